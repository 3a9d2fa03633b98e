// gfx950 kernels of the batched weighted isotonic fit.
//
// The fit of a row is the slope sequence of the lower convex hull of its
// cumulative sum diagram P_k = (W_k, S_k) (paper "Merge Hulls Without Copying
// Vertices: GPU Isotonic Regression", section 2.1, equations (2)-(3)).  The
// kernels build that hull in three levels (paper section 3):
//
//   thread  - the hull of its 16 consecutive points, a monotone chain whose
//             stack is a bit mask (section 3.1);
//   group   - the threads of a workgroup merge their hulls pairwise by walking
//             to the bridge and clearing the bits under it (section 3.2);
//   row     - chunk hulls, written once to the workspace, are merged up a tree
//             whose nodes are lists of segments of chunk hulls, at most one
//             per chunk (section 3.3, Definition 4.3, Theorem 4.4).
//
// and reconstruct the fit from the root list (section 3.4, Corollary 4.5).
// Rows of at most 4096 elements are finished inside one workgroup.
//
// All coordinates are f64: chunk-relative inside a chunk, plus f64 chunk starts
// from a scan of the chunk totals.  (The pages' float pairs and exponent
// filters, section 6 "Coordinates" and appendix B, exist because their GPU ran
// f64 at a thirty-second of the f32 rate; gfx950 runs f64 FMA at the f32 rate.)
#include "iso_kernels.hpp"

#include <math.h>

#include "iso_device.hpp"

namespace iso {
namespace {

// ----------------------------------------------------------------------------
// The hull of one workgroup's points.
//
// Thread L owns points L*P .. L*P+P of the block (P+1 points; its last point
// is thread L+1's first).  Bits 0..P-1 of mask[L] mark which of points
// L*P .. L*P+P-1 are vertices; the block's last point NT*P is always one.
// ----------------------------------------------------------------------------
template <int NT, int P, bool WT>
struct HullSmem {
    double S[NT * P + 1];            // block-relative S_k
    double W[WT ? NT * P + 1 : 1];   // block-relative W_k (weighted only)
    uint32_t mask[NT];
    uint32_t occ[(NT + 31) / 32];    // bit L: mask[L] != 0
    int32_t blo[NT];                 // bridge ends of the merge led by thread L
    int32_t bhi[NT];
    double red[NT / 64 + 1];
    int ired[NT / 64 + 1];
    int flag;
};

template <int NT, int P, bool WT>
struct Block {
    HullSmem<NT, P, WT>& sm;
    int len;  // real elements in the block; points beyond len repeat point len

    __device__ __forceinline__ Pt pt(int k) const {
        Pt p;
        p.s = sm.S[k];
        p.w = WT ? sm.W[k] : (double)min(k, len);
        return p;
    }

    // Highest vertex below point k, searching threads >= lo_lane.
    __device__ int prev_vertex(int k, int lo_lane) const {
        int Lk = k / P;
        int b = k - Lk * P;
        if (Lk < NT && b > 0) {
            uint32_t m = sm.mask[Lk] & ((1u << b) - 1u);
            if (m) return Lk * P + msb32(m);
        }
        int x = Lk - 1;
        while (x >= lo_lane) {
            int wi = x >> 5;
            uint32_t word = sm.occ[wi] & ((2u << (x & 31)) - 1u);
            if (word) {
                int c = (wi << 5) + msb32(word);
                if (c < lo_lane) break;
                return c * P + msb32(sm.mask[c]);
            }
            x = (wi << 5) - 1;
        }
        return lo_lane * P;  // the group's first point is always a vertex
    }

    // Lowest vertex above point k among threads < hi_lane, else the group's
    // last point hi_lane*P.
    __device__ int next_vertex(int k, int hi_lane) const {
        int Lk = k / P;
        int b = k - Lk * P;
        if (Lk < hi_lane) {
            uint32_t m = sm.mask[Lk] & ~((2u << b) - 1u);
            if (m) return Lk * P + lsb32(m);
        }
        int x = Lk + 1;
        while (x < hi_lane) {
            int wi = x >> 5;
            uint32_t word = sm.occ[wi] & ~((1u << (x & 31)) - 1u);
            if (word) {
                int c = (wi << 5) + lsb32(word);
                if (c >= hi_lane) break;
                return c * P + lsb32(sm.mask[c]);
            }
            x = (wi + 1) << 5;
        }
        return hi_lane * P;
    }
};

// Loads the block's elements, forms the block-relative cumulative sums, and
// leaves in sm.mask the vertices of the block's lower hull.  Returns this
// thread's element values (sign applied, sanitised) in yv.
template <int NT, int P, bool WT>
__device__ void block_hull(HullSmem<NT, P, WT>& sm, const float* __restrict__ gy,
                           const float* __restrict__ gw, int len, float sign, float (&yv)[P]) {
    const int L = threadIdx.x;
    const int base = L * P;
    float wv[P];
    int bad = 0;
    if (threadIdx.x == 0) sm.flag = 0;

    // ---- load (each thread its P consecutive elements) and check the data
    float yr[P], wr[P];
    const bool whole = base + P <= len;
    if (P % 4 == 0 && whole && ((((uintptr_t)(gy + base)) | (WT ? (uintptr_t)(gw + base) : 0)) & 15u) == 0) {
#pragma unroll
        for (int q = 0; q < P / 4; ++q) {
            float4 v = reinterpret_cast<const float4*>(gy + base)[q];
            yr[4 * q] = v.x; yr[4 * q + 1] = v.y; yr[4 * q + 2] = v.z; yr[4 * q + 3] = v.w;
            if (WT) {
                float4 u = reinterpret_cast<const float4*>(gw + base)[q];
                wr[4 * q] = u.x; wr[4 * q + 1] = u.y; wr[4 * q + 2] = u.z; wr[4 * q + 3] = u.w;
            }
        }
    } else {
#pragma unroll
        for (int b = 0; b < P; ++b) {
            int e = base + b;
            yr[b] = e < len ? gy[e] : 0.0f;
            if (WT) wr[b] = e < len ? gw[e] : 0.0f;
        }
    }
#pragma unroll
    for (int b = 0; b < P; ++b) {
        int e = base + b;
        bool in = e < len;
        float yy = yr[b];
        float ww = 1.0f;
        if (WT) ww = wr[b];
        if (in) {
            if (!isfinite(yy)) { bad |= kFlagNonfinite; yy = 0.0f; }
            if (WT && !(ww > 0.0f && isfinite(ww))) { bad |= kFlagWeight; ww = 1.0f; }
        } else {
            ww = 0.0f;
        }
        yv[b] = sign * yy;
        wv[b] = ww;
    }

    // ---- prefix sums (paper section 2.1, equation (2)), in f64
    double ps[P];
    double pw[P];
    double ls = 0.0, lw = 0.0;
#pragma unroll
    for (int b = 0; b < P; ++b) {
        if (WT) {
            ls += (double)wv[b] * (double)yv[b];  // exact product of two f32
            lw += (double)wv[b];
            pw[b] = lw;
        } else {
            ls += (double)yv[b];
        }
        ps[b] = ls;
    }
    double tot;
    double xs = wg_excl_scan<NT>(ls, sm.red, &tot);
    double xw = 0.0;
    if (WT) xw = wg_excl_scan<NT>(lw, sm.red, &tot);
#pragma unroll
    for (int b = 0; b < P; ++b) {
        sm.S[base + b + 1] = xs + ps[b];
        if (WT) sm.W[base + b + 1] = xw + pw[b];
    }
    if (L == 0) {
        sm.S[0] = 0.0;
        if (WT) sm.W[0] = 0.0;
    }
    if (bad) atomicOr(&sm.flag, bad);

    // ---- candidates: point k is a vertex only if the slope into it (the
    // value of element k-1) is below the slope out of it (element k).  Points
    // next to a padding element are kept as candidates; padding points
    // (beyond len) that are not thread ends are dropped, since they repeat
    // point len.
    uint32_t cand = 1u | (1u << P);
#pragma unroll
    for (int k = 1; k < P; ++k) {
        int pidx = base + k;
        bool realL = pidx - 1 < len, realR = pidx < len;
        bool c;
        if (pidx > len) c = false;
        else if (realL && realR) c = yv[k - 1] < yv[k];
        else c = true;
        if (c) cand |= 1u << k;
    }
    __syncthreads();

    Block<NT, P, WT> B{sm, len};

    // ---- thread hull: monotone chain over the candidates, the stack a bit
    // mask (paper section 3.1).  Each pass pops or pushes; both outcomes need
    // one LDS load, whose address is selected first.
    const uint32_t full = (P == 31) ? 0xffffffffu : ((2u << P) - 1u);
    uint32_t stk;
    if (cand == full) {
        stk = full;  // every point locally convex: the chain keeps them all
    } else {
        stk = 1u;
        int t = 0, u = -1;
        Pt T = B.pt(base), U = T;
        uint32_t rest = cand & ~1u;
        int c = lsb32(rest);
        Pt Cp = B.pt(base + c);
        for (int it = 0; it < 2 * P + 2 && c <= P; ++it) {
            bool pop = (u >= 0) && (cross3(U, T, Cp) <= 0.0);
            int addr;
            if (pop) {
                stk &= ~(1u << t);
                t = u;
                T = U;
                uint32_t below = stk & ((1u << u) - 1u);
                u = below ? msb32(below) : -1;
                addr = u < 0 ? 0 : u;
            } else {
                stk |= 1u << c;
                u = t;
                U = T;
                t = c;
                T = Cp;
                uint32_t above = cand & ~((2u << c) - 1u);
                c = above ? lsb32(above) : P + 1;
                addr = c > P ? P : c;
            }
            Pt Lp = B.pt(base + addr);
            if (pop) U = Lp;
            else Cp = Lp;
        }
    }
    uint32_t my = stk & ((1u << P) - 1u);
    sm.mask[L] = my;
    {
        unsigned long long bal = __ballot(my != 0u);
        if ((L & 31) == 0) sm.occ[L >> 5] = (uint32_t)(bal >> (L & 32));
    }
    __syncthreads();

    // ---- merge the thread hulls pairwise (paper section 3.2; Lemma 4.2's
    // walk).  The first thread of each pair of groups walks to the bridge;
    // then every thread clears its bits strictly inside the bridge.
    for (int r = 0; (1 << r) < NT; ++r) {
        const int g = 2 << r, half = 1 << r;
        if ((L & (g - 1)) == 0) {
            const int lo_lane = L, hi_lane = L + g;
            const int s = (L + half) * P;
            const int lo_pt = lo_lane * P, hi_pt = hi_lane * P;
            int a = B.prev_vertex(s, lo_lane);
            int b = B.next_vertex(s, hi_lane);
            Pt Pa = B.pt(a), Ps = B.pt(s), Pb = B.pt(b);
            if (cross3(Pa, Ps, Pb) > 0.0) {
                a = s;
                b = s;  // convex at s: nothing removed
            } else {
                // walk: a moves left while its turn towards b is not strictly
                // left, b moves right likewise, until neither moves.  Every
                // move removes a vertex, so the walk ends; the cap only guards.
                for (int pass = 0; pass < 2 * NT * P + 4; ++pass) {
                    bool moved = false;
                    while (a > lo_pt) {
                        int a2 = B.prev_vertex(a, lo_lane);
                        Pt P2 = B.pt(a2);
                        if (cross3(P2, Pa, Pb) <= 0.0) { a = a2; Pa = P2; moved = true; }
                        else break;
                    }
                    while (b < hi_pt) {
                        int b2 = B.next_vertex(b, hi_lane);
                        Pt P2 = B.pt(b2);
                        if (cross3(Pa, Pb, P2) <= 0.0) { b = b2; Pb = P2; moved = true; }
                        else break;
                    }
                    if (!moved) break;
                }
            }
            sm.blo[L] = a;
            sm.bhi[L] = b;
        }
        __syncthreads();
        {
            const int ldr = L & ~(g - 1);
            const int a = sm.blo[ldr], b = sm.bhi[ldr];
            int k0 = max(a + 1, base), k1 = min(b - 1, base + P - 1);
            if (k0 <= k1) {
                uint32_t clr = ((k1 - base == 31) ? 0xffffffffu : ((2u << (k1 - base)) - 1u)) &
                               ~((1u << (k0 - base)) - 1u);
                my &= ~clr;
                sm.mask[L] = my;
            }
            unsigned long long bal = __ballot(my != 0u);
            if ((L & 31) == 0) sm.occ[L >> 5] = (uint32_t)(bal >> (L & 32));
        }
        __syncthreads();
    }
}

// ----------------------------------------------------------------------------
// Short rows: the whole row in one workgroup, fit written directly.
// ----------------------------------------------------------------------------
template <int NT, int P, bool WT>
__global__ __launch_bounds__(NT) void k_short_rows(const float* __restrict__ y,
                                                   const float* __restrict__ w, int64_t n,
                                                   float sign, float* __restrict__ out,
                                                   int32_t* __restrict__ block_id,
                                                   int32_t* __restrict__ row_flag) {
    __shared__ HullSmem<NT, P, WT> sm;
    const int64_t row = blockIdx.x;
    const float* gy = y + row * n;
    const float* gw = WT ? w + row * n : nullptr;
    const int len = (int)n;
    float yv[P];
    block_hull<NT, P, WT>(sm, gy, gw, len, sign, yv);

    const int L = threadIdx.x;
    const int base = L * P;
    const uint32_t my = sm.mask[L];
    const int flag = sm.flag;
    if (L == 0) row_flag[row] = flag;
    float* go = out + row * n;
    int32_t* gb = block_id ? block_id + row * n : nullptr;
    if (flag & kFlagNonfinite) {
        for (int b = 0; b < P; ++b) {
            int e = base + b;
            if (e < len) {
                go[e] = __builtin_nanf("");
                if (gb) gb[e] = -1;
            }
        }
        return;
    }
    // vertex before this thread's points (max-scan from the left) and the first
    // vertex after them (min-scan from the right); vertex count before them.
    int lastv = my ? base + msb32(my) : -1;
    int firstv = my ? base + lsb32(my) : NT * P;
    int cnt = __popc(my);
    __shared__ int s_last[NT];
    __shared__ int s_first[NT];
    s_last[L] = lastv;
    s_first[L] = firstv;
    int total;
    int before = wg_excl_scan_int<NT>(cnt, sm.ired, &total);  // contains a barrier
    int prev_in = -1;
    int next_in = NT * P;
    for (int k = L - 1; k >= 0; --k) {
        int v = s_last[k];
        if (v >= 0) { prev_in = v; break; }
    }
    for (int k = L + 1; k < NT; ++k) {
        int v = s_first[k];
        if (v < NT * P) { next_in = v; break; }
    }
    Block<NT, P, WT> B{sm, len};
#pragma unroll
    for (int b = 0; b < P; ++b) {
        int e = base + b;
        if (e >= len) break;
        uint32_t upto = (b == 31) ? 0xffffffffu : ((2u << b) - 1u);
        uint32_t below = my & upto;
        uint32_t above = my & ~upto;
        int pv = below ? base + msb32(below) : prev_in;
        int nv = above ? base + lsb32(above) : next_in;
        float val;
        if (pv == e && nv == e + 1) {
            val = yv[b];  // both ends are vertices: the edge is the element itself
        } else {
            Pt A = B.pt(pv), C = B.pt(nv);
            val = (float)((C.s - A.s) / (C.w - A.w));
        }
        go[e] = sign * val;
        if (gb) gb[e] = before + __popc(below) - 1;  // point 0 is always a vertex
    }
}

// ----------------------------------------------------------------------------
// Long rows, phase 1: one workgroup per chunk builds the chunk's hull and
// writes it once to its slot (paper section 3.3), with the chunk's totals.
// ----------------------------------------------------------------------------
template <bool WT>
__global__ __launch_bounds__(kLongNT) void k_chunk_hulls(const float* __restrict__ y,
                                                         const float* __restrict__ w, int64_t n,
                                                         int m, float sign, LongWs ws) {
    constexpr int NT = kLongNT, P = kLongP, C = kChunk;
    __shared__ HullSmem<NT, P, WT> sm;
    const int64_t gid = blockIdx.x;  // row * m + chunk
    const int64_t row = gid / m;
    const int j = (int)(gid - row * m);
    const int64_t off = row * n + (int64_t)j * C;
    const int len = (int)min((int64_t)C, n - (int64_t)j * C);
    float yv[P];
    block_hull<NT, P, WT>(sm, y + off, WT ? w + off : nullptr, len, sign, yv);

    const int L = threadIdx.x;
    const int base = L * P;
    const uint32_t my = sm.mask[L];
    int total;
    int rank = wg_excl_scan_int<NT>(__popc(my), sm.ired, &total);
    const size_t slot = (size_t)gid * (C + 1);
    const int h = total + 1;
    WinRec* wr = ws.win + gid;
    // window entry of hull rank r, or -1 if r is in the middle of a long hull
    auto wslot = [&](int r) {
        if (h <= 2 * kWinK || r < kWinK) return r;
        return r >= h - kWinK ? kWinK + r - (h - kWinK) : -1;
    };
    uint32_t bits = my;
    while (bits) {
        int b = lsb32(bits);
        bits &= bits - 1u;
        int k = base + b;
        ws.slot_idx[slot + rank] = (uint16_t)min(k, len);
        ws.slot_S[slot + rank] = sm.S[k];
        if (WT) ws.slot_W[slot + rank] = sm.W[k];
        const int e = wslot(rank);
        if (e >= 0) wr->v[e] = make_double2(sm.S[k], WT ? sm.W[k] : (double)min(k, len));
        ++rank;
    }
    if (L == NT - 1) {
        // the chunk's last point (point len; padding repeats it) ends the hull
        ws.slot_idx[slot + total] = (uint16_t)len;
        ws.slot_S[slot + total] = sm.S[C];
        if (WT) ws.slot_W[slot + total] = sm.W[C];
        wr->v[wslot(total)] = make_double2(sm.S[C], WT ? sm.W[C] : (double)len);
        wr->h = h;
        ws.hull_cnt[gid] = h;
        ws.tot_S[gid] = sm.S[C];
        if (WT) ws.tot_W[gid] = sm.W[C];
        ws.chunk_flag[gid] = sm.flag;
    }
}

// ----------------------------------------------------------------------------
// Long rows, phase 2: the merge tree over segment lists (paper section 3.3,
// Algorithm 1, Definition 4.3, Theorem 4.4), one workgroup per row, a thread
// per merge, every level in one launch.  Then the per-chunk reconstruction
// records (section 3.4, Corollary 4.5).
// ----------------------------------------------------------------------------
// Bridge of the neighbouring lists L and R (Algorithm 1; Lemma 4.2): A is the
// last vertex of L that stays, B the first vertex of R that stays.  In the
// convex case A is the shared point s (kept once, in L) and B its successor.
struct Bridge {
    Cur A;
    Cur B;
};

// Tests the chain at the shared point s.  Returns true when it is convex (the
// bridge is then {A, B} as set); otherwise A, B are s's two neighbours, where
// the walk starts.
__device__ __forceinline__ bool bridge_start(const RowView X, const List Lq, const List Rq,
                                             int jr, Cur& A, Cur& B) {
    Cur sL = Lq.last();
    Cur sR = Rq.first();
    Pt Ps = Rq.pt(X, sR, jr);
    A = Lq.prev(sL);  // every node has at least its two end points
    B = Rq.next(sR);
    Pt PA = Lq.pt(X, A, jr), PB = Rq.pt(X, B, jr);
    if (cross3(PA, Ps, PB) > 0.0) {
        A = sL;
        return true;
    }
    return false;
}

// The walk of Lemma 4.2 by one thread: A moves left while its turn towards B is
// not strictly left, B moves right likewise, until neither moves.  Returns
// false if it gives up after `cap` steps (A, B then hold where it stopped; a
// resumed walk reaches the same bridge).
__device__ __forceinline__ bool walk_thread(const RowView X, const List Lq, const List Rq, int jr, Cur& A,
                            Cur& B, int cap) {
    Pt PA = Lq.pt(X, A, jr), PB = Rq.pt(X, B, jr);
    int steps = 0;
    for (;;) {
        bool moved = false;
        while (!Lq.is_first(A) && steps < cap) {
            Cur A2 = Lq.prev(A);
            Pt P2 = Lq.pt(X, A2, jr);
            if (cross3(P2, PA, PB) <= 0.0) { A = A2; PA = P2; moved = true; ++steps; }
            else break;
        }
        while (!Rq.is_last(B) && steps < cap) {
            Cur B2 = Rq.next(B);
            Pt P2 = Rq.pt(X, B2, jr);
            if (cross3(PA, PB, P2) <= 0.0) { B = B2; PB = P2; moved = true; ++steps; }
            else break;
        }
        if (!moved) return true;
        if (steps >= cap) return false;
    }
}

// Nested bisection (paper section 3.3, Theorem 5.2): A is the first vertex of L
// whose successor does not lie below A's tangent line to R; B is where that
// tangent touches R.  Used when a walk gives up.
__device__ __noinline__ Bridge bisect_bridge(const RowView X, const List Lq, const List Rq, int jr) {
    const Cur sL = Lq.last();
    const Cur sR = Rq.first();
    const Cur A0 = Lq.prev(sL);
    const Cur B0 = Rq.next(sR);
    const Cur RL = Rq.last();
    auto tangent = [&](Pt Pa) -> Cur {
        return find_first(Rq, B0, RL, [&](Cur r) -> bool {
            if (Rq.is_last(r)) return true;
            Pt Pr = Rq.pt(X, r, jr);
            Pt Pn = Rq.pt(X, Rq.next(r), jr);
            return cross3(Pa, Pr, Pn) > 0.0;
        });
    };
    Cur A = find_first(Lq, Lq.first(), A0, [&](Cur c) -> bool {
        if (c.seg == A0.seg && c.pos == A0.pos) return true;
        Pt Pc = Lq.pt(X, c, jr);
        Cur t = tangent(Pc);
        Pt Pt_ = Rq.pt(X, t, jr);
        Pt Pn = Lq.pt(X, Lq.next(c), jr);
        return cross3(Pc, Pt_, Pn) >= 0.0;
    });
    Cur B = tangent(Lq.pt(X, A, jr));
    return Bridge{A, B};
}

// For the 64 lanes of a wave: the vertex `lane` positions before (dir < 0) or
// after (dir > 0) cursor C along the list, or valid = false past its end.
// Every lane of the wave must call it with the same C and dir.
__device__ __forceinline__ Cur wave_offset(const List Lq, Cur C, int dir, int lane, bool& valid) {
    const int sj = C.seg + dir * lane;
    int cnt = 0;
    if (sj >= 0 && sj < Lq.n) {
        uint2 d = Lq.d[sj];
        if (lane == 0) cnt = dir < 0 ? C.pos - dlo(d) + 1 : dhi(d) - C.pos + 1;
        else cnt = dhi(d) - dlo(d) + 1;
    }
    int cum = cnt;
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
        int t = __shfl_up(cum, k);
        if (lane >= k) cum += t;
    }
    const int total = __shfl(cum, 63);
    valid = lane < total;
    // j = number of segments whose cumulative count is <= lane
    int j = 0;
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) {
        int c = __shfl(cum, j + k - 1);
        if (c <= lane) j += k;
    }
    int before = __shfl(cum, j > 0 ? j - 1 : 0);
    if (j == 0) before = 0;
    if (!valid) return C;
    const int seg = C.seg + dir * j;
    const uint2 d = Lq.d[seg];
    const int top = (j == 0) ? C.pos : (dir < 0 ? dhi(d) : dlo(d));
    return Cur{seg, top + dir * (lane - before)};
}

__device__ __forceinline__ Pt shfl_down_pt(Pt p, int k) {
    return Pt{__shfl_down(p.w, k), __shfl_down(p.s, k)};
}
__device__ __forceinline__ Cur bcast_cur(Cur c, int src) {
    return Cur{__shfl(c.seg, src), __shfl(c.pos, src)};
}

// The same walk by a whole wave: each step tests the next 63 candidates at
// once (the pages' warp-per-merge search, section 3.3, on 64 lanes).  The
// candidate where a sequential walk would stop is the first lane whose test
// holds.  Returns false if it gives up after `cap` steps.
__device__ __forceinline__ bool walk_wave(const RowView X, const List Lq, const List Rq, int jr, Cur& A, Cur& B,
                          int cap) {
    const int lane = threadIdx.x & 63;
    int steps = 0;
    for (;;) {
        bool moved = false;
        // A moves left
        for (;;) {
            Pt PB = Rq.pt(X, B, jr);
            bool valid;
            Cur v = wave_offset(Lq, A, -1, lane, valid);
            Pt Pv = valid ? Lq.pt(X, v, jr) : Pt{0.0, 0.0};
            Pt Pu = shfl_down_pt(Pv, 1);
            bool vnext = __shfl_down((int)valid, 1) != 0;
            bool stop = valid && lane < 63 && (!vnext || cross3(Pu, Pv, PB) > 0.0);
            unsigned long long bal = __ballot(stop);
            if (bal) {
                int i = __ffsll((long long)bal) - 1;
                if (i > 0) moved = true;
                A = bcast_cur(v, i);
                break;
            }
            A = bcast_cur(v, 63);
            moved = true;
            if (++steps >= cap) return false;
        }
        // B moves right
        for (;;) {
            Pt PA = Lq.pt(X, A, jr);
            bool valid;
            Cur v = wave_offset(Rq, B, +1, lane, valid);
            Pt Pv = valid ? Rq.pt(X, v, jr) : Pt{0.0, 0.0};
            Pt Pn = shfl_down_pt(Pv, 1);
            bool vnext = __shfl_down((int)valid, 1) != 0;
            bool stop = valid && lane < 63 && (!vnext || cross3(PA, Pv, Pn) > 0.0);
            unsigned long long bal = __ballot(stop);
            if (bal) {
                int i = __ffsll((long long)bal) - 1;
                if (i > 0) moved = true;
                B = bcast_cur(v, i);
                break;
            }
            B = bcast_cur(v, 63);
            moved = true;
            if (++steps >= cap) return false;
        }
        if (!moved) return true;
    }
}

// Writes the cut of one merge: L ends at A, R starts at B; records what the
// descriptor move needs.
__device__ __forceinline__ void apply_cut(uint2* D, int32_t* CNT, int2* MI, int k, int a, int b,
                                          int nR, Bridge br) {
    uint2 dl = D[a + br.A.seg];
    D[a + br.A.seg] = mkdesc(dchunk(dl), dlo(dl), br.A.pos);
    uint2 dr = D[b + br.B.seg];
    D[b + br.B.seg] = mkdesc(dchunk(dr), br.B.pos, dhi(dr));
    MI[k] = make_int2(br.A.seg + 1, br.B.seg);
    CNT[a] = br.A.seg + 1 + (nR - br.B.seg);
}

// One workgroup per row runs every level of the merge tree.  Segment lists
// live in LDS when the row has at most kMergeLdsMax chunks (else in the
// workspace).  Per level: one thread per merge finds its bridge and cuts the two
// boundary segments in place; then teams of threads move each right list's
// remaining descriptors down behind the left list's (through a scratch copy,
// since the two ranges may overlap).
template <bool WT, bool INLDS>
__global__ __launch_bounds__(kMergeNT) void k_merge_rows(int m, LongWs ws) {
    constexpr int NT = kMergeNT;
    extern __shared__ uint2 dyn_lds[];
    __shared__ double red[NT / 64 + 1];
    __shared__ int ired[NT / 64 + 1];
    __shared__ int sflag;
    __shared__ int s_nhard;
    __shared__ int4 s_hard[kHardCap];
    constexpr int NW = NT / 64;
    const int64_t row = blockIdx.x;
    const int64_t rb = row * m;
    const int tid = threadIdx.x;
    const int wid = tid >> 6, wlane = tid & 63;

    uint2* D;
    uint2* SCR;
    int32_t* CNT;
    int2* MI;
    int32_t* HC;
    double* STS;
    double* STW;
    if (INLDS) {
        D = dyn_lds;
        SCR = D + m;
        MI = reinterpret_cast<int2*>(SCR + m);
        STS = reinterpret_cast<double*>(MI + (m / 2 + 1));
        STW = STS + m;  // used when weighted
        CNT = reinterpret_cast<int32_t*>(STW + (WT ? m : 0));
        HC = CNT + m;
    } else {
        D = ws.desc + rb;
        SCR = ws.desc_scr + rb;
        CNT = ws.node_cnt + rb;
        MI = ws.merge_info + rb;
        HC = ws.hull_cnt + rb;
        STS = ws.st_S + rb;
        STW = WT ? ws.st_W + rb : nullptr;
    }

    // ---- row flags, chunk starts (exclusive scan of the chunk totals)
    if (tid == 0) sflag = 0;
    __syncthreads();
    int f = 0;
    for (int j = tid; j < m; j += NT) f |= ws.chunk_flag[rb + j];
    if (f) atomicOr(&sflag, f);
    double carryS = 0.0, carryW = 0.0;
    for (int t0 = 0; t0 < m; t0 += NT) {
        int j = t0 + tid;
        double vs = j < m ? ws.tot_S[rb + j] : 0.0;
        double tot;
        double xs = wg_excl_scan<NT>(vs, red, &tot);
        if (j < m) STS[j] = carryS + xs;
        carryS += tot;
        if (WT) {
            double vw = j < m ? ws.tot_W[rb + j] : 0.0;
            double xw = wg_excl_scan<NT>(vw, red, &tot);
            if (j < m) STW[j] = carryW + xw;
            carryW += tot;
        }
    }
    for (int j = tid; j < m; j += NT) {
        const int h = ws.hull_cnt[rb + j];
        if (INLDS) HC[j] = h;
        D[j] = mkdesc(j, 0, h - 1);
        CNT[j] = 1;
    }
    // warm this XCD's L2 with the compact hull ends of the whole row
    {
        const double2* wv = reinterpret_cast<const double2*>(ws.win + rb);
        const int nv2 = m * (int)(sizeof(WinRec) / sizeof(double2));
        double acc = 0.0;
        for (int i = tid; i < nv2; i += NT) acc += wv[i].x;
        keep(acc);
    }
    __syncthreads();
    if (tid == 0) ws.row_flag[row] = sflag;

    const size_t sl = (size_t)rb * (kChunk + 1);
    RowView X{ws.slot_idx + sl, ws.slot_S + sl, WT ? ws.slot_W + sl : nullptr, ws.win + rb, HC,
              STS, WT ? STW : nullptr, WT};

    // ---- the merge tree, level by level
    for (int span = 1; span < m; span <<= 1) {
        const int nm = (m - span + 2 * span - 1) / (2 * span);
        if (nm > NW) {
            // many merges: a thread each; walks that run long go to the waves
            if (tid == 0) s_nhard = 0;
            __syncthreads();
            for (int k = tid; k < nm; k += NT) {
                const int a = 2 * k * span, b = a + span;
                List Lq{D + a, CNT[a]};
                List Rq{D + b, CNT[b]};
                Bridge br;
                if (!bridge_start(X, Lq, Rq, b, br.A, br.B) &&
                    !walk_thread(X, Lq, Rq, b, br.A, br.B, kWalkCap)) {
                    int h = atomicAdd(&s_nhard, 1);
                    if (h < kHardCap) {
                        s_hard[h] = make_int4(k, br.A.seg, br.A.pos, (br.B.seg << 16) | br.B.pos);
                        continue;
                    }
                    br = bisect_bridge(X, Lq, Rq, b);
                }
                apply_cut(D, CNT, MI, k, a, b, Rq.n, br);
            }
            __syncthreads();
            const int nh = min(s_nhard, kHardCap);
            for (int h = wid; h < nh; h += NW) {
                const int4 hk = s_hard[h];
                const int k = hk.x, a = 2 * k * span, b = a + span;
                List Lq{D + a, CNT[a]};
                List Rq{D + b, CNT[b]};
                Bridge br{Cur{hk.y, hk.z}, Cur{hk.w >> 16, hk.w & 0xffff}};
                if (!walk_wave(X, Lq, Rq, b, br.A, br.B, kWaveWalkCap) && wlane == 0)
                    br = bisect_bridge(X, Lq, Rq, b);
                if (wlane == 0) apply_cut(D, CNT, MI, k, a, b, Rq.n, br);
            }
        } else {
            // few merges: a wave each
            for (int k = wid; k < nm; k += NW) {
                const int a = 2 * k * span, b = a + span;
                List Lq{D + a, CNT[a]};
                List Rq{D + b, CNT[b]};
                Bridge br;
                if (!bridge_start(X, Lq, Rq, b, br.A, br.B)) {
                    if (!walk_wave(X, Lq, Rq, b, br.A, br.B, kWaveWalkCap) && wlane == 0)
                        br = bisect_bridge(X, Lq, Rq, b);
                }
                if (wlane == 0) apply_cut(D, CNT, MI, k, a, b, Rq.n, br);
            }
        }
        __syncthreads();
        // move the right lists' tails: teams of ts threads per merge
        int ts = NT / nm;
        ts = ts < 1 ? 1 : (1 << (31 - __clz(ts)));
        const int teams = NT / ts;
        const int lane = tid & (ts - 1);
        for (int k = tid / ts; k < nm; k += teams) {
            const int b = (2 * k + 1) * span;
            const int rs = MI[k].y;
            const int nr = CNT[b] - rs;
            for (int i = lane; i < nr; i += ts) SCR[b + i] = D[b + rs + i];
        }
        __syncthreads();
        for (int k = tid / ts; k < nm; k += teams) {
            const int a = 2 * k * span, b = a + span;
            const int nl = MI[k].x;
            const int nr = CNT[b] - MI[k].y;
            for (int i = lane; i < nr; i += ts) D[a + nl + i] = SCR[b + i];
        }
        __syncthreads();
    }

    // ---- reconstruction records (Corollary 4.5)
    write_records<NT>(X, D, CNT[0], m, ws.vb + rb, ws.rec + rb, ired);
}

// ----------------------------------------------------------------------------
// Long rows, phase 3: every element takes the slope of the row-hull edge above
// it (paper equation (3), section 3.4).
// ----------------------------------------------------------------------------
template <bool WT>
__global__ __launch_bounds__(kLongNT) void k_expand(int64_t n, int m, float sign, LongWs ws,
                                                    float* __restrict__ out,
                                                    int32_t* __restrict__ block_id) {
    constexpr int NT = kLongNT, C = kChunk;
    constexpr int G = C / (4 * NT);  // groups of 4 consecutive elements per thread
    __shared__ int vidx[C + 1];
    __shared__ float vslope[C + 1];
    const int64_t gid = blockIdx.x;
    const int64_t row = gid / m;
    const int j = (int)(gid - row * m);
    const int64_t off = row * n + (int64_t)j * C;
    const int len = (int)min((int64_t)C, n - (int64_t)j * C);
    float* go = out + off;
    int32_t* gb = block_id ? block_id + off : nullptr;
    const int tid = threadIdx.x;
    // element groups e = 4 * (g * NT + tid): consecutive threads write
    // consecutive 16-byte groups
    const bool vec = ((((uintptr_t)go) | (uintptr_t)gb) & 15u) == 0;
    auto store4 = [&](int e, float4 v, int4 b) {
        if (vec && e + 4 <= len) {
            *reinterpret_cast<float4*>(go + e) = v;
            if (gb) *reinterpret_cast<int4*>(gb + e) = b;
        } else {
            const float vv[4] = {v.x, v.y, v.z, v.w};
            const int bb[4] = {b.x, b.y, b.z, b.w};
            for (int t = 0; t < 4 && e + t < len; ++t) {
                go[e + t] = vv[t];
                if (gb) gb[e + t] = bb[t];
            }
        }
    };
    if (ws.row_flag[row] & kFlagNonfinite) {
        const float nan = __builtin_nanf("");
        for (int g = 0; g < G; ++g) {
            int e = 4 * (g * NT + tid);
            if (e < len) store4(e, make_float4(nan, nan, nan, nan), make_int4(-1, -1, -1, -1));
        }
        return;
    }
    const ChunkRec rc = ws.rec[gid];
    if (rc.lo < 0) {
        const float v = sign * (float)rc.slope_in;
        const int b = rc.vb - 1;
        for (int g = 0; g < G; ++g) {
            int e = 4 * (g * NT + tid);
            if (e < len) store4(e, make_float4(v, v, v, v), make_int4(b, b, b, b));
        }
        return;
    }
    const int nv = rc.hi - rc.lo + 1;
    const size_t slot = (size_t)gid * (C + 1) + rc.lo;
    for (int v = tid; v < nv; v += NT) vidx[v] = ws.slot_idx[slot + v];
    for (int v = tid; v + 1 < nv; v += NT) {
        double ds = ws.slot_S[slot + v + 1] - ws.slot_S[slot + v];
        double dw = WT ? ws.slot_W[slot + v + 1] - ws.slot_W[slot + v]
                       : (double)((int)ws.slot_idx[slot + v + 1] - (int)ws.slot_idx[slot + v]);
        vslope[v] = sign * (float)(ds / dw);
    }
    __syncthreads();
    const float sin_ = sign * (float)rc.slope_in, sout = sign * (float)rc.slope_out;
    for (int g = 0; g < G; ++g) {
        const int e0 = 4 * (g * NT + tid);
        if (e0 >= len) break;
        // q = number of the chunk's surviving vertices at or before e0
        int lo = 0, hi = nv;
        while (lo < hi) {
            int mid = (lo + hi) >> 1;
            if (vidx[mid] <= e0) lo = mid + 1;
            else hi = mid;
        }
        int q = lo;
        float vv[4];
        int bb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int e = e0 + t;
            while (q < nv && vidx[q] <= e) ++q;
            vv[t] = (q == 0) ? sin_ : (q == nv ? sout : vslope[q - 1]);
            bb[t] = rc.vb + q - 1;
        }
        store4(e0, make_float4(vv[0], vv[1], vv[2], vv[3]), make_int4(bb[0], bb[1], bb[2], bb[3]));
    }
}

size_t merge_lds_bytes(int m, bool weighted) {
    // D, SCR (8 B each), MI (8 B per merge), STS (8 B), STW (8 B, weighted),
    // CNT, HC (4 B each)
    return (size_t)m * 16 + (size_t)(m / 2 + 1) * 8 + (size_t)m * (weighted ? 16 : 8) +
           (size_t)m * 8;
}

template <int NT, int P>
hipError_t launch_short_t(const float* y, const float* w, int64_t rows, int64_t n, float sign,
                          float* out, int32_t* block_id, int32_t* row_flag, hipStream_t st) {
    timed_begin(kPhaseShort, st);
    if (w)
        hipLaunchKernelGGL((k_short_rows<NT, P, true>), dim3((unsigned)rows), dim3(NT), 0, st, y, w,
                           n, sign, out, block_id, row_flag);
    else
        hipLaunchKernelGGL((k_short_rows<NT, P, false>), dim3((unsigned)rows), dim3(NT), 0, st, y,
                           w, n, sign, out, block_id, row_flag);
    timed_end(st);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_short(const float* y, const float* w, int64_t rows, int64_t n, float sign,
                        float* out, int32_t* block_id, int32_t* row_flag, hipStream_t st) {
    if (n <= 64) return launch_short_t<64, 1>(y, w, rows, n, sign, out, block_id, row_flag, st);
    if (n <= 128) return launch_short_t<64, 2>(y, w, rows, n, sign, out, block_id, row_flag, st);
    if (n <= 256) return launch_short_t<64, 4>(y, w, rows, n, sign, out, block_id, row_flag, st);
    if (n <= 512) return launch_short_t<64, 8>(y, w, rows, n, sign, out, block_id, row_flag, st);
    if (n <= 1024) return launch_short_t<64, 16>(y, w, rows, n, sign, out, block_id, row_flag, st);
    return launch_short_t<256, 16>(y, w, rows, n, sign, out, block_id, row_flag, st);
}

// The merge phase over segment lists: one workgroup per row, lists in LDS when
// they fit.
hipError_t launch_segment_merge(const LongShape& sh, const LongWs& ws, hipStream_t st) {
    const bool wt = sh.weighted;
    timed_begin(kPhaseMerge, st);
    if (sh.m <= kMergeLdsMax) {
        const size_t lds = merge_lds_bytes(sh.m, wt);
        static bool attr_set = false;
        if (!attr_set) {
            const int maxb = (int)merge_lds_bytes(kMergeLdsMax, true);
            (void)hipFuncSetAttribute((const void*)k_merge_rows<true, true>,
                                      hipFuncAttributeMaxDynamicSharedMemorySize, maxb);
            (void)hipFuncSetAttribute((const void*)k_merge_rows<false, true>,
                                      hipFuncAttributeMaxDynamicSharedMemorySize, maxb);
            attr_set = true;
        }
        if (wt)
            hipLaunchKernelGGL((k_merge_rows<true, true>), dim3((unsigned)sh.rows), dim3(kMergeNT), lds,
                               st, sh.m, ws);
        else
            hipLaunchKernelGGL((k_merge_rows<false, true>), dim3((unsigned)sh.rows), dim3(kMergeNT),
                               lds, st, sh.m, ws);
    } else {
        if (wt)
            hipLaunchKernelGGL((k_merge_rows<true, false>), dim3((unsigned)sh.rows), dim3(kMergeNT), 0,
                               st, sh.m, ws);
        else
            hipLaunchKernelGGL((k_merge_rows<false, false>), dim3((unsigned)sh.rows), dim3(kMergeNT),
                               0, st, sh.m, ws);
    }
    timed_end(st);
    return hipGetLastError();
}

hipError_t launch_long(const float* y, const float* w, const LongShape& sh, const LongWs& ws,
                       float* out, int32_t* block_id, bool copy_control, hipStream_t st) {
    const unsigned nblk = (unsigned)(sh.rows * sh.m);
    const bool wt = sh.weighted;
    timed_begin(kPhaseChunk, st);
    if (wt)
        hipLaunchKernelGGL(k_chunk_hulls<true>, dim3(nblk), dim3(kLongNT), 0, st, y, w, sh.n, sh.m,
                           sh.sign, ws);
    else
        hipLaunchKernelGGL(k_chunk_hulls<false>, dim3(nblk), dim3(kLongNT), 0, st, y, w, sh.n, sh.m,
                           sh.sign, ws);
    timed_end(st);
    hipError_t e = copy_control ? launch_copy_merge(sh, ws, st) : launch_segment_merge(sh, ws, st);
    if (e != hipSuccess) return e;
    timed_begin(kPhaseExpand, st);
    if (wt)
        hipLaunchKernelGGL(k_expand<true>, dim3(nblk), dim3(kLongNT), 0, st, sh.n, sh.m, sh.sign, ws,
                           out, block_id);
    else
        hipLaunchKernelGGL(k_expand<false>, dim3(nblk), dim3(kLongNT), 0, st, sh.n, sh.m, sh.sign,
                           ws, out, block_id);
    timed_end(st);
    return hipGetLastError();
}

}  // namespace iso
