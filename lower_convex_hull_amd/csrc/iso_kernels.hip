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
    // block-relative S_k and W_k, stored at sk(k) = k + k / P: each thread's
    // points plus one pad slot, so that threads reading their own points (and
    // walkers reading points P apart) hit different LDS banks
    double S[NT * (P + 1) + 1];
    double W[WT ? NT * (P + 1) + 1 : 1];
    int16_t prv[NT * P + 1];        // hull neighbours of each vertex (the walks' links)
    int16_t nxt[NT * P + 1];
    uint32_t mask[NT];
    int16_t bra[2 * NT];            // bridge ends of every merge, by round
    int16_t brb[2 * NT];
    double red[NT / 64 + 1];
    int ired[NT / 64 + 1];
    int flag;
};

template <int P>
__device__ __forceinline__ int sk(int k) {
    return k + k / P;
}

template <int NT, int P, bool WT>
struct Block {
    HullSmem<NT, P, WT>& sm;
    int len;  // real elements in the block; points beyond len repeat point len

    __device__ __forceinline__ Pt pt(int k) const {
        Pt p;
        p.s = sm.S[sk<P>(k)];
        p.w = WT ? sm.W[sk<P>(k)] : (double)min(k, len);
        return p;
    }
};

// Makes one lane's LDS writes visible to the other lanes of its wave and keeps
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
}

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
        sm.S[sk<P>(base + b + 1)] = xs + ps[b];
        if (WT) sm.W[sk<P>(base + b + 1)] = xw + pw[b];
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
    __syncthreads();

    // ---- links between consecutive vertices of the thread hulls; a thread's
    // last point is the next thread's first (bit 0, always a vertex)
    {
        const uint32_t pm = L > 0 ? sm.mask[L - 1] : 0u;
        int prev_v = L > 0 ? (L - 1) * P + msb32(pm) : 0;
        uint32_t bits = my;
        while (bits) {
            const int b = lsb32(bits);
            bits &= bits - 1u;
            const int k = base + b;
            sm.prv[k] = (int16_t)prev_v;
            sm.nxt[k] = (int16_t)(bits ? base + lsb32(bits) : base + P);
            prev_v = k;
        }
        if (L == NT - 1) sm.prv[NT * P] = (int16_t)prev_v;
    }
    __syncthreads();

    // ---- merge the thread hulls pairwise (paper section 3.2; Lemma 4.2's
    // walk).  The first thread of each pair of groups walks to the bridge over
    // the links and relinks its two ends; the rounds inside a wave need no
    // workgroup barrier.  The removed vertices' bits are cleared at the end.
    constexpr int R = __builtin_ctz(NT);
    for (int r = 0; r < R; ++r) {
        const int g = 2 << r, half = 1 << r;
        if ((L & (g - 1)) == 0) {
            const int lo_pt = L * P, hi_pt = (L + g) * P;
            const int s = (L + half) * P;
            int a = sm.prv[s];
            int b = sm.nxt[s];
            Pt Pa = B.pt(a), Ps = B.pt(s), Pb = B.pt(b);
            if (cross3(Pa, Ps, Pb) > 0.0) {
                a = s;
                b = s;  // convex at s: nothing removed
            } else {
                // a moves left while its turn towards b is not strictly left,
                // b moves right likewise, until neither moves.  Every move
                // removes a vertex, so the walk ends; the cap only guards.
                for (int pass = 0; pass < 2 * NT * P + 4; ++pass) {
                    bool moved = false;
                    while (a > lo_pt) {
                        const int a2 = sm.prv[a];
                        const Pt P2 = B.pt(a2);
                        if (cross3(P2, Pa, Pb) <= 0.0) { a = a2; Pa = P2; moved = true; }
                        else break;
                    }
                    while (b < hi_pt) {
                        const int b2 = sm.nxt[b];
                        const Pt P2 = B.pt(b2);
                        if (cross3(Pa, Pb, P2) <= 0.0) { b = b2; Pb = P2; moved = true; }
                        else break;
                    }
                    if (!moved) break;
                }
                sm.nxt[a] = (int16_t)b;
                sm.prv[b] = (int16_t)a;
            }
            sm.bra[(NT >> r) + (L >> (r + 1))] = (int16_t)a;
            sm.brb[(NT >> r) + (L >> (r + 1))] = (int16_t)b;
        }
        if (g < 64) wave_sync();
        else __syncthreads();
    }
    if (NT <= 64) __syncthreads();
    // ---- clear the bits of vertices strictly inside any bridge of this
    // thread's groups
    for (int r = 0; r < R; ++r) {
        const int i = (NT >> r) + (L >> (r + 1));
        const int a = sm.bra[i], b = sm.brb[i];
        const int k0 = max(a + 1, base), k1 = min(b - 1, base + P - 1);
        if (k0 <= k1) {
            const uint32_t clr = ((k1 - base == 31) ? 0xffffffffu : ((2u << (k1 - base)) - 1u)) &
                                 ~((1u << (k0 - base)) - 1u);
            my &= ~clr;
        }
    }
    sm.mask[L] = my;
    __syncthreads();
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
        ws.slot_S[slot + rank] = sm.S[sk<P>(k)];
        if (WT) ws.slot_W[slot + rank] = sm.W[sk<P>(k)];
        const int e = wslot(rank);
        if (e >= 0) wr->v[e] = make_double2(sm.S[sk<P>(k)], WT ? sm.W[sk<P>(k)] : (double)min(k, len));
        ++rank;
    }
    if (L == NT - 1) {
        // the chunk's last point (point len; padding repeats it) ends the hull
        ws.slot_idx[slot + total] = (uint16_t)len;
        ws.slot_S[slot + total] = sm.S[sk<P>(C)];
        if (WT) ws.slot_W[slot + total] = sm.W[sk<P>(C)];
        wr->v[wslot(total)] = make_double2(sm.S[sk<P>(C)], WT ? sm.W[sk<P>(C)] : (double)len);
        wr->h = h;
        ws.hull_cnt[gid] = h;
        ws.tot_S[gid] = sm.S[sk<P>(C)];
        if (WT) ws.tot_W[gid] = sm.W[sk<P>(C)];
        ws.chunk_flag[gid] = sm.flag;
    }
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
