// Device helpers shared by the fitting kernels (iso_kernels.hip) and the
// vertex-copying merge control (iso_copy.hip).  Internal to libiso.so.
#pragma once

#include "iso_kernels.hpp"

namespace iso {
namespace {

struct Pt {
    double w;
    double s;
};

// Phase stamp (measurement only): thread 0 of the workgroup records the
// 100 MHz real-time counter in slot k of its row of stamps, if there is one.
__device__ __forceinline__ void stamp(uint64_t* row, int k) {
    if (row && threadIdx.x == 0) row[k] = (uint64_t)wall_clock64();
}
__device__ __forceinline__ uint64_t* stamp_row(uint64_t* area, int64_t wg) {
    return area ? area + wg * kStampSlots : nullptr;
}

// z-component of (b - a) x (c - a).  For a, b, c in increasing abscissa, > 0
// means b lies strictly below the chord from a to c (a strict left turn), so b
// is a hull vertex of {a, b, c}; <= 0 means b is on or above the chord and is
// dropped (collinear middle points are not vertices, paper section 2.1).
// The two products are rounded separately (no fused multiply-add), so a
// repeated point or an exactly collinear triple gives exactly 0.
__device__ __forceinline__ double cross3(Pt a, Pt b, Pt c) {
    return mul_rn(b.w - a.w, c.s - a.s) - mul_rn(b.s - a.s, c.w - a.w);
}

// Makes one lane's LDS writes visible to the other lanes of its wave and keeps
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ int msb32(uint32_t x) { return 31 - __clz((int)x); }
__device__ __forceinline__ int lsb32(uint32_t x) { return __ffs((int)x) - 1; }

// ----------------------------------------------------------------------------
// Workgroup scans.
// ----------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ double wg_excl_scan(double v, double* red, double* total) {
    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    double x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        double t = __shfl_up(x, d);
        if (lane >= d) x += t;
    }
    double excl = __shfl_up(x, 1);
    if (lane == 0) excl = 0.0;
    if (lane == 63) red[wid] = x;
    __syncthreads();
    double before = 0.0, all = 0.0;
#pragma unroll
    for (int k = 0; k < NT / 64; ++k) {
        double t = red[k];
        if (k < wid) before += t;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + excl;
}

template <int NT>
__device__ __forceinline__ int wg_excl_scan_int(int v, int* red, int* total) {
    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int t = __shfl_up(x, d);
        if (lane >= d) x += t;
    }
    int excl = __shfl_up(x, 1);
    if (lane == 0) excl = 0;
    if (lane == 63) red[wid] = x;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int k = 0; k < NT / 64; ++k) {
        int t = red[k];
        if (k < wid) before += t;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + excl;
}

// Segment descriptors (Definition 4.3): the chunk (or group) a segment lies
// in and its first and last vertex positions.  uint2 packs the positions in
// 16 bits each (a chunk hull has at most kChunk + 1 vertices); int4 keeps 32
// bits (a group hull can be longer).
__device__ __forceinline__ int dchunk(uint2 d) { return (int)d.x; }
__device__ __forceinline__ int dlo(uint2 d) { return (int)(d.y & 0xffffu); }
__device__ __forceinline__ int dhi(uint2 d) { return (int)(d.y >> 16); }
__device__ __forceinline__ uint2 mkdesc(int j, int lo, int hi) {
    return make_uint2((uint32_t)j, (uint32_t)lo | ((uint32_t)hi << 16));
}
__device__ __forceinline__ int dchunk(int4 d) { return d.x; }
__device__ __forceinline__ int dlo(int4 d) { return d.y; }
__device__ __forceinline__ int dhi(int4 d) { return d.z; }
template <class DT>
__device__ __forceinline__ DT mkd(int j, int lo, int hi);
template <>
__device__ __forceinline__ uint2 mkd<uint2>(int j, int lo, int hi) {
    return mkdesc(j, lo, hi);
}
template <>
__device__ __forceinline__ int4 mkd<int4>(int j, int lo, int hi) {
    return make_int4(j, lo, hi, 0);
}

struct Cur {
    int seg;
    int pos;
};

// Where the points of a strictly increasing chunk (chunk flag kChunkInc) come
// from: the chunk's elements and its per-thread checkpoints.
struct IncSrc {
    const int32_t* cflag;  // chunk flags of the row (null: every chunk has a slot)
    const double* ckS;     // checkpoints of the row's chunks, kLongNT + 1 each
    const double* ckW;
    const void* y;         // the row's elements (f32, or f64 when f64)
    const void* w;
    float sign;
    int f64;
};

// ... for the chunks j0, j0+1, ... of a row (chunk j0 is chunk 0 of the view)
__device__ __forceinline__ IncSrc inc_src(const LongWs& ws, int64_t row, int m, int j0) {
    const int64_t cb = row * m + j0;
    const int64_t eb = row * ws.n + (int64_t)j0 * kChunk;
    const size_t es = ws.f64 ? 8 : 4;
    return IncSrc{ws.chunk_flag + cb, ws.ck_S + cb * (kLongNT + 1),
                  ws.ck_W ? ws.ck_W + cb * (kLongNT + 1) : nullptr,
                  static_cast<const char*>(ws.y) + eb * es,
                  ws.w ? static_cast<const char*>(ws.w) + eb * es : nullptr, ws.sign, ws.f64};
}

struct RowView {
    const uint16_t* idx;  // full slots (rarely read)
    const double* S;
    const double* W;
    const WinRec* win;    // compact hull ends
    const int32_t* hc;    // hull vertex counts
    const double* stS;    // chunk starts
    const double* stW;
    bool weighted;
    IncSrc inc;

    // The sums of elements 0..b of a thread's run, in the chunk kernel's order
    // and arithmetic (lw: the weights' sum when weighted).
    template <typename T>
    __device__ __forceinline__ double inc_sum(const T* gy, const T* gw, int b, double& lw) const {
        double ls = 0.0;
        lw = 0.0;
        const T sg = (T)inc.sign;
        for (int t = 0; t <= b; ++t) {
            T yy = gy[t];
            if (!isfinite(yy)) yy = T(0);
            const T yv = sg * yy;
            if (weighted) {
                T ww = gw[t];
                if (!(ww > T(0) && isfinite(ww))) ww = T(1);
                ls += (double)ww * (double)yv;
                lw += (double)ww;
            } else {
                ls += (double)yv;
            }
        }
        return ls;
    }

    // Point k of strictly increasing chunk j (chunk-relative), summed exactly
    // as the chunk kernel summed it: its thread's checkpoint plus that
    // thread's elements up to the point, in order.
    __device__ __forceinline__ Pt inc_point(int j, int k) const {
        constexpr int P = kLongP;
        Pt p;
        if (k == 0) return Pt{0.0, 0.0};
        const int L = (k - 1) / P, b = (k - 1) - L * P;
        const size_t c = (size_t)j * (kLongNT + 1) + L;
        if (b == P - 1) {
            p.s = inc.ckS[c + 1];
            p.w = weighted ? inc.ckW[c + 1] : (double)k;
            return p;
        }
        const int64_t e0 = (int64_t)j * kChunk + L * P;
        double ls = 0.0, lw = 0.0;
        if (inc.f64) {
            ls = inc_sum<double>(static_cast<const double*>(inc.y) + e0,
                                 weighted ? static_cast<const double*>(inc.w) + e0 : nullptr, b, lw);
        } else {
            ls = inc_sum<float>(static_cast<const float*>(inc.y) + e0,
                                weighted ? static_cast<const float*>(inc.w) + e0 : nullptr, b, lw);
        }
        p.s = inc.ckS[c] + ls;
        p.w = weighted ? inc.ckW[c] + lw : (double)k;
        return p;
    }

    // Vertex `pos` of chunk j's hull in chunk-relative coordinates: from the
    // compact window when it holds it, else from the full slot (or, for a
    // strictly increasing chunk, from its elements).
    __device__ __forceinline__ Pt vrel(int j, int pos) const {
        const int h = hc[j];
        int e = pos;
        if (h > 2 * kWinK && pos >= kWinK) e = pos >= h - kWinK ? kWinK + pos - (h - kWinK) : -1;
        Pt p;
        if (e >= 0) {
            const double2 v = win[j].v[e];
            p.s = v.x;
            p.w = v.y;
        } else if (inc.cflag && (inc.cflag[j] & kChunkInc)) {
            p = inc_point(j, pos);
        } else {
            const size_t o = (size_t)j * (kChunk + 1) + pos;
            p.s = S[o];
            p.w = weighted ? W[o] : (double)idx[o];
        }
        return p;
    }

    // The same vertex relative to chunk jr's start: the chunk-start difference
    // first, then the chunk-relative part.
    __device__ __forceinline__ Pt vtx(int j, int pos, int jr) const {
        const Pt v = vrel(j, pos);
        Pt p;
        p.s = (stS[j] - stS[jr]) + v.s;
        if (weighted) p.w = (stW[j] - stW[jr]) + v.w;
        else p.w = (double)((int64_t)(j - jr) * kChunk) + v.w;
        return p;
    }
};

template <class DT>
struct List {
    DT* d;
    int n;
    __device__ __forceinline__ Cur first() const { return Cur{0, dlo(d[0])}; }
    __device__ __forceinline__ Cur last() const { return Cur{n - 1, dhi(d[n - 1])}; }
    __device__ __forceinline__ bool is_first(Cur c) const { return c.seg == 0 && c.pos == dlo(d[0]); }
    __device__ __forceinline__ bool is_last(Cur c) const {
        return c.seg == n - 1 && c.pos == dhi(d[n - 1]);
    }
    __device__ __forceinline__ Cur prev(Cur c) const {
        return c.pos > dlo(d[c.seg]) ? Cur{c.seg, c.pos - 1} : Cur{c.seg - 1, dhi(d[c.seg - 1])};
    }
    __device__ __forceinline__ Cur next(Cur c) const {
        return c.pos < dhi(d[c.seg]) ? Cur{c.seg, c.pos + 1} : Cur{c.seg + 1, dlo(d[c.seg + 1])};
    }
    template <class V>
    __device__ __forceinline__ Pt pt(const V X, Cur c, int jr) const {
        return X.vtx(dchunk(d[c.seg]), c.pos, jr);
    }
};

// First vertex of the list range [X, Y] that satisfies a predicate which is
// false then true along the range and true at Y: bisection over segments (by
// each segment's last in-range vertex), then within one segment.
template <class DT, class F>
__device__ __forceinline__ Cur find_first(const List<DT> Lst, Cur X, Cur Y, F pred) {
    int lo = X.seg, hi = Y.seg;
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        Cur c{mid, mid == Y.seg ? Y.pos : dhi(Lst.d[mid])};
        if (pred(c)) hi = mid;
        else lo = mid + 1;
    }
    int plo = (lo == X.seg) ? X.pos : dlo(Lst.d[lo]);
    int phi = (lo == Y.seg) ? Y.pos : dhi(Lst.d[lo]);
    while (plo < phi) {
        int mid = (plo + phi) >> 1;
        if (pred(Cur{lo, mid})) phi = mid;
        else plo = mid + 1;
    }
    return Cur{lo, plo};
}

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
template <class V, class DT>
__device__ __forceinline__ bool bridge_start(const V X, const List<DT> Lq, const List<DT> Rq,
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
template <class V, class DT>
__device__ __forceinline__ bool walk_thread(const V X, const List<DT> Lq, const List<DT> Rq, int jr, Cur& A,
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
template <class V, class DT>
__device__ __forceinline__ Bridge bisect_bridge(const V X, const List<DT> Lq, const List<DT> Rq, int jr) {
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

__device__ __forceinline__ bool same(Cur a, Cur b) { return a.seg == b.seg && a.pos == b.pos; }

// Debug counter increment (no-op when the counters are off).
__device__ __forceinline__ void dbg_add(unsigned long long* dbg, int k, unsigned long long v = 1) {
    if (dbg && v) atomicAdd(dbg + k, v);
}

// The start of the middle edge of the list range [c0, c1] (c0 before c1):
// within one segment, the middle vertex pair; across segments, the edge from
// the middle segment's last vertex to the next segment's first (an edge of
// the chain, as consecutive vertices of the hull).
template <class DT>
__device__ __forceinline__ Cur mid_edge(const List<DT> Lq, Cur c0, Cur c1) {
    if (c0.seg == c1.seg) return Cur{c0.seg, (c0.pos + c1.pos - 1) >> 1};
    const int sm = (c0.seg + c1.seg - 1) >> 1;
    return Cur{sm, dhi(Lq.d[sm])};
}

// The three-case bridge search (paper appendix A, Lemma A.1, with lower
// hulls): for the non-convex case (the shared point s is not a vertex of the
// merged hull), keep a candidate range on each side ([a0, a1] of L without s,
// [b0, b1] of R without s) and compare the middle edge alpha of L's range with
// the middle edge beta of R's range, through the segment l r joining their
// midpoints:
//   (1) slope(alpha) >= slope(lr): the bridge's left end a* is not right of
//       alpha's left end;
//   (2) slope(lr) >= slope(beta): its right end b* is not left of beta's
//       right end;
//   (3) otherwise the lines of alpha and beta meet at gamma; if x(gamma) <=
//       x(s), a* is not left of alpha's right end; if x(gamma) >= x(s), b* is
//       not right of beta's left end.
// Each case discards a prefix or suffix of one range.  When one range is a
// single vertex, the bridge's other end is the tangent from it (a bisection
// with a turn predicate).  Slopes are compared by cross multiplication (the
// abscissa differences are positive); x(gamma) against x(s) by the sign of
// the difference of the two lines at x(s), scaled by both abscissa spans.
template <class V, class DT>
__device__ __forceinline__ Bridge three_case_bridge(const V X, const List<DT> Lq, const List<DT> Rq, int jr,
                                                    int* steps) {
    const Cur sR = Rq.first();
    const Pt S = Rq.pt(X, sR, jr);
    auto rel = [&](Pt p) { return Pt{p.w - S.w, p.s - S.s}; };
    Cur a0 = Lq.first(), a1 = Lq.prev(Lq.last());
    Cur b0 = Rq.next(sR), b1 = Rq.last();
    int it = 0;
    for (; it < 4 * 64 * 16 && !same(a0, a1) && !same(b0, b1); ++it) {
        const Cur am = mid_edge(Lq, a0, a1), an = Lq.next(am);
        const Cur bm = mid_edge(Rq, b0, b1), bn = Rq.next(bm);
        const Pt A0 = rel(Lq.pt(X, am, jr)), A1 = rel(Lq.pt(X, an, jr));
        const Pt B0 = rel(Rq.pt(X, bm, jr)), B1 = rel(Rq.pt(X, bn, jr));
        const double daw = A1.w - A0.w, das = A1.s - A0.s;
        const double dbw = B1.w - B0.w, dbs = B1.s - B0.s;
        const double lrw = (B0.w + B1.w) - (A0.w + A1.w), lrs = (B0.s + B1.s) - (A0.s + A1.s);
        const bool c1 = mul_rn(das, lrw) >= mul_rn(lrs, daw);  // slope(alpha) >= slope(lr)
        const bool c2 = mul_rn(lrs, dbw) >= mul_rn(dbs, lrw);  // slope(lr) >= slope(beta)
        if (c1) a1 = am;
        if (c2) b0 = bn;
        if (!c1 && !c2) {
            const double ca = mul_rn(A0.s, daw) - mul_rn(das, A0.w);
            const double cb = mul_rn(B0.s, dbw) - mul_rn(dbs, B0.w);
            const double D = mul_rn(ca, dbw) - mul_rn(cb, daw);
            if (D <= 0.0) a0 = an;
            if (D >= 0.0) b1 = bm;
        }
    }
    *steps = it;
    Bridge br;
    if (same(a0, a1)) {
        // a* is a0: b* is where the tangent from it touches R's range (the
        // rightmost point of contact)
        br.A = a0;
        const Pt Pa = Lq.pt(X, a0, jr);
        br.B = find_first(Rq, b0, b1, [&](Cur r) -> bool {
            if (same(r, b1)) return true;
            return cross3(Pa, Rq.pt(X, r, jr), Rq.pt(X, Rq.next(r), jr)) > 0.0;
        });
    } else {
        // b* is b0: a* is where the tangent from it touches L's range (the
        // leftmost point of contact)
        br.B = b0;
        const Pt Pb = Rq.pt(X, b0, jr);
        br.A = find_first(Lq, a0, a1, [&](Cur l) -> bool {
            if (same(l, a1)) return true;
            return cross3(Lq.pt(X, l, jr), Lq.pt(X, Lq.next(l), jr), Pb) <= 0.0;
        });
    }
    return br;
}

// For the 64 lanes of a wave: the vertex `lane` positions before (dir < 0) or
// after (dir > 0) cursor C along the list, or valid = false past its end.
// Every lane of the wave must call it with the same C and dir.
template <class DT>
__device__ __forceinline__ Cur wave_offset(const List<DT> Lq, Cur C, int dir, int lane, bool& valid) {
    const int sj = C.seg + dir * lane;
    int cnt = 0;
    if (sj >= 0 && sj < Lq.n) {
        DT d = Lq.d[sj];
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
    const DT d = Lq.d[seg];
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
template <class V, class DT>
__device__ __forceinline__ bool walk_wave(const V X, const List<DT> Lq, const List<DT> Rq, int jr, Cur& A, Cur& B,
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
template <class DT>
__device__ __forceinline__ void apply_cut(DT* D, int32_t* CNT, int2* MI, int k, int a, int b,
                                          int nR, Bridge br) {
    DT dl = D[a + br.A.seg];
    D[a + br.A.seg] = mkd<DT>(dchunk(dl), dlo(dl), br.A.pos);
    DT dr = D[b + br.B.seg];
    D[b + br.B.seg] = mkd<DT>(dchunk(dr), br.B.pos, dhi(dr));
    MI[k] = make_int2(br.A.seg + 1, br.B.seg);
    CNT[a] = br.A.seg + 1 + (nR - br.B.seg);
}

// Keeps a loaded value alive so the load that warms the cache is not removed.
__device__ __forceinline__ void keep(double v) { asm volatile("" ::"v"(v)); }

// Reconstruction records from the row's root list (paper section 3.4,
// Corollary 4.5): for every chunk, the range of its surviving hull vertices
// and the slopes of the edges into and out of it, or the one edge it lies
// under; and the number of root vertices before it (for block ids).
template <int NT>
__device__ __forceinline__ void write_records(const RowView X, const uint2* D, int nroot, int m, int32_t* vb,
                              ChunkRec* rec, int* ired) {
    const int tid = threadIdx.x;
    int carry = 0;
    for (int t0 = 0; t0 < nroot; t0 += NT) {
        int i = t0 + tid;
        int v = 0;
        if (i < nroot) {
            uint2 d = D[i];
            v = dhi(d) - dlo(d) + 1;
        }
        int tot;
        int x = wg_excl_scan_int<NT>(v, ired, &tot);
        if (i < nroot) vb[i] = carry + x;
        carry += tot;
    }
    __syncthreads();
    for (int j = tid; j < m; j += NT) {
        // first root descriptor whose chunk is >= j
        int lo = 0, hi = nroot - 1;
        while (lo < hi) {
            int mid = (lo + hi) >> 1;
            if (dchunk(D[mid]) >= j) hi = mid;
            else lo = mid + 1;
        }
        const int i = lo;
        const uint2 d = D[i];
        ChunkRec rc;
        rc.pad = 0;
        rc.vb = vb[i];
        if (dchunk(d) == j) {
            rc.lo = dlo(d);
            rc.hi = dhi(d);
            rc.slope_in = 0.0;
            rc.slope_out = 0.0;
            if (i > 0) {
                uint2 p = D[i - 1];
                Pt A = X.vtx(dchunk(p), dhi(p), j), Bv = X.vtx(j, dlo(d), j);
                rc.slope_in = (Bv.s - A.s) / (Bv.w - A.w);
            }
            if (i + 1 < nroot) {
                uint2 q = D[i + 1];
                Pt A = X.vtx(j, dhi(d), j), Bv = X.vtx(dchunk(q), dlo(q), j);
                rc.slope_out = (Bv.s - A.s) / (Bv.w - A.w);
            }
        } else {
            // the chunk lies under one edge, from the last vertex of the
            // previous segment to the first vertex of the next (i >= 1: chunk 0
            // always holds the row's first point)
            uint2 p = D[i - 1];
            Pt A = X.vtx(dchunk(p), dhi(p), j), Bv = X.vtx(dchunk(d), dlo(d), j);
            rc.lo = -1;
            rc.hi = -1;
            rc.slope_in = (Bv.s - A.s) / (Bv.w - A.w);
            rc.slope_out = rc.slope_in;
        }
        rec[j] = rc;
    }
}

// ----------------------------------------------------------------------------
// Compact hull arrays for the merge fast paths (hulls short enough that every
// vertex is in the window records): entry i holds (S, W) relative to a common
// origin and a tag naming the vertex's chunk and its position in that chunk's
// hull.  A node's hull sits at the start of its region and is merged with its
// neighbour's as in the chunk kernel: bridge, then the right array's kept
// entries are moved down behind the left array's kept ones.
// ----------------------------------------------------------------------------
__device__ __forceinline__ int mktag(int j, int pos) { return (j << kTagShift) | pos; }
__device__ __forceinline__ int tchunk(int t) { return t >> kTagShift; }
__device__ __forceinline__ int tpos(int t) { return t & ((1 << kTagShift) - 1); }

struct Arr {
    double* S;
    double* W;
    int32_t* tag;
    __device__ __forceinline__ Pt pt(int i) const { return Pt{W[i], S[i]}; }
};

// Bridge of the neighbouring compact hulls L = entries l0 .. l0+cL-1 and
// R = r0 .. r0+cR-1 (L's last vertex is R's first), found by a team of T lanes
// of one wave (lanes lane0 .. lane0+T-1; x is the lane's place in the team).
// The walk of Lemma 4.2 is kept, but each of its steps tests the next T
// candidates at once and a ballot finds where a lane-by-lane walk would stop.
// Returns (A, B): L keeps entries 0..A, R keeps B..cR-1.  Every lane of the
// wave calls it (the loops are wave-uniform); act marks lanes whose team has a
// merge.
__device__ __forceinline__ int2 team_bridge(const Arr& ar, int l0, int cL, int r0, int cR, int x,
                                            int T, int lane0, bool act) {
    const uint64_t tm = (T == 64) ? ~0ull : (((1ull << T) - 1ull) << lane0);
    int A = cL - 2, B = 1;
    bool run = act;
    if (act) {
        const Pt PA = ar.pt(l0 + A), Ps = ar.pt(r0), PB = ar.pt(r0 + 1);
        if (cross3(PA, Ps, PB) > 0.0) {
            A = cL - 1;  // convex at the shared point: kept once, in L
            run = false;
        }
    }
    for (;;) {
        if (__ballot(run) == 0) break;
        bool moved = false;
        // A moves left while its turn towards B is not strictly left
        {
            const Pt PB = run ? ar.pt(r0 + B) : Pt{0.0, 0.0};
            bool go = run;
            for (;;) {
                if (__ballot(go) == 0) break;
                bool stop = false;
                if (go) {
                    const int c = A - x;
                    stop = c <= 0 || cross3(ar.pt(l0 + c - 1), ar.pt(l0 + c), PB) > 0.0;
                }
                const uint64_t bal = __ballot(go && stop) & tm;
                if (go) {
                    const int xs = bal ? (__ffsll((long long)bal) - 1 - lane0) : T;
                    A -= xs;
                    if (xs > 0) moved = true;
                    if (xs < T) go = false;
                }
            }
        }
        // B moves right likewise
        {
            const Pt PA = run ? ar.pt(l0 + A) : Pt{0.0, 0.0};
            bool go = run;
            for (;;) {
                if (__ballot(go) == 0) break;
                bool stop = false;
                if (go) {
                    const int c = B + x;
                    stop = c >= cR - 1 || cross3(PA, ar.pt(r0 + c), ar.pt(r0 + c + 1)) > 0.0;
                }
                const uint64_t bal = __ballot(go && stop) & tm;
                if (go) {
                    const int xs = bal ? (__ffsll((long long)bal) - 1 - lane0) : T;
                    B += xs;
                    if (xs > 0) moved = true;
                    if (xs < T) go = false;
                }
            }
        }
        if (!moved) run = false;
    }
    return make_int2(A, B);
}

// The team moves R's kept entries r0+B .. r0+cR-1 to l0+A+1 onward.  The
// destination lies below the source, so copying forward T entries at a time,
// each step's reads before its writes, never overwrites an unread entry.
// Every lane of the wave calls it.
__device__ __forceinline__ void team_move(const Arr& ar, int l0, int A, int r0, int B, int cR, int x,
                                          int T, bool act) {
    const int n = act ? cR - B : 0;
    const int dst = l0 + A + 1, src = r0 + B;
    if (T == 64) {
        // one merge per wave: n is the same on every lane
        for (int i0 = 0; i0 < n; i0 += 64) {
            const int i = i0 + x;
            const bool a = i < n;
            double s = 0.0, w = 0.0;
            int t = 0;
            if (a) {
                s = ar.S[src + i];
                w = ar.W[src + i];
                t = ar.tag[src + i];
            }
            wave_sync();
            if (a) {
                ar.S[dst + i] = s;
                ar.W[dst + i] = w;
                ar.tag[dst + i] = t;
            }
            wave_sync();
        }
        return;
    }
    for (int i0 = 0;; i0 += T) {
        const int i = i0 + x;
        const bool a = i < n;
        if (__ballot(a) == 0) break;
        double s = 0.0, w = 0.0;
        int t = 0;
        if (a) {
            s = ar.S[src + i];
            w = ar.W[src + i];
            t = ar.tag[src + i];
        }
        wave_sync();
        if (a) {
            ar.S[dst + i] = s;
            ar.W[dst + i] = w;
            ar.tag[dst + i] = t;
        }
        wave_sync();
    }
}

// The bridge of two neighbouring compact hulls by one wave.  The walk of
// Lemma 4.2 stops at the one pair (A, B) whose line has A's neighbours in L
// and B's neighbours in R on or above it, A's left neighbour and B's right one
// strictly above (the outermost of collinear vertices).  These four local
// conditions single that pair out, so the wave tests the 8 x 8 pairs nearest
// the shared point at once (one per lane), then the 16 x 16 nearest (four per
// lane), and walks only when neither finds exactly one pair.  Every lane of
// the wave calls it.
__device__ __forceinline__ int2 wave_bridge(const Arr& ar, int l0, int cL, int r0, int cR, int lane) {
    // the loads of the shared-point test and of the 8 x 8 test are issued
    // together (addresses clamped into the arrays), so that the common cases
    // cost one round trip to LDS
    const int a8 = cL - 2 - (lane & 7), b8 = 1 + (lane >> 3);
    const int ac = max(a8, 0), bc = min(b8, cR - 1);
    const Pt PA = ar.pt(l0 + cL - 2), Ps = ar.pt(r0), PB = ar.pt(r0 + 1);
    const Pt La = ar.pt(l0 + ac), Ln = ar.pt(l0 + ac + 1), Rb = ar.pt(r0 + bc), Rp = ar.pt(r0 + bc - 1);
    const Pt Lp = ar.pt(l0 + max(ac - 1, 0)), Rn = ar.pt(r0 + min(bc + 1, cR - 1));
    if (cross3(PA, Ps, PB) > 0.0) return make_int2(cL - 1, 1);  // convex at the shared point
    {
        // the 8 x 8 pairs nearest the shared point, one per lane
        bool hit = false;
        if (a8 >= 0 && b8 <= cR - 1) {
            hit = (a8 == 0 || cross3(Lp, La, Rb) > 0.0) && (b8 == cR - 1 || cross3(La, Rb, Rn) > 0.0) &&
                  cross3(La, Ln, Rb) <= 0.0 && cross3(La, Rp, Rb) <= 0.0;
        }
        const uint64_t bal = __ballot(hit);
        if (__popcll(bal) == 1) {
            const int f = __ffsll((long long)bal) - 1;
            return make_int2(cL - 2 - (f & 7), 1 + (f >> 3));
        }
    }
    const int i = lane & 15, b0 = 1 + 4 * (lane >> 4);
    const int a = cL - 2 - i;
    unsigned msk = 0;
    if (a >= 0 && b0 <= cR - 1) {
        const Pt La = ar.pt(l0 + a), Ln = ar.pt(l0 + a + 1);
        const Pt Lp = a > 0 ? ar.pt(l0 + a - 1) : La;
        Pt Rr[6];  // R[b0-1 .. b0+4], clamped to R's last entry
#pragma unroll
        for (int k = 0; k < 6; ++k) Rr[k] = ar.pt(r0 + min(b0 - 1 + k, cR - 1));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int b = b0 + q;
            if (b <= cR - 1) {
                const bool c1 = a == 0 || cross3(Lp, La, Rr[q + 1]) > 0.0;
                const bool c2 = b == cR - 1 || cross3(La, Rr[q + 1], Rr[q + 2]) > 0.0;
                const bool c3 = cross3(La, Ln, Rr[q + 1]) <= 0.0;
                const bool c4 = cross3(La, Rr[q], Rr[q + 1]) <= 0.0;
                if (c1 && c2 && c3 && c4) msk |= 1u << q;
            }
        }
    }
    const uint64_t bal = __ballot(msk != 0);
    if (__popcll(bal) == 1) {
        const int f = __ffsll((long long)bal) - 1;
        const unsigned fm = (unsigned)__shfl((int)msk, f);
        if (__popc(fm) == 1) return make_int2(cL - 2 - (f & 15), 1 + 4 * (f >> 4) + (__ffs((int)fm) - 1));
    }
    return team_bridge(ar, l0, cL, r0, cR, lane, 64, 0, true);
}

// Merges the nodes of a compact-array tree: node k of the first level is
// entries k*E .. k*E+cnt[k]-1; at level l (span 2^l) node a and node a+span
// merge into node a, one wave per merge.  Leaves the root's hull in entries
// 0..cnt[0]-1.  There is no workgroup barrier between levels: node a's merges
// at every level belong to one wave, which records in ver[a] (LDS, zeroed by
// the caller before its last barrier) how many levels node a has been
// through; a merge waits only until its right node has been through every
// level at which that node had a partner (ver[a] also carries node a's vertex
// count, so the waiting wave reads both at once).  A wait is only ever for a
// lower level, so every wait ends.  Nodes 4u .. 4u+3 belong to wave u mod NW, and
// with 16 waves u's two bit pairs swap, so that the few merges of the upper
// levels (u a multiple of 2, 4, 8) land on waves of different SIMDs (wave w
// runs on SIMD w mod 4).
template <int NT>
__device__ __forceinline__ void merge_arrays(const Arr& ar, int32_t* cnt, int32_t* ver, int nn, int E,
                                             uint64_t* sr = nullptr /* phase stamps */) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int u0 = NW == 16 ? (((wid & 3) << 2) | (wid >> 2)) : wid;
    int lv = 0;
    for (int span = 1; span < nn; span <<= 1, ++lv) {
        // this wave's merges of the level: a = 4*u0 + 4*NW*j + r, a multiple of 2*span
        for (int a0 = 4 * u0; a0 < nn; a0 += 4 * NW) {
            for (int r = 0; r < 4; r += 2) {
                const int a = a0 + r, b = a + span;
                if ((a & (2 * span - 1)) != 0 || b >= nn) continue;
                // the last level below this one at which b merged with a partner
                int need = 0;
                for (int l2 = 0, s2 = 1; l2 < lv; ++l2, s2 <<= 1)
                    if (b + s2 < nn) need = l2 + 1;
                // ver[b] holds (levels done << 16) | b's vertex count since its
                // first merge; before that b's count is its initial cnt[b]
                const int cL = cnt[a], c0 = cnt[b];
                int v;
                while (((v = __hip_atomic_load(ver + b, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) >> 16) <
                       need)
                    __builtin_amdgcn_s_sleep(1);
                const int cR = need ? (v & 0xffff) : c0;
                const int2 br = wave_bridge(ar, a * E, cL, b * E, cR, lane);
                team_move(ar, a * E, br.x, b * E, br.y, cR, lane, 64, true);
                if (lane == 0) {
                    const int ca = br.x + 1 + cR - br.y;
                    cnt[a] = ca;
                    __hip_atomic_store(ver + a, ((lv + 1) << 16) | ca, __ATOMIC_RELEASE,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
                }
                wave_sync();  // the wave's next merge reads the count
                if (a == 0 && lv < 8) stamp(sr, 5 + lv);  // node 0 through level lv
            }
        }
    }
    __syncthreads();
}

// ----------------------------------------------------------------------------
// Local-bridge merge of compact hulls.  Nodes 0 .. nn-1 hold the lower hulls
// of consecutive runs of points (node k: entries k*E .. k*E+cnt[k]-1, its
// last vertex being node k+1's first).  Each node keeps the range of its
// vertices between its bridges (common lower tangents) with its two
// neighbours: from the bridge on its left, which touches it last at lc, to
// the bridge on its right, which touches it first at rc.  A node whose range
// is empty, or is one vertex at which the two bridges do not turn strictly
// left, has no vertex on the hull of itself and its neighbours, so none on
// the hull of the union: it is dropped and its neighbours are bridged
// directly.  Once no node is dropped, the ranges joined by the bridges form a
// convex chain (a vertex right of a bridge's last contact lies strictly above
// the bridge's line, one left of its first contact likewise) with every point
// on or above it: the hull of the union.  Where most of every node survives
// (hulls of long runs of points), one round of bridges between neighbours,
// all at once, replaces the levels of a merge tree.
// ----------------------------------------------------------------------------

// The tangent from point p (left of entries base+lo .. base+hi of a hull) to
// those entries: the first k in lo .. hi-1 whose entry lies strictly below
// the chord from p to entry k+1, else hi (the rightmost point of contact).
__device__ __forceinline__ int arr_tangent(const Arr& ar, int base, int lo, int hi, Pt p) {
    while (lo < hi) {
        const int k = (lo + hi) >> 1;
        if (cross3(p, ar.pt(base + k), ar.pt(base + k + 1)) > 0.0) hi = k;
        else lo = k + 1;
    }
    return lo;
}

// The bridge of node L (g entries from lb) and node R (h entries from rb) by
// one thread: a nested bisection over L (the first vertex of L whose
// successor does not lie strictly below the line from it to its tangent point
// on R), each step a bisection over R for the tangent (the paper's nested
// bisection, section 3.3, on arrays).  adj: R follows L directly, so L's last
// entry is R's first; unless the two turn convexly there, the bridge is the
// one of L without its last entry and R without its first, which passes on or
// below the shared point.
// Returns (A, B): L's point of contact (the leftmost on the bridge line) and
// R's (the rightmost); for a convex turn at the shared point, (g - 1, 1).
__device__ __forceinline__ int2 arr_bridge(const Arr& ar, int lb, int g, int rb, int h, bool adj) {
    int a = 0, b = g - 1, rlo = 0;
    if (adj) {
        if (cross3(ar.pt(lb + g - 2), ar.pt(lb + g - 1), ar.pt(rb + 1)) > 0.0) return make_int2(g - 1, 1);
        b = g - 2;
        rlo = 1;
    }
    int tb = -1;  // the tangent from L's entry b, once a step has found it
    while (a < b) {
        const int k = (a + b) >> 1;
        const Pt Pk = ar.pt(lb + k);
        const Pt Pn = ar.pt(lb + k + 1);
        const int t = arr_tangent(ar, rb, rlo, h - 1, Pk);
        if (cross3(Pk, Pn, ar.pt(rb + t)) > 0.0) {
            a = k + 1;
        } else {
            b = k;
            tb = t;
        }
    }
    const int t = tb >= 0 ? tb : arr_tangent(ar, rb, rlo, h - 1, ar.pt(lb + a));
    return make_int2(a, t);
}

// Merges nodes 0 .. nn-1 (E entries apart; MAXE bounds nn*E; nn <= 128) into
// node 0 and sets cnt[0].  lc, rc, nx, pv, dead, ko: nn ints each in LDS.
// Returns the number of rounds that dropped nodes, or -1, with the nodes
// untouched, if nodes are still being dropped after kLocalRounds rounds.
// Every thread of the workgroup calls it after a barrier that published the
// nodes.
constexpr int kLocalRounds = 8;
template <int NT, int E, int MAXE>
__device__ __forceinline__ int merge_local(const Arr& ar, int32_t* cnt, int nn, int32_t* lc, int32_t* rc,
                                            int32_t* nx, int32_t* pv, int32_t* dead, int32_t* ko,
                                            uint64_t* sr = nullptr /* phase stamps */) {
    constexpr int T = 8;  // measured against 1, 2, 4, 16, 32, 64
    const int tid = threadIdx.x, lane = tid & 63;
    // the bridges between neighbours, a team of T lanes each (the walk of
    // Lemma 4.2 testing T candidates a step); a wave without a pair skips it
    {
        const int x = tid & (T - 1);
        for (int g0 = 0; g0 < nn - 1; g0 += NT / T) {
            const int g = g0 + tid / T;
            if (g0 + (tid & ~63) / T < nn - 1) {
                const bool act = g < nn - 1;
                const int cL = act ? cnt[g] : 2, cR = act ? cnt[g + 1] : 2;
                const int2 br = team_bridge(ar, g * E, cL, (g + 1) * E, cR, x, T, lane & ~(T - 1), act);
                if (act && x == 0) {
                    rc[g] = br.x;
                    lc[g + 1] = br.y;
                }
            }
        }
        if (tid < nn) {
            nx[tid] = tid + 1;
            pv[tid] = tid - 1;
            dead[tid] = 0;
        }
        if (tid == 0) {
            lc[0] = 0;
            rc[nn - 1] = cnt[nn - 1] - 1;
        }
    }
    __syncthreads();
    stamp(sr, 5);  // bridges between neighbours found
    int round = 0;
    for (;; ++round) {
        // the first and last nodes keep their end points; any other node is
        // dropped if its range is empty or a vertex without a strict turn
        const int h = tid;
        bool drop = false;
        if (h > 0 && h < nn - 1 && !dead[h]) {
            const int c = lc[h], d = rc[h];
            if (c > d) {
                drop = true;
            } else if (c == d) {
                const int p = pv[h], q = nx[h];
                drop = !(cross3(ar.pt(p * E + rc[p]), ar.pt(h * E + c), ar.pt(q * E + lc[q])) > 0.0);
            }
        }
        if (!__syncthreads_or(drop)) break;
        if (round == kLocalRounds) return -1;  // (the same in every thread)
        if (drop) dead[h] = 1;
        __syncthreads();
        // a node whose next node went bridges to the next one left (the last
        // node is never dropped); it alone writes its rc and that node's lc
        if (h < nn - 1 && !dead[h] && dead[nx[h]]) {
            int q = nx[h];
            while (dead[q]) ++q;
            nx[h] = q;
            pv[q] = h;
            const int2 br = arr_bridge(ar, h * E, cnt[h], q * E, cnt[q], false);
            rc[h] = br.x;
            lc[q] = br.y;
        }
        __syncthreads();
    }
    stamp(sr, 6);  // ranges decided
    if (tid < 64) {
        // ko: kept entries before each node (two nodes a lane)
        const int t0 = 2 * lane, t1 = t0 + 1;
        const int v0 = t0 < nn && !dead[t0] ? rc[t0] - lc[t0] + 1 : 0;
        const int v1 = t1 < nn && !dead[t1] ? rc[t1] - lc[t1] + 1 : 0;
        int x = v0 + v1;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int u = __shfl_up(x, d);
            if (lane >= d) x += u;
        }
        const int ex = x - v0 - v1;
        if (t0 < nn) ko[t0] = ex;
        if (t1 < nn) ko[t1] = ex + v0;
        if (lane == 63) cnt[0] = x;  // no thread reads cnt past the last barrier
    }
    __syncthreads();
    // the kept entries to the front: every one read, then written
    constexpr int KQ = (MAXE + NT - 1) / NT;
    double vs[KQ], vw[KQ];
    int vt[KQ], dst[KQ];
#pragma unroll
    for (int q = 0; q < KQ; ++q) {
        const int e = tid + q * NT;
        dst[q] = -1;
        if (e < nn * E) {
            const int nd = e / E, pos = e - nd * E;
            if (!dead[nd] && pos >= lc[nd] && pos <= rc[nd]) {
                dst[q] = ko[nd] + pos - lc[nd];
                vs[q] = ar.S[e];
                vw[q] = ar.W[e];
                vt[q] = ar.tag[e];
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < KQ; ++q) {
        if (dst[q] >= 0) {
            ar.S[dst[q]] = vs[q];
            ar.W[dst[q]] = vw[q];
            ar.tag[dst[q]] = vt[q];
        }
    }
    __syncthreads();
    stamp(sr, 7);  // kept entries moved
    return round;
}

// Prefix counts over a row's root list D of nroot segments (at most one per
// chunk, in chunk order) for the reconstruction: vb[i] = root vertices before
// segment i (block ids), and fs[j] = segments in chunks before chunk j, which
// is the index of the first segment whose chunk is >= j.  rc (LDS, nroot
// ints) receives the segments' chunks so that fs is a binary search.
// root_fs takes rc as filled (and published by a barrier) by the caller.
template <int NT>
__device__ __forceinline__ void root_fs(int nroot, int m, int32_t* fs, const int32_t* rc) {
    // each thread a run of consecutive chunks: one binary search for the
    // first, then a step per chunk (a chunk holds at most one segment)
    const int kc = (m + NT - 1) / NT;
    const int c0 = min(m, (int)threadIdx.x * kc), c1 = min(m, c0 + kc);
    if (c0 < c1) {
        int lo = 0, hi = nroot;  // first segment whose chunk is >= c0
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (rc[mid] < c0) lo = mid + 1;
            else hi = mid;
        }
        for (int j = c0; j < c1; ++j) {
            while (lo < nroot && rc[lo] < j) ++lo;
            fs[j] = lo;
        }
    }
}

template <int NT>
__device__ __forceinline__ void root_prefixes(const uint2* D, int nroot, int m, int32_t* vb, int32_t* fs,
                                              int* ired, int32_t* rc) {
    const int tid = threadIdx.x;
    // each thread a run of consecutive segments: their chunks, and vb by one
    // workgroup scan of the runs' vertex counts
    const int ks = (nroot + NT - 1) / NT;
    const int i0 = min(nroot, tid * ks), i1 = min(nroot, i0 + ks);
    int loc = 0;
    for (int i = i0; i < i1; ++i) {
        const uint2 d = D[i];
        rc[i] = dchunk(d);
        loc += dhi(d) - dlo(d) + 1;
    }
    int tot;
    int x = wg_excl_scan_int<NT>(loc, ired, &tot);  // its barrier also publishes rc
    for (int i = i0; i < i1; ++i) {
        const uint2 d = D[i];
        vb[i] = x;
        x += dhi(d) - dlo(d) + 1;
    }
    root_fs<NT>(nroot, m, fs, rc);
}

// Bit of a row's root-segment count meaning that the merge stored the slope of
// the root edge into every root segment (rslope).
constexpr int kRootSlopes = 1 << 30;

// The reconstruction record of chunk j (Corollary 4.5) from the root list and
// its prefix counts: the range of the chunk's surviving hull vertices and the
// slopes of the edges into and out of it, or the one edge it lies under.  i is
// the first root segment whose chunk is >= j.  The edge slopes come from
// rslope when the merge stored them, else from the vertices (X).  Every load
// the record may need is issued before any is used.
template <class V>
__device__ __forceinline__ ChunkRec chunk_record(const V X, const uint2* D, int nroot_bits,
                                                 const int32_t* vb, int i, const double* rslope, int j) {
    const bool have = (nroot_bits & kRootSlopes) != 0;
    const int nroot = nroot_bits & ~kRootSlopes;
    const int ic = min(i, nroot - 1);
    const uint2 d = D[ic];
    const uint2 dp = D[max(ic - 1, 0)];
    const uint2 dn = D[min(ic + 1, nroot - 1)];
    const int vbi = vb[ic];
    double r_in = 0.0, r_out = 0.0;
    if (have) {
        r_in = rslope[max(ic, 1)];
        r_out = rslope[min(ic + 1, nroot - 1)];
    }
    auto vslope = [&](uint2 p, uint2 q) {  // the root edge from segment p's end to q's start
        const Pt A = X.vtx(dchunk(p), dhi(p), j), B = X.vtx(dchunk(q), dlo(q), j);
        return (B.s - A.s) / (B.w - A.w);
    };
    ChunkRec rc;
    rc.pad = 0;
    rc.vb = vbi;
    if (i < nroot && dchunk(d) == j) {
        rc.lo = dlo(d);
        rc.hi = dhi(d);
        rc.slope_in = i > 0 ? (have ? r_in : vslope(dp, d)) : 0.0;
        rc.slope_out = i + 1 < nroot ? (have ? r_out : vslope(d, dn)) : 0.0;
    } else {
        // the chunk lies under one edge, from the last vertex of the previous
        // segment to the first vertex of the next (chunk 0 always holds the
        // row's first point, so i >= 1; the last chunk holds its last point,
        // so i < nroot)
        rc.lo = -1;
        rc.hi = -1;
        rc.slope_in = have ? r_in : vslope(dp, d);
        rc.slope_out = rc.slope_in;
    }
    return rc;
}

}  // namespace
}  // namespace iso
