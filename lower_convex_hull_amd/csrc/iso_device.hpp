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

// z-component of (b - a) x (c - a).  For a, b, c in increasing abscissa, > 0
// means b lies strictly below the chord from a to c (a strict left turn), so b
// is a hull vertex of {a, b, c}; <= 0 means b is on or above the chord and is
// dropped (collinear middle points are not vertices, paper section 2.1).
__device__ __forceinline__ double cross3(Pt a, Pt b, Pt c) {
    return (b.w - a.w) * (c.s - a.s) - (b.s - a.s) * (c.w - a.w);
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

struct RowView {
    const uint16_t* idx;  // full slots (rarely read)
    const double* S;
    const double* W;
    const WinRec* win;    // compact hull ends
    const int32_t* hc;    // hull vertex counts
    const double* stS;    // chunk starts
    const double* stW;
    bool weighted;

    // Vertex `pos` of chunk j's hull in chunk-relative coordinates: from the
    // compact window when it holds it, else from the full slot.
    __device__ __forceinline__ Pt vrel(int j, int pos) const {
        const int h = hc[j];
        int e = pos;
        if (h > 2 * kWinK && pos >= kWinK) e = pos >= h - kWinK ? kWinK + pos - (h - kWinK) : -1;
        Pt p;
        if (e >= 0) {
            const double2 v = win[j].v[e];
            p.s = v.x;
            p.w = v.y;
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
__device__ Cur find_first(const List<DT> Lst, Cur X, Cur Y, F pred) {
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
__device__ void write_records(const RowView X, const uint2* D, int nroot, int m, int32_t* vb,
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

}  // namespace
}  // namespace iso
