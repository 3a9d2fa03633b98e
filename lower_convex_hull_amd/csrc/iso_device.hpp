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

__device__ __forceinline__ int dchunk(uint2 d) { return (int)d.x; }
__device__ __forceinline__ int dlo(uint2 d) { return (int)(d.y & 0xffffu); }
__device__ __forceinline__ int dhi(uint2 d) { return (int)(d.y >> 16); }
__device__ __forceinline__ uint2 mkdesc(int j, int lo, int hi) {
    return make_uint2((uint32_t)j, (uint32_t)lo | ((uint32_t)hi << 16));
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

    // Vertex `pos` of chunk j's hull, in coordinates relative to chunk jr's
    // start: the chunk-start difference first, then the chunk-relative part.
    __device__ __forceinline__ Pt vtx(int j, int pos, int jr) const {
        const int h = hc[j];
        int e = pos;
        if (h > 2 * kWinK && pos >= kWinK) e = pos >= h - kWinK ? kWinK + pos - (h - kWinK) : -1;
        double s, w;
        if (e >= 0) {
            const double2 v = win[j].v[e];
            s = v.x;
            w = v.y;
        } else {
            const size_t o = (size_t)j * (kChunk + 1) + pos;
            s = S[o];
            w = weighted ? W[o] : (double)idx[o];
        }
        Pt p;
        p.s = (stS[j] - stS[jr]) + s;
        if (weighted) p.w = (stW[j] - stW[jr]) + w;
        else p.w = (double)((int64_t)(j - jr) * kChunk) + w;
        return p;
    }
};

struct List {
    uint2* d;
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
    __device__ __forceinline__ Pt pt(const RowView X, Cur c, int jr) const {
        return X.vtx(dchunk(d[c.seg]), c.pos, jr);
    }
};

// First vertex of the list range [X, Y] that satisfies a predicate which is
// false then true along the range and true at Y: bisection over segments (by
// each segment's last in-range vertex), then within one segment.
template <class F>
__device__ Cur find_first(const List Lst, Cur X, Cur Y, F pred) {
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
