// The vertex-copying merge control (paper "Merge Hulls Without Copying
// Vertices: GPU Isotonic Regression", sections 7.3-7.4, the "grid copy"
// control): the chunk hulls of a long row are merged up the same tree as the
// segment lists, but every merged hull is materialised as a flat array of its
// vertices, rewritten at every level by a whole-GPU, coalesced copy.  It uses
// the same chunk hulls, bridge predicates, reconstruction records and slope
// expansion as the segment-list path, so the two differ only in the merge
// phase, whose bytes and time the benchmarks compare.
#include "iso_kernels.hpp"

#include "iso_device.hpp"

namespace iso {
namespace {

constexpr int kCopyNT = 256;

// One vertex of a flat hull array: chunk-relative S (and W), its chunk, its
// position in the chunk hull and its chunk-relative point index.
template <bool WT>
struct CpV;
template <>
struct CpV<false> {
    double s;
    int32_t chunk;
    uint16_t pos;
    uint16_t idx;
};
template <>
struct CpV<true> {
    double s;
    double w;
    int32_t chunk;
    uint16_t pos;
    uint16_t idx;
};

template <bool WT>
struct FlatView {
    const CpV<WT>* v;
    const double* stS;
    const double* stW;
    __device__ __forceinline__ Pt pt(int i, int jr) const {
        const CpV<WT> x = v[i];
        Pt p;
        p.s = (stS[x.chunk] - stS[jr]) + x.s;
        if constexpr (WT) p.w = (stW[x.chunk] - stW[jr]) + x.w;
        else p.w = (double)((int64_t)(x.chunk - jr) * kChunk + x.idx);
        return p;
    }
};

template <bool WT>
__device__ __forceinline__ CpV<WT>* buf(void* p) {
    return static_cast<CpV<WT>*>(p);
}

// Per row: chunk starts, row flags, and the flat array offsets of the chunk
// hulls (level 0 of the tree).
template <bool WT>
__global__ __launch_bounds__(1024) void k_cp_setup(int m, LongWs ws) {
    constexpr int NT = 1024;
    __shared__ double red[NT / 64 + 1];
    __shared__ int ired[NT / 64 + 1];
    __shared__ int sflag;
    const int64_t row = blockIdx.x, rb = row * m;
    const int tid = threadIdx.x;
    if (tid == 0) sflag = 0;
    __syncthreads();
    int f = 0;
    for (int j = tid; j < m; j += NT) f |= ws.chunk_flag[rb + j] & kFlagData;
    if (f) atomicOr(&sflag, f);
    double cS = 0.0, cW = 0.0;
    int cO = 0;
    for (int t0 = 0; t0 < m; t0 += NT) {
        const int j = t0 + tid;
        double tot;
        double xs = wg_excl_scan<NT>(j < m ? ws.tot_S[rb + j] : 0.0, red, &tot);
        if (j < m) ws.st_S[rb + j] = cS + xs;
        cS += tot;
        if (WT) {
            double xw = wg_excl_scan<NT>(j < m ? ws.tot_W[rb + j] : 0.0, red, &tot);
            if (j < m) ws.st_W[rb + j] = cW + xw;
            cW += tot;
        }
        const int h = j < m ? ws.hull_cnt[rb + j] : 0;
        int itot;
        int xo = wg_excl_scan_int<NT>(h, ired, &itot);
        if (j < m) {
            ws.cp_off[rb + j] = cO + xo;
            ws.cp_cnt[rb + j] = h;
        }
        cO += itot;
    }
    __syncthreads();
    if (tid == 0) ws.row_flag[row] = sflag;
}

// Level 0: every chunk hull copied from its slot into the row's flat array.
template <bool WT>
__global__ __launch_bounds__(kCopyNT) void k_cp_fill(int m, LongWs ws, void* out) {
    const int64_t gid = blockIdx.x, row = gid / m;
    const int j = (int)(gid - row * m);
    const int h = ws.hull_cnt[gid];
    const int o = ws.cp_off[gid];
    CpV<WT>* A = buf<WT>(out) + (size_t)row * m * (kChunk + 1);
    const size_t slot = (size_t)gid * (kChunk + 1);
    for (int p = threadIdx.x; p < h; p += kCopyNT) {
        CpV<WT> x;
        x.s = ws.slot_S[slot + p];
        if constexpr (WT) x.w = ws.slot_W[slot + p];
        x.chunk = j;
        x.pos = (uint16_t)p;
        x.idx = ws.slot_idx[slot + p];
        A[o + p] = x;
    }
}

// One level, bridges: a thread per merge walks (Lemma 4.2) the two flat arrays,
// falling back to the nested bisection (Theorem 5.2) after kWalkCap steps.
// Records how many vertices of L stay and where R starts.
template <bool WT>
__global__ __launch_bounds__(kCopyNT) void k_cp_bridge(int64_t rows, int m, int span, int nm,
                                                       LongWs ws, const void* in) {
    const int64_t t = (int64_t)blockIdx.x * kCopyNT + threadIdx.x;
    const int64_t row = t / nm;
    const int k = (int)(t - row * nm);
    if (row >= rows) return;
    const int64_t rb = row * m;
    const int a = 2 * k * span, b = a + span;
    FlatView<WT> F{buf<WT>(const_cast<void*>(in)) + (size_t)row * m * (kChunk + 1), ws.st_S + rb,
                   WT ? ws.st_W + rb : nullptr};
    const int l0 = ws.cp_off[rb + a], l1 = l0 + ws.cp_cnt[rb + a] - 1;  // l1: the shared point
    const int r0 = ws.cp_off[rb + b], r1 = r0 + ws.cp_cnt[rb + b] - 1;  // r0: the shared point
    const int jr = b;
    int A = l1 - 1, B = r0 + 1;
    Pt PA = F.pt(A, jr), PB = F.pt(B, jr);
    int keepL, startR;
    if (cross3(PA, F.pt(l1, jr), PB) > 0.0) {
        keepL = l1 - l0 + 1;
        startR = 1;
    } else {
        int steps = 0;
        bool done = false;
        for (;;) {
            bool moved = false;
            while (A > l0 && steps < kWalkCap) {
                Pt P2 = F.pt(A - 1, jr);
                if (cross3(P2, PA, PB) <= 0.0) { --A; PA = P2; moved = true; ++steps; }
                else break;
            }
            while (B < r1 && steps < kWalkCap) {
                Pt P2 = F.pt(B + 1, jr);
                if (cross3(PA, PB, P2) <= 0.0) { ++B; PB = P2; moved = true; ++steps; }
                else break;
            }
            if (!moved) { done = true; break; }
            if (steps >= kWalkCap) break;
        }
        if (!done) {
            auto tangent = [&](Pt Pa) {
                int lo = r0 + 1, hi = r1;  // first r with r == r1 or its successor above line (a, r)
                while (lo < hi) {
                    int mid = (lo + hi) >> 1;
                    if (cross3(Pa, F.pt(mid, jr), F.pt(mid + 1, jr)) > 0.0) hi = mid;
                    else lo = mid + 1;
                }
                return lo;
            };
            int lo = l0, hi = l1 - 1;  // first a whose successor is not below a's tangent
            while (lo < hi) {
                int mid = (lo + hi) >> 1;
                Pt Pm = F.pt(mid, jr);
                if (cross3(Pm, F.pt(tangent(Pm), jr), F.pt(mid + 1, jr)) >= 0.0) hi = mid;
                else lo = mid + 1;
            }
            A = lo;
            B = tangent(F.pt(A, jr));
        }
        keepL = A - l0 + 1;
        startR = B - r0;
    }
    ws.cp_cut[rb + a] = keepL;
    ws.cp_cut2[rb + a] = startR;
}

// One level, sizes: each node of the next level (slots multiple of 2 span)
// gets its vertex count and its offset in the other flat array.
__global__ __launch_bounds__(1024) void k_cp_scan(int m, int span, LongWs ws) {
    constexpr int NT = 1024;
    __shared__ int ired[NT / 64 + 1];
    const int64_t row = blockIdx.x, rb = row * m;
    const int nn = (m + 2 * span - 1) / (2 * span);
    int carry = 0;
    for (int t0 = 0; t0 < nn; t0 += NT) {
        const int q = t0 + threadIdx.x;
        int c = 0;
        if (q < nn) {
            const int a = 2 * q * span, b = a + span;
            c = b < m ? ws.cp_cut[rb + a] + ws.cp_cnt[rb + b] - ws.cp_cut2[rb + a] : ws.cp_cnt[rb + a];
        }
        int tot;
        int x = wg_excl_scan_int<NT>(c, ired, &tot);
        if (q < nn) {
            ws.cp_off2[rb + 2 * q * span] = carry + x;
            ws.cp_cnt2[rb + 2 * q * span] = c;
        }
        carry += tot;
    }
}

// One level, the copy: a thread per vertex of the row's flat array writes the
// vertex to its place in the other array if it survives the level's merge.
template <bool WT>
__global__ __launch_bounds__(kCopyNT) void k_cp_move(int m, int span, int blocks_per_row, LongWs ws,
                                                     const void* in, void* out) {
    const int64_t row = blockIdx.x / blocks_per_row;
    const int i = (int)((blockIdx.x - row * blocks_per_row) * kCopyNT + threadIdx.x);
    const int64_t rb = row * m;
    const int nn = (m + span - 1) / span;  // nodes at this level
    const int last = (nn - 1) * span;
    if (i >= ws.cp_off[rb + last] + ws.cp_cnt[rb + last]) return;
    // node containing i: last node t with off[t * span] <= i
    int lo = 0, hi = nn - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (ws.cp_off[rb + mid * span] <= i) lo = mid;
        else hi = mid - 1;
    }
    const int node = lo * span;
    const int local = i - ws.cp_off[rb + node];
    int dest = -1;
    if ((lo & 1) == 0) {
        const int parent = node;
        if (node + span < m) {
            if (local < ws.cp_cut[rb + parent]) dest = ws.cp_off2[rb + parent] + local;
        } else {
            dest = ws.cp_off2[rb + parent] + local;
        }
    } else {
        const int parent = node - span;
        const int sR = ws.cp_cut2[rb + parent];
        if (local >= sR) dest = ws.cp_off2[rb + parent] + ws.cp_cut[rb + parent] + (local - sR);
    }
    if (dest >= 0) {
        const size_t base = (size_t)row * m * (kChunk + 1);
        buf<WT>(out)[base + dest] = buf<WT>(const_cast<void*>(in))[base + i];
    }
}

// Reconstruction records from the root's flat array (paper section 3.4,
// Corollary 4.5), a thread per chunk: the root vertices of chunk j are a
// contiguous run of the array (sorted by chunk, then position), found by
// binary search; the edges into and out of the run, or the edge over an empty
// chunk, join neighbouring array entries.
template <bool WT>
__global__ __launch_bounds__(kCopyNT) void k_cp_records(int m, int bpr, LongWs ws, const void* in) {
    const int64_t row = blockIdx.x / bpr;
    const int j = (int)((blockIdx.x - row * bpr) * kCopyNT + threadIdx.x);
    if (j >= m) return;
    const int64_t rb = row * m;
    const CpV<WT>* V = buf<WT>(const_cast<void*>(in)) + (size_t)row * m * (kChunk + 1) + ws.cp_off[rb];
    const int cnt = ws.cp_cnt[rb];
    FlatView<WT> F{V, ws.st_S + rb, WT ? ws.st_W + rb : nullptr};
    auto lower = [&](int key) {  // first index whose chunk is >= key
        int lo = 0, hi = cnt;
        while (lo < hi) {
            int mid = (lo + hi) >> 1;
            if (V[mid].chunk >= key) hi = mid;
            else lo = mid + 1;
        }
        return lo;
    };
    const int i0 = lower(j), i1 = lower(j + 1);
    auto slope = [&](int a, int b) {
        Pt A = F.pt(a, j), B = F.pt(b, j);
        return (B.s - A.s) / (B.w - A.w);
    };
    ChunkRec rc;
    rc.pad = 0;
    rc.vb = i0;
    if (i0 < i1) {
        rc.lo = V[i0].pos;
        rc.hi = V[i1 - 1].pos;
        rc.slope_in = i0 > 0 ? slope(i0 - 1, i0) : 0.0;
        rc.slope_out = i1 < cnt ? slope(i1 - 1, i1) : 0.0;
    } else {
        rc.lo = -1;
        rc.hi = -1;
        rc.slope_in = slope(i0 - 1, i0);  // chunk 0 and the last chunk are never empty
        rc.slope_out = rc.slope_in;
    }
    ws.rec[rb + j] = rc;
}

template <bool WT>
hipError_t copy_merge_t(const LongShape& sh, const LongWs& ws, hipStream_t st) {
    const int m = sh.m;
    const unsigned R = (unsigned)sh.rows;
    timed_begin(kPhaseMerge, st);
    hipLaunchKernelGGL(k_cp_setup<WT>, dim3(R), dim3(1024), 0, st, m, ws);
    hipLaunchKernelGGL(k_cp_fill<WT>, dim3((unsigned)(sh.rows * m)), dim3(kCopyNT), 0, st, m, ws,
                       (void*)ws.cp_a);
    timed_end(st);
    void* in = ws.cp_a;
    void* out = ws.cp_b;
    LongWs w = ws;
    const int bpr = (int)(((int64_t)m * (kChunk + 1) + kCopyNT - 1) / kCopyNT);
    for (int span = 1; span < m; span <<= 1) {
        const int nm = (m - span + 2 * span - 1) / (2 * span);
        const int64_t nthreads = sh.rows * (int64_t)nm;
        timed_begin(kPhaseCopyBridge, st);
        hipLaunchKernelGGL(k_cp_bridge<WT>, dim3((unsigned)((nthreads + kCopyNT - 1) / kCopyNT)),
                           dim3(kCopyNT), 0, st, sh.rows, m, span, nm, w, (const void*)in);
        hipLaunchKernelGGL(k_cp_scan, dim3(R), dim3(1024), 0, st, m, span, w);
        timed_end(st);
        timed_begin(kPhaseCopyMove, st);
        hipLaunchKernelGGL(k_cp_move<WT>, dim3((unsigned)(R * (int64_t)bpr)), dim3(kCopyNT), 0, st,
                           m, span, bpr, w, (const void*)in, out);
        timed_end(st);
        // the next level reads the new offsets and counts
        int32_t* t;
        t = w.cp_off; w.cp_off = w.cp_off2; w.cp_off2 = t;
        t = w.cp_cnt; w.cp_cnt = w.cp_cnt2; w.cp_cnt2 = t;
        void* tv = in; in = out; out = tv;
    }
    timed_begin(kPhaseMerge, st);
    const int rbpr = (m + kCopyNT - 1) / kCopyNT;
    hipLaunchKernelGGL(k_cp_records<WT>, dim3((unsigned)(R * (int64_t)rbpr)), dim3(kCopyNT), 0, st, m,
                       rbpr, w, (const void*)in);
    timed_end(st);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_copy_merge(const LongShape& sh, const LongWs& ws, hipStream_t st) {
    return sh.weighted ? copy_merge_t<true>(sh, ws, st) : copy_merge_t<false>(sh, ws, st);
}

}  // namespace iso
