// Backward pass of the fit: the vector-Jacobian product (paper "Merge Hulls
// Without Copying Vertices: GPU Isotonic Regression", section 6, paragraph
// "Gradient").  The fit is constant on its blocks, each block's value the
// weighted mean z of y over it, so for a gradient g with respect to the fit,
// with G and W the sums of g and w over an element's block:
//
//     d/dy_i = w_i G / W ,        d/dw_i = (y_i - z) G / W .
//
// The blocks come from the forward pass's block ids (a block starts at a row's
// first element and wherever the id changes).  Sums are taken over blocks
// without atomics (same paragraph): a workgroup takes a tile of 2048 elements
// of a row; a row that fits in one tile is finished in one kernel (several
// short rows share a tile); a longer row takes three kernels, and the sums of
// blocks that cross tiles come from segmented scans over the tiles' boundary
// sums.  Every sum is f64 (the pages carry pairs of the working type for the
// same purpose); each output is rounded once to the I/O type.  Block ids are
// compared, never used as addresses, so ids that are not the forward's change
// the result but not what memory is touched.
#include "../../include/iso.h"
#include "iso_kernels.hpp"

#include <math.h>

namespace iso {
namespace {

constexpr int kVjpNT = 256;
constexpr int kVjpP = 8;
constexpr int kVjpT = kVjpNT * kVjpP;  // elements of a tile
constexpr int kCarryBlk = 256;  // tiles per workgroup of the carry kernels

// Boundary record of one tile of a long row: where its first and last block
// starts lie and the sums (g, w, w*y) over the stretch before the first start
// (the end of a block begun in an earlier tile) and from the last start on
// (the start of a block that may run into later tiles).
struct VjpRec {
    int32_t has;         // the tile holds a block start
    int32_t first_end;   // position of its first block start (len if none)
    int32_t last_start;  // position of its last block start (0 if none)
    int32_t nan;         // the row is a non-finite row of the fit (ids < 0)
    double head[3];      // sums over [0, first_end)
    double tail[3];      // sums over [last_start, len)
};

// Totals (g, w, w*y) of the blocks holding a tile's first and last elements.
struct VjpTot {
    double F[3];
    double L[3];
};

// A block of kCarryBlk tiles reduced: its forward value over the tails and its
// backward value over the heads (segmented: see phase 2).
struct CarryAgg {
    double fv[3];
    double bv[3];
    int32_t ff, bf;
    int32_t pad[2];
};

struct Sums {
    double a, b, c;  // sum g, sum w, sum w*y
};
__device__ __forceinline__ Sums operator+(Sums x, Sums y) { return Sums{x.a + y.a, x.b + y.b, x.c + y.c}; }

// Segmented inclusive scan over the wave, in lane order (FWD) or reverse lane
// order: a lane's (f, v) becomes the sum of v from the nearest flagged lane at
// or before it (in scan order) up to it, and f whether such a lane exists.
template <bool FWD>
__device__ __forceinline__ void wave_seg_scan(bool& f, Sums& v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int fo = FWD ? __shfl_up((int)f, d) : __shfl_down((int)f, d);
        const double ao = FWD ? __shfl_up(v.a, d) : __shfl_down(v.a, d);
        const double bo = FWD ? __shfl_up(v.b, d) : __shfl_down(v.b, d);
        const double co = FWD ? __shfl_up(v.c, d) : __shfl_down(v.c, d);
        const bool in = FWD ? lane >= d : lane + d < 64;
        if (in) {
            if (!f) v = Sums{v.a + ao, v.b + bo, v.c + co};
            f = f || fo != 0;
        }
    }
}

// The same over the workgroup (NT threads, wave totals through LDS); returns
// the exclusive value (fx, vx) of the calling thread: the sum from the nearest
// flagged thread strictly before it (in scan order) and whether there is one.
template <int NT, bool FWD>
__device__ __forceinline__ void wg_seg_scan_excl(bool f, Sums v, int* sf, Sums* sv, bool& fx, Sums& vx) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    bool fi = f;
    Sums vi = v;
    wave_seg_scan<FWD>(fi, vi);
    const int edge = FWD ? 63 : 0;
    if (lane == edge) {
        sf[wid] = fi ? 1 : 0;
        sv[wid] = vi;
    }
    __syncthreads();
    // carry: the waves before this one in scan order, folded in scan order
    bool cf = false;
    Sums cv{0.0, 0.0, 0.0};
    if (FWD) {
        for (int k = 0; k < wid; ++k) {
            if (sf[k]) { cf = true; cv = sv[k]; }
            else cv = cv + sv[k];
        }
    } else {
        for (int k = NW - 1; k > wid; --k) {
            if (sf[k]) { cf = true; cv = sv[k]; }
            else cv = cv + sv[k];
        }
    }
    // exclusive value: the previous lane's inclusive value (in scan order)
    const int fo = FWD ? __shfl_up((int)fi, 1) : __shfl_down((int)fi, 1);
    const Sums vo{FWD ? __shfl_up(vi.a, 1) : __shfl_down(vi.a, 1),
                  FWD ? __shfl_up(vi.b, 1) : __shfl_down(vi.b, 1),
                  FWD ? __shfl_up(vi.c, 1) : __shfl_down(vi.c, 1)};
    if (lane == (FWD ? 0 : 63)) {  // the wave's first lane in scan order
        fx = cf;
        vx = cv;
    } else if (fo) {
        fx = true;
        vx = vo;
    } else {
        fx = cf;
        vx = cv + vo;
    }
    __syncthreads();  // sf, sv are reused by the next scan
}

// Exclusive and total workgroup sums of one int per thread.
template <int NT>
__device__ __forceinline__ int wg_excl_count(int v, int* red, int& total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(x, d);
        if (lane >= d) x += t;
    }
    if (lane == 63) red[wid] = x;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int k = 0; k < NT / 64; ++k) {
        const int t = red[k];
        if (k < wid) before += t;
        all += t;
    }
    total = all;
    __syncthreads();
    return before + x - v;
}

// P consecutive values at p (vector loads when aligned and whole).
template <typename T, int P>
__device__ __forceinline__ void load_run(const T* __restrict__ p, int avail, T (&v)[P]) {
    constexpr int V = 16 / sizeof(T);
    if (avail >= P && (((uintptr_t)p) & 15u) == 0) {
#pragma unroll
        for (int q = 0; q < P / V; ++q) {
            if constexpr (sizeof(T) == 4) {
                const float4 t = reinterpret_cast<const float4*>(p)[q];
                v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
            } else {
                const double2 t = reinterpret_cast<const double2*>(p)[q];
                v[2 * q] = t.x; v[2 * q + 1] = t.y;
            }
        }
    } else {
#pragma unroll
        for (int b = 0; b < P; ++b) v[b] = b < avail ? p[b] : T(0);
    }
}

template <int P>
__device__ __forceinline__ void load_ids(const int32_t* __restrict__ p, int avail, int (&v)[P]) {
    if (avail >= P && (((uintptr_t)p) & 15u) == 0) {
#pragma unroll
        for (int q = 0; q < P / 4; ++q) {
            const int4 t = reinterpret_cast<const int4*>(p)[q];
            v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
        }
    } else {
#pragma unroll
        for (int b = 0; b < P; ++b) v[b] = b < avail ? p[b] : 0;
    }
}

template <typename T>
__device__ __forceinline__ T nan_of() {
    if constexpr (sizeof(T) == 4) return __builtin_nanf("");
    else return __builtin_nan("");
}

// Phase 1 (and the whole job for rows of at most kVjpT elements).
//   WHOLE: tile b holds rows b*kr .. b*kr+kr-1 whole (kr = kVjpT / n), so no
//          block crosses a tile and every element is written here.
//   else:  tile t of row r holds elements t*kVjpT .. of that row; blocks
//          wholly inside the tile are written here, the blocks holding the
//          tile's first and last elements by k_vjp_edges, and the tile's
//          boundary record goes to rec.
template <typename T, bool WT, bool GW, bool WHOLE>
__global__ __launch_bounds__(kVjpNT) void k_vjp_tiles(const T* __restrict__ g, const T* __restrict__ y,
                                                      const T* __restrict__ w,
                                                      const int32_t* __restrict__ bid, int64_t rows,
                                                      int64_t n, int mt, int kr, T* __restrict__ gy,
                                                      T* __restrict__ gw, VjpRec* __restrict__ rec) {
    constexpr int NT = kVjpNT, P = kVjpP;
    __shared__ double2 tab[kVjpT + 1];  // (G/W, z) of the tile's blocks, by ordinal
    __shared__ int sf[NT / 64], ired[NT / 64];
    __shared__ Sums sv[NT / 64];
    __shared__ Sums s_head, s_tail;
    __shared__ int s_fe, s_ls;
    int64_t base;
    int len, nrow = 0;
    bool first_tile = true;
    if (WHOLE) {
        const int64_t r0 = (int64_t)blockIdx.x * kr;
        nrow = (int)min((int64_t)kr, rows - r0);
        base = r0 * n;
        len = nrow * (int)n;
    } else {
        const int64_t row = blockIdx.x / mt;
        const int t = (int)(blockIdx.x - row * mt);
        base = row * n + (int64_t)t * kVjpT;
        len = (int)min((int64_t)kVjpT, n - (int64_t)t * kVjpT);
        first_tile = t == 0;
    }
    const int L = threadIdx.x, e0 = L * P;
    const int avail = min(P, len - e0);  // may be <= 0 for idle threads

    T gv[P], wv[P], yv[P];
    int bv[P];
    load_run<T, P>(g + base + e0, avail, gv);
    if (WT) load_run<T, P>(w + base + e0, avail, wv);
    if (GW) load_run<T, P>(y + base + e0, avail, yv);
    load_ids<P>(bid + base + e0, avail, bv);
    // block ids just before and just after this thread's run
    const int bprev = (e0 > 0 && e0 <= len) || (!WHOLE && !first_tile && e0 == 0) ? bid[base + e0 - 1] : 0;
    const int bnext = e0 + P < len ? bid[base + e0 + P] : 0;

    // block starts: a row's first element, or a change of id
    uint32_t fm = 0;
    int nx;  // next row start at or after e0 (tile-relative)
    if (WHOLE) nx = (int)(((int64_t)e0 + n - 1) / n * n);
    else nx = first_tile ? 0 : 0x7fffffff;
#pragma unroll
    for (int b = 0; b < P; ++b) {
        const int e = e0 + b;
        if (e < len) {
            bool st = false;
            if (e == nx) {
                st = true;
                nx = WHOLE ? nx + (int)n : 0x7fffffff;
            }
            const int pb = b == 0 ? bprev : bv[b - 1];
            if (st || bv[b] != pb) fm |= 1u << b;
        }
    }
    const bool next_start = e0 + P < len && (e0 + P == nx || bnext != bv[P - 1]);

    // this thread's sums: of the whole run (no start) or from its last start
    Sums run{0.0, 0.0, 0.0};
#pragma unroll
    for (int b = 0; b < P; ++b) {
        if (b < avail) {
            if ((fm >> b) & 1u) run = Sums{0.0, 0.0, 0.0};
            const double ww = WT ? (double)wv[b] : 1.0;
            run = Sums{run.a + (double)gv[b], run.b + ww, GW ? run.c + ww * (double)yv[b] : 0.0};
        }
    }
    bool fx;
    Sums cin;
    wg_seg_scan_excl<NT, true>(fm != 0, run, sf, sv, fx, cin);
    int total;
    const int cnt_ex = wg_excl_count<NT>(__popc(fm), ired, total);

    // walk the run: close each block at its last element (its totals into the
    // table, by ordinal = block starts at or before it in the tile)
    if (!WHOLE && L == 0) {
        s_fe = len;
        s_ls = 0;
    }
    run = cin;  // the open block's sums up to this run (reset at a start)
    int s = cnt_ex;
    __syncthreads();
#pragma unroll
    for (int b = 0; b < P; ++b) {
        if (b < avail) {
            const int e = e0 + b;
            if ((fm >> b) & 1u) {
                if (!WHOLE && s == 0) {  // the tile's first block start
                    s_head = run;
                    s_fe = e;
                }
                if (!WHOLE && s + 1 == total) s_ls = e;  // its last
                run = Sums{0.0, 0.0, 0.0};
                ++s;
            }
            const double ww = WT ? (double)wv[b] : 1.0;
            run = Sums{run.a + (double)gv[b], run.b + ww, GW ? run.c + ww * (double)yv[b] : 0.0};
            const bool last = e + 1 == len;
            const bool ends = last || (b + 1 < P ? ((fm >> (b + 1)) & 1u) != 0 : next_start);
            if (ends) {
                // a long row's blocks holding the tile's first or last element
                // are finished by the edge kernel
                const bool deferred = !WHOLE && (s == 0 || last);
                if (!deferred) tab[s] = make_double2(run.a / run.b, GW ? run.c / run.b : 0.0);
                if (!WHOLE && last) {
                    s_tail = run;
                    if (total == 0) s_head = run;
                }
            }
        }
    }
    __syncthreads();

    // write every element whose block is complete in the tile
    T oy[P], ow[P];
    uint32_t wm = 0;
    s = cnt_ex;
#pragma unroll
    for (int b = 0; b < P; ++b) {
        if (b < avail) {
            if ((fm >> b) & 1u) ++s;
            const bool deferred = !WHOLE && (s == 0 || s == total);
            if (!deferred) {
                wm |= 1u << b;
                const double2 rz = tab[s];
                const double ww = WT ? (double)wv[b] : 1.0;
                const bool bad = bv[b] < 0;
                oy[b] = bad ? nan_of<T>() : (T)(ww * rz.x);
                if (GW) ow[b] = bad ? nan_of<T>() : (T)(((double)yv[b] - rz.y) * rz.x);
            }
        }
    }
    T* py = gy ? gy + base + e0 : nullptr;
    T* pw = GW ? gw + base + e0 : nullptr;
    if (wm == (1u << P) - 1u && (((uintptr_t)py | (uintptr_t)pw) & 15u) == 0) {
        constexpr int V = 16 / sizeof(T);
#pragma unroll
        for (int q = 0; q < P / V; ++q) {
            if constexpr (sizeof(T) == 4) {
                if (py) reinterpret_cast<float4*>(py)[q] = make_float4(oy[4 * q], oy[4 * q + 1], oy[4 * q + 2], oy[4 * q + 3]);
                if (GW) reinterpret_cast<float4*>(pw)[q] = make_float4(ow[4 * q], ow[4 * q + 1], ow[4 * q + 2], ow[4 * q + 3]);
            } else {
                if (py) reinterpret_cast<double2*>(py)[q] = make_double2(oy[2 * q], oy[2 * q + 1]);
                if (GW) reinterpret_cast<double2*>(pw)[q] = make_double2(ow[2 * q], ow[2 * q + 1]);
            }
        }
    } else {
#pragma unroll
        for (int b = 0; b < P; ++b) {
            if ((wm >> b) & 1u) {
                if (py) py[b] = oy[b];
                if (GW) pw[b] = ow[b];
            }
        }
    }
    if (!WHOLE && L == 0) {
        VjpRec r;
        r.has = total > 0;
        r.first_end = s_fe;
        r.last_start = s_ls;
        r.nan = bv[0] < 0;
        r.head[0] = s_head.a; r.head[1] = s_head.b; r.head[2] = s_head.c;
        r.tail[0] = s_tail.a; r.tail[1] = s_tail.b; r.tail[2] = s_tail.c;
        rec[blockIdx.x] = r;
    }
}

// Phase 2: per long row, the totals of the blocks holding each tile's first
// and last elements.  With P_t the part of the block open at tile t's start
// that lies in earlier tiles and Q_t the part of the block open at its end
// that lies in later tiles (segmented scans over the tiles, forward of the
// tails and backward of the heads): F_t = P_t + head_t (+ Q_t when the tile
// holds no start) and L_t = tail_t + Q_t.  The scans run over many
// workgroups: each takes kCarryBlk consecutive tiles; k_vjp_agg reduces its
// tiles to one forward and one backward value, and k_vjp_apply folds the
// values of the blocks before (after) it, then scans its own tiles.  (A
// segmented value (f, v): v is the sum since the nearest tile holding a start,
// in scan order, that tile's own value included; f whether there is one.)

// One tile's boundary record (zero sums, no start, past the row's end).
__device__ __forceinline__ void load_carry_tile(const VjpRec* __restrict__ rec, int t, int mt, bool& f, Sums& tl,
                                                Sums& hd) {
    const VjpRec r = rec[min(t, mt - 1)];
    const bool in = t < mt;
    f = in && r.has != 0;
    tl = in ? Sums{r.tail[0], r.tail[1], r.tail[2]} : Sums{0.0, 0.0, 0.0};
    hd = in ? Sums{r.head[0], r.head[1], r.head[2]} : Sums{0.0, 0.0, 0.0};
}

// The inclusive value of the last thread in scan order, from an exclusive scan.
__device__ __forceinline__ void seg_fold(bool fx, Sums vx, bool f, Sums v, bool& fo, Sums& vo) {
    fo = fx || f;
    vo = f ? v : vx + v;
}

__global__ __launch_bounds__(kCarryBlk) void k_vjp_agg(const VjpRec* __restrict__ rec, int mt, int nb,
                                                       CarryAgg* __restrict__ agg) {
    constexpr int NT = kCarryBlk;
    __shared__ int sf[NT / 64];
    __shared__ Sums sv[NT / 64];
    const int64_t row = blockIdx.x;  // (grid: rows, blocks per row)
    const int t = (int)blockIdx.y * NT + (int)threadIdx.x;
    bool f;
    Sums tl, hd;
    load_carry_tile(rec + row * mt, t, mt, f, tl, hd);
    bool fx;
    Sums vx;
    wg_seg_scan_excl<NT, true>(f, tl, sf, sv, fx, vx);
    CarryAgg* a = agg + row * nb + blockIdx.y;
    if (threadIdx.x == NT - 1) {
        bool fo;
        Sums vo;
        seg_fold(fx, vx, f, tl, fo, vo);
        a->ff = fo ? 1 : 0;
        a->fv[0] = vo.a; a->fv[1] = vo.b; a->fv[2] = vo.c;
    }
    wg_seg_scan_excl<NT, false>(f, hd, sf, sv, fx, vx);
    if (threadIdx.x == 0) {
        bool fo;
        Sums vo;
        seg_fold(fx, vx, f, hd, fo, vo);
        a->bf = fo ? 1 : 0;
        a->bv[0] = vo.a; a->bv[1] = vo.b; a->bv[2] = vo.c;
    }
}

__global__ __launch_bounds__(kCarryBlk) void k_vjp_apply(const VjpRec* __restrict__ rec,
                                                         const CarryAgg* __restrict__ agg, int mt, int nb,
                                                         VjpTot* __restrict__ tot) {
    constexpr int NT = kCarryBlk;
    __shared__ int sf[NT / 64];
    __shared__ Sums sv[NT / 64];
    __shared__ Sums s_in[2];
    const int64_t row = blockIdx.x;  // (grid: rows, blocks per row)
    const int b = (int)blockIdx.y;
    const int t = b * NT + (int)threadIdx.x;
    bool f;
    Sums tl, hd;
    load_carry_tile(rec + row * mt, t, mt, f, tl, hd);
    // the values carried into this block: the blocks before it (forward) and
    // after it (backward), folded in rounds of NT blocks
    const CarryAgg* ar = agg + row * nb;
    Sums pin{0.0, 0.0, 0.0}, qin{0.0, 0.0, 0.0};
    for (int k0 = 0; k0 < b; k0 += NT) {  // blocks k0 .. min(b, k0+NT)-1, in order
        const int k = k0 + (int)threadIdx.x;
        bool af = false;
        Sums av{0.0, 0.0, 0.0};
        if (k < b) {
            af = ar[k].ff != 0;
            av = Sums{ar[k].fv[0], ar[k].fv[1], ar[k].fv[2]};
        }
        bool fx;
        Sums vx;
        wg_seg_scan_excl<NT, true>(af, av, sf, sv, fx, vx);
        if (threadIdx.x == NT - 1) {  // blocks past b add nothing
            bool fo;
            Sums vo;
            seg_fold(fx, vx, af, av, fo, vo);
            s_in[0] = fo ? vo : pin + vo;
        }
        __syncthreads();
        pin = s_in[0];
        __syncthreads();
    }
    for (int k1 = nb - 1; k1 > b; k1 -= NT) {  // blocks max(b+1, k1-NT+1) .. k1, in reverse
        const int k = k1 - (NT - 1) + (int)threadIdx.x;
        bool af = false;
        Sums av{0.0, 0.0, 0.0};
        if (k > b) {
            af = ar[k].bf != 0;
            av = Sums{ar[k].bv[0], ar[k].bv[1], ar[k].bv[2]};
        }
        bool fx;
        Sums vx;
        wg_seg_scan_excl<NT, false>(af, av, sf, sv, fx, vx);
        if (threadIdx.x == 0) {  // blocks at or before b add nothing
            bool fo;
            Sums vo;
            seg_fold(fx, vx, af, av, fo, vo);
            s_in[1] = fo ? vo : qin + vo;
        }
        __syncthreads();
        qin = s_in[1];
        __syncthreads();
    }
    // this block's tiles
    bool fx;
    Sums vx;
    wg_seg_scan_excl<NT, true>(f, tl, sf, sv, fx, vx);
    const Sums P = fx ? vx : pin + vx;
    wg_seg_scan_excl<NT, false>(f, hd, sf, sv, fx, vx);
    const Sums Qv = fx ? vx : qin + vx;
    if (t < mt) {
        const Sums F = f ? P + hd : P + hd + Qv;
        const Sums Lt = tl + Qv;
        VjpTot* o = tot + row * mt + t;
        o->F[0] = F.a; o->F[1] = F.b; o->F[2] = F.c;
        o->L[0] = Lt.a; o->L[1] = Lt.b; o->L[2] = Lt.c;
    }
}

// Phase 3: the elements of the blocks holding each tile's first and last
// elements, from the totals of phase 2.
template <typename T, bool WT, bool GW>
__global__ __launch_bounds__(kVjpNT) void k_vjp_edges(const T* __restrict__ y, const T* __restrict__ w,
                                                      int64_t n, int mt, const VjpRec* __restrict__ rec,
                                                      const VjpTot* __restrict__ tot, T* __restrict__ gy,
                                                      T* __restrict__ gw) {
    const int64_t row = blockIdx.x / mt;
    const int t = (int)(blockIdx.x - row * mt);
    const int64_t base = row * n + (int64_t)t * kVjpT;
    const int len = (int)min((int64_t)kVjpT, n - (int64_t)t * kVjpT);
    const VjpRec r = rec[blockIdx.x];
    const VjpTot q = tot[blockIdx.x];
    const double rF = q.F[0] / q.F[1], zF = GW ? q.F[2] / q.F[1] : 0.0;
    const double rL = q.L[0] / q.L[1], zL = GW ? q.L[2] / q.L[1] : 0.0;
    const int a1 = r.has ? r.first_end : len;  // [0, a1) takes F
    const int b0 = r.has ? r.last_start : len;  // [b0, len) takes L
    const bool bad = r.nan != 0;
    for (int e = threadIdx.x; e < len; e += kVjpNT) {
        if (e >= a1 && e < b0) continue;
        const bool first = e < a1;
        const double rr = first ? rF : rL, zz = first ? zF : zL;
        const int64_t i = base + e;
        const double ww = WT ? (double)w[i] : 1.0;
        if (gy) gy[i] = bad ? nan_of<T>() : (T)(ww * rr);
        if (GW) gw[i] = bad ? nan_of<T>() : (T)(((double)y[i] - zz) * rr);
    }
}

struct VjpPlan {
    bool whole = true;
    int mt = 0;   // tiles per row (long rows)
    int kr = 0;   // rows per tile (short rows)
    int64_t tiles = 0;
    size_t bytes = 0;
    size_t off_tot = 0;
    int nb = 0;           // blocks of kCarryBlk tiles per row (long rows)
    size_t off_agg = 0;
};

bool vjp_plan(int64_t rows, int64_t n, VjpPlan* p) {
    *p = VjpPlan();
    if (rows < 0 || n < 0) return false;
    if (rows == 0 || n == 0) return true;
    if (n > INT64_MAX / 16 / rows) return false;
    if (n <= kVjpT) {
        p->whole = true;
        p->kr = (int)(kVjpT / n);
        p->tiles = (rows + p->kr - 1) / p->kr;
        return p->tiles <= 0x7fffffffLL;
    }
    p->whole = false;
    const int64_t mt = (n + kVjpT - 1) / kVjpT;
    if (mt * rows > 0x7fffffffLL || rows > 0x7fffffffLL) return false;
    p->mt = (int)mt;
    p->tiles = mt * rows;
    const size_t rb = ((size_t)p->tiles * sizeof(VjpRec) + 255) / 256 * 256;
    p->off_tot = rb;
    if ((mt + kCarryBlk - 1) / kCarryBlk > 65535) return false;  // blocks of a row: the grid's y extent
    p->nb = (int)((mt + kCarryBlk - 1) / kCarryBlk);
    const size_t tb = ((size_t)p->tiles * sizeof(VjpTot) + 255) / 256 * 256;
    p->off_agg = rb + tb;
    p->bytes = p->off_agg + (size_t)rows * p->nb * sizeof(CarryAgg);
    return true;
}

template <typename T, bool WT, bool GW>
hipError_t launch_vjp_t(const T* g, const T* y, const T* w, const int32_t* bid, int64_t rows, int64_t n,
                        T* gy, T* gw, const VjpPlan& p, void* ws, hipStream_t st) {
    if (p.whole) {
        hipLaunchKernelGGL((k_vjp_tiles<T, WT, GW, true>), dim3((unsigned)p.tiles), dim3(kVjpNT), 0, st, g,
                           y, w, bid, rows, n, 0, p.kr, gy, gw, (VjpRec*)nullptr);
        return hipGetLastError();
    }
    VjpRec* rec = static_cast<VjpRec*>(ws);
    VjpTot* tot = reinterpret_cast<VjpTot*>(static_cast<char*>(ws) + p.off_tot);
    hipLaunchKernelGGL((k_vjp_tiles<T, WT, GW, false>), dim3((unsigned)p.tiles), dim3(kVjpNT), 0, st, g, y,
                       w, bid, rows, n, p.mt, 0, gy, gw, rec);
    CarryAgg* agg = reinterpret_cast<CarryAgg*>(static_cast<char*>(ws) + p.off_agg);
    const dim3 cg((unsigned)rows, (unsigned)p.nb);
    hipLaunchKernelGGL(k_vjp_agg, cg, dim3(kCarryBlk), 0, st, rec, p.mt, p.nb, agg);
    hipLaunchKernelGGL(k_vjp_apply, cg, dim3(kCarryBlk), 0, st, rec, agg, p.mt, p.nb, tot);
    hipLaunchKernelGGL((k_vjp_edges<T, WT, GW>), dim3((unsigned)p.tiles), dim3(kVjpNT), 0, st, y, w, n,
                       p.mt, rec, tot, gy, gw);
    return hipGetLastError();
}

bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes) {
    if (!a || !b) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bbytes && b0 < a0 + abytes;
}

template <typename T>
int vjp_entry(const T* g, const T* y, const T* w, const int32_t* block_id, int64_t rows, int64_t n, T* grad_y,
              T* grad_w, void* workspace, size_t workspace_bytes, void* stream) {
    if (rows < 0 || n < 0) return ISO_ERR_ARG;
    if (rows == 0 || n == 0) return ISO_OK;
    if (!g || !block_id || (!grad_y && !grad_w)) return ISO_ERR_ARG;
    if (grad_w && (!w || !y)) return ISO_ERR_ARG;
    VjpPlan p;
    if (!vjp_plan(rows, n, &p)) return ISO_ERR_ARG;
    const size_t nb = (size_t)rows * (size_t)n * sizeof(T);
    const size_t ib = (size_t)rows * (size_t)n * sizeof(int32_t);
    const void* ins[4] = {g, y, w, block_id};
    const size_t inb[4] = {nb, nb, nb, ib};
    for (int k = 0; k < 4; ++k)
        if (overlaps(grad_y, nb, ins[k], inb[k]) || overlaps(grad_w, nb, ins[k], inb[k])) return ISO_ERR_ARG;
    if (overlaps(grad_y, nb, grad_w, nb)) return ISO_ERR_ARG;
    if (((uintptr_t)g | (uintptr_t)y | (uintptr_t)w | (uintptr_t)block_id | (uintptr_t)grad_y |
         (uintptr_t)grad_w) & (sizeof(T) - 1))
        return ISO_ERR_ARG;
    if (p.bytes && (!workspace || workspace_bytes < p.bytes)) return ISO_ERR_WORKSPACE;
    if (p.bytes && ((uintptr_t)workspace & 255u)) return ISO_ERR_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (grad_w)
        e = launch_vjp_t<T, true, true>(g, y, w, block_id, rows, n, grad_y, grad_w, p, workspace, st);
    else if (w)
        e = launch_vjp_t<T, true, false>(g, y, w, block_id, rows, n, grad_y, nullptr, p, workspace, st);
    else
        e = launch_vjp_t<T, false, false>(g, y, nullptr, block_id, rows, n, grad_y, nullptr, p, workspace, st);
    return e == hipSuccess ? ISO_OK : ISO_ERR_HIP;
}

}  // namespace
}  // namespace iso

extern "C" {

size_t iso_vjp_workspace_bytes(int64_t rows, int64_t n) {
    iso::VjpPlan p;
    if (!iso::vjp_plan(rows, n, &p)) return 0;
    return p.bytes;
}

int iso_vjp(const float* g, const float* y, const float* w, const int32_t* block_id, int64_t rows,
            int64_t n, float* grad_y, float* grad_w, void* workspace, size_t workspace_bytes, void* stream) {
    return iso::vjp_entry<float>(g, y, w, block_id, rows, n, grad_y, grad_w, workspace, workspace_bytes,
                                 stream);
}

int iso_vjp_f64(const double* g, const double* y, const double* w, const int32_t* block_id, int64_t rows,
                int64_t n, double* grad_y, double* grad_w, void* workspace, size_t workspace_bytes,
                void* stream) {
    return iso::vjp_entry<double>(g, y, w, block_id, rows, n, grad_y, grad_w, workspace, workspace_bytes,
                                  stream);
}

}  // extern "C"
