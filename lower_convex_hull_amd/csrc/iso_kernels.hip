// gfx950 kernels of the batched weighted isotonic fit.
//
// The fit of a row is the slope sequence of the lower convex hull of its
// cumulative sum diagram P_k = (W_k, S_k) (paper "Merge Hulls Without Copying
// Vertices: GPU Isotonic Regression", section 2.1, equations (2)-(3)).  The
// kernels build that hull in three levels (paper section 3):
//
//   block   - a workgroup's hull of its 4096 points (iso_hull.hpp): top-down
//             quickhull levels over the locally convex points, or, where that
//             would need too many levels or vertices, each thread's monotone
//             chain (its LDS region as the stack) merged pairwise by walks to
//             the bridge with the kept vertices moved down (sections 3.1-3.2);
//   row     - chunk hulls, written once to the workspace, are merged up a tree
//             whose nodes are lists of segments of chunk hulls, at most one
//             per chunk (section 3.3, Definition 4.3, Theorem 4.4;
//             iso_merge.hip);
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
#include "iso_hull.hpp"

namespace iso {
namespace {


// ----------------------------------------------------------------------------
// Short rows: the whole row in one workgroup, fit written directly.
// ----------------------------------------------------------------------------
template <int NT, int P, bool WT, typename T>
__global__ __launch_bounds__(NT) void k_short_rows(const T* __restrict__ y,
                                                   const T* __restrict__ w, int64_t n,
                                                   float sign, T* __restrict__ out,
                                                   int32_t* __restrict__ block_id,
                                                   int32_t* __restrict__ row_flag) {
    __shared__ HullSmem<NT, P, WT, kHullBoth> sm;
    const int64_t row = blockIdx.x;
    const T* gy = y + row * n;
    const T* gw = WT ? w + row * n : nullptr;
    const int len = (int)n;
    const T sg = (T)sign;
    T yv[P];
    double ps[P], pw[P], s0, w0;
    const HullOut ho = block_hull<NT, P, WT, kHullBoth, T>(sm, gy, gw, len, sign, yv, ps, pw, s0, w0);

    const int L = threadIdx.x;
    const int base = L * P;
    const int flag = sm.flag;
    if (L == 0) row_flag[row] = flag;
    T* go = out + row * n;
    int32_t* gb = block_id ? block_id + row * n : nullptr;
    if (flag & kFlagNonfinite) {
        for (int b = 0; b < P; ++b) {
            int e = base + b;
            if (e < len) {
                go[e] = (T)__builtin_nan("");
                if (gb) gb[e] = -1;
            }
        }
        return;
    }
    if (ho.all) {
        // every point a vertex: each element is its own block
#pragma unroll
        for (int b = 0; b < P; ++b) {
            const int e = base + b;
            if (e < len) {
                go[e] = sg * yv[b];
                if (gb) gb[e] = e;
            }
        }
        return;
    }
    // q = the last hull vertex at or before this thread's first element
    const int h = ho.h;
    int lo = 0, hi = h;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((int)sm.idx[mid] <= base) lo = mid + 1;
        else hi = mid;
    }
    int q = lo - 1;
    int qs = -1;
    T slope = T(0);
#pragma unroll
    for (int b = 0; b < P; ++b) {
        const int e = base + b;
        if (e >= len) break;
        while ((int)sm.idx[q + 1] <= e) ++q;  // vertex q <= e < vertex q+1
        const int ka = sm.idx[q], kb = sm.idx[q + 1];
        T val;
        if (ka == e && kb == e + 1) {
            val = yv[b];  // both ends are vertices: the edge is the element itself
        } else {
            if (qs != q) {
                const double dw = WT ? sm.W[q + 1] - sm.W[q] : (double)(min(kb, len) - ka);
                slope = (T)((sm.S[q + 1] - sm.S[q]) / dw);
                qs = q;
            }
            val = slope;
        }
        go[e] = sg * val;
        if (gb) gb[e] = q;
    }
}


template <bool WT, typename T, bool ST>
__global__ __launch_bounds__(kLongNT, WT ? 3 : sizeof(T) == 8 ? 4 : 5) void k_chunk_hulls(
    const T* __restrict__ y, const T* __restrict__ w, int64_t n, int m, float sign, LongWs ws,
    int full_slots) {
    __shared__ HullSmem<kLongNT, kLongP, WT, kHullQuick> sm;
    uint64_t* const sr = ST ? stamp_row(ws.st_chunk, blockIdx.x) : nullptr;
    stamp(sr, 0);
    chunk_hull<kLongNT, kLongP, kHullQuick, WT, T>(y, w, n, m, sign, ws, full_slots, sm, blockIdx.x, sr);
    stamp(sr, 4);  // end
}

// The fallback for rows the first merge stage does not take (rows beyond the
// two-stage merge, and the vertex-copying control): a fixed grid walks the
// chunks and rebuilds the ones the chunk kernel marked in this call.
template <bool WT, typename T>
__global__ __launch_bounds__(kLongNT) void k_chunk_redo(const T* __restrict__ y,
                                                        const T* __restrict__ w, int64_t n,
                                                        int m, float sign, LongWs ws, int full_slots,
                                                        int64_t nchunks) {
    __shared__ HullSmem<kLongNT, kLongP, WT, kHullChains> sm;
    for (int64_t gid = blockIdx.x; gid < nchunks; gid += gridDim.x) {
        if (!(ws.chunk_flag[gid] & kChunkRedo)) continue;  // uniform: one load per workgroup
        chunk_hull<kLongNT, kLongP, kHullChains, WT, T>(y, w, n, m, sign, ws, full_slots, sm, gid);
        if (threadIdx.x == 0) dbg_add(ws.dbg, kDbgRebuilt);
        __syncthreads();
    }
}

// ----------------------------------------------------------------------------
// Long rows, phase 3: every element takes the slope of the row-hull edge above
// it (paper equation (3), section 3.4).
// ----------------------------------------------------------------------------
template <bool WT, typename T, bool ST>
__global__ __launch_bounds__(kExpNT) void k_expand(int64_t n, int m, float sign, LongWs ws,
                                                   T* __restrict__ out,
                                                   int32_t* __restrict__ block_id, int rec_done) {
    constexpr int NT = kExpNT, C = kChunk;
    constexpr int G = C / (4 * NT);  // groups of 4 consecutive elements per thread
    __shared__ int vidx[kExpTile + 1];
    __shared__ T vslope[kExpTile + 1];
    __shared__ double spS[NT], spW[WT ? NT : 1];
    __shared__ int spI[NT];
    __shared__ ChunkRec s_rc;
    __shared__ int s_inc, s_nan;
    const int64_t gid = blockIdx.x;
    const int64_t row = gid / m;
    const int j = (int)(gid - row * m);
    const int64_t off = row * n + (int64_t)j * C;
    const int len = (int)min((int64_t)C, n - (int64_t)j * C);
    const T sg = (T)sign;
    T* go = out + off;
    int32_t* gb = block_id ? block_id + off : nullptr;
    const int tid = threadIdx.x;
    uint64_t* const sr = ST ? stamp_row(ws.st_expand, gid) : nullptr;
    stamp(sr, 0);
    // element groups e = 4 * (g * NT + tid): consecutive threads write
    // consecutive groups of four
    const bool vec = ((((uintptr_t)go) | (uintptr_t)gb) & 15u) == 0;
    auto store4 = [&](int e, const T (&v)[4], const int (&b)[4]) {
        if (vec && e + 4 <= len) {
            // streaming stores: the output is not read again here
            typedef int i4v __attribute__((ext_vector_type(4)));
            if constexpr (sizeof(T) == 4) {
                typedef float f4v __attribute__((ext_vector_type(4)));
                __builtin_nontemporal_store(f4v{v[0], v[1], v[2], v[3]}, reinterpret_cast<f4v*>(go + e));
            } else {
                typedef double d2v __attribute__((ext_vector_type(2)));
                __builtin_nontemporal_store(d2v{v[0], v[1]}, reinterpret_cast<d2v*>(go + e));
                __builtin_nontemporal_store(d2v{v[2], v[3]}, reinterpret_cast<d2v*>(go + e + 2));
            }
            if (gb) __builtin_nontemporal_store(i4v{b[0], b[1], b[2], b[3]}, reinterpret_cast<i4v*>(gb + e));
        } else {
            for (int t = 0; t < 4 && e + t < len; ++t) {
                go[e + t] = v[t];
                if (gb) gb[e + t] = b[t];
            }
        }
    };
    // read while thread 0 forms the record: a strictly increasing chunk's
    // input (its fit is mostly its own elements), else the chunk's first NT
    // slot entries (every hull quickhull builds fits), so that a short
    // surviving range needs no further global read
    const bool incc = (ws.chunk_flag[gid] & kChunkInc) != 0;
    const T* gy = static_cast<const T*>(ws.y) + off;
    const bool vy = vec && (((uintptr_t)gy) & 15u) == 0;
    T ya[G][4];
    if (incc) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int e0 = 4 * (g * NT + tid);
            if (vy && e0 + 4 <= len) {
                if constexpr (sizeof(T) == 4) {
                    typedef float f4v __attribute__((ext_vector_type(4)));
                    const f4v t = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(gy + e0));
                    ya[g][0] = t.x; ya[g][1] = t.y; ya[g][2] = t.z; ya[g][3] = t.w;
                } else {
                    typedef double d2v __attribute__((ext_vector_type(2)));
                    const d2v t0 = __builtin_nontemporal_load(reinterpret_cast<const d2v*>(gy + e0));
                    const d2v t1 = __builtin_nontemporal_load(reinterpret_cast<const d2v*>(gy + e0 + 2));
                    ya[g][0] = t0.x; ya[g][1] = t0.y; ya[g][2] = t1.x; ya[g][3] = t1.y;
                }
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) ya[g][t] = e0 + t < len ? gy[e0 + t] : T(0);
            }
        }
    } else {
        const size_t s0 = (size_t)gid * (C + 1) + tid;
        const int si = ws.slot_idx[s0];
        const double ss = ws.slot_S[s0];
        const double sw = WT ? ws.slot_W[s0] : 0.0;
        spI[tid] = si;
        spS[tid] = ss;
        if (WT) spW[tid] = sw;
    }
    if (tid == 0) {
        // the row's flags, the chunk's flags and its first root segment, read
        // together; then the record
        const int64_t rb = row * m;
        const int rf = ws.row_flag[row];
        const int fsj = rec_done ? 0 : ws.node_cnt[rb + j];
        const int nrb = rec_done ? 0 : ws.root_n[row];
        ChunkRec r{};
        if (rf & kFlagNonfinite) {
            // the row comes out NaN: no record
        } else if (rec_done) {
            r = ws.rec[gid];
        } else {
            // this chunk's record from the row's root list (Corollary 4.5)
            const size_t sl = (size_t)rb * (C + 1);
            const RowView X{ws.slot_idx + sl, ws.slot_S + sl, WT ? ws.slot_W + sl : nullptr, ws.win + rb,
                            ws.hull_cnt + rb, ws.st_S + rb, WT ? ws.st_W + rb : nullptr, WT,
                            inc_src(ws, row, m, 0)};
            r = chunk_record(X, ws.desc_scr + rb, nrb, ws.vb + rb, fsj, ws.rslope + rb, j);
        }
        s_rc = r;
        s_inc = incc;
        s_nan = (rf & kFlagNonfinite) != 0;
    }
    __syncthreads();
    stamp(sr, 1);  // record ready
    if (s_nan) {
        const T nan = (T)__builtin_nan("");
        const T v4[4] = {nan, nan, nan, nan};
        const int b4[4] = {-1, -1, -1, -1};
        for (int g = 0; g < G; ++g) {
            int e = 4 * (g * NT + tid);
            if (e < len) store4(e, v4, b4);
        }
        stamp(sr, 4);
        return;
    }
    const ChunkRec rc = s_rc;
    if (rc.lo < 0) {
        const T v = sg * (T)rc.slope_in;
        const int b = rc.vb - 1;
        const T v4[4] = {v, v, v, v};
        const int b4[4] = {b, b, b, b};
        for (int g = 0; g < G; ++g) {
            int e = 4 * (g * NT + tid);
            if (e < len) store4(e, v4, b4);
        }
        stamp(sr, 4);
        return;
    }
    const int nv = rc.hi - rc.lo + 1;
    if (s_inc) {
        // every point of the chunk is a vertex at its own index: an element
        // between two surviving vertices is its own edge, so its fit is its
        // value (read at the start); elements before or after the surviving
        // range take the edges into and out of it
        const T sin_ = sg * (T)rc.slope_in, sout = sg * (T)rc.slope_out;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int e0 = 4 * (g * NT + tid);
            if (e0 >= len) break;
            T vv[4];
            int bb[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int e = e0 + t;
                vv[t] = e < rc.lo ? sin_ : (e >= rc.hi ? sout : ya[g][t]);
                bb[t] = rc.vb + (e < rc.lo ? 0 : min(e - rc.lo + 1, nv)) - 1;
            }
            store4(e0, vv, bb);
        }
        stamp(sr, 4);
        return;
    }
    const size_t slot = (size_t)gid * (C + 1) + rc.lo;
    const T sin_ = sg * (T)rc.slope_in, sout = sg * (T)rc.slope_out;
    // the slope of edge (v, v+1) of the surviving vertices, from the slot
    auto edge_slope = [&](int v) {
        const double ds = ws.slot_S[slot + v + 1] - ws.slot_S[slot + v];
        const double dw = WT ? ws.slot_W[slot + v + 1] - ws.slot_W[slot + v]
                             : (double)((int)ws.slot_idx[slot + v + 1] - (int)ws.slot_idx[slot + v]);
        return sg * (T)(ds / dw);
    };
    if (nv <= kExpTile) {
        if (rc.hi < NT) {
            // the surviving range lies in the entries read at the start
            if (tid < nv) vidx[tid] = spI[rc.lo + tid];
            if (tid + 1 < nv) {
                const int v = rc.lo + tid;
                const double dw = WT ? spW[v + 1] - spW[v] : (double)(spI[v + 1] - spI[v]);
                vslope[tid] = sg * (T)((spS[v + 1] - spS[v]) / dw);
            }
        } else {
            for (int v = tid; v < nv; v += NT) vidx[v] = ws.slot_idx[slot + v];
            for (int v = tid; v + 1 < nv; v += NT) vslope[v] = edge_slope(v);
        }
        __syncthreads();
        // q = number of the chunk's surviving vertices at or before each
        // group's first element: the groups' searches step together, one LDS
        // round trip per halving
        int qg[G];
#pragma unroll
        for (int g = 0; g < G; ++g) qg[g] = 0;
        for (int stp = 1 << (31 - __clz(nv)); stp > 0; stp >>= 1) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int e0 = 4 * (g * NT + tid);
                if (qg[g] + stp <= nv && vidx[qg[g] + stp - 1] <= e0) qg[g] += stp;
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int e0 = 4 * (g * NT + tid);
            if (e0 >= len) break;
            int q = qg[g];
            T vv[4];
            int bb[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int e = e0 + t;
                while (q < nv && vidx[q] <= e) ++q;
                vv[t] = (q == 0) ? sin_ : (q == nv ? sout : vslope[q - 1]);
                bb[t] = rc.vb + q - 1;
            }
            store4(e0, vv, bb);
        }
    } else {
        // many surviving vertices (a partly dense chunk): search the slot itself
        const uint16_t* vx = ws.slot_idx + slot;
        for (int g = 0; g < G; ++g) {
            const int e0 = 4 * (g * NT + tid);
            if (e0 >= len) break;
            int lo = 0, hi = nv;
            while (lo < hi) {
                int mid = (lo + hi) >> 1;
                if ((int)vx[mid] <= e0) lo = mid + 1;
                else hi = mid;
            }
            int q = lo, qs = -1;
            T sl = T(0);
            T vv[4];
            int bb[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int e = e0 + t;
                while (q < nv && (int)vx[q] <= e) ++q;
                if (q > 0 && q < nv && qs != q) {
                    sl = edge_slope(q - 1);
                    qs = q;
                }
                vv[t] = (q == 0) ? sin_ : (q == nv ? sout : sl);
                bb[t] = rc.vb + q - 1;
            }
            store4(e0, vv, bb);
        }
    }
    stamp(sr, 4);  // end
}

template <int NT, int P, typename T>
hipError_t launch_short_t(const T* y, const T* w, int64_t rows, int64_t n, float sign, T* out,
                          int32_t* block_id, int32_t* row_flag, hipStream_t st) {
    timed_begin(kPhaseShort, st);
    if (w)
        hipLaunchKernelGGL((k_short_rows<NT, P, true, T>), dim3((unsigned)rows), dim3(NT), 0, st, y, w,
                           n, sign, out, block_id, row_flag);
    else
        hipLaunchKernelGGL((k_short_rows<NT, P, false, T>), dim3((unsigned)rows), dim3(NT), 0, st, y,
                           w, n, sign, out, block_id, row_flag);
    timed_end(st);
    return hipGetLastError();
}

// One workgroup ORs every row's data flags into one int (read back by the
// checking path, so that a check copies four bytes whatever the batch).
__global__ __launch_bounds__(1024) void k_flags_or(const int32_t* __restrict__ f, int64_t rows,
                                                   int32_t* __restrict__ dst) {
    __shared__ int red[16];
    int v = 0;
    for (int64_t r = threadIdx.x; r < rows; r += 1024) v |= f[r];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) v |= __shfl_xor(v, d);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        int a = 0;
        for (int k = 0; k < 16; ++k) a |= red[k];
        *dst = a;
    }
}

// A plain streaming copy (16 bytes per lane per step, grid-stride): the
// practical HBM bandwidth ceiling the kernels are compared with.
__global__ __launch_bounds__(256) void k_copy_probe(const float4* __restrict__ src, float4* __restrict__ dst,
                                                    int64_t n16) {
    typedef float f4v __attribute__((ext_vector_type(4)));
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
        const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(src + i));
        __builtin_nontemporal_store(v, reinterpret_cast<f4v*>(dst + i));
    }
}

__global__ void k_zero_u64(unsigned long long* p, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0ull;
}

}  // namespace

hipError_t launch_zero_u64(unsigned long long* p, int n, hipStream_t st) {
    hipLaunchKernelGGL(k_zero_u64, dim3(1), dim3(64), 0, st, p, n);
    return hipGetLastError();
}

hipError_t launch_copy_probe(const void* src, void* dst, size_t bytes, hipStream_t st) {
    const int64_t n16 = (int64_t)(bytes / 16);
    int64_t g = (n16 + 255) / 256;
    if (g > 256 * 64) g = 256 * 64;  // 64 workgroups per CU, grid-stride beyond
    if (g < 1) g = 1;
    hipLaunchKernelGGL(k_copy_probe, dim3((unsigned)g), dim3(256), 0, st, static_cast<const float4*>(src),
                       static_cast<float4*>(dst), n16);
    return hipGetLastError();
}

hipError_t launch_flags_or(const int32_t* row_flag, int64_t rows, int32_t* dst, hipStream_t st) {
    hipLaunchKernelGGL(k_flags_or, dim3(1), dim3(1024), 0, st, row_flag, rows, dst);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_short(const T* y, const T* w, int64_t rows, int64_t n, float sign, T* out,
                        int32_t* block_id, int32_t* row_flag, hipStream_t st) {
    if (n <= 64) return launch_short_t<64, 1>(y, w, rows, n, sign, out, block_id, row_flag, st);
    if (n <= 128) return launch_short_t<64, 2>(y, w, rows, n, sign, out, block_id, row_flag, st);
    if (n <= 256) return launch_short_t<64, 4>(y, w, rows, n, sign, out, block_id, row_flag, st);
    if (n <= 512) return launch_short_t<64, 8>(y, w, rows, n, sign, out, block_id, row_flag, st);
    // a batch too small to fill the GPU with one wave (or four) per row gets
    // four times (twice) as many threads per row, each with fewer points:
    // shorter per-thread loops on the row's latency chain; a large batch keeps
    // the narrower workgroups, which do less work per row
    constexpr int64_t kFillWaves = 8192;  // waves the GPU holds at once (256 CUs x 32)
    if (n <= 1024) {
        if (rows * 4 <= kFillWaves) return launch_short_t<256, 4>(y, w, rows, n, sign, out, block_id, row_flag, st);
        return launch_short_t<64, 16>(y, w, rows, n, sign, out, block_id, row_flag, st);
    }
    if (rows * 8 <= kFillWaves) return launch_short_t<512, 8>(y, w, rows, n, sign, out, block_id, row_flag, st);
    return launch_short_t<256, 16>(y, w, rows, n, sign, out, block_id, row_flag, st);
}

template <typename T>
hipError_t launch_long(const T* y, const T* w, const LongShape& sh, const LongWs& ws0, T* out,
                       int32_t* block_id, bool copy_control, hipStream_t st) {
    const unsigned nblk = (unsigned)(sh.rows * sh.m);
    const bool wt = sh.weighted;
    LongWs ws = ws0;
    ws.y = y;
    ws.w = w;
    ws.n = sh.n;
    ws.sign = sh.sign;
    ws.f64 = sizeof(T) == 8;
    if (ws.dbg) {
        const hipError_t e = launch_zero_u64(ws.dbg, kDbgCount, st);
        if (e != hipSuccess) return e;
    }
    // the copy control reads every chunk hull from its slot
    const int full_slots = copy_control ? 1 : 0;
    // phase stamps (measurement only) come from separate instances of the
    // kernels, so that the others carry no stamp code
    const bool stamps = ws.st_chunk != nullptr && sizeof(T) == 4;
    timed_begin(kPhaseChunk, st);
    if (stamps) {
        if (wt)
            hipLaunchKernelGGL((k_chunk_hulls<true, T, true>), dim3(nblk), dim3(kLongNT), 0, st, y, w, sh.n,
                               sh.m, sh.sign, ws, full_slots);
        else
            hipLaunchKernelGGL((k_chunk_hulls<false, T, true>), dim3(nblk), dim3(kLongNT), 0, st, y, w, sh.n,
                               sh.m, sh.sign, ws, full_slots);
    } else {
        if (wt)
            hipLaunchKernelGGL((k_chunk_hulls<true, T, false>), dim3(nblk), dim3(kLongNT), 0, st, y, w, sh.n,
                               sh.m, sh.sign, ws, full_slots);
        else
            hipLaunchKernelGGL((k_chunk_hulls<false, T, false>), dim3(nblk), dim3(kLongNT), 0, st, y, w, sh.n,
                               sh.m, sh.sign, ws, full_slots);
    }
    timed_end(st);
    // chunks the chunk kernel gave up on are rebuilt by the first merge stage
    // (f32 input), else (f64 input, the copy control) by the fallback kernel
    if (copy_control || sizeof(T) == 8) {
        timed_begin(kPhaseChunkRedo, st);
        const unsigned nredo = nblk < kRedoGrid ? nblk : (unsigned)kRedoGrid;
        if (wt)
            hipLaunchKernelGGL((k_chunk_redo<true, T>), dim3(nredo), dim3(kLongNT), 0, st, y, w, sh.n, sh.m,
                               sh.sign, ws, full_slots, (int64_t)nblk);
        else
            hipLaunchKernelGGL((k_chunk_redo<false, T>), dim3(nredo), dim3(kLongNT), 0, st, y, w, sh.n,
                               sh.m, sh.sign, ws, full_slots, (int64_t)nblk);
        timed_end(st);
    }
    bool rec_done = true;
    hipError_t e = copy_control ? launch_copy_merge(sh, ws, st) : launch_segment_merge(sh, ws, st, &rec_done);
    if (e != hipSuccess) return e;
    timed_begin(kPhaseExpand, st);
    if (stamps) {
        if (wt)
            hipLaunchKernelGGL((k_expand<true, T, true>), dim3(nblk), dim3(kExpNT), 0, st, sh.n, sh.m, sh.sign,
                               ws, out, block_id, (int)rec_done);
        else
            hipLaunchKernelGGL((k_expand<false, T, true>), dim3(nblk), dim3(kExpNT), 0, st, sh.n, sh.m,
                               sh.sign, ws, out, block_id, (int)rec_done);
    } else {
        if (wt)
            hipLaunchKernelGGL((k_expand<true, T, false>), dim3(nblk), dim3(kExpNT), 0, st, sh.n, sh.m,
                               sh.sign, ws, out, block_id, (int)rec_done);
        else
            hipLaunchKernelGGL((k_expand<false, T, false>), dim3(nblk), dim3(kExpNT), 0, st, sh.n, sh.m,
                               sh.sign, ws, out, block_id, (int)rec_done);
    }
    timed_end(st);
    return hipGetLastError();
}

template hipError_t launch_short<float>(const float*, const float*, int64_t, int64_t, float, float*,
                                        int32_t*, int32_t*, hipStream_t);
template hipError_t launch_short<double>(const double*, const double*, int64_t, int64_t, float, double*,
                                         int32_t*, int32_t*, hipStream_t);
template hipError_t launch_long<float>(const float*, const float*, const LongShape&, const LongWs&, float*,
                                       int32_t*, bool, hipStream_t);
template hipError_t launch_long<double>(const double*, const double*, const LongShape&, const LongWs&,
                                        double*, int32_t*, bool, hipStream_t);

}  // namespace iso
