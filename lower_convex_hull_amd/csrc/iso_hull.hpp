// The hull of the points of one workgroup's block of a row, and the chunk
// stage of long rows built on it.  Shared by the fitting kernels
// (iso_kernels.hip) and the first merge stage (iso_merge.hip), which rebuilds
// the chunk hulls the chunk kernel gives up on.  Internal to libiso.so.
#pragma once

#include <math.h>

#include "iso_device.hpp"

namespace iso {
namespace {

// ----------------------------------------------------------------------------
// The hull of one workgroup's points, kept as compact vertex arrays in LDS.
//
// Thread L owns points L*P .. L*P+P (P+1 points; its last point is thread
// L+1's first) and a region of RS = P+1 array entries starting at L*RS.  Its
// thread hull, a monotone chain over its locally convex points (paper section
// 3.1), is built with the region as the stack.  Neighbouring hulls are then
// merged pairwise, level by level (section 3.2): one thread walks the two arrays
// to the bridge (Lemma 4.2), testing four candidates per LDS round trip since
// their positions are known, and the group's threads move the right array's
// kept vertices down behind the left array's kept ones.  A node of level r
// thus holds its hull at the start of its first thread's region, and the
// workgroup's hull ends up at the start of region 0.
// ----------------------------------------------------------------------------
// How a workgroup builds its hull: quickhull, then chains and merges if
// quickhull gives up (short rows); quickhull only, leaving a chunk it gives up
// on for the fallback kernel; or chains and merges only (that fallback).
constexpr int kHullBoth = 0, kHullQuick = 1, kHullChains = 2;

template <int NT, int P, bool WT, int MODE>
struct HullSmem {
    static constexpr int RS = P + 1;
    static constexpr int NR = MODE == kHullQuick ? 1 : NT * RS;  // region entries
    static constexpr int NQ = MODE == kHullChains ? 1 : kQhMax;  // quickhull entries
    double S[NR];                 // block-relative S of each array entry
    double W[WT ? NR : 1];        // block-relative W (weighted; else W is the index)
    uint16_t idx[NR];             // block point index of each entry
    int32_t cnt[MODE == kHullQuick ? 1 : NT];  // entries of the node stored from this region
    int32_t mvk[MODE == kHullQuick ? 1 : NT];  // per merge: kept entries of the left array
    int32_t mvb[MODE == kHullQuick ? 1 : NT];  // per merge: first kept entry of the right array
    double red[NT / 64 + 1];
    int ired[NT / 64 + 1];
    double end_s, end_w;          // S and W of point len (padding points repeat it)
    int flag;
    // quickhull: the points still live after the first level, compacted over
    // the workgroup in point order (S, W when weighted, and the block index;
    // room for CW entries per wave; the region arrays serve where they
    // exist), each wave's count of them, the vertex list
    // (two buffers), and per chord the key of the farthest point below it
    static constexpr int CW = MODE == kHullQuick ? (WT ? kQhWaveCapW : kQhWaveCap) : 64 * RS;
    static constexpr int NC = MODE == kHullQuick ? (NT / 64) * CW : 1;
    double cS[NC];
    double cW[WT ? NC : 1];
    uint16_t ck[NC];
    int32_t wcnt[NT / 64];
    int32_t qk[2][NQ];
    double qS[2][NQ], qW[2][NQ];
    unsigned long long qkey[2][NQ];
    int qn, qcur;
};

// A DPP move of an f64 within the wave (both 32-bit halves): lanes whose
// source lies outside the pattern, or whose row is not in RM, read +0.0.
template <int CTRL, int RM>
__device__ __forceinline__ double dpp_f64(double x) {
    const long long u = __double_as_longlong(x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)u, CTRL, RM, 0xf, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(u >> 32), CTRL, RM, 0xf, true);
    return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

// Inclusive f64 scan over the wave by DPP row shifts and row broadcasts
// (adding +0.0 where a lane has no source leaves its value unchanged).
__device__ __forceinline__ double wave_incl_scan_f64(double x) {
    x += dpp_f64<0x111, 0xf>(x);  // row_shr:1
    x += dpp_f64<0x112, 0xf>(x);  // row_shr:2
    x += dpp_f64<0x114, 0xf>(x);  // row_shr:4
    x += dpp_f64<0x118, 0xf>(x);  // row_shr:8
    x += dpp_f64<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp_f64<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

// Exclusive and inclusive workgroup scans of one f64 value per thread.  A
// lane's exclusive value is the previous lane's inclusive one, moved, and the
// wave totals are added in wave order, so thread L's inclusive value is
// bit-identical to thread L+1's exclusive value.
template <int NT>
__device__ __forceinline__ void wg_scan2(double v, double* red, double& excl, double& incl) {
    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const double x = wave_incl_scan_f64(v);
    const double ex = dpp_f64<0x138, 0xf>(x);  // wave_shr:1 (lane 0 reads +0.0)
    if (lane == 63) red[wid] = x;
    __syncthreads();
    double before = 0.0;
#pragma unroll
    for (int k = 0; k < NT / 64; ++k)
        if (k < wid) before += red[k];
    excl = before + ex;
    incl = before + x;
}

// Result of block_hull: every point 0..len is a vertex (`all`); or the hull's
// h vertices are entries 0..h-1 of the region arrays, or (quickhull-only
// mode) of the quickhull list qk/qS/qW[qcur]; or (quickhull-only mode) the
// block needs the fallback (`fail`).
struct HullOut {
    bool all;
    int h;
    bool fail;
};

// Loads the block's elements (T = float or double), forms the block-relative
// cumulative sums, and builds the block's lower hull.  Returns this thread's
// element values (sign applied, sanitised) in yv and its points' S (and W) in
// ps/pw: ps[b] is point base+b+1.
template <typename T, int P>
__device__ __forceinline__ void load_elems(const T* __restrict__ p, T (&v)[P]) {
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int q = 0; q < P / 4; ++q) {
            const float4 t = reinterpret_cast<const float4*>(p)[q];
            v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
        }
    } else {
#pragma unroll
        for (int q = 0; q < P / 2; ++q) {
            const double2 t = reinterpret_cast<const double2*>(p)[q];
            v[2 * q] = t.x; v[2 * q + 1] = t.y;
        }
    }
}

template <int NT, int P, bool WT, int MODE, typename T>
__device__ __forceinline__ HullOut block_hull(HullSmem<NT, P, WT, MODE>& sm, const T* __restrict__ gy,
                              const T* __restrict__ gw, int len, float sign, T (&yv)[P],
                              double (&ps)[P], double (&pw)[P], double& s0, double& w0,
                              uint64_t* sr = nullptr /* phase stamps */) {
    constexpr int RS = P + 1;
    const int L = threadIdx.x;
    const int base = L * P;
    const T sg = (T)sign;
    T wv[P];
    int bad = 0;
    if (threadIdx.x == 0) sm.flag = 0;
    // a full block (no padding) takes loops without per-element range tests
    const bool full = len == NT * P;

    // ---- load (each thread its P consecutive elements) and check the data
    T yr[P], wr[P];
    const bool whole = base + P <= len;
    if (P % 4 == 0 && whole && ((((uintptr_t)(gy + base)) | (WT ? (uintptr_t)(gw + base) : 0)) & 15u) == 0) {
        load_elems<T, P>(gy + base, yr);
        if (WT) load_elems<T, P>(gw + base, wr);
    } else {
#pragma unroll
        for (int b = 0; b < P; ++b) {
            int e = base + b;
            yr[b] = e < len ? gy[e] : T(0);
            if (WT) wr[b] = e < len ? gw[e] : T(0);
        }
    }
    // the element before this thread's first (for the increasing test)
    T yp = (L > 0 && base <= len) ? gy[base - 1] : T(0);
    if (!isfinite(yp)) yp = T(0);
    yp *= sg;
    if (full) {
#pragma unroll
        for (int b = 0; b < P; ++b) {
            T yy = yr[b];
            T ww = T(1);
            if (WT) ww = wr[b];
            if (!isfinite(yy)) { bad |= kFlagNonfinite; yy = T(0); }
            if (WT && !(ww > T(0) && isfinite(ww))) { bad |= kFlagWeight; ww = T(1); }
            yv[b] = sg * yy;
            wv[b] = ww;
        }
    } else {
#pragma unroll
        for (int b = 0; b < P; ++b) {
            int e = base + b;
            bool in = e < len;
            T yy = yr[b];
            T ww = T(1);
            if (WT) ww = wr[b];
            if (in) {
                if (!isfinite(yy)) { bad |= kFlagNonfinite; yy = T(0); }
                if (WT && !(ww > T(0) && isfinite(ww))) { bad |= kFlagWeight; ww = T(1); }
            } else {
                ww = T(0);
            }
            yv[b] = sg * yy;
            wv[b] = ww;
        }
    }

    // ---- prefix sums (paper section 2.1, equation (2)), in f64
    double ls = 0.0, lw = 0.0;
#pragma unroll
    for (int b = 0; b < P; ++b) {
        if (WT) {
            ls += (double)wv[b] * (double)yv[b];  // exact for f32 inputs (24 + 24 bits)
            lw += (double)wv[b];
            pw[b] = lw;
        } else {
            ls += (double)yv[b];
        }
        ps[b] = ls;
    }
    double xs, xs1, xw = 0.0, xw1 = 0.0;
    wg_scan2<NT>(ls, sm.red, xs, xs1);
    __syncthreads();
    if (WT) {
        wg_scan2<NT>(lw, sm.red, xw, xw1);
        __syncthreads();
    }
    // point base+b+1 for b < P-1 is xs + ps[b]; the thread's last point is the
    // next thread's first
#pragma unroll
    for (int b = 0; b < P - 1; ++b) {
        ps[b] = xs + ps[b];
        if (WT) pw[b] = xw + pw[b];
    }
    ps[P - 1] = xs1;
    if (WT) pw[P - 1] = xw1;
    s0 = xs;
    w0 = WT ? xw : (double)min(base, len);
    // point len: padding points (beyond len) become exact copies of it
    if (full) {
        if (L == NT - 1) {
            sm.end_s = ps[P - 1];
            sm.end_w = WT ? pw[P - 1] : (double)len;
        }
    } else {
#pragma unroll
        for (int b = 0; b < P; ++b) {
            if (base + b + 1 == len) {
                sm.end_s = ps[b];
                sm.end_w = WT ? pw[b] : (double)len;
            }
        }
    }
    if (bad) atomicOr(&sm.flag, bad);

    // ---- is the row strictly increasing here?  Then every point is a vertex
    // (each edge's slope is its element; paper section 2.1).
    bool inc = L == 0 || base >= len || yp < yv[0];
    if (full) {
#pragma unroll
        for (int b = 1; b < P; ++b) inc = inc && yv[b - 1] < yv[b];
    } else {
#pragma unroll
        for (int b = 1; b < P; ++b)
            if (base + b < len) inc = inc && yv[b - 1] < yv[b];
    }
    const bool all = __syncthreads_and(inc) != 0;  // also publishes end_s, end_w
    stamp(sr, 1);  // loads, sums, scan and the increasing test done
    if (!full && base + P > len) {
        const double es = sm.end_s, ew = sm.end_w;
        if (base >= len) { s0 = es; w0 = ew; }
#pragma unroll
        for (int b = 0; b < P; ++b)
            if (base + b + 1 > len) { ps[b] = es; if (WT) pw[b] = ew; }
    }
    if (all) return HullOut{true, len + 1, false};

    // ---- candidates: point k is a vertex only if the slope into it (element
    // k-1) is below the slope out of it (element k).  Points next to a padding
    // element are kept; padding points that are not thread ends are dropped.
    uint32_t cand = 1u | (1u << P);
    if (full) {
#pragma unroll
        for (int k = 1; k < P; ++k)
            if (yv[k - 1] < yv[k]) cand |= 1u << k;
    } else {
#pragma unroll
        for (int k = 1; k < P; ++k) {
            const int pidx = base + k;
            bool c;
            if (pidx > len) c = false;
            else if (pidx < len) c = yv[k - 1] < yv[k];
            else c = true;
            if (c) cand |= 1u << k;
        }
    }

    auto ent = [&](int i) -> Pt {
        Pt p;
        p.s = sm.S[i];
        p.w = WT ? sm.W[i] : (double)min((int)sm.idx[i], len);
        return p;
    };

    // ---- quickhull first: every chord of the current vertex list takes the
    // point farthest below it as a new vertex, and a point on or above its
    // chord is dropped, until no point is left.  Noise-like blocks finish in
    // a few levels with few vertices; a block that needs more levels or more
    // vertices falls back to the chains and merges below.
    if constexpr (MODE != kHullChains) {
        constexpr int CW = HullSmem<NT, P, WT, MODE>::CW;
        double* cS = MODE == kHullQuick ? sm.cS : sm.S;
        double* cW = MODE == kHullQuick ? sm.cW : sm.W;
        uint16_t* cK = MODE == kHullQuick ? sm.ck : sm.idx;
        // the key of a candidate: the positive f64 depth measure with its low
        // 13 bits giving way to the candidate's compact position (the thread's
        // point number in the first level), so that the largest key is the
        // farthest point and, on a tie, the lowest index
        auto mkkey = [](double c, int e) {
            return ((unsigned long long)__double_as_longlong(c) & ~0x1fffull) |
                   (unsigned long long)(0x1fff - e);
        };
        // live points: candidates below point len
        uint32_t alive = 0;
        if (full) {
            alive = (cand >> 1) & ((1u << P) - 1u);
            if (L == NT - 1) alive &= ~(1u << (P - 1));
        } else {
#pragma unroll
            for (int b = 0; b < P; ++b)
                if (((cand >> (b + 1)) & 1u) && base + b + 1 < len) alive |= 1u << b;
        }
        {
            // the thread's last point (base + P) is a candidate for the
            // chains as their shared end; here it is tested like the others,
            // against the next thread's first element (the wave's last lane
            // keeps it)
            const T nxt = __shfl_down(yv[0], 1);
            if ((L & 63) != 63 && base + P < len && !(yv[P - 1] < nxt)) alive &= ~(1u << (P - 1));
        }
        if constexpr (WT && MODE == kHullQuick) {
            // weighted: a vertex also lies strictly below the chord between
            // the points two before and two after it, which drops about a
            // quarter of the candidates and keeps the compact arrays (sized
            // for four workgroups per CU) from overflowing.  Lanes at a
            // wave's ends and points near the block's ends skip the test.
            const int lane = L & 63;
            const double pS2 = __shfl_up(ps[P - 2], 1), pW2 = __shfl_up(pw[P - 2], 1);
            const double nS0 = __shfl_down(ps[0], 1), nW0 = __shfl_down(pw[0], 1);
            const double nS1 = __shfl_down(ps[1], 1), nW1 = __shfl_down(pw[1], 1);
#pragma unroll
            for (int b = 0; b < P; ++b) {
                const int k = base + b + 1;
                bool ok = k - 2 >= 0 && k + 2 <= len && (b >= 1 || lane > 0 || L == 0) &&
                          (b <= P - 3 || lane < 63);
                if (b == 0 && L == 0) ok = false;  // point -1 does not exist
                if (ok && ((alive >> b) & 1u)) {
                    const Pt Pm = b >= 2 ? Pt{pw[b - 2], ps[b - 2]} : (b == 1 ? Pt{w0, s0} : Pt{pW2, pS2});
                    const Pt Pp = b <= P - 3 ? Pt{pw[b + 2], ps[b + 2]}
                                             : (b == P - 2 ? Pt{nW0, nS0} : Pt{nW1, nS1});
                    if (!(cross3(Pm, Pt{pw[b], ps[b]}, Pp) > 0.0)) alive &= ~(1u << b);
                }
            }
        }
        if (L == 0) {
            sm.qk[0][0] = 0;
            sm.qS[0][0] = 0.0;
            sm.qW[0][0] = 0.0;
            sm.qk[0][1] = len;
            sm.qS[0][1] = sm.end_s;
            sm.qW[0][1] = sm.end_w;
            sm.qn = 2;
            sm.qcur = 0;
        }
        if (L < kQhMax) {
            sm.qkey[0][L] = 0ull;
            sm.qkey[1][L] = 0ull;
        }
        // this thread's chord, the one over its reference point (base in the
        // first level, kref after it: vertex ci <= reference < vertex ci+1):
        // its ends A, B and B's index kB, kept in registers from level to
        // level; the list's size nv and buffer cb (the same in every thread);
        // the keys of a level in buffer lv & 1
        int ci = 0, kB = len, nv = 2, cb = 0, state = 0;
        Pt A{0.0, 0.0}, B{sm.end_w, sm.end_s};
        // level 0 has one chord, from point 0 to point len: the thread's own
        // points, from registers, without branches (with A at the origin the
        // depth is cross3(A, P, B) term for term).  It runs before the level
        // loop so that the register copies of the points end here.
        unsigned long long qbest0 = 0ull;
        if (alive) {
#pragma unroll
            for (int b = 0; b < P; ++b) {
                const int k = base + b + 1;
                const double c = mul_rn(WT ? pw[b] : (double)k, B.s) - mul_rn(ps[b], B.w);
                const bool live = ((alive >> b) & 1u) && c > 0.0;
                if (!live) alive &= ~(1u << b);
                const unsigned long long key = live ? mkkey(c, b) : 0ull;
                qbest0 = key > qbest0 ? key : qbest0;
            }
        }
        // the points still live go to the compact arrays in point order; this
        // thread's start e0 there comes from a scan of the live counts over
        // the wave and the counts of the waves before it.  With more live
        // points than the arrays hold nothing is stored and the block falls
        // back.
        int e0, over, wtot;
        {
            const int lane = L & 63, wid = L >> 6;
            const int cnt = __popc(alive);
            int inc = cnt;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int t = __shfl_up(inc, d);
                if (lane >= d) inc += t;
            }
            if (lane == 63) sm.wcnt[wid] = inc;
            __syncthreads();
            int woff = 0;
            wtot = 0;
#pragma unroll
            for (int w = 0; w < NT / 64; ++w) {
                const int c = sm.wcnt[w];
                woff += w < wid ? c : 0;
                wtot += c;
            }
            e0 = woff + inc - cnt;
            over = wtot > (NT / 64) * CW;
            if (!over && alive) {
#pragma unroll
                for (int b = 0; b < P; ++b) {
                    if ((alive >> b) & 1u) {
                        const int e = e0 + __popc(alive & ((1u << b) - 1u));
                        cS[e] = ps[b];
                        if (WT) cW[e] = pw[b];
                        cK[e] = (uint16_t)(base + b + 1);
                    }
                }
            }
            if (qbest0) {
                const int b = (int)(0x1fff - (qbest0 & 0x1fffull));
                qbest0 = (qbest0 & ~0x1fffull) | (unsigned long long)(0x1fff - (e0 + __popc(alive & ((1u << b) - 1u))));
            }
        }
        // from here on a thread works on an even share of the workgroup's
        // live points: entries e_lo .. e_lo + nloc - 1 of the compact arrays
        // (a later level runs as long as its most loaded thread, and live
        // points cluster near the hull), with kref the index just before its
        // first point in place of the thread's own base
        const int per = (wtot + NT - 1) / NT;
        const int lo = min(wtot, L * per);
        const int nloc = min(wtot, lo + per) - lo;
        const int e_lo = lo;
        alive = nloc > 0 && !over ? (1u << nloc) - 1u : 0u;
        __syncthreads();
        const int kref = alive ? (int)cK[e_lo] - 1 : 0;
        for (int lv = 0; lv < kQhLevels; ++lv) {
            unsigned long long* qkey = sm.qkey[lv & 1];
            const int32_t* vk = sm.qk[cb];
            int qi = ci;                        // this thread's last chord
            unsigned long long qbest = qbest0;  // and its best key there
            qbest0 = 0ull;
            if (lv > 0 && alive) {
                // chord i runs from A to B (index nk); the next chords come
                // from the list when this thread's points pass a vertex (a
                // point that became a vertex lies on its chords and drops
                // out).  The chord's differences are formed once per chord,
                // and the next live point's coordinates are read while the
                // current one is tested.
                double bc = 0.0;
                int be = 0;
                int i = ci, nk = kB;
                double Aw = A.w, As = A.s, dW = B.w - A.w, dS = B.s - A.s;
                uint32_t mm = alive;
                int b = lsb32(mm);
                int en = e_lo + b;
                double Sn = cS[en];
                double Wn = WT ? cW[en] : 0.0;
                int kn = cK[en];
                for (;;) {
                    const int k = kn, e = en;
                    const double Sk = Sn, Wk = WT ? Wn : (double)k;
                    mm &= mm - 1u;
                    const int b2 = mm ? lsb32(mm) : b;
                    en = e_lo + b2;
                    Sn = cS[en];
                    if (WT) Wn = cW[en];
                    kn = cK[en];
                    if (k >= nk) {
                        if (bc > 0.0) atomicMax(&qkey[i], mkkey(bc, be));
                        bc = 0.0;
                        be = 0;
                        do {
                            ++i;
                            nk = vk[i + 1];
                        } while (nk <= k);
                        Aw = sm.qW[cb][i];
                        As = sm.qS[cb][i];
                        dW = sm.qW[cb][i + 1] - Aw;
                        dS = sm.qS[cb][i + 1] - As;
                    }
                    const double c = mul_rn(Wk - Aw, dS) - mul_rn(Sk - As, dW);
                    const bool better = c > bc;  // bc >= 0, so a better point is live
                    alive = c > 0.0 ? alive : (alive & ~(1u << b));
                    bc = better ? c : bc;
                    be = better ? e : be;
                    if (!mm) break;
                    b = b2;
                }
                qi = i;
                qbest = bc > 0.0 ? mkkey(bc, be) : 0ull;
            }
            if (qbest) atomicMax(&qkey[qi], qbest);
            if (__syncthreads_or(lv == 0 && over)) {
                state = 2;  // too many live points for the compact arrays
                break;
            }
            // every wave reads the chords' keys: which chords found a point
            // (the same in every wave, so every thread takes the same exit)
            const int lane = L & 63;
            const unsigned long long kl = lane < nv - 1 ? qkey[lane] : 0ull;
            const uint64_t bal = __ballot(kl != 0ull);
            const int add = __popcll(bal);
            if (add == 0) {
                state = 1;  // no point left below any chord: done
                break;
            }
            if (nv + add > kQhMax) {
                state = 2;  // too many vertices: fall back
                break;
            }
            if (L < 64) {
                // wave 0 writes the new list, each chord's point after the
                // chord's start (coordinates from the compact arrays), and
                // clears the other key buffer (last read a level ago)
                const int pre = __popcll(bal & ((1ull << L) - 1ull));
                const int nb = 1 - cb;
                if (L < nv) {
                    sm.qk[nb][L + pre] = vk[L];
                    sm.qS[nb][L + pre] = sm.qS[cb][L];
                    sm.qW[nb][L + pre] = sm.qW[cb][L];
                    if (kl) {
                        const int e = (int)(0x1fff - (kl & 0x1fffull));
                        const int k = cK[e];
                        sm.qk[nb][L + pre + 1] = k;
                        sm.qS[nb][L + pre + 1] = cS[e];
                        sm.qW[nb][L + pre + 1] = WT ? cW[e] : (double)k;
                    }
                }
                sm.qkey[(lv & 1) ^ 1][L] = 0ull;
                if (L == 0) {
                    sm.qn = nv + add;
                    sm.qcur = nb;
                }
            }
            if (alive) {
                // this thread's chord in the new list: the half of the old
                // one that holds point kref
                const unsigned long long kc = qkey[ci];
                const int pre = __popcll(bal & ((1ull << ci) - 1ull));
                if (kc) {
                    const int e = (int)(0x1fff - (kc & 0x1fffull));
                    const int k = cK[e];
                    const Pt K{WT ? cW[e] : (double)k, cS[e]};
                    if (k <= kref) {
                        A = K;
                        ci += pre + 1;
                    } else {
                        B = K;
                        kB = k;
                        ci += pre;
                    }
                } else {
                    ci += pre;
                }
            }
            nv += add;
            cb = 1 - cb;
            __syncthreads();
            if (lv == 0) stamp(sr, 5);  // first quickhull level done
        }
        if (state == 1) {
            // the vertex list, made convex as computed (a near-tie may have
            // picked a point that is not quite the farthest)
            const int cb = sm.qcur, nv = sm.qn;
            if (L < 64) {
                bool ok = true;
                if (L >= 1 && L + 1 < nv)
                    ok = cross3(Pt{sm.qW[cb][L - 1], sm.qS[cb][L - 1]}, Pt{sm.qW[cb][L], sm.qS[cb][L]},
                                Pt{sm.qW[cb][L + 1], sm.qS[cb][L + 1]}) > 0.0;
                if (__ballot(!ok) != 0 && L == 0) {
                    // a monotone chain over the list, into the other buffer
                    const int nb = 1 - cb;
                    int dep = 0;
                    for (int t = 0; t < nv; ++t) {
                        const Pt Cp{sm.qW[cb][t], sm.qS[cb][t]};
                        while (dep >= 2 && cross3(Pt{sm.qW[nb][dep - 2], sm.qS[nb][dep - 2]},
                                                  Pt{sm.qW[nb][dep - 1], sm.qS[nb][dep - 1]}, Cp) <= 0.0)
                            --dep;
                        sm.qS[nb][dep] = Cp.s;
                        sm.qW[nb][dep] = Cp.w;
                        sm.qk[nb][dep] = sm.qk[cb][t];
                        ++dep;
                    }
                    sm.qcur = nb;
                    sm.qn = dep;
                }
            }
            __syncthreads();
            if (MODE == kHullQuick) return HullOut{false, sm.qn, false};
            // into entries 0..h-1 of the region arrays
            const int cq = sm.qcur, h = sm.qn;
            if (L < h) {
                sm.S[L] = sm.qS[cq][L];
                if (WT) sm.W[L] = sm.qW[cq][L];
                sm.idx[L] = (uint16_t)sm.qk[cq][L];
            }
            __syncthreads();
            return HullOut{false, h, false};
        }
        if (MODE == kHullQuick) return HullOut{false, 0, true};
    }

    if constexpr (MODE == kHullQuick) {
        return HullOut{false, 0, true};
    } else {
    // ---- thread hull: monotone chain, the region as its stack; pushes come
    // from registers, a pop reloads the entry under the new top
    const int r0 = L * RS;
    {
        Pt Top{w0, s0}, U{0.0, 0.0};  // the stack's top and the entry under it
        sm.S[r0] = s0;
        if (WT) sm.W[r0] = w0;
        sm.idx[r0] = (uint16_t)base;
        int dep = 1;
#pragma unroll
        for (int b = 1; b <= P; ++b) {
            if (!((cand >> b) & 1u)) continue;
            const Pt Cp{WT ? pw[b - 1] : (double)min(base + b, len), ps[b - 1]};
            while (dep >= 2 && cross3(U, Top, Cp) <= 0.0) {
                --dep;
                Top = U;
                if (dep >= 2) U = ent(r0 + dep - 2);
            }
            sm.S[r0 + dep] = Cp.s;
            if (WT) sm.W[r0 + dep] = Cp.w;
            sm.idx[r0 + dep] = (uint16_t)(base + b);
            ++dep;
            U = Top;
            Top = Cp;
        }
        sm.cnt[L] = dep;
    }
    __syncthreads();

    // ---- merge the hulls pairwise
    constexpr int R = __builtin_ctz(NT);
    for (int r = 0; r < R; ++r) {
        const int g = 2 << r, half = 1 << r;
        if (g > 64) __syncthreads();  // the two halves were built by different waves
        if ((L & (g - 1)) == 0) {
            const int a0 = L * RS, b0 = (L + half) * RS;
            const int cL = sm.cnt[L], cR = sm.cnt[L + half];
            int A = cL - 2, B = 1;
            Pt PA = ent(a0 + A), PB = ent(b0 + 1);
            const Pt Ps = ent(b0);
            if (cross3(PA, Ps, PB) > 0.0) {
                A = cL - 1;  // convex at the shared point: kept once, in L
            } else {
                // A moves left while its turn towards B is not strictly left,
                // B moves right likewise, until neither moves
                for (int pass = 0; pass < 2 * NT * RS; ++pass) {
                    bool moved = false;
                    while (A > 0) {
                        const Pt c1 = ent(a0 + A - 1), c2 = ent(a0 + max(A - 2, 0));
                        const Pt c3 = ent(a0 + max(A - 3, 0)), c4 = ent(a0 + max(A - 4, 0));
                        if (cross3(c1, PA, PB) > 0.0) break;
                        --A; PA = c1; moved = true;
                        if (A == 0 || cross3(c2, PA, PB) > 0.0) break;
                        --A; PA = c2;
                        if (A == 0 || cross3(c3, PA, PB) > 0.0) break;
                        --A; PA = c3;
                        if (A == 0 || cross3(c4, PA, PB) > 0.0) break;
                        --A; PA = c4;
                    }
                    while (B < cR - 1) {
                        const Pt c1 = ent(b0 + B + 1), c2 = ent(b0 + min(B + 2, cR - 1));
                        const Pt c3 = ent(b0 + min(B + 3, cR - 1)), c4 = ent(b0 + min(B + 4, cR - 1));
                        if (cross3(PA, PB, c1) > 0.0) break;
                        ++B; PB = c1; moved = true;
                        if (B == cR - 1 || cross3(PA, PB, c2) > 0.0) break;
                        ++B; PB = c2;
                        if (B == cR - 1 || cross3(PA, PB, c3) > 0.0) break;
                        ++B; PB = c3;
                        if (B == cR - 1 || cross3(PA, PB, c4) > 0.0) break;
                        ++B; PB = c4;
                    }
                    if (!moved) break;
                }
            }
            sm.mvk[L] = A + 1;
            sm.mvb[L] = B;
            sm.cnt[L] = A + 1 + cR - B;
        }
        if (g <= 64) wave_sync();
        else __syncthreads();
        // move the right array's kept entries down behind the left's (the
        // destination always lies below the source, so a forward copy in
        // steps of the group size never overwrites an entry it has yet to read)
        const int Lg = L & ~(g - 1), x = L & (g - 1);
        const int kept = sm.mvk[Lg];
        const int dst = Lg * RS + kept, src = (Lg + half) * RS + sm.mvb[Lg];
        const int n = sm.cnt[Lg] - kept;
        if (g <= 64) {
            for (int i0 = 0;; i0 += g) {
                const int i = i0 + x;
                const bool act = i < n;
                if (__ballot(act) == 0) break;
                double cs = 0.0, cw = 0.0;
                uint16_t ci = 0;
                if (act) {
                    cs = sm.S[src + i];
                    if (WT) cw = sm.W[src + i];
                    ci = sm.idx[src + i];
                }
                wave_sync();
                if (act) {
                    sm.S[dst + i] = cs;
                    if (WT) sm.W[dst + i] = cw;
                    sm.idx[dst + i] = ci;
                }
                wave_sync();
            }
        } else {
            // groups span waves: the same forward copy, a barrier between
            // each step's reads and writes (trip count uniform over the block)
            int nmax = 0;
            for (int q = 0; q < NT; q += g) nmax = max(nmax, sm.cnt[q] - sm.mvk[q]);
            for (int i0 = 0; i0 < nmax; i0 += g) {
                const int i = i0 + x;
                const bool act = i < n;
                double cs = 0.0, cw = 0.0;
                uint16_t ci = 0;
                if (act) {
                    cs = sm.S[src + i];
                    if (WT) cw = sm.W[src + i];
                    ci = sm.idx[src + i];
                }
                __syncthreads();
                if (act) {
                    sm.S[dst + i] = cs;
                    if (WT) sm.W[dst + i] = cw;
                    sm.idx[dst + i] = ci;
                }
            }
            __syncthreads();
        }
    }
    __syncthreads();
    return HullOut{false, sm.cnt[0], false};
    }
}

// ----------------------------------------------------------------------------
// Long rows, phase 1: a workgroup builds one chunk's hull and writes it once
// to the chunk's slot (paper section 3.3), with the chunk's totals.  The chunk
// kernel runs NT = 256 threads of P = 16 points in quickhull mode with little
// LDS and few registers, so that many workgroups share a CU; a chunk it gives
// up on gets the chunk flag kChunkRedo and a window header of h = 0, and is
// rebuilt with chains and merges (MODE kHullChains) by the first merge stage
// (NT = 1024, P = 4; f32 input) or by the fallback kernel.  Every chunk's flag and window
// header are written in every call, so the rebuild depends on no earlier call.
// ----------------------------------------------------------------------------
template <int NT, int P, int MODE, bool WT, typename T>
__device__ __forceinline__ void chunk_hull(const T* __restrict__ y, const T* __restrict__ w,
                                           int64_t n, int m, float sign, const LongWs& ws,
                                           int full_slots, HullSmem<NT, P, WT, MODE>& sm,
                                           int64_t gid /* row * m + chunk */,
                                           uint64_t* sr = nullptr /* phase stamps */) {
    constexpr int C = kChunk;
    static_assert(NT * P == C, "a workgroup covers one chunk");
    const int64_t row = gid / m;
    const int j = (int)(gid - row * m);
    const int64_t off = row * n + (int64_t)j * C;
    const int len = (int)min((int64_t)C, n - (int64_t)j * C);
    T yv[P];
    double ps[P], pw[P], s0, w0;
    const HullOut ho = block_hull<NT, P, WT, MODE, T>(sm, y + off, WT ? w + off : nullptr, len, sign, yv,
                                                   ps, pw, s0, w0, sr);
    stamp(sr, 2);  // hull built
    const int L = threadIdx.x;
    const int base = L * P;
    const int h = ho.h;
    const size_t slot = (size_t)gid * (C + 1);
    WinRec* wr = ws.win + gid;
    // window entry of hull rank r, or -1 if r is in the middle of a long hull
    auto wslot = [&](int r) {
        if (h <= 2 * kWinK || r < kWinK) return r;
        return r >= h - kWinK ? kWinK + r - (h - kWinK) : -1;
    };
    int cflag = sm.flag;
    int hw = h;  // the window header's vertex count (0: rebuilt later)
    if (NT == kLongNT && ho.all && !full_slots) {
        // every point 0..len is a vertex, at its own index: no slot; the
        // window, and each thread's first S (and W) as a checkpoint from which
        // a point is recomputed (with the chunk end as the last checkpoint)
        double* ck = ws.ck_S + (size_t)gid * (NT + 1);
        ck[L] = s0;
        if (L == NT - 1) ck[NT] = ps[P - 1];
        if (WT) {
            double* cw = ws.ck_W + (size_t)gid * (NT + 1);
            cw[L] = w0;
            if (L == NT - 1) cw[NT] = pw[P - 1];
        }
        if (L == 0) wr->v[0] = make_double2(0.0, 0.0);
        if (base + 1 < kWinK || base + P >= h - kWinK || h <= 2 * kWinK) {  // threads with window points
#pragma unroll
            for (int b = 0; b < P; ++b) {
                const int k = base + b + 1;
                const int e = k <= len ? wslot(k) : -1;
                if (e >= 0) wr->v[e] = make_double2(ps[b], WT ? pw[b] : (double)k);
            }
        }
        cflag |= kChunkInc;
    } else if (MODE == kHullQuick && (ho.all || ho.fail)) {
        // a full slot for an increasing chunk (it is staged through the
        // regions), or a hull quickhull gave up on: the second kernel
        cflag |= kChunkRedo;
        hw = 0;
    } else if constexpr (MODE == kHullQuick) {
        // the quickhull vertex list
        const int cq = sm.qcur;
        for (int i = L; i < h; i += NT) {
            const int k = min(sm.qk[cq][i], len);
            const double s = sm.qS[cq][i];
            const double wv = sm.qW[cq][i];
            ws.slot_idx[slot + i] = (uint16_t)k;
            ws.slot_S[slot + i] = s;
            if (WT) ws.slot_W[slot + i] = wv;
            const int e = wslot(i);
            if (e >= 0) wr->v[e] = make_double2(s, wv);
        }
    } else if (ho.all) {
        // every point 0..len is a vertex: stage the points' S (and W) in LDS
        // (point k at k + (k-1)/P, so that threads writing their own points hit
        // different banks), then write the slot with consecutive threads on
        // consecutive vertices
        __syncthreads();
#pragma unroll
        for (int b = 0; b < P; ++b) {
            const int k = base + b + 1;
            sm.S[k + (k - 1) / P] = ps[b];
            if (WT) sm.W[k + (k - 1) / P] = pw[b];
        }
        __syncthreads();
        for (int i = L; i <= len; i += NT) {
            const double s = i == 0 ? 0.0 : sm.S[i + (i - 1) / P];
            const double wv = WT ? (i == 0 ? 0.0 : sm.W[i + (i - 1) / P]) : (double)i;
            ws.slot_idx[slot + i] = (uint16_t)i;
            ws.slot_S[slot + i] = s;
            if (WT) ws.slot_W[slot + i] = wv;
            const int e = wslot(i);
            if (e >= 0) wr->v[e] = make_double2(s, wv);
        }
    } else {
        for (int i = L; i < h; i += NT) {
            const int k = min((int)sm.idx[i], len);
            const double s = sm.S[i];
            const double wv = WT ? sm.W[i] : (double)k;
            ws.slot_idx[slot + i] = (uint16_t)k;
            ws.slot_S[slot + i] = s;
            if (WT) ws.slot_W[slot + i] = wv;
            const int e = wslot(i);
            if (e >= 0) wr->v[e] = make_double2(s, wv);
        }
    }
    if (L == 0) {
        wr->h = hw;
        ws.hull_cnt[gid] = hw;
        ws.tot_S[gid] = sm.end_s;
        if (WT) ws.tot_W[gid] = sm.end_w;
        ws.chunk_flag[gid] = cflag;
    }
}

}  // namespace
}  // namespace iso
