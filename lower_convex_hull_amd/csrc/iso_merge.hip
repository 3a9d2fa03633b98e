// The merge phase of long rows: chunk hulls merged up a tree whose nodes are
// lists of segments of chunk hulls, at most one per chunk (paper "Merge Hulls
// Without Copying Vertices: GPU Isotonic Regression", section 3.3, Algorithm 1,
// Definition 4.3, Theorem 4.4), then the per-chunk reconstruction records
// (section 3.4, Corollary 4.5).
#include "iso_kernels.hpp"

#include <mutex>

#include "iso_device.hpp"
#include "iso_hull.hpp"

namespace iso {
namespace {

// ----------------------------------------------------------------------------
// Two-stage merge.  Stage 1: one workgroup per group of kGroup consecutive
// chunks merges their hulls (the tree's lower levels) with the chunk windows,
// lists and starts in LDS.  Stage 2: one workgroup per row merges the group
// hulls (the upper levels) with the group windows in LDS; a vertex outside a
// group window is found through the group's segment list.  Every walk step
// then reads LDS instead of a chain of cache misses.  Where every group hull
// fits its window, stage 2 bridges all neighbouring groups at once instead of
// running the upper levels (merge_local: each group keeps the vertices
// between its two bridges, and groups that keep none are dropped).
// ----------------------------------------------------------------------------

// Schedule, debug counters and tree level of one segment-list merge level.
struct MergeCtl {
    int sched;                 // kSched* bits
    unsigned long long* dbg;   // debug counters, or null
    int r;                     // tree level: the merged nodes span 2^(r+1) chunks
};

// Runs one level of merges of the lists stored in D (slots a, a + span, ...):
// a thread per merge when there are more merges than waves, handing walks that
// run long to the waves; a wave per merge otherwise (or always, with
// kSchedWaveAll).  With kSchedThreeCase the thread-per-merge walks are capped
// at 8 (r + log2 C) steps and finished by the three-case search.  Then moves
// each right list's kept descriptors down behind its left list's.  With debug
// counters, checks every merged list: at most one segment per chunk (node) of
// its range, in strictly increasing order, each with lo <= hi (Definition 4.3,
// Theorem 4.4).
// The level's merges are k = 0 .. nm-1 (nm = merges_at(m, span)); this
// workgroup runs merges kb .. ke-1 (all of them, or its share when a level is
// spread over several workgroups: merges touch disjoint ranges of D).
__host__ __device__ inline int merges_at(int m, int span) { return (m - span + 2 * span - 1) / (2 * span); }

template <int NT, bool EX, class V, class DT>
__device__ __forceinline__ void merge_level(const V X, DT* D, DT* SCR, int32_t* CNT, int2* MI, int m, int span,
                                            int kb, int ke, int* s_nhard, int4* s_hard, int hard_cap,
                                            const MergeCtl ctl0) {
    // the schedule variants and the debug checks exist only in the EX instances
    const MergeCtl ctl = EX ? ctl0 : MergeCtl{0, nullptr, ctl0.r};
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, wid = tid >> 6, wlane = tid & 63;
    const int nm = merges_at(m, span);
    const int nloc = ke - kb;
    if (nloc > NW && !(ctl.sched & kSchedWaveAll)) {
        if (tid == 0) *s_nhard = 0;
        __syncthreads();
        const bool three = EX && (ctl.sched & kSchedThreeCase) != 0;
        const int cap = three ? 8 * (ctl.r + 12) : kWalkCap;  // log2 C = 12
        for (int k = kb + tid; k < ke; k += NT) {
            const int a = 2 * k * span, b = a + span;
            List<DT> Lq{D + a, CNT[a]};
            List<DT> Rq{D + b, CNT[b]};
            Bridge br;
            if (!bridge_start(X, Lq, Rq, b, br.A, br.B) && !walk_thread(X, Lq, Rq, b, br.A, br.B, cap)) {
                if constexpr (EX) {
                    if (three) {
                        int st;
                        br = three_case_bridge(X, Lq, Rq, b, &st);
                        dbg_add(ctl.dbg, kDbgThreeCase);
                        apply_cut(D, CNT, MI, k, a, b, Rq.n, br);
                        continue;
                    }
                }
                {
                    int h = atomicAdd(s_nhard, 1);
                    if (h < hard_cap) {
                        s_hard[h] = make_int4(k, br.A.seg, br.A.pos, br.B.seg);
                        MI[k] = make_int2(br.B.pos, 0);  // parked until the wave finishes it
                        dbg_add(ctl.dbg, kDbgToWave);
                        continue;
                    }
                    br = bisect_bridge(X, Lq, Rq, b);
                    dbg_add(ctl.dbg, kDbgBisect);
                }
            }
            apply_cut(D, CNT, MI, k, a, b, Rq.n, br);
        }
        __syncthreads();
        const int nh = min(*s_nhard, hard_cap);
        for (int h = wid; h < nh; h += NW) {
            const int4 hk = s_hard[h];
            const int k = hk.x, a = 2 * k * span, b = a + span;
            List<DT> Lq{D + a, CNT[a]};
            List<DT> Rq{D + b, CNT[b]};
            Bridge br{Cur{hk.y, hk.z}, Cur{hk.w, MI[k].x}};
            if (!walk_wave(X, Lq, Rq, b, br.A, br.B, kWaveWalkCap) && wlane == 0) {
                br = bisect_bridge(X, Lq, Rq, b);
                dbg_add(ctl.dbg, kDbgBisect);
            }
            if (wlane == 0) apply_cut(D, CNT, MI, k, a, b, Rq.n, br);
        }
    } else {
        for (int k = kb + wid; k < ke; k += NW) {
            const int a = 2 * k * span, b = a + span;
            List<DT> Lq{D + a, CNT[a]};
            List<DT> Rq{D + b, CNT[b]};
            Bridge br;
            if (!bridge_start(X, Lq, Rq, b, br.A, br.B)) {
                if (!walk_wave(X, Lq, Rq, b, br.A, br.B, kWaveWalkCap) && wlane == 0) {
                    br = bisect_bridge(X, Lq, Rq, b);
                    dbg_add(ctl.dbg, kDbgBisect);
                }
            }
            if (wlane == 0) apply_cut(D, CNT, MI, k, a, b, Rq.n, br);
        }
    }
    __syncthreads();
    int ts = NT / nloc;
    ts = ts < 1 ? 1 : (1 << (31 - __clz(ts)));
    const int teams = NT / ts;
    const int lane = tid & (ts - 1);
    for (int k = kb + tid / ts; k < ke; k += teams) {
        const int b = (2 * k + 1) * span;
        const int rs = MI[k].y;
        const int nr = CNT[b] - rs;
        for (int i = lane; i < nr; i += ts) SCR[b + i] = D[b + rs + i];
    }
    __syncthreads();
    for (int k = kb + tid / ts; k < ke; k += teams) {
        const int a = 2 * k * span, b = a + span;
        const int nl = MI[k].x;
        const int nr = CNT[b] - MI[k].y;
        for (int i = lane; i < nr; i += ts) D[a + nl + i] = SCR[b + i];
    }
    __syncthreads();
    if (EX && ctl.dbg) {
        // the nodes of the next level this workgroup made (a = 2 span k), and
        // the last workgroup also the unpaired node at the end, if any
        unsigned long long bad = 0;
        const int kl = ke == nm ? ke + 1 : ke;
        for (int a = 2 * span * (kb + tid); a < m && a < 2 * span * kl; a += 2 * span * NT) {
            const int n = CNT[a], hi_node = min(m, a + 2 * span);
            if (n < 1 || n > hi_node - a) {
                ++bad;
                continue;
            }
            int prev = a - 1;
            for (int i = 0; i < n; ++i) {
                const DT d = D[a + i];
                const int c = dchunk(d);
                if (c <= prev || c >= hi_node || dlo(d) > dhi(d) || dlo(d) < 0) ++bad;
                prev = c;
            }
        }
        dbg_add(ctl.dbg, kDbgViolations, bad);
        if (tid == 0 && kb == 0) dbg_add(ctl.dbg, kDbgLevels);
    }
}

// Rows beyond the two-stage merge: after the first stage (k_group_merge, every
// group of kGroup chunks merged in parallel, its list left at its first chunk's
// slot), one workgroup per row runs the remaining levels of the merge tree with
// the segment lists in the workspace.  Per level: one thread per merge finds its
// bridge and cuts the two boundary segments in place; then teams of threads
// move each right list's remaining descriptors down behind the left list's
// (through a scratch copy, since the two ranges may overlap).  The chunk
// starts come from the first stage (group starts plus starts within groups);
// at the end the root list and its prefix counts are left for the expansion,
// which forms each chunk's record itself.
// MODE: 0 the production instance, 1 with phase stamps, 2 with the debug checks
// and schedule variants.
// Launched twice per call: the prelude (kMergeRowsPre), then, after the levels
// that k_merge_level spreads over workgroups, the remaining levels from span0
// on and the end (kMergeRowsTail).
constexpr int kMergeRowsPre = 1, kMergeRowsTail = 2;
template <bool WT, int MODE>
__global__ __launch_bounds__(kMergeNT) void k_merge_rows(int m, LongWs ws, int span0, int phases) {
    constexpr bool ST = MODE == 1, EX = MODE == 2;
    constexpr int NT = kMergeNT;
    __shared__ double red[NT / 64 + 1];
    __shared__ int ired[NT / 64 + 1];
    __shared__ int sflag;
    __shared__ int s_nhard;
    __shared__ int4 s_hard[kHardCap];
    const int64_t row = blockIdx.x;
    const int64_t rb = row * m;
    const int tid = threadIdx.x;
    const int wid = tid >> 6, wlane = tid & 63;

    uint64_t* const sr = ST ? stamp_row(ws.st_top, row) : nullptr;
    uint2* const D = ws.desc + rb;
    uint2* const SCR = ws.desc_scr + rb;
    int32_t* const CNT = ws.node_cnt + rb;
    int2* const MI = ws.merge_info + rb;
    int32_t* const HC = ws.hull_cnt + rb;
    double* const STS = ws.st_S + rb;
    double* const STW = WT ? ws.st_W + rb : nullptr;

    const size_t sl = (size_t)rb * (kChunk + 1);
    RowView X{ws.slot_idx + sl, ws.slot_S + sl, WT ? ws.slot_W + sl : nullptr, ws.win + rb, HC,
              STS, WT ? STW : nullptr, WT, inc_src(ws, row, m, 0)};
    if (phases & kMergeRowsPre) {
    stamp(sr, 0);
    // ---- row flags and group starts (an exclusive scan of the first stage's
    // group totals), then every chunk start as its group's start plus its
    // start within the group (both from the first stage)
    const int ng = (m + kGroup - 1) / kGroup;
    double* const gS = reinterpret_cast<double*>(MI);  // (the merge's scratch, free until the tree)
    double* const gW = gS + ng;
    if (tid == 0) sflag = 0;
    __syncthreads();
    int f = 0;
    double carryS = 0.0, carryW = 0.0;
    for (int g0 = 0; g0 < ng; g0 += NT) {
        const int g = g0 + tid;
        double2 t = make_double2(0.0, 0.0);
        if (g < ng) {
            const GroupWin* gw = ws.gwin + row * ng + g;
            f |= gw->flags;
            CNT[g * kGroup] = gw->nseg;  // the first stage's group lists: their segment counts
            t = ws.gtot[row * ng + g];
        }
        double tot;
        const double xs = wg_excl_scan<NT>(t.x, red, &tot);
        if (g < ng) gS[g] = carryS + xs;
        carryS += tot;
        if (WT) {
            const double xw = wg_excl_scan<NT>(t.y, red, &tot);
            if (g < ng) gW[g] = carryW + xw;
            carryW += tot;
        }
    }
    if (f) atomicOr(&sflag, f);
    __syncthreads();
    for (int j = tid; j < m; j += NT) {
        const double2 c = ws.cst[rb + j];
        STS[j] = gS[j / kGroup] + c.x;
        if (WT) STW[j] = gW[j / kGroup] + c.y;
    }
    __syncthreads();
    if (tid == 0) ws.row_flag[row] = sflag;
    stamp(sr, 1);  // prelude: flags, chunk starts, group list counts
    }
    if (!(phases & kMergeRowsTail)) return;
    stamp(sr, 3);  // the levels left to this kernel start

    // ---- the merge tree's remaining levels (tree level r: span 2^r chunks)
    for (int span = span0, r = 31 - __clz(span0); span < m; span <<= 1, ++r) {
        merge_level<NT, EX>(X, D, SCR, CNT, MI, m, span, 0, merges_at(m, span), &s_nhard, s_hard, kHardCap,
                            MergeCtl{ws.sched, ws.dbg, r});
        if (r - 6 < 11) stamp(sr, 5 + r - 6);  // through tree level r
    }

    stamp(sr, 2);  // merge tree done
    // ---- what the expansion needs for its records (Corollary 4.5): the root
    // list (into desc_scr), the root vertices before each segment (vb), and
    // each chunk's first root segment (into node_cnt, no longer a count);
    // each thread a run of consecutive segments, their chunks staged in the
    // merge's scratch (merge_info) for the search
    const int nroot = CNT[0];
    int32_t* const rcg = reinterpret_cast<int32_t*>(MI);
    {
        const int ks = (nroot + NT - 1) / NT;
        const int i0 = min(nroot, tid * ks), i1 = min(nroot, i0 + ks);
        int loc = 0;
        for (int i = i0; i < i1; ++i) {
            const uint2 d = D[i];
            SCR[i] = d;
            rcg[i] = dchunk(d);
            loc += dhi(d) - dlo(d) + 1;
        }
        int tot;
        int x = wg_excl_scan_int<NT>(loc, ired, &tot);  // its barriers also publish rcg
        for (int i = i0; i < i1; ++i) {
            const uint2 d = D[i];
            ws.vb[rb + i] = x;
            x += dhi(d) - dlo(d) + 1;
        }
    }
    __syncthreads();  // every thread has read CNT[0] before fs overwrites it
    root_fs<NT>(nroot, m, CNT, rcg);
    if (tid == 0) ws.root_n[row] = nroot;
    stamp(sr, 4);  // end
}


// One level of the merge tree of rows beyond the two-stage merge, spread over
// workgroups (grid: workgroups per row, rows): workgroup x runs merges
// x*per .. x*per+per-1 of its row, a wave per merge when per is at most the
// workgroup's waves.
template <bool WT, int MODE>
__global__ __launch_bounds__(kMergeNT) void k_merge_level(int m, int span, int per, LongWs ws) {
    constexpr bool EX = MODE == 2;
    constexpr int NT = kMergeNT;
    __shared__ int s_nhard;
    __shared__ int4 s_hard[kHardCap];
    const int64_t row = blockIdx.y;
    const int64_t rb = row * m;
    const int nm = merges_at(m, span);
    const int kb = (int)blockIdx.x * per, ke = min(nm, kb + per);
    if (kb >= ke) return;  // (the same in every thread)
    const size_t sl = (size_t)rb * (kChunk + 1);
    const RowView X{ws.slot_idx + sl, ws.slot_S + sl, WT ? ws.slot_W + sl : nullptr, ws.win + rb,
                    ws.hull_cnt + rb, ws.st_S + rb, WT ? ws.st_W + rb : nullptr, WT, inc_src(ws, row, m, 0)};
    merge_level<NT, EX>(X, ws.desc + rb, ws.desc_scr + rb, ws.node_cnt + rb, ws.merge_info + rb, m, span, kb, ke,
                        &s_nhard, s_hard, kHardCap, MergeCtl{ws.sched, ws.dbg, 31 - __clz(span)});
}

// Vertices of group hulls for the second stage: position p of group g's hull,
// relative to group gr's first point.
struct GroupView {
    const GroupWin* gw;  // group windows (LDS)
    const int32_t* gh;   // group hull vertex counts (LDS)
    const double* gS;    // group starts (LDS)
    const double* gW;
    const uint2* gdesc;  // group lists (chunk segments), stored from each group's first chunk
    const int32_t* gpre; // vertices before each segment of a group list
    const double2* cst;  // chunk starts relative to their group
    RowView C;           // chunk hull vertices (chunk-relative)
    bool weighted;

    __device__ __forceinline__ Pt vtx(int g, int pos, int gr) const {
        const int h = gh[g];
        int e = pos;
        if (h > 2 * kGWinK && pos >= kGWinK) e = pos >= h - kGWinK ? kGWinK + pos - (h - kGWinK) : -1;
        double s, w;
        if (e >= 0) {
            const double2 v = gw[g].v[e];
            s = v.x;
            w = v.y;
        } else {
            // the segment of the group's list that holds position pos
            const int base = g * kGroup;
            int lo = 0, hi = gw[g].nseg - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (gpre[base + mid] <= pos) lo = mid;
                else hi = mid - 1;
            }
            const uint2 d = gdesc[base + lo];
            const int j = dchunk(d);
            const Pt v = C.vrel(j, dlo(d) + (pos - gpre[base + lo]));
            const double2 c = cst[j];
            s = c.x + v.s;
            w = c.y + v.w;
        }
        Pt p;
        p.s = (gS[g] - gS[gr]) + s;
        p.w = (gW[g] - gW[gr]) + w;
        return p;
    }
};

template <bool WT, typename T, int MODE>
__global__ __launch_bounds__(kGroupNT) void k_group_merge(int m, int ng, LongWs ws) {
    constexpr bool ST = MODE == 1, EX = MODE == 2;
    constexpr int NT = kGroupNT, G = kGroup, E = 2 * kWinK, EG = 2 * kGWinK;
    static_assert(G == 64, "one wave numbers a group's segments");
    // the generic path's chunk windows, or the fast path's compact arrays, or
    // (before either) the rebuild of a chunk hull the chunk kernel gave up on
    using RedoSmem = HullSmem<NT, kChunk / NT, WT, kHullChains>;
    constexpr size_t kGen = sizeof(WinRec) * G;
    constexpr size_t kFast = (size_t)G * E * (8 + 8 + 4);
    constexpr size_t kPool0 = kGen > kFast ? kGen : kFast;
    __shared__ __align__(16) unsigned char pool[kPool0 > sizeof(RedoSmem) ? kPool0 : sizeof(RedoSmem)];
    __shared__ double lS[G], lW[G];
    __shared__ int32_t HC[G], CNT[G], VER[G], pre[G + 1];
    __shared__ uint2 D[G], SCR[G];
    __shared__ int2 MI[G / 2 + 1];
    __shared__ int s_nhard;
    __shared__ int4 s_hard[G / 2];
    __shared__ int ired[NT / 64 + 1];
    __shared__ int sflag, s_nseg;
    __shared__ int sfirst[G], slast[G];
    const int64_t gid = blockIdx.x;
    const int64_t row = gid / ng;
    const int g = (int)(gid - row * ng);
    const int64_t rb = row * m;
    const int j0 = g * G, gc = min(G, m - j0);
    const int tid = threadIdx.x, wid = tid >> 6, wlane = tid & 63;
    uint64_t* const sr = ST ? stamp_row(ws.st_group, gid) : nullptr;
    stamp(sr, 0);

    // the prelude's global reads, issued together: every chunk window (raw
    // 16-byte words, the hull count in each header) and the chunk totals
    constexpr int kW2 = (int)(sizeof(WinRec) / sizeof(double2));
    constexpr int kRaw = (G * kW2 + NT - 1) / NT;
    const int nraw = gc * kW2;
    const double2* wsrc = reinterpret_cast<const double2*>(ws.win + rb + j0);
    double2 raw[kRaw];
#pragma unroll
    for (int q = 0; q < kRaw; ++q) {
        const int i = tid + q * NT;
        raw[q] = i < nraw ? wsrc[i] : make_double2(0.0, 0.0);
    }
    double ts = 0.0, tw = 0.0;
    int cdf = 0;  // the chunk's data flags (a rebuild below leaves them as they are)
    if (wid == 0 && wlane < gc) {
        cdf = ws.chunk_flag[rb + j0 + wlane] & kFlagData;
        ts = ws.tot_S[rb + j0 + wlane];
        if (WT) tw = ws.tot_W[rb + j0 + wlane];
    }
    // hull counts; the fast path needs every chunk hull whole in its window
    bool ok = true, redo = false;
#pragma unroll
    for (int q = 0; q < kRaw; ++q) {
        const int i = tid + q * NT;
        if (i < nraw && i % kW2 == 0) {
            const int h = (int)(uint32_t)__double_as_longlong(raw[q].x);  // WinRec::h
            HC[i / kW2] = h;
            ok = ok && h <= E;
            redo = redo || h == 0;
        }
    }
    // (f64 input: the fallback kernel rebuilt them before this launch)
    if (sizeof(T) == 4 && __syncthreads_or(redo)) {
        // chunks the chunk kernel gave up on (header h = 0, written in this
        // call): the whole workgroup rebuilds each with chains and merges,
        // then every window word is read again
        RedoSmem& hs = *reinterpret_cast<RedoSmem*>(pool);
        for (int i = 0; i < gc; ++i) {
            if (HC[i] != 0) continue;  // the same in every thread
            if constexpr (sizeof(T) == 4)
                chunk_hull<NT, kChunk / NT, kHullChains, WT, float>(static_cast<const float*>(ws.y),
                                                                    static_cast<const float*>(ws.w), ws.n, m,
                                                                    ws.sign, ws, 0, hs, rb + j0 + i);
            if (tid == 0) dbg_add(ws.dbg, kDbgRebuilt);
            __syncthreads();
        }
        ok = true;
#pragma unroll
        for (int q = 0; q < kRaw; ++q) {
            const int i = tid + q * NT;
            raw[q] = i < nraw ? wsrc[i] : make_double2(0.0, 0.0);
            if (i < nraw && i % kW2 == 0) {
                const int h = (int)(uint32_t)__double_as_longlong(raw[q].x);
                HC[i / kW2] = h;
                ok = ok && h <= E;
            }
        }
    }
    if (wid == 0) {
        // chunk starts relative to the group: a scan of the chunk totals
        double is = ts, iw = tw;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            double us = __shfl_up(is, d), uw = __shfl_up(iw, d);
            if (wlane >= d) { is += us; iw += uw; }
        }
        double es = __shfl_up(is, 1), ew = __shfl_up(iw, 1);
        if (wlane == 0) { es = 0.0; ew = 0.0; }
        if (!WT) ew = (double)wlane * kChunk;  // unit weights: W is the point index
        if (wlane < gc) {
            lS[wlane] = es;
            lW[wlane] = ew;
            ws.cst[rb + j0 + wlane] = make_double2(es, ew);
        }
        const double totS = __shfl(is, 63), totW = __shfl(iw, 63);
        if (wlane == 0) ws.gtot[row * ng + g] = make_double2(totS, WT ? totW : 0.0);
    }
    const bool fast = __syncthreads_and(ok) != 0;
    stamp(sr, 1);  // prelude loaded (and any rebuilt chunks), starts scanned
    const size_t sl = (size_t)(rb + j0) * (kChunk + 1);
    GroupWin* gwo = ws.gwin + row * ng + g;
    int nseg, hg;
    if (fast) {
        // ---- every chunk hull is short: merge compact arrays in LDS
        double* aS = reinterpret_cast<double*>(pool);
        const Arr ar{aS, aS + G * E, reinterpret_cast<int32_t*>(aS + 2 * G * E)};
#pragma unroll
        for (int q = 0; q < kRaw; ++q) {
            const int r = tid + q * NT;
            const int i = r / kW2, e = r - i * kW2 - 1;  // word 0 is the header
            if (r < nraw && e >= 0 && e < HC[i]) {
                const int t = i * E + e;
                ar.S[t] = lS[i] + raw[q].x;
                ar.W[t] = lW[i] + raw[q].y;
                ar.tag[t] = mktag(i, e);
            }
        }
        for (int i = tid; i < gc; i += NT) {
            CNT[i] = HC[i];
            VER[i] = 0;
            sfirst[i] = -1;
        }
        __syncthreads();
        merge_arrays<NT>(ar, CNT, VER, gc, E, sr);
        stamp(sr, 2);  // merge tree done (compact arrays)
        hg = CNT[0];
        // the group's list: one segment per run of a chunk's vertices
        for (int t = tid; t < hg; t += NT) {
            const int c = tchunk(ar.tag[t]);
            if (t == 0 || tchunk(ar.tag[t - 1]) != c) sfirst[c] = t;
            if (t == hg - 1 || tchunk(ar.tag[t + 1]) != c) slast[c] = t;
        }
        __syncthreads();
        if (wid == 0) {
            const bool has = wlane < gc && sfirst[wlane] >= 0;
            const uint64_t bal = __ballot(has);
            const int sidx = __popcll(bal & ((1ull << wlane) - 1ull));
            if (has) {
                D[sidx] = mkdesc(wlane, tpos(ar.tag[sfirst[wlane]]), tpos(ar.tag[slast[wlane]]));
                pre[sidx] = sfirst[wlane];
            }
            if (wlane == 0) {
                s_nseg = __popcll(bal);
                pre[__popcll(bal)] = hg;
            }
        }
        __syncthreads();
        nseg = s_nseg;
        const int nwin = min(hg, EG);
        for (int t = tid; t < nwin; t += NT) {
            const int r = (hg <= EG || t < kGWinK) ? t : hg - EG + t;
            gwo->v[t] = make_double2(ar.S[r], ar.W[r]);
            gwo->tag[t] = mktag(j0 + tchunk(ar.tag[r]), tpos(ar.tag[r]));
        }
    } else {
        // ---- segment lists over the chunk hulls' windows
        WinRec* Wn = reinterpret_cast<WinRec*>(pool);
        {
            double2* dst = reinterpret_cast<double2*>(Wn);
#pragma unroll
            for (int q = 0; q < kRaw; ++q) {
                const int i = tid + q * NT;
                if (i < nraw) dst[i] = raw[q];
            }
        }
        for (int i = tid; i < gc; i += NT) {
            D[i] = mkdesc(i, 0, HC[i] - 1);
            CNT[i] = 1;
        }
        __syncthreads();
        const RowView X{ws.slot_idx + sl, ws.slot_S + sl, WT ? ws.slot_W + sl : nullptr, Wn, HC, lS, lW, WT,
                        inc_src(ws, row, m, j0)};
        // when the chain of chunk hulls turns strictly left at every junction
        // it is convex, so the group hull is the concatenation (each later
        // hull without its first point, the shared one)
        bool jc = true;
        if (tid + 1 < gc) {
            const int h = HC[tid];
            jc = cross3(X.vtx(tid, h - 2, tid + 1), X.vtx(tid + 1, 0, tid + 1), X.vtx(tid + 1, 1, tid + 1)) > 0.0;
        }
        if (__syncthreads_and(jc)) {
            for (int i = tid; i < gc; i += NT) D[i] = mkdesc(i, i == 0 ? 0 : 1, HC[i] - 1);
            if (tid == 0) CNT[0] = gc;
            __syncthreads();
        } else {
            for (int span = 1; span < gc; span <<= 1)
                merge_level<NT, EX>(X, D, SCR, CNT, MI, gc, span, 0, merges_at(gc, span), &s_nhard, s_hard, G / 2,
                                    MergeCtl{ws.sched, ws.dbg, 31 - __clz(span)});
        }
        stamp(sr, 2);  // merge tree done (segment lists)
        nseg = CNT[0];
        if (wid == 0) {
            int v = 0;
            if (wlane < nseg) v = dhi(D[wlane]) - dlo(D[wlane]) + 1;
            int x = v;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                int u = __shfl_up(x, d);
                if (wlane >= d) x += u;
            }
            if (wlane < nseg) pre[wlane + 1] = x;
            if (wlane == 0) pre[0] = 0;
        }
        __syncthreads();
        hg = pre[nseg];
        const int nwin = min(hg, EG);
        for (int t = tid; t < nwin; t += NT) {
            const int r = (hg <= EG || t < kGWinK) ? t : hg - EG + t;
            int lo = 0, hi = nseg - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (pre[mid] <= r) lo = mid;
                else hi = mid - 1;
            }
            const uint2 d = D[lo];
            const int pos = dlo(d) + (r - pre[lo]);
            const Pt v = X.vtx(dchunk(d), pos, 0);
            gwo->v[t] = make_double2(v.s, v.w);
            gwo->tag[t] = mktag(j0 + dchunk(d), pos);
        }
    }
    stamp(sr, 3);  // group window written
    for (int i = tid; i < nseg; i += NT) {
        const uint2 d = D[i];
        ws.desc[rb + j0 + i] = mkdesc(j0 + dchunk(d), dlo(d), dhi(d));
        ws.gpre[rb + j0 + i] = pre[i];
    }
    if (tid == 0) {
        gwo->h = hg;
        gwo->nseg = nseg;
        gwo->pre1 = pre[1];
    }
    if (wid == 0) {
        // the group's data flags, for the second stage
        int f = cdf;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) f |= __shfl_xor(f, d);
        if (wlane == 0) gwo->flags = f;
    }
    if (ng == 1) {
        // the group is the whole row: its list is the root
        if (tid == 0) sflag = 0;
        __syncthreads();
        int f = 0;
        for (int j = tid; j < m; j += NT) f |= ws.chunk_flag[rb + j] & kFlagData;
        if (f) atomicOr(&sflag, f);
        // the root list, its prefix counts and the chunk starts, for the
        // expansion's records
        for (int i = tid; i < nseg; i += NT) ws.desc_scr[rb + i] = D[i];
        for (int j = tid; j < m; j += NT) {
            ws.st_S[rb + j] = lS[j];
            if (WT) ws.st_W[rb + j] = lW[j];
        }
        root_prefixes<NT>(D, nseg, m, ws.vb + rb, ws.node_cnt + rb, ired, slast);
        if (fast) {
            // the root edge into each segment, from the group hull's entries
            const double* aS = reinterpret_cast<const double*>(pool);
            const double* aW = aS + G * E;
            for (int i = tid + 1; i < nseg; i += NT) {
                const int t = pre[i];
                ws.rslope[rb + i] = (aS[t] - aS[t - 1]) / (aW[t] - aW[t - 1]);
            }
        }
        if (tid == 0) {
            ws.row_flag[row] = sflag;
            ws.root_n[row] = nseg | (fast ? kRootSlopes : 0);
        }
    }
    stamp(sr, 4);  // end
}

// Dynamic LDS of the second stage: group starts gS, gW (8 B each), then
// either the segment-list path's D, SCR (16 B each), GW, MI (8 B per merge),
// CNT (4 B each, and 4 B spare), or the compact-array path's 2 kGWinK entries
// per group (S, W, tag) and CNT; after that the root segments' chunks (at most
// one segment per chunk and one per window entry).
__host__ __device__ inline size_t top_lds_main(int ng) {
    const size_t gen = (size_t)ng * (32 + sizeof(GroupWin) + 8) + (size_t)(ng / 2 + 1) * 8;
    const size_t fast = (size_t)ng * (2 * kGWinK) * 20 + (size_t)ng * 4;
    return (size_t)ng * 16 + (gen > fast ? gen : fast);
}
__host__ __device__ inline int top_root_cap(int ng, int m) { return m < ng * 2 * kGWinK ? m : ng * 2 * kGWinK; }
inline size_t top_lds_bytes(int ng, int m) { return top_lds_main(ng) + (size_t)top_root_cap(ng, m) * 4; }

template <bool WT, int MODE>
__global__ __launch_bounds__(kTopNT) void k_top_merge(int m, int ng, LongWs ws) {
    constexpr bool ST = MODE == 1, EX = MODE == 2;
    constexpr int NT = kTopNT, G = kGroup, E = 2 * kGWinK;
    extern __shared__ int4 top_lds[];
    __shared__ double red[NT / 64 + 1];
    __shared__ int ired[NT / 64 + 1];
    __shared__ int s_nhard;
    __shared__ int4 s_hard[kHardCap];
    __shared__ int s_ilo[kTopMax], s_ihi[kTopMax], s_off[kTopMax + 1];
    __shared__ int s_gh[kTopMax], s_gn[kTopMax], s_gf[kTopMax], s_ver[kTopMax];
    __shared__ int32_t s_lc[kTopMax], s_rc[kTopMax], s_nx[kTopMax], s_pv[kTopMax], s_dead[kTopMax], s_ko[kTopMax];
    const int64_t row = blockIdx.x;
    const int64_t rb = row * m, gb = row * ng;
    const int tid = threadIdx.x;
    uint64_t* const sr = ST ? stamp_row(ws.st_top, row) : nullptr;
    stamp(sr, 0);

    // the prelude's global reads, issued together: every group window (raw
    // 16-byte words; the header holds the hull count, segment count and data
    // flags) and the group totals
    constexpr int kW2 = (int)(sizeof(GroupWin) / sizeof(double2));
    constexpr int kRaw = (kTopMax * kW2 + NT - 1) / NT;
    const int nraw = ng * kW2;
    const double2* wsrc = reinterpret_cast<const double2*>(ws.gwin + gb);
    double2 raw[kRaw];
#pragma unroll
    for (int q = 0; q < kRaw; ++q) {
        const int i = tid + q * NT;
        raw[q] = i < nraw ? wsrc[i] : make_double2(0.0, 0.0);
    }
    constexpr int kRo = (kTopMax * kGroup + NT - 1) / NT;
    const int wid = tid >> 6, lane = tid & 63;
    double2 gt0 = make_double2(0.0, 0.0), gt1 = make_double2(0.0, 0.0);  // groups 2*lane, 2*lane+1
    if (wid == 0) {
        if (2 * lane < ng) gt0 = ws.gtot[gb + 2 * lane];
        if (2 * lane + 1 < ng) gt1 = ws.gtot[gb + 2 * lane + 1];
    }
    // group hull counts; the fast path needs every group hull whole in its window
    bool ok = true;
#pragma unroll
    for (int q = 0; q < kRaw; ++q) {
        const int i = tid + q * NT;
        if (i < nraw && i % kW2 == 0) {
            const uint64_t h01 = (uint64_t)__double_as_longlong(raw[q].x);  // h, nseg
            const int h = (int)(uint32_t)h01;
            s_gh[i / kW2] = h;
            s_gn[i / kW2] = (int)(uint32_t)(h01 >> 32);
            s_gf[i / kW2] = (int)(uint32_t)__double_as_longlong(raw[q].y);  // data flags
            ok = ok && h <= E;
        }
    }

    // group starts (exclusive scan of the group totals, two groups per lane)
    double* gS = reinterpret_cast<double*>(top_lds);
    double* gW = gS + ng;
    if (wid == 0) {
        double is = gt0.x + gt1.x, iw = gt0.y + gt1.y;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const double us = __shfl_up(is, d), uw = __shfl_up(iw, d);
            if (lane >= d) { is += us; iw += uw; }
        }
        double es = __shfl_up(is, 1), ew = __shfl_up(iw, 1);
        if (lane == 0) { es = 0.0; ew = 0.0; }
        if (2 * lane < ng) {
            gS[2 * lane] = es;
            gW[2 * lane] = WT ? ew : (double)((int64_t)(2 * lane) * G * kChunk);
        }
        if (2 * lane + 1 < ng) {
            gS[2 * lane + 1] = es + gt0.x;
            gW[2 * lane + 1] = WT ? ew + gt0.y : (double)((int64_t)(2 * lane + 1) * G * kChunk);
        }
    }
    const bool fast = (__syncthreads_and(ok) != 0) && ng <= kTopFastMax && m < kTagMaxChunks;
    stamp(sr, 1);  // prelude loaded, group starts scanned
    // the chunk starts relative to their groups (S only: unit weights), for
    // the row's chunk starts stored at the end (a row has at most kTopMax
    // groups of kGroup chunks): read now, behind the prelude's reads, while
    // the merges work in LDS
    double cstv[kRo];
#pragma unroll
    for (int q = 0; q < kRo; ++q) {
        const int j = tid + q * NT;
        if (!WT && j < m) cstv[q] = reinterpret_cast<const double*>(ws.cst + rb + j)[0];
    }
    uint2* R = ws.desc_scr + rb;  // the root list, as segments of chunk hulls
    // after both paths' LDS: the root segments' chunks (and, on the compact
    // path, their vertex prefix), for the record prefix counts
    int32_t* rcbuf = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(top_lds) + top_lds_main(ng));
    int nroot;
    if (fast) {
        // ---- every group hull is short: merge compact arrays in LDS
        double* aS = gW + ng;
        const Arr ar{aS, aS + ng * E, reinterpret_cast<int32_t*>(aS + 2 * ng * E)};
        int32_t* CNT = ar.tag + ng * E;
        // words 1..E of a window are its entries' (S, W), the next E/4 words
        // their tags, four to a word (unused entries are copied too)
#pragma unroll
        for (int q = 0; q < kRaw; ++q) {
            const int r = tid + q * NT;
            const int g = r / kW2, o = r - g * kW2;
            if (r < nraw && o >= 1) {
                if (o <= E) {
                    const int t = g * E + o - 1;
                    ar.S[t] = gS[g] + raw[q].x;
                    ar.W[t] = gW[g] + raw[q].y;
                } else {
                    const int t = g * E + 4 * (o - 1 - E);
                    const uint64_t x = (uint64_t)__double_as_longlong(raw[q].x);
                    const uint64_t y = (uint64_t)__double_as_longlong(raw[q].y);
                    ar.tag[t] = (int32_t)(uint32_t)x;
                    ar.tag[t + 1] = (int32_t)(uint32_t)(x >> 32);
                    ar.tag[t + 2] = (int32_t)(uint32_t)y;
                    ar.tag[t + 3] = (int32_t)(uint32_t)(y >> 32);
                }
            }
        }
        for (int g = tid; g < ng; g += NT) {
            CNT[g] = s_gh[g];
            s_ver[g] = 0;
        }
        __syncthreads();
        // group hulls keep most of their vertices: bridges between
        // neighbouring groups, all at once; the merge tree if groups are still
        // being dropped after a few rounds
        const bool tree = EX && (ws.sched & kSchedTreeTop) != 0;
        const int rounds =
            tree ? -1 : merge_local<NT, E, kTopFastMax * E>(ar, CNT, ng, s_lc, s_rc, s_nx, s_pv, s_dead, s_ko, sr);
        if (EX && tid == 0 && !tree && rounds != 0) dbg_add(ws.dbg, kDbgLocalRounds, rounds < 0 ? kLocalRounds : rounds);
        if (rounds < 0) merge_arrays<NT>(ar, CNT, s_ver, ng, E, sr);
        stamp(sr, 2);  // merge done (compact arrays)
        const int hr = CNT[0];
        // one root segment per run of a chunk's vertices; its chunk into rcbuf
        uint16_t* R16 = reinterpret_cast<uint16_t*>(R);
        uint32_t* R32 = reinterpret_cast<uint32_t*>(R);
        int carry = 0;
        for (int t0 = 0; t0 < hr; t0 += NT) {
            const int t = t0 + tid;
            int c = -1;
            bool st = false, en = false;
            if (t < hr) {
                c = tchunk(ar.tag[t]);
                st = t == 0 || tchunk(ar.tag[t - 1]) != c;
                en = t == hr - 1 || tchunk(ar.tag[t + 1]) != c;
            }
            int tot;
            const int x = wg_excl_scan_int<NT>(st ? 1 : 0, ired, &tot);
            const int sidx = carry + x - (st ? 0 : 1);  // this entry's segment
            if (st) {
                R32[2 * sidx] = (uint32_t)c;
                R16[4 * sidx + 2] = (uint16_t)tpos(ar.tag[t]);
                rcbuf[sidx] = c;
                ws.vb[rb + sidx] = t;  // root vertices before the segment
                // the root edge into the segment
                if (t > 0) ws.rslope[rb + sidx] = (ar.S[t] - ar.S[t - 1]) / (ar.W[t] - ar.W[t - 1]);
            }
            if (en) R16[4 * sidx + 3] = (uint16_t)tpos(ar.tag[t]);
            carry += tot;
        }
        nroot = carry;
    } else {
        // ---- segment lists over the group hulls' windows
        int4* D = reinterpret_cast<int4*>(gW + ng);
        int4* SCR = D + ng;
        GroupWin* GW = reinterpret_cast<GroupWin*>(SCR + ng);
        int2* MI = reinterpret_cast<int2*>(GW + ng);
        int32_t* CNT = reinterpret_cast<int32_t*>(MI + (ng / 2 + 1));
        const int32_t* GH = s_gh;
        {
            double2* dst = reinterpret_cast<double2*>(GW);
#pragma unroll
            for (int q = 0; q < kRaw; ++q) {
                const int i = tid + q * NT;
                if (i < nraw) dst[i] = raw[q];
            }
        }
        for (int g = tid; g < ng; g += NT) {
            D[g] = make_int4(g, 0, GH[g] - 1, 0);
            CNT[g] = 1;
        }
        __syncthreads();
        const size_t sl = (size_t)rb * (kChunk + 1);
        const RowView Cv{ws.slot_idx + sl, ws.slot_S + sl, WT ? ws.slot_W + sl : nullptr, ws.win + rb,
                         ws.hull_cnt + rb, ws.st_S + rb, WT ? ws.st_W + rb : nullptr, WT,
                         inc_src(ws, row, m, 0)};
        const GroupView X{GW, GH, gS, gW, ws.desc + rb, ws.gpre + rb, ws.cst + rb, Cv, WT};
        // a chain of group hulls turning strictly left at every junction is
        // the row hull: the concatenation
        bool jc = true;
        if (tid + 1 < ng) {
            const int h = GH[tid];
            jc = cross3(X.vtx(tid, h - 2, tid + 1), X.vtx(tid + 1, 0, tid + 1), X.vtx(tid + 1, 1, tid + 1)) > 0.0;
        }
        if (__syncthreads_and(jc)) {
            for (int g = tid; g < ng; g += NT) D[g] = make_int4(g, g == 0 ? 0 : 1, GH[g] - 1, 0);
            if (tid == 0) CNT[0] = ng;
            __syncthreads();
        } else {
            for (int span = 1; span < ng; span <<= 1)
                merge_level<NT, EX>(X, D, SCR, CNT, MI, ng, span, 0, merges_at(ng, span), &s_nhard, s_hard, kHardCap,
                                    MergeCtl{ws.sched, ws.dbg, 6 + 31 - __clz(span)});
        }
        stamp(sr, 2);  // merge tree done (segment lists)

        // the root list over groups, expanded into segments of chunk hulls:
        // first the range of group-list segments each root entry covers, then
        // one thread per output segment
        const int nr2 = CNT[0];
        auto seg_of = [&](int g, int p) {
            const int base = g * G;
            int a = 0, b = s_gn[g] - 1;
            while (a < b) {
                const int mid = (a + b + 1) >> 1;
                if (ws.gpre[rb + base + mid] <= p) a = mid;
                else b = mid - 1;
            }
            return a;
        };
        for (int t = tid; t < nr2; t += NT) {
            const int4 d = D[t];
            // a whole group list (always so where every merge was convex)
            // needs no search
            s_ilo[t] = d.y == 0 ? 0 : (d.y == 1 ? (GW[d.x].pre1 > 1 ? 0 : 1) : seg_of(d.x, d.y));
            s_ihi[t] = d.z == GH[d.x] - 1 ? s_gn[d.x] - 1 : seg_of(d.x, d.z);
        }
        __syncthreads();
        if (wid == 0) {
            // s_off: root segments before each root entry (two entries a lane)
            const int t0 = 2 * lane, t1 = t0 + 1;
            const int v0 = t0 < nr2 ? s_ihi[t0] - s_ilo[t0] + 1 : 0;
            const int v1 = t1 < nr2 ? s_ihi[t1] - s_ilo[t1] + 1 : 0;
            int x = v0 + v1;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int u = __shfl_up(x, d);
                if (lane >= d) x += u;
            }
            const int ex = x - v0 - v1;
            if (t0 <= nr2) s_off[t0] = ex;
            if (t1 <= nr2) s_off[t1] = ex + v0;
        }
        __syncthreads();
        nroot = s_off[nr2];
        // each thread a run of consecutive root segments (at most kRo, as a
        // row has at most one per chunk): every load first, then the
        // segments, their chunks (rcbuf) and vertex counts, and vb by one
        // workgroup scan
        const int ks = (nroot + NT - 1) / NT;
        const int o0 = min(nroot, tid * ks), no = min(nroot, o0 + ks) - o0;
        int4 ddv[kRo];
        uint2 dv[kRo];
        int iv[kRo], pv[kRo], av[kRo];
#pragma unroll
        for (int q = 0; q < kRo; ++q) {
            const int o = o0 + q;
            if (q < no) {
                int a = 0, b = nr2 - 1;
                while (a < b) {
                    const int mid = (a + b + 1) >> 1;
                    if (s_off[mid] <= o) a = mid;
                    else b = mid - 1;
                }
                av[q] = a;
                ddv[q] = D[a];
                iv[q] = s_ilo[a] + (o - s_off[a]);
                const int k = ddv[q].x * G + iv[q];
                dv[q] = ws.desc[rb + k];
                pv[q] = ws.gpre[rb + k];
            }
        }
        int loc = 0, len[kRo];
#pragma unroll
        for (int q = 0; q < kRo; ++q) {
            const int o = o0 + q;
            len[q] = 0;
            if (q < no) {
                const int a = av[q], i = iv[q];
                const uint2 d = dv[q];
                const int lo = i == s_ilo[a] ? dlo(d) + (ddv[q].y - pv[q]) : dlo(d);
                const int hi = i == s_ihi[a] ? dlo(d) + (ddv[q].z - pv[q]) : dhi(d);
                R[o] = mkdesc(dchunk(d), lo, hi);
                rcbuf[o] = dchunk(d);
                len[q] = hi - lo + 1;
                loc += len[q];
            }
        }
        int tot;
        int x = wg_excl_scan_int<NT>(loc, ired, &tot);
#pragma unroll
        for (int q = 0; q < kRo; ++q) {
            if (q < no) ws.vb[rb + o0 + q] = x;
            x += len[q];
        }
    }
    stamp(sr, 3);  // root list and its vertex prefix written
    // chunk starts of the row: group start plus the chunk's start in its group
#pragma unroll
    for (int q = 0; q < kRo; ++q) {
        const int j = tid + q * NT;
        if (j < m) {
            if (WT) {
                const double2 c = ws.cst[rb + j];
                ws.st_S[rb + j] = gS[j / G] + c.x;
                ws.st_W[rb + j] = gW[j / G] + c.y;
            } else {
                ws.st_S[rb + j] = gS[j / G] + cstv[q];
            }
        }
    }
    __syncthreads();
    // the first root segment of each chunk, for the expansion's records
    root_fs<NT>(nroot, m, ws.node_cnt + rb, rcbuf);
    if (tid == 0) {
        int f = 0;
        for (int g = 0; g < ng; ++g) f |= s_gf[g];
        ws.row_flag[row] = f;
        ws.root_n[row] = nroot | (fast ? kRootSlopes : 0);
    }
    stamp(sr, 4);  // end (chunk starts and each chunk's first root segment written)
}

// Debug check of each row's root list (ISO_F_DEBUG_INVARIANTS): at most one
// segment per chunk, in strictly increasing chunk order, each within its
// chunk hull (Definition 4.3, Theorem 4.4); the list starts at the row's
// first point and ends at its last; and every root vertex turns left or runs
// straight with its neighbours (the root list is a convex chain: its vertices
// include the hull's and lie on it).  Workgroup (row, part): part 0 checks the
// list, every part a stride of the vertices.
constexpr int kDbgParts = 64;
template <bool WT>
__global__ __launch_bounds__(256) void k_debug_root(int m, LongWs ws) {
    const int64_t row = blockIdx.x / kDbgParts;
    const int part = (int)(blockIdx.x - row * kDbgParts);
    const int64_t rb = row * m;
    const int tid = threadIdx.x;
    if (ws.row_flag[row] & kFlagNonfinite) return;
    const uint2* D = ws.desc_scr + rb;  // both merge paths leave the root list here
    const int nroot = ws.root_n[row] & ~kRootSlopes;
    const int32_t* HC = ws.hull_cnt + rb;
    unsigned long long bad = 0;
    if (nroot < 1 || nroot > m) {
        if (part == 0 && tid == 0) dbg_add(ws.dbg, kDbgViolations);
        return;
    }
    // a segment is readable when its chunk and positions lie within the chunk's hull
    auto ok_seg = [&](uint2 d) {
        const int c = dchunk(d);
        return c >= 0 && c < m && dlo(d) <= dhi(d) && dhi(d) < HC[c] && HC[c] <= kChunk + 1;
    };
    if (part == 0) {
        for (int i = tid; i < nroot; i += 256) {
            const uint2 d = D[i];
            if (!ok_seg(d)) ++bad;
            if (i > 0 && dchunk(D[i - 1]) >= dchunk(d)) ++bad;
        }
        if (tid == 0) {
            const uint2 f = D[0], l = D[nroot - 1];
            if (dchunk(f) != 0 || dlo(f) != 0 || dchunk(l) != m - 1 || dhi(l) != HC[m - 1] - 1) ++bad;
        }
    }
    // vertex v of the root chain: segment by binary search over the vertex prefix
    const int32_t* vb = ws.vb + rb;
    const uint2 dl = D[nroot - 1];
    const int64_t nv64 = ok_seg(dl) ? (int64_t)vb[nroot - 1] + dhi(dl) - dlo(dl) + 1 : 0;
    const int nv = (int)min(max(nv64, (int64_t)0), (int64_t)m * (kChunk + 1));
    const size_t sl = (size_t)rb * (kChunk + 1);
    const RowView X{ws.slot_idx + sl, ws.slot_S + sl, WT ? ws.slot_W + sl : nullptr, ws.win + rb, HC,
                    ws.st_S + rb, WT ? ws.st_W + rb : nullptr, WT, inc_src(ws, row, m, 0)};
    // vertex v, or false when the list does not hold it readably
    auto vert = [&](int v, Pt& p) {
        int lo = 0, hi = nroot - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (vb[mid] <= v) lo = mid;
            else hi = mid - 1;
        }
        const uint2 d = D[lo];
        const int pos = dlo(d) + (v - vb[lo]);
        if (!ok_seg(d) || pos < dlo(d) || pos > dhi(d)) return false;
        p = X.vtx(dchunk(d), pos, 0);
        return true;
    };
    unsigned long long checked = 0;
    for (int v = 1 + part * 256 + tid; v + 1 < nv; v += 256 * kDbgParts) {
        Pt a, b, c;
        if (!vert(v - 1, a) || !vert(v, b) || !vert(v + 1, c)) {
            ++bad;
            continue;
        }
        const double t1 = mul_rn(b.w - a.w, c.s - a.s), t2 = mul_rn(b.s - a.s, c.w - a.w);
        // a right turn beyond rounding: the chain is not convex there
        if (t1 - t2 < -1e-9 * (fabs(t1) + fabs(t2))) ++bad;
        if (!(b.w > a.w)) ++bad;
        ++checked;
    }
    dbg_add(ws.dbg, kDbgViolations, bad);
    dbg_add(ws.dbg, kDbgRootVerts, checked);
}

// The merge phase over segment lists: the first stage over every group of
// chunks, then the second stage (or, for very long rows, the row merge).
template <int MODE>
hipError_t launch_segment_merge_t(const LongShape& sh, const LongWs& ws, hipStream_t st, bool* rec_done) {
    const bool wt = sh.weighted;
    const int ng = (sh.m + kGroup - 1) / kGroup;
    const unsigned R = (unsigned)sh.rows;
    // first stage: every group of kGroup chunks
    timed_begin(kPhaseMerge, st);
    const dim3 grid(R * (unsigned)ng);
    if (ws.f64) {
        if (wt) hipLaunchKernelGGL((k_group_merge<true, double, MODE == 1 ? 0 : MODE>), grid, dim3(kGroupNT), 0, st, sh.m, ng, ws);
        else hipLaunchKernelGGL((k_group_merge<false, double, MODE == 1 ? 0 : MODE>), grid, dim3(kGroupNT), 0, st, sh.m, ng, ws);
    } else {
        if (wt) hipLaunchKernelGGL((k_group_merge<true, float, MODE>), grid, dim3(kGroupNT), 0, st, sh.m, ng, ws);
        else hipLaunchKernelGGL((k_group_merge<false, float, MODE>), grid, dim3(kGroupNT), 0, st, sh.m, ng, ws);
    }
    timed_end(st);
    if (two_stage_merge(sh.m)) {
        *rec_done = false;
        if (ng > 1) {
            const size_t lds = top_lds_bytes(ng, sh.m);
            static std::once_flag attr_once;
            std::call_once(attr_once, [] {
                const int maxb = (int)top_lds_bytes(kTopMax, kTopMax * kGroup);
                (void)hipFuncSetAttribute((const void*)k_top_merge<true, MODE>,
                                          hipFuncAttributeMaxDynamicSharedMemorySize, maxb);
                (void)hipFuncSetAttribute((const void*)k_top_merge<false, MODE>,
                                          hipFuncAttributeMaxDynamicSharedMemorySize, maxb);
            });
            timed_begin(kPhaseMergeTop, st);
            if (wt)
                hipLaunchKernelGGL((k_top_merge<true, MODE>), dim3(R), dim3(kTopNT), lds, st, sh.m, ng, ws);
            else
                hipLaunchKernelGGL((k_top_merge<false, MODE>), dim3(R), dim3(kTopNT), lds, st, sh.m, ng, ws);
            timed_end(st);
        }
        return hipGetLastError();
    }
    // very long rows: one workgroup per row merges the group lists through the
    // remaining levels, lists in the workspace
    // very long rows: the prelude, then the levels with more merges than a
    // workgroup has waves over several workgroups (a wave per merge), then
    // one workgroup per row for the last levels and the end
    *rec_done = false;
    timed_begin(kPhaseMergeTop, st);
    constexpr int per = kMergeNT / 64;
    if (wt)
        hipLaunchKernelGGL((k_merge_rows<true, MODE>), dim3(R), dim3(kMergeNT), 0, st, sh.m, ws, sh.m, kMergeRowsPre);
    else
        hipLaunchKernelGGL((k_merge_rows<false, MODE>), dim3(R), dim3(kMergeNT), 0, st, sh.m, ws, sh.m, kMergeRowsPre);
    int span = kGroup;
    for (; span < sh.m && merges_at(sh.m, span) > per; span <<= 1) {
        const dim3 grid((unsigned)((merges_at(sh.m, span) + per - 1) / per), R);
        if (wt) hipLaunchKernelGGL((k_merge_level<true, MODE>), grid, dim3(kMergeNT), 0, st, sh.m, span, per, ws);
        else hipLaunchKernelGGL((k_merge_level<false, MODE>), grid, dim3(kMergeNT), 0, st, sh.m, span, per, ws);
    }
    if (wt)
        hipLaunchKernelGGL((k_merge_rows<true, MODE>), dim3(R), dim3(kMergeNT), 0, st, sh.m, ws, span, kMergeRowsTail);
    else
        hipLaunchKernelGGL((k_merge_rows<false, MODE>), dim3(R), dim3(kMergeNT), 0, st, sh.m, ws, span, kMergeRowsTail);
    timed_end(st);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_segment_merge(const LongShape& sh, const LongWs& ws, hipStream_t st, bool* rec_done) {
    // phase stamps (measurement only, f32 input) come from separate instances
    // the debug checks and schedule variants, or else phase stamps (f32 input),
    // come from separate instances of the merge kernels
    hipError_t e;
    if (ws.dbg || ws.sched) e = launch_segment_merge_t<2>(sh, ws, st, rec_done);
    else if (ws.st_group != nullptr && !ws.f64) e = launch_segment_merge_t<1>(sh, ws, st, rec_done);
    else e = launch_segment_merge_t<0>(sh, ws, st, rec_done);
    if (e != hipSuccess || !ws.dbg) return e;
    const dim3 grid((unsigned)(sh.rows * kDbgParts));
    if (sh.weighted) hipLaunchKernelGGL(k_debug_root<true>, grid, dim3(256), 0, st, sh.m, ws);
    else hipLaunchKernelGGL(k_debug_root<false>, grid, dim3(256), 0, st, sh.m, ws);
    return hipGetLastError();
}

}  // namespace iso
