// Internal interface between the C ABI (iso_api.hip) and the gfx950 kernels
// (iso_kernels.hip).  Not installed; nothing outside libiso.so includes it.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace iso {

// An f64 product rounded on its own: the compiler may not fuse it with a
// neighbouring addition into a multiply-add (HIP's __dmul_rn is a plain
// product, which it may fuse).  Cross products built from two of these give
// exactly zero whenever the two products are equal.
__device__ __forceinline__ double mul_rn(double a, double b) {
#pragma clang fp contract(off)
    return a * b;
}

// Long rows are cut into chunks of kChunk points, one 256-thread workgroup
// each (16 points per thread).  Rows up to kShortMax elements are fitted whole
// by one workgroup and never touch the workspace.
constexpr int kLongNT = 256;
constexpr int kLongP = 16;
constexpr int kChunk = kLongNT * kLongP;  // 4096
constexpr int kShortMax = 4096;
constexpr int kQhMax = 64;          // vertices of a block hull built by quickhull
constexpr int kQhWaveCap = 576;     // room per wave for the live points after quickhull's first level (chunk kernel)
constexpr int kQhWaveCapW = 512;    // the same, weighted (four workgroups per CU fit the LDS)
constexpr int kQhLevels = 10;       // quickhull levels before the chains-and-merges fallback
constexpr int kRedoGrid = 768;      // workgroups of the fallback chunk kernel (3 per CU)
constexpr int kExpTile = 512;       // surviving vertices of a chunk the expansion keeps in LDS
constexpr int kExpNT = 128;        // threads of an expansion workgroup (one chunk, 32 elements each)
constexpr int kMergeNT = 1024;
constexpr int kWinK = 16;           // hull vertices kept at each end of a chunk's window
constexpr int kGWinK = 32;          // the same for a group hull's window
constexpr int kGroup = 64;          // chunks per group of the first merge stage
constexpr int kGroupNT = 1024;
constexpr int kTopNT = 1024;
constexpr int kTopMax = 72;         // groups per row the second stage keeps in LDS
constexpr int kTopFastMax = 72;     // groups per row for the second stage's compact-array path
constexpr int kWalkCap = 64;      // thread-walk steps before a merge is handed to a wave
constexpr int kWaveWalkCap = 64;  // wave-walk steps (63 vertices each) before bisection
constexpr int kHardCap = 256;     // merges per level a wave may take over

// Merge schedule variants (the paper's appendix A and section 7.4; measurement
// and stress only): every merge of a segment-list level by a wave, instead of
// a thread per merge with long walks handed to waves; or, at the levels run
// with a thread per merge, walks capped at 8 (r + log2 C) steps followed by
// the three-case bridge search instead of handing the merge to a wave.
constexpr int kSchedWaveAll = 1;
constexpr int kSchedThreeCase = 2;
// The second stage's compact-array merge by the merge tree instead of the
// bridges between neighbouring groups (measurement and stress only).
constexpr int kSchedTreeTop = 4;

// Debug counters (ISO_F_DEBUG_INVARIANTS), 8 x uint64 at the end of the workspace.
constexpr int kDbgViolations = 0;   // segment-list invariants found broken
constexpr int kDbgRebuilt = 1;      // chunk hulls rebuilt after the chunk kernel gave up
constexpr int kDbgToWave = 2;       // thread walks that reached their cap and went to a wave
constexpr int kDbgBisect = 3;       // nested bisections (walks beyond every cap)
constexpr int kDbgThreeCase = 4;    // three-case bridge searches
constexpr int kDbgLevels = 5;       // segment-list merge levels checked
constexpr int kDbgRootVerts = 6;    // root vertices checked for convexity
constexpr int kDbgLocalRounds = 7;  // rounds of the local-bridge merge that dropped groups
constexpr int kDbgCount = 8;

// Phase stamps per workgroup (ISO_F_PHASE_STAMPS).
constexpr int kStampSlots = 16;

// Per-row data flags written by the kernels (read back by the checking path).
constexpr int kFlagNonfinite = 1;
constexpr int kFlagWeight = 2;
constexpr int kFlagData = kFlagNonfinite | kFlagWeight;
// Chunk flag: the chunk's elements strictly increase, so every point is a
// hull vertex (position = point index) and the chunk's slot is not written;
// its points are recomputed from the input and the per-thread checkpoints.
constexpr int kChunkInc = 4;
// Chunk flag: the chunk kernel gave up on this chunk's hull (its window header
// then holds h = 0); the first merge stage or the fallback kernel rebuilds it.
constexpr int kChunkRedo = 8;

// Reconstruction record of one chunk, written by the merge phase.
//   lo < 0: no vertex of the row's hull lies in the chunk; every element of
//           the chunk lies under one edge of slope `slope_in`.
//   else:   the chunk's surviving hull vertices are its slot positions lo..hi;
//           slope_in is the edge into lo, slope_out the edge out of hi.
//   vb:     number of row-hull vertices in earlier chunks' segments (for the
//           block ids).
struct ChunkRec {
    int32_t lo;
    int32_t hi;
    int32_t vb;
    int32_t pad;
    double slope_in;
    double slope_out;
};

// A chunk hull's two ends in one compact record: its vertex count h and the
// chunk-relative (S, W) of its first kWinK and last kWinK vertices (all of them
// when h <= 2 kWinK).  The merge tree reads vertices here; only walks that
// reach the middle of a long chunk hull read the full slot.
struct WinRec {
    int32_t h;
    int32_t pad[3];
    double2 v[2 * kWinK];
};

// The same for the hull of a group of kGroup chunks (first merge stage): its
// vertex count, the number of segments in its list, its data flags, the (S, W) of its first
// and last kGWinK vertices relative to the group's first point, and for each
// of those the chunk and the position in that chunk's hull (packed by mktag).
struct GroupWin {
    int32_t h;
    int32_t nseg;
    int32_t flags;  // the group's data flags (kFlagData bits of its chunks)
    int32_t pre1;   // vertices in the first segment of the group's list
    double2 v[2 * kGWinK];
    int32_t tag[2 * kGWinK];
};

// A vertex's chunk and its position in that chunk's hull, in one int32.
constexpr int kTagShift = 13;  // positions 0..kChunk need 13 bits
constexpr int kTagMaxChunks = 1 << (31 - kTagShift);

// Device pointers of the long-row workspace (see plan_long in iso_api.hip).
struct LongWs {
    int32_t* chunk_flag;  // [R*m]
    double* tot_S;        // [R*m] chunk totals
    double* tot_W;        // [R*m] (weighted only)
    int32_t* hull_cnt;    // [R*m] vertices in each chunk hull
    uint16_t* slot_idx;   // [R*m*(C+1)] chunk-relative point index of each vertex
    double* slot_S;       // [R*m*(C+1)] chunk-relative S of each vertex
    double* slot_W;       // [R*m*(C+1)] chunk-relative W (weighted only)
    WinRec* win;          // [R*m] ends of each chunk hull
    double* st_S;         // [R*m] chunk starts (exclusive scan of totals)
    double* st_W;         // [R*m] (weighted only)
    uint2* desc;          // [R*m] segment descriptors (chunk, lo | hi << 16)
    int32_t* node_cnt;    // [R*m] segments in the list stored from this slot
    int32_t* vb;          // [R*m] scratch: vertex prefix over the root list
    uint2* desc_scr;      // [R*m] scratch for descriptor moves; the two-stage merge's root list
    GroupWin* gwin;       // [R*ng] group hull ends (ng = groups per row)
    double2* gtot;        // [R*ng] group totals (S, W)
    double2* cst;         // [R*m] chunk starts relative to their group's start
    int32_t* gpre;        // [R*m] vertices before each segment of a group's list
    int32_t* root_n;      // [R] segments in the root list (desc_scr) of each row
    double* rslope;       // [R*m] slope of the root edge into each root segment (from the previous one)
    double* ck_S;         // [R*m*(kLongNT+1)] S at each thread's first point (and the chunk end)
    double* ck_W;         // (weighted only)
    // the call's inputs, for points recomputed from them and chunks rebuilt
    const void* y;
    const void* w;
    int64_t n;
    float sign;
    int f64;              // y and w are f64 (else f32)
    int2* merge_info;     // [R*m] per merge: kept segments of L, first kept segment of R
    ChunkRec* rec;        // [R*m]
    int32_t* row_flag;    // [R]
    // merge schedule variants (kSched* bits; 0 = the default schedule)
    int sched;
    // debug counters (null unless ISO_F_DEBUG_INVARIANTS), kDbg* indices
    unsigned long long* dbg;
    // phase stamps (measurement only, null unless ISO_F_PHASE_STAMPS): per
    // workgroup kStampSlots 100 MHz real-time counter values
    uint64_t* st_chunk;   // [R*m]  chunk kernel
    uint64_t* st_group;   // [R*ng] first merge stage
    uint64_t* st_top;     // [R]    second merge stage (or the row merge)
    uint64_t* st_expand;  // [R*m]  expansion
    // grid-copy control only
    void* cp_a;           // [R*m*(C+1)] flat vertex buffers (ping), 16 B (24 B weighted) each
    void* cp_b;           // (pong)
    int32_t* cp_off;      // [R*m] node offsets (ping)
    int32_t* cp_cnt;      // [R*m] node vertex counts (ping)
    int32_t* cp_off2;     // [R*m] (pong)
    int32_t* cp_cnt2;     // [R*m]
    int32_t* cp_cut;      // [R*m] per merge: kept prefix of L (count) and start of R
    int32_t* cp_cut2;     // [R*m]
};

struct LongShape {
    int64_t rows;
    int64_t n;
    int m;         // chunks per row
    bool weighted;
    float sign;    // +1 increasing, -1 decreasing
};

// Phases of the launch timing (the ISO_PHASE_* values of iso.h).
constexpr int kPhaseShort = 0, kPhaseChunk = 1, kPhaseMerge = 2, kPhaseExpand = 3,
              kPhaseCopyBridge = 4, kPhaseCopyMove = 5, kPhaseMergeTop = 6, kPhaseChunkRedo = 7;

// Launch timing for benchmarks (iso_timing_enable / iso_timing_read): when
// enabled, timed_begin records an event before a launch and timed_end one
// after it, on the launch's stream.
void timed_begin(int phase, hipStream_t st);
void timed_end(hipStream_t st);

// The fit of rows of at most kShortMax elements (T = float or double).
template <typename T>
hipError_t launch_short(const T* y, const T* w, int64_t rows, int64_t n, float sign, T* out,
                        int32_t* block_id, int32_t* row_flag, hipStream_t st);

// The bandwidth probe: copies `bytes` (a multiple of 16, 16-byte aligned).
hipError_t launch_copy_probe(const void* src, void* dst, size_t bytes, hipStream_t st);

// ORs the rows' data flags into *dst (one int) on the device, for the check.
hipError_t launch_flags_or(const int32_t* row_flag, int64_t rows, int32_t* dst, hipStream_t st);

// The merge phase over segment lists (iso_merge.hip).  Leaves either the
// reconstruction records in ws.rec (*rec_done = true) or each row's root list
// in ws.desc_scr with its prefix counts, from which the expansion computes
// the records (*rec_done = false).
hipError_t launch_segment_merge(const LongShape& sh, const LongWs& ws, hipStream_t st, bool* rec_done);

// The merge phase of the vertex-copying control (iso_copy.hip); leaves the
// reconstruction records in ws.rec like the segment-list merge.
hipError_t launch_copy_merge(const LongShape& sh, const LongWs& ws, hipStream_t st);

// Clears the debug counters (a fill kernel, so that a captured graph may hold it).
hipError_t launch_zero_u64(unsigned long long* p, int n, hipStream_t st);

// Whether rows of m chunks take the two-stage merge (k_group_merge, then
// k_top_merge when there is more than one group); longer rows take
// k_group_merge, then k_merge_rows.
inline bool two_stage_merge(int m) { return (m + kGroup - 1) / kGroup <= kTopMax; }

// The fit of long rows: chunk hulls, merge, expansion (T = float or double).
template <typename T>
hipError_t launch_long(const T* y, const T* w, const LongShape& sh, const LongWs& ws, T* out,
                       int32_t* block_id, bool copy_control, hipStream_t st);

}  // namespace iso
