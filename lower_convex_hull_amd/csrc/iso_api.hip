// C ABI of libiso.so: argument checks, workspace planning, launches and the
// optional data check.  Declared in include/iso.h.
#include "../../include/iso.h"

#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "iso_kernels.hpp"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Offsets of the workspace arrays.  A short-row call only needs the per-row
// flags; a long-row call lays out every array of iso::LongWs.
struct Plan {
    bool empty = true;
    bool long_rows = false;
    int m = 0;
    size_t bytes = 0;
    size_t off_row_flag = 0;
    size_t off_flag_all = 0;  // one int: the OR of the row flags, for the check
    // long rows
    size_t off_chunk_flag = 0, off_tot_S = 0, off_tot_W = 0, off_hull_cnt = 0;
    size_t off_slot_idx = 0, off_slot_S = 0, off_slot_W = 0, off_st_S = 0, off_st_W = 0, off_win = 0;
    size_t off_desc = 0, off_node_cnt = 0, off_vb = 0, off_rec = 0, off_desc_scr = 0, off_mi = 0;
    size_t off_gwin = 0, off_gtot = 0, off_cst = 0, off_gpre = 0, off_root_n = 0, off_ck_S = 0, off_ck_W = 0, off_rslope = 0;
    size_t off_stamps = 0;  // phase stamps (ISO_F_PHASE_STAMPS), at the end
    size_t off_dbg = 0;     // debug counters (ISO_F_DEBUG_INVARIANTS), after the stamps
    size_t off_cp_a = 0, off_cp_b = 0, off_cp_off = 0, off_cp_cnt = 0, off_cp_off2 = 0,
           off_cp_cnt2 = 0, off_cp_cut = 0, off_cp_cut2 = 0;
};

bool plan(int64_t rows, int64_t n, bool weighted, bool copy_control, Plan* p, bool stamps = false,
          bool debug = false) {
    *p = Plan();
    if (rows < 0 || n < 0) return false;
    if (rows == 0 || n == 0) return true;
    if (n > INT64_MAX / 64 / rows) return false;
    p->empty = false;
    size_t at = 0;
    auto take = [&](size_t bytes) {
        size_t o = at;
        at = align_up(at + bytes);
        return o;
    };
    const size_t R = (size_t)rows;
    p->off_row_flag = take(R * sizeof(int32_t));
    p->off_flag_all = take(sizeof(int32_t));
    if (n <= iso::kShortMax) {
        if (rows > 0x7fffffffLL) return false;
        p->bytes = at;
        return true;
    }
    const int64_t m64 = (n + iso::kChunk - 1) / iso::kChunk;
    if (m64 * rows > 0x7fffffffLL) return false;  // one workgroup per chunk
    p->long_rows = true;
    p->m = (int)m64;
    const size_t M = R * (size_t)m64;
    const size_t SL = M * (size_t)(iso::kChunk + 1);
    p->off_chunk_flag = take(M * sizeof(int32_t));
    p->off_tot_S = take(M * sizeof(double));
    p->off_tot_W = weighted ? take(M * sizeof(double)) : 0;
    p->off_hull_cnt = take(M * sizeof(int32_t));
    p->off_slot_idx = take(SL * sizeof(uint16_t));
    p->off_slot_S = take(SL * sizeof(double));
    p->off_slot_W = weighted ? take(SL * sizeof(double)) : 0;
    p->off_win = take(M * sizeof(iso::WinRec));
    p->off_st_S = take(M * sizeof(double));
    p->off_st_W = weighted ? take(M * sizeof(double)) : 0;
    p->off_desc = take(M * sizeof(uint2));
    p->off_node_cnt = take(M * sizeof(int32_t));
    p->off_vb = take(M * sizeof(int32_t));
    p->off_rec = take(M * sizeof(iso::ChunkRec));
    p->off_desc_scr = take(M * sizeof(uint2));
    p->off_mi = take(M * sizeof(int2));
    const size_t NG = R * (size_t)((m64 + iso::kGroup - 1) / iso::kGroup);
    p->off_gwin = take(NG * sizeof(iso::GroupWin));
    p->off_gtot = take(NG * sizeof(double2));
    p->off_cst = take(M * sizeof(double2));
    p->off_gpre = take(M * sizeof(int32_t));
    p->off_root_n = take(R * sizeof(int32_t));
    p->off_rslope = take(M * sizeof(double));
    p->off_ck_S = take(M * (iso::kLongNT + 1) * sizeof(double));
    p->off_ck_W = weighted ? take(M * (iso::kLongNT + 1) * sizeof(double)) : 0;
    if (copy_control) {
        const size_t vb = weighted ? 24 : 16;  // bytes of one flat-array vertex
        p->off_cp_a = take(SL * vb);
        p->off_cp_b = take(SL * vb);
        p->off_cp_off = take(M * sizeof(int32_t));
        p->off_cp_cnt = take(M * sizeof(int32_t));
        p->off_cp_off2 = take(M * sizeof(int32_t));
        p->off_cp_cnt2 = take(M * sizeof(int32_t));
        p->off_cp_cut = take(M * sizeof(int32_t));
        p->off_cp_cut2 = take(M * sizeof(int32_t));
    }
    if (stamps) p->off_stamps = take((2 * M + NG + R) * iso::kStampSlots * sizeof(uint64_t));
    if (debug) p->off_dbg = take(iso::kDbgCount * sizeof(uint64_t));
    p->bytes = at;
    return true;
}

template <class T>
T* at(void* base, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

iso::LongWs long_ws(void* base, const Plan& p, bool weighted, bool copy_control, int64_t rows) {
    iso::LongWs ws{};
    if (p.off_stamps) {
        const int64_t M = rows * p.m, NG = rows * ((p.m + iso::kGroup - 1) / iso::kGroup);
        uint64_t* s0 = at<uint64_t>(base, p.off_stamps);
        ws.st_chunk = s0;
        ws.st_group = s0 + M * iso::kStampSlots;
        ws.st_top = ws.st_group + NG * iso::kStampSlots;
        ws.st_expand = ws.st_top + rows * iso::kStampSlots;
    }
    if (p.off_dbg) ws.dbg = at<unsigned long long>(base, p.off_dbg);
    ws.chunk_flag = at<int32_t>(base, p.off_chunk_flag);
    ws.tot_S = at<double>(base, p.off_tot_S);
    ws.tot_W = weighted ? at<double>(base, p.off_tot_W) : nullptr;
    ws.hull_cnt = at<int32_t>(base, p.off_hull_cnt);
    ws.slot_idx = at<uint16_t>(base, p.off_slot_idx);
    ws.slot_S = at<double>(base, p.off_slot_S);
    ws.slot_W = weighted ? at<double>(base, p.off_slot_W) : nullptr;
    ws.win = at<iso::WinRec>(base, p.off_win);
    ws.st_S = at<double>(base, p.off_st_S);
    ws.st_W = weighted ? at<double>(base, p.off_st_W) : nullptr;
    ws.desc = at<uint2>(base, p.off_desc);
    ws.node_cnt = at<int32_t>(base, p.off_node_cnt);
    ws.vb = at<int32_t>(base, p.off_vb);
    ws.rec = at<iso::ChunkRec>(base, p.off_rec);
    ws.desc_scr = at<uint2>(base, p.off_desc_scr);
    ws.gwin = at<iso::GroupWin>(base, p.off_gwin);
    ws.gtot = at<double2>(base, p.off_gtot);
    ws.cst = at<double2>(base, p.off_cst);
    ws.gpre = at<int32_t>(base, p.off_gpre);
    ws.root_n = at<int32_t>(base, p.off_root_n);
    ws.rslope = at<double>(base, p.off_rslope);
    ws.ck_S = at<double>(base, p.off_ck_S);
    ws.ck_W = weighted ? at<double>(base, p.off_ck_W) : nullptr;
    ws.merge_info = at<int2>(base, p.off_mi);
    ws.row_flag = at<int32_t>(base, p.off_row_flag);
    if (copy_control) {
        ws.cp_a = at<char>(base, p.off_cp_a);
        ws.cp_b = at<char>(base, p.off_cp_b);
        ws.cp_off = at<int32_t>(base, p.off_cp_off);
        ws.cp_cnt = at<int32_t>(base, p.off_cp_cnt);
        ws.cp_off2 = at<int32_t>(base, p.off_cp_off2);
        ws.cp_cnt2 = at<int32_t>(base, p.off_cp_cnt2);
        ws.cp_cut = at<int32_t>(base, p.off_cp_cut);
        ws.cp_cut2 = at<int32_t>(base, p.off_cp_cut2);
    }
    return ws;
}

bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes) {
    if (!a || !b) return false;
    uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bbytes && b0 < a0 + abytes;
}

constexpr uint32_t kKnownFlags = ISO_F_NOCHECK | ISO_F_DECREASING | ISO_F_COPY_CONTROL |
                                  ISO_F_DEBUG_INVARIANTS | ISO_F_WEIGHTED_HINT | ISO_F_PHASE_STAMPS |
                                  ISO_F_WAVE_MERGES | ISO_F_THREE_CASE | ISO_F_TREE_MERGES;

// Launch timing (benchmarks only).
struct Timing {
    std::mutex mu;
    bool on = false;
    struct Rec {
        int phase;
        hipEvent_t a, b;
    };
    std::vector<Rec> recs;
    int open = -1;  // index of the record awaiting its end event
};
Timing& timing() {
    static Timing t;
    return t;
}

// Per-device cached workspace of iso_fit.
struct Cache {
    std::mutex mu;
    std::vector<void*> ptr;
    std::vector<size_t> bytes;
};
Cache& cache() {
    static Cache c;
    return c;
}

// The fit on `stream` with `workspace`: argument checks, launches, and (without
// ISO_F_NOCHECK) the data check.  Allocates nothing, on the device or the host.
// T is the element type of y, w and out (float or double).
template <typename T>
int fit_body(const T* y, const T* w, int64_t rows, int64_t n, T* out, int32_t* block_id,
             void* workspace, size_t workspace_bytes, void* stream, uint32_t flags) {
    if (!y || !out || rows < 0 || n < 0 || (flags & ~kKnownFlags)) return ISO_ERR_ARG;
    if (rows == 0 || n == 0) return ISO_OK;
    const bool weighted = w != nullptr;
    const bool copy_control = (flags & ISO_F_COPY_CONTROL) != 0;
    Plan p;
    if (!plan(rows, n, weighted, copy_control, &p, (flags & ISO_F_PHASE_STAMPS) != 0,
              (flags & ISO_F_DEBUG_INVARIANTS) != 0))
        return ISO_ERR_ARG;
    const size_t nb = (size_t)rows * (size_t)n * sizeof(T);
    const size_t ib = (size_t)rows * (size_t)n * sizeof(int32_t);
    if (overlaps(out, nb, y, nb) || overlaps(out, nb, w, nb) || overlaps(block_id, ib, y, nb) ||
        overlaps(block_id, ib, w, nb) || overlaps(block_id, ib, out, nb))
        return ISO_ERR_ARG;
    if (((uintptr_t)y | (uintptr_t)out | (uintptr_t)w) & (sizeof(T) - 1)) return ISO_ERR_ARG;
    if ((uintptr_t)block_id & 3u) return ISO_ERR_ARG;
    if (!workspace || workspace_bytes < p.bytes) return ISO_ERR_WORKSPACE;
    if ((uintptr_t)workspace % kAlign) return ISO_ERR_ARG;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const float sign = (flags & ISO_F_DECREASING) ? -1.0f : 1.0f;
    int32_t* row_flag = at<int32_t>(workspace, p.off_row_flag);
    hipError_t e;
    if (!p.long_rows) {
        e = iso::launch_short<T>(y, w, rows, n, sign, out, block_id, row_flag, st);
    } else {
        iso::LongShape sh{rows, n, p.m, weighted, sign};
        iso::LongWs ws = long_ws(workspace, p, weighted, copy_control, rows);
        ws.sched = ((flags & ISO_F_WAVE_MERGES) ? iso::kSchedWaveAll : 0) |
                   ((flags & ISO_F_THREE_CASE) ? iso::kSchedThreeCase : 0) |
                   ((flags & ISO_F_TREE_MERGES) ? iso::kSchedTreeTop : 0);
        e = iso::launch_long<T>(y, w, sh, ws, out, block_id, copy_control, st);
    }
    if (e != hipSuccess) return ISO_ERR_HIP;
    if (flags & ISO_F_NOCHECK) return ISO_OK;

    int32_t* all = at<int32_t>(workspace, p.off_flag_all);
    if (iso::launch_flags_or(row_flag, rows, all, st) != hipSuccess) return ISO_ERR_HIP;
    int32_t any = 0;
    if (hipMemcpyAsync(&any, all, sizeof(any), hipMemcpyDeviceToHost, st) != hipSuccess)
        return ISO_ERR_HIP;
    unsigned long long viol = 0;
    if (p.long_rows && p.off_dbg &&
        hipMemcpyAsync(&viol, at<unsigned long long>(workspace, p.off_dbg) + iso::kDbgViolations,
                       sizeof(viol), hipMemcpyDeviceToHost, st) != hipSuccess)
        return ISO_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return ISO_ERR_HIP;
    if (viol) return ISO_ERR_INVARIANT;
    if (any & iso::kFlagWeight) return ISO_ERR_WEIGHT;
    if (any & iso::kFlagNonfinite) return ISO_WARN_NONFINITE;
    return ISO_OK;
}

}  // namespace

// The no-alloc entry point's workspace: a device array of ISO_NOALLOC_BYTES
// that every GPU the library runs on holds until the process ends.  Its name
// is not a device address in host code: the address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[ISO_NOALLOC_BYTES];

namespace {

struct ScratchTable {
    std::mutex mu;
    void* ptr[64] = {};
};
ScratchTable& scratch_table() {
    static ScratchTable t;
    return t;
}

// Device address of `scratch` on the current device (set up on the first call
// on each device), or nullptr on a HIP error.
void* scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    ScratchTable& t = scratch_table();
    std::lock_guard<std::mutex> lock(t.mu);
    if (!t.ptr[dev]) {
        void* q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
        t.ptr[dev] = q;
    }
    return t.ptr[dev];
}

// The blocking fit with the per-device cached workspace (iso_fit, iso_fit_f64).
template <typename T>
int cached_fit(const T* y, const T* w, int64_t rows, int64_t n, T* out) {
    if (!y || !out || rows < 0 || n < 0) return ISO_ERR_ARG;
    if (rows == 0 || n == 0) return ISO_OK;
    Plan p;
    if (!plan(rows, n, w != nullptr, false, &p)) return ISO_ERR_ARG;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return ISO_ERR_HIP;
    Cache& c = cache();
    std::lock_guard<std::mutex> lock(c.mu);
    if ((size_t)dev >= c.ptr.size()) {
        c.ptr.resize(dev + 1, nullptr);
        c.bytes.resize(dev + 1, 0);
    }
    if (c.bytes[dev] < p.bytes) {
        if (c.ptr[dev]) (void)hipFree(c.ptr[dev]);
        c.ptr[dev] = nullptr;
        c.bytes[dev] = 0;
        void* q = nullptr;
        if (hipMalloc(&q, p.bytes) != hipSuccess) {
            // A failed hipMalloc also sets the thread's last-error state; clear it so the
            // caller's next launch check does not report this failure a second time.
            (void)hipGetLastError();
            return ISO_ERR_NOMEM;
        }
        c.ptr[dev] = q;
        c.bytes[dev] = p.bytes;
    }
    return fit_body<T>(y, w, rows, n, out, nullptr, c.ptr[dev], c.bytes[dev], nullptr, 0u);
}

}  // namespace

namespace iso {

void timed_begin(int phase, hipStream_t st) {
    Timing& t = timing();
    std::lock_guard<std::mutex> lock(t.mu);
    if (!t.on) return;
    Timing::Rec r{phase, nullptr, nullptr};
    if (hipEventCreate(&r.a) != hipSuccess) return;
    if (hipEventCreate(&r.b) != hipSuccess) {
        (void)hipEventDestroy(r.a);
        return;
    }
    (void)hipEventRecord(r.a, st);
    t.recs.push_back(r);
    t.open = (int)t.recs.size() - 1;
}

void timed_end(hipStream_t st) {
    Timing& t = timing();
    std::lock_guard<std::mutex> lock(t.mu);
    if (!t.on || t.open < 0) return;
    (void)hipEventRecord(t.recs[t.open].b, st);
    t.open = -1;
}

}  // namespace iso

extern "C" {

int iso_copy_probe(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst || bytes % 16 || (((uintptr_t)src | (uintptr_t)dst) & 15u)) return ISO_ERR_ARG;
    if (overlaps(src, bytes, dst, bytes)) return ISO_ERR_ARG;
    if (bytes == 0) return ISO_OK;
    return iso::launch_copy_probe(src, dst, bytes, static_cast<hipStream_t>(stream)) == hipSuccess
               ? ISO_OK
               : ISO_ERR_HIP;
}

int iso_timing_enable(int on) {
    Timing& t = timing();
    std::lock_guard<std::mutex> lock(t.mu);
    t.on = on != 0;
    return ISO_OK;
}

int iso_timing_read(double* ms, int64_t* launches, int nphase) {
    Timing& t = timing();
    std::lock_guard<std::mutex> lock(t.mu);
    int status = 0;
    int count = 0;
    for (auto& r : t.recs) {
        float e = 0.0f;
        if (status == 0) {
            if (hipEventSynchronize(r.b) != hipSuccess ||
                hipEventElapsedTime(&e, r.a, r.b) != hipSuccess)
                status = ISO_ERR_HIP;
        }
        if (status == 0 && r.phase >= 0 && r.phase < nphase) {
            if (ms) ms[r.phase] += e;
            if (launches) launches[r.phase] += 1;
            ++count;
        }
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    t.recs.clear();
    t.open = -1;
    return status ? status : count;
}


const char* iso_status_str(int status) {
    switch (status) {
        case ISO_OK: return "ok";
        case ISO_WARN_NONFINITE: return "some rows hold non-finite values; their fit is NaN";
        case ISO_ERR_ARG: return "invalid argument";
        case ISO_ERR_WEIGHT: return "a weight is not positive and finite";
        case ISO_ERR_NOMEM: return "device workspace allocation failed";
        case ISO_ERR_HIP: return "HIP runtime error";
        case ISO_ERR_WORKSPACE: return "workspace too small";
        case ISO_ERR_DATA: return "non-finite score or outcome, or a negative score or segment";
        case ISO_ERR_INVARIANT: return "a segment-list invariant of the merge was violated (debug check)";
        default: return "unknown status";
    }
}

int64_t iso_chunk_size(int64_t n) { return n <= iso::kShortMax ? n : iso::kChunk; }
int64_t iso_short_row_max(void) { return iso::kShortMax; }

size_t iso_workspace_bytes(int64_t rows, int64_t n, uint32_t flags) {
    Plan p;
    if (!plan(rows, n, (flags & ISO_F_WEIGHTED_HINT) != 0, (flags & ISO_F_COPY_CONTROL) != 0, &p,
              (flags & ISO_F_PHASE_STAMPS) != 0, (flags & ISO_F_DEBUG_INVARIANTS) != 0))
        return 0;
    return p.bytes;
}

int iso_fit_ex(const float* y, const float* w, int64_t rows, int64_t n, float* out,
               int32_t* block_id, void* workspace, size_t workspace_bytes, void* stream,
               uint32_t flags) {
    return fit_body<float>(y, w, rows, n, out, block_id, workspace, workspace_bytes, stream, flags);
}

int iso_fit_ex_f64(const double* y, const double* w, int64_t rows, int64_t n, double* out,
                   int32_t* block_id, void* workspace, size_t workspace_bytes, void* stream,
                   uint32_t flags) {
    return fit_body<double>(y, w, rows, n, out, block_id, workspace, workspace_bytes, stream, flags);
}

int iso_fit_noalloc(const float* y, const float* w, int64_t rows, int64_t n, float* out,
                    int32_t* block_id, void* stream, uint32_t flags) {
    if (!y || !out || rows < 0 || n < 0 || (flags & ~kKnownFlags)) return ISO_ERR_ARG;
    if (rows == 0 || n == 0) return ISO_OK;
    Plan p;
    if (!plan(rows, n, w != nullptr, (flags & ISO_F_COPY_CONTROL) != 0, &p)) return ISO_ERR_ARG;
    if (p.bytes > (size_t)ISO_NOALLOC_BYTES) return ISO_ERR_WORKSPACE;
    void* ws = scratch_ptr();
    if (!ws) return ISO_ERR_HIP;
    return fit_body<float>(y, w, rows, n, out, block_id, ws, (size_t)ISO_NOALLOC_BYTES, stream, flags);
}

int iso_fit(const float* y, const float* w, int64_t rows, int64_t n, float* out) {
    return cached_fit<float>(y, w, rows, n, out);
}

int iso_fit_f64(const double* y, const double* w, int64_t rows, int64_t n, double* out) {
    return cached_fit<double>(y, w, rows, n, out);
}

void iso_release(void) {
    Cache& c = cache();
    std::lock_guard<std::mutex> lock(c.mu);
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (size_t d = 0; d < c.ptr.size(); ++d) {
        if (c.ptr[d]) {
            (void)hipSetDevice((int)d);
            (void)hipFree(c.ptr[d]);
        }
        c.ptr[d] = nullptr;
        c.bytes[d] = 0;
    }
    (void)hipSetDevice(cur);
}

}  // extern "C"
