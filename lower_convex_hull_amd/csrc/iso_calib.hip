// Calibration front end (paper "Merge Hulls Without Copying Vertices: GPU
// Isotonic Regression", section 7.7 "Case study: calibrating a click model";
// the blog note "Isotonic Regression on GPU"'s lab notebook, calibration
// cells): scores are keyed (with segments: segment index plus the score capped
// below 1), sorted with their outcomes, equal keys pooled into count-weighted
// means, each segment's means lifted by twice its index so that no block
// crosses a segment, fitted with the counts as weights, and the lift dropped.
// A curve is applied to new scores by linear interpolation between the
// distinct keys around each score, held at the end values outside them.
//
// The sort and the pooling reduction are rocPRIM device primitives (through
// hipCUB), used as a library sort; the keys, means, lift and interpolation
// are this file's kernels, and the fit is the library's own f64 path.
#include <hipcub/hipcub.hpp>

#include "../../include/iso.h"
#include "iso_kernels.hpp"

namespace iso {
namespace {

constexpr double kCap = 1.0 - 1e-12;  // scores are capped just below 1 when keyed by segment
constexpr int kCalNT = 256;

struct SumCnt {
    double s;  // sum of outcomes
    double c;  // count
};
struct ToSumCnt {
    __host__ __device__ SumCnt operator()(double o) const { return SumCnt{o, 1.0}; }
};
struct AddSumCnt {
    __host__ __device__ SumCnt operator()(const SumCnt& a, const SumCnt& b) const {
        return SumCnt{a.s + b.s, a.c + b.c};
    }
};

__device__ __forceinline__ double calib_key(double s, const int32_t* seg, int64_t i) {
    return seg ? __dadd_rn((double)seg[i], fmin(s, kCap)) : s;
}

// Keys of the scores; bad[0] |= 1 for a non-finite score or outcome, or (with
// segments) a negative segment id or a negative score.
__global__ __launch_bounds__(kCalNT) void k_calib_keys(const double* __restrict__ s,
                                                       const double* __restrict__ o,
                                                       const int32_t* __restrict__ seg, int64_t n,
                                                       double* __restrict__ keys, int* __restrict__ bad) {
    int b = 0;
    for (int64_t i = (int64_t)blockIdx.x * kCalNT + threadIdx.x; i < n; i += (int64_t)gridDim.x * kCalNT) {
        const double x = s[i];
        if (!isfinite(x) || !isfinite(o[i])) b = 1;
        if (seg && (seg[i] < 0 || !(x >= 0.0))) b = 1;
        keys[i] = calib_key(x, seg, i);
    }
    if (__ballot(b) != 0 && (threadIdx.x & 63) == 0) atomicOr(bad, 1);
}

// Pooled means (lifted by twice the segment index) and count weights.
__global__ __launch_bounds__(kCalNT) void k_calib_means(const double* __restrict__ xp,
                                                        const SumCnt* __restrict__ sc, int64_t k, int lift,
                                                        double* __restrict__ means, double* __restrict__ wts) {
    for (int64_t i = (int64_t)blockIdx.x * kCalNT + threadIdx.x; i < k; i += (int64_t)gridDim.x * kCalNT) {
        const SumCnt v = sc[i];
        const double m = v.s / v.c;
        means[i] = lift ? __dadd_rn(m, 2.0 * floor(xp[i])) : m;
        wts[i] = v.c;
    }
}

__global__ __launch_bounds__(kCalNT) void k_calib_unlift(const double* __restrict__ xp, int64_t k,
                                                         double* __restrict__ fp) {
    for (int64_t i = (int64_t)blockIdx.x * kCalNT + threadIdx.x; i < k; i += (int64_t)gridDim.x * kCalNT)
        fp[i] = __dsub_rn(fp[i], 2.0 * floor(xp[i]));
}

// First index in [lo, hi) whose key is >= x (hi if none).
__device__ __forceinline__ int64_t lower_bound(const double* xp, int64_t lo, int64_t hi, double x) {
    while (lo < hi) {
        const int64_t mid = lo + ((hi - lo) >> 1);
        if (xp[mid] < x) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(kCalNT) void k_calib_apply(const double* __restrict__ xp,
                                                        const double* __restrict__ fp, int64_t k,
                                                        const double* __restrict__ s,
                                                        const int32_t* __restrict__ seg, int64_t m,
                                                        double* __restrict__ out) {
    for (int64_t j = (int64_t)blockIdx.x * kCalNT + threadIdx.x; j < m; j += (int64_t)gridDim.x * kCalNT) {
        const double q = calib_key(s[j], seg, j);
        int64_t lo = 0, hi = k;
        if (seg) {
            // the query's own segment: keys in [g, g + 1)
            const double g = (double)seg[j];
            lo = lower_bound(xp, 0, k, g);
            hi = lower_bound(xp, lo, k, g + 1.0);
        }
        double v;
        if (hi <= lo || !(q == q) || (seg && seg[j] < 0)) {
            v = __builtin_nan("");
        } else if (hi - lo == 1) {
            v = fp[lo];
        } else {
            int64_t i = lower_bound(xp, lo, hi, q);
            i = i < lo + 1 ? lo + 1 : (i > hi - 1 ? hi - 1 : i);
            const double a = xp[i - 1], b = xp[i];
            double t = __ddiv_rn(__dsub_rn(q, a), fmax(__dsub_rn(b, a), 1e-300));
            t = fmin(fmax(t, 0.0), 1.0);
            v = __dadd_rn(fp[i - 1], mul_rn(t, __dsub_rn(fp[i], fp[i - 1])));
        }
        out[j] = v;
    }
}

unsigned grid_for(int64_t n) {
    const int64_t g = (n + kCalNT - 1) / kCalNT;
    return (unsigned)(g < 1 ? 1 : (g > 8192 ? 8192 : g));
}

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace layout of one calibration fit of n scores.
struct CalPlan {
    size_t off_keys, off_ks, off_os, off_sc, off_means, off_wts, off_misc, off_tmp, off_fit;
    size_t tmp_bytes, fit_bytes, bytes;
};

bool cal_plan(int64_t n, CalPlan* p) {
    if (n <= 0 || n > 0x7fffffffLL) return false;
    size_t sort_tmp = 0, rbk_tmp = 0;
    const double* kd = nullptr;
    double* kod = nullptr;
    if (hipcub::DeviceRadixSort::SortPairs(nullptr, sort_tmp, kd, kod, kd, kod, (int)n) != hipSuccess) return false;
    hipcub::TransformInputIterator<SumCnt, ToSumCnt, const double*> it(kd, ToSumCnt());
    SumCnt* scd = nullptr;
    int* nr = nullptr;
    if (hipcub::DeviceReduce::ReduceByKey(nullptr, rbk_tmp, kd, kod, it, scd, nr, AddSumCnt(), (int)n) !=
        hipSuccess)
        return false;
    const size_t N = (size_t)n;
    size_t at = 0;
    auto take = [&](size_t b) {
        const size_t o = at;
        at = up256(at + b);
        return o;
    };
    p->off_keys = take(N * 8);
    p->off_ks = take(N * 8);
    p->off_os = take(N * 8);
    p->off_sc = take(N * sizeof(SumCnt));
    p->off_means = take(N * 8);
    p->off_wts = take(N * 8);
    p->off_misc = take(16);
    p->tmp_bytes = sort_tmp > rbk_tmp ? sort_tmp : rbk_tmp;
    p->off_tmp = take(p->tmp_bytes);
    p->fit_bytes = iso_workspace_bytes(1, n, ISO_F_WEIGHTED_HINT);
    p->off_fit = take(p->fit_bytes);
    p->bytes = at;
    return true;
}

template <class T>
T* at(void* base, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes) {
    if (!a || !b) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bbytes && b0 < a0 + abytes;
}

}  // namespace
}  // namespace iso

extern "C" {

size_t iso_calib_workspace_bytes(int64_t n) {
    iso::CalPlan p;
    return iso::cal_plan(n, &p) ? p.bytes : 0;
}

int iso_calib_fit(const double* scores, const double* outcomes, const int32_t* segment, int64_t n,
                  double* xp, double* fp, int64_t* k_out, void* workspace, size_t workspace_bytes,
                  void* stream) {
    using namespace iso;
    if (!k_out || n < 0) return ISO_ERR_ARG;
    *k_out = 0;
    if (n == 0) return ISO_OK;
    if (!scores || !outcomes || !xp || !fp) return ISO_ERR_ARG;
    CalPlan p;
    if (!cal_plan(n, &p)) return ISO_ERR_ARG;
    const size_t nb = (size_t)n * 8;
    const void* ins[3] = {scores, outcomes, segment};
    const size_t inb[3] = {nb, nb, (size_t)n * 4};
    for (int q = 0; q < 3; ++q)
        if (overlaps(xp, nb, ins[q], inb[q]) || overlaps(fp, nb, ins[q], inb[q])) return ISO_ERR_ARG;
    if (overlaps(xp, nb, fp, nb)) return ISO_ERR_ARG;
    if (((uintptr_t)scores | (uintptr_t)outcomes | (uintptr_t)xp | (uintptr_t)fp) & 7u) return ISO_ERR_ARG;
    if ((uintptr_t)segment & 3u) return ISO_ERR_ARG;
    if (!workspace || workspace_bytes < p.bytes) return ISO_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 255u) return ISO_ERR_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    double* keys = at<double>(workspace, p.off_keys);
    double* ks = at<double>(workspace, p.off_ks);
    double* os = at<double>(workspace, p.off_os);
    SumCnt* sc = at<SumCnt>(workspace, p.off_sc);
    double* means = at<double>(workspace, p.off_means);
    double* wts = at<double>(workspace, p.off_wts);
    int* misc = at<int>(workspace, p.off_misc);  // [0] runs, [1] bad input
    void* tmp = at<void>(workspace, p.off_tmp);
    void* fitws = at<void>(workspace, p.off_fit);

    if (hipMemsetAsync(misc, 0, 8, st) != hipSuccess) return ISO_ERR_HIP;
    hipLaunchKernelGGL(k_calib_keys, dim3(grid_for(n)), dim3(kCalNT), 0, st, scores, outcomes, segment, n,
                       keys, misc + 1);
    if (hipGetLastError() != hipSuccess) return ISO_ERR_HIP;
    size_t tb = p.tmp_bytes;
    if (hipcub::DeviceRadixSort::SortPairs(tmp, tb, keys, ks, outcomes, os, (int)n, 0, 64, st) != hipSuccess)
        return ISO_ERR_HIP;
    tb = p.tmp_bytes;
    hipcub::TransformInputIterator<SumCnt, ToSumCnt, const double*> it(os, ToSumCnt());
    if (hipcub::DeviceReduce::ReduceByKey(tmp, tb, ks, xp, it, sc, misc, AddSumCnt(), (int)n, st) != hipSuccess)
        return ISO_ERR_HIP;
    int host[2] = {0, 0};
    if (hipMemcpyAsync(host, misc, 8, hipMemcpyDeviceToHost, st) != hipSuccess) return ISO_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return ISO_ERR_HIP;
    if (host[1]) return ISO_ERR_DATA;
    const int64_t k = host[0];
    if (k < 1 || k > n) return ISO_ERR_HIP;
    const int lift = segment ? 1 : 0;
    hipLaunchKernelGGL(k_calib_means, dim3(grid_for(k)), dim3(kCalNT), 0, st, xp, sc, k, lift, means, wts);
    if (hipGetLastError() != hipSuccess) return ISO_ERR_HIP;
    const int fs = iso_fit_ex_f64(means, wts, 1, k, fp, nullptr, fitws, p.fit_bytes, stream, ISO_F_NOCHECK);
    if (fs != ISO_OK) return fs;
    if (lift) {
        hipLaunchKernelGGL(k_calib_unlift, dim3(grid_for(k)), dim3(kCalNT), 0, st, xp, k, fp);
        if (hipGetLastError() != hipSuccess) return ISO_ERR_HIP;
    }
    *k_out = k;
    return ISO_OK;
}

int iso_calib_apply(const double* xp, const double* fp, int64_t k, const double* scores,
                    const int32_t* segment, int64_t m, double* out, void* stream) {
    using namespace iso;
    if (k < 1 || m < 0) return ISO_ERR_ARG;
    if (m == 0) return ISO_OK;
    if (!xp || !fp || !scores || !out) return ISO_ERR_ARG;
    if (((uintptr_t)xp | (uintptr_t)fp | (uintptr_t)scores | (uintptr_t)out) & 7u) return ISO_ERR_ARG;
    if ((uintptr_t)segment & 3u) return ISO_ERR_ARG;
    const size_t mb = (size_t)m * 8, kb = (size_t)k * 8;
    if (overlaps(out, mb, xp, kb) || overlaps(out, mb, fp, kb) || overlaps(out, mb, scores, mb) ||
        overlaps(out, mb, segment, (size_t)m * 4))
        return ISO_ERR_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(k_calib_apply, dim3(grid_for(m)), dim3(kCalNT), 0, st, xp, fp, k, scores, segment, m,
                       out);
    return hipGetLastError() == hipSuccess ? ISO_OK : ISO_ERR_HIP;
}

}  // extern "C"
