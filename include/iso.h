/*
 * iso.h - C ABI of the MI355X (gfx950) batched weighted isotonic-regression
 * library, libiso.so.
 *
 * The operation (paper "Merge Hulls Without Copying Vertices: GPU Isotonic
 * Regression", section 2.1, equations (1)-(3)): for every row y[0..n) with
 * weights w[0..n) > 0, compute the weighted least-squares non-decreasing fit
 *
 *     z* = argmin_{z_0 <= ... <= z_{n-1}}  sum_i w_i (z_i - y_i)^2 ,
 *
 * as the slope sequence of the lower convex hull of the cumulative sum diagram
 * P_k = (W_k, S_k), W_k = sum_{i<k} w_i, S_k = sum_{i<k} w_i y_i, P_0 = (0, 0):
 * z*_i is the slope of the hull edge above [W_i, W_{i+1}].  Rows are
 * independent problems of one common length (paper section 3, first paragraph;
 * rectangular batches only, section 6).
 *
 * Conventions shared by every entry point
 *   - y, w, out, block_id are DEVICE pointers (hipMalloc'd or torch CUDA
 *     tensors), row-major and contiguous: element (r, i) is at r*n + i.  They
 *     are caller-owned; the library never frees or retains them.
 *   - y, w, out are float32 and must be 4-byte aligned (the _f64 entry points:
 *     float64, 8-byte aligned); block_id is int32.
 *   - w == NULL means unit weights.
 *   - The fit is accumulated in f64 and each output value is rounded once to
 *     the output type (round to nearest even), as the paper's section 6
 *     ("Output") asks.  The output is not forced to be monotone (same
 *     section).
 *   - block_id (optional, NULL = not written): for each element, the 0-based
 *     index of its block (hull edge) within its row; non-decreasing along the
 *     row, +1 at every block start.  The paper's one-byte block-start flag
 *     (section 6, "Gradient") is block_id[i] != block_id[i-1].  Where adjacent
 *     blocks have equal means the library may split or pool them (a point on
 *     a hull edge changes no slope, section 4, after Corollary 4.5).
 *
 * Errors (return value; also see iso_status_str)
 *   ISO_OK               success.
 *   ISO_WARN_NONFINITE   some rows hold a NaN or infinity in y: those rows'
 *                        out is NaN and their block_id is -1; other rows are
 *                        exact.  (The paper keeps per-row NaN flags, section 6.)
 *   ISO_ERR_ARG          a NULL y or out, rows < 0 or n < 0, rows*n too large,
 *                        an output overlapping an input, or bad flags.
 *                        Nothing is launched.
 *   ISO_ERR_WEIGHT       some w_i <= 0 or non-finite (the problem needs
 *                        w_i > 0, section 2.1).  out is unspecified.
 *   ISO_ERR_NOMEM        iso_fit could not allocate its cached workspace.
 *                        Nothing launched; the HIP runtime's last-error
 *                        state that the failed hipMalloc set is cleared.
 *   ISO_ERR_HIP          a HIP runtime call or kernel launch failed.
 *   ISO_ERR_WORKSPACE    iso_fit_ex got a workspace smaller than
 *                        iso_workspace_bytes() asks for, or the shape needs
 *                        more than iso_fit_noalloc's ISO_NOALLOC_BYTES.
 *                        Nothing launched.
 *   ISO_ERR_DATA         iso_calib_fit got a non-finite score or outcome, or
 *                        (with segments) a negative score or segment id.
 *   ISO_ERR_INVARIANT    (ISO_F_DEBUG_INVARIANTS) a segment list of the merge
 *                        broke Definition 4.3 / Theorem 4.4 or the root
 *                        chain was not convex.
 *   rows == 0 or n == 0 is a no-op that returns ISO_OK.
 *
 * The two warning/error statuses that depend on the data (NONFINITE, WEIGHT)
 * are only reported when the call checks: iso_fit always does; iso_fit_ex
 * does unless ISO_F_NOCHECK is set (then it only enqueues work and returns
 * ISO_OK; NaN rows still come out NaN).
 */
#ifndef ISO_H
#define ISO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    ISO_OK = 0,
    ISO_WARN_NONFINITE = 1,
    ISO_ERR_ARG = -1,
    ISO_ERR_WEIGHT = -2,
    ISO_ERR_NOMEM = -3,
    ISO_ERR_HIP = -4,
    ISO_ERR_WORKSPACE = -5,
    ISO_ERR_DATA = -6,
    ISO_ERR_INVARIANT = -7
};

enum {
    /* Enqueue only: no device-to-host wait for the data checks. */
    ISO_F_NOCHECK = 1u,
    /* Non-increasing fit instead: the increasing fit of -y, negated (paper
     * section 2.1: the decreasing problem is the increasing one for -y). */
    ISO_F_DECREASING = 2u,
    /* Measurement control: merge the chunk hulls of long rows by copying the
     * surviving vertices at every level of the merge tree (the paper's
     * "grid copy" control, sections 7.3-7.4) instead of segment lists.  Same
     * result; more memory traffic.  Needs the larger workspace that
     * iso_workspace_bytes reports for this flag. */
    ISO_F_COPY_CONTROL = 4u,
    /* Tests: check the merge's segment lists on the device (paper section 4,
     * Definition 4.3, Theorem 4.4): after every segment-list merge level, each
     * list holds at most one segment per chunk of its range, in strictly
     * increasing chunk order, with lo <= hi; each row's root list starts at
     * the row's first point, ends at its last, keeps every segment inside its
     * chunk hull, and its vertices form a convex chain (no right turn beyond
     * rounding).  Also counts which merge paths ran.  The counters, 8 uint64,
     * sit at the end of the workspace (pass the flag to iso_workspace_bytes),
     * after any phase stamps: [0] violations, [1] chunk hulls rebuilt after
     * the chunk kernel gave up, [2] thread walks handed to a wave, [3] nested
     * bisections, [4] three-case searches, [5] levels checked, [6] root
     * vertices checked, [7] rounds of the second stage's bridges between
     * neighbouring groups that dropped a group.  A checked call returns
     * ISO_ERR_INVARIANT when [0] is not zero.  Long rows only; slower. */
    ISO_F_DEBUG_INVARIANTS = 8u,
    /* For iso_workspace_bytes only: size the workspace for a weighted call
     * (w != NULL).  Ignored by the fitting calls. */
    ISO_F_WEIGHTED_HINT = 0x100u,
    /* Measurement: on long rows, thread 0 of every workgroup of the chunk,
     * first-merge-stage, second-merge-stage and expansion kernels records the
     * device's 100 MHz real-time counter at its phase boundaries.  The stamps
     * take 64 bytes per workgroup at the end of the workspace (pass the flag to
     * iso_workspace_bytes too), from byte iso_workspace_bytes(rows, n, flags
     * without this bit) on: rows*m rows of 16 uint64 for the chunk kernel, then
     * rows*ng for the first merge stage (ng = ceil(m / 64)), rows for the
     * second stage, rows*m for the expansion (m = ceil(n / iso_chunk_size(n))).
     * Slots: chunk 0 start, 1 loads/sums/scan, 5 first quickhull level, 2 hull
     * built, 4 end; merge stages 0 start, 1 prelude, 2 merge tree, 3 lists and
     * windows written, 4 end, 5 + l node 0 through level l of a compact
     * merge tree; expansion 0 start, 1 record ready, 4 end.  Rows beyond the
 * two-stage merge use the second-stage row for the row merge: 0 start, 1
 * prelude done, 3 start of the levels left to one workgroup, 5 + (r - 6)
 * through tree level r, 2 tree done, 4 end. */
    ISO_F_PHASE_STAMPS = 0x200u,
    /* Merge-schedule variants (measurement and stress; paper section 7.4 and
     * appendix A).  Same result.  WAVE_MERGES: every merge of a segment-list
     * level is run by a wave (default: a thread per merge when a level has more
     * merges than the workgroup has waves, with walks that reach their cap
     * handed to waves).  THREE_CASE: at the levels with a thread per merge,
     * walks are capped at 8 (r + log2 C) steps (r the tree level, C the chunk
     * size) and finished by the three-case bridge search of Lemma A.1.  The
     * compact-array merges of short hulls are not affected.  TREE_MERGES: the
     * second stage merges short group hulls by the merge tree (default: the
     * bridges between neighbouring groups, all at once, with groups that keep
     * no vertex dropped round by round, and the tree after 8 such rounds). */
    ISO_F_WAVE_MERGES = 0x400u,
    ISO_F_THREE_CASE = 0x800u,
    ISO_F_TREE_MERGES = 0x1000u
};

/*
 * iso_fit - blocking fit on the null stream of the current device.
 *   y    [rows*n] f32, device.          w   [rows*n] f32 or NULL, device.
 *   out  [rows*n] f32, device, written.  May not overlap y or w.
 * Uses a workspace the library allocates once per device and grows on demand
 * (freed by iso_release).  Waits for the GPU and always runs the data checks.
 * Not safe to call concurrently from several host threads on one device.
 */
int iso_fit(const float* y, const float* w, int64_t rows, int64_t n, float* out);

/*
 * iso_fit_ex - the fit on a caller stream with a caller workspace.
 *   block_id        [rows*n] int32, device, or NULL.
 *   workspace       device buffer of at least iso_workspace_bytes(rows, n,
 *                   flags) bytes, 256-byte aligned; may be NULL only when
 *                   that size is 0.  Owned by the caller; its contents need
 *                   no initialisation and are scratch after the call.
 *   workspace_bytes its size.
 *   stream          a hipStream_t (NULL = the null stream).
 *   flags           ISO_F_* bits.
 * Without ISO_F_NOCHECK the call synchronises with `stream` to read the
 * device's per-row data flags.  Calls that share one workspace must not
 * overlap in time.
 */
int iso_fit_ex(const float* y, const float* w, int64_t rows, int64_t n, float* out,
               int32_t* block_id, void* workspace, size_t workspace_bytes, void* stream,
               uint32_t flags);

/*
 * iso_fit_ex_f64, iso_fit_f64 - the same fits with f64 y, w and out (8-byte
 * aligned), through the same kernels (the paper's operator takes f32 and f64
 * in one code path, section 6).  Every sum and predicate is f64 either way;
 * with f64 input the products w_i y_i are rounded in f64, and each output is
 * the f64 slope itself.  The workspace is the same as for f32
 * (iso_workspace_bytes).  Statuses and flags as for iso_fit_ex / iso_fit.
 */
int iso_fit_ex_f64(const double* y, const double* w, int64_t rows, int64_t n, double* out,
                   int32_t* block_id, void* workspace, size_t workspace_bytes, void* stream,
                   uint32_t flags);
int iso_fit_f64(const double* y, const double* w, int64_t rows, int64_t n, double* out);

/*
 * iso_fit_noalloc - iso_fit_ex without a caller workspace and without any
 * allocation, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *   y, w, out, block_id, stream, flags as for iso_fit_ex.
 * The workspace is a fixed device array of ISO_NOALLOC_BYTES that the library
 * holds on every device it runs on until the process ends; shapes whose
 * iso_workspace_bytes exceeds it return ISO_ERR_WORKSPACE with nothing
 * launched.  The call never calls hipMalloc, hipFree or any other allocating
 * routine (host or device); its first call on a device looks up the array's
 * device address once.  Every call on one device shares that array and leaves
 * its contents in it (the kernels need no initialised workspace), so calls on
 * one device must not overlap in time: overlapping calls race on it.  Without
 * ISO_F_NOCHECK the call synchronises with `stream` (not capturable then);
 * with it the call only enqueues work.
 */
#define ISO_NOALLOC_BYTES (64u << 20)
int iso_fit_noalloc(const float* y, const float* w, int64_t rows, int64_t n, float* out,
                    int32_t* block_id, void* stream, uint32_t flags);

/*
 * iso_vjp - the backward pass: the vector-Jacobian product of the fit (paper
 * section 6, paragraph "Gradient"; validated as its appendix C describes).
 * The fit is constant on its blocks, each block's value the weighted mean z of
 * y over the block, so for an element i with G and W the sums of g and of w
 * over its block:
 *     grad_y[i] = w_i G / W ,        grad_w[i] = (y_i - z) G / W
 * (wherever the blocks do not change; at a boundary between equal means the
 * fit is not differentiable and the blocks of the forward call are used).
 *   g         [rows*n] f32, device: the gradient with respect to the fit.
 *   y         [rows*n] f32, device: the forward call's y; needed only for
 *             grad_w (may be NULL when grad_w is NULL).
 *   w         [rows*n] f32, device: the forward call's weights, or NULL for
 *             unit weights.
 *   block_id  [rows*n] int32, device: the block ids the forward call wrote
 *             (iso_fit_ex or iso_fit_noalloc with a block_id buffer), for the
 *             same y, w and flags.  A block starts at a row's first element
 *             and wherever the id changes.  A row whose ids are negative (a
 *             non-finite row of the forward call) gets NaN gradients.
 *   grad_y    [rows*n] f32, device, written, or NULL.
 *   grad_w    [rows*n] f32, device, written, or NULL (needs y and w).
 *   workspace device buffer of iso_vjp_workspace_bytes(rows, n) bytes,
 *             256-byte aligned, contents need no initialisation (NULL when
 *             that size is 0: rows of at most 2048 elements).
 *   stream    hipStream_t (NULL = the null stream).  The call only enqueues.
 * A decreasing fit (ISO_F_DECREASING) has the same gradient formulas in y and
 * w, so the same call serves it.  Sums are f64, without atomics (the result
 * does not depend on scheduling); each output is rounded once to f32.
 * Returns ISO_OK, ISO_ERR_ARG (NULL g or block_id, no output, grad_w without y
 * or w, misaligned or overlapping buffers, bad sizes), ISO_ERR_WORKSPACE or
 * ISO_ERR_HIP; nothing is launched on an error.
 */
int iso_vjp(const float* g, const float* y, const float* w, const int32_t* block_id, int64_t rows,
            int64_t n, float* grad_y, float* grad_w, void* workspace, size_t workspace_bytes,
            void* stream);

/* The same with f64 g, y, w and gradients (8-byte aligned). */
int iso_vjp_f64(const double* g, const double* y, const double* w, const int32_t* block_id,
                int64_t rows, int64_t n, double* grad_y, double* grad_w, void* workspace,
                size_t workspace_bytes, void* stream);

/* Bytes of device workspace iso_vjp and iso_vjp_f64 need for this shape (0 for
 * rows of at most 2048 elements, or an empty or invalid shape). */
size_t iso_vjp_workspace_bytes(int64_t rows, int64_t n);

/*
 * Calibration front end (paper section 7.7, "Case study: calibrating a click
 * model"; the blog note's lab notebook, calibration cells), all f64.
 *
 * iso_calib_fit - an isotonic calibration curve from n scores and outcomes:
 *   1. each score is keyed: the score itself, or with segments
 *      segment[i] + min(score, 1 - 1e-12) (one curve per segment, all fitted
 *      as one problem laid end to end);
 *   2. the keys are sorted with their outcomes;
 *   3. equal keys are pooled: xp[r] is the r-th distinct key, with the count
 *      and the mean of the outcomes of its scores;
 *   4. with segments, each mean is lifted by twice its segment index, so that
 *      no block of the fit reaches across a segment boundary;
 *   5. the means are fitted, the counts as weights, by the f64 fit;
 *   6. the lift is dropped again: fp[r] is the curve at xp[r].
 *   scores, outcomes [n] f64, device.  segment [n] int32 >= 0, device, or NULL.
 *   xp, fp   [n] f64, device, written: the first *k_out entries are the curve.
 *   k_out    host pointer: the number of distinct keys.
 *   workspace device buffer of iso_calib_workspace_bytes(n) bytes, 256-byte
 *            aligned, contents need no initialisation.
 *   stream   hipStream_t (NULL = the null stream).
 * The call waits for the GPU once (for the number of distinct keys).  Returns
 * ISO_OK, ISO_ERR_ARG, ISO_ERR_DATA (non-finite score or outcome; with
 * segments a negative score or segment id), ISO_ERR_WORKSPACE or ISO_ERR_HIP.
 *
 * iso_calib_apply - the curve (xp, fp) of k distinct keys at m new scores:
 * the key of each score (as above; with segment != NULL the search stays in
 * that segment's keys), linear interpolation between the two keys around it,
 * held at the end values outside them.  A query whose segment has no keys, or
 * whose score is NaN, gets NaN.  Only enqueues.  Returns ISO_OK, ISO_ERR_ARG
 * or ISO_ERR_HIP.
 *
 * iso_calib_workspace_bytes - workspace of iso_calib_fit for n scores (0 for
 * an invalid n); queries the current device's sort configuration.
 */
int iso_calib_fit(const double* scores, const double* outcomes, const int32_t* segment, int64_t n,
                  double* xp, double* fp, int64_t* k_out, void* workspace, size_t workspace_bytes,
                  void* stream);
int iso_calib_apply(const double* xp, const double* fp, int64_t k, const double* scores,
                    const int32_t* segment, int64_t m, double* out, void* stream);
size_t iso_calib_workspace_bytes(int64_t n);

/* Bytes of device workspace iso_fit_ex needs for this shape and these flags
 * (weighted or not is part of the shape: pass ISO_F_WEIGHTED_HINT in flags
 * when w will be non-NULL).  Returns 0 for an empty or invalid shape. */
size_t iso_workspace_bytes(int64_t rows, int64_t n, uint32_t flags);

/* A static English description of a status code. */
const char* iso_status_str(int status);

/* Frees the workspace that iso_fit caches on each device it has used. */
void iso_release(void);

/* Chunk size (points per chunk hull) that long rows of length n use; rows
 * with n at most iso_short_row_max() are fitted whole by one workgroup. */
int64_t iso_chunk_size(int64_t n);
int64_t iso_short_row_max(void);

/*
 * Measurement hooks (for benchmarks; not needed to fit).  After
 * iso_timing_enable(1), every fitting call made from any host thread records a
 * HIP event on its stream before each of its kernel launches and after the
 * last, so each launch's device duration can be read.  iso_timing_read waits
 * for the recorded events, adds each launch's duration (ms) to
 * ms[phase] and 1 to launches[phase] for its phase (ISO_PHASE_*), for phase <
 * nphase, clears the record and returns the number of launches read (or
 * ISO_ERR_HIP).  Enabling adds the event records to the stream and so may
 * widen the gaps between launches; iso_timing_enable(0) stops recording.
 */
enum {
    ISO_PHASE_SHORT_ROWS = 0,  /* whole short rows in one kernel          */
    ISO_PHASE_CHUNK_HULLS = 1, /* prefix sums, chunk hulls, chunk slots   */
    ISO_PHASE_MERGE = 2,       /* segment-list merge (first stage) or its control's set-up */
    ISO_PHASE_EXPAND = 3,      /* slope expansion (the fit)               */
    ISO_PHASE_COPY_BRIDGE = 4, /* copy control: bridges of one level      */
    ISO_PHASE_COPY_MOVE = 5,   /* copy control: vertex rewrite of a level */
    ISO_PHASE_MERGE_TOP = 6,   /* second merge stage (group hulls of a row) */
    ISO_PHASE_CHUNK_REDO = 7,  /* chunk hulls the first chunk kernel left over */
    ISO_PHASE_COUNT = 8
};
int iso_timing_enable(int on);

/* Measurement probe: a plain streaming copy of `bytes` (a multiple of 16;
 * src and dst 16-byte aligned device buffers that do not overlap) on `stream`,
 * the practical HBM bandwidth ceiling the fit's kernels are measured against.
 * Only enqueues.  Returns ISO_OK, ISO_ERR_ARG or ISO_ERR_HIP. */
int iso_copy_probe(const void* src, void* dst, size_t bytes, void* stream);
int iso_timing_read(double* ms, int64_t* launches, int nphase);

#ifdef __cplusplus
}
#endif

#endif /* ISO_H */
