/*
 * ulysses.h — C ABI of libulysses.so: the Ulysses 4D all-to-all relayout on
 * one AMD Instinct MI355X (gfx950), with the W ranks of a sequence-parallel
 * group emulated as W separate shard buffers in the GPU's own HBM.
 *
 * What it computes (fast-ulysses 0.1.0 PyPI page, introduction and "Quick
 * start"; fast-ulysses 0.2.1 README, introduction, "Key features", "Quick
 * start" and "API"):
 *
 *   mode 0  W shards (b, S_j, n_global, d)  ->  W shards (b, s_global, H_r, d)
 *           out_r[bi][S][h][e] = in_j[bi][S - seq_off_j][head_off_r + h][e]
 *           where j is the rank whose sequence range holds the global row S;
 *   mode 1  the inverse: W shards (b, s_global, H_r, d) -> (b, S_r, n_global, d)
 *           out_r[bi][s][H][e] = in_j[bi][seq_off_r + s][H - head_off_j][e]
 *           where j is the rank whose head range holds the global head H.
 *
 * S_j = seq_splits[j] and H_r = head_splits[r] may be uneven ("Uneven
 * shards"); seq_off and head_off are their exclusive prefix sums.  Sequence
 * pieces are concatenated in rank order and rank r owns the contiguous head
 * block [head_off_r, head_off_r + H_r): the order torch.distributed's
 * permute + all_to_all_single + permute produces, which the pages give as the
 * equivalent baseline (0.1.0 "Results", 0.2.1 "Performance").
 *
 * Layout: every shard is one contiguous, row-major buffer with d innermost.
 * Element bytes are copied verbatim (NaN payloads, -0, fp8 encodings kept).
 *
 * Ownership: the caller allocates and owns every device buffer (sources,
 * destinations, windows, gammas, rotary tables) and keeps it alive until the
 * stream work completes.  The library never allocates or frees device memory
 * (the windows of ulysses_a2a_4d_chunked_static are a static array in the
 * library's own code object) and never synchronises a stream: each call
 * validates on the host and then enqueues asynchronously on the given stream.  A plan is host memory only,
 * immutable after creation, and may be shared by threads and reused.
 *
 * Errors: every call returns a status (ULYSSES_OK or a negative code below).
 * All validation happens before anything is enqueued, so on error nothing was
 * launched.  ulysses_last_error() returns a message for the calling thread's
 * most recent failure.  No C++ exception crosses this boundary.
 */
#ifndef ULYSSES_H
#define ULYSSES_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Ranks per group: 1..8, odd counts included (0.1.0 "What it does",
 * Limits; 0.2.1 "Limits"). */
#define ULYSSES_MAX_WORLD 8

/* Element types (0.2.1 "Limits").  The relayout is bytewise; the type fixes
 * the element size and which entry points accept it. */
enum ulysses_dtype {
    ULYSSES_BF16 = 0,
    ULYSSES_FP16 = 1,
    ULYSSES_FP32 = 2,
    ULYSSES_FP8_E4M3 = 3,
    ULYSSES_FP8_E5M2 = 4,
    ULYSSES_INT8 = 5,
    ULYSSES_UINT8 = 6
};

enum ulysses_status {
    ULYSSES_OK = 0,
    ULYSSES_EINVAL = -1,   /* bad world, mode, size, split, null pointer */
    ULYSSES_EALIGN = -2,   /* d*elem_size not a multiple of 16, or a base
                              pointer not 16-byte aligned (0.2.1 "Limits") */
    ULYSSES_EDTYPE = -3,   /* unknown dtype, or one the entry point refuses */
    ULYSSES_EWINDOW = -4,  /* per-rank window bytes exceed the plan's cap */
    ULYSSES_EOVERLAP = -5, /* a destination (or window) overlaps another
                              buffer of the same call */
    ULYSSES_EHIP = -6      /* the HIP runtime refused the launch */
};

typedef struct ulysses_plan ulysses_plan;

/*
 * Build a plan: validate the geometry and compute, on the host, every offset,
 * row pitch, piece extent and launch size the kernels need.  The plan is the
 * host-side addressing of the pages' a2a_plan (0.1.0 "What it does": the
 * relayout is a host plan, so there is no launch config and no autotune).
 *
 *   out               receives the plan; set to NULL on error.
 *   world             number of emulated ranks W, 1..ULYSSES_MAX_WORLD.
 *   b                 batch planes, >= 1 (the batch axis of every shard).
 *   d                 head dimension, >= 1; d*elem_size % 16 == 0 (EALIGN).
 *   seq_splits        host array of W sequence lengths S_j >= 0, sum >= 1.
 *   head_splits       host array of W head counts H_r >= 0, sum >= 1.
 *   dtype             enum ulysses_dtype.
 *   window_cap_bytes  per-rank staging-window cap for the plane-at-a-time
 *                     entry point (FastVideo "Ulysses performance on GB200":
 *                     at most 1 GiB of window per rank); 0 = no chunking.
 *
 * Limits checked here (EINVAL): one row of any shard at most 512 KiB, and one
 * batch plane of any shard below 2^31 16-byte vectors (32 GiB).
 */
int ulysses_plan_create(ulysses_plan **out, int world, int64_t b, int64_t d,
                        const int64_t *seq_splits, const int64_t *head_splits,
                        int dtype, int64_t window_cap_bytes);

/* Free a plan (NULL is ignored).  Nothing on a stream refers to it. */
void ulysses_plan_destroy(ulysses_plan *plan);

/*
 * Shape of rank `rank`'s shard: the input (is_dst = 0) or output (is_dst = 1)
 * of `mode`, written to shape[4] as (b, s, n, d).  Mode-0 input and mode-1
 * output are (b, S_r, n_global, d); mode-0 output and mode-1 input are
 * (b, s_global, H_r, d) (0.1.0 "Quick start"; 0.2.1 "Quick start").
 */
int ulysses_plan_shape(const ulysses_plan *plan, int mode, int rank, int is_dst,
                       int64_t shape[4]);

/*
 * Bytes one rank's staging window must hold for one batch plane of `mode`:
 * the largest per-rank destination plane, max_r s_global*H_r*d*esz (mode 0)
 * or max_r S_r*n_global*d*esz (mode 1).  FastVideo "Ulysses performance on
 * GB200" prints 896,000,000 for 250,000 tokens, 56 heads, d = 128, bf16 and
 * four ranks.  Returns a negative status on a bad plan or mode.
 */
int64_t ulysses_plan_window_bytes(const ulysses_plan *plan, int mode);

/*
 * Algorithmic bytes of one ulysses_a2a_4d call of `mode`: every element read
 * once and written once, 2 * b * s_global * n_global * d * esz.  Negative
 * status on a bad plan or mode.
 */
int64_t ulysses_plan_bytes(const ulysses_plan *plan, int mode);

/*
 * The relayout, all W ranks in one pass (0.1.0 introduction: the
 * sequence/head permutation is expressed as addressing, not as separate
 * permute kernels; 0.2.1 "API": all_to_all_4d with mode, seq_splits,
 * head_splits).
 *
 *   mode    0 or 1.
 *   src     host array of W device pointers, shard j of the mode's input shape.
 *   dst     host array of W device pointers, shard r of the mode's output shape.
 *   stream  HIP stream the work is enqueued on (0 = the null stream).
 *
 * Every pointer 16-byte aligned and non-null when its shard is non-empty.
 * Destinations must not overlap any source or each other (EOVERLAP).
 */
int ulysses_a2a_4d(const ulysses_plan *plan, int mode, const void *const *src,
                   void *const *dst, hipStream_t stream);

/*
 * The relayout of several tensors of the plan's geometry in one launch, e.g.
 * a layer's q, k and v, or a packed QKVG (fast-ulysses 0.1.0 "What it does":
 * q/k/v calls sharing one closing handshake; FastVideo "Ulysses performance
 * on GB200": packed QKV or QKVG).  Equal to ntensors ulysses_a2a_4d calls.
 *
 *   ntensors  1 .. ULYSSES_MAX_TENSORS.
 *   src, dst  host arrays of ntensors * W device pointers, tensor-major:
 *             entry t * W + r is rank r's shard of tensor t.
 *
 * Same pointer rules as ulysses_a2a_4d, over all tensors: no destination
 * may overlap any source or any other destination (EOVERLAP).
 */
#define ULYSSES_MAX_TENSORS 4
int ulysses_a2a_4d_multi(const ulysses_plan *plan, int mode, int ntensors,
                         const void *const *src, void *const *dst, hipStream_t stream);

/*
 * Plane-at-a-time relayout under a window cap (FastVideo "Ulysses
 * performance on GB200": one batch plane is exchanged at a time; each rank
 * keeps at most 1 GiB of window; the full output still needs its own
 * allocation).  For each batch plane p: the mode's relayout of plane p into
 * the W windows, then a copy of window r into plane p of dst r.  The result
 * equals ulysses_a2a_4d; the windows are scratch.
 *
 *   window  host array of W device pointers, each to at least
 *           ulysses_plan_window_bytes(plan, mode) bytes, 16-byte aligned,
 *           overlapping no source, destination or other window;
 *           or NULL: the window of plane p is plane p of the destination
 *           itself, so each plane's relayout writes straight into its final
 *           place and there is no copy-out (fast-ulysses 0.2.1 "Key
 *           features", "Performance" and "API": an output allocated up
 *           front and passed as out= removes the copy-out).
 *
 * EINVAL when the plan has no cap (window_cap_bytes == 0); EWINDOW when
 * ulysses_plan_window_bytes(plan, mode) exceeds the cap (with or without
 * windows: the destination plane then takes the window's place).
 */
int ulysses_a2a_4d_chunked(const ulysses_plan *plan, int mode, const void *const *src,
                           void *const *dst, void *const *window, hipStream_t stream);

/*
 * ulysses_a2a_4d_chunked with the library's own windows, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the W windows live in one static
 * device array of ULYSSES_STATIC_WINDOW_BYTES (64 MiB) that every GPU running
 * the library holds until the process ends.  The call itself allocates and
 * frees nothing.  Window r starts at r times the per-rank window bytes
 * rounded up to 256.
 *
 * The result equals ulysses_a2a_4d_chunked with caller windows.  The array
 * is shared by every call on a GPU and keeps the last call's contents (the
 * windows need no clearing: each plane's relayout writes every window byte
 * the copy-out reads), so calls that overlap in time on one GPU, e.g. on two
 * streams, race; serialise them.
 *
 * EINVAL when the plan has no cap; EWINDOW when the per-rank window bytes
 * exceed the cap, or when W windows do not fit the array; EHIP when the
 * array's address cannot be found on the stream's device.
 */
#define ULYSSES_STATIC_WINDOW_BYTES (64ll << 20)
int ulysses_a2a_4d_chunked_static(const ulysses_plan *plan, int mode, const void *const *src,
                                  void *const *dst, hipStream_t stream);

/*
 * Mode-0 relayout of q and k with QK RMSNorm and RoPE applied on the way
 * (0.1.0 "What it does": the QK RMSNorm + RoPE fusion inside the scatter
 * kernel; the pages give no formula, so the operation is fixed here).
 * For each destination row of d elements at GLOBAL sequence position S:
 *   ss  = sum of squares, fp32: one fused multiply-add chain per group of 8
 *         consecutive elements (ascending), then a pairwise tree over the d/8
 *         partial sums with adjacent pairing;
 *   inv = 1 / sqrt(ss / d + eps), each operation correctly rounded;
 *   y_i = (x_i * inv) * gamma_i;
 *   o_{2p}   = y_{2p} * cos[S][p] - y_{2p+1} * sin[S][p],
 *   o_{2p+1} = y_{2p} * sin[S][p] + y_{2p+1} * cos[S][p]   (products rounded,
 *         no fused multiply-add);  out = o rounded to bf16, nearest even.
 *
 *   q_src, k_src    W device pointers each, mode-0 input shards, bf16.
 *   q_dst, k_dst    W device pointers each, mode-0 output shards, bf16.
 *   gamma_q/gamma_k device, d floats each.
 *   eps             added to the mean square inside the square root.
 *   rope_cos/sin    device, [s_global][d/2] floats (ulysses_rope_table).
 *
 * The plan's dtype must be ULYSSES_BF16 (EDTYPE); d/8 must be a power of two
 * from 1 to 64, i.e. d in {8, 16, ..., 512} (EINVAL).  No destination may
 * overlap any source, table or gamma.
 */
int ulysses_a2a_4d_qknorm_rope(const ulysses_plan *plan,
                               const void *const *q_src, void *const *q_dst,
                               const void *const *k_src, void *const *k_dst,
                               const float *gamma_q, const float *gamma_k, float eps,
                               const float *rope_cos, const float *rope_sin,
                               hipStream_t stream);

/*
 * Host helper: the rotary table the fused entry point reads.  For S in
 * [0, s_global) and p in [0, d/2): w_p = theta^(-2p/d), angle = S * w_p, both
 * in double precision; cos_out[S*(d/2) + p] = (float)cos(angle) and
 * sin_out likewise (RoFormer's rotary position embedding, interleaved pairs).
 * cos_out and sin_out are HOST buffers of s_global*d/2 floats each.
 * EINVAL on theta <= 0, s_global < 0, odd d or null outputs.
 */
int ulysses_rope_table(double theta, int64_t s_global, int64_t d, float *cos_out,
                       float *sin_out);

/* Message of the calling thread's last failed call ("" if none).  The
 * pointer stays valid until that thread's next call into the library. */
const char *ulysses_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ULYSSES_H */
