/*
 * w4a16.h - C ABI of the W4A16 group-quantized linear layer for MI355X (gfx950).
 *
 * The operation (PerfXLLM page on Snapdragon 8 Gen2, 3532n.com/d/2322131):
 *   - §3.3 item 1 defines the product C[m, n] = A[m, k] . B[k, n]; here A is the
 *     dequantized weight matrix Wdeq[M, K] and B the activations X[K, N];
 *   - §3.3 item 2 is the same product with n = 1 (the decode-time GEMV);
 *   - §3.1 stores the weights as int4 codes with one scale and one zero per
 *     group of 128 weights.
 * Read here as
 *   C[m, n] = sum_k (q[m, k] - z[m, k / 128]) * s[m, k / 128] * X[k, n]
 * with fp16 s, X and C, 4-bit q and z, and fp32 accumulation.
 *
 * Layouts (all row-major, all device memory unless stated):
 *   q_packed  uint32 [M, K / 8]          nibble j (bits 4j..4j+3) of word w of
 *                                        row m holds q[m, 8w + j]
 *   scales    fp16   [M, G], G = K / 128
 *   z_packed  uint32 [M, ceil(G / 8)]    nibble j of word w of row m holds
 *                                        z[m, 8w + j]; padding nibbles are 0
 *   x         fp16   [K, N]              (N contiguous; [N, K] under
 *                                        W4A16_LAYOUT_TOKEN, see below)
 *   c         fp16   [M, N]              (N contiguous; [N, M] under
 *                                        W4A16_LAYOUT_TOKEN), written, never read
 *
 * Conventions shared by every entry point:
 *   - functions never throw, abort or allocate device memory, and never
 *     synchronize; work is enqueued on `stream` (a hipStream_t; NULL is the
 *     null stream) and its results are valid once that stream has reached it;
 *   - every argument is checked on the host before any HIP call; on failure
 *     the function returns a non-zero w4a16_status, writes nothing and
 *     records a message readable with w4a16_last_error();
 *   - the caller owns every buffer; no pointer is kept after the call.
 *   - base pointers must be 16-byte aligned (W4A16_ERR_MISALIGNED otherwise).
 *   - the output must not overlap any input (W4A16_ERR_INVALID_ARG).
 *   - NaN and Inf in scales or x propagate and are not checked.
 *   - results are bitwise repeatable for a given plan and shape: split
 *     reductions are summed in a fixed order, no float atomics are used.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4A16_OK = 0,
    W4A16_ERR_INVALID_ARG = 1,   /* bad size, null pointer, overlap, overflow  */
    W4A16_ERR_UNSUPPORTED = 2,   /* group_size other than 128, or a bad plan   */
    W4A16_ERR_MISALIGNED = 3,    /* a base pointer not 16-byte aligned         */
    W4A16_ERR_WORKSPACE = 4,     /* workspace missing or too small             */
    W4A16_ERR_HIP = 5            /* a HIP call failed (no device, launch error) */
} w4a16_status;

/* Static text for a status code ("unknown status" for other values). */
const char *w4a16_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none).  The
 * pointer stays valid until the next call on the same thread. */
const char *w4a16_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int w4a16_version(void);

/*
 * Round-to-nearest group quantizer: the step that produces the layer's
 * weights (PerfXLLM §3.1: weights only, int4, group size 128, a scale and a
 * zero per group), in its plain min/max form (AWQ's activation-aware scale
 * search is not part of it).  Per row m and group g of 128 k, in float32
 * with correctly rounded divides and round-half-to-even:
 *   lo = min(min_k w, 0), hi = max(max_k w, 0)
 *   s  = fp16(max(hi - lo, 1e-5) / 15)
 *   z  = clamp(rint(-lo / s), 0, 15)
 *   q  = clamp(rint(w / s) + z, 0, 15)
 *   w        : fp16 [M, K] row-major, finite values (NaN handling unspecified)
 *   q_packed : out, [M, K / 8] words, as w4a16_pack writes them
 *   scales   : out, fp16 [M, G]
 *   z_packed : out, [M, ceil(G / 8)] words (padding nibbles 0)
 * Requires M >= 1, K >= 128, K % 128 == 0, group_size == 128, 16-byte
 * aligned pointers and outputs that overlap neither each other nor w.
 * Bit-exact: the result is a pure function of w.  Work goes on stream.
 */
int w4a16_quantize(const void *w, int64_t M, int64_t K, int32_t group_size,
                   uint32_t *q_packed, void *scales, uint32_t *z_packed,
                   void *stream);

/*
 * Pack 4-bit codes into the storage format above (PerfXLLM §3.1 storage).
 *   q : uint8 [M, K] weight codes, or NULL to pack zeros only
 *   z : uint8 [M, K / group_size] zero codes, or NULL to pack weights only
 * Only the low nibble of each code is used.  q_packed / z_packed receive
 * [M, K / 8] and [M, ceil(G / 8)] words; a NULL output is allowed only with
 * a NULL input.  Requires M >= 1, K >= 128, K % 128 == 0, group_size == 128.
 * Bit-exact: the result is a pure function of the inputs.
 */
int w4a16_pack(const uint8_t *q, const uint8_t *z, int64_t M, int64_t K,
               int32_t group_size, uint32_t *q_packed, uint32_t *z_packed,
               void *stream);

/*
 * The GEMV of PerfXLLM §3.3 item 2: N = 1, c[M] = Wdeq . x[K].
 * Needs no workspace.  Same layouts and checks as w4a16_gemm with N = 1.
 */
int w4a16_gemv(const uint32_t *q_packed, const void *scales,
               const uint32_t *z_packed, const void *x, void *c, int64_t M,
               int64_t K, int32_t group_size, void *stream);

/*
 * Execution plan: which kernel runs and how the work is split.  Filled by
 * w4a16_plan_default(); tests and tuning may pass their own.
 *   kernel : W4A16_KERNEL_SKINNY (N <= 8, 16 or 32: weights streamed once,
 *            products on 16x16x32 fp16 MFMA, activations staged per wave in
 *            LDS), W4A16_KERNEL_NARROW (N <= 64: weights streamed once
 *            through a register ring, activations staged once per
 *            workgroup, 16x16x32 fp16 MFMA) or W4A16_KERNEL_TILED (tiles of
 *            BM x BN outputs, 32x32x16 fp16 MFMA; any N).
 *   skinny : ncol = N exactly (1..8, 16 or 32); rb = 1 (16 rows per wave);
 *            wm / wk = waves per workgroup along rows / along K
 *            (wm * wk <= 16); splitk = number of workgroups sharing one row
 *            tile along K (>= 1).  A wave takes at most 16 groups (8 for
 *            N > 4, 4 for N = 16, 2 for N = 32); plans beyond that, or whose
 *            staged activations exceed 160 KB of LDS, are rejected.
 *   tiled  : bm, bn = tile sizes (bm in {128, 256}, bn in {64, 128, 256},
 *            or bm = 512 with bn = 128 and wm = 8, or bm = 96 with
 *            bn = 64 and wm = 3);
 *            wm = waves along rows: 4 (each wave owns bm/4 rows and all
 *            bn columns), 2 (2 x 2 waves, bn >= 128), 8 (eight waves of
 *            64 rows, bm = 512) or 3 (three waves of 32 rows, bm = 96,
 *            pf <= 2, xpf <= 1, wk = 1); 0 means 4;
 *            pf = stages (groups of 128 k) of weights a wave loads ahead:
 *            0 or 1 (one) or 2 (two; not with wm = 2); xpf = stages of
 *            activations staged ahead: 0 or 1 (one); deeper pipelines,
 *            (pf, xpf) in {(2, 2), (3, 2), (4, 2), (3, 3), (4, 3)}, for
 *            wm = 4 and tiles of at most 256 x 64 outputs with bn <= 128;
 *            wk = K slices: 1 (0 means 1), or 2 for bm = 128, bn <= 128,
 *            wm = 4, pf <= 2, xpf <= 1 (a second grid of waves takes every
 *            other group; eight waves per workgroup);
 *            splitk as above; bm * K / 2 < 2^31 and N <= 2^23.
 *   narrow : ncol = 16, 32 or 64 staged columns (>= N); pf = groups of
 *            weights in flight per wave (4, 8 or 16); rb = 16-row blocks per
 *            wave (1 or 2, 0 means 2); wm = waves along rows (4, or 3 with
 *            wk = 1; 0 means 4), so 16 wm rb rows per workgroup; wk =
 *            waves along K per row block (1, 2 or 4; 0 means 1); splitk as
 *            above, with splitk * wk <= G, and large enough that a
 *            workgroup's activations, ceil(G / splitk) * 256 * ncol bytes
 *            plus its scales and zeros, fit in 160 KB of LDS;
 *            K <= 2^24 and 2 K N < 2^31.
 * Skinny plans with splitk > 1 and every tiled or narrow plan need a
 * workspace (w4a16_workspace_size_plan).  Fields a kernel does not use are
 * ignored.
 */
enum { W4A16_KERNEL_SKINNY = 1, W4A16_KERNEL_TILED = 2, W4A16_KERNEL_NARROW = 3 };

typedef struct {
    int32_t kernel;
    int32_t ncol;
    int32_t rb;
    int32_t wm;
    int32_t wk;
    int32_t bm;
    int32_t bn;
    int32_t splitk;
    int32_t pf;
    int32_t xpf;
} w4a16_plan;

/* The plan w4a16_gemm uses for this shape.  Returns a status. */
int w4a16_plan_default(int64_t M, int64_t N, int64_t K, int32_t group_size,
                       w4a16_plan *plan);

/* Name of the main kernel a plan (NULL: the default plan) launches for this
 * shape with x [K, N], as profilers print it without namespaces, e.g.
 * "skinny_kernel<1, 4>", "narrow_kernel<1, 4, 1, 1, 4, true>" or
 * "tiled_dx_kernel<512, 128, 8, 8, 2, 1>".  Kernels that read x in place
 * (narrow plans ending in "true", tiled_dx_kernel and tiled_k2_dx_kernel:
 * N a multiple of 8) are the call's only launch; the others (narrow plans
 * ending in "false", tiled_kernel and tiled_k2_kernel) follow
 * xpack_col_kernel, which rewrites x into 16-byte chunks.  Writes at most
 * len bytes including the terminating 0 into buf.
 * Returns a status; launches nothing. */
int w4a16_kernel_name(int64_t M, int64_t N, int64_t K, int32_t group_size,
                      const w4a16_plan *plan, char *buf, size_t len);

/* Workspace bytes a plan needs (0 for a skinny plan with splitk == 1); 0 on
 * invalid input. */
size_t w4a16_workspace_size_plan(int64_t M, int64_t N, int64_t K,
                                 int32_t group_size, const w4a16_plan *plan);

/* Workspace bytes w4a16_gemm needs with its default plan. */
size_t w4a16_gemm_workspace_size(int64_t M, int64_t N, int64_t K,
                                 int32_t group_size);

/*
 * The GEMM of PerfXLLM §3.3 item 1: c[M, N] = Wdeq[M, K] . x[K, N], with the
 * two regimes of that item (few tokens: bandwidth-bound skinny kernel; many
 * tokens: compute-bound tiled kernel) chosen by w4a16_plan_default().
 * Requires M >= 1, N >= 1, K >= 128, K % 128 == 0, group_size == 128.
 *
 * workspace: device memory of at least w4a16_gemm_workspace_size() bytes,
 * 16-byte aligned, or NULL when that size is 0.  Its first 64 KB hold one
 * arrival counter per output tile (split plans allow at most 16384 tiles);
 * fp32 partial sums follow, then (tiled and narrow kernels, only where they
 * do not read x in place: token-major x, or N not a multiple of 8) x
 * rewritten as 16-byte chunks of eight k of one column.  Before its first use the caller must fill at
 * least the first 64 KB with zeros; every call leaves the counters at zero
 * again, so one zero-fill serves all later calls of any shape.  Calls that
 * share a workspace must not run concurrently (one workspace per stream).
 */
int w4a16_gemm(const uint32_t *q_packed, const void *scales,
               const uint32_t *z_packed, const void *x, void *c, int64_t M,
               int64_t N, int64_t K, int32_t group_size, void *workspace,
               size_t workspace_bytes, void *stream);

/* w4a16_gemm with an explicit plan (W4A16_ERR_UNSUPPORTED for a plan the
 * shape cannot use). */
int w4a16_gemm_plan(const uint32_t *q_packed, const void *scales,
                    const uint32_t *z_packed, const void *x, void *c,
                    int64_t M, int64_t N, int64_t K, int32_t group_size,
                    const w4a16_plan *plan, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * Plan tuner, the "parameter tuning" of PerfXLLM §3.3 item 1: times the
 * candidate plans of this shape and layout on the caller's buffers and
 * returns the fastest.  Candidates: the default plan first, then skinny,
 * narrow and tiled plans over their fields (those the shape admits); plans
 * needing more than workspace_bytes are skipped.  Each candidate runs once
 * untimed, then iters times, each timed call bracketed by HIP events on
 * `stream`.  flush (optional, device memory, 16-byte aligned): flush_bytes
 * of it are overwritten before every timed call, so that the weights come
 * from HBM and not from the last-level cache (give more than 256 MB on
 * MI355X); NULL times warm calls.
 *   best    : out, the fastest plan
 *   best_us : out, its mean microseconds per call (may be NULL)
 *   n_tried : out, the number of plans timed (may be NULL)
 * Unlike every other entry point this one synchronizes the stream, writes c
 * and the workspace many times, and must not be called during graph
 * capture.  W4A16_ERR_WORKSPACE if no candidate fits the workspace; other
 * checks as w4a16_gemm_ex.
 */
int w4a16_tune(const uint32_t *q_packed, const void *scales,
               const uint32_t *z_packed, const void *x, void *c, int64_t M,
               int64_t N, int64_t K, int32_t group_size, int32_t layout,
               void *workspace, size_t workspace_bytes, void *flush,
               size_t flush_bytes, int32_t iters, w4a16_plan *best,
               float *best_us, int32_t *n_tried, void *stream);

/*
 * Activation and output layouts for the _ex entry points.
 *   W4A16_LAYOUT_KN    : x fp16 [K, N] and c fp16 [M, N] (the product of
 *                        PerfXLLM §3.3 item 1 as written; what w4a16_gemm
 *                        takes)
 *   W4A16_LAYOUT_TOKEN : x fp16 [N, K] and c fp16 [N, M], both row-major:
 *                        one row per token, the layout a model's hidden
 *                        states have, so that c = x . Wdeq^T feeds the next
 *                        layer without a transpose.  Same arithmetic, same
 *                        rounding: c_token[n, m] equals c_kn[m, n] bit for
 *                        bit under the same plan.
 * With N = 1 both layouts are the same memory.
 */
enum { W4A16_LAYOUT_KN = 0, W4A16_LAYOUT_TOKEN = 1 };

/*
 * w4a16_gemm for either layout, with an optional plan (NULL: the layout's
 * default plan, w4a16_plan_default_ex).  The skinny kernel takes the token
 * layout for N <= 8 (W4A16_ERR_UNSUPPORTED for its 16- and 32-column plans);
 * the narrow and tiled kernels take both layouts at any N they support.
 * Workspace needs are those of the plan, as for w4a16_gemm.  An unknown
 * layout is W4A16_ERR_INVALID_ARG.  Other checks, workspace rules and error
 * behaviour as w4a16_gemm.
 */
int w4a16_gemm_ex(const uint32_t *q_packed, const void *scales,
                  const uint32_t *z_packed, const void *x, void *c,
                  int64_t M, int64_t N, int64_t K, int32_t group_size,
                  int32_t layout, const w4a16_plan *plan, void *workspace,
                  size_t workspace_bytes, void *stream);

/* The plan w4a16_gemm_ex uses for this shape and layout (plan NULL there).
 * Returns a status. */
int w4a16_plan_default_ex(int64_t M, int64_t N, int64_t K, int32_t group_size,
                          int32_t layout, w4a16_plan *plan);

/* Workspace bytes w4a16_gemm_ex needs for this layout and plan (NULL: the
 * layout's default plan); 0 on invalid input or when none is needed. */
size_t w4a16_workspace_size_ex(int64_t M, int64_t N, int64_t K,
                               int32_t group_size, int32_t layout,
                               const w4a16_plan *plan);

/*
 * Residual add + RMS normalization, the first operator fusion of PerfXLLM
 * §3.2 (the residual network's addition and the normalization as one
 * operator; the normalization read as LLaMA's RMSNorm).  Token-major:
 *   h[n, k] = fp16(x[n, k] + residual[n, k])            (round to nearest even)
 *   y[n, k] = fp16(h[n, k] * rsqrt(mean_k h[n, k]^2 + eps) * gamma[k])
 * with the mean of squares taken in float32 over the stored fp16 h.
 *   x, residual : fp16 [N, K];  gamma : fp16 [K];  eps : finite, >= 0
 *   h           : out, fp16 [N, K]; may be residual itself (in-place
 *                 update of the stream), must not overlap it otherwise
 *   y           : out, fp16 [N, K]; overlaps nothing
 * Requires N >= 1, K >= 8, K % 8 == 0, 16-byte aligned pointers.  h is
 * bit-exact; y is within 2e-3 |y| + 1e-6 of the float64 result.
 */
int w4a16_add_rmsnorm(const void *x, const void *residual, const void *gamma,
                      float eps, void *h, void *y, int64_t N, int64_t K,
                      void *stream);

/*
 * The same normalization feeding the W4A16 product, token-major (the fused
 * prologue of a QKV or gate/up projection):
 *   h = fp16(x + residual);  c[n, m] = sum_k Wdeq[m, k] * y[n, k]
 * with y as in w4a16_add_rmsnorm and c fp16 [N, M].  y never reaches the
 * caller: with a skinny plan (N <= 8) of one split along K and h not the
 * residual itself, the skinny kernel stages fp16(h * gamma * 2^e) (e a
 * power of two per wave and token that brings the staged values to unit
 * mean square) and multiplies each token's sums by 2^-e and by the RMS
 * factor rsqrt(mean h^2 + eps) in its epilogue, after the workgroup's sums
 * of squares have met (one launch, no wait before the main loop);
 * otherwise y is written into the workspace, in the activation layout the
 * plan's kernel reads (the tiled and narrow kernels then skip their own
 * rewrite of the activations), and the call makes two launches.  The two
 * forms differ by one fp16 rounding of the activations (fp16(h gamma 2^e)
 * against fp16(y)), within the product's tolerance.  plan: NULL for the token-major
 * default plan
 * (w4a16_plan_default_ex with W4A16_LAYOUT_TOKEN).  workspace: at least
 * w4a16_gemm_add_rmsnorm_workspace_size() bytes, with the rules of
 * w4a16_gemm.  h may be residual itself; c overlaps nothing.  Other
 * requirements and errors as w4a16_gemm_ex and w4a16_add_rmsnorm.
 */
int w4a16_gemm_add_rmsnorm(const uint32_t *q_packed, const void *scales,
                           const uint32_t *z_packed, const void *x,
                           const void *residual, const void *gamma, float eps,
                           void *h, void *c, int64_t M, int64_t N, int64_t K,
                           int32_t group_size, const w4a16_plan *plan,
                           void *workspace, size_t workspace_bytes,
                           void *stream);

/* Workspace bytes of w4a16_gemm_add_rmsnorm for a plan (NULL: the
 * token-major default plan); 0 on invalid input. */
size_t w4a16_gemm_add_rmsnorm_workspace_size(int64_t M, int64_t N, int64_t K,
                                             int32_t group_size,
                                             const w4a16_plan *plan);

/*
 * One decode step of multi-head attention per sequence, the third fusion of
 * PerfXLLM §3.2 (the rotary encoding of Q and K, QK^T, the softmax and the
 * product with V in one operator; the rotary encoding read as LLaMA's:
 * channel pairs (2i, 2i + 1) turned by p * rope_base^(-2i / D)).  For each
 * sequence b with its new token at position p = pos[b]:
 *   q, k, v = the head slices of qkv[b] = [q | k | v]
 *   stores fp16(rope(k, p)) and v at position p of the caches, then
 *   out[b, h] = sum_{j <= p} softmax_j(scale * rope(q, p) . K[b, h, j]) V[b, h, j]
 *   qkv     : fp16 [B, 3 H D] (the QKV projection's token-major output)
 *   k_cache, v_cache : fp16 [B, H, S, D], updated at each sequence's p
 *   pos     : int32 [B] in device memory
 *   out     : fp16 [B, H D]
 *   max_len : a bound on p + 1 over the batch (1 <= max_len <= S): the
 *             work is split along it, so a tight bound is faster; a position
 *             outside [0, max_len) gives NaN outputs for its sequence and
 *             leaves its cache entries alone
 *   scale   : softmax scale, finite and > 0 (1 / sqrt(D) in LLaMA)
 * Requires D == 128 (W4A16_ERR_UNSUPPORTED otherwise), 1 <= B, H <= 65535,
 * max_len <= 262144 (the keys are split at most 1024 ways), 16-byte
 * aligned qkv, caches and out, and no overlap
 * between out, qkv, the caches and pos.  workspace: at least
 * w4a16_decode_attention_workspace_size() bytes (0 when the keys are not
 * split), with the zero-filled-counter rule of w4a16_gemm.  Results are
 * bitwise repeatable.
 */
int w4a16_decode_attention(const void *qkv, void *k_cache, void *v_cache,
                           const int32_t *pos, void *out, int64_t B, int64_t H,
                           int64_t D, int64_t S, int64_t max_len,
                           float rope_base, float scale, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Workspace bytes of w4a16_decode_attention (0 if none or on invalid
 * input). */
size_t w4a16_decode_attention_workspace_size(int64_t B, int64_t H, int64_t D,
                                             int64_t S, int64_t max_len);

/*
 * w4a16_decode_attention with an explicit workgroup shape (for tests and
 * tuning; results are the same up to the summation order of the split
 * merge): a workgroup of `waves` waves (4 or 8; 16 with 16 keys per wave)
 * takes waves * keys_per_wave consecutive keys of one head (keys_per_wave
 * 16, 32 or 64);
 * 0, 0 selects the default shape.  W4A16_ERR_UNSUPPORTED for other values,
 * or for a shape that splits the keys more than 1024 ways.
 */
int w4a16_decode_attention_plan(const void *qkv, void *k_cache, void *v_cache,
                                const int32_t *pos, void *out, int64_t B,
                                int64_t H, int64_t D, int64_t S,
                                int64_t max_len, float rope_base, float scale,
                                int32_t keys_per_wave, int32_t waves,
                                void *workspace, size_t workspace_bytes,
                                void *stream);

/* Workspace bytes of w4a16_decode_attention_plan for a shape (0, 0: the
 * default); 0 if none is needed or on invalid input. */
size_t w4a16_decode_attention_workspace_size_plan(int64_t B, int64_t H,
                                                  int64_t D, int64_t S,
                                                  int64_t max_len,
                                                  int32_t keys_per_wave,
                                                  int32_t waves);

/*
 * The gated activation of LLaMA's MLP on the fused gate/up projection's
 * output (the pages do not describe the MLP; this is the LLaMA-7B reading):
 *   act[n, i] = fp16(silu(gu[n, i]) * gu[n, I + i]),  silu(g) = g / (1 + e^-g)
 *   gu  : fp16 [N, 2 I], gate in columns 0 .. I - 1 (gate rows first in the
 *         fused weight), up in I .. 2 I - 1
 *   act : fp16 [N, I], overlapping nothing
 * Requires N >= 1, I >= 8, I % 8 == 0, 16-byte aligned pointers.  Within
 * 1e-3 |act| + 1e-6 of the float64 result.
 */
int w4a16_silu_mul(const void *gu, void *act, int64_t N, int64_t I,
                   void *stream);

/*
 * The down projection of the decoder layer's MLP with its gated activation
 * as a prologue (token-major):
 *   c[n, m] = sum_k Wdeq[m, k] * act[n, k],
 *   act[n, k] = fp16(silu(gu[n, k]) * gu[n, K + k])  (as w4a16_silu_mul)
 *   gu : fp16 [N, 2 K], the fused gate/up projection's output;  c : fp16 [N, M]
 * act never reaches memory: the skinny kernel forms it while staging the
 * activations, the tiled and narrow kernels while rewriting them into their
 * chunk layout.  Bit-identical to w4a16_silu_mul followed by w4a16_gemm_ex
 * (token layout) under the same plan.  plan NULL: the token-major default.
 * Workspace as w4a16_workspace_size_ex(M, N, K, 128, W4A16_LAYOUT_TOKEN,
 * plan); other requirements and errors as w4a16_gemm_ex.
 */
int w4a16_gemm_silu(const uint32_t *q_packed, const void *scales,
                    const uint32_t *z_packed, const void *gu, void *c,
                    int64_t M, int64_t N, int64_t K, int32_t group_size,
                    const w4a16_plan *plan, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * Measurement aid, not part of the layer: one launch that reads `bytes` of
 * `buf` once (16-byte non-temporal loads, `loads` KB per wave: 1, 2, 4, 8
 * or 16; `waves` waves per workgroup: 1, 2, 4, 8 or 16) and stores one
 * 32-bit word per wave into `sink` (w4a16_stream_read_sink_words(bytes,
 * waves, loads) words, caller-owned, overlapping nothing).  Its time per
 * launch is the attainable rate of a single read of that size, the floor
 * the memory-bound GEMV is held to (PerfXLLM §3.3 item 2: the GEMV is
 * memory-bound).  Requires bytes a positive multiple of 16 and 16-byte
 * aligned pointers.
 */
int64_t w4a16_stream_read_sink_words(int64_t bytes, int32_t waves, int32_t loads);
int w4a16_stream_read(const void *buf, int64_t bytes, uint32_t *sink,
                      int32_t waves, int32_t loads, void *stream);

/*
 * w4a16_gemm for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * default plan, kernels and results, bit for bit, with no workspace
 * argument.  The split-K partial sums, arrival counters and activation
 * chunks live in a fixed device array inside the library,
 * w4a16_gemm_noalloc_max_bytes() bytes (16 MiB) on each GPU it runs on,
 * held until the process ends; the first call on a device looks its address
 * up and clears its counters with a kernel on `stream`.  No call allocates
 * or frees memory.  A shape whose default plan needs more scratch than that
 * (w4a16_gemm_workspace_size above the maximum, e.g. the tiled kernel's
 * K x N activation chunks beyond 16 MiB, needed only when N is not a
 * multiple of 8) fails with W4A16_ERR_WORKSPACE
 * and writes nothing.  All calls on one GPU share the array: calls that may
 * run at the same time on that GPU (unordered streams) race and must not be
 * issued.  Other arguments, requirements and errors as w4a16_gemm.
 */
size_t w4a16_gemm_noalloc_max_bytes(void);
int w4a16_gemm_noalloc(const uint32_t *q_packed, const void *scales,
                       const uint32_t *z_packed, const void *x, void *c,
                       int64_t M, int64_t N, int64_t K, int32_t group_size,
                       void *stream);

/* One W4A16 linear layer's weights, as w4a16_gemm takes them. */
typedef struct {
    const uint32_t *q_packed;
    const void *scales;
    const uint32_t *z_packed;
} w4a16_linear;

/* The weights and caches of one LLaMA decoder layer (hidden size H D,
 * MLP width I). */
typedef struct {
    w4a16_linear qkv;       /* [3 H D, H D]: q rows, then k, then v      */
    w4a16_linear o;         /* [H D, H D]                                 */
    w4a16_linear gate_up;   /* [2 I, H D]: gate rows, then up rows        */
    w4a16_linear down;      /* [H D, I]                                   */
    const void *attn_norm;  /* fp16 [H D] gain of the attention's norm    */
    const void *mlp_norm;   /* fp16 [H D] gain of the MLP's norm          */
    void *k_cache;          /* fp16 [B, H, S, D]                          */
    void *v_cache;          /* fp16 [B, H, S, D]                          */
} w4a16_decoder_layer;

/*
 * One decode step of one LLaMA decoder layer, token-major, all on `stream`
 * (the generation phase of PerfXLLM §3.3, one input token per sequence,
 * with the fusions of §3.2):
 *   r   = fp16(x + r);  y = rmsnorm(r) * attn_norm          (w4a16_gemm_add_rmsnorm
 *   qkv = y . Wqkv^T                                           with the QKV weights)
 *   a   = decode attention(qkv, caches, pos)                  (w4a16_decode_attention)
 *   x   = a . Wo^T                                             (w4a16_gemm_ex)
 *   r   = fp16(x + r);  y = rmsnorm(r) * mlp_norm;  gu = y . Wgu^T
 *   x   = (silu(gate) * up) . Wdown^T                          (w4a16_gemm_silu)
 * residual (r) and x are fp16 [B, H D], both read and overwritten: on entry
 * x is the previous layer's output still to be added to the stream, on exit
 * this layer's.  Default plans, scale 1 / sqrt(D).  Every step is checked
 * before the first is enqueued; nothing allocates or synchronizes, so a
 * whole model's step can be captured in one graph.  workspace: at least
 * w4a16_decode_layer_workspace_size() bytes, 16-byte aligned, first 64 KB
 * zero before first use (kept zero).  Requirements of the steps above;
 * I % 128 == 0.
 */
int w4a16_decode_layer(const w4a16_decoder_layer *layer, int64_t B, int64_t H,
                       int64_t D, int64_t I, int64_t S, int64_t max_len,
                       const int32_t *pos, float eps, float rope_base,
                       void *residual, void *x, void *workspace,
                       size_t workspace_bytes, void *stream);

/* Workspace bytes of w4a16_decode_layer (0 on invalid input). */
size_t w4a16_decode_layer_workspace_size(int64_t B, int64_t H, int64_t D,
                                         int64_t I, int64_t S,
                                         int64_t max_len);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
