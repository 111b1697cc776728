/*
 * beam_moe.h -- C ABI of the BEAM masked-MoE layer forward pass on AMD
 * Instinct MI355X (gfx950).
 *
 * What the layer computes (BEAM page on aitrends.kr, "BEAM: Dynamic MoE
 * 라우팅을 위한 Binary Expert Activation Masking", method paragraph, Steps
 * 1-4, restated in its architecture paragraph):
 *
 *   Step 1  r = x Wr^T (+ b_r); keep the K largest r; g = softmax over them.
 *   Step 2  raw mask m_hat = sigmoid(z), z = x Wm^T (+ b_m), one mask logit
 *           per expert, read at the K candidates.
 *   Step 3  m = 1 when m_hat >= 0.5 (decided as z >= 0), else 0.
 *   Step 4  g_hat = g * m (not renormalised); y = sum_k g_hat_k E_k(x).
 *
 * Only the (token, expert) pairs with m = 1 run their expert (the ai-feeds.com
 * summary, section on inference: experts whose mask is 0 skip their FFN).
 * Experts are SwiGLU FFNs, E(x) = Wd (silu(Wg x) * (Wu x)).  Shared experts,
 * when the layer has them, are added to y with gate 1 and are never masked
 * (they are what the aitrends.kr page's limitation C refers to).
 *
 * Conventions for every call below:
 *   - All tensor pointers are DEVICE pointers, owned by the caller, 16-byte
 *     aligned, row-major and densely packed.  The library allocates nothing
 *     and keeps no state between calls except the optional profiler and the
 *     static workspace of beam_moe_forward_static.
 *   - `stream` is a hipStream_t (NULL = the default stream).  route and
 *     forward only enqueue work: they never synchronise the host.
 *   - Arguments are validated before anything is launched; on any error
 *     nothing is written.  A failed kernel launch returns BEAM_ERR_HIP.
 *   - T = 0 is a no-op returning BEAM_OK.
 *   - Results are bit-identical from run to run for identical inputs.
 *   - One workspace per concurrently running call: two calls in flight on the
 *     same workspace (different streams) race.
 */
#ifndef BEAM_MOE_H
#define BEAM_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BEAM_OK = 0,
  BEAM_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, bad shape or size  */
  BEAM_ERR_UNSUPPORTED = -2,  /* valid but outside what the kernels handle   */
  BEAM_ERR_WORKSPACE = -3,    /* workspace pointer null or too small         */
  BEAM_ERR_HIP = -4           /* a HIP runtime call or kernel launch failed  */
} beam_status;

typedef enum { BEAM_F32 = 0, BEAM_BF16 = 1 } beam_dtype;

/* Gate options (beam_moe_layer.gating, bits; 0 = the method as described
 * above).  The ai-feeds.com summary's section on the input and overall flow
 * applies the mask to the router's expert scores without fixing where the
 * softmax sits, so two common forms are offered besides Steps 1 and 4:
 *   BEAM_GATE_SOFTMAX_ALL  g_k = softmax over all E router logits, read at
 *                          the top-K experts (no renormalisation over K).
 *   BEAM_GATE_RENORM       after masking, g_hat_k = g_k m_k / sum_j g_j m_j
 *                          (0 for every slot when no slot survives).
 *   BEAM_GATE_BINARY       g_k = 1 on every top-K slot, so g_hat = m: the
 *                          {0,1} expert mask of the Stepped MoE page
 *                          (paper.rainbus.top, "Stepped MoE: Segment-Level
 *                          Routing with Configurable Inference Complexity",
 *                          section on the core method).  Combines with
 *                          BEAM_GATE_RENORM (g_hat = m / sum m), not with
 *                          BEAM_GATE_SOFTMAX_ALL (BEAM_ERR_INVALID_ARG).
 * The top-K set, its order and the mask bits do not depend on these bits. */
typedef enum {
  BEAM_GATE_SOFTMAX_ALL = 1,
  BEAM_GATE_RENORM = 2,
  BEAM_GATE_BINARY = 4
} beam_gate_flag;

/* Storage of the routed and shared expert weights (beam_moe_layer.
 * expert_format).  The masking combines with weight quantisation (the
 * ai-feeds.com summary, section on interfaces with existing products and
 * workflows, item 3):
 *   BEAM_WEIGHTS_DTYPE      every expert weight has the layer dtype.
 *   BEAM_WEIGHTS_FP8_E4M3   w_gate, w_up, w_down, ws_gate, ws_up, ws_down
 *                           hold OCP FP8 E4M3 codes (one byte per weight,
 *                           same shapes), and the weight in row r of a
 *                           matrix is e4m3(code) * scale[r], with one fp32
 *                           scale per output row: [E][I] for w_gate and
 *                           w_up, [E][D] for w_down, [n_shared][I_shared]
 *                           and [n_shared][D] for the shared experts.
 *                           Requires dtype BEAM_BF16 (x, y and the router
 *                           weights stay bf16) and D, I, I_shared multiples
 *                           of 128; every scale pointer in use must be
 *                           non-NULL and 16-byte aligned.  Products run in
 *                           bf16 MFMA on the exactly widened codes with fp32
 *                           accumulation; the scales multiply the fp32 sums.
 *                           Meant for decode: every batch runs the streaming
 *                           kernels with tiles of at most 64 token rows. */
typedef enum { BEAM_WEIGHTS_DTYPE = 0, BEAM_WEIGHTS_FP8_E4M3 = 1 } beam_weight_format;

/* Layer description.  Shapes: D hidden, E routed experts, K top-K, I routed
 * expert intermediate size, n_shared shared experts of intermediate size
 * I_shared.  Supported: 1 <= K <= min(E, 32), E <= 1024, D, I and I_shared
 * multiples of 64, D <= 16384, I <= 2^20, n_shared * I_shared <= 2^20, and
 * I * D and n_shared * I_shared * D below 2^31 (the kernels address rows with
 * 32-bit element offsets); per call T * K <= 2^30 and T * D < 2^31.  Shapes
 * outside these give BEAM_ERR_UNSUPPORTED (workspace size 0).  Every weight
 * tensor has the layer's dtype,
 * except the expert weights when expert_format is BEAM_WEIGHTS_FP8_E4M3.
 * Fields past `gating` may be left zero (= BEAM_WEIGHTS_DTYPE, no scales). */
typedef struct {
  int32_t D, E, K, I, n_shared, I_shared;
  int32_t dtype;               /* beam_dtype                                  */
  const void *w_router;        /* [E][D]  router weights Wr                   */
  const void *w_mask;          /* [E][D]  mask-router weights Wm              */
  const float *b_router;       /* [E] fp32 router bias, or NULL (= 0)         */
  const float *b_mask;         /* [E] fp32 mask-router bias, or NULL (= 0)    */
  const void *w_gate;          /* [E][I][D]  Wg                               */
  const void *w_up;            /* [E][I][D]  Wu                               */
  const void *w_down;          /* [E][D][I]  Wd                               */
  const void *ws_gate;         /* [n_shared][I_shared][D], NULL if n_shared=0 */
  const void *ws_up;           /* [n_shared][I_shared][D]                     */
  const void *ws_down;         /* [n_shared][D][I_shared]                     */
  int32_t gating;              /* beam_gate_flag bits; unknown bits are
                                  BEAM_ERR_INVALID_ARG                        */
  int32_t expert_format;       /* beam_weight_format; other values are
                                  BEAM_ERR_INVALID_ARG                        */
  const float *scale_gate;         /* FP8 only: [E][I] row scales of w_gate   */
  const float *scale_up;           /* [E][I] row scales of w_up               */
  const float *scale_down;         /* [E][D] row scales of w_down             */
  const float *scale_shared_gate;  /* [n_shared][I_shared] (ws_gate)          */
  const float *scale_shared_up;    /* [n_shared][I_shared] (ws_up)            */
  const float *scale_shared_down;  /* [n_shared][D] (ws_down)                 */
  int32_t segment_len;         /* Segment routing (Stepped MoE page, sections
                                  on the core method and the method steps):
                                  0 or 1 = every token routes itself; S > 1 =
                                  token t takes the routing (top-K set, g, m)
                                  of token t - t % S, the first token of its
                                  S-token segment of the batch, and runs those
                                  experts on its own x.  Negative values are
                                  BEAM_ERR_INVALID_ARG.                       */
  /* Optional second copies of the bf16 expert weights in the packed operand
   * layout written by beam_moe_pack_weights (same values, another
   * arrangement; NULL = absent).  Either all that the layer uses are given
   * (wp_gate, wp_up, wp_down, and the three shared ones when n_shared > 0,
   * 16-byte aligned) or none; only with dtype BEAM_BF16 and expert_format
   * BEAM_WEIGHTS_DTYPE.  Batches large enough for the prefill-shaped
   * kernels (128-token tiles) then read these, whose operand-layout loads
   * are whole cache lines; smaller batches read w_gate .. ws_down as always. */
  const void *wp_gate;         /* packed w_gate: E matrices [I][D]            */
  const void *wp_up;           /* packed w_up: E matrices [I][D]              */
  const void *wp_down;         /* packed w_down: E matrices [D][I]            */
  const void *wsp_gate;        /* packed ws_gate: one matrix [n_shared I_shared][D] */
  const void *wsp_up;          /* packed ws_up: one matrix [n_shared I_shared][D]   */
  const void *wsp_down;        /* packed ws_down: n_shared matrices [D][I_shared]   */
  /* Expected Avg-K of the layer (mean number of kept experts per token, the
   * figure the BEAM pages report; aitrends.kr results paragraph), or 0 when
   * unknown (then K is assumed).  A hint for choosing kernels only: with
   * packed weights and no shared experts, batches expected to give each
   * expert at least 256 surviving pairs (T x expected_avg_k / E) run the
   * expert-stationary prefill kernels, and on layers without shared
   * experts the decode-sized row tiles (16, 32 or 64 rows) are sized by
   * the same expected count.  The kernels it picks between compute the
   * same sums, possibly in another order: routing is unchanged, y agrees
   * within rounding.  Must be finite and in [0, K] (else
   * BEAM_ERR_INVALID_ARG). */
  float expected_avg_k;
} beam_moe_layer;

/* Routing results (device pointers, caller-owned). */
typedef struct {
  int32_t *topk_idx;      /* [T][K] experts by descending router logit; equal
                             logits are ordered by lower expert index         */
  float *gates;           /* [T][K] masked gates g_hat (0 where m = 0)        */
  uint32_t *mask;         /* [T] bit k = m of slot k                          */
  int32_t *expert_count;  /* [E] surviving pairs per expert                   */
} beam_route_out;

/* Host-side work accounting (beam_moe_stats / beam_moe_stats_host).
 * Avg-K, the average number of experts a token activates, is the measure
 * the aitrends.kr BEAM page reports its sparsity with (results paragraph:
 * Avg-K cut by 47-61% at mid sparsity, 0.14-0.56 at high sparsity); here it
 * is the number of surviving pairs over T.  The routed-expert FLOPs scale
 * with the surviving pairs, which is how the chatpaper.ai abstract's "up to
 * 85% fewer MoE-layer FLOPs" is counted: flops_reduction = 1 - Avg-K / K. */
typedef struct {
  int32_t T, E, K, active_experts;
  int64_t active_pairs;               /* sum of expert_count                  */
  double avg_k;                       /* active_pairs / T                     */
  double flops_routed;                /* 6 D I active_pairs                   */
  double flops_topk_routed;           /* 6 D I T K (plain top-K MoE)          */
  double flops_shared;                /* 6 D I_shared n_shared T              */
  double flops_router;                /* 4 E D T                              */
  double flops_reduction;             /* 1 - flops_routed / flops_topk_routed */
  double bytes_active_expert_weights; /* experts with a pair + shared, once
                                         (FP8: codes plus the row scales)     */
  double bytes_total_min;             /* + router weights + x + y             */
} beam_stats;

/* Bytes of workspace that route/forward need for batches of up to T_max
 * tokens.  Returns 0 for an invalid layer or T_max < 0. */
size_t beam_moe_workspace_size(const beam_moe_layer *layer, int32_t T_max);

/* Steps 1-3 of the method and the per-expert counts: fills every field of
 * *out (all four pointers required).  x: [T][D] in the layer dtype.
 * ws: device workspace of at least beam_moe_workspace_size(layer, T) bytes.  */
int beam_moe_route(const beam_moe_layer *layer, const void *x, int32_t T,
                   const beam_route_out *out, void *ws, size_t ws_bytes,
                   void *stream);

/* The whole layer, Steps 1-4: y [T][D] in the layer dtype.  out may be NULL
 * (routing is then kept in the workspace only); if given, all four of its
 * pointers are filled as by beam_moe_route.  y must not alias x. */
int beam_moe_forward(const beam_moe_layer *layer, const void *x, int32_t T,
                     void *y, const beam_route_out *out, void *ws,
                     size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the same
 * forward pass as beam_moe_forward, with its workspace taken from a static
 * device array of BEAM_STATIC_WORKSPACE_BYTES (128 MiB) inside the library
 * instead of a caller buffer.  Arguments and results are those of
 * beam_moe_forward; the current device (hipGetDevice) must be the one that
 * holds the tensors and the stream.
 *   - Batches whose workspace (beam_moe_workspace_size(layer, T)) exceeds
 *     BEAM_STATIC_WORKSPACE_BYTES are rejected with BEAM_ERR_WORKSPACE before
 *     anything is launched (every decode batch of up to 512 tokens of the
 *     DeepSeek-V2-Lite-, Mixtral- and fine-grained-shaped layers fits).
 *   - Calls no hipMalloc, hipFree or other allocating routine.  Each GPU the
 *     library runs on holds its own copy of the array from the first call on
 *     that GPU until the process ends (the first call per GPU also looks up
 *     the array's device address, a host-side runtime call).
 *   - Every call on one GPU shares that GPU's array: two calls that overlap
 *     in time on one GPU (different streams or threads) race and corrupt each
 *     other's results.  Serialise them on one stream.
 *   - The array keeps the last call's contents; nothing in it needs to start
 *     at zero (every call writes what it later reads). */
#define BEAM_STATIC_WORKSPACE_BYTES (128u << 20)
int beam_moe_forward_static(const beam_moe_layer *layer, const void *x,
                            int32_t T, void *y, const beam_route_out *out,
                            void *stream);

/* Packed operand layout of bf16 expert weights (for the wp_* / wsp_*
 * fields above).  Rearranges `mats` row-major matrices W [rows][cols], stored
 * one after another at w, into `packed` (same size, caller-owned, not
 * overlapping w), matrix by matrix:
 *   packed[m][(rb * cols/64 + kb) * 2048 + s * 512 + l * 8 + j]
 *     = W_m[32 rb + l % 32][64 kb + 16 s + 8 (l / 32) + j]
 * for rb < rows/32, kb < cols/64, s < 4, l < 64, j < 8: blocks of 32 rows x
 * 64 columns, and within a block the A operand of the gfx950
 * v_mfma_f32_32x32x16_bf16 instruction for lane l at k-step s.  A
 * 64-lane load of one k-step then reads 1 KB of contiguous memory.  rows must
 * be a multiple of 32, cols of 64, and rows * cols below 2^31.  Device
 * pointers, 16-byte aligned; enqueued on `stream`.  Meant to run once, when
 * the weights are loaded (for expert weights this is a layout of the layer's
 * parameters, like a transposition).  The routed gate and up weights are E
 * matrices [I][D], down E matrices [D][I]; the shared gate and up one matrix
 * [n_shared I_shared][D], the shared down n_shared matrices [D][I_shared]. */
int beam_moe_pack_weights(const void *w, int32_t mats, int32_t rows,
                          int32_t cols, void *packed, void *stream);

/* Mask-router training step: the loss value and straight-through gradient.
 * (BEAM page on aitrends.kr, method paragraph, training strategy: L = L_lm +
 * alpha L_bal + beta L_reg with L_reg = (1/K) sum_{i in TK} |m_hat_i|; the
 * straight-through estimator passes m_hat's gradient through the
 * binarisation, dm/dm_hat := 1.)  Over the batch, L_reg is the mean over the
 * T tokens.  Given dy = dL_lm/dy [T][D] (layer dtype) and beta, writes
 *   *lreg         L_reg (one fp32, device memory)
 *   dwm [E][D]    dL/dWm = sum over top-K candidates (t, k) of expert e of
 *                 dL/dz_k x_t, dL/dz_k = (g_k <dy_t, E_k(x_t)> + beta/(T K))
 *                 m_hat_k (1 - m_hat_k), with g the unmasked top-K softmax
 *                 and E_k evaluated for every candidate, masked or not
 *   dbm [E]       dL/db_m (same sums of dL/dz_k), or NULL to skip
 * all fp32, overwritten, device pointers (dwm 16-byte aligned).  Runs the
 * router and every candidate's expert, so it costs a plain top-K MoE forward;
 * needs the same workspace as beam_moe_forward.  Only the method's own gate
 * (gating 0) with per-token routing (segment_len <= 1) is supported
 * (otherwise BEAM_ERR_UNSUPPORTED).  Results are deterministic.  */
int beam_moe_mask_backward(const beam_moe_layer *layer, const void *x,
                           const void *dy, int32_t T, float beta, float *dwm,
                           float *dbm, float *lreg, void *ws, size_t ws_bytes,
                           void *stream);

/* Work accounting from the device expert counts of a route/forward call:
 * copies expert_count [E] (the expert_count field of a beam_route_out, or
 * any device array of E counts) to the host and SYNCHRONISES the stream.
 * Avg-K and FLOPs as defined above (aitrends.kr results paragraph;
 * chatpaper.ai abstract). */
int beam_moe_stats(const beam_moe_layer *layer, const int32_t *expert_count,
                   int32_t T, beam_stats *host_out, void *stream);

/* Same accounting (Avg-K and FLOPs as above) from host-resident counts [E];
 * touches no GPU. */
int beam_moe_stats_host(const beam_moe_layer *layer,
                        const int32_t *expert_count_host, int32_t T,
                        beam_stats *host_out);

/* Static, human-readable name of a status code. */
const char *beam_status_str(int status);

/* ---- Measurement helpers (not part of the layer) ------------------------ */

/* Per-kernel timing: while enabled, every kernel that route/forward launch is
 * bracketed by a pair of hipEvents recorded on the call's stream.  Up to
 * max_launches launches are recorded; later ones run untimed.  Not thread
 * safe; meant for a single benchmarking thread.  Host-side setup only. */
int beam_profile_begin(int32_t max_launches);

/* Waits for the recorded events, then reports per kernel name: number of
 * timed launches and their summed duration in ms.  names[i] receives a
 * pointer to a static string.  Returns the number of distinct kernels
 * (capped at max_out) and disables the profiler. */
int beam_profile_end(const char **names, int32_t *launches, double *total_ms,
                     int32_t max_out);

/* Plain device copy kernel (16-byte vector loads and stores) of `bytes`
 * (multiple of 16) from src to dst; used to calibrate memory counters. */
int beam_copy_kernel(void *dst, const void *src, size_t bytes, void *stream);

/* MFMA throughput probe: `blocks` workgroups of 4 waves, each wave running
 * `iters` rounds of four independent bf16 32x32x16 MFMA accumulation chains
 * on registers (blocks * iters * 4 * 4 * 32768 FLOPs per launch); one float
 * per thread is written to out [blocks * 256] so the work is kept.  Used to
 * measure the dense bf16 MFMA rate the chip sustains. */
int beam_mfma_loop(float *out, int32_t blocks, int32_t iters, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* BEAM_MOE_H */
