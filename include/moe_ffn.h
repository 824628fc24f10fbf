/*
 * moe_ffn.h — C ABI of the MI355X (gfx950) MoE feed-forward block.
 *
 * The block (Gemma 4 26B-A4B feed-forward layer):
 *   - router: z = x . W_r (+ optional per-expert bias b), softmax over all
 *     experts, keep the top_k largest, renormalise the kept weights to sum
 *     to 1 (archdb page "Gemma-4-26B-A4B": gating function softmax; selected
 *     expert weights renormalized; 128 routed experts, 8 selected per token).
 *     Equal logits go to the lower expert id.
 *   - routed experts: bias-free GeGLU MLPs
 *       E_e(x) = (gelu_tanh(x . Wg[e]) * (x . Wu[e])) . Wd[e]
 *     (archdb fields "FFN activation": GeGLU with tanh-approximate GELU;
 *     "FFN projections have bias terms": No; expert width 704).
 *   - always-on dense branch: the same GeGLU form with width 2112
 *     (gemma-llm API page gm.nn.Gemma4_26B_A4B, model description: every
 *     layer also has one dense MLP of width 2112 that all tokens pass through).
 *   - output: out[t] = sum_j w[t,j] * E_{e_j}(x_t) + Dense(x_t).
 * A config with num_experts = 0 is a plain dense feed-forward block: the
 * dense branch alone, no router (gemma-llm API page gm.nn.Gemma4_E4B:
 * enable_moe False, num_experts 0, embed_dim 2560, hidden_dim 10240).
 *
 * Data layout (all row-major, all caller-owned DEVICE memory unless noted):
 *   x        [T, H]      bf16
 *   router_w [H, E]      bf16  (never quantised: the NVFP4 checkpoint config
 *                               lists router.proj under "ignore"; NULL iff
 *                               num_experts == 0, as are router_b and w_*)
 *   router_b [E]         fp32 or NULL
 *   w_gate   [E, H, I]   bf16  (matrix e is [K=H, N=I], N contiguous)
 *   w_up     [E, H, I]   bf16
 *   w_down   [E, I, H]   bf16
 *   d_gate   [H, D]      bf16  (NULL iff dense_dim == 0)
 *   d_up     [H, D]      bf16
 *   d_down   [D, H]      bf16
 *   out      [T, H]      bf16
 * bf16 is passed as raw 16-bit storage (void*).  Every pointer must be
 * 16-byte aligned.
 *
 * NVFP4 weight-only matrices (NVFP4 checkpoint config, quantization_config
 * group_0.weights: 4-bit float e2m1 values, group_size 16, float8_e4m3fn
 * group scales, strategy tensor_group) are passed per projection as a
 * moe_ffn_nvfp4_t of G matrices (G = E for experts, 1 for the dense branch),
 * each [K, N] matrix stored out-major:
 *   q            [G, N, K/2] uint8: value (n,k) in byte q[g,n,k/2], low
 *                             nibble for even k
 *   scale        [G, N, K/16] uint8: float8_e4m3fn group scales
 *   tensor_scale [G] fp32
 *   w = e2m1(code) * e4m3(scale) * tensor_scale.
 *
 * FP8 weight-only matrices (a reading of the SFP8 footprint quoted for the
 * 26B model on the inference-research page: 28.8 GB against 57.7 GB in
 * BF16, i.e. one byte per weight; the page defines no encoding): OCP
 * float8_e4m3fn codes in the bf16 weights' [K, N] layout, one fp32 scale per
 * matrix, passed per projection as a moe_ffn_fp8_t of G matrices:
 *   q            [G, K, N] uint8 float8_e4m3fn
 *   tensor_scale [G] fp32
 *   w = e4m3(q) * tensor_scale.
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 * stream).  Every call that takes a stream only queues work on it and
 * returns at once; no call synchronises the device except when the
 * environment variable MOE_FFN_SYNC=1 is set (then each call waits for its
 * kernels and reports their errors).  No call allocates device memory after
 * moe_ffn_create, so a forward can be captured into a HIP graph.
 *
 * Errors: every entry point returns MOE_FFN_OK or a negative code and never
 * lets an exception cross the ABI; moe_ffn_last_error() gives the message
 * of the calling thread's last failure.  Arguments are validated before any
 * work is queued: a failing call has queued nothing.
 *
 * Concurrency: a handle owns one workspace, so at most one forward per
 * handle may be in flight; calls on one handle from two streams at once are
 * undefined.  Distinct handles are independent.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_ffn_handle moe_ffn_handle; /* opaque */

enum {
  MOE_FFN_OK = 0,
  MOE_FFN_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad T, bad handle */
  MOE_FFN_ERR_UNSUPPORTED = -2, /* shape or format this library does not run */
  MOE_FFN_ERR_HIP = -3,         /* a HIP runtime call or launch failed */
  MOE_FFN_ERR_OOM = -4          /* workspace allocation failed at create */
};

enum { MOE_FFN_W_BF16 = 0, MOE_FFN_W_NVFP4 = 1, MOE_FFN_W_FP8 = 2 };

/* config flags */
enum { MOE_FFN_ACCUMULATE = 1u << 0 }; /* out += block(x) (residual stack); out may alias x */

/* execution variants (moe_ffn_set_variant) */
enum {
  MOE_FFN_VARIANT_AUTO = 0,   /* weight streaming for small T, MFMA tiles for large T */
  MOE_FFN_VARIANT_STREAM = 1, /* force weight streaming (bf16 weights, T <= 64; else MFMA) */
  MOE_FFN_VARIANT_MFMA = 2    /* force MFMA tiles (any T) */
};

typedef struct {
  int32_t hidden;        /* H: 2816 (multiple of 256, at most 4096) */
  int32_t num_experts;   /* E: 128 (multiple of 4, 4..256), or 0: a dense FFN
                            (then top_k = expert_dim = 0 and dense_dim > 0,
                            else INVALID_ARG) */
  int32_t top_k;         /* k: 8 (1..min(E,16)) */
  int32_t expert_dim;    /* I: 704 (multiple of 64, at most 4096) */
  int32_t dense_dim;     /* D: 2112 (multiple of 64, at most 16384), or 0: no dense branch */
  int32_t max_tokens;    /* largest T a forward on this handle may use (>= 1);
                            x [T, H], h [T*k, I] and h_d [T, D] in bf16 must each
                            stay below 2 GiB at T = max_tokens */
  int32_t weight_format; /* MOE_FFN_W_BF16, MOE_FFN_W_NVFP4 or MOE_FFN_W_FP8 */
  uint32_t flags;        /* MOE_FFN_ACCUMULATE or 0 */
} moe_ffn_config;

typedef struct {
  const uint8_t *q;           /* [G, N, K/2] e2m1 codes, two per byte */
  const uint8_t *scale;       /* [G, N, K/16] float8_e4m3fn group scales */
  const float *tensor_scale;  /* [G] fp32 per-matrix scale */
} moe_ffn_nvfp4_t;

typedef struct {
  const uint8_t *q;           /* [G, K, N] float8_e4m3fn codes (N contiguous) */
  const float *tensor_scale;  /* [G] fp32 per-matrix scale */
} moe_ffn_fp8_t;

/* Bytes of device workspace a handle with this config allocates at create.
 * Returns INVALID_ARG for NULL pointers, UNSUPPORTED for shapes the library
 * does not run. */
int moe_ffn_workspace_bytes(const moe_ffn_config *cfg, size_t *bytes);

/* Validate cfg, allocate the workspace on the current HIP device, and return
 * a handle bound to that device.  On failure *out_handle is set to NULL. */
int moe_ffn_create(const moe_ffn_config *cfg, moe_ffn_handle **out_handle);

/* Free the workspace and the handle (waits for the handle's device to go
 * idle first).  NULL is accepted and ignored. */
int moe_ffn_destroy(moe_ffn_handle *h);

/* Force an execution variant for later forwards (tests and benchmarks). */
int moe_ffn_set_variant(moe_ffn_handle *h, int32_t variant);

/* Forward of the block for T tokens with bf16 weights (weight_format must be
 * MOE_FFN_W_BF16).  0 <= T <= max_tokens; T == 0 queues nothing.
 * router_bias may be NULL; d_gate/d_up/d_down must be NULL iff dense_dim==0;
 * router_w, router_bias and w_gate/w_up/w_down must be NULL iff
 * num_experts == 0 (INVALID_ARG otherwise).
 * With MOE_FFN_ACCUMULATE, out holds the residual on entry and receives
 * residual + block(x) (out == x allowed); otherwise out must not overlap x. */
int moe_ffn_forward(moe_ffn_handle *h, int32_t T, const void *x, const void *router_w,
                    const float *router_bias, const void *w_gate, const void *w_up,
                    const void *w_down, const void *d_gate, const void *d_up,
                    const void *d_down, void *out, void *stream);

/* The forward above for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no handle, no hipMalloc/hipFree, no allocating library call.
 * Its workspace is a static device array of 64 MiB that the library holds on
 * every GPU it runs on until the process ends (a shape and T whose workspace,
 * moe_ffn_workspace_bytes of cfg with max_tokens = T, exceeds 64 MiB return
 * UNSUPPORTED; at the 26B-A4B shape T <= 446 fits).  cfg (host memory) gives
 * the shape, weight_format (must be MOE_FFN_W_BF16) and flags; T must be in
 * [0, cfg->max_tokens]; every other argument, the validation and the result
 * are those of moe_ffn_forward on the current device.  Each call first clears
 * the counters the kernels need at zero.  Every call on one GPU shares that
 * GPU's array: two calls that overlap on one GPU (two streams, or two host
 * threads) race and give undefined results; calls on different GPUs are
 * independent.  Nothing of the call can be read back afterwards (no routing
 * or intermediates). */
int moe_ffn_forward_noalloc(const moe_ffn_config *cfg, int32_t T, const void *x, const void *router_w,
                            const float *router_bias, const void *w_gate, const void *w_up,
                            const void *w_down, const void *d_gate, const void *d_up,
                            const void *d_down, void *out, void *stream);

/* Same block with NVFP4 weight-only expert and dense matrices (weight_format
 * must be MOE_FFN_W_NVFP4).  Activations, router and output stay bf16; each
 * weight tile is decoded to bf16 on chip (an e2m1 x e4m3 product is exact in
 * bf16) and the fp32 tensor scale is applied to the fp32 accumulator.  The
 * dense descriptors must have NULL members iff dense_dim == 0, the expert
 * descriptors (and router_w) iff num_experts == 0. */
int moe_ffn_forward_nvfp4(moe_ffn_handle *h, int32_t T, const void *x, const void *router_w,
                          const float *router_bias, const moe_ffn_nvfp4_t *w_gate,
                          const moe_ffn_nvfp4_t *w_up, const moe_ffn_nvfp4_t *w_down,
                          const moe_ffn_nvfp4_t *d_gate, const moe_ffn_nvfp4_t *d_up,
                          const moe_ffn_nvfp4_t *d_down, void *out, void *stream);

/* Same block with FP8 weight-only expert and dense matrices (weight_format
 * must be MOE_FFN_W_FP8; the layout is given above).  Activations, router
 * and output stay bf16.  Small T streams the one-byte codes (half the bytes
 * of bf16) and widens them to fp32 in registers; the MFMA tiles convert each
 * weight tile to bf16 on chip (exact: e4m3 has 3 mantissa bits).  The fp32
 * per-matrix scale multiplies the fp32 sums.  Expert descriptors (and
 * router_w) must be NULL iff num_experts == 0, dense descriptors iff
 * dense_dim == 0; q must be 16-byte aligned, tensor_scale 4-byte aligned. */
int moe_ffn_forward_fp8(moe_ffn_handle *h, int32_t T, const void *x, const void *router_w,
                        const float *router_bias, const moe_ffn_fp8_t *w_gate, const moe_ffn_fp8_t *w_up,
                        const moe_ffn_fp8_t *w_down, const moe_ffn_fp8_t *d_gate,
                        const moe_ffn_fp8_t *d_up, const moe_ffn_fp8_t *d_down, void *out,
                        void *stream);

/* Same block with NVFP4 weights AND NVFP4 activations (W4A4; the NVFP4
 * checkpoint config's input_activations: e2m1 values, groups of 16 along K,
 * float8_e4m3fn group scales computed per call, a static global scale per
 * tensor).  weight_format must be MOE_FFN_W_NVFP4 and num_experts > 0.
 * in_scale: device fp32 [3], the static global scales of x (the input of
 * every gate/up projection), of the routed hidden rows h and of the dense
 * hidden rows h_d (unused when dense_dim == 0); each must be positive and
 * finite (a NaN scale gives undefined output).  Every 16-value group of a
 * row is quantised as
 *   s_g = e4m3(amax / (6 s)),  q = e2m1(v / (s_g s))   (nearest, ties to
 *   even, saturating; each operation one correctly rounded fp32 step),
 * and the projection reads q * s_g * s.  The router reads x unquantised.
 * Runs on the MFMA tiles for every T: the quantised values q * s_g are exact
 * in bf16, so the bf16 MFMA computes with them exactly and s joins the
 * weights' tensor scale on the fp32 accumulators. */
int moe_ffn_forward_w4a4(moe_ffn_handle *h, int32_t T, const void *x, const void *router_w,
                         const float *router_bias, const moe_ffn_nvfp4_t *w_gate, const moe_ffn_nvfp4_t *w_up,
                         const moe_ffn_nvfp4_t *w_down, const moe_ffn_nvfp4_t *d_gate,
                         const moe_ffn_nvfp4_t *d_up, const moe_ffn_nvfp4_t *d_down, const float *in_scale,
                         void *out, void *stream);

/* The NVFP4 activation quantiser of moe_ffn_forward_w4a4 on its own: rows x K
 * bf16 values (row-major, K a multiple of 16) to the bf16 values q * s_g of
 * each 16-group (the global scale *in_scale, device fp32, is not applied).
 * in == out is allowed.  Queues one kernel on `stream` on the current device;
 * needs no handle. */
int moe_ffn_quant_act_nvfp4(int64_t rows, int32_t K, const void *in, void *out, const float *in_scale,
                            void *stream);

/* The feed-forward sub-block of a layer with its sandwich norms and the
 * residual (archdb page "Gemma-4-26B-A4B": normalization RMSNorm, placement
 * sandwich (pre and post), epsilon 1e-06; API page gm.nn.Gemma4_26B_A4B
 * use_post_ffw_norm=True), bf16 weights:
 *   xn  = bf16(RMSNorm(x) * pre_scale)            RMSNorm(v) = v / sqrt(mean(v^2) + eps)
 *   out = x + RMSNorm(block(xn)) * post_scale     block = the forward above
 * One pre-norm feeds the router, the experts and the dense branch; one
 * post-norm acts on their sum (the pages show one norm on each side of the
 * block).  pre_scale, post_scale: [H] fp32 device gains as applied (a
 * checkpoint's stored offset, if any, is the caller's), 16-byte aligned.
 * eps finite and >= 0 (the pages' value is 1e-6).  out may be x (in place);
 * otherwise they must not overlap.  The handle must not carry
 * MOE_FFN_ACCUMULATE (the sub-block adds its own residual: UNSUPPORTED).
 * Routing and intermediates of the call describe block(xn).  The pre-norm
 * is timed with MOE_FFN_STAGE_ROUTE, the post-norm with the combine. */
int moe_ffn_forward_block(moe_ffn_handle *h, int32_t T, const void *x, const float *pre_scale,
                          const float *post_scale, float eps, const void *router_w,
                          const float *router_bias, const void *w_gate, const void *w_up,
                          const void *w_down, const void *d_gate, const void *d_up,
                          const void *d_down, void *out, void *stream);

/* Device-to-device copies of the routing of the last forward (or of the
 * last moe_ffn_align_only) into caller buffers; any destination may be NULL.
 *   topk_idx [T, k] int32 (ascending expert id per token), topk_w [T, k]
 *   fp32 (aligned with topk_idx), counts [E] int32, offsets [E+1] int32,
 *   perm [T*k] int32 (token of each expert-grouped row), pos [T*k] int32
 *   (row of slot (t, j)).  topk_w is not written by moe_ffn_align_only.
 * The weight-streaming variant never builds the grouping tables (its
 * kernels derive each expert's rows from topk_idx); after such a forward
 * this call first queues the grouping kernels on `stream`.  UNSUPPORTED for
 * a config without experts. */
int moe_ffn_get_routing(moe_ffn_handle *h, int32_t *topk_idx, float *topk_w, int32_t *counts,
                        int32_t *offsets, int32_t *perm, int32_t *pos, void *stream);

/* Intermediates of the last forward copied into caller device buffers;
 * any destination may be NULL.  h [T*k, I] bf16 (GeGLU hidden of each
 * routed row, expert-grouped order), y [T*k, H] bf16 (expert output per
 * row, same order), h_d [T, D] bf16 and y_d [T, H] bf16 (dense branch).
 * The weight-streaming variant keeps routed rows in (token, slot) order;
 * after such a forward this call queues the grouping kernels and a copy
 * into grouped order on `stream`.  A dense FFN (num_experts == 0) forward
 * on the MFMA tiles without MOE_FFN_ACCUMULATE writes its rows straight to
 * out, so asking for y_dense after it returns UNSUPPORTED. */
int moe_ffn_get_intermediates(moe_ffn_handle *h, void *h_rows, void *y_rows, void *h_dense,
                              void *y_dense, void *stream);

/* Test hook: run only the expert grouping (counts, offsets, perm, pos and
 * the tile lists) on caller-given routing topk_idx [T, k] int32 (device),
 * each row holding k distinct ids in [0, E) in ascending order.
 * UNSUPPORTED for a config without experts. */
int moe_ffn_align_only(moe_ffn_handle *h, int32_t T, const int32_t *topk_idx, void *stream);

/* Per-stage timing with HIP events recorded on the forward's stream.
 * Stages: */
enum {
  MOE_FFN_STAGE_ROUTE = 0,   /* router logits + top-k; streaming: the same
                                launch also runs the dense branch's gate/up */
  MOE_FFN_STAGE_ALIGN = 1,   /* grouping kernels (MFMA variant only) */
  MOE_FFN_STAGE_GATEUP = 2,  /* gate/up: MFMA = the routed + dense GEMM with the
                                GeGLU fused; streaming = the routed partial sums
                                and the dense ones the router launch left */
  MOE_FFN_STAGE_DOWN = 3,    /* down projections, routed + dense; streaming
                                with experts and bf16 weights: each down unit
                                forms its GeGLU rows from the gate/up partials */
  MOE_FFN_STAGE_COMBINE = 4, /* weighted sum + dense add */
  MOE_FFN_STAGE_GEGLU = 5,   /* streaming with FP8 weights or without
                                experts: GeGLU of the summed partials (else it
                                runs inside the down stage) */
  MOE_FFN_NUM_STAGES = 6
};
/* Start recording an event pair around every stage in stage_mask (bit s =
 * stage s) for each of the next max_samples forwards (later forwards are
 * not timed).  Creates host-side event objects only; forwards stay
 * asynchronous.  Not for forwards captured into a graph. */
int moe_ffn_profile_begin(moe_ffn_handle *h, uint32_t stage_mask, int32_t max_samples);
/* Wait for the recorded events, write the summed duration (ms) and the
 * number of timed launches of each stage into total_ms[MOE_FFN_NUM_STAGES]
 * and samples[MOE_FFN_NUM_STAGES] (either may be NULL), and stop recording. */
int moe_ffn_profile_end(moe_ffn_handle *h, float *total_ms, int32_t *samples);

/* Message of the calling thread's last failure ("" if none); never NULL. */
const char *moe_ffn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
