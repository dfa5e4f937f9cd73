/*
 * mxmoe.h -- C ABI of the MI355X (gfx950) sparse MoE layer with MXFP4 expert
 * weights and MXFP8 activations.
 *
 * The operation (one MoE layer, one GPU):
 *   router   : logits l = x W_r^T + b; per token the top_k experts by logit
 *              (ties -> lower index), weights w = sigmoid(l)/sum sigmoid(l)
 *              over the selected experts.  The pages give the router as
 *              "top-16" over 896 experts ("Kimi K3 Tech Intro", section 4.3
 *              "MXFP4 MoE + SiTU"; section 1 architecture table); the sigmoid
 *              score and the renormalisation are the readings taken.
 *   permute  : (token, slot) pairs regrouped expert by expert, tokens in
 *              ascending order inside an expert.
 *   quantise : x -> MXFP8 (E4M3 elements, one E8M0 scale per 32 elements
 *              along d): "MXFP4 weights and MXFP8 activations" ("Kimi K3 ...
 *              MoE推理系统工程分析"); bit formats per OCP MX v1.0.
 *   experts  : per routed and shared expert, [g | u] = A W_gu^T (MXFP8 x MXFP4,
 *              fp32 accumulate), h = silu(g) * u (SwiGLU, standing in for the
 *              SiTU activation the pages name but do not define), h -> MXFP8
 *              along d_ff, o = h W_dn^T.  Routed experts plus shared experts
 *              ("Kimi K3 Tech Intro", section 4.3; 2 shared per
 *              "Kimi K3本地部署指南", section 1 spec table).
 *   combine  : y[t] = sum_j w[t,j] o_(t,j) + sum_s o_s[t] (fp32, fixed order),
 *              rounded to bf16.
 *
 * Layouts (all device memory, all owned by the caller):
 *   x          bf16  [T][d_model] row-major
 *   y          bf16  [T][d_model] row-major
 *   router_w   fp32  [E][d_model];  router_b fp32 [E] or NULL (zero bias)
 *   Expert weights in canonical MXFP4 form are, per expert,
 *     W_gu  [2*d_ff][d_model]  (rows [0,d_ff) gate, [d_ff,2 d_ff) up)
 *     W_dn  [d_model][d_ff]
 *   each as codes u8 [rows][K/2] (E2M1 pairs, element 2i in the low nibble of
 *   byte i) and scales u8 [rows][K/32] (E8M0), K the reduction width.
 *   moe_forward takes them in that canonical form or in the packed tile
 *   order made by moe_pack_mx4 (below), and the caller says which in
 *   moe_weights.layout: MOE_WEIGHTS_CANONICAL or MOE_WEIGHTS_PACKED.  Either
 *   way gu_codes/gu_scales hold the E W_gu matrices back to back (same sizes
 *   in both forms), dn_codes/dn_scales the E W_dn matrices, sgu_* / sdn_*
 *   the shared ones, and the results are bit-identical.  The packed order is
 *   the fast one: a weight step of a 64-row group is one contiguous 4 KB and
 *   its scales one dword per lane, where the canonical form makes every
 *   copy a gather of 64-byte row pieces and 4-byte scale words.  Packing is
 *   a one-time load-time conversion.  A weight set with any other tag (for
 *   example a zero-initialised struct) is rejected with MOE_ERR_INVALID_ARG
 *   before anything is enqueued.
 *
 * Errors: every argument is checked on the host before anything is enqueued;
 * on an error nothing is written and the call returns a non-zero status
 * (details from moe_last_error(), thread-local).  Device work is enqueued on
 * `stream` (a hipStream_t, NULL = default stream) without host
 * synchronisation; asynchronous faults surface at the caller's next sync.
 * No call allocates or frees device memory.
 */
#ifndef MXMOE_H
#define MXMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad enum        */
  MOE_ERR_UNSUPPORTED = 2, /* shape outside what the kernels handle        */
  MOE_ERR_WORKSPACE = 3,   /* workspace missing, misaligned or too small   */
  MOE_ERR_DEVICE = 4       /* no usable gfx950 device or a launch failed   */
} moe_status;

typedef enum { MOE_SRC_BF16 = 0, MOE_SRC_FP32 = 1 } moe_src_dtype;

/* Layer shape.  d_model and d_ff: multiples of 128.  1 <= num_experts <= 1024.
 * 1 <= top_k <= min(32, num_experts).  0 <= num_shared <= 8.
 * 1 <= max_tokens <= 2^20.  flags: 0 (the layer with MXFP8 activations,
 * "A8W4") or MOE_FLAG_A16W4. */

/* The A16W4 variant ("Kimi K3 Tech Intro", sections 4.3 and 10 name A16W4
 * and A8W4 fused operators on MI355X): x stays bf16 into the gate_up
 * projection and h = silu(g)*u is rounded to bf16 (round to nearest even)
 * into the down projection; no MXFP8 activation anywhere; weights, router,
 * permutation and combine as in the A8W4 layer, at every token count: the
 * weight-streaming kernels below 24 rows per expert on average, 256-row
 * tiles on the bf16 MFMA from there on.  The x_codes, x_scales, h_codes and
 * h_scales taps must be NULL; h comes out through the h_bf16 tap. */
#define MOE_FLAG_A16W4 1u
typedef struct {
  int32_t d_model, d_ff, num_experts, top_k, num_shared;
  int64_t max_tokens;
  uint32_t flags;
} moe_config;

/* Opaque plan: host memory owned by the library; its shape is immutable after
 * moe_plan (only the optional profiling state below changes). */
typedef struct moe_plan_s moe_plan_t;

/* Layout tags of moe_weights.layout. */
#define MOE_WEIGHTS_CANONICAL 0x4E4E4143u /* every expert matrix as codes [N][K/2], scales [N][K/32] */
#define MOE_WEIGHTS_PACKED 0x3450584Du    /* every expert matrix made by moe_pack_mx4 */

typedef struct {
  const uint8_t *gu_codes, *gu_scales, *dn_codes, *dn_scales;
  const uint8_t *sgu_codes, *sgu_scales, *sdn_codes, *sdn_scales; /* NULL if num_shared==0 */
  const float *router_w;
  const float *router_b; /* may be NULL */
  uint32_t layout;       /* MOE_WEIGHTS_PACKED or MOE_WEIGHTS_CANONICAL */
} moe_weights;

/* Optional device outputs for inspection; each NULL pointer is skipped.
 * Permuted rows: R = T*top_k routed rows (expert-major, tokens ascending)
 * followed by num_shared blocks of T rows (shared expert s, token t at
 * T*top_k + s*T + t). */
/* Alignment: x_codes, x_scales, h_codes, h_scales, h_bf16, y_routed and
 * y_shared 16 bytes (the kernels move them in 16-byte pieces), every other
 * tap 4 bytes; a misaligned tap is rejected with MOE_ERR_INVALID_ARG. */
typedef struct {
  float *logits;          /* [T][E]   router logits incl. bias (fp32)        */
  int32_t *topk_ids;      /* [T][top_k] selected experts, ascending          */
  float *topk_w;          /* [T][top_k] routing weights                      */
  int32_t *expert_offsets;/* [E+1]    first permuted row of each expert      */
  int32_t *row_src;       /* [T*top_k] pair index t*top_k+j of each row      */
  int32_t *token_row;     /* [T][top_k] permuted row of each pair            */
  uint8_t *x_codes;       /* [T][d_model]  MXFP8 E4M3 codes of x             */
  uint8_t *x_scales;      /* [T][d_model/32] E8M0                            */
  uint8_t *h_codes;       /* [R][d_ff]     MXFP8 codes of h, permuted rows   */
  uint8_t *h_scales;      /* [R][d_ff/32]                                    */
  float *gu_acc;          /* [R][2*d_ff]   fp32 gate|up accumulators         */
  float *y_routed;        /* [T][d_model]  sum_j w o (fp32)                  */
  float *y_shared;        /* [T][d_model]  sum_s o_s (fp32)                  */
  uint16_t *h_bf16;       /* [R][d_ff] bf16 h, permuted rows (A16W4 only)    */
} moe_taps;

/* Packed MXFP4 matrix (one-time conversion at weight-load time).  For a
 * canonical matrix with `rows` rows (a multiple of 64) and reduction width k
 * (a multiple of 128): 64-row groups G, 128-wide K steps s, 16-row blocks
 * j = 0..3 of a group, lane l = 16*g + r (g = l/16, r = l%16), and
 *   row(G, j, r) = 64*G + 16*j + r                                (plain), or
 *   row(G, j, r) = (j/2)*(rows/2) + 32*G + 16*(j%2) + r      (interleave != 0:
 *                  group G pairs rows 32G..32G+31 of the two halves -- the
 *                  gate and up rows of the same outputs for W_gu):
 *   codes_p [rows/64][k/128][4][64][16]: entry (G, s, j, l) = canonical code
 *           bytes 64*s + 16*g .. +16 of row(G, j, r) (MX block 4*s + g);
 *   scales_p[rows/64][k/128][64][4]: byte j of entry (G, s, l) = canonical
 *           scale of row(G, j, r), block 4*s + g.
 * The four 16-row x 128-wide MFMA operands of a group and step are then 4 KB
 * contiguous in lane order, and their scales one dword per lane.
 * codes_p is rows*k/2 bytes; scales_p is moe_packed_scale_bytes(rows, k)
 * = rows*k/32 bytes (0 for sizes the layout does not cover). */
size_t moe_packed_scale_bytes(int64_t rows, int64_t k);
/* Pack `mats` matrices stored back to back (canonical codes [mats][rows][k/2],
 * scales [mats][rows][k/32]) into codes_p/scales_p (packed, back to back).
 * moe_forward expects W_gu (routed and shared) packed with interleave = 1 and
 * W_dn with interleave = 0.  Device buffers; codes and codes_p 16-byte
 * aligned, scales_p 4-byte aligned.  rows not a multiple of 64 or k not a
 * multiple of 128: MOE_ERR_UNSUPPORTED. */
moe_status moe_pack_mx4(const uint8_t *codes, const uint8_t *scales, int64_t mats, int64_t rows,
                        int64_t k, int interleave, uint8_t *codes_p, uint8_t *scales_p,
                        void *stream);

/* Validate `cfg` and build a plan (host only; no device call). */
moe_status moe_plan(const moe_config *cfg, moe_plan_t **out_plan);
void moe_plan_destroy(moe_plan_t *plan);

/* Bytes of device workspace moe_forward needs for num_tokens tokens. */
moe_status moe_workspace_bytes(const moe_plan_t *plan, int64_t num_tokens, size_t *out_bytes);

/* MXFP8-quantise rows of a bf16 or fp32 matrix along its columns: per row and
 * per 32 consecutive columns, e = clamp(floor(log2 amax) - 8, -127, 127)
 * (amax == 0 -> -127), codes = E4M3 round-to-nearest-even of v / 2^e with
 * saturation to +-448 (sign kept on zero), scale byte = e + 127.
 * src [rows][ld_src] (elements), codes [rows][cols], scales [rows][cols/32].
 * cols % 32 == 0, ld_src >= cols.  Inputs must be finite. */
moe_status moe_quantize_act(const void *src, moe_src_dtype dt, int64_t rows, int64_t cols,
                            int64_t ld_src, uint8_t *codes, uint8_t *scales, void *stream);

/* The whole layer for T = num_tokens tokens (0 <= T <= max_tokens; T == 0
 * enqueues nothing).  workspace: device memory of at least
 * moe_workspace_bytes(plan, T) bytes, 256-byte aligned; its contents on entry
 * do not matter.  Concurrent calls need distinct workspaces. */
moe_status moe_forward(const moe_plan_t *plan, const moe_weights *w, const void *x_bf16,
                       int64_t num_tokens, void *y_bf16, void *workspace, size_t workspace_bytes,
                       const moe_taps *taps, void *stream);

/* moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same layer, the same arguments and the same results as moe_forward, but the
 * workspace is a fixed scratch array of MOE_NOALLOC_SCRATCH_BYTES bytes that
 * the library's code object holds on every GPU it runs on, from the first
 * call on that device until the process ends.  The call allocates and frees
 * nothing and makes no host synchronisation.  Every call on one GPU uses that
 * GPU's one array and leaves its contents behind (no part of it has to start
 * at zero): calls that overlap on one GPU -- on two streams, or from two
 * threads without ordering -- race on it and must not be issued.  Token counts
 * whose moe_workspace_bytes exceeds MOE_NOALLOC_SCRATCH_BYTES are rejected
 * with MOE_ERR_WORKSPACE before anything is enqueued (at d_model = 7168,
 * 896 experts, top-16, d_ff = 2048, 2 shared: up to 256 tokens fit). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
moe_status moe_forward_noalloc(const moe_plan_t *plan, const moe_weights *w, const void *x_bf16,
                               int64_t num_tokens, void *y_bf16, const moe_taps *taps,
                               void *stream);

/* LatentMoE tail: y = MXFP8(RMSNorm(z)) W_up^T + s.  "Kimi K3 Tech Intro",
 * section 4.3 places a latent up-projection, an RMSNorm and an element-wise
 * add after the routed and shared experts; section 4.4 sends the routed
 * output through RMSNorm and the up projection and adds the shared output to
 * it directly.  Readings taken where the pages are silent: RMSNorm(z) =
 * z / sqrt(mean(z^2) + eps) * gamma per row; the normalised rows enter the
 * projection as MXFP8 (E4M3, one E8M0 scale per 32 columns, the quantiser of
 * moe_quantize_act) and W_up is MXFP4, like every other activation and weight
 * of the layer; fp32 accumulation; y rounded to bf16.
 *   z      fp32 [T][latent]   the routed experts' weighted sum (moe_forward's
 *                             y_routed tap when the experts run at the latent
 *                             width)
 *   s      fp32 [T][hidden]   the shared experts' output, or NULL (zero)
 *   y      bf16 [T][hidden]
 *   W_up   MXFP4 [hidden][latent], packed by moe_pack_mx4 with interleave 0
 *          (layout MOE_WEIGHTS_PACKED); gamma fp32 [latent]; or
 *          MOE_WEIGHTS_CANONICAL for W_up as codes [hidden][latent/2] and
 *          scales [hidden][latent/32].
 * latent and hidden: multiples of 128, both <= 65536;
 * 0 <= T <= 2^20 (T == 0 enqueues nothing); eps >= 0 and finite.
 * z, s, y, gamma and up_codes 16-byte aligned, up_scales 4 bytes; workspace
 * of moe_latent_tail_workspace_bytes bytes, 256-byte aligned, contents on
 * entry irrelevant.  Errors and streams as for moe_forward. */
typedef struct {
  const uint8_t *up_codes, *up_scales;
  const float *gamma;
  uint32_t layout; /* MOE_WEIGHTS_PACKED or MOE_WEIGHTS_CANONICAL */
} moe_tail_weights;

/* Optional device outputs (NULL = skip): the fp32 1/sqrt(mean(z^2)+eps) of
 * each row as computed (4-byte aligned) and the MXFP8 bytes of the normalised
 * rows (16-byte aligned). */
typedef struct {
  float *inv_rms;    /* [T]              */
  uint8_t *a_codes;  /* [T][latent]      */
  uint8_t *a_scales; /* [T][latent/32]   */
} moe_tail_taps;

moe_status moe_latent_tail_workspace_bytes(int64_t num_tokens, int32_t latent, int32_t hidden,
                                           size_t *out_bytes);
moe_status moe_latent_tail(int64_t num_tokens, int32_t latent, int32_t hidden, float eps,
                           const moe_tail_weights *w, const float *z, const float *s, void *y_bf16,
                           void *workspace, size_t workspace_bytes, const moe_tail_taps *taps,
                           void *stream);

/* One balancing step of the router bias from the expert loads of a forward:
 * b_e <- b_e + rate * sign(num_tokens*top_k/num_experts - c_e), with c_e =
 * expert_offsets[e+1] - expert_offsets[e] (moe_forward's expert_offsets tap
 * of that forward, num_tokens its token count): experts above the mean load
 * are made less likely, those below more likely.  "Kimi K3 Tech Intro"
 * (section 1 table, section 4.3) names "quantile balancing" for the router
 * without defining it; the router bias is the layer's only balancing hook,
 * and this step is the reading taken.  The sign is decided in integers, the
 * addition is one fp32 addition per expert.
 *   expert_offsets  int32 [E+1] device, 4-byte aligned
 *   router_b        fp32 [E] device, updated in place, 4-byte aligned
 *   rate            finite, >= 0
 * num_tokens == 0 enqueues nothing.  Errors and streams as for moe_forward. */
moe_status moe_router_bias_update(const moe_plan_t *plan, const int32_t *expert_offsets,
                                  int64_t num_tokens, float rate, float *router_b, void *stream);

/* Stages of moe_forward, for per-stage timing. */
typedef enum {
  MOE_STAGE_ROUTER = 0,  /* router logits                                   */
  MOE_STAGE_TOPK = 1,    /* top-k, routing weights, MXFP8 quantisation of x */
  MOE_STAGE_PERMUTE = 2, /* permutation and grouped-GEMM tile list          */
  MOE_STAGE_GATE_UP = 3, /* gate_up grouped GEMM + SwiGLU + MXFP8 of h      */
  MOE_STAGE_DOWN = 4,    /* down grouped GEMM                               */
  MOE_STAGE_COMBINE = 5, /* weighted combine -> y                           */
  MOE_NUM_STAGES = 6
} moe_stage;

/* Per-stage timing with HIP events recorded on the forward's stream: after
 * moe_profile_begin, each of the next max_calls (1..65536) moe_forward calls
 * on this plan records an event pair around every stage whose bit
 * (1u << stage) is set in stage_mask.  moe_profile_end waits for those events,
 * writes the summed milliseconds per stage to stage_ms[MOE_NUM_STAGES] (zero
 * for unrecorded stages) and the number of recorded calls to *calls, and stops
 * recording.  Host-side state of the plan; no device memory is allocated.
 * Each timed event pair leaves the GPU idle for a few microseconds between the
 * kernels it brackets, so calls being profiled are slower than plain ones.
 * Profiling a plan that is used by several threads at once is not supported. */
moe_status moe_profile_begin(moe_plan_t *plan, uint32_t stage_mask, int32_t max_calls);
moe_status moe_profile_end(moe_plan_t *plan, double *stage_ms, int32_t *calls);

const char *moe_status_string(moe_status s);
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MXMOE_H */
