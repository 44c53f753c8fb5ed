/*
 * moe.h -- C ABI of the MI355X (gfx950) Bailing/Ling mixture-of-experts FFN layer.
 *
 * The layer (sources: the model pages of the Ling / Bailing MoE family):
 *   router    logits = x W_r^T (+ optional router bias); scores = softmax over the
 *             experts (default) or sigmoid; an optional per-expert correction bias is
 *             added to a copy of the scores that is used for selection only
 *             [mlxcel #838 "Router: selection uses biased scores, weights come from
 *             unbiased scores"; Ling-2.6-flash-JANGTQ card, "Architecture
 *             (bailing_hybrid)", MoE routing paragraph];
 *   grouping  with n_group > 1 the experts form n_group contiguous groups, the
 *             topk_group best groups (group score: sum of the two largest biased
 *             scores) are kept, the other experts' selection scores are set to 0
 *             [mlxcel #838 "Architecture notes", "Defensive requirements"];
 *   top-k     the top_k experts by masked selection score; weights are the unbiased
 *             scores, renormalised by (sum + 1e-20) when top_k > 1 and
 *             norm_topk_prob, then always multiplied by routed_scaling_factor
 *             [mlxcel #838 "Router: ...", "moe_router_enable_routed_scaling is dead
 *             code upstream"];
 *   experts   SwiGLU MLP per expert: down(silu(gate x) * up x), weights stored
 *             [out, in] [mlxcel #838 "Validation checkpoint", "Weight remap"];
 *   combine   y = sum_j w_j expert_{S_j}(x) + shared(x), the shared expert being one
 *             MLP of width shared_intermediate added at weight 1.0
 *             [mlxcel #838 "Shared experts are one wide MLP, not N separate experts"].
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library never
 *     allocates or frees device memory, never synchronises the stream and never
 *     copies device data to the host.  Scratch memory is the caller's workspace,
 *     sized by moe_workspace_size().
 *   - Every call enqueues its kernels on `stream` (a hipStream_t; NULL = the null
 *     stream) and returns; outputs are valid once that stream's work completes.
 *   - All checks run on the host before anything is enqueued.  On an error nothing
 *     is launched, outputs are untouched, and moe_last_error() names the offending
 *     field or argument.  No C++ exception ever crosses this interface (the pages'
 *     "Defensive requirements": reject at load, never terminate at run time).
 *   - T == 0 is a valid no-op.
 *   - Row-major, densely packed tensors; all sizes are element counts.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* moe_stream_t; /* a hipStream_t */

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL_CONFIG = 1, /* a config field is out of range or inconsistent      */
  MOE_EINVAL_ARG = 2,    /* a null/misaligned pointer or a bad size             */
  MOE_EWORKSPACE = 3,    /* workspace missing or smaller than moe_workspace_size */
  MOE_EUNSUPPORTED = 4,  /* valid layer the gfx950 kernels do not implement      */
  MOE_EHIP = 5           /* a kernel launch failed (HIP runtime error)           */
} moe_status;

typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score_fn;

typedef enum {
  MOE_DT_F32 = 0,      /* IEEE fp32                                                  */
  MOE_DT_BF16 = 1,     /* bfloat16                                                    */
  MOE_DT_U8_AFFINE = 2, /* u8 code q + fp16 scale s + fp16 zero z per quant_group     */
                        /* consecutive elements of a row's reduction axis; w = s(q - z) */
  MOE_DT_U4_AFFINE = 3  /* the same with 4-bit codes q in [0, 15], two per byte along  */
                        /* the row: element 2i in the low nibble of byte i, 2i+1 in the */
                        /* high nibble.  Routed experts only; always runs the weight-   */
                        /* streaming path [4-bit routed experts: Ling-3.0-flash-GGUF     */
                        /* card, conversion recipe; the packing is not on the pages]     */
} moe_dtype;

typedef enum {
  MOE_PATH_AUTO = 0,    /* T <= 64, or at most min(20, 40960/hidden) routed tokens per
                           expert on average (T*top_k*max(hidden, 2048) <=
                           40960*num_experts): weight-streaming decode path; else the
                           tiled MFMA path */
  MOE_PATH_DECODE = 1,  /* force the weight-streaming path (any T)                      */
  MOE_PATH_PREFILL = 2  /* force the tiled grouped-GEMM path (bf16 activations only)    */
} moe_path;

/* Layer configuration.  Field names follow the Hugging Face config of the family
 * [mlxcel #838 "Config fields the checkpoint does not contain"]; defaults are those
 * of moe_config_default().                                                          */
typedef struct {
  int64_t hidden;              /* H                                                    */
  int64_t num_experts;         /* E, routed experts                                    */
  int64_t top_k;               /* k = num_experts_per_tok                              */
  int64_t moe_intermediate;    /* I, width of each routed expert                       */
  int64_t shared_intermediate; /* I_s = shared_dim * num_shared_experts; 0 = none      */
  int64_t n_group;             /* G (default 1 = no grouping)                          */
  int64_t topk_group;          /* g, groups kept when G > 1 (default 1)                */
  int32_t score_function;      /* moe_score_fn (default softmax)                       */
  int32_t norm_topk_prob;      /* 0/1 (default 1)                                      */
  int32_t use_expert_bias;     /* 0/1: selection-only correction bias (default 0)      */
  float routed_scaling_factor; /* always applied (default 1.0)                         */
  int32_t act_dtype;           /* x and y: MOE_DT_F32 or MOE_DT_BF16                   */
  int32_t router_dtype;        /* router weight: must equal act_dtype                  */
  int32_t expert_dtype;        /* routed experts: act_dtype, or U8/U4_AFFINE with bf16 x */
  int32_t shared_dtype;        /* shared expert: must equal act_dtype                  */
  int64_t quant_group;         /* 64 when expert_dtype is U8_AFFINE or U4_AFFINE       */
  int32_t path;                /* moe_path (default AUTO)                              */
} moe_config;

/* Weights of one layer (device pointers).  Layouts, [out, in] as in the checkpoint
 * [mlxcel #838 "Validation checkpoint"; stacked experts per "Weight remap"]:
 *   router       [E, H]  router_dtype
 *   router_bias  [E] fp32, nullable: added to the logits (the router's own bias)
 *   expert_bias  [E] fp32, the selection-only correction bias; required iff
 *                use_expert_bias
 *   gate, up     [E, I, H]; down [E, H, I]: expert_dtype (u8 codes when U8_AFFINE;
 *                packed u4 codes, [E, I, H/2] and [E, H, I/2] bytes, when U4_AFFINE)
 *   *_scale, *_zero  fp16 [E, I, H/quant_group] (gate, up) / [E, H, I/quant_group]
 *                (down); required iff expert_dtype is U8_AFFINE or U4_AFFINE (then
 *                4-byte aligned for U4_AFFINE), else ignored
 *   shared_gate, shared_up [I_s, H]; shared_down [H, I_s]: shared_dtype; required
 *                iff shared_intermediate > 0                                        */
typedef struct {
  const void* router;
  const float* router_bias;
  const float* expert_bias;
  const void* gate;
  const void* up;
  const void* down;
  const uint16_t* gate_scale;
  const uint16_t* gate_zero;
  const uint16_t* up_scale;
  const uint16_t* up_zero;
  const uint16_t* down_scale;
  const uint16_t* down_zero;
  const void* shared_gate;
  const void* shared_up;
  const void* shared_down;
} moe_weights;

/* Fills *cfg with the family's defaults (n_group 1, topk_group 1, softmax,
 * norm_topk_prob 1, no expert bias, routed_scaling_factor 1.0, bf16 everywhere,
 * quant_group 64, path AUTO) and zero sizes.  Never fails for a non-null cfg.    */
moe_status moe_config_default(moe_config* cfg);

/* Checks every field against the rules of the pages' "Defensive requirements"
 * (magnitude ceilings first, zero checks before divisibility, routing bounds):
 *   1 <= H <= 16384, 1 <= E <= 1024, 1 <= I <= 32768, 0 <= I_s <= 32768,
 *   1 <= k <= min(E, 16), G >= 1, 1 <= g <= G, and when G > 1: E % G == 0,
 *   E / G >= 2 (a group score needs two members), k <= g * E / G;
 *   score_function in {softmax, sigmoid}; routed_scaling_factor finite and > 0;
 *   flags in {0, 1}; dtype combination as documented in moe_config;
 *   quant_group == 64 for u8 and u4 experts.          -> MOE_EINVAL_CONFIG
 * Valid layers the kernels do not cover -> MOE_EUNSUPPORTED: H, I, I_s not
 * multiples of 64; G > 64; forced PREFILL path with fp32 activations; u4 experts
 * with H or I not multiples of 128, or with a forced PREFILL path.
 * Runs on the host only; needs no GPU.                                             */
moe_status moe_validate_config(const moe_config* cfg);

/* Bytes of device workspace a call with T tokens needs (the largest of
 * moe_route / moe_permute / moe_experts / moe_forward; one size fits all four).
 * The workspace is how this interface keeps the pages' ownership rule for the
 * native side: the caller owns every buffer and the library holds no device memory
 * of its own, so nothing is allocated, resized or freed behind the caller's back
 * [mlxcel #838 "Defensive requirements": validate at load, no failure at run time].
 * 0 <= T <= 2^20; the same config checks as moe_validate_config first.
 * Errors: MOE_EINVAL_CONFIG / MOE_EUNSUPPORTED (config), MOE_EINVAL_ARG (T out of
 * range, bytes null).  Needs no GPU.                                               */
moe_status moe_workspace_size(const moe_config* cfg, int64_t T, size_t* bytes);

/* The kernels a call with T tokens runs: *path_out = MOE_PATH_DECODE (weight-streaming
 * kernels) or MOE_PATH_PREFILL (tiled MFMA GEMMs), after cfg->path, the expert storage
 * (u4 experts always stream) and, for MOE_PATH_AUTO, the batch size rule documented
 * at moe_path.  Only the selected experts' weights are read on either path [Ling-3.0-
 * flash-GGUF card, "Measured performance"]; the choice changes speed, not results
 * beyond rounding.  Checks as moe_workspace_size.  Needs no GPU.                     */
moe_status moe_select_path(const moe_config* cfg, int64_t T, int32_t* path_out);

/* Router (steps: logits, scoring, correction bias, grouped mask, top-k, weights)
 * [mlxcel #838 "Router: selection uses biased scores, weights come from unbiased
 * scores" (the correction bias enters the selection copy only; renormalisation by
 * sum + 1e-20 when top_k > 1); "moe_router_enable_routed_scaling is dead code
 * upstream" (the factor is always applied); "Architecture notes" (groups kept,
 * the rest zeroed before top-k); Ling-2.6-flash-JANGTQ card, "Architecture
 * (bailing_hybrid)" (sigmoid, 8 groups -> top-4 groups -> top-8 experts)].
 *   x          [T, H] act_dtype
 *   router_w   [E, H] router_dtype; router_bias [E] fp32 nullable;
 *   expert_bias [E] fp32, required iff use_expert_bias
 *   topk_idx   [T, k] int32 out: experts by descending masked selection score,
 *              equal scores -> lower index first
 *   topk_w     [T, k] fp32 out: final routing weights (kept in fp32)
 *   ws         device workspace of ws_bytes >= moe_workspace_size(cfg, T)
 * Errors: MOE_EINVAL_CONFIG / MOE_EUNSUPPORTED (config), MOE_EINVAL_ARG (T out of
 * range; x or router_w null or not 16-byte aligned; a bias, topk_idx or topk_w null
 * where required or not 4-byte aligned), MOE_EWORKSPACE (ws null, not 256-byte
 * aligned or too small), MOE_EHIP (a launch failed).                               */
moe_status moe_route(const moe_config* cfg, int64_t T, const void* x, const void* router_w,
                     const float* router_bias, const float* expert_bias, int32_t* topk_idx,
                     float* topk_w, void* ws, size_t ws_bytes, moe_stream_t stream);

/* Token permutation by expert (histogram, exclusive scan, scatter): the grouping that
 * lets each selected expert's weights be read once per call [Ling-3.0-flash-GGUF
 * card, "Measured performance": decode reads only the selected experts].
 *   topk_idx  [T, k] int32 in; entries outside [0, E) are dropped (not counted)
 *   counts    [E] int32 out: slots routed to each expert
 *   offsets   [E + 1] int32 out: exclusive prefix sum of counts
 *   perm      [T * k] int32 out: slot ids t*k + j grouped by expert, expert e's run
 *             being perm[offsets[e] .. offsets[e+1]); the order inside a run is
 *             unspecified (the set is exact).  Trailing entries of dropped slots = -1.
 * Errors: as moe_route (topk_idx, counts, offsets, perm: non-null, 4-byte aligned).  */
moe_status moe_permute(const moe_config* cfg, int64_t T, const int32_t* topk_idx,
                       int32_t* counts, int32_t* offsets, int32_t* perm, void* ws,
                       size_t ws_bytes, moe_stream_t stream);

/* Expert stage with routing given by the caller (permutation, routed SwiGLU experts,
 * shared expert, weighted combine) [mlxcel #838 "Validation checkpoint" and "Weight
 * remap" (per-expert gate/up/down, gate_proj the SwiGLU gate); "Shared experts are
 * one wide MLP, not N separate experts" (weight 1.0, no routing)].
 *   x [T, H] act_dtype; w: layer weights (router fields unused);
 *   topk_idx [T, k] int32 (entries outside [0, E) contribute nothing);
 *   topk_w [T, k] fp32; y [T, H] act_dtype out.
 * Errors: as moe_route; weight pointers null or misaligned (16 bytes for matrices,
 * 2 bytes for u8 and 4 bytes for u4 scales and zero points) -> MOE_EINVAL_ARG.      */
moe_status moe_experts(const moe_config* cfg, int64_t T, const void* x, const moe_weights* w,
                       const int32_t* topk_idx, const float* topk_w, void* y, void* ws,
                       size_t ws_bytes, moe_stream_t stream);

/* The whole layer: y = MoE(x) = sum_j w_j expert_{S_j}(x) + shared(x)
 * [mlxcel #838 "Architecture notes" (router, routed experts and the shared expert of
 * one MoE layer) and "Shared experts are one wide MLP, not N separate experts" (the
 * shared output added at weight 1.0); the router as in moe_route].
 *   x [T, H] act_dtype; y [T, H] act_dtype out;
 *   topk_idx_out [T, k] int32, topk_w_out [T, k] fp32, expert_counts_out [E] int32:
 *   optional copies of the routing (nullable).
 * Errors: as moe_experts, plus the router pointers as moe_route.                     */
moe_status moe_forward(const moe_config* cfg, int64_t T, const void* x, const moe_weights* w,
                       void* y, int32_t* topk_idx_out, float* topk_w_out,
                       int32_t* expert_counts_out, void* ws, size_t ws_bytes,
                       moe_stream_t stream);

/* The whole layer as moe_forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The scratch memory is a fixed device array of the library,
 * MOE_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held from the library's first use on
 * that GPU until the process ends; the caller passes only inputs and outputs.  The
 * call allocates nothing and runs every launch on `stream` (no second stream).
 *   Same arguments, layouts and results as moe_forward without ws / ws_bytes.
 *   Limit: moe_workspace_size(cfg, T) <= MOE_NOALLOC_SCRATCH_BYTES (every decode
 *   batch of the family's layers; prefill batches up to several hundred tokens);
 *   larger calls -> MOE_EWORKSPACE with the bytes needed, nothing launched.
 *   Concurrency: all calls on one GPU share its scratch array; calls that overlap in
 *   time on one GPU (two streams, two host threads) race and give wrong results, so
 *   the caller serialises them.  No state carries over between calls: every kernel
 *   writes the scratch it reads within the same call.
 * Errors: as moe_forward, plus MOE_EHIP if the array's device address cannot be
 * obtained.                                                                         */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_forward_noalloc(const moe_config* cfg, int64_t T, const void* x, const moe_weights* w,
                               void* y, int32_t* topk_idx_out, float* topk_w_out,
                               int32_t* expert_counts_out, moe_stream_t stream);

/* Dense MLP of the layers in front of the MoE layers (`first_k_dense_replace`):
 *   y = (silu(x W_gᵀ) ⊙ (x W_uᵀ)) W_dᵀ
 * A plain gated MLP at the model's intermediate size [mlxcel #838 "Architecture
 * notes": the first_k_dense_replace layers before the MoE layers are dense MLPs;
 * Ling-2.6-flash-JANGTQ card, "Architecture" layer table: layer 0 is a dense MLP of
 * intermediate 9216].  It is the shared expert's computation and runs on its kernels
 * (weight streaming for T <= 192, tiled MFMA above).
 *   cfg          hidden, act_dtype and path are read; routing and expert fields are not
 *   intermediate MLP width I_d: a multiple of 64 in [64, 32768]
 *   x [T, H] and y [T, H] act_dtype; gate, up [I_d, H] and down [H, I_d] act_dtype
 *                (16-byte aligned device pointers)
 *   ws           device workspace of ws_bytes >= moe_dense_workspace_size(cfg, I_d, T)
 * Errors: MOE_EINVAL_CONFIG (hidden, act_dtype or path out of range), MOE_EUNSUPPORTED
 * (hidden or I_d not a multiple of 64; PREFILL with fp32), MOE_EINVAL_ARG (null or
 * misaligned pointers, I_d or T out of range), MOE_EWORKSPACE, MOE_EHIP.           */
moe_status moe_dense_workspace_size(const moe_config* cfg, int64_t intermediate, int64_t T, size_t* bytes);
moe_status moe_dense_mlp(const moe_config* cfg, int64_t intermediate, int64_t T, const void* x,
                         const void* gate, const void* up, const void* down, void* y, void* ws,
                         size_t ws_bytes, moe_stream_t stream);

/* Kernel timing with HIP events (for benchmarks).  While enabled, every launch of a
 * stage in `stage_mask` is bracketed by a pair of events recorded on its launch
 * stream, taken from a pool of `capacity` pairs created here (launches beyond the
 * pool are not timed).  moe_profile_collect() waits for the recorded events and
 * returns the summed duration and count of one stage's timed launches; the pool is
 * then reused from its start.  moe_profile_disable() destroys the pool.  Not
 * thread-safe: enable, run and collect from one host thread.  Needs a GPU.        */
typedef enum {
  MOE_STAGE_ROUTER = 1,      /* router logits                          */
  MOE_STAGE_TOPK = 2,        /* scoring, grouped mask, top-k, weights  */
  MOE_STAGE_PERMUTE = 4,     /* histogram, scan, scatter               */
  MOE_STAGE_UP = 8,          /* routed gate/up + SwiGLU                */
  MOE_STAGE_DOWN = 16,       /* routed down (weighted)                 */
  MOE_STAGE_SHARED_UP = 32,  /* shared gate/up + SwiGLU (tiled path)   */
  MOE_STAGE_SHARED_DOWN = 64,/* shared down + combine (tiled path)     */
  MOE_STAGE_COMBINE = 128    /* standalone combine                     */
} moe_stage;
moe_status moe_profile_enable(int32_t stage_mask, int32_t capacity);
moe_status moe_profile_collect(int32_t stage, float* total_ms, int32_t* launches);
moe_status moe_profile_disable(void);
moe_status moe_profile_reset(void); /* forget recorded pairs, keep the pool and mask */

/* Static description of a status code.  Every entry point reports failure as a
 * status value, never by throwing or aborting [mlxcel #838 "Defensive requirements":
 * invalid input is rejected when it is loaded, with an error, instead of failing
 * later].                                                                          */
const char* moe_status_str(moe_status s);

/* Message of the last failed call on this thread ("" when none).  It names the
 * offending config field or argument and the value it had [mlxcel #838 "Defensive
 * requirements": the error names the actual field].  The string stays valid until
 * the next call on this thread.                                                     */
const char* moe_last_error(void);

/* ABI version (incremented on any change of the structs or signatures).            */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
