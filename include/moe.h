/*
 * moe.h -- C ABI of libmoe.so: the forward and backward passes of one
 * mixture-of-experts layer on one AMD Instinct MI355X (gfx950), with the
 * routing variants (expert choice, a selection-only balancing bias and its
 * update, a per-sequence balance statistic).
 *
 * The layer (sources by page title and section):
 *   gating      p_e(x) = softmax(g(x))_e, g(x) = W_r x (+ b)
 *               ["MoE技术演进", "Adaptive Mixtures of Local Experts", gating equation]
 *   selection   top-k experts per token, optionally inside the best groups
 *               ["MoE技术演进", "DeepSeek-V2" item 3, device-limited routing]
 *               or per routing head inside the head's own expert partition
 *               ["多头 LatentMoE 与 Head Parallel", 方法论 items 1-2]
 *   keep rule   capacity C per expert, overflow through the residual
 *               ["MoE技术演进", "GShard" item 1]; or keep the best 90 % per
 *               expert by affinity ["MoE技术演进", "DeepSeek-V2" item 5];
 *               or no dropping ["MoE技术演进", "DeepSeek-V3" item 5]
 *   experts     FFN_e(u) = W2 relu(W1 u)  ["MoE技术演进", "GShard" item 3]
 *               or W2 (SiLU(W1 u) * W3 u) ["大语言模型并行策略（七）：专家并行",
 *               "MoE 模型的参数量分析": 3 d_model x d_moe matrices]
 *   combine     h = sum_shared FFN_i(u) + sum_kept g_e FFN_e(u) + u
 *               ["MoE技术演进", "DeepSeekMoE" item 2, shared-expert equation]
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless marked [host].  Matrices are
 *     row-major; weights use the [out, in] layout, so both operands of every
 *     product are contiguous along the contracted dimension.
 *   - The caller allocates every buffer, the workspace included.  The library
 *     never allocates or frees device memory, never synchronises the stream
 *     and keeps no pointer after a call returns.  Calls are reentrant.
 *   - Every call is asynchronous on `stream` and returns a moe_status.  All
 *     argument checks run on the host before anything is launched: a failed
 *     check launches nothing.  A launch failure returns MOE_ERR_HIP; with the
 *     environment variable MOE_DEBUG set, the failing launch and HIP's
 *     reason are also written to stderr.  A call clears HIP's last-error
 *     state (hipGetLastError) before its first launch, so an error that an
 *     earlier, unrelated HIP call left there is neither reported nor kept.
 *   - Row counts that depend on routing (R = kept assignments) are never read
 *     back to the host: buffers sized by R use moe_rows_upper_bound(), and
 *     the true R is offsets[E] on the device.  When that bound is 0 (capacity
 *     0), the buffers sized by it may be NULL.
 *   - "act" tensors (activations and expert weights) have cfg->act_dtype;
 *     the router weight has cfg->router_dtype; gates, logits, bias and the
 *     aux loss are float32; indices are int32.
 *   - The workspace `ws` must hold at least moe_workspace_bytes(cfg) bytes and
 *     be 256-byte aligned; its contents need not be initialised.
 *   - Every other device pointer must be 16-byte aligned (the kernels move
 *     16-byte vectors); a misaligned one returns MOE_ERR_ARG before any launch.
 *   - The library reads every field of the structs below as laid out in this
 *     header; fields are only ever appended, and each addition raises
 *     MOE_ABI_VERSION.  Zero-initialise a struct and set the fields you use
 *     (a NULL optional pointer is "not asked for").  A caller that may load a
 *     library built from another version of this header compares
 *     moe_abi_version() with its own MOE_ABI_VERSION before the first call:
 *     a library that reads fields the caller's structs do not have would read
 *     past them.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = -1,          /* null pointer, bad size or inconsistent config */
  MOE_ERR_UNSUPPORTED = -2,  /* valid request outside what the kernels support */
  MOE_ERR_WORKSPACE = -3,    /* ws_bytes < moe_workspace_bytes(cfg) or misaligned */
  MOE_ERR_HIP = -4           /* a HIP launch reported an error */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;
typedef enum { MOE_ACT_RELU = 0, MOE_ACT_SWIGLU = 1 } moe_act;
typedef enum { MOE_DROP_NONE = 0, MOE_DROP_CAPACITY = 1, MOE_DROP_AFFINITY = 2 } moe_drop;
/* Who chooses ["jiqizhixin.com article on LocMoE+", router-taxonomy paragraph]:
 *   TOKEN_CHOICE   every token picks top_k experts (per head)
 *   EXPERT_CHOICE  every expert picks its top-C tokens by gate, C = capacity.
 *                  Each token then has K = E assignment slots, slot j being
 *                  expert j (topk_idx[t][j] = j, topk_w[t][j] = p_{t,j}); the
 *                  keep rule is the experts' choice: per expert the min(C, T)
 *                  largest gates are kept, equal gates to the earlier token.
 *                  Requires n_heads == 1, n_groups == 0, renorm == 0,
 *                  latent_proj == 0 and drop == MOE_DROP_CAPACITY (the C);
 *                  top_k is not used. */
typedef enum { MOE_ROUTE_TOKEN_CHOICE = 0, MOE_ROUTE_EXPERT_CHOICE = 1 } moe_route_mode;
typedef enum {
  MOE_LOGITS_COMPUTE = 0,        /* compute scores from x and W_r; logits buffer unused (may be NULL) */
  MOE_LOGITS_COMPUTE_STORE = 1,  /* compute, and also write them to `logits` */
  MOE_LOGITS_LOAD = 2            /* read final scores (bias included) from `logits`; x, W_r, bias unused */
} moe_logits_mode;

/* [host] Layer shape and rules.  All fields are int32 so the layout is fixed. */
typedef struct moe_config {
  int32_t T;            /* tokens, >= 0 (T == 0: every call is a no-op returning MOE_OK) */
  int32_t d_model;      /* width of x and y; multiple of 64 */
  int32_t n_heads;      /* H >= 1 routing heads */
  int32_t d_head;       /* expert input width d_e; multiple of 64; with H == 1 and no latent
                           projection it equals d_model; otherwise H*d_head is the latent width */
  int32_t n_experts;    /* E routed experts in total, E = H * E_h, 1 <= E_h <= 256, E <= 1024 */
  int32_t top_k;        /* experts chosen per head, 1 <= top_k <= min(E_h, 8) */
  int32_t n_groups;     /* group-limited routing: groups per head (0 = off); divides E_h, <= 32 */
  int32_t topk_groups;  /* groups kept per token, 1..n_groups; top_k <= topk_groups*(E_h/n_groups) */
  int32_t renorm;       /* 1: chosen gates divided by their sum */
  int32_t drop;         /* moe_drop */
  int32_t capacity;     /* MOE_DROP_CAPACITY: integer C >= 0 (computed by the caller) */
  int32_t keep_num;     /* MOE_DROP_AFFINITY: keep ceil(keep_num*n_e/keep_den) of expert e's */
  int32_t keep_den;     /*   n_e assignments; 0 < keep_num <= keep_den */
  int32_t d_ff;         /* expert hidden width; multiple of 64 */
  int32_t act;          /* moe_act */
  int32_t n_shared;     /* always-active shared experts (H == 1 only), each d_ff wide */
  int32_t latent_proj;  /* 1: z = x W_in^T before routing and o W_out^T + x after */
  int32_t residual;     /* 1: combine adds the layer input (ignored with latent_proj: the
                           residual is added after the output projection) */
  int32_t act_dtype;    /* moe_dtype of activations and expert weights */
  int32_t router_dtype; /* moe_dtype of W_r; MOE_BF16 requires act_dtype == MOE_BF16 */
  int32_t route_mode;   /* moe_route_mode */
  int32_t sel_bias_gate;/* with a selection bias (moe_weights.sel_bias): 1 the gate of a chosen
                           expert is p + b (the formula as the page prints it), 0 it is p */
  int32_t seq_len;      /* > 0: report the per-sequence balance statistic over runs of seq_len
                           consecutive tokens (T % seq_len == 0, n_heads == 1); 0: off */
} moe_config;

/* Weights of one layer (device pointers; [out, in] layout). */
typedef struct moe_weights {
  const void *w_router;     /* [E, d_head] (== [H, E_h, d_head]), router_dtype */
  const float *router_bias; /* [E] or NULL: added to the scores before softmax and selection */
  const void *w1;           /* [E, d_ff, d_head]  gate projection (the only one for ReLU) */
  const void *w3;           /* [E, d_ff, d_head]  up projection (SwiGLU) or NULL (ReLU) */
  const void *w2;           /* [E, d_head, d_ff]  down projection */
  const void *ws1;          /* [n_shared*d_ff, d_model] shared experts, hidden widths concatenated */
  const void *ws3;          /* [n_shared*d_ff, d_model] (SwiGLU) or NULL */
  const void *ws2;          /* [d_model, n_shared*d_ff] */
  const void *w_in;         /* [H*d_head, d_model] latent in-projection, or NULL */
  const void *w_out;        /* [d_model, H*d_head] latent out-projection, or NULL */
  const float *sel_bias;    /* [E] float32 or NULL: balancing bias added to the probabilities for
                               the top-k choice only (token choice; see moe_route) */
} moe_weights;

/* Optional outputs and intermediates of moe_layer_fwd.  Every pointer may be
 * NULL; a NULL intermediate lives in the workspace instead.  Shapes use
 * K = H*top_k assignments per token and R_max = moe_rows_upper_bound(cfg). */
typedef struct moe_layer_io {
  float *logits;            /* [T, E] float32; role set by logits_mode */
  int32_t logits_mode;      /* moe_logits_mode; LOAD requires logits != NULL */
  int32_t *topk_idx;        /* [T, K] */
  float *topk_w;            /* [T, K] */
  int32_t *demand;          /* [E]  assignments per expert before the keep rule */
  int32_t *counts;          /* [E]  kept assignments per expert */
  int32_t *offsets;         /* [E+1] exclusive prefix sum of counts; offsets[E] = R */
  int32_t *row_of;          /* [T, K] row of each assignment in x_perm, -1 if dropped */
  int32_t *src_of;          /* [R_max] flat assignment (t*K + j) held by each row */
  float *aux_loss;          /* [1] GShard auxiliary loss (H == 1 only) */
  float *seq_loss;          /* [T / seq_len] per-sequence balance statistic (seq_len > 0), or NULL */
  void *z;                  /* [T, H*d_head] act: latent (latent_proj only) */
  void *x_perm;             /* [R_max, d_head] act: expert-contiguous expert inputs; if
                               NULL, none is written and the expert FFN reads its rows
                               from x (or z) directly (moe_expert_ffn_gather) */
  void *y_perm;             /* [R_max, d_head] act: expert outputs, same row order */
  void *shared_out;         /* [T, d_model] act: sum of the shared experts (n_shared > 0) */
  void *o;                  /* [T, H*d_head] act: combined head outputs (latent_proj only) */
  void *gu;                 /* [R_max, 2*d_ff] (SwiGLU: gate, then up) or [R_max, d_ff] (ReLU) act,
                               or NULL: the routed experts' pre-activations, rows as y_perm.
                               moe_layer_fwd writes them and moe_layer_bwd reads them instead
                               of recomputing the gate/up products, for layers whose routed
                               experts run the grouped GEMM (not the fused narrow-expert MLP:
                               bf16 with d_head 64, 128 or 256); ignored otherwise.  Pass the
                               same buffer to both calls, or NULL to both. */
} moe_layer_io;

/* [host] Workspace bytes every call below needs for `cfg` (0 for an invalid cfg). */
size_t moe_workspace_bytes(const moe_config *cfg);

/* [host] Upper bound on R, the number of kept assignments:
 * T*H*top_k for MOE_DROP_NONE / MOE_DROP_AFFINITY, min(T*top_k, E*C) for
 * MOE_DROP_CAPACITY, E*min(C, T) for expert choice.  -1 for an invalid cfg. */
int64_t moe_rows_upper_bound(const moe_config *cfg);

/* [host] Static string naming a moe_status value. */
const char *moe_status_str(int status);

/* Layout version of the structs in this header (see the conventions above). */
#define MOE_ABI_VERSION 1

/* [host] The MOE_ABI_VERSION the library was built with. */
int32_t moe_abi_version(void);

/* [host] MOE_OK if `cfg` is valid and supported, else the error moe_* calls would return.
 * Supported sizes: T*K, T*max(d_model, H*d_head, m*d_ff, m*n_shared*d_ff),
 * d_ff*d_head, n_shared*d_ff*d_model and H*d_head*d_model below 2^31
 * (m = 2 for SwiGLU, else 1; the GEMM addresses one group's operands with
 * 32-bit element offsets); MOE_ERR_UNSUPPORTED otherwise. */
int moe_check_config(const moe_config *cfg);

/*
 * moe_route -- scores, softmax, top-k and gates of every token.
 * ["MoE技术演进", "Adaptive Mixtures of Local Experts" (gating equation and
 * top-K selector); "GShard" item 1 (aux-loss equation); "DeepSeek-V2" item 3
 * (device-limited routing, here over expert groups); "多头 LatentMoE 与 Head
 * Parallel", 方法论 item 2 (per-head choice within a fixed partition)]
 *
 *   x         [T, H*d_head] act: router input (the latent z when latent_proj)
 *   w_router  [E, d_head] router_dtype; head h uses rows [h*E_h, (h+1)*E_h)
 *             and reads columns [h*d_head, (h+1)*d_head) of x
 *   bias      [E] float32 or NULL
 *   logits    [T, E] float32, per `mode` (a moe_logits_mode)
 *   topk_idx  [T, H*top_k] out: global expert ids (h*E_h + local); the k
 *             entries of a head are ordered by score descending, lower expert
 *             index first on equal scores (-0.0 and +0.0 are equal)
 *   topk_w    [T, H*top_k] out: softmax probability of each chosen expert over
 *             its head's E_h experts, divided by the chosen sum if cfg->renorm;
 *             evaluated in float64 and rounded to float32 once
 *   aux_loss  [1] float32 out or NULL: sum_e m_e * c_e / T with m_e the mean
 *             probability and c_e the number of choices of e; H == 1 only
 *             (MOE_ERR_UNSUPPORTED otherwise)
 * Expert choice (cfg->route_mode): topk_idx/topk_w are [T, E] with slot j =
 * expert j and the gate p_{t,j}; the experts choose in moe_dispatch.
 * Scores must be finite; non-finite scores give unspecified routing.
 * One kernel launch (two with aux_loss).
 */
int moe_route(const moe_config *cfg, const void *x, const void *w_router, const float *bias,
              float *logits, int mode, int32_t *topk_idx, float *topk_w,
              float *aux_loss, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_route_ex -- moe_route with the routing variants' extra inputs and outputs.
 * Arguments as for moe_route, plus:
 *   sel_bias  [E] float32 or NULL: balancing bias ["MoE技术演进", "DeepSeek-V3"
 *             item 1].  The top-k (and group scores) are taken on the float32
 *             keys p + b instead of the scores; the gate of a chosen expert is
 *             p + b if cfg->sel_bias_gate, else p (then renormalised if
 *             cfg->renorm).  Token choice only (MOE_ERR_UNSUPPORTED otherwise).
 *   seq_loss  [T / seq_len] float32 out or NULL (requires cfg->seq_len > 0):
 *             for each run of seq_len consecutive tokens, sum_e f_e P_e with
 *             f_e = (choices of e in the run) / seq_len and P_e the mean
 *             probability of e over the run ["MoE技术演进", "DeepSeek-V3"
 *             item 4: the sequence-wise balance loss is alpha times this]
 * moe_route(...) is moe_route_ex with sel_bias = seq_loss = NULL.
 */
int moe_route_ex(const moe_config *cfg, const void *x, const void *w_router, const float *bias,
                 const float *sel_bias, float *logits, int mode, int32_t *topk_idx, float *topk_w,
                 float *aux_loss, float *seq_loss, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_sel_bias_update -- one step of the balancing-bias update
 * ["MoE技术演进", "DeepSeek-V3" item 1: the bias of an overloaded expert falls
 * by gamma, that of an underloaded one rises by gamma (gamma = 0.001 there)].
 * Per head h: with n_e the load of expert e (e.g. moe_dispatch's demand) and
 * N_h the head's total, b_e -= gamma if n_e * E_h > N_h, b_e += gamma if
 * n_e * E_h < N_h, unchanged at the mean (integer comparison).
 *   load      [E] int32 in;  sel_bias [E] float32 in/out
 */
int moe_sel_bias_update(const moe_config *cfg, const int32_t *load, float *sel_bias, float gamma,
                        hipStream_t stream);

/*
 * moe_dispatch -- keep rule and permutation of tokens into an expert-contiguous buffer.
 * ["MoE技术演进", "GShard" item 1 (capacity C, overflow through the residual);
 * "DeepSeek-V2" item 5 (keep the top 90 % by affinity); "DeepSeek-V3" item 5
 * (no dropping); "大语言模型并行策略（七）：专家并行", "MoE 中的 all-to-all 通信"
 * (count tokens per expert, then fill each expert's buffer)]
 *
 * Flat assignment a = t*K + j (K = H*top_k), expert e(a) = topk_idx[a].
 *   NONE      every assignment kept
 *   CAPACITY  a kept iff fewer than C earlier assignments (smaller a) chose e(a)
 *   AFFINITY  per expert, the ceil(keep_num*n_e/keep_den) assignments with the
 *             largest topk_w are kept (equal gates: smaller a first)
 *   expert choice (cfg->route_mode): per expert, the min(C, T) assignments
 *             with the largest topk_w are kept (equal gates: smaller a first);
 *             K = E and a = t*E + e: slot j of every token is expert j (as
 *             moe_route writes it), so topk_idx is not read in this mode
 *
 *   topk_idx  [T, K] in, values in [0, E) (out-of-range values: undefined behaviour)
 *   topk_w    [T, K] in; read for AFFINITY and expert choice (may be NULL otherwise)
 *   x         [T, H*d_head] act: expert inputs (x, or z when latent_proj)
 *   demand    [E] out, counts [E] out, offsets [E+1] out (offsets[E] = R)
 *   row_of    [T, K] out: row of a in x_perm, or -1 if dropped
 *   src_of    [R_max] out: rows [0, R) hold the flat index of their assignment;
 *             rows of expert e are [offsets[e], offsets[e+1]) in ascending a
 *   x_perm    [R_max, d_head] act out: row r = columns [h*d_head, (h+1)*d_head)
 *             of x[src_of[r] / K], h = e(src_of[r]) / E_h (bitwise copy); may be
 *             NULL: then nothing is copied and x is not read (may be NULL too)
 * Results are deterministic (integer work only, no order-dependent atomics).
 */
int moe_dispatch(const moe_config *cfg, const int32_t *topk_idx, const float *topk_w,
                 const void *x, int32_t *demand, int32_t *counts, int32_t *offsets,
                 int32_t *row_of, int32_t *src_of, void *x_perm,
                 void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_dispatch_noalloc -- moe_dispatch for callers that cannot allocate or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Arguments, results and errors as for moe_dispatch,
 * without ws/ws_bytes: its scratch (per-chunk expert histograms and, for the
 * affinity rule and expert choice, the expert-sorted assignment list) lives in
 * a library-held device array of 8 MiB per GPU, allocated with the library's
 * code object and held until the process ends.  A configuration that needs
 * more (moe_dispatch's scratch grows with T*K and E) returns MOE_ERR_WORKSPACE
 * before any launch.  The array belongs to the current device: `stream` must be
 * a stream of the current device.  Every call on one GPU uses the same array,
 * so calls that overlap on one GPU (different streams, or threads) race;
 * calls in order on one stream do not.  The kernels overwrite every scratch
 * byte they read, so no clearing is needed between calls.  The entry point
 * itself allocates nothing and never synchronises.
 */
int moe_dispatch_noalloc(const moe_config *cfg, const int32_t *topk_idx, const float *topk_w, const void *x,
                         int32_t *demand, int32_t *counts, int32_t *offsets, int32_t *row_of, int32_t *src_of,
                         void *x_perm, hipStream_t stream);

/*
 * moe_check_topk -- checked mode for caller-supplied routing, to run before moe_dispatch.
 * [the top-K selector of "MoE技术演进", "Adaptive Mixtures of Local Experts":
 * each token names K distinct experts; per head inside the head's own experts,
 * "多头 LatentMoE 与 Head Parallel", 方法论 item 2]
 *
 * moe_dispatch's behaviour is undefined for a topk_idx it could not have got
 * from moe_route; this call tells whether one is such.  It counts the slots of
 * topk_idx [T, K] that name an expert outside their head's range
 * [h*E_h, (h+1)*E_h) (h = slot / top_k) or repeat an expert an earlier slot of
 * the same token and head named (expert choice: every slot j must be expert j),
 * and writes the count to *status: 0 means valid.
 *   topk_idx  [T, K] int32 in (device)
 *   status    [1] int32 out (device); written by one launch, so the caller may
 *             read it after synchronising the stream, or pass it on to its own
 *             kernels
 * Errors: MOE_ERR_ARG for a bad config or a NULL pointer.  One launch of one
 * block; allocates nothing, never synchronises.
 */
int moe_check_topk(const moe_config *cfg, const int32_t *topk_idx, int32_t *status, hipStream_t stream);

/*
 * moe_expert_ffn -- every routed expert on its rows of x_perm, plus the shared experts.
 * ["MoE技术演进", "GShard" item 3 (FFN_e); "DeepSeekMoE" item 2 (shared experts);
 * "大语言模型并行策略（七）：专家并行", "MoE 模型的参数量分析" (SwiGLU, 3 matrices)]
 *
 *   x_perm     [R_max, d_head] act, offsets [E+1] (from moe_dispatch)
 *   w1, w3, w2 per-expert weights (moe_weights layout); w3 NULL for ReLU
 *   y_perm     [R_max, d_head] act out: row r = FFN_e(x_perm[r]) for the expert
 *              e owning row r; rows >= offsets[E] untouched
 *   x_shared   [T, d_model] act (the layer input) or NULL when n_shared == 0
 *   ws1, ws3, ws2, shared_out [T, d_model] act out: sum over shared experts
 * Products accumulate in float32; the hidden activation is rounded to act_dtype.
 */
int moe_expert_ffn(const moe_config *cfg, const void *x_perm, const int32_t *offsets,
                   const void *w1, const void *w3, const void *w2, void *y_perm,
                   const void *x_shared, const void *ws1, const void *ws3, const void *ws2,
                   void *shared_out, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_expert_ffn_gather -- moe_expert_ffn with the token-to-expert copy fused
 * into the expert kernel's operand loads: no x_perm is read or written.
 * ["多头 LatentMoE 与 Head Parallel", 方法论 item 4 (IO-aware kernels: the
 * token-to-expert transfer is batched and fused with the expert computation,
 * cutting memory copies)]
 *
 *   x        [T, H*d_head] act: the expert inputs moe_dispatch was given (x, or z)
 *   src_of   [R_max], offsets [E+1] (from moe_dispatch, whose x_perm may be NULL)
 * Row r of expert e is read from x[src_of[r] / K], columns [h*d_head,
 * (h+1)*d_head), h = e / E_h: the row x_perm[r] would hold.  y_perm and
 * shared_out are bitwise those of moe_expert_ffn on that x_perm.  Other
 * arguments and errors as for moe_expert_ffn; additionally T * H * d_head
 * must be below 2^31 (MOE_ERR_UNSUPPORTED otherwise).
 */
int moe_expert_ffn_gather(const moe_config *cfg, const void *x, const int32_t *src_of,
                          const int32_t *offsets, const void *w1, const void *w3, const void *w2,
                          void *y_perm, const void *x_shared, const void *ws1, const void *ws3,
                          const void *ws2, void *shared_out, void *ws, size_t ws_bytes,
                          hipStream_t stream);

/*
 * moe_combine -- gate-weighted sum of the expert outputs, plus shared output and residual.
 * ["MoE技术演进", "GShard" item 3 (y_s = sum_e G_{s,e} FFN_e(x_s)); "DeepSeekMoE"
 * items 1-2 (+ u_t and the ungated shared experts)]
 *
 * For column c of head h = c / d_head:
 *   y[t, c] = residual[t, c] + shared_out[t, c]
 *             + sum_{j in head h, row_of[t,j] >= 0} topk_w[t,j] * y_perm[row_of[t,j], c - h*d_head]
 * accumulated in float32 in that order (residual, shared, then j ascending)
 * and rounded once.  A dropped assignment adds nothing.
 *   y_perm [R_max, d_head] (NULL allowed when R_max is 0), row_of [T, K], topk_w [T, K]
 *   residual [T, H*d_head] act or NULL, shared_out [T, H*d_head] act or NULL
 *   y [T, H*d_head] act out (the layer output when H == 1; o when latent_proj)
 */
int moe_combine(const moe_config *cfg, const void *y_perm, const int32_t *row_of,
                const float *topk_w, const void *residual, const void *shared_out, void *y,
                hipStream_t stream);

/*
 * moe_layer_fwd -- the whole layer: [z = x W_in^T] -> route -> dispatch ->
 * expert FFN (+ shared) -> combine -> [y = o W_out^T + x].  One stream, no host
 * synchronisation.  Without io->x_perm the expert FFN gathers its rows from the
 * expert input directly (as moe_expert_ffn_gather); y is the same either way.  x [T, d_model] act in, y [T, d_model] act out (distinct
 * from x).  `io` may be NULL.  Sources as for the four calls above, and
 * "多头 LatentMoE 与 Head Parallel", 方法论 item 1 (latent routing space).
 * A multi-head latent layer with top-1 per head, nothing dropped and a fused
 * expert MLP (bf16, d_head 64, 128 or 256) runs its combine inside the
 * expert FFN: io->o is then bitwise what moe_combine writes, and io->y_perm
 * is written only when given (the backward needs it).
 */
int moe_layer_fwd(const moe_config *cfg, const moe_weights *w, const void *x, void *y,
                  moe_layer_io *io, void *ws, size_t ws_bytes, hipStream_t stream);

/* ============================================================ backward
 * Gradients of  L = sum_t <dy_t, y_t> + aux_weight * l_aux
 *                  + seq_weight * sum_s sum_e f_{s,e} P_{s,e}  with the
 * forward's discrete decisions (top-k choice, keep rule) held fixed: those are
 * piecewise constant, so the gradient flows through the gate values, the
 * experts, the router probabilities, the shared experts, the residual and,
 * for the multi-head latent layer, the two projections (per head: softmax,
 * renormalisation and router over the head's own experts and slice).
 * ["MoE技术演进", "GShard" item 3 (FFN_e and the gate-weighted sum), item 1
 * (aux loss); "DeepSeekMoE" items 1-2 (gates, shared experts, residual);
 * "Adaptive Mixtures of Local Experts" (softmax gating equation);
 * "大语言模型并行策略（七）：专家并行", "MoE 模型的参数量分析" (SwiGLU experts);
 * "多头 LatentMoE 与 Head Parallel", 方法论 items 1-2 (latent space, heads)]
 */

/* Transposed weights for the backward products (caller-allocated, act dtype;
 * m = 2 for SwiGLU, 1 for ReLU):
 *   w13t  [E, d_head, m*d_ff]        row c of expert e = (W1[e][:, c], W3[e][:, c])
 *   w2t   [E, d_ff, d_head]          W2[e]^T
 *   ws13t [d_model, m*n_s*d_ff]      (Ws1[:, c], Ws3[:, c]); NULL when n_shared == 0
 *   ws2t  [n_s*d_ff, d_model]        Ws2^T;                 NULL when n_shared == 0
 *   w_in_t  [d_model, H*d_head]      W_in^T;                NULL without latent_proj
 *   w_out_t [H*d_head, d_model]      W_out^T;               NULL without latent_proj */
typedef struct moe_weights_t {
  void *w13t, *w2t, *ws13t, *ws2t, *w_in_t, *w_out_t;
} moe_weights_t;

/* Gradient outputs.  Weight gradients have the weights' shapes; expert and
 * shared-expert gradients are act_dtype, router gradients float32. */
typedef struct moe_grads {
  void *dx;          /* [T, d_model] act */
  float *dw_router;  /* [E, d_head] float32 */
  float *dbias;      /* [E] float32, or NULL */
  void *dw1, *dw3, *dw2;     /* [E, d_ff, d_head], [E, d_ff, d_head] (SwiGLU), [E, d_head, d_ff] */
  void *dws1, *dws3, *dws2;  /* shared experts (n_shared > 0) */
  void *dw_in, *dw_out;      /* [H*d_head, d_model], [d_model, H*d_head] (latent_proj) */
} moe_grads;

/* [host] Workspace bytes moe_layer_bwd needs (0 when cfg is invalid or the
 * backward does not support it). */
size_t moe_backward_workspace_bytes(const moe_config *cfg);

/* moe_transpose_weights -- fill `wt` from `w` (once per weight update). */
int moe_transpose_weights(const moe_config *cfg, const moe_weights *w, const moe_weights_t *wt,
                          hipStream_t stream);

/*
 * moe_layer_bwd -- the layer backward.
 *   w, wt      forward weights and their transposes (moe_transpose_weights)
 *   x          [T, d_model] act: the forward input
 *   dy         [T, d_model] act: upstream gradient of y
 *   aux_weight coefficient of l_aux in L (0: no aux term)
 *   seq_weight coefficient of the summed per-sequence balance terms in L
 *              (the statistic moe_route reports; alpha on the page,
 *              "MoE技术演进", "DeepSeek-V3" item 4); requires cfg->seq_len
 *              when nonzero (0: no such term)
 *   io         the forward's state: logits (the forward's scores, bias
 *              included: run it with MOE_LOGITS_COMPUTE_STORE), topk_idx,
 *              topk_w, demand, offsets, row_of, src_of, y_perm -- all
 *              required; with latent_proj also z and o
 *   g          gradient outputs (dbias may be NULL; shared ones required when
 *              n_shared > 0; dw3 required for SwiGLU; dw_in and dw_out with
 *              latent_proj)
 * Products accumulate in float32 and round once to act_dtype (weight
 * gradients per expert over all its rows); the router gradients stay float32.
 * Per-row and per-token sums run in a fixed order: results are bitwise
 * reproducible.  aux_weight must be 0 when n_heads > 1 (the aux loss is
 * defined for one head); a selection bias inside renormalised gates
 * (sel_bias_gate with renorm) is MOE_ERR_UNSUPPORTED.
 */
int moe_layer_bwd(const moe_config *cfg, const moe_weights *w, const moe_weights_t *wt, const void *x,
                  const void *dy, float aux_weight, float seq_weight, const moe_layer_io *io, moe_grads *g,
                  void *ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
