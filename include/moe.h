/*
 * moe.h - C ABI of the MI355X (gfx950) Mixture-of-Experts SwiGLU
 * feed-forward forward pass (libmoe.so).
 *
 * The layer (APEX-1 Mathematical Reference - Part 3, section 13.2):
 *
 *   MoE(x) = sum_s Expert_s(x)  +  sum_k g_k * Expert_{e_k}(x)
 *            (shared, always on)   (routed, top-K selected)
 *
 *   Expert(x) = W_down (SiLU(W_gate x) * (W_up x))        (section 12.2)
 *
 * computed as: fp32 router -> top-K and weights -> stable sorted dispatch of
 * the T*K (token, slot) assignments by expert -> grouped SwiGLU GEMMs over
 * contiguous expert slices -> atomic-free combine through the inverse
 * permutation, plus the shared experts.
 *
 * Conventions that hold for every entry point:
 *  - Pointers to tensors are DEVICE pointers to caller-owned memory. The
 *    library never allocates, frees or keeps a pointer after it returns.
 *    Descriptor structs are host memory, read during the call only.
 *  - Matrices are row-major and dense. Weights are stored "out x in", as a
 *    linear layer stores them: W_gate[e] is [d_ff, d_e], so W_gate x is a
 *    product with the transpose of the page's d x d_ff matrix.
 *  - act_dtype (MOE_F32 or MOE_BF16) is the type of x, of every expert,
 *    shared and latent weight, of the routed rows and of out. The router
 *    weight, the balance bias, the routing weights g and the RMSNorm gain
 *    are always fp32.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *    stream). No call synchronises with the host: outputs are valid once
 *    the stream has reached that point.
 *  - Return value: MOE_OK, or a negative moe_status. Arguments are checked
 *    on the host before anything is launched; a failed check launches
 *    nothing. MOE_ERR_HIP reports a launch failure.
 *  - Device arrays of activations, weights, routed rows, outputs, gradients
 *    and workspaces must be 16-byte aligned (the kernels move 16-byte
 *    chunks; torch's allocations are); index and count arrays need only
 *    their element's alignment.
 *  - T = 0 is valid and launches nothing. Experts that receive no tokens
 *    cost nothing (APEX-1 docs "10 - Mixture of Experts", BUG-08: an expert
 *    may get 0, 1 or many tokens).
 *  - Inputs must be finite; NaN / Inf behaviour is unspecified.
 *  - The library has no mutable global state apart from moe_forward_noalloc's
 *    per-device scratch (below); calls on different streams with disjoint
 *    outputs and workspaces may run concurrently.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,      /* a required pointer is NULL                      */
  MOE_ERR_SHAPE = -2,     /* T < 0, a width <= 0 or not a multiple of 8,
                             K < 1, K > E, K > 16, E > 1024, a size that
                             overflows the 32-bit row indices, or a device
                             array that is not 16-byte aligned            */
  MOE_ERR_MODE = -3,      /* unknown dtype / route mode, or a mode
                             combination this layer does not define         */
  MOE_ERR_WORKSPACE = -4, /* workspace smaller than moe_workspace_size()     */
  MOE_ERR_HIP = -5,       /* a kernel launch failed                          */
  MOE_ERR_SCRATCH = -6    /* moe_forward_noalloc: the layer needs more than
                             the library's static scratch (MOE_SCRATCH_BYTES),
                             or the stream is not on the current device     */
} moe_status;

/* Size of the static device scratch moe_forward_noalloc runs in. */
#define MOE_SCRATCH_BYTES ((size_t)64 << 20)

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Router rules.
 * MOE_ROUTE_TOPK_SOFTMAX (APEX-1 Math. Reference Part 3, 13.2):
 *   r = x W_router^T + b; pick the K largest r; g = softmax over those K.
 * MOE_ROUTE_SOFTMAX_TOPK ("A working MoE layer in PyTorch", the MoELayer
 *   forward): p = softmax(x W_router^T + b) over all E in fp32; pick the K
 *   largest p; g = p / (sum of the K picked). Equal to the rule above in
 *   exact arithmetic; gap and top scores are reported in probability space.
 * MOE_ROUTE_SIGMOID_BIAS ("StableLatentMoE and QuantileBalancer", section
 *   "FP32 router and training-only QB update" and "Flatten routing and
 *   recover original token order"): s = sigmoid(x W_router^T); c = s + b;
 *   pick the top K+1 of c and drop the last; g = s of the K picked (the
 *   uncorrected scores), divided by their sum only if renormalize is set.
 * In every rule g is finally multiplied by routed_scale. Equal scores rank
 * the lower expert id first; slots are ordered by descending score. */
typedef enum moe_route_mode {
  MOE_ROUTE_TOPK_SOFTMAX = 0,
  MOE_ROUTE_SOFTMAX_TOPK = 1,
  MOE_ROUTE_SIGMOID_BIAS = 2
} moe_route_mode;

/* Shape and mode of one layer. d_e = latent ? latent : d_model is the width
 * the routed experts run at. */
typedef struct moe_desc {
  int64_t T;           /* tokens (batch x sequence, flattened)               */
  int32_t d_model;     /* d (M for the latent layer)                         */
  int32_t d_ff;        /* per-expert intermediate width (I for latent)        */
  int32_t n_experts;   /* E, 1..1024                                          */
  int32_t top_k;       /* K, 1..min(E, 16)                                    */
  int32_t d_shared;    /* n_shared x shared width (shared FFNs concatenated
                          along the intermediate axis), 0 = no shared expert  */
  int32_t latent;      /* 0, or L: routed path runs at width L between a
                          down-projection M->L and an up-projection L->M
                          ("StableLatentMoE", "Construction separates shared
                          and routed capacities")                             */
  int32_t act_dtype;   /* moe_dtype                                           */
  int32_t route_mode;  /* moe_route_mode                                      */
  int32_t renormalize; /* MOE_ROUTE_SIGMOID_BIAS only: 1 = divide g by sum    */
  int32_t has_rmsnorm; /* latent only: RMSNorm of the routed sum in L          */
  float routed_scale;  /* multiplies every g (1.0 when unused)                */
  float rms_eps;       /* RMSNorm: R / sqrt(mean(R^2) + eps) * gamma          */
} moe_desc;

/* Weights of one layer (device pointers, caller-owned). */
typedef struct moe_weights {
  const float *w_router;  /* [E, d_model] fp32                                */
  const float *bias;      /* [E] fp32 balance bias, or NULL for zeros          */
  const void *w_gate;     /* [E, d_ff, d_e]  act                               */
  const void *w_up;       /* [E, d_ff, d_e]  act                               */
  const void *w_down;     /* [E, d_e, d_ff]  act                               */
  const void *ws_gate;    /* [d_shared, d_model] act (NULL if d_shared == 0)   */
  const void *ws_up;      /* [d_shared, d_model] act                           */
  const void *ws_down;    /* [d_model, d_shared] act                           */
  const void *w_lat_down; /* [L, d_model] act (latent only)                    */
  const void *w_lat_up;   /* [d_model, L] act (latent only)                    */
  const float *rms_gamma; /* [L] fp32, or NULL for ones (latent + rmsnorm)     */
} moe_weights;

/* Optional timing probe for moe_forward: if stage >= 0, ev_begin and ev_end
 * (hipEvent_t, created by the caller) are recorded on the stream right
 * before the first and right after the last kernel of that stage. With
 * repeat > 1 the kernels of a GEMM stage (latent_down, expert_gate_up,
 * expert_down, shared_gate_up) are enqueued that many times back to back
 * between the two events, each pass recomputing the same outputs from the
 * same inputs: (ev_end - ev_begin) / repeat then times one pass without the
 * events' own overhead (a benchmarking aid; the layer's result is the same).
 * Other stages ignore repeat. */
typedef enum moe_stage {
  MOE_STAGE_ROUTE = 0,         /* router GEMM + selection + weights          */
  MOE_STAGE_DISPATCH = 1,      /* histogram, scan, stable scatter            */
  MOE_STAGE_LATENT_DOWN = 2,   /* z = x W_lat_down^T (latent only)           */
  MOE_STAGE_EXPERT_GATE_UP = 3,/* grouped GEMM 1 with SiLU(gate) * up        */
  MOE_STAGE_EXPERT_DOWN = 4,   /* grouped GEMM 2 times the routing weight    */
  MOE_STAGE_SHARED_GATE_UP = 5,/* shared SwiGLU, first GEMM                  */
  MOE_STAGE_COMBINE = 6,       /* shared down GEMM + routed combine (or the
                                  latent combine, RMSNorm and up-projection) */
  MOE_STAGE_COUNT = 7
} moe_stage;

typedef struct moe_probe {
  int32_t stage;   /* moe_stage, or -1 for none */
  int32_t repeat;  /* passes of a GEMM stage between the events (0 or 1: one) */
  void *ev_begin;  /* hipEvent_t */
  void *ev_end;    /* hipEvent_t */
} moe_probe;

/* How moe_forward runs a layer (filled by moe_plan; host memory). */
typedef struct moe_plan_info {
  int32_t merged_shared;          /* 1: the shared experts' gate/up and down GEMMs
                                     run inside the grouped gate/up and down
                                     launches (stages expert_gate_up /
                                     expert_down), stage shared_gate_up is empty
                                     and stage combine is the gather-sum alone */
  int32_t gate_up_pipelined;      /* 1: grouped gate/up on the pipelined kernel */
  int32_t gate_up_tile_m;         /* its output tile: rows ...               */
  int32_t gate_up_tile_n;         /* ... x weight rows (gate + up halves)     */
  int32_t down_pipelined;
  int32_t down_tile_m;
  int32_t down_tile_n;
  int32_t router_per_token;       /* 1: one wavefront per token computes the
                                     fp32 logits (few experts, narrow model);
                                     0: matrix-core router GEMM             */
  int32_t dispatch_one_workgroup; /* 1: the whole dispatch in one workgroup  */
  int32_t backward_in_place;      /* moe_backward's products that read the
                                     weights in place (K-major) instead of
                                     transposed copies: bit 0 the W_down
                                     products, bit 1 the input gradient
                                     (W_gate, W_up), bit 2 the latent
                                     projections                           */
  int32_t persistent;             /* grouped GEMMs on the persistent kernel
                                     (one workgroup per CU over a fixed list
                                     of 256x256 tiles): bit 0 gate/up, bit 1
                                     down                                  */
} moe_plan_info;

/* Text of a status code (static storage). */
MOE_API const char *moe_strerror(int status);

/* Name of a moe_stage (static storage), or "?" for an unknown value. */
MOE_API const char *moe_stage_name(int stage);

/* Device workspace, in bytes, that moe_forward needs for this layer
 * (moe_dispatch, moe_expert_ffn and moe_combine need no more than this).
 * Writes *bytes; returns MOE_OK or a shape/mode error. */
MOE_API int moe_workspace_size(const moe_desc *desc, size_t *bytes);

/* Router (Math. Reference Part 3, 13.2 "Router" and "Top-K selection";
 * the three rules of moe_route_mode). For every token t:
 *   idx[t*K + k]  int32, expert of slot k (descending ranking score)
 *   g[t*K + k]    fp32 routing weight
 *   gap[t]        fp32, K-th minus (K+1)-th ranking score (+inf if K == E);
 *                 NULL to skip
 *   top_scores[t*(K+1) + r]  fp32, the K+1 largest ranking scores (the
 *                 (K+1)-th is -inf if K == E); NULL to skip. For the sigmoid
 *                 rule these are the bias-corrected scores whose last entry
 *                 is each token's balancing threshold ("QuantileBalancer").
 * The router product x W_router^T is fp32 whatever act_dtype is
 * ("StableLatentMoE", FP32 router with autocast disabled): for bf16 x the
 * fp32 weight is split exactly into three bf16 planes whose products with x
 * are exact, accumulated in fp32 on the matrix cores. x is [T, d_model] act.
 * ws must hold moe_workspace_size() bytes (split planes, partial logits). */
MOE_API int moe_route(const moe_desc *desc, const moe_weights *w, const void *x, int32_t *idx,
                      float *g, float *gap, float *top_scores, void *ws, size_t ws_bytes,
                      void *stream);

/* Sorted dispatch ("StableLatentMoE and QuantileBalancer", section "Dispatch
 * is a stable permutation, not token duplication in model state"): the T*K
 * assignments idx (as moe_route writes them) are sorted by expert id,
 * stably in t*K + k order:
 *   counts[e]          int32 [E], assignments of expert e
 *   offsets[e]         int32 [E+1], exclusive prefix sum (offsets[E] = T*K)
 *   perm[p]            int32 [T*K], flat slot t*K + k at sorted position p
 *   sorted_token[p]    int32 [T*K], = perm[p] / K
 *   inv[t*K + k]       int32 [T*K], sorted position of slot (t, k)
 *   sorted_w[p]        fp32 [T*K], g[perm[p]] (NULL to skip; g may then be
 *                      NULL)
 *   rows_sorted[p, :]  act [T*K, d_e], = rows[sorted_token[p], :] (NULL to
 *                      skip; rows may then be NULL). rows is x, or the latent
 *                      z = x W_lat_down^T for a latent layer.
 * Expert ids outside [0, E) are a caller error: such slots are dropped from
 * every output (no out-of-bounds access), leaving those outputs incomplete.
 * ws must hold moe_workspace_size() bytes. */
MOE_API int moe_dispatch(const moe_desc *desc, const int32_t *idx, const float *g, const void *rows,
                 int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *sorted_token,
                 int32_t *inv, float *sorted_w, void *rows_sorted, void *ws, size_t ws_bytes,
                 void *stream);

/* Grouped expert SwiGLU over contiguous expert slices (Math. Reference
 * Part 3, 12.2; "StableLatentMoE", "The actual grouped GEMM"; "A working MoE
 * layer in PyTorch", per-expert contiguous slices). For every sorted
 * position p in [offsets[e], offsets[e+1]):
 *   y_sorted[p, :] = row_scale[p] * W_down[e] (SiLU(W_gate[e] a_p) * (W_up[e] a_p))
 * with a_p = rows[row_index[p], :] if row_index is given (the gather is
 * fused into the GEMM's operand load), else rows[p, :]. rows is act
 * [*, d_e]; row_scale fp32 [T*K] or NULL for 1; y_sorted act [T*K, d_e].
 * The intermediate SiLU(gate) * up is rounded to act_dtype. */
MOE_API int moe_expert_ffn(const moe_desc *desc, const moe_weights *w, const void *rows,
                   const int32_t *row_index, const int32_t *offsets, const float *row_scale,
                   void *y_sorted, void *ws, size_t ws_bytes, void *stream);

/* Combine + shared experts (Math. Reference Part 3, 13.2; "StableLatentMoE",
 * "Return to model width"). For every token t, with R_t = sum over k = 0..K-1
 * (in that order, fp32) of y_sorted[inv[t*K + k], :]:
 *   out[t, :] = Shared(x_t) + R_t                                (latent = 0)
 *   out[t, :] = Shared(x_t) + W_lat_up RMSNorm(R_t)              (latent)
 * Shared is the SwiGLU FFN of width d_shared (absent if 0). No atomics: each
 * output row is written once. x [T, d_model] act; y_sorted act [T*K, d_e];
 * out act [T, d_model]. */
MOE_API int moe_combine(const moe_desc *desc, const moe_weights *w, const void *x, const void *y_sorted,
                const int32_t *inv, void *out, void *ws, size_t ws_bytes, void *stream);

/* The whole forward pass: route, dispatch, (latent down-projection), grouped
 * expert SwiGLU, shared experts and combine. out act [T, d_model].
 * counts: int32 [E] expert loads, or NULL.
 * n_near_ties: int32 [1], number of tokens whose K-th and (K+1)-th ranking
 *   scores (as this call computed them) differ by less than 1e-5, or NULL.
 * probe: optional timing probe, or NULL. */
MOE_API int moe_forward(const moe_desc *desc, const moe_weights *w, const void *x, void *out,
                int32_t *counts, int32_t *n_near_ties, void *ws, size_t ws_bytes,
                const moe_probe *probe, void *stream);

/* moe_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops such as decode, harnesses that
 * forbid hipMalloc): the same kernels and results as moe_forward, with its
 * workspace taken from a static device array of MOE_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends. The call
 * allocates nothing (no hipMalloc / hipFree, no allocating library call);
 * on its first call on a device it looks up that device's copy of the array
 * (hipGetSymbolAddress). The caller passes inputs and outputs as for
 * moe_forward. `stream` must belong to the current device.
 * Every call on one GPU shares that GPU's scratch, which keeps the previous
 * call's contents (nothing in the forward depends on them): calls that may
 * overlap on one GPU (different streams, or different host threads) race
 * and must be serialised by the caller.
 * Errors: as moe_forward, and MOE_ERR_SCRATCH when moe_workspace_size() of
 * the layer exceeds MOE_SCRATCH_BYTES (e.g. the d=7168, E=256, K=8 layer
 * fits up to 256 tokens, the d=512, E=4 layer up to ~4000) or the stream is
 * on another device; nothing is launched then. */
MOE_API int moe_forward_noalloc(const moe_desc *desc, const moe_weights *w, const void *x,
                                void *out, int32_t *counts, int32_t *n_near_ties, void *stream);

/* Gradients of the layer's parameters (fp32 DEVICE arrays, caller-owned; a
 * NULL member is not computed). Shapes as in moe_weights. */
typedef struct moe_grads {
  float *w_router;        /* [E, d_model]                              */
  float *w_gate, *w_up;   /* [E, d_ff, d_e]  (d_e = latent ? L : d_model) */
  float *w_down;          /* [E, d_e, d_ff]                            */
  float *ws_gate, *ws_up; /* [d_shared, d_model]                       */
  float *ws_down;         /* [d_model, d_shared]                       */
  float *w_lat_down;      /* [L, d_model]   (latent layers)            */
  float *w_lat_up;        /* [d_model, L]   (latent layers)            */
  float *rms_gamma;       /* [L]            (latent layers with RMSNorm) */
} moe_grads;

/* Device workspace, in bytes, that moe_backward needs for this layer (more
 * than moe_workspace_size: transposed weights of the experts and per-row
 * gradients). Errors as moe_backward's shape/mode checks. */
MOE_API int moe_backward_workspace_size(const moe_desc *desc, size_t *bytes);

/* Backward pass of the layer for an output gradient d_out [T, d_model] (act
 * dtype): the gradient of sum_t <d_out[t], MoE(x)[t]> with respect to x
 * (d_x [T, d_model], act dtype; NULL: not computed) and to the weights
 * (grads, fp32). The forward's routing and dispatch are recomputed from x
 * (nothing is kept from a forward call). Rules ("StableLatentMoE and
 * QuantileBalancer": gradients flow only into active experts):
 *  - the top-K selection is piecewise constant and passes no gradient; the
 *    routing weights pass theirs to the router logits (softmax over the
 *    selected, or sigmoid, as routed) and so to W_router and x; the balance
 *    bias gets none;
 *  - experts that no token selects get no weight gradient: their slices of
 *    grads->w_gate / w_up / w_down are left untouched; every other requested
 *    array is overwritten (not accumulated);
 *  - intermediate products are in the layer's dtype with fp32
 *    accumulation, like the forward (bf16 layers: bf16 operands; fp32
 *    layers: every product in fp32); router gradients are fp32.
 *  - latent layers ("StableLatentMoE and QuantileBalancer"): the routed sum
 *    and its RMSNorm are recomputed; gradients also reach W_lat_down,
 *    W_lat_up and the RMSNorm gain (rms_gamma NULL in w: a gain of ones,
 *    whose gradient is still reported if grads->rms_gamma is given).
 * Supported: d_model, d_ff, d_shared and L multiples of 32. Errors:
 * MOE_ERR_SHAPE (other widths, or operands beyond 4 GiB), MOE_ERR_NULL,
 * MOE_ERR_WORKSPACE (below moe_backward_workspace_size), MOE_ERR_HIP.
 * T == 0 is a no-op. */
MOE_API int moe_backward(const moe_desc *desc, const moe_weights *w, const void *x,
                         const void *d_out, void *d_x, const moe_grads *grads, void *ws,
                         size_t ws_bytes, void *stream);

/* The kernel plan moe_forward uses for this layer (it depends on the
 * descriptor only). Errors: a bad descriptor, MOE_ERR_NULL. */
MOE_API int moe_plan(const moe_desc *desc, moe_plan_info *info);

/* QuantileBalancer update ("StableLatentMoE and QuantileBalancer", sections
 * "QuantileBalancer: persistent biases, no gradient update" and "FP32 router
 * and training-only QB update"); sigmoid routing (MOE_ROUTE_SIGMOID_BIAS)
 * with top_k < n_experts only. From the router of this layer on x (fp32
 * logits as moe_route computes them, raw scores s = sigmoid(logits),
 * corrected scores s + bias with the current w->bias): per token the
 * threshold is the (K+1)-th largest corrected score; per expert e, new_bias[e]
 * is the value at position ceil(K (T-1) / E) of the ascending token-sorted
 * thresh - s[., e] (the p = K/E quantile, "higher" rule); the E values are
 * then centred by their mean (summed in fp64). new_bias: fp32 [E] device
 * array; it may be w->bias itself (the pages replace the buffer in place:
 * every read of the old bias precedes the write on the stream). The caller
 * applies it to later forwards (training-mode forwards only, per the page).
 * T == 0 is a no-op. Errors: MOE_ERR_MODE (other routing rules), MOE_ERR_SHAPE
 * (top_k >= n_experts, or a bad descriptor), MOE_ERR_NULL, MOE_ERR_WORKSPACE
 * (ws_bytes below moe_workspace_size, which includes this call's buffers
 * for sigmoid-routed layers), MOE_ERR_HIP. */
MOE_API int moe_quantile_balance(const moe_desc *desc, const moe_weights *w, const void *x,
                                 float *new_bias, void *ws, size_t ws_bytes, void *stream);

/* Router auxiliary losses of one training step, on this layer's router
 * logits r_t = x_t W_router^T (fp32, as moe_route computes them; the balance
 * bias is a non-gradient nudge and is not part of them):
 *  - losses[0], the load-balancing loss of "A working MoE layer in PyTorch"
 *    (the Switch loss its MoELayer computes): alpha * E * sum_e f_e * P_e with
 *    f_e = counts[e] / (T * top_k) and P_e the mean over the T tokens of
 *    softmax(r_t)_e;
 *  - losses[1], the router z-loss of the transformer book's mixture-of-experts
 *    chapter (MoEAuxiliaryLoss.router_z_loss, weight 0.001 there):
 *    z_weight * mean over tokens of logsumexp(r_t)^2.
 * counts: int32 [E] device array, the expert loads of the same T tokens (as
 * moe_forward / moe_dispatch return them). losses: fp32 [2] device array.
 * Any routing rule (the losses are defined on the softmax of the logits).
 * Sums are taken in a fixed order (per chunk of 16 to 64 tokens in fp32, then
 * over the chunks in fp64):
 * results are deterministic. Enqueued on stream, no host synchronisation.
 * T == 0 is a no-op (losses untouched). Errors: MOE_ERR_NULL, MOE_ERR_MODE
 * (alpha or z_weight not finite, or a bad descriptor), MOE_ERR_SHAPE,
 * MOE_ERR_WORKSPACE, MOE_ERR_HIP. */
MOE_API int moe_router_losses(const moe_desc *desc, const moe_weights *w, const void *x,
                              const int32_t *counts, float alpha, float z_weight, float *losses,
                              void *ws, size_t ws_bytes, void *stream);

/* Bias-based load balancing, one step ("APEX-1 Mathematical Reference -
 * Part 3", section 14.3; the sign rule of section 14.4). For a step of
 * n_tokens tokens routed top-k over n_experts experts with per-expert loads
 * counts[e] (as moe_forward / moe_dispatch return them), every bias[e] moves
 * by alpha * sign(1/E - counts[e] / (n_tokens * top_k)) and is clamped to
 * [-1, 1]. The sign is decided exactly on integers (n_tokens * top_k versus
 * E * counts[e]); the update is one fp32 add. bias: fp32 [E] device array,
 * updated in place (the same array moe_weights.bias points at); counts: int32
 * [E] device array. Enqueued on stream, no host synchronisation.
 * n_tokens == 0 is a no-op. Errors: MOE_ERR_NULL (counts or bias NULL),
 * MOE_ERR_SHAPE (n_experts outside 1..1024, top_k outside 1..n_experts,
 * n_tokens < 0, or n_tokens * top_k beyond int32), MOE_ERR_MODE (alpha not
 * finite), MOE_ERR_HIP (launch failure). */
MOE_API int moe_balance_bias(int32_t n_experts, int32_t top_k, int64_t n_tokens,
                             const int32_t *counts, float alpha, float *bias, void *stream);

/* Measurement helper, not a step of the layer: peak-rate microbenchmarks of
 * the part, so that fractions of peak can be stated against measured rates as
 * well as the datasheet's. Each of `groups` workgroups of `threads` (256: one
 * wavefront per SIMD, 512: two) holds 96 KB of LDS (one workgroup per CU)
 * and runs `iters` iterations of two halves; a half issues, per wavefront:
 *   mode 0: 8 independent v_mfma_f32_16x16x32_bf16 (131072 flops);
 *   mode 1: 4 independent v_mfma_f32_32x32x16_bf16 (131072 flops);
 *   mode 2: 8 conflict-free 16-byte LDS reads per lane (8 KB per wavefront);
 *   mode 3 / 4: mode 0 / 1 plus 3 16-byte LDS reads per lane whose data are
 *     the next half's MFMA operands (the read-to-MFMA ratio of a 64 x 128
 *     wavefront tile); mode 5 / 6: the same with 2 reads (a 128 x 128 tile);
 *   mode 7 .. 10: as mode 2, each read a GEMM operand fragment from stage
 *     rows of 128 bytes whose 16-byte units are XOR-swizzled: 7 / 8 the
 *     16x16x32 operand (16 rows per read) swizzled by row & 7 / by
 *     (row >> 1) & 7; 9 / 10 the 32x32x16 operand (32 rows), the same two.
 * clk: int64 [2 * groups] device array, per workgroup the shader clock cycles
 * (s_memtime) and the 100 MHz constant clock ticks (s_memrealtime) its loop
 * took. sink: uint32 [groups * threads] device array (results kept live).
 * Enqueued on stream. Errors: MOE_ERR_SHAPE (mode outside 0..10, threads not
 * 256 or 512, groups outside 1..2^20, iters < 1), MOE_ERR_NULL, MOE_ERR_HIP. */
MOE_API int moe_peak(int32_t mode, int32_t threads, int32_t groups, int32_t iters, int64_t *clk,
                     uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
