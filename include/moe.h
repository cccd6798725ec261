/*
 * moe.h -- C ABI of a dropless top-k mixture-of-experts FFN layer (forward and backward) for AMD MI355X
 * (gfx950, CDNA4). Every step runs in hand-written HIP kernels; this header carries no HIP
 * or framework types, only plain pointers and sizes.
 *
 * Pages the operations follow (cited by title and section):
 *   [L7.8]  "Mixture of Experts: routing, sorted dispatch, Switch aux loss, aux-free bias"
 *           (openlearn course module L7.8): §2 symbols, §2.1 routers table and output
 *           equation, §2.2 sorted dispatch, §2.3 load-balancing loss, §2.5 aux-free bias,
 *           §3 worked example, §4 interface, §5 pitfalls.
 *   [RB-15] "15. Mixture of Experts" (RustingBrain tutorial): §15.2 routing and "Dropless",
 *           §15.3 the z-loss.
 *   [nanoMoE] "nanoMoE: Mixture-of-Experts (MoE) LLMs from Scratch in PyTorch": the MLP /
 *           MLPExperts listings (GELU expert with optional biases).
 *
 * Conventions shared by every entry point
 *   - Memory: every tensor pointer is a DEVICE pointer owned by the caller. The library
 *     never allocates or frees device memory, and scratch memory comes from the caller's
 *     workspace `ws` of `ws_bytes` bytes (moe_forward_noalloc alone uses a static device
 *     array instead). No call's results depend on an earlier call. The only process-wide
 *     state is a per-device cache of the compute-unit count (read once per device, it sizes
 *     the persistent GEMM grids) and moe_forward_noalloc's per-device scratch address.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls
 *     enqueue kernels on it and return without synchronising (moe_get_device_error is the
 *     one exception). Outputs are valid once the stream reaches that point.
 *   - Layout: row-major everywhere. Expert weights are stacked per expert in nn.Linear's
 *     [out, in] layout, so both operands of every product are contiguous along the
 *     reduction axis. Index tensors are int32, gates and statistics float32.
 *   - Element type T (cfg->dtype): float32 or bfloat16 for x, all weights and biases,
 *     x_sorted, y_sorted and y. Accumulation is always float32. With bfloat16 the
 *     intermediate expert activation h and y_sorted are rounded to bfloat16
 *     (round-to-nearest-even); the combine sums in float32 and rounds once.
 *   - Assignments: token n's j-th choice is assignment a = n*k + j; A = N*k ([L7.8] §2.2).
 *   - Errors: arguments are validated on the host before anything is enqueued; an invalid
 *     call returns a non-zero moe_status and leaves every output untouched. Errors never
 *     cross the ABI as exceptions. A failed kernel launch returns MOE_ERR_HIP.
 *   - Limits: 0 <= N*k < 2^31, 1 <= E <= 1024, 1 <= k <= min(E, 32), d and d_ff in
 *     [8, 65536] and multiples of 8; the workspace and every T tensor 16-byte aligned, every
 *     int32 / float32 tensor 4-byte aligned (MOE_ERR_UNSUPPORTED otherwise; MOE_ERR_WORKSPACE
 *     for a misaligned workspace). N = 0 is valid: counts and statistics are written as zeros.
 *   - Device error word: the first int of the workspace. moe_dispatch overwrites it (0, or
 *     MOE_ERR_BAD_EXPERT_ID when it met an id outside [0, E)); moe_forward overwrites it with
 *     0; moe_expert_ffn sets it to MOE_ERR_INVALID_ARG when offsets is not a non-decreasing
 *     sequence in [0, A] starting at 0, and leaves it unchanged otherwise.
 *     moe_get_device_error reads and clears it.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* bad k, E, N, enum, flag combination or a NULL pointer */
  MOE_ERR_UNSUPPORTED = 2,   /* outside the limits above (sizes, alignment) */
  MOE_ERR_WORKSPACE = 3,     /* ws_bytes < moe_workspace_size(cfg, op) or ws == NULL */
  MOE_ERR_BAD_EXPERT_ID = 4, /* device-detected expert id outside [0, E) */
  MOE_ERR_HIP = 5            /* a HIP runtime call or kernel launch failed */
} moe_status;

/* [L7.8] §2.1 routers table. */
typedef enum {
  MOE_ROUTER_SOFTMAX_TOPK = 0, /* choose top k of p = softmax(z); w = p_T (renormalised if norm_topk) */
  MOE_ROUTER_TOPK_SOFTMAX = 1, /* choose top k of z; w = softmax over the k chosen logits */
  MOE_ROUTER_SIGMOID = 2       /* choose top k of sigmoid(z) + b; w = sigmoid(z_T) (renormalised if norm_topk) */
} moe_router;

/* Expert FFN. GELU (exact erf form): y = W2 gelu(W1 x + b1) + b2, biases optional
 * ([nanoMoE] MLPExperts). SwiGLU: y = W2 (silu(W1 x) * (W3 x)), W1 = gate, W3 = up, no biases. */
typedef enum { MOE_ACT_GELU = 0, MOE_ACT_SWIGLU = 1 } moe_act;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Layout of the routed experts' weights W1, W3 and W2 in moe_expert_ffn and moe_forward.
 * ROWMAJOR: [E,N,K] as each call states (N output features, K reduction).
 * TILED: written once by moe_pack_weights (bf16 only). Per expert, the N rows are taken in
 * blocks of 128, and each block is stored K-slab by K-slab, 32 reduction elements at a time:
 * element (e, n, k) sits at
 *   e*Np*Kp + (n/128)*128*Kp + (k/32)*128*32 + (n%128)*32 + k%32,
 * with Np = N rounded up to 128 and Kp = K rounded up to 32; the padding is zero. Each
 * 32-wide reduction slab of a 128-row block is then one contiguous 8 KiB run, which is how
 * the grouped GEMM reads it (same results as ROWMAJOR, bit for bit). */
typedef enum { MOE_WEIGHTS_ROWMAJOR = 0, MOE_WEIGHTS_TILED = 1 } moe_weight_layout;

/* Which call a workspace is sized for. */
typedef enum {
  MOE_OP_ROUTE = 0, MOE_OP_DISPATCH = 1, MOE_OP_EXPERT_FFN = 2, MOE_OP_COMBINE = 3, MOE_OP_FORWARD = 4,
  MOE_OP_SHARED_FFN = 5, MOE_OP_BACKWARD = 6
} moe_op;

/* One layer's configuration. Zero-initialise it (e.g. moe_config c = {0};) before setting
 * fields: a field added at the end later then means its default, 0. */
typedef struct {
  int64_t n_tokens;     /* N: tokens, every leading axis flattened ([L7.8] §2) */
  int32_t d_model;      /* d */
  int32_t n_experts;    /* E */
  int32_t top_k;        /* k */
  int32_t d_ff;         /* expert hidden width */
  int32_t router;       /* moe_router */
  int32_t norm_topk;    /* 1: renormalise the chosen gates to sum to 1; 0: keep them raw */
  int32_t act;          /* moe_act */
  int32_t has_bias;     /* 1: b1 [E,d_ff] and b2 [E,d] are given (GELU only) */
  int32_t dtype;        /* moe_dtype: element type T */
  float routed_scaling; /* every gate is multiplied by this after renormalisation ([L7.8] §2.1) */
  int32_t d_ff_shared;  /* hidden width S f of the shared expert(s), 0 = none ([L7.8] §2.1:
                           S shared experts of width f are one MLP of width S f; [RB-15] §15.4) */
  float capacity_factor; /* moe_forward only: 0 = dropless; > 0 = capacity-factor dispatch
                            (moe_dispatch_capacity) with this factor */
  int32_t weight_layout; /* moe_weight_layout of w1, w3 and w2 (moe_expert_ffn, moe_forward);
                            MOE_WEIGHTS_TILED needs dtype MOE_BF16, and moe_backward /
                            moe_forward_train return MOE_ERR_UNSUPPORTED with it */
} moe_config;

/* Number of statistics floats moe_route / moe_forward write: f[E], P[E], L, z_loss. */
#define MOE_STATS_LEN(E) (2 * (size_t)(E) + 2)

/* Workspace bytes that call `op` needs for this config (256-byte aligned sizes), or 0 when
 * the config is invalid. The first 256 bytes of every workspace hold the device error word
 * read by moe_get_device_error; a workspace may be reused by later calls on the same stream. */
size_t moe_workspace_size(const moe_config* cfg, int op);

/* Routing of N tokens ([L7.8] §2, §2.1; [RB-15] §15.2):
 *   z = x W_g^T + logit_bias                      (logit_bias [E] float32 or NULL: a fixed
 *                                                   per-expert offset that is part of z)
 *   p = softmax(z)                                 (float32, max-subtracted)
 *   s = z (+ sel_bias) for the softmax routers, sigmoid(z) + sel_bias for sigmoid
 *   T = the k largest s, largest first, ties to the lowest expert id
 *   w = gates by the routers table, times routed_scaling; sel_bias never enters w.
 * Switch statistics ([L7.8] §2.3): counts_e = assignments to e; f_e = counts_e / N;
 * P_e = mean_n p_{n,e}; L = E sum_e f_e P_e; and the router z-loss ([RB-15] §15.3)
 * z_loss = mean_n (logsumexp z_n)^2. The final reductions run in a fixed order, so the
 * statistics are bitwise reproducible.
 * In:  x [N,d] T; w_router [E,d] T; logit_bias, sel_bias [E] float32 or NULL.
 * Out: topk_ids [N,k] int32; topk_w [N,k] float32; counts [E] int32;
 *      stats [2E+2] float32 = f[0..E), P[E..2E), L at [2E], z_loss at [2E+1];
 *      logits_out [N,E] float32 (z) or NULL; gap_out [N] float32 or NULL, the margin
 *      s_(k) - s_(k+1) between the last chosen and the best unchosen score (+inf if k = E).
 * ws: moe_workspace_size(cfg, MOE_OP_ROUTE) bytes. */
moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* logit_bias, const float* sel_bias,
                     int32_t* topk_ids, float* topk_w, int32_t* counts, float* stats,
                     float* logits_out, float* gap_out,
                     void* ws, size_t ws_bytes, void* stream);

/* Sorted dispatch ([L7.8] §2.2, §3): assignment a = n*k + j is stably sorted by expert id.
 * Out: perm [A] int32 (sorted position i -> assignment a; the token is a / k);
 *      inv_perm [A] int32 (inv_perm[perm[i]] = i); counts [E] int32;
 *      offsets [E+1] int32 (offsets[e] is the START of expert e's slice, offsets[E] = A);
 *      x_sorted [A,d] T with x_sorted[i] = x[perm[i] / k] (a bit copy);
 *      gate_sorted [A] float32 = topk_w.flat[perm[i]] when both topk_w and gate_sorted are
 *      given (either may be NULL otherwise; x_sorted may be NULL to skip the row copy).
 * Ids outside [0, E) are dropped (no slot; inv_perm = -1; not counted) and set the device
 * error word in ws, which moe_get_device_error reports as MOE_ERR_BAD_EXPERT_ID.
 * ws: moe_workspace_size(cfg, MOE_OP_DISPATCH) bytes. */
moe_status moe_dispatch(const moe_config* cfg, const void* x, const int32_t* topk_ids,
                        const float* topk_w, void* x_sorted, int32_t* perm, int32_t* inv_perm,
                        int32_t* counts, int32_t* offsets, float* gate_sorted,
                        void* ws, size_t ws_bytes, void* stream);

/* Expert capacity of the capacity-factor dispatch ([nanoMoE] "Computing the expert
 * capacity"): floor(k * cf * N / E) in double precision, raised by one when odd. */
int64_t moe_expert_capacity(int32_t top_k, float capacity_factor, int64_t n_tokens, int32_t n_experts);

/* Capacity-factor (token-dropping) dispatch ([nanoMoE] "Expert Capacity"): each expert takes
 * at most cap = moe_expert_capacity(k, capacity_factor, N, E) assignments, ranked in k-major
 * order (every token's first choice before any second choice, tokens ascending), so top
 * choices win; the rest are dropped (no computation, no contribution; the kept ones keep
 * their router weight). The kept assignments of expert e form the contiguous rows
 * [offsets[e], offsets[e+1]) in rank order: a ragged batch of at most cap rows (the padding
 * of a fixed [E, cap] batch is never computed). moe_expert_ffn and moe_combine (inv_perm =
 * slot) run on this layout unchanged.
 * Out: slot [A] int32 (row of assignment a = n*k + j, or -1 if dropped); kept [E] int32;
 *      offsets [E+1] int32 (offsets[E] = kept rows); x_kept [A,d] T (NULL: no row copy);
 *      perm_kept [A] int32 (row -> assignment) or NULL; gate_kept [A] float32 = topk_w at
 *      each kept row when both are given. Ids outside [0, E) are dropped and flagged as in
 *      moe_dispatch. capacity_factor: finite, >= 0.
 * ws: moe_workspace_size(cfg, MOE_OP_DISPATCH) bytes. */
moe_status moe_dispatch_capacity(const moe_config* cfg, float capacity_factor, const void* x,
                                 const int32_t* topk_ids, const float* topk_w, void* x_kept,
                                 int32_t* perm_kept, int32_t* slot, int32_t* kept, int32_t* offsets,
                                 float* gate_kept, void* ws, size_t ws_bytes, void* stream);

/* Expert FFN over ragged per-expert slices ([L7.8] §2.2 "each expert runs once on its
 * slice"; [RB-15] "Dropless"): for every expert e and every row i in
 * [offsets[e], offsets[e+1]):  y_sorted[i] = FFN_e(x_sorted[i]) * gate_sorted[i].
 * Experts with an empty slice run nothing and their weights are never read.
 * In:  x_sorted [A,d] T; offsets [E+1] int32 (non-decreasing, offsets[0] = 0, offsets[E] <= A);
 *      w1 [E,d_ff,d] T (GELU fc or SwiGLU gate); w3 [E,d_ff,d] T (SwiGLU up; NULL for GELU);
 *      b1 [E,d_ff] T and b2 [E,d] T (has_bias only); w2 [E,d,d_ff] T;
 *      gate_sorted [A] float32 or NULL (NULL: no scaling).
 * Out: y_sorted [A,d] T (rows at or past offsets[E] are not written).
 * With cfg->weight_layout = MOE_WEIGHTS_TILED, w1, w3 and w2 are moe_pack_weights copies
 * (which = 0, 0, 1); the results are the same.
 * ws: moe_workspace_size(cfg, MOE_OP_EXPERT_FFN) bytes (holds h [A,d_ff] T). */
moe_status moe_expert_ffn(const moe_config* cfg, const void* x_sorted, const int32_t* offsets,
                          const void* w1, const void* w3, const void* b1,
                          const void* w2, const void* b2, const float* gate_sorted,
                          void* y_sorted, void* ws, size_t ws_bytes, void* stream);

/* Tiled weights (MOE_WEIGHTS_TILED, layout above), for the bf16 grouped GEMMs: a once-only
 * re-layout of static weights, done before moe_expert_ffn / moe_forward calls that read them.
 * which = 0: W1 or W3, [E,d_ff,d] (N = d_ff, K = d); which = 1: W2, [E,d,d_ff] (N = d,
 * K = d_ff).
 * moe_packed_weight_size: bytes of the tiled copy, E * Np * Kp * 2; 0 when the configuration
 * is invalid, not bf16, or which is neither 0 nor 1.
 * moe_pack_weights: w (row-major, device, 16-byte aligned) -> w_tiled (device, 16-byte
 * aligned, moe_packed_weight_size bytes, not overlapping w), on `stream`, padding zeroed.
 * The caller owns both buffers. MOE_ERR_UNSUPPORTED for dtype f32. */
size_t moe_packed_weight_size(const moe_config* cfg, int which);
moe_status moe_pack_weights(const moe_config* cfg, int which, const void* w, void* w_tiled, void* stream);

/* Combine ([L7.8] §2.2, §3): y[n] = sum_{j<k} g_{n,j} y_sorted[inv_perm[n*k+j]] (+ y_add[n]),
 * summed in float32 with j ascending, then y_add, and rounded to T once; g = topk_w [N,k]
 * float32, or 1 when topk_w is NULL (y_sorted already gate-scaled). y_add [N,d] T or NULL:
 * a term every token receives with weight 1 (the shared expert's output). Assignments with
 * inv_perm outside [0, A) contribute nothing. */
moe_status moe_combine(const moe_config* cfg, const void* y_sorted, const float* topk_w,
                       const int32_t* inv_perm, const void* y_add, void* y, void* stream);

/* The shared expert(s) ([L7.8] §2.1 Shared(x); [RB-15] §15.4): one dense MLP of width
 * F = cfg->d_ff_shared (> 0) over all N tokens, same activation as the routed experts:
 *   GELU:   y_shared = W2s gelu(W1s x + b1s) + b2s      (biases iff has_bias)
 *   SwiGLU: y_shared = W2s (silu(W1s x) * (W3s x))
 * In: x [N,d] T; s_w1 [F,d] T; s_w3 [F,d] T (SwiGLU) or NULL; s_b1 [F] T, s_b2 [d] T (GELU
 * with has_bias) or NULL; s_w2 [d,F] T. Out: y_shared [N,d] T (bf16: h rounded to bf16, as
 * for the routed experts). ws: moe_workspace_size(cfg, MOE_OP_SHARED_FFN) bytes. */
moe_status moe_shared_ffn(const moe_config* cfg, const void* x, const void* s_w1, const void* s_w3,
                          const void* s_b1, const void* s_w2, const void* s_b2, void* y_shared,
                          void* ws, size_t ws_bytes, void* stream);

/* The whole layer ([L7.8] §2.1 output equation): route -> dispatch -> expert FFN (gate
 * applied in the down-projection epilogue) -> combine -> statistics, on one stream with no
 * host synchronisation. Inputs and outputs as in the calls above; y [N,d] T. Routing's final
 * reduction also forms the dispatch offsets and per-block bases from its own histograms, so
 * the dispatch stage is a scatter and a row copy; results equal the separate calls'.
 * With cfg->d_ff_shared > 0 the shared expert's weights s_w1 .. s_b2 (as in moe_shared_ffn)
 * are required and Shared(x) is added in the combine; otherwise they must be NULL.
 * With cfg->capacity_factor > 0 the dispatch is moe_dispatch_capacity's (counts and the
 * statistics still describe the routing before any drop).
 * With cfg->weight_layout = MOE_WEIGHTS_TILED, w1, w3 and w2 are moe_pack_weights copies (the
 * shared expert's weights stay row-major); the results are the same.
 * perm, inv_perm, offsets: NULL, or int32 buffers that receive the dispatch arrays the call
 * itself used ([L7.8] §2.2): dropless, perm [A], inv_perm [A] and offsets [E+1] exactly as
 * moe_dispatch defines them for topk_ids; with cfg->capacity_factor > 0, moe_dispatch_capacity's
 * perm_kept (its first offsets[E] entries), slot and offsets. The call then writes them there
 * instead of into its workspace, so asking for them costs nothing. Each may be given alone.
 * stage_events: NULL, or 6 hipEvent_t (as void*) recorded on `stream` at the start, after
 * routing, after dispatch, after the up projection, after the down projection (and the
 * shared expert, when there is one) and at the end.
 * ws: moe_workspace_size(cfg, MOE_OP_FORWARD) bytes. */
moe_status moe_forward(const moe_config* cfg, const void* x, const void* w_router,
                       const float* logit_bias, const float* sel_bias,
                       const void* w1, const void* w3, const void* b1,
                       const void* w2, const void* b2,
                       const void* s_w1, const void* s_w3, const void* s_b1,
                       const void* s_w2, const void* s_b2,
                       void* y, int32_t* topk_ids, float* topk_w, int32_t* counts, float* stats,
                       int32_t* perm, int32_t* inv_perm, int32_t* offsets,
                       void* ws, size_t ws_bytes, void* const* stage_events, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): moe_forward with the same arguments minus the
 * workspace, perm / inv_perm / offsets and stage events. Its scratch is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds from module load to process
 * end; the call allocates and frees nothing. Configurations whose moe_workspace_size(cfg,
 * MOE_OP_FORWARD) exceeds MOE_NOALLOC_SCRATCH_BYTES are refused with MOE_ERR_WORKSPACE before
 * anything is enqueued: 128 MiB covers about 700 tokens at Mixtral width (d = 4096, E = 8, k = 2,
 * d_ff = 14336), of which 64 MiB are the down projection's split-K partials at any size. Every call on one GPU uses that GPU's single array, which keeps the last call's
 * contents: calls that overlap on one GPU (on different streams, or from several threads
 * without ordering) race and must not be issued. Results equal moe_forward's, bit for bit. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
moe_status moe_forward_noalloc(const moe_config* cfg, const void* x, const void* w_router,
                               const float* logit_bias, const float* sel_bias,
                               const void* w1, const void* w3, const void* b1,
                               const void* w2, const void* b2,
                               const void* s_w1, const void* s_w3, const void* s_b1,
                               const void* s_w2, const void* s_b2,
                               void* y, int32_t* topk_ids, float* topk_w, int32_t* counts, float* stats,
                               void* stream);

/* Gradients written by moe_backward: device pointers owned by the caller, each shaped like
 * the tensor it is the gradient of, element type T unless stated. */
typedef struct {
  void* dx;         /* [N,d] */
  void* dw_router;  /* [E,d] */
  void* dw1;        /* [E,d_ff,d] */
  void* dw3;        /* [E,d_ff,d] (SwiGLU) or NULL */
  void* db1;        /* [E,d_ff] (has_bias) or NULL */
  void* dw2;        /* [E,d,d_ff] */
  void* db2;        /* [E,d] (has_bias) or NULL */
  void* ds_w1;      /* shared expert (d_ff_shared > 0; NULL otherwise), shaped like s_w1 .. s_b2 */
  void* ds_w3;
  void* ds_b1;
  void* ds_w2;
  void* ds_b2;
  float* dz;        /* [N,E] float32 dJ/dz (router logits, logit_bias included) or NULL */
  float* dgate;     /* [N,k] float32 dJ/dw (the gates after routed_scaling) or NULL */
} moe_grads;

/* Backward of the dropless layer: the gradients of
 *     J = <dy, y> + aux_coef * L + z_coef * z_loss
 * (y the output of moe_forward with the same inputs and cfg->capacity_factor = 0; L and
 * z_loss the statistics of moe_route) with respect to x and every weight, by the chain
 * rule through [L7.8] §2.1 (output equation; routers table weights), §2.3 (L = E sum f P
 * with f piecewise constant, so only P = mean softmax(z) carries gradient) and [RB-15]
 * §15.3 (z-loss). The selection (top-k, sel_bias) carries none ([L7.8] §2.5). Nothing is
 * kept from a forward call: routing, dispatch and the up projection are recomputed (their
 * outputs topk_ids, topk_w, counts, stats are written as moe_route writes them).
 * bfloat16 only (T = MOE_BF16; MOE_ERR_UNSUPPORTED for float32 and for
 * capacity_factor > 0). Accumulation is float32; the pre-activations, the gate-scaled h,
 * the activation gradients and dx_sorted are rounded to bfloat16, dz is split into two
 * bfloat16 terms for the products with W_g and x; every gradient is rounded once.
 * In: the forward's inputs; dy [N,d] T; aux_coef, z_coef: finite.
 * Out: *grads (dw3 / db1 / db2 / shared gradients required exactly when the matching
 * weight is); topk_ids, topk_w, counts, stats as in moe_route.
 * saved: 0 = recompute as above. 1 = `ws` holds the state a moe_forward_train call left with
 * the same cfg and inputs, and topk_ids, topk_w, counts and stats hold that call's outputs:
 * they are then read, not written, and routing, dispatch and the up projections are not
 * recomputed. The gradients are the same bits as with saved = 0. The saved state survives
 * this call, so several backward calls may follow one moe_forward_train.
 * stage_events: NULL, or MOE_BWD_EVENTS hipEvent_t (as void*) recorded on `stream` at the
 * start, after the recomputed routing and dispatch, after the recomputed up projection, after
 * dh' (with the activation backward), after the router backward, after dx_sorted, after dW2,
 * after dW1 / dW3 (and the bias sums), after the shared expert's gradients and at the end
 * (router weight gradient, dz W_g and the dx combine).
 * ws: moe_workspace_size(cfg, MOE_OP_BACKWARD) bytes. */
#define MOE_BWD_EVENTS 10
moe_status moe_backward(const moe_config* cfg, const void* x, const void* w_router,
                        const float* logit_bias, const float* sel_bias,
                        const void* w1, const void* w3, const void* b1,
                        const void* w2, const void* b2,
                        const void* s_w1, const void* s_w3, const void* s_b1,
                        const void* s_w2, const void* s_b2,
                        const void* dy, float aux_coef, float z_coef, const moe_grads* grads,
                        int32_t* topk_ids, float* topk_w, int32_t* counts, float* stats, int saved,
                        void* ws, size_t ws_bytes, void* const* stage_events, void* stream);

/* The forward for training: the layer's output y and routing outputs as moe_forward's
 * (bfloat16, dropless only, like moe_backward), run so that its intermediates stay in the
 * workspace (moe_workspace_size(cfg, MOE_OP_BACKWARD) bytes) for moe_backward(saved = 1):
 * the logits, x_sorted, the up projection's pre-activations and the gate-scaled hidden
 * activations w_a h_a, from which the down projection computes y_sorted = (w_a h_a) W2^T +
 * w_a b2. y equals moe_forward's within the bfloat16 tolerance (h is rounded after the gate
 * is applied instead of before); ids, gates, counts and statistics are the same bits. */
moe_status moe_forward_train(const moe_config* cfg, const void* x, const void* w_router,
                             const float* logit_bias, const float* sel_bias,
                             const void* w1, const void* w3, const void* b1,
                             const void* w2, const void* b2,
                             const void* s_w1, const void* s_w3, const void* s_b1,
                             const void* s_w2, const void* s_b2,
                             void* y, int32_t* topk_ids, float* topk_w, int32_t* counts, float* stats,
                             void* ws, size_t ws_bytes, void* stream);

/* Aux-free load balancing, one update step ([L7.8] §2.5): with load_e = counts[e] and
 * mean = sum_e load_e / E,
 *     sel_bias[e] <- sel_bias[e] + rate * sign(mean - load_e)
 * so under-loaded experts become easier to select. The sign is decided exactly in integers
 * (sign(sum - E load_e)); the add is one float32 addition per expert. The bias enters
 * selection only (moe_route / moe_forward sel_bias), never the gates.
 * In: counts [E] int32 (e.g. moe_route's output for the last batch); rate: finite.
 * In/out: sel_bias [E] float32. No workspace. */
moe_status moe_update_bias(const moe_config* cfg, const int32_t* counts, float* sel_bias,
                           float rate, void* stream);

/* Synchronises `stream`, then reads and clears the device error word at the start of `ws`:
 * MOE_ERR_BAD_EXPERT_ID if the last dispatch on this workspace met an out-of-range id,
 * MOE_ERR_INVALID_ARG if an expert FFN call on it met a malformed offsets array (the call
 * clamped it, so no access left the buffers), MOE_ERR_HIP if the synchronisation or copy
 * failed, else MOE_OK. */
moe_status moe_get_device_error(void* ws, void* stream);

/* A static, human-readable name for a status code. */
const char* moe_status_string(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
