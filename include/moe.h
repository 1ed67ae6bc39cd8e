/*
 * moe.h -- C ABI of libmoe, a DeepSeekMoE layer forward pass for AMD Instinct
 * MI355X (gfx950).
 *
 * The layer is the one of the "DeepSeek-V3 Technical Report" (papers-reader
 * rewrite of arXiv 2412.19437):
 *   §2.1.2  DeepSeekMoE: for the FFN input u_t, the output is the sum of the
 *           N_s shared experts applied to u_t and of the K_r selected routed
 *           experts weighted by their gating values; affinities are
 *           s_{i,t} = sigmoid(u_t . e_i) with e_i the centroid of routed
 *           expert i; gating values are the selected affinities normalised
 *           over the selected experts.
 *   §2.1.2  auxiliary-loss-free balancing: a bias b_i is added to s_{i,t} for
 *           the top-K choice only (the gating value uses the un-biased s);
 *           after each step b_i moves by gamma against expert i's whole-batch
 *           load; node-limited routing keeps a token on at most M groups;
 *           no token is dropped.
 *   §3.3    FP8: activations quantised in 1 x N_c tiles and weights in
 *           N_c x N_c blocks (N_c = 128), each group with its own fp32 scale;
 *           partial sums accumulated in fp32 every N_c products.
 *   §4.2    shape: d = 7168, 1 shared + 256 routed experts, expert
 *           intermediate size 2048, 8 routed experts per token, at most 4
 *           nodes (groups) per token, gamma = 0.001.
 *
 * Conventions for every call
 *   - Return 0 (MOE_OK) or a negative moe_status.  Argument checks run on the
 *     host before any HIP call, so a rejected call touches no device state.
 *     moe_last_error() gives a message for the calling thread's last failure.
 *   - The moe_shape struct is host memory; every array argument is a device
 *     pointer to row-major contiguous storage, owned by the caller.  The
 *     library keeps no pointer after a call returns, but kernels read and
 *     write the buffers until the stream reaches them.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) without host synchronisation; expert loads never leave the GPU.
 *   - No call allocates device memory: scratch space comes from the caller's
 *     workspace `ws` of `ws_bytes` bytes (size it with moe_workspace_bytes);
 *     the workspace must be 256-byte aligned.
 *   - Matrices of weights are stored [out][in] (the reduction dimension is
 *     contiguous).  bf16 is stored as its 16-bit pattern; e4m3 is OCP E4M3FN
 *     (largest finite 448) in one byte.
 *   - Inputs must be finite; NaN and infinity are not checked.
 *   - Calls on different streams that share a buffer race, workspaces
 *     included (a workspace holds intermediate results and the expert
 *     kernel's tile-queue counters); the library holds no global mutable
 *     state, so calls on different data may overlap.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,   /* null pointer, non-positive size, bad alignment */
    MOE_ERR_UNSUPPORTED = -2,   /* shape or dtype combination outside the limits below */
    MOE_ERR_WORKSPACE = -3,     /* ws_bytes smaller than moe_workspace_bytes() */
    MOE_ERR_HIP = -4            /* a HIP runtime call or kernel launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_E4M3 = 2 } moe_dtype;

/* flags */
#define MOE_ADD_RESIDUAL 1u   /* moe_forward / moe_combine add u_t to the output */
/* moe_forward keeps the SwiGLU inputs a = W_gate x and b = W_up x of every
 * routed and shared row (fp32, the gate/up accumulators as they are) in its
 * workspace, which grows by (T*topk + T*n_shared) * 2 * inter * 4 bytes;
 * moe_backward with the same flag then forms the SwiGLU gradient from them
 * instead of recomputing the gate/up product: the same bits, without a second
 * pass over W_gate and W_up.  Forward and backward must agree on this flag. */
#define MOE_SAVE_SWIGLU_INPUTS 2u

/*
 * Shape and numerics of one layer (§2.1.2, §4.2).  Supported combinations
 * (act_dtype, router_dtype, w_dtype, out_dtype):
 *   (F32,  F32,  F32,  F32 )  fp32 everywhere
 *   (BF16, BF16, BF16, BF16)  bf16 storage, fp32 accumulation
 *   (BF16, BF16, E4M3, BF16)  bf16 u and centroids; expert GEMMs in e4m3 with
 *                             1x128 activation / 128x128 weight fp32 scales
 * Limits (MOE_ERR_UNSUPPORTED otherwise): n_routed % n_groups == 0,
 * 1 <= topk_groups <= n_groups <= 64, 1 <= topk <= 32,
 * topk <= topk_groups * n_routed / n_groups, n_routed <= 1024,
 * 0 <= n_shared <= 8, d and inter multiples of 128, quant_block == 128,
 * T * topk < 2^31, T * n_shared < 2^31.
 */
typedef struct moe_shape {
    int64_t T;              /* tokens in the batch (T >= 0; T == 0 is a no-op) */
    int32_t d;              /* hidden size (7168) */
    int32_t n_routed;       /* N_r routed experts (256) */
    int32_t n_shared;       /* N_s shared experts (1) */
    int32_t n_groups;       /* expert groups (nodes) G (8); group g = experts [g*N_r/G, (g+1)*N_r/G) */
    int32_t topk_groups;    /* M: groups a token may use (4) */
    int32_t topk;           /* K_r: routed experts per token (8) */
    int32_t inter;          /* expert intermediate size I (2048) */
    int32_t act_dtype;      /* u, x_perm (non-e4m3), H (non-e4m3) storage: MOE_F32 | MOE_BF16 */
    int32_t router_dtype;   /* centroids gate_w: equal to act_dtype */
    int32_t w_dtype;        /* expert weights and GEMM inputs: act_dtype, or MOE_E4M3 */
    int32_t out_dtype;      /* y_perm, y_shared, out: equal to act_dtype */
    int32_t quant_block;    /* N_c = 128 */
    float routed_scale;     /* factor on every gating value (1.0) */
    uint32_t flags;         /* MOE_ADD_RESIDUAL | MOE_SAVE_SWIGLU_INPUTS, or 0 */
} moe_shape;

/* ------------------------------------------------------------------------ */

/*
 * moe_route -- affinities, group-limited biased top-K, gating values
 * (§2.1.2; the group rule and tie rule are readings of the prose):
 *   s[t][i]  = sigmoid(sum_c u[t][c] * gate_w[i][c])   fp32 accumulation
 *   s'       = s + bias (one fp32 add; used for selection only)
 *   group g score = sum of its two largest s' (its only s' if N_r/G == 1);
 *   the topk_groups best groups are kept, other experts are excluded;
 *   the topk largest s' among kept experts are selected, slot order is
 *   decreasing s'; every tie goes to the lower index;
 *   topk_w[t][j] = routed_scale * s[t][e_j] / (s[t][e_0] + ... + s[t][e_{K-1}])
 *   with the sum taken left to right in fp32.
 * u [T][d] (act_dtype), gate_w [N_r][d] (router_dtype), bias [N_r] fp32.
 * scores_in [T][N_r] fp32 or NULL: when given, u and gate_w are not read and
 * selection runs on these affinities (bit-exact routing checks).
 * scores_out [T][N_r] fp32 or NULL; topk_idx [T][K] int32; topk_w [T][K] fp32.
 * ws: moe_workspace_bytes(shape, MOE_WS_ROUTE) bytes (256-byte aligned): the
 * affinities when scores_out is NULL, and for bf16 layers of 256 routed experts
 * in groups of a multiple of 16 experts with topk <= 16 the chunk partials of
 * a split-K gate GEMM (fp32 partial dot products over chunks of the hidden
 * dimension, summed in chunk order).  Given less workspace (at least the
 * affinities' when scores_out is NULL) the single-pass gate GEMM runs instead:
 * the affinities agree up to the order of the fp32 additions.
 */
int moe_route(const moe_shape *shape, const void *u, const void *gate_w, const float *bias,
              const float *scores_in, float *scores_out, int32_t *topk_idx, float *topk_w,
              void *ws, size_t ws_bytes, void *stream);

/*
 * moe_permute -- dispatch bookkeeping and row gather (§2.1.2: every
 * (token, slot) pair is kept; "whole-batch load" = pairs per expert):
 *   counts[i]   = #{(t, j) : topk_idx[t][j] == i}
 *   offsets     = exclusive prefix sum of counts, offsets[N_r] = T*K
 *   rows offsets[i] .. offsets[i+1]-1 belong to expert i, in increasing t
 *   perm_token[row] = t,   inv_perm[t*K + j] = row
 *   x_perm[row] = u[t]              when w_dtype != E4M3 (act_dtype copy)
 *   x_perm[row] = Q_1x128(u[t]) with x_scales[row][d/128] when w_dtype == E4M3
 *     (Q: scale = amax/448 in fp32, 1 for an all-zero tile; code =
 *      E4M3 round-to-nearest-even of clamp(x/scale, -448, 448); §3.3).
 * x_perm may be NULL (index outputs only); then u and x_scales are ignored.
 * topk_idx entries must lie in [0, N_r) and be distinct within a token.
 * ws: moe_workspace_bytes(shape, MOE_WS_PERMUTE).
 */
int moe_permute(const moe_shape *shape, const int32_t *topk_idx, const void *u,
                int32_t *counts, int32_t *offsets, int32_t *perm_token, int32_t *inv_perm,
                void *x_perm, float *x_scales, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_grouped_ffn -- SwiGLU experts over ragged row groups (§2.1.2 experts;
 * the SwiGLU form is the reading of the unstated expert FFN):
 *   for expert e and each of its rows r in [offsets[e], offsets[e+1]):
 *     a = W_gate[e] x_r,  b = W_up[e] x_r        (fp32 accumulation)
 *     h = SiLU(a) * b,    SiLU(a) = a / (1 + exp(-a)),   stored as
 *         act_dtype, or for E4M3 quantised per 1x128 tile of I (Q above)
 *     y[r] = W_down[e] h  (fp32 accumulation), stored in out_dtype
 *   x_r = x[gather[r]] when gather != NULL, else x[r].
 *   For E4M3 every 128-long block of the reduction is an fp32 partial sum of
 *   code products, multiplied by (activation scale * weight block scale) and
 *   added to the fp32 accumulator (§3.3 promotion every N_c products).
 * n_exp experts; offsets [n_exp+1] int32 on the device, offsets[0] = 0,
 * non-decreasing, offsets[n_exp] <= max_rows.
 * x [*][d] in act_dtype, or e4m3 with x_scales [*][d/128] fp32.
 * w_gate, w_up [n_exp][I][d]; w_down [n_exp][d][I] in w_dtype;
 * w_scales: NULL unless E4M3, then 3 device pointers to fp32 block scales
 * [n_exp][I/128][d/128], [n_exp][I/128][d/128], [n_exp][d/128][I/128]
 * (the array of 3 pointers itself is host memory).
 * y [max_rows][d] out_dtype.  ws: moe_ffn_workspace_bytes(shape, max_rows).
 */
int moe_grouped_ffn(const moe_shape *shape, int32_t n_exp, const int32_t *offsets, int64_t max_rows,
                    const int32_t *gather, const void *x, const float *x_scales,
                    const void *w_gate, const void *w_up, const void *w_down,
                    const float *const *w_scales, void *y, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_combine -- the layer output (§2.1.2 output equation; stripped on the
 * page, read as shared experts plus gate-weighted routed experts):
 *   out[t] = sum_j topk_w[t][j] * y_perm[inv_perm[t*K + j]]
 *          + sum_s y_shared[s][t]  (+ u[t] if MOE_ADD_RESIDUAL)
 * computed in fp32 and rounded once to out_dtype.
 * y_perm [T*K][d], y_shared [N_s][T][d] (NULL when N_s == 0), out [T][d] in
 * out_dtype; residual = u [T][d] (act_dtype), read only with the flag.
 */
int moe_combine(const moe_shape *shape, const void *y_perm, const int32_t *inv_perm, const float *topk_w,
                const void *y_shared, const void *residual, void *out, void *stream);

/*
 * moe_forward -- the whole layer: moe_route, dispatch, the routed and shared
 * grouped FFNs and moe_combine in one enqueue.  For E4M3, u is quantised
 * once per token (1x128) and rows are gathered inside the expert GEMM instead
 * of being copied.
 * routed_w = {W_gate [N_r][I][d], W_up [N_r][I][d], W_down [N_r][d][I]};
 * shared_w = the same with N_s (NULL when N_s == 0).  routed_s / shared_s:
 * the 3 block-scale arrays for E4M3, else NULL.  (Pointer arrays are host
 * memory; their elements are device pointers.)
 * Optional outputs (NULL to skip): topk_idx_out [T][K], topk_w_out [T][K],
 * counts_out [N_r], scores_out [T][N_r].
 * ws: moe_workspace_bytes(shape, MOE_WS_FORWARD).  After the call it holds the
 * layer's saved activations (affinities, selection, gates, dispatch, H and the
 * expert outputs) that moe_backward reads; scores_out, topk_idx_out and
 * topk_w_out receive copies.
 */
int moe_forward(const moe_shape *shape, const void *u, const void *gate_w, const float *bias,
                const void *const *routed_w, const float *const *routed_s,
                const void *const *shared_w, const float *const *shared_s,
                void *out, int32_t *topk_idx_out, float *topk_w_out, int32_t *counts_out,
                float *scores_out, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_forward_timed -- moe_forward that also records caller-created HIP
 * events (hipEvent_t) on `stream` at its stage boundaries, for per-kernel
 * timing without a profiler:
 *   stage_events[0] before the router        [1] after routing (affinities + selection)
 *   [2] after dispatch (and e4m3 quantisation of u)
 *   [3] after the gate/up expert kernel      [4] after the down expert kernel
 *   [5] after the combine
 * NULL entries (or a NULL array, 6 entries otherwise) are skipped.  The array
 * itself is host memory.  Results are identical to moe_forward.
 */
int moe_forward_timed(const moe_shape *shape, const void *u, const void *gate_w, const float *bias,
                      const void *const *routed_w, const float *const *routed_s,
                      const void *const *shared_w, const float *const *shared_s,
                      void *out, int32_t *topk_idx_out, float *topk_w_out, int32_t *counts_out,
                      float *scores_out, void *ws, size_t ws_bytes, void *stream, void *const *stage_events);

/*
 * moe_forward_static -- moe_forward for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The caller passes inputs and outputs only (arguments,
 * results and errors as for moe_forward); the workspace is a buffer of
 * MOE_STATIC_WS_BYTES that the library keeps in device memory, one per GPU it
 * runs on, for the life of the process.  No call allocates or frees memory.
 * Limit: shapes whose moe_workspace_bytes(shape, MOE_WS_FORWARD) exceeds
 * MOE_STATIC_WS_BYTES are rejected with MOE_ERR_WORKSPACE (at the V3 shape,
 * d = 7168 with 256 + 1 experts of I = 2048 in bf16, that is T above about 400
 * tokens: decode-size batches fit); MOE_SAVE_SWIGLU_INPUTS is rejected with
 * MOE_ERR_UNSUPPORTED (the saved activations stay in the library's buffer,
 * where moe_backward cannot read them).  Every call on one GPU shares that
 * GPU's buffer, which keeps the last call's intermediate results: calls that
 * overlap on one GPU (other streams, other host threads) race, so a caller
 * serialises them.
 */
#define MOE_STATIC_WS_BYTES ((size_t)64 << 20)
int moe_forward_static(const moe_shape *shape, const void *u, const void *gate_w, const float *bias,
                       const void *const *routed_w, const float *const *routed_s,
                       const void *const *shared_w, const float *const *shared_s,
                       void *out, int32_t *topk_idx_out, float *topk_w_out, int32_t *counts_out,
                       float *scores_out, void *stream);

/* ------------------------------------------------------------------------ */
/* backward                                                                 */

/*
 * moe_transpose_expert_weights -- the transposed weight copies moe_backward
 * reads (input gradients run through the same grouped expert kernel as the
 * forward, which wants the reduction dimension contiguous):
 *   wt[0] = W_down^T [n][I][d] per expert,
 *   wt[1] = [W_gate^T | W_up^T] [n][d][2I] per expert,
 * from w = {W_gate [n][I][d], W_up [n][I][d], W_down [n][d][I]} in
 * shape->w_dtype.  For E4M3 the 128 x 128 block scales follow their blocks:
 * w_s = the three forward scale grids ([n][I/128][d/128], .., [n][d/128][I/128])
 * and wt_s = {[n][I/128][d/128], [n][d/128][2I/128]}; NULL otherwise.  The
 * copies are bit-exact.  Rebuild them whenever the weights change.
 * n = N_r for the routed and N_s for the shared experts.  (Pointer arrays are
 * host memory; their elements are device pointers.)
 */
int moe_transpose_expert_weights(const moe_shape *shape, int32_t n, const void *const *w, const float *const *w_s,
                                 void *const *wt, float *const *wt_s, void *stream);

/*
 * moe_backward -- gradient of the layer (§2.1.2) for the selection that
 * moe_forward made, given dout = dL/dh'_t [T][d]; the selection and the bias
 * are piecewise constant and take no gradient (reading: the balancing bias
 * moves only by the moe_bias_update rule).  For output row t,
 *   dy_{t,j} = g_{t,j} dout_t,   dg_{t,j} = dout_t . y_{t,j}   (y = expert output)
 *   expert (SwiGLU h = SiLU(a) * b, a = W_gate x, b = W_up x, y = W_down h):
 *     dh = W_down^T dy,  da = dh b SiLU'(a),  db = dh SiLU(a),
 *     dx = W_gate^T da + W_up^T db,
 *     dW_down = sum dy h^T,  dW_gate = sum da x^T,  dW_up = sum db x^T
 *   gate g_j = rs s_j / D, D = sum_k s_k over the selected k (rs = routed_scale):
 *     ds_j = rs (dg_j / D - (sum_k dg_k s_k) / D^2),  dz_j = ds_j s_j (1 - s_j)
 *     (z = u . e, s = sigmoid(z)),
 *   du_t = sum_j dx_{t,j} + sum_shared dx + sum_j dz_j e_{sel_j},
 *   de_i = sum over slots routed to i of dz u_t.
 * E4M3 layers (§3.3: Fprop, Dgrad and Wgrad GEMMs in FP8): the Dgrad GEMMs take
 * dy, dout and [da | db] in 1 x 128 tiles along their reduction with the
 * transposed 128 x 128 weight blocks; the Wgrad GEMMs take both operands in
 * 128 x 1 tiles along each expert's rows (runs of 128 from its first row):
 * dy, dout, [da | db], and the forward's cached 1 x 128 tiles of H and u,
 * re-tiled; fp32 accumulation per run with both column scales.  The router
 * chain (dg, dz, du's centroid term, dgate_w) stays in fp32.
 * (With MOE_ADD_RESIDUAL the residual's own gradient, dout, is the caller's
 * to add: du holds the layer's part only.)
 * Inputs: u, gate_w, the weights and (E4M3) their scales exactly as passed to
 * moe_forward; routed_wt / routed_wt_s from moe_transpose_expert_weights,
 * shared_* likewise (NULL when N_s == 0); *_s and *_wt_s are NULL for
 * fp32 / bf16 layers.  fwd_ws/fwd_ws_bytes: the forward workspace of the
 * moe_forward call whose output dout refers to, untouched since (it holds the
 * scores, selection, dispatch, H and Y, which are the saved activations,
 * and with MOE_SAVE_SWIGLU_INPUTS the SwiGLU inputs a and b).
 * Storage: dout, du and the weight gradients in act_dtype (bf16 for E4M3
 * layers).  Outputs: du [T][d]; optional (NULL to skip): dgate_w [N_r][d]
 * fp32, d_routed_w = {dW_gate, dW_up, dW_down} (layout of the forward weights,
 * act_dtype), d_shared_w likewise, dtopk_w [T][K] fp32 = dL/dg.  Gradients
 * are written, not accumulated.  Sums run in fp32 in a fixed order
 * (deterministic).  ws: moe_backward_workspace_bytes(shape).
 * Errors: MOE_ERR_WORKSPACE when fwd_ws_bytes is smaller than
 * moe_workspace_bytes(shape, MOE_WS_FORWARD); MOE_ERR_INVALID_ARG for a NULL
 * required pointer or scale.
 */
int moe_backward(const moe_shape *shape, const void *u, const void *gate_w, const void *const *routed_w,
                 const float *const *routed_s, const void *const *routed_wt, const float *const *routed_wt_s,
                 const void *const *shared_w, const float *const *shared_s, const void *const *shared_wt,
                 const float *const *shared_wt_s, const void *fwd_ws, size_t fwd_ws_bytes, const void *dout, void *du,
                 float *dgate_w, void *const *d_routed_w, void *const *d_shared_w, float *dtopk_w, void *ws,
                 size_t ws_bytes, void *stream);

/*
 * moe_backward_timed -- moe_backward that also records caller-created HIP
 * events on `stream` at its stage boundaries:
 *   stage_events[0] before the combine gradient   [1] after it (dY, dg; e4m3: their 1 x 128 tiles)
 *   [2] after dH = dY W_down                      [3] after the SwiGLU gradient pass ([dA | dB], tiled)
 *   [4] after dX = [dA | dB] [W_gate ; W_up]      [5] after the token pass (du, dz)
 *   [6] after the centroid gradient               [7] after the weight-gradient operands' tiling
 *   [8] after dW_down                             (e4m3: run bases and 128 x 1 tiles; else empty)
 *   [9] after dW_gate / dW_up
 * NULL entries (or a NULL array, 10 entries otherwise) are skipped; skipped
 * optional outputs leave their stage empty.  Results are identical to
 * moe_backward.
 */
int moe_backward_timed(const moe_shape *shape, const void *u, const void *gate_w, const void *const *routed_w,
                       const float *const *routed_s, const void *const *routed_wt, const float *const *routed_wt_s,
                       const void *const *shared_w, const float *const *shared_s, const void *const *shared_wt,
                       const float *const *shared_wt_s, const void *fwd_ws, size_t fwd_ws_bytes, const void *dout,
                       void *du, float *dgate_w, void *const *d_routed_w, void *const *d_shared_w, float *dtopk_w,
                       void *ws, size_t ws_bytes, void *stream, void *const *stage_events);

/* Workspace bytes for moe_backward (0 when rejected). */
size_t moe_backward_workspace_bytes(const moe_shape *shape);

/* ------------------------------------------------------------------------ */
/* helpers                                                                  */

enum { MOE_WS_ROUTE = 0, MOE_WS_PERMUTE = 1, MOE_WS_FORWARD = 2 };

/* Workspace bytes for moe_route / moe_permute / moe_forward at this shape,
 * or 0 when the shape is rejected (see moe_last_error). */
size_t moe_workspace_bytes(const moe_shape *shape, int which);

/* Workspace bytes for moe_grouped_ffn with max_rows rows (0 when rejected). */
size_t moe_ffn_workspace_bytes(const moe_shape *shape, int64_t max_rows);

/*
 * moe_bias_update -- one auxiliary-loss-free step (§2.1.2; gamma = 0.001 in
 * §4.2): mean = fp32(T*K) / fp32(N_r);
 *   bias[i] = bias[i] + gamma * sign(mean - counts[i])   (sign(0) = 0)
 * (reading: "overloaded" = load above the mean; an exact tie leaves b_i).
 * counts [N_r] int32, bias [N_r] fp32 updated in place.
 */
int moe_bias_update(const moe_shape *shape, const int32_t *counts, float *bias, float gamma, void *stream);

/*
 * moe_seq_balance -- complementary sequence-wise balance statistic (§2.1.2: a
 * tiny loss alpha * sum_i f_i P_i kept beside the bias rule; §4.2: alpha =
 * 0.0001).  The pages name f_i and P_i without defining them; reading, for a
 * sequence of Ts tokens:
 *   f_i = N_r / (K * Ts) * (slots of the sequence routed to expert i),
 *   P_i = (1/Ts) * sum_t s_{i,t} / sum_k s_{k,t}   (affinity share over all
 *         routed experts, un-biased s).
 * Sequences are consecutive runs of seq_len tokens of the batch (the last one
 * may be shorter): n_seq = ceil(T / seq_len).
 * scores [T][N_r] fp32 (moe_route's scores_out), topk_idx [T][K] int32.
 * loss [n_seq] fp32; counts [n_seq][N_r] int32 and share [n_seq][N_r] fp32
 * (P_i) are optional (NULL).  fp32 sums in a fixed order (deterministic).
 * ws: moe_seq_balance_workspace_bytes(shape, seq_len).
 * Errors: MOE_ERR_INVALID_ARG for seq_len < 1 or a NULL required pointer.
 */
int moe_seq_balance(const moe_shape *shape, const float *scores, const int32_t *topk_idx, int64_t seq_len,
                    float alpha, float *loss, int32_t *counts, float *share, void *ws, size_t ws_bytes,
                    void *stream);

/* Workspace bytes for moe_seq_balance (0 when rejected). */
size_t moe_seq_balance_workspace_bytes(const moe_shape *shape, int64_t seq_len);

/*
 * moe_quantize_1x128 -- Q over 1x128 tiles of each row of x [rows][cols]
 * (x_dtype MOE_F32 or MOE_BF16; cols % 128 == 0): q [rows][cols] e4m3,
 * s [rows][cols/128] fp32 (§3.3 activation tiles).
 */
int moe_quantize_1x128(int64_t rows, int32_t cols, int32_t x_dtype, const void *x, uint8_t *q, float *s,
                       void *stream);

/*
 * moe_quantize_weights_128x128 -- Q over 128x128 blocks of nmat matrices
 * w [nmat][rows][cols] (w_dtype MOE_F32 or MOE_BF16; rows, cols % 128 == 0):
 * q [nmat][rows][cols] e4m3, s [nmat][rows/128][cols/128] fp32 (§3.3 weight
 * blocks).  Weight preparation, not part of the per-step path.
 */
int moe_quantize_weights_128x128(int64_t nmat, int32_t rows, int32_t cols, int32_t w_dtype, const void *w,
                                 uint8_t *q, float *s, void *stream);

/*
 * moe_quantize_128x1 -- Q over 128x1 tiles down the rows of segments, the
 * operands of the FP8 weight-gradient GEMMs.  §3.3 runs Wgrad in FP8 and
 * names 1x128 activation tiles and 128x128 weight blocks, but no tile for a
 * GEMM that reduces over tokens.  Reading (not the page's text): a tile is
 * 128 consecutive elements along the GEMM's reduction, which for a weight
 * gradient runs down the token rows, i.e. 128x1; the tile origin is not
 * stated either, read as runs of 128 list rows from each segment's first row.
 *   n_seg segments; offsets [n_seg+1] (device, int32, offsets[0] >= 0,
 *   nondecreasing, offsets[n_seg] <= max_rows): segment e owns list rows
 *   offsets[e] .. offsets[e+1]-1, cut into runs of 128 rows from its first
 *   row (the last run of a segment may be shorter);
 *   list row r reads x row gather[r] (gather NULL: row r);
 *   x [.][cols] MOE_BF16, or MOE_E4M3 codes with 1x128 fp32 scales
 *   x_s [.][cols/128] (decoded to fp32 before the re-quantisation);
 *   q [offsets[n_seg]][cols] e4m3 codes, rows offsets[0].. written;
 *   s [n_blocks][cols] fp32: one scale per run and column, runs numbered
 *   segment by segment; block_base [n_seg+1] (device, int32, out): the
 *   first run of each segment, block_base[n_seg] = n_blocks
 *   <= max_rows/128 + n_seg.
 * A scale is amax/448 over its run's column (1 for an all-zero column);
 * codes are round-to-nearest-even of clamp(v/scale, -448, 448).
 * Offsets that break the stated order are undefined behaviour.
 * Errors: INVALID_ARG for negative sizes or a NULL buffer; UNSUPPORTED for
 * cols % 128 != 0 or another x_dtype.  n_seg == 0 does nothing.
 */
int moe_quantize_128x1(int32_t n_seg, const int32_t *offsets, int64_t max_rows, int32_t cols, int32_t x_dtype,
                       const void *x, const float *x_s, const int32_t *gather, uint8_t *q, float *s,
                       int32_t *block_base, void *stream);

/* Message for the calling thread's last failed call ("" if none). */
const char *moe_last_error(void);

/* Library version string. */
const char *moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
