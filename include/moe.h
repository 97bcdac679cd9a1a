/*
 * moe.h — C ABI of the MI355X (gfx950) DeepSeekMoE feed-forward layer library.
 *
 * The layer (DeepSeek-V3 report as summarised on xyznot.com, "รายงานเชิงเทคนิคของ
 * DeepSeek-V3", Method §2 "DeepSeekMoE with auxiliary-loss-free balancing"):
 *
 *   s_{i,t}  = Sigmoid(u_t . e_i)                                  (affinity)
 *   g'_{i,t} = s_{i,t} if s_{i,t}+b_i in Topk({s_{j,t}+b_j}, K_r), else 0
 *   g_{i,t}  = g'_{i,t} / sum_j g'_{j,t}                           (normalised gate)
 *   h'_t     = u_t + sum_{shared} FFN(u_t) + sum_i g_{i,t} FFN_i(u_t)
 *   end of step: b_i -= gamma if expert i is overloaded, += gamma if underloaded.
 *
 * A forward pass is: moe_route -> moe_permute (shared expert as group 0) ->
 * [fp8_quant_tiles(u)] -> moe_grouped_ffn (shared and routed experts in one call)
 * -> moe_combine, then moe_bias_update at the end of a training step. The backward
 * pass (bf16) is moe_combine_backward -> moe_grouped_ffn_backward (or, after a
 * moe_grouped_ffn_train forward, moe_grouped_ffn_backward_saved) -> moe_router_backward.
 *
 * Conventions for every entry point:
 *  - Tensor arguments are DEVICE pointers owned by the caller. Row-major,
 *    0-based expert ids, int32 indices. The library never allocates and keeps no
 *    device state beyond its code objects; scratch memory comes in as a
 *    caller-owned `workspace` whose minimum size the *_workspace_size query gives.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call only enqueues work on it: no host synchronisation, no host reads
 *    of device data. Calls are thread-safe (stateless).
 *  - Every output is bitwise deterministic run to run (no floating-point atomics).
 *  - Errors: the return value is a moe_status_t. Arguments are validated on the
 *    host BEFORE any HIP call, so an invalid call enqueues nothing.
 *    moe_last_error() gives a thread-local message for the last failure.
 *    Values inside device buffers (expert ids, offsets, row indices) are not
 *    visible to the host; kernels bounds-check them where a bad value could
 *    cause an out-of-range access and then skip the offending entry.
 *  - dtype tags: MOE_F32, MOE_BF16 (bfloat16), MOE_FP8_E4M3 (OCP E4M3FN codes,
 *    one byte each, with fp32 scales).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status_t;

enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_VALUE = 1, /* null pointer, negative or inconsistent size */
  MOE_ERR_UNSUPPORTED = 2,   /* valid but unsupported shape / dtype combination */
  MOE_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the query says */
  MOE_ERR_HIP = 4            /* a HIP launch failed; moe_last_error() has HIP's message */
};

enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 };

#define MOE_ABI_VERSION 1
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 16

/* ------------------------------------------------------------------ router
 * Affinity, biased top-K selection and gate normalisation
 * ("รายงานเชิงเทคนิคของ DeepSeek-V3" Method §2, equations for s_{i,t}, g'_{i,t} and g_{i,t};
 * "Deepseek V3 国货之光 开源之光", section Auxiliary-Loss-Free Load Balancing: the bias b only picks
 * the experts and never enters the affinity used for the gates).
 *
 *   logit_{t,i} = u_t . centroids_i (+ logit_offset_i)     fp32 accumulation
 *   s_{t,i}     = 1 / (1 + exp(-logit_{t,i}))               fp32
 *   key_{t,i}   = fl32(s_{t,i} + bias_i)                    one fp32 add
 *   topk_idx[t] = the K experts with the largest keys, ordered by key
 *                 descending then expert index ascending (equal keys go to the
 *                 lower index)
 *   topk_gate[t,k] = s_{t,idx_k} / sum_k' s_{t,idx_k'}      fp32, k' ascending
 *
 * u            [T, H] in u_dtype (MOE_F32 or MOE_BF16). Ignored if affinity_in.
 * centroids    [N_r, H] fp32. Ignored if affinity_in.
 * bias         [N_r] fp32.
 * logit_offset [N_r] fp32 or NULL: added to the logit before the sigmoid (a
 *              workload knob that makes chosen experts hot); NULL normally.
 * affinity_in  [T, N_r] fp32 or NULL: if given, used as s directly (no GEMV, no
 *              sigmoid) — this compares selection on identical affinities.
 * affinity_out [T, N_r] fp32 or NULL: receives s.
 * topk_idx     [T, K] int32 out;  topk_gate [T, K] fp32 out.
 * workspace    >= moe_route_workspace_size(T, H, N_r) bytes (may be NULL if 0).
 * Limits: T >= 0 (T == 0 is a no-op), H >= 1, 1 <= N_r <= MOE_MAX_EXPERTS,
 * 1 <= K <= min(N_r, MOE_MAX_TOPK).
 */
size_t moe_route_workspace_size(int T, int H, int N_r);
moe_status_t moe_route(const void* u, int u_dtype, const float* centroids, const float* bias,
                       const float* logit_offset, const float* affinity_in, int T, int H, int N_r,
                       int K, float* affinity_out, int32_t* topk_idx, float* topk_gate,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Group-limited (node-limited) variant of moe_route: each token's K experts come from
 * at most topk_groups of n_groups groups ("DeepSeek：AI 領域的重大突破與開源策略",
 * innovation table, Node-Limited Routing: a token goes to at most M nodes;
 * "官方揭秘DeepSeek-V3模型训练全流程" §2.2: at most 4 nodes).
 * Group g holds experts [g*N_r/n_groups, (g+1)*N_r/n_groups). The pages do not say how
 * groups are chosen; this library's rule:
 *   score_{t,g} = fl32 sum of group g's K/topk_groups largest keys, largest first
 *   kept groups = the topk_groups largest scores (equal scores: lower group index)
 *   topk_idx[t] = Top-K as in moe_route over the kept groups' experts only
 * Gates are normalised over the selected unbiased s exactly as in moe_route. All other
 * arguments, outputs and the workspace are those of moe_route; n_groups = topk_groups = 1
 * is moe_route.
 * Limits (else MOE_ERR_UNSUPPORTED): 1 <= n_groups <= 64, N_r % n_groups == 0,
 * 1 <= topk_groups <= n_groups, K % topk_groups == 0, K/topk_groups <= N_r/n_groups.
 */
moe_status_t moe_route_group_limited(const void* u, int u_dtype, const float* centroids, const float* bias,
                                     const float* logit_offset, const float* affinity_in, int T, int H,
                                     int N_r, int K, int n_groups, int topk_groups, float* affinity_out,
                                     int32_t* topk_idx, float* topk_gate, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ dispatch
 * Single-GPU form of token dispatch: per-expert counts, exclusive offsets and a
 * stable row permutation; every one of the T*K assignments gets a row (no token
 * dropping: youleyou.com "官方揭秘DeepSeek-V3模型训练全流程" §2.2).
 * Histogram, scan and scatter are deterministic: their only atomics add integer counts
 * in LDS, and each row comes from a rank computed in (token, k) order. For T*K <= 4096
 * they run in one workgroup (the workspace is then unused); larger batches use chunked
 * kernels whose per-chunk counts live in the workspace.
 *
 *   counts[e]      = #{(t,k) : topk_idx[t,k] == e}
 *   rows are grouped by expert ascending, then token ascending:
 *   offsets[e]     = sum_{e' < e} counts[e'],  offsets[N_r] = number of valid entries
 *   row_token[r]   = token of row r
 *   slot_row[t*K+k]= row holding (t, k), or -1 if topk_idx[t,k] is outside [0, N_r)
 *
 * shared_rows = S > 0 also dispatches the always-on shared expert ("รายงานเชิงเทคนิคของ DeepSeek-V3"
 * Method §2: the shared experts take every token) as group 0 in front of the routed
 * experts, so one moe_grouped_ffn call computes shared and routed experts together:
 * rows [0, S) are group 0 with row_token[r] = r, routed expert e is group e + 1,
 * offsets has N_r + 2 entries (offsets[0] = 0, offsets[e+1] = S + sum_{e'<e} counts[e']),
 * and every row index above (row_token, slot_row) is shifted by S. counts stays per
 * routed expert.
 *
 * topk_idx [T, K] int32 in; counts [N_r], offsets [N_r+1] (or [N_r+2] with S > 0),
 * row_token [S + T*K], slot_row [T*K] int32 out. A token must not list the same expert
 * twice (moe_route never does). workspace >= moe_permute_workspace_size(T, K, N_r).
 */
size_t moe_permute_workspace_size(int T, int K, int N_r);
moe_status_t moe_permute(const int32_t* topk_idx, int T, int K, int N_r, int shared_rows,
                         int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* slot_row,
                         void* workspace, size_t workspace_bytes, void* stream);

/* moe_permute without a workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Same
 * arguments, layout and results as moe_permute (bit-identical: the same kernels), but
 * its per-chunk histograms live in a static device array of the library, one per GPU,
 * of moe_permute_noalloc_max_bytes() = 4 MiB, held until the process ends. It calls no
 * hipMalloc, hipFree or allocating routine. Calls whose moe_permute_workspace_size(T, K,
 * N_r) exceeds that size return MOE_ERR_WORKSPACE before any HIP call (for T > 512 the
 * histograms take T * N_r / 16 bytes, so e.g. T <= 262144 at N_r = 256). All calls on one GPU
 * share the array: calls that overlap in time on that GPU (different streams or threads)
 * race and must be serialised by the caller. The first call on a device looks the
 * array's address up on that device (hipGetSymbolAddress) and keeps it.
 */
size_t moe_permute_noalloc_max_bytes(void);
moe_status_t moe_permute_noalloc(const int32_t* topk_idx, int T, int K, int N_r, int shared_rows,
                                 int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* slot_row,
                                 void* stream);

/* Row gather of the dispatch: the rows each expert receives, as the all-to-all dispatch step of
 * "Deepseek V3 国货之光 开源之光" (databean.com.cn), section 分布式流水线 / 流水线分解, hands them
 * over; a permuted copy that an expert-parallel exchange or a library GEMM would consume (this
 * library's own grouped FFN gathers through row_token instead and does not need it):
 *
 *   x_perm[r, :] = x[row_token[r], :]          for r in [0, n), n = min(max(*n_rows, 0), max_rows)
 *   x_perm_scales[r, :] = x_scales[row_token[r], :]     (FP8 codes: H/128 fp32 scales per row)
 *
 * n_rows is read on the device, e.g. &offsets[N_r] of moe_permute (&offsets[N_r + 1] with a
 * shared group), so the host need not know the count. A row whose row_token is outside [0, T) is
 * written as zeros (codes 0, scales 0); rows r >= n are left untouched. Byte-exact copies.
 * x [T, H] of x_dtype (MOE_F32, MOE_BF16 or MOE_FP8_E4M3 codes with x_scales [T, H/128]); x_perm
 * [max_rows, H] of the same type (x_perm_scales [max_rows, H/128] for FP8). No workspace.
 * Limits (else MOE_ERR_UNSUPPORTED): x and x_perm 16-byte aligned, H * element size a multiple of
 * 16 bytes, H % 128 == 0 for FP8. With max_rows > 0, row_token, n_rows, x_perm (and x, x_scales,
 * x_perm_scales as the dtype needs them) must be non-NULL (else MOE_ERR_INVALID_VALUE).
 */
moe_status_t moe_gather_rows(const void* x, const float* x_scales, int x_dtype, int T, int H,
                             const int32_t* row_token, const int32_t* n_rows, int max_rows, void* x_perm,
                             float* x_perm_scales, void* stream);

/* ------------------------------------------------------------------ expert FFNs
 * Grouped SwiGLU expert FFN (the FFN_i of "รายงานเชิงเทคนิคของ DeepSeek-V3" Method §2, h'_t equation;
 * SwiGLU without biases is this library's reading — the pages only name FFN_i).
 * For group g in [0, n_groups) and rows r in [offsets[g], offsets[g+1]):
 *
 *   x_r  = X[row_index[r]]  (or X[r] if row_index is NULL)
 *   h_r  = SiLU(W_gate[g] x_r) * (W_up[g] x_r)          [I]   fp32 math
 *   Y[r] = W_down[g] h_r                                 [H]
 *
 * offsets [n_groups+1] int32 lives on the device (no host sync); total_rows is
 * the host-known upper bound of offsets[n_groups] and the row count of Y.
 * Rows past offsets[n_groups] are left untouched. The shared expert is
 * n_groups = 1 with offsets = {0, T}.
 * X       [x_rows, H]: x_dtype MOE_F32, MOE_BF16, or MOE_FP8_E4M3 codes with
 *         X_scales [x_rows, H/128] fp32 (one scale per 1x128 tile, as written by
 *         fp8_quant_tiles). A row index outside [0, x_rows) is never read out of
 *         bounds; that row's output is unspecified.
 * W_gate, W_up [n_groups, I, H]; W_down [n_groups, H, I] (K-contiguous rows) in
 *         w_dtype. For MOE_FP8_E4M3 the matching *_scales hold one fp32 scale
 *         per 128x128 block: Wg/Wu_scales [n_groups, I/128, H/128],
 *         Wd_scales [n_groups, H/128, I/128] ("官方揭秘DeepSeek-V3模型训练全流程" §4.3; "รายงานเชิงเทคนิคของ DeepSeek-V3"
 *         key ideas: 1x128 activation tiles, 128x128 weight blocks).
 * FP8 path: products of E4M3 codes accumulate in fp32 over each 128-wide K block,
 *         and each block's partial sum is multiplied by its activation and weight
 *         scales before it is added to the fp32 accumulator. h is re-quantized to
 *         E4M3 with 1x128 tiles (online absmax) before the down projection.
 * Supported (x_dtype, w_dtype): (F32, F32), (BF16, BF16), (FP8, FP8);
 *         y_dtype MOE_F32 or MOE_BF16. FP8 needs H % 128 == 0 and I % 128 == 0;
 *         BF16 needs H % 128 == 0 and I % 64 == 0.
 * X and the weights must be 16-byte aligned for BF16 and FP8 (MOE_ERR_UNSUPPORTED otherwise).
 * workspace >= moe_grouped_ffn_workspace_size(n_groups, total_rows, H, I, x_dtype).
 */
size_t moe_grouped_ffn_workspace_size(int n_groups, int total_rows, int H, int I, int x_dtype);
moe_status_t moe_grouped_ffn(int n_groups, const int32_t* offsets, int total_rows,
                             const int32_t* row_index, const void* X, const float* X_scales,
                             int x_rows, int x_dtype, const void* W_gate, const void* W_up,
                             const void* W_down, const float* Wg_scales, const float* Wu_scales,
                             const float* Wd_scales, int w_dtype, int H, int I, void* Y, int y_dtype,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Same as moe_grouped_ffn, and records events[0..3] (hipEvent_t passed as void*, each may be
 * NULL; events itself may be NULL) on `stream` before the gate/up GEMM kernel, after it, before
 * the down GEMM kernel (after the FP8 re-quantization of h, which the LDS-tiled FP8 gate/up kernel
 * does in its epilogue, so that events[1] and events[2] then coincide) and after the down GEMM
 * kernel, so a caller can time each kernel with hipEventElapsedTime. For measurement only.
 */
moe_status_t moe_grouped_ffn_profiled(int n_groups, const int32_t* offsets, int total_rows,
                                      const int32_t* row_index, const void* X, const float* X_scales,
                                      int x_rows, int x_dtype, const void* W_gate, const void* W_up,
                                      const void* W_down, const float* Wg_scales,
                                      const float* Wu_scales, const float* Wd_scales, int w_dtype,
                                      int H, int I, void* Y, int y_dtype, void* workspace,
                                      size_t workspace_bytes, void* stream, void* const* events);

/* Training form of moe_grouped_ffn for BF16 (x_dtype = w_dtype = MOE_BF16, no scales): the same
 * Y, and also the gate/up pre-activations of every row, z = W_gate[g] x and v = W_up[g] x, fp32
 * [total_rows, 2I] row-major (z in columns [0, I), v in [I, 2I)), exactly the values Y was
 * computed from, for moe_grouped_ffn_backward_saved (which then skips recomputing them). zv is
 * caller-owned, 4-byte aligned; rows outside every group are unspecified. events as in
 * moe_grouped_ffn_profiled (may be NULL). Same workspace as moe_grouped_ffn.
 */
moe_status_t moe_grouped_ffn_train(int n_groups, const int32_t* offsets, int total_rows,
                                   const int32_t* row_index, const void* X, int x_rows, const void* W_gate,
                                   const void* W_up, const void* W_down, int H, int I, void* Y, int y_dtype,
                                   float* zv, void* workspace, size_t workspace_bytes, void* stream,
                                   void* const* events);

/* ------------------------------------------------------------------ combine
 * Residual + shared + gate-weighted routed outputs ("รายงานเชิงเทคนิคของ DeepSeek-V3" Method §2, h'_t):
 *
 *   out[t] = u[t] + shared_y[t] + sum_{k ascending} topk_gate[t,k] * Y[slot_row[t*K+k]]
 *
 * fp32 arithmetic in that fixed order, rounded once to io_dtype.
 * u, out [T, H] in io_dtype (MOE_F32 / MOE_BF16); shared_y [T, H] in y_dtype or
 * NULL; Y [total_rows, H] in y_dtype; slot_row [T*K]; topk_gate [T, K] fp32.
 * Slot rows outside [0, total_rows) contribute nothing.
 */
moe_status_t moe_combine(const void* u, const void* shared_y, const void* Y,
                         const int32_t* slot_row, const float* topk_gate, int T, int K, int H,
                         int total_rows, int io_dtype, int y_dtype, void* out, void* stream);

/* ------------------------------------------------------------------ bias update
 * Auxiliary-loss-free balancing, end of step ("รายงานเชิงเทคนิคของ DeepSeek-V3" Method §2, gamma = 0.001;
 * "Deepseek V3 国货之光 开源之光", Auxiliary-Loss-Free Load Balancing section):
 *
 *   bias[i] = fl32(bias[i] - gamma)  if N_r*counts[i] > T*K   (overloaded)
 *   bias[i] = fl32(bias[i] + gamma)  if N_r*counts[i] < T*K   (underloaded)
 *   unchanged                        if equal to the batch mean
 *
 * counts [N_r] int32 (from moe_permute), bias [N_r] fp32 in place. gamma finite.
 */
moe_status_t moe_bias_update(const int32_t* counts, int N_r, int T, int K, float gamma,
                             float* bias, void* stream);

/* ------------------------------------------------------------------ FP8 quantization
 * Online-absmax E4M3 quantization with one scale per tile ("官方揭秘DeepSeek-V3模型训练全流程" §4.3:
 * 1x128 activation tiles, 128x128 weight blocks, max |x| taken online):
 *
 *   scale      = fl32(amax(tile) / 448)                       (fp32 division)
 *   codes[r,c] = E4M3FN(fl32(x[r,c] / scale)), round to nearest even,
 *                saturated to +-448, sign bit copied from x; never NaN
 *   an all-zero tile gets scale 0 and codes 0x00 / 0x80.
 *
 * x [rows, cols] in x_dtype (MOE_F32 or MOE_BF16); tile_rows in {1, 128},
 * tile_cols == 128, rows % tile_rows == 0, cols % 128 == 0.
 * codes [rows, cols] uint8; scales [rows/tile_rows, cols/128] fp32.
 * To quantize a stack of weight matrices [G, R, C] with 128x128 blocks, pass
 * rows = G*R (R % 128 == 0): blocks never straddle two matrices.
 * x and codes must be 16-byte aligned (MOE_ERR_UNSUPPORTED otherwise).
 * Non-finite inputs are outside the contract.
 */
moe_status_t fp8_quant_tiles(const void* x, int x_dtype, int rows, int cols, int tile_rows,
                             int tile_cols, uint8_t* codes, float* scales, void* stream);

/* ------------------------------------------------------------------ status */
/* ------------------------------------------------------------------ backward (bf16 operands)
 * Gradients of the layer for an upstream gradient dout of h' (training with the layer: "官方揭秘DeepSeek-V3模型训练全流程"
 * "官方揭秘DeepSeek-V3模型训练全流程" §4.3 trains the model, so this layer, with FP8 GEMMs; here
 * bf16 operands with fp32 accumulation and fp32 gradients). The top-K selection is piecewise
 * constant: no gradient flows through it or into the bias ("Deepseek V3 国货之光 开源之光", Auxiliary-Loss-Free Load Balancing section: b only
 * selects). Call order, each step enqueued on one stream:
 *   moe_combine_backward -> moe_grouped_ffn_backward -> moe_router_backward.
 * Every sum runs in a fixed order: all gradients are bitwise reproducible run to run.
 *
 * moe_combine_backward: for the forward combine out_t = u_t + shared_t + sum_k g_{t,k} Y[slot_row[t,k]]:
 *   dY[t]            = dout_t                       (shared expert rows [0, shared_rows), if any)
 *   dY[slot_row[t,k]]= g_{t,k} dout_t                (bf16)
 *   dgate[t,k]       = dout_t . Y[slot_row[t,k]]     (fp32)
 * dout [T, H] in io_dtype; Y [total_rows, H] in y_dtype (the forward's expert outputs); dY
 * [total_rows, H] bf16 out (rows not listed above are left untouched); dgate [T, K] fp32 out.
 * shared_rows is 0 or T (the layout moe_permute(shared_rows = T) produces).
 */
moe_status_t moe_combine_backward(const void* dout, int io_dtype, const void* Y, int y_dtype, const int32_t* slot_row,
                                  const float* topk_gate, int T, int K, int H, int shared_rows, int total_rows,
                                  void* dY, float* dgate, void* stream);

/* moe_grouped_ffn_backward: for the groups of moe_grouped_ffn (bf16), with z = W_g x, v = W_u x,
 * h = SiLU(z) v recomputed from X:
 *   dh = dY W_d, dz = dh v SiLU'(z), dv = dh SiLU(z)       (dz, dv rounded to bf16)
 *   dX[r]      = dz W_g + dv W_u                             fp32 [total_rows, H]
 *   dW_down[g] = sum over g's rows of dY^T h                 fp32 [n_groups, H, I]
 *   dW_gate[g] = sum over g's rows of dz^T x, dW_up likewise  fp32 [n_groups, I, H]
 * X, row_index, offsets, total_rows and the weights are those of the forward call; dY
 * [total_rows, H] bf16. Groups without rows get zero weight gradients; dX rows outside every
 * group are unspecified. H % 128 == 0 and I % 128 == 0; X, dY and the weights 16-byte aligned.
 * workspace >= moe_grouped_ffn_backward_workspace_size(n_groups, total_rows, H, I) bytes.
 * The _profiled form records events[0..3] (caller-created hipEvent_t) around the row GEMMs
 * (z/v recompute, dh, dX) and around the weight-gradient GEMMs.
 */
size_t moe_grouped_ffn_backward_workspace_size(int n_groups, int total_rows, int H, int I);
moe_status_t moe_grouped_ffn_backward(int n_groups, const int32_t* offsets, int total_rows, const int32_t* row_index,
                                      const void* X, int x_rows, const void* W_gate, const void* W_up,
                                      const void* W_down, const void* dY, int H, int I, float* dX, float* dW_gate,
                                      float* dW_up, float* dW_down, void* workspace, size_t workspace_bytes,
                                      void* stream);
moe_status_t moe_grouped_ffn_backward_profiled(int n_groups, const int32_t* offsets, int total_rows,
                                               const int32_t* row_index, const void* X, int x_rows,
                                               const void* W_gate, const void* W_up, const void* W_down,
                                               const void* dY, int H, int I, float* dX, float* dW_gate,
                                               float* dW_up, float* dW_down, void* workspace,
                                               size_t workspace_bytes, void* stream, void* const* events);

/* moe_grouped_ffn_backward_saved: moe_grouped_ffn_backward with the pre-activations zv
 * [total_rows, 2I] fp32 that moe_grouped_ffn_train wrote for the same call (same X, row_index,
 * offsets and weights) instead of recomputing them; the gradients are bitwise those of
 * moe_grouped_ffn_backward. events may be NULL (else as in the _profiled form). Same workspace.
 */
moe_status_t moe_grouped_ffn_backward_saved(int n_groups, const int32_t* offsets, int total_rows,
                                            const int32_t* row_index, const void* X, int x_rows,
                                            const void* W_gate, const void* W_up, const void* W_down,
                                            const void* dY, const float* zv, int H, int I, float* dX,
                                            float* dW_gate, float* dW_up, float* dW_down, void* workspace,
                                            size_t workspace_bytes, void* stream, void* const* events);

/* ------------------------------------------------------------------ backward (FP8 operands)
 * The FP8 layer's backward: every GEMM operand in E4M3 with an fp32 scale per tile, fp32
 * accumulation ("官方揭秘DeepSeek-V3模型训练全流程" §4.3, FP8 training: activations in 1x128 tiles,
 * weights in 128x128 blocks; §4.5: the backward needs operands quantized along another axis).
 * This library's reading: each operand is quantized (scale = fl32(amax/448), E4M3 round to nearest
 * even, saturating) from its high-precision value along its GEMM's reduction dimension:
 *   z = Q(x) Q(W_g)^T, v = Q(x) Q(W_u)^T              x: 1x128 tiles along H (recomputed from X)
 *   dh = Q(dy) Q(W_d)                                  dy: 1x128 tiles along H
 *   h = SiLU(z) v, dz = dh v SiLU'(z), dv = dh SiLU(z) fp32
 *   dX[r] = Q(dz) Q(W_g) + Q(dv) Q(W_u)                dz, dv: 1x128 tiles along I     fp32 [total_rows, H]
 *   dW_down[g] = Qr(dy)^T Qr(h), dW_gate[g] = Qr(dz)^T Qr(x), dW_up[g] = Qr(dv)^T Qr(x)   fp32
 * where Qr quantizes 128x1 tiles: 128 consecutive rows of group g (from its first row; the last
 * tile holds the rest) of one column. Call order: moe_combine_backward -> moe_grouped_ffn_backward_fp8
 * -> moe_router_backward (as for bf16).
 *
 * moe_fp8_transpose_weights (once per FP8 weight set, e.g. after fp8_quant_tiles of the weights):
 * the transposed codes the dgrad GEMMs read. A 128x128 block's codes and scale serve W and W^T:
 *   W_down_t[g][i][h] = W_down[g][h][i]                  [G, I, H] codes, Wd_t_scales [G, I/128, H/128]
 *   W_gate_up_t[g][h][i] = W_gate[g][i][h], W_gate_up_t[g][h][I + i] = W_up[g][i][h]
 *                                                        [G, H, 2I] codes, Wgu_t_scales [G, H/128, 2I/128]
 * Inputs: W_gate, W_up [G, I, H] with scales [G, I/128, H/128]; W_down [G, H, I] with [G, H/128, I/128].
 * H % 128 == 0, I % 128 == 0; codes 16-byte aligned.
 *
 * moe_grouped_ffn_backward_fp8: groups, offsets, row_index, X (bf16 u [x_rows, H]) and total_rows
 * as in the forward moe_grouped_ffn call; W_gate/W_up codes + scales as in the forward; the two
 * transposed weights from moe_fp8_transpose_weights; dY bf16 [total_rows, H] (moe_combine_backward).
 * Outputs fp32: dX [total_rows, H], dW_gate / dW_up [n_groups, I, H], dW_down [n_groups, H, I];
 * groups without rows get zero weight gradients. H % 128 == 0, I % 128 == 0, H <= 16384,
 * I <= 8192; X, dY, dX and the codes 16-byte aligned. workspace >=
 * moe_grouped_ffn_backward_fp8_workspace_size(n_groups, total_rows, H, I). events: NULL or 4
 * caller-created hipEvent_t recorded around the row GEMMs and around the weight-gradient GEMMs.
 */
moe_status_t moe_fp8_transpose_weights(int n_groups, int H, int I, const uint8_t* W_gate, const float* Wg_scales,
                                       const uint8_t* W_up, const float* Wu_scales, const uint8_t* W_down,
                                       const float* Wd_scales, uint8_t* W_down_t, float* Wd_t_scales,
                                       uint8_t* W_gate_up_t, float* Wgu_t_scales, void* stream);
size_t moe_grouped_ffn_backward_fp8_workspace_size(int n_groups, int total_rows, int H, int I);
moe_status_t moe_grouped_ffn_backward_fp8(int n_groups, const int32_t* offsets, int total_rows,
                                          const int32_t* row_index, const void* X, int x_rows,
                                          const uint8_t* W_gate, const float* Wg_scales, const uint8_t* W_up,
                                          const float* Wu_scales, const uint8_t* W_down_t, const float* Wd_t_scales,
                                          const uint8_t* W_gate_up_t, const float* Wgu_t_scales, const void* dY,
                                          int H, int I, float* dX, float* dW_gate, float* dW_up, float* dW_down,
                                          void* workspace, size_t workspace_bytes, void* stream,
                                          void* const* events);

/* moe_router_backward: gates, sigmoid and router ("รายงานเชิงเทคนิคของ DeepSeek-V3" Method §2: g = s / sum s over the
 * selected experts, s = Sigmoid(u . e)), plus the input gradient:
 *   ds_k      = (dgate_k - sum_j g_j dgate_j) / sum_j s_j,   dlogit_k = ds_k s_k (1 - s_k)
 *   du_t      = dout_t + dX_rows[t] (if shared_rows) + sum_k dX_rows[slot_row[t,k]]
 *               + sum_k dlogit_k centroids[idx_k]                       fp32 [T, H]
 *   dcentroids[i] = sum over routed rows r of expert i of dlogit_r u[row_token[r]]  fp32 [N_r, H]
 * affinity [T, N_r] is the forward's s (moe_route's affinity_out); offsets / row_token / slot_row
 * are moe_permute's (with shared_rows = 0 or T); dgate from moe_combine_backward; dX_rows from
 * moe_grouped_ffn_backward; dout and u [T, H] in io_dtype.
 * workspace >= moe_router_backward_workspace_size(total_rows) bytes (one float per row).
 */
size_t moe_router_backward_workspace_size(int total_rows);
moe_status_t moe_router_backward(const void* dout, const void* u, int io_dtype, const float* dX_rows,
                                 const int32_t* offsets, const int32_t* row_token, const int32_t* slot_row,
                                 int shared_rows, int total_rows, const float* affinity, const int32_t* topk_idx,
                                 const float* topk_gate, const float* dgate, const float* centroids, int T, int K,
                                 int H, int N_r, float* du, float* dcentroids, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ sequence-wise balance loss
 * The pages give only that a very small sequence-wise balance loss (alpha = 0.0001) complements the
 * bias rule ("รายงานเชิงเทคนิคของ DeepSeek-V3" Method §2, last sentence) to stop extreme imbalance inside one sequence
 * ("官方揭秘DeepSeek-V3模型训练全流程" §2.2); its formula is not on the pages. This library's reading, per sequence of
 * L = seq_len consecutive tokens (the last one may be shorter):
 *   f_i = N_r / (K L) * #{t in seq : i among topk_idx[t]}
 *   P_i = (1/L) * sum_{t in seq} s_{t,i} / sum_j s_{t,j}
 *   loss[q] = alpha * sum_i f_i P_i                       (fp32, deterministic)
 * affinity [T, N_r] fp32 (s, moe_route's affinity_out); topk_idx [T, K]; loss [ceil(T / seq_len)].
 * workspace >= moe_seq_balance_loss_workspace_size(T, N_r, seq_len) bytes.
 * Limits: 1 <= seq_len <= 16384, 1 <= K <= min(N_r, MOE_MAX_TOPK).
 */
size_t moe_seq_balance_loss_workspace_size(int T, int N_r, int seq_len);
moe_status_t moe_seq_balance_loss(const float* affinity, const int32_t* topk_idx, int T, int N_r, int K, int seq_len,
                                  float alpha, float* loss, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ expert-parallel payload
 * The send side of an expert-parallel dispatch, built and checked on one GPU (loop-back):
 * youleyou.com "官方揭秘DeepSeek-V3模型训练全流程" §4.3 (activations partly quantized to FP8
 * for communication) and §2.2 / §4.2 (a token is sent to a node once, at most 4 nodes).
 *
 * Rank r owns experts [r*N_r/n_ranks, (r+1)*N_r/n_ranks). Token t is sent to each rank that
 * owns at least one of its K experts, once per rank. Send rows are ordered by rank ascending,
 * then token ascending (atomic-free, deterministic):
 *   counts[r]       = rows sent to rank r;  offsets[r] = sum_{r'<r} counts[r'];
 *   offsets[n_ranks]= total rows (<= T*min(K, n_ranks))
 *   send_token[row] = the token of the row
 *   slot_send[t*K+k]= the row that carries token t to the rank of expert topk_idx[t,k]
 *                     (-1 if that id is outside [0, N_r))
 *   codes[row, :]   = E4M3FN codes of x[send_token[row]] quantized per 1x128 tile exactly as
 *                     fp8_quant_tiles(x, 1) does (so the receiver can feed them to the FP8
 *                     grouped FFN); scales[row, H/128] fp32.
 * x [T, H] bf16 or fp32 (16-byte aligned); topk_idx [T, K]; send_token [T*min(K, n_ranks)],
 * slot_send [T*K], codes [T*min(K, n_ranks), H] (16-byte aligned), scales
 * [T*min(K, n_ranks), H/128]: rows past offsets[n_ranks] are left untouched.
 * workspace >= moe_pack_fp8_payload_workspace_size(T, K, n_ranks) bytes.
 * Limits: 1 <= N_r <= MOE_MAX_EXPERTS, 1 <= K <= MOE_MAX_TOPK, n_ranks divides N_r,
 * H % 128 == 0.
 */
size_t moe_pack_fp8_payload_workspace_size(int T, int K, int n_ranks);
moe_status_t moe_pack_fp8_payload(const void* x, int x_dtype, int T, int H, const int32_t* topk_idx, int K,
                                  int N_r, int n_ranks, int32_t* counts, int32_t* offsets, int32_t* send_token,
                                  int32_t* slot_send, uint8_t* codes, float* scales, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Receive side: out[row, c] = fl32(decode(codes[row, c]) * scales[row, c/128]) (one rounding of
 * an exact product), stored as out_dtype (MOE_F32, or MOE_BF16 rounded to nearest even).
 * codes [rows, H] (8-byte aligned), scales [rows, H/128], out [rows, H]; H % 128 == 0. */
moe_status_t moe_unpack_fp8_payload(const uint8_t* codes, const float* scales, int rows, int H, void* out,
                                    int out_dtype, void* stream);

const char* moe_status_string(moe_status_t s);
const char* moe_last_error(void);
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
