// Internal helpers shared by the HIP kernels of the MoE layer library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- bf16 <-> fp32
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// round to nearest even; NaN stays a quiet NaN
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p, size_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void store(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// SiLU(z) * v in fp32
__device__ __forceinline__ float swiglu(float z, float v) { return z / (1.0f + __expf(-z)) * v; }

// ---------------------------------------------------------------- scheduling
// Workgroups are dealt round-robin to the 8 XCDs (id % 8). Remap so that each XCD
// receives a contiguous range of logical tile ids: neighbouring tiles (which share
// operands) then run on the same XCD and share its L2. `n` must be a multiple of 8.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int per = n >> 3;
  return (bid & 7) * per + (bid >> 3);
}

// Largest g in [0, n_groups) with prefix[g] <= m (prefix is non-decreasing, prefix[0] = 0).
__device__ __forceinline__ int find_group(const int* __restrict__ prefix, int n_groups, int m) {
  int lo = 0, hi = n_groups - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= m) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------- launchers (host)
hipError_t launch_route(const void* u, int u_dtype, const float* centroids, const float* bias,
                        const float* logit_offset, const float* affinity_in, int T, int H, int N_r,
                        int K, int n_groups, int topk_groups, float* affinity_out, int32_t* topk_idx,
                        float* topk_gate, void* ws, hipStream_t st);
size_t route_workspace(int T, int H, int N_r);

hipError_t launch_permute(const int32_t* topk_idx, int T, int K, int N_r, int shared_rows, int32_t* counts,
                          int32_t* offsets, int32_t* row_token, int32_t* slot_row, void* ws,
                          hipStream_t st);
hipError_t launch_gather_rows(const void* x, const float* x_scales, int T, int row_bytes, int n_sc,
                              const int32_t* row_token, const int32_t* n_rows, int max_rows, void* x_perm,
                              float* x_perm_scales, hipStream_t st);
size_t permute_workspace(int T, int K, int N_r);
// moe_permute_noalloc: the device address of the library's static per-device scratch array on
// the current device (looked up once per device); permute_workspace() must not exceed its size
constexpr size_t PERMUTE_SCRATCH_BYTES = (size_t)4 << 20;
hipError_t permute_scratch(void** ptr);

struct FfnArgs {
  int n_groups;
  const int32_t* offsets;
  int total_rows;
  const int32_t* row_index;
  const void* X;
  const float* X_scales;
  int x_rows;
  int x_dtype;
  const void* Wg;
  const void* Wu;
  const void* Wd;
  const float* Wg_s;
  const float* Wu_s;
  const float* Wd_s;
  int H, I;
  void* Y;
  int y_dtype;
  void* ws;
  float* ZV = nullptr;   // bf16 only: also write the pre-activations z | v [total_rows, 2I] fp32
};
// events (may be NULL): hipEvent_t[4] recorded before the gate/up GEMM, after it, before the
// down GEMM (after the FP8 re-quantization of h) and after the down GEMM; NULL entries are skipped.
hipError_t launch_grouped_ffn(const FfnArgs& a, hipStream_t st, void* const* events);
size_t grouped_ffn_workspace(int n_groups, int total_rows, int H, int I, int x_dtype);

hipError_t launch_combine(const void* u, const void* shared_y, const void* Y, const int32_t* slot_row,
                          const float* gate, int T, int K, int H, int total_rows, int io_dtype,
                          int y_dtype, void* out, hipStream_t st);
hipError_t launch_bias_update(const int32_t* counts, int N_r, int T, int K, float gamma, float* bias,
                              hipStream_t st);
hipError_t launch_fp8_quant(const void* x, int x_dtype, int rows, int cols, int tile_rows,
                            uint8_t* codes, float* scales, hipStream_t st);
hipError_t launch_fp8_quant_rows_gather(const void* x, int x_dtype, int x_rows, int rows, int cols,
                                        const int32_t* row_index, const int32_t* n_live, uint8_t* codes,
                                        float* scales, hipStream_t st);
hipError_t launch_fp8_quant_rows_scatter(const void* x, int x_dtype, int T, int cols, int K,
                                         const int32_t* owner, const int32_t* slot, int max_rows,
                                         uint8_t* codes, float* scales, hipStream_t st);

struct FfnBwdArgs {
  int n_groups;
  const int32_t* offsets;
  int total_rows;
  const int32_t* row_index;
  const void* X;
  int x_rows;
  const void *Wg, *Wu, *Wd, *dY;
  void *dX, *dWg, *dWu, *dWd;
  int H, I;
  void* ws;
  const float* zv = nullptr;   // pre-activations saved by the forward; NULL: recompute them
};
bool gate_up_preact_supported(int H, int I);
hipError_t launch_gate_up_preact(const int32_t* offsets, int n_groups, int total_rows, const int32_t* row_index,
                                 const void* X, int x_rows, const void* Wg, const void* Wu, int H, int I,
                                 int32_t* prefix, float* ZV, hipStream_t st);
// C[r][n] = sum_k A[r][k] B(k, n) over each group's rows (A [total_rows, K] bf16, C fp32
// [total_rows, N]), B(k, n) = k < split ? W0[g][k][n] : W1[g][k - split][n] (bf16, n contiguous):
// the LDS-tiled kernel with transposing B reads. prefix: n_groups + 1 ints of workspace.
bool rows_mn_supported(int N, int K, int split);
hipError_t launch_rows_mn(const int32_t* offsets, int n_groups, int total_rows, const void* A, const void* W0,
                          const void* W1, int split, int N, int K, int32_t* prefix, float* C, hipStream_t st);
// C[r][n] = sum_k A[r][k] W_g[n][k] over each group's rows: A E4M3 codes [total_rows, K] with 1x128
// scales As [total_rows, K/128], W E4M3 [n_groups, N, K] with 128x128 block scales [n_groups, N/128,
// K/128], C fp32 [total_rows, N] (the forward's down-GEMM kernels). N % 64 == 0, K % 128 == 0.
// prefix: n_groups + 1 ints of workspace.
hipError_t launch_fp8_rows_gemm(const int32_t* offsets, int n_groups, int total_rows, const uint8_t* A,
                                const float* As, const uint8_t* W, const float* Ws, int N, int K, float* C,
                                int32_t* prefix, hipStream_t st);
size_t grouped_ffn_backward_workspace(int n_groups, int total_rows, int H, int I);

// FP8 layer backward: the transposed weight codes the dgrad GEMMs read (once per weight set)
struct Fp8TransposeArgs {
  int n_groups, H, I;
  const uint8_t *Wg, *Wu, *Wd;
  const float *Wg_s, *Wu_s, *Wd_s;
  uint8_t *WdT, *WguT;      // [G, I, H], [G, H, 2I]
  float *WdT_s, *WguT_s;    // [G, I/128, H/128], [G, H/128, 2I/128]
};
hipError_t launch_fp8_transpose_weights(const Fp8TransposeArgs& a, hipStream_t st);
struct FfnBwdFp8Args {
  int n_groups;
  const int32_t* offsets;
  int total_rows;
  const int32_t* row_index;
  const void* X;            // bf16 [x_rows, H]
  int x_rows;
  const uint8_t *Wg, *Wu, *WdT, *WguT;
  const float *Wg_s, *Wu_s, *WdT_s, *WguT_s;
  const void* dY;           // bf16 [total_rows, H]
  float *dX, *dWg, *dWu, *dWd;
  int H, I;
  void* ws;
};
size_t grouped_ffn_backward_fp8_workspace(int n_groups, int total_rows, int H, int I);
hipError_t launch_grouped_ffn_backward_fp8(const FfnBwdFp8Args& a, hipStream_t st, void* const* events);
hipError_t launch_grouped_ffn_backward(const FfnBwdArgs& a, hipStream_t st, void* const* events);
hipError_t launch_combine_backward(const void* dout, int io_dtype, const void* Y, int y_dtype,
                                   const int32_t* slot_row, const float* gate, int T, int K, int H, int S,
                                   int total_rows, uint16_t* dY, float* dgate, hipStream_t st);
hipError_t launch_router_backward(const void* dout, const void* u, int io_dtype, const float* dX,
                                  const int32_t* offsets, int g0, const int32_t* row_token,
                                  const int32_t* slot_row, int S, int total_rows, const float* s,
                                  const int32_t* idx, const float* gate, const float* dgate, const float* E,
                                  int T, int K, int H, int N_r, float* du, float* dE, float* dlogit_rows,
                                  hipStream_t st);

size_t seq_balance_workspace(int T, int N_r, int seq_len);
hipError_t launch_seq_balance_loss(const float* s, const int32_t* idx, int T, int N_r, int K, int seq_len,
                                   float alpha, float* loss, void* ws, hipStream_t st);

size_t payload_workspace(int T, int K, int n_ranks);
hipError_t launch_pack_fp8_payload(const void* x, int x_dtype, int T, int H, const int32_t* topk_idx, int K,
                                   int N_r, int n_ranks, int32_t* counts, int32_t* offsets,
                                   int32_t* send_token, int32_t* slot_send, uint8_t* codes, float* scales,
                                   void* ws, hipStream_t st);
hipError_t launch_unpack_fp8_payload(const uint8_t* codes, const float* scales, int rows, int H, void* out,
                                     int out_dtype, hipStream_t st);

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace moe
