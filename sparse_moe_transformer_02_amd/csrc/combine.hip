// Residual + shared + gate-weighted routed combine, and the end-of-step bias update.
//
// "รายงานเชิงเทคนิคของ DeepSeek-V3" Method §2: h'_t = u_t + sum_shared FFN(u_t) + sum_i g_{i,t} FFN_i(u_t), and the
// auxiliary-loss-free rule b_i -= gamma (overloaded) / += gamma (underloaded), gamma = 0.001.
#include "common.h"

namespace moe {

namespace {

// One workgroup per token; each thread owns VEC consecutive features per pass.
// out = ((u + shared) + g_0 * Y_0) + g_1 * Y_1 + ... in fp32, one rounding at the store.
template <typename TIO, typename TY, int VEC>
__global__ __launch_bounds__(256) void combine_kernel(const TIO* __restrict__ u,
                                                      const TY* __restrict__ shared_y,
                                                      const TY* __restrict__ Y,
                                                      const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ gate, int K, int H,
                                                      int total_rows, TIO* __restrict__ out) {
  const int t = blockIdx.x;
  __shared__ int32_t rows[MOE_MAX_TOPK];
  __shared__ float gs[MOE_MAX_TOPK];
  if ((int)threadIdx.x < K) {
    const int r = slot_row[(size_t)t * K + threadIdx.x];
    rows[threadIdx.x] = (r >= 0 && r < total_rows) ? r : -1;
    gs[threadIdx.x] = gate[(size_t)t * K + threadIdx.x];
  }
  __syncthreads();
  for (int h0 = threadIdx.x * VEC; h0 < H; h0 += 256 * VEC) {
    float acc[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = Elem<TIO>::load(u, (size_t)t * H + h0 + v);
    if (shared_y) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[v] += Elem<TY>::load(shared_y, (size_t)t * H + h0 + v);
    }
    for (int k = 0; k < K; ++k) {
      const int r = rows[k];
      if (r < 0) continue;
      const float g = gs[k];
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[v] = fmaf(g, Elem<TY>::load(Y, (size_t)r * H + h0 + v), acc[v]);
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) Elem<TIO>::store(out, (size_t)t * H + h0 + v, acc[v]);
  }
}

// bf16 in and out, H % 8 == 0: 16-byte loads and stores of 8 features per thread and pass.
__device__ __forceinline__ void unpack8(const uint4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// 16 bytes that are read once: a non-temporal load (measured: combine at 4096 tokens 0.13 -> 0.10
// ms, at 8192 tokens 0.25 -> 0.21 ms)
__device__ __forceinline__ uint4 load_once(const uint16_t* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return uint4{v.x, v.y, v.z, v.w};
}

__global__ __launch_bounds__(256) void combine_bf16x8(const uint16_t* __restrict__ u,
                                                      const uint16_t* __restrict__ shared_y,
                                                      const uint16_t* __restrict__ Y,
                                                      const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ gate, int K, int H,
                                                      int total_rows, uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  __shared__ int32_t rows[MOE_MAX_TOPK];
  __shared__ float gs[MOE_MAX_TOPK];
  if ((int)threadIdx.x < K) {
    const int r = slot_row[(size_t)t * K + threadIdx.x];
    rows[threadIdx.x] = (r >= 0 && r < total_rows) ? r : -1;
    gs[threadIdx.x] = gate[(size_t)t * K + threadIdx.x];
  }
  __syncthreads();
  // blockIdx.y takes a contiguous share of the row's 8-feature chunks (several workgroups per
  // token when there are few tokens); the K routed rows' chunks are all loaded before the sums
  // so that their loads are in flight together
  const int chunks = H / 8, per = (chunks + gridDim.y - 1) / gridDim.y;
  const int c1 = min(chunks, (int)blockIdx.y * per + per);
  for (int c = blockIdx.y * per + threadIdx.x; c < c1; c += 256) {
    const int h0 = c * 8;
    uint4 yv[MOE_MAX_TOPK];
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK; ++k)
      if (k < K && rows[k] >= 0) yv[k] = load_once(Y + (size_t)rows[k] * H + h0);
    float acc[8], y[8];
    unpack8(load_once(u + (size_t)t * H + h0), acc);
    if (shared_y) {
      unpack8(load_once(shared_y + (size_t)t * H + h0), y);
#pragma unroll
      for (int v = 0; v < 8; ++v) acc[v] += y[v];
    }
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK; ++k) {
      if (k >= K || rows[k] < 0) continue;
      const float g = gs[k];
      unpack8(yv[k], y);
#pragma unroll
      for (int v = 0; v < 8; ++v) acc[v] = fmaf(g, y[v], acc[v]);
    }
    uint4 o;
    o.x = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
    o.y = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
    o.z = (uint32_t)f32_to_bf16(acc[4]) | ((uint32_t)f32_to_bf16(acc[5]) << 16);
    o.w = (uint32_t)f32_to_bf16(acc[6]) | ((uint32_t)f32_to_bf16(acc[7]) << 16);
    *reinterpret_cast<uint4*>(out + (size_t)t * H + h0) = o;
  }
}

__global__ void bias_update_kernel(const int32_t* __restrict__ counts, int N_r, long long mean_x_nr,
                                   float gamma, float* __restrict__ bias) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N_r) return;
  const long long load = (long long)N_r * counts[i];
  if (load > mean_x_nr) bias[i] = bias[i] - gamma;
  else if (load < mean_x_nr) bias[i] = bias[i] + gamma;
}

template <typename TIO, typename TY>
hipError_t combine_t(const void* u, const void* shared_y, const void* Y, const int32_t* slot_row,
                     const float* gate, int T, int K, int H, int total_rows, void* out, hipStream_t st) {
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(T), dim3(256), 0, st, static_cast<const TIO*>(u),
                       static_cast<const TY*>(shared_y), static_cast<const TY*>(Y), slot_row, gate, K,
                       H, total_rows, static_cast<TIO*>(out));
  };
  if (H % 8 == 0) go(combine_kernel<TIO, TY, 8>);
  else if (H % 4 == 0) go(combine_kernel<TIO, TY, 4>);
  else go(combine_kernel<TIO, TY, 1>);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const void* u, const void* shared_y, const void* Y, const int32_t* slot_row,
                          const float* gate, int T, int K, int H, int total_rows, int io_dtype,
                          int y_dtype, void* out, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  if (io_dtype == MOE_BF16 && y_dtype == MOE_BF16 && H % 8 == 0 && a16(u) && a16(Y) && a16(out) &&
      (shared_y == nullptr || a16(shared_y))) {
    const int split = max(1, min(8, 2048 / T));   // workgroups per token when tokens are few
    hipLaunchKernelGGL(combine_bf16x8, dim3(T, split), dim3(256), 0, st, static_cast<const uint16_t*>(u),
                       static_cast<const uint16_t*>(shared_y), static_cast<const uint16_t*>(Y), slot_row, gate,
                       K, H, total_rows, static_cast<uint16_t*>(out));
    return hipGetLastError();
  }
  if (io_dtype == MOE_BF16 && y_dtype == MOE_BF16)
    return combine_t<uint16_t, uint16_t>(u, shared_y, Y, slot_row, gate, T, K, H, total_rows, out, st);
  if (io_dtype == MOE_BF16 && y_dtype == MOE_F32)
    return combine_t<uint16_t, float>(u, shared_y, Y, slot_row, gate, T, K, H, total_rows, out, st);
  if (io_dtype == MOE_F32 && y_dtype == MOE_BF16)
    return combine_t<float, uint16_t>(u, shared_y, Y, slot_row, gate, T, K, H, total_rows, out, st);
  return combine_t<float, float>(u, shared_y, Y, slot_row, gate, T, K, H, total_rows, out, st);
}

hipError_t launch_bias_update(const int32_t* counts, int N_r, int T, int K, float gamma, float* bias,
                              hipStream_t st) {
  hipLaunchKernelGGL(bias_update_kernel, dim3((N_r + 255) / 256), dim3(256), 0, st, counts, N_r,
                     (long long)T * K, gamma, bias);
  return hipGetLastError();
}

}  // namespace moe
