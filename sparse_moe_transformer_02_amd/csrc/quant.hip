// Online-absmax E4M3FN quantization with one fp32 scale per 1x128 tile or 128x128 block.
//
// youleyou.com "官方揭秘DeepSeek-V3模型训练全流程" §4.3 and the "รายงานเชิงเทคนิคของ DeepSeek-V3" key-ideas FP8 bullet:
// activations get one scale per 1x128 tile, weights one per 128x128 block, from the current
// max |x|. scale = fl32(amax / 448); code = E4M3FN(fl32(x / scale)) rounded to nearest even and
// saturated at 448 (the largest finite E4M3FN value); zero tiles get scale 0.
#include "common.h"
#include "fp8.h"

namespace moe {

namespace {

template <typename TX> struct Load8;
template <> struct Load8<float> {
  __device__ __forceinline__ static void run(const float* p, float* v) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};
template <> struct Load8<uint16_t> {
  __device__ __forceinline__ static void run(const uint16_t* p, float* v) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

__device__ __forceinline__ uint2 encode8(const float* v, float scale) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= (uint32_t)e4m3_encode(scale == 0.f ? v[i] : v[i] / scale) << (8 * i);
    hi |= (uint32_t)e4m3_encode(scale == 0.f ? v[i + 4] : v[i + 4] / scale) << (8 * i);
  }
  return make_uint2(lo, hi);
}

// 1x128 tiles: 16 lanes per tile, 8 values per lane; a 256-thread block covers 16 tiles.
// Output row r quantizes input row row_index[r] (r itself if row_index is NULL); with n_live
// non-NULL only rows r < *n_live are written (a row count known on the device only). Gathered
// rows outside [0, x_rows) are skipped.
template <typename TX>
__global__ __launch_bounds__(256) void quant_rows(const TX* __restrict__ x, int x_rows, int rows, int cols,
                                                  const int32_t* __restrict__ row_index,
                                                  const int32_t* __restrict__ n_live,
                                                  uint8_t* __restrict__ codes,
                                                  float* __restrict__ scales) {
  const int tiles_per_row = cols >> 7;
  const long long tile = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int live_rows = n_live ? min(rows, max(*n_live, 0)) : rows;
  const long long ntiles = (long long)live_rows * tiles_per_row;
  const int sub = threadIdx.x & 15;
  const long long r = tile < ntiles ? tile / tiles_per_row : 0;
  const long long src = row_index ? (long long)row_index[r] : r;
  const bool live = tile < ntiles && src >= 0 && src < x_rows;   // uniform over the tile's 16 lanes
  const int c = live ? (int)(tile % tiles_per_row) * 128 + sub * 8 : 0;
  float v[8];
  if (live) Load8<TX>::run(x + src * cols + c, v);
  else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
  const float scale = amax / 448.0f;
  if (!live) return;
  *reinterpret_cast<uint2*>(codes + r * cols + c) = encode8(v, scale);
  if (sub == 0) scales[tile] = scale;
}

// The 1x128 tiles of each row t of x, quantized once as quant_rows does and written to every
// output row that carries token t: row slot[t*K + k] for each choice k with owner[t*K + k] >= 0
// (choices with owner < 0 share another choice's row or have none). Output rows outside
// [0, max_rows) are skipped.
template <typename TX>
__global__ __launch_bounds__(256) void quant_rows_scatter(const TX* __restrict__ x, int T, int cols, int K,
                                                          const int32_t* __restrict__ owner,
                                                          const int32_t* __restrict__ slot, int max_rows,
                                                          uint8_t* __restrict__ codes,
                                                          float* __restrict__ scales) {
  const int tiles_per_row = cols >> 7;
  const long long tile = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool live = tile < (long long)T * tiles_per_row;   // uniform over the tile's 16 lanes
  const int sub = threadIdx.x & 15;
  const long long t = live ? tile / tiles_per_row : 0;
  const int j = live ? (int)(tile % tiles_per_row) : 0;
  const int c = j * 128 + sub * 8;
  float v[8];
  if (live) Load8<TX>::run(x + t * cols + c, v);
  else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
  const float scale = amax / 448.0f;
  if (!live) return;
  const uint2 code = encode8(v, scale);
  for (int k = 0; k < K; ++k) {
    if (owner[t * K + k] < 0) continue;
    const int row = slot[t * K + k];
    if (row < 0 || row >= max_rows) continue;
    *reinterpret_cast<uint2*>(codes + (size_t)row * cols + c) = code;
    if (sub == 0) scales[(size_t)row * tiles_per_row + j] = scale;
  }
}

// 128x128 blocks: one 256-thread workgroup per block; thread (i) handles columns (i%16)*8..+8
// of rows i/16 + 16*j. Two passes over the block: max |x|, then encode.
template <typename TX>
__global__ __launch_bounds__(256) void quant_blocks(const TX* __restrict__ x, int rows, int cols,
                                                    uint8_t* __restrict__ codes,
                                                    float* __restrict__ scales) {
  __shared__ float red[4];
  const int bc = blockIdx.x, br = blockIdx.y;
  const int cc = bc * 128 + (threadIdx.x & 15) * 8;
  const size_t r0 = (size_t)br * 128 + (threadIdx.x >> 4);
  float amax = 0.f;
  for (int j = 0; j < 8; ++j) {
    float v[8];
    Load8<TX>::run(x + (r0 + 16 * j) * cols + cc, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float scale = amax / 448.0f;
  for (int j = 0; j < 8; ++j) {
    float v[8];
    Load8<TX>::run(x + (r0 + 16 * j) * cols + cc, v);
    *reinterpret_cast<uint2*>(codes + (r0 + 16 * j) * cols + cc) = encode8(v, scale);
  }
  if (threadIdx.x == 0) scales[(size_t)br * (cols >> 7) + bc] = scale;
}

}  // namespace

hipError_t launch_fp8_quant(const void* x, int x_dtype, int rows, int cols, int tile_rows,
                            uint8_t* codes, float* scales, hipStream_t st) {
  if (rows == 0 || cols == 0) return hipSuccess;
  if (tile_rows == 1) {
    const long long ntiles = (long long)rows * (cols / 128);
    dim3 grid((unsigned)((ntiles + 15) / 16));
    if (x_dtype == MOE_BF16)
      hipLaunchKernelGGL(quant_rows<uint16_t>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(x),
                         rows, rows, cols, nullptr, nullptr, codes, scales);
    else
      hipLaunchKernelGGL(quant_rows<float>, grid, dim3(256), 0, st, static_cast<const float*>(x), rows, rows,
                         cols, nullptr, nullptr, codes, scales);
  } else {
    dim3 grid(cols / 128, rows / 128);
    if (x_dtype == MOE_BF16)
      hipLaunchKernelGGL(quant_blocks<uint16_t>, grid, dim3(256), 0, st,
                         static_cast<const uint16_t*>(x), rows, cols, codes, scales);
    else
      hipLaunchKernelGGL(quant_blocks<float>, grid, dim3(256), 0, st, static_cast<const float*>(x),
                         rows, cols, codes, scales);
  }
  return hipGetLastError();
}

hipError_t launch_fp8_quant_rows_gather(const void* x, int x_dtype, int x_rows, int rows, int cols,
                                        const int32_t* row_index, const int32_t* n_live, uint8_t* codes,
                                        float* scales, hipStream_t st) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const long long ntiles = (long long)rows * (cols / 128);
  dim3 grid((unsigned)((ntiles + 15) / 16));
  if (x_dtype == MOE_BF16)
    hipLaunchKernelGGL(quant_rows<uint16_t>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(x), x_rows,
                       rows, cols, row_index, n_live, codes, scales);
  else
    hipLaunchKernelGGL(quant_rows<float>, grid, dim3(256), 0, st, static_cast<const float*>(x), x_rows, rows,
                       cols, row_index, n_live, codes, scales);
  return hipGetLastError();
}

hipError_t launch_fp8_quant_rows_scatter(const void* x, int x_dtype, int T, int cols, int K,
                                         const int32_t* owner, const int32_t* slot, int max_rows,
                                         uint8_t* codes, float* scales, hipStream_t st) {
  if (T == 0 || cols == 0) return hipSuccess;
  const long long ntiles = (long long)T * (cols / 128);
  dim3 grid((unsigned)((ntiles + 15) / 16));
  if (x_dtype == MOE_BF16)
    hipLaunchKernelGGL(quant_rows_scatter<uint16_t>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(x), T,
                       cols, K, owner, slot, max_rows, codes, scales);
  else
    hipLaunchKernelGGL(quant_rows_scatter<float>, grid, dim3(256), 0, st, static_cast<const float*>(x), T, cols,
                       K, owner, slot, max_rows, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
