// FP8 dispatch payload for expert parallelism: the send plan (one row per token and destination
// rank) and each row as 1x128-tile E4M3 codes + fp32 scales, and the receive-side dequantization.
//
// youleyou.com "官方揭秘DeepSeek-V3模型训练全流程" §4.3, low-precision storage and communication:
// part of the activations is quantized to FP8 for communication; §2.2 / §4.2: a token is sent to
// at most 4 nodes. Rank r owns experts [r*N_r/R, (r+1)*N_r/R); a token is sent to a rank once
// however many of its experts that rank owns. Rows are ordered by rank, then token.
//
// Pack = rank_ids (rank of each choice, -2 - k' for a repeat of choice k' on the same rank) ->
// the atomic-free dispatch kernels over R "experts" (repeats are skipped) -> repeat_slots (a
// repeat takes the row of its first choice) -> 1x128 quantization of each token once, its codes
// written to every row that carries it (a token goes to ~5 of 8 ranks at the FP8 workload's
// shape, and quantizing per row re-read and re-divided it that often).
#include "common.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void rank_ids(const int32_t* __restrict__ idx, int T, int K, int N_r,
                                                int per_rank, int32_t* __restrict__ rid) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)T * K) return;
  const int t = (int)(i / K), k = (int)(i % K);
  const int e = idx[i];
  if (e < 0 || e >= N_r) { rid[i] = -1; return; }
  const int r = e / per_rank;
  for (int kk = 0; kk < k; ++kk) {
    const int e2 = idx[(size_t)t * K + kk];
    if (e2 >= 0 && e2 < N_r && e2 / per_rank == r) { rid[i] = -2 - kk; return; }
  }
  rid[i] = r;
}

// the dispatch kernels left -1 in the slots of repeats; they take their first choice's row
__global__ __launch_bounds__(256) void repeat_slots(const int32_t* __restrict__ rid, int T, int K,
                                                    int32_t* __restrict__ slot) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)T * K) return;
  const int v = rid[i];
  if (v <= -2) slot[i] = slot[(i / K) * K + (-2 - v)];
}

// E4M3FN code -> fp32 (exact): sign, 4-bit exponent (bias 7), 3-bit mantissa; 0x7f / 0xff is NaN
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 24, ex = (c >> 3) & 15u, m = c & 7u;
  if (ex == 15u && m == 7u) return __uint_as_float(0x7fc00000u | sign);
  if (ex == 0u) {
    const float v = (float)m * 0x1p-9f;   // subnormal: m * 2^-9
    return sign ? -v : v;
  }
  return __uint_as_float(sign | ((ex + 120u) << 23) | (m << 20));
}

// one row of 128-column tiles per 16 lanes, 8 codes per lane: out = fl32(decode(code) * scale)
template <typename TO>
__global__ __launch_bounds__(256) void unpack_rows(const uint8_t* __restrict__ codes,
                                                   const float* __restrict__ scales, int rows, int cols,
                                                   TO* __restrict__ out) {
  const int tiles_per_row = cols >> 7;
  const long long tile = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (tile >= (long long)rows * tiles_per_row) return;
  const long long r = tile / tiles_per_row;
  const int c = (int)(tile % tiles_per_row) * 128 + (threadIdx.x & 15) * 8;
  const float sc = scales[tile];
  const uint2 w = *reinterpret_cast<const uint2*>(codes + r * cols + c);
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = e4m3_decode((w.x >> (8 * i)) & 0xffu) * sc;
    v[i + 4] = e4m3_decode((w.y >> (8 * i)) & 0xffu) * sc;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) Elem<TO>::store(out, r * cols + c + i, v[i]);
}

}  // namespace

// [rank ids: T*K int32][dispatch workspace over n_ranks groups]
size_t payload_workspace(int T, int K, int n_ranks) {
  return align256((size_t)T * K * sizeof(int32_t)) + permute_workspace(T, K, n_ranks);
}

hipError_t launch_pack_fp8_payload(const void* x, int x_dtype, int T, int H, const int32_t* topk_idx, int K,
                                   int N_r, int n_ranks, int32_t* counts, int32_t* offsets,
                                   int32_t* send_token, int32_t* slot_send, uint8_t* codes, float* scales,
                                   void* ws, hipStream_t st) {
  int32_t* rid = static_cast<int32_t*>(ws);
  void* pws = static_cast<char*>(ws) + align256((size_t)T * K * sizeof(int32_t));
  const long long n = (long long)T * K;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (n > 0) {
    hipLaunchKernelGGL(rank_ids, dim3(blocks), dim3(256), 0, st, topk_idx, T, K, N_r, N_r / n_ranks, rid);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch_permute(rid, T, K, n_ranks, 0, counts, offsets, send_token, slot_send, pws, st);
  if (e != hipSuccess || n == 0) return e;
  hipLaunchKernelGGL(repeat_slots, dim3(blocks), dim3(256), 0, st, rid, T, K, slot_send);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int max_rows = T * min(K, n_ranks);
  return launch_fp8_quant_rows_scatter(x, x_dtype, T, H, K, rid, slot_send, max_rows, codes, scales, st);
}

hipError_t launch_unpack_fp8_payload(const uint8_t* codes, const float* scales, int rows, int H, void* out,
                                     int out_dtype, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const long long ntiles = (long long)rows * (H / 128);
  dim3 grid((unsigned)((ntiles + 15) / 16));
  if (out_dtype == MOE_BF16)
    hipLaunchKernelGGL(unpack_rows<uint16_t>, grid, dim3(256), 0, st, codes, scales, rows, H,
                       static_cast<uint16_t*>(out));
  else
    hipLaunchKernelGGL(unpack_rows<float>, grid, dim3(256), 0, st, codes, scales, rows, H,
                       static_cast<float*>(out));
  return hipGetLastError();
}

}  // namespace moe
