// Sequence-wise balance loss value, one per sequence of seq_len consecutive tokens.
//
// The pages give only that a very small sequence-wise balance loss with alpha = 0.0001
// complements the bias rule (xyznot.com "รายงานเชิงเทคนิคของ DeepSeek-V3", Method §2, last
// sentence) to stop extreme imbalance inside one sequence ("官方揭秘DeepSeek-V3模型训练全流程" §2.2); the formula is
// not on the pages. This library computes the usual MoE balance loss within each sequence:
//   f_i = N_r / (K L) * #{t : i among the K selected},  P_i = (1/L) sum_t s_{i,t} / sum_j s_{j,t}
//   L_seq = alpha * sum_i f_i P_i
// Chunks of 64 tokens of a sequence are summed by one workgroup each (a wave per token), then one
// workgroup per sequence adds the chunk sums in order: deterministic.
#include "common.h"

namespace moe {

namespace {

constexpr int BL_CHUNK = 64;   // tokens per partial-sum workgroup

// Workgroup b = (sequence q, chunk ci) sums over its <= 64 tokens (a wave per token, tokens in
// order per wave, then the 4 waves in order): part[b][0][i] = sum_t s_{t,i} / sum_j s_{t,j} and
// part[b][1][i] = #{(t, k) : idx[t,k] = i}. Lane l holds experts l, l + 64, ... (NJ of them).
template <int NJ>
__global__ __launch_bounds__(256) void seq_balance_partial(const float* __restrict__ s, const int32_t* __restrict__ idx,
                                                           int T, int N_r, int K, int seq_len, int cps,
                                                           float* __restrict__ part) {
  __shared__ float sp[4][NJ * 64];
  __shared__ float sc[4][NJ * 64];
  const int q = blockIdx.x / cps, ci = blockIdx.x % cps;
  const int qs = q * seq_len;
  const int L = min(seq_len, T - qs);
  const int t0 = qs + ci * BL_CHUNK;
  const int n = min(BL_CHUNK, L - ci * BL_CHUNK);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float p[NJ], cn[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) p[j] = cn[j] = 0.f;
  for (int tt = wave; tt < n; tt += 4) {
    const float* row = s + (size_t)(t0 + tt) * N_r;
    float v[NJ], rs = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      v[j] = e < N_r ? row[e] : 0.f;
      rs += v[j];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) rs += __shfl_xor(rs, o);
    if (rs > 0.f) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) p[j] += v[j] / rs;
    }
    for (int k = 0; k < K; ++k) {
      const int e = idx[(size_t)(t0 + tt) * K + k];
#pragma unroll
      for (int j = 0; j < NJ; ++j) cn[j] += (e == lane + 64 * j) ? 1.f : 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    sp[wave][lane + 64 * j] = p[j];
    sc[wave][lane + 64 * j] = cn[j];
  }
  __syncthreads();
  float* out = part + (size_t)blockIdx.x * 2 * N_r;
  for (int e = threadIdx.x; e < N_r; e += 256) {
    out[e] = ((sp[0][e] + sp[1][e]) + sp[2][e]) + sp[3][e];
    out[N_r + e] = ((sc[0][e] + sc[1][e]) + sc[2][e]) + sc[3][e];
  }
}

// One workgroup per sequence: chunk partials summed in chunk order, then sum_i count_i P_i
__global__ __launch_bounds__(256) void seq_balance_final(const float* __restrict__ part, int T, int N_r, int K,
                                                         int seq_len, int cps, float alpha, float* __restrict__ loss) {
  __shared__ float red[4];
  const int q = blockIdx.x;
  const int L = min(seq_len, T - q * seq_len);
  const int nch = (L + BL_CHUNK - 1) / BL_CHUNK;
  float acc = 0.f;
  for (int e = threadIdx.x; e < N_r; e += 256) {
    float P = 0.f, C = 0.f;
    for (int c = 0; c < nch; ++c) {
      const float* pc = part + (size_t)(q * cps + c) * 2 * N_r;
      P += pc[e];
      C += pc[N_r + e];
    }
    acc = fmaf(C, P, acc);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float total = (red[0] + red[1]) + (red[2] + red[3]);
    loss[q] = alpha * ((float)N_r / ((float)K * (float)L)) * (total / (float)L);
  }
}

}  // namespace

size_t seq_balance_workspace(int T, int N_r, int seq_len) {
  if (T <= 0) return 0;
  const int nseq = (T + seq_len - 1) / seq_len;
  const int cps = (seq_len + BL_CHUNK - 1) / BL_CHUNK;
  return align256((size_t)nseq * cps * 2 * N_r * sizeof(float));
}

hipError_t launch_seq_balance_loss(const float* s, const int32_t* idx, int T, int N_r, int K, int seq_len,
                                   float alpha, float* loss, void* ws, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int nseq = (T + seq_len - 1) / seq_len;
  const int cps = (seq_len + BL_CHUNK - 1) / BL_CHUNK;
  float* part = static_cast<float*>(ws);
  const dim3 grid((unsigned)(nseq * cps));
  const int nj = (N_r + 63) / 64;
#define MOE_BAL(NJ) \
  hipLaunchKernelGGL(seq_balance_partial<NJ>, grid, dim3(256), 0, st, s, idx, T, N_r, K, seq_len, cps, part)
  if (nj <= 1) MOE_BAL(1);
  else if (nj <= 2) MOE_BAL(2);
  else if (nj <= 4) MOE_BAL(4);
  else if (nj <= 8) MOE_BAL(8);
  else MOE_BAL(16);
#undef MOE_BAL
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(seq_balance_final, dim3(nseq), dim3(256), 0, st, part, T, N_r, K, seq_len, cps, alpha, loss);
  return hipGetLastError();
}

}  // namespace moe
