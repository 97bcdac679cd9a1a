// Dispatch on one GPU: per-expert histogram, exclusive scan and stable row permutation.
//
// Every (token, choice) pair gets a row (no dropping: youleyou.com §2.2). Rows are grouped by
// expert ascending, and within an expert by token ascending. Nothing uses atomics, so the
// permutation is the same on every run:
//  1. perm_hist:    the T tokens are cut into chunks of PT tokens (16 for small batches, else
//                   64); workgroup b stages its chunk's
//                   ids in LDS and thread e counts how many equal e  -> cnt[b][e].
//                   Entries with an id outside [0, N_r) get slot_row = -1 here.
//  2. perm_scan:    one workgroup, thread e walks the chunks in order: cnt[b][e] becomes the
//                   number of e-rows before chunk b; then a block-wide exclusive scan over the
//                   experts gives offsets, and cnt[b][e] += offsets[e]. With an always-on
//                   shared expert (S rows), its identity rows [0, S) come first as group 0.
//  3. perm_scatter: workgroup b again; thread e walks its chunk in (token, k) order and hands
//                   out consecutive rows starting at cnt[b][e].
#include "common.h"

namespace moe {

namespace {

constexpr int PTHREADS = 256;

// tokens per chunk: small batches use short chunks (more workgroups, shorter serial scans)
inline int chunk_tokens(int T) { return T <= 512 ? 16 : 64; }

__global__ __launch_bounds__(PTHREADS) void perm_hist(const int32_t* __restrict__ idx, int T, int K,
                                                      int N_r, int PT, int32_t* __restrict__ cnt,
                                                      int32_t* __restrict__ slot_row) {
  extern __shared__ int4 ids4[];
  int32_t* ids = reinterpret_cast<int32_t*>(ids4);
  const int b = blockIdx.x;
  const int t0 = b * PT;
  const int n = min(PT, T - t0) * K;
  const int n4 = (n + 3) >> 2;
  for (int j = threadIdx.x; j < n4 * 4; j += PTHREADS) {
    const int v = j < n ? idx[(size_t)t0 * K + j] : -1;      // pad to a multiple of 4 with -1
    ids[j] = v;
    if (j < n && (v < 0 || v >= N_r)) slot_row[(size_t)t0 * K + j] = -1;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < N_r; e += PTHREADS) {
    int c = 0;
    for (int j = 0; j < n4; ++j) {
      const int4 v = ids4[j];
      c += (v.x == e) + (v.y == e) + (v.z == e) + (v.w == e);
    }
    cnt[(size_t)b * N_r + e] = c;
  }
}

__global__ __launch_bounds__(1024) void perm_scan(int32_t* __restrict__ cnt, int nchunks, int N_r,
                                                  int S, int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ row_token) {
  __shared__ int32_t wsum[16];
  const int e = threadIdx.x;
  int total = 0;
  if (e < N_r) {
    int b = 0;
    for (; b + 8 <= nchunks; b += 8) {          // 8 independent loads in flight, then in order
      int c[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) c[q] = cnt[(size_t)(b + q) * N_r + e];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        cnt[(size_t)(b + q) * N_r + e] = total;
        total += c[q];
      }
    }
    for (; b < nchunks; ++b) {
      const int c = cnt[(size_t)b * N_r + e];
      cnt[(size_t)b * N_r + e] = total;
      total += c;
    }
    counts[e] = total;
  }
  // exclusive scan of `total` over e (N_r <= 1024 = 16 waves of 64)
  const int lane = e & 63, w = e >> 6;
  int incl = total;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += wsum[i];
  // with an always-on shared group of S rows in front, routed expert e is group e + 1
  const int excl = S + base + incl - total;
  const int g = S > 0 ? e + 1 : e;
  if (e < N_r) {
    offsets[g] = excl;
    if (e == N_r - 1) offsets[g + 1] = excl + total;
    for (int b = 0; b < nchunks; ++b) cnt[(size_t)b * N_r + e] += excl;   // independent stores
  }
  if (S > 0) {
    if (e == 0) offsets[0] = 0;
    for (int r = e; r < S; r += 1024) row_token[r] = r;
  }
}

__global__ __launch_bounds__(PTHREADS) void perm_scatter(const int32_t* __restrict__ idx, int T, int K,
                                                         int N_r, int PT, const int32_t* __restrict__ cnt,
                                                         int32_t* __restrict__ row_token,
                                                         int32_t* __restrict__ slot_row) {
  extern __shared__ int4 ids4[];
  int32_t* ids = reinterpret_cast<int32_t*>(ids4);
  const int b = blockIdx.x;
  const int t0 = b * PT;
  const int n = min(PT, T - t0) * K;
  const int n4 = (n + 3) >> 2;
  for (int j = threadIdx.x; j < n4 * 4; j += PTHREADS) ids[j] = j < n ? idx[(size_t)t0 * K + j] : -1;
  __syncthreads();
  for (int e = threadIdx.x; e < N_r; e += PTHREADS) {
    int pos = cnt[(size_t)b * N_r + e];
    for (int j4 = 0; j4 < n4; ++j4) {
      const int4 v = ids4[j4];
      if (v.x != e && v.y != e && v.z != e && v.w != e) continue;
      const int vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (vv[q] == e) {
          const int j = j4 * 4 + q;
          row_token[pos] = t0 + j / K;
          slot_row[(size_t)t0 * K + j] = pos;
          ++pos;
        }
      }
    }
  }
}

}  // namespace

size_t permute_workspace(int T, int K, int N_r) {
  const int PT = chunk_tokens(T);
  const int nchunks = (T + PT - 1) / PT;
  return align256((size_t)nchunks * N_r * sizeof(int32_t));
}

hipError_t launch_permute(const int32_t* topk_idx, int T, int K, int N_r, int S, int32_t* counts,
                          int32_t* offsets, int32_t* row_token, int32_t* slot_row, void* ws,
                          hipStream_t st) {
  const int PT = chunk_tokens(T);
  const int nchunks = (T + PT - 1) / PT;
  int32_t* cnt = static_cast<int32_t*>(ws);
  const size_t lds = (size_t)(PT * K + 3) / 4 * 4 * sizeof(int32_t);
  if (nchunks > 0) {
    hipLaunchKernelGGL(perm_hist, dim3(nchunks), dim3(PTHREADS), lds, st, topk_idx, T, K, N_r, PT, cnt,
                       slot_row);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(perm_scan, dim3(1), dim3(1024), 0, st, cnt, nchunks, N_r, S, counts, offsets, row_token);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nchunks == 0) return e;
  hipLaunchKernelGGL(perm_scatter, dim3(nchunks), dim3(PTHREADS), lds, st, topk_idx, T, K, N_r, PT, cnt,
                     row_token, slot_row);
  return hipGetLastError();
}

}  // namespace moe
