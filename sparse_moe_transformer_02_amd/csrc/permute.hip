// Dispatch on one GPU: per-expert histogram, exclusive scan and stable row permutation.
//
// Every (token, choice) pair gets a row (no dropping: "官方揭秘DeepSeek-V3模型训练全流程" §2.2). Rows are grouped by
// expert ascending, and within an expert by token ascending. The permutation is the same on every
// run (the only atomics add integers in LDS, whose order cannot change a count):
//  1. perm_hist:    the T tokens are cut into chunks of PT tokens (16 for small batches, else
//                   64); workgroup b counts its chunk's ids per expert with integer adds in LDS
//                   -> cnt[b][e].
//                   Entries with an id outside [0, N_r) get slot_row = -1 here.
//  2. perm_scan:    one workgroup; 1024 / N_r threads per expert e split its walk over the
//                   chunks: cnt[b][e] becomes offsets[e] + the number of e-rows before chunk b,
//                   offsets coming from a block-wide exclusive scan of the per-expert totals.
//                   With an always-on shared expert (S rows), its identity rows [0, S) come
//                   first as group 0.
//  3. perm_scatter: workgroup b again hands out consecutive rows of each expert, starting at
//                   cnt[b][e], to its chunk's entries in (token, k) order (ranks within a wave by
//                   lane compares, per-wave counts in LDS).
// Small batches run all three steps in one workgroup instead (perm_fused), with the same result.
#include <mutex>

#include "common.h"

namespace moe {

namespace {

// Per-chunk histograms for moe_permute_noalloc: a static device array instead of a caller
// workspace, for callers that cannot allocate. Every GPU the library runs on holds its own copy
// (PERMUTE_SCRATCH_BYTES) until the process ends. perm_hist writes every entry the scan and the
// scatter read, so nothing in it has to start at zero; calls that overlap on one GPU share it
// and race.
static __device__ __align__(256) int32_t scratch[PERMUTE_SCRATCH_BYTES / sizeof(int32_t)];

constexpr int SCRATCH_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[SCRATCH_DEVICES];   // device address of `scratch` per device, once looked up

constexpr int PTHREADS = 256;

// tokens per chunk: small batches use short chunks (more workgroups, shorter serial scans)
inline int chunk_tokens(int T) { return T <= 512 ? 16 : 64; }

__global__ __launch_bounds__(PTHREADS) void perm_hist(const int32_t* __restrict__ idx, int T, int K,
                                                      int N_r, int PT, int32_t* __restrict__ cnt,
                                                      int32_t* __restrict__ slot_row) {
  __shared__ int32_t h[MOE_MAX_EXPERTS];
  const int b = blockIdx.x;
  const int t0 = b * PT;
  const int n = min(PT, T - t0) * K;
  for (int e = threadIdx.x; e < N_r; e += PTHREADS) h[e] = 0;
  __syncthreads();
  for (int j = threadIdx.x; j < n; j += PTHREADS) {
    const int v = idx[(size_t)t0 * K + j];
    if (v < 0 || v >= N_r) slot_row[(size_t)t0 * K + j] = -1;
    else atomicAdd(&h[v], 1);          // integer adds in LDS: the count does not depend on their order
  }
  __syncthreads();
  for (int e = threadIdx.x; e < N_r; e += PTHREADS) cnt[(size_t)b * N_r + e] = h[e];
}

// Q = 1024 / N_r threads share expert e's walk over the chunks: thread e + N_r q takes chunks
// [q P, q P + P), P = ceil(nchunks / Q). Pass 1 sums its chunks; the Q partial sums of e give
// each thread the rows of e before its first chunk and e's total; a block-wide scan of the totals
// gives the offsets; pass 2 writes, chunk by chunk, offsets[e] + the rows of e before it.
__global__ __launch_bounds__(1024) void perm_scan(int32_t* __restrict__ cnt, int nchunks, int N_r,
                                                  int S, int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ row_token) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t part[1024];        // part[q * N_r + e]: rows of e in thread (e, q)'s chunks
  __shared__ int32_t base_e[MOE_MAX_EXPERTS];
  const int tid = threadIdx.x;
  const int Q = 1024 / N_r;
  const int e = tid % N_r, q = tid / N_r;
  const bool walker = q < Q;
  const int P = (nchunks + Q - 1) / Q;
  const int b0 = min(nchunks, q * P), b1 = min(nchunks, b0 + P);
  int mine = 0;
  if (walker) {
    int b = b0;
    for (; b + 8 <= b1; b += 8) {               // 8 independent loads in flight
      int c[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = cnt[(size_t)(b + i) * N_r + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) mine += c[i];
    }
    for (; b < b1; ++b) mine += cnt[(size_t)b * N_r + e];
    part[tid] = mine;
  }
  __syncthreads();
  int before = 0, total = 0;                    // rows of e in chunks before b0; all rows of e
  if (walker) {
    for (int i = 0; i < Q; ++i) {
      const int v = part[i * N_r + e];
      before += i < q ? v : 0;
      total += v;
    }
  }
  // exclusive scan of the totals over the experts, on threads 0 .. N_r - 1 (q = 0)
  const int lane = tid & 63, w = tid >> 6;
  const int t_e = tid < N_r ? total : 0;
  int incl = t_e;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += wsum[i];
  if (tid < N_r) {
    // with an always-on shared group of S rows in front, routed expert e is group e + 1
    const int excl = S + base + incl - t_e;
    const int g = S > 0 ? tid + 1 : tid;
    counts[tid] = t_e;
    offsets[g] = excl;
    if (tid == N_r - 1) offsets[g + 1] = excl + t_e;
    base_e[tid] = excl;
  }
  __syncthreads();
  if (walker) {
    int run = base_e[e] + before;
    int b = b0;
    for (; b + 8 <= b1; b += 8) {
      int c[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = cnt[(size_t)(b + i) * N_r + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        cnt[(size_t)(b + i) * N_r + e] = run;
        run += c[i];
      }
    }
    for (; b < b1; ++b) {
      const int c = cnt[(size_t)b * N_r + e];
      cnt[(size_t)b * N_r + e] = run;
      run += c;
    }
  }
  if (S > 0) {
    if (tid == 0) offsets[0] = 0;
    for (int r = tid; r < S; r += 1024) row_token[r] = r;
  }
}

// Workgroup b hands out the rows of its chunk's entries in rounds of PTHREADS, entry j (token
// t0 + j / K, choice j % K) taken by thread j % PTHREADS: its row is cnt[b][e] + (rows of e in
// earlier rounds) + (rows of e in lower waves of the round) + (rows of e in lower lanes of its
// wave), i.e. the (token, k) order within the chunk that the scan's per-chunk bases assume. The
// per-wave counts go through LDS integer atomics, whose order cannot change a sum. (Walking the
// chunk once per expert instead took 24-33 us per call at 4096-16384 tokens.)
constexpr int SC_WAVES = PTHREADS / 64;
__global__ __launch_bounds__(PTHREADS) void perm_scatter(const int32_t* __restrict__ idx, int T, int K,
                                                         int N_r, int PT, const int32_t* __restrict__ cnt,
                                                         int32_t* __restrict__ row_token,
                                                         int32_t* __restrict__ slot_row) {
  __shared__ int32_t hist[SC_WAVES][MOE_MAX_EXPERTS];   // per-wave counts, then their row bases
  __shared__ int32_t run[MOE_MAX_EXPERTS];              // next free row of each expert in the chunk
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int t0 = b * PT;
  const int n = min(PT, T - t0) * K;
  for (int e = tid; e < N_r; e += PTHREADS) run[e] = cnt[(size_t)b * N_r + e];
  for (int j0 = 0; j0 < n; j0 += PTHREADS) {
    for (int i = tid; i < SC_WAVES * N_r; i += PTHREADS) hist[i / N_r][i % N_r] = 0;
    __syncthreads();
    const int j = j0 + tid;
    int v = j < n ? idx[(size_t)t0 * K + j] : -1;
    if (v < 0 || v >= N_r) v = -1;   // ids outside [0, N_r): no row (perm_hist set slot_row = -1)
    int rank = 0;                    // entries of the same expert in lower lanes of this wave
    for (int l = 0; l < 64; ++l) {
      const int u = __builtin_amdgcn_readlane(v, l);
      rank += (l < lane) & (u == v);
    }
    if (v >= 0) atomicAdd(&hist[w][v], 1);
    __syncthreads();
    for (int e = tid; e < N_r; e += PTHREADS) {   // the waves' row bases for expert e, in wave order
      int r = run[e];
      for (int q = 0; q < SC_WAVES; ++q) {
        const int c = hist[q][e];
        hist[q][e] = r;
        r += c;
      }
      run[e] = r;
    }
    __syncthreads();
    if (v >= 0) {
      const int pos = hist[w][v] + rank;
      row_token[pos] = t0 + j / K;
      slot_row[(size_t)t0 * K + j] = pos;
    }
    __syncthreads();   // every thread has read hist before the next round clears it
  }
}

// Small batches (0 < T K <= FUSED_MAX, decode) run the three steps in one workgroup of 1024
// threads with no workspace. Entry j (token j / K, choice j % K) is taken by thread j % 1024 in
// round j / 1024, each wave holding 64 consecutive entries of the round. Its row is offsets[e] +
// (rows of e in earlier rounds) + (rows of e in lower waves of the round) + (rows of e in lower
// lanes of the wave): the (token, k) order of the chunked kernels, so the result is the same. The
// counts go through LDS atomics, whose order cannot change an integer sum.
constexpr int FUSED_MAX = 4096, FUSED_WAVES = 16;
__global__ __launch_bounds__(1024) void perm_fused(const int32_t* __restrict__ idx, int T, int K, int N_r,
                                                   int S, int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ row_token,
                                                   int32_t* __restrict__ slot_row) {
  __shared__ int32_t ids[FUSED_MAX];
  __shared__ int32_t hist[FUSED_WAVES][MOE_MAX_EXPERTS];   // per-wave counts, then their row bases
  __shared__ int32_t run[MOE_MAX_EXPERTS];                 // total per expert, then its next free row
  __shared__ int32_t wsum[FUSED_WAVES];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = T * K;
  run[tid] = 0;
  for (int j = tid; j < n; j += 1024) {
    const int v = idx[j];
    const bool ok = v >= 0 && v < N_r;
    ids[j] = ok ? v : -1;
    if (!ok) slot_row[j] = -1;
  }
  __syncthreads();
  for (int j = tid; j < n; j += 1024)
    if (ids[j] >= 0) atomicAdd(&run[ids[j]], 1);
  __syncthreads();
  // exclusive scan of the totals over the experts (N_r <= 1024 = 16 waves of 64)
  const int e = tid;
  const int total = e < N_r ? run[e] : 0;
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
  if (e < N_r) {
    const int g = S > 0 ? e + 1 : e;
    counts[e] = total;
    offsets[g] = excl;
    if (e == N_r - 1) offsets[g + 1] = excl + total;
    run[e] = excl;
  }
  if (S > 0) {
    if (e == 0) offsets[0] = 0;
    for (int r = e; r < S; r += 1024) row_token[r] = r;
  }
  for (int j0 = 0; j0 < n; j0 += 1024) {
    for (int i = tid; i < FUSED_WAVES * N_r; i += 1024) hist[i / N_r][i % N_r] = 0;
    __syncthreads();
    const int j = j0 + tid;
    const int v = j < n ? ids[j] : -1;
    int rank = 0;      // entries of the same expert in lower lanes of this wave
    for (int l = 0; l < 64; ++l) {
      const int u = __builtin_amdgcn_readlane(v, l);
      rank += (l < lane) & (u == v);
    }
    if (v >= 0) atomicAdd(&hist[w][v], 1);
    __syncthreads();
    if (e < N_r) {     // the waves' row bases for expert e, in wave order
      int r = run[e];
      for (int q = 0; q < FUSED_WAVES; ++q) {
        const int c = hist[q][e];
        hist[q][e] = r;
        r += c;
      }
      run[e] = r;
    }
    __syncthreads();
    if (v >= 0) {
      const int pos = hist[w][v] + rank;
      row_token[pos] = j / K;
      slot_row[j] = pos;
    }
    __syncthreads();   // every thread has read hist before the next round clears it
  }
}

// Row gather of the dispatch: one workgroup per output row r < n = *n_rows, 16-byte copies of
// x[row_token[r]] (and of its scale row for FP8 codes); a row_token outside [0, T) gives zeros.
__global__ __launch_bounds__(256) void gather_rows(const uint4* __restrict__ x, const float* __restrict__ xs,
                                                   int T, int row_vecs, int n_sc,
                                                   const int32_t* __restrict__ row_token,
                                                   const int32_t* __restrict__ n_rows, int max_rows,
                                                   uint4* __restrict__ y, float* __restrict__ ys) {
  const int r = blockIdx.x;
  const int n = min(max(*n_rows, 0), max_rows);
  if (r >= n) return;
  const int t = row_token[r];
  const bool ok = t >= 0 && t < T;
  for (int i = threadIdx.x; i < row_vecs; i += 256)
    y[(size_t)r * row_vecs + i] = ok ? x[(size_t)t * row_vecs + i] : make_uint4(0u, 0u, 0u, 0u);
  if (ys)
    for (int i = threadIdx.x; i < n_sc; i += 256) ys[(size_t)r * n_sc + i] = ok ? xs[(size_t)t * n_sc + i] : 0.f;
}

}  // namespace

size_t permute_workspace(int T, int K, int N_r) {
  const int PT = chunk_tokens(T);
  const int nchunks = (T + PT - 1) / PT;
  return align256((size_t)nchunks * N_r * sizeof(int32_t));
}

hipError_t permute_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= SCRATCH_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    // the symbol's address on the current device; host code never passes `scratch` itself
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_permute(const int32_t* topk_idx, int T, int K, int N_r, int S, int32_t* counts,
                          int32_t* offsets, int32_t* row_token, int32_t* slot_row, void* ws,
                          hipStream_t st) {
  if (T > 0 && (long long)T * K <= FUSED_MAX) {
    hipLaunchKernelGGL(perm_fused, dim3(1), dim3(1024), 0, st, topk_idx, T, K, N_r, S, counts, offsets, row_token,
                       slot_row);
    return hipGetLastError();
  }
  const int PT = chunk_tokens(T);
  const int nchunks = (T + PT - 1) / PT;
  int32_t* cnt = static_cast<int32_t*>(ws);
  if (nchunks > 0) {
    hipLaunchKernelGGL(perm_hist, dim3(nchunks), dim3(PTHREADS), 0, st, topk_idx, T, K, N_r, PT, cnt,
                       slot_row);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(perm_scan, dim3(1), dim3(1024), 0, st, cnt, nchunks, N_r, S, counts, offsets, row_token);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nchunks == 0) return e;
  hipLaunchKernelGGL(perm_scatter, dim3(nchunks), dim3(PTHREADS), 0, st, topk_idx, T, K, N_r, PT, cnt,
                     row_token, slot_row);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const float* x_scales, int T, int row_bytes, int n_sc,
                              const int32_t* row_token, const int32_t* n_rows, int max_rows, void* x_perm,
                              float* x_perm_scales, hipStream_t st) {
  if (max_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows, dim3(max_rows), dim3(256), 0, st, static_cast<const uint4*>(x), x_scales, T,
                     row_bytes / 16, n_sc, row_token, n_rows, max_rows, static_cast<uint4*>(x_perm), x_perm_scales);
  return hipGetLastError();
}

}  // namespace moe
