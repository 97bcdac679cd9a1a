// Router: token-to-expert affinity, biased top-K selection, gate normalisation.
//
// xyznot.com "รายงานเชิงเทคนิคของ DeepSeek-V3", Method §2: s_{i,t} = Sigmoid(u_t . e_i);
// g'_{i,t} = s_{i,t} when s_{i,t}+b_i is among the top K_r of {s_{j,t}+b_j}; g = g' normalised.
// "Deepseek V3 国货之光 开源之光", Auxiliary-Loss-Free Load Balancing section: b only selects; the unbiased s feeds the gates.
//
// Kernels:
//  1. the [T, N_r] logit GEMM (K-contiguous u rows times K-contiguous centroid rows), with the
//     reduction dimension H split over `splits` workgroups when T is small (partial sums land
//     in the workspace):
//     - bf16 u (H % 32 == 0): on MFMA. Each fp32 centroid value is split exactly into three bf16
//       parts, e = hi + mid + lo with hi = RNE(e), mid = RNE(e - hi), lo = e - hi - mid (8 + 8 + 8
//       significand bits), so u.e = u.hi + u.mid + u.lo with exact products and fp32
//       accumulation (below 1024 tokens route_logits_mfma_f32c, fragments straight from memory
//       and the centroids split in registers; for T >= 1024 and H % 64 == 0 route_split_centroids,
//       then route_logits_lds, tiles staged through LDS; centroids without 16-byte alignment
//       route_split_centroids, then route_logits_mfma);
//     - otherwise fp32 FMA with 64x64 output tiles staged through LDS (route_logits).
//  2. route_select: one 64-lane wave per token. Adds the partial sums in a fixed order (so the
//     result is deterministic), applies the sigmoid, forms key = s + b and extracts the K best
//     (key desc, index asc) with K rounds of a wave-wide argmax over cross-lane shuffles.
#include "common.h"
#include "kloop.h"
#include "lds.h"

namespace moe {

namespace {

constexpr int RT_TILE = 64;   // tokens and experts per logits tile
constexpr int RT_KC = 16;     // reduction depth per LDS stage

template <typename TU>
__global__ __launch_bounds__(256) void route_logits(const TU* __restrict__ u,
                                                    const float* __restrict__ E, int T, int H,
                                                    int N_r, int kchunk, float* __restrict__ part) {
  __shared__ float As[RT_KC][RT_TILE + 4];   // u tile, [k][token]
  __shared__ float Bs[RT_KC][RT_TILE + 4];   // centroid tile, [k][expert]
  const int tid = threadIdx.x;
  const int i0 = blockIdx.x * RT_TILE;
  const int t0 = blockIdx.y * RT_TILE;
  const int kb = blockIdx.z * kchunk;
  const int ke = min(H, kb + kchunk);
  const int tx = tid & 15, ty = tid >> 4;
  const int lr = tid >> 2, lc = (tid & 3) * 4;
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;

  for (int k0 = kb; k0 < ke; k0 += RT_KC) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = k0 + lc + j;
      const bool kin = kk < ke;
      As[lc + j][lr] = (kin && t0 + lr < T) ? Elem<TU>::load(u, (size_t)(t0 + lr) * H + kk) : 0.f;
      Bs[lc + j][lr] = (kin && i0 + lr < N_r) ? E[(size_t)(i0 + lr) * H + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < RT_KC; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) { a[j] = As[kk][ty * 4 + j]; b[j] = Bs[kk][tx * 4 + j]; }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(a[x], b[y], acc[x][y]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int t = t0 + ty * 4 + x;
    if (t >= T) continue;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int i = i0 + tx * 4 + y;
      if (i < N_r) part[((size_t)blockIdx.z * T + t) * N_r + i] = acc[x][y];
    }
  }
}

// parts[p][i] for p = 0, 1, 2: the three bf16 parts of centroids[i] (exact: e = hi + mid + lo)
__global__ __launch_bounds__(256) void route_split_centroids(const float* __restrict__ E, long long n,
                                                             uint16_t* __restrict__ parts) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float e = E[i];
  const uint16_t hi = f32_to_bf16(e);
  const float r1 = e - bf16_to_f32(hi);
  const uint16_t mid = f32_to_bf16(r1);
  const float r2 = r1 - bf16_to_f32(mid);
  parts[i] = hi;
  parts[n + i] = mid;
  parts[2 * n + i] = f32_to_bf16(r2);
}

// Workgroup (4 waves, 2 x 2) = 64 tokens x 64 experts x one K chunk; a wave computes 32 tokens x
// 32 experts with separate accumulators for the hi, mid and lo parts, summed as (hi + mid) + lo.
constexpr int RM_TILE = 64;
__global__ __launch_bounds__(256) void route_logits_mfma(const uint16_t* __restrict__ u,
                                                         const uint16_t* __restrict__ parts, int T,
                                                         int H, int N_r, int kchunk,
                                                         float* __restrict__ part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, kq = (lane >> 4) * 8;
  const int t0 = blockIdx.y * RM_TILE + (wave >> 1) * 32;
  const int e0 = blockIdx.x * RM_TILE + (wave & 1) * 32;
  const int kb = blockIdx.z * kchunk;
  const int klen = min(H, kb + kchunk) - kb;
  const size_t n = (size_t)N_r * H;
  const uint16_t* pa[2];
  bool va[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int t = t0 + m * 16 + l16;
    va[m] = t < T;
    pa[m] = u + (size_t)(va[m] ? t : 0) * H + kb + kq;
  }
  const uint16_t* pb[6];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int e = min(e0 + f * 16 + l16, N_r - 1);
#pragma unroll
    for (int q = 0; q < 3; ++q) pb[f * 3 + q] = parts + q * n + (size_t)e * H + kb + kq;
  }
  f32x4 acc[2][6];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int j = 0; j < 6; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  kloop_bf16<2, 6, 2>(pa, va, pb, klen, acc);
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + m * 16 + (lane >> 4) * 4 + i;
      if (t >= T) continue;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int e = e0 + f * 16 + l16;
        if (e < N_r)
          part[((size_t)blockIdx.z * T + t) * N_r + e] = (acc[m][f * 3][i] + acc[m][f * 3 + 1][i]) + acc[m][f * 3 + 2][i];
      }
    }
}

// route_logits_mfma with the fp32 centroids read directly and split into their three bf16 parts
// in registers (hi = RNE(e), mid = RNE(e - hi), lo = RNE(e - hi - mid), the conversions by
// v_cvt_pk_bf16_f32: the same parts route_split_centroids writes), so small batches need neither
// the split kernel nor its 6 bytes per centroid value of traffic. Fragments, their order and the
// MFMA sequence of every accumulator are those of route_logits_mfma: the partial sums are the same.
// Blocks of RU 32-deep steps are double-buffered in registers as in kloop_bf16.
__device__ __forceinline__ void split_parts8(const float4& x0, const float4& x1, bf16x8& hi, bf16x8& mid,
                                             bf16x8& lo) {
  const float e[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h = (__bf16)e[i];
    const float r1 = e[i] - (float)h;      // exact
    const __bf16 m = (__bf16)r1;
    const float r2 = r1 - (float)m;        // exact
    hi[i] = h;
    mid[i] = m;
    lo[i] = (__bf16)r2;
  }
}

constexpr int RU = 2;
__global__ __launch_bounds__(256) void route_logits_mfma_f32c(const uint16_t* __restrict__ u,
                                                              const float* __restrict__ E, int T, int H,
                                                              int N_r, int kchunk, float* __restrict__ part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, kq = (lane >> 4) * 8;
  const int t0 = blockIdx.y * RM_TILE + (wave >> 1) * 32;
  const int e0 = blockIdx.x * RM_TILE + (wave & 1) * 32;
  const int kb = blockIdx.z * kchunk;
  const int klen = min(H, kb + kchunk) - kb;
  const uint16_t* pa[2];
  uint32_t msk[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int t = t0 + m * 16 + l16;
    msk[m] = t < T ? 0xffffffffu : 0u;
    pa[m] = u + (size_t)(t < T ? t : 0) * H + kb + kq;
  }
  const float* pe[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) pe[f] = E + (size_t)min(e0 + f * 16 + l16, N_r - 1) * H + kb + kq;
  f32x4 acc[2][6];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int j = 0; j < 6; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  struct Blk {
    float4 e[RU][2][2];
    bf16x8 a[RU][2];
  };
  auto load = [&](int k0, Blk& b) {
#pragma unroll
    for (int s = 0; s < RU; ++s) {
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        b.e[s][f][0] = *reinterpret_cast<const float4*>(pe[f] + k0 + 32 * s);
        b.e[s][f][1] = *reinterpret_cast<const float4*>(pe[f] + k0 + 32 * s + 4);
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) b.a[s][m] = ld_bf16x8(pa[m] + k0 + 32 * s);
    }
  };
  auto step = [&](const float4 (&e)[2][2], const bf16x8 (&a)[2]) {
    bf16x8 bp[6];
#pragma unroll
    for (int f = 0; f < 2; ++f) split_parts8(e[f][0], e[f][1], bp[f * 3], bp[f * 3 + 1], bp[f * 3 + 2]);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const bf16x8 am = mask_bf16x8(a[m], msk[m]);
#pragma unroll
      for (int j = 0; j < 6; ++j) acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, bp[j], acc[m][j], 0, 0, 0);
    }
  };
  auto mma = [&](const Blk& b) {
#pragma unroll
    for (int s = 0; s < RU; ++s) step(b.e[s], b.a[s]);
  };
  const int nblk = klen / (32 * RU);
  if (nblk > 0) {
    Blk b0, b1;
    load(0, b0);
    for (int blk = 0; blk < nblk; blk += 2) {
      load(min(blk + 1, nblk - 1) * 32 * RU, b1);
      mma(b0);
      if (blk + 1 >= nblk) break;
      load(min(blk + 2, nblk - 1) * 32 * RU, b0);
      mma(b1);
    }
  }
  for (int k0 = nblk * 32 * RU; k0 < klen; k0 += 32) {
    float4 e[2][2];
    bf16x8 a[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      e[f][0] = *reinterpret_cast<const float4*>(pe[f] + k0);
      e[f][1] = *reinterpret_cast<const float4*>(pe[f] + k0 + 4);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) a[m] = ld_bf16x8(pa[m] + k0);
    step(e, a);
  }
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + m * 16 + (lane >> 4) * 4 + i;
      if (t >= T) continue;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int e = e0 + f * 16 + l16;
        if (e < N_r)
          part[((size_t)blockIdx.z * T + t) * N_r + e] = (acc[m][f * 3][i] + acc[m][f * 3 + 1][i]) + acc[m][f * 3 + 2][i];
      }
    }
}

// LDS-tiled form of the same GEMM for large T: workgroup = 256 tokens x 64 experts x one K chunk,
// 8 waves (4 along tokens x 2 along experts). The B tile's 192 rows are the hi, mid and lo
// parts of the 64 experts (row p * 64 + e); a wave holds 64 tokens x 32 experts x 3 parts (4 x 6
// fragments) and writes (hi + mid) + lo. 64-deep K stages go through two LDS buffers (112 KB)
// by direct global->LDS loads, chunk c of row r in slot c ^ (r % 8).
constexpr int RL_T = 256, RL_E = 64, RL_RB = 128;
constexpr int RL_TA = RL_T * RL_RB, RL_TB = 3 * RL_E * RL_RB;
__global__ __launch_bounds__(512) void route_logits_lds(const uint16_t* __restrict__ u,
                                                        const uint16_t* __restrict__ parts, int T, int H,
                                                        int N_r, int kchunk, float* __restrict__ part) {
  __shared__ __align__(16) uint8_t sA0[RL_TA];
  __shared__ __align__(16) uint8_t sB0[RL_TB];
  __shared__ __align__(16) uint8_t sA1[RL_TA];
  __shared__ __align__(16) uint8_t sB1[RL_TB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e0 = blockIdx.x * RL_E, t0 = blockIdx.y * RL_T;
  const int kb = blockIdx.z * kchunk;
  const int nk = (min(H, kb + kchunk) - kb) / 64;
  const size_t n = (size_t)N_r * H;
  // wave w loads A rows [32w, 32w + 32) (4 x 8 rows) and B rows [24w, 24w + 24) (3 x 8 rows)
  const uint16_t* asrc[4];
  const uint16_t* bsrc[3];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = wave * 32 + j * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz_ch<8>(row);
    asrc[j] = u + (size_t)min(t0 + row, T - 1) * H + kb + c * 8;
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int row = wave * 24 + j * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz_ch<8>(row);
    const int pp = row / RL_E, e = min(e0 + row % RL_E, N_r - 1);
    bsrc[j] = parts + pp * n + (size_t)e * H + kb + c * 8;
  }
  auto stage = [&](int ks, uint8_t* sa, uint8_t* sb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(asrc[j] + ks * 64, sa + (wave * 32 + j * 8) * RL_RB);
#pragma unroll
    for (int j = 0; j < 3; ++j) dma16(bsrc[j] + ks * 64, sb + (wave * 24 + j * 8) * RL_RB);
  };
  const int wm = wave & 3, wn = wave >> 2;
  f32x4 acc[4][6];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int j = 0; j < 6; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const uint8_t* sa, const uint8_t* sb) {
#pragma unroll 1
    for (int kk = 0; kk < 2; ++kk) {
      const int c = kk * 4 + (lane >> 4);
      bf16x8 a[4], b[6];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int row = wm * 64 + m * 16 + (lane & 15);
        a[m] = *reinterpret_cast<const bf16x8*>(sa + row * RL_RB + (c ^ swz_ch<8>(row)) * 16);
      }
#pragma unroll
      for (int j = 0; j < 6; ++j) {   // j = part * 2 + fragment
        const int row = (j >> 1) * RL_E + wn * 32 + (j & 1) * 16 + (lane & 15);
        b[j] = *reinterpret_cast<const bf16x8*>(sb + row * RL_RB + (c ^ swz_ch<8>(row)) * 16);
      }
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int j = 0; j < 6; ++j) acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], b[j], acc[m][j], 0, 0, 0);
    }
  };
  if (nk > 0) {
    stage(0, sA0, sB0);
    for (int ks = 0; ks < nk; ks += 2) {
      wait_dma_keep_barrier<0>();
      if (ks + 1 < nk) stage(ks + 1, sA1, sB1);
      compute(sA0, sB0);
      if (ks + 1 >= nk) break;
      wait_dma_keep_barrier<0>();
      if (ks + 2 < nk) stage(ks + 2, sA0, sB0);
      compute(sA1, sB1);
    }
  }
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + wm * 64 + m * 16 + (lane >> 4) * 4 + i;
      if (t >= T) continue;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int e = e0 + wn * 32 + f * 16 + (lane & 15);
        if (e < N_r)
          part[((size_t)blockIdx.z * T + t) * N_r + e] = (acc[m][f][i] + acc[m][2 + f][i]) + acc[m][4 + f][i];
      }
    }
}

// a ranks before b: larger key, or equal key and smaller expert index
__device__ __forceinline__ bool ranks_before(float ka, int ea, float kb, int eb) {
  return ka > kb || (ka == kb && ea < eb);
}

// Group-limited selection (n_groups > 1): the experts form n_groups equal contiguous groups and a
// token's K experts come from at most topk_groups of them (node-limited routing, "DeepSeek：AI 領域的重大突破與開源策略"
// "DeepSeek：AI 領域的重大突破與開源策略" innovation table; "官方揭秘DeepSeek-V3模型训练全流程" §2.2: at most 4 nodes).
// How groups are chosen is not on the pages; this library scores a group by the fp32 sum of its
// K / topk_groups best keys, added best first, keeps the topk_groups best groups (equal scores:
// lower group index) and takes the Top-K over their experts only.
// Lane g < n_groups scores group g from the wave's keys staged in LDS; the kept groups come from
// topk_groups rounds of a wave-wide argmax; other groups' keys become -inf before the Top-K.
__device__ __forceinline__ uint64_t kept_groups(const float* __restrict__ kb, int lane, int N_r, int K,
                                               int n_groups, int topk_groups) {
  const int gsz = N_r / n_groups, per = K / topk_groups;
  float score = -INFINITY;
  if (lane < n_groups) {
    const float* gk = kb + lane * gsz;
    float pk = INFINITY;   // the previous pick; the next one ranks strictly after it
    int pe = -1;
    for (int r = 0; r < per; ++r) {
      float bk = -INFINITY;
      int be = 0x7fffffff;
      for (int i = 0; i < gsz; ++i) {
        const float v = gk[i];
        if (ranks_before(pk, pe, v, i) && ranks_before(v, i, bk, be)) { bk = v; be = i; }
      }
      score = r == 0 ? bk : score + bk;   // fp32, best key first
      pk = bk;
      pe = be;
    }
  }
  uint64_t keep = 0;
  bool taken = false;
  for (int m = 0; m < topk_groups; ++m) {
    const bool cand = lane < n_groups && !taken;
    float bs = cand ? score : -INFINITY;
    int bg = cand ? lane : 0x7fffffff;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float os = __shfl_xor(bs, off);
      const int og = __shfl_xor(bg, off);
      if (ranks_before(os, og, bs, bg)) { bs = os; bg = og; }
    }
    if (lane == bg) taken = true;
    if (bg < 64) keep |= 1ull << bg;
  }
  return keep;
}

template <int NJ, bool BATCH>
__global__ __launch_bounds__(256) void route_select(const float* __restrict__ part, int splits,
                                                    const float* __restrict__ logit_offset,
                                                    const float* __restrict__ affinity_in,
                                                    const float* __restrict__ bias, int T, int N_r,
                                                    int K, int n_groups, int topk_groups,
                                                    float* __restrict__ affinity_out,
                                                    int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_gate) {
  __shared__ float kbuf[4][MOE_MAX_EXPERTS];   // one token's keys per wave (group-limited only)
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float key[NJ], s[NJ];
  // logits: the split partials added in order z = 0, 1, ... for each expert. BATCH (many splits,
  // few tokens): the loads of all NJ experts of a batch of 8 splits are issued together (a lane past
  // the last expert reads the last expert's partials, unused); otherwise expert by expert, which
  // needs fewer registers (more waves per SIMD when the tokens are many)
  float logit[NJ];
  if (BATCH && !affinity_in) {
    const size_t zs = (size_t)T * N_r;
    const float* pz[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      logit[j] = 0.f;
      pz[j] = part + (size_t)t * N_r + min(lane + 64 * j, N_r - 1);
    }
    int z = 0;
    for (; z + 8 <= splits; z += 8) {
      float v[NJ][8];
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 8; ++q) v[j][q] = pz[j][(z + q) * zs];
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 8; ++q) logit[j] += v[j][q];
    }
    for (; z < splits; ++z) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) logit[j] += pz[j][z * zs];
    }
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    key[j] = -INFINITY;
    s[j] = 0.f;
    if (e < N_r) {
      float sv;
      if (affinity_in) {
        sv = affinity_in[(size_t)t * N_r + e];
      } else {
        float lg = 0.f;
        if (BATCH) {
          lg = logit[j];
        } else {
          const float* pz = part + (size_t)t * N_r + e;
          const size_t zs = (size_t)T * N_r;
          int z = 0;
          for (; z + 8 <= splits; z += 8) {
            float v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = pz[(z + q) * zs];
#pragma unroll
            for (int q = 0; q < 8; ++q) lg += v[q];
          }
          for (; z < splits; ++z) lg += pz[z * zs];
        }
        if (logit_offset) lg += logit_offset[e];
        sv = 1.0f / (1.0f + __expf(-lg));
      }
      if (affinity_out) affinity_out[(size_t)t * N_r + e] = sv;
      s[j] = sv;
      key[j] = sv + bias[e];
    }
  }
  if (n_groups > 1) {
    float* kb = kbuf[threadIdx.x >> 6];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      if (e < N_r) kb[e] = key[j];
    }
    // the wave's own LDS writes are complete and visible to all its lanes before the reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint64_t keep = kept_groups(kb, lane, N_r, K, n_groups, topk_groups);
    const int gsz = N_r / n_groups;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      if (e < N_r && !((keep >> (e / gsz)) & 1ull)) key[j] = -INFINITY;
    }
  }
  uint32_t taken = 0;
  int sel_e = 0;
  float sel_s = 0.f, ssum = 0.f;
  for (int k = 0; k < K; ++k) {
    float bk = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      if (e < N_r && !((taken >> j) & 1u) && ranks_before(key[j], e, bk, be)) { bk = key[j]; be = e; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ok = __shfl_xor(bk, off);
      const int oe = __shfl_xor(be, off);
      if (ranks_before(ok, oe, bk, be)) { bk = ok; be = oe; }
    }
    // every lane now holds the winner; its owner marks it taken and shares s
    const int jw = be >> 6, lw = be & 63;
    float sw = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (j == jw) sw = s[j];
    sw = __shfl(sw, lw);
    if (lane == lw) taken |= 1u << jw;
    ssum += sw;                       // k ascending: fixed summation order
    if (lane == k) { sel_e = be; sel_s = sw; }
  }
  if (lane < K) {
    topk_idx[(size_t)t * K + lane] = sel_e;
    topk_gate[(size_t)t * K + lane] = sel_s / ssum;
  }
}

// The LDS-tiled logits kernel serves bf16 u with H % 64 == 0 from this many tokens on
constexpr int RL_MIN_T = 1024;

bool use_lds_logits(int T, int H) { return T >= RL_MIN_T && H % 64 == 0; }

// K splits of the LDS-tiled kernel: about 512 workgroups, at least 512 of H per split
int route_splits_lds(int T, int H, int N_r) {
  const int tiles = ((T + RL_T - 1) / RL_T) * ((N_r + RL_E - 1) / RL_E);
  int splits = (512 + tiles - 1) / tiles;
  splits = max(1, min(splits, H / 512));
  const int kc = ((H + splits - 1) / splits + 63) / 64 * 64;
  return (H + kc - 1) / kc;
}

int route_splits(int T, int H, int N_r) {
  const int tiles = ((T + RT_TILE - 1) / RT_TILE) * ((N_r + RT_TILE - 1) / RT_TILE);
  int splits = (1024 + tiles - 1) / tiles;
  const int max_splits = (H + 255) / 256;          // keep at least 256 of H per split
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  return splits;
}

}  // namespace

// [partials: splits x T x N_r fp32][centroid parts: 3 x N_r x H bf16 (MFMA path only)]
static int max_splits(int T, int H, int N_r) {
  const int s = route_splits(T, H, N_r);
  return use_lds_logits(T, H) ? max(s, route_splits_lds(T, H, N_r)) : s;
}

size_t route_workspace(int T, int H, int N_r) {
  if (T <= 0) return 0;
  return align256((size_t)max_splits(T, H, N_r) * T * N_r * sizeof(float)) +
         ((H % 32 == 0) ? align256((size_t)3 * N_r * H * sizeof(uint16_t)) : 0);
}

hipError_t launch_route(const void* u, int u_dtype, const float* centroids, const float* bias,
                        const float* logit_offset, const float* affinity_in, int T, int H, int N_r,
                        int K, int n_groups, int topk_groups, float* affinity_out, int32_t* topk_idx,
                        float* topk_gate, void* ws, hipStream_t st) {
  if (T == 0) return hipSuccess;
  float* part = static_cast<float*>(ws);
  int splits = 0;
  if (!affinity_in) {
    splits = route_splits(T, H, N_r);
    int kchunk = (H + splits - 1) / splits;
    kchunk = (kchunk + RT_KC - 1) / RT_KC * RT_KC;
    splits = (H + kchunk - 1) / kchunk;
    dim3 grid((N_r + RT_TILE - 1) / RT_TILE, (T + RT_TILE - 1) / RT_TILE, splits);
    if (u_dtype == MOE_BF16 && H % 32 == 0 && ((uintptr_t)u & 15) == 0 && !use_lds_logits(T, H) &&
        ((uintptr_t)centroids & 15) == 0) {
      // small batches: the centroids split into bf16 parts inside the logits kernel
      int kc = (H + splits - 1) / splits;            // K chunks in whole 32-deep MFMA steps
      kc = (kc + 31) / 32 * 32;
      const int sp = (H + kc - 1) / kc;
      hipLaunchKernelGGL(route_logits_mfma_f32c, dim3((N_r + RM_TILE - 1) / RM_TILE, (T + RM_TILE - 1) / RM_TILE, sp),
                         dim3(256), 0, st, static_cast<const uint16_t*>(u), centroids, T, H, N_r, kc, part);
      splits = sp;
    } else if (u_dtype == MOE_BF16 && H % 32 == 0 && ((uintptr_t)u & 15) == 0) {
      uint16_t* parts = reinterpret_cast<uint16_t*>(
          static_cast<char*>(ws) + align256((size_t)max_splits(T, H, N_r) * T * N_r * sizeof(float)));
      const long long n = (long long)N_r * H;
      hipLaunchKernelGGL(route_split_centroids, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, centroids,
                         n, parts);
      if (use_lds_logits(T, H)) {
        const int sp = route_splits_lds(T, H, N_r);
        const int kc = ((H + sp - 1) / sp + 63) / 64 * 64;
        hipLaunchKernelGGL(route_logits_lds, dim3((N_r + RL_E - 1) / RL_E, (T + RL_T - 1) / RL_T, sp), dim3(512), 0,
                           st, static_cast<const uint16_t*>(u), parts, T, H, N_r, kc, part);
        splits = sp;
      } else {
        int kc = (H + splits - 1) / splits;            // K chunks in whole 32-deep MFMA steps
        kc = (kc + 31) / 32 * 32;
        const int sp = (H + kc - 1) / kc;
        hipLaunchKernelGGL(route_logits_mfma, dim3((N_r + RM_TILE - 1) / RM_TILE, (T + RM_TILE - 1) / RM_TILE, sp),
                           dim3(256), 0, st, static_cast<const uint16_t*>(u), parts, T, H, N_r, kc, part);
        splits = sp;
      }
    } else if (u_dtype == MOE_BF16)
      hipLaunchKernelGGL(route_logits<uint16_t>, grid, dim3(256), 0, st,
                         static_cast<const uint16_t*>(u), centroids, T, H, N_r, kchunk, part);
    else
      hipLaunchKernelGGL(route_logits<float>, grid, dim3(256), 0, st, static_cast<const float*>(u),
                         centroids, T, H, N_r, kchunk, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid((T + 3) / 4);
  const int nj = (N_r + 63) / 64;
  const bool batch = splits >= 16;   // few tokens (measured: T = 128 40 -> 35 us; no gain at T >= 4096)
#define MOE_SEL(NJ)                                                                               \
  hipLaunchKernelGGL((batch ? route_select<NJ, true> : route_select<NJ, false>), grid, dim3(256), 0, st, \
                     part, splits, logit_offset, affinity_in, bias, T, N_r, K, n_groups, topk_groups, \
                     affinity_out, topk_idx, topk_gate)
  if (nj <= 1) MOE_SEL(1);
  else if (nj <= 2) MOE_SEL(2);
  else if (nj <= 4) MOE_SEL(4);
  else if (nj <= 8) MOE_SEL(8);
  else MOE_SEL(16);
#undef MOE_SEL
  return hipGetLastError();
}

}  // namespace moe
