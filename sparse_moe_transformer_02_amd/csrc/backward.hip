// Backward pass of the DeepSeekMoE layer (bf16 operands, fp32 accumulation and gradients).
//
// xyznot.com "รายงานเชิงเทคนิคของ DeepSeek-V3", Method §2: h'_t = u_t + shared FFN(u_t) +
// sum_i g_{i,t} FFN_i(u_t), g = s / sum(s) over the selected experts, s = Sigmoid(u . e).
// The selection (Top-K over s + b) is piecewise constant: no gradient flows through it or
// into b. Per expert row (SwiGLU FFN, z = W_g x, v = W_u x, h = SiLU(z) v, y = W_d h):
//   dh = dy W_d,  dz = dh v SiLU'(z),  dv = dh SiLU(z),  dx = dz W_g + dv W_u,
//   dW_d += dy^T h,  dW_g += dz^T x,  dW_u += dv^T x.
// The layer: dy = g dout for a routed row (dout for the shared expert's row), dg = dout . y,
// ds_k = (dg_k - sum_j g_j dg_j) / S, dlogit = ds s (1 - s), du = dout + sum dx + sum dlogit e,
// de_i = sum over i's rows of dlogit u.
//
// GEMMs. Where H and I are multiples of 512 the row GEMMs run on the forward's LDS-tiled kernel
// (ffn.hip): the z/v recompute as its gate/up GEMM with fp32 pre-activations out, dh and dx with
// the MN-major weights staged as k-rows and read through transposing LDS loads. The kernels here:
// one 128 x 128-tile family (4 waves, each 64 x 64 with 16x16x32 bf16 MFMAs, K staged 32 deep
// through LDS, operands K-contiguous in LDS; an operand held in global memory with its M/N index
// contiguous ("MN-major") is transposed on the way into LDS):
//   bwd_rows:    C[r][n] = sum_k A[r][k] B(n, k) over a group's rows r (row GEMMs for other shapes)
//   bwd_wgrad:   C_g[m][n] = sum over group g's rows r of A[r][m] B[r][n] (dW_d, dW_g, dW_u) for
//                decode-sized groups
//   wgrad_tiled: the same from transposed, 64-padded copies of the operands (groups of 32+ rows)
// Every sum runs in a fixed order: gradients are bitwise reproducible.
#include "common.h"
#include "lds.h"
#include "tiles.h"

namespace moe {

namespace {

constexpr int BT = 128;            // tile rows and columns
constexpr int BK = 32;             // K per stage (one MFMA k-step)
constexpr int LROW = BK + 8;       // LDS row pitch in bf16 (80 bytes: 16-byte aligned, skewed banks)
constexpr int BWD_GM = 8;          // row tiles per band (they share weight tiles in L2)

// 16 MFMAs of a wave's 64 x 64 sub-tile for one 32-deep stage held in LDS
__device__ __forceinline__ void mma_stage(const uint16_t* __restrict__ sA, const uint16_t* __restrict__ sB,
                                          int wm, int wn, int lane, f32x4 (&acc)[4][4]) {
  const int r = lane & 15, c = (lane >> 4) * 8;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = *reinterpret_cast<const bf16x8*>(sA + (wm * 64 + i * 16 + r) * LROW + c);
    b[i] = *reinterpret_cast<const bf16x8*>(sB + (wn * 64 + i * 16 + r) * LROW + c);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
}

// A stage of one operand: 512 chunks of 8 bf16, two per thread.
//  K-major:  chunk c -> tile row c / 4, k = (c % 4) * 8 .. +8   (one 16-byte load, one LDS write)
//  MN-major: chunk c -> k = c % 32, tile rows (c / 32) * 8 .. +8 (one 16-byte load, 8 LDS writes);
//            a wave's 64 lanes then write 32 consecutive k of two rows 8 apart per store, which
//            fall in distinct LDS banks (rows 8 apart with lanes spread over the row index all
//            hit the same two banks at this row pitch)
__device__ __forceinline__ void put_kmajor(uint16_t* __restrict__ s, uint4 v0, uint4 v1) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = threadIdx.x + 256 * j;
    *reinterpret_cast<uint4*>(s + (c >> 2) * LROW + (c & 3) * 8) = j ? v1 : v0;
  }
}

__device__ __forceinline__ void put_mnmajor(uint16_t* __restrict__ s, uint4 v0, uint4 v1) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = threadIdx.x + 256 * j;
    const int k = c & 31, m0 = (c >> 5) * 8;
    const uint4 v = j ? v1 : v0;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[(m0 + 2 * i) * LROW + k] = (uint16_t)(w[i] & 0xffffu);
      s[(m0 + 2 * i + 1) * LROW + k] = (uint16_t)(w[i] >> 16);
    }
  }
}

__device__ __forceinline__ uint4 ld16(const uint16_t* p, bool ok) {
  return ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0u, 0u, 0u, 0u);
}

// fp32 weight-gradient tiles are written once and never read back by the GEMMs. The tiled
// kernel (groups of 32+ rows) stores them non-temporally so that they do not evict the operand
// tiles that other workgroups still read from L2 (prefill: 17.7 -> 13.8 ms for the three
// gradients); the direct kernel (decode-sized groups) keeps plain stores, which measured faster
// there (6.4 vs 11.3 ms).
template <bool NT>
__device__ __forceinline__ void wgrad_store(float* p, float v) {
  if (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// ----------------------------------------------------------------------------- row GEMMs
// For the rows r of each group g (tiles of 128 rows x 128 columns, items from the tile prefix):
//   C[r][n] = sum_k A[src(r)][k] * B_g(n, k),  k in [0, K)
// A: K-major [*, lda], row src(r) = row_index[r] when GATHER (rows outside [0, a_rows) read 0).
// B_KMAJOR:  B_g(n, k) = (n < split ? B0 : B1)[g][n mod split][k]   ([split, K] per group)
// otherwise: B_g(n, k) = (k < split ? B0 : B1)[g][k mod split][n]   ([split, N] per group)
template <bool B_KMAJOR, bool GATHER>
__global__ __launch_bounds__(256) void bwd_rows(const int32_t* __restrict__ off, const int32_t* __restrict__ prefix,
                                                int n_groups, int total_rows, const int32_t* __restrict__ row_index,
                                                int a_rows, const uint16_t* __restrict__ A, int lda, int K,
                                                const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1,
                                                int split, int N, float* __restrict__ C, int ldc) {
  __shared__ __align__(16) uint16_t sA[BT * LROW];
  __shared__ __align__(16) uint16_t sB[BT * LROW];
  int nt;
  Tile t;
  if (!find_tile(off, prefix, n_groups, total_rows, BT, N / BT, BWD_GM, nt, t)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const size_t gstride = (size_t)split * (B_KMAJOR ? K : N);
  // per-thread chunk sources
  const uint16_t* ap[2];
  bool aok[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = threadIdx.x + 256 * j;
    const int r = t.r0 + (c >> 2);
    int src = -1;
    if (r < t.r1) src = GATHER ? row_index[r] : r;
    aok[j] = src >= 0 && src < a_rows;
    ap[j] = A + (size_t)(aok[j] ? src : 0) * lda + (c & 3) * 8;
  }
  auto load_b = [&](int k0, int j) -> uint4 {
    const int c = threadIdx.x + 256 * j;
    if (B_KMAJOR) {
      const int n = nt * BT + (c >> 2), k = k0 + (c & 3) * 8;
      const uint16_t* base = n < split ? B0 + t.g * gstride + (size_t)n * K : B1 + t.g * gstride + (size_t)(n - split) * K;
      return *reinterpret_cast<const uint4*>(base + k);
    }
    const int k = k0 + (c & 31), n = nt * BT + (c >> 5) * 8;
    const uint16_t* base = k < split ? B0 + t.g * gstride + (size_t)k * N : B1 + t.g * gstride + (size_t)(k - split) * N;
    return *reinterpret_cast<const uint4*>(base + n);
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 a0 = ld16(ap[0], aok[0]), a1 = ld16(ap[1], aok[1]);
  uint4 b0 = load_b(0, 0), b1 = load_b(0, 1);
  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();                         // the previous stage's fragments are consumed
    put_kmajor(sA, a0, a1);
    if (B_KMAJOR) put_kmajor(sB, b0, b1); else put_mnmajor(sB, b0, b1);
    __syncthreads();
    if (k0 + BK < K) {                       // next stage's loads fly during this stage's MFMAs
      a0 = ld16(ap[0] + k0 + BK, aok[0]);
      a1 = ld16(ap[1] + k0 + BK, aok[1]);
      b0 = load_b(k0 + BK, 0);
      b1 = load_b(k0 + BK, 1);
    }
    mma_stage(sA, sB, wm, wn, lane, acc);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = t.r0 + wm * 64 + i * 16 + (lane >> 4) * 4 + q;
      if (r >= t.r1) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) C[(size_t)r * ldc + nt * BT + wn * 64 + j * 16 + (lane & 15)] = acc[i][j][q];
    }
}

// ----------------------------------------------------------------------------- weight gradients
// C_g[m][n] = sum over rows r of group g of A[r][m] * B[src(r)][n]; one workgroup per 128 x 128
// output tile of one group (work item = (g * mt + tile m) * nt + tile n, split over the XCDs).
// A: [*, lda] bf16 with m contiguous; B: [*, ldb] with n contiguous, src(r) = row_index[r] when
// GATHER (rows outside [0, b_rows) read 0). A group without rows gets zeros.
template <bool GATHER>
__global__ __launch_bounds__(256) void bwd_wgrad(const int32_t* __restrict__ off, int n_groups, int total_rows,
                                                 const uint16_t* __restrict__ A, int lda,
                                                 const uint16_t* __restrict__ B, int ldb,
                                                 const int32_t* __restrict__ row_index, int b_rows, int M, int N,
                                                 float* __restrict__ C) {
  __shared__ __align__(16) uint16_t sA[BT * LROW];
  __shared__ __align__(16) uint16_t sB[BT * LROW];
  const int mt = M / BT, ntl = N / BT;
  const int w = xcd_item(n_groups * mt * ntl);
  if (w < 0) return;
  const int g = w / (mt * ntl), tm = (w / ntl) % mt, tn = w % ntl;
  int r0, r1;
  group_rows(off, g, total_rows, r0, r1);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  auto load_a = [&](int k0, int j) -> uint4 {
    const int c = threadIdx.x + 256 * j;
    const int r = r0 + k0 + (c & 31), x0 = (c >> 5) * 8;
    const bool live = r < r1;
    return ld16(A + (size_t)(live ? r : 0) * lda + tm * BT + x0, live);
  };
  auto load_b = [&](int k0, int j) -> uint4 {
    const int c = threadIdx.x + 256 * j;
    const int r = r0 + k0 + (c & 31), x0 = (c >> 5) * 8;
    int src = -1;
    if (r < r1) src = GATHER ? row_index[r] : r;
    const bool bl = src >= 0 && src < b_rows;
    return ld16(B + (size_t)(bl ? src : 0) * ldb + tn * BT + x0, bl);
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int K = r1 - r0;
  uint4 a0 = make_uint4(0u, 0u, 0u, 0u), a1 = a0, b0 = a0, b1 = a0;
  if (K > 0) {
    a0 = load_a(0, 0); a1 = load_a(0, 1);
    b0 = load_b(0, 0); b1 = load_b(0, 1);
  }
  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
    put_mnmajor(sA, a0, a1);
    put_mnmajor(sB, b0, b1);
    __syncthreads();
    if (k0 + BK < K) {
      a0 = load_a(k0 + BK, 0); a1 = load_a(k0 + BK, 1);
      b0 = load_b(k0 + BK, 0); b1 = load_b(k0 + BK, 1);
    }
    mma_stage(sA, sB, wm, wn, lane, acc);
  }
  float* Cg = C + (size_t)g * M * N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = tm * BT + wm * 64 + i * 16 + (lane >> 4) * 4 + q;
#pragma unroll
      for (int j = 0; j < 4; ++j) wgrad_store<false>(&Cg[(size_t)m * N + tn * BT + wn * 64 + j * 16 + (lane & 15)], acc[i][j][q]);
    }
}

// ----------------------------------------------------------------------------- weight gradients, tiled
// The weight gradients reduce over a group's rows. Their operands are first transposed into
// feature-major buffers OpT [F, Rp] in which group g owns the columns [poff[g], poff[g] + Pg),
// Pg = rows_g rounded up to 64 (zeros past rows_g), so that both operands are K-contiguous:
//   C_g[m][n] = sum over g's columns c of At[m][c] * Bt[n][c]
// (16-byte loads and 16-byte LDS writes, no transposition inside the GEMM).
constexpr int TP = 64;   // transpose tile, and the column padding of each group

// 64 padded columns x 64 features per workgroup: rows of src (gathered through row_index when
// given) -> columns of dst [F, ldd]
__global__ __launch_bounds__(256) void transpose_pad(const int32_t* __restrict__ off, const int32_t* __restrict__ poff,
                                                     int n_groups, int total_rows, const uint16_t* __restrict__ src,
                                                     int lds_src, int src_rows, const int32_t* __restrict__ row_index,
                                                     int F, uint16_t* __restrict__ dst, int ldd) {
  __shared__ uint16_t tile[TP][TP + 2];
  const int c0 = blockIdx.x * TP, f0 = blockIdx.y * TP;
  if (c0 >= poff[n_groups]) return;
  const int g = find_group(poff, n_groups, c0);
  int r0, r1;
  group_rows(off, g, total_rows, r0, r1);
  const int lc0 = c0 - poff[g];              // first local column of this block inside group g
  // load: thread -> (row j of the block, 4 features)
  for (int q = threadIdx.x; q < TP * (TP / 4); q += 256) {
    const int j = q / (TP / 4), f = (q % (TP / 4)) * 4;
    const int r = r0 + lc0 + j;
    uint2 v = make_uint2(0u, 0u);
    if (r < r1) {
      const int sr = row_index ? row_index[r] : r;
      if (sr >= 0 && sr < src_rows) v = *reinterpret_cast<const uint2*>(src + (size_t)sr * lds_src + f0 + f);
    }
    tile[j][f] = (uint16_t)(v.x & 0xffffu);
    tile[j][f + 1] = (uint16_t)(v.x >> 16);
    tile[j][f + 2] = (uint16_t)(v.y & 0xffffu);
    tile[j][f + 3] = (uint16_t)(v.y >> 16);
  }
  __syncthreads();
  // store: thread -> (feature f, 4 columns)
  for (int q = threadIdx.x; q < TP * (TP / 4); q += 256) {
    const int f = q / (TP / 4), j = (q % (TP / 4)) * 4;
    uint2 v;
    v.x = (uint32_t)tile[j][f] | ((uint32_t)tile[j + 1][f] << 16);
    v.y = (uint32_t)tile[j + 2][f] | ((uint32_t)tile[j + 3][f] << 16);
    *reinterpret_cast<uint2*>(dst + (size_t)(f0 + f) * ldd + c0 + j) = v;
  }
}

// 128 x 128 output tile of one group per 256-thread workgroup (20 KB of LDS, so several run on a
// CU and their epilogues overlap other workgroups' loads): both operands K-contiguous, staged 32
// deep with the next stage's loads in registers during this stage's MFMAs.
__global__ __launch_bounds__(256) void wgrad_tiled(const int32_t* __restrict__ off, const int32_t* __restrict__ poff,
                                                   int n_groups, int total_rows, const uint16_t* __restrict__ At,
                                                   const uint16_t* __restrict__ Bt, int ld, int M, int N,
                                                   float* __restrict__ C) {
  __shared__ __align__(16) uint16_t sA[BT * LROW];
  __shared__ __align__(16) uint16_t sB[BT * LROW];
  const int mt = M / BT, ntl = N / BT;
  const int w = xcd_item(n_groups * mt * ntl);
  if (w < 0) return;
  const int g = w / (mt * ntl), tm = (w / ntl) % mt, tn = w % ntl;
  int r0, r1;
  group_rows(off, g, total_rows, r0, r1);
  const size_t c0 = poff[g];
  // padded columns past rows_g hold zeros; never past the buffer, whatever the offsets say
  const long long room = c0 < (size_t)ld ? ((long long)ld - (long long)c0) / BK * BK : 0;
  const int K = (int)min((long long)((r1 - r0 + BK - 1) / BK * BK), room);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const uint16_t* ap[2];
  const uint16_t* bp[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = threadIdx.x + 256 * j;
    ap[j] = At + (size_t)(tm * BT + (c >> 2)) * ld + c0 + (c & 3) * 8;
    bp[j] = Bt + (size_t)(tn * BT + (c >> 2)) * ld + c0 + (c & 3) * 8;
  }
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 a0 = make_uint4(0u, 0u, 0u, 0u), a1 = a0, b0 = a0, b1 = a0;
  if (K > 0) {
    a0 = *reinterpret_cast<const uint4*>(ap[0]);
    a1 = *reinterpret_cast<const uint4*>(ap[1]);
    b0 = *reinterpret_cast<const uint4*>(bp[0]);
    b1 = *reinterpret_cast<const uint4*>(bp[1]);
  }
  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
    put_kmajor(sA, a0, a1);
    put_kmajor(sB, b0, b1);
    __syncthreads();
    if (k0 + BK < K) {
      a0 = *reinterpret_cast<const uint4*>(ap[0] + k0 + BK);
      a1 = *reinterpret_cast<const uint4*>(ap[1] + k0 + BK);
      b0 = *reinterpret_cast<const uint4*>(bp[0] + k0 + BK);
      b1 = *reinterpret_cast<const uint4*>(bp[1] + k0 + BK);
    }
    mma_stage(sA, sB, wm, wn, lane, acc);
  }
  float* Cg = C + (size_t)g * M * N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = tm * BT + wm * 64 + i * 16 + (lane >> 4) * 4 + q;
#pragma unroll
      for (int j = 0; j < 4; ++j) wgrad_store<true>(&Cg[(size_t)m * N + tn * BT + wn * 64 + j * 16 + (lane & 15)], acc[i][j][q]);
    }
}

// ----------------------------------------------------------------------------- SwiGLU backward
// ZV [rows, 2I] fp32 (z then v), dH [rows, I] fp32 -> Hh [rows, I] bf16 (h = SiLU(z) v, for dW_d)
// and dZV [rows, 2I] bf16 (dz = dh v SiLU'(z), dv = dh SiLU(z)).
__global__ __launch_bounds__(256) void bwd_swiglu(const float* __restrict__ ZV, const float* __restrict__ dH,
                                                  long long rows, int I, uint16_t* __restrict__ Hh,
                                                  uint16_t* __restrict__ dZV) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * I) return;
  const long long r = i / I;
  const int c = (int)(i % I);
  const float z = ZV[r * 2 * I + c], v = ZV[r * 2 * I + I + c], dh = dH[i];
  const float sig = 1.0f / (1.0f + __expf(-z));
  const float a = z * sig;
  Hh[i] = f32_to_bf16(a * v);
  dZV[r * 2 * I + c] = f32_to_bf16(dh * v * sig * (1.0f + z * (1.0f - sig)));
  dZV[r * 2 * I + I + c] = f32_to_bf16(dh * a);
}

// ----------------------------------------------------------------------------- layer pieces
// V consecutive elements as fp32 (V = 1, 4 or 8; V > 1 needs 4 * V-byte (fp32) or 2 * V-byte (bf16)
// aligned addresses)
template <int V>
__device__ __forceinline__ void ldv(const uint16_t* p, float (&v)[V]) {
  if constexpr (V == 1) {
    v[0] = bf16_to_f32(*p);
  } else {
    uint32_t w[V / 2];
    if constexpr (V == 4) {
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      w[0] = u.x; w[1] = u.y;
    } else {
      const uint4 u = *reinterpret_cast<const uint4*>(p);
      w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
    }
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
      v[2 * i] = bf16_to_f32((uint16_t)(w[i] & 0xffffu));
      v[2 * i + 1] = bf16_to_f32((uint16_t)(w[i] >> 16));
    }
  }
}
template <int V>
__device__ __forceinline__ void ldv(const float* p, float (&v)[V]) {
  if constexpr (V == 1) {
    v[0] = *p;
  } else {
#pragma unroll
    for (int i = 0; i < V / 4; ++i) {
      const float4 f = reinterpret_cast<const float4*>(p)[i];
      v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
  }
}
template <int V>
__device__ __forceinline__ void stv_bf16(uint16_t* p, const float (&v)[V]) {
  if constexpr (V == 1) {
    *p = f32_to_bf16(v[0]);
  } else {
    uint32_t w[V / 2];
#pragma unroll
    for (int i = 0; i < V / 2; ++i) w[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
    if constexpr (V == 4) *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
    else *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// One workgroup per token: dY rows (shared row t: dout_t; routed row of (t, k): g_{t,k} dout_t)
// and dgate_{t,k} = dout_t . Y[slot_row[t,k]] (fp32, fixed-order block reduction). Each thread
// takes V consecutive elements at a time (V = 8 when H % 8 == 0 and the rows are 16-byte aligned).
template <typename TIO, typename TY, int V>
__global__ __launch_bounds__(256) void combine_bwd(const TIO* __restrict__ dout, const TY* __restrict__ Y,
                                                   const int32_t* __restrict__ slot_row,
                                                   const float* __restrict__ gate, int K, int H, int S,
                                                   int total_rows, uint16_t* __restrict__ dY,
                                                   float* __restrict__ dgate) {
  __shared__ float red[MOE_MAX_TOPK][4];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float part[MOE_MAX_TOPK];
  int rows[MOE_MAX_TOPK];
  float gs[MOE_MAX_TOPK];
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK; ++k) {
    part[k] = 0.f;
    rows[k] = -1;
    gs[k] = 0.f;
    if (k < K) {
      const int r = slot_row[(size_t)t * K + k];
      rows[k] = (r >= 0 && r < total_rows) ? r : -1;
      gs[k] = gate[(size_t)t * K + k];
    }
  }
  for (int c = threadIdx.x; c < H / V; c += 256) {
    const size_t h = (size_t)c * V;
    float d[V];
    ldv<V>(dout + (size_t)t * H + h, d);
    if (S > 0 && t < S) stv_bf16<V>(dY + (size_t)t * H + h, d);
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK; ++k) {
      if (k < K && rows[k] >= 0) {
        float y[V], gd[V];
        ldv<V>(Y + (size_t)rows[k] * H + h, y);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          part[k] = fmaf(d[e], y[e], part[k]);
          gd[e] = gs[k] * d[e];
        }
        stv_bf16<V>(dY + (size_t)rows[k] * H + h, gd);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK; ++k) {
    if (k >= K) break;
    float v = part[k];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0) red[k][wave] = v;
  }
  __syncthreads();
  if ((int)threadIdx.x < K) {
    const int k = threadIdx.x;
    dgate[(size_t)t * K + k] = rows[k] >= 0 ? (red[k][0] + red[k][1]) + (red[k][2] + red[k][3]) : 0.f;
  }
}

// One workgroup per token: gate and sigmoid backward (dlogit for its K choices, also written per
// routed row for the centroid gradient) and the input gradient
//   du_t = dout_t + dX[shared row t] + sum_k dX[slot_row[t,k]] + sum_k dlogit_k e_{idx_k}
// (V consecutive elements per thread at a time, each summed in that order)
template <typename TIO, int V>
__global__ __launch_bounds__(256) void router_input_bwd(const TIO* __restrict__ dout, const float* __restrict__ dX,
                                                        const int32_t* __restrict__ slot_row, int S,
                                                        int total_rows, const float* __restrict__ s,
                                                        const int32_t* __restrict__ idx,
                                                        const float* __restrict__ gate,
                                                        const float* __restrict__ dgate,
                                                        const float* __restrict__ E, int K, int H, int N_r,
                                                        float* __restrict__ du, float* __restrict__ dlogit_rows) {
  __shared__ float dl[MOE_MAX_TOPK];
  __shared__ int ex[MOE_MAX_TOPK];
  __shared__ int rw[MOE_MAX_TOPK];
  const int t = blockIdx.x;
  if (threadIdx.x == 0) {
    float ssum = 0.f, gd = 0.f;
    for (int k = 0; k < K; ++k) {
      const int e = idx[(size_t)t * K + k];
      const float sk = (e >= 0 && e < N_r) ? s[(size_t)t * N_r + e] : 0.f;
      ssum += sk;
      gd = fmaf(gate[(size_t)t * K + k], dgate[(size_t)t * K + k], gd);
    }
    for (int k = 0; k < K; ++k) {
      const int e = idx[(size_t)t * K + k];
      const bool ok = e >= 0 && e < N_r && ssum > 0.f;
      const float sk = ok ? s[(size_t)t * N_r + e] : 0.f;
      const float d = ok ? (dgate[(size_t)t * K + k] - gd) / ssum * sk * (1.f - sk) : 0.f;
      const int r = slot_row[(size_t)t * K + k];
      dl[k] = d;
      ex[k] = ok ? e : -1;
      rw[k] = (r >= 0 && r < total_rows) ? r : -1;
      if (rw[k] >= 0) dlogit_rows[rw[k]] = d;
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < H / V; c += 256) {
    const size_t h = (size_t)c * V;
    float acc[V], x[V];
    ldv<V>(dout + (size_t)t * H + h, acc);
    if (S > 0 && t < S) {
      ldv<V>(dX + (size_t)t * H + h, x);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] += x[e];
    }
    for (int k = 0; k < K; ++k)
      if (rw[k] >= 0) {
        ldv<V>(dX + (size_t)rw[k] * H + h, x);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] += x[e];
      }
    for (int k = 0; k < K; ++k)
      if (ex[k] >= 0) {
        ldv<V>(E + (size_t)ex[k] * H + h, x);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] = fmaf(dl[k], x[e], acc[e]);
      }
    if constexpr (V == 1) {
      du[(size_t)t * H + h] = acc[0];
    } else {
#pragma unroll
      for (int i = 0; i < V / 4; ++i)
        reinterpret_cast<float4*>(du + (size_t)t * H + h)[i] = make_float4(acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]);
    }
  }
}

// dE_i[h] = sum over routed rows r of expert i (group i + g0, in row order) of dlogit_r u[row_token[r]][h];
// each thread owns V consecutive h (V = 4 when H % 4 == 0 and the rows are 16-byte aligned)
template <typename TU, int V>
__global__ __launch_bounds__(256) void centroid_bwd(const int32_t* __restrict__ off, int g0, int total_rows,
                                                    const int32_t* __restrict__ row_token,
                                                    const float* __restrict__ dlogit_rows,
                                                    const TU* __restrict__ u, int T, int H,
                                                    float* __restrict__ dE) {
  const int i = blockIdx.y;
  const int h = (blockIdx.x * 256 + threadIdx.x) * V;
  if (h >= H) return;
  int r0, r1;
  group_rows(off, i + g0, total_rows, r0, r1);
  float acc[V] = {};
  for (int r = r0; r < r1; ++r) {
    const int tok = row_token[r];
    if (tok >= 0 && tok < T) {
      const float d = dlogit_rows[r];
      float x[V];
      ldv<V>(u + (size_t)tok * H + h, x);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = fmaf(d, x[e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < V; ++e) dE[(size_t)i * H + h + e] = acc[e];
}

// The transposed-operand weight-gradient path (64-column group padding) pays off once groups
// average 32 rows or more; below that (decode) the padding multiplies the operand reads and the
// direct kernel, which transposes inside, is faster (measured at the V3 decode shape).
constexpr int TILED_WGRAD_MIN_AVG_ROWS = 32;
inline bool tiled_wgrad(int n_groups, int total_rows, int H, int I) {
  return H % 128 == 0 && I % 128 == 0 && total_rows >= TILED_WGRAD_MIN_AVG_ROWS * (long long)n_groups;
}

// padded column count bound of the transposed operands: every group rounded up to 64
inline size_t padded_cols(int n_groups, int total_rows) {
  return ((size_t)total_rows + (size_t)TP * n_groups + TP - 1) / TP * TP;
}

#ifndef MOE_ROWS_MN
#define MOE_ROWS_MN 1
#endif
inline bool rows_mn_tiled(int H, int I) { return MOE_ROWS_MN && H % 512 == 0 && I % 512 == 0; }

struct BwdWs {
  size_t prefix, zv, dh, hh, dzv, tr, total;
};

BwdWs bwd_layout(int n_groups, int total_rows, int H, int I) {
  BwdWs L{};
  size_t o = 0;
  const size_t rows = (size_t)total_rows;
  L.prefix = o; o += align256((size_t)3 * (n_groups + 1) * sizeof(int32_t));
  L.zv = o; o += align256(rows * 2 * I * sizeof(float));
  L.dh = o; o += align256(rows * I * sizeof(float));
  L.hh = o; o += align256(rows * I * sizeof(uint16_t));
  L.dzv = o; o += align256(rows * 2 * I * sizeof(uint16_t));
  L.tr = o;
  if (tiled_wgrad(n_groups, total_rows, H, I))
    o += align256(padded_cols(n_groups, total_rows) * (2 * (size_t)H + 3 * (size_t)I) * sizeof(uint16_t));
  L.total = o;
  return L;
}

}  // namespace

size_t grouped_ffn_backward_workspace(int n_groups, int total_rows, int H, int I) {
  if (total_rows == 0) return 0;
  return bwd_layout(n_groups, total_rows, H, I).total;
}

hipError_t launch_grouped_ffn_backward(const FfnBwdArgs& a, hipStream_t st, void* const* ev) {
  if (a.total_rows == 0 && a.n_groups == 0) return hipSuccess;
  const int H = a.H, I = a.I;
  const BwdWs L = bwd_layout(a.n_groups, a.total_rows, H, I);
  char* ws = static_cast<char*>(a.ws);
  int32_t* prefix_i = reinterpret_cast<int32_t*>(ws + L.prefix);   // column tiles of 2I / I wide rows
  int32_t* prefix_h = prefix_i + (a.n_groups + 1);
  // pre-activations z | v: saved by the forward, else recomputed into the workspace
  const float* ZV = a.zv ? a.zv : reinterpret_cast<const float*>(ws + L.zv);
  float* dH = reinterpret_cast<float*>(ws + L.dh);
  uint16_t* Hh = reinterpret_cast<uint16_t*>(ws + L.hh);
  uint16_t* dZV = reinterpret_cast<uint16_t*>(ws + L.dzv);
  const uint16_t* X = static_cast<const uint16_t*>(a.X);
  const uint16_t* Wg = static_cast<const uint16_t*>(a.Wg);
  const uint16_t* Wu = static_cast<const uint16_t*>(a.Wu);
  const uint16_t* Wd = static_cast<const uint16_t*>(a.Wd);
  const uint16_t* dY = static_cast<const uint16_t*>(a.dY);
  auto mark = [&](int i) {
    if (ev && ev[i]) (void)hipEventRecord(static_cast<hipEvent_t>(ev[i]), st);
  };
  if (a.total_rows > 0) {
    const long long ms = (a.total_rows + BT - 1) / BT + a.n_groups;
    auto pad8 = [](long long n) { return (unsigned)((n + 7) / 8 * 8); };
    // z / v recompute (N = 2I: gate rows then up rows), dh = dY W_d (N = I), dx = [dz dv] [W_g; W_u] (N = H)
    mark(0);
    float* zv_out = reinterpret_cast<float*>(ws + L.zv);
    if (a.zv) {
      // saved by the forward: nothing to recompute
    } else if (gate_up_preact_supported(H, I)) {     // the forward's LDS-tiled gate/up GEMM, z and v out
      hipError_t e = launch_gate_up_preact(a.offsets, a.n_groups, a.total_rows, a.row_index, X, a.x_rows, Wg, Wu, H,
                                           I, prefix_i, zv_out, st);
      if (e != hipSuccess) return e;
    } else {
      hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, a.offsets, a.n_groups, a.total_rows, BT,
                         2 * I / BT, prefix_i);
      if (a.row_index)
        hipLaunchKernelGGL((bwd_rows<true, true>), dim3(pad8(ms * (2 * I / BT))), dim3(256), 0, st, a.offsets,
                           prefix_i, a.n_groups, a.total_rows, a.row_index, a.x_rows, X, H, H, Wg, Wu, I, 2 * I, zv_out,
                           2 * I);
      else
        hipLaunchKernelGGL((bwd_rows<true, false>), dim3(pad8(ms * (2 * I / BT))), dim3(256), 0, st, a.offsets,
                           prefix_i, a.n_groups, a.total_rows, a.row_index, a.x_rows, X, H, H, Wg, Wu, I, 2 * I, zv_out,
                           2 * I);
    }
    // dh and dx: LDS-tiled with transposing weight reads where the shapes allow it
    const bool mn = rows_mn_tiled(H, I) && rows_mn_supported(I, H, H) && rows_mn_supported(H, 2 * I, I);
    if (mn) {
      hipError_t e = launch_rows_mn(a.offsets, a.n_groups, a.total_rows, dY, Wd, Wd, H, I, H, prefix_i, dH, st);
      if (e != hipSuccess) return e;
    } else {
      hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, a.offsets, a.n_groups, a.total_rows, BT,
                         I / BT, prefix_i);
      hipLaunchKernelGGL((bwd_rows<false, false>), dim3(pad8(ms * (I / BT))), dim3(256), 0, st, a.offsets, prefix_i,
                         a.n_groups, a.total_rows, static_cast<const int32_t*>(nullptr), a.total_rows, dY, H, H, Wd,
                         Wd, H, I, dH, I);
    }
    const long long n = (long long)a.total_rows * I;
    hipLaunchKernelGGL(bwd_swiglu, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, ZV, dH,
                       (long long)a.total_rows, I, Hh, dZV);
    if (mn) {
      hipError_t e = launch_rows_mn(a.offsets, a.n_groups, a.total_rows, dZV, Wg, Wu, I, H, 2 * I, prefix_h,
                                    static_cast<float*>(a.dX), st);
      if (e != hipSuccess) return e;
    } else {
      hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, a.offsets, a.n_groups, a.total_rows, BT,
                         H / BT, prefix_h);
      hipLaunchKernelGGL((bwd_rows<false, false>), dim3(pad8(ms * (H / BT))), dim3(256), 0, st, a.offsets, prefix_h,
                         a.n_groups, a.total_rows, static_cast<const int32_t*>(nullptr), a.total_rows, dZV, 2 * I,
                         2 * I, Wg, Wu, I, H, static_cast<float*>(a.dX), H);
    }
    mark(1);
  } else {
    mark(0);
    mark(1);
  }
  // weight gradients: dW_d = dY^T h, dW_g = dz^T x, dW_u = dv^T x (zeros for groups without rows)
  mark(2);
  if (tiled_wgrad(a.n_groups, a.total_rows, H, I) && a.total_rows > 0) {   // no rows: no workspace, zeros below
    int32_t* poff = prefix_h + (a.n_groups + 1);
    const size_t Rp = padded_cols(a.n_groups, a.total_rows);
    uint16_t* dYT = reinterpret_cast<uint16_t*>(ws + L.tr);
    uint16_t* XT = dYT + (size_t)H * Rp;
    uint16_t* HhT = XT + (size_t)H * Rp;
    uint16_t* dZT = HhT + (size_t)I * Rp;
    uint16_t* dVT = dZT + (size_t)I * Rp;
    hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, a.offsets, a.n_groups, a.total_rows, TP, TP,
                       poff);
    const unsigned cb = (unsigned)(Rp / TP);
    auto tr = [&](const uint16_t* src, int lds_src, int src_rows, const int32_t* ri, int F, uint16_t* dst) {
      hipLaunchKernelGGL(transpose_pad, dim3(cb, F / TP), dim3(256), 0, st, a.offsets, poff, a.n_groups,
                         a.total_rows, src, lds_src, src_rows, ri, F, dst, (int)Rp);
    };
    tr(dY, H, a.total_rows, nullptr, H, dYT);
    tr(X, H, a.x_rows, a.row_index, H, XT);
    tr(Hh, I, a.total_rows, nullptr, I, HhT);
    tr(dZV, 2 * I, a.total_rows, nullptr, I, dZT);
    tr(dZV + I, 2 * I, a.total_rows, nullptr, I, dVT);
    auto gemm = [&](const uint16_t* At, const uint16_t* Bt, int M, int N, void* C) {
      const int items = a.n_groups * (M / BT) * (N / BT);
      hipLaunchKernelGGL(wgrad_tiled, dim3((unsigned)((items + 7) / 8 * 8)), dim3(256), 0, st, a.offsets, poff,
                         a.n_groups, a.total_rows, At, Bt, (int)Rp, M, N, static_cast<float*>(C));
    };
    gemm(dYT, HhT, H, I, a.dWd);
    gemm(dZT, XT, I, H, a.dWg);
    gemm(dVT, XT, I, H, a.dWu);
    mark(3);
    return hipGetLastError();
  }
  const int dwd_items = a.n_groups * (H / BT) * (I / BT);
  const unsigned grid_w = (unsigned)((dwd_items + 7) / 8 * 8);
  hipLaunchKernelGGL((bwd_wgrad<false>), dim3(grid_w), dim3(256), 0, st, a.offsets, a.n_groups, a.total_rows, dY,
                     H, Hh, I, static_cast<const int32_t*>(nullptr), a.total_rows, H, I, static_cast<float*>(a.dWd));
  auto wgrad_x = [&](const uint16_t* dzv, float* dW) {
    if (a.row_index)
      hipLaunchKernelGGL((bwd_wgrad<true>), dim3(grid_w), dim3(256), 0, st, a.offsets, a.n_groups, a.total_rows,
                         dzv, 2 * I, X, H, a.row_index, a.x_rows, I, H, dW);
    else
      hipLaunchKernelGGL((bwd_wgrad<false>), dim3(grid_w), dim3(256), 0, st, a.offsets, a.n_groups, a.total_rows,
                         dzv, 2 * I, X, H, a.row_index, a.x_rows, I, H, dW);
  };
  wgrad_x(dZV, static_cast<float*>(a.dWg));
  wgrad_x(dZV + I, static_cast<float*>(a.dWu));
  mark(3);
  return hipGetLastError();
}

hipError_t launch_combine_backward(const void* dout, int io_dtype, const void* Y, int y_dtype,
                                   const int32_t* slot_row, const float* gate, int T, int K, int H, int S,
                                   int total_rows, uint16_t* dY, float* dgate, hipStream_t st) {
  if (T == 0) return hipSuccess;
  auto go = [&](auto kern, auto* d, auto* y) {
    hipLaunchKernelGGL(kern, dim3(T), dim3(256), 0, st, d, y, slot_row, gate, K, H, S, total_rows, dY, dgate);
  };
  const uint16_t* db = static_cast<const uint16_t*>(dout);
  const float* df = static_cast<const float*>(dout);
  const uint16_t* yb = static_cast<const uint16_t*>(Y);
  const float* yf = static_cast<const float*>(Y);
  auto al16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  const bool vec = H % 8 == 0 && al16(dout) && al16(Y) && al16(dY);
  if (vec) {
    if (io_dtype == MOE_BF16 && y_dtype == MOE_BF16) go(combine_bwd<uint16_t, uint16_t, 8>, db, yb);
    else if (io_dtype == MOE_BF16) go(combine_bwd<uint16_t, float, 8>, db, yf);
    else if (y_dtype == MOE_BF16) go(combine_bwd<float, uint16_t, 8>, df, yb);
    else go(combine_bwd<float, float, 8>, df, yf);
  } else {
    if (io_dtype == MOE_BF16 && y_dtype == MOE_BF16) go(combine_bwd<uint16_t, uint16_t, 1>, db, yb);
    else if (io_dtype == MOE_BF16) go(combine_bwd<uint16_t, float, 1>, db, yf);
    else if (y_dtype == MOE_BF16) go(combine_bwd<float, uint16_t, 1>, df, yb);
    else go(combine_bwd<float, float, 1>, df, yf);
  }
  return hipGetLastError();
}

hipError_t launch_router_backward(const void* dout, const void* u, int io_dtype, const float* dX,
                                  const int32_t* offsets, int g0, const int32_t* row_token,
                                  const int32_t* slot_row, int S, int total_rows, const float* s,
                                  const int32_t* idx, const float* gate, const float* dgate, const float* E,
                                  int T, int K, int H, int N_r, float* du, float* dE, float* dlogit_rows,
                                  hipStream_t st) {
  if (T > 0) {
    auto al16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
    const bool vec = H % 4 == 0 && al16(dout) && al16(dX) && al16(E) && al16(du);
    auto go = [&](auto kern, auto* d) {
      hipLaunchKernelGGL(kern, dim3(T), dim3(256), 0, st, d, dX, slot_row, S, total_rows, s, idx, gate, dgate, E, K,
                         H, N_r, du, dlogit_rows);
    };
    const uint16_t* db = static_cast<const uint16_t*>(dout);
    const float* df = static_cast<const float*>(dout);
    if (io_dtype == MOE_BF16) {
      if (vec) go(router_input_bwd<uint16_t, 4>, db); else go(router_input_bwd<uint16_t, 1>, db);
    } else {
      if (vec) go(router_input_bwd<float, 4>, df); else go(router_input_bwd<float, 1>, df);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bool vec = H % 4 == 0 && ((uintptr_t)u & 15) == 0;
  const int V = vec ? 4 : 1;
  dim3 grid((H / V + 255) / 256, N_r);
  auto go = [&](auto kern, auto* x) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, offsets, g0, total_rows, row_token, dlogit_rows, x, T, H, dE);
  };
  const uint16_t* ub = static_cast<const uint16_t*>(u);
  const float* uf = static_cast<const float*>(u);
  if (io_dtype == MOE_BF16) {
    if (vec) go(centroid_bwd<uint16_t, 4>, ub); else go(centroid_bwd<uint16_t, 1>, ub);
  } else {
    if (vec) go(centroid_bwd<float, 4>, uf); else go(centroid_bwd<float, 1>, uf);
  }
  return hipGetLastError();
}

}  // namespace moe
