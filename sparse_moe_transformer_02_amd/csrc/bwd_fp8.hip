// Backward pass of the grouped SwiGLU expert FFN with E4M3 GEMM operands.
//
// "官方揭秘DeepSeek-V3模型训练全流程" §4.3 trains with FP8 GEMMs (activations in 1x128 tiles,
// weights in 128x128 blocks, fp32 accumulation); §4.5 notes that the backward needs its operands
// quantized along another axis. This library's reading: every GEMM operand is quantized from its
// high-precision value along that GEMM's reduction dimension.
//   z, v  = Q(x) Q(W_g)^T, Q(x) Q(W_u)^T          x in 1x128 tiles along H (the forward's operands)
//   dh    = Q(dy) Q(W_d)                          dy in 1x128 tiles along H; Q(W_d) read as W_d^T
//   h     = SiLU(z) v, dz = dh v SiLU'(z), dv = dh SiLU(z)          (fp32)
//   dx    = [Q(dz) Q(dv)] [Q(W_g); Q(W_u)]        dz, dv in 1x128 tiles along I
//   dW_d  = Qr(dy)^T Qr(h), dW_g = Qr(dz)^T Qr(x), dW_u = Qr(dv)^T Qr(x)
// with Qr the 128x1 tiles over each expert's rows (dispatch order; a last partial tile).
//
// The row GEMMs run on the forward's FP8 down-GEMM kernels (ffn.hip): z and v against the
// forward's weight codes, dh and dx against transposed copies of the codes (a 128x128 block's
// codes and scale serve W and W^T alike), made once per weight set by moe_fp8_transpose_weights.
// The weight-gradient operands are quantized straight into feature-major, 128-padded buffers
// (quant_cols_t) so that both operands of wgrad_fp8 are K-contiguous.
#include "common.h"
#include "fp8.h"
#include "lds.h"
#include "tiles.h"

#ifndef MOE_WGRAD_FP8_LDS
#define MOE_WGRAD_FP8_LDS 1   // 256 x 256 LDS-shared weight-gradient tiles where M and N allow
#endif

namespace moe {

namespace {

template <typename TX> __device__ __forceinline__ float ld1(const TX* p);
template <> __device__ __forceinline__ float ld1<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld1<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// 128x1 tiles over each group's rows, written feature-major. Group g's rows [s, e) own the padded
// columns [poff[g], poff[g + 1]) of the outputs, poff[g + 1] - poff[g] = ceil((e - s) / 128) * 128.
// For the block of rows s + 128 b .. (at most 128) and feature f:
//   scalesT[f][poff[g] / 128 + b] = fl32(amax / 448),
//   codesT[f][poff[g] + 128 b + i] = E4M3(fl32(x[s + 128 b + i][f] / scale))   (0 past the group's rows)
// x row r is src[row_index[r]] when row_index is given (rows outside [0, src_rows) read as 0).
// One workgroup per (padded 128-row block, 64 features): thread (q, f) takes rows 32 q .. 32 q + 31.
template <typename TX>
__global__ __launch_bounds__(256) void quant_cols_t(const int32_t* __restrict__ off, const int32_t* __restrict__ poff,
                                                    int n_groups, int total_rows, const TX* __restrict__ src, int ld,
                                                    int src_rows, const int32_t* __restrict__ row_index,
                                                    uint8_t* __restrict__ codesT, float* __restrict__ scalesT, int Rp) {
  __shared__ float red[4][64];
  const int c0 = blockIdx.x * 128;
  if (c0 >= poff[n_groups]) return;
  const int g = find_group(poff, n_groups, c0);
  int s, e;
  group_rows(off, g, total_rows, s, e);
  const int r0 = s + (c0 - poff[g]);
  const int nr = min(128, e - r0);
  const int fl = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int f = blockIdx.y * 64 + fl;
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int row = 32 * q + i;
    float x = 0.f;
    if (row < nr) {
      const int sr = row_index ? row_index[r0 + row] : r0 + row;
      if (sr >= 0 && sr < src_rows) x = ld1<TX>(src + (size_t)sr * ld + f);
    }
    v[i] = x;
    amax = fmaxf(amax, fabsf(x));
  }
  red[q][fl] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0][fl], red[1][fl]), fmaxf(red[2][fl], red[3][fl]));
  const float scale = amax / 448.0f;
  uint32_t w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float x = v[4 * j + b];
      word |= e4m3_encode(scale == 0.f ? x : x / scale) << (8 * b);
    }
    w[j] = word;
  }
  uint8_t* dst = codesT + (size_t)f * Rp + c0 + 32 * q;
  *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  *reinterpret_cast<uint4*>(dst + 16) = make_uint4(w[4], w[5], w[6], w[7]);
  if (q == 0) scalesT[(size_t)f * (Rp / 128) + blockIdx.x] = scale;
}

// h = SiLU(z) v, dz = dh v SiLU'(z), dv = dh SiLU(z) in fp32, SiLU'(z) = sig (1 + z (1 - sig)).
// z, v, dh, h [rows, I]; dzv [rows, 2I] (dz, then dv).
__global__ __launch_bounds__(256) void swiglu_bwd_f32(const float* __restrict__ Z, const float* __restrict__ V,
                                                      const float* __restrict__ dH, long long rows, int I,
                                                      float* __restrict__ Hf, float* __restrict__ dZV) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * I) return;
  const long long r = i / I;
  const int c = (int)(i % I);
  const float z = Z[i], v = V[i], dh = dH[i];
  const float sig = 1.0f / (1.0f + __expf(-z));
  const float a = z * sig;
  Hf[i] = a * v;
  dZV[r * 2 * I + c] = dh * v * sig * (1.0f + z * (1.0f - sig));
  dZV[r * 2 * I + I + c] = dh * a;
}

constexpr int E8M0_UNIT = 0x7f7f7f7f;   // unit hardware block scale (2^0) in all four bytes

__device__ __forceinline__ i32x8 ldg_fp8x32(const uint8_t* p) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint4 b = *reinterpret_cast<const uint4*>(p + 16);
  return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// Weight gradients: for group g, C_g[m][n] = sum over the group's 128-deep padded blocks kb of
//   mfma(At[m][kb], Bt[n][kb]) * (sA[m][kb] * sB[n][kb])
// At [M, Rp] / Bt [N, Rp] E4M3 feature-major (quant_cols_t), sA [M, Rp/128], sB [N, Rp/128];
// C fp32 [n_groups, M, N]; groups without rows get zeros. A 256-thread workgroup per 128 x 128
// tile of one group; wave (wm, wn) owns 64 x 64 (4 x 4 fragments of 16x16x128 MFMAs) and loads
// its fragments and scales straight from memory (several workgroups per CU hide the latency).
// Stores are non-temporal (the gradients are written once, after every read).
__global__ __launch_bounds__(256) void wgrad_fp8(const int32_t* __restrict__ poff, int n_groups,
                                                 const uint8_t* __restrict__ At, const float* __restrict__ sA,
                                                 const uint8_t* __restrict__ Bt, const float* __restrict__ sB,
                                                 int Rp, int M, int N, float* __restrict__ C) {
  const int mt = M / 128, ntl = N / 128;
  const int w = xcd_item(n_groups * mt * ntl);
  if (w < 0) return;
  const int g = w / (mt * ntl), tm = (w / ntl) % mt, tn = w % ntl;
  const int c0 = poff[g];
  const int nb = (poff[g + 1] - c0) >> 7;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int nsb = Rp >> 7;
  const int kq = (lane >> 4) * 32;
  // this lane's operand rows: A row m0 + 16 f + lane % 16, B row n0 + 16 f + lane % 16; its
  // accumulator rows m0 + 16 f + 4 (lane / 16) + i take the scales of A rows, its column the
  // scale of B row n0 + 16 f + lane % 16
  const int m0 = tm * 128 + wm * 64, n0 = tn * 128 + wn * 64;
  const uint8_t* pa = At + (size_t)(m0 + (lane & 15)) * Rp + c0 + kq;
  const uint8_t* pb = Bt + (size_t)(n0 + (lane & 15)) * Rp + c0 + kq;
  const float* psa = sA + (size_t)(m0 + (lane >> 4) * 4) * nsb + (c0 >> 7);
  const float* psb = sB + (size_t)(n0 + (lane & 15)) * nsb + (c0 >> 7);
  const size_t frag = (size_t)16 * Rp, sfrag = (size_t)16 * nsb;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kb = 0; kb < nb; ++kb) {
    i32x8 a[4], b[4];
    float sa[4][4], sb[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      a[f] = ldg_fp8x32(pa + f * frag + kb * 128);
      b[f] = ldg_fp8x32(pb + f * frag + kb * 128);
      sb[f] = psb[f * sfrag + kb];
#pragma unroll
      for (int i = 0; i < 4; ++i) sa[f][i] = psa[f * sfrag + i * nsb + kb];
    }
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
#pragma unroll
      for (int fn = 0; fn < 4; ++fn) {
        const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[fm], b[fn], f32x4{0.f, 0.f, 0.f, 0.f}, 0,
                                                                        0, 0, E8M0_UNIT, 0, E8M0_UNIT);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[fm][fn][i] = fmaf(p[i], sa[fm][i] * sb[fn], acc[fm][fn][i]);
      }
  }
  float* Cg = C + (size_t)g * M * N;
#pragma unroll
  for (int fm = 0; fm < 4; ++fm)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = tm * 128 + wm * 64 + fm * 16 + (lane >> 4) * 4 + i;
#pragma unroll
      for (int fn = 0; fn < 4; ++fn) {
        const int n = tn * 128 + wn * 64 + fn * 16 + (lane & 15);
        __builtin_nontemporal_store(acc[fm][fn][i], Cg + (size_t)m * N + n);
      }
    }
}

// The same weight gradients with 256 x 256 tiles (M and N multiples of 256) whose operands are
// shared through LDS: per 128-deep block the tile's 256 A rows and 256 B rows (128 bytes each, chunk c
// of row r in slot c ^ (r mod 8), the conflict-free layout of the forward's LDS-tiled kernels) and
// their 512 scales are staged by direct-to-LDS loads, the next block's loads in flight during this
// block's MFMAs. 8 waves: wave (wm = w & 3, wn = w >> 2) owns rows 64 wm .. +64 and columns
// 128 wn .. +128 (4 x 8 fragments). Each wave's row fragments sit behind a (never false) row-count
// branch, which keeps the compiler from front-loading every LDS read and MFMA result of a block and
// running out of registers at two waves per SIMD.
__global__ __launch_bounds__(512) void wgrad_fp8_lds(const int32_t* __restrict__ poff, int n_groups,
                                                     const uint8_t* __restrict__ At, const float* __restrict__ sA,
                                                     const uint8_t* __restrict__ Bt, const float* __restrict__ sB,
                                                     int Rp, int M, int N, float* __restrict__ C) {
  constexpr int TILE = 256 * 128;
  __shared__ __align__(16) uint8_t lA[2][TILE];
  __shared__ __align__(16) uint8_t lB[2][TILE];
  __shared__ __align__(16) float lsA[2][256];
  __shared__ __align__(16) float lsB[2][256];
  const int mt = M / 256, ntl = N / 256;
  const int w = xcd_item(n_groups * mt * ntl);
  if (w < 0) return;
  const int g = w / (mt * ntl), tm = (w / ntl) % mt, tn = w % ntl;
  const int c0 = poff[g];
  const int nb = (poff[g + 1] - c0) >> 7;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 3, wn = wave >> 2;
  const int nsb = Rp >> 7;
  const uint8_t* asrc[4];
  const uint8_t* bsrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = wave * 32 + j * 8 + (lane >> 3);
    const int c = swz(row, lane & 7);
    asrc[j] = At + (size_t)(tm * 256 + row) * Rp + c0 + c * 16;
    bsrc[j] = Bt + (size_t)(tn * 256 + row) * Rp + c0 + c * 16;
  }
  // scales: waves 0..3 stage 64 A rows' each, waves 4..7 64 B rows' each
  const float* ssrc = wave < 4 ? sA + (size_t)(tm * 256 + wave * 64 + lane) * nsb + (c0 >> 7)
                               : sB + (size_t)(tn * 256 + (wave - 4) * 64 + lane) * nsb + (c0 >> 7);
  auto stage = [&](int kb, int b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int base = (wave * 32 + j * 8) * 128;
      dma16(asrc[j] + kb * 128, lA[b] + base);
      dma16(bsrc[j] + kb * 128, lB[b] + base);
    }
    dma4(ssrc + kb, wave < 4 ? lsA[b] + wave * 64 : lsB[b] + (wave - 4) * 64);
  };
  const int nmf = min(4, (M - tm * 256 - wm * 64) >> 4);   // 4: every tile is full
  f32x4 acc[4][8];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int cq = lane >> 4;
  auto frag = [&](const uint8_t* base, int row) {
    const uint4 lo = *reinterpret_cast<const uint4*>(base + row * 128 + swz(row, cq) * 16);
    const uint4 hi = *reinterpret_cast<const uint4*>(base + row * 128 + swz(row, cq + 4) * 16);
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  auto compute = [&](int b) {
    i32x8 a[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) a[m] = frag(lA[b], wm * 64 + m * 16 + (lane & 15));
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      i32x8 bf[4];
      float sb[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int col = wn * 128 + (half * 4 + jj) * 16 + (lane & 15);
        bf[jj] = frag(lB[b], col);
        sb[jj] = lsB[b][col];
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (m < nmf) {
          const f32x4 sa4 = *reinterpret_cast<const f32x4*>(&lsA[b][wm * 64 + m * 16 + cq * 4]);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[m], bf[jj], f32x4{0.f, 0.f, 0.f, 0.f},
                                                                            0, 0, 0, E8M0_UNIT, 0, E8M0_UNIT);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[m][half * 4 + jj][i] = fmaf(p[i], sa4[i] * sb[jj], acc[m][half * 4 + jj][i]);
          }
        }
      }
    }
  };
  if (nb > 0) {
    stage(0, 0);
    wait_dma();
    __syncthreads();
    for (int kb = 0; kb < nb; ++kb) {
      if (kb + 1 < nb) stage(kb + 1, (kb + 1) & 1);
      compute(kb & 1);
      wait_dma();
      __syncthreads();
    }
  }
  float* Cg = C + (size_t)g * M * N;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = tm * 256 + wm * 64 + m * 16 + cq * 4 + i;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int col = tn * 256 + wn * 128 + j * 16 + (lane & 15);
        __builtin_nontemporal_store(acc[m][j][i], Cg + (size_t)row * N + col);
      }
    }
}

// dst[g][c][coff + r] = src[g][r][c] for E4M3 codes src [G, R, C], dst rows of ldd bytes: one
// 64 x 64 tile per workgroup through LDS.
__global__ __launch_bounds__(256) void transpose_codes(const uint8_t* __restrict__ src, int R, int C,
                                                       uint8_t* __restrict__ dst, int ldd, int coff) {
  __shared__ uint8_t tile[64][64 + 4];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64, g = blockIdx.z;
  const uint8_t* s = src + (size_t)g * R * C;
  uint8_t* d = dst + (size_t)g * C * ldd;
  {
    const int j = threadIdx.x >> 2, cc = (threadIdx.x & 3) * 16;
    const uint4 v = *reinterpret_cast<const uint4*>(s + (size_t)(r0 + j) * C + c0 + cc);
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 16; ++k) tile[j][cc + k] = (uint8_t)(wv[k >> 2] >> (8 * (k & 3)));
  }
  __syncthreads();
  {
    const int c = threadIdx.x >> 2, rr = (threadIdx.x & 3) * 16;
    uint32_t wv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 16; ++k) wv[k >> 2] |= (uint32_t)tile[rr + k][c] << (8 * (k & 3));
    *reinterpret_cast<uint4*>(d + (size_t)(c0 + c) * ldd + coff + r0 + rr) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
}

// dst[g][cb][coff + rb] = src[g][rb][cb] for block scales src [G, RB, CB], dst rows of ldd floats
__global__ __launch_bounds__(256) void transpose_scales(const float* __restrict__ src, int G, int RB, int CB,
                                                        float* __restrict__ dst, int ldd, int coff) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)G * RB * CB) return;
  const int g = (int)(i / ((long long)RB * CB)), rb = (int)((i / CB) % RB), cb = (int)(i % CB);
  dst[((size_t)g * CB + cb) * ldd + coff + rb] = src[i];
}

// padded row-block bound: every group's rows rounded up to 128
inline size_t padded_rows(int n_groups, int total_rows) {
  return ((size_t)total_rows + (size_t)128 * n_groups + 127) / 128 * 128;
}

struct Fp8BwdWs {
  size_t prefix, xc, xs, z, v, dyc, dys, dh, h, dzv, dzvc, dzvs, tr, total;
  size_t Rp;
};

Fp8BwdWs fp8_bwd_layout(int n_groups, int total_rows, int H, int I) {
  Fp8BwdWs L{};
  size_t o = 0;
  const size_t rows = (size_t)total_rows;
  L.Rp = padded_rows(n_groups, total_rows);
  L.prefix = o; o += align256((size_t)3 * (n_groups + 1) * sizeof(int32_t));
  L.xc = o; o += align256(rows * H);
  L.xs = o; o += align256(rows * (H / 128) * sizeof(float));
  L.z = o; o += align256(rows * I * sizeof(float));
  L.v = o; o += align256(rows * I * sizeof(float));
  L.dyc = o; o += align256(rows * H);
  L.dys = o; o += align256(rows * (H / 128) * sizeof(float));
  L.dh = o; o += align256(rows * I * sizeof(float));
  L.h = o; o += align256(rows * I * sizeof(float));
  L.dzv = o; o += align256(rows * 2 * I * sizeof(float));
  L.dzvc = o; o += align256(rows * 2 * I);
  L.dzvs = o; o += align256(rows * (2 * I / 128) * sizeof(float));
  // feature-major weight-gradient operands: dy^T, x^T [H, Rp]; h^T, dz^T, dv^T [I, Rp]; codes and scales
  L.tr = o;
  if (total_rows > 0)
    for (int F : {H, H, I, I, I}) o += align256((size_t)F * L.Rp) + align256((size_t)F * (L.Rp / 128) * sizeof(float));
  L.total = o;
  return L;
}

}  // namespace

size_t grouped_ffn_backward_fp8_workspace(int n_groups, int total_rows, int H, int I) {
  return fp8_bwd_layout(n_groups, total_rows, H, I).total;   // the group prefixes even without rows
}

hipError_t launch_fp8_transpose_weights(const Fp8TransposeArgs& a, hipStream_t st) {
  const int G = a.n_groups, H = a.H, I = a.I;
  if (G == 0) return hipSuccess;
  // W_d [G, H, I] -> W_d^T [G, I, H]
  hipLaunchKernelGGL(transpose_codes, dim3(I / 64, H / 64, G), dim3(256), 0, st, a.Wd, H, I, a.WdT, H, 0);
  // W_g, W_u [G, I, H] -> [W_g | W_u]^T [G, H, 2I]
  hipLaunchKernelGGL(transpose_codes, dim3(H / 64, I / 64, G), dim3(256), 0, st, a.Wg, I, H, a.WguT, 2 * I, 0);
  hipLaunchKernelGGL(transpose_codes, dim3(H / 64, I / 64, G), dim3(256), 0, st, a.Wu, I, H, a.WguT, 2 * I, I);
  const long long nd = (long long)G * (H / 128) * (I / 128);
  const unsigned gs = (unsigned)((nd + 255) / 256);
  hipLaunchKernelGGL(transpose_scales, dim3(gs), dim3(256), 0, st, a.Wd_s, G, H / 128, I / 128, a.WdT_s, H / 128, 0);
  hipLaunchKernelGGL(transpose_scales, dim3(gs), dim3(256), 0, st, a.Wg_s, G, I / 128, H / 128, a.WguT_s,
                     2 * I / 128, 0);
  hipLaunchKernelGGL(transpose_scales, dim3(gs), dim3(256), 0, st, a.Wu_s, G, I / 128, H / 128, a.WguT_s,
                     2 * I / 128, I / 128);
  return hipGetLastError();
}

hipError_t launch_grouped_ffn_backward_fp8(const FfnBwdFp8Args& a, hipStream_t st, void* const* ev) {
  const int H = a.H, I = a.I, rows = a.total_rows;
  auto mark = [&](int i) {
    if (ev && ev[i]) (void)hipEventRecord(static_cast<hipEvent_t>(ev[i]), st);
  };
  const Fp8BwdWs L = fp8_bwd_layout(a.n_groups, rows, H, I);
  char* ws = static_cast<char*>(a.ws);
  int32_t* prefix = reinterpret_cast<int32_t*>(ws + L.prefix);
  int32_t* poff = prefix + 2 * (a.n_groups + 1);
  uint8_t* Xc = reinterpret_cast<uint8_t*>(ws + L.xc);
  float* Xs = reinterpret_cast<float*>(ws + L.xs);
  float* Z = reinterpret_cast<float*>(ws + L.z);
  float* V = reinterpret_cast<float*>(ws + L.v);
  uint8_t* dYc = reinterpret_cast<uint8_t*>(ws + L.dyc);
  float* dYs = reinterpret_cast<float*>(ws + L.dys);
  float* dH = reinterpret_cast<float*>(ws + L.dh);
  float* Hf = reinterpret_cast<float*>(ws + L.h);
  float* dZV = reinterpret_cast<float*>(ws + L.dzv);
  uint8_t* dZVc = reinterpret_cast<uint8_t*>(ws + L.dzvc);
  float* dZVs = reinterpret_cast<float*>(ws + L.dzvs);
  const size_t Rp = L.Rp;
  hipError_t e = hipSuccess;
  mark(0);
  if (rows > 0) {
    // z, v: the forward's GEMM operands (u rows gathered and quantized 1x128, the weight codes)
    e = launch_fp8_quant_rows_gather(a.X, MOE_BF16, a.x_rows, rows, H, a.row_index, nullptr, Xc, Xs, st);
    if (e == hipSuccess)
      e = launch_fp8_rows_gemm(a.offsets, a.n_groups, rows, Xc, Xs, a.Wg, a.Wg_s, I, H, Z, prefix, st);
    if (e == hipSuccess)
      e = launch_fp8_rows_gemm(a.offsets, a.n_groups, rows, Xc, Xs, a.Wu, a.Wu_s, I, H, V, prefix, st);
    // dh = Q(dy) Q(W_d): dy 1x128 along H, W_d^T codes
    if (e == hipSuccess) e = launch_fp8_quant(a.dY, MOE_BF16, rows, H, 1, dYc, dYs, st);
    if (e == hipSuccess)
      e = launch_fp8_rows_gemm(a.offsets, a.n_groups, rows, dYc, dYs, a.WdT, a.WdT_s, I, H, dH, prefix, st);
    if (e != hipSuccess) return e;
    const long long n = (long long)rows * I;
    hipLaunchKernelGGL(swiglu_bwd_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, Z, V, dH,
                       (long long)rows, I, Hf, dZV);
    // dx = [Q(dz) Q(dv)] against [W_g | W_u]^T: one GEMM with K = 2I (1x128 tiles never straddle dz / dv)
    e = launch_fp8_quant(dZV, MOE_F32, rows, 2 * I, 1, dZVc, dZVs, st);
    if (e == hipSuccess)
      e = launch_fp8_rows_gemm(a.offsets, a.n_groups, rows, dZVc, dZVs, a.WguT, a.WguT_s, H, 2 * I, a.dX, prefix,
                               st);
    if (e != hipSuccess) return e;
  }
  mark(1);
  mark(2);
  // weight gradients from 128x1-tiled, feature-major operands
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, a.offsets, a.n_groups, rows, 128, 128, poff);
  uint8_t* tc = reinterpret_cast<uint8_t*>(ws + L.tr);
  auto take = [&](int F, uint8_t*& codes, float*& scales) {
    codes = tc;
    tc += align256((size_t)F * Rp);
    scales = reinterpret_cast<float*>(tc);
    tc += align256((size_t)F * (Rp / 128) * sizeof(float));
  };
  uint8_t *dYT = nullptr, *XT = nullptr, *hT = nullptr, *dzT = nullptr, *dvT = nullptr;
  float *dYTs = nullptr, *XTs = nullptr, *hTs = nullptr, *dzTs = nullptr, *dvTs = nullptr;
  if (rows > 0) {   // without rows every group has no blocks: wgrad_fp8 reads nothing and writes zeros
    take(H, dYT, dYTs);
    take(H, XT, XTs);
    take(I, hT, hTs);
    take(I, dzT, dzTs);
    take(I, dvT, dvTs);
  }
  if (rows > 0) {
    const unsigned nblk = (unsigned)(Rp / 128);
    hipLaunchKernelGGL(quant_cols_t<uint16_t>, dim3(nblk, H / 64), dim3(256), 0, st, a.offsets, poff, a.n_groups,
                       rows, static_cast<const uint16_t*>(a.dY), H, rows, static_cast<const int32_t*>(nullptr), dYT,
                       dYTs, (int)Rp);
    hipLaunchKernelGGL(quant_cols_t<uint16_t>, dim3(nblk, H / 64), dim3(256), 0, st, a.offsets, poff, a.n_groups,
                       rows, static_cast<const uint16_t*>(a.X), H, a.x_rows, a.row_index, XT, XTs, (int)Rp);
    hipLaunchKernelGGL(quant_cols_t<float>, dim3(nblk, I / 64), dim3(256), 0, st, a.offsets, poff, a.n_groups, rows,
                       static_cast<const float*>(Hf), I, rows, static_cast<const int32_t*>(nullptr), hT, hTs,
                       (int)Rp);
    hipLaunchKernelGGL(quant_cols_t<float>, dim3(nblk, I / 64), dim3(256), 0, st, a.offsets, poff, a.n_groups, rows,
                       static_cast<const float*>(dZV), 2 * I, rows, static_cast<const int32_t*>(nullptr), dzT, dzTs,
                       (int)Rp);
    hipLaunchKernelGGL(quant_cols_t<float>, dim3(nblk, I / 64), dim3(256), 0, st, a.offsets, poff, a.n_groups, rows,
                       static_cast<const float*>(dZV + I), 2 * I, rows, static_cast<const int32_t*>(nullptr), dvT,
                       dvTs, (int)Rp);
  }
  auto gemm = [&](const uint8_t* At, const float* sA, const uint8_t* Bt, const float* sB, int M, int N, float* C) {
    if (MOE_WGRAD_FP8_LDS && M % 256 == 0 && N % 256 == 0) {
      const long long items = (long long)a.n_groups * (M / 256) * (N / 256);
      hipLaunchKernelGGL(wgrad_fp8_lds, dim3((unsigned)((items + 7) / 8 * 8)), dim3(512), 0, st, poff, a.n_groups, At,
                         sA, Bt, sB, (int)Rp, M, N, C);
      return;
    }
    const long long items = (long long)a.n_groups * (M / 128) * (N / 128);
    hipLaunchKernelGGL(wgrad_fp8, dim3((unsigned)((items + 7) / 8 * 8)), dim3(256), 0, st, poff, a.n_groups, At, sA,
                       Bt, sB, (int)Rp, M, N, C);
  };
  gemm(dYT, dYTs, hT, hTs, H, I, a.dWd);
  gemm(dzT, dzTs, XT, XTs, I, H, a.dWg);
  gemm(dvT, dvTs, XT, XTs, I, H, a.dWu);
  mark(3);
  return hipGetLastError();
}

}  // namespace moe
