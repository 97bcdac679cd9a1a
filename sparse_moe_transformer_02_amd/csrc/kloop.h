// Register-streaming bf16 MFMA K loop shared by the expert GEMMs and the router GEMM.
#pragma once

#include "common.h"

namespace moe {

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// v with every bit cleared when m == 0 (m is 0 or all ones)
__device__ __forceinline__ bf16x8 mask_bf16x8(bf16x8 v, uint32_t m) {
  u32x4 x = __builtin_bit_cast(u32x4, v);
  x &= m;
  return __builtin_bit_cast(bf16x8, x);
}

// K loop shared by the bf16 GEMMs: acc[m][j] += A_m (16 rows) x B_j (16 columns) over K.
// Blocks of U 32-deep steps are double-buffered in registers: the loads of block i+1 are in
// flight while block i's MFMAs run, so each wave keeps U*(RM+NB) to 2*U*(RM+NB) 16-byte loads
// outstanding. Every load is unconditional (the tail re-reads the last block, its data unused)
// so the compiler's wait counts stay exact; A rows past the tile point at a valid row and are
// zeroed with a mask after the load.
template <int RM, int NB, int U>
__device__ __forceinline__ void kloop_bf16(const uint16_t* const (&pa)[RM], const bool (&va)[RM],
                                           const uint16_t* const (&pb)[NB], int K,
                                           f32x4 (&acc)[RM][NB]) {
  uint32_t msk[RM];
#pragma unroll
  for (int m = 0; m < RM; ++m) msk[m] = va[m] ? 0xffffffffu : 0u;
  const int nblk = K / (32 * U);
  auto load = [&](int blk, bf16x8 (&b)[U][NB], bf16x8 (&a)[U][RM]) {
    const int k0 = blk * 32 * U;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < NB; ++j) b[u][j] = ld_bf16x8(pb[j] + k0 + 32 * u);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < RM; ++m) a[u][m] = ld_bf16x8(pa[m] + k0 + 32 * u);
  };
  auto mma = [&](const bf16x8 (&b)[U][NB], const bf16x8 (&a)[U][RM]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < RM; ++m) {
        const bf16x8 am = mask_bf16x8(a[u][m], msk[m]);
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, b[u][j], acc[m][j], 0, 0, 0);
      }
  };
  if (nblk > 0) {
    bf16x8 b0[U][NB], a0[U][RM], b1[U][NB], a1[U][RM];
    load(0, b0, a0);
    for (int blk = 0; blk < nblk; blk += 2) {
      load(min(blk + 1, nblk - 1), b1, a1);
      mma(b0, a0);
      if (blk + 1 >= nblk) break;
      load(min(blk + 2, nblk - 1), b0, a0);
      mma(b1, a1);
    }
  }
  for (int k0 = nblk * 32 * U; k0 < K; k0 += 32) {
    bf16x8 b[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) b[j] = ld_bf16x8(pb[j] + k0);
#pragma unroll
    for (int m = 0; m < RM; ++m) {
      const bf16x8 am = mask_bf16x8(ld_bf16x8(pa[m] + k0), msk[m]);
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, b[j], acc[m][j], 0, 0, 0);
    }
  }
}


}  // namespace moe
