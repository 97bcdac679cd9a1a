// Grouped SwiGLU expert FFN: Y[r] = W_down[g] (SiLU(W_gate[g] x_r) * (W_up[g] x_r)).
//
// The FFN_i terms of the "รายงานเชิงเทคนิคของ DeepSeek-V3" Method §2 h'_t equation (SwiGLU without biases is this
// library's reading; the pages only name FFN_i). Group sizes live on the device: a small kernel
// turns the offsets into a prefix of row tiles per group, and each GEMM workgroup maps its id to
// (row tile, column tile) through that prefix, so the host never learns the counts.
//
// Work items are split into 8 contiguous ranges, one per XCD (workgroup ids are dealt to the
// XCDs round-robin), so the column tiles of one row tile run on one XCD and share its L2.
//
// Paths:
//  * fp32: SIMT dot products, for small fp32 layers.
//  * bf16: v_mfma_f32_16x16x32_bf16. Decode-sized groups (16 rows or fewer on average): the
//    weight-streaming kernels (persistent workgroups, 1 KB / 512 B runs of every weight row staged
//    through LDS) where H and I are multiples of 512, else the register-streaming kernels (each
//    lane streams 16 contiguous bytes of a weight row per 32-deep step into the B operand; a wave
//    owns 16 output columns and 16*RM rows). Larger groups: the LDS-tiled kernels.
//  * fp8 (E4M3FN, "官方揭秘DeepSeek-V3模型训练全流程" §4.3 recipe): v_mfma_scale_f32_16x16x128_f8f6f4 with unit
//    hardware scales; each MFMA covers exactly one 128-deep K block, so its fp32 result is
//    multiplied by the row's 1x128 activation scale and the 128x128 weight-block scale and added
//    to the fp32 accumulator. h is written in fp32, re-quantized per 1x128 tile, then GEMM2.
//    The same three kernel families as bf16.
#include <type_traits>

#include "common.h"
#include "fp8.h"
#include "kloop.h"
#include "lds.h"
#include "tiles.h"

namespace moe {

namespace {

constexpr int DIRECT_GM = 8;   // row tiles per band on the direct (register-streaming) path

__device__ __forceinline__ int x_row(const int32_t* __restrict__ row_index, int r, int r1, int x_rows) {
  if (r >= r1) return -1;
  const int tok = row_index ? row_index[r] : r;
  return (tok >= 0 && tok < x_rows) ? tok : -1;
}

// -------------------------------------------------------------------- fp32 SIMT path
// 16 rows x 16 columns per workgroup, one output per thread.
__global__ __launch_bounds__(256) void ffn1_f32(const int32_t* __restrict__ off,
                                                const int32_t* __restrict__ prefix, int n_groups,
                                                int total_rows, const int32_t* __restrict__ row_index,
                                                const float* __restrict__ X, int x_rows,
                                                const float* __restrict__ Wg,
                                                const float* __restrict__ Wu, int H, int I,
                                                float* __restrict__ Hf) {
  const int n_nt = (I + 15) / 16;
  int nt;
  Tile t;
  if (!find_tile(off, prefix, n_groups, total_rows, 16, n_nt, DIRECT_GM, nt, t)) return;
  const int r = t.r0 + (threadIdx.x >> 4);
  const int n = nt * 16 + (threadIdx.x & 15);
  if (r >= t.r1 || n >= I) return;
  const int tok = x_row(row_index, r, t.r1, x_rows);
  float z = 0.f, v = 0.f;
  if (tok >= 0) {
    const float* x = X + (size_t)tok * H;
    const float* wg = Wg + ((size_t)t.g * I + n) * H;
    const float* wu = Wu + ((size_t)t.g * I + n) * H;
    for (int k = 0; k < H; ++k) { z = fmaf(x[k], wg[k], z); v = fmaf(x[k], wu[k], v); }
  }
  Hf[(size_t)r * I + n] = swiglu(z, v);
}

template <typename TY>
__global__ __launch_bounds__(256) void ffn2_f32(const int32_t* __restrict__ off,
                                                const int32_t* __restrict__ prefix, int n_groups,
                                                int total_rows, const float* __restrict__ Hf,
                                                const float* __restrict__ Wd, int H, int I,
                                                TY* __restrict__ Y) {
  const int n_nt = (H + 15) / 16;
  int nt;
  Tile t;
  if (!find_tile(off, prefix, n_groups, total_rows, 16, n_nt, DIRECT_GM, nt, t)) return;
  const int r = t.r0 + (threadIdx.x >> 4);
  const int n = nt * 16 + (threadIdx.x & 15);
  if (r >= t.r1 || n >= H) return;
  const float* h = Hf + (size_t)r * I;
  const float* wd = Wd + ((size_t)t.g * H + n) * I;
  float y = 0.f;
  for (int k = 0; k < I; ++k) y = fmaf(h[k], wd[k], y);
  Elem<TY>::store(Y, (size_t)r * H + n, y);
}

// -------------------------------------------------------------------- bf16 MFMA path
// GEMM1 + SwiGLU. Workgroup = 4 waves; wave w owns h columns [nt*64 + 16w, +16) for rows
// [r0, r0 + 16*RM). Lane l supplies row / weight-row (l % 16) and k-slice 8*(l / 16) .. +8 of
// each 32-deep step; the accumulator holds rows 4*(l/16)+i, column l % 16.
template <int RM>
__global__ __launch_bounds__(256) void ffn1_bf16(const int32_t* __restrict__ off,
                                                 const int32_t* __restrict__ prefix, int n_groups,
                                                 int total_rows, const int32_t* __restrict__ row_index,
                                                 const uint16_t* __restrict__ X, int x_rows,
                                                 const uint16_t* __restrict__ Wg,
                                                 const uint16_t* __restrict__ Wu, int H, int I,
                                                 uint16_t* __restrict__ Hb, float* __restrict__ ZV) {
  const int n_nt = I / 64;
  int nt;
  Tile t;
  if (!find_tile(off, prefix, n_groups, total_rows, 16 * RM, n_nt, DIRECT_GM, nt, t)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, kq = (lane >> 4) * 8;
  const int n = nt * 64 + wave * 16 + l16;
  const uint16_t* pb[2] = {Wg + ((size_t)t.g * I + n) * H + kq, Wu + ((size_t)t.g * I + n) * H + kq};
  const uint16_t* pa[RM];
  bool va[RM];
#pragma unroll
  for (int m = 0; m < RM; ++m) {
    const int tok = x_row(row_index, t.r0 + m * 16 + l16, t.r1, x_rows);
    va[m] = tok >= 0;
    pa[m] = X + (size_t)(tok >= 0 ? tok : 0) * H + kq;
  }
  f32x4 acc[RM][2];
#pragma unroll
  for (int m = 0; m < RM; ++m) acc[m][0] = acc[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  kloop_bf16<RM, 2, (RM == 1 ? 4 : (RM == 2 ? 3 : 2))>(pa, va, pb, H, acc);
#pragma unroll
  for (int m = 0; m < RM; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = t.r0 + m * 16 + (lane >> 4) * 4 + i;
      if (r >= t.r1) continue;
      Hb[(size_t)r * I + n] = f32_to_bf16(swiglu(acc[m][0][i], acc[m][1][i]));
      if (ZV) {                 // pre-activations z | v for the backward pass
        ZV[(size_t)r * 2 * I + n] = acc[m][0][i];
        ZV[(size_t)r * 2 * I + I + n] = acc[m][1][i];
      }
    }
}

// GEMM2: Y rows [r0, r0+16*RM) x columns [nt*64*RN + wave*16*RN, +16*RN).
template <int RM, int RN, typename TY>
__global__ __launch_bounds__(256) void ffn2_bf16(const int32_t* __restrict__ off,
                                                 const int32_t* __restrict__ prefix, int n_groups,
                                                 int total_rows, const uint16_t* __restrict__ Hb,
                                                 const uint16_t* __restrict__ Wd, int H, int I,
                                                 TY* __restrict__ Y) {
  const int n_nt = H / (64 * RN);
  int nt;
  Tile t;
  if (!find_tile(off, prefix, n_groups, total_rows, 16 * RM, n_nt, DIRECT_GM, nt, t)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, kq = (lane >> 4) * 8;
  const int nb = nt * 64 * RN + wave * 16 * RN;
  const uint16_t* pb[RN];
#pragma unroll
  for (int j = 0; j < RN; ++j) pb[j] = Wd + ((size_t)t.g * H + nb + j * 16 + l16) * I + kq;
  const uint16_t* pa[RM];
  bool va[RM];
#pragma unroll
  for (int m = 0; m < RM; ++m) {
    const int r = t.r0 + m * 16 + l16;
    va[m] = r < t.r1;
    pa[m] = Hb + (size_t)(va[m] ? r : t.r0) * I + kq;
  }
  f32x4 acc[RM][RN];
#pragma unroll
  for (int m = 0; m < RM; ++m)
#pragma unroll
    for (int j = 0; j < RN; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  kloop_bf16<RM, RN, (RM == 1 ? 4 : (RM + RN <= 4 ? 3 : 2))>(pa, va, pb, I, acc);
#pragma unroll
  for (int m = 0; m < RM; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = t.r0 + m * 16 + (lane >> 4) * 4 + i;
      if (r >= t.r1) continue;
#pragma unroll
      for (int j = 0; j < RN; ++j) Elem<TY>::store(Y, (size_t)r * H + nb + j * 16 + l16, acc[m][j][i]);
    }
}

// -------------------------------------------------------------------- weight-streaming bf16 path
// Decode-sized groups (at most 16 rows per row tile) when both K dimensions are multiples of 512:
// every weight byte feeds at most 16 rows, so the GEMM is a stream of weights and runs at the rate
// HBM delivers them. One persistent 256-thread workgroup per CU walks a contiguous range of items
// (the last few of every range are shared out at the end, see run_with_pool).
// An item is a 16-row tile of one group x 64 NF weight rows: in MODE 1 (gate/up + SwiGLU) each
// 16-row MFMA fragment of a wave holds the gate rows and the matching up rows of 8 h columns, in
// MODE 2 (down) 16 rows of W_down. K streams through two LDS buffers in stages of SKB bytes of
// every weight row and every live activation row, one direct-to-LDS load per 1 KB (non-temporal
// when the group has no other row tile), so HBM sees long runs of every weight row, and the next
// stage (possibly of the next item; gate/up: the next two) is in flight while the current one goes
// through the MFMAs.
// The 16-byte chunk c of tile row r lands in slot c ^ (r mod 16), so the fragment reads of 16 rows
// hit every bank once. K is summed in the same 32-deep steps, in the same order, as the
// register-streaming kernels above.
// NF: MFMA column fragments (16 weight rows each) per wave, 64 NF weight rows per item; SKB: bytes
// of each row per stage (1 KB: one row per direct load; 512 B: two rows per load). Measured at
// the decode shape: gate/up (1, 1 KB) and down (2, 512 B), both 64 KB of weights per stage; the
// other pairings were slower, and 32 KB stages far slower.
// NWV: waves per workgroup; waves 0..3 run the MFMAs, all of them issue loads (8 waves with
// load-only waves 4..7 measured within noise of 4)
constexpr int ST1_NF = 1, ST1_SKB = 1024, ST2_NF = 2, ST2_SKB = 512, ST_NWV = 4;
#ifndef STREAM_TAIL
#define STREAM_TAIL 4   // gate/up: items per workgroup range that go to the shared end-of-launch pool
#endif
#ifndef MOE_STREAM_POOL2
#define MOE_STREAM_POOL2 1   // the down GEMM's launch shares its tail items too
#endif
#ifndef MOE_STREAM_LA2
#define MOE_STREAM_LA2 1   // gate/up: two stages in flight (0: one, refilled after the next stage landed)
#endif
template <int MODE, typename TY, int NF, int SKB, int NWV>
__global__ __launch_bounds__(64 * NWV) void ffn_stream_bf16(const int32_t* __restrict__ off,
                                                       const int32_t* __restrict__ prefix, int n_groups,
                                                       int total_rows, const int32_t* __restrict__ row_index,
                                                       const uint16_t* __restrict__ X, int x_rows,
                                                       const uint16_t* __restrict__ W0,
                                                       const uint16_t* __restrict__ W1, int N, int K,
                                                       void* __restrict__ out, float* __restrict__ zv,
                                                       int32_t* __restrict__ pool = nullptr) {
  static_assert(SKB == 1024 || SKB == 512, "1 KB or 512 B of each row per stage");
  constexpr int SK = SKB / 2;                 // bf16 K per stage
  constexpr int KT = SKB / 64;                // 32-deep MFMA steps per stage
  constexpr int CPR = SKB / 16;               // 16-byte chunks of a row per stage
  constexpr int RPL = 1024 / SKB;             // rows per 1 KB direct load
  constexpr int RPW = 16 * NF;                // weight rows per wave
  constexpr int A_BYTES = 16 * SKB, BUF = A_BYTES + 4 * RPW * SKB;
  constexpr int AW = 16 / NWV, BW = 4 * RPW / NWV;   // activation / weight rows each wave loads
  static_assert(MODE != 1 || (RPL == 1 && BW == RPW), "gate/up: one row per load, a fragment's rows per wave");
  __shared__ __align__(16) uint8_t lds[2 * BUF];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lrow = lane / CPR, lchunk = lane % CPR;   // row within a direct load, and chunk slot
  const int n_items = prefix[n_groups];
  const int i0 = (int)((long long)n_items * blockIdx.x / gridDim.x);
  const int i1 = (int)((long long)n_items * (blockIdx.x + 1) / gridDim.x);
  if (i0 >= i1) return;
  const int S = K / SK;

  // source row of tile row r (MODE 1 gathers through row_index), or -1 for a row outside X
  auto src_row = [&](int r) {
    const int tk = MODE == 1 && row_index ? row_index[r] : r;
    return (tk >= 0 && tk < x_rows) ? tk : -1;
  };
  // item -> group g (items [pb, pe) of the group, rows [s, e)), rows [r0, r1) of the item, its
  // first weight row c0, and a bit per tile row that holds data. The row tiles of one column tile
  // are adjacent items, so a group with several row tiles reads each weight tile again from L2.
  // A workgroup's items are consecutive: the group is looked up only when the item leaves it.
  // w0 / w1: this wave's first weight row of the item in W0 / W1 (MODE 1: gate / up rows);
  // asrc[j]: this lane's source of activation load j of the wave (at k = 0), loaded when bit j of
  // alive is set (the load holds a live row); both are fixed per item, so a stage adds only k0
  constexpr int NJA = AW / RPL;
  struct It {
    int g, pb, pe, s, e, r0, r1, c0;
    uint32_t bits, alive;
    bool once;
    const uint16_t* asrc[NJA];
    const uint16_t* w0;
    const uint16_t* w1;
  };
  struct Out {   // what computing and storing an item need
    int r0, r1, c0;
    uint32_t bits;
  };
  auto out_of = [](const It& it) { return Out{it.r0, it.r1, it.c0, it.bits}; };
  auto item = [&](int w, const It* prev) {
    It it;
    if (prev && w < prev->pe) {
      it.g = prev->g; it.pb = prev->pb; it.pe = prev->pe; it.s = prev->s; it.e = prev->e;
    } else {
      it.g = find_group(prefix, n_groups, w);
      it.pb = prefix[it.g];
      it.pe = prefix[it.g + 1];
      group_rows(off, it.g, total_rows, it.s, it.e);
    }
    const int mt = max((it.e - it.s + 15) >> 4, 1);
    const int local = w - it.pb;
    it.r0 = it.s + 16 * (local % mt);
    it.r1 = min(it.e, it.r0 + 16);
    it.c0 = (local / mt) * (MODE == 1 ? 2 * RPW : 4 * RPW);   // h columns (MODE 1) or rows of W_down
    it.once = mt == 1;
    const size_t wrow = (size_t)it.g * N + it.c0 + (MODE == 1 ? (RPW / 2) * wave : BW * wave);
    it.w0 = W0 + wrow * K;
    it.w1 = MODE == 1 ? W1 + wrow * K : nullptr;
    it.bits = 0;
    int vsrc = -1;   // lane l: source row of tile row l % 16 (-1 for none)
    for (int j = 0; j < 16 && it.r0 + j < it.r1; ++j) {
      const int sr = src_row(it.r0 + j);
      if (sr >= 0) it.bits |= 1u << j;
      if ((lane & 15) == j) vsrc = sr;
    }
    // activation rows AW w .. AW w + AW - 1, RPL per load; a lane whose row holds no data re-reads
    // a live row of its load
    it.alive = 0;
#pragma unroll
    for (int j = 0; j < NJA; ++j) {
      const int row0 = AW * wave + j * RPL, row = row0 + lrow;
      it.asrc[j] = X;
      if (it.r0 + row0 >= it.r1 || !((it.bits >> row0) & ((1u << RPL) - 1u))) continue;
      it.alive |= 1u << j;
      auto src_of = [&](int r) {
        if constexpr (MODE == 1 && RPL == 1) return __builtin_amdgcn_readlane(vsrc, r);   // r is uniform
        else return src_row(it.r0 + r);
      };
      int src = ((it.bits >> row) & 1u) ? src_of(row) : -1;
      if (src < 0) src = src_of(row0 + ((it.bits >> row0) & 1u ? 0 : 1));
      it.asrc[j] = X + (size_t)src * K + ((lchunk ^ (row & 15)) << 3);
    }
    return it;
  };
  // all-ones for lanes whose activation row holds data (missing rows multiply as zeros)
  auto row_mask = [&](const Out& it) { return ((it.bits >> (lane & 15)) & 1u) ? 0xffffffffu : 0u; };
  const unsigned lds0 = __builtin_amdgcn_readfirstlane((unsigned)(size_t)MOE_LDS(lds));
  auto issue = [&](const It& it, int s, int b, auto nt) {
    constexpr bool NT = decltype(nt)::value;
    const unsigned la = lds0 + b * BUF, lb = la + A_BYTES;
    const int k0 = s * SK;
#pragma unroll
    for (int j = 0; j < NJA; ++j)
      if ((it.alive >> j) & 1u) dma16_at<false>(it.asrc[j] + k0, la + (AW * wave + j * RPL) * SKB);
    // weight rows BW w .. BW w + BW - 1: a uniform row base plus each lane's byte offset
#pragma unroll
    for (int j = 0; j < BW / RPL; ++j) {
      const int rl = j * RPL;                  // first row of the load, counted from the wave's first
      const int row = BW * wave + rl + lrow;   // tile row of this lane's chunk (row % 16 sets the slot)
      const uint16_t* base;
      unsigned voff = (unsigned)((lchunk ^ (row & 15)) << 4);
      // MODE 1: fragment f of the wave holds the gate rows, then the up rows, of h columns
      // c0 + RPW/2 w + 8 f .. + 8
      if (MODE == 1) {
        base = ((rl & 15) < 8 ? it.w0 : it.w1) + (size_t)(8 * (rl / 16) + (rl & 7)) * K + k0;
      } else {
        base = it.w0 + (size_t)rl * K + k0;
        voff += (unsigned)(lrow * K * 2);
      }
      dma16_sv<NT>(base, voff, lb + (BW * wave + rl) * SKB);
    }
  };
  auto compute = [&](int b, uint32_t amsk, f32x4 (&acc)[NF]) {
    const uint8_t* sa = lds + b * BUF;
    const uint8_t* sb = sa + A_BYTES + RPW * wave * SKB;
    const int r = lane & 15, q = lane >> 4;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const int slot = (4 * t + q) ^ r;
      const bf16x8 av = mask_bf16x8(*reinterpret_cast<const bf16x8*>(sa + r * SKB + slot * 16), amsk);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(sb + (16 * f + r) * SKB + slot * 16);
        acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[f], 0, 0, 0);
      }
    }
  };
  // lane l holds rows 4 (l / 16) + i of the tile, weight row RPW w + 16 f + l % 16
  auto epilogue = [&](const Out& it, const f32x4 (&acc)[NF]) {
    const int col = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = it.r0 + 4 * (lane >> 4) + i;
      if (MODE == 1) {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const float v = __shfl_xor(acc[f][i], 8);    // the up value of this lane's h column
          if (r < it.r1 && col < 8) {
            const int hc = it.c0 + (RPW / 2) * wave + 8 * f + col;
            static_cast<uint16_t*>(out)[(size_t)r * N + hc] = f32_to_bf16(swiglu(acc[f][i], v));
            if (zv) {               // pre-activations z | v for the backward pass
              zv[(size_t)r * 2 * N + hc] = acc[f][i];
              zv[(size_t)r * 2 * N + N + hc] = v;
            }
          }
        }
      } else if (r < it.r1) {
#pragma unroll
        for (int f = 0; f < NF; ++f)
          Elem<TY>::store(static_cast<TY*>(out), (size_t)r * N + it.c0 + RPW * wave + 16 * f + col, acc[f][i]);
      }
    }
  };

  // With a pool counter (zeroed by the tile-prefix launch before this one): the last STREAM_TAIL
  // items of every workgroup's range form a shared pool, claimed one at a time (through the counter,
  // the index passed to the other waves in LDS, free once the ring has drained) by the workgroups
  // that end their own part first, so the last ones end together. run(a0, a1) streams items
  // [a0, a1) and drains the ring.
  auto run_with_pool = [&](auto&& run) {
    const int tail = pool ? min(STREAM_TAIL, i1 - i0) : 0;
    run(i0, i1 - tail);
    if (!pool) return;
    const int G = (int)gridDim.x;
    int* const slot = reinterpret_cast<int*>(lds);
    for (;;) {
      lds_reads_barrier();   // every wave is past its last read of the ring
      if (threadIdx.x == 0) *slot = atomicAdd(pool, 1);
      lds_reads_barrier();   // the claimed index is in LDS
      const int p = __builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile int*>(slot));
      lds_reads_barrier();   // every wave has read it before the ring is refilled
      if (p >= G * STREAM_TAIL) break;
      const int ob = p % G;  // owner workgroup of the claimed item, and its place in the tail
      const int lo = (int)((long long)n_items * ob / G), hi = (int)((long long)n_items * (ob + 1) / G);
      const int w = max(lo, hi - STREAM_TAIL) + p / G;
      if (w < hi) run(w, w + 1);
    }
  };
  constexpr bool LA2 = MOE_STREAM_LA2 && MODE == 1;
  if constexpr (LA2) {
    // Items [a0, a1) with two stages in flight: buffer b is refilled (stage gs + 2) as soon as every
    // wave is done computing stage gs from it, instead of after stage gs + 1 has landed (gate/up
    // 2.22 -> 2.19 ms at the decode shape; the down GEMM's 512-byte stages measured 1.09 -> 1.14 ms
    // with it and keep one stage in flight). The wait at the top lets the loads of stage gs + 1, the
    // youngest memory instructions, stay in flight (their count is exact per wave); a finished
    // item's stores are older, so the wait covers them.
    auto run = [&](int a0, int a1) {
      if (a0 >= a1) return;
      const long long total = (long long)(a1 - a0) * S;
      It ld = item(a0, nullptr);   // item of the next stage to load
      Out cu = out_of(ld);         // item of the stage being computed
      int ld_w = a0, ld_s = 0, cs = 0;
      uint32_t amsk = row_mask(cu);
      f32x4 acc[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
      Out q0 = cu, q1 = cu;        // item and load count of the stage in each buffer
      int n0 = 0, n1 = 0;
      auto load_next = [&](int b) {
        if (ld.once) issue(ld, ld_s, b, std::true_type{});
        else issue(ld, ld_s, b, std::false_type{});
        const int n = BW / RPL + __builtin_popcount(ld.alive);   // direct loads this wave just issued
        if (b) { q1 = out_of(ld); n1 = n; }
        else { q0 = out_of(ld); n0 = n; }
        if (++ld_s == S) {
          ld_s = 0;
          if (++ld_w < a1) ld = item(ld_w, &ld);
        }
      };
      f32x4 done[NF];
      Out done_it = cu;
      bool pending = false;
      load_next(0);
      if (total > 1) load_next(1);
      for (long long gs = 0; gs < total; ++gs) {
        const int b = (int)(gs & 1);
        if (gs + 1 < total) wait_vm_n_barrier<BW / RPL, BW / RPL + NJA>(b ? n0 : n1);
        else wait_dma_keep_barrier<0>();
        if (pending) {
          if (wave < 4) epilogue(done_it, done);
          pending = false;
        }
        if (wave < 4) compute(b, amsk, acc);
        if (++cs == S) {
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            done[f] = acc[f];
            acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
          done_it = cu;
          pending = true;
          cs = 0;
          cu = b ? q0 : q1;      // stage gs + 1 starts the next item
          amsk = row_mask(cu);
        }
        if (gs + 2 < total) {
          lds_reads_barrier();   // every wave is done reading buffer b
          load_next(b);
        }
      }
      if (pending && wave < 4) epilogue(done_it, done);
    };
    run_with_pool(run);
    return;
  }
  // one stage in flight
  auto run = [&](int a0, int a1) {
    if (a0 >= a1) return;
    const long long total = (long long)(a1 - a0) * S;
    It ld = item(a0, nullptr);   // item of the next stage to load
    Out cu = out_of(ld);         // item of the stage being computed
    Out issued = cu;             // item of the stage last loaded
    int ld_w = a0, ld_s = 0, cs = 0;
    uint32_t amsk = row_mask(cu);
    f32x4 acc[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto load_next = [&](int b) {
      if (ld.once) issue(ld, ld_s, b, std::true_type{});
      else issue(ld, ld_s, b, std::false_type{});
      issued = out_of(ld);
      if (++ld_s == S) {
        ld_s = 0;
        if (++ld_w < a1) ld = item(ld_w, &ld);
      }
    };
    f32x4 done[NF];
    Out done_it = cu;
    bool pending = false;
    // a finished item's results are stored after the next stage's loads have been issued: the wait at
    // the top of each iteration then covers the stores together with those loads instead of after them
    load_next(0);
    for (long long gs = 0; gs < total; ++gs) {
      // this wave's loads of stage gs landed; after the barrier everyone's have, and every wave is
      // done reading the other buffer
      wait_dma_keep_barrier<0>();
      if (gs + 1 < total) load_next((int)((gs + 1) & 1));
      if (pending) {
        if (wave < 4) epilogue(done_it, done);
        pending = false;
      }
      if (wave < 4) compute((int)(gs & 1), amsk, acc);
      if (++cs == S) {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          done[f] = acc[f];
          acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        done_it = cu;
        pending = true;
        cs = 0;
        cu = issued;             // stage gs + 1, just loaded, starts the next item
        amsk = row_mask(cu);
      }
    }
    if (pending && wave < 4) epilogue(done_it, done);
  };
  run_with_pool(run);
}

// -------------------------------------------------------------------- LDS-tiled bf16 path
// For groups with many rows (prefill): 256 x 256 or 128 x 512 tiles (activation rows x weight
// rows), 8 waves each computing 64 rows x 128 columns with v_mfma_f32_16x16x32_bf16 (4 x 8
// fragments). K is staged through a ring of NBUF LDS buffers, filled by direct global->LDS
// loads (global_load_lds_dwordx4 from inline asm, which the compiler does not track: lane l's 16
// bytes land at base + 16*l) issued NBUF-1 stages ahead; every wave issues the same number of
// loads per stage, so waiting for "all but the last NBUF-2 stages" is an exact vmcnt.
// A tile row holds RB bytes = CH chunks of 16 bytes; chunk c of row r sits in slot c ^ (r % CH).
// With that layout the 16-row fragment reads (ds_read_b128) show no LDS bank conflicts on gfx950
// (SQ_LDS_BANK_CONFLICT = 0 in a micro-benchmark; an unswizzled tile takes 3x longer).
// For the gate/up GEMM each 128-row block of the B tile is 64 gate rows followed by the 64 up
// rows of the same h columns, so every wave ends with gate and up of the same columns in one
// lane and applies SwiGLU in registers.
// Measured on MI355X: a plain stream of 64 KB global->LDS blocks per CU reaches about 6.2 TB/s
// from HBM (the practical ceiling; a device copy reaches less), and 26-34 TB/s from L2.
#ifndef MOE_LDS_RB
#define MOE_LDS_RB 128   // bytes per tile row per stage (128: 64-deep bf16 stages, 64: 32-deep)
#endif
#ifndef MOE_LDS_NBUF
#define MOE_LDS_NBUF 2   // LDS ring depth (NBUF * 640 * RB bytes <= 160 KB for 128 x 512 tiles)
#endif

#ifndef MOE_LDS_WM
#define MOE_LDS_WM 0     // tile shape where H % 512 == 0 and I % 256 == 0: 0 = mixed per group, 2 = 128 x 512
#endif

#ifndef MOE_LDS_GM
#define MOE_LDS_GM 8     // row tiles per band: they run side by side and share weight tiles in L2
#endif

constexpr int LB_M = 256;          // rows per tile
constexpr int LB_TILE = 256 * 128; // bytes of one 128-byte-row operand tile (fp8 path)

struct Item {
  int g, nt, r0, r1;
};

// MODE 1: gate/up GEMM + SwiGLU, out = h [rows, N = I] bf16 (W0 = W_gate, W1 = W_up)
// MODE 2: down GEMM, out = Y [rows, N = H] in TY (W0 = W_down)
// MODE 3: the gate/up GEMM of MODE 1 without SwiGLU: out = [z | v] [rows, 2N] fp32 (the
//         pre-activations the backward pass differentiates through)
// MODE 4: out[r][n] = sum_k X[r][k] B(k, n) in fp32 [rows, N], with B stored K-major by rows of
//         n: B(k, n) = (k < split ? W0[g][k][n] : W1[g][k - split][n]) (the backward's dh = dy W_d
//         and dx = dz W_g + dv W_u). A stage of B is 64 k-rows of the tile's 512 n, one 1 KB
//         direct load each, with 16-byte chunk c of k-row q stored at slot c ^ bmn_swz(q); the
//         MFMA B fragments (8 consecutive k of one n per lane) come out of it through transposing
//         LDS reads (ds_read_b64_tr_b16), two per fragment.
// WM waves along M, 8 / WM along N, each wave 64 rows x 128 weight rows:
//   WM = 2: 128-row x 512-weight-row tiles (MODE 4 always; a group's tail of <= 128 rows in the
//           mixed launch).
//   WM = 4: 256-row x 256-weight-row tiles (the mixed launch's whole 256-row tiles; every tile
//           where H % 512 != 0 or I % 256 != 0, with H % 256 == 0 and I % 128 == 0).
//   WM = 0: the mixed launch (kernel below), used whenever H % 512 == 0 and I % 256 == 0.
typedef short i16x4 __attribute__((ext_vector_type(4)));

// LDS slot swizzle of the 16-byte chunks of an MN-major B stage row (k-row q of 64): spreads the
// 16 k-rows x 32 bytes of one transposing fragment read over all banks (2 accesses per bank with
// 64 banks, 4 with 32: the minimum for 512 bytes)
__device__ __forceinline__ int bmn_swz(int q) { return ((q & 3) << 1) | (((q >> 3) & 3) << 3); }

// B fragment (columns ncol0 .. +16, k = 32 ks + 8 (lane / 16) .. +8 per lane) of an MN-major stage
// (64 k-rows of 1 KB). ds_read_b64_tr_b16 on a 16-lane group: lane i receives element i % 4 of the
// 8 bytes addressed by lanes 4q + i / 4, q = 0..3, as its element q; so lane 16 G + s addresses k-row
// 32 ks + 8 G + 4 h + s / 4, columns ncol0 + 4 (s % 4) .. +4, and ends with k = 8 G + 4 h + q of
// column ncol0 + s (h = 0, 1: the two halves of the fragment).
__device__ __forceinline__ bf16x8 ld_b_mn(const uint8_t* sb, int ks, int ncol0, int lane) {
  const int G = lane >> 4, sl = lane & 15;
  const int c = (ncol0 >> 3) + ((sl & 3) >> 1);
  i16x4 v[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = ks * 32 + 8 * G + 4 * h + (sl >> 2);
    const uint8_t* p = sb + q * 1024 + ((c ^ bmn_swz(q)) << 4) + ((sl & 1) << 3);
    v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  }
  const i16x4 lo = v[0], hi = v[1];
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, w);
}

// One tile (item `it`: group, column tile, rows) of the LDS-tiled GEMM; `lds` holds NBUF ring
// buffers of (BM + BW) * RB bytes, activation tile first. NTW: the weight tiles are loaded
// non-temporally (the group's only row tile: no other workgroup stages them, and such loads
// stream from HBM faster); a group's several row tiles share them through L2 instead. The MN-major
// weight stages of MODE 4 measured slower that way and keep plain loads.
template <int MODE, typename TY, int RB, int NBUF, int WM, int NW, bool NTW>
__device__ __forceinline__ void lds_tile(const Item& it, const int32_t* __restrict__ row_index,
                                         const uint16_t* __restrict__ X, int x_rows,
                                         const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1,
                                         int N, int K, void* __restrict__ out, int split, float* __restrict__ zv,
                                         uint8_t* lds) {
  constexpr int WN = NW / WM;
  constexpr bool NTB = NTW && MODE != 4;
  constexpr int BM = 64 * WM;            // activation rows per tile
  constexpr int BW = 128 * WN;           // weight rows per tile
  constexpr int CH = RB / 16;            // 16-byte chunks per tile row
  constexpr int BK = RB / 2;             // bf16 K per stage
  constexpr int KS = BK / 32;            // MFMA k-steps per stage
  constexpr int TA = BM * RB, TB = BW * RB;
  constexpr int RPI = 1024 / RB;         // tile rows per 1 KB wave load
  constexpr int AR = BM / NW, BR = BW / NW;   // tile rows each wave loads
  constexpr int NJA = AR / RPI, NJB = BR / RPI;
  constexpr int DMA_PER_STAGE = NJA + NJB;
  static_assert(NJA * RPI == AR && NJB * RPI == BR, "tile rows per wave must be whole loads");
  auto bufA = [&](int b) -> uint8_t* { return lds + b * (TA + TB); };
  auto bufB = [&](int b) -> uint8_t* { return lds + b * (TA + TB) + TA; };

  constexpr bool GU = MODE == 1 || MODE == 3;   // gate/up operands (gathered rows, paired weight rows)
  constexpr bool BMN = MODE == 4;               // B stored MN-major, read through transposing loads
  static_assert(!BMN || (BW == 512 && RB == 128 && NJB == 8 && NW == 8), "MN-major B: 64 k-rows of 1 KB, 8 per wave");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar branches below
  const int rows = it.r1 - it.r0;

  // direct-load sources: wave w fills activation rows [AR w, AR w + AR) and weight rows
  // [BR w, BR w + BR), RPI rows per load
  const uint16_t* asrc[NJA];
  const uint16_t* bsrc[NJB];
  const int tok0 = GU ? (row_index ? row_index[it.r0] : it.r0) : it.r0;
  const int tok_first = (tok0 >= 0 && tok0 < x_rows) ? tok0 : 0;
#pragma unroll
  for (int j = 0; j < NJA; ++j) {
    const int row = wave * AR + j * RPI + lane / CH;
    const int c = (lane % CH) ^ swz_ch<CH>(row);   // logical chunk that belongs in this slot
    const int r = it.r0 + row;
    int src = tok_first;                           // rows past the tile re-read a valid row
    if (r < it.r1) {
      const int tk = GU && row_index ? row_index[r] : r;
      src = (tk >= 0 && tk < x_rows) ? tk : tok_first;
    }
    asrc[j] = X + (size_t)src * K + c * 8;
  }
  int boff[BMN ? NJB : 1];   // MN-major: offset of this lane's chunk inside a stage's k-rows
#pragma unroll
  for (int j = 0; j < NJB; ++j) {
    const int row = wave * BR + j * RPI + lane / CH;
    const int c = (lane % CH) ^ swz_ch<CH>(row);
    if (BMN) {
      const int q = wave * NJB + j;              // k-row of the stage; lane = slot of its 64 chunks
      boff[j] = q * N + it.nt * BW + ((lane ^ bmn_swz(q)) << 3);
      bsrc[j] = nullptr;
    } else if (GU) {
      // each 128-row block: 64 gate rows, then the 64 up rows of the same h columns
      const int q = row >> 7, w = row & 127;
      const int hcol = it.nt * (BW / 2) + q * 64 + (w & 63);
      bsrc[j] = (w < 64 ? W0 : W1) + ((size_t)it.g * N + hcol) * K + c * 8;
    } else {
      bsrc[j] = W0 + ((size_t)it.g * N + it.nt * BW + row) * K + c * 8;
    }
  }
  auto stage = [&](int k0, uint8_t* sa, uint8_t* sb) {
#pragma unroll
    for (int j = 0; j < NJA; ++j) dma16(asrc[j] + k0, sa + (wave * AR + j * RPI) * RB);
    if (BMN) {   // a stage never straddles split (both are multiples of 64)
      const uint16_t* wb = k0 < split ? W0 + ((size_t)it.g * split + k0) * N
                                      : W1 + ((size_t)it.g * (K - split) + (k0 - split)) * N;
#pragma unroll
      for (int j = 0; j < NJB; ++j) {
        if (NTB) dma16_nt(wb + boff[BMN ? j : 0], sb + (wave * NJB + j) * 1024);
        else dma16(wb + boff[BMN ? j : 0], sb + (wave * NJB + j) * 1024);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NJB; ++j) {
        if (NTB) dma16_nt(bsrc[j] + k0, sb + (wave * BR + j * RPI) * RB);
        else dma16(bsrc[j] + k0, sb + (wave * BR + j * RPI) * RB);
      }
    }
  };

  const int wm = wave % WM, wn = wave / WM;
  const int nmf = max(0, min(4, (rows - wm * 64 + 15) >> 4));   // row fragments with data
  f32x4 acc[4][8];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragments of k-step ks: the next k-step's LDS reads are issued before this one's MFMAs
  auto load_frags = [&](const uint8_t* sa, const uint8_t* sb, int ks, bf16x8 (&a)[4], bf16x8 (&b)[8]) {
    const int c = ks * 4 + (lane >> 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (BMN) {
        b[j] = ld_b_mn(sb, ks, wn * 128 + j * 16, lane);
      } else {
        const int row = wn * 128 + j * 16 + (lane & 15);
        b[j] = *reinterpret_cast<const bf16x8*>(sb + row * RB + (c ^ swz_ch<CH>(row)) * 16);
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int row = wm * 64 + m * 16 + (lane & 15);
      a[m] = *reinterpret_cast<const bf16x8*>(sa + row * RB + (c ^ swz_ch<CH>(row)) * 16);
    }
  };
  auto mma = [&](const bf16x8 (&a)[4], const bf16x8 (&b)[8]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m < nmf) {   // row fragments past the tile hold stale data: skip their MFMAs
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], b[j], acc[m][j], 0, 0, 0);
      }
    }
  };
  auto compute = [&](const uint8_t* sa, const uint8_t* sb) {
    bf16x8 a0[4], b0[8], a1[4], b1[8];
    load_frags(sa, sb, 0, a0, b0);
#pragma unroll
    for (int ks = 0; ks < KS; ks += 2) {
      if (ks + 1 < KS) load_frags(sa, sb, ks + 1, a1, b1);
      mma(a0, b0);
      if (ks + 1 >= KS) break;
      if (ks + 2 < KS) load_frags(sa, sb, ks + 2, a0, b0);
      mma(a1, b1);
    }
  };

  const int nk = K / BK;
  // prologue: stages 0 .. NBUF-2 (clamped: the tail re-reads the last stage into a free buffer)
#pragma unroll
  for (int b = 0; b < NBUF - 1; ++b) stage(min(b, nk - 1) * BK, bufA(b), bufB(b));
  for (int kt0 = 0; kt0 < nk; kt0 += NBUF) {
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      const int kt = kt0 + b;
      if (kt >= nk) break;
      // this wave's loads of stage kt landed; after the barrier everyone's have, and every wave is
      // done reading the buffer of stage kt-1
      wait_dma_keep_barrier<DMA_PER_STAGE * (NBUF - 2)>();
      const int nb = (b + NBUF - 1) % NBUF;           // the buffer stage kt-1 used
      stage(min(kt + NBUF - 1, nk - 1) * BK, bufA(nb), bufB(nb));
      compute(bufA(b), bufB(b));
    }
  }

#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (m >= nmf) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = it.r0 + wm * 64 + m * 16 + (lane >> 4) * 4 + i;
      if (r >= it.r1) continue;
      if (MODE == 1) {
        uint16_t* Hb = static_cast<uint16_t*>(out);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = it.nt * (BW / 2) + wn * 64 + j * 16 + (lane & 15);
          Hb[(size_t)r * N + col] = f32_to_bf16(swiglu(acc[m][j][i], acc[m][j + 4][i]));
          if (zv) {             // pre-activations z | v for the backward pass
            zv[(size_t)r * 2 * N + col] = acc[m][j][i];
            zv[(size_t)r * 2 * N + N + col] = acc[m][j + 4][i];
          }
        }
      } else if (MODE == 3) {
        float* ZV = static_cast<float*>(out);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = it.nt * (BW / 2) + wn * 64 + j * 16 + (lane & 15);
          ZV[(size_t)r * 2 * N + col] = acc[m][j][i];
          ZV[(size_t)r * 2 * N + N + col] = acc[m][j + 4][i];
        }
      } else {
        TY* Y = static_cast<TY*>(out);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int col = it.nt * BW + wn * 128 + j * 16 + (lane & 15);
          Elem<TY>::store(Y, (size_t)r * N + col, acc[m][j][i]);
        }
      }
    }
  }
}

// The LDS-tiled GEMM kernel. WM = 2 or 4: every tile has that shape. WM = 0 (mixed): groups are
// cut into 256-row x 256-weight-row tiles (WM = 4 shape) and a tail of at most 128 rows becomes
// one 128-row x 512-weight-row tile (WM = 2 shape). Group sizes sit just above 128 at prefill,
// where 128-row tiles alone would give half the experts a second tile of a few rows that stages
// every weight tile again; per 256 rows the 256 x 256 shape also stages a fifth fewer bytes.
template <int MODE, typename TY, int RB, int NBUF, int WM, int NW>
__global__ __launch_bounds__(NW * 64) void ffn_lds_bf16(const int32_t* __restrict__ off,
                                                    const int32_t* __restrict__ prefix, int n_groups,
                                                    int total_rows, const int32_t* __restrict__ row_index,
                                                    const uint16_t* __restrict__ X, int x_rows,
                                                    const uint16_t* __restrict__ W0,
                                                    const uint16_t* __restrict__ W1, int N, int K,
                                                    void* __restrict__ out, int split = 0,
                                                    float* __restrict__ zv = nullptr) {
  constexpr bool GU = MODE == 1 || MODE == 3;
  constexpr int ROWS = WM == 4 ? 512 : 640;   // tile rows (activation + weight) per ring buffer
  __shared__ __align__(16) uint8_t lds[NBUF * ROWS * RB];
  Item it;
  Tile t;
  if constexpr (WM != 0) {
    constexpr int BW = 128 * (NW / WM);
    if (!find_tile(off, prefix, n_groups, total_rows, 64 * WM, GU ? N / (BW / 2) : N / BW, MOE_LDS_GM, it.nt, t))
      return;
    it.g = t.g;
    it.r0 = t.r0;
    it.r1 = t.r1;
    if (MODE != 4 && __builtin_amdgcn_readfirstlane((int)t.once))
      lds_tile<MODE, TY, RB, NBUF, WM, NW, MODE != 4>(it, row_index, X, x_rows, W0, W1, N, K, out, split, zv, lds);
    else
      lds_tile<MODE, TY, RB, NBUF, WM, NW, false>(it, row_index, X, x_rows, W0, W1, N, K, out, split, zv, lds);
  } else {
    static_assert(MODE != 4, "MN-major B tiles are 128 x 512 only");
    int big;
    if (!find_tile_mixed(off, prefix, n_groups, total_rows, GU ? N / 256 : N / 512, GU ? N / 128 : N / 256,
                         MOE_LDS_GM, it.nt, t, big))
      return;
    it.g = t.g;
    it.r0 = t.r0;
    it.r1 = t.r1;
    if (big) {
      if (__builtin_amdgcn_readfirstlane((int)t.once)) lds_tile<MODE, TY, RB, NBUF, 4, NW, true>(it, row_index, X, x_rows, W0, W1, N, K, out, split, zv, lds);
      else lds_tile<MODE, TY, RB, NBUF, 4, NW, false>(it, row_index, X, x_rows, W0, W1, N, K, out, split, zv, lds);
    } else {
      if (__builtin_amdgcn_readfirstlane((int)t.once)) lds_tile<MODE, TY, RB, NBUF, 2, NW, true>(it, row_index, X, x_rows, W0, W1, N, K, out, split, zv, lds);
      else lds_tile<MODE, TY, RB, NBUF, 2, NW, false>(it, row_index, X, x_rows, W0, W1, N, K, out, split, zv, lds);
    }
  }
}

// -------------------------------------------------------------------- fp8 MFMA path
constexpr int E8M0_ONE = 0x7f7f7f7f;   // unit hardware block scale (2^0) in all four bytes

__device__ __forceinline__ i32x8 ld_fp8x32(const uint8_t* p) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint4 b = *reinterpret_cast<const uint4*>(p + 16);
  return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

__device__ __forceinline__ f32x4 mfma_fp8_block(const i32x8& a, const i32x8& b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                         E8M0_ONE, 0, E8M0_ONE);
}

__device__ __forceinline__ i32x8 mask_i32x8(i32x8 v, uint32_t m) { return v & (int)m; }

// K loop shared by the fp8 GEMMs, one 128-deep block per step:
//   acc[m][j][i] += mfma(A_m, B_j)[i] * (sa[m][i] * sw[j])
// sa[m][i]: 1x128 activation scale of accumulator row i of row-block m (psa pointers, zero
// for rows past the tile); sw[j]: the 128x128 weight-block scale of column group j (pws).
// Blocks of U steps are double-buffered in registers like the bf16 loop.
template <int RM, int NB, int U>
__device__ __forceinline__ void kloop_fp8(const uint8_t* const (&pa)[RM], const bool (&va)[RM],
                                          const float* const (&psa)[RM][4], const uint32_t (&sam)[RM][4],
                                          const uint8_t* const (&pb)[NB], const float* const (&pws)[NB],
                                          int nkb, f32x4 (&acc)[RM][NB]) {
  uint32_t msk[RM];
#pragma unroll
  for (int m = 0; m < RM; ++m) msk[m] = va[m] ? 0xffffffffu : 0u;
  struct Stage {
    i32x8 a[U][RM], b[U][NB];
    float sa[U][RM][4], sw[U][NB];
  };
  const int nblk = nkb / U;
  auto load = [&](int kb0, Stage& st) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = kb0 + u;
#pragma unroll
      for (int j = 0; j < NB; ++j) { st.b[u][j] = ld_fp8x32(pb[j] + kb * 128); st.sw[u][j] = pws[j][kb]; }
#pragma unroll
      for (int m = 0; m < RM; ++m) {
        st.a[u][m] = ld_fp8x32(pa[m] + kb * 128);
#pragma unroll
        for (int i = 0; i < 4; ++i) st.sa[u][m][i] = psa[m][i][kb];
      }
    }
  };
  auto mma = [&](const Stage& st) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < RM; ++m) {
        const i32x8 am = mask_i32x8(st.a[u][m], msk[m]);
        float sa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[i] = __uint_as_float(__float_as_uint(st.sa[u][m][i]) & sam[m][i]);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const f32x4 p = mfma_fp8_block(am, st.b[u][j]);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[m][j][i] = fmaf(p[i], sa[i] * st.sw[u][j], acc[m][j][i]);
        }
      }
  };
  if (nblk > 0) {
    Stage s0, s1;
    load(0, s0);
    for (int blk = 0; blk < nblk; blk += 2) {
      load(min(blk + 1, nblk - 1) * U, s1);
      mma(s0);
      if (blk + 1 >= nblk) break;
      load(min(blk + 2, nblk - 1) * U, s0);
      mma(s1);
    }
  }
  for (int kb = nblk * U; kb < nkb; ++kb) {
    Stage st;
#pragma unroll
    for (int j = 0; j < NB; ++j) { st.b[0][j] = ld_fp8x32(pb[j] + kb * 128); st.sw[0][j] = pws[j][kb]; }
#pragma unroll
    for (int m = 0; m < RM; ++m) {
      st.a[0][m] = ld_fp8x32(pa[m] + kb * 128);
#pragma unroll
      for (int i = 0; i < 4; ++i) st.sa[0][m][i] = psa[m][i][kb];
    }
#pragma unroll
    for (int m = 0; m < RM; ++m) {
      const i32x8 am = mask_i32x8(st.a[0][m], msk[m]);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const f32x4 p = mfma_fp8_block(am, st.b[0][j]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sa = __uint_as_float(__float_as_uint(st.sa[0][m][i]) & sam[m][i]);
          acc[m][j][i] = fmaf(p[i], sa * st.sw[0][j], acc[m][j][i]);
        }
      }
    }
  }
}

// GEMM1 + SwiGLU in fp8. Lane l supplies row / weight-row l % 16 and the 32 codes
// 32*(l/16) .. +32 of each 128-deep block; rows of the accumulator are 4*(l/16)+i.
template <int RM>
__global__ __launch_bounds__(256) void ffn1_fp8(const int32_t* __restrict__ off,
                                                const int32_t* __restrict__ prefix, int n_groups,
                                                int total_rows, const int32_t* __restrict__ row_index,
                                                const uint8_t* __restrict__ X,
                                                const float* __restrict__ Xs, int x_rows,
                                                const uint8_t* __restrict__ Wg,
                                                const uint8_t* __restrict__ Wu,
                                                const float* __restrict__ Wgs,
                                                const float* __restrict__ Wus, int H, int I,
                                                float* __restrict__ Hf) {
  const int n_nt = I / 64;
  int nt;
  Tile t;
  if (!find_tile(off, prefix, n_groups, total_rows, 16 * RM, n_nt, DIRECT_GM, nt, t)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, kq = (lane >> 4) * 32;
  const int nkb = H / 128;
  const int n = nt * 64 + wave * 16 + l16;
  const uint8_t* pb[2] = {Wg + ((size_t)t.g * I + n) * H + kq, Wu + ((size_t)t.g * I + n) * H + kq};
  const size_t wsrow = ((size_t)t.g * (I / 128) + (nt * 64 + wave * 16) / 128) * nkb;
  const float* pws[2] = {Wgs + wsrow, Wus + wsrow};
  const uint8_t* pa[RM];
  bool va[RM];
  const float* psa[RM][4];
  uint32_t sam[RM][4];
#pragma unroll
  for (int m = 0; m < RM; ++m) {
    const int tok = x_row(row_index, t.r0 + m * 16 + l16, t.r1, x_rows);
    va[m] = tok >= 0;
    pa[m] = X + (size_t)(tok >= 0 ? tok : 0) * H + kq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tk = x_row(row_index, t.r0 + m * 16 + (lane >> 4) * 4 + i, t.r1, x_rows);
      psa[m][i] = Xs + (size_t)(tk >= 0 ? tk : 0) * nkb;
      sam[m][i] = tk >= 0 ? 0xffffffffu : 0u;
    }
  }
  f32x4 acc[RM][2];
#pragma unroll
  for (int m = 0; m < RM; ++m) acc[m][0] = acc[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  kloop_fp8<RM, 2, (RM == 1 ? 2 : 1)>(pa, va, psa, sam, pb, pws, nkb, acc);
#pragma unroll
  for (int m = 0; m < RM; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = t.r0 + m * 16 + (lane >> 4) * 4 + i;
      if (r < t.r1) Hf[(size_t)r * I + n] = swiglu(acc[m][0][i], acc[m][1][i]);
    }
}

template <int RM, int RN, typename TY>
__global__ __launch_bounds__(256) void ffn2_fp8(const int32_t* __restrict__ off,
                                                const int32_t* __restrict__ prefix, int n_groups,
                                                int total_rows, const uint8_t* __restrict__ Hc,
                                                const float* __restrict__ Hs,
                                                const uint8_t* __restrict__ Wd,
                                                const float* __restrict__ Wds, int H, int I,
                                                TY* __restrict__ Y) {
  const int n_nt = H / (64 * RN);
  int nt;
  Tile t;
  if (!find_tile(off, prefix, n_groups, total_rows, 16 * RM, n_nt, DIRECT_GM, nt, t)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, kq = (lane >> 4) * 32;
  const int nkb = I / 128;
  const int nb = nt * 64 * RN + wave * 16 * RN;
  const uint8_t* pb[RN];
  const float* pws[RN];
#pragma unroll
  for (int j = 0; j < RN; ++j) {
    pb[j] = Wd + ((size_t)t.g * H + nb + j * 16 + l16) * I + kq;
    pws[j] = Wds + ((size_t)t.g * (H / 128) + (nb + j * 16) / 128) * nkb;
  }
  const uint8_t* pa[RM];
  bool va[RM];
  const float* psa[RM][4];
  uint32_t sam[RM][4];
#pragma unroll
  for (int m = 0; m < RM; ++m) {
    const int r = t.r0 + m * 16 + l16;
    va[m] = r < t.r1;
    pa[m] = Hc + (size_t)(va[m] ? r : t.r0) * I + kq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ro = t.r0 + m * 16 + (lane >> 4) * 4 + i;
      psa[m][i] = Hs + (size_t)(ro < t.r1 ? ro : t.r0) * nkb;
      sam[m][i] = ro < t.r1 ? 0xffffffffu : 0u;
    }
  }
  f32x4 acc[RM][RN];
#pragma unroll
  for (int m = 0; m < RM; ++m)
#pragma unroll
    for (int j = 0; j < RN; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  kloop_fp8<RM, RN, (RM + RN <= 2 ? 2 : 1)>(pa, va, psa, sam, pb, pws, nkb, acc);
#pragma unroll
  for (int m = 0; m < RM; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = t.r0 + m * 16 + (lane >> 4) * 4 + i;
      if (r >= t.r1) continue;
#pragma unroll
      for (int j = 0; j < RN; ++j) Elem<TY>::store(Y, (size_t)r * H + nb + j * 16 + l16, acc[m][j][i]);
    }
}

// -------------------------------------------------------------------- weight-streaming fp8 path
// Contiguous item ranges of the fp8 streaming kernel, one per workgroup, balanced by cost: when group 0
// has more than one 16-row tile (in the layer: the shared expert, which holds all T tokens) each of
// its nh items (items 0 .. nh - 1) counts (16 + HV) / 16 of another item, as it stages a full
// activation tile and re-reads its weights from L2. Measured at the decode shape: HV = 2 took the
// FP8 layer from 2.06 to 2.00-2.02 ms (HV = 1 and 4 within that spread); the bf16 kernel, whose
// workgroups holding group 0 also end last, measured no gain and keeps equal item counts.
// Cost of items [0, w): 16 w + HV min(w, nh); workgroup b takes the items whose cost prefix starts
// in [C b / G, C (b + 1) / G).
__device__ __forceinline__ int stream_bound(int b, int G, int n, int nh) {
  constexpr long long HV = 2;
  const long long total = 16LL * n + HV * nh;
  const long long t = total * b / G;
  const long long heavy = (16 + HV) * (long long)nh;
  const long long w = t <= heavy ? (t + 15 + HV) / (16 + HV) : nh + (t - heavy + 15) / 16;
  return (int)min(w, (long long)n);
}
__device__ __forceinline__ int stream_heavy(const int32_t* __restrict__ off, const int32_t* __restrict__ prefix,
                                            int n_groups, int total_rows) {
  if (n_groups < 2) return 0;
  int s, e;
  group_rows(off, 0, total_rows, s, e);
  return e - s > 16 ? prefix[1] - prefix[0] : 0;
}

// The weight-streaming scheme of ffn_stream_bf16 for E4M3 codes at decode-sized groups: 16-row
// tiles x 128 weight rows per item (each wave two 16-row MFMA column fragments; in MODE 1 each
// fragment holds the gate rows, then the up rows, of 8 h columns), stages of 512 bytes (four
// 128-deep scale blocks) of every weight row and live activation row, plus the stage's 1x128
// activation scales (one 4-byte direct load per lane). Each fragment's 128x128 weight-block scales
// are uniform per wave and come in by scalar loads one stage ahead. The arithmetic is that of the
// register-streaming fp8 kernels: per block, acc += mfma(A, B) * (activation scale * weight scale).
template <int MODE, typename TY>
__global__ __launch_bounds__(256) void ffn_stream_fp8(const int32_t* __restrict__ off,
                                                      const int32_t* __restrict__ prefix, int n_groups,
                                                      int total_rows, const int32_t* __restrict__ row_index,
                                                      const uint8_t* __restrict__ X, const float* __restrict__ Xs,
                                                      int x_rows, const uint8_t* __restrict__ W0,
                                                      const uint8_t* __restrict__ W1, const float* __restrict__ S0,
                                                      const float* __restrict__ S1, int N, int K,
                                                      void* __restrict__ out) {
  constexpr int SKB = 512, KBS = SKB / 128;   // bytes of each row per stage, scale blocks per stage
  constexpr int CPR = SKB / 16, RPW = 32;     // 16-byte chunks per row run, weight rows per wave
  constexpr int A_BYTES = 16 * SKB, B_BYTES = 4 * RPW * SKB, SC_BYTES = 16 * KBS * 4;
  constexpr int BUF = A_BYTES + B_BYTES + SC_BYTES;
  __shared__ __align__(16) uint8_t lds[2 * BUF];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_items = prefix[n_groups];
  const int nh = stream_heavy(off, prefix, n_groups, total_rows);
  const int i0 = stream_bound(blockIdx.x, gridDim.x, n_items, nh);
  const int i1 = stream_bound(blockIdx.x + 1, gridDim.x, n_items, nh);
  if (i0 >= i1) return;
  const int S = K / SKB, nkb = K / 128;

  auto src_row = [&](int r) {
    const int tk = MODE == 1 && row_index ? row_index[r] : r;
    return (tk >= 0 && tk < x_rows) ? tk : -1;
  };
  struct It {
    int g, pb, pe, s, e, r0, r1, c0;
    int sc_src;     // per lane: source row of the activation scales this lane loads (row lane / 4)
    uint32_t bits;
    bool once;
  };
  auto item = [&](int w, const It* prev) {
    It it;
    if (prev && w < prev->pe) {
      it.g = prev->g; it.pb = prev->pb; it.pe = prev->pe; it.s = prev->s; it.e = prev->e;
    } else {
      it.g = find_group(prefix, n_groups, w);
      it.pb = prefix[it.g];
      it.pe = prefix[it.g + 1];
      group_rows(off, it.g, total_rows, it.s, it.e);
    }
    const int mt = max((it.e - it.s + 15) >> 4, 1);
    const int local = w - it.pb;
    it.r0 = it.s + 16 * (local % mt);
    it.r1 = min(it.e, it.r0 + 16);
    it.c0 = (local / mt) * (MODE == 1 ? 2 * RPW : 4 * RPW);   // h columns (MODE 1) or rows of W_down
    it.once = mt == 1;
    it.bits = 0;
    for (int j = 0; j < 16 && it.r0 + j < it.r1; ++j)
      if (src_row(it.r0 + j) >= 0) it.bits |= 1u << j;
    // rows without data load the scales of a row that has them (or of row 0 of X); they are masked.
    // Built from uniform (scalar) loads: a vector load here would make the compiler drain the
    // stage loads in flight before using it.
    const int first = it.bits ? __builtin_ctz(it.bits) : 0;
    const int fsrc = max(src_row(it.r0 + first), 0);
    it.sc_src = fsrc;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if ((it.bits >> j) & 1u) {
        const int sj = src_row(it.r0 + j);
        if (lane / KBS == j) it.sc_src = sj;
      }
    return it;
  };
  // weight rows of fragment f of this wave: block row of the 128x128 scales, and (MODE 1) h column 0
  auto frag_col = [&](const It& it, int f) { return MODE == 1 ? it.c0 + 16 * wave + 8 * f : it.c0 + RPW * wave + 16 * f; };
  const int lrow = lane / CPR, lchunk = lane % CPR;
  auto issue = [&](const It& it, int s, int b) {
    uint8_t* sa = lds + b * BUF;
    uint8_t* sb = sa + A_BYTES;
    float* ss = reinterpret_cast<float*>(sb + B_BYTES);
    const int k0 = s * SKB;
#pragma unroll
    for (int j = 0; j < 2; ++j) {              // activation rows 4w .. 4w + 3, two per load
      const int row0 = 4 * wave + 2 * j;
      if (it.r0 + row0 >= it.r1 || !((it.bits >> row0) & 3u)) continue;
      const int row = row0 + lrow;
      // the pair's source rows are uniform; a row without data re-reads the other one (masked)
      const int s0 = (it.bits >> row0) & 1u ? src_row(it.r0 + row0) : -1;
      const int s1 = (it.bits >> (row0 + 1)) & 1u ? src_row(it.r0 + row0 + 1) : -1;
      const int src = lrow ? (s1 >= 0 ? s1 : s0) : (s0 >= 0 ? s0 : s1);
      dma16(X + (size_t)src * K + k0 + ((lchunk ^ (row & 15)) << 4), sa + row0 * SKB);
    }
#pragma unroll
    for (int j = 0; j < RPW / 2; ++j) {        // weight rows RPW w .. RPW w + RPW - 1, two per load
      const int row0 = RPW * wave + 2 * j, row = row0 + lrow;
      const int f = (2 * j) / 16;
      const uint8_t* wr;
      if (MODE == 1) wr = ((row & 15) < 8 ? W0 : W1) + ((size_t)it.g * N + frag_col(it, f) + (row & 7)) * K;
      else wr = W0 + ((size_t)it.g * N + frag_col(it, f) + (row & 15)) * K;
      const uint8_t* p = wr + k0 + ((lchunk ^ (row & 15)) << 4);
      if (it.once) dma16_nt(p, sb + row0 * SKB);
      else dma16(p, sb + row0 * SKB);
    }
    if (wave == 0)                             // 1x128 scales of the 16 rows' stage blocks: [row][block]
      dma4(Xs + (size_t)it.sc_src * nkb + s * KBS + lane % KBS, ss);
  };
  // this wave's weight-block scales for one stage: [fragment][gate, up][block]
  struct Ws {
    float v[2][2][KBS];
  };
  auto wscales = [&](const It& it, int s) {
    Ws w;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const size_t base = ((size_t)it.g * (N / 128) + frag_col(it, f) / 128) * nkb + s * KBS;
#pragma unroll
      for (int kk = 0; kk < KBS; ++kk) {
        w.v[f][0][kk] = S0[base + kk];
        w.v[f][1][kk] = MODE == 1 ? S1[base + kk] : w.v[f][0][kk];
      }
    }
    return w;
  };
  auto compute = [&](int b, const It& it, const Ws& w, f32x4 (&acc)[2]) {
    const uint8_t* sa = lds + b * BUF;
    const uint8_t* sb = sa + A_BYTES + RPW * wave * SKB;
    const float* ss = reinterpret_cast<const float*>(sa + A_BYTES + B_BYTES);
    const int r = lane & 15, q = lane >> 4;
    const uint32_t amsk = ((it.bits >> r) & 1u) ? 0xffffffffu : 0u;
    const bool up = MODE == 1 && r >= 8;      // this lane's column of each fragment is an up row
#pragma unroll
    for (int kk = 0; kk < KBS; ++kk) {
      const int c0 = 8 * kk + 2 * q;           // lane group q: the 32 codes 32q .. 32q + 31 of the block
      const uint4 alo = *reinterpret_cast<const uint4*>(sa + r * SKB + ((c0 ^ r) << 4));
      const uint4 ahi = *reinterpret_cast<const uint4*>(sa + r * SKB + (((c0 + 1) ^ r) << 4));
      const i32x8 av = mask_i32x8(i32x8{(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w,
                                        (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w}, amsk);
      float sai[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * q + i;
        sai[i] = ((it.bits >> row) & 1u) ? ss[row * KBS + kk] : 0.f;
      }
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int br = 16 * f + r;
        const uint4 blo = *reinterpret_cast<const uint4*>(sb + br * SKB + ((c0 ^ r) << 4));
        const uint4 bhi = *reinterpret_cast<const uint4*>(sb + br * SKB + (((c0 + 1) ^ r) << 4));
        const i32x8 bv = i32x8{(int)blo.x, (int)blo.y, (int)blo.z, (int)blo.w,
                               (int)bhi.x, (int)bhi.y, (int)bhi.z, (int)bhi.w};
        const f32x4 p = mfma_fp8_block(av, bv);
        const float sw = up ? w.v[f][1][kk] : w.v[f][0][kk];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[f][i] = fmaf(p[i], sai[i] * sw, acc[f][i]);
      }
    }
  };
  auto epilogue = [&](const It& it, const f32x4 (&acc)[2]) {
    const int col = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = it.r0 + 4 * (lane >> 4) + i;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        if (MODE == 1) {
          const float v = __shfl_xor(acc[f][i], 8);   // the up value of this lane's h column
          if (r < it.r1 && col < 8) static_cast<float*>(out)[(size_t)r * N + frag_col(it, f) + col] = swiglu(acc[f][i], v);
        } else if (r < it.r1) {
          Elem<TY>::store(static_cast<TY*>(out), (size_t)r * N + frag_col(it, f) + col, acc[f][i]);
        }
      }
    }
  };

  const long long total = (long long)(i1 - i0) * S;
  It ld = item(i0, nullptr), cu = ld, issued = ld;
  int ld_w = i0, ld_s = 0, cs = 0;
  Ws w_cur = wscales(cu, 0), w_nxt = w_cur;
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  auto load_next = [&](int b) {
    issue(ld, ld_s, b);
    issued = ld;
    w_nxt = wscales(ld, ld_s);
    if (++ld_s == S) {
      ld_s = 0;
      if (++ld_w < i1) ld = item(ld_w, &ld);
    }
  };
  f32x4 done[2];
  It done_it = cu;
  bool pending = false;
  load_next(0);
  w_cur = w_nxt;
  for (long long gs = 0; gs < total; ++gs) {
    wait_dma_keep_barrier<0>();
    const Ws w_this = w_cur;
    if (gs + 1 < total) load_next((int)((gs + 1) & 1));
    if (pending) {
      epilogue(done_it, done);
      pending = false;
    }
    compute((int)(gs & 1), cu, w_this, acc);
    w_cur = w_nxt;
    if (++cs == S) {
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        done[f] = acc[f];
        acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      done_it = cu;
      pending = true;
      cs = 0;
      cu = issued;
    }
  }
  if (pending) epilogue(done_it, done);
}

// -------------------------------------------------------------------- LDS-tiled fp8 path
// Same tiling as ffn_lds_bf16, with one 128-deep E4M3 K block per stage (a 128-byte tile row):
// each fragment pair is one v_mfma_scale_f32_16x16x128_f8f6f4 whose fp32 result is multiplied
// by (activation 1x128 tile scale x weight 128x128 block scale) and added to the fp32
// accumulator. The stage's 256 activation scales are loaded into LDS next to the tiles
// (4-byte direct loads); the weight block scales are uniform per wave (scalar loads).
// MODE 1: gate/up GEMM + SwiGLU -> h as E4M3 codes [rows, N = I] (out) with one fp32 scale per 1x128
// tile (out_scales [rows, N / 128]); MODE 2: down GEMM -> Y [rows, N = H].

#ifndef MOE_FP8_GM
#define MOE_FP8_GM 2     // row tiles per band in the fp8 LDS kernel
#endif

template <int MODE, typename TY>
__global__ __launch_bounds__(512) void ffn_lds_fp8(const int32_t* __restrict__ off,
                                                   const int32_t* __restrict__ prefix, int n_groups,
                                                   int total_rows, const int32_t* __restrict__ row_index,
                                                   const uint8_t* __restrict__ X,
                                                   const float* __restrict__ Xs, int x_rows,
                                                   const uint8_t* __restrict__ W0,
                                                   const uint8_t* __restrict__ W1,
                                                   const float* __restrict__ S0,
                                                   const float* __restrict__ S1, int N, int K,
                                                   void* __restrict__ out, float* __restrict__ out_scales = nullptr) {
  __shared__ __align__(16) uint8_t sA0[LB_TILE];
  __shared__ __align__(16) uint8_t sB0[LB_TILE];
  __shared__ __align__(16) uint8_t sA1[LB_TILE];
  __shared__ __align__(16) uint8_t sB1[LB_TILE];
  __shared__ __align__(16) float sS0[LB_M];
  __shared__ __align__(16) float sS1[LB_M];
  const int n_nt = MODE == 1 ? N / 128 : N / 256;
  const int nkb = K / 128;
  int nt;
  Tile t;
  if (!find_tile(off, prefix, n_groups, total_rows, LB_M, n_nt, MOE_FP8_GM, nt, t, true)) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rows = t.r1 - t.r0;

  const int tok0 = MODE == 1 ? (row_index ? row_index[t.r0] : t.r0) : t.r0;
  const int tok_first = (tok0 >= 0 && tok0 < x_rows) ? tok0 : 0;
  auto src_row = [&](int row) {
    const int r = t.r0 + row;
    if (r >= t.r1) return tok_first;
    const int tk = MODE == 1 && row_index ? row_index[r] : r;
    return (tk >= 0 && tk < x_rows) ? tk : tok_first;
  };
  const uint8_t* asrc[4];
  const uint8_t* bsrc[4];
  bool aload[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = wave * 32 + j * 8 + (lane >> 3);
    const int c = swz(row, lane & 7);
    asrc[j] = X + (size_t)src_row(row) * K + c * 16;
    aload[j] = wave * 32 + j * 8 < rows;
    if (MODE == 1) {
      const int half = row >> 7, w = row & 127;
      const int hcol = nt * 128 + half * 64 + (w & 63);
      bsrc[j] = (w < 64 ? W0 : W1) + ((size_t)t.g * N + hcol) * K + c * 16;
    } else {
      bsrc[j] = W0 + ((size_t)t.g * N + nt * 256 + row) * K + c * 16;
    }
  }
  // activation scales: waves 0..3 each load 64 rows' scales per stage
  const float* ssrc = Xs + (size_t)src_row((wave & 3) * 64 + lane) * nkb;
  const bool sload = wave < 4 && (wave & 3) * 64 < rows;
  // the group's only row tile loads its weights non-temporally, as the bf16 kernel does
  const bool w_once = __builtin_amdgcn_readfirstlane((int)t.once) != 0;
  auto stage = [&](int kb, uint8_t* sa, uint8_t* sb, float* ss) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int base = (wave * 32 + j * 8) * 128;
      if (aload[j]) dma16(asrc[j] + kb * 128, sa + base);
      if (w_once) dma16_nt(bsrc[j] + kb * 128, sb + base);
      else dma16(bsrc[j] + kb * 128, sb + base);
    }
    if (sload) dma4(ssrc + kb, ss + (wave & 3) * 64);
  };

  // row fragment m of wave wm holds the tile's rows 16 (4m + wm) .. +16: a tile with fewer rows
  // than 256 spreads its fragments evenly over the four wm waves
  const int wm = wave & 3, wn = wave >> 2;
  const int nmf = max(0, min(4, (((rows + 15) >> 4) - wm + 3) >> 2));
  // weight block scales of this wave's columns: [t.g][block][kb]
  const float* sw0;
  const float* sw1;
  if (MODE == 1) {
    sw0 = S0 + ((size_t)t.g * (N / 128) + nt) * nkb;   // gate block of h columns nt*128..+128
    sw1 = S1 + ((size_t)t.g * (N / 128) + nt) * nkb;   // up block
  } else {
    sw0 = S0 + ((size_t)t.g * (N / 128) + nt * 2 + wn) * nkb;
    sw1 = sw0;
  }
  // The K loop reads them from registers: lane l holds blocks l and l + 64 (K <= 16384), picked out
  // per stage with a uniform lane index. A load inside the loop would be the only one the compiler
  // tracks, and its wait would also drain the next stage's loads already in flight.
  float wr0[2], wr1[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kb = lane + 64 * h;
    wr0[h] = kb < nkb ? sw0[kb] : 0.f;
    wr1[h] = kb < nkb ? sw1[kb] : 0.f;
  }
  auto wscale = [&](const float (&wr)[2], int kb) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, kb < 64 ? wr[0] : wr[1]),
                                                               kb & 63));
  };
  f32x4 acc[4][8];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int kb, const uint8_t* sa, const uint8_t* sb, const float* ss) {
    const float w0 = wscale(wr0, kb), w1 = wscale(wr1, kb);
    // lane group q supplies chunks q and q + 4 of the 128-byte block (any K order works as
    // long as A and B use the same one); this is the conflict-free bf16 fragment pattern
    const int c0 = lane >> 4;
    i32x8 a[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int row = (4 * m + wm) * 16 + (lane & 15);
      const uint4 lo = *reinterpret_cast<const uint4*>(sa + row * 128 + swz(row, c0) * 16);
      const uint4 hi = *reinterpret_cast<const uint4*>(sa + row * 128 + swz(row, c0 + 4) * 16);
      a[m] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      i32x8 b[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int row = wn * 128 + (half * 4 + jj) * 16 + (lane & 15);
        const uint4 lo = *reinterpret_cast<const uint4*>(sb + row * 128 + swz(row, c0) * 16);
        const uint4 hi = *reinterpret_cast<const uint4*>(sb + row * 128 + swz(row, c0 + 4) * 16);
        b[jj] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      // MODE 1: fragments 0..3 are gate columns, 4..7 the up columns; MODE 2: one block
      const float w = (MODE == 1 && half == 1) ? w1 : w0;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (m < nmf) {
          const f32x4 sa4 = *reinterpret_cast<const f32x4*>(ss + (4 * m + wm) * 16 + (lane >> 4) * 4);
          f32x4 s4;
#pragma unroll
          for (int i = 0; i < 4; ++i) s4[i] = sa4[i] * w;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const f32x4 p = mfma_fp8_block(a[m], b[jj]);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[m][half * 4 + jj][i] = fmaf(p[i], s4[i], acc[m][half * 4 + jj][i]);
          }
        }
      }
    }
  };

  stage(0, sA0, sB0, sS0);
  asm volatile("" ::"v"(wr0[0]), "v"(wr0[1]), "v"(wr1[0]), "v"(wr1[1]));   // scale loads complete here
  wait_dma();
  __syncthreads();
  for (int kb = 0; kb < nkb; kb += 2) {
    if (kb + 1 < nkb) stage(kb + 1, sA1, sB1, sS1);
    compute(kb, sA0, sB0, sS0);
    wait_dma();
    __syncthreads();
    if (kb + 1 >= nkb) break;
    if (kb + 2 < nkb) stage(kb + 2, sA0, sB0, sS0);
    compute(kb + 1, sA1, sB1, sS1);
    wait_dma();
    __syncthreads();
  }

  if constexpr (MODE == 1) {
    // h = SwiGLU(z, v), quantized here: the tile holds all 128 h columns of its rows, one 1x128
    // tile each. The row's max |h| over this wave's 64 columns (4 fragments x 16 lanes), then over
    // the two column waves through LDS (the scale buffers are free after the last k-step's
    // barrier); the scale and the codes are the row quantizer's: amax / 448, E4M3(h / scale).
    uint8_t* Hc = static_cast<uint8_t*>(out);
    float hv[4][4][4];
    float am[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        am[m][i] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          hv[m][j][i] = swiglu(acc[m][j][i], acc[m][j + 4][i]);
          am[m][i] = fmaxf(am[m][i], fabsf(hv[m][j][i]));
        }
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) am[m][i] = fmaxf(am[m][i], __shfl_xor(am[m][i], o, 16));
      }
    float* mine = wn == 0 ? sS0 : sS1;
    const float* other = wn == 0 ? sS1 : sS0;
    if ((lane & 15) == 0) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[(4 * m + wm) * 16 + (lane >> 4) * 4 + i] = am[m][i];
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m >= nmf) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (4 * m + wm) * 16 + (lane >> 4) * 4 + i;
        const int r = t.r0 + row;
        if (r >= t.r1) continue;
        const float scale = fmaxf(am[m][i], other[row]) / 448.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = nt * 128 + wn * 64 + j * 16 + (lane & 15);
          Hc[(size_t)r * N + col] = (uint8_t)e4m3_encode(scale == 0.f ? hv[m][j][i] : hv[m][j][i] / scale);
        }
        if (wn == 0 && (lane & 15) == 0) out_scales[(size_t)r * (N / 128) + nt] = scale;
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m >= nmf) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = t.r0 + (4 * m + wm) * 16 + (lane >> 4) * 4 + i;
        if (r >= t.r1) continue;
        TY* Y = static_cast<TY*>(out);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int col = nt * 256 + wn * 128 + j * 16 + (lane & 15);
          Elem<TY>::store(Y, (size_t)r * N + col, acc[m][j][i]);
        }
      }
    }
  }
}

// -------------------------------------------------------------------- host side
inline unsigned pad8(long long n) { return (unsigned)((n + 7) / 8 * 8); }

inline long long mslots(int total_rows, int n_groups, int BM) {
  return (total_rows + BM - 1) / BM + n_groups;
}

struct WsLayout {
  size_t prefix, hf, hb, hc, hs, total;
};

WsLayout ws_layout(int n_groups, int total_rows, int H, int I, int x_dtype) {
  WsLayout L{};
  size_t o = 0;
  // two tile prefixes, then the pool counters of the two streaming launches
  L.prefix = o; o += align256(((size_t)2 * (n_groups + 1) + 2) * sizeof(int32_t));
  const size_t rows = (size_t)total_rows;
  if (x_dtype == MOE_F32 || x_dtype == MOE_FP8_E4M3) { L.hf = o; o += align256(rows * I * sizeof(float)); }
  if (x_dtype == MOE_BF16) { L.hb = o; o += align256(rows * I * sizeof(uint16_t)); }
  if (x_dtype == MOE_FP8_E4M3) {
    L.hc = o; o += align256(rows * I);
    L.hs = o; o += align256(rows * (I / 128) * sizeof(float));
  }
  L.total = o;
  return L;
}

int pick_rm(int total_rows, int n_groups) {
  const long long avg = n_groups > 0 ? ((long long)total_rows + n_groups - 1) / n_groups : 0;
  if (avg <= 16) return 1;
  if (avg <= 32) return 2;
  return 4;
}

inline void mark(void* const* ev, int i, hipStream_t st) {
  if (ev && ev[i]) (void)hipEventRecord(static_cast<hipEvent_t>(ev[i]), st);
}

template <typename TY>
hipError_t run_f32(const FfnArgs& a, const WsLayout& L, hipStream_t st, void* const* ev) {
  char* ws = static_cast<char*>(a.ws);
  int32_t* prefix = reinterpret_cast<int32_t*>(ws + L.prefix);
  int32_t* prefix2 = prefix + (a.n_groups + 1);
  float* Hf = reinterpret_cast<float*>(ws + L.hf);
  const int nt1 = (a.I + 15) / 16, nt2 = (a.H + 15) / 16;
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, a.offsets, a.n_groups, a.total_rows,
                     16, nt1, prefix);
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, a.offsets, a.n_groups, a.total_rows,
                     16, nt2, prefix2);
  const long long ms = mslots(a.total_rows, a.n_groups, 16);
  mark(ev, 0, st);
  hipLaunchKernelGGL(ffn1_f32, dim3(pad8(ms * nt1)), dim3(256), 0, st, a.offsets, prefix,
                     a.n_groups, a.total_rows, a.row_index, static_cast<const float*>(a.X), a.x_rows,
                     static_cast<const float*>(a.Wg), static_cast<const float*>(a.Wu), a.H, a.I, Hf);
  mark(ev, 1, st);
  mark(ev, 2, st);
  hipLaunchKernelGGL(ffn2_f32<TY>, dim3(pad8(ms * nt2)), dim3(256), 0, st, a.offsets, prefix2,
                     a.n_groups, a.total_rows, Hf, static_cast<const float*>(a.Wd), a.H, a.I,
                     static_cast<TY*>(a.Y));
  mark(ev, 3, st);
  return hipGetLastError();
}

template <int RM, typename TY>
hipError_t run_bf16(const FfnArgs& a, const WsLayout& L, hipStream_t st, void* const* ev) {
  char* ws = static_cast<char*>(a.ws);
  int32_t* prefix = reinterpret_cast<int32_t*>(ws + L.prefix);
  int32_t* prefix2 = prefix + (a.n_groups + 1);
  uint16_t* Hb = reinterpret_cast<uint16_t*>(ws + L.hb);
  constexpr int BM = 16 * RM;
  constexpr int RN = 2;   // two 16-column weight fragments per wave (measured best at decode)
  const int nt1 = a.I / 64, nt2 = a.H / (64 * RN);
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, a.offsets, a.n_groups, a.total_rows,
                     BM, nt1, prefix);
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, a.offsets, a.n_groups, a.total_rows,
                     BM, nt2, prefix2);
  const long long ms = mslots(a.total_rows, a.n_groups, BM);
  mark(ev, 0, st);
  hipLaunchKernelGGL(ffn1_bf16<RM>, dim3(pad8(ms * nt1)), dim3(256), 0, st, a.offsets, prefix,
                     a.n_groups, a.total_rows, a.row_index, static_cast<const uint16_t*>(a.X), a.x_rows,
                     static_cast<const uint16_t*>(a.Wg), static_cast<const uint16_t*>(a.Wu), a.H, a.I, Hb, a.ZV);
  mark(ev, 1, st);
  mark(ev, 2, st);
  hipLaunchKernelGGL((ffn2_bf16<RM, RN, TY>), dim3(pad8(ms * nt2)), dim3(256), 0, st,
                     a.offsets, prefix2, a.n_groups, a.total_rows, Hb, static_cast<const uint16_t*>(a.Wd),
                     a.H, a.I, static_cast<TY*>(a.Y));
  mark(ev, 3, st);
  return hipGetLastError();
}

// both K dimensions split into whole stages, whole items per group
inline bool stream_supported(const FfnArgs& a) { return a.H % 512 == 0 && a.I % 512 == 0; }

template <typename TY>
hipError_t run_bf16_stream(const FfnArgs& a, const WsLayout& L, hipStream_t st, void* const* ev) {
  char* ws = static_cast<char*>(a.ws);
  int32_t* prefix1 = reinterpret_cast<int32_t*>(ws + L.prefix);
  int32_t* prefix2 = prefix1 + (a.n_groups + 1);
  int32_t* pool = STREAM_TAIL > 0 ? prefix2 + (a.n_groups + 1) : nullptr;
  int32_t* pool2 = STREAM_TAIL > 0 && MOE_STREAM_POOL2 ? pool + 1 : nullptr;
  uint16_t* Hb = reinterpret_cast<uint16_t*>(ws + L.hb);
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, a.offsets, a.n_groups, a.total_rows, 16,
                     a.I / (32 * ST1_NF), prefix1, 0, pool, a.H / (64 * ST2_NF), prefix2, pool2);
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)max(cus, 1);    // one workgroup per CU (the LDS ring fills a CU)
  mark(ev, 0, st);
  hipLaunchKernelGGL((ffn_stream_bf16<1, uint16_t, ST1_NF, ST1_SKB, ST_NWV>), dim3(grid), dim3(64 * ST_NWV), 0, st, a.offsets, prefix1, a.n_groups,
                     a.total_rows, a.row_index, static_cast<const uint16_t*>(a.X), a.x_rows,
                     static_cast<const uint16_t*>(a.Wg), static_cast<const uint16_t*>(a.Wu), a.I, a.H,
                     static_cast<void*>(Hb), a.ZV, pool);
  mark(ev, 1, st);
  mark(ev, 2, st);
  hipLaunchKernelGGL((ffn_stream_bf16<2, TY, ST2_NF, ST2_SKB, ST_NWV>), dim3(grid), dim3(64 * ST_NWV), 0, st, a.offsets, prefix2, a.n_groups,
                     a.total_rows, static_cast<const int32_t*>(nullptr), static_cast<const uint16_t*>(Hb),
                     a.total_rows, static_cast<const uint16_t*>(a.Wd), static_cast<const uint16_t*>(nullptr), a.H,
                     a.I, a.Y, static_cast<float*>(nullptr), pool2);
  mark(ev, 3, st);
  return hipGetLastError();
}

template <typename TY, int WM, int NW = 8, int RB = MOE_LDS_RB, int NBUF = MOE_LDS_NBUF>
hipError_t run_bf16_lds(const FfnArgs& a, const WsLayout& L, hipStream_t st, void* const* ev) {
  char* ws = static_cast<char*>(a.ws);
  int32_t* prefix1 = reinterpret_cast<int32_t*>(ws + L.prefix);
  int32_t* prefix2 = prefix1 + (a.n_groups + 1);
  uint16_t* Hb = reinterpret_cast<uint16_t*>(ws + L.hb);
  // WM = 0 (mixed tiles): prefixes and grid in units of 128-row x 512-weight-row tiles; a 256-row
  // tile has twice as many column tiles
  constexpr int W = WM == 0 ? 2 : WM;
  constexpr int BM = 64 * W, BW = 128 * (NW / W);
  const int nt1 = a.I / (BW / 2), nt2 = a.H / BW;
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, a.offsets, a.n_groups, a.total_rows,
                     BM, nt1, prefix1, WM == 0 ? 2 * nt1 : 0);
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, a.offsets, a.n_groups, a.total_rows,
                     BM, nt2, prefix2, WM == 0 ? 2 * nt2 : 0);
  const long long ms = mslots(a.total_rows, a.n_groups, BM);
  mark(ev, 0, st);
  hipLaunchKernelGGL((ffn_lds_bf16<1, uint16_t, RB, NBUF, WM, NW>), dim3(pad8(ms * nt1)), dim3(NW * 64), 0, st,
                     a.offsets, prefix1, a.n_groups, a.total_rows, a.row_index, static_cast<const uint16_t*>(a.X),
                     a.x_rows, static_cast<const uint16_t*>(a.Wg), static_cast<const uint16_t*>(a.Wu), a.I, a.H,
                     static_cast<void*>(Hb), 0, a.ZV);
  mark(ev, 1, st);
  mark(ev, 2, st);
  hipLaunchKernelGGL((ffn_lds_bf16<2, TY, RB, NBUF, WM, NW>), dim3(pad8(ms * nt2)), dim3(NW * 64), 0, st,
                     a.offsets, prefix2, a.n_groups, a.total_rows, static_cast<const int32_t*>(nullptr),
                     static_cast<const uint16_t*>(Hb), a.total_rows, static_cast<const uint16_t*>(a.Wd),
                     static_cast<const uint16_t*>(nullptr), a.H, a.I, a.Y);
  mark(ev, 3, st);
  return hipGetLastError();
}

template <int RM, typename TY>
hipError_t run_fp8(const FfnArgs& a, const WsLayout& L, hipStream_t st, void* const* ev) {
  char* ws = static_cast<char*>(a.ws);
  int32_t* prefix = reinterpret_cast<int32_t*>(ws + L.prefix);
  int32_t* prefix2 = prefix + (a.n_groups + 1);
  float* Hf = reinterpret_cast<float*>(ws + L.hf);
  uint8_t* Hc = reinterpret_cast<uint8_t*>(ws + L.hc);
  float* Hs = reinterpret_cast<float*>(ws + L.hs);
  constexpr int BM = 16 * RM;
  constexpr int RN = RM == 1 ? 1 : 2;
  const int nt1 = a.I / 64, nt2 = a.H / (64 * RN);
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, a.offsets, a.n_groups, a.total_rows,
                     BM, nt1, prefix);
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, a.offsets, a.n_groups, a.total_rows,
                     BM, nt2, prefix2);
  const long long ms = mslots(a.total_rows, a.n_groups, BM);
  mark(ev, 0, st);
  hipLaunchKernelGGL(ffn1_fp8<RM>, dim3(pad8(ms * nt1)), dim3(256), 0, st, a.offsets, prefix,
                     a.n_groups, a.total_rows, a.row_index, static_cast<const uint8_t*>(a.X), a.X_scales,
                     a.x_rows, static_cast<const uint8_t*>(a.Wg), static_cast<const uint8_t*>(a.Wu), a.Wg_s,
                     a.Wu_s, a.H, a.I, Hf);
  mark(ev, 1, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_fp8_quant(Hf, MOE_F32, a.total_rows, a.I, 1, Hc, Hs, st);
  if (e != hipSuccess) return e;
  mark(ev, 2, st);
  hipLaunchKernelGGL((ffn2_fp8<RM, RN, TY>), dim3(pad8(ms * nt2)), dim3(256), 0, st,
                     a.offsets, prefix2, a.n_groups, a.total_rows, Hc, Hs, static_cast<const uint8_t*>(a.Wd),
                     a.Wd_s, a.H, a.I, static_cast<TY*>(a.Y));
  mark(ev, 3, st);
  return hipGetLastError();
}

template <typename TY>
hipError_t run_fp8_stream(const FfnArgs& a, const WsLayout& L, hipStream_t st, void* const* ev) {
  char* ws = static_cast<char*>(a.ws);
  int32_t* prefix1 = reinterpret_cast<int32_t*>(ws + L.prefix);
  int32_t* prefix2 = prefix1 + (a.n_groups + 1);
  float* Hf = reinterpret_cast<float*>(ws + L.hf);
  uint8_t* Hc = reinterpret_cast<uint8_t*>(ws + L.hc);
  float* Hs = reinterpret_cast<float*>(ws + L.hs);
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, a.offsets, a.n_groups, a.total_rows, 16,
                     a.I / 64, prefix1);
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, a.offsets, a.n_groups, a.total_rows, 16,
                     a.H / 128, prefix2);
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)max(cus, 1);
  mark(ev, 0, st);
  hipLaunchKernelGGL((ffn_stream_fp8<1, float>), dim3(grid), dim3(256), 0, st, a.offsets, prefix1, a.n_groups,
                     a.total_rows, a.row_index, static_cast<const uint8_t*>(a.X), a.X_scales, a.x_rows,
                     static_cast<const uint8_t*>(a.Wg), static_cast<const uint8_t*>(a.Wu), a.Wg_s, a.Wu_s, a.I, a.H,
                     static_cast<void*>(Hf));
  mark(ev, 1, st);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_fp8_quant(Hf, MOE_F32, a.total_rows, a.I, 1, Hc, Hs, st);
  if (e != hipSuccess) return e;
  mark(ev, 2, st);
  hipLaunchKernelGGL((ffn_stream_fp8<2, TY>), dim3(grid), dim3(256), 0, st, a.offsets, prefix2, a.n_groups,
                     a.total_rows, static_cast<const int32_t*>(nullptr), static_cast<const uint8_t*>(Hc),
                     static_cast<const float*>(Hs), a.total_rows, static_cast<const uint8_t*>(a.Wd),
                     static_cast<const uint8_t*>(nullptr), a.Wd_s, static_cast<const float*>(nullptr), a.H, a.I,
                     a.Y);
  mark(ev, 3, st);
  return hipGetLastError();
}

template <typename TY>
hipError_t run_fp8_lds(const FfnArgs& a, const WsLayout& L, hipStream_t st, void* const* ev) {
  char* ws = static_cast<char*>(a.ws);
  int32_t* prefix1 = reinterpret_cast<int32_t*>(ws + L.prefix);
  int32_t* prefix2 = prefix1 + (a.n_groups + 1);
  uint8_t* Hc = reinterpret_cast<uint8_t*>(ws + L.hc);
  float* Hs = reinterpret_cast<float*>(ws + L.hs);
  const int nt1 = a.I / 128, nt2 = a.H / 256;
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, a.offsets, a.n_groups, a.total_rows,
                     LB_M, nt1, prefix1);
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, a.offsets, a.n_groups, a.total_rows,
                     LB_M, nt2, prefix2);
  const long long ms = mslots(a.total_rows, a.n_groups, LB_M);
  mark(ev, 0, st);
  hipLaunchKernelGGL((ffn_lds_fp8<1, float>), dim3(pad8(ms * nt1)), dim3(512), 0, st, a.offsets, prefix1,
                     a.n_groups, a.total_rows, a.row_index, static_cast<const uint8_t*>(a.X), a.X_scales,
                     a.x_rows, static_cast<const uint8_t*>(a.Wg), static_cast<const uint8_t*>(a.Wu), a.Wg_s,
                     a.Wu_s, a.I, a.H, static_cast<void*>(Hc), Hs);   // h quantized in the epilogue
  mark(ev, 1, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  mark(ev, 2, st);
  hipLaunchKernelGGL((ffn_lds_fp8<2, TY>), dim3(pad8(ms * nt2)), dim3(512), 0, st, a.offsets, prefix2,
                     a.n_groups, a.total_rows, static_cast<const int32_t*>(nullptr),
                     static_cast<const uint8_t*>(Hc), static_cast<const float*>(Hs), a.total_rows,
                     static_cast<const uint8_t*>(a.Wd), static_cast<const uint8_t*>(nullptr), a.Wd_s,
                     static_cast<const float*>(nullptr), a.H, a.I, a.Y);
  mark(ev, 3, st);
  return hipGetLastError();
}

template <typename TY>
hipError_t dispatch_ffn(const FfnArgs& a, const WsLayout& L, hipStream_t st, void* const* ev) {
  const int rm = pick_rm(a.total_rows, a.n_groups);
  if (a.x_dtype == MOE_F32) return run_f32<TY>(a, L, st, ev);
  if (a.x_dtype == MOE_BF16) {
    if (rm == 1 && stream_supported(a)) return run_bf16_stream<TY>(a, L, st, ev);
    if (rm == 1) return run_bf16<1, TY>(a, L, st, ev);
    if (rm == 2) return run_bf16<2, TY>(a, L, st, ev);
    if (a.H % 512 == 0 && a.I % 256 == 0) return run_bf16_lds<TY, MOE_LDS_WM>(a, L, st, ev);
    if (a.H % 256 == 0 && a.I % 128 == 0) return run_bf16_lds<TY, 4>(a, L, st, ev);
    return run_bf16<4, TY>(a, L, st, ev);
  }
  if (rm == 1 && stream_supported(a)) return run_fp8_stream<TY>(a, L, st, ev);
  if (rm == 1) return run_fp8<1, TY>(a, L, st, ev);
  if (rm == 2) return run_fp8<2, TY>(a, L, st, ev);
  if (a.H % 256 == 0 && a.H <= 16384 && a.I <= 16384) return run_fp8_lds<TY>(a, L, st, ev);
  return run_fp8<4, TY>(a, L, st, ev);
}

}  // namespace

bool gate_up_preact_supported(int H, int I) { return H % 512 == 0 && I % 256 == 0; }

hipError_t launch_gate_up_preact(const int32_t* offsets, int n_groups, int total_rows, const int32_t* row_index,
                                 const void* X, int x_rows, const void* Wg, const void* Wu, int H, int I,
                                 int32_t* prefix, float* ZV, hipStream_t st) {
  constexpr int WM = MOE_LDS_WM, NW = 8, BM = 128, BW = 512;   // mixed tiles counted in 128 x 512 units
  const int nt = I / (BW / 2);
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, offsets, n_groups, total_rows, BM, nt, prefix,
                     WM == 0 ? 2 * nt : 0);
  const long long ms = mslots(total_rows, n_groups, BM);
  hipLaunchKernelGGL((ffn_lds_bf16<3, float, MOE_LDS_RB, MOE_LDS_NBUF, WM, NW>), dim3(pad8(ms * nt)), dim3(NW * 64),
                     0, st, offsets, prefix, n_groups, total_rows, row_index, static_cast<const uint16_t*>(X), x_rows,
                     static_cast<const uint16_t*>(Wg), static_cast<const uint16_t*>(Wu), I, H, static_cast<void*>(ZV));
  return hipGetLastError();
}

hipError_t launch_fp8_rows_gemm(const int32_t* offsets, int n_groups, int total_rows, const uint8_t* A,
                                const float* As, const uint8_t* W, const float* Ws, int N, int K, float* C,
                                int32_t* prefix, hipStream_t st) {
  if (total_rows == 0) return hipSuccess;
  const int rm = pick_rm(total_rows, n_groups);
  if (rm == 1 && K % 512 == 0 && N % 128 == 0) {           // decode-sized groups: weight streaming
    hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, offsets, n_groups, total_rows, 16, N / 128,
                       prefix);
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((ffn_stream_fp8<2, float>), dim3((unsigned)max(cus, 1)), dim3(256), 0, st, offsets, prefix,
                       n_groups, total_rows, static_cast<const int32_t*>(nullptr), A, As, total_rows, W,
                       static_cast<const uint8_t*>(nullptr), Ws, static_cast<const float*>(nullptr), N, K,
                       static_cast<void*>(C));
    return hipGetLastError();
  }
  if (rm == 4 && N % 256 == 0 && K <= 16384) {                // LDS-tiled
    hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, offsets, n_groups, total_rows, LB_M, N / 256,
                       prefix);
    const long long ms = mslots(total_rows, n_groups, LB_M);
    hipLaunchKernelGGL((ffn_lds_fp8<2, float>), dim3(pad8(ms * (N / 256))), dim3(512), 0, st, offsets, prefix,
                       n_groups, total_rows, static_cast<const int32_t*>(nullptr), A, As, total_rows, W,
                       static_cast<const uint8_t*>(nullptr), Ws, static_cast<const float*>(nullptr), N, K,
                       static_cast<void*>(C));
    return hipGetLastError();
  }
  auto reg = [&](auto rm_c, auto rn_c) {                       // register-streamed
    constexpr int RM = decltype(rm_c)::value, RN = decltype(rn_c)::value;
    hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, offsets, n_groups, total_rows, 16 * RM,
                       N / (64 * RN), prefix);
    const long long ms = mslots(total_rows, n_groups, 16 * RM);
    hipLaunchKernelGGL((ffn2_fp8<RM, RN, float>), dim3(pad8(ms * (N / (64 * RN)))), dim3(256), 0, st, offsets,
                       prefix, n_groups, total_rows, A, As, W, Ws, N, K, C);
    return hipGetLastError();
  };
  if (rm == 1) return N % 64 == 0 ? reg(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{}) : hipErrorInvalidValue;
  if (N % 128 != 0) return hipErrorInvalidValue;
  if (rm == 2) return reg(std::integral_constant<int, 2>{}, std::integral_constant<int, 2>{});
  return reg(std::integral_constant<int, 4>{}, std::integral_constant<int, 2>{});
}

bool rows_mn_supported(int N, int K, int split) {
  return N % 512 == 0 && K % 64 == 0 && split % 64 == 0 && split > 0 && split <= K;
}

hipError_t launch_rows_mn(const int32_t* offsets, int n_groups, int total_rows, const void* A, const void* W0,
                          const void* W1, int split, int N, int K, int32_t* prefix, float* C, hipStream_t st) {
  constexpr int WM = 2, NW = 8, BM = 64 * WM, BW = 128 * (NW / WM);
  const int nt = N / BW;
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, offsets, n_groups, total_rows, BM, nt, prefix);
  const long long ms = mslots(total_rows, n_groups, BM);
  hipLaunchKernelGGL((ffn_lds_bf16<4, float, MOE_LDS_RB, MOE_LDS_NBUF, WM, NW>), dim3(pad8(ms * nt)), dim3(NW * 64),
                     0, st, offsets, prefix, n_groups, total_rows, static_cast<const int32_t*>(nullptr),
                     static_cast<const uint16_t*>(A), total_rows, static_cast<const uint16_t*>(W0),
                     static_cast<const uint16_t*>(W1), N, K, static_cast<void*>(C), split);
  return hipGetLastError();
}

size_t grouped_ffn_workspace(int n_groups, int total_rows, int H, int I, int x_dtype) {
  if (total_rows == 0) return 0;
  return ws_layout(n_groups, total_rows, H, I, x_dtype).total;
}

hipError_t launch_grouped_ffn(const FfnArgs& a, hipStream_t st, void* const* events) {
  if (a.total_rows == 0) return hipSuccess;
  const WsLayout L = ws_layout(a.n_groups, a.total_rows, a.H, a.I, a.x_dtype);
  if (a.y_dtype == MOE_BF16) return dispatch_ffn<uint16_t>(a, L, st, events);
  return dispatch_ffn<float>(a, L, st, events);
}

}  // namespace moe
