// Device-side tile bookkeeping shared by the grouped GEMMs: group sizes stay on the device, a
// one-workgroup kernel turns the offsets into a prefix of work items per group, and every
// workgroup maps its id to (group, row tile, column tile) through that prefix.
#pragma once
#include "common.h"

namespace moe {
namespace {

__device__ __forceinline__ void group_rows(const int32_t* __restrict__ off, int g, int total_rows,
                                           int& s, int& e) {
  s = min(max(off[g], 0), total_rows);
  e = min(max(off[g + 1], s), total_rows);
}

// prefix[g] = sum over groups g' < g of ceil(rows_g' / BM) * mult  (mult = work items per row tile);
// with mult_big > 0, groups are cut into 2 BM-row tiles of mult_big items each, and a tail of at
// most BM rows into one BM-row tile of mult items (the mapping of find_tile_mixed)
// counter (optional): set to 0, for a launch after this one that hands out work through it.
// prefix2 (optional, mult_big = 0 only): a second prefix over the same row tiles with mult2 items per
// tile, and its own counter2 (one launch for the two GEMMs of a grouped FFN)
__global__ __launch_bounds__(1024) void tile_prefix_kernel(const int32_t* __restrict__ off,
                                                           int n_groups, int total_rows, int BM, int mult,
                                                           int32_t* __restrict__ prefix, int mult_big = 0,
                                                           int32_t* __restrict__ counter = nullptr,
                                                           int mult2 = 0, int32_t* __restrict__ prefix2 = nullptr,
                                                           int32_t* __restrict__ counter2 = nullptr) {
  __shared__ int wsum[16];
  const int g = threadIdx.x;
  if (counter && g == 0) *counter = 0;
  if (counter2 && g == 0) *counter2 = 0;
  int c = 0;
  if (g < n_groups) {
    int s, e;
    group_rows(off, g, total_rows, s, e);
    c = (e - s + BM - 1) / BM * (prefix2 ? 1 : mult);   // with prefix2: row tiles, scaled below
    if (mult_big > 0) {                 // whole 2 BM-row tiles, then a BM-row tile for a tail of <= BM rows
      const int n = e - s, r = n % (2 * BM);
      c = (n / (2 * BM) + (r > BM)) * mult_big + (r > 0 && r <= BM) * mult;
    }
  }
  const int lane = g & 63, w = g >> 6;
  int incl = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += wsum[i];
  if (g < n_groups) {
    const int m1 = prefix2 ? mult : 1;
    prefix[g] = (base + incl - c) * m1;
    if (g == n_groups - 1) prefix[n_groups] = (base + incl) * m1;
    if (prefix2) {
      prefix2[g] = (base + incl - c) * mult2;
      if (g == n_groups - 1) prefix2[n_groups] = (base + incl) * mult2;
    }
  }
}

// Work item of this workgroup, or -1. Items [0, W) are split into 8 contiguous parts, part x
// going to the workgroups with id % 8 == x (the ones on XCD x). Needs gridDim.x >= 8*ceil(W/8).
__device__ __forceinline__ int xcd_item(int W) {
  const int x = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int P = (W + 7) >> 3;
  if (local >= P) return -1;
  const int w = x * P + local;
  return w < W ? w : -1;
}

struct Tile {
  int g, r0, r1;
  bool once;   // the group has this one row tile only
};

// Work item of this workgroup: `prefix` counts items per group (row tiles x n_nt column tiles).
// Inside a group, items run in bands of GM row tiles with the column tile as the slower index:
// the band's row tiles run side by side on one XCD and share each weight tile through its L2,
// and a row tile's activations are shared by the band's column tiles. Returns the group, the
// column tile and the rows [r0, r1). With `balanced`, a group's rows are shared evenly by its row
// tiles (ceil(rows / tiles) each) instead of filling BM-row tiles and leaving a short last one:
// row tiles that stream the same weight tiles then advance through K at the same pace, so the
// weights they share are still in L2 when the second one reads them.
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ off,
                                          const int32_t* __restrict__ prefix, int n_groups,
                                          int total_rows, int BM, int n_nt, int GM, int& nt, Tile& t,
                                          bool balanced = false) {
  const int W = prefix[n_groups];
  const int w = xcd_item(W);
  if (w < 0) return false;
  t.g = find_group(prefix, n_groups, w);
  int s, e;
  group_rows(off, t.g, total_rows, s, e);
  const int mtiles = (e - s + BM - 1) / BM;
  const int local = w - prefix[t.g];
  const int band = local / (GM * n_nt);
  const int in_band = local - band * GM * n_nt;
  const int bsize = min(GM, mtiles - band * GM);
  nt = in_band / bsize;
  const int mt = band * GM + (in_band - nt * bsize);
  const int per = balanced && mtiles > 0 ? (e - s + mtiles - 1) / mtiles : BM;
  t.once = mtiles == 1;
  t.r0 = s + mt * per;
  t.r1 = min(e, t.r0 + per);
  return t.r0 < t.r1;
}

// find_tile for mixed tiles (prefix from tile_prefix_kernel with BM = 128, mult = n_nt_small,
// mult_big = n_nt_big): a group is cut into 256-row tiles (big = 1, n_nt_big column tiles each),
// and a tail of 1..128 rows becomes one 128-row tile (n_nt_small column tiles); a tail of
// 129..255 rows is a 256-row tile too. The 256-row tiles run in bands of GM as in find_tile; in
// the last band each tail tile follows the 256-row tiles that stage the same weight rows.
__device__ __forceinline__ bool find_tile_mixed(const int32_t* __restrict__ off,
                                                const int32_t* __restrict__ prefix, int n_groups, int total_rows,
                                                int n_nt_small, int n_nt_big, int GM, int& nt, Tile& t, int& big) {
  const int W = prefix[n_groups];
  const int w = xcd_item(W);
  if (w < 0) return false;
  t.g = find_group(prefix, n_groups, w);
  int s, e;
  group_rows(off, t.g, total_rows, s, e);
  const int n = e - s, r = n % 256;
  const int mtiles = n / 256 + (r > 128);      // 256-row tiles
  const int tail = r > 0 && r <= 128;          // one 128-row tile for the rest
  const int local = w - prefix[t.g];
  t.once = mtiles + tail == 1;
  auto tail_tile = [&](int nts) {
    big = 0;
    nt = nts;
    t.r0 = s + mtiles * 256;
    t.r1 = e;
    return nt < n_nt_small && t.r0 < t.r1;
  };
  auto big_tile = [&](int ntb, int mt) {
    big = 1;
    nt = ntb;
    t.r0 = s + mt * 256;
    t.r1 = min(e, t.r0 + 256);
    return t.r0 < t.r1;
  };
  if (mtiles == 0) return tail_tile(local);
  // bands before the last: as in find_tile
  const int nbands = (mtiles + GM - 1) / GM;
  const int before = (nbands - 1) * GM * n_nt_big;
  if (local < before) {
    const int band = local / (GM * n_nt_big);
    const int in_band = local - band * GM * n_nt_big;
    nt = in_band / GM;
    return big_tile(nt, band * GM + (in_band - nt * GM));
  }
  // the last band: for each tail column tile s, the band's 256-row tiles of big column tiles 2s and
  // 2s + 1 (the same weight rows), then the tail tile s, so that it runs beside them and finds
  // those weight rows in L2 instead of streaming them again (n_nt_big == 2 n_nt_small)
  const int bsize = mtiles - (nbands - 1) * GM;
  const int per = 2 * bsize + tail;
  const int j = local - before;
  const int sidx = j / per, q = j - sidx * per;
  if (q >= 2 * bsize) return tail_tile(sidx);
  return big_tile(2 * sidx + q / bsize, (nbands - 1) * GM + q % bsize);
}

}  // namespace
}  // namespace moe
