// C ABI entry points: host-side argument validation, then asynchronous kernel launches.
// Every check runs before the first HIP call, so a rejected call enqueues nothing.
#include <cmath>
#include <cstdio>
#include <string>

#include "common.h"

namespace {

thread_local std::string g_last_error;

moe_status_t fail(moe_status_t s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

moe_status_t ok() {
  g_last_error.clear();
  return MOE_OK;
}

moe_status_t hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(MOE_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

#define REQUIRE(cond, status, msg) \
  do {                             \
    if (!(cond)) return fail(status, msg); \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

moe_status_t check_ws(void* ws, size_t have, size_t need, const char* fn) {
  if (need == 0) return MOE_OK;
  if (ws == nullptr || have < need)
    return fail(MOE_ERR_WORKSPACE, std::string(fn) + ": workspace needs " + std::to_string(need) +
                                       " bytes, got " + std::to_string(ws ? have : 0));
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_VALUE: return "MOE_ERR_INVALID_VALUE";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

// ------------------------------------------------------------------------- router
size_t moe_route_workspace_size(int T, int H, int N_r) {
  if (T <= 0 || H <= 0 || N_r <= 0) return 0;
  return moe::route_workspace(T, H, N_r);
}

static moe_status_t route_impl(const char* name, const void* u, int u_dtype, const float* centroids,
                               const float* bias, const float* logit_offset, const float* affinity_in, int T,
                               int H, int N_r, int K, int n_groups, int topk_groups, float* affinity_out,
                               int32_t* topk_idx, float* topk_gate, void* workspace, size_t workspace_bytes,
                               void* stream) {
  REQUIRE(T >= 0 && H >= 1, MOE_ERR_INVALID_VALUE, std::string(name) + ": need T >= 0 and H >= 1");
  REQUIRE(N_r >= 1 && N_r <= MOE_MAX_EXPERTS, MOE_ERR_UNSUPPORTED, std::string(name) + ": N_r must be in [1, 1024]");
  REQUIRE(K >= 1 && K <= N_r && K <= MOE_MAX_TOPK, MOE_ERR_UNSUPPORTED,
          std::string(name) + ": K must be in [1, min(N_r, 16)]");
  REQUIRE(n_groups >= 1 && n_groups <= 64 && N_r % n_groups == 0, MOE_ERR_UNSUPPORTED,
          std::string(name) + ": n_groups must be in [1, 64] and divide N_r");
  REQUIRE(topk_groups >= 1 && topk_groups <= n_groups && K % topk_groups == 0 &&
              K / topk_groups <= N_r / n_groups,
          MOE_ERR_UNSUPPORTED,
          std::string(name) + ": need 1 <= topk_groups <= n_groups, K % topk_groups == 0 and "
                              "K / topk_groups <= N_r / n_groups");
  REQUIRE(bias && topk_idx && topk_gate, MOE_ERR_INVALID_VALUE,
          std::string(name) + ": bias, topk_idx and topk_gate are required");
  if (!affinity_in) {
    REQUIRE(u && centroids, MOE_ERR_INVALID_VALUE,
            std::string(name) + ": u and centroids are required without affinity_in");
    REQUIRE(u_dtype == MOE_F32 || u_dtype == MOE_BF16, MOE_ERR_UNSUPPORTED,
            std::string(name) + ": u_dtype must be F32 or BF16");
    moe_status_t s = check_ws(workspace, workspace_bytes, moe::route_workspace(T, H, N_r), name);
    if (s != MOE_OK) return s;
  }
  if (T == 0) return ok();
  return hip_status(moe::launch_route(u, u_dtype, centroids, bias, logit_offset, affinity_in, T, H, N_r, K,
                                      n_groups, topk_groups, affinity_out, topk_idx, topk_gate, workspace,
                                      as_stream(stream)),
                    name);
}

moe_status_t moe_route(const void* u, int u_dtype, const float* centroids, const float* bias,
                       const float* logit_offset, const float* affinity_in, int T, int H, int N_r,
                       int K, float* affinity_out, int32_t* topk_idx, float* topk_gate,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return route_impl("moe_route", u, u_dtype, centroids, bias, logit_offset, affinity_in, T, H, N_r, K, 1, 1,
                    affinity_out, topk_idx, topk_gate, workspace, workspace_bytes, stream);
}

moe_status_t moe_route_group_limited(const void* u, int u_dtype, const float* centroids, const float* bias,
                                     const float* logit_offset, const float* affinity_in, int T, int H,
                                     int N_r, int K, int n_groups, int topk_groups, float* affinity_out,
                                     int32_t* topk_idx, float* topk_gate, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return route_impl("moe_route_group_limited", u, u_dtype, centroids, bias, logit_offset, affinity_in, T, H,
                    N_r, K, n_groups, topk_groups, affinity_out, topk_idx, topk_gate, workspace,
                    workspace_bytes, stream);
}

// ------------------------------------------------------------------------- dispatch
size_t moe_permute_workspace_size(int T, int K, int N_r) {
  if (T < 0 || K <= 0 || N_r <= 0) return 0;
  return moe::permute_workspace(T, K, N_r);
}

moe_status_t moe_permute(const int32_t* topk_idx, int T, int K, int N_r, int shared_rows,
                         int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* slot_row,
                         void* workspace, size_t workspace_bytes, void* stream) {
  REQUIRE(T >= 0 && shared_rows >= 0, MOE_ERR_INVALID_VALUE, "moe_permute: T and shared_rows must be >= 0");
  REQUIRE(N_r >= 1 && N_r <= MOE_MAX_EXPERTS, MOE_ERR_UNSUPPORTED, "moe_permute: N_r must be in [1, 1024]");
  REQUIRE(K >= 1 && K <= MOE_MAX_TOPK, MOE_ERR_UNSUPPORTED, "moe_permute: K must be in [1, 16]");
  REQUIRE(counts && offsets, MOE_ERR_INVALID_VALUE, "moe_permute: counts and offsets are required");
  REQUIRE(T == 0 || (topk_idx && row_token && slot_row), MOE_ERR_INVALID_VALUE,
          "moe_permute: topk_idx, row_token and slot_row are required");
  REQUIRE((long long)T * K + shared_rows <= 0x7fffffffLL, MOE_ERR_UNSUPPORTED, "moe_permute: row count overflows int32");
  REQUIRE(shared_rows == 0 || row_token, MOE_ERR_INVALID_VALUE, "moe_permute: row_token is required");
  moe_status_t s = check_ws(workspace, workspace_bytes, moe::permute_workspace(T, K, N_r), "moe_permute");
  if (s != MOE_OK) return s;
  return hip_status(moe::launch_permute(topk_idx, T, K, N_r, shared_rows, counts, offsets, row_token, slot_row,
                                        workspace, as_stream(stream)),
                    "moe_permute");
}

size_t moe_permute_noalloc_max_bytes(void) { return moe::PERMUTE_SCRATCH_BYTES; }

moe_status_t moe_permute_noalloc(const int32_t* topk_idx, int T, int K, int N_r, int shared_rows,
                                 int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* slot_row,
                                 void* stream) {
  REQUIRE(T >= 0 && shared_rows >= 0, MOE_ERR_INVALID_VALUE, "moe_permute_noalloc: T and shared_rows must be >= 0");
  REQUIRE(N_r >= 1 && N_r <= MOE_MAX_EXPERTS, MOE_ERR_UNSUPPORTED, "moe_permute_noalloc: N_r must be in [1, 1024]");
  REQUIRE(K >= 1 && K <= MOE_MAX_TOPK, MOE_ERR_UNSUPPORTED, "moe_permute_noalloc: K must be in [1, 16]");
  REQUIRE(counts && offsets, MOE_ERR_INVALID_VALUE, "moe_permute_noalloc: counts and offsets are required");
  REQUIRE(T == 0 || (topk_idx && row_token && slot_row), MOE_ERR_INVALID_VALUE,
          "moe_permute_noalloc: topk_idx, row_token and slot_row are required");
  REQUIRE((long long)T * K + shared_rows <= 0x7fffffffLL, MOE_ERR_UNSUPPORTED,
          "moe_permute_noalloc: row count overflows int32");
  REQUIRE(shared_rows == 0 || row_token, MOE_ERR_INVALID_VALUE, "moe_permute_noalloc: row_token is required");
  const size_t need = moe::permute_workspace(T, K, N_r);
  if (need > moe::PERMUTE_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE, "moe_permute_noalloc: T = " + std::to_string(T) + " with N_r = " +
                                       std::to_string(N_r) + " needs " + std::to_string(need) +
                                       " bytes of scratch, more than its static " +
                                       std::to_string(moe::PERMUTE_SCRATCH_BYTES) + " bytes");
  void* scratch = nullptr;
  hipError_t e = moe::permute_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e, "moe_permute_noalloc (scratch lookup)");
  return hip_status(moe::launch_permute(topk_idx, T, K, N_r, shared_rows, counts, offsets, row_token, slot_row,
                                        scratch, as_stream(stream)),
                    "moe_permute_noalloc");
}

moe_status_t moe_gather_rows(const void* x, const float* x_scales, int x_dtype, int T, int H,
                             const int32_t* row_token, const int32_t* n_rows, int max_rows, void* x_perm,
                             float* x_perm_scales, void* stream) {
  REQUIRE(T >= 0 && H >= 1 && max_rows >= 0, MOE_ERR_INVALID_VALUE,
          "moe_gather_rows: need T >= 0, H >= 1 and max_rows >= 0");
  REQUIRE(x_dtype == MOE_F32 || x_dtype == MOE_BF16 || x_dtype == MOE_FP8_E4M3, MOE_ERR_UNSUPPORTED,
          "moe_gather_rows: x_dtype must be F32, BF16 or FP8_E4M3");
  const int esize = x_dtype == MOE_F32 ? 4 : (x_dtype == MOE_BF16 ? 2 : 1);
  REQUIRE((long long)H * esize % 16 == 0, MOE_ERR_UNSUPPORTED,
          "moe_gather_rows: a row must be a whole number of 16-byte vectors (H * element size % 16 == 0)");
  REQUIRE(x_dtype != MOE_FP8_E4M3 || H % 128 == 0, MOE_ERR_UNSUPPORTED,
          "moe_gather_rows: FP8 codes need H % 128 == 0 (one scale per 1x128 tile)");
  REQUIRE((long long)H * esize <= 0x7fffffffLL && (long long)max_rows * H * esize <= 0x7fffffffffffLL &&
              (long long)T * H * esize <= 0x7fffffffffffLL,
          MOE_ERR_UNSUPPORTED, "moe_gather_rows: sizes too large");
  if (max_rows == 0) return MOE_OK;
  REQUIRE(row_token && n_rows && x_perm, MOE_ERR_INVALID_VALUE,
          "moe_gather_rows: row_token, n_rows and x_perm are required");
  REQUIRE(T == 0 || x, MOE_ERR_INVALID_VALUE, "moe_gather_rows: x is required");
  REQUIRE(x_dtype != MOE_FP8_E4M3 || (x_perm_scales && (T == 0 || x_scales)), MOE_ERR_INVALID_VALUE,
          "moe_gather_rows: FP8 codes need x_scales and x_perm_scales");
  REQUIRE((T == 0 || aligned16(x)) && aligned16(x_perm), MOE_ERR_UNSUPPORTED,
          "moe_gather_rows: x and x_perm must be 16-byte aligned");
  const bool fp8 = x_dtype == MOE_FP8_E4M3;
  return hip_status(moe::launch_gather_rows(x, fp8 ? x_scales : nullptr, T, H * esize, fp8 ? H / 128 : 0,
                                            row_token, n_rows, max_rows, x_perm, fp8 ? x_perm_scales : nullptr,
                                            as_stream(stream)),
                    "moe_gather_rows");
}

// ------------------------------------------------------------------------- expert FFNs
size_t moe_grouped_ffn_workspace_size(int n_groups, int total_rows, int H, int I, int x_dtype) {
  if (n_groups <= 0 || total_rows < 0 || H <= 0 || I <= 0) return 0;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16 && x_dtype != MOE_FP8_E4M3) return 0;
  return moe::grouped_ffn_workspace(n_groups, total_rows, H, I, x_dtype);
}

static moe_status_t grouped_ffn_impl(int n_groups, const int32_t* offsets, int total_rows,
                             const int32_t* row_index, const void* X, const float* X_scales,
                             int x_rows, int x_dtype, const void* W_gate, const void* W_up,
                             const void* W_down, const float* Wg_scales, const float* Wu_scales,
                             const float* Wd_scales, int w_dtype, int H, int I, void* Y, int y_dtype,
                             void* workspace, size_t workspace_bytes, void* stream, void* const* events,
                             float* zv = nullptr, bool want_zv = false) {
  REQUIRE(n_groups >= 1 && n_groups <= MOE_MAX_EXPERTS, MOE_ERR_UNSUPPORTED,
          "moe_grouped_ffn: n_groups must be in [1, 1024]");
  REQUIRE(!want_zv || x_dtype == MOE_BF16, MOE_ERR_UNSUPPORTED,
          "moe_grouped_ffn_train: saved pre-activations are built for BF16 only");
  REQUIRE(!want_zv || total_rows == 0 || zv, MOE_ERR_INVALID_VALUE, "moe_grouped_ffn_train: zv is required");
  REQUIRE(total_rows >= 0 && x_rows >= 0 && H >= 1 && I >= 1, MOE_ERR_INVALID_VALUE,
          "moe_grouped_ffn: need total_rows >= 0, x_rows >= 0, H >= 1, I >= 1");
  REQUIRE(offsets, MOE_ERR_INVALID_VALUE, "moe_grouped_ffn: offsets is required");
  REQUIRE(y_dtype == MOE_F32 || y_dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, "moe_grouped_ffn: y_dtype must be F32 or BF16");
  REQUIRE(x_dtype == w_dtype, MOE_ERR_UNSUPPORTED, "moe_grouped_ffn: x_dtype and w_dtype must match");
  REQUIRE(x_dtype == MOE_F32 || x_dtype == MOE_BF16 || x_dtype == MOE_FP8_E4M3, MOE_ERR_UNSUPPORTED,
          "moe_grouped_ffn: unknown dtype");
  REQUIRE((long long)total_rows * H <= 0x7fffffffffffLL && (long long)n_groups * I * H <= 0x7fffffffffffLL,
          MOE_ERR_UNSUPPORTED, "moe_grouped_ffn: sizes too large");
  if (x_dtype == MOE_BF16)
    REQUIRE(H % 128 == 0 && I % 64 == 0, MOE_ERR_UNSUPPORTED, "moe_grouped_ffn: bf16 needs H % 128 == 0 and I % 64 == 0");
  if (x_dtype == MOE_FP8_E4M3) {
    REQUIRE(H % 128 == 0 && I % 128 == 0, MOE_ERR_UNSUPPORTED, "moe_grouped_ffn: fp8 needs H % 128 == 0 and I % 128 == 0");
    REQUIRE(total_rows == 0 || (X_scales && Wg_scales && Wu_scales && Wd_scales), MOE_ERR_INVALID_VALUE,
            "moe_grouped_ffn: fp8 needs X_scales and all three weight scale arrays");
  }
  REQUIRE(total_rows == 0 || (X && W_gate && W_up && W_down && Y), MOE_ERR_INVALID_VALUE,
          "moe_grouped_ffn: X, W_gate, W_up, W_down and Y are required");
  REQUIRE(total_rows == 0 || x_rows >= 1, MOE_ERR_INVALID_VALUE, "moe_grouped_ffn: rows to compute but X is empty");
  REQUIRE(x_dtype == MOE_F32 || (aligned16(X) && aligned16(W_gate) && aligned16(W_up) && aligned16(W_down)),
          MOE_ERR_UNSUPPORTED, "moe_grouped_ffn: X and the weights must be 16-byte aligned");
  moe_status_t s = check_ws(workspace, workspace_bytes,
                            moe::grouped_ffn_workspace(n_groups, total_rows, H, I, x_dtype), "moe_grouped_ffn");
  if (s != MOE_OK) return s;
  if (total_rows == 0) return ok();
  moe::FfnArgs a{n_groups, offsets, total_rows, row_index, X, X_scales, x_rows, x_dtype, W_gate, W_up,
                 W_down, Wg_scales, Wu_scales, Wd_scales, H, I, Y, y_dtype, workspace, want_zv ? zv : nullptr};
  return hip_status(moe::launch_grouped_ffn(a, as_stream(stream), events), "moe_grouped_ffn");
}

moe_status_t moe_grouped_ffn(int n_groups, const int32_t* offsets, int total_rows,
                             const int32_t* row_index, const void* X, const float* X_scales,
                             int x_rows, int x_dtype, const void* W_gate, const void* W_up,
                             const void* W_down, const float* Wg_scales, const float* Wu_scales,
                             const float* Wd_scales, int w_dtype, int H, int I, void* Y, int y_dtype,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return grouped_ffn_impl(n_groups, offsets, total_rows, row_index, X, X_scales, x_rows, x_dtype, W_gate,
                          W_up, W_down, Wg_scales, Wu_scales, Wd_scales, w_dtype, H, I, Y, y_dtype,
                          workspace, workspace_bytes, stream, nullptr);
}

moe_status_t moe_grouped_ffn_profiled(int n_groups, const int32_t* offsets, int total_rows,
                                      const int32_t* row_index, const void* X, const float* X_scales,
                                      int x_rows, int x_dtype, const void* W_gate, const void* W_up,
                                      const void* W_down, const float* Wg_scales,
                                      const float* Wu_scales, const float* Wd_scales, int w_dtype,
                                      int H, int I, void* Y, int y_dtype, void* workspace,
                                      size_t workspace_bytes, void* stream, void* const* events) {
  return grouped_ffn_impl(n_groups, offsets, total_rows, row_index, X, X_scales, x_rows, x_dtype, W_gate,
                          W_up, W_down, Wg_scales, Wu_scales, Wd_scales, w_dtype, H, I, Y, y_dtype,
                          workspace, workspace_bytes, stream, events);
}

moe_status_t moe_grouped_ffn_train(int n_groups, const int32_t* offsets, int total_rows,
                                   const int32_t* row_index, const void* X, int x_rows, const void* W_gate,
                                   const void* W_up, const void* W_down, int H, int I, void* Y, int y_dtype,
                                   float* zv, void* workspace, size_t workspace_bytes, void* stream,
                                   void* const* events) {
  return grouped_ffn_impl(n_groups, offsets, total_rows, row_index, X, nullptr, x_rows, MOE_BF16, W_gate, W_up,
                          W_down, nullptr, nullptr, nullptr, MOE_BF16, H, I, Y, y_dtype, workspace, workspace_bytes,
                          stream, events, zv, true);
}

// ------------------------------------------------------------------------- combine / bias
moe_status_t moe_combine(const void* u, const void* shared_y, const void* Y,
                         const int32_t* slot_row, const float* topk_gate, int T, int K, int H,
                         int total_rows, int io_dtype, int y_dtype, void* out, void* stream) {
  REQUIRE(T >= 0 && H >= 1 && total_rows >= 0, MOE_ERR_INVALID_VALUE, "moe_combine: need T >= 0, H >= 1, total_rows >= 0");
  REQUIRE(K >= 1 && K <= MOE_MAX_TOPK, MOE_ERR_UNSUPPORTED, "moe_combine: K must be in [1, 16]");
  REQUIRE(io_dtype == MOE_F32 || io_dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, "moe_combine: io_dtype must be F32 or BF16");
  REQUIRE(y_dtype == MOE_F32 || y_dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, "moe_combine: y_dtype must be F32 or BF16");
  REQUIRE(T == 0 || (u && Y && slot_row && topk_gate && out), MOE_ERR_INVALID_VALUE,
          "moe_combine: u, Y, slot_row, topk_gate and out are required");
  if (T == 0) return ok();
  return hip_status(moe::launch_combine(u, shared_y, Y, slot_row, topk_gate, T, K, H, total_rows, io_dtype,
                                        y_dtype, out, as_stream(stream)),
                    "moe_combine");
}

moe_status_t moe_bias_update(const int32_t* counts, int N_r, int T, int K, float gamma, float* bias,
                             void* stream) {
  REQUIRE(N_r >= 1 && N_r <= MOE_MAX_EXPERTS, MOE_ERR_UNSUPPORTED, "moe_bias_update: N_r must be in [1, 1024]");
  REQUIRE(T >= 0 && K >= 1, MOE_ERR_INVALID_VALUE, "moe_bias_update: need T >= 0 and K >= 1");
  REQUIRE(std::isfinite(gamma), MOE_ERR_INVALID_VALUE, "moe_bias_update: gamma must be finite");
  REQUIRE(counts && bias, MOE_ERR_INVALID_VALUE, "moe_bias_update: counts and bias are required");
  return hip_status(moe::launch_bias_update(counts, N_r, T, K, gamma, bias, as_stream(stream)), "moe_bias_update");
}

// ------------------------------------------------------------------------- fp8
moe_status_t fp8_quant_tiles(const void* x, int x_dtype, int rows, int cols, int tile_rows,
                             int tile_cols, uint8_t* codes, float* scales, void* stream) {
  REQUIRE(rows >= 0 && cols >= 0, MOE_ERR_INVALID_VALUE, "fp8_quant_tiles: rows and cols must be >= 0");
  REQUIRE(x_dtype == MOE_F32 || x_dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, "fp8_quant_tiles: x_dtype must be F32 or BF16");
  REQUIRE((tile_rows == 1 || tile_rows == 128) && tile_cols == 128, MOE_ERR_UNSUPPORTED,
          "fp8_quant_tiles: tiles must be 1x128 or 128x128");
  REQUIRE(rows % tile_rows == 0 && cols % 128 == 0, MOE_ERR_UNSUPPORTED,
          "fp8_quant_tiles: rows must be a multiple of tile_rows and cols of 128");
  REQUIRE(tile_rows == 1 || rows / 128 <= 65535, MOE_ERR_UNSUPPORTED, "fp8_quant_tiles: too many block rows");
  REQUIRE((long long)rows * (cols / 128) <= 0x7fffffffLL * 16LL, MOE_ERR_UNSUPPORTED, "fp8_quant_tiles: too many tiles");
  REQUIRE(rows == 0 || cols == 0 || (x && codes && scales), MOE_ERR_INVALID_VALUE,
          "fp8_quant_tiles: x, codes and scales are required");
  REQUIRE(aligned16(x) && aligned16(codes), MOE_ERR_UNSUPPORTED, "fp8_quant_tiles: x and codes must be 16-byte aligned");
  return hip_status(moe::launch_fp8_quant(x, x_dtype, rows, cols, tile_rows, codes, scales, as_stream(stream)),
                    "fp8_quant_tiles");
}

// ------------------------------------------------------------------------- backward
size_t moe_grouped_ffn_backward_workspace_size(int n_groups, int total_rows, int H, int I) {
  if (n_groups <= 0 || total_rows < 0 || H <= 0 || I <= 0) return 0;
  return moe::grouped_ffn_backward_workspace(n_groups, total_rows, H, I);
}

static moe_status_t ffn_backward_impl(int n_groups, const int32_t* offsets, int total_rows, const int32_t* row_index,
                                      const void* X, int x_rows, const void* W_gate, const void* W_up,
                                      const void* W_down, const void* dY, int H, int I, float* dX, float* dW_gate,
                                      float* dW_up, float* dW_down, void* workspace, size_t workspace_bytes,
                                      void* stream, void* const* events, const float* zv = nullptr,
                                      bool want_zv = false) {
  const char* fn = want_zv ? "moe_grouped_ffn_backward_saved" : "moe_grouped_ffn_backward";
  REQUIRE(!want_zv || total_rows == 0 || zv, MOE_ERR_INVALID_VALUE, std::string(fn) + ": zv is required");
  REQUIRE(n_groups >= 1 && n_groups <= MOE_MAX_EXPERTS, MOE_ERR_UNSUPPORTED,
          std::string(fn) + ": n_groups must be in [1, 1024]");
  REQUIRE(total_rows >= 0 && x_rows >= 0 && H >= 1 && I >= 1, MOE_ERR_INVALID_VALUE,
          std::string(fn) + ": need total_rows >= 0, x_rows >= 0, H >= 1, I >= 1");
  REQUIRE(H % 128 == 0 && I % 128 == 0, MOE_ERR_UNSUPPORTED, std::string(fn) + ": needs H % 128 == 0 and I % 128 == 0");
  REQUIRE((long long)total_rows * 2 * I <= 0x7fffffffffffLL && (long long)n_groups * I * H <= 0x7fffffffffffLL,
          MOE_ERR_UNSUPPORTED, std::string(fn) + ": sizes too large");
  REQUIRE((long long)n_groups * (H / 128) * (I / 128) <= 0x7fffffffLL, MOE_ERR_UNSUPPORTED,
          std::string(fn) + ": too many weight-gradient tiles");
  REQUIRE(offsets && W_gate && W_up && W_down && dW_gate && dW_up && dW_down, MOE_ERR_INVALID_VALUE,
          std::string(fn) + ": offsets, the weights and the weight gradients are required");
  REQUIRE(total_rows == 0 || (X && dY && dX && x_rows >= 1), MOE_ERR_INVALID_VALUE,
          std::string(fn) + ": X, dY and dX are required when there are rows");
  REQUIRE(aligned16(X) && aligned16(W_gate) && aligned16(W_up) && aligned16(W_down) && aligned16(dY),
          MOE_ERR_UNSUPPORTED, std::string(fn) + ": X, dY and the weights must be 16-byte aligned");
  moe_status_t s = check_ws(workspace, workspace_bytes, moe::grouped_ffn_backward_workspace(n_groups, total_rows, H, I), fn);
  if (s != MOE_OK) return s;
  moe::FfnBwdArgs a{n_groups, offsets, total_rows, row_index, X, x_rows, W_gate, W_up, W_down, dY,
                    dX, dW_gate, dW_up, dW_down, H, I, workspace, want_zv ? zv : nullptr};
  return hip_status(moe::launch_grouped_ffn_backward(a, as_stream(stream), events), fn);
}

moe_status_t moe_grouped_ffn_backward(int n_groups, const int32_t* offsets, int total_rows, const int32_t* row_index,
                                      const void* X, int x_rows, const void* W_gate, const void* W_up,
                                      const void* W_down, const void* dY, int H, int I, float* dX, float* dW_gate,
                                      float* dW_up, float* dW_down, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  return ffn_backward_impl(n_groups, offsets, total_rows, row_index, X, x_rows, W_gate, W_up, W_down, dY, H, I, dX,
                           dW_gate, dW_up, dW_down, workspace, workspace_bytes, stream, nullptr);
}

moe_status_t moe_grouped_ffn_backward_profiled(int n_groups, const int32_t* offsets, int total_rows,
                                               const int32_t* row_index, const void* X, int x_rows,
                                               const void* W_gate, const void* W_up, const void* W_down,
                                               const void* dY, int H, int I, float* dX, float* dW_gate,
                                               float* dW_up, float* dW_down, void* workspace,
                                               size_t workspace_bytes, void* stream, void* const* events) {
  REQUIRE(events, MOE_ERR_INVALID_VALUE, "moe_grouped_ffn_backward_profiled: events is required");
  return ffn_backward_impl(n_groups, offsets, total_rows, row_index, X, x_rows, W_gate, W_up, W_down, dY, H, I, dX,
                           dW_gate, dW_up, dW_down, workspace, workspace_bytes, stream, events);
}

moe_status_t moe_grouped_ffn_backward_saved(int n_groups, const int32_t* offsets, int total_rows,
                                            const int32_t* row_index, const void* X, int x_rows,
                                            const void* W_gate, const void* W_up, const void* W_down,
                                            const void* dY, const float* zv, int H, int I, float* dX,
                                            float* dW_gate, float* dW_up, float* dW_down, void* workspace,
                                            size_t workspace_bytes, void* stream, void* const* events) {
  return ffn_backward_impl(n_groups, offsets, total_rows, row_index, X, x_rows, W_gate, W_up, W_down, dY, H, I, dX,
                           dW_gate, dW_up, dW_down, workspace, workspace_bytes, stream, events, zv, true);
}

moe_status_t moe_fp8_transpose_weights(int n_groups, int H, int I, const uint8_t* W_gate, const float* Wg_scales,
                                       const uint8_t* W_up, const float* Wu_scales, const uint8_t* W_down,
                                       const float* Wd_scales, uint8_t* W_down_t, float* Wd_t_scales,
                                       uint8_t* W_gate_up_t, float* Wgu_t_scales, void* stream) {
  const char* fn = "moe_fp8_transpose_weights";
  REQUIRE(n_groups >= 0 && H >= 1 && I >= 1, MOE_ERR_INVALID_VALUE, std::string(fn) + ": need n_groups >= 0, H, I >= 1");
  REQUIRE(H % 128 == 0 && I % 128 == 0, MOE_ERR_UNSUPPORTED, std::string(fn) + ": needs H % 128 == 0 and I % 128 == 0");
  REQUIRE(n_groups == 0 || (W_gate && Wg_scales && W_up && Wu_scales && W_down && Wd_scales && W_down_t && Wd_t_scales &&
                            W_gate_up_t && Wgu_t_scales),
          MOE_ERR_INVALID_VALUE, std::string(fn) + ": every pointer is required");
  REQUIRE(aligned16(W_gate) && aligned16(W_up) && aligned16(W_down) && aligned16(W_down_t) && aligned16(W_gate_up_t),
          MOE_ERR_UNSUPPORTED, std::string(fn) + ": the codes must be 16-byte aligned");
  REQUIRE((long long)n_groups * H * I <= 0x7fffffffffffLL, MOE_ERR_UNSUPPORTED, std::string(fn) + ": sizes too large");
  moe::Fp8TransposeArgs a{n_groups, H, I, W_gate, W_up, W_down, Wg_scales, Wu_scales, Wd_scales,
                          W_down_t, W_gate_up_t, Wd_t_scales, Wgu_t_scales};
  return hip_status(moe::launch_fp8_transpose_weights(a, as_stream(stream)), fn);
}

size_t moe_grouped_ffn_backward_fp8_workspace_size(int n_groups, int total_rows, int H, int I) {
  if (n_groups <= 0 || total_rows < 0 || H <= 0 || I <= 0 || H % 128 || I % 128) return 0;
  return moe::grouped_ffn_backward_fp8_workspace(n_groups, total_rows, H, I);
}

moe_status_t moe_grouped_ffn_backward_fp8(int n_groups, const int32_t* offsets, int total_rows,
                                          const int32_t* row_index, const void* X, int x_rows,
                                          const uint8_t* W_gate, const float* Wg_scales, const uint8_t* W_up,
                                          const float* Wu_scales, const uint8_t* W_down_t, const float* Wd_t_scales,
                                          const uint8_t* W_gate_up_t, const float* Wgu_t_scales, const void* dY,
                                          int H, int I, float* dX, float* dW_gate, float* dW_up, float* dW_down,
                                          void* workspace, size_t workspace_bytes, void* stream,
                                          void* const* events) {
  const char* fn = "moe_grouped_ffn_backward_fp8";
  REQUIRE(n_groups >= 1 && n_groups <= MOE_MAX_EXPERTS + 1, MOE_ERR_UNSUPPORTED,
          std::string(fn) + ": n_groups must be in [1, 1025]");
  REQUIRE(total_rows >= 0 && x_rows >= 0 && H >= 1 && I >= 1, MOE_ERR_INVALID_VALUE,
          std::string(fn) + ": need total_rows >= 0, x_rows >= 0, H >= 1, I >= 1");
  REQUIRE(H % 128 == 0 && I % 128 == 0, MOE_ERR_UNSUPPORTED, std::string(fn) + ": needs H % 128 == 0 and I % 128 == 0");
  REQUIRE(H <= 16384 && I <= 8192, MOE_ERR_UNSUPPORTED, std::string(fn) + ": needs H <= 16384 and I <= 8192");
  REQUIRE((long long)total_rows * 2 * I <= 0x7fffffffffffLL && (long long)n_groups * I * H <= 0x7fffffffffffLL &&
              (long long)total_rows + 128LL * n_groups <= 0x7fffffffLL,
          MOE_ERR_UNSUPPORTED, std::string(fn) + ": sizes too large");
  REQUIRE((long long)n_groups * (H / 128) * (I / 128) <= 0x7fffffffLL, MOE_ERR_UNSUPPORTED,
          std::string(fn) + ": too many weight-gradient tiles");
  REQUIRE(offsets && W_gate && Wg_scales && W_up && Wu_scales && W_down_t && Wd_t_scales && W_gate_up_t &&
              Wgu_t_scales && dW_gate && dW_up && dW_down,
          MOE_ERR_INVALID_VALUE, std::string(fn) + ": offsets, the weights, their scales and the weight gradients are required");
  REQUIRE(total_rows == 0 || (X && dY && dX && x_rows >= 1), MOE_ERR_INVALID_VALUE,
          std::string(fn) + ": X, dY and dX are required when there are rows");
  REQUIRE(aligned16(X) && aligned16(dY) && aligned16(W_gate) && aligned16(W_up) && aligned16(W_down_t) &&
              aligned16(W_gate_up_t) && aligned16(dX),
          MOE_ERR_UNSUPPORTED, std::string(fn) + ": X, dY, dX and the weight codes must be 16-byte aligned");
  moe_status_t s = check_ws(workspace, workspace_bytes, moe::grouped_ffn_backward_fp8_workspace(n_groups, total_rows, H, I), fn);
  if (s != MOE_OK) return s;
  moe::FfnBwdFp8Args a{n_groups, offsets, total_rows, row_index, X, x_rows, W_gate, W_up, W_down_t, W_gate_up_t,
                       Wg_scales, Wu_scales, Wd_t_scales, Wgu_t_scales, dY, dX, dW_gate, dW_up, dW_down, H, I, workspace};
  return hip_status(moe::launch_grouped_ffn_backward_fp8(a, as_stream(stream), events), fn);
}

moe_status_t moe_combine_backward(const void* dout, int io_dtype, const void* Y, int y_dtype, const int32_t* slot_row,
                                  const float* topk_gate, int T, int K, int H, int shared_rows, int total_rows,
                                  void* dY, float* dgate, void* stream) {
  const char* fn = "moe_combine_backward";
  REQUIRE(T >= 0 && H >= 1 && shared_rows >= 0 && total_rows >= 0, MOE_ERR_INVALID_VALUE,
          std::string(fn) + ": need T >= 0, H >= 1, shared_rows >= 0, total_rows >= 0");
  REQUIRE(K >= 1 && K <= MOE_MAX_TOPK, MOE_ERR_UNSUPPORTED, std::string(fn) + ": K must be in [1, 16]");
  REQUIRE(shared_rows == 0 || shared_rows == T, MOE_ERR_UNSUPPORTED,
          std::string(fn) + ": shared_rows must be 0 or T (the shared expert's identity rows)");
  REQUIRE((io_dtype == MOE_F32 || io_dtype == MOE_BF16) && (y_dtype == MOE_F32 || y_dtype == MOE_BF16),
          MOE_ERR_UNSUPPORTED, std::string(fn) + ": dtypes must be F32 or BF16");
  REQUIRE(T == 0 || (dout && Y && slot_row && topk_gate && dY && dgate), MOE_ERR_INVALID_VALUE,
          std::string(fn) + ": every pointer is required");
  return hip_status(moe::launch_combine_backward(dout, io_dtype, Y, y_dtype, slot_row, topk_gate, T, K, H, shared_rows,
                                                 total_rows, static_cast<uint16_t*>(dY), dgate, as_stream(stream)),
                    fn);
}

size_t moe_router_backward_workspace_size(int total_rows) {
  return total_rows <= 0 ? 0 : (((size_t)total_rows * sizeof(float) + 255) & ~(size_t)255);
}

moe_status_t moe_router_backward(const void* dout, const void* u, int io_dtype, const float* dX_rows,
                                 const int32_t* offsets, const int32_t* row_token, const int32_t* slot_row,
                                 int shared_rows, int total_rows, const float* affinity, const int32_t* topk_idx,
                                 const float* topk_gate, const float* dgate, const float* centroids, int T, int K,
                                 int H, int N_r, float* du, float* dcentroids, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  const char* fn = "moe_router_backward";
  REQUIRE(T >= 0 && H >= 1 && total_rows >= 0, MOE_ERR_INVALID_VALUE, std::string(fn) + ": need T >= 0, H >= 1");
  REQUIRE(N_r >= 1 && N_r <= MOE_MAX_EXPERTS, MOE_ERR_UNSUPPORTED, std::string(fn) + ": N_r must be in [1, 1024]");
  REQUIRE(K >= 1 && K <= N_r && K <= MOE_MAX_TOPK, MOE_ERR_UNSUPPORTED, std::string(fn) + ": K must be in [1, min(N_r, 16)]");
  REQUIRE(shared_rows == 0 || shared_rows == T, MOE_ERR_UNSUPPORTED, std::string(fn) + ": shared_rows must be 0 or T");
  REQUIRE(io_dtype == MOE_F32 || io_dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, std::string(fn) + ": io_dtype must be F32 or BF16");
  REQUIRE(offsets && centroids && dcentroids, MOE_ERR_INVALID_VALUE,
          std::string(fn) + ": offsets, centroids and dcentroids are required");
  REQUIRE(T == 0 || (dout && u && dX_rows && row_token && slot_row && affinity && topk_idx && topk_gate && dgate && du),
          MOE_ERR_INVALID_VALUE, std::string(fn) + ": every per-token pointer is required");
  moe_status_t s = check_ws(workspace, workspace_bytes, moe_router_backward_workspace_size(total_rows), fn);
  if (s != MOE_OK) return s;
  return hip_status(moe::launch_router_backward(dout, u, io_dtype, dX_rows, offsets, shared_rows > 0 ? 1 : 0, row_token,
                                                slot_row, shared_rows, total_rows, affinity, topk_idx, topk_gate,
                                                dgate, centroids, T, K, H, N_r, du, dcentroids,
                                                static_cast<float*>(workspace), as_stream(stream)),
                    fn);
}

// ------------------------------------------------------------------------- balance loss
size_t moe_seq_balance_loss_workspace_size(int T, int N_r, int seq_len) {
  if (T <= 0 || N_r <= 0 || seq_len <= 0) return 0;
  return moe::seq_balance_workspace(T, N_r, seq_len);
}

moe_status_t moe_seq_balance_loss(const float* affinity, const int32_t* topk_idx, int T, int N_r, int K, int seq_len,
                                  float alpha, float* loss, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "moe_seq_balance_loss";
  REQUIRE(T >= 0, MOE_ERR_INVALID_VALUE, std::string(fn) + ": T must be >= 0");
  REQUIRE(N_r >= 1 && N_r <= MOE_MAX_EXPERTS, MOE_ERR_UNSUPPORTED, std::string(fn) + ": N_r must be in [1, 1024]");
  REQUIRE(K >= 1 && K <= N_r && K <= MOE_MAX_TOPK, MOE_ERR_UNSUPPORTED, std::string(fn) + ": K must be in [1, min(N_r, 16)]");
  REQUIRE(seq_len >= 1 && seq_len <= 16384, MOE_ERR_UNSUPPORTED, std::string(fn) + ": seq_len must be in [1, 16384]");
  REQUIRE(std::isfinite(alpha), MOE_ERR_INVALID_VALUE, std::string(fn) + ": alpha must be finite");
  REQUIRE(T == 0 || (affinity && topk_idx && loss), MOE_ERR_INVALID_VALUE, std::string(fn) + ": every pointer is required");
  moe_status_t s = check_ws(workspace, workspace_bytes, moe::seq_balance_workspace(T, N_r, seq_len), fn);
  if (s != MOE_OK) return s;
  return hip_status(moe::launch_seq_balance_loss(affinity, topk_idx, T, N_r, K, seq_len, alpha, loss, workspace,
                                                 as_stream(stream)),
                    fn);
}

// ------------------------------------------------------------------------- EP dispatch payload
size_t moe_pack_fp8_payload_workspace_size(int T, int K, int n_ranks) {
  if (T < 0 || K <= 0 || n_ranks <= 0) return 0;
  return moe::payload_workspace(T, K, n_ranks);
}

moe_status_t moe_pack_fp8_payload(const void* x, int x_dtype, int T, int H, const int32_t* topk_idx, int K,
                                  int N_r, int n_ranks, int32_t* counts, int32_t* offsets, int32_t* send_token,
                                  int32_t* slot_send, uint8_t* codes, float* scales, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  REQUIRE(T >= 0 && H >= 0, MOE_ERR_INVALID_VALUE, "moe_pack_fp8_payload: T and H must be >= 0");
  REQUIRE(N_r >= 1 && N_r <= MOE_MAX_EXPERTS, MOE_ERR_UNSUPPORTED, "moe_pack_fp8_payload: N_r must be in [1, 1024]");
  REQUIRE(K >= 1 && K <= MOE_MAX_TOPK, MOE_ERR_UNSUPPORTED, "moe_pack_fp8_payload: K must be in [1, 16]");
  REQUIRE(n_ranks >= 1 && N_r % n_ranks == 0, MOE_ERR_UNSUPPORTED, "moe_pack_fp8_payload: n_ranks must divide N_r");
  REQUIRE(H % 128 == 0, MOE_ERR_UNSUPPORTED, "moe_pack_fp8_payload: H must be a multiple of 128");
  REQUIRE(x_dtype == MOE_F32 || x_dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, "moe_pack_fp8_payload: x_dtype must be F32 or BF16");
  REQUIRE((long long)T * K <= 0x7fffffffLL, MOE_ERR_UNSUPPORTED, "moe_pack_fp8_payload: T * K overflows int32");
  REQUIRE(counts && offsets, MOE_ERR_INVALID_VALUE, "moe_pack_fp8_payload: counts and offsets are required");
  REQUIRE(T == 0 || (topk_idx && send_token && slot_send), MOE_ERR_INVALID_VALUE,
          "moe_pack_fp8_payload: topk_idx, send_token and slot_send are required");
  REQUIRE(T == 0 || H == 0 || (x && codes && scales), MOE_ERR_INVALID_VALUE,
          "moe_pack_fp8_payload: x, codes and scales are required");
  REQUIRE(aligned16(x) && aligned16(codes), MOE_ERR_UNSUPPORTED, "moe_pack_fp8_payload: x and codes must be 16-byte aligned");
  moe_status_t s = check_ws(workspace, workspace_bytes, moe::payload_workspace(T, K, n_ranks), "moe_pack_fp8_payload");
  if (s != MOE_OK) return s;
  return hip_status(moe::launch_pack_fp8_payload(x, x_dtype, T, H, topk_idx, K, N_r, n_ranks, counts, offsets,
                                                 send_token, slot_send, codes, scales, workspace, as_stream(stream)),
                    "moe_pack_fp8_payload");
}

moe_status_t moe_unpack_fp8_payload(const uint8_t* codes, const float* scales, int rows, int H, void* out,
                                    int out_dtype, void* stream) {
  REQUIRE(rows >= 0 && H >= 0, MOE_ERR_INVALID_VALUE, "moe_unpack_fp8_payload: rows and H must be >= 0");
  REQUIRE(H % 128 == 0, MOE_ERR_UNSUPPORTED, "moe_unpack_fp8_payload: H must be a multiple of 128");
  REQUIRE(out_dtype == MOE_F32 || out_dtype == MOE_BF16, MOE_ERR_UNSUPPORTED,
          "moe_unpack_fp8_payload: out_dtype must be F32 or BF16");
  REQUIRE((long long)rows * (H / 128) <= 0x7fffffffLL * 16LL, MOE_ERR_UNSUPPORTED, "moe_unpack_fp8_payload: too many tiles");
  REQUIRE(rows == 0 || H == 0 || (codes && scales && out), MOE_ERR_INVALID_VALUE,
          "moe_unpack_fp8_payload: codes, scales and out are required");
  REQUIRE(((uintptr_t)codes & 7) == 0, MOE_ERR_UNSUPPORTED, "moe_unpack_fp8_payload: codes must be 8-byte aligned");
  return hip_status(moe::launch_unpack_fp8_payload(codes, scales, rows, H, out, out_dtype, as_stream(stream)),
                    "moe_unpack_fp8_payload");
}

}  // extern "C"
