// iq_api.hip -- the C ABI of libiq.so (declared in include/iq.h): host-side
// validation, workspace queries, then the launches.  No entry point allocates
// device memory or synchronises the stream; every size a launch depends on is
// checked before the first kernel is enqueued.

#include <atomic>
#include <mutex>

#include "iq.h"
#include "iq_common.hpp"
#include "iq_internal.hpp"

// Scratch of iq_quantize_noalloc, for callers that cannot allocate.  Each
// device the library runs on holds its own copy until the process ends.  Host
// code never uses the array's name as an address (on the host it names a
// stand-in, not device memory): it uses the device address that
// hipGetSymbolAddress returns, looked up once per device.
static __device__ __align__(256) unsigned char scratch[IQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_dev[kMaxDevices];  // device address of `scratch` per device, once known
std::mutex g_scratch_mu;

// The current device's address of `scratch` (nullptr on a HIP error).
void *noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void *p = g_scratch_dev[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_dev[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_dev[dev].store(p, std::memory_order_release);
  }
  return p;
}

struct FmtRow {
  int block_bytes, grid_size, choice_groups, num_choices, groups_per_choice;
};
// ModelOpt PR #2513 (sizes, grids) and "[1/5] Let the GGML IQ encoders take
// fixed per-group choices" (choice units and their ranges).
constexpr FmtRow kFmt[5] = {
    {66, 256, 8, 16, 4},   // IQ2_XXS
    {74, 512, 16, 16, 2},  // IQ2_XS
    {82, 1024, 16, 16, 2}, // IQ2_S
    {50, 2048, 8, 16, 4},  // IQ1_S
    {56, 2048, 16, 8, 2},  // IQ1_M
};

constexpr int64_t kMaxGrid = (int64_t(1) << 31) - 1;  // workgroups in one grid dimension

bool bad_fmt(int fmt) { return fmt < 0 || fmt > 4; }
bool bad_dtype(int dt) { return dt != IQ_DTYPE_F32 && dt != IQ_DTYPE_BF16; }
bool fits(int64_t wgs) { return wgs >= 0 && wgs <= kMaxGrid; }

// Shape checks shared by the encoder entry points and their workspace queries.
int check_encode_shape(int64_t rows, int64_t cols, int64_t rpe, int fmt, int64_t units_per_wg_col) {
  if (rows < 0 || cols <= 0 || cols % 256 != 0) return IQ_ERR_SHAPE;
  if (rpe < 1 || rows % rpe != 0) return IQ_ERR_SHAPE;
  if (cols / 256 > (int64_t(1) << 24) || rows > (int64_t(1) << 40)) return IQ_ERR_SHAPE;
  const int64_t E = rows / rpe, nb = cols / 256;
  if (rows > (int64_t(1) << 40) / nb) return IQ_ERR_SHAPE;  // blocks: keeps the products below in range
  // search workgroups: experts x 64-row tiles x column sets
  if (!fits(E * ((rpe + 63) / 64) * nb * units_per_wg_col)) return IQ_ERR_SHAPE;
  // norm-table, importance-check and anchor launches
  const int64_t gblocks = (E * (cols / 8) * kFmt[fmt].grid_size + 255) / 256;
  if (!fits(gblocks + (E * nb + 3) / 4) || !fits((rows * nb + 7) / 8)) return IQ_ERR_SHAPE;
  return IQ_OK;
}

// search workgroups per block column: 32 groups over the groups per workgroup
// (eight for IQ2_XXS, IQ2_XS and IQ1_M, four for IQ2_S and IQ1_S)
int64_t wg_cols(int fmt) { return (fmt == IQ_FMT_IQ2_S || fmt == IQ_FMT_IQ1_S) ? 8 : 4; }

int check_workspace(size_t need, const void *ws, size_t ws_bytes) {
  if (need == 0) return IQ_OK;
  if (!ws) return IQ_ERR_NULL;
  if (ws_bytes < need) return IQ_ERR_WORKSPACE;
  return IQ_OK;
}

int check_collect_args(int dtype, int64_t T, int64_t K, const int32_t *ids, int top_k, int num_experts,
                       int chunk_rows) {
  if (bad_dtype(dtype)) return IQ_ERR_DTYPE;
  if (T < 0 || K <= 0 || num_experts < 1 || chunk_rows < 1) return IQ_ERR_ARG;
  if (ids && top_k < 1) return IQ_ERR_ARG;
  if (!ids && num_experts != 1 && T != 0) return IQ_ERR_ARG;  // no tokens: ids may be NULL
  if (static_cast<int64_t>(num_experts) * K > (int64_t(1) << 40)) return IQ_ERR_ARG;
  return IQ_OK;
}

int check_collect_grids(int64_t T, int64_t K, bool routed, int E, int chunk_rows) {
  if (T == 0) return IQ_OK;
  const iq::CollectPlan P = iq::plan_collect(T, K, routed, E, chunk_rows);
  if (!fits(P.wchunks * P.nsub * E * P.ntile) || !fits((static_cast<int64_t>(E) * K + 255) / 256) ||
      !fits(P.wchunks * ((chunk_rows + 255) / 256)))
    return IQ_ERR_ARG;
  return IQ_OK;
}

int check_hessian_args(int dtype, int64_t T, int64_t K, const int32_t *ids, int top_k, int num_experts,
                       int chunk_rows) {
  const int rc = check_collect_args(dtype, T, K, ids, top_k, num_experts, chunk_rows);
  if (rc != IQ_OK) return rc;
  if (K % 256 != 0) return IQ_ERR_SHAPE;
  if (static_cast<int64_t>(num_experts) * K > (int64_t(1) << 30) || T > (int64_t(1) << 31) - 1) return IQ_ERR_ARG;
  if (T == 0) return IQ_OK;
  const iq::HessPlan P = iq::plan_hessian(T, K, ids ? top_k : 0, num_experts, chunk_rows);
  const int64_t nb = K / 256, per_e = nb * 65536;
  if (ids) {
    if (!fits(P.smax * nb * 10) || !fits(P.hmax * ((per_e + 255) / 256)) ||
        !fits(P.nchunks * ((chunk_rows + 255) / 256)) || T * top_k > (int64_t(1) << 32))
      return IQ_ERR_ARG;
  } else if (!fits(num_experts * nb * 10 * P.nsplit)) {
    return IQ_ERR_ARG;
  }
  return IQ_OK;
}

iq::EncArgs enc_args(const void *w, int dtype, int64_t rows, int64_t cols, int64_t rpe, const float *grid,
                     const float *importance, int32_t *status) {
  iq::EncArgs A{};
  A.w = w;
  A.dtype = dtype;
  A.rows = rows;
  A.cols = cols;
  A.rpe = rpe;
  A.E = rows / rpe;
  A.nb = static_cast<int>(cols / 256);
  A.grid = grid;
  A.imp = importance;
  A.status = status;
  return A;
}

int quantize_common(int fmt, const void *w, int dtype, int64_t rows, int64_t cols, int64_t rows_per_expert,
                    const float *grid, const float *importance, const uint8_t *choices, uint8_t *out,
                    void *workspace, size_t workspace_bytes, int32_t *status, bool every, hipEvent_t ev0,
                    hipEvent_t ev1, hipStream_t stream) {
  if (bad_fmt(fmt)) return IQ_ERR_FMT;
  if (bad_dtype(dtype)) return IQ_ERR_DTYPE;
  if (!grid || (rows != 0 && (!w || !out))) return IQ_ERR_NULL;
  int rc = check_encode_shape(rows, cols, rows_per_expert, fmt, wg_cols(fmt));
  if (rc != IQ_OK) return rc;
  const size_t need = rows ? iq::plan_quantize(fmt, rows, cols, rows_per_expert, importance != nullptr).bytes : 0;
  if ((rc = check_workspace(need, workspace, workspace_bytes)) != IQ_OK) return rc;
  iq::EncArgs A = enc_args(w, dtype, rows, cols, rows_per_expert, grid, importance, status);
  A.choices = choices;
  A.out = out;
  A.copies = every ? kFmt[fmt].num_choices : 1;
  A.copy_stride = rows * (cols / 256) * kFmt[fmt].block_bytes;
  return iq::launch_quantize(fmt, A, every, workspace, ev0, ev1, stream) == 0 ? IQ_OK : IQ_ERR_HIP;
}

}  // namespace

extern "C" {

int iq_format_info(int fmt, iq_format_info_t *out) {
  if (bad_fmt(fmt)) return IQ_ERR_FMT;
  if (!out) return IQ_ERR_NULL;
  out->block_values = 256;
  out->block_bytes = kFmt[fmt].block_bytes;
  out->grid_size = kFmt[fmt].grid_size;
  out->choice_groups = kFmt[fmt].choice_groups;
  out->num_choices = kFmt[fmt].num_choices;
  out->groups_per_choice = kFmt[fmt].groups_per_choice;
  return IQ_OK;
}

int iq_imatrix_collect_workspace_size(int64_t T, int64_t K, int top_k, int num_experts, int chunk_rows,
                                      size_t *bytes) {
  if (!bytes) return IQ_ERR_NULL;
  if (T < 0 || K <= 0 || num_experts < 1 || chunk_rows < 1 || top_k < 0) return IQ_ERR_ARG;
  if (static_cast<int64_t>(num_experts) * K > (int64_t(1) << 40)) return IQ_ERR_ARG;
  *bytes = T ? iq::plan_collect(T, K, top_k > 0, num_experts, chunk_rows).bytes : 0;
  return IQ_OK;
}

int iq_imatrix_collect(const void *x, int dtype, int64_t T, int64_t K, const int32_t *ids, int top_k,
                       int num_experts, int chunk_rows, float *sums, int64_t *counts, void *workspace,
                       size_t workspace_bytes, int32_t *status, hipStream_t stream) {
  int rc = check_collect_args(dtype, T, K, ids, top_k, num_experts, chunk_rows);
  if (rc != IQ_OK) return rc;
  if (!sums || !counts || (T != 0 && !x)) return IQ_ERR_NULL;
  if ((rc = check_collect_grids(T, K, ids != nullptr, num_experts, chunk_rows)) != IQ_OK) return rc;
  const size_t need = T ? iq::plan_collect(T, K, ids != nullptr, num_experts, chunk_rows).bytes : 0;
  if ((rc = check_workspace(need, workspace, workspace_bytes)) != IQ_OK) return rc;
  return iq::launch_collect(x, dtype, T, K, ids, ids ? top_k : 0, num_experts, chunk_rows, sums, counts, status,
                            workspace, stream) == 0
             ? IQ_OK
             : IQ_ERR_HIP;
}

int iq_hessian_collect_workspace_size(int64_t T, int64_t K, int top_k, int num_experts, int chunk_rows,
                                      size_t *bytes) {
  if (!bytes) return IQ_ERR_NULL;
  if (T < 0 || K <= 0 || num_experts < 1 || chunk_rows < 1 || top_k < 0) return IQ_ERR_ARG;
  if (K % 256 != 0) return IQ_ERR_SHAPE;
  if (static_cast<int64_t>(num_experts) * K > (int64_t(1) << 30) || T > (int64_t(1) << 31) - 1) return IQ_ERR_ARG;
  *bytes = T ? iq::plan_hessian(T, K, top_k, num_experts, chunk_rows).bytes : 0;
  return IQ_OK;
}

int iq_hessian_collect(const void *x, int dtype, int64_t T, int64_t K, const int32_t *ids, int top_k,
                       int num_experts, int chunk_rows, float *hess, void *workspace, size_t workspace_bytes,
                       int32_t *status, hipStream_t stream) {
  int rc = check_hessian_args(dtype, T, K, ids, top_k, num_experts, chunk_rows);
  if (rc != IQ_OK) return rc;
  if (!hess || (T != 0 && !x)) return IQ_ERR_NULL;
  const size_t need = T ? iq::plan_hessian(T, K, ids ? top_k : 0, num_experts, chunk_rows).bytes : 0;
  if ((rc = check_workspace(need, workspace, workspace_bytes)) != IQ_OK) return rc;
  return iq::launch_hessian(x, dtype, T, K, ids, ids ? top_k : 0, num_experts, chunk_rows, hess, status, workspace,
                            stream) == 0
             ? IQ_OK
             : IQ_ERR_HIP;
}

int iq_imatrix_importance(const float *sums, const int64_t *counts, int num_experts, int64_t K, float floor_rel,
                          float *importance, int32_t *status, hipStream_t stream) {
  if (!sums || !counts || !importance) return IQ_ERR_NULL;
  if (num_experts < 1 || K <= 0 || !(floor_rel >= 0.0f) || floor_rel > 3.0e38f) return IQ_ERR_ARG;
  return iq::launch_importance(sums, counts, num_experts, K, floor_rel, importance, status, stream) == 0
             ? IQ_OK
             : IQ_ERR_HIP;
}

int iq_imatrix_merge(const float *src_sums, const int64_t *src_counts, int num_experts, int64_t K, float *sums,
                     int64_t *counts, int32_t *status, hipStream_t stream) {
  if (!src_sums || !src_counts || !sums || !counts) return IQ_ERR_NULL;
  if (num_experts < 1 || K <= 0) return IQ_ERR_ARG;
  const int64_t n = static_cast<int64_t>(num_experts) * K;
  if (n / 256 >= (int64_t(1) << 31)) return IQ_ERR_ARG;
  // in place: the sources may not overlap the accumulators
  auto overlap = [](const void *a, const void *b, int64_t bytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + bytes && y < x + bytes;
  };
  if (overlap(src_sums, sums, n * static_cast<int64_t>(sizeof(float))) ||
      overlap(src_counts, counts, num_experts * static_cast<int64_t>(sizeof(int64_t))))
    return IQ_ERR_ARG;
  return iq::launch_merge(src_sums, src_counts, num_experts, K, sums, counts, status, stream) == 0 ? IQ_OK
                                                                                                 : IQ_ERR_HIP;
}

int iq_quantize_workspace_size(int fmt, int64_t rows, int64_t cols, int64_t rows_per_expert, int weighted,
                               size_t *bytes) {
  if (bad_fmt(fmt)) return IQ_ERR_FMT;
  if (!bytes) return IQ_ERR_NULL;
  const int rc = check_encode_shape(rows, cols, rows_per_expert, fmt, wg_cols(fmt));
  if (rc != IQ_OK) return rc;
  *bytes = rows ? iq::plan_quantize(fmt, rows, cols, rows_per_expert, weighted != 0).bytes : 0;
  return IQ_OK;
}

int iq_quantize(int fmt, const void *w, int dtype, int64_t rows, int64_t cols, int64_t rows_per_expert,
                const float *grid, const float *importance, const uint8_t *choices, uint8_t *out, void *workspace,
                size_t workspace_bytes, int32_t *status, hipStream_t stream) {
  return quantize_common(fmt, w, dtype, rows, cols, rows_per_expert, grid, importance, choices, out, workspace,
                         workspace_bytes, status, false, nullptr, nullptr, stream);
}

int iq_quantize_noalloc(int fmt, const void *w, int dtype, int64_t rows, int64_t cols, int64_t rows_per_expert,
                        const float *grid, const float *importance, const uint8_t *choices, uint8_t *out,
                        int32_t *status, hipStream_t stream) {
  // the host checks of iq_quantize first, so a bad call never touches HIP
  if (bad_fmt(fmt)) return IQ_ERR_FMT;
  if (bad_dtype(dtype)) return IQ_ERR_DTYPE;
  if (!grid || (rows != 0 && (!w || !out))) return IQ_ERR_NULL;
  const int rc = check_encode_shape(rows, cols, rows_per_expert, fmt, wg_cols(fmt));
  if (rc != IQ_OK) return rc;
  if (rows == 0) return IQ_OK;
  if (iq::plan_quantize(fmt, rows, cols, rows_per_expert, importance != nullptr).bytes > IQ_NOALLOC_SCRATCH_BYTES)
    return IQ_ERR_WORKSPACE;
  void *ws = noalloc_scratch();
  if (!ws) return IQ_ERR_HIP;
  return quantize_common(fmt, w, dtype, rows, cols, rows_per_expert, grid, importance, choices, out, ws,
                         IQ_NOALLOC_SCRATCH_BYTES, status, false, nullptr, nullptr, stream);
}

int iq_quantize_timed(int fmt, const void *w, int dtype, int64_t rows, int64_t cols, int64_t rows_per_expert,
                      const float *grid, const float *importance, const uint8_t *choices, uint8_t *out,
                      void *workspace, size_t workspace_bytes, int32_t *status, hipEvent_t search_start,
                      hipEvent_t search_stop, hipStream_t stream) {
  if (!search_start || !search_stop) return IQ_ERR_NULL;
  return quantize_common(fmt, w, dtype, rows, cols, rows_per_expert, grid, importance, choices, out, workspace,
                         workspace_bytes, status, false, search_start, search_stop, stream);
}

int iq_quantize_every_choice(int fmt, const void *w, int dtype, int64_t rows, int64_t cols, int64_t rows_per_expert,
                             const float *grid, const float *importance, uint8_t *out, void *workspace,
                             size_t workspace_bytes, int32_t *status, hipStream_t stream) {
  return quantize_common(fmt, w, dtype, rows, cols, rows_per_expert, grid, importance, nullptr, out, workspace,
                         workspace_bytes, status, true, nullptr, nullptr, stream);
}

int iq_choice_search_workspace_size(int fmt, int64_t rows, int64_t cols, int64_t rows_per_expert, int weighted,
                                    size_t *bytes) {
  if (bad_fmt(fmt)) return IQ_ERR_FMT;
  if (!bytes) return IQ_ERR_NULL;
  const int rc = check_encode_shape(rows, cols, rows_per_expert, fmt, wg_cols(fmt));
  if (rc != IQ_OK) return rc;
  *bytes = rows ? iq::plan_choice_search(fmt, rows, cols, rows_per_expert, weighted != 0).bytes : 0;
  return IQ_OK;
}

int iq_choice_search(int fmt, const void *w, int dtype, int64_t rows, int64_t cols, int64_t rows_per_expert,
                     const float *grid, const float *importance, const float *hess, float perc_damp,
                     uint8_t *choices, uint8_t *out, void *workspace, size_t workspace_bytes, int32_t *status,
                     hipStream_t stream) {
  if (bad_fmt(fmt)) return IQ_ERR_FMT;
  if (bad_dtype(dtype)) return IQ_ERR_DTYPE;
  if (!grid || (rows != 0 && (!w || !hess || !choices))) return IQ_ERR_NULL;
  int rc = check_encode_shape(rows, cols, rows_per_expert, fmt, wg_cols(fmt));
  if (rc != IQ_OK) return rc;
  if (!(perc_damp >= 0.0f) || perc_damp > 3.0e38f) return IQ_ERR_ARG;
  const size_t need =
      rows ? iq::plan_choice_search(fmt, rows, cols, rows_per_expert, importance != nullptr).bytes : 0;
  if ((rc = check_workspace(need, workspace, workspace_bytes)) != IQ_OK) return rc;
  iq::EncArgs A = enc_args(w, dtype, rows, cols, rows_per_expert, grid, importance, status);
  A.out = out;
  return iq::launch_choice_search(fmt, A, hess, perc_damp, choices, workspace, stream) == 0 ? IQ_OK : IQ_ERR_HIP;
}

int iq_dequantize(int fmt, const uint8_t *packed, int64_t rows, int64_t cols, const float *grid, void *out,
                  int dtype, hipStream_t stream) {
  if (bad_fmt(fmt)) return IQ_ERR_FMT;
  if (bad_dtype(dtype)) return IQ_ERR_DTYPE;
  if (!grid || (rows != 0 && (!packed || !out))) return IQ_ERR_NULL;
  if (rows < 0 || cols <= 0 || cols % 256 != 0) return IQ_ERR_SHAPE;
  if (rows > (int64_t(1) << 40) / (cols / 256) || rows * (cols / 256) * 32 / 256 >= (int64_t(1) << 31))
    return IQ_ERR_SHAPE;
  return iq::launch_decode(fmt, packed, rows, cols, grid, out, dtype, stream) == 0 ? IQ_OK : IQ_ERR_HIP;
}

const char *iq_error_string(int code) {
  switch (code) {
    case IQ_OK: return "ok";
    case IQ_ERR_FMT: return "unknown format";
    case IQ_ERR_DTYPE: return "unknown dtype";
    case IQ_ERR_NULL: return "required pointer is NULL";
    case IQ_ERR_SHAPE: return "invalid shape";
    case IQ_ERR_ARG: return "invalid argument";
    case IQ_ERR_HIP: return "HIP launch failure";
    case IQ_ERR_WORKSPACE: return "workspace smaller than the size query returns";
  }
  return "unknown error code";
}

}  // extern "C"
