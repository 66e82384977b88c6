// iq_api.hip -- the C ABI of libiq.so (declared in include/iq.h): host-side
// validation, then the launches.  No entry point synchronises the stream.

#include "iq.h"
#include "iq_common.hpp"
#include "iq_internal.hpp"

namespace {

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

thread_local hipEvent_t t_search_start = nullptr, t_search_stop = nullptr;

bool bad_fmt(int fmt) { return fmt < 0 || fmt > 4; }
bool bad_dtype(int dt) { return dt != IQ_DTYPE_F32 && dt != IQ_DTYPE_BF16; }

}  // namespace

namespace iq {
void take_search_events(hipEvent_t *start, hipEvent_t *stop) {
  *start = t_search_start;
  *stop = t_search_stop;
  t_search_start = t_search_stop = nullptr;
}
}  // namespace iq

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

int iq_imatrix_collect(const void *x, int dtype, int64_t T, int64_t K, const int32_t *ids, int top_k,
                       int num_experts, int chunk_rows, float *sums, int64_t *counts, int32_t *status,
                       hipStream_t stream) {
  if (bad_dtype(dtype)) return IQ_ERR_DTYPE;
  if (!sums || !counts || (T != 0 && !x)) return IQ_ERR_NULL;
  if (T < 0 || K <= 0 || num_experts < 1 || chunk_rows < 1) return IQ_ERR_ARG;
  if (ids && top_k < 1) return IQ_ERR_ARG;
  if (!ids && num_experts != 1 && T != 0) return IQ_ERR_ARG;  // no tokens: ids may be NULL
  if (static_cast<int64_t>(num_experts) * K > (int64_t(1) << 40)) return IQ_ERR_ARG;
  return iq::launch_collect(x, dtype, T, K, ids, ids ? top_k : 0, num_experts, chunk_rows, sums, counts, status,
                            stream) == 0
             ? IQ_OK
             : IQ_ERR_HIP;
}

int iq_hessian_collect(const void *x, int dtype, int64_t T, int64_t K, const int32_t *ids, int top_k,
                       int num_experts, int chunk_rows, float *hess, int32_t *status, hipStream_t stream) {
  if (bad_dtype(dtype)) return IQ_ERR_DTYPE;
  if (!hess || (T != 0 && !x)) return IQ_ERR_NULL;
  if (T < 0 || K <= 0 || num_experts < 1 || chunk_rows < 1) return IQ_ERR_ARG;
  if (ids && top_k < 1) return IQ_ERR_ARG;
  if (!ids && num_experts != 1 && T != 0) return IQ_ERR_ARG;  // no tokens: ids may be NULL
  if (K % 256 != 0) return IQ_ERR_SHAPE;
  if (static_cast<int64_t>(num_experts) * K > (int64_t(1) << 30) || T > (int64_t(1) << 31) - 1) return IQ_ERR_ARG;
  return iq::launch_hessian(x, dtype, T, K, ids, ids ? top_k : 0, num_experts, chunk_rows, hess, status, stream) == 0
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

static int quantize_common(int fmt, const void *w, int dtype, int64_t rows, int64_t cols, int64_t rows_per_expert,
                           const float *grid, const float *importance, const uint8_t *choices, uint8_t *out,
                           int32_t *status, bool every, hipStream_t stream) {
  if (bad_fmt(fmt)) return IQ_ERR_FMT;
  if (bad_dtype(dtype)) return IQ_ERR_DTYPE;
  if (!grid || (rows != 0 && (!w || !out))) return IQ_ERR_NULL;
  if (rows < 0 || cols <= 0 || cols % 256 != 0) return IQ_ERR_SHAPE;
  if (rows_per_expert < 1 || rows % rows_per_expert != 0) return IQ_ERR_SHAPE;
  if (cols / 256 > (int64_t(1) << 24) || rows > (int64_t(1) << 40)) return IQ_ERR_SHAPE;
  iq::EncArgs A{};
  A.w = w;
  A.dtype = dtype;
  A.rows = rows;
  A.cols = cols;
  A.rpe = rows_per_expert;
  A.E = rows / rows_per_expert;
  A.nb = static_cast<int>(cols / 256);
  A.grid = grid;
  A.imp = importance;
  A.choices = choices;
  A.out = out;
  A.copies = every ? kFmt[fmt].num_choices : 1;
  A.copy_stride = rows * (cols / 256) * kFmt[fmt].block_bytes;
  A.status = status;
  // workgroups: experts x 64-row tiles x column sets; must fit one grid dimension
  const int64_t wgg = (fmt == IQ_FMT_IQ1_M) ? 8 : 4;
  const int64_t total = A.E * ((rows_per_expert + 63) / 64) * A.nb * (32 / wgg);
  if (total >= (int64_t(1) << 31)) return IQ_ERR_SHAPE;
  return iq::launch_quantize(fmt, A, every, stream) == 0 ? IQ_OK : IQ_ERR_HIP;
}

int iq_quantize(int fmt, const void *w, int dtype, int64_t rows, int64_t cols, int64_t rows_per_expert,
                const float *grid, const float *importance, const uint8_t *choices, uint8_t *out,
                int32_t *status, hipStream_t stream) {
  return quantize_common(fmt, w, dtype, rows, cols, rows_per_expert, grid, importance, choices, out, status, false,
                         stream);
}

int iq_quantize_every_choice(int fmt, const void *w, int dtype, int64_t rows, int64_t cols, int64_t rows_per_expert,
                             const float *grid, const float *importance, uint8_t *out, int32_t *status,
                             hipStream_t stream) {
  return quantize_common(fmt, w, dtype, rows, cols, rows_per_expert, grid, importance, nullptr, out, status, true,
                         stream);
}

int iq_choice_search(int fmt, const void *w, int dtype, int64_t rows, int64_t cols, int64_t rows_per_expert,
                     const float *grid, const float *importance, const float *hess, float perc_damp,
                     uint8_t *choices, uint8_t *out, int32_t *status, hipStream_t stream) {
  if (bad_fmt(fmt)) return IQ_ERR_FMT;
  if (bad_dtype(dtype)) return IQ_ERR_DTYPE;
  if (!grid || (rows != 0 && (!w || !hess || !choices))) return IQ_ERR_NULL;
  if (rows < 0 || cols <= 0 || cols % 256 != 0) return IQ_ERR_SHAPE;
  if (rows_per_expert < 1 || rows % rows_per_expert != 0) return IQ_ERR_SHAPE;
  if (cols / 256 > (int64_t(1) << 24) || rows > (int64_t(1) << 40)) return IQ_ERR_SHAPE;
  if (!(perc_damp >= 0.0f) || perc_damp > 3.0e38f) return IQ_ERR_ARG;
  iq::EncArgs A{};
  A.w = w;
  A.dtype = dtype;
  A.rows = rows;
  A.cols = cols;
  A.rpe = rows_per_expert;
  A.E = rows / rows_per_expert;
  A.nb = static_cast<int>(cols / 256);
  A.grid = grid;
  A.imp = importance;
  A.out = out;
  A.status = status;
  const int64_t wgg = (fmt == IQ_FMT_IQ1_M) ? 8 : 4;
  const int64_t total = A.E * ((rows_per_expert + 63) / 64) * A.nb * (32 / wgg);
  if (total >= (int64_t(1) << 31)) return IQ_ERR_SHAPE;
  return iq::launch_choice_search(fmt, A, hess, perc_damp, choices, stream) == 0 ? IQ_OK : IQ_ERR_HIP;
}

int iq_dequantize(int fmt, const uint8_t *packed, int64_t rows, int64_t cols, const float *grid, void *out,
                  int dtype, hipStream_t stream) {
  if (bad_fmt(fmt)) return IQ_ERR_FMT;
  if (bad_dtype(dtype)) return IQ_ERR_DTYPE;
  if (!grid || (rows != 0 && (!packed || !out))) return IQ_ERR_NULL;
  if (rows < 0 || cols <= 0 || cols % 256 != 0) return IQ_ERR_SHAPE;
  if (rows * (cols / 256) * 32 / 256 >= (int64_t(1) << 31)) return IQ_ERR_SHAPE;
  return iq::launch_decode(fmt, packed, rows, cols, grid, out, dtype, stream) == 0 ? IQ_OK : IQ_ERR_HIP;
}

int iq_time_next_search(hipEvent_t start, hipEvent_t stop) {
  if ((start == nullptr) != (stop == nullptr)) return IQ_ERR_NULL;
  t_search_start = start;
  t_search_stop = stop;
  return IQ_OK;
}

const char *iq_error_string(int code) {
  switch (code) {
    case IQ_OK: return "ok";
    case IQ_ERR_FMT: return "unknown format";
    case IQ_ERR_DTYPE: return "unknown dtype";
    case IQ_ERR_NULL: return "required pointer is NULL";
    case IQ_ERR_SHAPE: return "invalid shape";
    case IQ_ERR_ARG: return "invalid argument";
    case IQ_ERR_HIP: return "HIP allocation or launch failure";
  }
  return "unknown error code";
}

}  // extern "C"
