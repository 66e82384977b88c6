// iq_internal.hpp -- argument block and launcher declarations shared by the
// libiq translation units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iq {

struct EncArgs {
  const void *w;
  int dtype;
  int64_t rows, cols, rpe, E;
  int nb;                  // blocks per row (cols / 256)
  const float *grid;
  const float *imp;        // [E, cols] or null (flat)
  const uint8_t *choices;  // [rows, nb, units] or null
  uint8_t *out;
  int64_t copies, copy_stride;  // payload copies (every-choice: num_choices) and bytes between them
  int32_t *status;
  uint32_t *rec;           // field records (choice search): [num_choices][nb][32 groups][rows]
  uint16_t *d_out;         // copy of the fp16 block scales [rows][nb] (choice search), or null
  // filled by the launcher
  float *gtab;             // weighted norms [tables][NG][N]
  int64_t gtab_e_stride, gtab_cg_stride;
  uint16_t *dscr;          // fp16 scale bits per block
  int64_t tiles_per_e, total_wg;
};

// events registered by iq_time_next_search for this host thread (cleared on take)
void take_search_events(hipEvent_t *start, hipEvent_t *stop);

int launch_quantize(int fmt, EncArgs A, bool every_choice, hipStream_t stream);
int launch_choice_search(int fmt, EncArgs A, const float *hess, float perc_damp, uint8_t *choices,
                         hipStream_t stream);
int launch_decode(int fmt, const uint8_t *packed, int64_t rows, int64_t cols, const float *grid, void *out,
                  int dtype, hipStream_t stream);
int launch_collect(const void *x, int dtype, int64_t T, int64_t K, const int32_t *ids, int top_k, int E,
                   int chunk_rows, float *sums, int64_t *counts, int32_t *status, hipStream_t stream);
int launch_hessian(const void *x, int dtype, int64_t T, int64_t K, const int32_t *ids, int top_k, int E,
                   int chunk_rows, float *hess, int32_t *status, hipStream_t stream);
int launch_merge(const float *src, const int64_t *src_counts, int E, int64_t K, float *sums, int64_t *counts,
                 int32_t *status, hipStream_t stream);
int launch_importance(const float *sums, const int64_t *counts, int E, int64_t K, float floor_rel,
                      float *imp, int32_t *status, hipStream_t stream);

}  // namespace iq
