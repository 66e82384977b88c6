// iq_internal.hpp -- argument block, workspace plans and launcher declarations
// shared by the libiq translation units (not part of the C ABI).
//
// Every launcher takes the caller's workspace (device memory it owns) and
// carves its scratch from it; none allocates.  A workspace plan is a pure
// function of the call's sizes: the *_workspace_size queries and the
// launchers evaluate the same plan, so a workspace of the queried size always
// fits.  Launchers enqueue nothing before their sizes are known to be valid,
// and return at the first failed launch without enqueuing anything after it.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
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
  // filled by the launcher
  float *gtab;             // weighted norms [tables][NG][N]
  int64_t gtab_e_stride, gtab_cg_stride;
  uint16_t *dscr;          // fp16 scale bits per block
  int64_t tiles_per_e, total_wg;
};

// Scratch layout inside a workspace: the base is rounded up to 256 bytes (the
// byte counts include that slack) and every part starts 256-byte aligned.
constexpr size_t kWsAlign = 256;
inline size_t ws_up(size_t v) { return (v + kWsAlign - 1) & ~(kWsAlign - 1); }
inline char *ws_base(void *ws) {
  return reinterpret_cast<char *>((reinterpret_cast<uintptr_t>(ws) + kWsAlign - 1) & ~uintptr_t(kWsAlign - 1));
}

// Encoder scratch: weighted-norm tables, fp16 block scales, importance flags.
struct QuantPlan {
  int64_t ntab;              // norm tables (weighted: E * cols / 8; flat: one)
  size_t goff, doff, foff;   // offsets of the three parts
  size_t bytes;              // total, including the alignment slack
};
QuantPlan plan_quantize(int fmt, int64_t rows, int64_t cols, int64_t rpe, bool weighted);

// Choice-search scratch: the field records and damping terms, then an encoder
// scratch for the record sweep (whose fp16 scales the choice search reads).
struct ChoicePlan {
  size_t roff, loff, foff, qoff;   // records, damping terms, reached flags, encoder scratch
  QuantPlan q;
  size_t bytes;
};
ChoicePlan plan_choice_search(int fmt, int64_t rows, int64_t cols, int64_t rpe, bool weighted);

// Collector scratch, bounded independently of T: chunks are reduced in windows
// of `wchunks` chunks whose slice partials (and, routed, routing bitmaps and
// repeat flags) reuse one region.
struct CollectPlan {
  int64_t nchunks, wchunks, nsub, slice_len, ntile;
  int W;                     // bitmap words per (chunk, expert)
  size_t boff, doff, bytes;  // partials at 0, then bitmaps, repeat flags
};
CollectPlan plan_collect(int64_t T, int64_t K, bool routed, int E, int chunk_rows);

// Hessian scratch: split partials; routed: bitmaps, repeat flags, list
// lengths and starts, the cut experts and the token lists.
struct HessPlan {
  int64_t nchunks, nsplit, split_len, target, smax, pmax, hmax;
  int W;
  size_t off_b, off_d, off_n, off_l, bytes;
};
HessPlan plan_hessian(int64_t T, int64_t K, int top_k, int E, int chunk_rows);

int launch_quantize(int fmt, EncArgs A, bool every_choice, void *ws, hipEvent_t search_start,
                    hipEvent_t search_stop, hipStream_t stream);
int launch_choice_search(int fmt, EncArgs A, const float *hess, float perc_damp, uint8_t *choices, void *ws,
                         hipStream_t stream);
int launch_decode(int fmt, const uint8_t *packed, int64_t rows, int64_t cols, const float *grid, void *out,
                  int dtype, hipStream_t stream);
int launch_collect(const void *x, int dtype, int64_t T, int64_t K, const int32_t *ids, int top_k, int E,
                   int chunk_rows, float *sums, int64_t *counts, int32_t *status, void *ws, hipStream_t stream);
int launch_hessian(const void *x, int dtype, int64_t T, int64_t K, const int32_t *ids, int top_k, int E,
                   int chunk_rows, float *hess, int32_t *status, void *ws, hipStream_t stream);
int launch_merge(const float *src, const int64_t *src_counts, int E, int64_t K, float *sums, int64_t *counts,
                 int32_t *status, hipStream_t stream);
int launch_importance(const float *sums, const int64_t *counts, int E, int64_t K, float floor_rel,
                      float *imp, int32_t *status, hipStream_t stream);

}  // namespace iq
