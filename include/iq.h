/*
 * iq.h -- C ABI of libiq.so: importance-weighted GGML IQ codebook encoding
 * (IQ2_XXS, IQ2_XS, IQ2_S, IQ1_S, IQ1_M) and imatrix collection on one
 * MI355X (gfx950).
 *
 * Conventions for every entry point
 *  - Pointers marked (device) must point to device memory of the current HIP
 *    device; (host) pointers to host memory.  The caller owns every buffer.
 *  - The library allocates no memory and keeps no state between calls (the
 *    one exception, iq_quantize_noalloc, says so).  Calls that need scratch
 *    take a caller-owned device workspace: `*_workspace_size` returns its size
 *    in bytes for the call's sizes (0: none needed, workspace may be NULL);
 *    any alignment is accepted.  The workspace is overwritten; it must not be
 *    used by another call while this call's work is in flight.
 *  - Work is enqueued on `stream` (0 = the null stream) and is asynchronous:
 *    a return of IQ_OK means "validated and enqueued", not "finished".
 *  - Every return code except IQ_ERR_HIP is host-detected before anything is
 *    enqueued: no kernel ran and no output or workspace byte was touched.
 *    IQ_ERR_HIP means a kernel launch failed: the kernels of this call before
 *    it may already be enqueued (outputs and workspace then hold partial
 *    results), nothing after it is.
 *  - Problems only the device can see (non-finite data, out-of-range fixed
 *    choices or expert ids, fp16 overflow of a block scale) are OR-ed into
 *    *status (device, int32, optional) as IQ_STATUS_* bits; the caller reads it
 *    after synchronising.  The library never synchronises the stream itself.
 *  - Dense tensors are row-major and contiguous.  Sizes are in elements.
 *
 * Sources are cited by page title and section:
 *  [2735]     "Add imatrix calibration for the GGML formats and use it for fused
 *             MoE experts" (ModelOpt PR), description.
 *  [2513]     ModelOpt PR #2513: IQ2_XXS / IQ2_S / IQ1_M commit messages, IQ1_M body.
 *  [3157]     "[1/5] Let the GGML IQ encoders take fixed per-group choices"
 *             (ModelOpt PR), description and review, and the squashed follow-ups
 *             on that page (#3158 local_hessian, #3159 every-choice encode).
 *  [recipes]  modelopt_recipes folder page, IQ1_M CUDA encoder commit.
 *  [coverage] "MoE expert coverage in imatrix calibration", Facts.
 */
#ifndef IQ_H
#define IQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The five layouts ([2513] commit messages: IQ2_XXS 2.0625 bits/weight,
 * IQ2_S 2.5625, IQ1_M 1.75, IQ1_S 1.75 - 0.1875; IQ2_XS 9-bit index + 7-bit
 * sign index per 8 values and a 4-bit scale per 16). */
typedef enum {
  IQ_FMT_IQ2_XXS = 0, /* 66-byte blocks, 256-entry grid           */
  IQ_FMT_IQ2_XS = 1,  /* 74-byte blocks, 512-entry grid           */
  IQ_FMT_IQ2_S = 2,   /* 82-byte blocks, 1024-entry grid          */
  IQ_FMT_IQ1_S = 3,   /* 50-byte blocks, 2048-entry signed grid   */
  IQ_FMT_IQ1_M = 4    /* 56-byte blocks, same 2048-entry grid     */
} iq_fmt;

typedef enum { IQ_DTYPE_F32 = 0, IQ_DTYPE_BF16 = 1 } iq_dtype;

/* Return codes (all but IQ_ERR_HIP host-detected: nothing enqueued). */
#define IQ_OK 0
#define IQ_ERR_FMT (-1)    /* unknown format                                  */
#define IQ_ERR_DTYPE (-2)  /* unknown dtype                                   */
#define IQ_ERR_NULL (-3)   /* a required pointer is NULL (data pointers of an
                              empty input -- rows == 0 or T == 0 -- may be NULL;
                              the call then enqueues nothing and returns IQ_OK) */
#define IQ_ERR_SHAPE (-4)  /* cols % 256 != 0, rows % rows_per_expert != 0, ... */
#define IQ_ERR_ARG (-5)    /* other invalid argument (top_k, chunk_rows, ...)   */
#define IQ_ERR_HIP (-6)    /* a kernel launch failed (see the conventions)    */
#define IQ_ERR_WORKSPACE (-7) /* workspace smaller than its size query returns */

/* Device status bits, OR-ed into *status. */
#define IQ_STATUS_NONFINITE 1  /* non-finite weight (block encoded as zeros) or activation */
#define IQ_STATUS_OVERFLOW 2   /* fp16 block scale overflowed (block encoded as zeros)    */
#define IQ_STATUS_BADCHOICE 4  /* fixed choice >= num_choices (block encoded as zeros)    */
#define IQ_STATUS_BADIMP 8     /* importance outside [0, 2^64] (block zeros) or a non-finite /
                                  negative statistic (expert flat)                          */
#define IQ_STATUS_BADID 16     /* routed expert id outside [0, num_experts) (pair skipped) */

/* Geometry of one layout ([3157]: each format records choice_groups and
 * num_choices). */
typedef struct {
  int32_t block_values;      /* 256 values per block ([2735] "Checked up front")   */
  int32_t block_bytes;       /* 66 / 74 / 82 / 50 / 56                             */
  int32_t grid_size;         /* codebook entries, each 8 floats                    */
  int32_t choice_groups;     /* choice units per block: 8 / 16 / 16 / 8 / 16       */
  int32_t num_choices;       /* choices per unit: 16 / 16 / 16 / 16 / 8            */
  int32_t groups_per_choice; /* 8-value groups sharing one choice: 4 / 2 / 2 / 4 / 2 */
} iq_format_info_t;

/* Fill *out (host) with the geometry of `fmt`.  Returns IQ_OK or IQ_ERR_FMT /
 * IQ_ERR_NULL. */
int iq_format_info(int fmt, iq_format_info_t *out);

/* imatrix collection ([2735] "What imatrix does": per input column the second
 * moment E[x_j^2]; "Bounded memory": rows are squared 1,024 at a time;
 * [coverage] Facts: a token's squares are added only to the experts in its
 * top-k, with one counts entry per expert).
 *
 *  x        (device) [T, K] activations, dtype f32 or bf16.
 *  ids      (device) [T, top_k] int32 routed expert ids, or NULL for a dense
 *           weight (then num_experts must be 1 and top_k is ignored; with
 *           T == 0 ids may be NULL for any num_experts).
 *  chunk_rows  rows reduced per chunk (1024 in [2735]); each chunk is reduced
 *           in fixed slices whose partial sums are added to `sums` in order,
 *           so results do not depend on the launch and repeat bit for bit.
 *  sums     (device) [num_experts, K] f32, ACCUMULATED: sums[e][j] += sum over
 *           the (t, s) pairs with ids[t][s] == e of x[t][j]^2 (a duplicate id in
 *           one token counts per occurrence).
 *  counts   (device) [num_experts] int64, ACCUMULATED: counts[e] += number of
 *           such pairs (dense: += T).
 *  workspace, workspace_bytes  (device) scratch of at least
 *           iq_imatrix_collect_workspace_size(T, K, ids ? top_k : 0, num_experts,
 *           chunk_rows) bytes.  Chunks are reduced in windows of several
 *           chunks, so the size is bounded independently of T (slice partials
 *           of one window, and for routed tokens its routing bitmaps).
 *  status   (device, nullable): IQ_STATUS_NONFINITE when a row that reached an
 *           expert holds a non-finite value (only touched experts are checked);
 *           IQ_STATUS_BADID for ids outside [0, num_experts) (those pairs skip).
 * Errors: IQ_ERR_NULL (x, sums, counts, or a needed workspace), IQ_ERR_DTYPE,
 * IQ_ERR_ARG (T < 0, K <= 0, top_k < 1 with ids, num_experts < 1,
 * chunk_rows < 1, sizes whose launches would not fit a grid),
 * IQ_ERR_WORKSPACE, IQ_ERR_HIP. */
int iq_imatrix_collect(const void *x, int dtype, int64_t T, int64_t K, const int32_t *ids,
                       int top_k, int num_experts, int chunk_rows, float *sums, int64_t *counts,
                       void *workspace, size_t workspace_bytes, int32_t *status, hipStream_t stream);

/* Workspace bytes iq_imatrix_collect needs; top_k = 0 for a dense
 * collection (ids NULL).  *bytes (host).  Errors: IQ_ERR_NULL, IQ_ERR_ARG. */
int iq_imatrix_collect_workspace_size(int64_t T, int64_t K, int top_k, int num_experts, int chunk_rows,
                                      size_t *bytes);

/* Merge of two collections' statistics ([coverage] Facts: the GGUF imatrix
 * format stores in_sum2 and counts per tensor so that files can be merged;
 * [2735] "Single rank": summing the statistics of data-parallel ranks is the
 * same addition).
 *
 *  sums[e][j] = sums[e][j] + src_sums[e][j] (one fp32 addition, round to
 *  nearest even); counts[e] += src_counts[e] (exact).  Merging in a fixed
 *  order therefore repeats bit for bit; merges in different orders agree
 *  within the fp32 rounding of each addition.
 *  src_sums (device) [E, K] f32, src_counts (device) [E] int64: read only,
 *           e.g. a collection loaded from a statistics file.
 *  sums, counts (device) [E, K] f32 and [E] int64, ACCUMULATED in place.
 *  status   (device, nullable): IQ_STATUS_NONFINITE when a source sum of an
 *           expert with src_counts[e] != 0 is not finite (the value is still
 *           added; experts the source did not touch are not checked).
 * Errors: IQ_ERR_NULL (any array), IQ_ERR_ARG (E < 1, K <= 0, or a source
 * array overlapping its accumulator). */
int iq_imatrix_merge(const float *src_sums, const int64_t *src_counts, int num_experts, int64_t K,
                     float *sums, int64_t *counts, int32_t *status, hipStream_t stream);

/* Importance from collected statistics ([2735] "What imatrix does" and "Why
 * the square root": the search weight is sqrt(E[x_j^2]), floored ("Shared
 * floor"); [coverage] Facts: counts[e] == 0 gives weight 1 on every channel).
 *
 *  importance[e][j] = sqrt(max(m_j, floor_rel * mean_j m_j)), m_j = sums[e][j] /
 *  counts[e] (fp32, IEEE division and square root).  The mean is the plain
 *  one: the m_j added in fp64 in ascending j, divided by K in fp64, rounded to
 *  fp32.  Experts with counts 0, a mean that is 0, or a non-finite / negative
 *  m_j (IQ_STATUS_BADIMP) get all ones.
 *  sums (device) [E, K] f32; counts (device) [E] int64; importance (device)
 *  [E, K] f32 (may alias nothing).  floor_rel: 1e-6 is the default used here.
 * Errors: IQ_ERR_NULL, IQ_ERR_ARG (E < 1, K <= 0, floor_rel < 0 or not finite). */
int iq_imatrix_importance(const float *sums, const int64_t *counts, int num_experts, int64_t K,
                          float floor_rel, float *importance, int32_t *status, hipStream_t stream);

/* Importance-weighted IQ encode ([2513] commit messages: fixed anchored fp16
 * super-block scale, single-pass grid search, IQ2_XXS/XS even-parity sign
 * index with the weakest element flipped, IQ2_S full sign mask, IQ1 +-1/8
 * delta with lower-shift-then-lower-entry ties; [3157]: one choice per unit
 * by least importance-weighted squared error, or fixed by the caller, in
 * which case only the entry search runs).
 *
 *  w           (device) [rows, cols] weight, f32 or bf16; cols % 256 == 0.
 *  rows_per_expert  rows sharing one importance row: row r uses importance row
 *              r / rows_per_expert ([coverage] Facts: the slice for each
 *              expert is applied separately, chunks never cross experts).
 *              Pass rows for a dense weight.  rows % rows_per_expert == 0.
 *  grid        (device) [grid_size, 8] f32 codebook (IQ2: magnitudes; IQ1:
 *              signed values).
 *  importance  (device) [rows / rows_per_expert, cols] f32 search weights
 *              a_j, or NULL for the plain (flat, a_j = 1) search.  Use
 *              iq_imatrix_importance to build it; a row of ones is the flat
 *              search for an idle expert ([2735] "Idle experts").
 *  choices     (device) [rows, cols/256, choice_groups] uint8 fixed choices,
 *              or NULL to search them.  IQ2: local scale in [0,16); IQ1_S:
 *              (delta_sign << 3) | local scale; IQ1_M: local scale in [0,8).
 *  out         (device) [rows, cols/256, block_bytes] uint8 payload.
 *  workspace, workspace_bytes  (device) scratch of at least
 *              iq_quantize_workspace_size(fmt, rows, cols, rows_per_expert,
 *              importance != NULL) bytes: the weighted norms of every grid entry
 *              per (expert, 8-column group), the fp16 block scales and the
 *              importance flags.
 *  status      (device, nullable) IQ_STATUS_* bits.
 * Every block is written; a block holding a non-finite value, an importance
 * value outside [0, 2^64], an out-of-range choice, an fp16-overflowing scale,
 * or only zeros is written as all-zero bytes ([3157] review: all-zero block ->
 * all-zero payload).  The grid's values are taken to lie in the layout's
 * alphabet range (IQ2 magnitudes in [0, 5], IQ1 values in [-1, 1]), which the
 * scale anchor assumes.
 * Errors: IQ_ERR_FMT, IQ_ERR_DTYPE, IQ_ERR_NULL (w, grid, out, or a needed
 * workspace), IQ_ERR_SHAPE (rows < 0, cols <= 0 or % 256, rows_per_expert < 1
 * or not dividing rows, sizes whose launches would not fit a grid),
 * IQ_ERR_WORKSPACE, IQ_ERR_HIP. */
int iq_quantize(int fmt, const void *w, int dtype, int64_t rows, int64_t cols,
                int64_t rows_per_expert, const float *grid, const float *importance,
                const uint8_t *choices, uint8_t *out, void *workspace, size_t workspace_bytes,
                int32_t *status, hipStream_t stream);

/* Workspace bytes iq_quantize and iq_quantize_every_choice need (weighted:
 * importance given).  *bytes (host).  Errors: IQ_ERR_FMT, IQ_ERR_NULL,
 * IQ_ERR_SHAPE. */
int iq_quantize_workspace_size(int fmt, int64_t rows, int64_t cols, int64_t rows_per_expert, int weighted,
                               size_t *bytes);

/* Bytes of the static device scratch iq_quantize_noalloc works in (64 MiB). */
#define IQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* iq_quantize for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid it): same
 * arguments, results and errors as iq_quantize, without a workspace.  Its
 * scratch is a static device array of IQ_NOALLOC_SCRATCH_BYTES that each GPU
 * the library runs on holds until the process ends; the first call on a
 * device looks up that device's address (hipGetSymbolAddress), and no call
 * allocates or frees anything.  Every call on a device shares its array and
 * leaves it holding that call's scratch, so calls that overlap on one GPU
 * (other streams, other threads) race: serialise them.
 * Limit: iq_quantize_workspace_size(fmt, rows, cols, rows_per_expert,
 * importance != NULL) must not exceed IQ_NOALLOC_SCRATCH_BYTES -- e.g. any
 * dense weight up to 17408 x 5120, or 128 experts x 2048 columns in the
 * IQ2 layouts -- else IQ_ERR_WORKSPACE before anything is enqueued.
 * IQ_ERR_HIP also reports a failed address lookup. */
int iq_quantize_noalloc(int fmt, const void *w, int dtype, int64_t rows, int64_t cols,
                        int64_t rows_per_expert, const float *grid, const float *importance,
                        const uint8_t *choices, uint8_t *out, int32_t *status, hipStream_t stream);

/* iq_quantize, also recording `search_start` on `stream` just before its
 * search kernel and `search_stop` just after it, so hipEventElapsedTime gives
 * that kernel's duration alone (a measurement aid, not part of the method).
 * Both events must have been created on the current device.
 * Errors: as iq_quantize, plus IQ_ERR_NULL for a NULL event. */
int iq_quantize_timed(int fmt, const void *w, int dtype, int64_t rows, int64_t cols,
                      int64_t rows_per_expert, const float *grid, const float *importance,
                      const uint8_t *choices, uint8_t *out, void *workspace, size_t workspace_bytes,
                      int32_t *status, hipEvent_t search_start, hipEvent_t search_stop, hipStream_t stream);

/* Every-choice encode ([3157] series, squashed #3159 "one-pass every-choice
 * encode": each 256-column block encoded under every choice from a single
 * sweep, byte-identical to the forced encodes).
 *  out (device) [num_choices, rows, cols/256, block_bytes]: out[c] is exactly
 *  the payload iq_quantize writes with `choices` set to c for every unit
 *  (IQ1_S: c = (delta_sign << 3) | local scale).
 *  Other arguments, the workspace (iq_quantize_workspace_size), status bits
 *  and errors as iq_quantize (no `choices`). */
int iq_quantize_every_choice(int fmt, const void *w, int dtype, int64_t rows, int64_t cols,
                             int64_t rows_per_expert, const float *grid, const float *importance,
                             uint8_t *out, void *workspace, size_t workspace_bytes, int32_t *status,
                             hipStream_t stream);

/* Local-Hessian choice search ([3157] series, squashed #3158 "local_hessian
 * for GGML IQ": encode each block under every choice; give each choice unit its
 * best choice under its own block of the damped input Hessian; revisit the units
 * twice, each taking the choice that most lowers the block's layer-output error
 * dw H dw^T with the others held; blocks damped by perc_damp as GPTQ damps).
 *  hess     (device) [rows / rows_per_expert, cols/256, 256, 256] f32: the
 *           256-column diagonal blocks of each expert's input Hessian X^T X.
 *  perc_damp  H_b + perc_damp * mean(diag H_b) * I is used (0.3 in [3158]).
 *  choices  (device) [rows, cols/256, choice_groups] uint8 OUT: the picks, to be
 *           passed to iq_quantize (IQ1_S: (delta_sign << 3) | local scale).
 *           A block no calibration token reached (all-zero diag H_b, e.g. an
 *           idle expert's) keeps the encoder's own choices, so its payload is
 *           iq_quantize's ([3158] Testing: a never-reached weight is encoded
 *           plainly).
 *  out      (device, nullable) [rows, cols/256, block_bytes] uint8 OUT: when
 *           given, the payload under the picks -- byte for byte what iq_quantize
 *           writes with `choices` -- packed from the every-choice fields the
 *           search already holds, so no second sweep is needed.
 *  workspace, workspace_bytes  (device) scratch of at least
 *           iq_choice_search_workspace_size(...) bytes: every group's fields
 *           under every choice (num_choices * rows * cols/8 * 4 bytes), the
 *           damping terms, the reached flags and an encoder workspace.
 *  importance, grid, w, rows_per_expert, status: as iq_quantize (the codebook
 *  search keeps the importance weighting).
 * Errors: as iq_quantize, plus IQ_ERR_NULL (hess, choices) and IQ_ERR_ARG
 * (perc_damp negative or not finite). */
int iq_choice_search(int fmt, const void *w, int dtype, int64_t rows, int64_t cols,
                     int64_t rows_per_expert, const float *grid, const float *importance,
                     const float *hess, float perc_damp, uint8_t *choices, uint8_t *out,
                     void *workspace, size_t workspace_bytes, int32_t *status, hipStream_t stream);

/* Workspace bytes iq_choice_search needs (weighted: importance given).
 * Errors: IQ_ERR_FMT, IQ_ERR_NULL, IQ_ERR_SHAPE. */
int iq_choice_search_workspace_size(int fmt, int64_t rows, int64_t cols, int64_t rows_per_expert,
                                    int weighted, size_t *bytes);

/* Hessian diagonal blocks for iq_choice_search ([3157] series, squashed #3158
 * "local_hessian for GGML IQ": the layer-output error is measured under the
 * 256-column diagonal blocks of each weight's input Hessian X^T X, gathered
 * from the same calibration tokens as the imatrix, routed per expert).
 *  x, dtype, T, K, ids, top_k, num_experts, chunk_rows: as iq_imatrix_collect;
 *           K must be a multiple of 256.
 *  hess     (device) [num_experts, K/256, 256, 256] f32, ACCUMULATED:
 *           hess[e][b][i][j] += sum over the (t, s) pairs with ids[t][s] == e of
 *           x[t][256b + i] * x[t][256b + j] (dense: every token, e = 0).  Each
 *           block is exactly symmetric.  Tokens are added in ascending order
 *           (a token naming e twice, twice in a row) in fixed splits: token
 *           ranges for a dense input; for routed input, an expert's list is cut
 *           into equal shares only when it holds more entries than a length set
 *           by T, top_k and K (256 to 1,024 entries, more if the partial blocks
 *           would pass 512 MiB), else taken whole.  Partial blocks are added in
 *           split order, so results repeat bit for bit.
 *  workspace, workspace_bytes  (device) scratch of at least
 *           iq_hessian_collect_workspace_size(T, K, ids ? top_k : 0,
 *           num_experts, chunk_rows) bytes: split partial blocks (at most
 *           512 MiB for routed tokens) and, routed, the token lists.
 *  status   (device, nullable): IQ_STATUS_NONFINITE when a token that reached an
 *           expert holds a non-finite value; IQ_STATUS_BADID as
 *           iq_imatrix_collect.
 * Errors: as iq_imatrix_collect, plus IQ_ERR_NULL (hess), IQ_ERR_SHAPE (K not a
 * multiple of 256) and IQ_ERR_ARG (num_experts * K above 2^30, T of 2^31 or
 * more). */
int iq_hessian_collect(const void *x, int dtype, int64_t T, int64_t K, const int32_t *ids, int top_k,
                       int num_experts, int chunk_rows, float *hess, void *workspace, size_t workspace_bytes,
                       int32_t *status, hipStream_t stream);

/* Workspace bytes iq_hessian_collect needs; top_k = 0 for dense tokens.
 * Errors: IQ_ERR_NULL, IQ_ERR_ARG, IQ_ERR_SHAPE. */
int iq_hessian_collect_workspace_size(int64_t T, int64_t K, int top_k, int num_experts, int chunk_rows,
                                      size_t *bytes);

/* Decode ([2513]: dequantize_row semantics; IQ1_M d reassembled from the top
 * nibbles of the four scale words, one 3-bit scale per two groups).
 *  packed (device) [rows, cols/256, block_bytes]; grid (device) [grid_size, 8];
 *  out (device) [rows, cols] f32 or bf16 (bf16: round to nearest even).
 *  IQ2: out = +-(s * g), s = d * (2 ls + 1) / 8.  IQ1: out = s * (g +- 1/8),
 *  s = d * (2 ls + 1).
 * Errors: IQ_ERR_FMT, IQ_ERR_DTYPE, IQ_ERR_NULL, IQ_ERR_SHAPE. */
int iq_dequantize(int fmt, const uint8_t *packed, int64_t rows, int64_t cols, const float *grid,
                  void *out, int dtype, hipStream_t stream);

/* Short text for a return code (static storage). */
const char *iq_error_string(int code);

#ifdef __cplusplus
}
#endif
#endif /* IQ_H */
