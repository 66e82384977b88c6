// iq_collect.hip -- imatrix collection and importance on gfx950.
//
// What is computed (pages cited by title and section):
//  * "Add imatrix calibration for the GGML formats and use it for fused MoE
//    experts", description: per input column the second moment E[x_j^2]; the
//    input hook squares 1,024 rows at a time ("Bounded memory"); each routed
//    expert gets its own statistic over the tokens routed to it; a weight no
//    token reaches gets the plain search ("Idle experts"); the search weight is
//    the floored square root ("Why the square root", "Shared floor").
//  * "MoE expert coverage in imatrix calibration", Facts: squares are added only
//    to the experts in a token's top-k, a per-expert counts vector records the
//    tokens seen, non-finite values are checked only for touched experts, and an
//    expert with count 0 receives weight 1 on every channel.
//
// Design.  No floating-point atomics: a pass marks, per 1,024-row chunk and
// expert, which tokens route there (bitmaps built with integer atomics, whose
// result does not depend on order); a second pass reduces each (chunk, expert,
// 128-column tile) with 16 waves that each own a fixed slice of the chunk's
// rows, combined in wave order; a last pass adds the chunk partials to the
// running sums in chunk order.  The sums therefore repeat bit for bit, and no
// x^2 temporary of the activation's size is ever materialised.

#include "iq_common.hpp"
#include "iq_internal.hpp"

namespace iq {

// Pass 1 (routed): membership bitmaps bm[chunk][e][words] and counts.
__global__ void __launch_bounds__(256) collect_route_kernel(const int32_t *__restrict__ ids, int64_t T,
                                                             int top_k, int E, int chunk_rows, int W,
                                                             uint32_t *__restrict__ bm,
                                                             int64_t *__restrict__ counts,
                                                             int32_t *status) {
  const int64_t chunk = blockIdx.x;
  uint32_t *reg = bm + chunk * static_cast<int64_t>(E) * W;
  for (int64_t i = threadIdx.x; i < static_cast<int64_t>(E) * W; i += blockDim.x) reg[i] = 0u;
  __syncthreads();
  const int64_t t0 = chunk * chunk_rows;
  const int64_t n = (T - t0 < chunk_rows) ? (T - t0) : chunk_rows;
  int st = 0;
  for (int64_t p = threadIdx.x; p < n; p += blockDim.x) {
    for (int s = 0; s < top_k; ++s) {
      const int e = ids[(t0 + p) * top_k + s];
      if (e < 0 || e >= E) { st |= ST_BADID; continue; }
      atomicOr(&reg[static_cast<int64_t>(e) * W + (p >> 5)], 1u << (p & 31));
      atomicAdd(reinterpret_cast<unsigned long long *>(counts + e), 1ull);
    }
  }
  raise_status(status, st);
}

// Pass 2: partial[chunk][e][K] = sum over the chunk's rows routed to e of x^2.
// Workgroup = 16 waves x 64 lanes over a 128-column tile; lane owns 2 columns;
// wave w owns rows [w * rpw, (w + 1) * rpw) of the chunk and adds them in row
// order, loading 16 rows per batch; the 16 wave partials are then added in wave
// order.
constexpr int kTile = 128, kBatch = 16;

template <int DT, bool PAIR>
__global__ void __launch_bounds__(1024) collect_partial_kernel(const void *__restrict__ x, int64_t T, int64_t K,
                                                                const int32_t *__restrict__ ids, int top_k,
                                                                int E, int chunk_rows, int W,
                                                                const uint32_t *__restrict__ bm,
                                                                float *__restrict__ partial, int32_t *status) {
  __shared__ float s_part[16][kTile];
  const int64_t ntile = (K + kTile - 1) / kTile;
  const int64_t tile = blockIdx.x % ntile;
  const int64_t ce = blockIdx.x / ntile;  // chunk * E + e
  const int e = static_cast<int>(ce % E);
  const int64_t chunk = ce / E;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: row bookkeeping stays scalar
  const int lane = threadIdx.x & 63;
  const int64_t t0 = chunk * chunk_rows;
  const int64_t n = (T - t0 < chunk_rows) ? (T - t0) : chunk_rows;
  const int64_t rpw = (((chunk_rows + 15) / 16) + 63) / 64 * 64;  // rows per wave, whole 64-row words
  const int64_t cl = tile * kTile + lane * 2;             // this lane's first column
  // lanes past the last column read a valid column and their results are dropped
  const int64_t c0 = cl < K ? cl : (PAIR ? K - 2 : K - 1);
  float acc0 = 0.0f, acc1 = 0.0f;
  bool finite = true;
  for (int64_t base = wave * rpw; base < (wave + 1) * rpw && base < n; base += 64) {
    const int64_t cnt = (n - base < 64) ? (n - base) : 64;
    const uint64_t live = cnt == 64 ? ~0ull : ((1ull << cnt) - 1ull);
    uint64_t mm = live;
    if (ids) {
      const uint32_t *wrow = bm + ce * W;
      const uint64_t lo = wrow[base >> 5];
      const uint64_t hi = ((base >> 5) + 1 < W) ? wrow[(base >> 5) + 1] : 0u;
      mm = (lo | (hi << 32)) & live;
    }
    while (mm) {
      // next kBatch member rows in ascending order; empty slots reuse a valid
      // row and contribute an exact zero, so the loads need no branches
      int64_t tok[kBatch];
      bool ok[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        ok[u] = mm != 0;
        tok[u] = t0 + base + (ok[u] ? __builtin_ctzll(mm) : 0);
        mm &= mm - 1;
      }
      float v0[kBatch], v1[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int64_t off = tok[u] * K + c0;
        if (PAIR) {  // even K: one 2-column load
          if (DT == 1) {
            const uint32_t q = *reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(x) + off);
            v0[u] = __uint_as_float(q << 16);
            v1[u] = __uint_as_float(q & 0xffff0000u);
          } else {
            const float2 q = *reinterpret_cast<const float2 *>(static_cast<const float *>(x) + off);
            v0[u] = q.x;
            v1[u] = q.y;
          }
        } else {
          const int64_t o1 = (c0 + 1 < K) ? off + 1 : off;
          v0[u] = DT == 1 ? bf16_to_f32(static_cast<const uint16_t *>(x)[off]) : static_cast<const float *>(x)[off];
          v1[u] = DT == 1 ? bf16_to_f32(static_cast<const uint16_t *>(x)[o1]) : static_cast<const float *>(x)[o1];
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        int mult = ok[u] ? 1 : 0;
        if (ids && ok[u]) {  // multiplicity of e in this token's top-k (usually 1)
          mult = 0;
          for (int s2 = 0; s2 < top_k; ++s2) mult += ids[tok[u] * top_k + s2] == e;
        }
        const float a0 = mult ? v0[u] : 0.0f, a1 = mult ? v1[u] : 0.0f;
        finite = finite && finite_f(a0) && finite_f(a1);
        acc0 = __builtin_fmaf(a0, a0, acc0);
        acc1 = __builtin_fmaf(a1, a1, acc1);
        for (int rep = 1; rep < mult; ++rep) {
          acc0 = __builtin_fmaf(a0, a0, acc0);
          acc1 = __builtin_fmaf(a1, a1, acc1);
        }
      }
    }
  }
  s_part[wave][lane * 2] = acc0;
  s_part[wave][lane * 2 + 1] = acc1;
  if (!finite) raise_status(status, ST_NONFINITE);
  __syncthreads();
  if (threadIdx.x < kTile) {  // columns past K (clamped lanes) are not stored
    const int64_t col = tile * kTile + threadIdx.x;
    float p = s_part[0][threadIdx.x];
#pragma unroll
    for (int w = 1; w < 16; ++w) p = p + s_part[w][threadIdx.x];
    if (col < K) partial[ce * K + col] = p;
  }
}

// Pass 3: sums[e][j] += partial[0][e][j]; += partial[1][e][j]; ... (chunk order)
__global__ void __launch_bounds__(256) collect_combine_kernel(const float *__restrict__ partial, int64_t nchunks,
                                                               int64_t EK, float *__restrict__ sums,
                                                               int64_t *counts, int64_t dense_T) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i == 0 && dense_T > 0) counts[0] += dense_T;
  if (i >= EK) return;
  float s = sums[i];
  for (int64_t c = 0; c < nchunks; ++c) s = s + partial[c * EK + i];
  sums[i] = s;
}

int launch_collect(const void *x, int dtype, int64_t T, int64_t K, const int32_t *ids, int top_k, int E,
                   int chunk_rows, float *sums, int64_t *counts, int32_t *status, hipStream_t stream) {
  if (T == 0) return 0;
  const int64_t nchunks = (T + chunk_rows - 1) / chunk_rows;
  const int W = (chunk_rows + 31) / 32 + 1;  // +1: a 64-bit read past the last word stays in the row
  const int64_t EK = static_cast<int64_t>(E) * K;
  const size_t pbytes = static_cast<size_t>(nchunks) * EK * sizeof(float);
  const size_t bbytes = ids ? static_cast<size_t>(nchunks) * E * W * sizeof(uint32_t) : 0;
  void *scratch = nullptr;
  if (hipMallocAsync(&scratch, pbytes + bbytes + 256, stream) != hipSuccess) return -1;
  float *partial = static_cast<float *>(scratch);
  uint32_t *bm = reinterpret_cast<uint32_t *>(static_cast<char *>(scratch) + ((pbytes + 255) & ~size_t(255)));
  if (ids)
    hipLaunchKernelGGL(collect_route_kernel, dim3(static_cast<unsigned>(nchunks)), dim3(256), 0, stream, ids, T,
                       top_k, E, chunk_rows, W, bm, counts, status);
  const int64_t ntile = (K + kTile - 1) / kTile;
  const dim3 g2(static_cast<unsigned>(nchunks * E * ntile));
  const bool pair = (K & 1) == 0;
  if (dtype == 1 && pair)
    hipLaunchKernelGGL((collect_partial_kernel<1, true>), g2, dim3(1024), 0, stream, x, T, K, ids, top_k, E,
                       chunk_rows, W, bm, partial, status);
  else if (dtype == 1)
    hipLaunchKernelGGL((collect_partial_kernel<1, false>), g2, dim3(1024), 0, stream, x, T, K, ids, top_k, E,
                       chunk_rows, W, bm, partial, status);
  else if (pair)
    hipLaunchKernelGGL((collect_partial_kernel<0, true>), g2, dim3(1024), 0, stream, x, T, K, ids, top_k, E,
                       chunk_rows, W, bm, partial, status);
  else
    hipLaunchKernelGGL((collect_partial_kernel<0, false>), g2, dim3(1024), 0, stream, x, T, K, ids, top_k, E,
                       chunk_rows, W, bm, partial, status);
  hipLaunchKernelGGL(collect_combine_kernel, dim3(static_cast<unsigned>((EK + 255) / 256)), dim3(256), 0, stream,
                     partial, nchunks, EK, sums, counts, ids ? int64_t(0) : T);
  const hipError_t le = hipGetLastError();
  hipFreeAsync(scratch, stream);
  return le == hipSuccess ? 0 : -1;
}

// ---------------------------------------------------------------------------
// Importance.  a_j = sqrt(max(m_j, floor_rel * mean)), m_j = sums_j / count.
// The mean is defined through an exact fixed-point sum so that any reduction
// order gives the same bits: with M = max_j m_j = f 2^eM (f in [0.5, 1)),
// L = ceil(log2 K) and s = 62 - eM - L, total = sum_j floor(m_j 2^s) is an
// integer below 2^62 and mean = fp32(fp64(total) 2^-s / K).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t fixed_term(float m, int s) {
  const uint32_t bits = __float_as_uint(m);
  const uint32_t eb = (bits >> 23) & 0xffu;
  const uint64_t mant = eb ? ((bits & 0x7fffffu) | 0x800000u) : (bits & 0x7fffffu);
  const int ex = eb ? static_cast<int>(eb) - 150 : -149;
  const int sh = ex + s;
  if (sh >= 0) return mant << sh;
  if (-sh >= 64) return 0;
  return mant >> (-sh);
}

__device__ __forceinline__ int frexp_exponent(float m) {  // m > 0: m = f 2^e, f in [0.5, 1)
  const uint32_t bits = __float_as_uint(m);
  const uint32_t eb = (bits >> 23) & 0xffu;
  if (eb) return static_cast<int>(eb) - 126;
  return (32 - __builtin_clz(bits & 0x7fffffu)) - 149;
}

__global__ void __launch_bounds__(1024) importance_kernel(const float *__restrict__ sums,
                                                          const int64_t *__restrict__ counts, int64_t K,
                                                          float floor_rel, int L, float *__restrict__ imp,
                                                          int32_t *status) {
  constexpr int NT = 1024, NW = NT / 64;
  __shared__ float s_f[NW];
  __shared__ int s_i[NW];
  __shared__ unsigned long long s_u[NW];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *se = sums + static_cast<int64_t>(e) * K;
  float *ie = imp + static_cast<int64_t>(e) * K;
  const int64_t c = counts[e];
  bool flat = c <= 0;
  float mx = 0.0f;
  int bad = 0;
  if (!flat) {
    const float fc = static_cast<float>(c);
    for (int64_t j = tid; j < K; j += NT) {
      const float m = se[j] / fc;
      bad |= !(finite_f(m) && m >= 0.0f);
      mx = fmaxf(mx, m);
      ie[j] = m;  // m_j kept in the output until the floor is known
    }
    for (int o = 32; o > 0; o >>= 1) {
      mx = fmaxf(mx, __shfl_xor(mx, o));
      bad |= __shfl_xor(bad, o);
    }
    if (lane == 0) { s_f[wave] = mx; s_i[wave] = bad; }
    __syncthreads();
    mx = s_f[0];
    bad = s_i[0];
    for (int w = 1; w < NW; ++w) { mx = fmaxf(mx, s_f[w]); bad |= s_i[w]; }
    if (bad && tid == 0) raise_status(status, ST_BADIMP);
    flat = bad || mx == 0.0f;
  }
  if (flat) {
    __syncthreads();
    for (int64_t j = tid; j < K; j += NT) ie[j] = 1.0f;
    return;
  }
  const int s = 62 - frexp_exponent(mx) - L;
  unsigned long long tot = 0;
  for (int64_t j = tid; j < K; j += NT) tot += fixed_term(ie[j], s);
  for (int o = 32; o > 0; o >>= 1) tot += __shfl_xor(tot, o);
  if (lane == 0) s_u[wave] = tot;
  __syncthreads();
  tot = 0;
  for (int w = 0; w < NW; ++w) tot += s_u[w];
  const float mean = static_cast<float>(ldexp(static_cast<double>(tot), -s) / static_cast<double>(K));
  const float fl = floor_rel * mean;
  for (int64_t j = tid; j < K; j += NT) ie[j] = sqrtf(fmaxf(ie[j], fl));
}

int launch_importance(const float *sums, const int64_t *counts, int E, int64_t K, float floor_rel, float *imp,
                      int32_t *status, hipStream_t stream) {
  int L = 0;
  while ((int64_t(1) << L) < K) ++L;
  hipLaunchKernelGGL(importance_kernel, dim3(static_cast<unsigned>(E)), dim3(1024), 0, stream, sums, counts, K,
                     floor_rel, L, imp, status);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace iq
