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
// result does not depend on order); a second pass reduces each (slice of a
// chunk, expert, 512-column tile) with 4 waves that take the slice's member
// tokens in turn (member m to wave m mod 4, each wave in token order, 8 rows per
// load batch of 16-byte loads), the wave partials combined in wave order; a
// last pass adds the slice partials to the running sums in slice order (chunk
// by chunk).  The sums therefore repeat bit for bit, and no x^2 temporary of
// the activation's size is ever materialised.

#include <type_traits>

#include "iq_common.hpp"
#include "iq_internal.hpp"

namespace iq {

// Pass 1 (routed): membership bitmaps bm[chunk - chunk0][e][words] and a
// per-token flag dup[t - chunk0 * chunk_rows] for tokens that name one expert
// twice, for the chunks of one window starting at chunk0.  One workgroup per
// 256 positions of a chunk: it clears its own 8 words of every expert's row
// (the chunk's last workgroup also the row's tail), then marks.
__global__ void __launch_bounds__(256) collect_route_kernel(const int32_t *__restrict__ ids, int64_t T,
                                                             int top_k, int E, int chunk_rows, int W,
                                                             int64_t chunk0, uint32_t *__restrict__ bm,
                                                             uint8_t *__restrict__ dup, int32_t *status) {
  const int nsub = (chunk_rows + 255) / 256;
  const int64_t lchunk = blockIdx.x / nsub;
  const int64_t chunk = chunk0 + lchunk;
  const int sub = static_cast<int>(blockIdx.x % nsub);
  uint32_t *reg = bm + lchunk * static_cast<int64_t>(E) * W;
  const int w0 = sub * 8;
  const int w1 = sub == nsub - 1 ? W : w0 + 8;
  for (int64_t i = threadIdx.x; i < static_cast<int64_t>(E) * (w1 - w0); i += blockDim.x)
    reg[(i / (w1 - w0)) * W + w0 + i % (w1 - w0)] = 0u;
  __syncthreads();
  const int64_t t0 = chunk * chunk_rows;
  const int64_t n = (T - t0 < chunk_rows) ? (T - t0) : chunk_rows;
  const int64_t p = static_cast<int64_t>(sub) * 256 + threadIdx.x;
  int st = 0;
  if (p < n) {
    bool rep = false;  // an expert named twice by this token
    for (int s = 0; s < top_k; ++s) {
      const int e = ids[(t0 + p) * top_k + s];
      if (e < 0 || e >= E) { st |= ST_BADID; continue; }
      for (int s2 = 0; s2 < s; ++s2) rep = rep || ids[(t0 + p) * top_k + s2] == e;
      atomicOr(&reg[static_cast<int64_t>(e) * W + (p >> 5)], 1u << (p & 31));
    }
    if (dup) dup[lchunk * chunk_rows + p] = rep ? 1 : 0;
  }
  raise_status(status, st);
}

// Pass 2: partial[slice][e][K] = sum over the slice's member tokens (routed to
// e; dense: all) of x^2, for the slices of one window (chunks chunk0 on; the
// bitmaps and repeat flags are the window's).  Workgroup = NW waves over a 512-column tile, 8
// columns per lane; member m of the slice (ascending tokens, a token routed
// twice to e counted twice) goes to wave m mod NW, which adds its members in
// token order, 8 rows per batch of 16-byte loads.  Routed slices (at most 1,024
// positions) first list their members in LDS from the bitmap words, one word
// per lane.
constexpr int kCPL = 8, kCTile = 64 * kCPL, kCBatch = 8, kMaxRoutedSlice = 1024;

template <int DT, bool VEC, int NW, bool ROUTED>
__global__ void __launch_bounds__(64 * NW) collect_slice_kernel(const void *__restrict__ x, int64_t T, int64_t K,
                                                                 const int32_t *__restrict__ ids, int top_k, int E,
                                                                 int chunk_rows, int W,
                                                                 const uint32_t *__restrict__ bm,
                                                                 const uint8_t *__restrict__ dup, int64_t chunk0,
                                                                 int nsub, int slice_len, float *__restrict__ partial,
                                                                 int64_t *__restrict__ counts, int32_t *status) {
  __shared__ float s_acc[NW][kCTile];
  __shared__ int s_cnt[NW];
  __shared__ int s_mem[ROUTED ? kMaxRoutedSlice : 1];
  __shared__ int s_nmem;
  const int64_t ntile = (K + kCTile - 1) / kCTile;
  const int64_t tile = blockIdx.x % ntile;
  const int64_t rest = blockIdx.x / ntile;  // slice * E + e
  const int e = static_cast<int>(rest % E);
  const int64_t slice = rest / E;
  const int64_t lchunk = slice / nsub;
  const int64_t chunk = chunk0 + lchunk;
  const int sub = static_cast<int>(slice % nsub);
  const int64_t cbase = chunk * chunk_rows;
  const int64_t n = (T - cbase < chunk_rows) ? (T - cbase) : chunk_rows;
  const int64_t p_lo = static_cast<int64_t>(sub) * slice_len;
  const int64_t p_hi = (p_lo + slice_len < n) ? p_lo + slice_len : n;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: token bookkeeping stays scalar
  const int lane = threadIdx.x & 63;
  const int64_t col = tile * kCTile + lane * kCPL;
  // lanes past the last column read a valid column and their results are dropped
  const int64_t colv = VEC ? (col < K ? col : K - kCPL) : col;

  int64_t nmem = p_hi > p_lo ? p_hi - p_lo : 0;  // dense: the positions themselves
  if (ROUTED) {
    if (wave == 0) {
      // lane l lists the members in word l of the slice: positions p_lo + 32 l + bit
      const int64_t nw = (nmem + 31) / 32;
      uint32_t word = 0u;
      if (lane < nw) {
        word = bm[(lchunk * E + e) * W + (p_lo >> 5) + lane];
        const int64_t lim = nmem - 32 * static_cast<int64_t>(lane);
        if (lim < 32) word &= (1u << lim) - 1u;
      }
      const int cnt = __builtin_popcount(word);
      int pre = cnt;  // inclusive prefix over lanes
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(pre, d);
        if (lane >= d) pre += o;
      }
      int at = pre - cnt;
      while (word) {
        s_mem[at++] = static_cast<int>(p_lo + 32 * lane + __builtin_ctz(word));
        word &= word - 1u;
      }
      if (lane == 63) s_nmem = pre;
    }
    __syncthreads();
    nmem = s_nmem;
  }

  float acc[kCPL];
#pragma unroll
  for (int j = 0; j < kCPL; ++j) acc[j] = 0.0f;
  bool finite = true;
  int pairs = 0;  // routed (token, slot) pairs seen by this wave
  for (int64_t m0 = wave; m0 < nmem; m0 += static_cast<int64_t>(NW) * kCBatch) {
    int64_t tok[kCBatch];
    int mult[kCBatch];
#pragma unroll
    for (int u = 0; u < kCBatch; ++u) {
      const int64_t mi = m0 + static_cast<int64_t>(u) * NW;
      const bool ok = mi < nmem;
      const int64_t q = ok ? (ROUTED ? s_mem[mi] : p_lo + mi) : (ROUTED ? s_mem[0] : p_lo);
      tok[u] = cbase + q;
      mult[u] = ok ? 1 : 0;
    }
    if (ROUTED) {
#pragma unroll
      for (int u = 0; u < kCBatch; ++u) {
        if (mult[u] && dup[tok[u] - chunk0 * chunk_rows]) {  // rare: count the repeats of e in this token's ids
          int c = 0;
          for (int s2 = 0; s2 < top_k; ++s2) c += ids[tok[u] * top_k + s2] == e;
          mult[u] = c;
        }
        pairs += mult[u];
      }
    }
    float v[kCBatch][kCPL];
#pragma unroll
    for (int u = 0; u < kCBatch; ++u) {
      const int64_t off = tok[u] * K + colv;
      if (VEC) {
        if (DT == 1) {
          const uint4 q = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + off);
          const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            v[u][2 * h] = __uint_as_float(qq[h] << 16);
            v[u][2 * h + 1] = __uint_as_float(qq[h] & 0xffff0000u);
          }
        } else {
          const float4 q0 = *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + off);
          const float4 q1 = *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + off + 4);
          v[u][0] = q0.x; v[u][1] = q0.y; v[u][2] = q0.z; v[u][3] = q0.w;
          v[u][4] = q1.x; v[u][5] = q1.y; v[u][6] = q1.z; v[u][7] = q1.w;
        }
      } else {
#pragma unroll
        for (int j = 0; j < kCPL; ++j) {
          const int64_t c = col + j < K ? off + j : tok[u] * K + (K - 1);
          v[u][j] = DT == 1 ? bf16_to_f32(static_cast<const uint16_t *>(x)[c]) : static_cast<const float *>(x)[c];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kCBatch; ++u) {
      for (int rep = 0; rep < mult[u]; ++rep) {
#pragma unroll
        for (int j = 0; j < kCPL; ++j) {
          if (col + j < K) finite = finite && finite_f(v[u][j]);
          acc[j] = __builtin_fmaf(v[u][j], v[u][j], acc[j]);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kCPL; ++j) s_acc[wave][lane * kCPL + j] = acc[j];
  if (ROUTED && lane == 0) s_cnt[wave] = pairs;
  if (!finite) raise_status(status, ST_NONFINITE);
  __syncthreads();
  if (ROUTED && tile == 0 && threadIdx.x == 0) {  // one column tile counts the expert's pairs
    int64_t c = 0;
    for (int w = 0; w < NW; ++w) c += s_cnt[w];
    if (c) atomicAdd(reinterpret_cast<unsigned long long *>(counts + e), static_cast<unsigned long long>(c));
  }
  for (int c = threadIdx.x; c < kCTile; c += blockDim.x) {
    const int64_t cc = tile * kCTile + c;
    float p = s_acc[0][c];
#pragma unroll
    for (int w = 1; w < NW; ++w) p = p + s_acc[w][c];
    if (cc < K) partial[rest * K + cc] = p;
  }
}

// Pass 3: sums[e][j] += partial[0][e][j]; += partial[1][e][j]; ... (slice order)
__global__ void __launch_bounds__(256) collect_combine_kernel(const float *__restrict__ partial, int64_t nchunks,
                                                               int64_t EK, float *__restrict__ sums,
                                                               int64_t *counts, int64_t dense_T) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i == 0 && dense_T > 0) counts[0] += dense_T;
  if (i >= EK) return;
  float s = sums[i];
  int64_t c = 0;
  for (; c + 8 <= nchunks; c += 8) {
    float p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) p[u] = partial[(c + u) * EK + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) s = s + p[u];
  }
  for (; c < nchunks; ++c) s = s + partial[c * EK + i];
  sums[i] = s;
}

template <int DT, bool VEC, int NW, bool ROUTED>
static void launch_slices(dim3 g, hipStream_t stream, const void *x, int64_t T, int64_t K, const int32_t *ids,
                          int top_k, int E, int chunk_rows, int W, const uint32_t *bm, const uint8_t *dup,
                          int64_t chunk0, int nsub, int slice_len, float *partial, int64_t *counts,
                          int32_t *status) {
  hipLaunchKernelGGL((collect_slice_kernel<DT, VEC, NW, ROUTED>), g, dim3(64 * NW), 0, stream, x, T, K, ids, top_k, E,
                     chunk_rows, W, bm, dup, chunk0, nsub, slice_len, partial, counts, status);
}

// Slices: dense workgroups of 16 waves, routed ones of 4; a window holds
// enough chunks for ~4,096 (chunk, expert, column tile) units (at least one
// chunk), and each of its chunks is cut into nsub slices so the window's
// launch has >= 128 (dense) / 512 (routed) workgroups; routed slices hold at
// most 1,024 positions.  The partials of a window are added to the sums in
// slice order before the next window reuses them, which is the same sequence
// of fp32 additions as one pass over all slices.
constexpr int64_t kWindowUnits = 4096;

CollectPlan plan_collect(int64_t T, int64_t K, bool routed, int E, int chunk_rows) {
  CollectPlan p{};
  p.nchunks = (T + chunk_rows - 1) / chunk_rows;
  p.W = (chunk_rows + 31) / 32 + 1;
  p.ntile = (K + kCTile - 1) / kCTile;
  const int64_t units = static_cast<int64_t>(E) * p.ntile;  // per chunk
  int64_t wc = (kWindowUnits + units - 1) / units;
  p.wchunks = p.nchunks < wc ? p.nchunks : wc;
  if (p.wchunks < 1) p.wchunks = 1;
  const int64_t want = routed ? 512 : 128;
  int64_t nsub = (want + p.wchunks * units - 1) / (p.wchunks * units);
  if (routed && nsub < (chunk_rows + kMaxRoutedSlice - 1) / kMaxRoutedSlice)
    nsub = (chunk_rows + kMaxRoutedSlice - 1) / kMaxRoutedSlice;
  const int64_t max_sub = (chunk_rows + 31) / 32;
  if (nsub > max_sub) nsub = max_sub;
  if (nsub < 1) nsub = 1;
  p.slice_len = ((chunk_rows + nsub - 1) / nsub + 31) / 32 * 32;
  p.nsub = (chunk_rows + p.slice_len - 1) / p.slice_len;
  const size_t pbytes = static_cast<size_t>(p.wchunks) * p.nsub * E * K * sizeof(float);
  const size_t bbytes = routed ? static_cast<size_t>(p.wchunks) * E * p.W * sizeof(uint32_t) : 0;
  const size_t dbytes = routed ? static_cast<size_t>(p.wchunks) * chunk_rows : 0;
  p.boff = ws_up(pbytes);
  p.doff = p.boff + ws_up(bbytes);
  p.bytes = p.doff + ws_up(dbytes) + kWsAlign;
  return p;
}

int launch_collect(const void *x, int dtype, int64_t T, int64_t K, const int32_t *ids, int top_k, int E,
                   int chunk_rows, float *sums, int64_t *counts, int32_t *status, void *ws, hipStream_t stream) {
  if (T == 0) return 0;
  const CollectPlan P = plan_collect(T, K, ids != nullptr, E, chunk_rows);
  char *base = ws_base(ws);
  float *partial = reinterpret_cast<float *>(base);
  uint32_t *bm = ids ? reinterpret_cast<uint32_t *>(base + P.boff) : nullptr;
  uint8_t *dup = ids ? reinterpret_cast<uint8_t *>(base + P.doff) : nullptr;
  const int64_t EK = static_cast<int64_t>(E) * K;
  const bool vec = K % kCPL == 0;  // 16-byte (bf16) / 32-byte (f32) aligned rows, whole 8-column lanes
  const int ns = static_cast<int>(P.nsub), sl = static_cast<int>(P.slice_len);
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using BT = std::true_type;
  using BF = std::false_type;
  using WR = std::integral_constant<int, 4>;
  using WD = std::integral_constant<int, 16>;
  for (int64_t c0 = 0; c0 < P.nchunks; c0 += P.wchunks) {
    const int64_t nc = P.nchunks - c0 < P.wchunks ? P.nchunks - c0 : P.wchunks;
    const int64_t nslices = nc * P.nsub;
    if (ids) {
      hipLaunchKernelGGL(collect_route_kernel, dim3(static_cast<unsigned>(nc * ((chunk_rows + 255) / 256))),
                         dim3(256), 0, stream, ids, T, top_k, E, chunk_rows, P.W, c0, bm, dup, status);
      if (hipGetLastError() != hipSuccess) return -1;
    }
    const dim3 g2(static_cast<unsigned>(nslices * E * P.ntile));
    const uint32_t *bmc = bm;
    auto go = [&](auto dt, auto v, auto nw, auto r) {
      launch_slices<decltype(dt)::value, decltype(v)::value, decltype(nw)::value, decltype(r)::value>(
          g2, stream, x, T, K, ids, top_k, E, chunk_rows, P.W, bmc, dup, c0, ns, sl, partial, counts, status);
    };
    if (ids) {
      if (dtype == 1) { if (vec) go(I1{}, BT{}, WR{}, BT{}); else go(I1{}, BF{}, WR{}, BT{}); }
      else { if (vec) go(I0{}, BT{}, WR{}, BT{}); else go(I0{}, BF{}, WR{}, BT{}); }
    } else {
      if (dtype == 1) { if (vec) go(I1{}, BT{}, WD{}, BF{}); else go(I1{}, BF{}, WD{}, BF{}); }
      else { if (vec) go(I0{}, BT{}, WD{}, BF{}); else go(I0{}, BF{}, WD{}, BF{}); }
    }
    if (hipGetLastError() != hipSuccess) return -1;
    hipLaunchKernelGGL(collect_combine_kernel, dim3(static_cast<unsigned>((EK + 255) / 256)), dim3(256), 0, stream,
                       partial, nslices, EK, sums, counts, (ids || c0 > 0) ? int64_t(0) : T);
    if (hipGetLastError() != hipSuccess) return -1;
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Importance.  a_j = sqrt(max(m_j, floor_rel * mean)), m_j = sums_j / count
// (IEEE fp32 division and square root).  The mean is the plain one: the m_j
// added one after another in fp64, j ascending from 0, the total divided by K
// in fp64 and rounded to fp32.
//
// When no partial sum can round, every order of additions gives that running
// sum, so the workgroup adds the m_j in parallel.  The non-negative fp32 m_j
// are all integer multiples of q, the least ulp among the nonzero ones, and so
// is every partial sum in any order; a partial sum below 2^53 q is then exact
// in fp64.  All of them lie below the true total S, so S < 2^53 q suffices.
// The parallel fp64 total S' of n non-negative terms satisfies
// S <= S' (1 + (n + 4) 2^-52) (each of at most n - 1 additions rounds by a
// relative 2^-53), so S' (1 + (n + 4) 2^-52) < 2^53 q proves it, and S' is
// then exactly the running sum.
//
// Otherwise the running sum is one dependent chain: wave 0 walks it 64 values
// at a time -- each lane converts one m_j to fp64 into LDS, then every lane
// reads the 64 values back into registers (a broadcast) and adds them in
// order, so each add of the chain takes VGPR operands only; the next 64 are
// loaded while it adds.  Lanes past K add +0.0, which leaves the sum unchanged
// (it starts at +0 and only meets non-negative values).  A flagged expert
// (a value negative or not finite) takes flat weights without a mean.
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(1024) importance_kernel(const float *__restrict__ sums,
                                                          const int64_t *__restrict__ counts, int64_t K,
                                                          float floor_rel, float *__restrict__ imp,
                                                          int32_t *status) {
  constexpr int NT = 1024, NW = NT / 64;
  __shared__ int s_i[NW], s_u[NW];
  __shared__ double s_s[NW];
  __shared__ float s_mean;
  __shared__ __attribute__((aligned(16))) double s_chain[64];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *se = sums + static_cast<int64_t>(e) * K;
  float *ie = imp + static_cast<int64_t>(e) * K;
  const int64_t c = counts[e];
  if (c <= 0) {  // idle expert: flat weights
    for (int64_t j = tid; j < K; j += NT) ie[j] = 1.0f;
    return;
  }
  const float fc = static_cast<float>(c);
  int bad = 0;
  int umin = 1 << 20;  // least ulp exponent among the nonzero m_j
  double part = 0.0;
  for (int64_t j = tid; j < K; j += NT) {
    const float m = se[j] / fc;
    bad |= !(finite_f(m) && m >= 0.0f);
    if (m > 0.0f) {
      const int ef = static_cast<int>(__float_as_uint(m) >> 23);  // biased exponent (sign is 0)
      umin = min(umin, (ef > 1 ? ef : 1) - 150);
    }
    part += static_cast<double>(m);
    ie[j] = m;  // m_j kept in the output until the floor is known
  }
  for (int o = 32; o > 0; o >>= 1) {
    bad |= __shfl_xor(bad, o);
    umin = min(umin, __shfl_xor(umin, o));
    part += __shfl_xor(part, o);
  }
  if (lane == 0) {
    s_i[wave] = bad;
    s_u[wave] = umin;
    s_s[wave] = part;
  }
  __syncthreads();
  bad = 0;
  umin = 1 << 20;
  double tot = 0.0;
  for (int w = 0; w < NW; ++w) {
    bad |= s_i[w];
    umin = min(umin, s_u[w]);
    tot += s_s[w];
  }
  // exact in any order when tot (1 + (K + 4) 2^-52) < 2^53 q (all-zero: tot = 0)
  const bool exact = umin > (1 << 19) || tot * (1.0 + static_cast<double>(K + 4) * 0x1p-52) < ldexp(1.0, umin + 53);
  if (wave == 0 && !bad) {
    if (exact) {
      if (lane == 0) s_mean = static_cast<float>(tot / static_cast<double>(K));
    } else {
      double acc = 0.0;
      float nxt = lane < K ? se[lane] : 0.0f;
      for (int64_t j0 = 0; j0 < K; j0 += 64) {
        s_chain[lane] = j0 + lane < K ? static_cast<double>(nxt / fc) : 0.0;
        nxt = j0 + 64 + lane < K ? se[j0 + 64 + lane] : 0.0f;
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        double v[64];
#pragma unroll
        for (int l = 0; l < 64; l += 2) {
          const double2 q = reinterpret_cast<const double2 *>(s_chain)[l / 2];
          v[l] = q.x;
          v[l + 1] = q.y;
        }
#pragma unroll
        for (int l = 0; l < 64; ++l) acc = acc + v[l];
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
      }
      if (lane == 0) s_mean = static_cast<float>(acc / static_cast<double>(K));
    }
  }
  __syncthreads();
  if (bad && tid == 0) raise_status(status, ST_BADIMP);
  const float mean = bad ? 0.0f : s_mean;
  if (bad || mean == 0.0f) {  // nothing usable: flat weights
    for (int64_t j = tid; j < K; j += NT) ie[j] = 1.0f;
    return;
  }
  const float fl = floor_rel * mean;
  for (int64_t j = tid; j < K; j += NT) ie[j] = sqrtf(fmaxf(ie[j], fl));
}

int launch_importance(const float *sums, const int64_t *counts, int E, int64_t K, float floor_rel, float *imp,
                      int32_t *status, hipStream_t stream) {
  hipLaunchKernelGGL(importance_kernel, dim3(static_cast<unsigned>(E)), dim3(1024), 0, stream, sums, counts, K,
                     floor_rel, imp, status);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ---------------------------------------------------------------------------
// Merge of two collections' statistics (the GGUF imatrix files keep in_sum2
// and counts per tensor so that they can be merged; summing ranks' statistics
// is the same operation): sums[e][j] = sums[e][j] + src[e][j], one fp32
// addition per element; counts[e] += src_counts[e].  One thread per element,
// or per 4 elements as one 16-byte access when K and the pointers allow;
// non-finite source values of an expert the source touched raise the
// non-finite bit.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) merge_kernel(const float *__restrict__ src, const int64_t *__restrict__ src_counts,
                                                    int E, int64_t K, float *__restrict__ sums,
                                                    int64_t *__restrict__ counts, bool vec, int32_t *status) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < E) counts[i] += src_counts[i];
  const int64_t n = static_cast<int64_t>(E) * K;
  int st = 0;
  if (vec) {
    if (4 * i >= n) return;
    const int64_t e = 4 * i / K;
    const float4 v = reinterpret_cast<const float4 *>(src)[i];
    float4 d = reinterpret_cast<float4 *>(sums)[i];
    if (src_counts[e] != 0 && !(finite_f(v.x) && finite_f(v.y) && finite_f(v.z) && finite_f(v.w)))
      st = ST_NONFINITE;
    d.x = d.x + v.x; d.y = d.y + v.y; d.z = d.z + v.z; d.w = d.w + v.w;
    reinterpret_cast<float4 *>(sums)[i] = d;
  } else {
    if (i >= n) return;
    const float v = src[i];
    if (src_counts[i / K] != 0 && !finite_f(v)) st = ST_NONFINITE;
    sums[i] = sums[i] + v;
  }
  raise_status(status, st);
}

int launch_merge(const float *src, const int64_t *src_counts, int E, int64_t K, float *sums, int64_t *counts,
                 int32_t *status, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(E) * K;
  const bool vec = (K & 3) == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(sums) & 15) == 0;
  const int64_t threads = vec ? n / 4 : n;
  const int64_t total = threads > E ? threads : E;
  hipLaunchKernelGGL(merge_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, stream, src,
                     src_counts, E, K, sums, counts, vec, status);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ---------------------------------------------------------------------------
// Routed token lists (for the Hessian blocks): each expert's member tokens in
// ascending order, built once from the routing bitmaps, so that a wave reads
// its next tokens with one coalesced load instead of walking bitmap words.
// An entry is the token index, with bit 31 set when the token names the
// expert more than once (the reader then repeats it).  lstart[e] is the
// expert's first entry, lstart[E] the total.
// ---------------------------------------------------------------------------
// entries per expert: one wave per expert, popcounts of its bitmap words
__global__ void __launch_bounds__(256) route_count_kernel(const uint32_t *__restrict__ bm, int64_t nchunks, int E,
                                                           int W, int64_t *__restrict__ lens) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (e >= E) return;
  int64_t n = 0;
  for (int64_t i = lane; i < nchunks * W; i += 64) {
    const int64_t c = i / W, q = i % W;
    n += __builtin_popcount(bm[(c * E + e) * W + q]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o);
  if (lane == 0) lens[e] = n;
}

// lstart = exclusive prefix sum of lens (one workgroup of 1,024 threads, each a
// contiguous run of experts)
__global__ void __launch_bounds__(1024) route_scan_kernel(const int64_t *__restrict__ lens, int E, int64_t target,
                                                          int64_t *__restrict__ lstart, int64_t *__restrict__ sstart,
                                                          int64_t *__restrict__ pstart, int32_t *__restrict__ heavy) {
  // three exclusive scans over the experts: list entries, Hessian splits
  // (ceil(len / target), at least one) and partial slots (the splits of the
  // experts cut into more than one); then the cut experts in order
  __shared__ int64_t s_part[3][1024];
  const int per = (E + 1023) / 1024;
  const int e0 = threadIdx.x * per, e1 = e0 + per < E ? e0 + per : E;
  auto nsp = [&](int64_t len) -> int64_t { return len > target ? (len + target - 1) / target : 1; };
  int64_t own[3] = {0, 0, 0};
  for (int e = e0; e < e1; ++e) {
    const int64_t n = nsp(lens[e]);
    own[0] += lens[e];
    own[1] += n;
    own[2] += n > 1 ? n : 0;
  }
  for (int k = 0; k < 3; ++k) s_part[k][threadIdx.x] = own[k];
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive scans over the 1,024 runs
    int64_t v[3];
    for (int k = 0; k < 3; ++k) v[k] = threadIdx.x >= o ? s_part[k][threadIdx.x - o] : 0;
    __syncthreads();
    for (int k = 0; k < 3; ++k) s_part[k][threadIdx.x] += v[k];
    __syncthreads();
  }
  int64_t run[3];
  for (int k = 0; k < 3; ++k) run[k] = s_part[k][threadIdx.x] - own[k];
  for (int e = e0; e < e1; ++e) {
    const int64_t n = nsp(lens[e]);
    lstart[e] = run[0];
    sstart[e] = run[1];
    pstart[e] = run[2];
    run[0] += lens[e];
    run[1] += n;
    run[2] += n > 1 ? n : 0;
  }
  if (threadIdx.x == 1023) {
    lstart[E] = s_part[0][1023];
    sstart[E] = s_part[1][1023];
    pstart[E] = s_part[2][1023];
  }
  __syncthreads();
  if (threadIdx.x == 0) {  // the cut experts, ascending (few: each holds more than target entries)
    int h = 0;
    for (int e = 0; e < E; ++e)
      if (sstart[e + 1] - sstart[e] > 1) heavy[h++] = e;
    heavy[E] = h;
  }
}

// the lists: one workgroup per expert walks its bitmap words in token order,
// 256 words at a time (a word per thread, positions by a workgroup scan of the
// popcounts), and writes each member with its repeat flag
__global__ void __launch_bounds__(256) route_list_kernel(const uint32_t *__restrict__ bm,
                                                          const uint8_t *__restrict__ dup, int64_t nchunks, int E,
                                                          int W, int chunk_rows, const int64_t *__restrict__ lstart,
                                                          uint32_t *__restrict__ list) {
  __shared__ int s_w[4];
  const int e = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t base = lstart[e];
  const int64_t nw = nchunks * W;
  for (int64_t i0 = 0; i0 < nw; i0 += 256) {
    const int64_t i = i0 + threadIdx.x;
    uint32_t bits = 0u;
    int64_t c = 0, q = 0;
    if (i < nw) {
      c = i / W;
      q = i % W;
      bits = bm[(c * E + e) * W + q];
    }
    const int n = __builtin_popcount(bits);
    int incl = n;  // inclusive scan within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    if (lane == 63) s_w[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      before += w < wave ? s_w[w] : 0;
      total += s_w[w];
    }
    int64_t pos = base + before + incl - n;
    const int64_t t0 = c * chunk_rows + q * 32;
    for (uint32_t b = bits; b; b &= b - 1u) {
      const int64_t t = t0 + __builtin_ctz(b);
      list[pos++] = static_cast<uint32_t>(t) | (dup[t] ? 0x80000000u : 0u);
    }
    base += total;
    __syncthreads();  // s_w is rewritten by the next round
  }
}

// ---------------------------------------------------------------------------
// Hessian diagonal blocks for the local-Hessian choice search (ModelOpt PR
// #3158: the layer-output error is taken over the 256-column diagonal blocks
// of the input Hessian).  hess[e][b] += sum over the (token, slot) pairs
// routed to e of x_t,b x_t,b^T, x_t,b the token's 256 columns of block b.
//
// A dense contraction, so it runs on the matrix cores.  One wave computes one
// 64x64 tile (ti <= tj of the 4x4 tiles of a block; the mirror tile is written
// from the same registers, so the result is exactly symmetric) as 2x2 MFMA
// 32x32 tiles (bf16: v_mfma_f32_32x32x16_bf16, whose products are exact in
// fp32; f32: v_mfma_f32_32x32x2_f32) over one token range.  Each step stages
// 32 tokens transposed in LDS ([column][token], padded rows), the operand
// layout the MFMA reads.  Tokens are taken in ascending order, each as often
// as it is routed to e; token ranges ("splits") give the chip enough waves
// when E * blocks is small, and their partial tiles are added in split order,
// so the sums repeat bit for bit.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kHTok = 32;  // tokens per step

// bf16 input: held to three waves per SIMD (156 registers, none spilled; 2%
// faster than the two that 144 VGPRs + 64 AGPRs allow); fp32, whose staging
// needs more registers, would spill at three and keeps two.
template <int DT>
__global__ void __launch_bounds__(64, DT == 1 ? 3 : 1) hessian_kernel(const void *__restrict__ x, int64_t T, int64_t K,
                                                     const int32_t *__restrict__ ids, int top_k, int E,
                                                     const uint32_t *__restrict__ list,
                                                     const int64_t *__restrict__ lstart,
                                                     const int64_t *__restrict__ sstart,
                                                     const int64_t *__restrict__ pstart, int64_t nsplit,
                                                     int64_t split_len, float *__restrict__ hess,
                                                     float *__restrict__ partial, int32_t *status) {
  constexpr int RS = DT == 1 ? 40 : 33;  // LDS row: 32 tokens + padding (bf16 80 B, f32 132 B)
  using elem_t = typename std::conditional<DT == 1, uint16_t, float>::type;
  __shared__ __attribute__((aligned(16))) elem_t sA[64][RS];
  __shared__ __attribute__((aligned(16))) elem_t sB[64][RS];
  __shared__ int s_tok[kHTok];
  const int64_t nb = K / 256;
  // Dense: workgroup = (split, block, tile) with uniform token splits.
  // Routed: workgroup = (split slot, block, tile); the slots are numbered expert
  // by expert (sstart), an expert holding ceil(len / target) of them.  One slot:
  // the expert's whole list, added into hess; several: equal shares of the list,
  // each written to its own partial slot (pstart) for the combine.
  int64_t t0, t1, slot_e = 0;
  int e, b, tp;
  float *Hdst;
  bool accumulate;
  if (ids == nullptr) {
    const int64_t ntiles = static_cast<int64_t>(E) * nb * 10;
    const int64_t split = blockIdx.x / ntiles, rem = blockIdx.x % ntiles;
    tp = static_cast<int>(rem % 10);
    b = static_cast<int>((rem / 10) % nb);
    e = static_cast<int>(rem / 10 / nb);
    t0 = split * split_len;
    t1 = (t0 + split_len < T) ? t0 + split_len : T;
    accumulate = nsplit == 1;
    Hdst = accumulate ? hess + (static_cast<int64_t>(e) * nb + b) * 65536
                      : partial + ((split * E + e) * nb + b) * 65536;
  } else {
    const int64_t slot = blockIdx.x / (nb * 10), rem = blockIdx.x % (nb * 10);
    if (slot >= sstart[E]) return;  // the grid is sized for the most slots the lists allow
    tp = static_cast<int>(rem % 10);
    b = static_cast<int>(rem / 10);
    int lo = 0, hi = E;  // the expert: sstart[e] <= slot < sstart[e + 1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sstart[mid] <= slot) lo = mid; else hi = mid;
    }
    e = lo;
    slot_e = slot - sstart[e];
    const int64_t n = sstart[e + 1] - sstart[e];
    const int64_t ls = lstart[e], len = lstart[e + 1] - ls;
    t0 = ls + slot_e * len / n;
    t1 = ls + (slot_e + 1) * len / n;
    accumulate = n == 1;
    Hdst = accumulate ? hess + (static_cast<int64_t>(e) * nb + b) * 65536
                      : partial + ((pstart[e] + slot_e) * nb + b) * 65536;
  }
  int ti = 0;
  while (tp >= 4 - ti) { tp -= 4 - ti; ++ti; }
  const int tj = ti + tp;
  const int lane = threadIdx.x;
  const int64_t colA = static_cast<int64_t>(b) * 256 + ti * 64, colB = static_cast<int64_t>(b) * 256 + tj * 64;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  // token stream.  Dense: the range in order.  Routed: the list entries
  // [t0, t1), 32 per batch; their load is issued one batch ahead.  An entry
  // flagged as naming e more than once sends that batch down a path where lane
  // 0 repeats the token as often as e appears in its ids.
  int64_t cur = t0;
  int pending = 0;        // repeats of `last` still to place (routed slow path)
  int last = 0;
  bool finite = true;
  uint32_t ent = 0u;      // routed: list entry cur + lane (lanes < 32), loaded ahead
  auto fetch = [&]() {
    ent = (ids != nullptr && lane < kHTok && cur + lane < t1) ? list[cur + lane] : 0u;
  };
  fetch();
  // next batch of tokens into s_tok; returns how many (uniform)
  auto fill = [&]() -> int {
    int nt = 0;
    if (ids == nullptr) {
      nt = static_cast<int>((t1 - cur < kHTok) ? t1 - cur : kHTok);
      if (lane < kHTok) s_tok[lane] = lane < nt ? static_cast<int>(cur + lane) : -1;
      cur += nt;
      return nt;
    }
    const int64_t avail = t1 - cur;
    const uint64_t flagged = __ballot(lane < kHTok && lane < avail && (ent >> 31));
    if (pending == 0 && flagged == 0) {
      nt = static_cast<int>(avail < kHTok ? avail : kHTok);
      if (lane < kHTok) s_tok[lane] = lane < nt ? static_cast<int>(ent & 0x7fffffffu) : -1;
      cur += nt;
      fetch();
      return nt;
    }
    if (lane == 0) {
      while (nt < kHTok) {
        if (pending > 0) {
          s_tok[nt++] = last;
          --pending;
          continue;
        }
        if (cur >= t1) break;
        const uint32_t en = list[cur++];
        last = static_cast<int>(en & 0x7fffffffu);
        int mult = 1;
        if (en >> 31) {
          mult = 0;
          for (int s = 0; s < top_k; ++s) mult += ids[static_cast<int64_t>(last) * top_k + s] == e;
        }
        s_tok[nt++] = last;
        pending = mult - 1;
      }
      for (int q = nt; q < kHTok; ++q) s_tok[q] = -1;
    }
    // lane 0 advanced the stream: every lane takes its state
    cur = static_cast<int64_t>(__shfl(static_cast<long long>(cur), 0));
    pending = __shfl(pending, 0);
    last = __shfl(last, 0);
    fetch();
    return __shfl(nt, 0);
  };
  // this lane's share of a batch: bf16 -- column pair cp of both tiles for token
  // octets g = lane/32, lane/32 + 2; f32 -- 4 columns of one token, 8 times
  constexpr int NLD = DT == 1 ? 16 : 32;
  uint32_t ra[NLD], rb[NLD];
  auto issue = [&]() {
    if (DT == 1) {
      const int cp = lane & 31;
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int g = (lane >> 5) + 2 * it;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int tok = s_tok[8 * g + j];
          ra[it * 8 + j] = 0u;
          rb[it * 8 + j] = 0u;
          if (tok >= 0) {
            const uint16_t *xr = static_cast<const uint16_t *>(x) + static_cast<int64_t>(tok) * K;
            ra[it * 8 + j] = *reinterpret_cast<const uint32_t *>(xr + colA + 2 * cp);
            rb[it * 8 + j] = *reinterpret_cast<const uint32_t *>(xr + colB + 2 * cp);
          }
        }
      }
    } else {
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int qd = lane + 64 * it;
        const int tt = qd >> 4, cc = (qd & 15) * 4;
        const int tok = s_tok[tt];
        float4 va = make_float4(0.f, 0.f, 0.f, 0.f), vb = make_float4(0.f, 0.f, 0.f, 0.f);
        if (tok >= 0) {
          const float *xr = static_cast<const float *>(x) + static_cast<int64_t>(tok) * K;
          va = *reinterpret_cast<const float4 *>(xr + colA + cc);
          vb = *reinterpret_cast<const float4 *>(xr + colB + cc);
        }
        ra[4 * it] = __float_as_uint(va.x); ra[4 * it + 1] = __float_as_uint(va.y);
        ra[4 * it + 2] = __float_as_uint(va.z); ra[4 * it + 3] = __float_as_uint(va.w);
        rb[4 * it] = __float_as_uint(vb.x); rb[4 * it + 1] = __float_as_uint(vb.y);
        rb[4 * it + 2] = __float_as_uint(vb.z); rb[4 * it + 3] = __float_as_uint(vb.w);
      }
    }
  };
  auto stage = [&]() {
    if (DT == 1) {
      const int cp = lane & 31;
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int g = (lane >> 5) + 2 * it;
        const uint32_t *va = ra + it * 8, *vb = rb + it * 8;
        uint4 a0, a1, b0, b1;
        uint32_t *pa0 = &a0.x, *pa1 = &a1.x, *pb0 = &b0.x, *pb1 = &b1.x;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pa0[j] = (va[2 * j] & 0xffffu) | (va[2 * j + 1] << 16);
          pa1[j] = (va[2 * j] >> 16) | (va[2 * j + 1] & 0xffff0000u);
          pb0[j] = (vb[2 * j] & 0xffffu) | (vb[2 * j + 1] << 16);
          pb1[j] = (vb[2 * j] >> 16) | (vb[2 * j + 1] & 0xffff0000u);
          finite = finite && finite_f(__uint_as_float(va[2 * j] << 16)) &&
                   finite_f(__uint_as_float(va[2 * j] & 0xffff0000u)) &&
                   finite_f(__uint_as_float(va[2 * j + 1] << 16)) &&
                   finite_f(__uint_as_float(va[2 * j + 1] & 0xffff0000u));
        }
        *reinterpret_cast<uint4 *>(&sA[2 * cp][8 * g]) = a0;
        *reinterpret_cast<uint4 *>(&sA[2 * cp + 1][8 * g]) = a1;
        *reinterpret_cast<uint4 *>(&sB[2 * cp][8 * g]) = b0;
        *reinterpret_cast<uint4 *>(&sB[2 * cp + 1][8 * g]) = b1;
      }
    } else {
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int qd = lane + 64 * it;
        const int tt = qd >> 4, cc = (qd & 15) * 4;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float av = __uint_as_float(ra[4 * it + c]);
          sA[cc + c][tt] = av;
          sB[cc + c][tt] = __uint_as_float(rb[4 * it + c]);
          finite = finite && finite_f(av);
        }
      }
    }
  };
  int nt = fill();
  __syncthreads();
  if (nt > 0) {
    issue();
    stage();
  }
  __syncthreads();
  while (nt > 0) {
    // the next batch's tokens and loads are in flight while this one multiplies
    const int nn = fill();
    __syncthreads();
    if (nn > 0) issue();
    if (DT == 1) {
#pragma unroll
      for (int ks = 0; ks < kHTok / 16; ++ks) {
        bf16x8_t a[2], bb[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          a[m] = *reinterpret_cast<const bf16x8_t *>(&sA[m * 32 + (lane & 31)][16 * ks + 8 * (lane >> 5)]);
          bb[m] = *reinterpret_cast<const bf16x8_t *>(&sB[m * 32 + (lane & 31)][16 * ks + 8 * (lane >> 5)]);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int n = 0; n < 2; ++n)
            acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m], bb[n], acc[m][n], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < kHTok / 2; ++ks) {
        float a[2], bb[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          a[m] = sA[m * 32 + (lane & 31)][2 * ks + (lane >> 5)];
          bb[m] = sB[m * 32 + (lane & 31)][2 * ks + (lane >> 5)];
        }
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int n = 0; n < 2; ++n)
            acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[m], bb[n], acc[m][n], 0, 0, 0);
      }
    }
    __syncthreads();
    if (nn > 0) stage();
    __syncthreads();
    nt = nn;
  }
  if (!finite) raise_status(status, ST_NONFINITE);
  // Per 32 x 32 product: its 16 values and their mirror images (off-diagonal
  // tiles) are read together, then added and written, so the read latency is
  // paid once per product rather than once per value.
  float *Hb = Hdst;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const bool mirror = ti != tj;
      const int col = tj * 64 + n * 32 + (lane & 31);
      float od[16], om[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = ti * 64 + m * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        od[q] = accumulate ? Hb[row * 256 + col] : 0.0f;
        om[q] = accumulate && mirror ? Hb[col * 256 + row] : 0.0f;
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = ti * 64 + m * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        const float v = acc[m][n][q];
        Hb[row * 256 + col] = accumulate ? od[q] + v : v;
        if (mirror) Hb[col * 256 + row] = accumulate ? om[q] + v : v;
      }
    }
}

// hess[i] += partial[0][i] + partial[1][i] + ... in split order.
__global__ void __launch_bounds__(256) hessian_combine_kernel(const float *__restrict__ partial, int64_t nsplit,
                                                              int64_t n, float *__restrict__ hess) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  float s = partial[i];
  for (int64_t k = 1; k < nsplit; ++k) s = s + partial[k * n + i];
  hess[i] = hess[i] + s;
}

// Routed: for each expert cut into several splits (heavy[0 .. heavy[E])),
// hess += partial[first] + partial[first + 1] + ... in split order.
__global__ void __launch_bounds__(256) hessian_combine_routed_kernel(const float *__restrict__ partial,
                                                                     const int64_t *__restrict__ sstart,
                                                                     const int64_t *__restrict__ pstart,
                                                                     const int32_t *__restrict__ heavy, int E,
                                                                     int64_t per_e, float *__restrict__ hess) {
  const int64_t chunks = (per_e + 255) / 256;
  const int64_t h = blockIdx.x / chunks;
  if (h >= heavy[E]) return;
  const int64_t i = (blockIdx.x % chunks) * 256 + threadIdx.x;
  if (i >= per_e) return;
  const int e = heavy[h];
  const int64_t n = sstart[e + 1] - sstart[e];
  const float *p = partial + pstart[e] * per_e + i;
  float s = p[0];
  for (int64_t k = 1; k < n; ++k) s = s + p[k * per_e];
  float *d = hess + static_cast<int64_t>(e) * per_e + i;
  *d = *d + s;
}

// Dense: uniform token splits, enough waves for 256 CUs with at least 256
// tokens each.  Routed: an expert whose list holds more than `target` entries
// is cut into ceil(len / target) splits, target sized for ~2,048 workgroups
// over the launch (256 .. 1,024 entries), so the busiest expert's lists do not
// run as one serial chain; the cut experts' partials stay within 512 MiB.
HessPlan plan_hessian(int64_t T, int64_t K, int top_k, int E, int chunk_rows) {
  HessPlan p{};
  const bool routed = top_k > 0;
  p.nchunks = (T + chunk_rows - 1) / chunk_rows;
  p.W = (chunk_rows + 31) / 32 + 1;
  const int64_t nb = K / 256;
  const int64_t ntiles = static_cast<int64_t>(E) * nb * 10;
  const int64_t per_e = nb * 65536;  // floats of one expert's blocks
  const int64_t hn = static_cast<int64_t>(E) * per_e;
  p.nsplit = 1;
  p.split_len = T;
  if (!routed) {
    if (ntiles < 2048) {
      p.nsplit = (2048 + ntiles - 1) / ntiles;
      const int64_t by_tokens = (T + 255) / 256;
      if (p.nsplit > by_tokens) p.nsplit = by_tokens;
      if (p.nsplit < 1) p.nsplit = 1;
    }
    p.split_len = ((T + p.nsplit - 1) / p.nsplit + kHTok - 1) / kHTok * kHTok;
    if (p.split_len < kHTok) p.split_len = kHTok;
    p.nsplit = (T + p.split_len - 1) / p.split_len;
  } else {
    const int64_t total = T * top_k;
    p.target = (total * nb * 10 + 2047) / 2048;
    p.target = p.target < 256 ? 256 : (p.target > 1024 ? 1024 : p.target);
    p.target = (p.target + kHTok - 1) / kHTok * kHTok;
    auto ceil_div = [](int64_t a, int64_t d) { return (a + d - 1) / d; };
    // partial slots: only cut experts hold them, fewer than 2 total / target
    p.pmax = 2 * ceil_div(total, p.target);
    while (p.pmax > 2 && p.pmax * per_e * static_cast<int64_t>(sizeof(float)) > (int64_t(512) << 20)) {
      p.target *= 2;
      p.pmax = 2 * ceil_div(total, p.target);
    }
    p.smax = E + ceil_div(total, p.target);  // sum over experts of max(1, ceil(len / target))
    p.hmax = ceil_div(total, p.target);      // cut experts: each holds more than target entries
    if (p.hmax > E) p.hmax = E;
  }
  const size_t pbytes = routed ? static_cast<size_t>(p.pmax) * per_e * sizeof(float)
                               : (p.nsplit > 1 ? static_cast<size_t>(p.nsplit) * hn * sizeof(float) : 0);
  const size_t bbytes = routed ? static_cast<size_t>(p.nchunks) * E * p.W * sizeof(uint32_t) : 0;
  const size_t dbytes = routed ? static_cast<size_t>(T) : 0;
  const size_t nbytes = routed ? static_cast<size_t>(4 * E + 3) * sizeof(int64_t) + (E + 1) * sizeof(int32_t) : 0;
  const size_t lbytes = routed ? static_cast<size_t>(T) * top_k * sizeof(uint32_t) : 0;
  p.off_b = ws_up(pbytes);
  p.off_d = p.off_b + ws_up(bbytes);
  p.off_n = p.off_d + ws_up(dbytes);
  p.off_l = p.off_n + ws_up(nbytes);
  p.bytes = p.off_l + ws_up(lbytes) + kWsAlign;
  return p;
}

int launch_hessian(const void *x, int dtype, int64_t T, int64_t K, const int32_t *ids, int top_k, int E,
                   int chunk_rows, float *hess, int32_t *status, void *ws, hipStream_t stream) {
  if (T == 0) return 0;
  const HessPlan P = plan_hessian(T, K, ids ? top_k : 0, E, chunk_rows);
  const int64_t nb = K / 256;
  const int64_t ntiles = static_cast<int64_t>(E) * nb * 10;
  const int64_t per_e = nb * 65536;
  const int64_t hn = static_cast<int64_t>(E) * per_e;
  char *base = ws_base(ws);
  float *partial = reinterpret_cast<float *>(base);
  uint32_t *bm = ids ? reinterpret_cast<uint32_t *>(base + P.off_b) : nullptr;
  uint8_t *dup = ids ? reinterpret_cast<uint8_t *>(base + P.off_d) : nullptr;
  int64_t *lens = ids ? reinterpret_cast<int64_t *>(base + P.off_n) : nullptr;
  int64_t *lstart = ids ? lens + E : nullptr;
  int64_t *sstart = ids ? lstart + (E + 1) : nullptr;
  int64_t *pstart = ids ? sstart + (E + 1) : nullptr;
  int32_t *heavy = ids ? reinterpret_cast<int32_t *>(pstart + (E + 1)) : nullptr;
  uint32_t *list = ids ? reinterpret_cast<uint32_t *>(base + P.off_l) : nullptr;
  if (ids) {
    hipLaunchKernelGGL(collect_route_kernel, dim3(static_cast<unsigned>(P.nchunks * ((chunk_rows + 255) / 256))),
                       dim3(256), 0, stream, ids, T, top_k, E, chunk_rows, P.W, int64_t(0), bm, dup, status);
    if (hipGetLastError() != hipSuccess) return -1;
    hipLaunchKernelGGL(route_count_kernel, dim3(static_cast<unsigned>((E + 3) / 4)), dim3(256), 0, stream,
                       static_cast<const uint32_t *>(bm), P.nchunks, E, P.W, lens);
    if (hipGetLastError() != hipSuccess) return -1;
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, stream, static_cast<const int64_t *>(lens), E,
                       P.target, lstart, sstart, pstart, heavy);
    if (hipGetLastError() != hipSuccess) return -1;
    hipLaunchKernelGGL(route_list_kernel, dim3(static_cast<unsigned>(E)), dim3(256), 0, stream,
                       static_cast<const uint32_t *>(bm), static_cast<const uint8_t *>(dup), P.nchunks, E, P.W,
                       chunk_rows, static_cast<const int64_t *>(lstart), list);
    if (hipGetLastError() != hipSuccess) return -1;
  }
  const dim3 g(static_cast<unsigned>(ids ? P.smax * nb * 10 : ntiles * P.nsplit));
  if (dtype == 1)
    hipLaunchKernelGGL(hessian_kernel<1>, g, dim3(64), 0, stream, x, T, K, ids, top_k, E,
                       static_cast<const uint32_t *>(list), static_cast<const int64_t *>(lstart),
                       static_cast<const int64_t *>(sstart), static_cast<const int64_t *>(pstart), P.nsplit,
                       P.split_len, hess, partial, status);
  else
    hipLaunchKernelGGL(hessian_kernel<0>, g, dim3(64), 0, stream, x, T, K, ids, top_k, E,
                       static_cast<const uint32_t *>(list), static_cast<const int64_t *>(lstart),
                       static_cast<const int64_t *>(sstart), static_cast<const int64_t *>(pstart), P.nsplit,
                       P.split_len, hess, partial, status);
  if (hipGetLastError() != hipSuccess) return -1;
  if (ids)
    hipLaunchKernelGGL(hessian_combine_routed_kernel, dim3(static_cast<unsigned>(P.hmax * ((per_e + 255) / 256))),
                       dim3(256), 0, stream, static_cast<const float *>(partial),
                       static_cast<const int64_t *>(sstart), static_cast<const int64_t *>(pstart),
                       static_cast<const int32_t *>(heavy), E, per_e, hess);
  else if (P.nsplit > 1)
    hipLaunchKernelGGL(hessian_combine_kernel, dim3(static_cast<unsigned>((hn + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const float *>(partial), P.nsplit, hn, hess);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace iq
