// iq_encode.hip -- importance-weighted GGML IQ encoder and decoder for gfx950.
//
// What is computed (pages cited by title and section):
//  * ModelOpt PR #2513, commit messages: every 256-value block gets a fixed
//    anchored fp16 super-block scale d, then a single-pass search of the grid;
//    IQ2_XXS / IQ2_XS use an even-parity 7-bit sign index and flip the weakest
//    element to fix parity; IQ2_S keeps the input signs and compares
//    magnitudes; IQ1 values carry a +-1/8 delta, IQ1_S per 32 values, IQ1_M per
//    group with ties going to the lower shift, then the lower entry; IQ1_M's
//    anchor ratio is clamp(0.58 + 0.035 * peak_to_rms, 0.65, 0.95), IQ1_S's 0.61.
//  * ModelOpt PR "[1/5] Let the GGML IQ encoders take fixed per-group choices":
//    each choice unit takes the local scale (IQ1_S: and delta sign) with the
//    least importance-weighted squared error; given choices, only the entry
//    search runs; an all-zero block gives an all-zero payload.
//  * "Add imatrix calibration for the GGML formats ...", description: the
//    search weight of column j is a_j = sqrt(E[x_j^2]).
//
// Arithmetic.  For a group of 8 values x_j with weights a_j, entry g_k and
// local scale s, the weighted error is sum a_j (y_j - s u_j)^2 =
// sum a_j y_j^2 + s (s G - 2 P) with G = sum a_j u_j^2, P = sum a_j y_j u_j.
// The search ranks t = fmaf(s, G, -2P) (fp32, contraction off, explicit fmaf);
// per (group, slot) it keeps the first minimum over entries, each choice unit
// takes the choice with the least sum over its groups of s * t_min (left to
// right, lowest choice on ties).
//  IQ2: y = |x|, u = g; -2P is the fmaf chain of (-2 a_j y_j) * g_kj; with an odd
//       number of negative inputs (IQ2_XXS/XS) the cheapest single flip
//       F = min_j a_j y_j g_kj is charged: -2P' = fmaf(4, F, -2P).
//  IQ1: y = x, u = g + delta (delta = +1/8 for shift 0, -1/8 for shift 1);
//       -2P = fmaf(delta, S, Q) with Q the fmaf chain of (-2 a_j x_j) g_kj and
//       S = sum (-2 a_j x_j), i.e. per-entry grid terms plus one shift term.
//
// gfx950 design.  One wave per 8-value group and 64 rows per wave: the grid
// entry and the weighted norm G_k are then the same for all 64 lanes, so they
// arrive as scalar loads and cost no LDS bandwidth; G_k is precomputed once per
// (expert, column group) by the preparation kernel and copied to a VGPR per
// entry so the candidate FMAs can co-issue across waves.  (IQ2_XXS/XS waves
// take 64 (group, row) items dealt by sign parity instead, and read the norms
// from an LDS copy of the workgroup's tables.)  The sweep keeps, per
// slot, a running minimum per chunk of CH entries (v_min3 pairs; CH = 32, 16
// for IQ2_XXS, 8 in the every-choice sweeps) and the index of the chunk
// holding the first minimum; after the unit's choice is known the chosen chunk
// is rescanned to recover the exact entry.  A workgroup holds the groups whose
// payload bytes nobody else writes (one 32-value sub-block; IQ1_M: 64 values),
// exchanges per-slot minima through LDS to score its choice units, and packs
// its bytes itself.  The file ends with the local-Hessian choice search and
// its damping pass.

#include "iq_common.hpp"
#include "iq_internal.hpp"

namespace iq {

// ---------------------------------------------------------------------------
// Workgroup order: the hardware deals consecutive workgroups round robin to the
// 8 XCDs.  Remap so each XCD gets a contiguous range of logical work (the same
// column groups over all their row tiles), which keeps each column group's
// weighted-norm table in one XCD's L2.  The search kernel orders that range
// sub-block fastest, so the workgroups that share a block's payload lines run
// together and their partial writes merge in L2.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t xcd_remap(int64_t i, int64_t total) {
  const int64_t q = total >> 3, r = total & 7;
  const int64_t x = i & 7, j = i >> 3;
  return x * q + (x < r ? x : r) + j;
}

// ---------------------------------------------------------------------------
// Importance check: one wave per (expert, block), 4 values per lane;
// flags[e * nb + b] = 1 when the block's 256 importance values hold a value
// outside [0, 2^64]: NaN, negative, or above any floored square root of a
// finite fp32 second moment (sqrt(FLT_MAX) < 2^64).  Within that range, and
// with a finite fp16 block scale, every fp32 intermediate of the search stays
// finite (the largest, a unit score, is below 1e34).
// ---------------------------------------------------------------------------
constexpr float kImpMax = 18446744073709551616.0f;  // 2^64

__device__ __forceinline__ bool imp_ok(float a) { return a >= 0.0f && a <= kImpMax; }

__device__ __forceinline__ void impcheck_block(int64_t blk, const float *__restrict__ imp, int64_t n,
                                               uint8_t *__restrict__ flags) {
  const int64_t i = blk * 4 + (threadIdx.x >> 6);  // (e * nb + b)
  const int lane = threadIdx.x & 63;
  if (i >= n) return;
  const float4 q = reinterpret_cast<const float4 *>(imp + i * 256)[lane];  // cols = nb * 256
  const bool ok = imp_ok(q.x) && imp_ok(q.y) && imp_ok(q.z) && imp_ok(q.w);
  const uint64_t bad = __ballot(!ok);
  if (lane == 0) flags[i] = bad ? 1 : 0;
}

// ---------------------------------------------------------------------------
// Anchor: 32 lanes per block, 8 contiguous values per lane (coalesced), two
// blocks per wave.  amax and finiteness reduce across the 32 lanes (exact); the
// IQ1_M sum of squares is the sequential chain over j = 0..255, run by one lane
// from an LDS copy of the block.  Writes the fp16 scale bits (0 = all-zero
// block) to dscr and, for layouts with a leading d field, to the payload.
// ---------------------------------------------------------------------------
template <int F>
__global__ void __launch_bounds__(256) anchor_kernel(EncArgs A, const uint8_t *__restrict__ impflags) {
  using G = Geo<F>;
  __shared__ float s_blk[F == IQ1_M ? 8 : 1][F == IQ1_M ? 256 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, sl = lane & 31;
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * 2 + half;
  const bool live = i < A.rows * A.nb;
  const int64_t ii = live ? i : 0;
  const int64_t r = ii / A.nb;
  const int b = static_cast<int>(ii % A.nb);
  const int64_t e = r / A.rpe;
  float v[8];
  load8(A.w, A.dtype, r * A.cols + static_cast<int64_t>(b) * 256 + sl * 8, v);
  float amax = 0.0f;
  int finite = 1;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    finite &= finite_f(v[j]) ? 1 : 0;
    amax = fmaxf(amax, fabsf(v[j]));
  }
  int chok = 1;
  if (A.choices && sl < G::UNITS) chok = A.choices[ii * G::UNITS + sl] < G::NC;
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) {
    amax = fmaxf(amax, __shfl_xor(amax, o));
    finite &= __shfl_xor(finite, o);
    chok &= __shfl_xor(chok, o);
  }
  float ss = 0.0f;
  if (F == IQ1_M) {
    const int q = wave * 2 + half;
#pragma unroll
    for (int j = 0; j < 8; ++j) s_blk[q][sl * 8 + j] = v[j];
    __syncthreads();
    if (sl == 0 && finite)
      for (int j = 0; j < 256; ++j) ss = __builtin_fmaf(s_blk[q][j], s_blk[q][j], ss);
  }
  if (!live || sl != 0) return;
  int st = 0;
  uint16_t h = 0;
  if (!finite) {
    st |= ST_NONFINITE;
  } else if (amax > 0.0f) {
    float ratio = 1.0f;                 // IQ2: no ratio is printed on the pages; 1
    if (F == IQ1_S) ratio = 0.61f;
    if (F == IQ1_M) {                   // peak-to-RMS over the 256-value block
      const float rms = sqrtf(ss * (1.0f / 256.0f));
      const float p = amax / rms;
      ratio = fminf(fmaxf(__builtin_fmaf(0.035f, p, 0.58f), 0.65f), 0.95f);
    }
    const float qmax = G::IQ1 ? 15.0f : 19.375f;  // top multiplier * top magnitude
    const float d = (ratio * amax) / qmax;
    h = f32_to_f16_bits(d);
    if ((h & 0x7c00u) == 0x7c00u) {
      st |= ST_OVERFLOW;
      h = 0;
    } else if ((h & 0x7fffu) == 0) {
      h = 0;
    }
  }
  if (impflags && impflags[e * A.nb + b]) { st |= ST_BADIMP; h = 0; }
  if (!chok) { st |= ST_BADCHOICE; h = 0; }
  A.dscr[ii] = h;
  if (F != IQ1_M)
    for (int64_t c = 0; c < A.copies; ++c) *reinterpret_cast<uint16_t *>(A.out + c * A.copy_stride + ii * G::BYTES) = h;
  raise_status(A.status, st);
}

// ---------------------------------------------------------------------------
// Weighted norms of every grid entry for one (expert, column group):
// IQ2: G_k = sum_j a_j g_kj^2;  IQ1: G^h_k = sum_j a_j (g_kj + delta_h)^2.
// Thread per (table, entry).  Flat weights use a single table (a_j = 1).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load_entry(const float *p, float g[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 4);
  g[0] = a.x; g[1] = a.y; g[2] = a.z; g[3] = a.w;
  g[4] = b.x; g[5] = b.y; g[6] = b.z; g[7] = b.w;
}

// IQ2 weighted norm of one entry: the fmaf chain over j = 0..7 (the table pass
// and the in-lane rescans evaluate it this way, so they hold the same value)
__device__ __forceinline__ float iq2_norm(const float a[8], const float g[8]) {
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s = __builtin_fmaf(a[j], g[j] * g[j], s);
  return s;
}

template <int F>
__device__ __forceinline__ void gterm_block(int64_t blk, const float *__restrict__ grid,
                                            const float *__restrict__ imp, int64_t ntab, float *__restrict__ gtab) {
  using G = Geo<F>;
  const int64_t i = blk * 256 + threadIdx.x;
  if (i >= ntab * G::N) return;
  const int k = static_cast<int>(i % G::N);
  // N is a multiple of the block size, so a block lies in one table: the
  // importance values are wave-uniform
  static_assert(G::N % 256 == 0, "a 256-thread block covers entries of one table");
  const int64_t tab = blk * 256 / G::N;  // = e * (cols / 8) + cg
  float a[8], g[8];
  load_entry(grid + static_cast<int64_t>(k) * 8, g);
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = imp ? imp[tab * 8 + j] : 1.0f;  // importance row e, columns 8cg..8cg+7
  if (!G::IQ1) {
    gtab[tab * G::N + k] = iq2_norm(a, g);
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float delta = h ? -0.125f : 0.125f;
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float u = g[j] + delta;
        s = __builtin_fmaf(a[j], u * u, s);
      }
      gtab[(tab * 2 + h) * G::N + k] = s;
    }
  }
}

// One launch for the two preparation passes: blocks [0, gblocks) build the
// weighted-norm tables, the rest check the importance blocks.
template <int F>
__global__ void __launch_bounds__(256) prep_kernel(const float *__restrict__ grid, const float *__restrict__ imp,
                                                   int64_t ntab, float *__restrict__ gtab, int64_t gblocks,
                                                   int64_t nflags, uint8_t *__restrict__ flags) {
  const int64_t blk = blockIdx.x;
  if (blk < gblocks) gterm_block<F>(blk, grid, imp, ntab, gtab);
  else impcheck_block(blk - gblocks, imp, nflags, flags);
}

// ---------------------------------------------------------------------------
// Per-lane group state and the per-entry reduced errors.
// ---------------------------------------------------------------------------
template <int F>
struct GroupState {
  float ax[8];   // IQ2: a_j |x_j|
  float nax[8];  // IQ2: -2 a_j |x_j| ; IQ1: -2 a_j x_j
  float f4;      // IQ2 parity: 4 for an odd count of negative inputs, else 0
  float S2;      // IQ1: sum_j -2 a_j x_j
  uint32_t neg;  // IQ2: negative mask
  bool odd;

  __device__ __forceinline__ void init(const float x[8], const float a[8]) {
    neg = 0;
    S2 = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (!Geo<F>::IQ1) {
        const float v = fabsf(x[j]);
        neg |= (x[j] < 0.0f ? 1u : 0u) << j;
        ax[j] = a[j] * v;
        nax[j] = -2.0f * ax[j];
      } else {
        ax[j] = 0.0f;
        nax[j] = -2.0f * (a[j] * x[j]);
        S2 = S2 + nax[j];
      }
    }
    odd = Geo<F>::PARITY && (__builtin_popcount(neg) & 1);
    f4 = odd ? 4.0f : 0.0f;
  }

  // IQ2: -2 P'_k for grid entry g;  IQ1: Q_k (before the shift term).  PAR
  // false drops the parity term, which is exact for an even-parity group
  // (f4 = 0: the term adds +0 to a sum that is never -0)
  template <bool PAR = Geo<F>::PARITY>
  __device__ __forceinline__ float term(const float g[8]) const {
    float p = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) p = __builtin_fmaf(nax[j], g[j], p);
    if (PAR) {
      float fm = ax[0] * g[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) fm = fminf(fm, ax[j] * g[j]);
      p = __builtin_fmaf(f4, fm, p);
    }
    return p;
  }

  // element flipped to fix parity for entry g: the first j with least a_j |x_j| g_j
  __device__ __forceinline__ int flip_index(const float g[8]) const {
    int jm = 0;
    float fm = ax[0] * g[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
      const float f = ax[j] * g[j];
      if (f < fm) { fm = f; jm = j; }
    }
    return jm;
  }
};

// Copy a wave-uniform (SGPR) value into a VGPR.  On gfx950 a VALU op that
// reads an SGPR cannot be co-issued with another wave's VALU op, while all-VGPR
// fp32 FMA/MUL/ADD ops can; the 16 candidate FMAs per grid entry read the
// weighted norm, so one copy per entry lets them all co-issue.
__device__ __forceinline__ float to_vgpr(float s) {
  float v;
  asm("v_mov_b32 %0, %1" : "=v"(v) : "s"(s));
  return v;
}


// ---------------------------------------------------------------------------
// Rescan one CH-entry chunk under one (scale, shift) slot: the first entry with
// the least reduced error -- the same fp32 values the sweep compared -- and
// its sign mask (IQ2) or shift bit (IQ1).  par = false (a wave whose groups
// all have even parity) drops the parity term as that wave's sweep did.
// ---------------------------------------------------------------------------
template <int F, int CH>
__device__ __forceinline__ void rescan_chunk(const float *__restrict__ grid, const float *gt, const GroupState<F> &S,
                                             int chs, float ssel, int hsel, bool par, int &kb, uint32_t &mfield) {
  using G = Geo<F>;
  constexpr int N = G::N;
  const float dsel = hsel ? -0.125f : 0.125f;
  float bt = __builtin_inff();
  kb = chs * CH;
  auto scan = [&](auto pc) {
    constexpr bool PAR = decltype(pc)::value;
    for (int i = 0; i < CH; ++i) {
      const int k = chs * CH + i;
      float g[8];
      load_entry(grid + static_cast<int64_t>(k) * 8, g);
      const float q2 = S.template term<PAR>(g);
      float t;
      if (!G::IQ1) {
        t = __builtin_fmaf(ssel, gt[k], q2);
      } else {
        const float pn = __builtin_fmaf(dsel, S.S2, q2);
        t = __builtin_fmaf(ssel, gt[hsel * N + k], pn);
      }
      if (t < bt) { bt = t; kb = k; }
    }
  };
  if (G::PARITY && par) scan(std::integral_constant<bool, G::PARITY>{});
  else scan(std::integral_constant<bool, false>{});
  if (!G::IQ1) {
    uint32_t mask = S.neg;
    if (S.odd) {
      float g[8];
      load_entry(grid + static_cast<int64_t>(kb) * 8, g);
      mask ^= 1u << S.flip_index(g);
    }
    mfield = mask;
  } else {
    mfield = static_cast<uint32_t>(hsel);
  }
}

// IQ2 layouts rescan from a copy of the grid in LDS: chunk c's entry i sits at
// float (CH c + i) * 8 + 4 c, so lanes rescanning different chunks read
// different banks.  The weighted norm G_k is recomputed in the lane with the
// same fmaf chain that built the table the sweep read, so it is the same value.
template <int CH>
__device__ __forceinline__ int lds_entry(int k) { return k * 8 + (k / CH) * 4; }

template <int F, int CH, bool TAB>
__device__ __forceinline__ void rescan_chunk_lds(const float *s_grid, const float *gnorm, const float a[8],
                                                 const GroupState<F> &S, int chs, float ssel, bool par, int &kb,
                                                 uint32_t &mfield) {
  float bt = __builtin_inff();
  kb = chs * CH;
  const float *base = s_grid + lds_entry<CH>(chs * CH);
  auto scan = [&](auto pc) {
    constexpr bool PAR = decltype(pc)::value;
#pragma unroll 4
    for (int i = 0; i < CH; ++i) {
      float g[8];
      load_entry(base + i * 8, g);
      // the weighted norm: the workgroup's LDS table (TAB), else the same fmaf
      // chain in the lane
      const float gk = TAB ? gnorm[chs * CH + i] : iq2_norm(a, g);
      const float t = __builtin_fmaf(ssel, gk, S.template term<PAR>(g));
      if (t < bt) { bt = t; kb = chs * CH + i; }
    }
  };
  if (Geo<F>::PARITY && par) scan(std::integral_constant<bool, Geo<F>::PARITY>{});
  else scan(std::integral_constant<bool, false>{});
  uint32_t mask = S.neg;
  if (S.odd) {
    float g[8];
    load_entry(s_grid + lds_entry<CH>(kb), g);
    mask ^= 1u << S.flip_index(g);
  }
  mfield = mask;
}

// One group's fields in a packed block: grid index k, sign mask (IQ2), local
// scale ls, delta sign h (IQ1), and the block's fp16 scale bits d16.
struct GroupFields {
  uint32_t d16, k, mask, ls, h;
};

// A group's fields as one word: k | mask << 11 | ls << 19 | h << 23.
__device__ __forceinline__ uint32_t pack_record(const GroupFields &f) {
  return f.k | (f.mask << 11) | (f.ls << 19) | (f.h << 23);
}

// ---------------------------------------------------------------------------
// Pack one packed unit's bytes of one row's block from the LDS field tables:
// k[g][row], m[g][row] (IQ2 sign mask / IQ1 shift), c[u][row] (unit choice),
// the unit's PG groups first.  Packed unit sb is: IQ2_XXS/XS/S, IQ1_S the
// 32-value sub-block sb; IQ1_M the 64 values of scale word sb.
// ---------------------------------------------------------------------------
template <int F>
__device__ __forceinline__ void pack_bytes(uint8_t *blk, int sb, int lane, const uint16_t (*s_k)[64],
                                           const uint8_t (*s_m)[64], const uint8_t (*s_c)[64], uint32_t d16) {
  if (F == IQ2_XXS) {  // 4 index bytes, then (4 x 7-bit sign index | scale << 28)
    uint8_t *p = blk + 2 + 8 * sb;
    uint32_t word = static_cast<uint32_t>(s_c[0][lane]) << 28;
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      p[l] = static_cast<uint8_t>(s_k[l][lane]);
      word |= (static_cast<uint32_t>(s_m[l][lane]) & 0x7fu) << (7 * l);
    }
    reinterpret_cast<uint16_t *>(p + 4)[0] = static_cast<uint16_t>(word);
    reinterpret_cast<uint16_t *>(p + 4)[1] = static_cast<uint16_t>(word >> 16);
  } else if (F == IQ2_XS) {  // 4 x (9-bit index | 7-bit sign index << 9), scale byte
#pragma unroll
    for (int l = 0; l < 4; ++l)
      reinterpret_cast<uint16_t *>(blk + 2 + 2 * (4 * sb + l))[0] =
          static_cast<uint16_t>(s_k[l][lane] | ((s_m[l][lane] & 0x7fu) << 9));
    blk[66 + sb] = static_cast<uint8_t>(s_c[0][lane] | (s_c[1][lane] << 4));
  } else if (F == IQ2_S) {  // low index bytes, sign masks, high index bits, scale byte
    uint32_t hi = 0;
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      blk[2 + 4 * sb + l] = static_cast<uint8_t>(s_k[l][lane] & 0xff);
      blk[34 + 4 * sb + l] = s_m[l][lane];
      hi |= ((s_k[l][lane] >> 8) & 3u) << (2 * l);
    }
    blk[66 + sb] = static_cast<uint8_t>(hi);
    blk[74 + sb] = static_cast<uint8_t>(s_c[0][lane] | (s_c[1][lane] << 4));
  } else if (F == IQ1_S) {  // low index bytes, (4 x 3 high bits | scale << 12 | shift << 15)
    const uint32_t c = s_c[0][lane];
    uint32_t w = ((c & 7u) << 12) | ((c >> 3) << 15);
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      blk[2 + 4 * sb + l] = static_cast<uint8_t>(s_k[l][lane] & 0xff);
      w |= ((s_k[l][lane] >> 8) & 7u) << (3 * l);
    }
    reinterpret_cast<uint16_t *>(blk + 34 + 2 * sb)[0] = static_cast<uint16_t>(w);
  } else {  // IQ1_M, 8 groups: low index bytes, qh nibbles, scale word with d nibble sb
#pragma unroll
    for (int l = 0; l < 8; ++l) blk[8 * sb + l] = static_cast<uint8_t>(s_k[l][lane] & 0xff);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const uint32_t lo = ((s_k[2 * qq][lane] >> 8) & 7u) | (static_cast<uint32_t>(s_m[2 * qq][lane]) << 3);
      const uint32_t hi = ((s_k[2 * qq + 1][lane] >> 8) & 7u) | (static_cast<uint32_t>(s_m[2 * qq + 1][lane]) << 3);
      blk[32 + 4 * sb + qq] = static_cast<uint8_t>(lo | (hi << 4));
    }
    uint32_t w = ((d16 >> (4 * sb)) & 0xfu) << 12;
#pragma unroll
    for (int u = 0; u < 4; ++u) w |= (s_c[u][lane] & 7u) << (3 * u);
    reinterpret_cast<uint16_t *>(blk + 48 + 2 * sb)[0] = static_cast<uint16_t>(w);
  }
}

// Copy the grid into LDS in the rescan layout (whole workgroup; ends with a barrier).
template <int N, int CH>
__device__ __forceinline__ void stage_grid(const float *__restrict__ grid, float *s_grid) {
  for (int i = threadIdx.x; i < N * 2; i += blockDim.x) {
    const int k = i >> 1;
    *reinterpret_cast<float4 *>(s_grid + lds_entry<CH>(k) + (i & 1) * 4) = reinterpret_cast<const float4 *>(grid)[i];
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Search + pack.  Workgroup = WGG waves (groups) x 64 rows of one expert.
// ---------------------------------------------------------------------------
// MODE: SEARCH scores every choice per unit; FIXED takes the caller's choices;
// EVERY writes one payload per choice (out[c] == the FIXED payload with every
// unit set to c) from a single sweep; RECORDS writes the same groups' fields
// as one word per (choice, group, row) for the choice search.
enum Mode : int { SEARCH = 0, FIXED_CHOICES = 1, EVERY = 2, RECORDS = 3 };

// Waves per SIMD the compiler must fit (each measured): the IQ1 searches run
// six (IQ1_M's eight-wave workgroups fit three to a CU instead of two, at the
// cost of three spilled registers; IQ1_S spills two), IQ2_S five (six spills
// sixteen registers and runs slower), the others keep their register budget.
template <int F, int MODE>
constexpr int search_min_waves() {
  constexpr bool SF = MODE == SEARCH || MODE == FIXED_CHOICES;
  return SF && (F == IQ1_M || F == IQ1_S)              ? 6
         : SF && F == IQ2_S                            ? 5
         : F == IQ2_XXS || F == IQ2_XS || F == IQ1_M ? 4
                                                       : 1;
}

template <int F, int MODE>
__global__ void __launch_bounds__(64 * Geo<F>::WGG, (search_min_waves<F, MODE>())) search_kernel(EncArgs A) {
  using G = Geo<F>;
  constexpr bool FIXED = MODE == FIXED_CHOICES;
  constexpr int WGG = G::WGG, GPU = G::GPU, N = G::N;
  // chunk of the first-minimum tracking: the every-choice sweeps rescan 16
  // times per lane, so they keep shorter chunks (more bookkeeping, shorter rescans)
  // (IQ1_M takes 16: with 8 its every-choice sweep needs more registers than
  // four waves per SIMD allow; IQ2_S takes 16 too: its parity-free 1,024-entry
  // sweep spends more on the per-chunk bookkeeping than the longer rescans
  // cost); the 256-entry IQ2_XXS sweep, whose one rescan weighs more against
  // its short sweep, takes 16, as do the IQ2_XS search (measured ~1% faster
  // than with 32) and the fixed-choice sweeps of IQ2_S and IQ1_M, which track
  // one slot (two shifts) and so gain less from long chunks
  constexpr bool EV = MODE == EVERY || MODE == RECORDS;
  constexpr int CH = EV ? (F == IQ1_M || F == IQ2_S ? 16 : 8)
                        : (F == IQ2_XXS || (!FIXED && F == IQ2_XS) || (FIXED && (F == IQ2_S || F == IQ1_M)) ? 16
                                                                                                           : 32),
                NCH = N / CH;
  constexpr int UPW = WGG / GPU;                 // choice units per workgroup
  constexpr int SBS = 32 / WGG;                  // workgroups per block column
  // slots swept per lane: IQ2 16 choices; IQ1 8 scales x 2 shifts;
  // fixed choices: one slot (IQ1_M: its two shifts)
  constexpr int NSLOT = FIXED ? (F == IQ1_M ? 2 : 1) : 16;

  // s_u: the per-slot minima exchanged for scoring (search), or, for the IQ2
  // layouts' every-choice sweeps (16 rescans per lane), the grid copy the
  // rescans read
  constexpr bool LDS_RESCAN = !G::IQ1 && (MODE == EVERY || MODE == RECORDS);
  constexpr int BEST_F = MODE == SEARCH ? WGG * NSLOT * 64 : 1;
  constexpr int GRID_F = LDS_RESCAN ? N * 8 + (N / CH) * 4 : 1;
  __shared__ __attribute__((aligned(16))) float s_u[BEST_F > GRID_F ? BEST_F : GRID_F];
  float (*s_best)[NSLOT][64] = reinterpret_cast<float (*)[NSLOT][64]>(s_u);
  __shared__ uint16_t s_k[WGG][64];
  __shared__ uint8_t s_m[WGG][64];
  __shared__ uint8_t s_c[UPW][64];
  // Parity-sorted items (IQ2_XXS/XS, every mode): the workgroup's WGG x 64
  // (group, row) items are dealt to the waves odd-parity first, so of the
  // eight waves about three hold only even-parity groups and sweep without the
  // parity term (and at most one mixes both).  A wave then mixes groups, so the weighted norms come from an LDS
  // copy of the workgroup's tables instead of scalar loads (the every-choice
  // rescans read the same copy), and the LDS field tables are indexed by each
  // item's group and row.
  constexpr bool SORTED = G::PARITY;
  __shared__ uint16_t s_items[SORTED ? WGG * 64 : 1];
  __shared__ int s_nodd[SORTED ? WGG : 1];
  // row stride N + 2: the (up to WGG) groups a wave reads per entry pair sit in
  // different banks
  __shared__ __attribute__((aligned(8))) float s_g[SORTED ? WGG : 1][SORTED ? N + 2 : 1];

  const int64_t L = xcd_remap(blockIdx.x, A.total_wg);
  const int sb = static_cast<int>(L % SBS);
  const int64_t Lt = L / SBS;
  const int64_t tile = Lt % A.tiles_per_e;
  const int64_t q = Lt / A.tiles_per_e;
  const int b = static_cast<int>(q % A.nb);
  const int64_t e = q / A.nb;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // this thread's item: group gw of the workgroup, row rl of the tile
  int gw = wave, rl = lane;
  bool all_even = false;  // wave-uniform
  if (SORTED) {
    const int64_t rn = e * A.rpe + (tile * 64 + lane < A.rpe ? tile * 64 + lane : A.rpe - 1);  // lane = row
    float xn[8];
    load8(A.w, A.dtype, rn * A.cols + (static_cast<int64_t>(b) * 32 + sb * WGG + wave) * 8, xn);
    uint32_t neg = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) neg |= (xn[j] < 0.0f ? 1u : 0u) << j;
    const bool odd = __builtin_popcount(neg) & 1;
    const uint64_t bal = __ballot(odd);
    if (lane == 0) s_nodd[wave] = __builtin_popcountll(bal);
    for (int i = threadIdx.x; i < WGG * N; i += 64 * WGG) {
      const int64_t cgw = static_cast<int64_t>(b) * 32 + sb * WGG + i / N;
      s_g[i / N][i % N] = A.gtab[e * A.gtab_e_stride + cgw * A.gtab_cg_stride + i % N];
    }
    __syncthreads();
    int n_odd = 0, before = 0;
#pragma unroll
    for (int w = 0; w < WGG; ++w) {
      n_odd += s_nodd[w];
      before += w < wave ? s_nodd[w] : 0;
    }
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    const int pos = odd ? before + __builtin_popcountll(bal & below)
                        : n_odd + (wave * 64 - before) + __builtin_popcountll(~bal & below);
    s_items[pos] = static_cast<uint16_t>((wave << 6) | lane);
    __syncthreads();
    const int it = s_items[wave * 64 + lane];
    gw = it >> 6;
    rl = it & 63;
    all_even = wave * 64 >= __builtin_amdgcn_readfirstlane(n_odd);
  }
  const int64_t rin = tile * 64 + rl;
  const bool valid = rin < A.rpe;
  const int64_t r = e * A.rpe + (valid ? rin : A.rpe - 1);
  const int gi = sb * WGG + gw;                    // group within the block
  const int64_t cg = static_cast<int64_t>(b) * 32 + gi;
  const int uw = gw / GPU;                         // unit within the workgroup
  const int unit = gi / GPU;                       // unit within the block

  const uint16_t d16 = A.dscr[r * A.nb + b];
  const bool zero_blk = d16 == 0;
  const float d = f16_bits_to_f32(d16);

  float x[8], a[8];
  load8(A.w, A.dtype, r * A.cols + cg * 8, x);
  if (A.imp) {
    const float *ap = A.imp + e * A.cols + cg * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = ap[j];
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = 1.0f;
  }
  GroupState<F> S;
  S.init(x, a);
  const float *gt = A.gtab + e * A.gtab_e_stride + cg * A.gtab_cg_stride;  // [NG][N]

  // ---- slot scales -------------------------------------------------------
  float sc[G::IQ1 ? 8 : 16];
  int fixed_c = 0;
  if (FIXED) {
    int c = A.choices[(r * A.nb + b) * G::UNITS + unit];
    fixed_c = c < G::NC ? c : G::NC - 1;  // out-of-range choices only occur in zeroed blocks
  }
  if (!G::IQ1) {
#pragma unroll
    for (int c = 0; c < 16; ++c) sc[c] = d * (static_cast<float>(2 * c + 1) * 0.125f);
  } else {
#pragma unroll
    for (int l = 0; l < 8; ++l) sc[l] = d * static_cast<float>(2 * l + 1);
  }
  // per-lane fixed slot parameters
  float fs = 0.0f;        // fixed: local scale
  int fh = 0;             // fixed IQ1_S: shift
  if (FIXED) {
    if (!G::IQ1) fs = d * (static_cast<float>(2 * fixed_c + 1) * 0.125f);
    else fs = d * static_cast<float>(2 * (fixed_c & 7) + 1);
    fh = (F == IQ1_S) ? (fixed_c >> 3) : 0;
  }
  const float fdelta = fh ? -0.125f : 0.125f;

  // ---- sweep -------------------------------------------------------------
  float best[NSLOT];
  int bidx[NSLOT];
#pragma unroll
  for (int s = 0; s < NSLOT; ++s) { best[s] = __builtin_inff(); bidx[s] = 0; }

  auto sweep = [&](auto par) {
  constexpr bool PAR = decltype(par)::value;
  for (int ch = 0; ch < NCH; ++ch) {
    float cm[NSLOT];
#pragma unroll
    for (int s = 0; s < NSLOT; ++s) cm[s] = __builtin_inff();
#pragma unroll
    for (int i = 0; i < CH; i += 2) {
      const int k = ch * CH + i;
      float t0[NSLOT], t1[NSLOT];
      float2 gk2 = make_float2(0.0f, 0.0f);
      if (SORTED) gk2 = *reinterpret_cast<const float2 *>(&s_g[gw][k]);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        float *t = p ? t1 : t0;
        const float *gp = A.grid + static_cast<int64_t>(k + p) * 8;
        float g[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) g[j] = gp[j];
        const float q2 = S.template term<PAR>(g);
        if (!G::IQ1) {
          const float Gk = SORTED ? (p ? gk2.y : gk2.x) : to_vgpr(gt[k + p]);
          if (FIXED) {
            t[0] = __builtin_fmaf(fs, Gk, q2);
          } else {
#pragma unroll
            for (int c = 0; c < 16; ++c) t[c] = __builtin_fmaf(sc[c], Gk, q2);
          }
        } else {
          const float G0 = to_vgpr(gt[k + p]), G1 = to_vgpr(gt[N + k + p]);
          const float p0 = __builtin_fmaf(0.125f, S.S2, q2);
          const float p1 = __builtin_fmaf(-0.125f, S.S2, q2);
          if (FIXED) {
            if (F == IQ1_M) {
              t[0] = __builtin_fmaf(fs, G0, p0);
              t[1] = __builtin_fmaf(fs, G1, p1);
            } else {
              const float pf = __builtin_fmaf(fdelta, S.S2, q2);
              t[0] = __builtin_fmaf(fs, fh ? G1 : G0, pf);
            }
          } else {
#pragma unroll
            for (int l = 0; l < 8; ++l) {
              t[l] = __builtin_fmaf(sc[l], G0, p0);
              t[8 + l] = __builtin_fmaf(sc[l], G1, p1);
            }
          }
        }
      }
#pragma unroll
      for (int s = 0; s < NSLOT; ++s) cm[s] = fminf(fminf(cm[s], t0[s]), t1[s]);
    }
#pragma unroll
    for (int s = 0; s < NSLOT; ++s) {
      const bool upd = cm[s] < best[s];
      best[s] = upd ? cm[s] : best[s];
      bidx[s] = upd ? ch : bidx[s];
    }
  }
  };
  if constexpr (SORTED) {
    if (all_even) sweep(std::integral_constant<bool, false>{});
    else sweep(std::integral_constant<bool, true>{});
  } else {
    sweep(std::integral_constant<bool, G::PARITY>{});
  }

  // ---- every choice: one field record per choice and group ----------------
  if (LDS_RESCAN) stage_grid<N, CH>(A.grid, s_u);
  if (MODE == RECORDS) {
    uint32_t *rp = A.rec + (static_cast<int64_t>(b) * 32 + gi) * A.rows + r;
    const int64_t cstride = static_cast<int64_t>(A.nb) * 32 * A.rows;
#pragma unroll
    for (int c = 0; c < G::NC; ++c) {
      int slot = c;
      if (F == IQ1_M) slot = (best[8 + c] < best[c]) ? 8 + c : c;  // tie: the lower shift
      int chs = bidx[c];
      if (F == IQ1_M) chs = (slot != c) ? bidx[8 + c] : chs;
      const float ssel = G::IQ1 ? sc[c & 7] : sc[c];
      int kb;
      uint32_t mfield;
      if (LDS_RESCAN) rescan_chunk_lds<F, CH, SORTED>(s_u, SORTED ? &s_g[gw][0] : s_u, a, S, chs, ssel, !all_even, kb, mfield);
      else rescan_chunk<F, CH>(A.grid, gt, S, chs, ssel, G::IQ1 ? (slot >> 3) : 0, !all_even, kb, mfield);
      GroupFields f;
      f.d16 = d16;
      f.k = static_cast<uint32_t>(kb);
      f.mask = G::IQ1 ? 0u : mfield;
      f.ls = static_cast<uint32_t>(F == IQ1_S ? (c & 7) : c);
      f.h = F == IQ1_S ? static_cast<uint32_t>(c >> 3) : (F == IQ1_M ? mfield : 0u);
      if (d16 == 0) { f.k = 0; f.mask = 0; f.ls = 0; f.h = 0; }
      if (valid) rp[c * cstride] = pack_record(f);
    }
    return;
  }

  // ---- every choice: one payload per choice --------------------------------
  if (MODE == EVERY) {
#pragma unroll
    for (int c = 0; c < G::NC; ++c) {
      int slot = c;
      if (F == IQ1_M) slot = (best[8 + c] < best[c]) ? 8 + c : c;  // tie: the lower shift
      int chs = bidx[c];
      if (F == IQ1_M) chs = (slot != c) ? bidx[8 + c] : chs;
      const float ssel = G::IQ1 ? sc[c & 7] : sc[c];
      int kb;
      uint32_t mfield;
      if (LDS_RESCAN) rescan_chunk_lds<F, CH, SORTED>(s_u, SORTED ? &s_g[gw][0] : s_u, a, S, chs, ssel, !all_even, kb, mfield);
      else rescan_chunk<F, CH>(A.grid, gt, S, chs, ssel, G::IQ1 ? (slot >> 3) : 0, !all_even, kb, mfield);
      int cu = c;
      if (d16 == 0) { kb = 0; mfield = 0; cu = 0; }
      __syncthreads();  // the previous choice's bytes have been read from LDS
      s_k[gw][rl] = static_cast<uint16_t>(kb);
      s_m[gw][rl] = static_cast<uint8_t>(mfield);
      if (gw % GPU == 0) s_c[uw][rl] = static_cast<uint8_t>(cu);
      __syncthreads();
      // wave p packs packed unit p of the workgroup for the tile's rows, lane = row
      constexpr int PPW = WGG / G::PG;
      if (wave < PPW && tile * 64 + lane < A.rpe) {
        const int64_t rp = e * A.rpe + tile * 64 + lane;
        pack_bytes<F>(A.out + c * A.copy_stride + (rp * A.nb + b) * G::BYTES, sb * PPW + wave, lane,
                      s_k + wave * G::PG, s_m + wave * G::PG, s_c + wave * (G::PG / GPU), A.dscr[rp * A.nb + b]);
      }
    }
    return;
  }

  // ---- choice per unit ---------------------------------------------------
  int cu = 0;     // unit choice (IQ1_S: (h << 3) | ls)
  int slot = 0;   // slot of this lane's group under that choice
  if (FIXED) {
    cu = fixed_c;
    slot = (F == IQ1_M) ? (best[1] < best[0] ? 1 : 0) : 0;
  } else {
    // each (unit, row) is scored once: wave p < UPW scores unit p for row
    // lane (the unit's other groups would repeat the same sums) and hands the
    // choice to the unit's items through LDS; the row's block scale comes
    // through LDS too, since a lane's item row need not be its lane's row
    __shared__ float s_drow[64];
    __shared__ uint8_t s_cu[UPW][64];
#pragma unroll
    for (int s = 0; s < NSLOT; ++s) s_best[gw][s][rl] = best[s];
    if (gw == 0) s_drow[rl] = d;
    __syncthreads();
    if (wave < UPW) {
      const float dr = s_drow[lane];
      float bs = 0.0f;
      int cs = 0;
#pragma unroll
      for (int c = 0; c < G::NC; ++c) {
        // the slot scales as the sweep formed them (sc[] of the row)
        const float s = G::IQ1 ? dr * static_cast<float>(2 * (F == IQ1_S ? (c & 7) : c) + 1)
                               : dr * (static_cast<float>(2 * c + 1) * 0.125f);
        float score = 0.0f;
#pragma unroll
        for (int i = 0; i < GPU; ++i) {
          const int w = wave * GPU + i;
          float bb;
          if (F == IQ1_M) {
            const float b0 = s_best[w][c][lane], b1 = s_best[w][8 + c][lane];
            bb = (b1 < b0) ? b1 : b0;          // tie: the lower shift
          } else {
            bb = s_best[w][c][lane];
          }
          const float ev = s * bb;
          score = (i == 0) ? ev : score + ev;
        }
        if (c == 0 || score < bs) { bs = score; cs = c; }
      }
      s_cu[wave][lane] = static_cast<uint8_t>(cs);
    }
    __syncthreads();
    cu = s_cu[uw][rl];
    if (F == IQ1_M) {
      float b0 = best[0], b1 = best[8];
#pragma unroll
      for (int c = 1; c < 8; ++c) {
        b0 = (cu == c) ? best[c] : b0;
        b1 = (cu == c) ? best[8 + c] : b1;
      }
      slot = (b1 < b0) ? 8 + cu : cu;
    } else {
      slot = cu;
    }
  }

  // ---- rescan the chosen chunk for the exact entry ----------------------
  int chs = bidx[0];
#pragma unroll
  for (int s = 1; s < NSLOT; ++s) chs = (slot == s) ? bidx[s] : chs;
  float ssel;
  int hsel;
  if (FIXED) {
    ssel = fs;
    hsel = (F == IQ1_M) ? slot : fh;
  } else {
    ssel = sc[0];
    if (!G::IQ1) {
#pragma unroll
      for (int c = 1; c < 16; ++c) ssel = (slot == c) ? sc[c] : ssel;
    } else {
#pragma unroll
      for (int l = 1; l < 8; ++l) ssel = ((slot & 7) == l) ? sc[l] : ssel;
    }
    hsel = G::IQ1 ? (slot >> 3) : 0;
  }
  int kb;
  uint32_t mfield;
  rescan_chunk<F, CH>(A.grid, SORTED ? &s_g[gw][0] : gt, S, chs, ssel, hsel, !all_even, kb, mfield);
  if (zero_blk) { kb = 0; mfield = 0; cu = 0; }

  // ---- pack ----------------------------------------------------------------
  s_k[gw][rl] = static_cast<uint16_t>(kb);
  s_m[gw][rl] = static_cast<uint8_t>(mfield);
  if (gw % GPU == 0) s_c[uw][rl] = static_cast<uint8_t>(cu);
  __syncthreads();
  // wave p packs packed unit p of the workgroup's PPW, lane = row (the row and
  // its scale are recomputed here rather than kept through the sweep)
  constexpr int PPW = WGG / G::PG;
  if (wave >= PPW || tile * 64 + lane >= A.rpe) return;
  const int64_t rp = e * A.rpe + tile * 64 + lane;
  pack_bytes<F>(A.out + (rp * A.nb + b) * G::BYTES, sb * PPW + wave, lane, s_k + wave * G::PG, s_m + wave * G::PG,
                s_c + wave * (G::PG / GPU), A.dscr[rp * A.nb + b]);
}

// ---------------------------------------------------------------------------
// Decode: one thread per group.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ld16(const uint8_t *p) { return *reinterpret_cast<const uint16_t *>(p); }

// Decode group g (0..31) of one block into 8 fp32 values.
template <int F>
__device__ __forceinline__ GroupFields group_fields(const uint8_t *blk, int g) {
  using G = Geo<F>;
  GroupFields f;
  f.mask = 0;
  f.h = 0;
  const int u = g / G::GPU;
  if (F == IQ2_XXS) {
    f.d16 = ld16(blk);
    const int ib = g >> 2, l = g & 3;
    const uint32_t word = ld16(blk + 2 + 8 * ib + 4) | (ld16(blk + 2 + 8 * ib + 6) << 16);
    f.k = blk[2 + 8 * ib + l];
    const uint32_t si = (word >> (7 * l)) & 0x7fu;
    f.mask = si | ((__builtin_popcount(si) & 1u) << 7);
    f.ls = word >> 28;
  } else if (F == IQ2_XS) {
    f.d16 = ld16(blk);
    const uint32_t v = ld16(blk + 2 + 2 * g);
    f.k = v & 511u;
    const uint32_t si = v >> 9;
    f.mask = si | ((__builtin_popcount(si) & 1u) << 7);
    const uint32_t sbyte = blk[66 + (u >> 1)];
    f.ls = (u & 1) ? (sbyte >> 4) : (sbyte & 15u);
  } else if (F == IQ2_S) {
    f.d16 = ld16(blk);
    f.k = blk[2 + g] | (((blk[66 + (g >> 2)] >> (2 * (g & 3))) & 3u) << 8);
    f.mask = blk[34 + g];
    const uint32_t sbyte = blk[74 + (u >> 1)];
    f.ls = (u & 1) ? (sbyte >> 4) : (sbyte & 15u);
  } else if (F == IQ1_S) {
    f.d16 = ld16(blk);
    const uint32_t w = ld16(blk + 34 + 2 * (g >> 2));
    f.k = blk[2 + g] | (((w >> (3 * (g & 3))) & 7u) << 8);
    f.ls = (w >> 12) & 7u;
    f.h = w >> 15;
  } else {
    f.d16 = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) f.d16 |= (ld16(blk + 48 + 2 * w) >> 12) << (4 * w);
    const uint32_t nb = blk[32 + (g >> 1)];
    const uint32_t nib = (g & 1) ? (nb >> 4) : (nb & 15u);
    f.k = blk[g] | ((nib & 7u) << 8);
    f.h = nib >> 3;
    f.ls = (ld16(blk + 48 + 2 * (u >> 2)) >> (3 * (u & 3))) & 7u;
  }
  return f;
}

// The group's 8 values from its fields (d: the block scale as fp32).
template <int F>
__device__ __forceinline__ void group_values(float d, uint32_t k, uint32_t mask, uint32_t ls, uint32_t h,
                                             const float *__restrict__ grid, float y[8]) {
  using G = Geo<F>;
  float gv[8];
  load_entry(grid + static_cast<int64_t>(k) * 8, gv);
  if (!G::IQ1) {
    const float s = d * (static_cast<float>(2 * ls + 1) * 0.125f);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = s * gv[j];
      y[j] = ((mask >> j) & 1u) ? -v : v;
    }
  } else {
    const float s = d * static_cast<float>(2 * ls + 1);
    const float delta = h ? -0.125f : 0.125f;
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = s * (gv[j] + delta);
  }
}

template <int F>
__device__ __forceinline__ void decode_group(const uint8_t *blk, int g, const float *__restrict__ grid, float y[8]) {
  const GroupFields f = group_fields<F>(blk, g);
  group_values<F>(f16_bits_to_f32(static_cast<uint16_t>(f.d16)), f.k, f.mask, f.ls, f.h, grid, y);
}

template <int F>
__global__ void __launch_bounds__(256) decode_kernel(const uint8_t *__restrict__ packed, int64_t ngroups,
                                                      const float *__restrict__ grid, void *out, int dtype) {
  using G = Geo<F>;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= ngroups) return;
  float y[8];
  decode_group<F>(packed + (i >> 5) * G::BYTES, static_cast<int>(i & 31), grid, y);
  if (dtype == 1) {
    uint4 o;
    o.x = f32_to_bf16(y[0]) | (static_cast<uint32_t>(f32_to_bf16(y[1])) << 16);
    o.y = f32_to_bf16(y[2]) | (static_cast<uint32_t>(f32_to_bf16(y[3])) << 16);
    o.z = f32_to_bf16(y[4]) | (static_cast<uint32_t>(f32_to_bf16(y[5])) << 16);
    o.w = f32_to_bf16(y[6]) | (static_cast<uint32_t>(f32_to_bf16(y[7])) << 16);
    reinterpret_cast<uint4 *>(out)[i] = o;
  } else {
    float4 *o = reinterpret_cast<float4 *>(out) + 2 * i;
    o[0] = make_float4(y[0], y[1], y[2], y[3]);
    o[1] = make_float4(y[4], y[5], y[6], y[7]);
  }
}

// ---------------------------------------------------------------------------
// Local-Hessian choice search (ModelOpt PR #3158).  Damping of the diagonal
// Hessian blocks: lambda = perc_damp * mean(diag H_b), the diagonal summed in
// fp64 (j ascending) and the mean rounded to fp32.  One wave per block: the
// lanes fetch the 256 diagonal entries (each in its own cache line) together,
// then lane 0 walks the running sum from LDS.  The same pass flags the blocks
// no calibration token reached (an all-zero diagonal) for the choice search.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(64) damping_kernel(const float *__restrict__ hess, float perc_damp,
                                                      float *__restrict__ lam, uint8_t *__restrict__ reached) {
  __shared__ double s_d[256];
  const int64_t i = blockIdx.x;
  const float *H = hess + i * 65536;
  bool nonzero = false;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = static_cast<int>(threadIdx.x) + 64 * t;
    const float h = H[j * 257];
    s_d[j] = static_cast<double>(h);
    nonzero = nonzero || h != 0.0f;
  }
  // a calibration token reached the block iff some column's sum of squares
  // (a diagonal entry) is nonzero
  const uint64_t any = __ballot(nonzero);
  __syncthreads();
  if (threadIdx.x == 0) {
    double acc = 0.0;
    for (int j = 0; j < 256; ++j) acc += s_d[j];
    lam[i] = perc_damp * static_cast<float>(acc / 256.0);
    reached[i] = any != 0 ? 1 : 0;
  }
}

// the unit's weights (the same under every choice)
template <int F>
__device__ __forceinline__ void unit_weights(const EncArgs &A, int64_t r, int b, int u, float *x) {
  using G = Geo<F>;
#pragma unroll
  for (int gi = 0; gi < G::GPU; ++gi)
    load8(A.w, A.dtype, r * A.cols + static_cast<int64_t>(b) * 256 + (u * G::GPU + gi) * 8, x + gi * 8);
}

template <int F>
__device__ __forceinline__ void record_values(float d, uint32_t rec, const float *__restrict__ grid, float y[8]) {
  group_values<F>(d, rec & 2047u, (rec >> 11) & 255u, (rec >> 19) & 15u, (rec >> 23) & 1u, grid, y);
}

// The same values in two steps, so the grid loads can be issued well before
// the values are needed: record_entry fetches the entry, record_finish applies
// the scale and signs (or shift) exactly as group_values does.
__device__ __forceinline__ void record_entry(uint32_t rec, const float *__restrict__ grid, float gv[8]) {
  load_entry(grid + static_cast<int64_t>(rec & 2047u) * 8, gv);
}
template <int F>
__device__ __forceinline__ void record_finish(float d, uint32_t rec, const float gv[8], float y[8]) {
  using G = Geo<F>;
  const uint32_t mask = (rec >> 11) & 255u, ls = (rec >> 19) & 15u, h = (rec >> 23) & 1u;
  if (!G::IQ1) {
    const float s = d * (static_cast<float>(2 * ls + 1) * 0.125f);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = s * gv[j];
      y[j] = ((mask >> j) & 1u) ? -v : v;
    }
  } else {
    const float s = d * static_cast<float>(2 * ls + 1);
    const float delta = h ? -0.125f : 0.125f;
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = s * (gv[j] + delta);
  }
}


typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x32 __attribute__((ext_vector_type(32)));

// One wave's cross-term part on the matrix cores: dst[i * 64 + row] =
// sum_k h[i][k] dw_row[k] for the unit's UV rows i and the wave's 64 rows
// (lane = row; dw holds the lane's own row), k ascending from zero.  The fp32
// MFMA forms that take one k per step (32x32x1 in two blocks, 16x16x1 in four)
// round each step as one fmaf does, so the result is the fmaf chain
// part = fmaf(h_ik, dw_k, part) bit for bit.  H's row i is the A operand
// (lane i of each block holds it, read from hrow + i * SH), dw the B operand,
// so each block is 32 (16) rows of the wave; the accumulator's element (i, row)
// sits in register r of lane l as decoded below.
template <int UV, int SH>
__device__ __forceinline__ void unit_part_mfma(const float *hrow, const float dw[UV], float *dst, int lane) {
  const float4 *h4 = reinterpret_cast<const float4 *>(hrow + (lane & (UV - 1)) * SH);
  if constexpr (UV == 32) {
    f32x32 acc = {};
#pragma unroll
    for (int k4 = 0; k4 < UV / 4; ++k4) {
      const float4 h = h4[k4];
      acc = __builtin_amdgcn_mfma_f32_32x32x1f32(h.x, dw[4 * k4 + 0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x1f32(h.y, dw[4 * k4 + 1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x1f32(h.z, dw[4 * k4 + 2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x1f32(h.w, dw[4 * k4 + 3], acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const int i = 8 * ((r & 15) >> 2) + 4 * (lane >> 5) + (r & 3), row = 32 * (r >> 4) + (lane & 31);
      dst[i * 64 + row] = acc[r];
    }
  } else {
    static_assert(UV == 16, "units of 16 or 32 columns");
    f32x16 acc = {};
#pragma unroll
    for (int k4 = 0; k4 < UV / 4; ++k4) {
      const float4 h = h4[k4];
      acc = __builtin_amdgcn_mfma_f32_16x16x1f32(h.x, dw[4 * k4 + 0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x1f32(h.y, dw[4 * k4 + 1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x1f32(h.z, dw[4 * k4 + 2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x1f32(h.w, dw[4 * k4 + 3], acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 4 * (lane >> 4) + (r & 3), row = 16 * (r >> 2) + (lane & 15);
      dst[i * 64 + row] = acc[r];
    }
  }
}

// y = H dw for one choice of the wave's own unit, on the matrix cores, in the
// lanes' own layout: y[i] = sum_k ha_i[k] dw[k], k ascending from zero (the
// fmaf chain, bit for bit), where lane l holds in ha the row i = l % UV of the
// damped block and in dw its own row's residual.  The accumulator's layout is
// unit_part_mfma's; the exchanges then give every lane all UV values of its own
// row.  UV = 32: register r holds (i, row) = (8 (r % 16 / 4) + 4 (l / 32) + r % 4,
// 32 (r / 16) + l % 32), so one permlane32 swap per register pair (r, r + 16)
// trades the upper lanes' low registers for the lower lanes' high ones, leaving
// i = 8 (r / 4) + r % 4 in register r and i = 8 (r / 4) + 4 + r % 4 in r + 16.
// UV = 16: register 4 b + e holds (i, row) = (4 (l / 16) + e, 16 b + l % 16):
// four lane groups of 4 x 4 tiles, transposed by a permlane32 stage (groups
// 0 <-> 2, 1 <-> 3) and a permlane16 stage (0 <-> 1, 2 <-> 3), leaving i = r in
// register r.
template <int UV>
__device__ __forceinline__ void unit_hdw_mfma(const float ha[UV], const float dw[UV], float y[UV]) {
  if constexpr (UV == 32) {
    f32x32 acc = {};
#pragma unroll
    for (int k = 0; k < UV; ++k) acc = __builtin_amdgcn_mfma_f32_32x32x1f32(ha[k], dw[k], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[r]), __float_as_uint(acc[16 + r]), false, false);
      y[8 * (r >> 2) + (r & 3)] = __uint_as_float(sw[0]);
      y[8 * (r >> 2) + 4 + (r & 3)] = __uint_as_float(sw[1]);
    }
  } else {
    f32x16 acc = {};
#pragma unroll
    for (int k = 0; k < UV; ++k) acc = __builtin_amdgcn_mfma_f32_16x16x1f32(ha[k], dw[k], acc, 0, 0, 0);
    uint32_t t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) t[r] = __float_as_uint(acc[r]);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const auto sw = __builtin_amdgcn_permlane32_swap(t[4 * b + e], t[4 * (b + 2) + e], false, false);
        t[4 * b + e] = sw[0];
        t[4 * (b + 2) + e] = sw[1];
      }
#pragma unroll
    for (int b = 0; b < 4; b += 2)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const auto sw = __builtin_amdgcn_permlane16_swap(t[4 * b + e], t[4 * (b + 1) + e], false, false);
        t[4 * b + e] = sw[0];
        t[4 * (b + 1) + e] = sw[1];
      }
#pragma unroll
    for (int r = 0; r < 16; ++r) y[r] = __uint_as_float(t[r]);
  }
}

// Local-Hessian choice search (ModelOpt PR #3158's choice_search): from the
// payloads of every choice, give each unit its best choice under its own
// damped diagonal Hessian block, then revisit the units twice, each taking the
// choice that most lowers the block error dw H dw^T with the others held.
// Evaluation order (fp32, explicit fmaf): unit error e = sum_i dw_i (sum_j
// H_ij dw_j), i and j ascending over the unit's columns; the cross term
// r = sum over the other units v of H_uv dw_v is gathered unit by unit (an
// fmaf chain over v's columns from zero per unit, the units' parts added in
// ascending order); a candidate scores fmaf(2, dw . r, e); first minimum wins.
// The damped block is H + lambda I, lambda = perc_damp * mean(diag H).
//
// One workgroup per (expert, 64-row tile, block) with one wave per unit:
// lanes are rows, H is shared by the 64 rows, and wave v keeps its unit's
// weights and current residual in registers.  The products with H run on the
// matrix cores as [UV x UV] . [UV x 64 rows] MFMA chains (one column per step,
// so each is the fmaf chain above bit for bit), H's rows as the A operand and
// the lanes' residuals as B.  The every-choice sweep hands over each group's
// fields under every choice as one word per (choice, group, row), rows
// contiguous, so the residuals come from coalesced loads rather than from
// packed bytes.  Step A: wave v scores every choice of unit v
// (unit_hdw_mfma); the own-block errors do not change between passes, so each
// wave keeps those of the choices it scores later.  A revisit of unit u: every
// other wave v forms its part H_uv dw_v (unit_part_mfma); the waves add the
// parts in unit order (each a slice of the rows of r); the waves score unit
// u's choices between them, with u's weights passed through LDS; wave u takes
// the first minimum.
// With A.out set, the workgroup then packs its block's payload under the
// picks from the same field records (the every-choice sweep's fields under
// choice c are the fixed-choice encoder's fields under c).
template <int F>
__global__ void __launch_bounds__(64 * Geo<F>::UNITS) choice_search_kernel(EncArgs A, const uint32_t *__restrict__ rec,
                                                                          const uint16_t *__restrict__ dblk,
                                                                          const float *__restrict__ hess,
                                                                          const float *__restrict__ lamv,
                                                                          const uint8_t *__restrict__ reached,
                                                                          uint8_t *__restrict__ choices) {
  using G = Geo<F>;
  constexpr int U = G::UNITS, UV = 8 * G::GPU, NC = G::NC, GPU = G::GPU;
  constexpr int NCW = (NC + U - 1) / U;     // choices of the revisited unit scored per wave
  constexpr int NI = (UV + U - 1) / U;      // cross-term rows summed per wave
  static_assert(U * NC <= U * UV, "the error table fits the parts buffer");
  static_assert(32 * 64 * 3 + U * 64 <= U * UV * 64 * 4, "the payload fields fit the parts buffer");
  // s_buf holds the table of own-block errors [unit][choice][row] after step A,
  // then the parts H_uv dw_v [v][i][row] of the unit being revisited
  __shared__ float s_buf[U * UV * 64];
  __shared__ float s_r[UV][64];      // its cross term
  __shared__ float s_x[UV][64];      // its weights
  __shared__ float s_f[NC][64];      // its candidates' scores
  // the revisited unit's rows of the damped-free block H (UV x 256), staged
  // one revisit ahead: each thread prefetches HV4 float4 into registers at the
  // start of a revisit and stores them once the parts have been formed
  // (rows padded to SH floats, so the lanes' operand reads of the parts spread
  // over the banks)
  constexpr int HROW = UV * 256, NT = 64 * U, HV4 = HROW / 4 / NT, SH = 256 + 4;
  static_assert(HROW % (4 * NT) == 0, "whole float4 per thread");
  __shared__ __attribute__((aligned(16))) float s_h[UV * SH];
  const int64_t L = xcd_remap(blockIdx.x, A.total_wg);
  const int64_t tile = L % A.tiles_per_e;
  const int64_t q = L / A.tiles_per_e;
  const int b = static_cast<int>(q % A.nb);
  const int64_t e = q / A.nb;
  const int v = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // this wave's unit
  const int lane = threadIdx.x & 63;
  const int64_t rin = tile * 64 + lane;
  const bool valid = rin < A.rpe;
  const int64_t r = e * A.rpe + (valid ? rin : A.rpe - 1);
  const float *H = hess + (e * A.nb + b) * 65536;
  const float lam = lamv[e * A.nb + b];
  // record of (choice c, group g) for this lane's row
  const int64_t rstride = A.rows;
  const uint32_t *rrow = rec + static_cast<int64_t>(b) * 32 * rstride + r;
  const int64_t cstride = A.nb * 32 * rstride;

  // the picks out, and with A.out the payload under them
  auto finish = [&](int pick) {
    if (valid) choices[(r * A.nb + b) * U + v] = static_cast<uint8_t>(pick);
    if (!A.out) return;

    // payload under the picks: each wave stages its unit's fields (the parts
    // buffer is free: in the search its last reader is two barriers back, and
    // the never-reached path below does not use it), then wave sb packs packed
    // unit sb as the search kernel does
    constexpr int PG = G::PG, SBS = 32 / PG, UPW = PG / GPU;
    uint16_t(*p_k)[64] = reinterpret_cast<uint16_t(*)[64]>(s_buf);
    uint8_t(*p_m)[64] = reinterpret_cast<uint8_t(*)[64]>(s_buf + 32 * 64 / 2);
    uint8_t(*p_c)[64] = reinterpret_cast<uint8_t(*)[64]>(s_buf + 32 * 64 / 2 + 32 * 64 / 4);
    const uint16_t d16 = dblk[r * A.nb + b];
#pragma unroll
    for (int gi = 0; gi < GPU; ++gi) {
      const uint32_t wd = rrow[pick * cstride + (v * GPU + gi) * rstride];
      p_k[v * GPU + gi][lane] = static_cast<uint16_t>(wd & 2047u);
      p_m[v * GPU + gi][lane] = static_cast<uint8_t>(G::IQ1 ? (wd >> 23) & 1u : (wd >> 11) & 255u);
    }
    p_c[v][lane] = static_cast<uint8_t>(d16 ? pick : 0);
    __syncthreads();
    if (v < SBS && valid) {
      uint8_t *blk = A.out + (r * A.nb + b) * G::BYTES;
      pack_bytes<F>(blk, v, lane, p_k + v * PG, p_m + v * PG, p_c + v * UPW, d16);
      if (F != IQ1_M && v == 0) *reinterpret_cast<uint16_t *>(blk) = d16;
    }
  };

  // R21: a block no calibration token reached (its Hessian diagonal, each
  // column's sum of squares, all zero: flagged by damping_kernel) keeps the
  // encoder's own choices.  One flag per block, so the whole workgroup takes
  // this path.  Each unit scores every choice from the field records with the
  // fp32 operations of the search's unit scoring: the record under choice c
  // holds the group's first-minimum entry (and IQ1_M's better shift), whose
  // reduced error is the slot minimum the search compared.
  if (!reached[e * A.nb + b]) {
    float xu[UV], au[UV];
    unit_weights<F>(A, r, b, v, xu);
#pragma unroll
    for (int j = 0; j < UV; ++j)
      au[j] = A.imp ? A.imp[e * A.cols + static_cast<int64_t>(b) * 256 + v * UV + j] : 1.0f;
    const float d = f16_bits_to_f32(dblk[r * A.nb + b]);
    GroupState<F> S[GPU];
#pragma unroll
    for (int gi = 0; gi < GPU; ++gi) S[gi].init(xu + gi * 8, au + gi * 8);
    float bs = 0.0f;
    int own = 0;
#pragma unroll 1
    for (int c = 0; c < NC; ++c) {
      float score = 0.0f;
#pragma unroll
      for (int gi = 0; gi < GPU; ++gi) {
        const uint32_t rcg = rrow[c * cstride + (v * GPU + gi) * rstride];
        float g[8];
        record_entry(rcg, A.grid, g);
        const float q2 = S[gi].template term<G::PARITY>(g);
        const float *a = au + gi * 8;
        float s, t;
        if (!G::IQ1) {
          s = d * (static_cast<float>(2 * c + 1) * 0.125f);
          t = __builtin_fmaf(s, iq2_norm(a, g), q2);
        } else {
          const float delta = ((rcg >> 23) & 1u) ? -0.125f : 0.125f;
          float gh = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float u = g[j] + delta;
            gh = __builtin_fmaf(a[j], u * u, gh);
          }
          s = d * static_cast<float>(2 * (F == IQ1_S ? (c & 7) : c) + 1);
          t = __builtin_fmaf(s, gh, __builtin_fmaf(delta, S[gi].S2, q2));
        }
        const float ev = s * t;
        score = gi == 0 ? ev : score + ev;
      }
      if (c == 0 || score < bs) { bs = score; own = c; }
    }
    finish(own);
    return;
  }

  // step A: every choice of unit v under its own damped block; the U diagonal sub-blocks H_vv ([v][i][j], U * UV * UV = HROW floats) are
  // staged in s_h first
  for (int t4 = threadIdx.x; t4 < HROW / 4; t4 += NT) {
    const int vv = t4 / (UV * UV / 4), rem = t4 % (UV * UV / 4);
    const int i = rem / (UV / 4), j4 = rem % (UV / 4);
    reinterpret_cast<float4 *>(s_h)[t4] =
        *reinterpret_cast<const float4 *>(H + static_cast<int64_t>(vv * UV + i) * 256 + vv * UV + 4 * j4);
  }
  float xv[UV], dwv[UV];
  unit_weights<F>(A, r, b, v, xv);
  const float d = f16_bits_to_f32(dblk[r * A.nb + b]);
  int pick = 0;
  {
    // one choice at a time on the matrix cores (unit_hdw_mfma); the next
    // choice's field words and grid entries are fetched while this one's
    // product runs
    uint32_t rcs[GPU];
    float gvs[UV];
#pragma unroll
    for (int gi = 0; gi < GPU; ++gi) rcs[gi] = rrow[(v * GPU + gi) * rstride];
#pragma unroll
    for (int gi = 0; gi < GPU; ++gi) record_entry(rcs[gi], A.grid, &gvs[gi * 8]);
    __syncthreads();  // s_h holds every H_vv
    // this lane's row of the damped block H_vv + lambda I (the A operand)
    float ha[UV];
    {
      const int ia = lane & (UV - 1);
      const float *Hi = s_h + (v * UV + ia) * UV;
#pragma unroll
      for (int k = 0; k < UV; ++k) {
        const float h = Hi[k];
        ha[k] = k == ia ? h + lam : h;
      }
    }
    float best = 0.0f;
#pragma unroll 1
    for (int c = 0; c < NC; ++c) {
      float dw[UV];
#pragma unroll
      for (int gi = 0; gi < GPU; ++gi) {
        float y[8];
        record_finish<F>(d, rcs[gi], &gvs[gi * 8], y);
#pragma unroll
        for (int j = 0; j < 8; ++j) dw[gi * 8 + j] = xv[gi * 8 + j] - y[j];
      }
      const int cn = c + 1 < NC ? c + 1 : c;
#pragma unroll
      for (int gi = 0; gi < GPU; ++gi) rcs[gi] = rrow[cn * cstride + (v * GPU + gi) * rstride];
#pragma unroll
      for (int gi = 0; gi < GPU; ++gi) record_entry(rcs[gi], A.grid, &gvs[gi * 8]);
      float yv[UV];
      unit_hdw_mfma<UV>(ha, dw, yv);
      float err = 0.0f;
#pragma unroll
      for (int i = 0; i < UV; ++i) err = __builtin_fmaf(dw[i], yv[i], err);
      s_buf[(v * NC + c) * 64 + lane] = err;
      if (c == 0 || err < best) { best = err; pick = c; }
    }
  }
#pragma unroll
  for (int gi = 0; gi < GPU; ++gi) {
    float y[8];
    record_values<F>(d, rrow[pick * cstride + (v * GPU + gi) * rstride], A.grid, y);
#pragma unroll
    for (int j = 0; j < 8; ++j) dwv[gi * 8 + j] = xv[gi * 8 + j] - y[j];
  }
  __syncthreads();
  // each wave keeps the errors of the choices it scores in the passes
  float qk[NCW][U];
#pragma unroll
  for (int k = 0; k < NCW; ++k)
#pragma unroll
    for (int u = 0; u < U; ++u) qk[k][u] = v + U * k < NC ? s_buf[(u * NC + v + U * k) * 64 + lane] : 0.0f;
  // the prefetched rows are held in one vector value: as an array of float4
  // the compiler would place them in LDS, storing each load as it arrives and
  // so waiting for it at once
  typedef float hvec_t __attribute__((ext_vector_type(4 * HV4)));
  hvec_t hpre;
  auto h_load = [&](const float *src) {
#pragma unroll
    for (int t = 0; t < HV4; ++t) {
      const float4 x = reinterpret_cast<const float4 *>(src)[threadIdx.x + t * NT];
      hpre[4 * t] = x.x;
      hpre[4 * t + 1] = x.y;
      hpre[4 * t + 2] = x.z;
      hpre[4 * t + 3] = x.w;
    }
  };
  auto h_store = [&]() {
#pragma unroll
    for (int t = 0; t < HV4; ++t) {
      const int f = threadIdx.x + t * NT;
      *reinterpret_cast<float4 *>(s_h + (f >> 6) * SH + 4 * (f & 63)) =
          make_float4(hpre[4 * t], hpre[4 * t + 1], hpre[4 * t + 2], hpre[4 * t + 3]);
    }
  };
  h_load(H);
  h_store();
  __syncthreads();
  // the fields of this wave's share of a revisited unit's choices do not
  // depend on the picks: they are loaded one revisit ahead, and their grid
  // entries are fetched as the revisit starts, to be used after the cross term
  uint32_t rc[NCW][GPU];
#pragma unroll
  for (int k = 0; k < NCW; ++k)
#pragma unroll
    for (int gi = 0; gi < GPU; ++gi) rc[k][gi] = v + U * k < NC ? rrow[(v + U * k) * cstride + gi * rstride] : 0u;
  // two passes over the units in ascending order
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll 1
    for (int u = 0; u < U; ++u) {
      const bool more = pass == 0 || u + 1 < U;  // a next revisit exists
      const int un = (u + 1) % U;
      if (more) h_load(H + un * HROW);
      // (the 32-column units score two choices per wave: their entries would
      // not fit the register budget, so they are fetched when scored)
      constexpr bool EARLY = NCW * UV <= 16;
      float gvc[NCW][UV];
      if (EARLY) {
#pragma unroll
        for (int k = 0; k < NCW; ++k)
#pragma unroll
          for (int gi = 0; gi < GPU; ++gi) record_entry(rc[k][gi], A.grid, &gvc[k][gi * 8]);
      }
      uint32_t rcn[NCW][GPU];
#pragma unroll
      for (int k = 0; k < NCW; ++k)
#pragma unroll
        for (int gi = 0; gi < GPU; ++gi)
          rcn[k][gi] = more && v + U * k < NC ? rrow[(v + U * k) * cstride + (un * GPU + gi) * rstride] : 0u;
      if (v != u) {
        unit_part_mfma<UV, SH>(s_h + v * UV, dwv, s_buf + v * UV * 64, lane);
      } else {  // the unit's weights, reloaded rather than kept in registers
        float xu[UV];
        unit_weights<F>(A, r, b, v, xu);
#pragma unroll
        for (int i = 0; i < UV; ++i) s_x[i][lane] = xu[i];
      }
      __syncthreads();
      if (more) h_store();  // every wave has formed its part: the next revisit's rows replace these
      // cross term rows i = v, v + U, ...: the parts added in unit order
#pragma unroll
      for (int t = 0; t < NI; ++t) {
        const int i = v + U * t;
        if (i < UV) {
          float pv[U];
#pragma unroll
          for (int w = 0; w < U; ++w) pv[w] = s_buf[(w * UV + i) * 64 + lane];  // [u] unused
          float acc = 0.0f;
#pragma unroll
          for (int w = 0; w < U; ++w) acc = w != u ? acc + pv[w] : acc;
          s_r[i][lane] = acc;
        }
      }
      __syncthreads();
      // group by group: the group's weights and cross term are read from LDS
      // once for all of this wave's choices (each choice's dot product is
      // still one fmaf chain over the unit's columns in ascending order)
      float dwc[NCW][UV];
      float dot[NCW];
#pragma unroll
      for (int k = 0; k < NCW; ++k) dot[k] = 0.0f;
#pragma unroll
      for (int gi = 0; gi < GPU; ++gi) {
        float xs[8], rs[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xs[j] = s_x[gi * 8 + j][lane];
          rs[j] = s_r[gi * 8 + j][lane];
        }
#pragma unroll
        for (int k = 0; k < NCW; ++k) {
          if (v + U * k < NC) {
            float y[8];
            if (!EARLY) record_entry(rc[k][gi], A.grid, &gvc[k][gi * 8]);
            record_finish<F>(d, rc[k][gi], &gvc[k][gi * 8], y);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              dwc[k][gi * 8 + j] = xs[j] - y[j];
              dot[k] = __builtin_fmaf(dwc[k][gi * 8 + j], rs[j], dot[k]);
            }
          }
        }
      }
#pragma unroll
      for (int k = 0; k < NCW; ++k) {
        const int c = v + U * k;
        if (c < NC) {
          float qu = qk[k][0];
#pragma unroll
          for (int w = 1; w < U; ++w) qu = u == w ? qk[k][w] : qu;
          s_f[c][lane] = __builtin_fmaf(2.0f, dot[k], qu);
        }
      }
      __syncthreads();
      // every wave finds each row's pick; the wave that scored it hands its
      // residual to wave u through s_r (free until the next cross term)
      float best = s_f[0][lane];
      int pk = 0;
      for (int c = 1; c < NC; ++c) {
        const float f = s_f[c][lane];
        if (f < best) { best = f; pk = c; }
      }
#pragma unroll
      for (int k = 0; k < NCW; ++k)
        if (pk == v + U * k) {
#pragma unroll
          for (int j = 0; j < UV; ++j) s_r[j][lane] = dwc[k][j];
        }
      __syncthreads();
      if (v == u) {
        pick = pk;
#pragma unroll
        for (int j = 0; j < UV; ++j) dwv[j] = s_r[j][lane];
      }
#pragma unroll
      for (int k = 0; k < NCW; ++k)
#pragma unroll
        for (int gi = 0; gi < GPU; ++gi) rc[k][gi] = rcn[k][gi];
    }
  }
  finish(pick);
}

// ---------------------------------------------------------------------------
// Host launchers.  Workspace plans first (pure functions of the sizes), then
// the launches: each is checked, and a failed launch returns at once.
// ---------------------------------------------------------------------------
namespace {
constexpr int kGridN[5] = {256, 512, 1024, 2048, 2048};
constexpr int kNC[5] = {16, 16, 16, 16, 8};
bool launched_ok() { return hipGetLastError() == hipSuccess; }
}  // namespace

QuantPlan plan_quantize(int fmt, int64_t rows, int64_t cols, int64_t rpe, bool weighted) {
  QuantPlan p{};
  const int64_t nb = cols / 256, E = rows / rpe;
  const int NG = fmt >= IQ1_S ? 2 : 1;
  p.ntab = weighted ? E * (cols / 8) : 1;
  const size_t gbytes = static_cast<size_t>(p.ntab) * NG * kGridN[fmt] * sizeof(float);
  const size_t dbytes = static_cast<size_t>(rows) * nb * sizeof(uint16_t);
  const size_t fbytes = weighted ? static_cast<size_t>(E) * nb : 0;
  p.goff = 0;
  p.doff = ws_up(gbytes);
  p.foff = p.doff + ws_up(dbytes);
  p.bytes = p.foff + ws_up(fbytes) + kWsAlign;
  return p;
}

ChoicePlan plan_choice_search(int fmt, int64_t rows, int64_t cols, int64_t rpe, bool weighted) {
  ChoicePlan p{};
  const int64_t nblocks = rows * (cols / 256), nl = (rows / rpe) * (cols / 256);
  p.q = plan_quantize(fmt, rows, cols, rpe, weighted);
  p.roff = 0;
  p.loff = ws_up(static_cast<size_t>(kNC[fmt]) * nblocks * 32 * sizeof(uint32_t));
  p.foff = p.loff + ws_up(static_cast<size_t>(nl) * sizeof(float));
  p.qoff = p.foff + ws_up(static_cast<size_t>(nl));
  p.bytes = p.qoff + p.q.bytes;  // the encoder part keeps its own slack
  return p;
}

template <int F>
static int launch_quantize_t(EncArgs A, int mode, void *ws, hipEvent_t ev0, hipEvent_t ev1, hipStream_t stream) {
  using G = Geo<F>;
  const int64_t nblocks = A.rows * A.nb;
  if (nblocks == 0) return 0;
  const QuantPlan P = plan_quantize(F, A.rows, A.cols, A.rpe, A.imp != nullptr);
  const int NG = G::IQ1 ? 2 : 1;
  const int64_t cgs = A.cols / 8;
  char *base = ws_base(ws);
  A.gtab = reinterpret_cast<float *>(base + P.goff);
  A.dscr = reinterpret_cast<uint16_t *>(base + P.doff);
  uint8_t *impflags = A.imp ? reinterpret_cast<uint8_t *>(base + P.foff) : nullptr;
  A.gtab_e_stride = A.imp ? cgs * NG * G::N : 0;
  A.gtab_cg_stride = A.imp ? NG * G::N : 0;
  A.tiles_per_e = (A.rpe + 63) / 64;
  A.total_wg = A.E * A.tiles_per_e * A.nb * (32 / G::WGG);

  const int64_t gblocks = (P.ntab * G::N + 255) / 256;
  const int64_t nf = impflags ? A.E * A.nb : 0;
  hipLaunchKernelGGL(prep_kernel<F>, dim3(static_cast<unsigned>(gblocks + (nf + 3) / 4)), dim3(256), 0, stream,
                     A.grid, A.imp, P.ntab, A.gtab, gblocks, nf, impflags);
  if (!launched_ok()) return -1;
  hipLaunchKernelGGL(anchor_kernel<F>, dim3(static_cast<unsigned>((nblocks + 7) / 8)), dim3(256), 0, stream, A,
                     static_cast<const uint8_t *>(impflags));
  if (!launched_ok()) return -1;
  if (ev0 && hipEventRecord(ev0, stream) != hipSuccess) return -1;
  const dim3 grid_dim(static_cast<unsigned>(A.total_wg)), block_dim(64 * G::WGG);
  if (mode == RECORDS)
    hipLaunchKernelGGL((search_kernel<F, RECORDS>), grid_dim, block_dim, 0, stream, A);
  else if (mode == EVERY)
    hipLaunchKernelGGL((search_kernel<F, EVERY>), grid_dim, block_dim, 0, stream, A);
  else if (A.choices)
    hipLaunchKernelGGL((search_kernel<F, FIXED_CHOICES>), grid_dim, block_dim, 0, stream, A);
  else
    hipLaunchKernelGGL((search_kernel<F, SEARCH>), grid_dim, block_dim, 0, stream, A);
  if (!launched_ok()) return -1;
  if (ev1 && hipEventRecord(ev1, stream) != hipSuccess) return -1;
  return 0;
}

int launch_quantize(int fmt, EncArgs A, bool every, void *ws, hipEvent_t ev0, hipEvent_t ev1, hipStream_t stream) {
  const int mode = every ? EVERY : SEARCH;
  switch (fmt) {
    case IQ2_XXS: return launch_quantize_t<IQ2_XXS>(A, mode, ws, ev0, ev1, stream);
    case IQ2_XS: return launch_quantize_t<IQ2_XS>(A, mode, ws, ev0, ev1, stream);
    case IQ2_S: return launch_quantize_t<IQ2_S>(A, mode, ws, ev0, ev1, stream);
    case IQ1_S: return launch_quantize_t<IQ1_S>(A, mode, ws, ev0, ev1, stream);
    case IQ1_M: return launch_quantize_t<IQ1_M>(A, mode, ws, ev0, ev1, stream);
  }
  return -1;
}

template <int F>
static int launch_decode_t(const uint8_t *packed, int64_t rows, int64_t cols, const float *grid, void *out,
                           int dtype, hipStream_t stream) {
  const int64_t ng = rows * (cols / 256) * 32;
  if (ng == 0) return 0;
  hipLaunchKernelGGL(decode_kernel<F>, dim3(static_cast<unsigned>((ng + 255) / 256)), dim3(256), 0, stream,
                     packed, ng, grid, out, dtype);
  return launched_ok() ? 0 : -1;
}

int launch_decode(int fmt, const uint8_t *packed, int64_t rows, int64_t cols, const float *grid, void *out,
                  int dtype, hipStream_t stream) {
  switch (fmt) {
    case IQ2_XXS: return launch_decode_t<IQ2_XXS>(packed, rows, cols, grid, out, dtype, stream);
    case IQ2_XS: return launch_decode_t<IQ2_XS>(packed, rows, cols, grid, out, dtype, stream);
    case IQ2_S: return launch_decode_t<IQ2_S>(packed, rows, cols, grid, out, dtype, stream);
    case IQ1_S: return launch_decode_t<IQ1_S>(packed, rows, cols, grid, out, dtype, stream);
    case IQ1_M: return launch_decode_t<IQ1_M>(packed, rows, cols, grid, out, dtype, stream);
  }
  return -1;
}

template <int F>
static int launch_choice_search_t(EncArgs A, const float *hess, float perc_damp, uint8_t *choices, void *ws,
                                  hipStream_t stream) {
  using G = Geo<F>;
  const int64_t nblocks = A.rows * A.nb;
  if (nblocks == 0) return 0;
  const int64_t nl = A.E * A.nb;
  const ChoicePlan P = plan_choice_search(F, A.rows, A.cols, A.rpe, A.imp != nullptr);
  char *base = ws_base(ws);
  uint32_t *rec = reinterpret_cast<uint32_t *>(base + P.roff);
  float *lam = reinterpret_cast<float *>(base + P.loff);
  uint8_t *reached = reinterpret_cast<uint8_t *>(base + P.foff);
  void *qws = base + P.qoff;
  // the record sweep's fp16 block scales, read by the choice search
  const uint16_t *dblk = reinterpret_cast<const uint16_t *>(ws_base(qws) + P.q.doff);
  EncArgs E = A;
  E.choices = nullptr;
  E.out = nullptr;
  E.copies = 0;
  E.rec = rec;
  if (launch_quantize_t<F>(E, RECORDS, qws, nullptr, nullptr, stream) != 0) return -1;
  hipLaunchKernelGGL(damping_kernel, dim3(static_cast<unsigned>(nl)), dim3(64), 0, stream, hess, perc_damp, lam,
                     reached);
  if (!launched_ok()) return -1;
  A.tiles_per_e = (A.rpe + 63) / 64;
  A.total_wg = A.E * A.tiles_per_e * A.nb;
  hipLaunchKernelGGL(choice_search_kernel<F>, dim3(static_cast<unsigned>(A.total_wg)), dim3(64 * G::UNITS), 0,
                     stream, A, static_cast<const uint32_t *>(rec), dblk, hess, static_cast<const float *>(lam),
                     static_cast<const uint8_t *>(reached), choices);
  return launched_ok() ? 0 : -1;
}

int launch_choice_search(int fmt, EncArgs A, const float *hess, float perc_damp, uint8_t *choices, void *ws,
                         hipStream_t stream) {
  switch (fmt) {
    case IQ2_XXS: return launch_choice_search_t<IQ2_XXS>(A, hess, perc_damp, choices, ws, stream);
    case IQ2_XS: return launch_choice_search_t<IQ2_XS>(A, hess, perc_damp, choices, ws, stream);
    case IQ2_S: return launch_choice_search_t<IQ2_S>(A, hess, perc_damp, choices, ws, stream);
    case IQ1_S: return launch_choice_search_t<IQ1_S>(A, hess, perc_damp, choices, ws, stream);
    case IQ1_M: return launch_choice_search_t<IQ1_M>(A, hess, perc_damp, choices, ws, stream);
  }
  return -1;
}

}  // namespace iq
