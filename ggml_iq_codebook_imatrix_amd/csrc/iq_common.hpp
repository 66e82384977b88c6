// iq_common.hpp -- device-side definitions shared by the libiq kernels.
//
// Layout facts restated from the pages (cited by page title and section):
//  * block sizes: ModelOpt PR #2513 commit messages (IQ2_XXS 2.0625 bits per
//    weight, IQ2_S 2.5625, IQ1_M 1.75, IQ1_S 0.1875 below IQ1_M); IQ2_XS holds a
//    9-bit index and a 7-bit sign index per group plus a 4-bit scale per 16.
//  * grid sizes 256 / 512 / 1024 / 2048 (same messages: "256-entry grid",
//    "twice IQ2_XS's", "2048-entry grid ... shared with IQ1_S").
//  * choices: ModelOpt PR "[1/5] Let the GGML IQ encoders take fixed per-group
//    choices": one local scale (plus, for IQ1_S, the delta sign) per choice unit;
//    IQ2 units take 16 choices, IQ1_S 16, IQ1_M 8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iq {

enum Fmt : int { IQ2_XXS = 0, IQ2_XS = 1, IQ2_S = 2, IQ1_S = 3, IQ1_M = 4 };

// Per-format geometry.  GPU = 8-value groups per choice unit; NC = choices per
// unit; PG = groups per packed unit, the smallest set of groups whose payload
// bytes no other set touches; WGG = groups (one wave each) per search
// workgroup, a multiple of PG (eight for the layouts whose groups are sorted
// by parity, so the sort deals from more items).
template <int F> struct Geo;
template <> struct Geo<IQ2_XXS> {
  static constexpr int BYTES = 66, N = 256, GPU = 4, UNITS = 8, NC = 16, PG = 4, WGG = 8;
  static constexpr bool IQ1 = false, PARITY = true;
};
template <> struct Geo<IQ2_XS> {
  static constexpr int BYTES = 74, N = 512, GPU = 2, UNITS = 16, NC = 16, PG = 4, WGG = 8;
  static constexpr bool IQ1 = false, PARITY = true;
};
template <> struct Geo<IQ2_S> {
  static constexpr int BYTES = 82, N = 1024, GPU = 2, UNITS = 16, NC = 16, PG = 4, WGG = 4;
  static constexpr bool IQ1 = false, PARITY = false;
};
template <> struct Geo<IQ1_S> {
  static constexpr int BYTES = 50, N = 2048, GPU = 4, UNITS = 8, NC = 16, PG = 4, WGG = 4;
  static constexpr bool IQ1 = true, PARITY = false;
};
template <> struct Geo<IQ1_M> {
  static constexpr int BYTES = 56, N = 2048, GPU = 2, UNITS = 16, NC = 8, PG = 8, WGG = 8;
  static constexpr bool IQ1 = true, PARITY = false;
};

// status bits (mirror include/iq.h)
constexpr int ST_NONFINITE = 1, ST_OVERFLOW = 2, ST_BADCHOICE = 4, ST_BADIMP = 8, ST_BADID = 16;

__device__ __forceinline__ void raise_status(int32_t *status, int bits) {
  if (status && bits) atomicOr(status, bits);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// fp16 bits <-> fp32 via the hardware conversions (IEEE, round to nearest even)
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = static_cast<_Float16>(f);
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

// Load 8 consecutive values (a group) as fp32.
__device__ __forceinline__ void load8(const void *base, int dtype, int64_t idx, float v[8]) {
  if (dtype == 1) {
    const uint4 q = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + idx);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(base) + idx);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

__device__ __forceinline__ bool finite_f(float x) { return (__float_as_uint(x) & 0x7f800000u) != 0x7f800000u; }

}  // namespace iq
