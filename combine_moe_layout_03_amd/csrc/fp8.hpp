// Per-128-channel E4M3 cast of bf16 rows on gfx950, for the FP8 dispatch of
// the NeMo AutoModel page "nemo_automodel.components.moe.uccl_ep.buffer"
// (Buffer.low_latency_dispatch: use_fp8, round_scale, use_ue8m0; returns).
//
// A lane holds one 16-byte vector (8 bf16 channels), so the 128 channels that
// share a scale are the 16 lanes of one DPP row: the group maximum is a
// four-step rotate-and-max inside the row, with no LDS and no cross-row
// traffic. Then, per group:
//   amax  = max |x| (at least 1e-4, so an all-zero group has a finite scale),
//   scale = amax / 448 (448 = largest finite E4M3 value), a correctly rounded
//           float division; with round_scale, rounded up to a power of two;
//   code  = E4M3 of x / scale (correctly rounded float division, then the
//           hardware's round-to-nearest-even conversion to OCP E4M3).
// The per-element quotient costs one multiply and two fmas instead of a full
// division: with y = RN(1/scale), q = RN(x*y) is within one ulp of x/scale,
// the remainder x - scale*q is exact in one fma, and q + remainder*y rounds to
// RN(x/scale) (Markstein's theorem; the identity is also checked exhaustively
// on the CPU for every bf16 significand of x against every float significand
// of the scale). Quotients too small for a normal float give a signed zero
// code either way, so copying the sign of x settles them.
// The UE8M0 form of a power-of-two scale is its biased exponent byte.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kFp8RoundScale = 1;  // scales rounded up to powers of two
constexpr int kFp8Ue8m0 = 2;       // scales stored as packed exponent bytes
constexpr int kFp8ScaleRows = 4;   // receive-side scales row-major [rows][...]
constexpr int kFp8Group = 128;     // channels per scale

typedef uint32_t fp8_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Maximum over the 16 lanes of this lane's DPP row (row_ror by 8, 4, 2, 1).
// Every lane of the wave must execute it.
__device__ __forceinline__ uint32_t row16_max(uint32_t m) {
  m = umax32(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x128, 0xf, 0xf, false));
  m = umax32(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x124, 0xf, 0xf, false));
  m = umax32(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x122, 0xf, 0xf, false));
  m = umax32(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x121, 0xf, 0xf, false));
  return m;
}

__device__ __forceinline__ float fp8_bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float fp8_bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Four floats -> four E4M3 codes, channel order in little-endian bytes.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// RN(x / s) given y = RN(1/s), for finite x (see above).
__device__ __forceinline__ float div_by_scale(float x, float s, float y) {
#pragma clang fp contract(off)
  const float q = x * y;
  const float r = __builtin_fmaf(-s, q, x);
  return __builtin_copysignf(__builtin_fmaf(r, y, q), x);
}

struct Fp8Lane {
  uint32_t lo, hi;  // codes of the lane's 8 channels
  float scale;      // the group's scale (equal in its 16 lanes)
};

// Cast one lane's 8 bf16 values; the lane's DPP row is the 128-channel group.
template <int kFlags>
__device__ __forceinline__ Fp8Lane fp8_cast_lane(fp8_u32x4 v) {
  // (kFp8ScaleRows only changes where the caller stores the scales)
  // |x| as bf16 bit patterns: for finite values the integer order is the
  // magnitude order
  uint32_t m = umax32(umax32(v.x & 0x7fffu, v.x >> 16 & 0x7fffu),
                      umax32(v.y & 0x7fffu, v.y >> 16 & 0x7fffu));
  m = umax32(m, umax32(umax32(v.z & 0x7fffu, v.z >> 16 & 0x7fffu),
                       umax32(v.w & 0x7fffu, v.w >> 16 & 0x7fffu)));
  m = row16_max(m);
  float amax = __uint_as_float(m << 16);
  if (amax < 1e-4f) amax = 1e-4f;
  float s = amax / 448.0f;
  if (kFlags & kFp8RoundScale) {
    uint32_t b = __float_as_uint(s);
    if (b & 0x7fffffu) b = (b & 0xff800000u) + 0x800000u;  // next power of two up
    s = __uint_as_float(b);
  }
  const float y = 1.0f / s;  // correctly rounded (exact for a power of two)
  Fp8Lane r;
  r.lo = e4m3x4(div_by_scale(fp8_bf16_lo(v.x), s, y), div_by_scale(fp8_bf16_hi(v.x), s, y),
                div_by_scale(fp8_bf16_lo(v.y), s, y), div_by_scale(fp8_bf16_hi(v.y), s, y));
  r.hi = e4m3x4(div_by_scale(fp8_bf16_lo(v.z), s, y), div_by_scale(fp8_bf16_hi(v.z), s, y),
                div_by_scale(fp8_bf16_lo(v.w), s, y), div_by_scale(fp8_bf16_hi(v.w), s, y));
  r.scale = s;
  return r;
}

// The four UE8M0 bytes of a wave's 512 channels (groups in lanes 0, 16, 32,
// 48), packed group 4w+b into byte b; wave-uniform.
__device__ __forceinline__ uint32_t ue8m0_word(float scale) {
  const int e = (int)(__float_as_uint(scale) >> 23);
  return (uint32_t)__builtin_amdgcn_readlane(e, 0) |
         (uint32_t)__builtin_amdgcn_readlane(e, 16) << 8 |
         (uint32_t)__builtin_amdgcn_readlane(e, 32) << 16 |
         (uint32_t)__builtin_amdgcn_readlane(e, 48) << 24;
}

}  // namespace moe
