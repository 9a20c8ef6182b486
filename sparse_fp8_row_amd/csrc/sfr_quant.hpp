// Device functions of the row-wise dynamic FP8 quantization, shared by the
// quantization kernels and the fused decode kernel, so both produce the same
// codes by the same arithmetic.
#pragma once

#include "sfr_device.hpp"

namespace sfr {

__device__ __forceinline__ uint32_t mag_max8(uint4 c, uint32_t m) {
  // |bf16| order == unsigned order of the low 15 bits (finite inputs)
  uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = max(m, w[i] & 0x7FFFu);
    m = max(m, (w[i] >> 16) & 0x7FFFu);
  }
  return m;
}

// Wavefront maximum, uniform in every lane, without LDS-path instructions:
// DPP row_shr 1, 2, 4, 8 (controls 0x111 .. 0x118; lanes shifted in from
// outside the 16-lane row read 0) leave each row's maximum in its lane 15,
// then four readlanes.
__device__ __forceinline__ uint32_t wave_max(uint32_t m) {
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x111, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x112, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x114, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x118, 0xF, 0xF, false));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)m, 15), b = (uint32_t)__builtin_amdgcn_readlane((int)m, 31);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)m, 47), d = (uint32_t)__builtin_amdgcn_readlane((int)m, 63);
  return max(max(a, b), max(c, d));
}

// True when q = fl32(x * rcp) is known to encode to the same FP8 code as
// fl32(x / scale) (see cast8).
template <int FMT>
__device__ __forceinline__ bool quotient_settled(float x, float q) {
  constexpr uint32_t kMinNormal = (FMT == FMT_E4M3) ? 0x3C800000u : 0x38800000u;  // 2^-6, 2^-14
  constexpr uint32_t kLowMask = (FMT == FMT_E4M3) ? 0xFFFFFu : 0x1FFFFFu;
  constexpr uint32_t kMid = (FMT == FMT_E4M3) ? 0x80000u : 0x100000u;
  const uint32_t b = __float_as_uint(q) & 0x7FFFFFFFu;
  // |low - kMid| > 8, as one wrapping add and compare (low < kMid - 8 wraps
  // to a large value)
  const bool far = ((b & kLowMask) + (8u - kMid)) > 16u;
  // bitwise, not short-circuit, so the test is straight-line code
  return ((b >= kMinNormal) & (b < 0x7F800000u) & far) | (x == 0.0f);
}

// Smallest scale for which cast8 forms the quotients with one fma
// correction (below it: the tested product, see cast8).
constexpr float kFmaQuotientMinScale = 0x1p-80f;

// 8 bf16 -> 8 FP8 bytes.  `scale` > 0, `rcp` = fl32(1 / scale): the codes of
// fl32(x / scale) (IEEE binary32 division), clamped to +/-fmax and rounded to
// nearest even by the hardware converter.  The row's elements satisfy
// |x| <= amax with scale = fl32(amax / fmax).
//
// From scale 2^-80 up the quotient is q0 = fl32(x * rcp), corrected once:
// q = fma(-fma(q0, scale, -x), rcp, q0) (the residual negated twice, so that
// x = -0 keeps its sign).  q is not always fl32(x / scale) -- it can differ
// by a unit in the last place -- but it always gives the same FP8 code: this
// was checked by enumerating every bf16 amax and every bf16 x with
// |x| <= amax, for both formats (about 2.1e9 pairs; codes first differ at
// scales below 2^-106).
//
// Below 2^-80 the quotients are formed as q = fl32(x * rcp), which differs
// from x / scale by at most 2^-23 relative, so fl32(x / scale) lies within a
// few binary32 steps of q.  An FP8 code only changes where the value crosses
// the midpoint between two FP8 neighbours; in the FP8 normal range that
// midpoint has the low 20 (e4m3) or 21 (e5m2) bits of the binary32 pattern
// equal to 0x80000 / 0x100000.  When q's low bits are more than 8 steps from
// it, q and fl32(x / scale) round to the same code (at binade edges the low
// bits are near 0 or all ones, far from the midpoint).  Zero divides to a
// signed zero (taken as is: rcp is infinite when scale is below 2^-128).  An
// element the test cannot settle -- near a midpoint, in the FP8 subnormal
// range, or not finite -- takes the IEEE division (one branch per 8
// elements).
template <int FMT>
__device__ __forceinline__ uint2 cast8(uint4 c, float scale, float rcp) {
  constexpr float fmax = Fp8<FMT>::fmax;
  uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float x[8], t[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
  if (__builtin_expect(scale >= kFmaQuotientMinScale, 1)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q0 = x[i] * rcp;
      const float rn = __builtin_fmaf(q0, scale, -x[i]);
      t[i] = __builtin_fmaf(-rn, rcp, q0);
    }
  } else {
    bool settled = true;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // a zero keeps its sign (x * rcp would give NaN when rcp is infinite)
      t[i] = x[i] == 0.0f ? x[i] : x[i] * rcp;
      settled &= quotient_settled<FMT>(x[i], t[i]);
    }
    if (!settled) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (!quotient_settled<FMT>(x[i], t[i])) t[i] = x[i] / scale;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = fminf(fmaxf(t[i], -fmax), fmax);
  int lo = cvt_pk_fp8<FMT, false>(t[0], t[1], 0);
  lo = cvt_pk_fp8<FMT, true>(t[2], t[3], lo);
  int hi = cvt_pk_fp8<FMT, false>(t[4], t[5], 0);
  hi = cvt_pk_fp8<FMT, true>(t[6], t[7], hi);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// All-zero row: keep each zero's sign (0x00 / 0x80).
__device__ __forceinline__ uint2 zero8(uint4 c) {
  uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t b[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t s0 = (w[i] >> 15) & 1u, s1 = (w[i] >> 31) & 1u;
    b[i / 2] |= ((s0 << 7) | (s1 << 15)) << (16 * (i % 2));
  }
  return make_uint2(b[0], b[1]);
}

}  // namespace sfr
