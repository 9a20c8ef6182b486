// Device-side helpers shared by the gfx950 kernels of the sparse FP8 row-wise
// linear layer.  Internal header: not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfr {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

enum { FMT_E4M3 = 0, FMT_E5M2 = 1 };
enum { OUT_BF16 = 0, OUT_F32 = 1 };

// Largest finite magnitude of each OCP FP8 format.
template <int FMT> struct Fp8;
template <> struct Fp8<FMT_E4M3> { static constexpr float fmax = 448.0f; };
template <> struct Fp8<FMT_E5M2> { static constexpr float fmax = 57344.0f; };

// Two binary32 values -> two FP8 bytes with the gfx950 converter, written into
// bytes [0,1] (HI=false) or [2,3] (HI=true) of `old`.  The converter rounds to
// nearest even and keeps the sign of zero; inputs are clamped to +/-fmax by the
// caller, which makes the cast saturating.
template <int FMT, bool HI>
__device__ __forceinline__ int cvt_pk_fp8(float a, float b, int old) {
  if constexpr (FMT == FMT_E4M3) return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
  else return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, HI);
}

// binary32 -> bf16 bits, round to nearest even (finite inputs; overflow gives inf).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// 2:4 sparse x dense FP8 MFMA, 16x16 output, 128 dense k per instruction.
// A (sparse weight, format WF): lane l holds row l%16, kept values of dense
// k = 32*(l/16) .. +31 (16 bytes) with their 2-bit positions in `idx`.
// B (dense activation, format XF): lane l holds column l%16, bytes 0..15 are
// k = 16*(l/16) .. +15 and bytes 16..31 are k = 64 + 16*(l/16) .. +15.
// D: lane l holds rows 4*(l/16) .. +3 of column l%16.
template <int XF, int WF>
__device__ __forceinline__ v4f smfmac16(v4i a, v8i b, v4f c, int idx) {
  if constexpr (WF == FMT_E4M3 && XF == FMT_E4M3)
    return __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(a, b, c, idx, 0, 0);
  else if constexpr (WF == FMT_E4M3 && XF == FMT_E5M2)
    return __builtin_amdgcn_smfmac_f32_16x16x128_fp8_bf8(a, b, c, idx, 0, 0);
  else if constexpr (WF == FMT_E5M2 && XF == FMT_E4M3)
    return __builtin_amdgcn_smfmac_f32_16x16x128_bf8_fp8(a, b, c, idx, 0, 0);
  else
    return __builtin_amdgcn_smfmac_f32_16x16x128_bf8_bf8(a, b, c, idx, 0, 0);
}

// The same instruction through inline assembly, with the accumulator pinned in
// the accumulation registers (the compiler otherwise may keep a large
// accumulator set there but select the instruction's VGPR form and copy each
// accumulator out and back around every MFMA).  volatile keeps these in
// program order with each other and with memory operations.  The compiler
// does not see inside the asm, so the two hazards on the accumulator are the
// caller's: a plain write of it must precede its first MFMA by >= 5 wait
// states (acc_fence), and its result must not be read sooner than 19 wait
// states after the MFMA that wrote it (mfma_drain, then acc_fence).
template <int XF, int WF>
__device__ __forceinline__ void smfmac16_acc(v4f& c, const v4i& a, const v8i& b, int idx) {
  if constexpr (WF == FMT_E4M3 && XF == FMT_E4M3)
    asm volatile("v_smfmac_f32_16x16x128_fp8_fp8 %0, %1, %2, %3" : "+a"(c) : "v"(a), "v"(b), "v"(idx));
  else if constexpr (WF == FMT_E4M3 && XF == FMT_E5M2)
    asm volatile("v_smfmac_f32_16x16x128_fp8_bf8 %0, %1, %2, %3" : "+a"(c) : "v"(a), "v"(b), "v"(idx));
  else if constexpr (WF == FMT_E5M2 && XF == FMT_E4M3)
    asm volatile("v_smfmac_f32_16x16x128_bf8_fp8 %0, %1, %2, %3" : "+a"(c) : "v"(a), "v"(b), "v"(idx));
  else
    asm volatile("v_smfmac_f32_16x16x128_bf8_bf8 %0, %1, %2, %3" : "+a"(c) : "v"(a), "v"(b), "v"(idx));
}

// Orders every later use of c after this point, 5 wait states on.
__device__ __forceinline__ void acc_fence(v4f& c) { asm volatile("s_nop 4" : "+a"(c)); }

// 24 wait states: an MFMA issued before this has written its result after it.
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::); }

}  // namespace sfr
