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

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Two binary32 values -> two bf16 rounded to nearest even, a in the low half,
// in one instruction (V_CVT_PK_BF16_F32; subnormals kept, as the kernels run
// with binary32 denormals on; overflow gives inf, NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, bf2));
}

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

// ---------------------------------------------------------------------------
// binary32-grade accumulation on the 16-bit sparse matrix instruction.
//
// The FP8 instruction above adds the 64 products of one instruction in fixed
// point 13 bits below the largest of them, so a product under 2^-13 of the
// largest is dropped.  V_SMFMAC_F32_16X16X64_BF16 aligns its terms (the
// accumulator included) 24 bits below the largest and truncates toward zero:
// the error of a long sum is that of a binary32 sum.  Every OCP FP8 value
// (subnormals included) is exactly a bf16 value and every product of two is
// exact in binary32, so one 128-k FP8 step can run as two bf16 instructions
// on exactly widened codes (V_CVT_SCALEF32_PK_BF16_{FP8,BF8} with scale 1).
//
// Layout (gfx950, measured): the bf16 instruction is the FP8 one at half the
// k.  A lane l holds row l%16 and the 8 kept values of virtual k
// 16*(l/16) .. +15 with a 16-bit index (nibble j = positions of group j);
// B lane l holds column l%16, elements 0..7 = virtual k 8*(l/16) .. +7 and
// elements 8..15 = virtual k 32 + 8*(l/16) .. +7.  Half h (0, 1) of an FP8
// step uses, in every lane, FP8 A bytes 4h..4h+3 and 8+4h..8+4h+3 (groups
// 2h, 2h+1, 4+2h, 5+2h of the lane), index bytes h and 2+h, and FP8 B bytes
// 8h..8h+7 and 16+8h..16+8h+7.  This pairs every kept weight value with the
// activation of its own k and moves no data between lanes; the two halves
// together cover the step's 128 k once.
// ---------------------------------------------------------------------------
enum { ACC_F32 = 0, ACC_F8 = 1 };

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v16bf __attribute__((ext_vector_type(16)));

// Bytes 0,1 (HI = false) or 2,3 (HI = true) of w, FP8 format FMT, as two bf16
// values (exact).
template <int FMT, bool HI>
__device__ __forceinline__ int widen2(int w) {
  if constexpr (FMT == FMT_E4M3) return __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  else return __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI));
}

// Half H of an FP8 A fragment (16 kept bytes) as the bf16 instruction's A operand.
template <int FMT, int H>
__device__ __forceinline__ v4i widen_a_half(const v4i& a) {
  return v4i{widen2<FMT, false>(a[H]), widen2<FMT, true>(a[H]), widen2<FMT, false>(a[2 + H]),
             widen2<FMT, true>(a[2 + H])};
}

// Half H of an FP8 B fragment (32 bytes) as the bf16 instruction's B operand.
template <int FMT, int H>
__device__ __forceinline__ v8i widen_b_half(const v8i& b) {
  return v8i{widen2<FMT, false>(b[2 * H]),     widen2<FMT, true>(b[2 * H]),
             widen2<FMT, false>(b[2 * H + 1]), widen2<FMT, true>(b[2 * H + 1]),
             widen2<FMT, false>(b[4 + 2 * H]), widen2<FMT, true>(b[4 + 2 * H]),
             widen2<FMT, false>(b[5 + 2 * H]), widen2<FMT, true>(b[5 + 2 * H])};
}

// Index of half H: bytes H and 2+H of the FP8 step's index word, in both
// 16-bit halves (the instruction reads one of them).
template <int H>
__device__ __forceinline__ int idx_half(int idx) {
  return (int)__builtin_amdgcn_perm(0u, (uint32_t)idx, H ? 0x03010301u : 0x02000200u);
}

__device__ __forceinline__ v4f smfmac16_bf16(const v4i& aw, const v8i& bw, v4f c, int ix) {
  return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(v8bf, aw), __builtin_bit_cast(v16bf, bw), c, ix,
                                                   0, 0);
}

// One 128-k step, c += A(a, idx) * B(b), with the accumulation ACC.
template <int XF, int WF, int ACC>
__device__ __forceinline__ v4f mma_step(const v4i& a, const v8i& b, v4f c, int idx) {
  if constexpr (ACC == ACC_F8) {
    return smfmac16<XF, WF>(a, b, c, idx);
  } else {
    c = smfmac16_bf16(widen_a_half<WF, 0>(a), widen_b_half<XF, 0>(b), c, idx_half<0>(idx));
    return smfmac16_bf16(widen_a_half<WF, 1>(a), widen_b_half<XF, 1>(b), c, idx_half<1>(idx));
  }
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
