// Row-wise dynamic FP8 quantization on gfx950.
//
// Method: pytorch/ao PR #1671 ("Add CUTLASS-based row-wise scaled sparse FP8
// kernel"): FP8 activations with one scale per row, quantized dynamically, and
// casts that never produce NaN.  The amax is a deterministic reduction, the
// property the review of pytorch/ao PR #1455 ("[float8nocompile] ...
// atomic_max-based algo ...") asks to keep; here it is an exact integer max
// over the bf16 magnitude bits, reduced inside one wavefront, so no atomics
// and no cross-workgroup step exist at all.
//
// The per-element division x / scale is done as a multiplication by the
// row's reciprocal with an exactness check (cast8): the IEEE
// division runs only for the rare elements whose FP8 rounding the check cannot
// settle, so the codes are those of the plain division.
//
// Layout: one 64-lane wavefront owns one row.  Lane l holds 16-byte chunks
// (8 bf16) l, l+64, l+128, ... of its row in registers between the amax sweep
// and the cast sweep, so each input byte is read from HBM once.  Rows longer
// than 32 chunks per lane (cols > 16384) take a two-sweep path that reads the
// row again (from L2 in practice).
#include "sfr_device.hpp"
#include "sfr_launch.hpp"

namespace sfr {
namespace {

constexpr int kRowsPerBlock = 4;  // 4 wavefronts of 64 lanes

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

__device__ __forceinline__ uint32_t wave_max(uint32_t m) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  return m;
}

// True when q = fl32(x * rcp) is known to encode to the same FP8 code as
// fl32(x / scale) (see cast8).
template <int FMT>
__device__ __forceinline__ bool quotient_settled(float x, float q) {
  constexpr uint32_t kMinNormal = (FMT == FMT_E4M3) ? 0x3C800000u : 0x38800000u;  // 2^-6, 2^-14
  constexpr uint32_t kLowMask = (FMT == FMT_E4M3) ? 0xFFFFFu : 0x1FFFFFu;
  constexpr uint32_t kMid = (FMT == FMT_E4M3) ? 0x80000u : 0x100000u;
  const uint32_t b = __float_as_uint(q) & 0x7FFFFFFFu;
  const uint32_t low = b & kLowMask;
  const uint32_t dist = low > kMid ? low - kMid : kMid - low;
  return (b >= kMinNormal && b < 0x7F800000u && dist > 8u) || x == 0.0f;
}

// 8 bf16 -> 8 FP8 bytes.  `scale` > 0, `rcp` = fl32(1 / scale): the codes of
// fl32(x / scale) (IEEE binary32 division), clamped to +/-fmax and rounded to
// nearest even by the hardware converter.
//
// The quotients are formed as q = fl32(x * rcp), which differs from x / scale
// by at most 2^-23 relative, so fl32(x / scale) lies within a few binary32
// steps of q.  An FP8 code only changes where the value crosses the midpoint
// between two FP8 neighbours; in the FP8 normal range that midpoint has the
// low 20 (e4m3) or 21 (e5m2) bits of the binary32 pattern equal to 0x80000 /
// 0x100000.  When q's low bits are more than 8 steps from it, q and
// fl32(x / scale) round to the same code (at binade edges the low bits are
// near 0 or all ones, far from the midpoint).  Zero divides to a signed zero
// (taken as is: rcp is infinite when scale is below 2^-128).  An element the
// test cannot settle -- near a midpoint, in the FP8 subnormal
// range, or not finite -- takes the IEEE division (one branch per 8 elements).
template <int FMT>
__device__ __forceinline__ uint2 cast8(uint4 c, float scale, float rcp) {
  constexpr float fmax = Fp8<FMT>::fmax;
  uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float x[8], t[8];
  bool settled = true;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // a zero keeps its sign (x * rcp would give NaN when rcp is infinite)
    t[i] = x[i] == 0.0f ? x[i] : x[i] * rcp;
    settled = settled && quotient_settled<FMT>(x[i], t[i]);
  }
  if (__builtin_expect(!settled, 0)) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (!quotient_settled<FMT>(x[i], t[i])) t[i] = x[i] / scale;
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

template <int FMT, int R>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                            int64_t cols, uint8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;  // uniform per wavefront
  const int64_t nchunks = cols >> 3;
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * cols);
  uint2* qr = reinterpret_cast<uint2*>(q + row * cols);

  if constexpr (R > 0) {
    uint4 buf[R];
    uint32_t m = 0;
    if (nchunks == 64 * R) {
      // whole row in R chunks per lane: unconditional loads, all in flight at once
#pragma unroll
      for (int i = 0; i < R; ++i) buf[i] = xr[lane + 64 * i];
    } else {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int64_t c = lane + 64 * i;
        buf[i] = c < nchunks ? xr[c] : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) m = mag_max8(buf[i], m);
    m = wave_max(m);
    const float amax = bf16_to_f32(m);
    const float s = amax / Fp8<FMT>::fmax;
    const float r = 1.0f / s;
    if (lane == 0) scale[row] = (m == 0) ? 0.0f : s;
    if (m == 0) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int64_t c = lane + 64 * i;
        if (c < nchunks) qr[c] = zero8(buf[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int64_t c = lane + 64 * i;
        if (c < nchunks) qr[c] = cast8<FMT>(buf[i], s, r);
      }
    }
  } else {
    uint32_t m = 0;
    for (int64_t c = lane; c < nchunks; c += 64) m = mag_max8(xr[c], m);
    m = wave_max(m);
    const float amax = bf16_to_f32(m);
    const float s = amax / Fp8<FMT>::fmax;
    const float r = 1.0f / s;
    if (lane == 0) scale[row] = (m == 0) ? 0.0f : s;
    if (m == 0) {
      for (int64_t c = lane; c < nchunks; c += 64) qr[c] = zero8(xr[c]);
    } else {
      for (int64_t c = lane; c < nchunks; c += 64) qr[c] = cast8<FMT>(xr[c], s, r);
    }
  }
}

template <int FMT>
hipError_t launch_fmt(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, float* scale,
                      hipStream_t stream) {
  const int64_t per_lane = ((cols >> 3) + 63) / 64;
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(256);
#define SFR_Q(R) hipLaunchKernelGGL((quantize_rows_kernel<FMT, R>), grid, block, 0, stream, x, rows, cols, q, scale)
  // R = chunks per lane; rows of exactly 64 * R chunks (K = 4096 -> 8, K = 14336
  // -> 28) take the unconditional-load path
  if (per_lane <= 1) SFR_Q(1);
  else if (per_lane <= 2) SFR_Q(2);
  else if (per_lane <= 4) SFR_Q(4);
  else if (per_lane <= 8) SFR_Q(8);
  else if (per_lane <= 16) SFR_Q(16);
  else if (per_lane <= 28) SFR_Q(28);
  else if (per_lane <= 32) SFR_Q(32);
  else SFR_Q(0);
#undef SFR_Q
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Tensor-wise variant: one scale for the whole tensor.  Two launches over the
// same split of the tensor into blocks of `per_block` 16-byte chunks: the
// first writes each block's magnitude maximum to its own workspace slot; the
// second has every block reduce all slots (the same exact integer max in every
// block, no atomics, so the result is deterministic by construction), derive
// the scale and cast its chunks exactly as the row-wise kernel does.
// ---------------------------------------------------------------------------
constexpr int kTensorThreads = 256;
constexpr int64_t kTensorMaxBlocks = 512;

// chunks per block: a multiple of the block size, at most kTensorMaxBlocks blocks
__host__ __device__ inline int64_t tensor_chunks_per_block(int64_t chunks) {
  int64_t per = (chunks + kTensorMaxBlocks - 1) / kTensorMaxBlocks;
  per = (per + kTensorThreads - 1) / kTensorThreads * kTensorThreads;
  return per < kTensorThreads ? kTensorThreads : per;
}

__device__ __forceinline__ uint32_t block_max(uint32_t m, uint32_t* red) {
  m = wave_max(m);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = m;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int w = 1; w < kTensorThreads / 64; ++w) r = max(r, red[w]);
  return r;
}

__global__ __launch_bounds__(kTensorThreads) void tensor_amax_kernel(const uint4* __restrict__ x, int64_t chunks,
                                                                     int64_t per_block, uint32_t* __restrict__ part) {
  __shared__ uint32_t red[kTensorThreads / 64];
  const int64_t c0 = (int64_t)blockIdx.x * per_block;
  const int64_t c1 = min(c0 + per_block, chunks);
  uint32_t m = 0;
  int64_t c = c0 + threadIdx.x;
  // four loads in flight per thread
  for (; c + 3 * kTensorThreads < c1; c += 4 * kTensorThreads) {
    const uint4 v0 = x[c], v1 = x[c + kTensorThreads], v2 = x[c + 2 * kTensorThreads], v3 = x[c + 3 * kTensorThreads];
    m = mag_max8(v0, m);
    m = mag_max8(v1, m);
    m = mag_max8(v2, m);
    m = mag_max8(v3, m);
  }
  for (; c < c1; c += kTensorThreads) m = mag_max8(x[c], m);
  m = block_max(m, red);
  if (threadIdx.x == 0) part[blockIdx.x] = m;
}

template <int FMT>
__global__ __launch_bounds__(kTensorThreads) void tensor_cast_kernel(const uint4* __restrict__ x, int64_t chunks,
                                                                     int64_t per_block,
                                                                     const uint32_t* __restrict__ part, int nparts,
                                                                     uint2* __restrict__ q, float* __restrict__ scale) {
  __shared__ uint32_t red[kTensorThreads / 64];
  uint32_t m = 0;
  for (int i = threadIdx.x; i < nparts; i += kTensorThreads) m = max(m, part[i]);
  m = block_max(m, red);
  const float amax = bf16_to_f32(m);
  const float s = amax / Fp8<FMT>::fmax;
  const float r = 1.0f / s;
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale = (m == 0) ? 0.0f : s;
  const int64_t c0 = (int64_t)blockIdx.x * per_block;
  const int64_t c1 = min(c0 + per_block, chunks);
  if (m == 0) {
    for (int64_t c = c0 + threadIdx.x; c < c1; c += kTensorThreads) q[c] = zero8(x[c]);
    return;
  }
  int64_t c = c0 + threadIdx.x;
  for (; c + 3 * kTensorThreads < c1; c += 4 * kTensorThreads) {
    const uint4 v0 = x[c], v1 = x[c + kTensorThreads], v2 = x[c + 2 * kTensorThreads], v3 = x[c + 3 * kTensorThreads];
    q[c] = cast8<FMT>(v0, s, r);
    q[c + kTensorThreads] = cast8<FMT>(v1, s, r);
    q[c + 2 * kTensorThreads] = cast8<FMT>(v2, s, r);
    q[c + 3 * kTensorThreads] = cast8<FMT>(v3, s, r);
  }
  for (; c < c1; c += kTensorThreads) q[c] = cast8<FMT>(x[c], s, r);
}

}  // namespace

int64_t tensor_workspace_bytes(int64_t rows, int64_t cols) {
  const int64_t chunks = rows * cols / 8;
  const int64_t per = tensor_chunks_per_block(chunks);
  return 4 * ((chunks + per - 1) / per);
}

hipError_t launch_quantize_tensor(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* q, float* scale,
                                  void* workspace, hipStream_t stream) {
  const int64_t chunks = rows * cols / 8;
  const int64_t per = tensor_chunks_per_block(chunks);
  const int nb = (int)((chunks + per - 1) / per);
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint32_t* part = static_cast<uint32_t*>(workspace);
  hipLaunchKernelGGL(tensor_amax_kernel, dim3(nb), dim3(kTensorThreads), 0, stream, xv, chunks, per, part);
  if (fmt == FMT_E4M3)
    hipLaunchKernelGGL(tensor_cast_kernel<FMT_E4M3>, dim3(nb), dim3(kTensorThreads), 0, stream, xv, chunks, per, part,
                       nb, reinterpret_cast<uint2*>(q), scale);
  else
    hipLaunchKernelGGL(tensor_cast_kernel<FMT_E5M2>, dim3(nb), dim3(kTensorThreads), 0, stream, xv, chunks, per, part,
                       nb, reinterpret_cast<uint2*>(q), scale);
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* q,
                           float* scale, hipStream_t stream) {
  if (fmt == FMT_E4M3) return launch_fmt<FMT_E4M3>(x, rows, cols, q, scale, stream);
  return launch_fmt<FMT_E5M2>(x, rows, cols, q, scale, stream);
}

}  // namespace sfr
