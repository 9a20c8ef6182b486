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
// row's reciprocal with one fma correction (cast8; for scales from 2^-80 up,
// checked to give the codes of the plain division for every bf16 input),
// below that scale with an exactness check that sends the rare elements it
// cannot settle to the IEEE division; either way the codes are those of the
// plain division.
//
// Layout: one 64-lane wavefront owns one row.  Lane l holds 16-byte chunks
// (8 bf16) l, l+64, l+128, ... of its row in registers between the amax sweep
// and the cast sweep, so each input byte is read from HBM once.  Rows longer
// than 32 chunks per lane (cols > 16384) take a two-sweep path that reads the
// row again (from L2 in practice).
#include <atomic>

#include "sfr_device.hpp"
#include "sfr_launch.hpp"
#include "sfr_quant.hpp"

namespace sfr {
namespace {

constexpr int kRowsPerBlock = 4;  // 4 wavefronts of 64 lanes

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
    } else if (nchunks == 64 * R) {
#pragma unroll
      for (int i = 0; i < R; ++i) qr[lane + 64 * i] = cast8<FMT>(buf[i], s, r);
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

// Few rows (decode): one workgroup per row, so a row's casts spread over
// four SIMDs instead of one wavefront (a lone row of 4096 elements is
// otherwise ~1300 dependent ALU instructions on one SIMD): one 8-element
// chunk per thread up to K = 8192 (256, 512 or 1024 threads), two above (a
// 14336-element row: 2 chunks per thread instead of 7 with 256 threads:
// 22.9 -> 17.5 us for quantization + linear layer at M = 16, N = 4096).  CPT chunks of 8 elements per thread, all loads in flight at once; the
// amax is reduced across the wavefronts through LDS.
template <int FMT, int CPT, int NT>
__global__ __launch_bounds__(NT) void quantize_row_per_block_kernel(const uint16_t* __restrict__ x, int64_t cols,
                                                                    uint8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ uint32_t red[NT / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int nchunks = (int)(cols >> 3);
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * cols);
  uint2* qr = reinterpret_cast<uint2*>(q + row * cols);
  uint4 buf[CPT];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + NT * i;
    buf[i] = c < nchunks ? xr[c] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < CPT; ++i) m = mag_max8(buf[i], m);
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) m = max(m, red[w]);
  const float amax = bf16_to_f32(m);
  const float s = amax / Fp8<FMT>::fmax;
  const float r = 1.0f / s;
  if (tid == 0) scale[row] = (m == 0) ? 0.0f : s;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + NT * i;
    if (c < nchunks) qr[c] = m == 0 ? zero8(buf[i]) : cast8<FMT>(buf[i], s, r);
  }
}

template <int FMT>
hipError_t launch_fmt(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, float* scale,
                      hipStream_t stream) {
  if (rows <= 64 && cols <= 16384) {
    const int64_t chunks = cols >> 3;
#define SFR_QB(C, T)                                                                                 \
  hipLaunchKernelGGL((quantize_row_per_block_kernel<FMT, C, T>), dim3((unsigned)rows), dim3(T), 0, stream, x, \
                     cols, q, scale)
    if (chunks <= 256) SFR_QB(1, 256);
    else if (chunks <= 512) SFR_QB(1, 512);
    else if (chunks <= 1024) SFR_QB(1, 1024);
    else SFR_QB(2, 1024);
#undef SFR_QB
    return hipGetLastError();
  }
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
constexpr int64_t kTensorMaxBlocks = 1024;  // cast pass at 8192 x 4096: 29 us with 512 blocks, 23 with 1024

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

// Workspace of quantize_tensorwise_fp8_noalloc: one per device, for
// callers that cannot allocate.  Its largest use is one slot per block of
// the cast pass (kTensorMaxBlocks 32-bit slots); every slot a call reads is
// written by that call's first pass, so nothing needs clearing between calls.
// Host code must use the address hipGetSymbolAddress returns for the current
// device, never the array's name.
static __device__ __align__(256) uint32_t scratch[kTensorMaxBlocks];

int64_t noalloc_workspace_bytes() { return (int64_t)sizeof(scratch); }

// The current device's copy of `scratch` (looked up once per device).
static hipError_t scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> cache[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    cache[dev].store(p, std::memory_order_release);  // every thread stores the same address
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_quantize_tensor_noalloc(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* q,
                                          float* scale, hipStream_t stream) {
  if (tensor_workspace_bytes(rows, cols) > noalloc_workspace_bytes()) return hipErrorInvalidValue;
  void* work = nullptr;
  hipError_t e = scratch_address(&work);
  if (e != hipSuccess) return e;
  return launch_quantize_tensor(x, rows, cols, fmt, q, scale, work, stream);
}

hipError_t launch_quantize(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* q,
                           float* scale, hipStream_t stream) {
  if (fmt == FMT_E4M3) return launch_fmt<FMT_E4M3>(x, rows, cols, q, scale, stream);
  return launch_fmt<FMT_E5M2>(x, rows, cols, q, scale, stream);
}

}  // namespace sfr
