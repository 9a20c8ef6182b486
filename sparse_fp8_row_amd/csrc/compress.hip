// 2:4 semi-structured compression of an FP8 matrix on gfx950.
//
// Method: pytorch/ao PR #1671 ("Add CUTLASS-based row-wise scaled sparse FP8
// kernel"): a converter of FP8 data to the 2:4 sparse format, which must treat
// -0.0 as a zero (the bug that PR found in the upstream compressor).  Each
// group of four consecutive k keeps its two largest magnitudes, ties going to
// the lower index.
//
// Selection: each byte of a group becomes the composite key
//     (low 7 bits << 2) | (3 - index)
// which orders by magnitude (the low 7 bits of an OCP FP8 byte order finite
// magnitudes, +0 and -0 alike) and then by lower index; all four keys differ,
// so the two largest keys name the kept pair.  Integer-only, hence bit-exact.
//
// Layout of the output (format version 1): values[n, k/2] holds the kept bytes
// of each group in ascending index order (-0.0 written as 0x00); meta[n, k/8]
// holds one nibble i0 | (i1 << 2) per group, even group in the low nibble.
// One thread turns 32 input bytes (8 groups) into 16 value bytes and one
// 32-bit metadata word, with 16-byte loads and stores.
//
// The same selection on bf16 bits is the weight's 2:4 pruning before
// quantization (prune_bf16_kernel).
#include "sfr_device.hpp"
#include "sfr_launch.hpp"

namespace sfr {
namespace {

__device__ __forceinline__ uint32_t group_select(uint32_t g, uint32_t* vals16) {
  uint32_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) key[i] = (((g >> (8 * i)) & 0x7Fu) << 2) | (3u - i);
  const uint32_t a = max(key[0], key[1]), b = min(key[0], key[1]);
  const uint32_t c = max(key[2], key[3]), d = min(key[2], key[3]);
  const uint32_t first = max(a, c);
  const uint32_t second = max(min(a, c), max(b, d));
  const uint32_t ia = 3u - (first & 3u), ib = 3u - (second & 3u);
  const uint32_t i0 = min(ia, ib), i1 = max(ia, ib);
  uint32_t v0 = (g >> (8 * i0)) & 0xFFu, v1 = (g >> (8 * i1)) & 0xFFu;
  v0 = (v0 == 0x80u) ? 0u : v0;
  v1 = (v1 == 0x80u) ? 0u : v1;
  *vals16 = v0 | (v1 << 8);
  return i0 | (i1 << 2);
}

__global__ __launch_bounds__(256) void compress_kernel(const uint4* __restrict__ w, int64_t nthreads,
                                                       uint4* __restrict__ values,
                                                       uint32_t* __restrict__ meta) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= nthreads) return;
  const uint4 lo = w[2 * t], hi = w[2 * t + 1];
  const uint32_t words[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  uint32_t out[4] = {0, 0, 0, 0};
  uint32_t mw = 0;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    uint32_t v16;
    const uint32_t nib = group_select(words[g], &v16);
    out[g / 2] |= v16 << (16 * (g % 2));
    mw |= nib << (4 * g);
  }
  values[t] = make_uint4(out[0], out[1], out[2], out[3]);
  meta[t] = mw;
}

// 2:4 pruning of a bf16 matrix: per group of four, the two largest
// magnitudes keep their bits and the other two become +0.0.  Composite keys
// (low 15 bits << 2) | (3 - index) order finite bf16 magnitudes (+0 and -0
// alike) and then the lower index, so the two largest keys name the
// survivors, exactly as in group_select.  One thread per 16 bytes (two
// groups); in place is allowed (each thread reads its bytes before writing
// them).
__device__ __forceinline__ uint64_t prune_group_bf16(uint64_t g) {
  uint32_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) key[i] = ((uint32_t)((g >> (16 * i)) & 0x7FFFu) << 2) | (3u - i);
  const uint32_t a = max(key[0], key[1]), b = min(key[0], key[1]);
  const uint32_t c = max(key[2], key[3]), d = min(key[2], key[3]);
  const uint32_t first = max(a, c);
  const uint32_t second = max(min(a, c), max(b, d));
  const uint32_t ia = 3u - (first & 3u), ib = 3u - (second & 3u);
  const uint64_t keep = (0xFFFFull << (16 * ia)) | (0xFFFFull << (16 * ib));
  return g & keep;
}

__global__ __launch_bounds__(256) void prune_bf16_kernel(const uint4* w, int64_t nthreads, uint4* out) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= nthreads) return;
  const uint4 v = w[t];
  const uint64_t g0 = prune_group_bf16(((uint64_t)v.y << 32) | v.x);
  const uint64_t g1 = prune_group_bf16(((uint64_t)v.w << 32) | v.z);
  out[t] = make_uint4((uint32_t)g0, (uint32_t)(g0 >> 32), (uint32_t)g1, (uint32_t)(g1 >> 32));
}

}  // namespace

hipError_t launch_prune_bf16(const uint16_t* w, int64_t n, int64_t k, uint16_t* out, hipStream_t stream) {
  // k % 8 == 0: each thread's 8 elements are two whole groups of one row
  const int64_t nthreads = n * k / 8;
  const dim3 grid((unsigned)((nthreads + 255) / 256)), block(256);
  hipLaunchKernelGGL(prune_bf16_kernel, grid, block, 0, stream, reinterpret_cast<const uint4*>(w), nthreads,
                     reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

hipError_t launch_compress(const uint8_t* w, int64_t n, int64_t k, uint8_t* values, uint8_t* meta,
                           hipStream_t stream) {
  // k % 32 == 0, so each thread's 32 bytes lie in one row and the flattened
  // offsets 32t (input), 16t (values) and 4t (meta) line up.
  const int64_t nthreads = n * k / 32;
  const dim3 grid((unsigned)((nthreads + 255) / 256)), block(256);
  hipLaunchKernelGGL(compress_kernel, grid, block, 0, stream, reinterpret_cast<const uint4*>(w), nthreads,
                     reinterpret_cast<uint4*>(values), reinterpret_cast<uint32_t*>(meta));
  return hipGetLastError();
}

}  // namespace sfr
