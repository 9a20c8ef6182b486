// Block-sparse (BSR) bf16 weight: conversion from dense and the linear layer.
//
// Source: pytorch/ao PR #1734 ("promote blocksparse from prototype, make it
// faster"): a weight stored in 64 x 64 blocks, most of them zero (sparsity
// level 0.9 in its measurements), multiplied by a dense activation whose row
// count is padded up to 16 in decode, with deep load pipelining mattering
// most.  The page names no number format; here the weight, activation and
// output are bf16 and the sum is binary32 (bf16 products are exact in it).
//
// Layout (the usual compressed-sparse-row structure over blocks): crow
// [n/64 + 1] block-row pointers, col [nnz] block-column indices (ascending in
// a block row), values [nnz][64][64] bf16, each block row-major.
#include "sfr_device.hpp"
#include "sfr_launch.hpp"

namespace sfr {
namespace {

constexpr int BS = 64;  // block edge

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Non-zero test of one 64 x 64 block of w [., k] (bf16 bits) by one
// wavefront: lane l reads 16-byte chunk l % 8 of rows 8 i + l / 8, i = 0..7
// (eight 1 KB loads, one 128-byte line per row).  +0.0 and -0.0 are zero.
__device__ __forceinline__ bool block_nonzero(const uint16_t* __restrict__ w, int64_t k, int64_t br, int64_t bc,
                                              int lane) {
  const uint8_t* base = reinterpret_cast<const uint8_t*>(w + (br * BS) * k + bc * BS);
  uint32_t any = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 v = *reinterpret_cast<const uint4*>(base + (int64_t)(8 * i + (lane >> 3)) * k * 2 + 16 * (lane & 7));
    any |= (v.x | v.y | v.z | v.w) & 0x7FFF7FFFu;
  }
  return __builtin_amdgcn_ballot_w64(any != 0) != 0;
}

// crow[br + 1] = number of kept blocks of block row br (one workgroup of 4
// wavefronts per block row, the wavefronts taking every 4th block column).
__global__ __launch_bounds__(256) void bsr_count_kernel(const uint16_t* __restrict__ w, int64_t k,
                                                        int32_t* __restrict__ crow) {
  __shared__ int cnt[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t br = blockIdx.x, nbc = k / BS;
  int c = 0;
  for (int64_t bc = wave; bc < nbc; bc += 4) c += block_nonzero(w, k, br, bc, lane) ? 1 : 0;
  if (lane == 0) cnt[wave] = c;
  __syncthreads();
  if (threadIdx.x == 0) crow[br + 1] = cnt[0] + cnt[1] + cnt[2] + cnt[3];
}

// In-place inclusive scan of crow[1 .. nbr] (counts -> block-row pointers)
// and crow[0] = 0: one workgroup of 1024 threads, chunk by chunk with a
// running carry (Hillis-Steele within a chunk).
__global__ __launch_bounds__(1024) void bsr_scan_kernel(int32_t* __restrict__ crow, int64_t nbr) {
  __shared__ int buf[1024];
  __shared__ int carry;
  const int t = threadIdx.x;
  if (t == 0) {
    carry = 0;
    crow[0] = 0;
  }
  __syncthreads();
  for (int64_t c0 = 0; c0 < nbr; c0 += 1024) {
    const int64_t i = c0 + t;
    int v = i < nbr ? crow[i + 1] : 0;
    buf[t] = v;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const int add = t >= d ? buf[t - d] : 0;
      __syncthreads();
      buf[t] += add;
      __syncthreads();
    }
    if (i < nbr) crow[i + 1] = carry + buf[t];
    __syncthreads();
    if (t == 1023) carry += buf[1023];
    __syncthreads();
  }
}

// Fill col and values of one block row per workgroup.  Block columns are
// taken 256 at a time: the 4 wavefronts test them (every 4th), an exclusive
// scan of the 256 flags gives each kept block its slot after the ones before
// it, and the wavefronts copy their kept blocks (eight 1 KB loads and stores
// each) to values[crow[br] + slot].
__global__ __launch_bounds__(256) void bsr_fill_kernel(const uint16_t* __restrict__ w, int64_t k,
                                                       const int32_t* __restrict__ crow, int32_t* __restrict__ col,
                                                       uint16_t* __restrict__ values) {
  __shared__ int flag[256];
  __shared__ int pos[256];
  __shared__ int carry;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, t = threadIdx.x;
  const int64_t br = blockIdx.x, nbc = k / BS;
  const int64_t first = crow[br];
  if (t == 0) carry = 0;
  for (int64_t c0 = 0; c0 < nbc; c0 += 256) {
    for (int b = wave; b < 256; b += 4) {
      const bool kept = c0 + b < nbc && block_nonzero(w, k, br, c0 + b, lane);
      if (lane == 0) flag[b] = kept ? 1 : 0;
    }
    __syncthreads();
    pos[t] = flag[t];
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
      const int add = t >= d ? pos[t - d] : 0;
      __syncthreads();
      pos[t] += add;
      __syncthreads();
    }
    for (int b = wave; b < 256; b += 4) {
      if (!flag[b]) continue;
      const int64_t j = first + carry + pos[b] - 1;  // inclusive scan: slot = pos - 1
      const int64_t bc = c0 + b;
      if (lane == 0) col[j] = (int32_t)bc;
      const uint8_t* src = reinterpret_cast<const uint8_t*>(w + (br * BS) * k + bc * BS);
      uint8_t* dst = reinterpret_cast<uint8_t*>(values + j * BS * BS);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 8 * i + (lane >> 3);
        *reinterpret_cast<uint4*>(dst + row * 128 + 16 * (lane & 7)) =
            *reinterpret_cast<const uint4*>(src + (int64_t)row * k * 2 + 16 * (lane & 7));
      }
    }
    __syncthreads();
    if (t == 0) carry += pos[255];
    __syncthreads();
  }
}

// out[m, n] = sum_k x[m, k] W[n, k] (+ bias[n]) for the BSR weight W.
// A workgroup owns 16 output rows n (a quarter of a block row) and 16
// activation rows m (workgroup id / (N / 16)); its NW wavefronts take every
// NW-th kept block of the block row.  Per block, two 16x16x32 bf16 MFMAs: A = the block's 16
// rows, k = 32 s + 8 g .. + 7 for lane group g, B = the activation at the
// block's columns, same k.  Any one-to-one k order works as long as A and B
// use the same one; the 16-byte chunk per lane keeps the loads contiguous.
// Loads of up to U blocks are issued before their MFMAs (the weight blocks'
// with the block-column load, the activation's once the columns are in).  Activation rows >= M read row
// M - 1 (an MFMA output column depends on its own B column only; those
// columns are never stored).  The partial tiles are summed in fixed order.
template <int OUT, int NW, int U>
__global__ __launch_bounds__(64 * NW) void bsr_linear_kernel(const uint16_t* __restrict__ x, int M, int64_t K,
                                                         const int32_t* __restrict__ crow,
                                                         const int32_t* __restrict__ col,
                                                         const uint16_t* __restrict__ values, int64_t N,
                                                         const uint16_t* __restrict__ bias, void* __restrict__ out) {
  __shared__ v4f red[NW][64];
  // each wavefront's U 2 KB block slices (16 rows x 128 bytes), filled by
  // global->LDS loads of whole lines: load h of a slice takes rows 8h..8h+7,
  // lane l the 16-byte chunk (l % 8) ^ (row % 8) of row 8h + l / 8, written
  // at 16 l -- so chunk c of row r sits at chunk c ^ (r % 8), and the
  // operand reads of 8 consecutive rows at one chunk hit distinct banks.
  // (Loaded as MFMA operands straight from memory, each 1 KB load touched
  // 16 half lines.)
  __shared__ __attribute__((aligned(1024))) uint8_t wbuf[NW][U * 2048];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t tiles_n = N / 16;
  const int64_t n0 = ((int64_t)blockIdx.x % tiles_n) * 16, br = n0 / BS, rowoff = n0 % BS;
  const int m0 = (int)((int64_t)blockIdx.x / tiles_n) * 16;
  const int j0 = crow[br], j1 = crow[br + 1];
  const int64_t kmax = K / BS - 1;
  const uint8_t* xrow = reinterpret_cast<const uint8_t*>(x + (int64_t)min(m0 + r16, M - 1) * K) + 16 * g;
  // this lane's part of a slice load, and its operand chunks (step s: k = 32 s + 8 g .. + 7)
  const uint8_t* vload = reinterpret_cast<const uint8_t*>(values) + (rowoff + (lane >> 3)) * (BS * 2) +
                         16 * ((lane & 7) ^ ((lane >> 3) & 7));
  const int a_rd0 = r16 * 128 + 16 * (g ^ (r16 & 7)), a_rd1 = r16 * 128 + 16 * ((4 + g) ^ (r16 & 7));
  uint8_t* const mine = wbuf[wave];
  v4f acc0 = v4f{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  for (int jb = j0 + wave; jb < j1; jb += NW * U) {
    const int live = min(U, (j1 - jb + NW - 1) / NW);  // blocks of this group (uniform)
    v4i a[U][2], b[U][2];
    // the weight slices first: their addresses need the block index only
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u < live) {
        const uint8_t* vb = vload + (int64_t)(jb + NW * u) * (BS * BS * 2);
#pragma unroll
        for (int h = 0; h < 2; ++h)
          __builtin_amdgcn_global_load_lds((void*)(vb + h * 8 * (BS * 2)), (void*)(mine + u * 2048 + h * 1024), 16, 0, 0);
      }
    }
    // then the block columns, as uniform (scalar) loads: waiting for them
    // does not wait for the slices, which stream meanwhile; then the
    // activation at those columns (a corrupt index is clamped so the read
    // stays inside x)
    int64_t bc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) bc[u] = col[__builtin_amdgcn_readfirstlane(jb + NW * min(u, live - 1))];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u < live) {
        const uint8_t* xb = xrow + min((int64_t)(uint32_t)bc[u], kmax) * (BS * 2);
#pragma unroll
        for (int s = 0; s < 2; ++s) b[u][s] = *reinterpret_cast<const v4i*>(xb + 64 * s);
      }
    }
    // every load has landed (the activation loads and the global->LDS ones
    // share the counter); then the slices' operand chunks
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), other counters at maximum (gfx9 encoding)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u < live) {
        a[u][0] = *reinterpret_cast<const v4i*>(mine + u * 2048 + a_rd0);
        a[u][1] = *reinterpret_cast<const v4i*>(mine + u * 2048 + a_rd1);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u < live) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const v8bf av = __builtin_bit_cast(v8bf, a[u][s]);
          const v8bf bv = __builtin_bit_cast(v8bf, b[u][s]);
          if (s) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc1, 0, 0, 0);
          else acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc0, 0, 0, 0);
        }
      }
    }
    // the LDS reads above fed the MFMAs, so the slices are free for the next group
  }
  red[wave][lane] = acc0 + acc1;
  __syncthreads();
  if (wave == 0) {
    v4f t = red[0][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) t += red[w][lane];
    const int64_t n = n0 + 4 * g;
    v4f y = t;
    if (bias) {
      const uint2 b2 = *reinterpret_cast<const uint2*>(bias + n);
      y[0] += bf16_to_f32(b2.x & 0xFFFFu);
      y[1] += bf16_to_f32(b2.x >> 16);
      y[2] += bf16_to_f32(b2.y & 0xFFFFu);
      y[3] += bf16_to_f32(b2.y >> 16);
    }
    const int m = m0 + r16;
    if (m < M) {
      if constexpr (OUT == OUT_BF16) {
        uint16_t* o = reinterpret_cast<uint16_t*>(out) + (int64_t)m * N + n;
        const uint32_t lo = pack_bf16x2(y[0], y[1]);
        const uint32_t hi = pack_bf16x2(y[2], y[3]);
        *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
      } else {
        *reinterpret_cast<v4f*>(reinterpret_cast<float*>(out) + (int64_t)m * N + n) = y;
      }
    }
  }
}

}  // namespace

hipError_t launch_bsr_count(const uint16_t* w, int64_t n, int64_t k, int32_t* crow, hipStream_t stream) {
  const int64_t nbr = n / BS;
  if (nbr > 0) {
    hipLaunchKernelGGL(bsr_count_kernel, dim3((unsigned)nbr), dim3(256), 0, stream, w, k, crow);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bsr_scan_kernel, dim3(1), dim3(1024), 0, stream, crow, nbr);
  return hipGetLastError();
}

hipError_t launch_bsr_fill(const uint16_t* w, int64_t n, int64_t k, const int32_t* crow, int32_t* col,
                           uint16_t* values, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(bsr_fill_kernel, dim3((unsigned)(n / BS)), dim3(256), 0, stream, w, k, crow, col, values);
  return hipGetLastError();
}

hipError_t launch_bsr_linear(const uint16_t* x, int64_t m, int64_t k, const int32_t* crow, const int32_t* col,
                             const uint16_t* values, int64_t n, const uint16_t* bias, void* out, int out_fmt,
                             hipStream_t stream) {
  const dim3 grid((unsigned)((n / 16) * ((m + 15) / 16)));
  // 8 wavefronts of up to 2 blocks per group: at sparsity 0.9 a block row
  // keeps about 6 of 64 blocks, so most wavefronts run one short group and
  // the workgroup's loads all go out at once (measured best or within noise
  // of 1-16 wavefronts and groups of 1-8 blocks on the Llama shapes)
  if (out_fmt == OUT_BF16)
    hipLaunchKernelGGL((bsr_linear_kernel<OUT_BF16, 8, 2>), grid, dim3(512), 0, stream, x, (int)m, k, crow, col,
                       values, n, bias, out);
  else
    hipLaunchKernelGGL((bsr_linear_kernel<OUT_F32, 8, 2>), grid, dim3(512), 0, stream, x, (int)m, k, crow, col,
                       values, n, bias, out);
  return hipGetLastError();
}

}  // namespace sfr
