// Host-side launchers of the gfx950 kernels (internal; the C ABI validates
// arguments before calling these).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfr {

hipError_t launch_quantize(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* q,
                           float* scale, hipStream_t stream);

// Tensor-wise quantization: workspace of tensor_workspace_bytes(rows, cols).
int64_t tensor_workspace_bytes(int64_t rows, int64_t cols);
hipError_t launch_quantize_tensor(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* q, float* scale,
                                  void* workspace, hipStream_t stream);
// The same on the library's own per-device workspace of noalloc_workspace_bytes().
int64_t noalloc_workspace_bytes();
hipError_t launch_quantize_tensor_noalloc(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* q,
                                          float* scale, hipStream_t stream);

hipError_t launch_compress(const uint8_t* w, int64_t n, int64_t k, uint8_t* values, uint8_t* meta,
                           hipStream_t stream);

// 2:4 pruning of a bf16 matrix (k % 8 == 0); out may be w.
hipError_t launch_prune_bf16(const uint16_t* w, int64_t n, int64_t k, uint16_t* out, hipStream_t stream);

struct LinearArgs {
  const uint8_t* xq;
  const float* xs;
  const uint8_t* values;
  const uint8_t* meta;
  const float* ws;
  const uint16_t* bias;  // may be null
  void* out;
  int64_t m, n, k;
  int x_fmt, w_fmt, out_fmt;
  int xs_stride, ws_stride;  // 1: one scale per row; 0: one scale for the operand
};

hipError_t launch_linear(const LinearArgs& a, hipStream_t stream);

// Kernel configurations of the linear layer.  algo < 0: the built-in choice.
enum LinearAlgo {
  ALGO_DECODE_LDS = 0,     // m <= 16, k % 1024 == 0: 16 weight rows per workgroup, one 1024-k unit per wavefront via LDS
  ALGO_DECODE_REG = 1,     // m <= 16: 16 weight rows per workgroup, streamed to registers
  ALGO_TILED_64 = 2,       // 64 x 64 tiles, 4 wavefronts
  ALGO_TILED_128 = 3,      // 128 x 128 tiles, 4 wavefronts
  ALGO_TILED_256 = 4,      // 256 x 256 tiles, 8 wavefronts
  ALGO_WIDE_256 = 5,       // 256 x 256 tiles, 4 software-pipelined wavefronts (k >= 512)
  ALGO_DECODE_LDS_32 = 6,  // as ALGO_DECODE_LDS with 32 weight rows per workgroup (n % 32 == 0)
  ALGO_TILED_256x128 = 7,  // 256 (n) x 128 (m) tiles, 8 wavefronts, one workgroup per CU
  ALGO_COUNT = 8
};
// Flag of an algorithm id: FP8 matrix-instruction accumulation (products of
// one instruction added 13 bits below the largest) instead of the default
// binary32-grade accumulation on exactly widened operands.
constexpr int ALGO_ACC_F8_FLAG = 0x100;
bool linear_algo_valid(int algo);
const char* linear_algo_name(int algo);
bool linear_algo_supported(int algo, int64_t m, int64_t n, int64_t k);
int linear_default_algo(int64_t m, int64_t n, int64_t k);
hipError_t launch_linear_algo(const LinearArgs& a, int algo, hipStream_t stream);

// Row-wise quantization of x into (xq, xs) and the linear layer on them (a's
// xq / xs are ignored) with algorithm `algo` (< 0: the built-in choice): one
// fused launch for small decode shapes on the built-in configuration, else two.
hipError_t launch_linear_dynamic(const uint16_t* x, uint8_t* xq, float* xs, const LinearArgs& a, int algo,
                                 hipStream_t stream);

// Block-sparse (BSR, 64 x 64 blocks) bf16 weight.
hipError_t launch_bsr_count(const uint16_t* w, int64_t n, int64_t k, int32_t* crow, hipStream_t stream);
hipError_t launch_bsr_fill(const uint16_t* w, int64_t n, int64_t k, const int32_t* crow, int32_t* col,
                           uint16_t* values, hipStream_t stream);
hipError_t launch_bsr_linear(const uint16_t* x, int64_t m, int64_t k, const int32_t* crow, const int32_t* col,
                             const uint16_t* values, int64_t n, const uint16_t* bias, void* out, int out_fmt,
                             hipStream_t stream);

}  // namespace sfr
