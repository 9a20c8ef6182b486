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

hipError_t launch_compress(const uint8_t* w, int64_t n, int64_t k, uint8_t* values, uint8_t* meta,
                           hipStream_t stream);

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

// Row-wise quantization of x into (xq, xs) and the linear layer on them (a's
// xq / xs are ignored): one fused launch for small decode shapes, else two.
hipError_t launch_linear_dynamic(const uint16_t* x, uint8_t* xq, float* xs, const LinearArgs& a,
                                 hipStream_t stream);

}  // namespace sfr
