// C ABI of the sparse FP8 row-wise linear layer: argument validation and
// dispatch to the gfx950 kernels.  The contract of every entry point is
// documented in include/sparse_fp8_row.h.
#include "sparse_fp8_row.h"

#include "sfr_launch.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool fp8_ok(int dt) { return dt == SFR_E4M3 || dt == SFR_E5M2; }
bool scale_ok(int kind) { return kind == SFR_SCALE_ROW || kind == SFR_SCALE_TENSOR; }
// Bound on rows * cols of any one tensor, keeping every grid within HIP's limits.
constexpr int64_t kMaxElems = (int64_t)1 << 40;

sfr_status launch_status(hipError_t e) { return e == hipSuccess ? SFR_OK : SFR_ERR_LAUNCH; }

}  // namespace

extern "C" {

sfr_status quantize_rowwise_fp8(const uint16_t* x, int64_t rows, int64_t cols, sfr_fp8_t dt, uint8_t* q,
                                float* scale, void* stream) {
  if (!fp8_ok(dt)) return SFR_ERR_DTYPE;
  if (rows < 0 || rows > SFR_MAX_DIM || cols <= 0 || cols > SFR_MAX_DIM || cols % 8 != 0 ||
      rows * cols > kMaxElems)
    return SFR_ERR_SHAPE;
  if (rows == 0) return SFR_OK;
  if (!x || !q || !scale) return SFR_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || !aligned16(scale)) return SFR_ERR_ALIGN;
  return launch_status(sfr::launch_quantize(x, rows, cols, dt, q, scale, static_cast<hipStream_t>(stream)));
}

int64_t sfr_quantize_tensorwise_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || rows > SFR_MAX_DIM || cols <= 0 || cols > SFR_MAX_DIM || cols % 8 != 0 || rows * cols > kMaxElems)
    return 0;
  return sfr::tensor_workspace_bytes(rows, cols);
}

sfr_status quantize_tensorwise_fp8(const uint16_t* x, int64_t rows, int64_t cols, sfr_fp8_t dt, uint8_t* q,
                                   float* scale, void* workspace, int64_t workspace_bytes, void* stream) {
  if (!fp8_ok(dt)) return SFR_ERR_DTYPE;
  if (rows < 0 || rows > SFR_MAX_DIM || cols <= 0 || cols > SFR_MAX_DIM || cols % 8 != 0 ||
      rows * cols > kMaxElems)
    return SFR_ERR_SHAPE;
  if (rows == 0) return SFR_OK;
  if (workspace_bytes < sfr::tensor_workspace_bytes(rows, cols)) return SFR_ERR_SHAPE;
  if (!x || !q || !scale || !workspace) return SFR_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || !aligned16(scale) || !aligned16(workspace)) return SFR_ERR_ALIGN;
  return launch_status(
      sfr::launch_quantize_tensor(x, rows, cols, dt, q, scale, workspace, static_cast<hipStream_t>(stream)));
}

sfr_status quantize_tensorwise_fp8_noalloc(const uint16_t* x, int64_t rows, int64_t cols, sfr_fp8_t dt, uint8_t* q,
                                           float* scale, void* stream) {
  if (!fp8_ok(dt)) return SFR_ERR_DTYPE;
  if (rows < 0 || rows > SFR_MAX_DIM || cols <= 0 || cols > SFR_MAX_DIM || cols % 8 != 0 ||
      rows * cols > kMaxElems)
    return SFR_ERR_SHAPE;
  if (rows == 0) return SFR_OK;
  if (sfr::tensor_workspace_bytes(rows, cols) > sfr::noalloc_workspace_bytes()) return SFR_ERR_SHAPE;
  if (!x || !q || !scale) return SFR_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || !aligned16(scale)) return SFR_ERR_ALIGN;
  return launch_status(
      sfr::launch_quantize_tensor_noalloc(x, rows, cols, dt, q, scale, static_cast<hipStream_t>(stream)));
}

sfr_status compress_2to4_fp8(const uint8_t* w, int64_t n, int64_t k, sfr_fp8_t dt, uint8_t* values, uint8_t* meta,
                             void* stream) {
  if (!fp8_ok(dt)) return SFR_ERR_DTYPE;
  if (n < 0 || n > SFR_MAX_DIM || k <= 0 || k > SFR_MAX_DIM || k % 128 != 0 || n * k > kMaxElems)
    return SFR_ERR_SHAPE;
  if (n == 0) return SFR_OK;
  if (!w || !values || !meta) return SFR_ERR_NULL;
  if (!aligned16(w) || !aligned16(values) || !aligned16(meta)) return SFR_ERR_ALIGN;
  return launch_status(sfr::launch_compress(w, n, k, values, meta, static_cast<hipStream_t>(stream)));
}

sfr_status prune_2to4_bf16(const uint16_t* w, int64_t n, int64_t k, uint16_t* out, void* stream) {
  if (n < 0 || n > SFR_MAX_DIM || k <= 0 || k > SFR_MAX_DIM || k % 8 != 0 || n * k > kMaxElems)
    return SFR_ERR_SHAPE;
  if (n == 0) return SFR_OK;
  if (!w || !out) return SFR_ERR_NULL;
  if (!aligned16(w) || !aligned16(out)) return SFR_ERR_ALIGN;
  return launch_status(sfr::launch_prune_bf16(w, n, k, out, static_cast<hipStream_t>(stream)));
}

int sfr_linear_algo_count(void) { return sfr::ALGO_COUNT; }

int sfr_linear_algo_valid(int algo) { return sfr::linear_algo_valid(algo) ? 1 : 0; }

const char* sfr_linear_algo_name(int algo) { return sfr::linear_algo_name(algo); }

int sfr_linear_algo_supported(int algo, int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || n % 16 != 0 || k <= 0 || k % 128 != 0) return 0;
  return sfr::linear_algo_supported(algo, m, n, k) ? 1 : 0;
}

int sfr_linear_default_algo(int64_t m, int64_t n, int64_t k) { return sfr::linear_default_algo(m, n, k); }

sfr_status sparse_fp8_scaled_linear_algo(const uint8_t* xq, sfr_fp8_t x_dt, const float* xs, sfr_scale_t xs_kind,
                                         int64_t m, int64_t k, const uint8_t* values, const uint8_t* meta,
                                         sfr_fp8_t w_dt, const float* ws, sfr_scale_t ws_kind, int64_t n,
                                         const uint16_t* bias, void* out, sfr_out_t out_dt, int algo,
                                         void* stream) {
  if (!fp8_ok(x_dt) || !fp8_ok(w_dt) || (out_dt != SFR_OUT_BF16 && out_dt != SFR_OUT_F32) || !scale_ok(xs_kind) ||
      !scale_ok(ws_kind) || (algo != SFR_ALGO_DEFAULT && !sfr::linear_algo_valid(algo)))
    return SFR_ERR_DTYPE;
  if (m < 0 || m > SFR_MAX_DIM || n < 0 || n > SFR_MAX_DIM || n % 16 != 0 || k <= 0 || k > SFR_MAX_DIM ||
      k % 128 != 0 || m * k > kMaxElems || n * k > kMaxElems || m * n > kMaxElems)
    return SFR_ERR_SHAPE;
  if (m == 0 || n == 0) return SFR_OK;
  if (algo != SFR_ALGO_DEFAULT && !sfr::linear_algo_supported(algo, m, n, k)) return SFR_ERR_SHAPE;
  if (!xq || !xs || !values || !meta || !ws || !out) return SFR_ERR_NULL;
  if (!aligned16(xq) || !aligned16(xs) || !aligned16(values) || !aligned16(meta) || !aligned16(ws) ||
      !aligned16(out) || (bias && !aligned16(bias)))
    return SFR_ERR_ALIGN;
  sfr::LinearArgs a{xq, xs, values, meta, ws, bias, out, m, n, k, (int)x_dt, (int)w_dt, (int)out_dt,
                    xs_kind == SFR_SCALE_ROW ? 1 : 0, ws_kind == SFR_SCALE_ROW ? 1 : 0};
  return launch_status(sfr::launch_linear_algo(a, algo, static_cast<hipStream_t>(stream)));
}

sfr_status sparse_fp8_scaled_linear(const uint8_t* xq, sfr_fp8_t x_dt, const float* xs, sfr_scale_t xs_kind, int64_t m,
                                    int64_t k, const uint8_t* values, const uint8_t* meta, sfr_fp8_t w_dt,
                                    const float* ws, sfr_scale_t ws_kind, int64_t n, const uint16_t* bias, void* out,
                                    sfr_out_t out_dt, void* stream) {
  return sparse_fp8_scaled_linear_algo(xq, x_dt, xs, xs_kind, m, k, values, meta, w_dt, ws, ws_kind, n, bias, out,
                                       out_dt, SFR_ALGO_DEFAULT, stream);
}

sfr_status sparse_fp8_rowwise_linear_dynamic_algo(const uint16_t* x, sfr_fp8_t x_dt, int64_t m, int64_t k,
                                                  const uint8_t* values, const uint8_t* meta, sfr_fp8_t w_dt,
                                                  const float* ws, sfr_scale_t ws_kind, int64_t n,
                                                  const uint16_t* bias, void* out, sfr_out_t out_dt, uint8_t* xq,
                                                  float* xs, int algo, void* stream) {
  if (!fp8_ok(x_dt) || !fp8_ok(w_dt) || (out_dt != SFR_OUT_BF16 && out_dt != SFR_OUT_F32) || !scale_ok(ws_kind) ||
      (algo != SFR_ALGO_DEFAULT && !sfr::linear_algo_valid(algo)))
    return SFR_ERR_DTYPE;
  if (m < 0 || m > SFR_MAX_DIM || n < 0 || n > SFR_MAX_DIM || n % 16 != 0 || k <= 0 || k > SFR_MAX_DIM ||
      k % 128 != 0 || m * k > kMaxElems || n * k > kMaxElems || m * n > kMaxElems)
    return SFR_ERR_SHAPE;
  if (m == 0 || n == 0) return SFR_OK;
  if (algo != SFR_ALGO_DEFAULT && !sfr::linear_algo_supported(algo, m, n, k)) return SFR_ERR_SHAPE;
  if (!x || !values || !meta || !ws || !out || !xq || !xs) return SFR_ERR_NULL;
  if (!aligned16(x) || !aligned16(values) || !aligned16(meta) || !aligned16(ws) || !aligned16(out) ||
      !aligned16(xq) || !aligned16(xs) || (bias && !aligned16(bias)))
    return SFR_ERR_ALIGN;
  sfr::LinearArgs a{xq, xs, values, meta, ws, bias, out, m, n, k, (int)x_dt, (int)w_dt, (int)out_dt, 1,
                    ws_kind == SFR_SCALE_ROW ? 1 : 0};
  return launch_status(sfr::launch_linear_dynamic(x, xq, xs, a, algo, static_cast<hipStream_t>(stream)));
}

sfr_status sparse_fp8_rowwise_linear_dynamic(const uint16_t* x, sfr_fp8_t x_dt, int64_t m, int64_t k,
                                             const uint8_t* values, const uint8_t* meta, sfr_fp8_t w_dt,
                                             const float* ws, sfr_scale_t ws_kind, int64_t n, const uint16_t* bias,
                                             void* out, sfr_out_t out_dt, uint8_t* xq, float* xs, void* stream) {
  return sparse_fp8_rowwise_linear_dynamic_algo(x, x_dt, m, k, values, meta, w_dt, ws, ws_kind, n, bias, out, out_dt,
                                                xq, xs, SFR_ALGO_DEFAULT, stream);
}

sfr_status sparse_fp8_rowwise_linear(const uint8_t* xq, sfr_fp8_t x_dt, const float* xs, int64_t m, int64_t k,
                                     const uint8_t* values, const uint8_t* meta, sfr_fp8_t w_dt, const float* ws,
                                     int64_t n, const uint16_t* bias, void* out, sfr_out_t out_dt, void* stream) {
  return sparse_fp8_scaled_linear(xq, x_dt, xs, SFR_SCALE_ROW, m, k, values, meta, w_dt, ws, SFR_SCALE_ROW, n, bias,
                                  out, out_dt, stream);
}

sfr_status bsr_count_bf16(const uint16_t* w, int64_t n, int64_t k, int32_t* crow, void* stream) {
  if (n < 0 || n > SFR_MAX_DIM || n % SFR_BSR_BLOCK != 0 || k <= 0 || k > SFR_MAX_DIM || k % SFR_BSR_BLOCK != 0 ||
      n * k > kMaxElems)
    return SFR_ERR_SHAPE;
  if (!crow || (n > 0 && !w)) return SFR_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(crow) & 3u) || (w && !aligned16(w))) return SFR_ERR_ALIGN;
  return launch_status(sfr::launch_bsr_count(w, n, k, crow, static_cast<hipStream_t>(stream)));
}

sfr_status bsr_fill_bf16(const uint16_t* w, int64_t n, int64_t k, const int32_t* crow, int32_t* col,
                         uint16_t* values, void* stream) {
  if (n < 0 || n > SFR_MAX_DIM || n % SFR_BSR_BLOCK != 0 || k <= 0 || k > SFR_MAX_DIM || k % SFR_BSR_BLOCK != 0 ||
      n * k > kMaxElems)
    return SFR_ERR_SHAPE;
  if (n == 0) return SFR_OK;
  if (!w || !crow) return SFR_ERR_NULL;
  if (!aligned16(w) || (reinterpret_cast<uintptr_t>(crow) & 3u) || (reinterpret_cast<uintptr_t>(col) & 3u) ||
      (values && !aligned16(values)))
    return SFR_ERR_ALIGN;
  return launch_status(sfr::launch_bsr_fill(w, n, k, crow, col, values, static_cast<hipStream_t>(stream)));
}

sfr_status bsr_linear_bf16(const uint16_t* x, int64_t m, int64_t k, const int32_t* crow, const int32_t* col,
                           const uint16_t* values, int64_t n, const uint16_t* bias, void* out, sfr_out_t out_dt,
                           void* stream) {
  if (out_dt != SFR_OUT_BF16 && out_dt != SFR_OUT_F32) return SFR_ERR_DTYPE;
  if (m < 0 || m > SFR_MAX_DIM || n < 0 || n > SFR_MAX_DIM || n % SFR_BSR_BLOCK != 0 || k <= 0 ||
      k > SFR_MAX_DIM || k % SFR_BSR_BLOCK != 0 || m * k > kMaxElems || n * k > kMaxElems || m * n > kMaxElems ||
      (n / 16) * ((m + 15) / 16) > INT32_MAX)
    return SFR_ERR_SHAPE;
  if (m == 0 || n == 0) return SFR_OK;
  if (!x || !crow || !out) return SFR_ERR_NULL;
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(crow) & 3u) || (reinterpret_cast<uintptr_t>(col) & 3u) ||
      (values && !aligned16(values)) || !aligned16(out) || (bias && !aligned16(bias)))
    return SFR_ERR_ALIGN;
  return launch_status(sfr::launch_bsr_linear(x, m, k, crow, col, values, n, bias, out, (int)out_dt,
                                              static_cast<hipStream_t>(stream)));
}

const char* sfr_status_string(sfr_status s) {
  switch (s) {
    case SFR_OK: return "ok";
    case SFR_ERR_NULL: return "null pointer";
    case SFR_ERR_SHAPE: return "invalid shape";
    case SFR_ERR_ALIGN: return "pointer not 16-byte aligned";
    case SFR_ERR_DTYPE: return "invalid dtype";
    case SFR_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

int sfr_format_version(void) { return SFR_FORMAT_VERSION; }

}  // extern "C"
