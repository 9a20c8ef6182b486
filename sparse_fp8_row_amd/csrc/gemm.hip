// Row-wise scaled linear layer with a 2:4 sparse FP8 weight, on gfx950.
//
// Method: pytorch/ao PR #1671 ("Add CUTLASS-based row-wise scaled sparse FP8
// kernel"): out[m, n] = xs[m] * ws[n] * sum_k xq[m, k] * wq[n, k] (+ bias[n]),
// FP8 activation, 2:4 sparse FP8 weight, one kernel instantiation per
// (activation, weight) dtype pair (pytorch/ao issue #3516, file table).  The
// row/column scales and the bias are applied in the epilogue of the same
// kernel, and the result leaves as bf16.
//
// Instruction: V_SMFMAC_F32_16X16X128_{FP8,BF8}_{FP8,BF8}.  The sparse A
// operand is the compressed weight (16 output rows, 128 dense k per
// instruction, 64 kept bytes per row plus 2-bit positions), the dense B
// operand is the activation transposed (16 tokens x 128 k), so one
// instruction computes a 16(n) x 16(m) block of out^T.  The weight's 4-bit
// group nibbles (i0 | i1 << 2, eight groups per 32-bit word) are exactly the
// instruction's index operand, so metadata goes from memory to the matrix core
// untouched.  Each lane of a D block holds four consecutive n of one m, which
// is what a row-major [M, N] output wants: 8-byte bf16 stores.
//
// Two kernels:
//  * tiled:  a workgroup computes a BN x BM tile of out^T.  Per 128-wide k step
//    it stages BN rows of compressed weight (64 B values + 16 B metadata per
//    row) and BM rows of activation (128 B per row) in LDS, double-buffered:
//    the global loads of step k+1 are in flight while the MFMAs of step k run.
//    LDS rows are XOR-swizzled in 16-byte chunks so that the 16 lanes of a
//    quarter-wave read 16 different 16-byte bank groups.  Tiles are assigned so
//    that each XCD (workgroup id mod 8) works on one contiguous run of tiles,
//    walked in groups of G n-tiles, which keeps the weight and activation
//    panels that neighbouring workgroups share in that XCD's L2.
//  * decode: for M <= 16, where the weight read is everything.  A workgroup
//    owns 16 weight rows; its eight wavefronts split the k steps between them,
//    stream the compressed weight straight from HBM into registers (no LDS
//    staging: every byte is used by exactly one instruction), and reduce
//    their partial 16x16 sums through LDS in a fixed order (deterministic).
//    Tokens beyond M are zero columns of B, the padding-to-16 idea of
//    pytorch/ao PR #1734 ("promote blocksparse from prototype ...").
#include "sfr_device.hpp"
#include "sfr_launch.hpp"

namespace sfr {
namespace {

constexpr int KSTEP = 128;  // dense k per MFMA and per pipeline stage

template <int OUT>
__device__ __forceinline__ void store4(void* out, int64_t ld, int64_t m, int64_t n, v4f y) {
  if constexpr (OUT == OUT_BF16) {
    uint16_t* o = reinterpret_cast<uint16_t*>(out) + m * ld + n;
    const uint32_t lo = f32_to_bf16_rne(y[0]) | (f32_to_bf16_rne(y[1]) << 16);
    const uint32_t hi = f32_to_bf16_rne(y[2]) | (f32_to_bf16_rne(y[3]) << 16);
    *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
  } else {
    float* o = reinterpret_cast<float*>(out) + m * ld + n;
    *reinterpret_cast<v4f*>(o) = y;
  }
}

// y = acc * (xs * ws) (+ bias), binary32.
__device__ __forceinline__ v4f epilogue4(v4f acc, float xsm, const float* __restrict__ ws,
                                         const uint16_t* __restrict__ bias, int64_t n) {
  const v4f w4 = *reinterpret_cast<const v4f*>(ws + n);
  v4f y;
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = acc[i] * (xsm * w4[i]);
  if (bias) {
    const uint2 b = *reinterpret_cast<const uint2*>(bias + n);
    y[0] += bf16_to_f32(b.x & 0xFFFFu);
    y[1] += bf16_to_f32(b.x >> 16);
    y[2] += bf16_to_f32(b.y & 0xFFFFu);
    y[3] += bf16_to_f32(b.y >> 16);
  }
  return y;
}

// ---------------------------------------------------------------------------
// Tiled kernel
// ---------------------------------------------------------------------------
template <int XF, int WF, int OUT, int BN, int BM, int WN, int WM, int G>
struct Tiled {
  static constexpr int NT = 64 * WN * WM;
  static constexpr int TN = BN / WN, TM = BM / WM;  // wavefront tile
  static constexpr int FN = TN / 16, FM = TM / 16;  // 16x16 blocks per wavefront
  static constexpr int W_BYTES = BN * 64, META_BYTES = BN * 16, X_BYTES = BM * 128;
  static constexpr int STAGE = W_BYTES + META_BYTES + X_BYTES;
  static constexpr int LDS = 2 * STAGE;
  // 16-byte chunks per stage and per thread
  static constexpr int W_CH = BN * 4, M_CH = BN, X_CH = BM * 8;
  static constexpr int W_PT = (W_CH + NT - 1) / NT, M_PT = (M_CH + NT - 1) / NT, X_PT = (X_CH + NT - 1) / NT;
  static_assert(BN % (16 * WN) == 0 && BM % (16 * WM) == 0, "tile");
  static_assert(W_CH % NT == 0 || W_PT == 1, "weight chunks");
  static_assert(X_CH % NT == 0, "activation chunks");
};

template <int XF, int WF, int OUT, int BN, int BM, int WN, int WM, int G>
__global__ __launch_bounds__(64 * WN * WM) void linear_tiled_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xs, const uint8_t* __restrict__ values,
    const uint8_t* __restrict__ meta, const float* __restrict__ ws, const uint16_t* __restrict__ bias,
    void* __restrict__ out, int M, int N, int K, int tiles_m, int tiles_n) {
  using C = Tiled<XF, WF, OUT, BN, BM, WN, WM, G>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  // ---- tile assignment: contiguous runs per XCD, grouped along n ----
  const int T = tiles_m * tiles_n;
  const int per_xcd = (T + 7) / 8;
  const int lid = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (lid >= T) return;
  const int group = lid / (G * tiles_m);
  const int first_n = group * G;
  const int gsize = min(tiles_n - first_n, G);
  const int within = lid - group * G * tiles_m;
  const int tn = first_n + within % gsize;
  const int tm = within / gsize;
  const int n0 = tn * BN, m0 = tm * BM;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave / WM, wm = wave % WM;
  const int r16 = lane & 15, lg = lane >> 4;

  const int64_t ldv = K / 2, ldm = K / 8, ldx = K;

  // ---- global -> register staging addresses (rows clamped into range) ----
  const uint8_t* gw[C::W_PT];
  int sw_off[C::W_PT];
  bool w_on[C::W_PT];
#pragma unroll
  for (int i = 0; i < C::W_PT; ++i) {
    const int c = tid + i * C::NT;
    w_on[i] = c < C::W_CH;
    const int r = (c >> 2) % BN, j = c & 3;
    const int64_t row = min(n0 + r, N - 1);
    gw[i] = values + row * ldv + 16 * j;
    sw_off[i] = r * 64 + 16 * (j ^ ((r >> 2) & 3));
  }
  const uint8_t* gm[C::M_PT];
  int sm_off[C::M_PT];
  bool m_on[C::M_PT];
#pragma unroll
  for (int i = 0; i < C::M_PT; ++i) {
    const int r = tid + i * C::NT;
    m_on[i] = r < C::M_CH;
    const int64_t row = min(n0 + (r % BN), N - 1);
    gm[i] = meta + row * ldm;
    sm_off[i] = C::W_BYTES + (r % BN) * 16;
  }
  const uint8_t* gx[C::X_PT];
  int sx_off[C::X_PT];
#pragma unroll
  for (int i = 0; i < C::X_PT; ++i) {
    const int c = tid + i * C::NT;
    const int r = c >> 3, j = c & 7;
    const int64_t row = min(m0 + r, M - 1);
    gx[i] = xq + row * ldx + 16 * j;
    sx_off[i] = C::W_BYTES + C::META_BYTES + r * 128 + 16 * (j ^ ((r >> 1) & 7));
  }

  uint4 rw[C::W_PT], rm[C::M_PT], rx[C::X_PT];
  auto gload = [&](int kt) {
    const int64_t kb = (int64_t)kt * KSTEP;
#pragma unroll
    for (int i = 0; i < C::W_PT; ++i)
      if (w_on[i]) rw[i] = *reinterpret_cast<const uint4*>(gw[i] + kb / 2);
#pragma unroll
    for (int i = 0; i < C::M_PT; ++i)
      if (m_on[i]) rm[i] = *reinterpret_cast<const uint4*>(gm[i] + kb / 8);
#pragma unroll
    for (int i = 0; i < C::X_PT; ++i) rx[i] = *reinterpret_cast<const uint4*>(gx[i] + kb);
  };
  auto sstore = [&](int stage) {
    uint8_t* base = smem + stage * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::W_PT; ++i)
      if (w_on[i]) *reinterpret_cast<uint4*>(base + sw_off[i]) = rw[i];
#pragma unroll
    for (int i = 0; i < C::M_PT; ++i)
      if (m_on[i]) *reinterpret_cast<uint4*>(base + sm_off[i]) = rm[i];
#pragma unroll
    for (int i = 0; i < C::X_PT; ++i) *reinterpret_cast<uint4*>(base + sx_off[i]) = rx[i];
  };

  // ---- LDS read offsets of this lane's MFMA operands ----
  int a_off[C::FN], i_off[C::FN], b_off0[C::FM], b_off1[C::FM];
#pragma unroll
  for (int f = 0; f < C::FN; ++f) {
    const int r = wn * C::TN + f * 16 + r16;
    a_off[f] = r * 64 + 16 * (lg ^ ((r >> 2) & 3));
    i_off[f] = C::W_BYTES + r * 16 + 4 * lg;
  }
#pragma unroll
  for (int f = 0; f < C::FM; ++f) {
    const int r = wm * C::TM + f * 16 + r16;
    const int sw = (r >> 1) & 7;
    b_off0[f] = C::W_BYTES + C::META_BYTES + r * 128 + 16 * (lg ^ sw);
    b_off1[f] = C::W_BYTES + C::META_BYTES + r * 128 + 16 * ((4 + lg) ^ sw);
  }

  v4f acc[C::FN][C::FM];
#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int KT = K / KSTEP;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const uint8_t* base = smem + cur * C::STAGE;
    v8i b[C::FM];
#pragma unroll
    for (int f = 0; f < C::FM; ++f) {
      const v4i lo = *reinterpret_cast<const v4i*>(base + b_off0[f]);
      const v4i hi = *reinterpret_cast<const v4i*>(base + b_off1[f]);
      b[f] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const v4i a = *reinterpret_cast<const v4i*>(base + a_off[fn]);
      const int idx = *reinterpret_cast<const int*>(base + i_off[fn]);
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) acc[fn][fm] = smfmac16<XF, WF>(a, b[fm], acc[fn][fm], idx);
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: scales, bias, bf16, store ----
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int m = m0 + wm * C::TM + fm * 16 + r16;
    if (m >= M) continue;
    const float xsm = xs[m];
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int n = n0 + wn * C::TN + fn * 16 + 4 * lg;
      if (n >= N) continue;
      store4<OUT>(out, N, m, n, epilogue4(acc[fn][fm], xsm, ws, bias, n));
    }
  }
}

// ---------------------------------------------------------------------------
// Decode kernel (M <= 16)
// ---------------------------------------------------------------------------
constexpr int DEC_WAVES = 8;
constexpr int DEC_UNROLL = 4;

template <int XF, int WF, int OUT>
__global__ __launch_bounds__(64 * DEC_WAVES) void linear_decode_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xs, const uint8_t* __restrict__ values,
    const uint8_t* __restrict__ meta, const float* __restrict__ ws, const uint16_t* __restrict__ bias,
    void* __restrict__ out, int M, int N, int K) {
  __shared__ v4f red[DEC_WAVES][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int KT = K / KSTEP;

  const uint8_t* vrow = values + (int64_t)(n0 + r16) * (K / 2) + 16 * lg;
  const uint8_t* mrow = meta + (int64_t)(n0 + r16) * (K / 8) + 4 * lg;
  const bool xon = r16 < M;
  const uint8_t* xrow = xq + (int64_t)min(r16, M - 1) * K + 16 * lg;

  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  for (int s0 = wave; s0 < KT; s0 += DEC_WAVES * DEC_UNROLL) {
    v4i a[DEC_UNROLL];
    int idx[DEC_UNROLL];
    v8i b[DEC_UNROLL];
#pragma unroll
    for (int u = 0; u < DEC_UNROLL; ++u) {
      const int s = s0 + u * DEC_WAVES;
      if (s < KT) {
        a[u] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(vrow + (int64_t)s * 64));
        idx[u] = __builtin_nontemporal_load(reinterpret_cast<const int*>(mrow + (int64_t)s * 16));
        if (xon) {
          const v4i lo = *reinterpret_cast<const v4i*>(xrow + (int64_t)s * 128);
          const v4i hi = *reinterpret_cast<const v4i*>(xrow + (int64_t)s * 128 + 64);
          b[u] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
          b[u] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        }
      }
    }
#pragma unroll
    for (int u = 0; u < DEC_UNROLL; ++u)
      if (s0 + u * DEC_WAVES < KT) acc = smfmac16<XF, WF>(a[u], b[u], acc, idx[u]);
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    v4f t = red[0][lane];
#pragma unroll
    for (int w = 1; w < DEC_WAVES; ++w) t += red[w][lane];
    const int m = r16;
    const int n = n0 + 4 * lg;
    if (m < M) store4<OUT>(out, N, m, n, epilogue4(t, xs[m], ws, bias, n));
  }
}

// ---------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------
template <int XF, int WF, int OUT, int BN, int BM, int WN, int WM, int G>
hipError_t run_tiled(const LinearArgs& a, hipStream_t stream) {
  using C = Tiled<XF, WF, OUT, BN, BM, WN, WM, G>;
  const int tiles_m = (int)((a.m + BM - 1) / BM), tiles_n = (int)((a.n + BN - 1) / BN);
  const int T = tiles_m * tiles_n;
  const int grid = 8 * ((T + 7) / 8);
  auto kern = linear_tiled_kernel<XF, WF, OUT, BN, BM, WN, WM, G>;
  static bool attr_set = false;  // benign race: every thread sets the same value
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), C::LDS, stream, a.xq, a.xs, a.values, a.meta, a.ws,
                     a.bias, a.out, (int)a.m, (int)a.n, (int)a.k, tiles_m, tiles_n);
  return hipGetLastError();
}

template <int XF, int WF, int OUT>
hipError_t run_linear(const LinearArgs& a, hipStream_t stream) {
  if (a.m <= 16) {
    hipLaunchKernelGGL((linear_decode_kernel<XF, WF, OUT>), dim3((unsigned)(a.n / 16)), dim3(64 * DEC_WAVES), 0,
                       stream, a.xq, a.xs, a.values, a.meta, a.ws, a.bias, a.out, (int)a.m, (int)a.n, (int)a.k);
    return hipGetLastError();
  }
  const int64_t big = ((a.m + 255) / 256) * ((a.n + 255) / 256);
  const int64_t mid = ((a.m + 127) / 128) * ((a.n + 127) / 128);
  if (big >= 512) return run_tiled<XF, WF, OUT, 256, 256, 2, 4, 8>(a, stream);
  if (mid >= 256) return run_tiled<XF, WF, OUT, 128, 128, 2, 2, 8>(a, stream);
  return run_tiled<XF, WF, OUT, 64, 64, 2, 2, 8>(a, stream);
}

template <int XF, int WF>
hipError_t run_out(const LinearArgs& a, hipStream_t stream) {
  if (a.out_fmt == OUT_BF16) return run_linear<XF, WF, OUT_BF16>(a, stream);
  return run_linear<XF, WF, OUT_F32>(a, stream);
}

}  // namespace

hipError_t launch_linear(const LinearArgs& a, hipStream_t stream) {
  if (a.x_fmt == FMT_E4M3 && a.w_fmt == FMT_E4M3) return run_out<FMT_E4M3, FMT_E4M3>(a, stream);
  if (a.x_fmt == FMT_E4M3 && a.w_fmt == FMT_E5M2) return run_out<FMT_E4M3, FMT_E5M2>(a, stream);
  if (a.x_fmt == FMT_E5M2 && a.w_fmt == FMT_E4M3) return run_out<FMT_E5M2, FMT_E4M3>(a, stream);
  return run_out<FMT_E5M2, FMT_E5M2>(a, stream);
}

}  // namespace sfr
