// Row-wise scaled linear layer with a 2:4 sparse FP8 weight, on gfx950.
//
// Method: pytorch/ao PR #1671 ("Add CUTLASS-based row-wise scaled sparse FP8
// kernel"): out[m, n] = xs[m] * ws[n] * sum_k xq[m, k] * wq[n, k] (+ bias[n]),
// FP8 activation, 2:4 sparse FP8 weight, one kernel instantiation per
// (activation, weight) dtype pair (pytorch/ao issue #3516, file table).  The
// row/column scales and the bias are applied in the epilogue of the same
// kernel, and the result leaves as bf16.
//
// Instructions: V_SMFMAC_F32_16X16X128_{FP8,BF8}_{FP8,BF8}.  The sparse A
// operand is the compressed weight (16 output rows, 128 dense k per
// instruction, 64 kept bytes per row plus 2-bit positions), the dense B
// operand is the activation transposed (16 tokens x 128 k), so one
// instruction computes a 16(n) x 16(m) block of out^T.  The weight's 4-bit
// group nibbles (i0 | i1 << 2, eight groups per 32-bit word) are exactly the
// instruction's index operand, so metadata goes from memory to the matrix core
// untouched.  Each lane of a D block holds four consecutive n of one m, which
// is what a row-major [M, N] output wants: 8-byte bf16 stores.
//
// Accumulation (template parameter ACC).  The FP8 instruction adds the
// products of one instruction in fixed point 13 bits below the largest of
// them, which is outside the layer's binary32 accuracy on cancelling inputs,
// so by default (ACC_F32) each 128-k step runs as two
// V_SMFMAC_F32_16X16X64_BF16 instructions on operands widened exactly to
// bf16 (sfr_device.hpp, mma_step); ACC_F8 (algorithm ids with the FP8
// accumulation flag) runs the FP8 instruction.  Same layouts, same loads.
//
// Kernels:
//  * tiled (linear_tiled_kernel): a workgroup computes a BN x BM tile of
//    out^T.  Per 128-wide k step it stages BN rows of compressed weight (64 B
//    values, metadata in blocks of steps) and BM rows of activation (128 B per
//    row) in LDS with global->LDS loads, in S buffers: the loads of step k+S-1
//    are in flight while the MFMAs of step k run.  LDS rows are XOR-swizzled
//    in 16-byte chunks so that the lanes the LDS serves together read
//    different banks.  Tiles are assigned so that each XCD (workgroup id
//    mod 8) works on one contiguous run of tiles, walked in groups of G
//    n-tiles, which keeps the weight and activation panels that neighbouring
//    workgroups share in that XCD's L2.
//  * persistent (linear_persistent_kernel): the prefill configuration, one
//    workgroup per CU walking 256 x 256 tiles; 8 wavefronts (64 x 128 each,
//    two per SIMD), wavefronts 0-3 also issue the global->LDS loads of the
//    next stage and 4-7 store the previous tile's output.
//  * wide (linear_wide_kernel, ACC_F8 only): 256 x 256 tiles on 4 wavefronts
//    (128 x 128 each, accumulators in the accumulation registers).
//  * decode (linear_decode_unit_kernel): for M <= 64, where the weight read is
//    everything.  A workgroup owns 16 or 32 weight rows; its wavefronts split
//    the k range in units of 1024, each putting its unit's weight block into
//    its own LDS region (global->LDS, whole cache lines) and its activation
//    into registers, then reduce their partial 16x16 sums through LDS in a
//    fixed order (deterministic).  Tokens beyond M are padding columns of B
//    whose outputs are never stored, the padding-to-16 idea of pytorch/ao PR
//    #1734 ("promote blocksparse from prototype ...").
//    linear_decode_kernel streams the weight into registers instead (any K
//    that is a multiple of 128), and linear_decode_unit_fused1_kernel also
//    quantizes 1 to 4 bf16 activation rows itself.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "sfr_device.hpp"
#include "sfr_launch.hpp"
#include "sfr_quant.hpp"

namespace sfr {
namespace {

constexpr int KSTEP = 128;  // dense k per MFMA and per pipeline stage

template <int OUT>
__device__ __forceinline__ void store4(void* out, int64_t ld, int64_t m, int64_t n, v4f y) {
  if constexpr (OUT == OUT_BF16) {
    uint16_t* o = reinterpret_cast<uint16_t*>(out) + m * ld + n;
    const uint32_t lo = pack_bf16x2(y[0], y[1]);
    const uint32_t hi = pack_bf16x2(y[2], y[3]);
    *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
  } else {
    float* o = reinterpret_cast<float*>(out) + m * ld + n;
    *reinterpret_cast<v4f*>(o) = y;
  }
}

// Weight scales of outputs n .. n+3: four row scales, or the one tensor scale.
__device__ __forceinline__ v4f load_ws4(const float* __restrict__ ws, int n, int ws_stride) {
  if (ws_stride) return *reinterpret_cast<const v4f*>(ws + n);
  const float w = ws[0];
  return v4f{w, w, w, w};
}

// Epilogue of a wavefront's FN x FM grid of 16x16 blocks (block (fn, fm) at
// rows nb + 16 fn, columns mb + 16 fm of the product; lane (r16, lg) holds
// n = 4 lg .. 4 lg + 3 of column m = r16).  Every scale and bias load is
// issued before the first store: a wait for a load also waits for all stores
// issued before it, so loads interleaved with the stores would each cost a
// full store round trip.  Loads are clamped into range and the stores masked.
template <int OUT, int FN, int FM>
__device__ __forceinline__ void store_tile(const v4f (&acc)[FN][FM], const float* __restrict__ xs,
                                           const float* __restrict__ ws, const uint16_t* __restrict__ bias,
                                           void* __restrict__ out, int M, int N, int mb, int nb, int r16, int lg,
                                           int xs_stride, int ws_stride) {
  float xsv[FM];
  v4f wsv[FN];
  uint2 bv[FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) xsv[fm] = xs[min(mb + fm * 16 + r16, M - 1) * xs_stride];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const int nc = min(nb + fn * 16 + 4 * lg, N - 4);
    wsv[fn] = load_ws4(ws, nc, ws_stride);
    bv[fn] = bias ? *reinterpret_cast<const uint2*>(bias + nc) : make_uint2(0u, 0u);
  }
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int m = mb + fm * 16 + r16;
    if (m >= M) continue;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int n = nb + fn * 16 + 4 * lg;
      if (n >= N) continue;
      v4f y;
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = acc[fn][fm][i] * (xsv[fm] * wsv[fn][i]);
      if (bias) {
        y[0] += bf16_to_f32(bv[fn].x & 0xFFFFu);
        y[1] += bf16_to_f32(bv[fn].x >> 16);
        y[2] += bf16_to_f32(bv[fn].y & 0xFFFFu);
        y[3] += bf16_to_f32(bv[fn].y >> 16);
      }
      store4<OUT>(out, N, m, n, y);
    }
  }
}

// bf16 epilogue through LDS (NT = 1: non-temporal stores).  The accumulator
// layout gives each store instruction 16 rows x 32 bytes, and output written
// that way reached about half of what plain full-line writes reach (3.6
// against 7 TB/s), which made the stores of the 256 x 256 kernel a fifth of
// its time.  So a wavefront
// writes its finished FN x FM block, scaled and rounded, row-major into
// `region` (FM * 16 rows of FN * 32 bytes, each 16-byte chunk at
// chunk ^ (row % chunks-per-row) so the writes and the reads spread over the
// banks), and reads it back so that consecutive lanes hold consecutive
// 16-byte chunks of a row: every store instruction then writes whole rows
// of the tile (whole cache lines when a row is 128 bytes or more).  N is a
// multiple of 16 (checked at the boundary), so a chunk that starts below N
// lies wholly inside the row.  The caller makes the LDS free first (every
// wavefront done with its last stage); each wavefront uses only its own region.
template <int FN, int FM, int NT = 0>
__device__ __forceinline__ void store_tile_bf16_lds(const v4f (&acc)[FN][FM], const float* __restrict__ xs,
                                                    const float* __restrict__ ws, const uint16_t* __restrict__ bias,
                                                    uint16_t* __restrict__ out, int M, int N, int mb, int nb, int r16,
                                                    int lg, int lane, int xs_stride, int ws_stride, uint8_t* region) {
  constexpr int CPR = FN * 2;               // 16-byte chunks per row (8 outputs each)
  constexpr int ROWS = FM * 16, RPI = 64 / CPR;  // rows, rows per 64-lane pass
  static_assert((CPR & (CPR - 1)) == 0 && CPR <= 64, "chunks per row");
  float xsv[FM];
  v4f wsv[FN];
  uint2 bv[FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) xsv[fm] = xs[min(mb + fm * 16 + r16, M - 1) * xs_stride];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const int nc = min(nb + fn * 16 + 4 * lg, N - 4);
    wsv[fn] = load_ws4(ws, nc, ws_stride);
    bv[fn] = bias ? *reinterpret_cast<const uint2*>(bias + nc) : make_uint2(0u, 0u);
  }
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int row = fm * 16 + r16;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      v4f y;
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = acc[fn][fm][i] * (xsv[fm] * wsv[fn][i]);
      if (bias) {
        y[0] += bf16_to_f32(bv[fn].x & 0xFFFFu);
        y[1] += bf16_to_f32(bv[fn].x >> 16);
        y[2] += bf16_to_f32(bv[fn].y & 0xFFFFu);
        y[3] += bf16_to_f32(bv[fn].y >> 16);
      }
      const uint32_t lo = pack_bf16x2(y[0], y[1]);
      const uint32_t hi = pack_bf16x2(y[2], y[3]);
      // outputs n = 16 fn + 4 lg .. + 3: chunk 2 fn + lg / 2, half lg % 2
      const int c = (2 * fn + (lg >> 1)) ^ (row & (CPR - 1));
      *reinterpret_cast<uint2*>(region + row * (CPR * 16) + c * 16 + 8 * (lg & 1)) = make_uint2(lo, hi);
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // this wavefront's LDS writes are done
#pragma unroll
  for (int t = 0; t < ROWS / RPI; ++t) {
    const int row = t * RPI + lane / CPR, c = lane % CPR;
    const uint4 v = *reinterpret_cast<const uint4*>(region + row * (CPR * 16) + 16 * (c ^ (row & (CPR - 1))));
    const int m = mb + row, n = nb + 8 * c;
    if (m < M && n < N) {
      uint4* o = reinterpret_cast<uint4*>(out + (int64_t)m * N + n);
      if constexpr (NT) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(o));
      } else {
        *o = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Tiled kernel
// ---------------------------------------------------------------------------
// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without the release fence of __syncthreads (which would
// wait for every outstanding global->LDS load, including later stages').  Each
// wavefront waits for its own loads of the stage it is about to read before
// arriving; the empty asm keeps the compiler from moving LDS accesses across.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Barrier after this wavefront's LDS operations (only) have completed: global
// loads in flight stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), other counters at maximum
  stage_barrier();
}

// LDS row swizzles (16-byte chunks).  The LDS serves a 128-bit read 8 lanes at
// a time, 128 bytes per clock; the 8 lanes of a group read 8 consecutive rows
// at the same logical chunk, so the physical chunk is XORed with the row such
// that those 8 reads cover all 32 banks exactly once.
//   activation rows (128 B = 8 chunks): chunk ^ (row & 7)
//   weight rows     (64 B = 4 chunks, two rows per 128 B): chunk ^ ((row >> 1) & 3)
__device__ __forceinline__ int x_chunk(int row, int j) { return j ^ (row & 7); }
__device__ __forceinline__ int w_chunk(int row, int j) { return j ^ ((row >> 1) & 3); }

// MB = 0: each stage holds its k step's metadata.  MB > 0: metadata moves in
// blocks of MB k steps (16 * MB bytes of each weight row, whole 128-byte
// lines for MB = 8) into two LDS buffers of their own after the stages.
template <int BN, int BM, int WN, int WM, int S, int MB = 0>
struct Tiled {
  static constexpr int NW = WN * WM, NT = 64 * NW;
  static constexpr int TN = BN / WN, TM = BM / WM;  // wavefront tile
  static constexpr int FN = TN / 16, FM = TM / 16;  // 16x16 blocks per wavefront
  static constexpr int W_BYTES = BN * 64, META_BYTES = MB ? 0 : BN * 16, X_BYTES = BM * 128;
  static constexpr int STAGE = W_BYTES + META_BYTES + X_BYTES;
  static constexpr int META_BLOCK = MB ? BN * 16 * MB : 0;  // one metadata block buffer
  static constexpr int MAIN = S * STAGE + 2 * META_BLOCK;
  static constexpr int EPI = NW * FN * FM * 512;  // bf16 epilogue staging (store_tile_bf16_lds)
  static constexpr int LDS = MAIN > EPI ? MAIN : EPI;
  static_assert(BN % 64 == 0 && BM % 8 == 0, "tile");
  static_assert(BN % (16 * WN) == 0 && BM % (16 * WM) == 0, "wave tile");
  static_assert(LDS <= 160 * 1024, "LDS");
  static_assert(S >= 2, "stages");
  static_assert(MB == 0 || (MB == 8 && S >= 2 && S <= 9 && BN % (8 * NW) == 0), "metadata blocks: 8 steps");
};

// Global -> LDS loader of one pipeline stage.  The stage is W_INSTR + M_INSTR
// + X_INSTR load instructions of 1 KB (64 lanes x 16 bytes, written to LDS at
// 1024 q + 16 lane); each region is split evenly over the wavefronts.  The XOR
// swizzle of the LDS rows is applied by choosing which global chunk a lane
// fetches; a lane's chunk is the same for every instruction of a region (the
// swizzles depend on row bits that one instruction's 16 or 8 rows do not
// change), so only the row moves.  Rows past the matrix edge are clamped to
// the last row (read, never stored).
template <int BN, int BM, int NW, bool META = true>
struct StageLoader {
  static constexpr int W_INSTR = BN / 16, M_INSTR = META ? BN / 64 : 0, X_INSTR = BM / 8;
  static constexpr int W_PW = W_INSTR / NW, X_PW = X_INSTR / NW;
  static constexpr int M_PW = (M_INSTR + NW - 1) / NW;
  static constexpr int PER_WAVE_MIN = W_PW + X_PW + M_INSTR / NW;  // loads per stage, every wavefront
  static_assert(W_INSTR % NW == 0 && X_INSTR % NW == 0, "loads split evenly");
  static_assert(M_INSTR % NW == 0 || M_INSTR < NW, "metadata loads");
  const uint8_t* values;
  const uint8_t* meta;
  const uint8_t* xq;
  int64_t ldv, ldm, ldx;
  int n_last, m_last;
  int w_row0, w_col, m_row0, x_row0, x_col;
  int wave;

  __device__ StageLoader(const uint8_t* v, const uint8_t* mt, const uint8_t* x, int K, int N, int M, int n0, int m0,
                         int wave_, int lane)
      : values(v), meta(mt), xq(x), ldv(K / 2), ldm(K / 8), ldx(K), n_last(N - 1), m_last(M - 1), wave(wave_) {
    w_row0 = n0 + wave * W_PW * 16 + (lane >> 2);
    w_col = 16 * ((lane & 3) ^ ((lane >> 3) & 3));
    m_row0 = n0 + wave * 64 + lane;
    x_row0 = m0 + wave * X_PW * 8 + (lane >> 3);
    x_col = 16 * ((lane & 7) ^ ((lane >> 3) & 7));
  }

  // Load j (0 <= j < PER_WAVE_MIN, a compile-time constant once unrolled) of
  // this wavefront's share of stage kt: weight rows, then metadata, then
  // activation rows.  Only for loaders where every wavefront has a metadata load.
  __device__ __forceinline__ void issue_one(uint8_t* stage_base, int kt, int j) const {
    static_assert(M_INSTR % NW == 0, "one metadata share per wavefront");
    const int64_t kb = (int64_t)kt * 128;
    if (j < W_PW) {
      const uint8_t* g = values + (int64_t)min(w_row0 + 16 * j, n_last) * ldv + w_col + kb / 2;
      __builtin_amdgcn_global_load_lds((void*)g, (void*)(stage_base + (wave * W_PW + j) * 1024), 16, 0, 0);
    } else if (j < W_PW + M_PW) {
      const int q = j - W_PW;
      const uint8_t* g = meta + (int64_t)min(m_row0 + 64 * NW * q, n_last) * ldm + kb / 8;
      __builtin_amdgcn_global_load_lds((void*)g, (void*)(stage_base + (W_INSTR + wave + NW * q) * 1024), 16, 0, 0);
    } else {
      const int q = j - W_PW - M_PW;
      const uint8_t* g = xq + (int64_t)min(x_row0 + 8 * q, m_last) * ldx + x_col + kb;
      __builtin_amdgcn_global_load_lds((void*)g, (void*)(stage_base + (W_INSTR + M_INSTR + wave * X_PW + q) * 1024),
                                       16, 0, 0);
    }
  }

  __device__ __forceinline__ void issue(uint8_t* stage_base, int kt) const {
    const int64_t kb = (int64_t)kt * 128;
#pragma unroll
    for (int j = 0; j < W_PW; ++j) {
      const uint8_t* g = values + (int64_t)min(w_row0 + 16 * j, n_last) * ldv + w_col + kb / 2;
      __builtin_amdgcn_global_load_lds((void*)g, (void*)(stage_base + (wave * W_PW + j) * 1024), 16, 0, 0);
    }
    if (M_INSTR > 0 && (M_INSTR >= NW || wave < M_INSTR)) {
#pragma unroll
      for (int j = 0; j < M_PW; ++j) {
        const uint8_t* g = meta + (int64_t)min(m_row0 + 64 * NW * j, n_last) * ldm + kb / 8;
        __builtin_amdgcn_global_load_lds((void*)g, (void*)(stage_base + (W_INSTR + wave + NW * j) * 1024), 16, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < X_PW; ++j) {
      const uint8_t* g = xq + (int64_t)min(x_row0 + 8 * j, m_last) * ldx + x_col + kb;
      __builtin_amdgcn_global_load_lds((void*)g,
                                       (void*)(stage_base + (W_INSTR + M_INSTR + wave * X_PW + j) * 1024), 16, 0, 0);
    }
  }
};

template <int XF, int WF, int OUT, int BN, int BM, int WN, int WM, int G, int S, int ORD, int OCC, int MB, int NT,
          int ACC>
__global__ __launch_bounds__(64 * WN * WM, OCC) void linear_tiled_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xs, const uint8_t* __restrict__ values,
    const uint8_t* __restrict__ meta, const float* __restrict__ ws, const uint16_t* __restrict__ bias,
    void* __restrict__ out, int M, int N, int K, int tiles_m, int tiles_n, int xs_stride, int ws_stride) {
  using C = Tiled<BN, BM, WN, WM, S, MB>;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

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
  const int64_t ldm = K / 8;

  // ---- this wavefront's share of the per-stage loads (global -> LDS) ----
  const StageLoader<BN, BM, C::NW, MB == 0> loader(values, meta, xq, K, N, M, n0, m0, wave, lane);
  auto issue = [&](int kt, int slot) { loader.issue(smem + slot * C::STAGE, kt); };
  constexpr int LPW = StageLoader<BN, BM, C::NW, MB == 0>::PER_WAVE_MIN;
  const int KT = K / KSTEP;

  // ---- metadata blocks (MB > 0): block b = k steps MB b .. MB b + MB - 1,
  // row r's 16-byte chunk of step s at chunk s ^ (r % 8) of the row's 16 MB
  // bytes, in buffer b % 2.  One 1 KB load = 8 rows x 8 chunks; each
  // wavefront loads BN / (8 NW) of them.  Chunks past the last k step repeat
  // that step's chunk (loaded, never read). ----
  uint8_t* const meta_lds = smem + S * C::STAGE;
  auto issue_meta = [&](int blk) {
    if constexpr (MB > 0) {
      constexpr int PW = BN / (8 * C::NW);
      const int s = min((lane & 7) ^ ((lane >> 3) & 7), KT - MB * blk - 1);
#pragma unroll
      for (int j = 0; j < PW; ++j) {
        const int row = (wave * PW + j) * 8 + (lane >> 3);
        const uint8_t* g = meta + (int64_t)min(n0 + row, N - 1) * ldm + 16 * (MB * blk + s);
        __builtin_amdgcn_global_load_lds((void*)g, (void*)(meta_lds + (blk & 1) * C::META_BLOCK + (wave * PW + j) * 1024),
                                         16, 0, 0);
      }
    }
  };

  // ---- LDS read offsets of this lane's MFMA operands ----
  int a_off[C::FN], i_off[C::FN], b_off0[C::FM], b_off1[C::FM];
#pragma unroll
  for (int f = 0; f < C::FN; ++f) {
    const int r = wn * C::TN + f * 16 + r16;
    a_off[f] = r * 64 + 16 * w_chunk(r, lg);
    // MB > 0: offset from the stage base to the row's metadata (step chunk added per step)
    i_off[f] = MB ? (int)(meta_lds - smem) + r * (16 * MB) + 4 * lg : C::W_BYTES + r * 16 + 4 * lg;
  }
#pragma unroll
  for (int f = 0; f < C::FM; ++f) {
    const int r = wm * C::TM + f * 16 + r16;
    b_off0[f] = C::W_BYTES + C::META_BYTES + r * 128 + 16 * x_chunk(r, lg);
    b_off1[f] = C::W_BYTES + C::META_BYTES + r * 128 + 16 * x_chunk(r, 4 + lg);
  }

  v4f acc[C::FN][C::FM];
#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  issue_meta(0);
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < KT) issue(s, s);

  for (int kt = 0; kt < KT; ++kt) {
    // stage kt has landed once at most the loads of the S-2 later stages are
    // pending (a metadata block issued after stage kt only makes the wait
    // stricter; it was issued at least one step earlier)
    if (kt + S - 2 < KT) wait_vmcnt<LPW * (S - 2)>();
    else wait_vmcnt<0>();
    stage_barrier();
    // block kt / MB + 1 goes to the buffer that block kt / MB - 1 used, free
    // since every wavefront passed this barrier after its last step
    if constexpr (MB > 0)
      if (kt % MB == 0 && kt + MB < KT) issue_meta(kt / MB + 1);
    if (kt + S - 1 < KT) issue(kt + S - 1, (kt + S - 1) % S);
    const uint8_t* base = smem + (kt % S) * C::STAGE;
    // metadata of step kt relative to the stage base: chunk (kt % MB) ^ (row % 8), rows % 8 = r16 % 8
    const int mo = MB ? 16 * ((kt % (MB ? MB : 1)) ^ (r16 & 7)) + ((kt / (MB ? MB : 1)) & 1) * C::META_BLOCK -
                            (int)(base - smem)
                      : 0;
    if constexpr (ACC == ACC_F32) {
      // binary32-grade accumulation: every weight fragment widened once per
      // step (both halves), then one activation block at a time, each half
      // widened once and fed to the FN instructions of that half
      v4i aw[2][C::FN];
      int ix[2][C::FN];
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        const v4i a = *reinterpret_cast<const v4i*>(base + a_off[fn]);
        const int idx = *reinterpret_cast<const int*>(base + i_off[fn] + mo);
        aw[0][fn] = widen_a_half<WF, 0>(a);
        aw[1][fn] = widen_a_half<WF, 1>(a);
        ix[0][fn] = idx_half<0>(idx);
        ix[1][fn] = idx_half<1>(idx);
      }
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
        const v4i lo = *reinterpret_cast<const v4i*>(base + b_off0[fm]);
        const v4i hi = *reinterpret_cast<const v4i*>(base + b_off1[fm]);
        const v8i b = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const v8i b0 = widen_b_half<XF, 0>(b);
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) acc[fn][fm] = smfmac16_bf16(aw[0][fn], b0, acc[fn][fm], ix[0][fn]);
        const v8i b1 = widen_b_half<XF, 1>(b);
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) acc[fn][fm] = smfmac16_bf16(aw[1][fn], b1, acc[fn][fm], ix[1][fn]);
      }
    } else if constexpr (ORD == 0) {
      // all weight operands of the wavefront tile, then one activation block at
      // a time: each 32-byte B fragment feeds FN instructions
      v4i a[C::FN];
      int idx[C::FN];
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        a[fn] = *reinterpret_cast<const v4i*>(base + a_off[fn]);
        idx[fn] = *reinterpret_cast<const int*>(base + i_off[fn] + mo);
      }
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
        const v4i lo = *reinterpret_cast<const v4i*>(base + b_off0[fm]);
        const v4i hi = *reinterpret_cast<const v4i*>(base + b_off1[fm]);
        const v8i b = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) acc[fn][fm] = smfmac16<XF, WF>(a[fn], b, acc[fn][fm], idx[fn]);
      }
    } else {
      // all activation blocks, then the weight blocks one ahead of their MFMAs
      v8i b[C::FM];
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
        const v4i lo = *reinterpret_cast<const v4i*>(base + b_off0[fm]);
        const v4i hi = *reinterpret_cast<const v4i*>(base + b_off1[fm]);
        b[fm] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      v4i a[2];
      int idx[2];
      a[0] = *reinterpret_cast<const v4i*>(base + a_off[0]);
      idx[0] = *reinterpret_cast<const int*>(base + i_off[0] + mo);
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        if (fn + 1 < C::FN) {
          a[(fn + 1) & 1] = *reinterpret_cast<const v4i*>(base + a_off[fn + 1]);
          idx[(fn + 1) & 1] = *reinterpret_cast<const int*>(base + i_off[fn + 1] + mo);
        }
        if constexpr (ORD == 2) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
          acc[fn][fm] = smfmac16<XF, WF>(a[fn & 1], b[fm], acc[fn][fm], idx[fn & 1]);
        if constexpr (ORD == 2) __builtin_amdgcn_s_setprio(0);
      }
    }
  }

  // ---- epilogue: scales, bias, bf16, store (bf16 through LDS, once every
  // wavefront is done with the last stage) ----
  if constexpr (OUT == OUT_BF16) {
    lds_barrier();
    store_tile_bf16_lds<C::FN, C::FM, NT>(acc, xs, ws, bias, reinterpret_cast<uint16_t*>(out), M, N, m0 + wm * C::TM,
                                      n0 + wn * C::TN, r16, lg, lane, xs_stride, ws_stride,
                                      smem + wave * (C::FN * C::FM * 512));
  } else {
    store_tile<OUT>(acc, xs, ws, bias, out, M, N, m0 + wm * C::TM, n0 + wn * C::TN, r16, lg, xs_stride, ws_stride);
  }
}

// ---------------------------------------------------------------------------
// Persistent 256 x 256 kernel (bf16 output)
// ---------------------------------------------------------------------------
// The tiled kernel's scheme (two 48 KB stages, metadata in 8-step blocks,
// eight wavefronts of 64(n) x 128(m), one barrier per k step) with three
// changes:
//  * global -> LDS loads through buffer descriptors based at the tile's first
//    row: the k step and each load's row offset are scalar, so a load needs
//    one vector offset per operand kind instead of a 64-bit address each, and
//    rows past the matrix edge read zeros (those outputs are never stored);
//  * wavefronts 0-3 issue every load and wait for them; wavefronts 4-7 never
//    wait on the memory counter (gfx9 counts stores in it too), so they can
//    issue a tile's output stores and go straight on into the next tile;
//  * one workgroup per CU walks its XCD's run of tiles: the next tile's first
//    stage and metadata block are put in flight before the output is staged,
//    so their latency overlaps the epilogue.
// Epilogue per half of the tile: every wavefront writes its scaled bf16 rows
// into its own 8 KB LDS region (in stage slot 1 and metadata buffer 1, which
// the next tile's first loads do not touch), then the store wavefronts each
// write two regions out as whole 128-byte row segments.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  // raw buffer, 32-bit data format in the last descriptor word (gfx9)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// One 1 KB buffer -> LDS load: lane l's 16 bytes at voff + soff land at lds + 16 l.
__device__ __forceinline__ void buffer_lds16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, int voff, int soff) {
  // the LDS address and the scalar offset are uniform; saying so keeps the
  // compiler from looping over their values
  const uint32_t a = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)lds);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(uintptr_t)a, 16, voff, __builtin_amdgcn_readfirstlane(soff), 0,
                                           0);
}

// Loads of one BN x BM tile, shared by NL wavefronts (lw = 0 .. NL-1).  LDS
// layouts are those of the tiled kernel: a stage is BN / 16 1 KB blocks of
// weight values then BM / 8 of activation; a metadata block BN / 8 blocks.
template <int BN, int BM, int NL>
struct TileBufferLoader {
  static constexpr int MB = 8;
  static constexpr int W_INSTR = BN / 16, X_INSTR = BM / 8, M_INSTR = BN / 8;
  static constexpr int W_PW = W_INSTR / NL, X_PW = X_INSTR / NL, M_PW = M_INSTR / NL;
  static_assert(W_INSTR % NL == 0 && X_INSTR % NL == 0 && M_INSTR % NL == 0, "loads split evenly");
  __amdgpu_buffer_rsrc_t rx, rw, rm;
  int ldx, ldv, ldm, vx, vw, lw, lane;
  // requires max(BN, BM) * K < 2^31 (every offset and range fits the descriptor)
  __device__ TileBufferLoader(const uint8_t* xq, const uint8_t* values, const uint8_t* meta, int M, int N, int K, int m0,
                              int n0, int lw_, int lane_)
      : ldx(K), ldv(K / 2), ldm(K / 8), lw(lw_), lane(lane_) {
    const int rows_m = min(M - m0, BM), rows_n = min(N - n0, BN);
    rx = buffer_rsrc(xq + (int64_t)m0 * K, rows_m * K);
    rw = buffer_rsrc(values + (int64_t)n0 * (K / 2), rows_n * (K / 2));
    rm = buffer_rsrc(meta + (int64_t)n0 * (K / 8), rows_n * (K / 8));
    // lane -> (row within the load, swizzled 16-byte chunk), as in StageLoader
    vx = (lane >> 3) * ldx + 16 * ((lane & 7) ^ ((lane >> 3) & 7));
    vw = (lane >> 2) * ldv + 16 * ((lane & 3) ^ ((lane >> 3) & 3));
  }
  __device__ __forceinline__ void stage(uint8_t* base, int kt) const {
#pragma unroll
    for (int j = 0; j < W_PW; ++j)
      buffer_lds16(rw, base + (lw * W_PW + j) * 1024, vw, (lw * W_PW + j) * 16 * ldv + kt * 64);
#pragma unroll
    for (int q = 0; q < X_PW; ++q)
      buffer_lds16(rx, base + (W_INSTR + lw * X_PW + q) * 1024, vx, (lw * X_PW + q) * 8 * ldx + kt * 128);
  }
  // metadata block blk: row r's chunk of step s at chunk s ^ (r % 8); chunks
  // past the last k step repeat that step's chunk
  __device__ __forceinline__ void metablock(uint8_t* buf, int blk, int KT) const {
    const int s = min((lane & 7) ^ ((lane >> 3) & 7), KT - MB * blk - 1);
    const int vm = (lane >> 3) * ldm + 16 * s;
#pragma unroll
    for (int j = 0; j < M_PW; ++j)
      buffer_lds16(rm, buf + (lw * M_PW + j) * 1024, vm, (lw * M_PW + j) * 8 * ldm + 16 * MB * blk);
  }
};

// NT = 1: output stores are non-temporal.  OUT_F32: every wavefront stores
// its own binary32 block straight from its accumulators (the diagnostic
// output; the loader wavefronts then also wait for their stores).
template <int XF, int WF, int OUT, int ACC, int BN, int BM, int WN, int WM, int NL, int G, int OCC, int NT = 0>
__global__ __launch_bounds__(64 * WN * WM, OCC) void linear_persistent_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xs, const uint8_t* __restrict__ values,
    const uint8_t* __restrict__ meta, const float* __restrict__ ws, const uint16_t* __restrict__ bias,
    void* __restrict__ out_, int M, int N, int K, int tiles_m, int tiles_n, int xs_stride, int ws_stride) {
  uint16_t* const out = reinterpret_cast<uint16_t*>(out_);
  constexpr int S = 2, MB = 8;
  using C = Tiled<BN, BM, WN, WM, S, MB>;
  using L = TileBufferLoader<BN, BM, NL>;
  // epilogue: each wavefront stages half its block (TM / 2 rows of 128 bytes)
  // per pass; the NW - NL store wavefronts write out PER regions each
  constexpr int RB = C::TM / 2 * 128, PER = C::NW / (C::NW - NL);
  static_assert(C::TN == 64 && C::FM % 2 == 0, "128-byte rows of whole 16x16 blocks");
  static_assert(NL > 0 && NL < C::NW && C::NW % (C::NW - NL) == 0, "loader and store wavefronts");
  static_assert(C::NW * RB <= C::STAGE + C::META_BLOCK, "regions fit in stage slot 1 and metadata buffer 1");
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  // ---- tiles: XCD x (workgroup id mod 8) owns a contiguous run, grouped
  // along n as in the tiled kernel; its workgroups take every nslot-th ----
  const int T = tiles_m * tiles_n;
  const int per_xcd = (T + 7) / 8;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8, nslot = gridDim.x / 8;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave / WM, wm = wave % WM;
  const int r16 = lane & 15, lg = lane >> 4;
  const bool loader_wave = wave < NL;
  const int lw = loader_wave ? wave : 0;
  const int KT = K / KSTEP;
  auto tile_of = [&](int it, int& n0, int& m0) -> bool {
    const int j = slot + nslot * it;
    if (j >= per_xcd) return false;
    const int lid = xcd * per_xcd + j;
    if (lid >= T) return false;
    const int group = lid / (G * tiles_m);
    const int first_n = group * G;
    const int gsize = min(tiles_n - first_n, G);
    const int within = lid - group * G * tiles_m;
    n0 = (first_n + within % gsize) * BN;
    m0 = (within / gsize) * BM;
    return true;
  };

  // ---- LDS read offsets (as in the tiled kernel with MB = 8) ----
  uint8_t* const meta_lds = smem + S * C::STAGE;
  int a_off[C::FN], i_off[C::FN], b_off0[C::FM], b_off1[C::FM];
#pragma unroll
  for (int f = 0; f < C::FN; ++f) {
    const int r = wn * C::TN + f * 16 + r16;
    a_off[f] = r * 64 + 16 * w_chunk(r, lg);
    i_off[f] = (int)(meta_lds - smem) + r * (16 * MB) + 4 * lg;
  }
#pragma unroll
  for (int f = 0; f < C::FM; ++f) {
    const int r = wm * C::TM + f * 16 + r16;
    b_off0[f] = C::W_BYTES + r * 128 + 16 * x_chunk(r, lg);
    b_off1[f] = C::W_BYTES + r * 128 + 16 * x_chunk(r, 4 + lg);
  }
  // epilogue regions: stage slot 1 first, then metadata buffer 1
  constexpr int IN_SLOT = C::STAGE / RB;
  auto region = [&](int w) -> uint8_t* {
    return w < IN_SLOT ? smem + C::STAGE + w * RB : meta_lds + C::META_BLOCK + (w - IN_SLOT) * RB;
  };

  int n0, m0;
  if (!tile_of(0, n0, m0)) return;
  if (loader_wave) {
    const L first(xq, values, meta, M, N, K, m0, n0, lw, lane);
    first.metablock(meta_lds, 0, KT);
    first.stage(smem, 0);
  }
  for (int it = 0;; ++it) {
    const L loader(xq, values, meta, M, N, K, m0, n0, lw, lane);
    v4f acc[C::FN][C::FM];
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
      for (int j = 0; j < C::FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int kt = 0; kt < KT; ++kt) {
      // the loaders' loads of stage kt (and of its metadata block) have
      // landed once they have none pending; the barrier tells everyone
      if (loader_wave) wait_vmcnt<0>();
      stage_barrier();
      if (loader_wave) {
        if (kt % MB == 0 && kt + MB < KT)
          loader.metablock(meta_lds + ((kt / MB + 1) & 1) * C::META_BLOCK, kt / MB + 1, KT);
        if (kt + 1 < KT) loader.stage(smem + ((kt + 1) % S) * C::STAGE, kt + 1);
      }
      const uint8_t* base = smem + (kt % S) * C::STAGE;
      const int mo = 16 * ((kt % MB) ^ (r16 & 7)) + ((kt / MB) & 1) * C::META_BLOCK - (int)(base - smem);
      if constexpr (ACC == ACC_F32) {
        // The step as 2 FM (activation block, half) pairs, in that order (see
        // smfmac16_bf16).  Both halves of the weight fragments are widened
        // at the start; each activation block is read whole (two 16-byte LDS
        // reads, PD blocks ahead) and the operand of pair q + 1 is widened
        // while the FN instructions of pair q run: 8 / FN of those
        // conversions follow each instruction (and in pair 0 also one
        // fragment's second weight half), held in place by scheduling
        // barriers, so they issue while the matrix core is busy instead of
        // between its instruction groups.
        v4i a[C::FN];
        int idx[C::FN];
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
          a[fn] = *reinterpret_cast<const v4i*>(base + a_off[fn]);
          idx[fn] = *reinterpret_cast<const int*>(base + i_off[fn] + mo);
        }
        constexpr int PD = 2;
        auto read_b = [&](int fm) __attribute__((always_inline)) {
          const v4i lo = *reinterpret_cast<const v4i*>(base + b_off0[fm]);
          const v4i hi = *reinterpret_cast<const v4i*>(base + b_off1[fm]);
          return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        };
        v8i braw[C::FM];
#pragma unroll
        for (int f = 0; f < PD; ++f) braw[f] = read_b(f);
        v4i aw[2][C::FN];
        int ix[2][C::FN];
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
          aw[0][fn] = widen_a_half<WF, 0>(a[fn]);
          ix[0][fn] = idx_half<0>(idx[fn]);
        }
        v8i bw[2];
        bw[0] = widen_b_half<XF, 0>(braw[0]);
        constexpr int EPF = 8 / C::FN;  // conversions after each instruction
        static_assert(8 % C::FN == 0, "conversions spread evenly over the instructions");
#pragma unroll
        for (int q = 0; q < 2 * C::FM; ++q) {
          const int fm = q >> 1, h = q & 1;
          if (h == 0 && fm + PD < C::FM) braw[fm + PD] = read_b(fm + PD);
          // pair q + 1 uses half nh of block nfm; its element e (widen_b_half)
          // is half (e & 1) of FP8 word 2 nh + ((e >> 1) & 1) + 4 (e >> 2)
          const bool more = q + 1 < 2 * C::FM;
          const int nfm = fm + h, nh = h ^ 1;
#pragma unroll
          for (int fn = 0; fn < C::FN; ++fn) {
            acc[fn][fm] = smfmac16_bf16(aw[h][fn], bw[h], acc[fn][fm], ix[h][fn]);
            if (more) {
#pragma unroll
              for (int e = fn * EPF; e < (fn + 1) * EPF; ++e) {
                const int w = braw[nfm][2 * nh + ((e >> 1) & 1) + 4 * (e >> 2)];
                bw[nh][e] = (e & 1) ? widen2<XF, true>(w) : widen2<XF, false>(w);
              }
            }
            if (q == 0) {
              aw[1][fn] = widen_a_half<WF, 1>(a[fn]);
              ix[1][fn] = idx_half<1>(idx[fn]);
            }
            // program order is issue order: each instruction is followed by
            // the conversions that can run while it occupies the matrix core
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        continue;
      }
      v8i b[C::FM];
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
        const v4i lo = *reinterpret_cast<const v4i*>(base + b_off0[fm]);
        const v4i hi = *reinterpret_cast<const v4i*>(base + b_off1[fm]);
        b[fm] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      v4i a[2];
      int idx[2];
      a[0] = *reinterpret_cast<const v4i*>(base + a_off[0]);
      idx[0] = *reinterpret_cast<const int*>(base + i_off[0] + mo);
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        if (fn + 1 < C::FN) {
          a[(fn + 1) & 1] = *reinterpret_cast<const v4i*>(base + a_off[fn + 1]);
          idx[(fn + 1) & 1] = *reinterpret_cast<const int*>(base + i_off[fn + 1] + mo);
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
          acc[fn][fm] = smfmac16<XF, WF>(a[fn & 1], b[fm], acc[fn][fm], idx[fn & 1]);
        __builtin_amdgcn_s_setprio(0);
      }
    }

    // ---- epilogue ----
    int nn0 = 0, nm0 = 0;
    const bool next = tile_of(it + 1, nn0, nm0);
    const int mb = m0 + wm * C::TM, nb = n0 + wn * C::TN;
    if constexpr (OUT == OUT_F32) {
      lds_barrier();  // every wavefront is done with the last step's LDS reads
      if (next && loader_wave) {
        const L nl(xq, values, meta, M, N, K, nm0, nn0, lw, lane);
        nl.metablock(meta_lds, 0, KT);
        nl.stage(smem, 0);
      }
      store_tile<OUT_F32>(acc, xs, ws, bias, out_, M, N, mb, nb, r16, lg, xs_stride, ws_stride);
      if (!next) break;
      n0 = nn0;
      m0 = nm0;
      continue;
    }
    float xsv[C::FM];
    v4f wsv[C::FN];
    uint2 bv[C::FN];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) xsv[fm] = xs[min(mb + fm * 16 + r16, M - 1) * xs_stride];
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int nc = min(nb + fn * 16 + 4 * lg, N - 4);
      wsv[fn] = load_ws4(ws, nc, ws_stride);
      bv[fn] = bias ? *reinterpret_cast<const uint2*>(bias + nc) : make_uint2(0u, 0u);
    }
    lds_barrier();  // every wavefront is done with the last step's LDS reads
    if (next && loader_wave) {
      const L nl(xq, values, meta, M, N, K, nm0, nn0, lw, lane);
      nl.metablock(meta_lds, 0, KT);
      nl.stage(smem, 0);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // rows m = wm * TM + h TM / 2 .. of this wavefront's block, 128 bytes
      // each, 16-byte chunk c at c ^ (row % 8)
      uint8_t* reg = region(wave);
#pragma unroll
      for (int q = 0; q < C::FM / 2; ++q) {
        const int fm = h * (C::FM / 2) + q, row = q * 16 + r16;
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
          v4f y;
#pragma unroll
          for (int i = 0; i < 4; ++i) y[i] = acc[fn][fm][i] * (xsv[fm] * wsv[fn][i]);
          if (bias) {
            y[0] += bf16_to_f32(bv[fn].x & 0xFFFFu);
            y[1] += bf16_to_f32(bv[fn].x >> 16);
            y[2] += bf16_to_f32(bv[fn].y & 0xFFFFu);
            y[3] += bf16_to_f32(bv[fn].y >> 16);
          }
          const uint32_t lo = pack_bf16x2(y[0], y[1]);
          const uint32_t hi = pack_bf16x2(y[2], y[3]);
          const int c = (2 * fn + (lg >> 1)) ^ (row & 7);
          *reinterpret_cast<uint2*>(reg + row * 128 + c * 16 + 8 * (lg & 1)) = make_uint2(lo, hi);
        }
      }
      lds_barrier();  // every region written
      if (!loader_wave) {
        // N is a multiple of 16, so a chunk starting below N lies inside the row
#pragma unroll
        for (int q = 0; q < PER; ++q) {
          const int sw = PER * (wave - NL) + q;
          const int swn = sw / WM, swm = sw % WM;
          const uint8_t* sreg = region(sw);
#pragma unroll
          for (int t = 0; t < C::TM / 16; ++t) {
            const int row = t * 8 + (lane >> 3), c = lane & 7;
            const uint4 v = *reinterpret_cast<const uint4*>(sreg + row * 128 + 16 * (c ^ (row & 7)));
            const int m = m0 + swm * C::TM + h * (C::TM / 2) + row, n = n0 + swn * C::TN + 8 * c;
            if (m < M && n < N) {
              uint4* o = reinterpret_cast<uint4*>(out + (int64_t)m * N + n);
              if constexpr (NT) {
                typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
                __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(o));
              } else {
                *o = v;
              }
            }
          }
        }
      }
      lds_barrier();  // the store wavefronts have read every region
    }
    if (!next) break;
    n0 = nn0;
    m0 = nm0;
  }
}

// ---------------------------------------------------------------------------
// Software-pipelined tiled kernel: 256 x 256 tile, four wavefronts (one per
// SIMD), each owning a 128 x 128 block of the tile (64 accumulators of 16x16,
// held in the accumulation registers).
// ---------------------------------------------------------------------------
// With one wavefront per SIMD nothing else hides a wavefront's own LDS latency,
// so the reads are pipelined in registers:
//   * the activation fragments of a k step stream through a ring of RING
//     registers sets, read PF m blocks ahead of their MFMAs;
//   * the weight fragments and the first PF activation fragments of step kt+1
//     are read during the last m blocks of step kt.
// That needs stage kt+1 in LDS before step kt ends, so the workgroup barrier
// sits inside the step, before m block SWITCH: by then each wavefront has
// issued every LDS read of stage kt (and waited for them), and stage kt+1 has
// landed.  Past the barrier, stage kt's slot is free and receives stage kt+3:
// three LDS stages give each global->LDS load two steps to land.
template <int XF, int WF, int OUT, int G>
__global__ __launch_bounds__(256, 1) void linear_wide_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xs, const uint8_t* __restrict__ values,
    const uint8_t* __restrict__ meta, const float* __restrict__ ws, const uint16_t* __restrict__ bias,
    void* __restrict__ out, int M, int N, int K, int tiles_m, int tiles_n, int xs_stride, int ws_stride) {
  constexpr int BN = 256, BM = 256, S = 3;
  using C = Tiled<BN, BM, 2, 2, S>;
  using L = StageLoader<BN, BM, C::NW>;
  constexpr int FN = C::FN, FM = C::FM;  // 8 x 8
  constexpr int LPW = L::PER_WAVE_MIN;   // global->LDS loads per stage and wavefront
  constexpr int PF = 2, RING = 4, SWITCH = FM - PF;
  static_assert(RING >= PF + 1 && FM % RING == 0, "activation ring");
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

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
  const int wn = wave / 2, wm = wave % 2;
  const int r16 = lane & 15, lg = lane >> 4;

  const L loader(values, meta, xq, K, N, M, n0, m0, wave, lane);
  const int KT = K / KSTEP;

  // LDS operand offsets: block f of the wavefront sits 16 f rows further on,
  // and the swizzles depend only on row bits 0-2, which f does not change, so
  // each offset is a per-lane base plus a compile-time multiple of f.
  const int a_base = (wn * C::TN + r16) * 64 + 16 * w_chunk(r16, lg);        // + 1024 f
  const int i_base = C::W_BYTES + (wn * C::TN + r16) * 16 + 4 * lg;         // + 256 f
  const int b_base0 = C::W_BYTES + C::META_BYTES + (wm * C::TM + r16) * 128 + 16 * x_chunk(r16, lg);      // + 2048 f
  const int b_base1 = C::W_BYTES + C::META_BYTES + (wm * C::TM + r16) * 128 + 16 * x_chunk(r16, 4 + lg);  // + 2048 f
  auto read_b = [&](const uint8_t* base, int fm) __attribute__((always_inline)) {
    const v4i lo = *reinterpret_cast<const v4i*>(base + b_base0 + 2048 * fm);
    const v4i hi = *reinterpret_cast<const v4i*>(base + b_base1 + 2048 * fm);
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  auto read_a = [&](const uint8_t* base, v4i(&a)[FN], int(&idx)[FN]) __attribute__((always_inline)) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      a[fn] = *reinterpret_cast<const v4i*>(base + a_base + 1024 * fn);
      idx[fn] = *reinterpret_cast<const int*>(base + i_base + 256 * fn);
    }
  };

  v4f acc[FN][FM];

  // prologue: stages 0..2 in flight, stage 0 landed and visible (KT >= 4)
#pragma unroll
  for (int s = 0; s < S; ++s) loader.issue(smem + s * C::STAGE, s);
  wait_vmcnt<(S - 1) * LPW>();
  stage_barrier();

  // Two sets of weight fragments, used by alternate steps: the set for step
  // kt+1 is loaded while step kt's MFMAs read the other, so no register an
  // MFMA may still be reading is rewritten by an ALU copy.
  v4i a0[FN], a1[FN];
  int i0[FN], i1[FN];
  v8i b[RING];
  read_a(smem, a0, i0);
#pragma unroll
  for (int f = 0; f < PF; ++f) b[f] = read_b(smem, f);

  // The global->LDS loads of one stage are spread over FM positions, at most
  // two per m block: positions 0 .. FM-SWITCH-1 are m blocks SWITCH .. FM-1 of
  // step kt (after its barrier), the rest m blocks 0 .. SWITCH-1 of step kt+1,
  // all before the wait for the stage at step kt+1's barrier.  So the address
  // unit never queues a whole stage's loads ahead of the wavefront's MFMAs.
  static_assert((LPW + 1) / 2 <= FM, "issue schedule");
  auto issue_at = [&](uint8_t* base, int stage, int p) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 2 * p; j < 2 * p + 2; ++j)
      if (j < LPW) loader.issue_one(base, stage, j);
  };

  // One k step on weight set (a, idx), loading set (an, in) for step kt+1.
  // NEXT: a step kt+1 exists; WAIT: global->LDS loads of this wavefront allowed
  // to stay pending once stage kt+1 has landed; CONT: finish issuing stage
  // kt+2 (begun in step kt-1) in m blocks 0 .. SWITCH-1; BEGIN: start issuing
  // stage kt+3 (into stage kt's slot) at the barrier.
  auto step = [&](auto next_c, auto wait_c, auto cont_c, auto begin_c, int kt, v4i(&a)[FN], int(&idx)[FN],
                  v4i(&an)[FN], int(&in)[FN]) __attribute__((always_inline)) {
    constexpr bool NEXT = decltype(next_c)::value, CONT = decltype(cont_c)::value;
    constexpr bool BEGIN = decltype(begin_c)::value;
    constexpr int WAIT = decltype(wait_c)::value;
    const int slot = kt % S, nslot = (kt + 1) % S, pslot = (kt + 2) % S;
    const uint8_t* cur = smem + slot * C::STAGE;
    const uint8_t* nxt = smem + nslot * C::STAGE;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if constexpr (CONT) {
        if (fm < SWITCH) issue_at(smem + pslot * C::STAGE, kt + 2, FM - SWITCH + fm);
      }
      if constexpr (NEXT) {
        if (fm == SWITCH) {
          wait_vmcnt<WAIT>();
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wavefront's reads of stage kt are done
          stage_barrier();
          read_a(nxt, an, in);
        }
      }
      if constexpr (BEGIN) {
        if (fm >= SWITCH) issue_at(smem + slot * C::STAGE, kt + S, fm - SWITCH);
      }
      if (fm + PF < FM) b[(fm + PF) % RING] = read_b(cur, fm + PF);
      else if constexpr (NEXT) b[(fm + PF) % RING] = read_b(nxt, fm + PF - FM);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) smfmac16_acc<XF, WF>(acc[fn][fm], a[fn], b[fm % RING], idx[fn]);
    }
  };
  using T1 = std::true_type;
  using F0 = std::false_type;
  // loads a wavefront may leave pending once stage kt+1 has landed: those of
  // stage kt+2, if it exists
  using WL = std::integral_constant<int, LPW>;
  using W0 = std::integral_constant<int, 0>;
  // The whole step sequence, straight-line for one parity of KT, so that the
  // fragment set of every step is known at compile time (KT >= 4):
  //   step 0 begins stage 3; steps 1 .. KT-4 continue and begin stages;
  //   step KT-3 only continues; steps KT-2 and KT-1 issue nothing.
  // Accumulator set-up, steps and epilogue all sit inside each parity's path,
  // so no accumulator is live where the two paths split or join.
  auto steps = [&](auto odd_c) __attribute__((always_inline)) {
    constexpr bool ODD = decltype(odd_c)::value;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        acc_fence(acc[i][j]);
      }
    step(T1{}, WL{}, F0{}, T1{}, 0, a0, i0, a1, i1);
    int kt = 1;
    if constexpr (ODD) step(T1{}, WL{}, T1{}, T1{}, kt++, a1, i1, a0, i0);
    // pairs (kt even when ODD, odd otherwise); KT - 4 - ODD steps remain before step KT-3
    for (; kt + S + 1 < KT; kt += 2) {
      if constexpr (ODD) {
        step(T1{}, WL{}, T1{}, T1{}, kt, a0, i0, a1, i1);
        step(T1{}, WL{}, T1{}, T1{}, kt + 1, a1, i1, a0, i0);
      } else {
        step(T1{}, WL{}, T1{}, T1{}, kt, a1, i1, a0, i0);
        step(T1{}, WL{}, T1{}, T1{}, kt + 1, a0, i0, a1, i1);
      }
    }
    // kt == KT - 3: odd when KT is even
    if constexpr (ODD) {
      step(T1{}, WL{}, T1{}, F0{}, kt, a0, i0, a1, i1);
      step(T1{}, W0{}, F0{}, F0{}, kt + 1, a1, i1, a0, i0);
      step(F0{}, W0{}, F0{}, F0{}, kt + 2, a0, i0, a1, i1);
    } else {
      step(T1{}, WL{}, T1{}, F0{}, kt, a1, i1, a0, i0);
      step(T1{}, W0{}, F0{}, F0{}, kt + 1, a0, i0, a1, i1);
      step(F0{}, W0{}, F0{}, F0{}, kt + 2, a1, i1, a0, i0);
    }
    mfma_drain();
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc_fence(acc[i][j]);
    if constexpr (OUT == OUT_BF16) {
      lds_barrier();
      store_tile_bf16_lds<FN, FM>(acc, xs, ws, bias, reinterpret_cast<uint16_t*>(out), M, N, m0 + wm * C::TM,
                                  n0 + wn * C::TN, r16, lg, lane, xs_stride, ws_stride, smem + wave * (FN * FM * 512));
    } else {
      store_tile<OUT>(acc, xs, ws, bias, out, M, N, m0 + wm * C::TM, n0 + wn * C::TN, r16, lg, xs_stride, ws_stride);
    }
  };
  if (KT & 1) steps(T1{});
  else steps(F0{});
}

template <int XF, int WF, int OUT, int G>
hipError_t run_wide(const LinearArgs& a, hipStream_t stream) {
  using C = Tiled<256, 256, 2, 2, 3>;
  if (a.k < 4 * KSTEP) return hipErrorInvalidValue;  // the step sequence needs K >= 512
  const int tiles_m = (int)((a.m + 255) / 256), tiles_n = (int)((a.n + 255) / 256);
  const int T = tiles_m * tiles_n;
  const int grid = 8 * ((T + 7) / 8);
  auto kern = linear_wide_kernel<XF, WF, OUT, G>;
  constexpr int lds = C::LDS;
  static bool attr_set = false;  // benign race: every thread sets the same value
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), lds, stream, a.xq, a.xs, a.values, a.meta, a.ws,
                     a.bias, a.out, (int)a.m, (int)a.n, (int)a.k, tiles_m, tiles_n, a.xs_stride, a.ws_stride);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode kernel (M <= 16)
// ---------------------------------------------------------------------------
// NWV wavefronts per workgroup, each taking k steps wave, wave + NWV, ... (U of
// them per pass).  All of a pass's loads are issued before its first MFMA and
// nothing in between branches, so a wavefront has U * 4 loads in flight.
// Steps past the end re-read the last step (in bounds) and add a zero A operand.
template <int XF, int WF, int OUT, int ACC, int NWV, int U, bool NT = true>
__global__ __launch_bounds__(64 * NWV) void linear_decode_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xs, const uint8_t* __restrict__ values,
    const uint8_t* __restrict__ meta, const float* __restrict__ ws, const uint16_t* __restrict__ bias,
    void* __restrict__ out, int M, int N, int K, int xs_stride, int ws_stride) {
  __shared__ v4f red[NWV][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int KT = K / KSTEP;

  const uint8_t* vrow = values + (int64_t)(n0 + r16) * (K / 2) + 16 * lg;
  const uint8_t* mrow = meta + (int64_t)(n0 + r16) * (K / 8) + 4 * lg;
  const bool xon = r16 < M;
  const uint8_t* xrow = xq + (int64_t)min(r16, M - 1) * K + 16 * lg;
  const v4i z4 = v4i{0, 0, 0, 0};

  // epilogue operands, fetched up front so their latency hides under the stream
  const int m = r16, n = n0 + 4 * lg;
  float xsm = 0.f;
  v4f w4 = v4f{0.f, 0.f, 0.f, 0.f};
  uint2 b2 = make_uint2(0, 0);
  if (wave == 0) {
    xsm = xs[min(m, M - 1) * xs_stride];
    w4 = load_ws4(ws, n, ws_stride);
    if (bias) b2 = *reinterpret_cast<const uint2*>(bias + n);
  }

  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  for (int s0 = wave; s0 < KT; s0 += NWV * U) {
    v4i a[U], blo[U], bhi[U];
    int idx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t s = min(s0 + u * NWV, KT - 1);
      if constexpr (NT) {
        a[u] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(vrow + s * 64));
        idx[u] = __builtin_nontemporal_load(reinterpret_cast<const int*>(mrow + s * 16));
      } else {
        a[u] = *reinterpret_cast<const v4i*>(vrow + s * 64);
        idx[u] = *reinterpret_cast<const int*>(mrow + s * 16);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t s = min(s0 + u * NWV, KT - 1);
      blo[u] = *reinterpret_cast<const v4i*>(xrow + s * 128);
      bhi[u] = *reinterpret_cast<const v4i*>(xrow + s * 128 + 64);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every load of the pass ahead of the MFMAs
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = s0 + u * NWV < KT;
      const v4i av = live ? a[u] : z4;
      const v4i lo = xon ? blo[u] : z4, hi = xon ? bhi[u] : z4;
      const v8i b = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      acc = mma_step<XF, WF, ACC>(av, b, acc, idx[u]);
    }
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    v4f t = red[0][lane];
#pragma unroll
    for (int w = 1; w < NWV; ++w) t += red[w][lane];
    v4f y;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = t[i] * (xsm * w4[i]);
    if (bias) {
      y[0] += bf16_to_f32(b2.x & 0xFFFFu);
      y[1] += bf16_to_f32(b2.x >> 16);
      y[2] += bf16_to_f32(b2.y & 0xFFFFu);
      y[3] += bf16_to_f32(b2.y >> 16);
    }
    if (m < M) store4<OUT>(out, N, m, n, y);
  }
}

// b[s] = lanes 2s (low half) and 2s + 1 (high half) of each 16-lane row of x,
// broadcast to the row (DPP row_newbcast, control 0x150 + lane)
template <int S>
__device__ __forceinline__ v8i row_bcast_pair(const v4i& x) {
  v8i r;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    r[d] = __builtin_amdgcn_update_dpp(0, x[d], 0x150 + 2 * S, 0xF, 0xF, false);
    r[4 + d] = __builtin_amdgcn_update_dpp(0, x[d], 0x151 + 2 * S, 0xF, 0xF, false);
  }
  return r;
}
template <int... S>
__device__ __forceinline__ void row_bcast_steps(v8i (&b)[8], const v4i& x, std::integer_sequence<int, S...>) {
  ((b[S] = row_bcast_pair<S>(x)), ...);
}

// One unit's 8 MFMA steps for a single activation row: step S's operand is
// broadcast from x1 (row_bcast_pair<S>) just before its MFMA, so only one
// step's operand is live at a time.
template <int XF, int WF, int ACC, int S>
__device__ __forceinline__ void x1_step(v4f& acc0, v4f& acc1, const v4i& x1, const uint8_t* region, uint32_t a_even,
                                        uint32_t a_odd, uint32_t i_row, int r7) {
  const v4i a = *reinterpret_cast<const v4i*>(region + ((S & 1) ? a_odd : a_even) + 128 * (S >> 1));
  const int idx = *reinterpret_cast<const int*>(region + i_row + 16 * (S ^ r7));
  const v8i b = row_bcast_pair<S>(x1);
  if constexpr (S & 1) acc1 = mma_step<XF, WF, ACC>(a, b, acc1, idx);
  else acc0 = mma_step<XF, WF, ACC>(a, b, acc0, idx);
}
template <int XF, int WF, int ACC, int... S>
__device__ __forceinline__ void x1_unit(v4f& acc0, v4f& acc1, const v4i& x1, const uint8_t* region, uint32_t a_even,
                                        uint32_t a_odd, uint32_t i_row, int r7, std::integer_sequence<int, S...>) {
  (x1_step<XF, WF, ACC, S>(acc0, acc1, x1, region, a_even, a_odd, i_row, r7), ...);
}

// Decode kernel, one k unit per wavefront.  A workgroup owns RT * 16 weight
// rows and K / 1024 "units" of 1024 k (8 MFMA steps) each; wavefront w takes
// units w, w + NW, ...  For a unit it puts the unit's compressed values
// (512 contiguous bytes per row) and metadata (128 bytes per row) in flight
// into its own RT * 10 KB of LDS with 1 KB buffer->LDS loads, in two halves
// of 4 steps (unit_two_halves), and the activation operands of the unit's 8
// steps straight into registers (shared by the RT row tiles); it waits for
// the first half of its own loads only and runs those 4 * RT MFMAs while the
// second half lands, then the rest: no workgroup barrier before the final
// fixed-order reduction, so every wavefront computes as soon as its data is
// there while the others' loads stream.  LDS holds only the weight block, so
// several workgroups share a CU.  Each 16-byte chunk of a row is stored at
// chunk ^ (row & 7) (a permutation inside 128-byte groups, applied to the
// source addresses of each 1 KB load), which makes the MFMA-layout LDS reads
// conflict-free.  RT = 2 halves the activation traffic (every workgroup reads
// all of the activation) at half the workgroups.  Its 20 KB of LDS per
// wavefront allow at most two workgroups per CU with four or more wavefronts,
// so its register budget is that of two (256 per lane): the 64 registers of
// activation operands and the widened operands of the binary32-grade step
// then fit without spilling.
constexpr int kUnitK = 1024;
constexpr int kUnitLds = 16 * kUnitK / 2 + 16 * kUnitK / 8;  // 10 KB per 16 rows
enum { XM_DIRECT = 0, XM_ONE_ROW = 1, XM_PERMUTED = 2 };
constexpr int kHalfLds = kUnitLds / 2;  // one half unit (4 steps) of 16 rows: 4 KB values + 1 KB metadata

// Offsets of the unit kernel's two-half layout.  Half h of a unit (its steps
// 4h .. 4h + 3) of row tile t sits at (h * RT + t) * kHalfLds of the
// wavefront's region: 16 rows x 256 bytes of values, then 16 rows x 64 bytes
// of metadata.  Values load i (0..3) of a half brings rows 4i .. 4i + 3, lane
// L the row's 16-byte chunk (L % 16) ^ (row & 7) (row & 7 = 4 (i & 1) + L / 16)
// to 16 L; the metadata load brings row L / 4, step (L % 4) ^ (row & 3) of the
// half.  Reads of step s (s4 = s % 4): lane (r16, lg) finds values chunk
// 4 s4 + lg of row r16 at chunk (4 s4 + lg) ^ (r16 & 7) and the metadata of
// step s4 at chunk s4 ^ (r16 & 3), which keeps the 128-bit reads of 8
// consecutive rows on distinct banks.
struct UnitHalfOffsets {
  uint32_t voff[2], moff, a_even, a_odd, i_row;
  int r3;
  __device__ UnitHalfOffsets(int lane, int K) {
    const int r16 = lane & 15, lg = lane >> 4, r7 = r16 & 7;
#pragma unroll
    for (int p = 0; p < 2; ++p)
      voff[p] = (uint32_t)((lane >> 4) * (K / 2) + 16 * ((lane & 15) ^ (4 * p + (lane >> 4))));
    moff = (uint32_t)((lane >> 2) * (K / 8) + 16 * ((lane & 3) ^ ((lane >> 2) & 3)));
    a_even = r16 * 256 + 16 * ((4 * ((r7 >> 2) & 1)) | (lg ^ (r7 & 3)));
    a_odd = r16 * 256 + 16 * ((4 * (((r7 >> 2) & 1) ^ 1)) | (lg ^ (r7 & 3)));
    i_row = 4096 + r16 * 64 + 4 * lg;
    r3 = r16 & 3;
  }
};

// Global -> LDS loads of half h of unit u0 for RT row tiles into hb, through
// buffer descriptors of the workgroup's weight rows (rv: values, rm:
// metadata): the lane offsets stay in fixed registers and everything else is
// a scalar offset.
template <int RT>
__device__ __forceinline__ void unit_half_loads(uint8_t* __restrict__ hb, __amdgpu_buffer_rsrc_t rv,
                                                __amdgpu_buffer_rsrc_t rm, const UnitHalfOffsets& o, int u0, int h,
                                                int K) {
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    uint8_t* dst = hb + t * kHalfLds;
    const int sv = 16 * t * (K / 2) + u0 * (kUnitK / 2) + 256 * h;
#pragma unroll
    for (int i = 0; i < 4; ++i) buffer_lds16(rv, dst + i * 1024, (int)o.voff[i & 1], sv + 4 * i * (K / 2));
    buffer_lds16(rm, dst + 4096, (int)o.moff, 16 * t * (K / 8) + u0 * (kUnitK / 8) + 64 * h);
  }
}

// b[d] = the value b[d] of lane xsrc / 4, for the 8 words of one step's
// activation (ds_bpermute), with the wait for the results in the same block.
// Written as assembly because the compiler treats its own lane permutation as
// an LDS access and would make it wait for every global->LDS load in flight,
// including those of the unit's second half; the permutation neither reads
// nor writes LDS memory.
__device__ __forceinline__ void bpermute8(v8i& b, int xsrc) {
  int r0, r1, r2, r3, r4, r5, r6, r7;
  asm volatile(
      "ds_bpermute_b32 %0, %8, %9\n\t"
      "ds_bpermute_b32 %1, %8, %10\n\t"
      "ds_bpermute_b32 %2, %8, %11\n\t"
      "ds_bpermute_b32 %3, %8, %12\n\t"
      "ds_bpermute_b32 %4, %8, %13\n\t"
      "ds_bpermute_b32 %5, %8, %14\n\t"
      "ds_bpermute_b32 %6, %8, %15\n\t"
      "ds_bpermute_b32 %7, %8, %16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
      : "v"(xsrc), "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]), "v"(b[4]), "v"(b[5]), "v"(b[6]), "v"(b[7]));
  b = v8i{r0, r1, r2, r3, r4, r5, r6, r7};
}

// Steps S0 .. S0 + 3 of a unit from half hb (RT row tiles), activation b.
template <int XF, int WF, int ACC, int RT, int XM, int S0>
__device__ __forceinline__ void unit_half_steps(const uint8_t* __restrict__ hb, v8i (&b)[8], v4f (&acc0)[RT],
                                                v4f (&acc1)[RT], const UnitHalfOffsets& o, int xsrc) {
#pragma unroll
  for (int s = S0; s < S0 + 4; ++s) {
    const int s4 = s & 3;
    if constexpr (XM == XM_PERMUTED) bpermute8(b[s], xsrc);
    if constexpr (ACC == ACC_F32) {
      // the activation half widened once for the RT row tiles
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const v8i bw = hh ? widen_b_half<XF, 1>(b[s]) : widen_b_half<XF, 0>(b[s]);
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const uint8_t* rt = hb + t * kHalfLds;
          const v4i a = *reinterpret_cast<const v4i*>(rt + ((s4 & 1) ? o.a_odd : o.a_even) + 128 * (s4 >> 1));
          const int idx = *reinterpret_cast<const int*>(rt + o.i_row + 16 * (s4 ^ o.r3));
          const v4i aw = hh ? widen_a_half<WF, 1>(a) : widen_a_half<WF, 0>(a);
          const int ix = hh ? idx_half<1>(idx) : idx_half<0>(idx);
          if (s & 1) acc1[t] = smfmac16_bf16(aw, bw, acc1[t], ix);
          else acc0[t] = smfmac16_bf16(aw, bw, acc0[t], ix);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const uint8_t* rt = hb + t * kHalfLds;
        const v4i a = *reinterpret_cast<const v4i*>(rt + ((s4 & 1) ? o.a_odd : o.a_even) + 128 * (s4 >> 1));
        const int idx = *reinterpret_cast<const int*>(rt + o.i_row + 16 * (s4 ^ o.r3));
        if (s & 1) acc1[t] = smfmac16<XF, WF>(a, b[s], acc1[t], idx);
        else acc0[t] = smfmac16<XF, WF>(a, b[s], acc0[t], idx);
      }
    }
  }
}

// One unit of the unit kernel in two halves: the loads of half 0 (and the
// activation of its steps) go out before those of half 1, so the wavefront
// computes steps 0-3 while the rest of its block is still in flight
// (measured against one wait for the whole unit: 0.45-0.87 us faster at
// M = 4 and 16 on the Llama shapes, the same at M = 1).  h0 and h1 are
// restrict parameters of an inlined function, so the compiler can tell the
// reads of half 0 from the pending loads of half 1 and waits for half 0
// alone.
template <int XF, int WF, int ACC, int RT, int XM>
__device__ __forceinline__ void unit_two_halves(uint8_t* __restrict__ h0, uint8_t* __restrict__ h1,
                                                __amdgpu_buffer_rsrc_t rv, __amdgpu_buffer_rsrc_t rm,
                                                const uint8_t* __restrict__ xq, const uint8_t* xrow,
                                                const UnitHalfOffsets& o, int u0, int K, int r16, int lg, int xsrc,
                                                v4f (&acc0)[RT], v4f (&acc1)[RT]) {
  v8i b[8];
  v4i x1;
  if constexpr (XM == XM_ONE_ROW) {
    // one activation row: lane (r16, lg) holds chunk 8 (r16 >> 1) + 4 (r16 & 1) + lg
    // of the unit, i.e. the half r16 & 1 of step r16 >> 1 that lane group lg needs
    x1 = *reinterpret_cast<const v4i*>(xq + u0 * kUnitK + 128 * (r16 >> 1) + 64 * (r16 & 1) + 16 * lg);
    // the memory clobbers keep the issue order the counts below assume
    asm volatile("" ::: "memory");
    unit_half_loads<RT>(h0, rv, rm, o, u0, 0, K);
    asm volatile("" ::: "memory");
    unit_half_loads<RT>(h1, rv, rm, o, u0, 1, K);
    asm volatile("" ::: "memory");
    wait_vmcnt<5 * RT>();  // x1 and half 0 have landed
    __builtin_amdgcn_sched_barrier(0);
    // step s's operand: lanes 2s and 2s + 1 of each 16-lane row, broadcast
    // to the whole row (DPP row_newbcast)
    row_bcast_steps(b, x1, std::make_integer_sequence<int, 8>{});
  } else {
    const uint8_t* xp = xrow + u0 * kUnitK;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int s = 4 * hf; s < 4 * hf + 4; ++s) {
        const v4i l = *reinterpret_cast<const v4i*>(xp + s * 128);
        const v4i h = *reinterpret_cast<const v4i*>(xp + s * 128 + 64);
        b[s] = __builtin_shufflevector(l, h, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      // the memory clobbers keep the issue order the counts below assume
      asm volatile("" ::: "memory");
      unit_half_loads<RT>(hf ? h1 : h0, rv, rm, o, u0, hf, K);
      asm volatile("" ::: "memory");
    }
    // nothing that uses the loaded operands (the lane permutations included)
    // moves above this point
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<8 + 5 * RT>();  // the activation of steps 0-3 and half 0 have landed
    __builtin_amdgcn_sched_barrier(0);
  }
  unit_half_steps<XF, WF, ACC, RT, XM, 0>(h0, b, acc0, acc1, o, xsrc);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<0>();
  __builtin_amdgcn_sched_barrier(0);
  unit_half_steps<XF, WF, ACC, RT, XM, 4>(h1, b, acc0, acc1, o, xsrc);
}
template <int XF, int WF, int OUT, int ACC, int RT, int XM, int MAXW = 8>
__global__ __launch_bounds__(64 * MAXW, RT == 1 ? 4 : 2) void linear_decode_unit_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xs, const uint8_t* __restrict__ values,
    const uint8_t* __restrict__ meta, const float* __restrict__ ws, const uint16_t* __restrict__ bias,
    void* __restrict__ out, int M, int N, int K, int xs_stride, int ws_stride) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NW = blockDim.x / 64;
  const int r16 = lane & 15, lg = lane >> 4;
  const int NU = K / kUnitK;
  uint8_t* region = smem + wave * (RT * kUnitLds);
  const UnitHalfOffsets o(lane, K);
  // workgroup row blockIdx.y takes activation rows mb .. mb + 15 (M up to
  // 64: the weight block is read once per 16 rows, mostly from L2).  Rows
  // past the last, Mc, read row Mc - 1: MFMA output column m depends on
  // activation row m alone, and those columns are never stored.
  // Activation loads (XM): XM_ONE_ROW, M == 1: one 16-byte chunk per lane,
  // broadcast per step (below).  XM_DIRECT: in the MFMA layout (lane (m, g):
  // row m, chunk g), sixteen rows under sixteen neighbouring lanes, which the
  // vector memory unit serves as one cache access per lane.  XM_PERMUTED:
  // row-contiguously (lane L: row L / 4, chunk L % 4 of each 64-byte half
  // step, four neighbouring lanes on one 64-byte run), then moved into the
  // MFMA layout by a lane permutation (ds_bpermute, eight per step); it pays
  // for itself when most of the 16 rows are distinct (measured: M = 16
  // faster by up to 1.9 us, M = 4 slower by 0.4-0.8 us than XM_DIRECT).
  const int mb = blockIdx.y * 16, Mc = min(M - mb, 16);
  const uint8_t* xrow =
      XM == XM_PERMUTED ? xq + (int64_t)(mb + min(lane >> 2, Mc - 1)) * K + 16 * (lane & 3)
                        : xq + (int64_t)(mb + min(r16, Mc - 1)) * K + 16 * lg;
  const int xsrc = 4 * (4 * r16 + lg);  // byte address of the source lane of (r16, lg)

  const int m = r16;
  float xsm = 0.f;
  v4f w4[RT];
  uint2 b2[RT];
  if (wave == 0) {
    xsm = xs[(mb + min(m, Mc - 1)) * xs_stride];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int n = (blockIdx.x * RT + t) * 16 + 4 * lg;
      w4[t] = load_ws4(ws, n, ws_stride);
      b2[t] = bias ? *reinterpret_cast<const uint2*>(bias + n) : make_uint2(0, 0);
    }
  }

  v4f acc0[RT], acc1[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc0[t] = acc1[t] = v4f{0.f, 0.f, 0.f, 0.f};
  // the workgroup's RT * 16 weight rows (N is a multiple of 16 RT)
  const int64_t n0 = (int64_t)blockIdx.x * RT * 16;
  const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(values + n0 * (K / 2), RT * 16 * (K / 2));
  const __amdgpu_buffer_rsrc_t rm = buffer_rsrc(meta + n0 * (K / 8), RT * 16 * (K / 8));
  for (int u0 = wave; u0 < NU; u0 += NW) {
    unit_two_halves<XF, WF, ACC, RT, XM>(region, region + RT * kHalfLds, rv, rm, xq, xrow, o, u0, K, r16, lg, xsrc,
                                         acc0, acc1);
    // the region's reads are complete (their values fed the MFMAs) before
    // the next unit's loads overwrite it
    __builtin_amdgcn_s_waitcnt(0xC07F);
  }
  // fixed-order reduction: each wavefront's partial tiles into its own region
#pragma unroll
  for (int t = 0; t < RT; ++t) reinterpret_cast<v4f*>(region)[t * 64 + lane] = acc0[t] + acc1[t];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      v4f sum = reinterpret_cast<const v4f*>(smem)[t * 64 + lane];
      for (int w = 1; w < NW; ++w) sum += reinterpret_cast<const v4f*>(smem + w * (RT * kUnitLds))[t * 64 + lane];
      v4f y;
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = sum[i] * (xsm * w4[t][i]);
      if (bias) {
        y[0] += bf16_to_f32(b2[t].x & 0xFFFFu);
        y[1] += bf16_to_f32(b2[t].x >> 16);
        y[2] += bf16_to_f32(b2[t].y & 0xFFFFu);
        y[3] += bf16_to_f32(b2[t].y >> 16);
      }
      if (m < Mc) store4<OUT>(out, N, mb + m, (blockIdx.x * RT + t) * 16 + 4 * lg, y);
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel configurations ("algorithms") and the default choice by shape
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------
template <int XF, int WF, int OUT, int ACC, int BN, int BM, int WN, int WM, int G, int S, int ORD = 0, int OCC = 1,
          int MB = 0, int NT = 0>
hipError_t run_tiled(const LinearArgs& a, hipStream_t stream) {
  using C = Tiled<BN, BM, WN, WM, S, MB>;
  const int tiles_m = (int)((a.m + BM - 1) / BM), tiles_n = (int)((a.n + BN - 1) / BN);
  const int T = tiles_m * tiles_n;
  const int grid = 8 * ((T + 7) / 8);
  auto kern = linear_tiled_kernel<XF, WF, OUT, BN, BM, WN, WM, G, S, ORD, OCC, MB, NT, ACC>;
  static bool attr_set = false;  // benign race: every thread sets the same value
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), C::LDS, stream, a.xq, a.xs, a.values, a.meta, a.ws,
                     a.bias, a.out, (int)a.m, (int)a.n, (int)a.k, tiles_m, tiles_n, a.xs_stride, a.ws_stride);
  return hipGetLastError();
}

// The persistent kernel needs every per-tile offset in 32 bits.
inline bool persistent_ok(const LinearArgs& a, int tile) { return a.k * tile < ((int64_t)1 << 31); }

// Compute units of the current device (cached per device).
inline int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 8) c = 256;
    cus[dev] = c;  // benign race: every thread stores the same value
  }
  return cus[dev];
}

// Deep-pipeline form of a tiled configuration: at most `per_cu` tiles of
// tile x tile per compute unit and K >= min_k.
inline bool tiled_deep(const LinearArgs& a, int tile, int per_cu, int64_t min_k) {
  const int64_t tiles = ((a.m + tile - 1) / tile) * ((a.n + tile - 1) / tile);
  return a.k >= min_k && tiles <= (int64_t)per_cu * device_cus();
}

template <int XF, int WF, int OUT, int ACC, int BN, int BM, int WN, int WM, int NL, int G, int OCC, int NT = 0>
hipError_t run_persistent(const LinearArgs& a, hipStream_t stream) {
  using C = Tiled<BN, BM, WN, WM, 2, 8>;
  const int tiles_m = (int)((a.m + BM - 1) / BM), tiles_n = (int)((a.n + BN - 1) / BN);
  const int T = tiles_m * tiles_n;
  // a multiple of 8 workgroups (the XCD mapping), at most OCC per CU
  const int grid = std::max(8, std::min(8 * ((T + 7) / 8), (OCC * device_cus() / 8) * 8));
  auto kern = linear_persistent_kernel<XF, WF, OUT, ACC, BN, BM, WN, WM, NL, G, OCC, NT>;
  static bool attr_set = false;  // benign race: every thread sets the same value
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), C::LDS, stream, a.xq, a.xs, a.values, a.meta, a.ws, a.bias, a.out,
                     (int)a.m, (int)a.n, (int)a.k, tiles_m, tiles_n, a.xs_stride, a.ws_stride);
  return hipGetLastError();
}

// Wavefronts per workgroup of the unit decode kernel: the K / 1024 units
// spread evenly over at most 8 wavefronts.
inline int unit_waves(int64_t k, int maxw = 8) {
  const int nu = (int)(k / kUnitK), per = (nu + maxw - 1) / maxw;
  return (nu + per - 1) / per;
}

// Wavefronts per workgroup of the unit kernel: at most 8, so that several
// workgroups share a CU.  Up to 16 (one unit per wavefront up to K = 16384,
// 160 KB of LDS at most) for the binary32-grade step with 16 weight rows and
// 2..16 activation rows per workgroup, more than 8 units of K and workgroups
// that all fit on the CUs at once: the widening work after each wavefront's
// wait is then spread over twice the wavefronts instead of following a
// second unit's wait.  Measured on the down projection (N = 4096,
// K = 14336): M = 16 12.41 -> 11.75 us, M = 4 10.75 -> 10.68 us; one row
// (the broadcast form, little work per unit) 9.23 -> 9.46 us, and FP8
// accumulation (no widening) 11.92 -> 12.02 us at M = 16, so those keep 8.
template <int RT, int ACC, int XM>
inline int unit_max_waves(const LinearArgs& a) {
  if (RT != 1 || ACC != ACC_F32 || XM == XM_ONE_ROW || a.k <= 8 * kUnitK) return 8;
  return (a.n / 16) * ((a.m + 15) / 16) <= device_cus() ? 16 : 8;
}

template <int XF, int WF, int OUT, int ACC, int RT, int XM, int MAXW>
hipError_t run_decode_unit_waves(const LinearArgs& a, hipStream_t stream) {
  auto kern = linear_decode_unit_kernel<XF, WF, OUT, ACC, RT, XM, MAXW>;
  const int nw = unit_waves(a.k, MAXW);
  const unsigned lds = (unsigned)(nw * RT * kUnitLds);
  static bool attr_set = false;  // benign race: every thread sets the same value
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, MAXW * RT * kUnitLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)(a.n / (16 * RT)), (unsigned)((a.m + 15) / 16)), dim3(64 * nw), lds, stream,
                     a.xq, a.xs, a.values,
                     a.meta, a.ws, a.bias, a.out, (int)a.m, (int)a.n, (int)a.k, a.xs_stride, a.ws_stride);
  return hipGetLastError();
}

template <int XF, int WF, int OUT, int ACC, int RT, int XM>
hipError_t run_decode_unit_cfg(const LinearArgs& a, hipStream_t stream) {
  if constexpr (RT == 1 && ACC == ACC_F32 && XM != XM_ONE_ROW) {
    if (unit_max_waves<RT, ACC, XM>(a) == 16) return run_decode_unit_waves<XF, WF, OUT, ACC, RT, XM, 16>(a, stream);
  }
  return run_decode_unit_waves<XF, WF, OUT, ACC, RT, XM, 8>(a, stream);
}

template <int XF, int WF, int OUT, int ACC, int RT>
hipError_t run_decode_unit(const LinearArgs& a, hipStream_t stream) {
  // the permuted activation loads above 8 rows on the shapes whose weight
  // stream is long enough to hide the permutation (measured on the Llama
  // shapes at M = 16 with the two-half units: 0.2-0.7 us faster at
  // N = 14336 or K = 14336, 0.19 us slower at N = 6144, K = 4096)
  if (a.m == 1) return run_decode_unit_cfg<XF, WF, OUT, ACC, RT, XM_ONE_ROW>(a, stream);
  if (a.m <= 8 || (a.n < 8192 && a.k < 8192)) return run_decode_unit_cfg<XF, WF, OUT, ACC, RT, XM_DIRECT>(a, stream);
  return run_decode_unit_cfg<XF, WF, OUT, ACC, RT, XM_PERMUTED>(a, stream);
}

// ---------------------------------------------------------------------------
// Decode from the bf16 activation, 1 to 4 rows: quantization fused in front
// of the unit kernel.
// ---------------------------------------------------------------------------
// linear_decode_unit_kernel's units, LDS regions and reduction, for MR = 1, 2
// or 4 activation rows that the kernel first quantizes itself, exactly as
// quantize_rowwise_fp8 does.  Every wavefront puts the bf16 chunks of its
// units (each row's, for lane (r, g) the 16 elements 8 (r >> 1) + 4 (r & 1)
// + g of a unit) and then its first unit's weight block in flight, all as
// global->LDS loads (fused_first_loads), and reads the chunks back once only
// the weight loads are pending.  Each row's maximum (over lanes by DPP, over
// wavefronts through LDS; every wavefront reading the whole row instead
// measured slower), the scales, their reciprocals and cast8 follow; the LDS
// exchange waits for the weight block too (any LDS access waits for pending
// global->LDS loads), so the casts run a few hundred cycles after the
// stream, against a second launch.  With one row the codes stay in
// registers and each step broadcasts its operand across the 16-lane rows
// (x1_unit); with several, each row's codes go back to the wavefront's
// staging area and each lane reads its own row's operand there (xl_unit).
// Workgroup 0 also writes the codes and the scales to xq / xs.  Every
// workgroup repeats the casts of all its rows, which is why the host takes
// this path only for few rows and workgroups (fused_decode_ok).  A
// wavefront holds at most 2 units of the activation (K <= 16384 with 8
// wavefronts).
constexpr int kFusedMaxUnitsPerWave = 2;
constexpr int kCodeRow = kUnitK + 16;  // LDS stride of a row's codes (several rows)

// First loads of the fused decode kernel: the wavefront's activation chunks
// (global -> LDS into xl), then its first unit's weight block (into wl), a
// wait until only the weight loads are pending, and the activation chunks
// read back.  xl and wl are restrict parameters of an inlined function, so
// the compiler can tell the activation reads from the pending weight loads
// and does not make them wait for the whole stream.
template <int UPW, int MR>
__device__ __forceinline__ void fused_first_loads(uint8_t* __restrict__ xl, uint8_t* __restrict__ wl,
                                                  const uint16_t* __restrict__ x, const uint8_t* vu, const uint8_t* mu,
                                                  const uint32_t (&voff)[4], uint32_t moff, int M, int K, int NU,
                                                  int wave, int NW, int xoff, int lane, uint4 (&xa)[UPW][MR][2]) {
#pragma unroll
  for (int c = 0; c < UPW; ++c) {
    const int u0 = min(wave + c * NW, NU - 1);
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      const uint16_t* xr = x + (int64_t)min(r, M - 1) * K + (int64_t)u0 * kUnitK + xoff;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        __builtin_amdgcn_global_load_lds((void*)(xr + 8 * h), (void*)(xl + ((c * MR + r) * 2 + h) * 1024), 16, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
    __builtin_amdgcn_global_load_lds((void*)(vu + (int64_t)i * K + voff[i & 3]), (void*)(wl + i * 1024), 16, 0, 0);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    __builtin_amdgcn_global_load_lds((void*)(mu + (int64_t)i * K + moff), (void*)(wl + 8192 + i * 1024), 16, 0, 0);
  wait_vmcnt<10>();
#pragma unroll
  for (int c = 0; c < UPW; ++c)
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
      for (int h = 0; h < 2; ++h) xa[c][r][h] = reinterpret_cast<const uint4*>(xl + ((c * MR + r) * 2 + h) * 1024)[lane];
}

// Step S of a unit for several activation rows: lane (m, g) reads its row's
// operand (the codes 128 S + 16 g and 128 S + 64 + 16 g of the unit, as
// row_bcast_pair would broadcast them) from the codes the wavefront stored in
// LDS; cb points at the lane's row of the unit, offset by 16 g.
template <int XF, int WF, int ACC, int S>
__device__ __forceinline__ void xl_step(v4f& acc0, v4f& acc1, const uint8_t* cb, const uint8_t* region,
                                        uint32_t a_even, uint32_t a_odd, uint32_t i_row, int r7) {
  const v4i a = *reinterpret_cast<const v4i*>(region + ((S & 1) ? a_odd : a_even) + 128 * (S >> 1));
  const int idx = *reinterpret_cast<const int*>(region + i_row + 16 * (S ^ r7));
  const v4i lo = *reinterpret_cast<const v4i*>(cb + 128 * S);
  const v4i hi = *reinterpret_cast<const v4i*>(cb + 128 * S + 64);
  const v8i b = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  if constexpr (S & 1) acc1 = mma_step<XF, WF, ACC>(a, b, acc1, idx);
  else acc0 = mma_step<XF, WF, ACC>(a, b, acc0, idx);
}
template <int XF, int WF, int ACC, int... S>
__device__ __forceinline__ void xl_unit(v4f& acc0, v4f& acc1, const uint8_t* cb, const uint8_t* region,
                                        uint32_t a_even, uint32_t a_odd, uint32_t i_row, int r7,
                                        std::integer_sequence<int, S...>) {
  (xl_step<XF, WF, ACC, S>(acc0, acc1, cb, region, a_even, a_odd, i_row, r7), ...);
}

template <int XF, int WF, int OUT, int ACC, int NWMAX, int MR>
__global__ __launch_bounds__(64 * NWMAX, NWMAX <= 4 ? 4 : 2) void linear_decode_unit_fused1_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ xq, float* __restrict__ xs,
    const uint8_t* __restrict__ values, const uint8_t* __restrict__ meta, const float* __restrict__ ws,
    const uint16_t* __restrict__ bias, void* __restrict__ out, int M, int N, int K, int ws_stride) {
  // dynamic LDS: the weight regions, then the activation chunks, then the
  // wavefront maxima
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  // a wavefront holds 2 units with 8 wavefronts (K up to 16384; 1 or 2 rows)
  static_assert(MR < 4 || NWMAX <= 4, "3 or 4 rows: K up to 4096");
  constexpr int UPW0 = NWMAX == 8 ? kFusedMaxUnitsPerWave : 1;
  static_assert((UPW0 * MR - 1) * kCodeRow + kUnitK <= UPW0 * MR * 2048, "codes fit the staging area");
  uint8_t* xbase = smem + NWMAX * kUnitLds;
  uint32_t* wmax = reinterpret_cast<uint32_t*>(xbase + NWMAX * UPW0 * MR * 2048);  // [NW][MR]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NW = blockDim.x / 64;
  const int r16 = lane & 15, lg = lane >> 4;
  const int NU = K / kUnitK;
  // this wavefront's units: 1, or 2 when there are more units than 8 wavefronts
  constexpr int UPW = UPW0;
  const int nuw = (NU - wave + NW - 1) / NW;
  uint8_t* region = smem + wave * kUnitLds;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int vrow_l = lane >> 5, vc = lane & 31, mrow_l = lane >> 3, mc = lane & 7;
  uint32_t voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = (uint32_t)(vrow_l * (K / 2) + 16 * (vc ^ ((2 * i + vrow_l) & 7)));
  const uint32_t moff = (uint32_t)(mrow_l * (K / 8) + 16 * (mc ^ (mrow_l & 7)));
  const int r7 = r16 & 7;
  const uint32_t a_even = r16 * 512 + 16 * ((4 * ((r7 >> 2) & 1)) | (lg ^ (r7 & 3)));
  const uint32_t a_odd = r16 * 512 + 16 * ((4 * (((r7 >> 2) & 1) ^ 1)) | (lg ^ (r7 & 3)));
  const uint32_t i_row = 8192 + r16 * 128 + 4 * lg;
  // this lane's 16 activation elements of a unit (and its 16 code bytes)
  const int xoff = 128 * (r16 >> 1) + 64 * (r16 & 1) + 16 * lg;

  auto dma = [&](int u0) __attribute__((always_inline)) {
    const uint8_t* vu = values + n0 * (K / 2) + u0 * (kUnitK / 2);
    const uint8_t* mu = meta + n0 * (K / 8) + u0 * (kUnitK / 8);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_global_load_lds((void*)(vu + (int64_t)i * K + voff[i & 3]), (void*)(region + i * 1024), 16, 0,
                                       0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_global_load_lds((void*)(mu + (int64_t)i * K + moff), (void*)(region + 8192 + i * 1024), 16, 0,
                                       0);
  };

  // 1. epilogue operands, the activation of this wavefront's units, then the
  // first unit's weight loads
  const int n = (int)n0 + 4 * lg;
  v4f w4 = v4f{0.f, 0.f, 0.f, 0.f};
  uint2 b2 = make_uint2(0, 0);
  if (wave == 0) {
    w4 = load_ws4(ws, n, ws_stride);
    if (bias) b2 = *reinterpret_cast<const uint2*>(bias + n);
  }
  // the activation chunks by global->LDS loads too (lane l's 16 bytes at
  // 16 l of each 1 KB), issued before the weight loads: all pending loads are
  // then of one kind and complete in issue order, so once at most the weight
  // loads are pending (vmcnt(10)) the activation has landed
  uint4 xa[UPW][MR][2];
  uint8_t* xw = xbase + wave * UPW0 * MR * 2048;
  fused_first_loads<UPW, MR>(xw, region, x, values + n0 * (K / 2) + wave * (kUnitK / 2),
                             meta + n0 * (K / 8) + wave * (kUnitK / 8), voff, moff, M, K, NU, wave, NW, xoff, lane,
                             xa);

  // 2. each row's maximum over lanes, then wavefronts
  uint32_t mx[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    mx[r] = 0;
#pragma unroll
    for (int c = 0; c < UPW; ++c)
      if (c < nuw) mx[r] = mag_max8(xa[c][r][1], mag_max8(xa[c][r][0], mx[r]));
    mx[r] = wave_max(mx[r]);
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < MR; ++r) wmax[wave * MR + r] = mx[r];
  }
  lds_barrier();
  float sc[MR], rc[MR];
  bool zr[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    uint32_t mm = wmax[r];
    for (int w = 1; w < NW; ++w) mm = max(mm, wmax[w * MR + r]);
    zr[r] = mm == 0;
    sc[r] = bf16_to_f32(mm) / Fp8<XF>::fmax;
    rc[r] = 1.0f / sc[r];
  }

  // 3. codes of this wavefront's units (workgroup 0 also stores them)
  v4i x1[UPW][MR];
  const bool out0 = blockIdx.x == 0;
#pragma unroll
  for (int c = 0; c < UPW; ++c) {
    if (c < nuw) {
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        const uint2 lo = zr[r] ? zero8(xa[c][r][0]) : cast8<XF>(xa[c][r][0], sc[r], rc[r]);
        const uint2 hi = zr[r] ? zero8(xa[c][r][1]) : cast8<XF>(xa[c][r][1], sc[r], rc[r]);
        x1[c][r] = v4i{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
        if (out0 && r < M) *reinterpret_cast<v4i*>(xq + (int64_t)r * K + (wave + c * NW) * kUnitK + xoff) = x1[c][r];
        // several rows: the codes go to this wavefront's staging area (its
        // bf16 chunks are already in registers), in k order per row and unit,
        // rows 1040 bytes apart so that the rows' operand reads of a step
        // fall in different LDS banks
        if constexpr (MR > 1) *reinterpret_cast<v4i*>(xw + (c * MR + r) * kCodeRow + xoff) = x1[c][r];
      }
    }
  }
  // lane (m, g) scales output column m by row min(m, MR - 1)'s scale
  float xsm = zr[0] ? 0.0f : sc[0];
#pragma unroll
  for (int r = 1; r < MR; ++r)
    if (r == MR - 1 ? r16 >= r : r16 == r) xsm = zr[r] ? 0.0f : sc[r];
  if (out0 && tid < M) {
    float v = zr[0] ? 0.0f : sc[0];
#pragma unroll
    for (int r = 1; r < MR; ++r)
      if (tid == r) v = zr[r] ? 0.0f : sc[r];
    xs[tid] = v;
  }

  // 4. the units: weight block in LDS, the codes broadcast per step, MFMAs
  v4f acc0 = v4f{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
  for (int c = 0; c < UPW; ++c) {
    if (c < nuw) {
      if (c > 0) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // the previous unit's LDS reads are done
        dma(wave + c * NW);
      }
      wait_vmcnt<0>();
      if constexpr (MR == 1)
        x1_unit<XF, WF, ACC>(acc0, acc1, x1[c][0], region, a_even, a_odd, i_row, r7,
                             std::make_integer_sequence<int, 8>{});
      else
        xl_unit<XF, WF, ACC>(acc0, acc1, xw + (c * MR + min(r16, MR - 1)) * kCodeRow + 16 * lg, region, a_even, a_odd,
                             i_row, r7, std::make_integer_sequence<int, 8>{});
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  // 5. fixed-order reduction of the partial tiles, epilogue
  reinterpret_cast<v4f*>(region)[lane] = acc0 + acc1;
  __syncthreads();
  if (wave == 0) {
    v4f t = reinterpret_cast<const v4f*>(smem)[lane];
    for (int w = 1; w < NW; ++w) t += reinterpret_cast<const v4f*>(smem + w * kUnitLds)[lane];
    v4f y;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = t[i] * (xsm * w4[i]);
    if (bias) {
      y[0] += bf16_to_f32(b2.x & 0xFFFFu);
      y[1] += bf16_to_f32(b2.x >> 16);
      y[2] += bf16_to_f32(b2.y & 0xFFFFu);
      y[3] += bf16_to_f32(b2.y >> 16);
    }
    if (r16 < M) store4<OUT>(out, N, r16, n, y);
  }
}

// Fused path of the bf16-activation entry point, where one launch beats
// quantization + linear layer (measured against them on the Llama shapes,
// N 4096 .. 14336, K 4096 .. 14336, 1 .. 4 rows: one launch 0.9 .. 2.1 us
// faster where chosen).  Every workgroup quantizes all the rows it uses, so
// the redundant casts grow with rows x workgroups; above K = 4096 the 8
// wavefronts' weight blocks and activation chunks take most of the LDS, one
// workgroup per CU.
//  - 1 or 2 rows, K a multiple of 1024: up to 4096 always; up to 16384 while
//    the workgroups (16 weight rows each) fit the CUs once (at N = 6144,
//    K = 8192 two launches were 1.6 .. 2.8 us faster);
//  - 3 or 4 rows: K up to 4096 and workgroups that fit the CUs once (at
//    N = 4096 one launch is 0.15 us faster; at 6144, 14336 and K = 8192 two
//    launches are faster: 8.67 against 9.35 us at N = 6144 since the unit
//    kernel computes the first half of each unit while the second lands).
inline int fused_rows(int64_t m) { return m == 1 ? 1 : m == 2 ? 2 : 4; }
inline bool fused_decode_ok(int64_t m, int64_t n, int64_t k) {
  if (m < 1 || m > 4 || k % kUnitK != 0) return false;
  const int64_t wgs = n / 16, cus = device_cus();
  if (m <= 2) return k <= 4 * kUnitK || (k <= 16 * kUnitK && wgs <= cus);
  return k <= 4 * kUnitK && wgs <= cus;
}

template <int XF, int WF, int OUT, int ACC, int NWMAX, int MR>
hipError_t run_decode_fused_nw(const uint16_t* x, uint8_t* xq, float* xs, const LinearArgs& a, int nw,
                               hipStream_t stream) {
  constexpr int UPW = NWMAX == 8 ? kFusedMaxUnitsPerWave : 1;
  constexpr unsigned lds = NWMAX * kUnitLds + NWMAX * UPW * MR * 2048 + 4 * NWMAX * MR;
  static_assert(lds <= 160 * 1024, "LDS");
  auto kern = linear_decode_unit_fused1_kernel<XF, WF, OUT, ACC, NWMAX, MR>;
  static bool attr_set = false;  // benign race: every thread sets the same value
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)(a.n / 16)), dim3(64 * nw), lds, stream, x, xq, xs, a.values, a.meta, a.ws,
                     a.bias, a.out, (int)a.m, (int)a.n, (int)a.k, a.ws_stride);
  return hipGetLastError();
}

template <int XF, int WF, int OUT, int ACC, int MR>
hipError_t run_decode_fused_rows(const uint16_t* x, uint8_t* xq, float* xs, const LinearArgs& a, hipStream_t stream) {
  // the static LDS is sized for the smallest of 2, 4, 8 wavefronts that covers
  // the units, so small K keeps several workgroups per CU
  const int nw = unit_waves(a.k);
  if (nw <= 2) return run_decode_fused_nw<XF, WF, OUT, ACC, 2, MR>(x, xq, xs, a, nw, stream);
  if (nw <= 4) return run_decode_fused_nw<XF, WF, OUT, ACC, 4, MR>(x, xq, xs, a, nw, stream);
  if constexpr (MR < 4) return run_decode_fused_nw<XF, WF, OUT, ACC, 8, MR>(x, xq, xs, a, nw, stream);
  return hipErrorInvalidValue;  // 3 or 4 rows: fused_decode_ok keeps K <= 4096
}

template <int XF, int WF, int OUT, int ACC>
hipError_t run_decode_fused(const uint16_t* x, uint8_t* xq, float* xs, const LinearArgs& a, hipStream_t stream) {
  const int mr = fused_rows(a.m);
  if (mr == 1) return run_decode_fused_rows<XF, WF, OUT, ACC, 1>(x, xq, xs, a, stream);
  if (mr == 2) return run_decode_fused_rows<XF, WF, OUT, ACC, 2>(x, xq, xs, a, stream);
  return run_decode_fused_rows<XF, WF, OUT, ACC, 4>(x, xq, xs, a, stream);
}

template <int XF, int WF, int OUT, int ACC>
hipError_t run_decode_reg(const LinearArgs& a, hipStream_t stream) {
  const int64_t kt = a.k / KSTEP;
  const dim3 grid((unsigned)(a.n / 16));
#define SFR_DEC(NWV, U)                                                                                      \
  hipLaunchKernelGGL((linear_decode_kernel<XF, WF, OUT, ACC, NWV, U>), grid, dim3(64 * NWV), 0, stream, a.xq, a.xs, \
                     a.values, a.meta, a.ws, a.bias, a.out, (int)a.m, (int)a.n, (int)a.k, a.xs_stride, a.ws_stride)
  if (kt <= 8) SFR_DEC(8, 1);
  else if (kt <= 16) SFR_DEC(8, 2);
  else if (kt <= 32) SFR_DEC(8, 4);
  else if (kt <= 64) SFR_DEC(16, 4);
  else if (kt <= 112) SFR_DEC(16, 7);
  else SFR_DEC(16, 8);  // loops for kt > 128
#undef SFR_DEC
  return hipGetLastError();
}

template <int XF, int WF, int OUT, int ACC>
hipError_t run_algo(const LinearArgs& a, int cfg, hipStream_t stream) {
  switch (cfg) {
    case ALGO_DECODE_LDS: return run_decode_unit<XF, WF, OUT, ACC, 1>(a, stream);
    case ALGO_DECODE_REG: return run_decode_reg<XF, WF, OUT, ACC>(a, stream);
    // Four stages instead of two where few tiles share a CU (one or two
    // workgroups per CU hide little latency by themselves) and K is long
    // enough for the deeper pipeline to pay: each load then has three k steps
    // to land.  Same arithmetic, same order, bit-identical output.
    case ALGO_TILED_64:
      if (tiled_deep(a, 64, 2, 8192)) return run_tiled<XF, WF, OUT, ACC, 64, 64, 2, 2, 8, 4, 0, 1, 8, 1>(a, stream);
      return run_tiled<XF, WF, OUT, ACC, 64, 64, 2, 2, 8, 2, 0, 1, 8, 1>(a, stream);
    case ALGO_TILED_128:
      if (tiled_deep(a, 128, 1, 4096)) return run_tiled<XF, WF, OUT, ACC, 128, 128, 2, 2, 8, 4, 0, 1, 8, 1>(a, stream);
      return run_tiled<XF, WF, OUT, ACC, 128, 128, 2, 2, 8, 2, 0, 1, 8, 1>(a, stream);
    case ALGO_TILED_256:
      // non-temporal output stores: the GEMM's speed is the same, and the
      // next kernel's traffic no longer waits behind its dirty lines
      if (persistent_ok(a, 256)) return run_persistent<XF, WF, OUT, ACC, 256, 256, 4, 2, 4, 8, 1, 1>(a, stream);
      return run_tiled<XF, WF, OUT, ACC, 256, 256, 4, 2, 8, 2, 2, 1, 8, 1>(a, stream);
    case ALGO_DECODE_LDS_32: return run_decode_unit<XF, WF, OUT, ACC, 2>(a, stream);
    case ALGO_TILED_256x128:
      // the persistent kernel with half-height tiles: for shapes whose
      // 256 x 256 tiles leave most CUs idle
      if (persistent_ok(a, 256)) return run_persistent<XF, WF, OUT, ACC, 256, 128, 4, 2, 4, 8, 1, 1>(a, stream);
      return run_tiled<XF, WF, OUT, ACC, 256, 128, 4, 2, 8, 2, 2, 1, 8, 1>(a, stream);
    default:  // ALGO_WIDE_256: FP8 accumulation only (checked by linear_algo_supported)
      if constexpr (ACC == ACC_F8) return run_wide<XF, WF, OUT, 8>(a, stream);
      else return hipErrorInvalidValue;
  }
}

template <int XF, int WF>
hipError_t run_out(const LinearArgs& a, int cfg, int acc, hipStream_t stream) {
  if (acc == ACC_F8) {
    if (a.out_fmt == OUT_BF16) return run_algo<XF, WF, OUT_BF16, ACC_F8>(a, cfg, stream);
    return run_algo<XF, WF, OUT_F32, ACC_F8>(a, cfg, stream);
  }
  if (a.out_fmt == OUT_BF16) return run_algo<XF, WF, OUT_BF16, ACC_F32>(a, cfg, stream);
  return run_algo<XF, WF, OUT_F32, ACC_F32>(a, cfg, stream);
}

}  // namespace

const char* linear_algo_name(int algo) {
  static const char* const names[2][ALGO_COUNT] = {
      {"decode_lds", "decode_reg", "tiled_64x64", "tiled_128x128", "tiled_256x256", nullptr, "decode_lds_32",
       "tiled_256x128"},
      {"decode_lds+f8acc", "decode_reg+f8acc", "tiled_64x64+f8acc", "tiled_128x128+f8acc", "tiled_256x256+f8acc",
       "wide_256x256+f8acc", "decode_lds_32+f8acc", "tiled_256x128+f8acc"}};
  if (algo < 0 || (algo & ~(ALGO_ACC_F8_FLAG | 0xFF)) != 0) return nullptr;
  const int cfg = algo & 0xFF;
  const bool f8 = (algo & ALGO_ACC_F8_FLAG) != 0;
  if (cfg >= ALGO_COUNT || (cfg == ALGO_WIDE_256 && !f8)) return nullptr;  // FP8 accumulation only
  return names[f8 ? 1 : 0][cfg];
}

bool linear_algo_valid(int algo) { return linear_algo_name(algo) != nullptr; }

bool linear_algo_supported(int algo, int64_t m, int64_t n, int64_t k) {
  if (!linear_algo_valid(algo)) return false;
  switch (algo & 0xFF) {
    case ALGO_DECODE_LDS: return m <= 64 && k % kUnitK == 0;
    case ALGO_DECODE_REG: return m <= 16;
    case ALGO_TILED_64:
    case ALGO_TILED_128:
    case ALGO_TILED_256:
    case ALGO_TILED_256x128: return true;
    case ALGO_WIDE_256: return (algo & ALGO_ACC_F8_FLAG) && k >= 4 * KSTEP;
    case ALGO_DECODE_LDS_32: return m <= 64 && k % kUnitK == 0 && n % 32 == 0;
    default: return false;
  }
}

// The built-in kernel configuration: up to 16 rows the unit decode kernel
// when K allows (32 weight rows per workgroup for several activation rows and
// N >= 6144, where the activation traffic it halves costs more than the
// workgroups it gives up), else the register-streaming decode kernel; 17..64
// rows and above as explained at each rule.
static int default_config(int64_t m, int64_t n, int64_t k) {
  if (m <= 16) {
    if (m >= 2 && n >= 6144 && linear_algo_supported(ALGO_DECODE_LDS_32, m, n, k)) return ALGO_DECODE_LDS_32;
    return linear_algo_supported(ALGO_DECODE_LDS, m, n, k) ? ALGO_DECODE_LDS : ALGO_DECODE_REG;
  }
  const int64_t cus = device_cus();
  // 17..64 rows: the unit decode kernels over 16-row activation blocks (the
  // weight block is read once per block, mostly from L2), unless above 32
  // rows the 64x64 tiles alone cover about 3/4 of the CUs: then the tiled
  // kernel, which reads the weight once, is as fast (measured on the Llama
  // shapes: decode 2-3x faster at N = 4096 / 6144 and at K = 14336, the
  // tiled kernels 10-25% faster at N = 14336, K = 4096, M >= 48)
  if (m <= 64 && linear_algo_supported(ALGO_DECODE_LDS, m, n, k) && !(m > 32 && 4 * ((n + 63) / 64) >= 3 * cus)) {
    if ((m > 24 || n >= 14336 || k >= 8192) && linear_algo_supported(ALGO_DECODE_LDS_32, m, n, k))
      return ALGO_DECODE_LDS_32;
    return ALGO_DECODE_LDS;
  }
  // Rounds of tiles over the CUs: one 256x256 tile per CU at a time, two
  // 128x128 ones.  A 128x128 round takes about 0.65 of a 256x256 one
  // (measured on the Llama shapes at M = 1024..4096), so the 256x256
  // configuration wins once it needs at most 2/3 as many rounds, and always
  // from two full rounds on.
  const int64_t t256 = ((m + 255) / 256) * ((n + 255) / 256);
  const int64_t t128 = ((m + 127) / 128) * ((n + 127) / 128);
  const int64_t t2x1 = ((m + 127) / 128) * ((n + 255) / 256);
  const int64_t r256 = (t256 + cus - 1) / cus, r128 = (t128 + 2 * cus - 1) / (2 * cus);
  if (t256 >= 2 * cus || 3 * r256 <= 2 * r128) return ALGO_TILED_256;
  // One round of 256(n) x 128(m) persistent tiles covering 3/4 to all of the
  // CUs: 11-15% faster than the 128x128 tiles (measured on the Llama shapes
  // at M = 512 (N = 14336), 1024 (N = 6144) and 2048 (N = 4096, K = 4096 and
  // 14336)); with fewer tiles too many CUs idle.
  if (4 * t2x1 >= 3 * cus && t2x1 <= cus) return ALGO_TILED_256x128;
  if (t128 >= cus) return ALGO_TILED_128;
  return ALGO_TILED_64;
}

// The built-in choice: binary32-grade accumulation everywhere (the stated
// accuracy of the layer holds for every input).
int linear_default_algo(int64_t m, int64_t n, int64_t k) { return default_config(m, n, k); }

hipError_t launch_linear_algo(const LinearArgs& a, int algo, hipStream_t stream) {
  if (algo < 0) algo = linear_default_algo(a.m, a.n, a.k);
  const int cfg = algo & 0xFF, acc = (algo & ALGO_ACC_F8_FLAG) ? ACC_F8 : ACC_F32;
  if (a.x_fmt == FMT_E4M3 && a.w_fmt == FMT_E4M3) return run_out<FMT_E4M3, FMT_E4M3>(a, cfg, acc, stream);
  if (a.x_fmt == FMT_E4M3 && a.w_fmt == FMT_E5M2) return run_out<FMT_E4M3, FMT_E5M2>(a, cfg, acc, stream);
  if (a.x_fmt == FMT_E5M2 && a.w_fmt == FMT_E4M3) return run_out<FMT_E5M2, FMT_E4M3>(a, cfg, acc, stream);
  return run_out<FMT_E5M2, FMT_E5M2>(a, cfg, acc, stream);
}

hipError_t launch_linear(const LinearArgs& a, hipStream_t stream) { return launch_linear_algo(a, -1, stream); }

template <int XF, int WF>
hipError_t run_fused_out(const uint16_t* x, uint8_t* xq, float* xs, const LinearArgs& a, int acc, hipStream_t stream) {
  if (acc == ACC_F8) {
    if (a.out_fmt == OUT_BF16) return run_decode_fused<XF, WF, OUT_BF16, ACC_F8>(x, xq, xs, a, stream);
    return run_decode_fused<XF, WF, OUT_F32, ACC_F8>(x, xq, xs, a, stream);
  }
  if (a.out_fmt == OUT_BF16) return run_decode_fused<XF, WF, OUT_BF16, ACC_F32>(x, xq, xs, a, stream);
  return run_decode_fused<XF, WF, OUT_F32, ACC_F32>(x, xq, xs, a, stream);
}

hipError_t launch_linear_dynamic(const uint16_t* x, uint8_t* xq, float* xs, const LinearArgs& a, int algo,
                                 hipStream_t stream) {
  const int dflt = linear_default_algo(a.m, a.n, a.k);
  if (algo < 0) algo = dflt;
  if (!fused_decode_ok(a.m, a.n, a.k) || (algo & 0xFF) != (dflt & 0xFF)) {
    // two launches: the row-wise quantization, then the linear layer
    hipError_t e = launch_quantize(x, a.m, a.k, a.x_fmt, xq, xs, stream);
    if (e != hipSuccess) return e;
    LinearArgs b = a;
    b.xq = xq;
    b.xs = xs;
    return launch_linear_algo(b, algo, stream);
  }
  const int acc = (algo & ALGO_ACC_F8_FLAG) ? ACC_F8 : ACC_F32;
  if (a.x_fmt == FMT_E4M3 && a.w_fmt == FMT_E4M3) return run_fused_out<FMT_E4M3, FMT_E4M3>(x, xq, xs, a, acc, stream);
  if (a.x_fmt == FMT_E4M3 && a.w_fmt == FMT_E5M2) return run_fused_out<FMT_E4M3, FMT_E5M2>(x, xq, xs, a, acc, stream);
  if (a.x_fmt == FMT_E5M2 && a.w_fmt == FMT_E4M3) return run_fused_out<FMT_E5M2, FMT_E4M3>(x, xq, xs, a, acc, stream);
  return run_fused_out<FMT_E5M2, FMT_E5M2>(x, xq, xs, a, acc, stream);
}

}  // namespace sfr
