/*
 * CPU oracle for the row-wise-scaled FP8 linear layer with a 2:4 sparse weight.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code with the HIP library.
 *
 * Sources (web pages on pytorch/ao):
 *  [P1] "Add CUTLASS-based row-wise scaled sparse FP8 kernel" (PR #1671):
 *       the operator is a row-wise scaled linear for an FP8 activation and a
 *       2:4 sparse FP8 weight; the activation is quantized dynamically; the
 *       dense->sparse converter must treat -0.0 as zero; FP16->FP8 casts must
 *       not produce NaN.
 *  [P4] "Making torchao ABI compatible ..." (issue #3516), file table: the four
 *       (activation, weight) dtype pairs e4m3/e5m2 x e4m3/e5m2.
 *  [P5] "[float8nocompile] ... atomic_max-based algo ..." (PR #1455), review
 *       thread: the amax reduction should stay deterministic.
 *  [P2] "promote blocksparse from prototype, make it faster" (PR #1734): a
 *       weight stored block-sparse (BSR) with blocks of 64 x 64 and most
 *       blocks zero (sparsity level 0.9 in its numbers), multiplied by a
 *       dense activation whose decode row count is padded up to 16.  The page
 *       names no number format; read here as the model's bf16 weight and
 *       activation with a binary32-or-better sum and a bf16 result.
 * The formats' constants (e4m3 max 448, e5m2 max 57344) are the OCP FP8
 * definitions; the pages only name the dtypes.
 *
 * Every function is written for obviousness, not speed.  Floating-point
 * arithmetic is IEEE binary32/binary64 with no contraction (built with
 * -ffp-contract=off -fno-fast-math).  Loops over independent outputs may run
 * under OpenMP; no sum is reordered.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_E4M3 0
#define ORC_E5M2 1

/* ------------------------------------------------------------------------- */
/* FP8 codec.  [P4] file table names e4m3 and e5m2; bit layouts are OCP FP8.  */
/* ------------------------------------------------------------------------- */

/* Exact value of an FP8 byte.  e4m3 ("fn" variant): 1 sign, 4 exponent bits
 * (bias 7), 3 mantissa bits, no infinities, S.1111.111 is NaN.  e5m2: 1 sign,
 * 5 exponent bits (bias 15), 2 mantissa bits, IEEE-style inf/NaN at exponent
 * 31.  Exponent field 0 encodes subnormals f * 2^(1-bias-mbits). */
double orc_fp8_decode(uint8_t b, int fmt)
{
    int s = b >> 7;
    double v;
    if (fmt == ORC_E4M3) {
        int e = (b >> 3) & 15, f = b & 7;
        if (e == 15 && f == 7) return NAN;
        if (e == 0) v = ldexp((double)f, -9);                /* f/8 * 2^-6 */
        else v = ldexp(1.0 + f / 8.0, e - 7);
    } else {
        int e = (b >> 2) & 31, f = b & 3;
        if (e == 31) return f ? NAN : (s ? -INFINITY : INFINITY);
        if (e == 0) v = ldexp((double)f, -16);               /* f/4 * 2^-14 */
        else v = ldexp(1.0 + f / 4.0, e - 15);
    }
    return s ? -v : v;
}

/* Largest finite magnitude code: e4m3 0x7E (448), e5m2 0x7B (57344). */
int orc_fp8_max_code(int fmt) { return fmt == ORC_E4M3 ? 0x7E : 0x7B; }

/* Number of binary places of the smallest subnormal: every finite value of
 * the format is an integer multiple of 2^-orc_fp8_frac_bits(fmt). */
int orc_fp8_frac_bits(int fmt) { return fmt == ORC_E4M3 ? 9 : 16; }

/* Saturating round-to-nearest-even encode of a finite binary32 value.
 * Definition: the sign is kept (so -0.0 and negative underflow give a signed
 * zero); a magnitude at or above the format's maximum gives the maximum (the
 * cast must not produce NaN or inf, [P1] on NaNs from FP16->FP8); otherwise
 * the result is the representable magnitude nearest to |v|, and at an exact
 * midpoint the code whose mantissa LSB is 0.  The finite non-negative codes
 * 0x00..max are ordered by value, so the two neighbours are found by bisection
 * over codes, and the midpoint test is exact in binary64. */
uint8_t orc_fp8_encode(float v, int fmt)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    int cmax = orc_fp8_max_code(fmt);
    if (a >= orc_fp8_decode((uint8_t)cmax, fmt)) return (uint8_t)(sign | cmax);
    int lo = 0, hi = cmax;                 /* dec(lo) <= a < dec(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (orc_fp8_decode((uint8_t)mid, fmt) <= a) lo = mid; else hi = mid;
    }
    double twice_mid = orc_fp8_decode((uint8_t)lo, fmt) + orc_fp8_decode((uint8_t)hi, fmt);
    double twice_a = 2.0 * a;
    int c;
    if (twice_a < twice_mid) c = lo;
    else if (twice_a > twice_mid) c = hi;
    else c = (lo & 1) ? hi : lo;           /* tie: even mantissa LSB */
    return (uint8_t)(sign | c);
}

/* ------------------------------------------------------------------------- */
/* bfloat16                                                                   */
/* ------------------------------------------------------------------------- */

float orc_bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a binary64 value to the nearest bfloat16 (8-bit significand, the
 * binary32 exponent range), ties to even, overflow to infinity.  Written as
 * "scale the value so that one bf16 unit in the last place is 1, round to
 * an integer, scale back". */
uint16_t orc_bf16_from_double(double y)
{
    if (isnan(y)) return 0x7FC0;
    uint16_t sign = signbit(y) ? 0x8000 : 0;
    double a = fabs(y);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                 /* a = f * 2^e, f in [0.5,1): a in [2^(e-1), 2^e) */
    int ex = e - 1;               /* floor(log2 a) */
    if (ex < -126) ex = -126;     /* bf16 subnormals share the 2^-133 quantum */
    double q = ldexp(1.0, ex - 7);
    double r = nearbyint(a / q);  /* a/q is exact (power-of-two scaling) */
    double res = r * q;           /* exact */
    float f = (float)res;         /* exact, or +inf on overflow */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (u >> 16));
}

/* ------------------------------------------------------------------------- */
/* Row-wise dynamic quantization.  [P1]: row-wise scaled linear, dynamically   */
/* quantized FP8 activation; [P5]: the amax must be a deterministic max.       */
/* ------------------------------------------------------------------------- */

/* For each row r of x[rows, cols] (bf16 bits, row-major):
 *   amax  = max_k |x[r,k]|                         (exact)
 *   scale = fl32(amax / fmax)                      (IEEE binary32 division)
 *   q[r,k]= encode(fl32(x[r,k] / scale))           (binary32 division, then
 *                                                   saturating RNE to FP8)
 * A row with amax == 0 gets scale 0 and codes that keep each zero's sign. */
void orc_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int fmt,
                       uint8_t* q, float* scale)
{
    const float fmax = (float)orc_fp8_decode((uint8_t)orc_fp8_max_code(fmt), fmt);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * cols;
        uint8_t* qr = q + r * cols;
        float amax = 0.0f;
        for (int64_t k = 0; k < cols; ++k) {
            float a = fabsf(orc_bf16_to_float(xr[k]));
            if (a > amax) amax = a;
        }
        if (amax == 0.0f) {
            scale[r] = 0.0f;
            for (int64_t k = 0; k < cols; ++k) qr[k] = (xr[k] & 0x8000) ? 0x80 : 0x00;
            continue;
        }
        float s = amax / fmax;
        scale[r] = s;
        for (int64_t k = 0; k < cols; ++k) {
            float t = orc_bf16_to_float(xr[k]) / s;
            qr[k] = orc_fp8_encode(t, fmt);
        }
    }
}

/* Tensor-wise dynamic quantization ([P5]: one scale for the whole tensor, its
 * amax a deterministic reduction).  It is the row-wise quantization above of
 * the tensor read as one row of rows*cols elements: a single exact amax, one
 * scale, the same division and encoding for every element. */
void orc_quantize_tensor(const uint16_t* x, int64_t rows, int64_t cols, int fmt,
                         uint8_t* q, float* scale)
{
    orc_quantize_rows(x, 1, rows * cols, fmt, q, scale);
}

/* ------------------------------------------------------------------------- */
/* 2:4 selection and compression.  [P1]: converter to the sparse format; the  */
/* converter must treat -0.0 as zero.                                          */
/* ------------------------------------------------------------------------- */

/* Magnitude key of an FP8 byte: for both OCP formats the unsigned order of
 * the 7 low bits equals the order of finite magnitudes, and +0 / -0 share key
 * 0, which is how -0.0 counts as zero. */
static int mag_key(uint8_t b) { return b & 0x7F; }

/* Position j outranks position i when its magnitude is larger, or equal with
 * a lower index (ties go to the lower index). */
static int outranks(const uint8_t* g, int j, int i)
{
    return mag_key(g[j]) > mag_key(g[i]) || (mag_key(g[j]) == mag_key(g[i]) && j < i);
}

/* Formulation 1 (ranking): keep the positions outranked by fewer than two
 * others.  Returns the kept indices in ascending order. */
void orc_select_rank(const uint8_t g[4], int* i0, int* i1)
{
    int kept[2], n = 0;
    for (int i = 0; i < 4; ++i) {
        int beaten = 0;
        for (int j = 0; j < 4; ++j)
            if (j != i && outranks(g, j, i)) ++beaten;
        if (beaten < 2) kept[n++] = i;
    }
    *i0 = kept[0];
    *i1 = kept[1];
}

/* Formulation 2 (pairs): of the six pairs {a<b}, take the one whose members
 * both outrank both non-members. */
void orc_select_pairs(const uint8_t g[4], int* i0, int* i1)
{
    *i0 = -1;
    *i1 = -1;
    for (int a = 0; a < 4; ++a)
        for (int b = a + 1; b < 4; ++b) {
            int ok = 1;
            for (int c = 0; c < 4; ++c) {
                if (c == a || c == b) continue;
                if (!outranks(g, a, c) || !outranks(g, b, c)) ok = 0;
            }
            if (ok) { *i0 = a; *i1 = b; }
        }
}

/* Compressed layout (this library's own): for row n and group g of four
 * consecutive k (k = 4g .. 4g+3):
 *   values[n, 2g], values[n, 2g+1]: the kept bytes in ascending index order,
 *       a kept negative zero stored as 0x00;
 *   meta[n, g/2], bits 4*(g%2) .. 4*(g%2)+3: nibble i0 | (i1 << 2).
 * values is [n, k/2] and meta is [n, k/8], both row-major bytes. */
void orc_compress_2to4(const uint8_t* w, int64_t n, int64_t k, uint8_t* values, uint8_t* meta)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        const uint8_t* wr = w + r * k;
        uint8_t* vr = values + r * (k / 2);
        uint8_t* mr = meta + r * (k / 8);
        memset(mr, 0, (size_t)(k / 8));
        for (int64_t g = 0; g < k / 4; ++g) {
            int i0, i1;
            orc_select_rank(wr + 4 * g, &i0, &i1);
            uint8_t b0 = wr[4 * g + i0], b1 = wr[4 * g + i1];
            vr[2 * g] = (b0 == 0x80) ? 0x00 : b0;
            vr[2 * g + 1] = (b1 == 0x80) ? 0x00 : b1;
            mr[g / 2] |= (uint8_t)((i0 | (i1 << 2)) << (4 * (g % 2)));
        }
    }
}

/* Inverse of the layout above: kept bytes back at their positions, 0x00 at
 * the dropped ones. */
void orc_decompress_2to4(const uint8_t* values, const uint8_t* meta, int64_t n, int64_t k, uint8_t* w)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        const uint8_t* vr = values + r * (k / 2);
        const uint8_t* mr = meta + r * (k / 8);
        uint8_t* wr = w + r * k;
        memset(wr, 0, (size_t)k);
        for (int64_t g = 0; g < k / 4; ++g) {
            int nib = (mr[g / 2] >> (4 * (g % 2))) & 0xF;
            int i0 = nib & 3, i1 = (nib >> 2) & 3;
            wr[4 * g + i0] = vr[2 * g];
            wr[4 * g + i1] = vr[2 * g + 1];
        }
    }
}

/* Byte-level pruning of a dense FP8 matrix: the bytes compress would keep
 * (with -0 written as +0), 0x00 elsewhere. */
void orc_prune_2to4(const uint8_t* w, int64_t n, int64_t k, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t g = 0; g < k / 4; ++g) {
            const uint8_t* gr = w + r * k + 4 * g;
            uint8_t* o = out + r * k + 4 * g;
            int i0, i1;
            orc_select_pairs(gr, &i0, &i1);
            for (int i = 0; i < 4; ++i) {
                uint8_t b = (i == i0 || i == i1) ? gr[i] : 0x00;
                o[i] = (b == 0x80) ? 0x00 : b;
            }
        }
    }
}

/* 2:4 magnitude pruning of a dense bf16 matrix (the weight is pruned before
 * it is quantized: [P1], the 2:4 sparse weight; a group's two largest
 * magnitudes survive).  For row r and group g (k = 4g .. 4g+3): position j
 * survives when fewer than two positions of the group outrank it, where i
 * outranks j if |w_i| > |w_j|, or |w_i| == |w_j| and i < j (ties go to the
 * lower index).  Magnitudes are compared as values: +0.0 and -0.0 are both
 * zero (and tie).  Surviving entries keep their bits; the others become
 * +0.0.  Finite inputs only. */
static int bf16_outranks(const uint16_t* g, int i, int j)
{
    const double a = fabs((double)orc_bf16_to_float(g[i])), b = fabs((double)orc_bf16_to_float(g[j]));
    return a > b || (a == b && i < j);
}

void orc_prune_2to4_bf16(const uint16_t* w, int64_t n, int64_t k, uint16_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t g = 0; g < k / 4; ++g) {
            const uint16_t* gr = w + r * k + 4 * g;
            uint16_t* o = out + r * k + 4 * g;
            for (int j = 0; j < 4; ++j) {
                int above = 0;
                for (int i = 0; i < 4; ++i)
                    if (i != j && bf16_outranks(gr, i, j)) ++above;
                o[j] = above < 2 ? gr[j] : (uint16_t)0x0000;
            }
        }
    }
}

/* Exhaustive agreement of the two selection formulations over every 4-byte
 * group (2^32 of them).  Returns the number of disagreements, and the number
 * of groups whose chosen pair is not a valid ascending pair. */
void orc_check_all_groups(int64_t* disagree, int64_t* invalid)
{
    int64_t d = 0, bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : d, bad)
    for (int64_t hi = 0; hi < 65536; ++hi) {
        for (uint32_t lo = 0; lo < 65536; ++lo) {
            uint32_t u = ((uint32_t)hi << 16) | lo;
            uint8_t g[4] = {(uint8_t)u, (uint8_t)(u >> 8), (uint8_t)(u >> 16), (uint8_t)(u >> 24)};
            int a0, a1, b0, b1;
            orc_select_rank(g, &a0, &a1);
            orc_select_pairs(g, &b0, &b1);
            if (a0 != b0 || a1 != b1) ++d;
            if (!(0 <= a0 && a0 < a1 && a1 < 4)) ++bad;
        }
    }
    *disagree = d;
    *invalid = bad;
}

/* ------------------------------------------------------------------------- */
/* The linear layer.  [P1]: row-wise scaled linear with sparse FP8 weight:     */
/*   out[m,n] = xs[m] * ws[n] * sum_k xq[m,k] * wq[n,k]  (+ bias[n])           */
/* where wq is the 2:4 weight the compressed (values, meta) encode.            */
/* ------------------------------------------------------------------------- */

/* Integer units of an FP8 value: dec(b) = units(b) * 2^-frac_bits. */
static int64_t fp8_units(uint8_t b, int fmt)
{
    return (int64_t)ldexp(orc_fp8_decode(b, fmt), orc_fp8_frac_bits(fmt));
}

/* Evaluate the layer at the output positions (rows[i], cols[j]) for
 * i < nr, j < nc.  For each position it produces:
 *   y_exact[i,j] : fl64( S * fl64(xs*ws) ) (+ bias), with S the exact dot
 *                  product (summed in 128-bit integers, then one rounding)
 *   acc32[i,j]   : the dot product summed serially in binary32 over
 *                  ascending k (the products are exact in binary32)
 *   sabs[i,j]    : fl64( sum_k |xq*wq| ) * xs * ws  (the tolerance scale)
 * bias may be NULL.  The weight is first decompressed, so the sum runs over
 * the dense pruned weight row. */
void orc_linear(const uint8_t* xq, int xfmt, const float* xs, int64_t m, int64_t k,
                const uint8_t* values, const uint8_t* meta, int wfmt, const float* ws, int64_t n,
                const uint16_t* bias, const int64_t* rows, int64_t nr, const int64_t* cols, int64_t nc,
                double* y_exact, float* acc32, double* sabs)
{
    (void)m;
    (void)n;
    int fb = orc_fp8_frac_bits(xfmt) + orc_fp8_frac_bits(wfmt);
#pragma omp parallel for schedule(dynamic)
    for (int64_t j = 0; j < nc; ++j) {
        int64_t c = cols[j];
        uint8_t wrow[k > 0 ? k : 1];
        orc_decompress_2to4(values + c * (k / 2), meta + c * (k / 8), 1, k, wrow);
        for (int64_t i = 0; i < nr; ++i) {
            int64_t r = rows[i];
            const uint8_t* xr = xq + r * k;
            __int128 s = 0, sa = 0;
            float f = 0.0f;
            for (int64_t kk = 0; kk < k; ++kk) {
                __int128 p = (__int128)fp8_units(xr[kk], xfmt) * fp8_units(wrow[kk], wfmt);
                s += p;
                sa += p < 0 ? -p : p;
                float prod = (float)orc_fp8_decode(xr[kk], xfmt) * (float)orc_fp8_decode(wrow[kk], wfmt);
                f = f + prod;
            }
            double t = (double)xs[r] * (double)ws[c];      /* exact: 24x24 bits */
            double S = ldexp((double)s, -fb);
            double y = S * t;
            if (bias) y = y + (double)orc_bf16_to_float(bias[c]);
            y_exact[i * nc + j] = y;
            acc32[i * nc + j] = f;
            sabs[i * nc + j] = ldexp((double)sa, -fb) * t;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Block-sparse (BSR) weight and linear layer.  [P2]: blocks of bs x bs        */
/* (bs = 64 there), stored as the usual compressed-sparse-row structure over  */
/* blocks: crow (block-row pointers), col (block-column indices) and the      */
/* kept blocks' values.                                                       */
/* ------------------------------------------------------------------------- */

/* A bs x bs block of w[n, k] (bf16 bits, row-major) at block row br and block
 * column bc is kept when any element is non-zero by value: +0.0 (0x0000) and
 * -0.0 (0x8000) both count as zero, every other code (subnormals, NaN, inf
 * included) as non-zero. */
static int bsr_block_kept(const uint16_t* w, int64_t k, int64_t bs, int64_t br, int64_t bc)
{
    for (int64_t r = 0; r < bs; ++r)
        for (int64_t c = 0; c < bs; ++c)
            if ((w[(br * bs + r) * k + bc * bs + c] & 0x7FFF) != 0) return 1;
    return 0;
}

/* crow[0 .. n/bs]: crow[0] = 0 and crow[i + 1] = crow[i] + (number of kept
 * blocks in block row i).  Returns the total number of kept blocks. */
int64_t orc_bsr_count(const uint16_t* w, int64_t n, int64_t k, int64_t bs, int32_t* crow)
{
    int64_t nbr = n / bs, nbc = k / bs, total = 0;
    crow[0] = 0;
    for (int64_t br = 0; br < nbr; ++br) {
        for (int64_t bc = 0; bc < nbc; ++bc) total += bsr_block_kept(w, k, bs, br, bc);
        crow[br + 1] = (int32_t)total;
    }
    return total;
}

/* col[crow[i] ..]: the kept block columns of block row i in ascending order;
 * values[j]: block j copied as bs x bs row-major bf16 bits. */
void orc_bsr_fill(const uint16_t* w, int64_t n, int64_t k, int64_t bs, const int32_t* crow, int32_t* col,
                  uint16_t* values)
{
    int64_t nbr = n / bs, nbc = k / bs;
    for (int64_t br = 0; br < nbr; ++br) {
        int64_t j = crow[br];
        for (int64_t bc = 0; bc < nbc; ++bc) {
            if (!bsr_block_kept(w, k, bs, br, bc)) continue;
            col[j] = (int32_t)bc;
            for (int64_t r = 0; r < bs; ++r)
                for (int64_t c = 0; c < bs; ++c)
                    values[(j * bs + r) * bs + c] = w[(br * bs + r) * k + bc * bs + c];
            ++j;
        }
    }
}

/* The dense matrix the structure describes: zero outside the kept blocks. */
void orc_bsr_to_dense(const int32_t* crow, const int32_t* col, const uint16_t* values, int64_t n, int64_t k,
                      int64_t bs, uint16_t* w)
{
    memset(w, 0, (size_t)(n * k) * sizeof(uint16_t));
    for (int64_t br = 0; br < n / bs; ++br)
        for (int64_t j = crow[br]; j < crow[br + 1]; ++j)
            for (int64_t r = 0; r < bs; ++r)
                for (int64_t c = 0; c < bs; ++c)
                    w[(br * bs + r) * k + (int64_t)col[j] * bs + c] = values[(j * bs + r) * bs + c];
}

/* out[r, c] = sum_k x[r, k] * W[c, k] (+ bias[c]) for the BSR weight W, at the
 * positions (rows[i], cols[j]).  The sum runs over the kept blocks of block
 * row c / bs in stored order and, inside a block, over ascending k, in
 * binary64 (each bf16 x bf16 product is exact in binary64; zero blocks add
 * nothing, so this is the dense definition).  Also returns
 * sabs = sum |x * w| (the tolerance scale) and acc32, the same sum taken
 * serially in binary32 (without bias). */
void orc_bsr_linear(const uint16_t* x, int64_t m, int64_t k, const int32_t* crow, const int32_t* col,
                    const uint16_t* values, int64_t n, int64_t bs, const uint16_t* bias, const int64_t* rows,
                    int64_t nr, const int64_t* cols, int64_t nc, double* y, float* acc32, double* sabs)
{
    (void)m;
    (void)n;
#pragma omp parallel for schedule(dynamic)
    for (int64_t j = 0; j < nc; ++j) {
        int64_t c = cols[j], br = c / bs, rin = c % bs;
        for (int64_t i = 0; i < nr; ++i) {
            const uint16_t* xr = x + rows[i] * k;
            double s = 0.0, sa = 0.0;
            float f = 0.0f;
            for (int64_t b = crow[br]; b < crow[br + 1]; ++b) {
                const uint16_t* wr = values + (b * bs + rin) * bs;
                const uint16_t* xb = xr + (int64_t)col[b] * bs;
                for (int64_t kk = 0; kk < bs; ++kk) {
                    double p = (double)orc_bf16_to_float(xb[kk]) * (double)orc_bf16_to_float(wr[kk]);
                    s += p;
                    sa += fabs(p);
                    f = f + (float)p;   /* the product is exact in binary32 too */
                }
            }
            if (bias) s = s + (double)orc_bf16_to_float(bias[c]);
            y[i * nc + j] = s;
            acc32[i * nc + j] = f;
            sabs[i * nc + j] = sa;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Array forms of the element functions, for the Python side.                 */
/* ------------------------------------------------------------------------- */

void orc_fp8_decode_array(const uint8_t* b, int64_t n, int fmt, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_decode(b[i], fmt);
}

void orc_fp8_encode_array(const float* v, int64_t n, int fmt, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_encode(v[i], fmt);
}

void orc_bf16_from_double_array(const double* y, int64_t n, uint16_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_double(y[i]);
}

/* Kept index pairs of ngroups 4-byte groups, by either formulation. */
void orc_select_array(const uint8_t* groups, int64_t ngroups, int formulation, int32_t* i0, int32_t* i1)
{
    for (int64_t g = 0; g < ngroups; ++g) {
        int a, b;
        if (formulation == 0) orc_select_rank(groups + 4 * g, &a, &b);
        else orc_select_pairs(groups + 4 * g, &a, &b);
        i0[g] = a;
        i1[g] = b;
    }
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
