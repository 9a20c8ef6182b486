/*
 * Sanitizer driver for the CPU oracle (test infrastructure only).
 *
 * Built by tests/test_oracle_sanitize.py with gcc and AddressSanitizer +
 * UndefinedBehaviorSanitizer together with sfr_oracle.c (no OpenMP, so every
 * loop runs in this thread), it calls every exported oracle function on
 * small seeded inputs and checks a few invariants that the pinning tests
 * also check, so that an out-of-bounds access, an overflow or another
 * undefined operation anywhere in the oracle stops the run.  Exit status 0
 * means every call ran clean and every invariant held.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_fp8_decode(uint8_t b, int fmt);
int orc_fp8_max_code(int fmt);
int orc_fp8_frac_bits(int fmt);
uint8_t orc_fp8_encode(float v, int fmt);
float orc_bf16_to_float(uint16_t h);
uint16_t orc_bf16_from_double(double y);
void orc_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* q, float* scale);
void orc_quantize_tensor(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* q, float* scale);
void orc_select_rank(const uint8_t g[4], int* i0, int* i1);
void orc_select_pairs(const uint8_t g[4], int* i0, int* i1);
void orc_compress_2to4(const uint8_t* w, int64_t n, int64_t k, uint8_t* values, uint8_t* meta);
void orc_decompress_2to4(const uint8_t* values, const uint8_t* meta, int64_t n, int64_t k, uint8_t* w);
void orc_prune_2to4(const uint8_t* w, int64_t n, int64_t k, uint8_t* out);
void orc_prune_2to4_bf16(const uint16_t* w, int64_t n, int64_t k, uint16_t* out);
void orc_linear(const uint8_t* xq, int xfmt, const float* xs, int64_t m, int64_t k, const uint8_t* values,
                const uint8_t* meta, int wfmt, const float* ws, int64_t n, const uint16_t* bias, const int64_t* rows,
                int64_t nr, const int64_t* cols, int64_t nc, double* y_exact, float* acc32, double* sabs);
int64_t orc_bsr_count(const uint16_t* w, int64_t n, int64_t k, int64_t bs, int32_t* crow);
void orc_bsr_fill(const uint16_t* w, int64_t n, int64_t k, int64_t bs, const int32_t* crow, int32_t* col,
                  uint16_t* values);
void orc_bsr_to_dense(const int32_t* crow, const int32_t* col, const uint16_t* values, int64_t n, int64_t k,
                      int64_t bs, uint16_t* w);
void orc_bsr_linear(const uint16_t* x, int64_t m, int64_t k, const int32_t* crow, const int32_t* col,
                    const uint16_t* values, int64_t n, int64_t bs, const uint16_t* bias, const int64_t* rows,
                    int64_t nr, const int64_t* cols, int64_t nc, double* y, float* acc32, double* sabs);
void orc_fp8_decode_array(const uint8_t* b, int64_t n, int fmt, double* out);
void orc_fp8_encode_array(const float* v, int64_t n, int fmt, uint8_t* out);
void orc_bf16_from_double_array(const double* y, int64_t n, uint16_t* out);
void orc_select_array(const uint8_t* groups, int64_t ngroups, int formulation, int32_t* i0, int32_t* i1);
int orc_num_threads(void);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void)
{
    /* xorshift64*: a seeded source of test bytes, nothing more */
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (uint32_t)((state * 0x2545F4914F6CDD1Dull) >> 32);
}

/* bf16 bits of a value spread over many binades, about 1 in 16 an exact zero */
static uint16_t random_bf16(void)
{
    uint32_t r = next_u32();
    if ((r & 15) == 0) return (uint16_t)((r >> 4) & 0x8000);
    double v = ((double)(r >> 8) / 16777216.0 + 0.5) * ldexp(1.0, (int)((r >> 4) & 15) - 8);
    return orc_bf16_from_double((r & 0x10) ? -v : v);
}

static int failures = 0;
#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "invariant failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                    \
        }                                                                  \
    } while (0)

int main(void)
{
    /* FP8 codec: every finite code survives decode -> encode */
    for (int fmt = 0; fmt < 2; ++fmt) {
        for (int b = 0; b < 256; ++b) {
            double v = orc_fp8_decode((uint8_t)b, fmt);
            if (isnan(v) || isinf(v)) continue;
            CHECK(orc_fp8_encode((float)v, fmt) == (uint8_t)b);
        }
        CHECK(orc_fp8_decode((uint8_t)orc_fp8_max_code(fmt), fmt) == (fmt == 0 ? 448.0 : 57344.0));
        CHECK(orc_fp8_frac_bits(fmt) == (fmt == 0 ? 9 : 16));
        uint8_t codes[256];
        double vals[256];
        float fv[256];
        for (int b = 0; b < 256; ++b) codes[b] = (uint8_t)b;
        orc_fp8_decode_array(codes, 256, fmt, vals);
        for (int b = 0; b < 256; ++b) fv[b] = isnan(vals[b]) ? 0.0f : (float)vals[b];
        orc_fp8_encode_array(fv, 256, fmt, codes);
    }
    double dv[5] = {0.0, -0.0, 1.0, -3.140625, 1e-40};
    uint16_t hv[5];
    orc_bf16_from_double_array(dv, 5, hv);
    CHECK(hv[2] == 0x3F80 && hv[1] == 0x8000);
    CHECK(orc_bf16_to_float(0x3F80) == 1.0f);

    /* quantization: 5 x 96 rows, row 2 all zeros */
    enum { R = 5, C = 96 };
    uint16_t x[R * C];
    uint8_t q[R * C];
    float s[R];
    for (int i = 0; i < R * C; ++i) x[i] = random_bf16();
    for (int c = 0; c < C; ++c) x[2 * C + c] = (uint16_t)(c & 1 ? 0x8000 : 0x0000);
    for (int fmt = 0; fmt < 2; ++fmt) {
        orc_quantize_rows(x, R, C, fmt, q, s);
        CHECK(s[2] == 0.0f);
        for (int i = 0; i < R * C; ++i) CHECK((q[i] & 0x7F) <= orc_fp8_max_code(fmt));
        orc_quantize_tensor(x, R, C, fmt, q, s);
        CHECK(s[0] > 0.0f);
    }

    /* selection: both formulations agree on random groups */
    uint8_t groups[4 * 4096];
    int32_t a0[4096], a1[4096], b0[4096], b1[4096];
    for (int i = 0; i < 4 * 4096; ++i) groups[i] = (uint8_t)next_u32();
    orc_select_array(groups, 4096, 0, a0, a1);
    orc_select_array(groups, 4096, 1, b0, b1);
    for (int g = 0; g < 4096; ++g) CHECK(a0[g] == b0[g] && a1[g] == b1[g] && a0[g] < a1[g]);
    int i0, i1;
    const uint8_t neg_zeros[4] = {0x80, 0x80, 0x80, 0x80};
    orc_select_rank(neg_zeros, &i0, &i1);
    CHECK(i0 == 0 && i1 == 1);
    orc_select_pairs(neg_zeros, &i0, &i1);
    CHECK(i0 == 0 && i1 == 1);

    /* compression round trip on an 8 x 64 FP8 matrix */
    enum { N = 8, K = 64 };
    uint8_t w[N * K], vals8[N * K / 2], meta[N * K / 8], back[N * K], pruned[N * K];
    for (int i = 0; i < N * K; ++i) w[i] = (uint8_t)next_u32();
    orc_compress_2to4(w, N, K, vals8, meta);
    orc_decompress_2to4(vals8, meta, N, K, back);
    orc_prune_2to4(w, N, K, pruned);
    CHECK(memcmp(back, pruned, sizeof back) == 0);
    uint16_t wb[N * K], wbp[N * K];
    for (int i = 0; i < N * K; ++i) wb[i] = random_bf16();
    orc_prune_2to4_bf16(wb, N, K, wbp);
    for (int g = 0; g < N * K / 4; ++g) {
        int zeros = 0;
        for (int j = 0; j < 4; ++j) zeros += wbp[4 * g + j] == 0;
        CHECK(zeros >= 2);
    }

    /* linear layer at every position of a 5 x 8 output, K = 64 */
    uint8_t xq[R * K];
    float xs[R], ws[N];
    uint16_t bias[N];
    for (int i = 0; i < R * K; ++i) xq[i] = (uint8_t)(next_u32() % 0x7C) | (uint8_t)(next_u32() & 0x80);  /* finite in both formats */
    for (int r = 0; r < R; ++r) xs[r] = 0.25f * (float)(r + 1);
    for (int c = 0; c < N; ++c) {
        ws[c] = 0.5f + (float)c;
        bias[c] = random_bf16();
    }
    int64_t rows[R], cols[N];
    for (int r = 0; r < R; ++r) rows[r] = r;
    for (int c = 0; c < N; ++c) cols[c] = c;
    for (int i = 0; i < N * K; ++i) w[i] = (uint8_t)(next_u32() % 0x7C);
    orc_compress_2to4(w, N, K, vals8, meta);
    double y[R * N], sabs[R * N];
    float acc[R * N];
    for (int xf = 0; xf < 2; ++xf)
        for (int wf = 0; wf < 2; ++wf) {
            orc_linear(xq, xf, xs, R, K, vals8, meta, wf, ws, N, bias, rows, R, cols, N, y, acc, sabs);
            orc_linear(xq, xf, xs, R, K, vals8, meta, wf, ws, N, NULL, rows, R, cols, N, y, acc, sabs);
            for (int i = 0; i < R * N; ++i) CHECK(fabs(y[i]) <= sabs[i] * (1.0 + 1e-12) + 1e-300);
        }

    /* block-sparse weight: 128 x 128 with 64 x 64 blocks, block (0, 1) zero */
    enum { BN = 128, BK = 128, BS = 64 };
    static uint16_t bw[BN * BK], bdense[BN * BK], bvals[BN * BK];
    for (int i = 0; i < BN * BK; ++i) bw[i] = random_bf16();
    for (int r = 0; r < BS; ++r)
        for (int c = BS; c < 2 * BS; ++c) bw[r * BK + c] = (uint16_t)((r + c) & 1 ? 0x8000 : 0);
    int32_t crow[BN / BS + 1], col[(BN / BS) * (BK / BS)];
    int64_t nnz = orc_bsr_count(bw, BN, BK, BS, crow);
    CHECK(nnz == 3 && crow[0] == 0 && crow[BN / BS] == 3);
    orc_bsr_fill(bw, BN, BK, BS, crow, col, bvals);
    orc_bsr_to_dense(crow, col, bvals, BN, BK, BS, bdense);
    for (int i = 0; i < BN * BK; ++i) CHECK((bdense[i] & 0x7FFF) == (bw[i] & 0x7FFF));
    static uint16_t bx[3 * BK], bbias[BN];
    for (int i = 0; i < 3 * BK; ++i) bx[i] = random_bf16();
    for (int i = 0; i < BN; ++i) bbias[i] = random_bf16();
    int64_t brows[3] = {0, 1, 2}, bcols[4] = {0, 63, 64, 127};
    double by[12], bsabs[12];
    float bacc[12];
    orc_bsr_linear(bx, 3, BK, crow, col, bvals, BN, BS, bbias, brows, 3, bcols, 4, by, bacc, bsabs);
    orc_bsr_linear(bx, 3, BK, crow, col, bvals, BN, BS, NULL, brows, 3, bcols, 4, by, bacc, bsabs);
    for (int i = 0; i < 12; ++i) CHECK(fabs(by[i]) <= bsabs[i] * (1.0 + 1e-12) + 1e-300);

    CHECK(orc_num_threads() >= 1);
    if (failures) {
        fprintf(stderr, "%d invariant(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: clean\n");
    return 0;
}
