/*
 * Exhaustive check of the quotient the HIP quantization kernels form for
 * scales from 2^-80 up (the fma-corrected product of sfr_quant.hpp's cast8):
 *
 *   q0 = fl32(x * rcp), rn = fma(q0, scale, -x), q = fma(-rn, rcp, q0),
 *   with scale = fl32(amax / fmax) and rcp = fl32(1 / scale).
 *
 * Row-wise dynamic quantization (pytorch/ao PR #1671, "Add CUTLASS-based
 * row-wise scaled sparse FP8 kernel": FP8 activations with one scale per row,
 * quantized dynamically) defines each code as the FP8 encoding of the
 * binary32 quotient x / scale.  For every positive finite bf16 amax and every
 * bf16 x with |x| <= amax (both signs, zeros included), in both formats, this
 * program compares the FP8 code of q with the code of the IEEE quotient, both
 * encoded by the oracle's orc_fp8_encode (where the two binary32 values are
 * bitwise equal the codes are equal without encoding).  Rows whose scale is
 * so small that 1 / scale overflows are skipped (the kernels take the
 * division path there).
 *
 * Prints, per format, the pair count, the pairs whose codes differ with scale
 * >= 2^-80, and the largest scale at which any codes differ.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

uint8_t orc_fp8_encode(float v, int fmt);

static float bf16(uint32_t h)
{
    uint32_t u = h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

int main(void)
{
    const float fmaxes[2] = {448.0f, 57344.0f};
    for (int fmt = 0; fmt < 2; ++fmt) {
        const float fmax = fmaxes[fmt];
        long pairs = 0, bad_above = 0;
        float worst = 0.0f;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, bad_above) reduction(max : worst)
        for (int am = 1; am < 0x7F80; ++am) {
            const float amax = bf16((uint32_t)am);
            const float scale = amax / fmax;
            const float rcp = 1.0f / scale;
            if (!isfinite(rcp)) continue;
            for (int xm = 0; xm <= am; ++xm) {
                for (int sg = 0; sg < 2; ++sg) {
                    const float x = bf16((uint32_t)xm | ((uint32_t)sg << 15));
                    const float ref = x / scale;
                    const float q0 = x * rcp;
                    const float rn = fmaf(q0, scale, -x);
                    const float q = fmaf(-rn, rcp, q0);
                    ++pairs;
                    if (bits(q) == bits(ref)) continue;
                    if (orc_fp8_encode(q, fmt) == orc_fp8_encode(ref, fmt)) continue;
                    if (scale > worst) worst = scale;
                    if (scale >= 0x1p-80f) ++bad_above;
                }
            }
        }
        printf("fmt %d pairs %ld differing_from_2^-80 %ld largest_differing_scale %a\n", fmt, pairs, bad_above,
               (double)worst);
    }
    return 0;
}
