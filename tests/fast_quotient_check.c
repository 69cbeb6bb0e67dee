/*
 * Exhaustive check of the division-free quotient the fp8 store kernels use
 * (quotient_fast in the HIP sources), restated here in C: for every finite
 * bf16 group maximum A >= 2^-4 and every bf16 x with |x| <= A (both signs),
 *
 *     s = A / fmax, r = 1 / s                (IEEE float32 divisions)
 *     q0 = x * r, e = fma(q0, s, -x), q1 = fma(-e, r, q0)
 *
 * (the residual is taken negated, so a zero quotient keeps the sign of x),
 * must give the same fp8 code as the IEEE quotient x / s does, both encoded
 * by the CPU oracle.  The format is the first argument: "e4m3" (fmax = 448)
 * or "e5m2" (fmax = 57344).  Prints the number of pairs checked and of
 * mismatches (expected 0); exit status 1 on any mismatch, 2 on bad usage.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kv_oracle.h"

static float f_of(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }

int main(int argc, char** argv)
{
    if (argc != 2 || (strcmp(argv[1], "e4m3") != 0 && strcmp(argv[1], "e5m2") != 0)) {
        fprintf(stderr, "usage: %s e4m3|e5m2\n", argv[0]);
        return 2;
    }
    const int e5m2 = strcmp(argv[1], "e5m2") == 0;
    const float fmax = e5m2 ? 57344.0f : 448.0f;
    long long checked = 0, bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(+ : checked, bad)
    for (int ah = 0x3D80; ah < 0x7F80; ++ah) {
        const float A = f_of((uint32_t)ah << 16), s = A / fmax, r = 1.0f / s;
        for (uint32_t h = 0; h <= (uint32_t)ah; ++h) {
            for (int sg = 0; sg < 2; ++sg) {
                const float x = f_of((h | (sg ? 0x8000u : 0u)) << 16);
                const float q0 = x * r, e = fmaf(q0, s, -x), fast = fmaf(-e, r, q0);
                const float exact = x / s;
                ++checked;
                if (e5m2 ? kvo_e5m2_encode(fast) != kvo_e5m2_encode(exact)
                         : kvo_e4m3_encode(fast) != kvo_e4m3_encode(exact))
                    ++bad;
            }
        }
    }
    printf("checked %lld mismatches %lld\n", checked, bad);
    return bad != 0;
}
