/*
 * Exhaustive check of the division-free (q - MAX) / MAX the CacheGen
 * dequantiser uses (cg_unit in the HIP sources), restated here in C: for
 * every MAX in [1, 63] (bin counts 4 .. 129) and every c = q - MAX in
 * [-MAX, MAX],
 *
 *     r = 1 / MAX, p = c * r, e = fma(-p, MAX, c), u = fma(e, r, p)
 *
 * must equal the IEEE float32 quotient c / MAX that the oracle computes, bit
 * for bit (sign of zero included).  Prints the counts; exit status 1 on any
 * mismatch.
 */
#include <math.h>
#include <stdio.h>
#include <string.h>

static unsigned bits(float f) { unsigned b; memcpy(&b, &f, 4); return b; }

int main(void)
{
    int checked = 0, bad = 0;
    for (int MAX = 1; MAX <= 63; ++MAX) {
        volatile float m = (float)MAX;
        const float r = 1.0f / m;
        for (int c = -MAX; c <= MAX; ++c) {
            volatile float cf = (float)c;
            const float p = cf * r, e = fmaf(-p, m, cf), u = fmaf(e, r, p);
            ++checked;
            if (bits(u) != bits(cf / m)) ++bad;
        }
    }
    printf("checked %d mismatches %d\n", checked, bad);
    return bad != 0;
}
