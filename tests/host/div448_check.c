/* The FP8 epilogue computes scale = amax / 448 as
 *     q = RN(amax * c),  c = RN(1/448),  scale = RN(q + RN(amax - 448 q) * c)
 * (two FMAs) where amax >= 2^-116, and by division below.  This program checks,
 * for every float in the binades it is given, that the three-instruction form
 * equals the IEEE quotient bit for bit.
 *
 * usage: div448_check E0 E1 [E0 E1 ...]   every x in [2^E0, 2^E1)
 * prints "OK <count>" or the first mismatch; exit status 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t to_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

int main(int argc, char **argv) {
    const float c = 1.0f / 448.0f;
    unsigned long long n = 0;
    if (argc < 3 || (argc - 1) % 2 != 0) {
        fprintf(stderr, "usage: %s E0 E1 [E0 E1 ...]\n", argv[0]);
        return 2;
    }
    for (int a = 1; a + 1 < argc; a += 2) {
        const int e0 = atoi(argv[a]), e1 = atoi(argv[a + 1]);
        const uint32_t lo = to_bits(ldexpf(1.0f, e0));
        const uint32_t hi = e1 >= 128 ? 0x7f800000u : to_bits(ldexpf(1.0f, e1));
        for (uint32_t u = lo; u < hi; ++u) {
            const volatile float x = from_bits(u);
            const float ref = x / 448.0f;
            const float q = x * c;
            const float s = fmaf(fmaf(-q, 448.0f, x), c, q);
            if (to_bits(s) != to_bits(ref)) {
                printf("MISMATCH x=0x%08x: 0x%08x vs IEEE 0x%08x\n", u, to_bits(s), to_bits(ref));
                return 1;
            }
            ++n;
        }
    }
    printf("OK %llu\n", n);
    return 0;
}
