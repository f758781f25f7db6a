// Pins the device-side division used for reference means (div_small in the HIP
// sources): exhaustive check that for every sum s of at most 8 OCP FP8 e4m3fn values (a multiple of
// 2^-9 with |s| <= 8*448) and k = 1..8, q = s*r, e = fma(-q,k,s), q' = fma(e,r,q)
// with r = RN(1/k) equals the correctly rounded s/k.
#include <math.h>
#include <stdio.h>
int main(void) {
    long bad = 0, total = 0;
    for (int k = 1; k <= 8; ++k) {
        const float kf = (float)k;
        const float r = 1.0f / kf;  // RN(1/k)
        for (long n = -1835008; n <= 1835008; ++n) {
            const float s = (float)ldexp((double)n, -9);  // exact: |n| < 2^21
            const float ref = (float)((double)s / (double)k);
            float q = s * r;
            const float e = fmaf(-q, kf, s);
            q = fmaf(e, r, q);
            ++total;
            if (q != ref && !(q == 0.0f && ref == 0.0f)) {
                if (bad < 5) printf("k=%d n=%ld s=%.9g got %.9g want %.9g\n", k, n, s, q, ref);
                ++bad;
            }
        }
    }
    printf("checked %ld, mismatches %ld\n", total, bad);
    return bad != 0;
}
