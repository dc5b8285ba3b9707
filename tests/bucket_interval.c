#include <math.h>
#include <stdio.h>
#include <stdint.h>
#include <stdlib.h>
/* Checks, with the float32 arithmetic of the register-path top-k, that the
   clamped bucket 1 + clamp(int(fma(v, -s, vmax*s)), 0, KB-3) equals b exactly
   when the fma result lies in [b-1, b) (the first bucket open below, the last
   open above), and that -inf falls in no bucket.  Rows span ranges from 1 down
   to 1e-8 of their largest value, where the rounded vmax*s makes the fma result
   negative. */
#define KB 2048
static uint64_t st = 88172645463325252ull;
static double urand(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return (st >> 11) * (1.0 / 9007199254740992.0); }
static int bucket_new(float v, float s, float off) { int i = (int)fmaf(v, -s, off); if (i > KB - 3) i = KB - 3; if (i < 0) i = 0; return 1 + i; }
static int bucket_old(float v, float s, float off) { int i = (int)fmaf(v, -s, off); if (i > KB - 3) i = KB - 3; return 1 + i; }
int main(void) {
    long bad = 0, neg_old = 0, checked = 0;
    for (int row = 0; row < 20000; ++row) {
        int n = 64;
        float base = (float)((urand() - 0.5) * pow(10.0, urand() * 12 - 4));
        float spread = (float)(fabs(base) * pow(10.0, -urand() * 8) + 1e-30);
        float v[64];
        float mx = -INFINITY, mn = INFINITY;
        for (int i = 0; i < n; ++i) {
            v[i] = base + spread * (float)urand();
            if (urand() < 0.2) v[i] = base;  /* ties at the minimum */
            mx = fmaxf(mx, v[i]); mn = fminf(mn, v[i]);
        }
        float span = mx - mn;
        float sc = (span > 0.0f && isfinite(span)) ? (float)(KB - 3) / span : 0.0f;
        float off = mx * sc;
        for (int i = 0; i < n; ++i) {
            int b = bucket_new(v[i], sc, off);
            if (bucket_old(v[i], sc, off) < 1) ++neg_old;
            float f = fmaf(v[i], -sc, off);
            for (int bs = 1; bs <= KB - 2; bs += (bs < 4 || bs > KB - 6) ? 1 : 97) {
                float lo = bs <= 1 ? -INFINITY : (float)(bs - 1), hi = bs >= KB - 2 ? INFINITY : (float)bs;
                int by_f = (f >= lo) && (f < hi);
                if (by_f != (b == bs)) ++bad;
                ++checked;
            }
            if (!(b >= 1 && b <= KB - 2)) ++bad;
            float fi = fmaf(-INFINITY, -sc, off);
            for (int bs = 1; bs <= KB - 2; bs += KB - 3)
                if ((fi >= (bs <= 1 ? -INFINITY : (float)(bs - 1))) && (fi < (bs >= KB - 2 ? INFINITY : (float)bs))) ++bad;
        }
    }
    printf("checked %ld mismatches %ld rows-values where the old bucket went below 1: %ld\n", checked, bad, neg_old);
    return bad != 0;
}
