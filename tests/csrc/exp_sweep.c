/* Exhaustive accuracy sweep of the oracle's fp32 exponential against the fp64 libm exp.
 * Usage: exp_sweep  -> prints "maxulp <v> at <x>  checked <n>  special_fail <k>". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

float oracle_exp(float x);

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

int main(void) {
    const float lo = -0x1.5d589ep+6f;  /* smallest input whose exp is a normal float */
    const float hi = 0x1.62e42ep+6f;   /* largest input whose exp is finite */
    double maxulp = 0.0;
    float worst = 0.0f;
    long long checked = 0, special_fail = 0;
#pragma omp parallel
    {
        double my_max = 0.0; float my_worst = 0.0f; long long my_n = 0, my_fail = 0;
#pragma omp for schedule(dynamic, 1 << 20)
        for (long long b = 0; b < (1LL << 32); ++b) {
            float x = f_of((uint32_t)b);
            if (x != x) { if (oracle_exp(x) == oracle_exp(x)) my_fail++; continue; }
            float y = oracle_exp(x);
            if (x > 0x1.62e430p+6f) { if (!(isinf(y) && y > 0)) my_fail++; continue; }
            if (x < lo) { if (y != 0.0f) my_fail++; continue; }
            if (x > hi) continue; /* the single input between the cut-offs overflows in the scaling */
            double r = exp((double)x);
            int e; frexp(r, &e);
            double ulp = ldexp(1.0, e - 24);
            double err = fabs((double)y - r) / ulp;
            if (err > my_max) { my_max = err; my_worst = x; }
            my_n++;
        }
#pragma omp critical
        {
            if (my_max > maxulp) { maxulp = my_max; worst = my_worst; }
            checked += my_n; special_fail += my_fail;
        }
    }
    printf("maxulp %.6f at %a checked %lld special_fail %lld\n", maxulp, worst, checked, special_fail);
    return 0;
}
