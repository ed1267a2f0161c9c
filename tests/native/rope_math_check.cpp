// Host check of the executor's double-precision RoPE angle routines against
// the C library in long double.  Prints one line per routine:
//   <name> <max error> <count>
// (relative error for log2/exp2/angle, absolute for sin/cos).
#define GPUOS_HD
#include "rope_math.h"

#include <math.h>
#include <stdint.h>
#include <stdio.h>

using namespace gpuos::rmath;

static uint64_t st = 0x9E3779B97F4A7C15ull;
static double uni() {  // SplitMix64 -> [0, 1)
    uint64_t z = (st += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * 0x1.0p-53;
}

int main() {
    long double e_log = 0, e_exp = 0, e_sin = 0, e_cos = 0, e_ang = 0;
    const int n = 200000;
    for (int i = 0; i < n; ++i) {
        const double x = exp2(60.0 * uni() - 20.0);
        e_log = fmaxl(e_log, fabsl((log2_d(x) - log2l(x)) / log2l(x)));
        const double y = 80.0 * uni() - 40.0;
        e_exp = fmaxl(e_exp, fabsl((exp2_d(y) - exp2l(y)) / exp2l(y)));
        // angles up to 65535 radians, plus points next to multiples of pi/2
        double a = 65535.0 * uni();
        if (i % 4 == 1) a = nearbyint(a) * 1.5707963267948966;
        if (i % 4 == 2) a = 1e-3 * uni();
        double s, c;
        sincos_d(a, &s, &c);
        e_sin = fmaxl(e_sin, fabsl(s - sinl(a)));
        e_cos = fmaxl(e_cos, fabsl(c - cosl(a)));
    }
    const double thetas[] = {10000.0, 500000.0, 10.0, 1e6};
    const uint32_t dims[] = {64, 128, 256, 96};
    const double positions[] = {0.0, 1.0, 17.0, 4095.0, 65534.0};
    for (double th : thetas)
        for (uint32_t D : dims)
            for (uint32_t pi = 0; pi < D / 2; ++pi)
                for (double pos : positions) {
                    const long double ref = (long double)pos * powl((long double)th, -2.0L * pi / D);
                    const double g = rope_angle(pos, log2_d(th), pi, D);
                    if (ref != 0) e_ang = fmaxl(e_ang, fabsl((g - ref) / ref));
                    else if (g != 0) e_ang = 1;
                }
    printf("log2 %.3Le %d\nexp2 %.3Le %d\nsin %.3Le %d\ncos %.3Le %d\nangle %.3Le %d\n",
           e_log, n, e_exp, n, e_sin, n, e_cos, n, e_ang, 4 * 4 * 5);
    return 0;
}
