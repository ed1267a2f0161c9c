// Double-precision exp2, log2 and sincos for RoPE angles.
//
// RoPE rotates pair i of a head by pos * theta^(-2i/D) radians (RoFormer,
// section 3.2; the GPUOS digest lists RoPE among the micro-ops).  Angles
// reach a few thousand radians, and a bf16 result must stay within one ulp
// of the exactly rounded rotation even where the two products cancel, so
// the angle and its sine and cosine are computed in double.  These routines
// are short on purpose: a persistent executor keeps every op body in one
// kernel, and library pow/sincos would add a few thousand instructions to
// it.  Each is accurate to a few double ulps over the arguments used here:
//  - log2_d: x > 0 normal.  x = m 2^e with m in [sqrt(1/2), sqrt(2)),
//    ln m = 2 atanh(s), s = (m-1)/(m+1), |s| <= 0.172, series to s^21.
//  - exp2_d: |y| < 1000.  y = n + f, |f| <= 1/2; e^(f ln 2) by its Taylor
//    series to degree 14 (|f ln 2| <= 0.347); scaled by 2^n.
//  - sincos_d: 0 <= a < 2^20.  a = k pi/2 + r with pi/2 split in three
//    doubles (32 + 32 + 53 bits, so k pi/2_hi and k pi/2_mid are exact for
//    k < 2^21) and fused multiply-adds; sin r and cos r by their Taylor
//    series to degree 19 and 20 on |r| <= pi/4 (plus rounding); the
//    quadrant k mod 4 swaps and negates them.
#pragma once
#include <math.h>
#include <stdint.h>

#ifndef GPUOS_HD
#define GPUOS_HD __host__ __device__
#endif

namespace gpuos {
namespace rmath {

constexpr double SQRT2 = 1.4142135623730951;
constexpr double LN2 = 0.6931471805599453;
constexpr double LOG2E = 1.4426950408889634;
constexpr double TWO_OVER_PI = 0.6366197723675814;
constexpr double PIO2_1 = 1.5707963267341256;      // pi/2 to 32 bits
constexpr double PIO2_2 = 6.077100506303966e-11;   // the next 32 bits
constexpr double PIO2_3 = 2.0222662487959506e-21;  // the next 53 bits

constexpr double inv_fact(int n) {
    double f = 1.0;
    for (int i = 2; i <= n; ++i) f *= (double)i;
    return 1.0 / f;
}

// sign(N) / |N|!, as a compile-time constant
template <int N>
struct Coef {
    static constexpr double v = (N < 0 ? -1.0 : 1.0) * inv_fact(N < 0 ? -N : N);
};

GPUOS_HD inline double log2_d(double x) {
    int e = 0;
    double m = frexp(x, &e);  // [0.5, 1)
    if (m < SQRT2 * 0.5) {
        m *= 2.0;
        e -= 1;
    }
    const double s = (m - 1.0) / (m + 1.0);
    const double s2 = s * s;
    double p = 1.0 / 21.0;
    p = fma(p, s2, 1.0 / 19.0);
    p = fma(p, s2, 1.0 / 17.0);
    p = fma(p, s2, 1.0 / 15.0);
    p = fma(p, s2, 1.0 / 13.0);
    p = fma(p, s2, 1.0 / 11.0);
    p = fma(p, s2, 1.0 / 9.0);
    p = fma(p, s2, 1.0 / 7.0);
    p = fma(p, s2, 1.0 / 5.0);
    p = fma(p, s2, 1.0 / 3.0);
    const double lnm = 2.0 * fma(s * s2, p, s);
    return fma(lnm, LOG2E, (double)e);
}

GPUOS_HD inline double exp2_d(double y) {
    const double n = rint(y);
    const double t = (y - n) * LN2;
    double p = Coef<14>::v;
    p = fma(p, t, Coef<13>::v);
    p = fma(p, t, Coef<12>::v);
    p = fma(p, t, Coef<11>::v);
    p = fma(p, t, Coef<10>::v);
    p = fma(p, t, Coef<9>::v);
    p = fma(p, t, Coef<8>::v);
    p = fma(p, t, Coef<7>::v);
    p = fma(p, t, Coef<6>::v);
    p = fma(p, t, Coef<5>::v);
    p = fma(p, t, Coef<4>::v);
    p = fma(p, t, Coef<3>::v);
    p = fma(p, t, Coef<2>::v);
    p = fma(p, t, 1.0);
    p = fma(p, t, 1.0);
    return ldexp(p, (int)n);
}

GPUOS_HD inline void sincos_d(double a, double* sn, double* cs) {
    const double k = rint(a * TWO_OVER_PI);
    double r = fma(-k, PIO2_1, a);
    r = fma(-k, PIO2_2, r);
    r = fma(-k, PIO2_3, r);
    const double r2 = r * r;
    // sin r = r (1 - r^2/3! + r^4/5! - ...), cos r = 1 - r^2/2! + ...
    double ps = Coef<-19>::v;
    ps = fma(ps, r2, Coef<17>::v);
    ps = fma(ps, r2, Coef<-15>::v);
    ps = fma(ps, r2, Coef<13>::v);
    ps = fma(ps, r2, Coef<-11>::v);
    ps = fma(ps, r2, Coef<9>::v);
    ps = fma(ps, r2, Coef<-7>::v);
    ps = fma(ps, r2, Coef<5>::v);
    ps = fma(ps, r2, Coef<-3>::v);
    const double s = fma(r * r2, ps, r);
    double pc = Coef<20>::v;
    pc = fma(pc, r2, Coef<-18>::v);
    pc = fma(pc, r2, Coef<16>::v);
    pc = fma(pc, r2, Coef<-14>::v);
    pc = fma(pc, r2, Coef<12>::v);
    pc = fma(pc, r2, Coef<-10>::v);
    pc = fma(pc, r2, Coef<8>::v);
    pc = fma(pc, r2, Coef<-6>::v);
    pc = fma(pc, r2, Coef<4>::v);
    pc = fma(pc, r2, Coef<-2>::v);
    const double c = fma(r2, pc, 1.0);
    const int q = (int)((long long)k & 3);
    const double s1 = (q & 1) ? c : s;
    const double c1 = (q & 1) ? s : c;
    *sn = (q & 2) ? -s1 : s1;
    *cs = ((q + 1) & 2) ? -c1 : c1;
}

// pos * theta^(-2i/D): the rotation angle of pair i at position pos
GPUOS_HD inline double rope_angle(double pos, double log2_theta, uint32_t i, uint32_t D) {
    return pos * exp2_d(-2.0 * (double)i / (double)D * log2_theta);
}

}  // namespace rmath
}  // namespace gpuos
