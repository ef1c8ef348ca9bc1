// Float elementary functions of the device code, also compiled for the host so that
// their accuracy can be swept against a float64 libm on the CPU.
//
// cossin_rev: (cos, sin) of 2 pi r for r in [-1/2, 1/2].  The quadrant comes from
// rint(4 r); on the remaining f in [-1/2, 1/2], sin(pi f / 2) = f S(f^2) and
// cos(pi f / 2) = C(f^2) with S of degree 3 and C of degree 4 in f^2, fitted here by
// iteratively reweighted least squares (Lawson's method towards the minimax fit;
// aberration_phase_variance_amd/csrc/fit_math_polys.py).  Max error about 1e-7.
//
// atan2_f: octant reduction to t = min(|x|, |y|) / max(|x|, |y|) in [0, 1], then
// atan(t) = t P(t^2) with P of degree 7 in t^2 (8 coefficients), fitted the same way
// on the relative error over (0, 1]; the octant is undone afterwards.  Evaluated in
// float (host sweep against float64 libm): relative error at most 2.9e-7 at every
// angle; absolute error at most 1.9e-7 rad for |phase| <= pi/4 and 3.9e-7 rad near
// +-pi, where one float ulp is already 2.4e-7.  atan2(0, 0) = 0; NaN inputs give NaN.
// On the device the division is the hardware reciprocal (about 1 ulp); on the host
// it is exact.
#pragma once

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define SSB_HD __host__ __device__
#define SSB_INLINE __forceinline__
#else
#include <cmath>
#define SSB_HD
#define SSB_INLINE inline
#endif

#ifndef SSB_ATAN_TERMS
#define SSB_ATAN_TERMS 8
#endif

namespace ssb {

SSB_HD SSB_INLINE float rcp_approx(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_rcpf(x);
#else
    return 1.0f / x;
#endif
}

// (cos, sin) of 2 pi r into c, s
SSB_HD SSB_INLINE void cossin_rev_cs(float r, float& c, float& s) {
    const float x = 4.0f * r;
    const float q = rintf(x);
    const float f = x - q;
    const float s2 = f * f;
    const float sn = f * fmaf(fmaf(fmaf(-4.592288285e-03f, s2, 7.967590541e-02f), s2, -6.459629536e-01f), s2,
                              1.570796251e+00f);
    const float cs = fmaf(fmaf(fmaf(fmaf(9.040214936e-04f, s2, -2.086028829e-02f), s2, 2.536692321e-01f), s2,
                               -1.233700514e+00f),
                          s2, 1.0f);
    const int qi = (int)q & 3;
    const float sb = (qi & 1) ? cs : sn;
    const float cb = (qi & 1) ? sn : cs;
    c = ((qi + 1) & 2) ? -cb : cb;
    s = (qi & 2) ? -sb : sb;
}

// atan(t) for t in [0, 1]
SSB_HD SSB_INLINE float atan_unit(float t) {
    const float s = t * t;
#if SSB_ATAN_TERMS == 7
    float p = 8.250554092e-03f;
    p = fmaf(p, s, -3.822105378e-02f);
    p = fmaf(p, s, 8.530547470e-02f);
    p = fmaf(p, s, -1.356764287e-01f);
    p = fmaf(p, s, 1.990287155e-01f);
    p = fmaf(p, s, -3.332884312e-01f);
#elif SSB_ATAN_TERMS == 8
    float p = -4.822450690e-03f;
    p = fmaf(p, s, 2.473379672e-02f);
    p = fmaf(p, s, -6.020280346e-02f);
    p = fmaf(p, s, 9.968453646e-02f);
    p = fmaf(p, s, -1.404132247e-01f);
    p = fmaf(p, s, 1.997421384e-01f);
    p = fmaf(p, s, -3.333239257e-01f);
#else
    float p = 2.903556684e-03f;
    p = fmaf(p, s, -1.628302597e-02f);
    p = fmaf(p, s, 4.303940013e-02f);
    p = fmaf(p, s, -7.533679157e-02f);
    p = fmaf(p, s, 1.065467894e-01f);
    p = fmaf(p, s, -1.420713365e-01f);
    p = fmaf(p, s, 1.999305487e-01f);
    p = fmaf(p, s, -3.333309293e-01f);
#endif
    p = fmaf(p, s, 1.0f);
    return t * p;
}

SSB_HD SSB_INLINE float atan2_f(float y, float x) {
    const float ax = fabsf(x), ay = fabsf(y);
    const float mx = fmaxf(ax, ay), mn = fminf(ax, ay);
    const float t = mx > 0.f ? mn * rcp_approx(mx) : 0.f;
    float a = atan_unit(t);
    a = ay > ax ? 1.57079632679489662f - a : a;
    a = x < 0.f ? 3.14159265358979324f - a : a;
    a = copysignf(a, y);
    return (x != x || y != y) ? x + y : a;
}

}  // namespace ssb
