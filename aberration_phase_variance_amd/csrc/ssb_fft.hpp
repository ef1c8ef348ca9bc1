// Wave-level radix-R Stockham FFT for gfx950 (64-lane wavefronts).
//
// An FFT of length N is done by a group of L = N/R lanes.  Lane j (0 <= j < L)
// holds x[j + r L] for r = 0..R-1 in registers, both on entry and on exit
// (natural order).  Each of the log_R(N) passes twiddles, does a radix-R DFT in
// registers, and (except the last) exchanges through a group-private LDS buffer
// of N complex values.  A wave holds 64/L groups.  Lanes of one group exchange
// only with each other, so no workgroup barrier is needed, only wave-level
// ordering of the LDS accesses.
#pragma once

#include <hip/hip_runtime.h>

#include "ssb_math.hpp"

namespace ssb {

// (cos, sin) of 2 pi r for r in [-1/2, 1/2] (ssb_math.hpp)
__device__ __forceinline__ float2 cossin_rev(float r) {
    float c, s;
    cossin_rev_cs(r, c, s);
    return make_float2(c, s);
}

__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
// multiply by SIGN * i
template <int SIGN>
__device__ __forceinline__ float2 mul_si(float2 v) {
    return SIGN > 0 ? make_float2(-v.y, v.x) : make_float2(v.y, -v.x);
}

// Keep the compiler from moving LDS accesses across this point; the hardware
// executes one wave's LDS operations in order.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int SIGN>
__device__ __forceinline__ void dft2(float2 (&x)[2]) {
    float2 a = x[0];
    x[0] = cadd(a, x[1]);
    x[1] = csub(a, x[1]);
}

template <int SIGN>
__device__ __forceinline__ void dft4v(float2& x0, float2& x1, float2& x2, float2& x3) {
    float2 a = cadd(x0, x2), b = csub(x0, x2), c = cadd(x1, x3), d = mul_si<SIGN>(csub(x1, x3));
    x0 = cadd(a, c);
    x2 = csub(a, c);
    x1 = cadd(b, d);
    x3 = csub(b, d);
}

template <int SIGN>
__device__ __forceinline__ void dft4(float2 (&x)[4]) {
    dft4v<SIGN>(x[0], x[1], x[2], x[3]);
}

template <int SIGN>
__device__ __forceinline__ void dft8(float2 (&x)[8]) {
    float2 e0 = x[0], e1 = x[2], e2 = x[4], e3 = x[6];
    float2 o0 = x[1], o1 = x[3], o2 = x[5], o3 = x[7];
    dft4v<SIGN>(e0, e1, e2, e3);
    dft4v<SIGN>(o0, o1, o2, o3);
    const float c = 0.70710678118654752440f;
    // o_k * exp(SIGN i pi k / 4)
    float2 t1 = make_float2(c * (o1.x - SIGN * o1.y), c * (o1.y + SIGN * o1.x));
    float2 t2 = mul_si<SIGN>(o2);
    float2 t3 = make_float2(c * (-o3.x - SIGN * o3.y), c * (SIGN * o3.x - o3.y));
    x[0] = cadd(e0, o0);
    x[4] = csub(e0, o0);
    x[1] = cadd(e1, t1);
    x[5] = csub(e1, t1);
    x[2] = cadd(e2, t2);
    x[6] = csub(e2, t2);
    x[3] = cadd(e3, t3);
    x[7] = csub(e3, t3);
}

template <int R, int SIGN>
__device__ __forceinline__ void dft(float2 (&x)[R]) {
    if constexpr (R == 2) dft2<SIGN>(x);
    else if constexpr (R == 4) dft4<SIGN>(x);
    else dft8<SIGN>(x);
}

template <int N> struct FftShape;
template <> struct FftShape<512> { static constexpr int R = 8, P = 3; };
template <> struct FftShape<256> { static constexpr int R = 4, P = 4; };
template <> struct FftShape<128> { static constexpr int R = 2, P = 7; };
template <> struct FftShape<64>  { static constexpr int R = 4, P = 3; };
template <> struct FftShape<32>  { static constexpr int R = 2, P = 5; };
template <> struct FftShape<1024> { static constexpr int R = 16, P = 3; };   // radices 16, 8, 8 (below)

// LDS scratch (complex values) one transform's exchanges need.
// Exchange address of register r after radix-8 pass p of the 512-point transform
// in the padded layout p(i) = i + i/8 (one pad slot per 8 values, 576 slots): a lane
// base plus a constant, so no lane addresses need to stay live.  Writes of pass 0:
// p(8 j + r) = 9 j + r; writes of pass 1: p(64 (j/8) + j%8 + 8 r) = 72 (j/8) + j%8 + 9 r;
// reads: p(j + 64 r) = j + j/8 + 72 r.  Unlike the XOR swizzles it leaves some 2-way
// bank conflicts.
__device__ __forceinline__ int pad512_write(int p, int j, int r) {
    return p == 0 ? 9 * j + r : 72 * (j >> 3) + (j & 7) + 9 * r;
}
__device__ __forceinline__ int pad512_read(int j, int r) { return j + (j >> 3) + 72 * r; }

// Bijective LDS index maps for the exchange after pass p.  The write and the
// read of one exchange use the same map, so values are unchanged; the maps only
// spread each 64-lane access across banks.  For N = 512 (radix 8) they remove
// the bank conflicts of both exchanges (checked against 32- and 64-bank models);
// other sizes keep the plain index.
template <int N>
__device__ __forceinline__ int exch_swizzle(int p, int i) {
    if constexpr (N == 512) {
        if (p == 0) return i ^ (((i >> 3) ^ (i >> 6)) & 7);
        return i ^ ((((i) ^ (i >> 6)) & 7) << 3);
    } else {
        return i;
    }
}

template <int N, int SIGN>
struct WaveFFT {
    static constexpr int R = FftShape<N>::R;
    static constexpr int P = FftShape<N>::P;
    static constexpr int L = N / R;        // lanes per FFT
    static constexpr int W = 64 / L;       // FFTs per wave
    static constexpr int NT = (P > 1 ? P - 1 : 1);
    static constexpr int SCRATCH = N;      // LDS values one transform's exchanges use

    float2 tw[NT][R - 1];                  // per-lane twiddles of passes 1..P-1

    // j: lane index inside the group.
    __device__ __forceinline__ void init(int j) {
        int ns = R;
#pragma unroll
        for (int p = 1; p < P; ++p) {
            const int k = j & (ns - 1);
#pragma unroll
            for (int r = 1; r < R; ++r) {
                // exp(SIGN * 2 pi i k r / (ns R)): sincospi of an exact dyadic argument
                float s, c;
                sincospif((float)(SIGN * 2 * k * r) / (float)(ns * R), &s, &c);
                tw[p - 1][r - 1] = make_float2(c, s);
            }
            ns *= R;
        }
    }

    // The same twiddles for radix 8 from three sincospi per pass (r = 1, 2, 4) and
    // complex products for r = 3, 5, 6, 7 (two roundings more on those).
    __device__ __forceinline__ void init_products(int j) {
        static_assert(R == 8, "radix-8 products");
        int ns = R;
#pragma unroll
        for (int p = 1; p < P; ++p) {
            const int k = j & (ns - 1);
            // w1 = exp(2 pi i SIGN k / (ns R)) from the fitted sincos (about 15
            // instructions instead of about 40 for sincospi), w2 and w4 by squaring
            // (each squaring at most doubles its 1e-7 error)
            const float2 w1 = cossin_rev((float)(SIGN * k) / (float)(ns * R));
            const float2 w2 = make_float2(fmaf(w1.x, w1.x, -w1.y * w1.y), 2.f * w1.x * w1.y);
            const float2 w4 = make_float2(fmaf(w2.x, w2.x, -w2.y * w2.y), 2.f * w2.x * w2.y);
            tw[p - 1][0] = w1;
            tw[p - 1][1] = w2;
            tw[p - 1][2] = cmul(w1, w2);
            tw[p - 1][3] = w4;
            tw[p - 1][4] = cmul(w4, w1);
            tw[p - 1][5] = cmul(w4, w2);
            tw[p - 1][6] = cmul(w4, tw[p - 1][2]);
            ns *= R;
        }
    }

    // The same twiddles read from a table in global memory laid out as WaveFFTT's
    // (filled once with WaveFFTT<N, SIGN>::fill): no transcendentals per workgroup.
    __device__ __forceinline__ void load(const float2* __restrict__ tab, int j) {
        int ns = R, base = 0;
#pragma unroll
        for (int p = 1; p < P; ++p) {
            const int k = j & (ns - 1);
#pragma unroll
            for (int r = 1; r < R; ++r) tw[p - 1][r - 1] = tab[base + (r - 1) * ns + k];
            base += (R - 1) * ns;
            ns *= R;
        }
    }

    // In-place transform of the group's values; buf holds N complex values private
    // to this group (clobbered).
    __device__ __forceinline__ void run(float2 (&x)[R], float2* buf, int j) const {
        int ns = 1;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            if (p > 0) {
#pragma unroll
                for (int r = 1; r < R; ++r) x[r] = cmul(x[r], tw[p - 1][r - 1]);
            }
            dft<R, SIGN>(x);
            if (p == P - 1) break;
            const int k = j & (ns - 1);
            const int base = (j - k) * R + k;
            wave_lds_fence();
#pragma unroll
            for (int r = 0; r < R; ++r) buf[exch_swizzle<N>(p, base + r * ns)] = x[r];
            wave_lds_fence();
#pragma unroll
            for (int r = 0; r < R; ++r) x[r] = buf[exch_swizzle<N>(p, j + r * L)];
            ns *= R;
        }
    }
};

// The same transform with the per-lane twiddles read from a workgroup table in
// LDS instead of held in registers (frees 2 (R-1) complex registers per lane).
// Table layout: for pass p = 1..P-1 (ns = R^p) a block [R-1][ns] of
// exp(SIGN 2 pi i k r / (ns R)), r = 1..R-1, k < ns; N - R entries in all.
template <int N, int SIGN>
struct WaveFFTT {
    static constexpr int R = FftShape<N>::R;
    static constexpr int P = FftShape<N>::P;
    static constexpr int L = N / R;
    static constexpr int W = 64 / L;
    static constexpr int TABLE = N - R;
    // LDS values one transform's exchanges use: N = 512 takes the padded layout here,
    // which keeps no lane addresses live across the row pass's loop
    static constexpr int SCRATCH = N == 512 ? N + N / 8 : N;

    __device__ static void fill(float2* tab, int tid, int nthreads) {
        for (int e = tid; e < TABLE; e += nthreads) {
            int base = 0, ns = R;
            // locate the pass block holding entry e
            while (e >= base + (R - 1) * ns) {
                base += (R - 1) * ns;
                ns *= R;
            }
            const int off = e - base;
            const int r = off / ns + 1, k = off % ns;
            float s, c;
            sincospif((float)(SIGN * 2 * k * r) / (float)(ns * R), &s, &c);
            tab[e] = make_float2(c, s);
        }
    }

    __device__ __forceinline__ void run(float2 (&x)[R], float2* buf, int j, const float2* tab) const {
        int ns = 1, base = 0;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            if (p > 0) {
                const int k = j & (ns - 1);
#pragma unroll
                for (int r = 1; r < R; ++r) x[r] = cmul(x[r], tab[base + (r - 1) * ns + k]);
                base += (R - 1) * ns;
            }
            dft<R, SIGN>(x);
            if (p == P - 1) break;
            const int k = j & (ns - 1);
            const int bb = (j - k) * R + k;
            wave_lds_fence();
            if constexpr (N == 512) {
#pragma unroll
                for (int r = 0; r < R; ++r) buf[pad512_write(p, j, r)] = x[r];
                wave_lds_fence();
#pragma unroll
                for (int r = 0; r < R; ++r) x[r] = buf[pad512_read(j, r)];
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) buf[exch_swizzle<N>(p, bb + r * ns)] = x[r];
                wave_lds_fence();
#pragma unroll
                for (int r = 0; r < R; ++r) x[r] = buf[exch_swizzle<N>(p, j + r * L)];
            }
            ns *= R;
        }
    }
};

// ---------------------------------------------------------------- N = 1024
// One wave per transform, lane j holds x[j + 64 r] for r < 16, in and out.  Mixed
// radices 16, 8, 8 in self-sorting (Stockham) form: pass 0 is a radix-16 DFT of the
// lane's own values; passes 1 and 2 are radix 8 on 128 virtual lanes jv = j + 64 h
// (h = 0, 1), the lane's values with r = h + 2 r'.  Pass p reads a[jv + (N/R_p) r],
// twiddles by exp(SIGN 2 pi i k r / (ns R_p)) with k = jv mod ns, applies the DFT and
// writes position (jv - k) R_p + k + r ns, ns being the product of the earlier
// radices; the last pass leaves X[jv + 128 r'] in the lane.

// radix-16 DFT in registers: 4 x radix 4 over n1 (n = 4 n1 + n2), twiddles
// exp(SIGN 2 pi i n2 k1 / 16), 4 x radix 4 over n2 (k = k1 + 4 k2)
template <int SIGN>
__device__ __forceinline__ void dft16(float2 (&x)[16]) {
    const float c1 = 0.92387953251128675613f, s1 = 0.38268343236508977173f, h2 = 0.70710678118654752440f;
    // w[m] = exp(SIGN 2 pi i m / 16) for the products m = n2 k1 that occur
    auto w16 = [&](int m) -> float2 {
        switch (m) {
            case 1: return make_float2(c1, SIGN * s1);
            case 2: return make_float2(h2, SIGN * h2);
            case 3: return make_float2(s1, SIGN * c1);
            case 4: return make_float2(0.f, (float)SIGN);
            case 6: return make_float2(-h2, SIGN * h2);
            default: return make_float2(-c1, -SIGN * s1);   // m = 9
        }
    };
#pragma unroll
    for (int n2 = 0; n2 < 4; ++n2) dft4v<SIGN>(x[n2], x[4 + n2], x[8 + n2], x[12 + n2]);
    // now x[4 k1 + n2] holds y[n2][k1]
#pragma unroll
    for (int n2 = 1; n2 < 4; ++n2)
#pragma unroll
        for (int k1 = 1; k1 < 4; ++k1) x[4 * k1 + n2] = cmul(x[4 * k1 + n2], w16(n2 * k1));
    float2 y[16];
#pragma unroll
    for (int k1 = 0; k1 < 4; ++k1) {
        float2 a0 = x[4 * k1], a1 = x[4 * k1 + 1], a2 = x[4 * k1 + 2], a3 = x[4 * k1 + 3];
        dft4v<SIGN>(a0, a1, a2, a3);
        y[k1] = a0;
        y[k1 + 4] = a1;
        y[k1 + 8] = a2;
        y[k1 + 12] = a3;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) x[k] = y[k];
}

// LDS index map of the N = 1024 exchanges: one pad slot after every 16 values,
// p(i) = i + i / 16, so a transform needs N + N/16 slots (SCRATCH).  Every
// exchange address is then a per-lane base plus a per-register constant (the
// instruction's immediate offset), and the stride-16 writes of pass 0 (17 j + r)
// spread over the banks.  The transform below writes p out per access pattern
// (base + constant), which the compiler cannot derive from p itself:
//   pass-0 write  p(16 j + r)                       = 17 j + r
//   radix-8 reads p(j + 64 h + 128 r)               = (j + j/16) + 68 h + 136 r
//   pass-1 write  p(128 (j/16 + 4 h) + j%16 + 16 r) = (136 (j/16) + j%16) + 544 h + 17 r

// Twiddles of the N = 1024 passes.  Pass 1: t[r-1] = exp(SIGN 2 pi i k r / 128),
// k = j mod 16.  Pass 2: exp(SIGN 2 pi i jv r / 1024) for jv = j (ta) and j + 64 (tb).
// Either from the table laid out as WaveFFTT<1024>'s, or computed: r = 1 from the
// fitted sincos, r = 2 and 4 by squaring, the other r as products; tb = ta times
// exp(SIGN i pi r / 8).
template <int SIGN>
__device__ __forceinline__ void tw1024_products(float2 (&t)[7], int k, float den) {
    const float2 w1 = cossin_rev((float)(SIGN * k) / den);
    const float2 w2 = make_float2(fmaf(w1.x, w1.x, -w1.y * w1.y), 2.f * w1.x * w1.y);
    const float2 w4 = make_float2(fmaf(w2.x, w2.x, -w2.y * w2.y), 2.f * w2.x * w2.y);
    t[0] = w1;
    t[1] = w2;
    t[2] = cmul(w1, w2);
    t[3] = w4;
    t[4] = cmul(w4, w1);
    t[5] = cmul(w4, w2);
    t[6] = cmul(w4, t[2]);
}

template <int SIGN>
__device__ __forceinline__ void tw1024_shift64(const float2 (&ta)[7], float2 (&tb)[7]) {
    const float c1 = 0.92387953251128675613f, s1 = 0.38268343236508977173f, h2 = 0.70710678118654752440f;
    const float2 c[7] = {make_float2(c1, SIGN * s1), make_float2(h2, SIGN * h2), make_float2(s1, SIGN * c1),
                         make_float2(0.f, (float)SIGN),  make_float2(-s1, SIGN * c1),
                         make_float2(-h2, SIGN * h2),   make_float2(-c1, SIGN * s1)};
#pragma unroll
    for (int r = 0; r < 7; ++r) tb[r] = cmul(ta[r], c[r]);
}

template <class T>
__device__ __forceinline__ void tw1024_load1(const T* tab, int j, float2 (&t)[7]) {
#pragma unroll
    for (int r = 1; r < 8; ++r) t[r - 1] = tab[(r - 1) * 16 + (j & 15)];
}
// Pass-2 block of the table: [r-1][64] (k < 64); the k + 64 rows are formed as
// tb = ta exp(SIGN i pi r / 8).  The half-size table (4.5 KB) lets the row pass keep
// four workgroups per CU in LDS (pass 2 at N = 1024: 2.85 against 3.26 ms).
constexpr int kTw1024Pass2 = 64;
template <int SIGN, class T>
__device__ __forceinline__ void tw1024_load2(const T* tab, int j, float2 (&ta)[7], float2 (&tb)[7]) {
#pragma unroll
    for (int r = 1; r < 8; ++r) ta[r - 1] = tab[112 + (r - 1) * kTw1024Pass2 + j];
    tw1024_shift64<SIGN>(ta, tb);
}

// The transform; get1(t) and get2(ta, tb) produce each pass's twiddles right before
// that pass, so that at most one pass's twiddles are live.
template <int SIGN, class Get1, class Get2>
__device__ __forceinline__ void fft1024_run(float2 (&x)[16], float2* buf, int j, Get1 get1, Get2 get2) {
    dft16<SIGN>(x);
    wave_lds_fence();
#pragma unroll
    for (int r = 0; r < 16; ++r) buf[17 * j + r] = x[r];
    wave_lds_fence();
    // pass 1: radix 8, ns = 16
    const float2* rd = buf + j + (j >> 4);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 8; ++r) x[8 * h + r] = rd[68 * h + 136 * r];
    {
        float2 t1[7];
        get1(t1);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float2 y[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) y[r] = r == 0 ? x[8 * h] : cmul(x[8 * h + r], t1[r - 1]);
            dft8<SIGN>(y);
#pragma unroll
            for (int r = 0; r < 8; ++r) x[8 * h + r] = y[r];
        }
    }
    wave_lds_fence();
    float2* wr = buf + 136 * (j >> 4) + (j & 15);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 8; ++r) wr[544 * h + 17 * r] = x[8 * h + r];
    wave_lds_fence();
    // pass 2: radix 8, ns = 128, k = jv
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 8; ++r) x[8 * h + r] = rd[68 * h + 136 * r];
    float2 t2a[7], t2b[7];
    get2(t2a, t2b);
    float2 out[16];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float2 y[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) y[r] = r == 0 ? x[8 * h] : cmul(x[8 * h + r], h == 0 ? t2a[r - 1] : t2b[r - 1]);
        dft8<SIGN>(y);
#pragma unroll
        for (int r = 0; r < 8; ++r) out[h + 2 * r] = y[r];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = out[r];
}

// Twiddle table of the N = 1024 transform: pass 1 block [r-1][16] (k < 16, over 128),
// then pass 2 block [r-1][kTw1024Pass2] (k < kTw1024Pass2, over 1024).
template <int SIGN>
struct WaveFFTT<1024, SIGN> {
    static constexpr int N = 1024, R = 16, P = 3, L = 64, W = 1;
    static constexpr int TABLE = 7 * 16 + 7 * kTw1024Pass2;
    static constexpr int SCRATCH = N + N / 16;

    __device__ static void fill(float2* tab, int tid, int nthreads) {
        for (int e = tid; e < TABLE; e += nthreads) {
            int r, k, den;
            if (e < 112) {
                r = e / 16 + 1;
                k = e % 16;
                den = 128;
            } else {
                r = (e - 112) / kTw1024Pass2 + 1;
                k = (e - 112) % kTw1024Pass2;
                den = 1024;
            }
            float s, c;
            sincospif((float)(SIGN * 2 * k * r) / (float)den, &s, &c);
            tab[e] = make_float2(c, s);
        }
    }

    // tab: the table (in LDS for the row pass), read pass by pass
    __device__ __forceinline__ void run(float2 (&x)[16], float2* buf, int j, const float2* tab) const {
        fft1024_run<SIGN>(
            x, buf, j, [&](float2 (&t)[7]) { tw1024_load1(tab, j, t); },
            [&](float2 (&ta)[7], float2 (&tb)[7]) { tw1024_load2<SIGN>(tab, j, ta, tb); });
    }
};

// Register form: load() takes the table from global memory pass by pass during
// run(); init() / init_products() select twiddles computed from six sincospi
// inside run() instead.
template <int SIGN>
struct WaveFFT<1024, SIGN> {
    static constexpr int N = 1024, R = 16, P = 3, L = 64, W = 1;
    static constexpr int SCRATCH = N + N / 16;
    const float2* tab = nullptr;

    __device__ __forceinline__ void init(int) { tab = nullptr; }
    __device__ __forceinline__ void init_products(int) { tab = nullptr; }
    __device__ __forceinline__ void load(const float2* __restrict__ t, int) { tab = t; }
    __device__ __forceinline__ void run(float2 (&x)[16], float2* buf, int j) const {
        if (tab) {
            const float2* t = tab;
            fft1024_run<SIGN>(
                x, buf, j, [&](float2 (&t1)[7]) { tw1024_load1(t, j, t1); },
                [&](float2 (&ta)[7], float2 (&tb)[7]) { tw1024_load2<SIGN>(t, j, ta, tb); });
        } else {
            fft1024_run<SIGN>(
                x, buf, j, [&](float2 (&t1)[7]) { tw1024_products<SIGN>(t1, j & 15, 128.0f); },
                [&](float2 (&ta)[7], float2 (&tb)[7]) {
                    tw1024_products<SIGN>(ta, j, 1024.0f);
                    tw1024_shift64<SIGN>(ta, tb);
                });
        }
    }
};

}  // namespace ssb
