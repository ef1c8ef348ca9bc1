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

namespace ssb {

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
            float2 w1, w2, w4;
            sincospif((float)(SIGN * 2 * k) / (float)(ns * R), &w1.y, &w1.x);
            sincospif((float)(SIGN * 4 * k) / (float)(ns * R), &w2.y, &w2.x);
            sincospif((float)(SIGN * 8 * k) / (float)(ns * R), &w4.y, &w4.x);
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
#pragma unroll
            for (int r = 0; r < R; ++r) buf[exch_swizzle<N>(p, bb + r * ns)] = x[r];
            wave_lds_fence();
#pragma unroll
            for (int r = 0; r < R; ++r) x[r] = buf[exch_swizzle<N>(p, j + r * L)];
            ns *= R;
        }
    }
};

}  // namespace ssb
