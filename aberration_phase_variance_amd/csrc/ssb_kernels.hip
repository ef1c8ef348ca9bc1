// HIP kernels of the SSB phase-variance path for gfx950.
//
// Layouts (complex64 = float2):
//   G cache        main [n_bf][N][N/2]   (v = 0 .. N/2-1), nyq [n_bf][N]   (v = N/2)
//   intermediate   main [trial][cap][N][N/2],             nyq [trial][cap][N]
//   S1 partials    float [trial][gcap][N][N] (one image per 32-BF group)
// Splitting the Nyquist column off keeps every main row a power-of-two run of
// complex values (2 KiB at N = 512), so rows and column tiles stay aligned.
//
// The per-BF 2-D inverse transform follows the two-pass structure the pages
// describe (Checkpoints page, "fftA intermediate and M5 hardware floor": a
// correct + column IFFT pass and a row IFFT + atan2 moments pass over
// 257 + 512 transforms per BF).  Here the row pass transforms two rows at once:
// the corrected spectrum is anti-Hermitian apart from the DC term and the
// Nyquist column, so the imaginary part of the object is the real inverse
// transform of -i * (column result) and its real part is fixed by columns 0 and
// N/2 (plus the DC).  Packing row y0 into the real part and row y1 into the
// imaginary part of one complex transform gives both.
#include "ssb_internal.hpp"
#include "ssb_fft.hpp"

#include <algorithm>

namespace ssb {

namespace {

constexpr int kTC = 16;       // columns per column-pass tile
constexpr int kPad = 1;       // LDS row padding (complex values)

enum ColMode { COL_CORRECT_INV = 0, COL_PLAIN_FWD = 1, COL_PLAIN_INV = 2 };

__device__ __forceinline__ double aperture_weight(double r2, const GeomDev& g) {
    if (r2 >= g.hi2) return 0.0;
    if (r2 <= g.lo2) return 1.0;
    const double a = (g.ra - sqrt(r2)) / g.w + 0.5;
    return fmin(fmax(a, 0.0), 1.0);
}

// C = G * T for half-plane entry (u, v) of the BF pixel at k = (kx, ky) pixels.
// T = conj(Gamma)/|Gamma| with Gamma = a(k) e^{i delta} [(a_- - a_+) cos chi_q - i (a_- + a_+) sin chi_q],
// where a_-+ = a(k -+ q), delta = 2 pi * 2 k^T M q and chi_q = 2 pi q^T M q: the
// definition's two shifted probe phases chi(k) - chi(k -+ q) = +-delta - chi_q
// regrouped, so the magnitude never comes from cancellation.  Geometry and phase
// arguments are double; the phasors and the product are float.
__device__ __forceinline__ float2 correct_entry(float2 gv, int u, int v, double kx, double ky,
                                                const TrialConst& m, const GeomDev& g) {
    const double fy = (double)(u < g.h ? u : u - g.n);
    const double fx = (double)v;
    const double qx0 = g.s * fx, qy0 = g.s * fy;
    const double qx = g.crot * qx0 - g.srot * qy0;
    const double qy = g.srot * qx0 + g.crot * qy0;
    const double dxm = kx - qx, dym = ky - qy, dxp = kx + qx, dyp = ky + qy;
    const double am = aperture_weight(dxm * dxm + dym * dym, g);
    const double apl = aperture_weight(dxp * dxp + dyp * dyp, g);
    if (am == 0.0 && apl == 0.0) return make_float2(0.f, 0.f);
    const double mqx = m.mxx * qx + m.mxy * qy;
    const double mqy = m.mxy * qx + m.myy * qy;
    const double d = 2.0 * (kx * mqx + ky * mqy);
    const double cq = qx * mqx + qy * mqy;
    const float dr = (float)(d - rint(d));
    const float cr = (float)(cq - rint(cq));
    float sd, cd, sc, cc;
    sincospif(2.0f * dr, &sd, &cd);
    sincospif(2.0f * cr, &sc, &cc);
    const float br = (float)(am - apl) * cc;   // Re conj(bracket)
    const float bi = (float)(am + apl) * sc;   // Im conj(bracket)
    const float mag2 = br * br + bi * bi;
    if (mag2 == 0.0f) return make_float2(0.f, 0.f);
    const float inv = rsqrtf(mag2);
    const float tr = (cd * br + sd * bi) * inv;
    const float ti = (cd * bi - sd * br) * inv;
    return make_float2(gv.x * tr - gv.y * ti, gv.x * ti + gv.y * tr);
}

// Column pass: one workgroup = one plane x one tile of kTC columns (or the
// Nyquist column), one trial.  Coalesced tile load (optionally corrected) into
// LDS, one wave-level FFT per column, coalesced store.  in == out is allowed
// (the whole tile is read before any store).
template <int N, int MODE>
__global__ __launch_bounds__(256) void k_cols(const float2* in_m, const float2* in_n, float2* out_m,
                                              float2* out_n, int64_t out_tstride_m,
                                              int64_t out_tstride_n, int64_t bf0,
                                              const double2* __restrict__ kb,
                                              const uint8_t* __restrict__ active,
                                              const TrialConst* __restrict__ tc, GeomDev geo) {
    constexpr int H = N / 2;
    constexpr int LD = N + kPad;
    constexpr int SIGN = (MODE == COL_PLAIN_FWD) ? -1 : 1;
    using F = WaveFFT<N, SIGN>;
    __shared__ float2 tile[kTC * LD];

    const int tid = threadIdx.x;
    const int plane = blockIdx.y;
    const int trial = blockIdx.z;
    const bool nyq = blockIdx.x == H / kTC;
    const int v0 = blockIdx.x * kTC;

    double kx = 0.0, ky = 0.0;
    TrialConst m{};
    if constexpr (MODE == COL_CORRECT_INV) {
        if (!active[bf0 + plane]) return;          // zero-aperture BF: phase is exactly 0
        const double2 k = kb[bf0 + plane];
        kx = k.x;
        ky = k.y;
        m = tc[trial];
    }
    const float2* pin_m = in_m + (int64_t)plane * N * H;
    const float2* pin_n = in_n + (int64_t)plane * N;
    float2* pout_m = out_m + (int64_t)trial * out_tstride_m + (int64_t)plane * N * H;
    float2* pout_n = out_n + (int64_t)trial * out_tstride_n + (int64_t)plane * N;

    if (!nyq) {
        const int c = tid % kTC;
        for (int u = tid / kTC; u < N; u += 256 / kTC) {
            float2 gv = pin_m[(int64_t)u * H + v0 + c];
            if constexpr (MODE == COL_CORRECT_INV) {
                gv = (u == 0 && v0 + c == 0) ? make_float2(0.f, 0.f)
                                             : correct_entry(gv, u, v0 + c, kx, ky, m, geo);
            }
            tile[c * LD + u] = gv;
        }
    } else {
        for (int u = tid; u < N; u += 256) {
            float2 gv = pin_n[u];
            if constexpr (MODE == COL_CORRECT_INV) gv = correct_entry(gv, u, H, kx, ky, m, geo);
            tile[u] = gv;
        }
    }
    __syncthreads();

    const int lane = tid & 63;
    const int grp = (tid >> 6) * F::W + lane / F::L;
    const int j = lane % F::L;
    constexpr int NG = 4 * F::W;
    F fft;
    fft.init(j);
    const int ncols = nyq ? 1 : kTC;
    for (int c = grp; c < ncols; c += NG) {
        float2 x[F::R];
#pragma unroll
        for (int r = 0; r < F::R; ++r) x[r] = tile[c * LD + j + r * F::L];
        fft.run(x, &tile[c * LD], j);
        wave_lds_fence();
#pragma unroll
        for (int r = 0; r < F::R; ++r) tile[c * LD + j + r * F::L] = x[r];
    }
    __syncthreads();

    if (!nyq) {
        const int c = tid % kTC;
        for (int y = tid / kTC; y < N; y += 256 / kTC) pout_m[(int64_t)y * H + v0 + c] = tile[c * LD + y];
    } else {
        for (int y = tid; y < N; y += 256) pout_n[y] = tile[y];
    }
}

// Assemble Z(v) = B0(v) + i B1(v), B_k = -i * (column result of row y_k),
// extended Hermitian (B(N - v) = conj B(v)), with only real parts kept at
// v = 0 and v = N/2; lane j gets v = j + r L.
template <int N, int R, int L>
__device__ __forceinline__ void assemble_row_pair(const float2* r0, const float2* r1, float2 h0, float2 h1,
                                                  int j, float2 (&x)[R]) {
    constexpr int H = N / 2;
#pragma unroll
    for (int r = 0; r < R / 2; ++r) {
        const int v = j + r * L;
        float2 a0 = r0[v], a1 = r1[v];
        if (v == 0) {
            a0.x = 0.f;
            a1.x = 0.f;
        }
        x[r] = make_float2(a0.y + a1.x, a1.y - a0.x);
    }
#pragma unroll
    for (int r = R / 2; r < R; ++r) {
        const int v = j + r * L;
        if (v == H) {
            x[r] = make_float2(h0.y, h1.y);
        } else {
            const int w = N - v;
            const float2 a0 = r0[w], a1 = r1[w];
            x[r] = make_float2(a0.y - a1.x, a0.x + a1.y);
        }
    }
}

// Pass 2: one workgroup = 4*W row pairs x one 32-BF group x one trial.  Loops
// over the group's BF pixels in order, accumulating per-pixel phase sums in
// registers (float) and the squared phase (double per lane).
template <int N>
__global__ __launch_bounds__(256) void k_pass2(const float2* __restrict__ im, const float2* __restrict__ in,
                                               int cap, const uint8_t* __restrict__ active, int64_t bf0,
                                               int cb, float dcf, float* __restrict__ part_s1,
                                               double* __restrict__ part_s2, int gcap) {
    constexpr int H = N / 2;
    using F = WaveFFT<N, +1>;
    constexpr int R = F::R, L = F::L;
    __shared__ float2 buf[4 * F::W][N];
    __shared__ double red[4];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int grp = wave * F::W + lane / L;
    const int j = lane % L;
    const int rp = blockIdx.x * (4 * F::W) + grp;
    const int y0 = 2 * rp;
    const int g = blockIdx.y;
    const int t = blockIdx.z;
    const int b_lo = g * kGroupBF;
    const int b_hi = min(cb, b_lo + kGroupBF);

    F fft;
    fft.init(j);
    float s1a[R], s1b[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        s1a[r] = 0.f;
        s1b[r] = 0.f;
    }
    double s2 = 0.0;
    const float sgn = (j & 1) ? -1.f : 1.f;   // (-1)^x for x = j + r L, L even

    for (int b = b_lo; b < b_hi; ++b) {
        if (!active[bf0 + b]) continue;
        const int64_t pl = (int64_t)t * cap + b;
        const float2* r0 = im + (pl * N + y0) * H;
        const float2* r1 = r0 + H;
        const float2 h0 = in[pl * N + y0], h1 = in[pl * N + y0 + 1];
        const float2 z0 = r0[0], z1 = r1[0];
        float2 x[R];
        assemble_row_pair<N, R, L>(r0, r1, h0, h1, j, x);
        fft.run(x, buf[grp], j);
        const float den0 = dcf + z0.x + sgn * h0.x;
        const float den1 = dcf + z1.x + sgn * h1.x;
        float p2 = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float pa = atan2f(x[r].x, den0);
            const float pb = atan2f(x[r].y, den1);
            s1a[r] += pa;
            s1b[r] += pb;
            p2 += pa * pa + pb * pb;
        }
        s2 += (double)p2;
    }

    float* o = part_s1 + (((int64_t)t * gcap + g) * N + y0) * N;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        o[j + r * L] = s1a[r];
        o[N + j + r * L] = s1b[r];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s2 += __shfl_xor(s2, off);
    if (lane == 0) red[wave] = s2;
    __syncthreads();
    if (tid == 0) part_s2[((int64_t)t * gcap + g) * gridDim.x + blockIdx.x] = ((red[0] + red[1]) + red[2]) + red[3];
}

// S1run[t][p] += sum over groups g (in order) of part_s1[t][g][p], in double.
__global__ __launch_bounds__(256) void k_accum_s1(const float* __restrict__ part, int gcap, int ng,
                                                  int64_t n2, double* __restrict__ s1run) {
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int t = blockIdx.y;
    if (p >= n2) return;
    double acc = s1run[t * n2 + p];
    const float* src = part + (int64_t)t * gcap * n2 + p;
    for (int g = 0; g < ng; ++g) acc += (double)src[(int64_t)g * n2];
    s1run[t * n2 + p] = acc;
}

// S2run[t] += sum over groups g (in order) of (fixed-tree sum over row blocks).
__global__ __launch_bounds__(64) void k_accum_s2(const double* __restrict__ part, int gcap, int ng, int rb,
                                                 double* __restrict__ s2run) {
    const int t = blockIdx.x;
    const int lane = threadIdx.x;
    double run = s2run[t];
    for (int g = 0; g < ng; ++g) {
        const double* src = part + ((int64_t)t * gcap + g) * rb;
        double v = 0.0;
        for (int i = lane; i < rb; i += 64) v += src[i];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
        run += v;
    }
    if (lane == 0) s2run[t] = run;
}

__global__ __launch_bounds__(256) void k_fill(double* p, int64_t count) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < count) p[i] = 0.0;
}

// loss[t] = S2/(n_bf N^2) - (1/N^2) sum_px (S1/n_bf)^2, fixed-order double reduction.
__global__ __launch_bounds__(1024) void k_loss(const double* __restrict__ s1run, const double* __restrict__ s2run,
                                               int64_t n2, double nbf, double* __restrict__ loss,
                                               float* __restrict__ mean_phase) {
    __shared__ double sh[1024];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    double acc = 0.0;
    for (int64_t p = tid; p < n2; p += 1024) {
        const double mval = s1run[t * n2 + p] / nbf;
        acc += mval * mval;
        if (t == 0 && mean_phase) mean_phase[p] = (float)mval;
    }
    sh[tid] = acc;
    __syncthreads();
    for (int s = 512; s > 0; s >>= 1) {
        if (tid < s) sh[tid] += sh[tid + s];
        __syncthreads();
    }
    if (tid == 0) loss[t] = s2run[t] / (nbf * (double)n2) - sh[0] / (double)n2;
}

// Row transform of the cached spectra: counts rows y0, y1 packed as one complex
// forward FFT, split by Hermitian symmetry.  Also the exact integer scan sum of
// every BF pixel.
template <int N>
__global__ __launch_bounds__(256) void k_g_rows(const uint32_t* __restrict__ counts, int64_t b0,
                                                float2* __restrict__ gm, float2* __restrict__ gn,
                                                unsigned long long* __restrict__ bfsum) {
    constexpr int H = N / 2;
    using F = WaveFFT<N, -1>;
    constexpr int R = F::R, L = F::L;
    __shared__ float2 buf[4 * F::W][N];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int grp = (tid >> 6) * F::W + lane / L;
    const int j = lane % L;
    const int64_t b = b0 + blockIdx.y;
    const int y0 = 2 * (blockIdx.x * (4 * F::W) + grp);

    const uint32_t* c0 = counts + (b * N + y0) * N;
    const uint32_t* c1 = c0 + N;
    float2 x[R];
    unsigned long long sum = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t i0 = c0[j + r * L], i1 = c1[j + r * L];
        sum += (unsigned long long)i0 + (unsigned long long)i1;
        x[r] = make_float2((float)i0, (float)i1);
    }
    F fft;
    fft.init(j);
    fft.run(x, buf[grp], j);
    wave_lds_fence();
#pragma unroll
    for (int r = 0; r < R; ++r) buf[grp][j + r * L] = x[r];
    wave_lds_fence();
    float2* g0 = gm + (b * N + y0) * H;
    float2* g1 = g0 + H;
#pragma unroll
    for (int r = 0; r < R / 2; ++r) {
        const int v = j + r * L;
        const float2 z = x[r];
        const float2 zm = buf[grp][(N - v) & (N - 1)];
        // X0 = (Z(v) + conj Z(N-v))/2, X1 = (Z(v) - conj Z(N-v))/(2i)
        g0[v] = make_float2(0.5f * (z.x + zm.x), 0.5f * (z.y - zm.y));
        g1[v] = make_float2(0.5f * (z.y + zm.y), -0.5f * (z.x - zm.x));
    }
    if (j == 0) {
        const float2 z = x[R / 2];            // v = N/2
        gn[b * N + y0] = make_float2(z.x, 0.f);
        gn[b * N + y0 + 1] = make_float2(z.y, 0.f);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    if (lane == 0) atomicAdd(&bfsum[b], sum);
}

// Object: sum over all BF pixels of the corrected half-plane spectrum, one
// segment of BF pixels per grid row (double accumulation, BF order).
template <int N>
__global__ __launch_bounds__(256) void k_obj_sum(const float2* __restrict__ gm, const float2* __restrict__ gn,
                                                 const double2* __restrict__ kb,
                                                 const uint8_t* __restrict__ active, TrialConst m,
                                                 GeomDev geo, int64_t nbf, int seglen,
                                                 double2* __restrict__ part) {
    constexpr int H = N / 2;
    constexpr int NE = N * (H + 1);
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= NE) return;
    const int u = e / (H + 1), v = e % (H + 1);
    const int64_t b_lo = (int64_t)blockIdx.y * seglen;
    const int64_t b_hi = min(nbf, b_lo + seglen);
    double ax = 0.0, ay = 0.0;
    if (!(u == 0 && v == 0)) {
        for (int64_t b = b_lo; b < b_hi; ++b) {
            if (!active[b]) continue;
            const float2 gv = v < H ? gm[(b * N + u) * H + v] : gn[b * N + u];
            const double2 k = kb[b];
            const float2 c = correct_entry(gv, u, v, k.x, k.y, m, geo);
            ax += c.x;
            ay += c.y;
        }
    }
    part[(int64_t)blockIdx.y * NE + e] = make_double2(ax, ay);
}

template <int N>
__global__ __launch_bounds__(256) void k_obj_reduce(const double2* __restrict__ part, int nseg,
                                                    float2* __restrict__ pm, float2* __restrict__ pn) {
    constexpr int H = N / 2;
    constexpr int NE = N * (H + 1);
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= NE) return;
    double ax = 0.0, ay = 0.0;
    for (int s = 0; s < nseg; ++s) {
        const double2 p = part[(int64_t)s * NE + e];
        ax += p.x;
        ay += p.y;
    }
    const int u = e / (H + 1), v = e % (H + 1);
    const float2 val = make_float2((float)ax, (float)ay);
    if (v < H) pm[u * H + v] = val;
    else pn[u] = val;
}

template <int N>
__global__ __launch_bounds__(256) void k_obj_rows(const float2* __restrict__ pm, const float2* __restrict__ pn,
                                                  float dcs, float scale, float* __restrict__ phase,
                                                  float2* __restrict__ psi) {
    constexpr int H = N / 2;
    using F = WaveFFT<N, +1>;
    constexpr int R = F::R, L = F::L;
    __shared__ float2 buf[4 * F::W][N];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int grp = (tid >> 6) * F::W + lane / L;
    const int j = lane % L;
    const int y0 = 2 * (blockIdx.x * (4 * F::W) + grp);
    const float2* r0 = pm + y0 * H;
    const float2* r1 = r0 + H;
    const float2 h0 = pn[y0], h1 = pn[y0 + 1];
    const float2 z0 = r0[0], z1 = r1[0];
    float2 x[R];
    assemble_row_pair<N, R, L>(r0, r1, h0, h1, j, x);
    F fft;
    fft.init(j);
    fft.run(x, buf[grp], j);
    const float sgn = (j & 1) ? -1.f : 1.f;
    const float den0 = dcs + z0.x + sgn * h0.x;
    const float den1 = dcs + z1.x + sgn * h1.x;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int xx = j + r * L;
        phase[y0 * N + xx] = atan2f(x[r].x, den0);
        phase[(y0 + 1) * N + xx] = atan2f(x[r].y, den1);
        if (psi) {
            psi[y0 * N + xx] = make_float2(den0 * scale, x[r].x * scale);
            psi[(y0 + 1) * N + xx] = make_float2(den1 * scale, x[r].y * scale);
        }
    }
}

template <int N>
int row_blocks() {
    return (N / 2) / (4 * WaveFFT<N, 1>::W);
}

template <int N>
hipError_t g_rows_n(const uint32_t* counts, int64_t nbf, float2* gm, float2* gn, unsigned long long* bfsum,
                    hipStream_t st) {
    for (int64_t b0 = 0; b0 < nbf; b0 += 65535) {
        const int nb = (int)std::min<int64_t>(65535, nbf - b0);
        hipLaunchKernelGGL(k_g_rows<N>, dim3(row_blocks<N>(), nb), dim3(256), 0, st, counts, b0, gm, gn, bfsum);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int N, int MODE>
hipError_t cols_n(const float2* in_m, const float2* in_n, float2* out_m, float2* out_n, int64_t planes,
                  int trials, int64_t out_tstride_m, int64_t out_tstride_n, int64_t bf0, const double2* kb,
                  const uint8_t* active, const TrialConst* tc, GeomDev geo, hipStream_t st) {
    constexpr int H = N / 2;
    for (int64_t p0 = 0; p0 < planes; p0 += 65535) {
        const int np = (int)std::min<int64_t>(65535, planes - p0);
        hipLaunchKernelGGL((k_cols<N, MODE>), dim3(H / kTC + 1, np, trials), dim3(256), 0, st,
                           in_m + p0 * N * H, in_n + p0 * N, out_m + p0 * N * H, out_n + p0 * N,
                           out_tstride_m, out_tstride_n, bf0 + p0, kb, active, tc, geo);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

#define SSB_DISPATCH_N(n, CALL)            \
    switch (n) {                           \
        case 32: { constexpr int NN = 32; return CALL; }   \
        case 64: { constexpr int NN = 64; return CALL; }   \
        case 128: { constexpr int NN = 128; return CALL; } \
        case 256: { constexpr int NN = 256; return CALL; } \
        case 512: { constexpr int NN = 512; return CALL; } \
        default: return hipErrorInvalidValue;               \
    }

hipError_t launch_g_rows(int n, const uint32_t* counts, int64_t nbf, float2* gm, float2* gn,
                         unsigned long long* bfsum, hipStream_t st) {
    SSB_DISPATCH_N(n, (g_rows_n<NN>(counts, nbf, gm, gn, bfsum, st)))
}

hipError_t launch_g_cols(int n, float2* gm, float2* gn, int64_t nbf, hipStream_t st) {
    GeomDev geo{};
    SSB_DISPATCH_N(n, (cols_n<NN, COL_PLAIN_FWD>(gm, gn, gm, gn, nbf, 1, 0, 0, 0, nullptr, nullptr, nullptr,
                                                  geo, st)))
}

hipError_t launch_pass1(int n, const float2* gm, const float2* gn, const double2* kb, const uint8_t* active,
                        const TrialConst* tc, int n_trials, GeomDev geo, int64_t bf0, int cb, int cap,
                        float2* im, float2* in, hipStream_t st) {
    const int64_t nn = n;
    const int64_t ts_m = (int64_t)cap * nn * (nn / 2);
    const int64_t ts_n = (int64_t)cap * nn;
    SSB_DISPATCH_N(n, (cols_n<NN, COL_CORRECT_INV>(gm + bf0 * nn * (nn / 2), gn + bf0 * nn, im, in, cb, n_trials,
                                                    ts_m, ts_n, bf0, kb, active, tc, geo, st)))
}

int pass2_row_blocks(int n) {
    switch (n) {
        case 32: return row_blocks<32>();
        case 64: return row_blocks<64>();
        case 128: return row_blocks<128>();
        case 256: return row_blocks<256>();
        default: return row_blocks<512>();
    }
}

template <int N>
static hipError_t pass2_n(const float2* im, const float2* in, int cap, const uint8_t* active, int64_t bf0,
                          int cb, int n_trials, double dc, float* part_s1, double* part_s2, int gcap,
                          hipStream_t st) {
    const int ng = (cb + kGroupBF - 1) / kGroupBF;
    hipLaunchKernelGGL(k_pass2<N>, dim3(row_blocks<N>(), ng, n_trials), dim3(256), 0, st, im, in, cap, active,
                       bf0, cb, (float)dc, part_s1, part_s2, gcap);
    return hipGetLastError();
}

hipError_t launch_pass2(int n, const float2* im, const float2* in, int cap, const uint8_t* active, int64_t bf0,
                        int cb, int n_trials, double dc, float* part_s1, double* part_s2, int gcap,
                        hipStream_t st) {
    SSB_DISPATCH_N(n, (pass2_n<NN>(im, in, cap, active, bf0, cb, n_trials, dc, part_s1, part_s2, gcap, st)))
}

hipError_t launch_accum(int n, const float* part_s1, const double* part_s2, int gcap, int ng, int n_trials,
                        double* s1run, double* s2run, hipStream_t st) {
    const int64_t n2 = (int64_t)n * n;
    hipLaunchKernelGGL(k_accum_s1, dim3((unsigned)((n2 + 255) / 256), n_trials), dim3(256), 0, st, part_s1, gcap,
                       ng, n2, s1run);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_accum_s2, dim3(n_trials), dim3(64), 0, st, part_s2, gcap, ng, pass2_row_blocks(n), s2run);
    return hipGetLastError();
}

hipError_t launch_fill(double* p, int64_t count, hipStream_t st) {
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st, p, count);
    return hipGetLastError();
}

hipError_t launch_loss(int n, const double* s1run, const double* s2run, int n_trials, double n_bf, double* loss,
                       float* mean_phase, hipStream_t st) {
    hipLaunchKernelGGL(k_loss, dim3(n_trials), dim3(1024), 0, st, s1run, s2run, (int64_t)n * n, n_bf, loss,
                       mean_phase);
    return hipGetLastError();
}

int obj_segments(int64_t nbf) {
    // enough segments to fill the chip, at least 16 BF per segment
    int64_t seg = (nbf + 15) / 16;
    return (int)std::max<int64_t>(1, std::min<int64_t>(64, seg));
}

template <int N>
static hipError_t obj_sum_n(const float2* gm, const float2* gn, const double2* kb, const uint8_t* active,
                            TrialConst tc, GeomDev geo, int64_t nbf, double2* part, int nseg,
                            hipStream_t st) {
    constexpr int NE = N * (N / 2 + 1);
    const int seglen = (int)((nbf + nseg - 1) / nseg);
    hipLaunchKernelGGL(k_obj_sum<N>, dim3((NE + 255) / 256, nseg), dim3(256), 0, st, gm, gn, kb, active, tc, geo,
                       nbf, seglen, part);
    return hipGetLastError();
}

hipError_t launch_obj_sum(int n, const float2* gm, const float2* gn, const double2* kb, const uint8_t* active,
                          TrialConst tc, GeomDev geo, int64_t nbf, double2* part, int nseg,
                          hipStream_t st) {
    SSB_DISPATCH_N(n, (obj_sum_n<NN>(gm, gn, kb, active, tc, geo, nbf, part, nseg, st)))
}

template <int N>
static hipError_t obj_reduce_n(const double2* part, int nseg, float2* pm, float2* pn, hipStream_t st) {
    constexpr int NE = N * (N / 2 + 1);
    hipLaunchKernelGGL(k_obj_reduce<N>, dim3((NE + 255) / 256), dim3(256), 0, st, part, nseg, pm, pn);
    return hipGetLastError();
}

hipError_t launch_obj_reduce(int n, const double2* part, int nseg, float2* pm, float2* pn, hipStream_t st) {
    SSB_DISPATCH_N(n, (obj_reduce_n<NN>(part, nseg, pm, pn, st)))
}

hipError_t launch_obj_cols(int n, float2* pm, float2* pn, hipStream_t st) {
    GeomDev geo{};
    SSB_DISPATCH_N(n, (cols_n<NN, COL_PLAIN_INV>(pm, pn, pm, pn, 1, 1, 0, 0, 0, nullptr, nullptr, nullptr, geo,
                                                  st)))
}

template <int N>
static hipError_t obj_rows_n(const float2* pm, const float2* pn, double dcsum, double scale, float* phase,
                             float2* psi, hipStream_t st) {
    hipLaunchKernelGGL(k_obj_rows<N>, dim3(row_blocks<N>()), dim3(256), 0, st, pm, pn, (float)dcsum, (float)scale,
                       phase, psi);
    return hipGetLastError();
}

hipError_t launch_obj_rows(int n, const float2* pm, const float2* pn, double dcsum, double scale, float* phase,
                           float2* psi, hipStream_t st) {
    SSB_DISPATCH_N(n, (obj_rows_n<NN>(pm, pn, dcsum, scale, phase, psi, st)))
}

}  // namespace ssb
