// HIP kernels of the SSB phase-variance path for gfx950.
//
// Layouts (complex64 = float2):
//   G cache        main [n_bf][N/2/8][N][8]   (v = 0 .. N/2-1 in tiles of 8 columns),
//                  nyq [n_bf][N]              (v = N/2)
//   intermediate   main [trial][cap][N/2/8][N][8],  nyq [trial][cap][N]
//   S1 partials    float [trial][gcap][N][N] (one image per 32-BF group)
// The tile-major main planes make one 8-column tile of one BF pixel a contiguous
// 32 KiB block at N = 512 (the unit pass 1 reads and writes), and two consecutive
// rows of a tile share one 128-byte line (the unit pass 2 reads).
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
#include <mutex>

// Scratch of the no-allocation loss entry point (for callers that cannot allocate):
// every chunk buffer of one call lives here.  Each device holds its own copy from
// the library's load until the process ends.  Host code must use the address
// hipGetSymbolAddress returns on that device, never this name.
static __device__ __align__(256) char scratch[(size_t)256 << 20];

namespace ssb {

size_t scratch_bytes() { return sizeof(scratch); }

hipError_t scratch_address(void** out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

namespace {

// Compile-time tuning constants.
#ifndef SSB_PASS1_THREADS
#define SSB_PASS1_THREADS 256 // pass-1 workgroup size
#endif
#ifndef SSB_PASS1_MIN_WAVES
#define SSB_PASS1_MIN_WAVES 5 // pass-1 register budget at N = 512: resident waves per SIMD
#endif
#ifndef SSB_P1_SWZ
#define SSB_P1_SWZ 1 // pass-1 LDS tile: row u of column c at u ^ ((c mod 8) << SSB_P1_SWZ)
#endif
#ifndef SSB_PASS1_MIN_WAVES_BATCH
#define SSB_PASS1_MIN_WAVES_BATCH 3 // the same with several trials per workgroup (168 VGPRs; at 4 it spills)
#endif
#ifndef SSB_PASS1_TB
#define SSB_PASS1_TB 8 // trials per pass-1 workgroup in batches
#endif
#ifndef SSB_PASS2_MIN_WAVES_1024
#define SSB_PASS2_MIN_WAVES_1024 4 // the same at N = 1024 (LDS also allows 4 workgroups per CU)
#endif
#ifndef SSB_PASS2_OBJ_FP_WAVES
#define SSB_PASS2_OBJ_FP_WAVES 4 // full-plane row pass with the object sums: resident waves per SIMD
#endif
#ifndef SSB_PASS2_MIN_WAVES
#define SSB_PASS2_MIN_WAVES 7 // pass-2 register budget (N <= 512, half plane): resident waves per SIMD
#endif

// columns per column-pass tile (LDS: kTC x (N + 1) complex values)
template <int N> constexpr int cols_tc() { return N >= 1024 ? 8 : 16; }
constexpr int kPad = 1;       // LDS row padding (complex values)

enum ColMode { COL_PLAIN_FWD = 1, COL_PLAIN_INV = 2 };

// exp(-2 pi i x) for x in revolutions, reduced in double first.
__device__ __forceinline__ float2 phasor_rev_neg(double x) {
    const float2 cs = cossin_rev((float)(x - rint(x)));
    return make_float2(cs.x, -cs.y);
}

// Phase-ramp chains of a wave that holds 8 consecutive rows x 8 consecutive columns of
// a tile (row r0 + lane / 8, column v0 + lane % 8): the start exp(-i (u beta + v alpha))
// of the chain over rows u below N/2 (ea), of the chain over rows u - N (eb) and the step
// exp(-i rs beta) (st).  The starts factor into a row phasor and a column phasor, so
// each lane computes one phasor (of one of the 8 rows, one of the 8 columns, the step,
// or exp(i (N/2) beta)) and gathers the factors it needs from the other lanes, instead
// of three phasors per lane.  (beta, alpha in revolutions.)
__device__ __forceinline__ void wave_chain_starts(int lane, int r0, int v0, int rs, int h, double alpha,
                                                  double beta, float2& ea, float2& eb, float2& st) {
    const int idx = lane < 8 ? r0 + lane : lane < 16 ? v0 + lane - 8 : lane == 16 ? rs : -h;
    const float2 ph = phasor_rev_neg((double)idx * (lane >= 8 && lane < 16 ? alpha : beta));
    auto from = [&](int src) { return make_float2(__shfl(ph.x, src), __shfl(ph.y, src)); };
    auto uni = [&](int src) {
        return make_float2(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(ph.x), src)),
                           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ph.y), src)));
    };
    ea = cmul(from(lane >> 3), from(8 + (lane & 7)));
    st = uni(16);
    eb = cmul(ea, uni(17));
}

// The same for a wave that holds 16 consecutive rows x 4 column pairs (row r0 + lane / 4,
// columns v0 + 2 (lane % 4) and the next): also e1 = exp(-i alpha), the step from a
// pair's first column to its second.
__device__ __forceinline__ void wave_chain_starts_pair(int lane, int r0, int v0, int rs, int h, double alpha,
                                                       double beta, float2& ea, float2& eb, float2& st,
                                                       float2& e1) {
    const bool col = lane >= 16 && lane < 20;
    const int idx = lane < 16 ? r0 + lane : col ? v0 + 2 * (lane - 16) : lane == 20 ? rs : lane == 21 ? -h : 1;
    const float2 ph = phasor_rev_neg((double)idx * (col || lane >= 22 ? alpha : beta));
    auto from = [&](int src) { return make_float2(__shfl(ph.x, src), __shfl(ph.y, src)); };
    auto uni = [&](int src) {
        return make_float2(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(ph.x), src)),
                           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ph.y), src)));
    };
    ea = cmul(from(lane >> 2), from(16 + (lane & 3)));
    st = uni(20);
    eb = cmul(ea, uni(21));
    e1 = uni(22);
}

// Squared distance |k + sg q(u', v)|^2 (pixels^2) of one shifted aperture center,
// sg = -1 for A(k - q) and +1 for A(k + q), in double.  Every support and flat-top
// decision of the correction is taken on this value.
__device__ __forceinline__ double shifted_r2(double kx, double ky, double sg, int up, int v, const GeomDev& g) {
    const double qx = fma(g.qux, (double)up, g.qvx * v);
    const double qy = fma(g.quy, (double)up, g.qvy * v);
    const double dx = kx + sg * qx, dy = ky + sg * qy;
    return fma(dx, dx, dy * dy);
}

// Soft aperture weight on the edge ring (lo2 < r2 < hi2): clip((R_a - r)/w + 1/2)
// with R_a - r = (R_a^2 - r^2)/(R_a + r), the difference taken in double.
__device__ __forceinline__ float edge_weight(double r2, const GeomDev& g) {
    const float num = (float)(g.ra2 - r2);
    const float den = (float)g.ra + __builtin_amdgcn_sqrtf((float)r2);
    const float a = fmaf(num * __builtin_amdgcn_rcpf(den), (float)g.inv_w, 0.5f);
    return fminf(fmaxf(a, 0.f), 1.f);
}

// Signed rows u' in [-H, H) of column v where r2(u') = |k + sg q(u', v)|^2 is below
// R2 (strict) or at most R2, as [lo, lo + len).  The set is a disk cut by a line, so
// it is one interval; its ends come from the roots of the quadratic in u' and are
// then settled with the exact test on shifted_r2 itself.
template <bool STRICT>
__device__ void row_interval(double kx, double ky, double sg, int v, int H, double R2, const GeomDev& g, int& lo,
                             int& len) {
    auto inside = [&](int up) {
        const double r = shifted_r2(kx, ky, sg, up, v, g);
        return STRICT ? r < R2 : r <= R2;
    };
    // r2(u') = |P + u' D|^2 with P = k + sg v qv, D = sg qu
    const double px = kx + sg * (g.qvx * v), py = ky + sg * (g.qvy * v);
    const double dx = sg * g.qux, dy = sg * g.quy;
    const double dd = dx * dx + dy * dy, pd = px * dx + py * dy, pp = px * px + py * py;
    const double disc = pd * pd - dd * (pp - R2);
    const double c = -pd / dd;
    double ra_ = c, rb_ = c;
    if (disc > 0.0) {
        const double hw = sqrt(disc) / dd;
        ra_ = c - hw;
        rb_ = c + hw;
    }
    int a = (int)fmax(fmin(ceil(ra_), (double)H), (double)(-H - 1));
    int b = (int)fmax(fmin(floor(rb_), (double)H), (double)(-H - 1));
    a = max(a, -H);
    b = min(b, H - 1);
    if (a > b) {
        // no integer strictly between the roots: only a rounding tie can hold one
        const int cand = (int)fmax(fmin(rint(c), (double)(H - 1)), (double)(-H));
        if (!inside(cand)) {
            lo = 0;
            len = 0;
            return;
        }
        a = b = cand;
    }
    for (int it = 0; it < 4 && a > -H && inside(a - 1); ++it) --a;
    for (int it = 0; it < 4 && a <= b && !inside(a); ++it) ++a;
    for (int it = 0; it < 4 && b < H - 1 && inside(b + 1); ++it) ++b;
    for (int it = 0; it < 4 && b >= a && !inside(b); --b, ++it) {}
    lo = a;
    len = b >= a ? b - a + 1 : 0;
}

__device__ __forceinline__ unsigned pack_lo_len(int lo, int len) {
    return ((unsigned)lo & 0xffffu) | ((unsigned)len << 16);
}
__device__ __forceinline__ int unpack_lo(unsigned p) { return (int)(short)(p & 0xffffu); }
__device__ __forceinline__ int unpack_len(unsigned p) { return (int)(p >> 16); }

// 64-bit load through a buffer resource: an offset at or past the resource's size
// returns zero without touching memory (predicated loads with no branch).
typedef int ssb_v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ float2 load_or_zero(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
// 16 bytes (two complex values) or zeros, like load_or_zero.
__device__ __forceinline__ float4 load4_or_zero(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// The same with the non-temporal cache policy (aux bit 1): for data read once per
// evaluation (the spectra in pass 1: 3.29 -> 3.22 ms).  Not for the row pass's
// loads: rows y0 and y0 + 1 of a tile share lines that other waves read too
// (non-temporal there: pass 2 2.02 -> 2.54 ms).
__device__ __forceinline__ float2 load_or_zero_nt(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 2));
}
// Non-temporal store of one complex value (pass 1's column results, read back only
// by the next kernel: 3.29 -> 3.14 ms).
__device__ __forceinline__ void store_nt(float2* p, float2 v) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    f32x2 w;
    w.x = v.x;
    w.y = v.y;
    __builtin_nontemporal_store(w, reinterpret_cast<f32x2*>(p));
}
// Two adjacent complex values as one 16-byte store (p 16-byte aligned), non-temporal or not.
__device__ __forceinline__ void store2_nt(float2* p, float2 a, float2 b) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    f32x4 w;
    w.x = a.x;
    w.y = a.y;
    w.z = b.x;
    w.w = b.y;
    __builtin_nontemporal_store(w, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ void store2(float2* p, float2 a, float2 b) {
    *reinterpret_cast<float4*>(p) = make_float4(a.x, a.y, b.x, b.y);
}
constexpr int kNoLoad = (int)0x80000000;

// (cos, sin) of 2 pi q^T M q
__device__ __forceinline__ float2 chi_phasor(double qx, double qy, const TrialConst& m) {
    const double cq = qx * (m.mxx * qx + m.mxy * qy) + qy * (m.mxy * qx + m.myy * qy);
    const float2 ph = phasor_rev_neg(cq);
    return make_float2(ph.x, -ph.y);
}

// atan_unit and atan2_f: ssb_math.hpp

// Plain column pass (spectrum builder, object): one workgroup = one plane x one
// tile of kTC columns (or the Nyquist column).  Coalesced tile load into LDS, one
// wave-level FFT per column, coalesced store.  in == out is allowed (the whole tile
// is read before any store).
template <int N, int MODE>
__global__ __launch_bounds__(256) void k_cols(const float2* in_m, const float2* in_n, float2* out_m,
                                              float2* out_n, const float2* __restrict__ twt) {
    constexpr int H = N / 2;
    constexpr int SIGN = (MODE == COL_PLAIN_FWD) ? -1 : 1;
    using F = WaveFFT<N, SIGN>;
    constexpr int LD = F::SCRATCH + kPad;   // a column's slot is also its transform's scratch
    constexpr int kTC = cols_tc<N>();
    __shared__ float2 tile[kTC * LD];

    const int tid = threadIdx.x;
    const int plane = blockIdx.y;
    const bool nyq = blockIdx.x == H / kTC;
    const int v0 = blockIdx.x * kTC;
    const float2* pin_m = in_m + (int64_t)plane * N * H;
    const float2* pin_n = in_n + (int64_t)plane * N;
    float2* pout_m = out_m + (int64_t)plane * N * H;
    float2* pout_n = out_n + (int64_t)plane * N;

    if (!nyq) {
        // all of the thread's loads in flight before the LDS stores
        constexpr int ROWS = 256 / kTC, IT = N / ROWS;
        const int c = tid % kTC, u0 = tid / kTC;
        float2 v[IT];
#pragma unroll
        for (int k = 0; k < IT; ++k) v[k] = pin_m[tm_index(N, u0 + k * ROWS, v0 + c)];
#pragma unroll
        for (int k = 0; k < IT; ++k) tile[c * LD + u0 + k * ROWS] = v[k];
    } else {
        for (int u = tid; u < N; u += 256) tile[u] = pin_n[u];
    }
    __syncthreads();

    const int lane = tid & 63;
    const int grp = (tid >> 6) * F::W + lane / F::L;
    const int j = lane % F::L;
    constexpr int NG = 4 * F::W;
    F fft;
    fft.load(twt, j);
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
        for (int y = tid / kTC; y < N; y += 256 / kTC) pout_m[tm_index(N, y, v0 + c)] = tile[c * LD + y];
    } else {
        for (int y = tid; y < N; y += 256) pout_n[y] = tile[y];
    }
}

// exp(i chi_q) = (cos, sin)(2 pi q^T M q) of every half-plane entry, per trial
// (BF independent): main [t] x tile-major [N/2/8][N][8], nyq [t][N].
// Pass 1 at N = 512 copies each tile's block of the chi_q table straight into its LDS
// tile, so the table is stored per layout tile as that tile's LDS image: column c of
// the tile at c * N, row u at u ^ ((c & 7) << SSB_P1_SWZ) (the tile's XOR swizzle).  Other sizes
// keep the tile-major [tile][u][8] layout of the spectra.
template <int N> constexpr bool chi_in_lds() { return N == 512; }
template <int N> __host__ __device__ __forceinline__ int64_t chi_index(int u, int v) {
    if constexpr (chi_in_lds<N>()) {
        const int c = v % kTileW;
        return (int64_t)(v / kTileW) * N * kTileW + c * N + (u ^ ((c & 7) << SSB_P1_SWZ));
    } else {
        return tm_index(N, u, v);
    }
}

template <int N>
__global__ __launch_bounds__(256) void k_chiq(const TrialConst* __restrict__ tc, GeomDev geo,
                                              float2* __restrict__ chm, float2* __restrict__ chn) {
    constexpr int H = N / 2;
    constexpr int NE = N * (H + 1);
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= NE) return;
    const int t = blockIdx.y;
    const int u = e / (H + 1), v = e % (H + 1);
    const double up = (double)(u < H ? u : u - N);
    const float2 val = chi_phasor(fma(geo.qux, up, geo.qvx * v), fma(geo.quy, up, geo.qvy * v), tc[t]);
    if (v < H) chm[(int64_t)t * N * H + chi_index<N>(u, v)] = val;
    else chn[(int64_t)t * N + u] = val;
}

// Correction support of every (BF, column) pair, from the geometry alone: for each
// shifted aperture the rows with nonzero weight (r2 < hi2) and the rows with weight
// exactly 1 (r2 <= lo2), packed as four (lo, len) pairs:
//   x = minus nonzero, y = plus nonzero, z = minus flat, w = plus flat.
template <int N>
__global__ __launch_bounds__(256) void k_support(const double2* __restrict__ kb, GeomDev geo, int64_t nbf,
                                                 uint4* __restrict__ sup) {
    constexpr int H = N / 2;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= nbf * (H + 1)) return;
    const int64_t b = e / (H + 1);
    const int v = (int)(e % (H + 1));
    const double2 k = kb[b];
    int lo, len;
    uint4 o;
    row_interval<true>(k.x, k.y, -1.0, v, H, geo.hi2, geo, lo, len);
    o.x = pack_lo_len(lo, len);
    row_interval<true>(k.x, k.y, 1.0, v, H, geo.hi2, geo, lo, len);
    o.y = pack_lo_len(lo, len);
    if (geo.lo2 >= 0.0) {
        row_interval<false>(k.x, k.y, -1.0, v, H, geo.lo2, geo, lo, len);
        o.z = pack_lo_len(lo, len);
        row_interval<false>(k.x, k.y, 1.0, v, H, geo.lo2, geo, lo, len);
        o.w = pack_lo_len(lo, len);
    } else {
        o.z = 0;
        o.w = 0;
    }
    sup[e] = o;
}

// vend[b] = 1 + the last column with any support (columns from vend on are all
// zero after the correction); at least 1 for an active BF pixel, 0 for an inactive
// one.  nsup[b] = number of half-plane entries with nonzero transfer (q = 0 aside).
template <int N>
__global__ __launch_bounds__(256) void k_vend(const uint4* __restrict__ sup, const uint8_t* __restrict__ active,
                                              int64_t nbf, int* __restrict__ vend, int* __restrict__ nsup) {
    constexpr int H = N / 2;
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nbf) return;
    int ve = 0, ns = 0;
    if (active[b]) {
        ve = 1;
        for (int v = 0; v <= H; ++v) {
            const uint4 o = sup[b * (H + 1) + v];
            const int lm = unpack_lo(o.x), nm = unpack_len(o.x), lp = unpack_lo(o.y), np = unpack_len(o.y);
            const int ov = max(0, min(lm + nm, lp + np) - max(lm, lp));
            const int cnt = nm + np - ov;
            if (cnt > 0) ve = v + 1;
            ns += cnt;
            // the q = 0 entry carries the DC, not a corrected value
            if (v == 0 && ((unsigned)(0 - lm) < (unsigned)nm || (unsigned)(0 - lp) < (unsigned)np)) ns -= 1;
        }
    }
    vend[b] = ve;
    nsup[b] = ns;
}

// Twiddle table of the wave-level FFT (WaveFFTT layout), filled once per handle.
template <int N, int SIGN>
__global__ __launch_bounds__(256) void k_twiddles(float2* __restrict__ tab) {
    WaveFFTT<N, SIGN>::fill(tab, threadIdx.x, 256);
}

// Per-BF phase slopes of delta = v alpha + u' beta (revolutions).
__device__ __forceinline__ void delta_slopes(double kx, double ky, const TrialConst& m, const GeomDev& g,
                                             double& alpha, double& beta) {
    const double px = m.mxx * kx + m.mxy * ky;
    const double py = m.mxy * kx + m.myy * ky;
    alpha = 2.0 * (px * g.qvx + py * g.qvy);
    beta = 2.0 * (px * g.qux + py * g.quy);
}

// Corrected value C = G T of one half-plane entry, T = conj(Gamma)/|Gamma|.  With chi
// quadratic, chi(k) - chi(k -+ q) = +-delta - chi_q where delta = 2 pi * 2 k^T M q
// (bilinear) and chi_q = 2 pi q^T M q, so
//   Gamma = a(k) e^{i delta} [(a_- - a_+) cos chi_q - i (a_- + a_+) sin chi_q],
// the definition's two shifted probe factors regrouped so that |Gamma| never comes
// from cancellation, and a(k) > 0 drops out of T.
// Inputs: the support flags (inm: A(k - q) has
// nonzero weight, inp: A(k + q) does; edge(edm, edp): that weight is on the edge ring, not
// the flat top), the spectrum value g, exp(i chi_q) = ch and e = exp(-i delta).
// With one sideband the bracket is a positive multiple of (+-cos chi_q, sin chi_q), so
// its weight cancels in T whether or not it lies on an edge ring.  With two on the flat
// tops it is (0, sign sin chi_q) (zero when sin chi_q is zero).  Only an entry inside
// both shifted apertures with at least one weight on its edge ring evaluates the
// weights and normalizes the bracket, so the edge flags (edge(edm, edp): the weight of
// A(k - q), A(k + q) is on its edge ring) are asked for only there.
template <class Edge>
__device__ __forceinline__ float2 correct_entry(float2 g, float2 ch, float2 e, bool inm, bool inp, Edge edge,
                                                int up, int v, double kx, double ky, const GeomDev& geo) {
    float br, bi;
    if (inm && inp) {
        bool edm, edp;
        edge(edm, edp);
        if (edm || edp) {
            // keep the rarely needed double-precision distances inside this branch (an
            // empty asm makes the row index opaque, so nothing here is hoisted out of a
            // caller's loop where it would hold registers)
            int upo = up;
            asm volatile("" : "+v"(upo));
            float am = 1.f, apl = 1.f;
            if (edm) am = edge_weight(shifted_r2(kx, ky, -1.0, upo, v, geo), geo);
            if (edp) apl = edge_weight(shifted_r2(kx, ky, 1.0, upo, v, geo), geo);
            br = (am - apl) * ch.x;
            bi = (am + apl) * ch.y;
            const float mag2 = fmaf(br, br, bi * bi);
            const float inv = mag2 > 0.f ? __builtin_amdgcn_rsqf(mag2) : 0.f;
            br *= inv;
            bi *= inv;
        } else {
            br = 0.f;
            bi = ch.y > 0.f ? 1.f : (ch.y < 0.f ? -1.f : 0.f);
        }
    } else {
        br = inm ? ch.x : -ch.x;
        bi = ch.y;
    }
    return cmul(g, make_float2(e.x * br - e.y * bi, e.x * bi + e.y * br));
}

// Corrected value of the entry at signed row up and signed column v, any lattice
// point (including the column -N/2 and the row +N/2, which the half-plane tables do
// not hold): support and flat-top flags from the shifted distances themselves (the
// rule the support tables encode), exp(i chi_q) in double, E_u(up) E_v(v).  The same
// bits as the table path for an entry both can form.
__device__ float2 correct_direct(float2 g, int up, int v, double kx, double ky, const TrialConst& m,
                                 const GeomDev& geo, double alpha, double beta) {
    const double rm = shifted_r2(kx, ky, -1.0, up, v, geo);
    const double rp = shifted_r2(kx, ky, 1.0, up, v, geo);
    const bool inm = rm < geo.hi2, inp = rp < geo.hi2;
    if (!inm && !inp) return make_float2(0.f, 0.f);
    auto edge = [&](bool& edm, bool& edp) {
        edm = !(geo.lo2 >= 0.0 && rm <= geo.lo2);
        edp = !(geo.lo2 >= 0.0 && rp <= geo.lo2);
    };
    const float2 ch = chi_phasor(fma(geo.qux, (double)up, geo.qvx * v), fma(geo.quy, (double)up, geo.qvy * v), m);
    const float2 e = cmul(phasor_rev_neg((double)up * beta), phasor_rev_neg((double)v * alpha));
    return correct_entry(g, ch, e, inm, inp, edge, up, v, kx, ky, geo);
}

// Full-plane variant, the Nyquist lines of one BF pixel.  Correcting every entry of
// the N x N plane on its own differs from the half plane's anti-Hermitian extension
// only on the Nyquist column and row: off them, -q of a lattice q is again a lattice
// point, G(-q) = conj G(q) and T(-q) = -conj T(q).  The object therefore gains
//   (-1)^x A(y) + (-1)^y B(x)    (unnormalized, as the row pass's values),
// A = inverse transform over u of dC(u) = G(u, N/2) [T(u, -N/2) - T(u, +N/2)], and
// B = inverse transform over v of dR(v) = conj(G(N/2, v') [T(-N/2, v') - T(+N/2, v')])
// at v = N - v' for v' = 1 .. N/2 - 1 (zero elsewhere).  (u, v) are the signed
// row and column of q.
__device__ __forceinline__ float2 nyq_col_delta(float2 g, int up, double kx, double ky, const TrialConst& m,
                                                const GeomDev& geo, double alpha, double beta) {
    const int H = geo.h;
    const float2 a = correct_direct(g, up, -H, kx, ky, m, geo, alpha, beta);
    const float2 b = correct_direct(g, up, H, kx, ky, m, geo, alpha, beta);
    return make_float2(a.x - b.x, a.y - b.y);
}
__device__ __forceinline__ float2 nyq_row_delta(float2 g, int vp, double kx, double ky, const TrialConst& m,
                                                const GeomDev& geo, double alpha, double beta) {
    const int H = geo.h;
    const float2 a = correct_direct(g, -H, vp, kx, ky, m, geo, alpha, beta);
    const float2 b = correct_direct(g, H, vp, kx, ky, m, geo, alpha, beta);
    return make_float2(a.x - b.x, -(a.y - b.y));
}

// A and B of every BF pixel of a chunk and trial: one workgroup per (BF, trial);
// the deltas in LDS, then two wave-level inverse transforms.  Out: na, nb
// [t][cap][N] (natural order).
template <int N>
__global__ __launch_bounds__(256) void k_nyq_lines(const float2* __restrict__ gm, const float2* __restrict__ gn,
                                                   const double2* __restrict__ kb,
                                                   const uint8_t* __restrict__ active,
                                                   const TrialConst* __restrict__ tc, GeomDev geo, int64_t bf0,
                                                   int cap, float2* __restrict__ na, float2* __restrict__ nb,
                                                   const float2* __restrict__ twt) {
    constexpr int H = N / 2;
    using F = WaveFFT<N, +1>;
    __shared__ float2 lc[F::SCRATCH];
    __shared__ float2 lr[F::SCRATCH];
    const int bl = blockIdx.x, t = blockIdx.y;
    const int64_t b = bf0 + bl;
    if (!active[b]) return;                       // pass 2 skips inactive BF pixels
    const double2 k = kb[b];
    const TrialConst m = tc[t];
    double alpha, beta;
    delta_slopes(k.x, k.y, m, geo, alpha, beta);
    const int tid = threadIdx.x;
    for (int u = tid; u < N; u += 256)
        lc[u] = nyq_col_delta(gn[b * N + u], u < H ? u : u - N, k.x, k.y, m, geo, alpha, beta);
    for (int v = tid; v < N; v += 256) {
        float2 d = make_float2(0.f, 0.f);
        if (v > H) {
            const int vp = N - v;
            d = nyq_row_delta(gm[b * N * H + tm_index(N, H, vp)], vp, k.x, k.y, m, geo, alpha, beta);
        }
        lr[v] = d;
    }
    __syncthreads();
    const int lane = tid & 63;
    const int grp = (tid >> 6) * F::W + lane / F::L;
    const int j = lane % F::L;
    if (grp < 2) {
        float2* src = grp == 0 ? lc : lr;
        float2* dst = (grp == 0 ? na : nb) + ((int64_t)t * cap + bl) * N;
        F fft;
        fft.load(twt, j);
        float2 x[F::R];
#pragma unroll
        for (int r = 0; r < F::R; ++r) x[r] = src[j + r * F::L];
        fft.run(x, src, j);
#pragma unroll
        for (int r = 0; r < F::R; ++r) dst[j + r * F::L] = x[r];
    }
}

// Pass 1: correction + column inverse transforms.  One workgroup = one BF pixel x
// one tile of TC columns (or the Nyquist column) x one trial; the waves share the
// tile's column FFTs.  Tiles at or past the BF pixel's last supported column (vend) are
// all zero after the correction: they are neither computed nor written, and pass 2
// does not read them.
//   1. support from the per-column intervals (integer compares); the spectrum
//      entries with nonzero transfer and their exp(i chi_q) (per-trial table) are
//      loaded into registers through buffer resources, zero-transfer entries get
//      an out-of-range offset and read as exact zeros without a memory access;
//      the BF pixel's phase slopes are formed while those loads are in flight;
//   2. each entry is corrected into the LDS tile: on the flat tops of the
//      apertures the bracket is already a unit phasor, on an edge ring it is
//      normalized;
//   3. one wave-level inverse FFT per column;  4. coalesced store.
// exp(-i delta) = E(u', v) = exp(-2 pi i (u' beta + v alpha)): each thread keeps
// one column and walks its rows RS apart, so its phasors are two geometric chains
// (rows below N/2, and rows from N/2 on taken as u - N) advanced by exp(-2 pi i RS
// beta); the chain starts and the step are reduced in double.
// 1024-point columns take 512 threads: a thread's share of the tile (N TC / threads
// entries) stays at 16, the most the per-thread support word holds.
template <int N> constexpr int pass1_threads() { return N >= 1024 ? 512 : SSB_PASS1_THREADS; }

// One pass-1 tile; NYQ selects the Nyquist column at compile time so that every
// row index, LDS address and load offset of the unrolled entry loops is a
// compile-time step from the thread's first row.
// LDS tile: one slot per column, which is also its transform's scratch.  Where the
// transform's scratch is exactly N values the slots are packed (pitch N) and row u
// of column c sits at u ^ 2 (c mod 8): the XOR changes bits 1..3 only, so a column
// stays a permutation of its own slot and row steps of 32 leave it alone.  An 8-byte
// LDS access is served 16 lanes at a time over 32 four-byte banks (the bank-conflict
// counter shows it: the earlier u ^ 4 (c mod 8), conflict-free for 32 lanes at a time,
// logged about one conflict cycle per LDS instruction).  16 lanes holding 8 columns x
// 2 consecutive rows (the correction and the stores) then hit 16 distinct 8-byte
// slots modulo 16, and 16 consecutive rows of one column (the transform's reads) stay
// a permutation of an aligned group of 16: pass 1 2.64 -> 2.62 ms.  8 columns of 512
// values take exactly 32 KB.  Padded transforms (1,024 points) keep the pitch
// SCRATCH + 32/TC (no swizzle).  (Five workgroups per CU would fit this LDS but need at
// most 96 VGPRs: forced there, the kernel spills loaded values to scratch right after
// their loads, 4.2-4.4 ms against 3.0 ms at the compiler's 127 VGPRs, four workgroups.)
template <int N> constexpr bool pass1_swz() { return WaveFFT<N, +1>::SCRATCH == N; }
template <int N, int TC> constexpr int pass1_ld() { return pass1_swz<N>() ? N : WaveFFT<N, +1>::SCRATCH + 32 / TC; }
template <int N> __device__ __forceinline__ int pass1_row(int c, int u) {
    if constexpr (pass1_swz<N>()) return u ^ ((c & 7) << SSB_P1_SWZ);
    else return u;
}
// TB trials per workgroup (TB > 1 for batches): the tile's spectrum entries, support
// flags and BF offset are loaded once and stay in registers while each trial, in turn,
// brings its own chi_q block, phase chains, correction, transforms and stores (the
// pages' fused candidates: geometry, aperture weights and the spectrum fetch shared,
// each candidate with its own correction and transforms).  The arithmetic of each
// trial is the single-trial path's, so a trial's results do not depend on TB.
// chsrc / out: trial t0's block; the next trial's is ch_step / out_step values on.
template <int N, int TC, bool NYQ, bool STREAM, int TB>
__device__ __forceinline__ void pass1_tile(const float2* __restrict__ gsrc, const float2* __restrict__ chsrc,
                                           int64_t ch_step, const double2 k, const uint4 sr,
                                           const TrialConst* __restrict__ tcp, int nt, const GeomDev& geo,
                                           float2* __restrict__ out, int64_t out_step, float2* tile, int v0,
                                           int csub) {
    constexpr int H = N / 2;
    constexpr int LD = pass1_ld<N, TC>();
    constexpr int NT = pass1_threads<N>();
    constexpr int RS = NYQ ? NT : NT / TC;    // rows per sweep
    constexpr int PM = (N + RS - 1) / RS;     // entries per thread
    constexpr int SSTRIDE = NYQ ? 1 : kTileW; // row stride inside the source tile
    static_assert(NYQ || kTileW % TC == 0, "a pass-1 tile is part of one layout tile");
    using F = WaveFFT<N, +1>;

    const int tid = threadIdx.x;
    const int c = NYQ ? 0 : tid % TC;
    const int v = v0 + c;
    int ustart = NYQ ? tid : tid / TC;
    int lo_m = unpack_lo(sr.x), len_m = unpack_len(sr.x);
    int lo_p = unpack_lo(sr.y), len_p = unpack_len(sr.y);

    // 1. support and loads into registers (all loads in flight together)
    // gsrc / chsrc: the layout tile's block (main: [N][kTileW]; this workgroup's
    // columns start at csub) or the Nyquist column
    // CL: the tile's chi_q block is stored as the tile's LDS image (chi_index) and is
    // copied into the LDS tile asynchronously (16 bytes per lane, no registers held),
    // each entry reading its value back from its own slot at the correction.
    constexpr bool CL = chi_in_lds<N>() && !NYQ;
    static_assert(!CL || RS <= H, "the copied block is waited for in the two-chain path");
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(gsrc, N * (NYQ ? 1 : kTileW) * 8);
    auto copy_chi = [&](const float2* chs) {
        if constexpr (CL) {
            static_assert(TC == kTileW && LD == N, "the chi_q block is the tile's LDS image");
            const __amdgpu_buffer_rsrc_t rc = make_rsrc(chs, N * kTileW * 8);
            constexpr int WAVE_BYTES = N * kTileW * 8 / (NT / 64);
            const int lane = tid & 63;
            const int wb = (tid >> 6) * WAVE_BYTES;
#pragma unroll
            for (int q = 0; q < WAVE_BYTES / 1024; ++q)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (lds_ptr_t)((char*)tile + wb + q * 1024), 16,
                                                         wb + q * 1024 + lane * 16, 0, 0, 0);
            asm volatile("" ::: "memory");   // the copies stay ahead of every later load
        }
    };
    copy_chi(chsrc);
    const int off0 = (ustart * SSTRIDE + csub + c) * 8;
    float2 gv[PM], chv[CL ? 1 : PM];
    // entry i in the support of either shifted aperture (DC excluded): evaluated at
    // the loads and again at the correction, which is cheaper than packing the two
    // flags of each entry into a word and unpacking them (pass 1 2.92 -> 2.86 ms)
    auto flags = [&](int i, bool& inm, bool& inp) {
        const int u = ustart + i * RS;
        const int up = (NYQ || RS > H) ? (u < H ? u : u - N) : (i < PM / 2 ? u : u - N);
        inm = (unsigned)(up - lo_m) < (unsigned)len_m;
        inp = (unsigned)(up - lo_p) < (unsigned)len_p;
        return (NYQ ? u < N : true) && (inm || inp) && (u != 0 || v != 0);
    };
    auto load_chv = [&](const float2* chs) {
        if constexpr (!CL) {
            const __amdgpu_buffer_rsrc_t rc = make_rsrc(chs, N * (NYQ ? 1 : kTileW) * 8);
#pragma unroll
            for (int i = 0; i < PM; ++i) {
                bool inm, inp;
                chv[i] = load_or_zero(rc, flags(i, inm, inp) ? off0 + i * RS * SSTRIDE * 8 : kNoLoad);
            }
        }
    };
#pragma unroll
    for (int i = 0; i < PM; ++i) {
        bool inm, inp;
        const int off = flags(i, inm, inp) ? off0 + i * RS * SSTRIDE * 8 : kNoLoad;
        gv[i] = STREAM ? load_or_zero_nt(rg, off) : load_or_zero(rg, off);
    }
    load_chv(chsrc);

    int flo_m = unpack_lo(sr.z), flen_m = unpack_len(sr.z);
    int flo_p = unpack_lo(sr.w), flen_p = unpack_len(sr.w);
    static_assert(NYQ || RS % 32 == 0 || !pass1_swz<N>(), "row steps leave the swizzled bits alone");
    float2* trow = tile + c * LD + pass1_row<N>(c, ustart);
    const int lane = tid & 63;
    const int grp = (tid >> 6) * F::W + lane / F::L;
    const int j = lane % F::L;
    constexpr int NG = (NT / 64) * F::W;
    constexpr int NCOLS = NYQ ? 1 : TC;
    // row j + r L of column cc: with L a multiple of 32 the swizzle leaves r L alone
    auto slot = [&](int cc, int r) {
        if constexpr (F::L % 32 == 0) return cc * LD + pass1_row<N>(cc, j) + r * F::L;
        else return cc * LD + pass1_row<N>(cc, j + r * F::L);
    };

    const int ntr = TB == 1 ? 1 : nt;
    for (int tt = 0; tt < ntr; ++tt) {
        if constexpr (TB > 1) {
            // opaque per trial: what derives from the row start and the support intervals
            // is formed again in each trial instead of held in registers across the
            // transforms (which would spill)
            asm volatile("" : "+v"(ustart), "+v"(lo_m), "+v"(len_m), "+v"(lo_p), "+v"(len_p));
            asm volatile("" : "+v"(flo_m), "+v"(flen_m), "+v"(flo_p), "+v"(flen_p));
        }
        if (tt > 0) {
            // every thread's stores of the previous trial have read the tile before the
            // next chi_q block lands in it
            __syncthreads();
            copy_chi(chsrc + tt * ch_step);
            load_chv(chsrc + tt * ch_step);
        }
        const TrialConst m = tcp[tt];
        // the phase slopes of this BF pixel while the loads are in flight
        double alpha, beta;
        delta_slopes(k.x, k.y, m, geo, alpha, beta);
        const double av = (double)v * alpha;

        // 2. correction into the LDS tile
        auto entry = [&](int i, float2 e) {
            const int u = ustart + i * RS;
            // outside the support the predicated load left gv[i] zero, which is the stored value
            float2 val = gv[i];
            bool inm, inp;
            if (flags(i, inm, inp)) {
                const int up = (NYQ || RS > H) ? (u < H ? u : u - N) : (i < PM / 2 ? u : u - N);
                auto edge = [&](bool& edm, bool& edp) {
                    int uo = up;   // opaque: the tests stay in the branch that needs them
                    asm volatile("" : "+v"(uo));
                    edm = (unsigned)(uo - flo_m) >= (unsigned)flen_m;
                    edp = (unsigned)(uo - flo_p) >= (unsigned)flen_p;
                };
                float2 ch;
                if constexpr (CL) ch = trow[i * RS];
                else ch = chv[i];
                val = correct_entry(gv[i], ch, e, inm, inp, edge, up, v, k.x, k.y, geo);
            }
            trow[i * RS] = val;
        };
        if constexpr (!NYQ && RS <= H) {
            // PM/2 rows below N/2, then PM/2 rows from N/2 on; two chains
            static_assert(PM % 2 == 0 && (PM / 2) * RS == H, "rows split at N/2");
            float2 ea, eb, st;
            static_assert(TC == 8 && NT / TC == RS, "a wave is 8 rows x 8 columns of the tile");
            wave_chain_starts(lane, (tid >> 6) * 8, v0, RS, H, alpha, beta, ea, eb, st);
            if constexpr (CL) {
                // every wave's copies have landed before any thread reads a slot another
                // wave filled.  The compiler tracks the copies to the LDS as outstanding
                // vector memory operations: before this barrier it waits only until the
                // operations issued after them (the spectrum loads, any spill) are the
                // only ones left, so the spectrum loads stay in flight and each entry
                // waits for its own load (a CPU test checks this in the built assembly)
                __syncthreads();
            }
#pragma unroll
            for (int i = 0; i < PM / 2; ++i) {
                entry(i, ea);
                entry(i + PM / 2, eb);
                ea = cmul(ea, st);
                eb = cmul(eb, st);
            }
        } else {
#pragma unroll
            for (int i = 0; i < PM; ++i) {
                const int u = ustart + i * RS;
                if (NYQ ? u < N : true) entry(i, phasor_rev_neg(fma((double)(u < H ? u : u - N), beta, av)));
            }
        }
        __syncthreads();

        // 3. column transforms.  The twiddles are computed here rather than loaded
        // from the shared table: loaded at this point their latency is exposed, loaded
        // early they hold registers through the correction (both measured slower),
        // while this arithmetic fills issue slots of waves waiting on memory.  For
        // radix 8 only r = 1, 2, 4 take a sincospi; r = 3, 5, 6, 7 are their products.
        F fft;
        if constexpr (F::R == 8 || N == 1024) fft.init_products(j);   // sincospi for r = 1, 2, 4, the rest products
        else fft.init(j);
        for (int cc = grp; cc < NCOLS; cc += NG) {
            float2 x[F::R];
#pragma unroll
            for (int r = 0; r < F::R; ++r) x[r] = tile[slot(cc, r)];
            fft.run(x, &tile[cc * LD], j);
            wave_lds_fence();
#pragma unroll
            for (int r = 0; r < F::R; ++r) tile[slot(cc, r)] = x[r];
        }
        __syncthreads();

        // 4. store, in the row pass's form (out: the layout tile's block of the column-result
        // plane, or the Nyquist column).  The row pass transforms rows y0 = 2p and y0 + 1
        // together as Z(v) = B0(v) + i B1(v), B_k = -i C(y_k, v) (C: the column results),
        // extended Hermitian; both Z(v) = (C0.y + C1.x, C1.y - C0.x) and
        // Z(N - v) = (C0.y - C1.x, C0.x + C1.y) come from the same two values, so they are
        // formed here, where vector issue has room, and stored as one 16-byte unit
        // [Z(v), Z(N - v)] per row pair and column (the pair's two 64-byte rows hold its
        // 8 columns' units).  At v = 0 the unit is [(C0.y, C1.y), (C0.x, C1.x)]: the
        // transform takes only the imaginary parts there, and the real parts are the
        // object's real part along the two rows.  The Nyquist column's unit per row pair is
        // [(C0.y, C1.y), (C0.x, C1.x)] in the same way.  Bitwise the sums the row pass formed
        // itself; the row pass loses its assembly arithmetic, its cross-lane permutes and two
        // of its loads per BF pixel (pass 2 1.88-1.92 -> 1.73-1.77 ms with half the permutes
        // left, pass 1 2.40 -> 2.45 ms, 4.44-4.55 -> 4.33 ms per evaluation in one run).
        float2* ot = out + tt * out_step;
        if constexpr (!NYQ && TC == 8) {
            // unit q = (p, c) = (q / 8, q % 8): 16 bytes per lane, 8 lanes per 128-byte row
            // pair, at 2 q values into the tile's block; rows 2p and 2p + 1 of a column are
            // adjacent LDS slots (the swizzle leaves bit 0 alone, and steps of NT / 4 rows
            // leave it as it is).  The DC form only in the first tile (a uniform branch).
            constexpr int UNITS = (N / 2) * TC;
            constexpr int KU = (UNITS + NT - 1) / NT;
            static_assert(UNITS % NT == 0 || KU == 1, "whole sweeps, or one partial sweep");
            static_assert((NT / 4) % 16 == 0 || !pass1_swz<N>(), "row steps leave the swizzled bits alone");
            const int cc = tid & 7;
            const float2* src = tile + cc * LD + pass1_row<N>(cc, 2 * (tid >> 3));
            float2* dst = ot + csub + 2 * tid;
            auto sweep = [&](auto dcv) {
                constexpr bool DC = decltype(dcv)::value;
#pragma unroll
                for (int k = 0; k < KU; ++k) {
                    if (UNITS % NT != 0 && tid + k * NT >= UNITS) break;
                    const float2 c0 = src[k * (NT / 4)], c1 = src[k * (NT / 4) + 1];
                    float2 zs = make_float2(c0.y + c1.x, c1.y - c0.x);
                    float2 zm = make_float2(c0.y - c1.x, c0.x + c1.y);
                    if (DC && cc == 0) {
                        zs = make_float2(c0.y, c1.y);
                        zm = make_float2(c0.x, c1.x);
                    }
                    if constexpr (STREAM) store2_nt(dst + 2 * k * NT, zs, zm);
                    else store2(dst + 2 * k * NT, zs, zm);
                }
            };
            if (v0 == 0) sweep(std::true_type{});
            else sweep(std::false_type{});
        } else if (!NYQ) {
            static_assert(NYQ || TC == 8, "main tiles are whole layout tiles");
        } else {
            for (int pr = tid; pr < N / 2; pr += NT) {
                const float2 c0 = tile[2 * pr], c1 = tile[2 * pr + 1];
                const float2 zs = make_float2(c0.y, c1.y), zm = make_float2(c0.x, c1.x);
                if constexpr (STREAM) store2_nt(ot + 2 * pr, zs, zm);
                else store2(ot + 2 * pr, zs, zm);
            }
        }
    }
}

// STREAM: non-temporal spectrum loads and column-result stores, for launches whose
// spectrum tiles are not read again soon: one trial, or a chunk whose spectra
// exceed the 256 MB MALL.  With many trials the chunk is small (32 BF at 200 trials)
// and each trial row of the grid re-reads its tiles from the MALL; there the
// default policy is kept (200-trial batch: 5.30 against 5.55 ms per trial).
// Register budget: with the chi_q block copied to the LDS (N = 512) the kernel fits
// the budget of SSB_PASS1_MIN_WAVES waves per SIMD, which the 32 KB tile's LDS also
// allows (five 32 KB tiles fill the 160 KB of a CU).
// With TB > 1 trials per workgroup the spectrum entries stay in registers through the
// transforms: a 168-VGPR budget (three waves per SIMD; at four the compiler spills).
template <int N, int TB> constexpr int pass1_min_waves() {
    return chi_in_lds<N>() ? (TB > 1 ? SSB_PASS1_MIN_WAVES_BATCH : SSB_PASS1_MIN_WAVES) : 1;
}

template <int N, int TC, bool STREAM, int TB>
__global__ __launch_bounds__(pass1_threads<N>(), (pass1_min_waves<N, TB>())) void k_pass1(const float2* __restrict__ gm,
                                                         const float2* __restrict__ gn,
                                                         const float2* __restrict__ chm,
                                                         const float2* __restrict__ chn,
                                                         const double2* __restrict__ kb,
                                                         const uint4* __restrict__ sup,
                                                         const int* __restrict__ vend,
                                                         const TrialConst* __restrict__ tc, GeomDev geo,
                                                         int64_t bf0, int cap, float2* __restrict__ im,
                                                         float2* __restrict__ in, int n_trials) {
    constexpr int H = N / 2;
    constexpr int LD = pass1_ld<N, TC>();
    __shared__ float2 tile[TC * LD];

    // trials [t, t + nt) of this workgroup
    const int t = blockIdx.y * TB;
    const int nt = min(TB, n_trials - t);
    // Workgroup -> (BF, tile).  Up to N = 512 BF-major: the H/TC main tiles of a BF,
    // then its Nyquist tile (the per-trial chi_q table, 1 MB, stays in L2 anyway).
    // At N = 1024 tile-major: the workgroups running together share one column
    // tile, so that tile's slice of the 4.2 MB chi_q table stays in L2 instead of
    // being refetched for every BF pixel (pass 1 4.4 ms against 4.8 ms; BF-major
    // is the faster order at 512).  (Giving the two tiles that share 128-byte rows
    // ids 8 apart, so that they run on the same XCD, halves the fetched bytes at 512
    // but measured slower.)
    constexpr int NTM = H / TC;
    int bl, tix;
    if constexpr (N >= 1024) {
        const int cbk = (int)(gridDim.x / (NTM + 1));
        tix = (int)(blockIdx.x / cbk);
        bl = (int)(blockIdx.x % cbk);
    } else {
        bl = (int)(blockIdx.x / (NTM + 1));
        tix = (int)(blockIdx.x % (NTM + 1));
    }
    const int64_t b = bf0 + bl;
    const bool nyq = tix == NTM;
    const int v0 = nyq ? H : tix * TC;
    const int lt = v0 / kTileW;                   // the layout tile holding these columns
    // layout tiles wholly past the last supported column are all zero (every column
    // of an inactive BF); they are neither computed nor written, and pass 2 reads
    // them as zeros.  A layout tile with any supported column is written whole.
    if ((nyq ? H : lt * kTileW) >= vend[b]) return;
    const double2 k = kb[b];
    if (!nyq) {
        const int64_t tb = (int64_t)lt * N * kTileW;      // the layout tile's block in a plane
        const int v = v0 + (int)threadIdx.x % TC;
        pass1_tile<N, TC, false, STREAM, TB>(gm + b * N * H + tb, chm + (int64_t)t * N * H + tb, (int64_t)N * H, k,
                                             sup[b * (H + 1) + v], tc + t, nt, geo,
                                             im + ((int64_t)t * cap + bl) * N * H + tb, (int64_t)cap * N * H, tile,
                                             v0, v0 - lt * kTileW);
    } else {
        pass1_tile<N, TC, true, STREAM, TB>(gn + b * N, chn + (int64_t)t * N, (int64_t)N, k, sup[b * (H + 1) + H],
                                            tc + t, nt, geo, in + ((int64_t)t * cap + bl) * N, (int64_t)cap * N,
                                            tile, v0, 0);
    }
}

// Raw column-pass values a row pair needs: lane j gets v = j + r L for r < R/2
// (direct, loaded) and the mirrored w = N - v for r >= R/2 (permuted from other
// lanes' direct values), plus the v = 0 and v = N/2 entries of both rows.
// (The object's row transform reads its column results in this raw form; the row pass
// reads pass 1's row-pair form, RowPairUnits below.)
template <int N, int R, int L>
struct RowPairRaw {
    float2 d0[R / 2], d1[R / 2], m0[R / 2], m1[R / 2];
    float2 h0, h1, z0, z1;

    // plane: one BF pixel's column results (tile-major [N/2/8][N][8]); nyqc: its
    // Nyquist column [N].  Tiles past the last supported column (ve) were not written
    // by pass 1: the buffer resource ends at the last written tile, so their loads
    // return zero without a memory access (columns at or past ve inside that tile
    // hold pass 1's zeros).  Row y0 + 1 of a tile follows row y0 (the same 128-byte
    // line).  Column j + r L sits r (L/8) tiles after column j, so every load is a
    // per-lane base plus a constant.
    __device__ __forceinline__ void load(const float2* plane, const float2* nyqc, int y0, int j, int ve) {
        constexpr int H = N / 2;
        static_assert(L % kTileW == 0, "a lane group spans whole tiles");
        constexpr int TILE = N * kTileW * 8;             // bytes of one tile of a plane
        constexpr int RSTEP = (L / kTileW) * TILE;       // bytes from column v to column v + L
        const int ntile = min((ve + kTileW - 1) / kTileW, H / kTileW);
        const __amdgpu_buffer_rsrc_t rp = make_rsrc(plane, ntile * TILE);
        // base: column j.  The empty asm makes it opaque, so the R offsets derived
        // from it are formed at each call rather than hoisted out of the caller's loop.
        int od = (int)tm_index(N, y0, j) * 8;
        asm volatile("" : "+v"(od));
#pragma unroll
        for (int r = 0; r < R / 2; ++r) {
            d0[r] = load_or_zero(rp, od + r * RSTEP);
            d1[r] = load_or_zero(rp, od + r * RSTEP + kTileW * 8);
        }
        // the DC column (in the first tile: zero when ve = 0 leaves the resource empty)
        // and the Nyquist column (a resource of N values only when ve > H; pass 1 did not
        // write it otherwise), as predicated loads: no branch, no zeroing
        z0 = load_or_zero(rp, (int)tm_index(N, y0, 0) * 8);
        z1 = load_or_zero(rp, (int)tm_index(N, y0 + 1, 0) * 8);
        const __amdgpu_buffer_rsrc_t rn = make_rsrc(nyqc, ve > H ? N * 8 : 0);
        h0 = load_or_zero(rn, y0 * 8);
        h1 = load_or_zero(rn, (y0 + 1) * 8);
    }

    // Mirrored columns w = N/2 - j - r L from the direct values already loaded: for
    // j > 0, w = (L - j) + (R/2 - 1 - r) L is lane L - j's direct value R/2 - 1 - r
    // (one cross-lane permute per float, instead of a second load of the same lines:
    // row pass 2.02-2.07 -> 1.99 ms); for j = 0, w = (R/2 - r) L is the lane's own
    // (r >= 1; r = 0 is the Nyquist column, replaced in assemble).
    __device__ __forceinline__ void mirror(int j) {
        const int lane = (int)threadIdx.x & 63;
        const int addr = (lane - j + ((L - j) & (L - 1))) * 4;
#pragma unroll
        for (int r = 0; r < R / 2; ++r) {
            const int rs = R / 2 - 1 - r;
            m0[r].x = __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(d0[rs].x)));
            m0[r].y = __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(d0[rs].y)));
            m1[r].x = __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(d1[rs].x)));
            m1[r].y = __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(d1[rs].y)));
        }
        if (j == 0) {
#pragma unroll
            for (int r = 1; r < R / 2; ++r) {
                m0[r] = d0[R / 2 - r];
                m1[r] = d1[R / 2 - r];
            }
        }
    }

    // Z(v) = B0(v) + i B1(v), B_k = -i * (column result of row y_k), extended
    // Hermitian (B(N - v) = conj B(v)) with only real parts kept at v = 0 and N/2.
    __device__ __forceinline__ void assemble(int j, float2 (&x)[R]) {
        constexpr int H = N / 2;
        mirror(j);
#pragma unroll
        for (int r = 0; r < R / 2; ++r) {
            float2 a0 = d0[r], a1 = d1[r];
            if (j + r * L == 0) {
                a0.x = 0.f;
                a1.x = 0.f;
            }
            x[r] = make_float2(a0.y + a1.x, a1.y - a0.x);
        }
#pragma unroll
        for (int r = 0; r < R / 2; ++r) {
            if (j + (r + R / 2) * L == H) {
                x[r + R / 2] = make_float2(h0.y, h1.y);
            } else {
                x[r + R / 2] = make_float2(m0[r].y - m1[r].x, m0[r].x + m1[r].y);
            }
        }
    }
};

// The row pass's inputs in pass 1's row-pair form: per row pair and column v a 16-byte
// unit [Z(v), Z(N - v)] (Z as in RowPairRaw::assemble, formed by pass 1), at v = 0
// [Z(0), (Re C(y0, 0), Re C(y0 + 1, 0))], and per row pair of the Nyquist column
// [Z(N/2), (Re C(y0, N/2), Re C(y0 + 1, N/2))].  Lane j loads the Z(v) halves of its direct
// units (v = j + r L) and the Z(N - w) halves of the units at its mirrored columns
// w = N/2 - j - r L, which give x[r + R/2] = Z(v + N/2) directly; for j = 0 and r = 0 that
// is the Nyquist unit (the offset of column N/2 lies past the plane's resource and loads
// zero; the Nyquist unit's value is selected instead).  Bitwise the values RowPairRaw
// assembles.  (Taking the mirrored halves from lane L - j's own 16-byte loads with cross-lane
// permutes instead: pass 2 1.724-1.734 against 1.709-1.722 ms, in a 200-trial batch 1.774
// against 1.727 ms per trial.)
template <int N, int R, int L>
struct RowPairUnits {
    float2 s[R / 2], d[R / 2];
    float4 hn;        // the Nyquist unit
    float2 zr;        // real parts of the DC column on rows y0, y0 + 1

    __device__ __forceinline__ void load(const float2* plane, const float2* nyqc, int y0, int j, int ve) {
        constexpr int H = N / 2;
        static_assert(L % kTileW == 0, "a lane group spans whole tiles");
        constexpr int TILE = N * kTileW * 8;
        constexpr int RSTEP = (L / kTileW) * TILE;
        const int ntile = min((ve + kTileW - 1) / kTileW, H / kTileW);
        const __amdgpu_buffer_rsrc_t rp = make_rsrc(plane, ntile * TILE);
        int od = (int)tm_index(N, y0, j) * 8 + (j % kTileW) * 8;
        const int w0 = H - j;
        int om = (int)tm_index(N, y0, w0) * 8 + (w0 % kTileW) * 8 + 8;
        asm volatile("" : "+v"(od), "+v"(om));
#pragma unroll
        for (int r = 0; r < R / 2; ++r) {
            s[r] = load_or_zero(rp, od + r * RSTEP);
            d[r] = load_or_zero(rp, om - r * RSTEP);
        }
        zr = load_or_zero(rp, y0 * (kTileW * 8) + 8);
        const __amdgpu_buffer_rsrc_t rn = make_rsrc(nyqc, ve > H ? N * 8 : 0);
        hn = load4_or_zero(rn, y0 * 8);
    }

    __device__ __forceinline__ void assemble(int j, float2 (&x)[R]) {
#pragma unroll
        for (int r = 0; r < R / 2; ++r) {
            x[r] = s[r];
            x[r + R / 2] = (r == 0 && j == 0) ? make_float2(hn.x, hn.y) : d[r];
        }
    }
    __device__ __forceinline__ float dc_re0() const { return zr.x; }
    __device__ __forceinline__ float dc_re1() const { return zr.y; }
    __device__ __forceinline__ float ny_re0() const { return hn.z; }
    __device__ __forceinline__ float ny_re1() const { return hn.w; }
};

// Pass 2: one workgroup = 4*W row pairs x one 32-BF group x one trial.  Loops
// over the group's BF pixels in order, accumulating per-pixel phase sums in
// registers (float) and the squared phase (double per lane).  (Loading the next
// BF's column values during the current transform measured slower: the extra
// registers cost more than it hides.)
// FP: the full-plane variant; each BF pixel's object gains (-1)^x A(y) + (-1)^y B(x)
// from na, nb [t][cap][N] (k_nyq_lines), so the real part varies along a row: the
// wave test and the reciprocal of the atan2 fast path are per sample.
// Register budget: 72 VGPRs (7 waves per SIMD, which is also what the LDS allows: seven
// 22.5 KB workgroups per CU) fit the half-plane row pass up to N = 512 without spills
// (1.908 -> 1.880 ms against 78 VGPRs and 6 waves; earlier 2.07 against 2.19 ms for 6
// against 5 waves);
// 128 (4 waves) at N = 1024 (2.85 against 3.26 ms at 136, 3 waves); the
// full-plane form 96 up to N = 512 (5 waves, 44 bytes of spills; 2.31-2.32 -> 2.24 ms against the
// compiler's 124 VGPRs and 4 waves) and the compiler's choice at N = 1024.
// OBJ: the row pass also sums each pixel's object O_b over the group's BF pixels (the
// half plane's 18 sums per lane take the budget of five waves per SIMD, 94 VGPRs, or at
// 1,024 points of three, 161 VGPRs; the full plane's 32 that of SSB_PASS2_OBJ_FP_WAVES)
template <int N, bool FP, bool OBJ = false>
constexpr int pass2_min_waves() {
    return OBJ ? (FP ? SSB_PASS2_OBJ_FP_WAVES : (N <= 512 ? 5 : 3))
               : FP ? (N <= 512 ? 5 : 1) : (N <= 512 ? SSB_PASS2_MIN_WAVES : SSB_PASS2_MIN_WAVES_1024);
}

// part_obj (OBJ only): per trial and group, N * N sums of Im O_b over the group's active BF
// pixels (row-major, like part_s1), then for the half plane 2 N sums of Re O_b per row and
// column parity (there Re O_b depends on the column only through its parity: the DC term,
// the v = 0 column's real part along the row, and the Nyquist column's, with sign (-1)^x),
// for the full plane N * N sums of Re O_b per pixel
template <int N, bool FP, bool OBJ = false>
__global__ __launch_bounds__(256, (pass2_min_waves<N, FP, OBJ>())) void k_pass2(const float2* __restrict__ im, const float2* __restrict__ in,
                                               int cap, const uint8_t* __restrict__ active,
                                               const int* __restrict__ vend, int64_t bf0,
                                               int cb, float dcf, float* __restrict__ part_s1,
                                               double* __restrict__ part_s2, int gcap,
                                               const float2* __restrict__ gtw,
                                               const float2* __restrict__ na, const float2* __restrict__ nb,
                                               float* __restrict__ part_obj) {
    // FFT twiddles from an LDS copy of the table (not registers: 4 waves per SIMD)
    using F = WaveFFTT<N, +1>;
    __shared__ float2 twt[F::TABLE];
    constexpr int H = N / 2;
    constexpr int R = F::R, L = F::L;
    __shared__ float2 buf[4 * F::W][F::SCRATCH];
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

    // The group's activity flags and last supported columns, one BF pixel per lane,
    // read once: inside the loop they come from a ballot mask and lane reads (scalar
    // values), so each BF pixel's column loads issue at once instead of after a
    // dependent flag load and its wait.
    static_assert(kGroupBF <= 64, "one BF pixel of a group per lane");
    const int gl = lane < b_hi - b_lo ? lane : 0;
    const bool act_l = lane < b_hi - b_lo && active[bf0 + b_lo + gl];
    const int ve_l = vend[bf0 + b_lo + gl];
    const uint64_t amask = __ballot(act_l);
    auto next_active = [&](int b) {
        const uint64_t m = b - b_lo < 64 ? amask >> (b - b_lo) : 0;
        return m ? b + (int)__builtin_ctzll(m) : b_hi;
    };
    auto vend_of = [&](int b) { return __builtin_amdgcn_readlane(ve_l, b - b_lo); };
    auto plane_ptr = [&](int b) { return im + ((int64_t)t * cap + b) * N * H; };
    auto nyq_ptr = [&](int b) { return in + ((int64_t)t * cap + b) * N; };

    RowPairUnits<N, R, L> cur;
    int b = next_active(b_lo);

    F fft;
    for (int e = tid; e < F::TABLE; e += 256) twt[e] = gtw[e];
    __syncthreads();
    float s1a[R], s1b[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        s1a[r] = 0.f;
        s1b[r] = 0.f;
    }
    double s2 = 0.0;
    const float sgn = (j & 1) ? -1.f : 1.f;   // (-1)^x for x = j + r L, L even
    float oa[OBJ ? R : 1], ob[OBJ ? R : 1], rea = 0.f, reb = 0.f;
    float qa[OBJ && FP ? R : 1], qb[OBJ && FP ? R : 1];
#pragma unroll
    for (int r = 0; r < (OBJ ? R : 1); ++r) oa[r] = ob[r] = 0.f;
#pragma unroll
    for (int r = 0; r < (OBJ && FP ? R : 1); ++r) qa[r] = qb[r] = 0.f;

    while (b < b_hi) {
        const int bn = next_active(b + 1);
        cur.load(plane_ptr(b), nyq_ptr(b), y0, j, vend_of(b));
        float2 x[R];
        cur.assemble(j, x);
        float2 av0, av1, bv[FP ? R : 1];
        if constexpr (FP) {
            const int64_t o = ((int64_t)t * cap + b) * N;
            av0 = na[o + y0];
            av1 = na[o + y0 + 1];
#pragma unroll
            for (int r = 0; r < R; ++r) bv[r] = nb[o + j + r * L];
        }
        fft.run(x, buf[grp], j, twt);
        const float den0 = dcf + cur.dc_re0() + sgn * cur.ny_re0();
        const float den1 = dcf + cur.dc_re1() + sgn * cur.ny_re1();
        float p2 = 0.f;
        if constexpr (FP) {
            // rows y0 (even: (-1)^y = +1) and y0 + 1 (odd: -1)
            const float r0 = fmaf(sgn, av0.x, den0), i0 = sgn * av0.y;
            const float r1 = fmaf(sgn, av1.x, den1), i1 = sgn * av1.y;
            // Re O > 0 and |Im O| <= Re O for every sample of the wave: the [0, 1]
            // polynomial of Im O / Re O with a reciprocal per sample (the general
            // atan2's phase bits on those inputs); else the general atan2
            bool easy = true;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float ra = r0 + bv[r].x, rb = r1 - bv[r].x;
                x[r].x += i0 + bv[r].y;
                x[r].y += i1 - bv[r].y;
                bv[r] = make_float2(ra, rb);
                easy = easy && ra > 0.f && rb > 0.f && fabsf(x[r].x) <= ra && fabsf(x[r].y) <= rb;
            }
            if constexpr (OBJ) {
                // O_b on rows y0 and y0 + 1: real parts bv[r], imaginary parts x[r]
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    oa[r] += x[r].x;
                    ob[r] += x[r].y;
                    qa[r] += bv[r].x;
                    qb[r] += bv[r].y;
                }
            }
            if (__all(easy)) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float pa = atan_unit(x[r].x * __builtin_amdgcn_rcpf(bv[r].x));
                    float pb = atan_unit(x[r].y * __builtin_amdgcn_rcpf(bv[r].y));
                    asm("" : "+v"(pa), "+v"(pb));   // each phase rounded before it is summed
                    s1a[r] += pa;
                    s1b[r] += pb;
                    p2 = fmaf(pb, pb, fmaf(pa, pa, p2));
                }
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float pa = atan2_f(x[r].x, bv[r].x);
                    float pb = atan2_f(x[r].y, bv[r].y);
                    asm("" : "+v"(pa), "+v"(pb));
                    s1a[r] += pa;
                    s1b[r] += pb;
                    p2 = fmaf(pb, pb, fmaf(pa, pa, p2));
                }
            }
        } else {
            // Re O > 0 and |Im O| <= Re O for every sample of the wave: atan2 is the
            // odd polynomial of Im O / Re O, with one reciprocal per row (the real part
            // depends on the pixel only through its parity): the same phase bits as the
            // general atan2 on those inputs (only the sums may round differently, where the
            // compiler fuses the polynomial's last multiply into the accumulation).
            // The test takes each row's largest |Im O| (three-input maxima) against its real
            // part, and the four tests' lane masks are combined in scalar registers: six
            // vector instructions fewer per BF pixel than a compare per sample (a NaN sample
            // makes the sums NaN on either path).
            float ma = fabsf(x[0].x), mb = fabsf(x[0].y);
#pragma unroll
            for (int r = 1; r < R; ++r) {
                ma = fmaxf(ma, fabsf(x[r].x));
                mb = fmaxf(mb, fabsf(x[r].y));
            }
            // LLVM predicates 2: ordered >, 5: ordered <=
            const uint64_t easy_m = __builtin_amdgcn_fcmpf(den0, 0.f, 2) & __builtin_amdgcn_fcmpf(den1, 0.f, 2) &
                                    __builtin_amdgcn_fcmpf(ma, den0, 5) & __builtin_amdgcn_fcmpf(mb, den1, 5);
            if constexpr (OBJ) {
                // O_b on rows y0 and y0 + 1: real parts den0, den1; imaginary parts x[r]
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    oa[r] += x[r].x;
                    ob[r] += x[r].y;
                }
                rea += den0;
                reb += den1;
            }
            if (easy_m == __builtin_amdgcn_read_exec()) {
                const float i0 = __builtin_amdgcn_rcpf(den0), i1 = __builtin_amdgcn_rcpf(den1);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float pa = atan_unit(x[r].x * i0);
                    float pb = atan_unit(x[r].y * i1);
                    // each phase rounded on its own before it is summed: the polynomial's
                    // last multiply is never fused into the sums, in any variant of this
                    // kernel, so the object-summing variant gives the same moments bitwise
                    asm("" : "+v"(pa), "+v"(pb));
                    s1a[r] += pa;
                    s1b[r] += pb;
                    p2 = fmaf(pb, pb, fmaf(pa, pa, p2));
                }
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float pa = atan2_f(x[r].x, den0);
                    float pb = atan2_f(x[r].y, den1);
                    asm("" : "+v"(pa), "+v"(pb));
                    s1a[r] += pa;
                    s1b[r] += pb;
                    p2 = fmaf(pb, pb, fmaf(pa, pa, p2));
                }
            }
        }
        s2 += (double)p2;
        b = bn;
    }

    float* o = part_s1 + (((int64_t)t * gcap + g) * N + y0) * N;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        o[j + r * L] = s1a[r];
        o[N + j + r * L] = s1b[r];
    }
    if constexpr (OBJ) {
        float* po = part_obj + ((int64_t)t * gcap + g) * obj_sum_count(N, FP);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            po[(int64_t)y0 * N + j + r * L] = oa[r];
            po[(int64_t)(y0 + 1) * N + j + r * L] = ob[r];
        }
        if constexpr (FP) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                po[(int64_t)N * N + (int64_t)y0 * N + j + r * L] = qa[r];
                po[(int64_t)N * N + (int64_t)(y0 + 1) * N + j + r * L] = qb[r];
            }
        } else if (j < 2) {
            // Re sums per row and column parity: lanes 0 (even columns) and 1 (odd)
            po[(int64_t)N * N + 2 * y0 + j] = rea;
            po[(int64_t)N * N + 2 * (y0 + 1) + j] = reb;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s2 += __shfl_xor(s2, off);
    if (lane == 0) red[wave] = s2;
    __syncthreads();
    if (tid == 0) part_s2[((int64_t)t * gcap + g) * gridDim.x + blockIdx.x] = ((red[0] + red[1]) + red[2]) + red[3];
}

// S1run[t][p] += sum over groups g (in order) of part_s1[t][g][p], in double.
// first: the range's first chunk, whose sums start from zero (no clearing launch)
__global__ __launch_bounds__(256) void k_accum_s1(const float* __restrict__ part, int gcap, int ng,
                                                  int64_t n2, double* __restrict__ s1run, int first) {
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int t = blockIdx.y;
    if (p >= n2) return;
    double acc = first ? 0.0 : s1run[t * n2 + p];
    const float* src = part + (int64_t)t * gcap * n2 + p;
    // groups added in order; the loads of 8 groups are issued together
    int g = 0;
    for (; g + 8 <= ng; g += 8) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = src[(int64_t)(g + k) * n2];
#pragma unroll
        for (int k = 0; k < 8; ++k) acc += (double)v[k];
    }
    for (; g < ng; ++g) acc += (double)src[(int64_t)g * n2];
    s1run[t * n2 + p] = acc;
}

// S2run[t] += sum over groups g (in order) of (sum over row blocks in order).  One
// thread per group forms its group's sum; one thread then adds the group sums in
// group order.  Independent of how groups are chunked.
__global__ __launch_bounds__(256) void k_accum_s2(const double* __restrict__ part, int gcap, int ng, int rb,
                                                  double* __restrict__ s2run, int first) {
    __shared__ double gs[256];
    const int t = blockIdx.x;
    double run = 0.0;
    if (threadIdx.x == 0 && !first) run = s2run[t];
    for (int g0 = 0; g0 < ng; g0 += 256) {
        const int g = g0 + threadIdx.x;
        double v = 0.0;
        if (g < ng) {
            // added in order; the loads of 8 row blocks are issued together (one dependent
            // load per row block took 0.021 ms)
            const double* src = part + ((int64_t)t * gcap + g) * rb;
            int i = 0;
            for (; i + 8 <= rb; i += 8) {
                double w[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) w[k] = src[i + k];
#pragma unroll
                for (int k = 0; k < 8; ++k) v += w[k];
            }
            for (; i < rb; ++i) v += src[i];
        }
        gs[threadIdx.x] = v;
        __syncthreads();
        if (threadIdx.x == 0) {
            const int m = min(256, ng - g0);
            for (int i = 0; i < m; ++i) run += gs[i];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) s2run[t] = run;
}

// The object redraw from the row pass's sums (one trial): per pixel (y, x), the object
// summed over every BF pixel is Re = acc[N^2 + 2 y + x mod 2] (half plane) or
// acc[N^2 + y N + x] (full plane), plus re_extra (the inactive BF pixels contribute their
// DC term only), and Im = acc[y N + x]; its phase is the phase of the mean object.
__global__ __launch_bounds__(256) void k_obj_from_sums(const double* __restrict__ acc, int n, int fp,
                                                        double re_extra, double scale, float* __restrict__ phase,
                                                        float2* __restrict__ psi) {
    const int64_t n2 = (int64_t)n * n;
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (p >= n2) return;
    const int y = (int)(p / n), x = (int)(p - (int64_t)y * n);
    const double re = (fp ? acc[n2 + p] : acc[n2 + 2 * y + (x & 1)]) + re_extra;
    const double imv = acc[p];
    phase[p] = (float)atan2(imv, re);
    if (psi) psi[p] = make_float2((float)(re * scale), (float)(imv * scale));
}

__global__ __launch_bounds__(64) void k_set_trials(TrialBlock blk, int count, TrialConst* __restrict__ out) {
    const int i = threadIdx.x;
    if (i < count) out[i] = blk.t[i];
}

__global__ __launch_bounds__(256) void k_fill(double* p, int64_t count) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < count) p[i] = 0.0;
}

// Per-block sums of (S1/n_bf)^2 over fixed pixel blocks (and the mean phase of
// trial 0), then loss[t] = S2/(n_bf N^2) - (1/N^2) sum_blocks, in block order.
constexpr int kLossBlocks = 256;

__global__ __launch_bounds__(256) void k_loss_partial(const double* __restrict__ s1run, int64_t n2, double nbf,
                                                      double* __restrict__ lpart, float* __restrict__ mean_phase) {
    __shared__ double sh[256];
    const int t = blockIdx.y;
    const int64_t per = (n2 + kLossBlocks - 1) / kLossBlocks;
    const int64_t p0 = blockIdx.x * per, p1 = min(n2, p0 + per);
    double acc = 0.0;
    for (int64_t p = p0 + threadIdx.x; p < p1; p += 256) {
        const double mval = s1run[t * n2 + p] / nbf;
        acc += mval * mval;
        if (t == 0 && mean_phase) mean_phase[p] = (float)mval;
    }
    sh[threadIdx.x] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) lpart[(int64_t)t * kLossBlocks + blockIdx.x] = sh[0];
}

__global__ __launch_bounds__(64) void k_loss(const double* __restrict__ lpart, const double* __restrict__ s2run,
                                             int64_t n2, double nbf, double* __restrict__ loss) {
    // the block sums staged through the LDS by the whole wave, then added in block order
    // by one thread
    __shared__ double ls[kLossBlocks];
    const int t = blockIdx.x;
    for (int i = threadIdx.x; i < kLossBlocks; i += 64) ls[i] = lpart[(int64_t)t * kLossBlocks + i];
    __syncthreads();
    if (threadIdx.x != 0) return;
    double sum = 0.0;
    for (int i = 0; i < kLossBlocks; ++i) sum += ls[i];
    loss[t] = s2run[t] / (nbf * (double)n2) - sum / (double)n2;
}

// Row transform of the cached spectra: counts rows y0, y1 packed as one complex
// forward FFT, split by Hermitian symmetry.  Also the exact integer scan sum of
// every BF pixel.
template <int N>
__global__ __launch_bounds__(256) void k_g_rows(const uint32_t* __restrict__ counts, int64_t b0,
                                                float2* __restrict__ gm, float2* __restrict__ gn,
                                                unsigned long long* __restrict__ bfsum,
                                                const float2* __restrict__ twt) {
    constexpr int H = N / 2;
    using F = WaveFFT<N, -1>;
    constexpr int R = F::R, L = F::L;
    __shared__ float2 buf[4 * F::W][F::SCRATCH];

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
    fft.load(twt, j);
    fft.run(x, buf[grp], j);
    wave_lds_fence();
#pragma unroll
    for (int r = 0; r < R; ++r) buf[grp][j + r * L] = x[r];
    wave_lds_fence();
    float2* g0 = gm + b * N * H;
#pragma unroll
    for (int r = 0; r < R / 2; ++r) {
        const int v = j + r * L;
        const float2 z = x[r];
        const float2 zm = buf[grp][(N - v) & (N - 1)];
        // X0 = (Z(v) + conj Z(N-v))/2, X1 = (Z(v) - conj Z(N-v))/(2i); rows y0, y0 + 1
        // of a tile are adjacent (one 128-byte line per 8 columns)
        const int64_t e = tm_index(N, y0, v);
        g0[e] = make_float2(0.5f * (z.x + zm.x), 0.5f * (z.y - zm.y));
        g0[e + kTileW] = make_float2(0.5f * (z.y + zm.y), -0.5f * (z.x - zm.x));
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

// Object: sum over the BF pixels of one segment of the corrected half-plane
// spectrum.  One workgroup = one column tile (as in pass 1) x one BF segment; each
// thread keeps its tile entries' running sums in registers (float, at most a
// segment's worth of terms) and loops over the segment's BF pixels in order:
// support from the per-column intervals, predicated loads, the same correction as
// pass 1 (exp(-i delta) from two phasor chains per thread, no workgroup barrier in the
// loop; exp(i chi_q) once per entry).  Tiles at or past a BF pixel's last supported
// column skip it.  Partials per segment: the float sums themselves (added in double
// by k_obj_reduce, so storing them as float loses nothing and halves their traffic).
// Grid: x = segment, y = column tile.  Workgroups are dispatched x fastest, so every
// segment of tile 0 goes first: the support, and with it the work, shrinks with the
// column (tile 0 holds about 26 M of the 503 M support entries at 512^2, the last main
// tile 1 M), and the lightest items fill the tail (object sum 1.51 -> 1.30 ms against
// the tile-fastest order).
// 1024 threads at N = 1024 keep a thread's share of the tile at 8 entries, as at 512.
template <int N> constexpr int obj_threads() { return N >= 1024 ? 1024 : 512; }

// Object sum of one main column tile with a thread on two adjacent columns of its rows
// (row rr + (NT/4) k, columns 2 (tid % 4) and the next): both columns of a row in one
// 16-byte load (half the load instructions of one column per thread), the second
// column's phase ramp the first's times exp(-i alpha) (object sum 1.025-1.029 ->
// 0.932-0.943 ms; the object's phase moves by at most 1.8e-7 rad, rounding).
template <int N, int TC>
__device__ __forceinline__ void obj_tile_pair(const float2* __restrict__ gm, const double2* __restrict__ kb,
                                              const uint4* __restrict__ sup, const int* __restrict__ vend,
                                              const TrialConst& m, const GeomDev& geo, int64_t nbf, int seglen,
                                              float2* __restrict__ part, int tix, int seg) {
    constexpr int H = N / 2;
    constexpr int NE = N * (H + 1);
    constexpr int NT = obj_threads<N>();
    constexpr int RQ = NT / 4;                 // rows per sweep
    constexpr int PK = N / RQ;                 // rows per thread
    static_assert(TC == 8 && PK % 2 == 0 && (PK / 2) * RQ == H && RQ % 16 == 0, "two chains split at N/2");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int cA = 2 * (tid & 3);
    const int rr = tid >> 2;
    const int v0 = tix * TC, vA = v0 + cA, vB = vA + 1;
    const int64_t tb = (int64_t)tix * N * TC;
    const int64_t b_lo = (int64_t)seg * seglen;
    const int64_t b_hi = min(nbf, b_lo + seglen);

    float2 chv[2 * PK], acc[2 * PK];           // entry 2k + (column B)
#pragma unroll
    for (int k = 0; k < PK; ++k) {
        const int u = rr + k * RQ;
        const double up = (double)(u < H ? u : u - N);
        chv[2 * k] = chi_phasor(fma(geo.qux, up, geo.qvx * vA), fma(geo.quy, up, geo.qvy * vA), m);
        chv[2 * k + 1] = chi_phasor(fma(geo.qux, up, geo.qvx * vB), fma(geo.quy, up, geo.qvy * vB), m);
        acc[2 * k] = make_float2(0.f, 0.f);
        acc[2 * k + 1] = make_float2(0.f, 0.f);
    }
    int64_t wbase = b_lo;
    uint64_t wmask = 0;
    auto load_window = [&]() {
        const int64_t bl = wbase + lane;
        bool has = false;
        if (bl < b_hi) has = v0 < vend[bl];
        wmask = __ballot(has);
    };
    auto next_bf = [&]() -> int64_t {
        while (wmask == 0) {
            wbase += 64;
            if (wbase >= b_hi) return b_hi;
            load_window();
        }
        const int64_t bx = wbase + __builtin_ctzll(wmask);
        wmask &= wmask - 1;
        return bx;
    };
    load_window();
    int64_t b = next_bf();
    uint4 snA = make_uint4(0, 0, 0, 0), snB = snA;
    double2 kn = make_double2(0.0, 0.0);
    if (b < b_hi) {
        snA = sup[b * (H + 1) + vA];
        snB = sup[b * (H + 1) + vB];
        kn = kb[b];
    }
    while (b < b_hi) {
        const uint4 sA = snA, sB = snB;
        const double2 k = kn;
        const int64_t bn = next_bf();
        if (bn < b_hi) {
            snA = sup[bn * (H + 1) + vA];
            snB = sup[bn * (H + 1) + vB];
            kn = kb[bn];
        }
        const __amdgpu_buffer_rsrc_t rg = make_rsrc(gm + b * N * H + tb, N * TC * 8);
        auto upk = [&](int kk) { return rr + kk * RQ - (kk < PK / 2 ? 0 : N); };
        auto inA = [&](int up, bool& mm, bool& pp) {
            mm = (unsigned)(up - unpack_lo(sA.x)) < (unsigned)unpack_len(sA.x);
            pp = (unsigned)(up - unpack_lo(sA.y)) < (unsigned)unpack_len(sA.y);
            return (mm || pp) && (up != 0 || vA != 0);
        };
        auto inB = [&](int up, bool& mm, bool& pp) {
            mm = (unsigned)(up - unpack_lo(sB.x)) < (unsigned)unpack_len(sB.x);
            pp = (unsigned)(up - unpack_lo(sB.y)) < (unsigned)unpack_len(sB.y);
            return mm || pp;
        };
        float4 gv[PK];
#pragma unroll
        for (int kk = 0; kk < PK; ++kk) {
            bool mm, pp;
            const int up = upk(kk);
            const bool on = inA(up, mm, pp) || inB(up, mm, pp);
            gv[kk] = load4_or_zero(rg, on ? ((rr + kk * RQ) * TC + cA) * 8 : kNoLoad);
        }
        double alpha, beta;
        delta_slopes(k.x, k.y, m, geo, alpha, beta);
        float2 ea, eb, st, e1;
        wave_chain_starts_pair(lane, (tid >> 6) * 16, v0, RQ, H, alpha, beta, ea, eb, st, e1);
        auto entry = [&](int kk, bool colB, float2 g, float2 e) {
            const int up = upk(kk);
            bool inm, inp;
            if (colB ? inB(up, inm, inp) : inA(up, inm, inp)) {
                const uint4 sr = colB ? sB : sA;
                auto edge = [&](bool& edm, bool& edp) {
                    int uo = up;   // opaque: the tests stay in the branch that needs them
                    asm volatile("" : "+v"(uo));
                    edm = (unsigned)(uo - unpack_lo(sr.z)) >= (unsigned)unpack_len(sr.z);
                    edp = (unsigned)(uo - unpack_lo(sr.w)) >= (unsigned)unpack_len(sr.w);
                };
                const int i = 2 * kk + (colB ? 1 : 0);
                const float2 cv = correct_entry(g, chv[i], e, inm, inp, edge, up, colB ? vB : vA, k.x, k.y, geo);
                acc[i].x += cv.x;
                acc[i].y += cv.y;
            }
        };
#pragma unroll
        for (int kk = 0; kk < PK / 2; ++kk) {
            const float4 ga = gv[kk], gb = gv[kk + PK / 2];
            entry(kk, false, make_float2(ga.x, ga.y), ea);
            entry(kk, true, make_float2(ga.z, ga.w), cmul(ea, e1));
            entry(kk + PK / 2, false, make_float2(gb.x, gb.y), eb);
            entry(kk + PK / 2, true, make_float2(gb.z, gb.w), cmul(eb, e1));
            ea = cmul(ea, st);
            eb = cmul(eb, st);
        }
        b = bn;
    }
#pragma unroll
    for (int k = 0; k < PK; ++k) {
        const int u = rr + k * RQ;
        float2* o = part + (int64_t)seg * NE + (int64_t)u * (H + 1) + vA;
        o[0] = acc[2 * k];
        o[1] = acc[2 * k + 1];
    }
}

template <int N, int TC>
__global__ __launch_bounds__(obj_threads<N>()) void k_obj_sum(const float2* __restrict__ gm,
                                                         const float2* __restrict__ gn,
                                                         const double2* __restrict__ kb,
                                                         const uint4* __restrict__ sup,
                                                         const int* __restrict__ vend, TrialConst m, GeomDev geo,
                                                         int64_t nbf, int seglen, float2* __restrict__ part) {
    constexpr int H = N / 2;
    constexpr int NE = N * (H + 1);
    constexpr int NT = obj_threads<N>();
    constexpr int RS = NT / TC;
    constexpr int PER = (N + RS - 1) / RS;
    constexpr int PERN = (N + NT - 1) / NT;
    constexpr int PM = PER > PERN ? PER : PERN;

    const int tid = threadIdx.x;
    const int tix = blockIdx.y, seg = blockIdx.x;
    const bool nyq = tix == H / TC;
    // main tiles from N = 256 on: two columns per thread (obj_tile_pair)
    constexpr int PKP = N / (obj_threads<N>() / 4);
    if constexpr (TC == 8 && PKP >= 2 && PKP % 2 == 0) {
        if (!nyq) {
            obj_tile_pair<N, TC>(gm, kb, sup, vend, m, geo, nbf, seglen, part, tix, seg);
            return;
        }
    }
    const int c = nyq ? 0 : tid % TC;
    const int v0 = nyq ? H : tix * TC;
    const int v = v0 + c;
    const int ustart = nyq ? tid : tid / TC;
    const int ustep = nyq ? NT : RS;
    const int nent = nyq ? PERN : PER;
    static_assert(TC == kTileW, "object tiles are the layout's tiles");
    const int sstride = nyq ? 1 : TC;             // row stride inside the tile block
    const int64_t tb = (int64_t)tix * N * TC;      // this tile's block in a plane
    const int64_t b_lo = (int64_t)seg * seglen;
    const int64_t b_hi = min(nbf, b_lo + seglen);

    float2 chv[PM], acc[PM];
#pragma unroll
    for (int i = 0; i < PM; ++i) {
        const int u = ustart + i * ustep;
        const int up = u < H ? u : u - N;
        chv[i] = chi_phasor(fma(geo.qux, (double)up, geo.qvx * v), fma(geo.quy, (double)up, geo.qvy * v), m);
        acc[i] = make_float2(0.f, 0.f);
    }

    // BF pixels with support in this tile, in order, 64 at a time: one last-supported-
    // column value per lane and a ballot, so stepping to the next one takes no dependent
    // load (inactive BF pixels have none).  The next one's column support and k are
    // fetched while the current one is corrected.
    const int lane = tid & 63;
    int64_t wbase = b_lo;
    uint64_t wmask = 0;
    auto load_window = [&]() {
        const int64_t bl = wbase + lane;
        bool has = false;
        if (bl < b_hi) has = v0 < vend[bl];
        wmask = __ballot(has);
    };
    auto next_bf = [&]() -> int64_t {
        while (wmask == 0) {
            wbase += 64;
            if (wbase >= b_hi) return b_hi;
            load_window();
        }
        const int64_t bx = wbase + __builtin_ctzll(wmask);
        wmask &= wmask - 1;
        return bx;
    };
    load_window();
    int64_t b = next_bf();
    uint4 srn = make_uint4(0, 0, 0, 0);
    double2 kn = make_double2(0.0, 0.0);
    if (b < b_hi) {
        srn = sup[b * (H + 1) + v];
        kn = kb[b];
    }
    while (b < b_hi) {
        const uint4 sr = srn;
        const double2 k = kn;
        const int64_t bn = next_bf();
        if (bn < b_hi) {
            srn = sup[bn * (H + 1) + v];
            kn = kb[bn];
        }
        const int lo_m = unpack_lo(sr.x), len_m = unpack_len(sr.x);
        const int lo_p = unpack_lo(sr.y), len_p = unpack_len(sr.y);
        const int flo_m = unpack_lo(sr.z), flen_m = unpack_len(sr.z);
        const int flo_p = unpack_lo(sr.w), flen_p = unpack_len(sr.w);
        const __amdgpu_buffer_rsrc_t rg =
            nyq ? make_rsrc(gn + b * N, N * 8) : make_rsrc(gm + b * N * H + tb, N * TC * 8);
        float2 gv[PM];
        // entry i in the support of either shifted aperture (DC excluded); evaluated
        // again at the correction instead of kept as flag bits through the loads
        auto on_of = [&](int i, bool& inm, bool& inp) {
            const int u = ustart + i * ustep;
            const int up = u < H ? u : u - N;
            inm = (unsigned)(up - lo_m) < (unsigned)len_m;
            inp = (unsigned)(up - lo_p) < (unsigned)len_p;
            return i < nent && u < N && (inm || inp) && (u != 0 || v != 0);
        };
#pragma unroll
        for (int i = 0; i < PM; ++i) {
            const int u = ustart + i * ustep;
            bool inm, inp;
            gv[i] = load_or_zero(rg, on_of(i, inm, inp) ? (u * sstride + c) * 8 : kNoLoad);
        }
        // phase ramps exp(-i delta) of this BF while its spectrum loads are in flight: per
        // thread one chain over its rows below N/2 and one over its rows from N/2 on (steps
        // of RS rows), as in pass 1; the Nyquist tile's one entry per thread directly
        double alpha, beta;
        delta_slopes(k.x, k.y, m, geo, alpha, beta);
        const double av = (double)v * alpha;
        float2 ea, eb, st;
        if (!nyq && (PM % 2 == 0 && (PM / 2) * RS == H)) {
            static_assert(TC == 8, "a wave is 8 rows x 8 columns of the tile");
            wave_chain_starts(lane, (tid >> 6) * 8, v0, RS, H, alpha, beta, ea, eb, st);
        } else {
            ea = phasor_rev_neg(fma((double)(ustart < H ? ustart : ustart - N), beta, av));
            eb = ea;
            st = make_float2(1.f, 0.f);
        }
        auto entry = [&](int i, float2 e) {
            bool inm, inp;
            if (on_of(i, inm, inp)) {
                const int u = ustart + i * ustep;
                const int up = u < H ? u : u - N;
                auto edge = [&](bool& edm, bool& edp) {
                    int uo = up;   // opaque: the tests stay in the branch that needs them
                    asm volatile("" : "+v"(uo));
                    edm = (unsigned)(uo - flo_m) >= (unsigned)flen_m;
                    edp = (unsigned)(uo - flo_p) >= (unsigned)flen_p;
                };
                const float2 cv = correct_entry(gv[i], chv[i], e, inm, inp, edge, up, v, k.x, k.y, geo);
                acc[i].x += cv.x;
                acc[i].y += cv.y;
            }
        };
        if constexpr (PM % 2 == 0 && (PM / 2) * RS == H) {
#pragma unroll
            for (int i = 0; i < PM / 2; ++i) {
                entry(i, ea);
                entry(i + PM / 2, eb);
                ea = cmul(ea, st);
                eb = cmul(eb, st);
            }
        } else {
            // small transforms (a thread's rows do not split evenly at N/2): each entry's
            // phasor directly
#pragma unroll
            for (int i = 0; i < PM; ++i) {
                const int u = ustart + i * ustep;
                entry(i, phasor_rev_neg(fma((double)(u < H ? u : u - N), beta, av)));
            }
        }
        b = bn;
    }
#pragma unroll
    for (int i = 0; i < PM; ++i) {
        const int u = ustart + i * ustep;
        if (i < nent && u < N)
            part[(int64_t)seg * NE + (int64_t)u * (H + 1) + v] = acc[i];
    }
}

template <int N>
__global__ __launch_bounds__(256) void k_obj_reduce(const float2* __restrict__ part, int nseg,
                                                    float2* __restrict__ pm, float2* __restrict__ pn) {
    constexpr int H = N / 2;
    constexpr int NE = N * (H + 1);
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= NE) return;
    double ax = 0.0, ay = 0.0;
    int s = 0;
    for (; s + 8 <= nseg; s += 8) {             // segments added in order, 8 loads in flight
        float2 p[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) p[k] = part[(int64_t)(s + k) * NE + e];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            ax += p[k].x;
            ay += p[k].y;
        }
    }
    for (; s < nseg; ++s) {
        const float2 p = part[(int64_t)s * NE + e];
        ax += p.x;
        ay += p.y;
    }
    const int u = e / (H + 1), v = e % (H + 1);
    const float2 val = make_float2((float)ax, (float)ay);
    if (v < H) pm[tm_index(N, u, v)] = val;
    else pn[u] = val;
}

// FP: the full-plane variant adds (-1)^x A(y) + (-1)^y B(x) from nab = [A | B]
// (BF sums, k_obj_nyq_fin).
template <int N, bool FP>
__global__ __launch_bounds__(256) void k_obj_rows(const float2* __restrict__ pm, const float2* __restrict__ pn,
                                                  float dcs, float scale, float* __restrict__ phase,
                                                  float2* __restrict__ psi, const float2* __restrict__ twt,
                                                  const float2* __restrict__ nab) {
    constexpr int H = N / 2;
    using F = WaveFFT<N, +1>;
    constexpr int R = F::R, L = F::L;
    __shared__ float2 buf[4 * F::W][F::SCRATCH];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int grp = (tid >> 6) * F::W + lane / L;
    const int j = lane % L;
    const int y0 = 2 * (blockIdx.x * (4 * F::W) + grp);
    RowPairRaw<N, R, L> raw;
    raw.load(pm, pn, y0, j, H + 1);   // every column present
    float2 x[R];
    raw.assemble(j, x);
    F fft;
    fft.load(twt, j);
    fft.run(x, buf[grp], j);
    const float sgn = (j & 1) ? -1.f : 1.f;
    const float den0 = dcs + raw.z0.x + sgn * raw.h0.x;
    const float den1 = dcs + raw.z1.x + sgn * raw.h1.x;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int xx = j + r * L;
        float re0 = den0, im0 = x[r].x, re1 = den1, im1 = x[r].y;
        if constexpr (FP) {
            const float2 a0 = nab[y0], a1 = nab[y0 + 1], bx = nab[N + xx];
            re0 = fmaf(sgn, a0.x, re0) + bx.x;
            im0 = fmaf(sgn, a0.y, im0) + bx.y;
            re1 = fmaf(sgn, a1.x, re1) - bx.x;
            im1 = fmaf(sgn, a1.y, im1) - bx.y;
        }
        phase[y0 * N + xx] = atan2_f(im0, re0);
        phase[(y0 + 1) * N + xx] = atan2_f(im1, re1);
        if (psi) {
            psi[y0 * N + xx] = make_float2(re0 * scale, im0 * scale);
            psi[(y0 + 1) * N + xx] = make_float2(re1 * scale, im1 * scale);
        }
    }
}

// Full-plane object: per BF segment (in order) the sums of dC(u) and dR(v) (the
// Nyquist-line differences, as k_nyq_lines forms them), float per segment, in
// double partials part [seg][2N] = [dC | dR].
template <int N>
__global__ __launch_bounds__(256) void k_obj_nyq(const float2* __restrict__ gm, const float2* __restrict__ gn,
                                                 const double2* __restrict__ kb, const int* __restrict__ vend,
                                                 TrialConst m, GeomDev geo, int64_t nbf, int seglen,
                                                 double2* __restrict__ part) {
    constexpr int H = N / 2;
    constexpr int PC = (N + 255) / 256;
    const int tid = threadIdx.x;
    const int64_t b_lo = (int64_t)blockIdx.x * seglen;
    const int64_t b_hi = min(nbf, b_lo + seglen);
    float2 ac[PC], ar[PC];
#pragma unroll
    for (int i = 0; i < PC; ++i) {
        ac[i] = make_float2(0.f, 0.f);
        ar[i] = make_float2(0.f, 0.f);
    }
    for (int64_t b = b_lo; b < b_hi; ++b) {
        if (vend[b] == 0) continue;               // inactive BF pixel: zero transfer
        const double2 k = kb[b];
        double alpha, beta;
        delta_slopes(k.x, k.y, m, geo, alpha, beta);
#pragma unroll
        for (int i = 0; i < PC; ++i) {
            const int u = tid + i * 256;
            if (u < N) {
                const float2 dc = nyq_col_delta(gn[b * N + u], u < H ? u : u - N, k.x, k.y, m, geo, alpha, beta);
                ac[i].x += dc.x;
                ac[i].y += dc.y;
                if (u > H) {
                    const int vp = N - u;
                    const float2 dr = nyq_row_delta(gm[b * N * H + tm_index(N, H, vp)], vp, k.x, k.y, m, geo,
                                                    alpha, beta);
                    ar[i].x += dr.x;
                    ar[i].y += dr.y;
                }
            }
        }
    }
    double2* o = part + (int64_t)blockIdx.x * 2 * N;
#pragma unroll
    for (int i = 0; i < PC; ++i) {
        const int u = tid + i * 256;
        if (u < N) {
            o[u] = make_double2(ac[i].x, ac[i].y);
            o[N + u] = make_double2(ar[i].x, ar[i].y);
        }
    }
}

// Sum of the segment partials (in order, double), then A and B by two inverse
// transforms: nab = [A (N) | B (N)].
template <int N>
__global__ __launch_bounds__(256) void k_obj_nyq_fin(const double2* __restrict__ part, int nseg,
                                                     float2* __restrict__ nab, const float2* __restrict__ twt) {
    using F = WaveFFT<N, +1>;
    __shared__ float2 l2[2][F::SCRATCH];
    const int tid = threadIdx.x;
    for (int e = tid; e < 2 * N; e += 256) {
        double ax = 0.0, ay = 0.0;
        for (int sg = 0; sg < nseg; ++sg) {
            const double2 p = part[(int64_t)sg * 2 * N + e];
            ax += p.x;
            ay += p.y;
        }
        l2[e / N][e % N] = make_float2((float)ax, (float)ay);
    }
    __syncthreads();
    const int lane = tid & 63;
    const int grp = (tid >> 6) * F::W + lane / F::L;
    const int j = lane % F::L;
    if (grp < 2) {
        F fft;
        fft.load(twt, j);
        float2 x[F::R];
#pragma unroll
        for (int r = 0; r < F::R; ++r) x[r] = l2[grp][j + r * F::L];
        fft.run(x, l2[grp], j);
#pragma unroll
        for (int r = 0; r < F::R; ++r) nab[grp * N + j + r * F::L] = x[r];
    }
}

template <int N>
int row_blocks() {
    return (N / 2) / (4 * WaveFFT<N, 1>::W);
}

template <int N>
hipError_t g_rows_n(const uint32_t* counts, int64_t nbf, float2* gm, float2* gn, unsigned long long* bfsum,
                    const float2* tw, hipStream_t st) {
    for (int64_t b0 = 0; b0 < nbf; b0 += 65535) {
        const int nb = (int)std::min<int64_t>(65535, nbf - b0);
        hipLaunchKernelGGL(k_g_rows<N>, dim3(row_blocks<N>(), nb), dim3(256), 0, st, counts, b0, gm, gn, bfsum, tw);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int N, int MODE>
hipError_t cols_n(const float2* in_m, const float2* in_n, float2* out_m, float2* out_n, int64_t planes,
                  const float2* tw, hipStream_t st) {
    constexpr int H = N / 2;
    for (int64_t p0 = 0; p0 < planes; p0 += 65535) {
        const int np = (int)std::min<int64_t>(65535, planes - p0);
        hipLaunchKernelGGL((k_cols<N, MODE>), dim3(H / cols_tc<N>() + 1, np), dim3(256), 0, st, in_m + p0 * N * H,
                           in_n + p0 * N, out_m + p0 * N * H, out_n + p0 * N, tw);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Columns per pass-1 workgroup: one layout tile.  (Half tiles, 4 columns with 256
// threads, reach 7 waves per SIMD at 71 VGPRs but ran 6.2-6.5 ms against 3.2-3.3 ms
// at N = 512: both halves pull the tile's whole 64-byte rows, and the row-phase
// table then built per workgroup and the twiddles were paid per half.)
template <int N> constexpr int pass1_tc() { return kTileW; }

template <int N>
hipError_t pass1_n(const float2* gm, const float2* gn, const float2* chm, const float2* chn, const double2* kb,
                   const uint4* sup, const int* vend, const TrialConst* tc, int n_trials, GeomDev geo, int64_t bf0,
                   int cb, int cap, float2* im, float2* in, hipStream_t st) {
    constexpr int H = N / 2;
    constexpr int TC = pass1_tc<N>();
    // one launch per chunk: (H/TC + 1) tiles per BF in x, groups of TB trials in y
    constexpr int TB = SSB_PASS1_TB;
    const dim3 grid1((unsigned)((int64_t)cb * (H / TC + 1)), n_trials);
    const dim3 gridb((unsigned)((int64_t)cb * (H / TC + 1)), (n_trials + TB - 1) / TB);
    const bool stream = n_trials == 1 || (int64_t)cb * N * (H + 1) * 8 > ((int64_t)192 << 20);
    if (n_trials == 1 || TB == 1) {
        if (stream)
            hipLaunchKernelGGL((k_pass1<N, TC, true, 1>), grid1, dim3(pass1_threads<N>()), 0, st, gm, gn, chm, chn, kb,
                               sup, vend, tc, geo, bf0, cap, im, in, n_trials);
        else
            hipLaunchKernelGGL((k_pass1<N, TC, false, 1>), grid1, dim3(pass1_threads<N>()), 0, st, gm, gn, chm, chn,
                               kb, sup, vend, tc, geo, bf0, cap, im, in, n_trials);
    } else {
        if (stream)
            hipLaunchKernelGGL((k_pass1<N, TC, true, TB>), gridb, dim3(pass1_threads<N>()), 0, st, gm, gn, chm, chn,
                               kb, sup, vend, tc, geo, bf0, cap, im, in, n_trials);
        else
            hipLaunchKernelGGL((k_pass1<N, TC, false, TB>), gridb, dim3(pass1_threads<N>()), 0, st, gm, gn, chm, chn,
                               kb, sup, vend, tc, geo, bf0, cap, im, in, n_trials);
    }
    return hipGetLastError();
}

template <int N>
hipError_t chiq_n(const TrialConst* tc, int n_trials, GeomDev geo, float2* chm, float2* chn, hipStream_t st) {
    constexpr int NE = N * (N / 2 + 1);
    hipLaunchKernelGGL(k_chiq<N>, dim3((NE + 255) / 256, n_trials), dim3(256), 0, st, tc, geo, chm, chn);
    return hipGetLastError();
}

template <int N>
hipError_t support_n(const double2* kb, const uint8_t* active, GeomDev geo, int64_t nbf, uint4* sup, int* vend,
                     int* nsup, hipStream_t st) {
    const int64_t ne = nbf * (N / 2 + 1);
    hipLaunchKernelGGL(k_support<N>, dim3((unsigned)((ne + 255) / 256)), dim3(256), 0, st, kb, geo, nbf, sup);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_vend<N>, dim3((unsigned)((nbf + 255) / 256)), dim3(256), 0, st, sup, active, nbf, vend,
                       nsup);
    return hipGetLastError();
}

}  // namespace

#define SSB_DISPATCH_N(n, CALL)            \
    switch (n) {                           \
        case 32: { constexpr int NN = 32; return CALL; }   \
        case 64: { constexpr int NN = 64; return CALL; }   \
        case 128: { constexpr int NN = 128; return CALL; } \
        case 256: { constexpr int NN = 256; return CALL; } \
        case 512: { constexpr int NN = 512; return CALL; } \
        case 1024: { constexpr int NN = 1024; return CALL; } \
        default: return hipErrorInvalidValue;               \
    }

hipError_t launch_g_rows(int n, const uint32_t* counts, int64_t nbf, float2* gm, float2* gn,
                         unsigned long long* bfsum, const float2* tw_fwd, hipStream_t st) {
    SSB_DISPATCH_N(n, (g_rows_n<NN>(counts, nbf, gm, gn, bfsum, tw_fwd, st)))
}

hipError_t launch_g_cols(int n, float2* gm, float2* gn, int64_t nbf, const float2* tw_fwd, hipStream_t st) {
    SSB_DISPATCH_N(n, (cols_n<NN, COL_PLAIN_FWD>(gm, gn, gm, gn, nbf, tw_fwd, st)))
}

int twiddle_count(int n) {
    switch (n) {
        case 32: return WaveFFTT<32, 1>::TABLE;
        case 64: return WaveFFTT<64, 1>::TABLE;
        case 128: return WaveFFTT<128, 1>::TABLE;
        case 256: return WaveFFTT<256, 1>::TABLE;
        case 1024: return WaveFFTT<1024, 1>::TABLE;
        default: return WaveFFTT<512, 1>::TABLE;
    }
}

template <int N>
static hipError_t twiddles_n(float2* tw_inv, float2* tw_fwd, hipStream_t st) {
    hipLaunchKernelGGL((k_twiddles<N, 1>), dim3(1), dim3(256), 0, st, tw_inv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_twiddles<N, -1>), dim3(1), dim3(256), 0, st, tw_fwd);
    return hipGetLastError();
}

hipError_t launch_twiddles(int n, float2* tw_inv, float2* tw_fwd, hipStream_t st) {
    SSB_DISPATCH_N(n, (twiddles_n<NN>(tw_inv, tw_fwd, st)))
}

hipError_t launch_chiq(int n, const TrialConst* tc, int n_trials, GeomDev geo, float2* chm, float2* chn,
                       hipStream_t st) {
    SSB_DISPATCH_N(n, (chiq_n<NN>(tc, n_trials, geo, chm, chn, st)))
}

hipError_t launch_pass1(int n, const float2* gm, const float2* gn, const float2* chm, const float2* chn,
                        const double2* kb, const uint4* sup, const int* vend, const TrialConst* tc, int n_trials,
                        GeomDev geo, int64_t bf0, int cb, int cap, float2* im, float2* in, hipStream_t st) {
    SSB_DISPATCH_N(n, (pass1_n<NN>(gm, gn, chm, chn, kb, sup, vend, tc, n_trials, geo, bf0, cb, cap, im, in, st)))
}

int pass2_row_blocks(int n) {
    switch (n) {
        case 32: return row_blocks<32>();
        case 64: return row_blocks<64>();
        case 128: return row_blocks<128>();
        case 256: return row_blocks<256>();
        case 1024: return row_blocks<1024>();
        default: return row_blocks<512>();
    }
}

template <int N>
static hipError_t pass2_n(const float2* im, const float2* in, int cap, const uint8_t* active, const int* vend,
                          int64_t bf0, int cb, int n_trials, double dc, float* part_s1, double* part_s2, int gcap,
                          const float2* tw, const float2* na, const float2* nb, float* part_obj, hipStream_t st) {
    const int ng = (cb + kGroupBF - 1) / kGroupBF;
    const dim3 grid(row_blocks<N>(), ng, n_trials);
    if (part_obj) {
        if (na) {
            if constexpr (pass2_obj_sizes(N, true))
                hipLaunchKernelGGL((k_pass2<N, true, true>), grid, dim3(256), 0, st, im, in, cap, active, vend, bf0,
                                   cb, (float)dc, part_s1, part_s2, gcap, tw, na, nb, part_obj);
            else
                return hipErrorInvalidValue;
        } else {
            if constexpr (pass2_obj_sizes(N, false))
                hipLaunchKernelGGL((k_pass2<N, false, true>), grid, dim3(256), 0, st, im, in, cap, active, vend, bf0,
                                   cb, (float)dc, part_s1, part_s2, gcap, tw, na, nb, part_obj);
            else
                return hipErrorInvalidValue;
        }
    } else if (na) {
        hipLaunchKernelGGL((k_pass2<N, true>), grid, dim3(256), 0, st, im, in, cap, active, vend, bf0, cb, (float)dc,
                           part_s1, part_s2, gcap, tw, na, nb, part_obj);
    } else {
        hipLaunchKernelGGL((k_pass2<N, false>), grid, dim3(256), 0, st, im, in, cap, active, vend, bf0, cb,
                           (float)dc, part_s1, part_s2, gcap, tw, na, nb, part_obj);
    }
    return hipGetLastError();
}

hipError_t launch_pass2(int n, const float2* im, const float2* in, int cap, const uint8_t* active,
                        const int* vend, int64_t bf0, int cb, int n_trials, double dc, float* part_s1,
                        double* part_s2, int gcap, const float2* tw_inv, const float2* na, const float2* nb,
                        float* part_obj, hipStream_t st) {
    SSB_DISPATCH_N(n, (pass2_n<NN>(im, in, cap, active, vend, bf0, cb, n_trials, dc, part_s1, part_s2, gcap, tw_inv,
                                   na, nb, part_obj, st)))
}

template <int N>
static hipError_t nyq_lines_n(const float2* gm, const float2* gn, const double2* kb, const uint8_t* active,
                              const TrialConst* tc, int n_trials, GeomDev geo, int64_t bf0, int cb, int cap,
                              float2* na, float2* nb, const float2* tw, hipStream_t st) {
    hipLaunchKernelGGL(k_nyq_lines<N>, dim3(cb, n_trials), dim3(256), 0, st, gm, gn, kb, active, tc, geo, bf0, cap,
                       na, nb, tw);
    return hipGetLastError();
}

hipError_t launch_nyq_lines(int n, const float2* gm, const float2* gn, const double2* kb, const uint8_t* active,
                            const TrialConst* tc, int n_trials, GeomDev geo, int64_t bf0, int cb, int cap, float2* na,
                            float2* nb, const float2* tw_inv, hipStream_t st) {
    SSB_DISPATCH_N(n, (nyq_lines_n<NN>(gm, gn, kb, active, tc, n_trials, geo, bf0, cb, cap, na, nb, tw_inv, st)))
}

hipError_t launch_support(int n, const double2* kb, const uint8_t* active, GeomDev geo, int64_t nbf, uint4* sup,
                          int* vend, int* nsup, hipStream_t st) {
    SSB_DISPATCH_N(n, (support_n<NN>(kb, active, geo, nbf, sup, vend, nsup, st)))
}

int pass1_tile(int n) { return kTileW; }     // pass 1 writes whole layout tiles

hipError_t launch_accum(int n, const float* part_s1, const double* part_s2, int gcap, int ng, int n_trials,
                        double* s1run, double* s2run, bool first, hipStream_t st) {
    const int64_t n2 = (int64_t)n * n;
    hipLaunchKernelGGL(k_accum_s1, dim3((unsigned)((n2 + 255) / 256), n_trials), dim3(256), 0, st, part_s1, gcap,
                       ng, n2, s1run, (int)first);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_accum_s2, dim3(n_trials), dim3(256), 0, st, part_s2, gcap, ng, pass2_row_blocks(n), s2run,
                       (int)first);
    return hipGetLastError();
}

hipError_t launch_accum_obj(int n, bool fp, const float* part_obj, int gcap, int ng, int n_trials, double* acc,
                            bool first, hipStream_t st) {
    const int64_t n2 = obj_sum_count(n, fp);
    hipLaunchKernelGGL(k_accum_s1, dim3((unsigned)((n2 + 255) / 256), n_trials), dim3(256), 0, st, part_obj, gcap,
                       ng, n2, acc, (int)first);
    return hipGetLastError();
}

hipError_t launch_obj_from_sums(int n, bool fp, const double* acc, double re_extra, double scale, float* phase,
                                float2* psi, hipStream_t st) {
    const int64_t n2 = (int64_t)n * n;
    hipLaunchKernelGGL(k_obj_from_sums, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, st, acc, n, (int)fp,
                       re_extra, scale, phase, psi);
    return hipGetLastError();
}

hipError_t launch_set_trials(const TrialBlock& blk, int count, TrialConst* dev, hipStream_t st) {
    if (count <= 0) return hipSuccess;
    if (count > kTrialBlock) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_set_trials, dim3(1), dim3(64), 0, st, blk, count, dev);
    return hipGetLastError();
}

hipError_t launch_fill(double* p, int64_t count, hipStream_t st) {
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st, p, count);
    return hipGetLastError();
}

int loss_blocks() { return kLossBlocks; }

hipError_t launch_loss(int n, const double* s1run, const double* s2run, int n_trials, double n_bf, double* lpart,
                       double* loss, float* mean_phase, hipStream_t st) {
    const int64_t n2 = (int64_t)n * n;
    hipLaunchKernelGGL(k_loss_partial, dim3(kLossBlocks, n_trials), dim3(256), 0, st, s1run, n2, n_bf, lpart,
                       mean_phase);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_loss, dim3(n_trials), dim3(64), 0, st, lpart, s2run, n2, n_bf, loss);
    return hipGetLastError();
}

int obj_segments(int64_t nbf) {
    // enough segments to fill the chip, at least 16 BF per segment; at most 48 (with two
    // columns per thread, 48 against 64 took the sum and its reduction from 0.93-0.95 to
    // 0.92-0.93 ms at 512^2; 32, 40 and 96 were slower)
    int64_t seg = (nbf + 15) / 16;
    return (int)std::max<int64_t>(1, std::min<int64_t>(48, seg));
}

template <int N>
static hipError_t obj_sum_n(const float2* gm, const float2* gn, const double2* kb, const uint4* sup,
                            const int* vend, TrialConst tc, GeomDev geo, int64_t nbf, float2* part, int nseg,
                            hipStream_t st) {
    constexpr int TC = kTileW;
    const int seglen = (int)((nbf + nseg - 1) / nseg);
    const dim3 grid(nseg, N / 2 / TC + 1);
    hipLaunchKernelGGL((k_obj_sum<N, TC>), grid, dim3(obj_threads<N>()), 0, st, gm, gn, kb, sup,
                       vend, tc, geo, nbf, seglen, part);
    return hipGetLastError();
}

hipError_t launch_obj_sum(int n, const float2* gm, const float2* gn, const double2* kb, const uint4* sup,
                          const int* vend, TrialConst tc, GeomDev geo, int64_t nbf, float2* part, int nseg,
                          hipStream_t st) {
    SSB_DISPATCH_N(n, (obj_sum_n<NN>(gm, gn, kb, sup, vend, tc, geo, nbf, part, nseg, st)))
}

template <int N>
static hipError_t obj_reduce_n(const float2* part, int nseg, float2* pm, float2* pn, hipStream_t st) {
    constexpr int NE = N * (N / 2 + 1);
    hipLaunchKernelGGL(k_obj_reduce<N>, dim3((NE + 255) / 256), dim3(256), 0, st, part, nseg, pm, pn);
    return hipGetLastError();
}

hipError_t launch_obj_reduce(int n, const float2* part, int nseg, float2* pm, float2* pn, hipStream_t st) {
    SSB_DISPATCH_N(n, (obj_reduce_n<NN>(part, nseg, pm, pn, st)))
}

hipError_t launch_obj_cols(int n, float2* pm, float2* pn, const float2* tw_inv, hipStream_t st) {
    SSB_DISPATCH_N(n, (cols_n<NN, COL_PLAIN_INV>(pm, pn, pm, pn, 1, tw_inv, st)))
}

template <int N>
static hipError_t obj_rows_n(const float2* pm, const float2* pn, double dcsum, double scale, float* phase,
                             float2* psi, const float2* tw, const float2* nab, hipStream_t st) {
    if (nab)
        hipLaunchKernelGGL((k_obj_rows<N, true>), dim3(row_blocks<N>()), dim3(256), 0, st, pm, pn, (float)dcsum,
                           (float)scale, phase, psi, tw, nab);
    else
        hipLaunchKernelGGL((k_obj_rows<N, false>), dim3(row_blocks<N>()), dim3(256), 0, st, pm, pn, (float)dcsum,
                           (float)scale, phase, psi, tw, nab);
    return hipGetLastError();
}

hipError_t launch_obj_rows(int n, const float2* pm, const float2* pn, double dcsum, double scale, float* phase,
                           float2* psi, const float2* tw_inv, const float2* nab, hipStream_t st) {
    SSB_DISPATCH_N(n, (obj_rows_n<NN>(pm, pn, dcsum, scale, phase, psi, tw_inv, nab, st)))
}

template <int N>
static hipError_t obj_nyq_n(const float2* gm, const float2* gn, const double2* kb, const int* vend, TrialConst tc,
                            GeomDev geo, int64_t nbf, double2* part, int nseg, float2* nab, const float2* tw,
                            hipStream_t st) {
    const int seglen = (int)((nbf + nseg - 1) / nseg);
    hipLaunchKernelGGL(k_obj_nyq<N>, dim3(nseg), dim3(256), 0, st, gm, gn, kb, vend, tc, geo, nbf, seglen, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_obj_nyq_fin<N>, dim3(1), dim3(256), 0, st, part, nseg, nab, tw);
    return hipGetLastError();
}

hipError_t launch_obj_nyq(int n, const float2* gm, const float2* gn, const double2* kb, const int* vend,
                          TrialConst tc, GeomDev geo, int64_t nbf, double2* part, int nseg, float2* nab,
                          const float2* tw_inv, hipStream_t st) {
    SSB_DISPATCH_N(n, (obj_nyq_n<NN>(gm, gn, kb, vend, tc, geo, nbf, part, nseg, nab, tw_inv, st)))
}

}  // namespace ssb
