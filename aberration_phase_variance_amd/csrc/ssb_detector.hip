// Detector side of the SSB path on gfx950: the exact detector sum over every scan
// frame (the mean diffraction pattern), the probe-disk fit (on the host, or on the
// device from the device sums), and the
// gather of the BF pixels into the BF-major counts ssb_prepare takes (declared in
// ssb.h).
//
// The detector sum is a streaming integer reduction: every frame is read once,
// 16 bytes (four pixels) per lane, coalesced across the frame, non-temporal; each workgroup
// sums a block of frames in 64-bit registers and adds its partials to the output
// with 64-bit integer atomics, so the result is exact and independent of order.
// The gather is a tiled transpose: a workgroup reads 64 frames x 64 BF pixels
// (runs of neighbouring BF pixels are contiguous in a frame), every load of a
// thread in flight before the first LDS store, turns the tile in LDS and writes
// 64 scan positions per BF pixel contiguously.  (Longer BF runs would use more of
// each 128-byte line, but tiles of 8,192 values measured slower: 7.8 to 8.0 ms
// against 4.8 to 5.2 ms at 64 x 64, and 6.6 to 6.9 ms before the loads were
// issued together.)
#include "../../include/ssb.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <string>
#include <vector>

namespace ssb {
int set_error(int code, const std::string& msg);
void clear_error();
bool in_bf_disk(const ssb_geometry* g, int i, int j);
}  // namespace ssb

namespace {

constexpr int kSumFrames = 1024;   // frames per workgroup of the detector sum
#ifndef SSB_GATHER_FRAMES
#define SSB_GATHER_FRAMES 64
#endif
#ifndef SSB_GATHER_BF
#define SSB_GATHER_BF 64
#endif
#ifndef SSB_GATHER_XCD
#define SSB_GATHER_XCD 1   // BF tiles of one frame block on one XCD (0: a 2-D grid)
#endif
constexpr int kTileS = SSB_GATHER_FRAMES;   // gather tile: scan positions ...
constexpr int kTileB = SSB_GATHER_BF;       // ... x BF pixels
static_assert(kTileS * kTileB % 256 == 0, "whole tile rows per thread");

__global__ __launch_bounds__(256) void k_zero_u64(unsigned long long* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0ull;
}

// Four pixels per lane; frames [nf][4 * nq] viewed as uint4 [nf][nq].
__global__ __launch_bounds__(256) void k_detsum4(const uint4* __restrict__ frames, int64_t nf, int nq,
                                                 unsigned long long* __restrict__ sums) {
    const int q = blockIdx.x * 256 + threadIdx.x;
    if (q >= nq) return;
    const int64_t f0 = (int64_t)blockIdx.y * kSumFrames;
    const int64_t f1 = f0 + kSumFrames < nf ? f0 + kSumFrames : nf;
    unsigned long long a0 = 0, a1 = 0, a2 = 0, a3 = 0;
    const uint4* p = frames + f0 * nq + q;
    int64_t f = f0;
    // 16 frames in flight per lane; non-temporal loads (the frames are read once)
    // took the sum from 6.45 to 5.85 ms on the full frames
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    constexpr int U = 16;
    for (; f + U <= f1; f += U) {
        u32x4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) v[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + (int64_t)k * nq));
#pragma unroll
        for (int k = 0; k < U; ++k) {
            a0 += v[k].x;
            a1 += v[k].y;
            a2 += v[k].z;
            a3 += v[k].w;
        }
        p += (int64_t)U * nq;
    }
    for (; f < f1; ++f, p += nq) {
        const uint4 v = *p;
        a0 += v.x;
        a1 += v.y;
        a2 += v.z;
        a3 += v.w;
    }
    atomicAdd(&sums[4 * q + 0], a0);
    atomicAdd(&sums[4 * q + 1], a1);
    atomicAdd(&sums[4 * q + 2], a2);
    atomicAdd(&sums[4 * q + 3], a3);
}

// One pixel per lane (detector sizes whose pixel count is not a multiple of 4).
__global__ __launch_bounds__(256) void k_detsum1(const uint32_t* __restrict__ frames, int64_t nf, int np,
                                                 unsigned long long* __restrict__ sums) {
    const int px = blockIdx.x * 256 + threadIdx.x;
    if (px >= np) return;
    const int64_t f0 = (int64_t)blockIdx.y * kSumFrames;
    const int64_t f1 = f0 + kSumFrames < nf ? f0 + kSumFrames : nf;
    unsigned long long a = 0;
    for (int64_t f = f0; f < f1; ++f) a += frames[f * np + px];
    atomicAdd(&sums[px], a);
}

__global__ __launch_bounds__(256) void k_gather(const uint32_t* __restrict__ frames, int64_t np, int64_t nscan,
                                                const int* __restrict__ pix, int64_t nbf,
                                                uint32_t* __restrict__ out) {
    __shared__ uint32_t t[kTileS][kTileB + 1];
    const int tid = threadIdx.x;
#if SSB_GATHER_XCD
    // Workgroup id L -> (frame block x, BF tile y).  Consecutive ids go to the eight
    // XCDs in turn, so x = 8 (L / 8 / ny) + L % 8 keeps every BF tile of one frame block
    // on one XCD, dispatched one after another: the 128-byte lines two neighbouring BF
    // tiles share (a BF run rarely ends on a line boundary) are fetched into that XCD's
    // L2 once.
    const int64_t ny = (nbf + kTileB - 1) / kTileB;
    const int64_t L = blockIdx.x;
    const int64_t r = L / 8;
    const int64_t x = (r / ny) * 8 + L % 8, y = r % ny;
    if (x * kTileS >= nscan) return;
    const int64_t s0 = x * kTileS;
    const int64_t b0 = y * kTileB;
#else
    const int64_t s0 = (int64_t)blockIdx.x * kTileS;
    const int64_t b0 = (int64_t)blockIdx.y * kTileB;
#endif
    // every load of the thread in flight before the first LDS store
    constexpr int PER = kTileS * kTileB / 256;
    uint32_t v[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int e = tid + k * 256;
        const int sl = e / kTileB, bl = e % kTileB;
        const int64_t s = s0 + sl, b = b0 + bl;
        v[k] = (s < nscan && b < nbf) ? frames[s * np + pix[b]] : 0u;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int e = tid + k * 256;
        t[e / kTileB][e % kTileB] = v[k];
    }
    __syncthreads();
    for (int e = tid; e < kTileS * kTileB; e += 256) {
        const int bl = e / kTileS, sl = e % kTileS;
        const int64_t s = s0 + sl, b = b0 + bl;
        if (s < nscan && b < nbf) out[b * nscan + s] = t[sl][bl];
    }
}

// The probe-disk fit of ssb_fit_probe on the device, one workgroup: the mean and the
// variance of the mean pattern summed by one thread in pixel order (the host fit's order,
// so every double is the host's), then the mask's count and index sums and the disk's
// pixel counts, exact integers, split over the threads.  out[0..6] takes the fit in the
// order of ssb_probe_fit; out[7] is 1 when no pixel lies above the threshold; out[8], out[9]
// the mean and the summed squared deviations; out[10..] the mean pattern.
__global__ __launch_bounds__(256) void k_fit_probe(const unsigned long long* __restrict__ sums, double frames,
                                                   int det_n, double* __restrict__ out) {
    // every product rounded on its own, as in the host fit (no fused multiply-add)
#pragma clang fp contract(off)
    __shared__ double sh_thr;
    __shared__ long long red[3][256];
    const int tid = threadIdx.x;
    const int64_t np = (int64_t)det_n * det_n;
    // the mean pattern, one division per pixel, split over the threads (m: np doubles
    // after the 10 result slots); the workgroup barrier makes it visible to thread 0
    double* m = out + 10;
    for (int64_t p = tid; p < np; p += 256) m[p] = (double)sums[p] / frames;
    __syncthreads();
    if (tid == 0) {
        double mu = 0.0;
        for (int64_t p = 0; p < np; ++p) mu += m[p];
        mu /= (double)np;
        double var = 0.0;
        for (int64_t p = 0; p < np; ++p) {
            const double d = m[p] - mu;
            var += d * d;
        }
        // the correctly rounded square root (the host's): the hardware root's neighbour
        // whose square lies nearest the argument, residuals formed exactly by an FMA
        const double a = var / (double)np;
        double r = sqrt(a);
        const double lo = nextafter(r, 0.0), hi = nextafter(r, 2.0 * r + 1.0);
        if (fabs(fma(lo, lo, -a)) < fabs(fma(r, r, -a))) r = lo;
        if (fabs(fma(hi, hi, -a)) < fabs(fma(r, r, -a))) r = hi;
        out[8] = mu;
        out[9] = var;
        sh_thr = mu + r;
    }
    __syncthreads();
    const double thr = sh_thr;
    long long n = 0, si = 0, sj = 0;
    for (int64_t p = tid; p < np; p += 256)
        if (m[p] > thr) {
            ++n;
            si += p / det_n;
            sj += p % det_n;
        }
    red[0][tid] = n;
    red[1][tid] = si;
    red[2][tid] = sj;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w)
            for (int k = 0; k < 3; ++k) red[k][tid] += red[k][tid + w];
        __syncthreads();
    }
    const long long n_disk = red[0][0], ti = red[1][0], tj = red[2][0];
    __syncthreads();
    if (n_disk == 0) {
        if (tid == 0) out[7] = 1.0;
        return;
    }
    const double cy = (double)ti / (double)n_disk, cx = (double)tj / (double)n_disk;
    const double r2 = (double)n_disk / M_PI;
    // the BF rule: squares rounded on their own, then added
    long long nbf = 0, nz = 0;
    for (int64_t p = tid; p < np; p += 256) {
        const double di = (double)(p / det_n) - cy, dj = (double)(p % det_n) - cx;
        if (di * di + dj * dj <= r2) {
            if (sums[p] > 0) ++nbf;
            else ++nz;
        }
    }
    red[0][tid] = nbf;
    red[1][tid] = nz;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w)
            for (int k = 0; k < 2; ++k) red[k][tid] += red[k][tid + w];
        __syncthreads();
    }
    if (tid == 0) {
        out[0] = cy;
        out[1] = cx;
        out[2] = r2;
        out[3] = thr;
        out[4] = (double)n_disk;
        out[5] = (double)red[0][0];
        out[6] = (double)red[1][0];
        out[7] = 0.0;
    }
}

bool device_pointer(const void* p) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged;
}

int hip_error(hipError_t e, const char* what) {
    return ssb::set_error(e == hipErrorOutOfMemory ? SSB_ENOMEM : SSB_EDEVICE,
                          std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

extern "C" int ssb_detector_sum(const uint32_t* frames, int32_t scan_n, int32_t det_n, uint64_t* sums,
                                void* stream) {
    ssb::clear_error();
    if (!frames || !sums) return ssb::set_error(SSB_EINVAL, "null argument");
    if (scan_n < 1 || det_n < 1) return ssb::set_error(SSB_EINVAL, "scan_n and det_n must be positive");
    if (!device_pointer(frames) || !device_pointer(sums))
        return ssb::set_error(SSB_EINVAL, "frames and sums must be device pointers");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t nf = (int64_t)scan_n * scan_n;
    const int64_t np = (int64_t)det_n * det_n;
    if (np > (int64_t)1 << 30) return ssb::set_error(SSB_EINVAL, "detector too large");
    auto* out = reinterpret_cast<unsigned long long*>(sums);
    hipLaunchKernelGGL(k_zero_u64, dim3((unsigned)((np + 255) / 256)), dim3(256), 0, st, out, np);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "detector sum");
    const unsigned nblk = (unsigned)((nf + kSumFrames - 1) / kSumFrames);
    const bool quads = np % 4 == 0 && (reinterpret_cast<uintptr_t>(frames) & 15) == 0;
    if (quads) {
        const int nq = (int)(np / 4);
        hipLaunchKernelGGL(k_detsum4, dim3((unsigned)((nq + 255) / 256), nblk), dim3(256), 0, st,
                           reinterpret_cast<const uint4*>(frames), nf, nq, out);
    } else {
        hipLaunchKernelGGL(k_detsum1, dim3((unsigned)((np + 255) / 256), nblk), dim3(256), 0, st, frames, nf,
                           (int)np, out);
    }
    e = hipGetLastError();
    return e == hipSuccess ? SSB_OK : hip_error(e, "detector sum");
}

extern "C" int ssb_fit_probe(const uint64_t* sums, int32_t scan_n, int32_t det_n, ssb_probe_fit* out) {
    ssb::clear_error();
    if (!sums || !out) return ssb::set_error(SSB_EINVAL, "null argument");
    if (scan_n < 1 || det_n < 1) return ssb::set_error(SSB_EINVAL, "scan_n and det_n must be positive");
    const int64_t np = (int64_t)det_n * det_n;
    const double frames = (double)scan_n * (double)scan_n;
    // mean pattern, then its mean and population standard deviation over all pixels
    std::vector<double> m((size_t)np);
    double mu = 0.0;
    for (int64_t p = 0; p < np; ++p) {
        m[p] = (double)sums[p] / frames;
        mu += m[p];
    }
    mu /= (double)np;
    double var = 0.0;
    for (int64_t p = 0; p < np; ++p) {
        const double d = m[p] - mu;
        var += d * d;
    }
    const double thr = mu + std::sqrt(var / (double)np);
    // mask centroid (exact integer sums of the indices) and area radius
    int64_t n_disk = 0, si = 0, sj = 0;
    for (int i = 0; i < det_n; ++i)
        for (int j = 0; j < det_n; ++j)
            if (m[(int64_t)i * det_n + j] > thr) {
                ++n_disk;
                si += i;
                sj += j;
            }
    if (n_disk == 0) return ssb::set_error(SSB_EINVAL, "no detector pixel above the probe threshold");
    ssb_probe_fit f;
    f.det_cy = (double)si / (double)n_disk;
    f.det_cx = (double)sj / (double)n_disk;
    f.bf_r2 = (double)n_disk / M_PI;
    f.threshold = thr;
    f.n_disk = n_disk;
    f.n_bf = 0;
    f.n_zero = 0;
    ssb_geometry g{};
    g.det_n = det_n;
    g.det_cy = f.det_cy;
    g.det_cx = f.det_cx;
    g.bf_r2 = f.bf_r2;
    for (int i = 0; i < det_n; ++i)
        for (int j = 0; j < det_n; ++j)
            if (ssb::in_bf_disk(&g, i, j)) {
                if (sums[(int64_t)i * det_n + j] > 0) ++f.n_bf;
                else ++f.n_zero;
            }
    *out = f;
    return SSB_OK;
}

extern "C" int ssb_fit_probe_device(const uint64_t* sums, int32_t scan_n, int32_t det_n, ssb_probe_fit* out,
                                    void* stream) {
    ssb::clear_error();
    if (!sums || !out) return ssb::set_error(SSB_EINVAL, "null argument");
    if (scan_n < 1 || det_n < 1) return ssb::set_error(SSB_EINVAL, "scan_n and det_n must be positive");
    if (!device_pointer(sums)) return ssb::set_error(SSB_EINVAL, "sums must be a device pointer");
    hipStream_t st = static_cast<hipStream_t>(stream);
    double* dev = nullptr;
    hipError_t e = hipMalloc(&dev, (10 + (size_t)det_n * det_n) * sizeof(double));
    if (e != hipSuccess) return ssb::set_error(SSB_ENOMEM, std::string("probe fit result: ") + hipGetErrorString(e));
    double res[10];
    hipLaunchKernelGGL(k_fit_probe, dim3(1), dim3(256), 0, st, reinterpret_cast<const unsigned long long*>(sums),
                       (double)scan_n * (double)scan_n, det_n, dev);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpyAsync(res, dev, sizeof(res), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    (void)hipFree(dev);
    if (e != hipSuccess) return ssb::set_error(SSB_EDEVICE, std::string("probe fit: ") + hipGetErrorString(e));
    if (res[7] != 0.0) return ssb::set_error(SSB_EINVAL, "no detector pixel above the probe threshold");
    ssb_probe_fit f;
    f.det_cy = res[0];
    f.det_cx = res[1];
    f.bf_r2 = res[2];
    f.threshold = res[3];
    f.n_disk = (int64_t)res[4];
    f.n_bf = (int64_t)res[5];
    f.n_zero = (int64_t)res[6];
    *out = f;
    return SSB_OK;
}

extern "C" int ssb_gather_bf(const uint32_t* frames, const ssb_geometry* g, uint32_t* counts, int64_t n_bf,
                             void* stream) {
    ssb::clear_error();
    if (!frames || !g || !counts) return ssb::set_error(SSB_EINVAL, "null argument");
    if (g->scan_n < 1 || g->det_n < 1) return ssb::set_error(SSB_EINVAL, "scan_n and det_n must be positive");
    if (!std::isfinite(g->bf_r2) || !std::isfinite(g->det_cy) || !std::isfinite(g->det_cx))
        return ssb::set_error(SSB_EINVAL, "non-finite BF disk");
    if (!device_pointer(frames) || !device_pointer(counts))
        return ssb::set_error(SSB_EINVAL, "frames and counts must be device pointers");
    std::vector<int> pix;
    for (int i = 0; i < g->det_n; ++i)
        for (int j = 0; j < g->det_n; ++j)
            if (ssb::in_bf_disk(g, i, j)) pix.push_back(i * g->det_n + j);
    if ((int64_t)pix.size() != n_bf)
        return ssb::set_error(SSB_ESHAPE, "n_bf = " + std::to_string(n_bf) + " but the BF rule selects " +
                                              std::to_string(pix.size()) + " detector pixels");
    if (n_bf == 0) return SSB_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int* dpix = nullptr;
    hipError_t e = hipMalloc(&dpix, pix.size() * sizeof(int));
    if (e != hipSuccess) return hip_error(e, "gather allocation");
    const int64_t nscan = (int64_t)g->scan_n * g->scan_n;
    const int64_t np = (int64_t)g->det_n * g->det_n;
    if ((e = hipMemcpyAsync(dpix, pix.data(), pix.size() * sizeof(int), hipMemcpyHostToDevice, st)) == hipSuccess) {
#if SSB_GATHER_XCD
        const int64_t nx8 = ((nscan + kTileS - 1) / kTileS + 7) / 8 * 8;
        const int64_t nblk = nx8 * ((n_bf + kTileB - 1) / kTileB);
        if (nblk > 0x7fffffff) {
            (void)hipStreamSynchronize(st);
            (void)hipFree(dpix);
            return ssb::set_error(SSB_EINVAL, "gather grid too large");
        }
        const dim3 grid((unsigned)nblk);
#else
        const dim3 grid((unsigned)((nscan + kTileS - 1) / kTileS), (unsigned)((n_bf + kTileB - 1) / kTileB));
#endif
        hipLaunchKernelGGL(k_gather, grid, dim3(256), 0, st, frames, np, nscan, dpix, n_bf, counts);
        e = hipGetLastError();
    }
    // the pixel list lives for this call only: wait for the kernel before freeing it
    const hipError_t e2 = hipStreamSynchronize(st);
    (void)hipFree(dpix);
    if (e != hipSuccess) return hip_error(e, "gather");
    if (e2 != hipSuccess) return hip_error(e2, "gather");
    return SSB_OK;
}
