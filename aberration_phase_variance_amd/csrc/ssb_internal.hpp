// Internal declarations shared by the host layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssb {

// Reduction group: S1 partial images are summed over this many consecutive BF
// pixels in float, then added group by group, in order, in double.  Fixed so that
// every result is independent of chunking and batch size.
constexpr int kGroupBF = 32;

// Per-trial aberration constants: chi(k)/(2 pi) = k^T M k with k in detector
// pixels (revolutions), M = (lambda dk^2 / 2) [[C10 + C12 c, C12 s], [C12 s, C10 - C12 c]],
// c = cos 2 phi12, s = sin 2 phi12.
struct TrialConst {
    double mxx, mxy, myy, pad;
};

// Geometry as the kernels see it.
// Half-plane layout of the spectrum cache, the per-trial chi_q table, the column
// results and the object's plane: the columns v < N/2 in tiles of kTileW,
// [tile][row u][kTileW] (one tile of one plane is N * kTileW contiguous complex
// values); the Nyquist column v = N/2 is a separate [N] array.
constexpr int kTileW = 8;
__host__ __device__ constexpr int64_t tm_index(int n, int u, int v) {
    return ((int64_t)(v / kTileW) * n + u) * kTileW + (v % kTileW);
}

struct GeomDev {
    int n;            // N
    int h;            // N / 2
    double s;         // q step (detector pixels per scan-frequency index)
    double crot, srot;
    // q(u', v) = (qvx v + qux u', qvy v + quy u') detector pixels, u' the signed row index
    double qvx, qux, qvy, quy;
    double inv_w;     // 1 / w
    double ra;        // aperture radius (pixels)
    double ra2;       // ra^2
    double w;         // edge width (pixels)
    double lo2;       // (ra - w/2)^2, or -1 when ra < w/2 (no flat top)
    double hi2;       // (ra + w/2)^2
};

// Trial constants passed to the device by value (kernel arguments), kTrialBlock at a
// time: no host staging buffer and no copy engine.
constexpr int kTrialBlock = 16;
struct TrialBlock {
    TrialConst t[kTrialBlock];
};
hipError_t launch_set_trials(const TrialBlock& blk, int count, TrialConst* dev, hipStream_t st);

// The no-allocation scratch (ssb_loss_noalloc): a file-scope device array of
// scratch_bytes() bytes, one per device, kept until the process ends.  scratch_address
// returns its device address on the current device (looked up once per device).
size_t scratch_bytes();
hipError_t scratch_address(void** out);

// Launchers (defined in ssb_kernels.hip).  All return the hipError_t of the
// launch; grids are chunked internally to keep every dimension in range.
// FFT twiddle tables (inverse and forward sign, twiddle_count(n) entries each),
// filled once per handle; the transforms below read their twiddles from them
// (pass 1 computes its own: measured faster there).
int twiddle_count(int n);
hipError_t launch_twiddles(int n, float2* tw_inv, float2* tw_fwd, hipStream_t st);
hipError_t launch_g_rows(int n, const uint32_t* counts, int64_t nbf, float2* gm, float2* gn,
                         unsigned long long* bfsum, const float2* tw_fwd, hipStream_t st);
hipError_t launch_g_cols(int n, float2* gm, float2* gn, int64_t nbf, const float2* tw_fwd, hipStream_t st);

// Pass 1: correction + column inverse transforms of the BF chunk [bf0, bf0 + cb)
// for n_trials trials into the intermediate (main [t][cap][N][H], nyq [t][cap][N]).
// exp(2 pi i q^T M q) over the half plane for each trial: main [t][N][N/2], nyq [t][N].
hipError_t launch_chiq(int n, const TrialConst* tc, int n_trials, GeomDev geo, float2* chm, float2* chn,
                       hipStream_t st);
hipError_t launch_pass1(int n, const float2* gm, const float2* gn, const float2* chm, const float2* chn,
                        const double2* kb, const uint4* sup, const int* vend, const TrialConst* tc, int n_trials,
                        GeomDev geo, int64_t bf0, int cb, int cap, float2* im, float2* in, hipStream_t st);
// Pass 2: row transforms, atan2 and moments, one partial per 32-BF group.  With part_obj
// (scan sizes and variants where pass2_obj_sizes holds; at 1,024 points the full plane's
// sums would not fit the row pass's registers) it also writes each group's object sums:
// [t][g] blocks of obj_sum_count(n, fp) floats (N * N sums of Im O_b, then the sums of
// Re O_b: 2 N per row and column parity for the half plane, N * N for the full plane).
constexpr bool pass2_obj_sizes(int n, bool fp) { return fp ? n <= 512 : n <= 1024; }
constexpr int64_t obj_sum_count(int n, bool fp) { return (int64_t)n * n + (fp ? (int64_t)n * n : 2 * n); }
hipError_t launch_pass2(int n, const float2* im, const float2* in, int cap, const uint8_t* active,
                        const int* vend, int64_t bf0, int cb, int n_trials, double dc, float* part_s1,
                        double* part_s2, int gcap, const float2* tw_inv, const float2* na, const float2* nb,
                        float* part_obj, hipStream_t st);
// acc[t][i] (+)= sum over groups g < ng, in order, of part_obj[t][g][i] (double), i < obj_sum_count(n, fp)
hipError_t launch_accum_obj(int n, bool fp, const float* part_obj, int gcap, int ng, int n_trials, double* acc,
                            bool first, hipStream_t st);
// Phase (and psi, when not null) of the object summed over all BF pixels from one trial's
// accumulated row-pass sums: Re = acc's Re sum + re_extra, Im = acc's pixel sum;
// psi = (Re, Im) * scale.
hipError_t launch_obj_from_sums(int n, bool fp, const double* acc, double re_extra, double scale, float* phase,
                                float2* psi, hipStream_t st);
// Full-plane variant: the Nyquist-line terms A, B ([t][cap][N] each) of the chunk's
// BF pixels (pass 2 adds them when na is not null).
hipError_t launch_nyq_lines(int n, const float2* gm, const float2* gn, const double2* kb, const uint8_t* active,
                            const TrialConst* tc, int n_trials, GeomDev geo, int64_t bf0, int cb, int cap, float2* na,
                            float2* nb, const float2* tw_inv, hipStream_t st);
// Correction support per (BF, column) from the geometry: sup [n_bf][N/2+1] of four
// packed (lo, len) row intervals (minus/plus aperture, nonzero weight / flat top),
// vend [n_bf] = 1 + the last column with any support (0 for an inactive BF), and
// nsup [n_bf] = nonzero-transfer entries per BF.
hipError_t launch_support(int n, const double2* kb, const uint8_t* active, GeomDev geo, int64_t nbf, uint4* sup,
                          int* vend, int* nsup, hipStream_t st);
// Columns per pass-1 tile (pass 1 writes whole tiles below vend).
int pass1_tile(int n);
int pass2_row_blocks(int n);
hipError_t launch_accum(int n, const float* part_s1, const double* part_s2, int gcap, int ng,
                        int n_trials, double* s1run, double* s2run, bool first, hipStream_t st);
hipError_t launch_fill(double* p, int64_t count, hipStream_t st);
int loss_blocks();
hipError_t launch_loss(int n, const double* s1run, const double* s2run, int n_trials, double n_bf,
                       double* lpart, double* loss, float* mean_phase, hipStream_t st);
// Object: sum of corrected spectra over all BF, then one 2-D inverse transform.
int obj_segments(int64_t nbf);
hipError_t launch_obj_sum(int n, const float2* gm, const float2* gn, const double2* kb, const uint4* sup,
                          const int* vend, TrialConst tc, GeomDev geo, int64_t nbf, float2* part, int nseg,
                          hipStream_t st);
hipError_t launch_obj_reduce(int n, const float2* part, int nseg, float2* pm, float2* pn,
                             hipStream_t st);
hipError_t launch_obj_cols(int n, float2* pm, float2* pn, const float2* tw_inv, hipStream_t st);
hipError_t launch_obj_rows(int n, const float2* pm, const float2* pn, double dcsum, double scale, float* phase,
                           float2* psi, const float2* tw_inv, const float2* nab, hipStream_t st);
// Full-plane object: BF sums of the Nyquist-line terms, nab = [A | B] (2N complex);
// part holds nseg x 2N double2 partials.
hipError_t launch_obj_nyq(int n, const float2* gm, const float2* gn, const double2* kb, const int* vend,
                          TrialConst tc, GeomDev geo, int64_t nbf, double2* part, int nseg, float2* nab,
                          const float2* tw_inv, hipStream_t st);

}  // namespace ssb
