/*
 * ssb.h - C ABI of the MI355X (gfx950) single-side-band (SSB) phase-variance library.
 *
 * The objective follows the quantem.gpu maintainer pages "SSB performance notes"
 * and "Later SSB performance checkpoints".  For every bright-field (BF) detector
 * pixel b the cached scan spectrum G_b (a forward real 2-D DFT of that pixel's
 * scan counts, Hermitian half plane) is multiplied by the SSB aberration
 * correction T_b, extended to the full plane by C(-q) = -conj(C(q)), inverse
 * transformed (a 2-D inverse DFT done as column then row transforms), its phase
 * taken with atan2, and the per-scan-pixel phase moments are reduced over all BF
 * pixels to the phase-variance loss
 *
 *     L = S2 / (n_bf N^2) - (1/N^2) sum_px (S1 / n_bf)^2,
 *     S1(px) = sum_b phi_b(px),  S2 = sum_b sum_px phi_b(px)^2.
 *
 * The correction is T = conj(Gamma)/|Gamma| (0 where Gamma = 0) with
 * Gamma(q) = conj(A(k)) A(k - q) - A(k) conj(A(k + q)) and the probe
 * A(k) = a(k) exp(-i chi(k)): soft aperture a(k) = clip((R_a - |k|)/w + 1/2, 0, 1),
 * chi = pi lambda |k|^2 C10 + pi lambda C12 ((kx^2 - ky^2) cos 2phi12 + 2 kx ky sin 2phi12).
 * Notes page, sections "MPS zero-transfer q-space checkpoint" (both shifted
 * apertures, zero transfer), "MPS dead inactive-write elimination checkpoint"
 * (v8 follow-ups: two shifted-phase sincos, gamma normalization) and
 * "Automatic whole-probe sparse-storage checkpoint" (the anti-Hermitian relation,
 * the DC value).  The q = 0 term is the scalar DC = mean over BF of the scan sum.
 *
 * Conventions.  Detector pixel (i, j) is row i, column j; k_b = (j - cx, i - cy)
 * in pixels.  The BF set is every detector pixel with (i-cy)^2 + (j-cx)^2 <= bf_r2,
 * in row-major order; counts are passed in that order.  Scan frequency (u, v) of
 * the half plane (u in [0, N), v in [0, N/2]) is q = Rot(rho) * s * (v, u') in
 * detector pixels, u' = u for u < N/2 and u - N otherwise; v = N/2 is +N/2.
 *
 * Errors.  Every int-returning call returns SSB_OK (0) or a negative code and
 * sets a thread-local message readable with ssb_last_error().  Nothing throws
 * across this boundary.  A handle is not safe for concurrent calls; different
 * handles are independent.  All device work is issued on the caller's HIP stream
 * (NULL = the default stream).  Every call that returns host results
 * synchronizes that stream before returning.
 */
#ifndef SSB_H
#define SSB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    SSB_OK = 0,
    SSB_EINVAL = -1,   /* null pointer, non-finite or out-of-range argument, bad handle */
    SSB_ESHAPE = -2,   /* n_bf does not match the BF rule, or a range is outside [0, n_bf] */
    SSB_ENOMEM = -3,   /* a device allocation failed */
    SSB_EDEVICE = -4   /* a HIP runtime error; the message carries hipGetErrorString */
};

/* Workload geometry.  Lengths are in detector pixels unless stated otherwise.
 * The scan sampling enters as q_step_px, the detector pixels one scan-frequency
 * index spans, 1/(N * scan step * dk); a caller holding the scan step in Angstrom
 * forms it.  Passing the ratio itself keeps q on an exact lattice when it is dyadic
 * (e.g. D/N), so every support and flat-top decision of the correction is exact and
 * reproducible; deriving it from a step in Angstrom would round it and turn the
 * lattice's exact ties with the aperture edge into near ties.  bf_r2 is a double
 * because the probe-disk fit (ssb_fit_probe) gives a non-integer radius squared. */
typedef struct ssb_geometry {
    int32_t scan_n;        /* N: scan side, a power of two in [32, 1024] */
    int32_t det_n;         /* D: detector side, > 0 */
    double bf_r2;          /* BF disk radius squared (pixels^2), >= 0 */
    double det_cy;         /* detector center row (pixels) */
    double det_cx;         /* detector center column (pixels) */
    double q_step_px;      /* detector pixels per scan-frequency index: 1/(N * scan step * dk), > 0 */
    double dk;             /* detector sampling in 1/Angstrom per pixel, > 0 */
    double wavelength_A;   /* electron wavelength in Angstrom, > 0 */
    double alpha_rad;      /* probe semi-angle in rad, > 0; aperture radius R_a = alpha/(lambda dk) px */
    double rotation_rad;   /* scan-to-detector rotation rho, finite */
    double edge_px;        /* width w of the soft aperture edge (pixels), > 0 */
} ssb_geometry;

typedef struct ssb_info {
    int64_t n_bf;          /* logical BF pixels (all count in the normalization) */
    int64_t n_active_bf;   /* BF pixels with a(k_b) > 0 */
    int32_t scan_n;
    int32_t det_n;
    int64_t spectrum_bytes;/* device bytes of the cached half-plane spectra */
    double dc;             /* DC value: mean over BF of the exact integer scan sums */
    int64_t chunk_bf;      /* current cap on BF pixels per intermediate chunk */
    int64_t support_entries; /* half-plane entries with nonzero transfer, summed over BF (q = 0 aside) */
    int64_t columns_written; /* column results (N values each) the column pass writes per trial, all BF */
    int64_t columns_read;    /* column results the row pass reads per trial, all BF (zero columns skipped) */
    int32_t variant;         /* SSB_VARIANT_HALF_PLANE or SSB_VARIANT_FULL_PLANE (ssb_set_variant) */
    int32_t pad;
    int64_t workspace_bytes; /* device workspace the handle holds (loss + object) */
    int32_t reserved_trials; /* loss calls with at most this many trials allocate nothing (ssb_reserve) */
    int32_t pad2;
} ssb_info;

typedef struct ssb_handle ssb_handle;

/*
 * ssb_prepare: validate the geometry, select the BF pixels, and build the cached
 * spectra G_b = rfft2(counts_b) for every BF pixel on the device (complex64,
 * BF-major).  Checkpoints page, "fftA intermediate and M5 hardware floor"
 * (complex64 Hermitian G cache) and Notes page, "BF-major G_qk materialization".
 *
 *   g        host pointer to the geometry (copied).
 *   counts   DEVICE pointer, uint32 [n_bf][N][N], BF-major in BF order, scan
 *            row-major.  Counts up to 2^24 convert to float exactly.  Only read;
 *            the caller may free it once this call returns.
 *   n_bf     must equal the number of detector pixels selected by the BF rule.
 *   stream   hipStream_t or NULL.
 *   out      receives a new handle that owns all device memory it uses.
 * Errors: SSB_EINVAL (null, non-finite or out-of-range geometry, counts not a
 * device pointer), SSB_ESHAPE (n_bf mismatch), SSB_ENOMEM, SSB_EDEVICE.
 */
int ssb_prepare(const ssb_geometry* g, const uint32_t* counts, int64_t n_bf,
                void* stream, ssb_handle** out);

/*
 * ssb_loss: phase-variance loss for n_trials aberration sets.  One exact
 * evaluation covers every BF pixel and every scan pixel (Checkpoints page,
 * "2026-09-11 full-aperture Apple M5 floor checkpoint": all 8,937 BF terms of the
 * 512 x 512 scan, no crop or BF reduction), reduced from the phase-sum image and
 * the squared-phase partials (Notes page, "Standard-only CUDA native 512
 * calibration"); candidates of a batch share the spectrum fetch and keep their own
 * correction, transforms and loss (Notes page, "MPS fused candidate-pair
 * checkpoint").
 *   params      HOST float [n_trials][3] = {C10 nm, C12 nm, phi12 rad}; each value
 *               is taken as given in float32 (the evaluation's exact input; Notes
 *               page, "MPS wider exact-simplex checkpoint").
 *   losses      HOST double [n_trials], written on success.
 *   mean_phase  optional DEVICE float [N][N] receiving S1/n_bf of trial 0, or NULL.
 * Each trial's loss is bitwise independent of n_trials, of its position in the
 * batch and of the chunk size.  Synchronizes the stream before returning.
 * Allocates nothing when n_trials <= the reserved trial count (1 after
 * ssb_prepare; see ssb_reserve); a larger batch grows the handle's workspace once.
 * Errors: SSB_EINVAL (null handle/params/losses, n_trials outside [1, 65535],
 * non-finite parameter), SSB_ENOMEM, SSB_EDEVICE.
 */
int ssb_loss(ssb_handle* h, const float* params, int32_t n_trials, double* losses,
             float* mean_phase, void* stream);

/*
 * ssb_loss_noalloc: ssb_loss for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, results and errors as ssb_loss, and the same kernels, but every
 * per-call buffer lives in a fixed scratch array of 256 MiB that each device holds
 * from the library's load until the process ends; no hipMalloc, hipFree or other
 * allocating call is made, on the device or the host (trial constants reach the
 * device as kernel arguments).  The BF chunk is the largest multiple of 32 pixels
 * whose buffers fit the scratch (results are bitwise those of ssb_loss, which do not
 * depend on the chunk); a call whose trials do not fit even with 32-BF chunks is
 * rejected with SSB_EINVAL (at N = 512 one call takes up to 7 trials, at N = 1024
 * one).  Every handle on a device shares that device's scratch, which keeps the
 * last call's contents: calls that overlap on one device race, so issue them on
 * one stream or serialize them.  Call with the handle's device current.
 * Synchronizes the stream before returning.
 */
int ssb_loss_noalloc(ssb_handle* h, const float* params, int32_t n_trials, double* losses,
                     float* mean_phase, void* stream);

/*
 * ssb_reserve: size the handle's device workspace, host staging and pinned host
 * landing area for the losses (at least 16 trials) for loss calls of up to max_trials
 * trials (any BF range, either variant, any chunk cap), so that such calls, and
 * ssb_moments, ssb_object and ssb_loss_object, allocate nothing afterwards.
 * ssb_prepare reserves one trial (and the object sums ssb_loss_object uses).  Reservations only grow.  Errors: SSB_EINVAL
 * (bad handle, max_trials outside [1, 65535]), SSB_ENOMEM, SSB_EDEVICE.
 */
int ssb_reserve(ssb_handle* h, int32_t max_trials);

/*
 * ssb_moments: phase moments of one trial over the BF range [bf_begin, bf_end)
 * (one device's share when the BF set is split).  S1 = sum of phi_b per scan
 * pixel and S2 = sum of phi_b^2 over the range, the pieces of the loss above.
 *   params3  HOST float[3].
 *   s1       DEVICE double [N][N], overwritten.
 *   s2       HOST double, written on success.
 * Synchronizes the stream.  Errors: SSB_EINVAL, SSB_ESHAPE (bad range),
 * SSB_ENOMEM, SSB_EDEVICE.
 */
int ssb_moments(ssb_handle* h, const float* params3, int64_t bf_begin, int64_t bf_end,
                double* s1, double* s2, void* stream);

/*
 * ssb_object: phase-of-mean object redraw.  psi = ifft2(full plane of
 * mean_b C_b) and phase = atan2(Im psi, Re psi) (Notes page, "Standard-only CUDA
 * native 512 calibration": the public output is the phase of the mean).
 *   params3  HOST float[3].
 *   phase    DEVICE float [N][N].
 *   psi      optional DEVICE complex64 [N][N] (interleaved re, im) or NULL.
 * Asynchronous on the stream; allocates nothing (its workspace is reserved by
 * ssb_prepare).  Errors: SSB_EINVAL, SSB_EDEVICE.
 */
int ssb_object(ssb_handle* h, const float* params3, float* phase, float* psi, void* stream);

/*
 * ssb_loss_object: one trial's loss and its phase-of-mean object from one pass over
 * the cached spectra (the loss of ssb_loss and the object of ssb_object, Notes page,
 * "Standard-only CUDA native 512 calibration").  The object transform is linear, so
 * the mean object equals the mean of the per-BF objects O_b that the loss already
 * forms before taking their phases: the row pass also sums O_b over each 32-BF group,
 * and the sums are added in double in group order.  The loss is bitwise that of
 * ssb_loss; phase and psi agree with ssb_object to float rounding (the two sum in
 * different orders).  Either variant; only the full-plane variant of 1,024-point scans
 * runs ssb_loss and then ssb_object (the returned results are those two calls').
 *   params3  HOST float[3].
 *   loss     HOST double, written on success.
 *   phase    DEVICE float [N][N].
 *   psi      optional DEVICE complex64 [N][N] (interleaved re, im) or NULL.
 * Synchronizes the stream before returning.  Allocates nothing (ssb_prepare reserves
 * its buffers).  Errors: SSB_EINVAL (null handle/params/loss/phase, non-finite
 * parameter), SSB_ENOMEM, SSB_EDEVICE.
 */
int ssb_loss_object(ssb_handle* h, const float* params3, double* loss, float* phase, float* psi,
                    void* stream);

/*
 * ssb_spectrum: copy the cached spectrum of BF pixel bf as complex64
 * [N][N/2 + 1] (interleaved re, im, logical half-plane order) into the DEVICE
 * buffer out.  Asynchronous.  Errors: SSB_EINVAL, SSB_ESHAPE, SSB_EDEVICE.
 */
int ssb_spectrum(const ssb_handle* h, int64_t bf, float* out, void* stream);

/*
 * ssb_set_chunk: cap the BF pixels whose intermediate is resident at once
 * (rounded up to the fixed 32-BF reduction group; also bounded by the library's
 * 48 GiB intermediate budget; 0 restores the budget-only choice).  Results do not
 * depend on it (bitwise); it bounds workspace memory.
 */
int ssb_set_chunk(ssb_handle* h, int64_t chunk_bf);

/*
 * ssb_set_variant: which corrected plane ssb_loss, ssb_moments and ssb_object
 * transform (per handle; default SSB_VARIANT_HALF_PLANE).
 *
 *   SSB_VARIANT_HALF_PLANE  the corrected half plane v = 0 .. N/2, extended to the
 *       full plane by C(-q) = -conj(C(q)) (columns 0 and N/2 as computed, N/2 taken
 *       as +N/2).  Notes page, "Automatic whole-probe sparse-storage checkpoint"
 *       (the anti-Hermitian relation and its 257-row intermediate).
 *   SSB_VARIANT_FULL_PLANE  every entry of the N x N plane corrected on its own,
 *       index N/2 taken as -N/2 on both axes; the same passage's accepted evaluator.
 *       It differs from the half plane only on the Nyquist column and row, which
 *       the library adds to each BF pixel's object as two line terms.
 *
 * Errors: SSB_EINVAL (bad handle or variant).
 */
enum { SSB_VARIANT_HALF_PLANE = 0, SSB_VARIANT_FULL_PLANE = 1 };
int ssb_set_variant(ssb_handle* h, int32_t variant);

/*
 * Stage profiling.  When enabled, the library records a pair of HIP events on
 * the caller's stream around each stage's kernel launches and accumulates their
 * elapsed times (and the BF-plane x trial units each stage processed).
 */
enum {
    SSB_STAGE_PASS1 = 0,     /* correction + column inverse transforms */
    SSB_STAGE_PASS2 = 1,     /* row inverse transforms + atan2 + phase moments */
    SSB_STAGE_REDUCE = 2,    /* clears, ordered S1/S2 accumulation, loss reduction */
    SSB_STAGE_OBJ_SUM = 3,   /* object: corrected-spectrum sum over all BF */
    SSB_STAGE_OBJ_FFT = 4,   /* object: partial reduction, 2-D inverse transform, phase */
    SSB_NUM_STAGES = 5
};

typedef struct ssb_profile_data {
    double ms[SSB_NUM_STAGES];         /* accumulated event time per stage */
    int64_t launches[SSB_NUM_STAGES];  /* timed stage invocations */
    int64_t units[SSB_NUM_STAGES];     /* active BF planes x trials processed (passes 1-2, object sum) */
} ssb_profile_data;

/*
 * ssb_profile: mode 1 enables profiling and clears the totals, mode 0 disables it,
 * mode 2 leaves the state unchanged.  If out is not NULL it receives the totals
 * after waiting for every recorded event.  Errors: SSB_EINVAL, SSB_EDEVICE.
 */
int ssb_profile(ssb_handle* h, int mode, ssb_profile_data* out);

/*
 * Detector side, before ssb_prepare: the mean diffraction pattern as an exact
 * integer detector sum over every scan frame, the probe-disk fit that selects the
 * BF pixels, and the gather of those pixels into BF-major counts (Notes page,
 * sections "Cross-backend and native-size validation notes": mean diffraction
 * pattern, mean-plus-standard-deviation probe fit and disk crop on the device;
 * "Automatic full-probe MPS optimizer": the fitted center and radius select the
 * positive-count pixels of the disk; "Automatic-probe detector-sum reduction":
 * exact integer sums from frame-block partials).
 *
 * Frames are DEVICE uint32 [scan_n * scan_n][det_n * det_n]: frame y * scan_n + x
 * is the whole detector at scan position (y, x), row-major (row i, column j).
 */

/*
 * ssb_detector_sum: sums[p] = sum over all frames of frame[p], exact (uint64).
 *   frames  DEVICE uint32 frames as above (only read).
 *   sums    DEVICE uint64 [det_n * det_n], overwritten.
 * Asynchronous on the stream.  Errors: SSB_EINVAL (null or host pointer,
 * scan_n < 1 or det_n < 1), SSB_EDEVICE.
 */
int ssb_detector_sum(const uint32_t* frames, int32_t scan_n, int32_t det_n, uint64_t* sums, void* stream);

typedef struct ssb_probe_fit {
    double det_cy, det_cx;  /* disk center: unweighted centroid of the mask (pixels) */
    double bf_r2;           /* disk radius squared: mask area / pi (pixels^2) */
    double threshold;       /* mean + population std of the mean pattern over all pixels */
    int64_t n_disk;         /* mask pixels: mean pattern strictly above the threshold */
    int64_t n_bf;           /* pixels with (i-cy)^2 + (j-cx)^2 <= bf_r2 and a positive sum */
    int64_t n_zero;         /* pixels inside that disk with a zero sum (not BF) */
} ssb_probe_fit;

/*
 * ssb_fit_probe: the probe-disk fit on the host from HOST sums [det_n * det_n]
 * (ssb_detector_sum's output copied back); the mean pattern is sums / scan_n^2.
 * The BF set is the disk rule of ssb_geometry with (det_cy, det_cx, bf_r2) from
 * the fit when n_zero is 0 (then n_bf is what ssb_prepare expects).
 * Errors: SSB_EINVAL (null, sizes < 1, no pixel above the threshold).
 */
int ssb_fit_probe(const uint64_t* sums, int32_t scan_n, int32_t det_n, ssb_probe_fit* out);

/*
 * ssb_fit_probe_device: the same fit from DEVICE sums [det_n * det_n] (ssb_detector_sum's
 * output, left on the device); out is a HOST struct.  One workgroup forms the mean and the
 * variance of the mean pattern in pixel order, as the host fit does, so every field is
 * bitwise ssb_fit_probe's on the same sums; the mask and disk counts are exact integers.
 * Allocates and frees a result buffer of 8 (det_n^2 + 10) bytes; synchronizes the stream.  Errors: SSB_EINVAL
 * (null, sizes < 1, sums not a device pointer, no pixel above the threshold), SSB_ENOMEM,
 * SSB_EDEVICE.
 */
int ssb_fit_probe_device(const uint64_t* sums, int32_t scan_n, int32_t det_n, ssb_probe_fit* out,
                         void* stream);

/*
 * ssb_gather_bf: BF-major counts [n_bf][scan_n][scan_n] (the layout ssb_prepare
 * takes, BF pixels in row-major detector order by the geometry's disk rule) from
 * the DEVICE frames.  counts is a DEVICE buffer, overwritten.  Only scan_n, det_n,
 * det_cy, det_cx and bf_r2 of the geometry are used.  Synchronizes the stream
 * (a temporary device list of the BF pixels is freed before returning).
 * Errors: SSB_EINVAL (null or host pointer, bad geometry), SSB_ESHAPE (n_bf differs
 * from the rule's count), SSB_ENOMEM, SSB_EDEVICE.
 */
int ssb_gather_bf(const uint32_t* frames, const ssb_geometry* g, uint32_t* counts, int64_t n_bf, void* stream);

/*
 * Aberration fit: a batch of trial parameter sets, then Nelder-Mead refinement of
 * the exact loss from the batch's best trial (Notes page, "MPS wider
 * exact-simplex checkpoint" and "Final exact MPS optimizer handoff": axis steps of
 * 5% of each starting value with floors of 2 nm on C12 and 0.04 rad on phi12,
 * rounded to two decimals; stop when the simplex's loss spread is at most fatol
 * and its coordinate spread at most xatol; a request whose float32 inputs equal an
 * earlier evaluation's reuses that loss instead of evaluating again).
 *
 * The simplex moves are the standard ones: reflection 1, expansion 2, outside and
 * inside contraction 1/2, shrink 1/2 towards the best vertex; vertices are kept
 * sorted by loss (ties keep their order).
 */
typedef struct ssb_fit_options {
    double fatol;          /* loss spread tolerance (default 3e-6) */
    double xatol;          /* coordinate spread tolerance, max over the three coordinates (default 0.1) */
    double step_frac;      /* initial axis step as a fraction of the start value (default 0.05) */
    double step_floor[3];  /* minimum |step| per axis: C10 nm, C12 nm, phi12 rad (default 0.01, 2.0, 0.04) */
    int32_t max_evals;     /* cap on physical loss evaluations in the refinement, 0 = none */
    int32_t max_iter;      /* cap on simplex iterations, 0 = 600 */
} ssb_fit_options;

typedef struct ssb_fit_result {
    double best[3];        /* refined (C10 nm, C12 nm, phi12 rad) as the simplex holds them */
    double loss;           /* exact loss at float32(best) */
    int32_t batch_best;    /* index of the batch trial the refinement started from (first minimum) */
    int32_t requests;      /* loss requests made by the simplex */
    int32_t evals;         /* physical evaluations among them (the rest were memoized) */
    int32_t iterations;    /* simplex iterations */
    int32_t converged;     /* 1 if the tolerances were met, 0 if a cap stopped it */
    int32_t pad;
    double batch_loss;     /* loss of that batch trial */
} ssb_fit_result;

/* Loss of one float32 parameter triple, for ssb_nelder_mead.  Returns the loss;
 * a non-finite value aborts the minimization with SSB_EINVAL. */
typedef double (*ssb_objective)(const float* params3, void* ctx);

/*
 * ssb_nelder_mead: the refinement above on any objective (host only).
 *   x0      HOST double[3] start.
 *   opt     options (NULL = defaults).
 *   f, ctx  objective; called once per distinct float32 triple.
 *   res     result (batch_best = -1, batch_loss = the start's loss).
 *   trace   optional HOST double [trace_cap][4]: (float32 C10, C12, phi12, loss) of
 *           each physical evaluation in order; the count is res->evals.
 * Errors: SSB_EINVAL (null argument, non-finite start or objective value).
 */
int ssb_nelder_mead(const double* x0, const ssb_fit_options* opt, ssb_objective f, void* ctx,
                    ssb_fit_result* res, double* trace, int32_t trace_cap);

/*
 * ssb_fit: evaluate the HOST float trials [n_trials][3] as one batch (ssb_loss),
 * then refine from the first trial with the lowest loss with ssb_nelder_mead on
 * ssb_loss.  trace as above (refinement evaluations only).  Synchronizes the stream.
 * Errors: those of ssb_loss and ssb_nelder_mead.
 */
int ssb_fit(ssb_handle* h, const float* trials, int32_t n_trials, const ssb_fit_options* opt,
            ssb_fit_result* res, double* trace, int32_t trace_cap, void* stream);

/* ssb_query: fill *info.  Errors: SSB_EINVAL. */
int ssb_query(const ssb_handle* h, ssb_info* info);

/* ssb_release: free the handle and its device memory; NULL is a no-op. */
void ssb_release(ssb_handle* h);

/* Thread-local text of the last error on this thread ("" if none). */
const char* ssb_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SSB_H */
