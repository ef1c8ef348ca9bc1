// Host side of the C ABI declared in include/ssb.h.
#include "../../include/ssb.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "ssb_internal.hpp"

using namespace ssb;

namespace ssb {
bool in_bf_disk(const ssb_geometry* g, int i, int j);
}

namespace {
// |k|^2 < hi2 with the squares rounded separately (the oracle's rounding).
bool active_pixel(double di, double dj, double hi2) {
#pragma clang fp contract(off)
    const double a = di * di, b = dj * dj;
    return a + b < hi2;
}
}  // namespace

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    if (e == hipErrorOutOfMemory) return fail(SSB_ENOMEM, "%s: %s", what, hipGetErrorString(e));
    return fail(SSB_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

#define SSB_HIP(call, what)                          \
    do {                                             \
        hipError_t e_ = (call);                      \
        if (e_ != hipSuccess) return hip_fail(e_, what); \
    } while (0)

constexpr uint64_t kMagic = 0x5353424d49333535ull;   // "SSBMI355"
constexpr uint64_t kDead = 0xdeadbeefdeadbeefull;
// Intermediate budget for one chunk (all trials): bounds workspace memory.  Large
// enough that a 200-trial batch at 512^2 runs in 224-BF chunks (each chunk folds every
// trial's 2 MB double phase-sum image once, so small chunks cost reduction traffic),
// small against the 288 GB of one device.
constexpr double kInterBudget = 48.0 * 1024 * 1024 * 1024;

template <class T>
T* align_up(char* base, size_t& off, size_t count) {
    off = (off + 255) & ~size_t(255);
    T* p = reinterpret_cast<T*>(base + off);
    off += count * sizeof(T);
    return p;
}

}  // namespace

struct ssb_handle {
    uint64_t magic;
    ssb_geometry g;
    int n, h;
    int device;
    int64_t n_bf, n_active;
    GeomDev geo;
    double dc;
    int64_t chunk_user;
    int variant;          // SSB_VARIANT_HALF_PLANE or SSB_VARIANT_FULL_PLANE
    float2* gm = nullptr;
    float2* gn = nullptr;
    double2* kb = nullptr;
    uint8_t* active = nullptr;
    unsigned long long* bfsum = nullptr;
    uint4* sup = nullptr;      // correction support intervals [n_bf][N/2+1]
    int* vend = nullptr;       // 1 + last supported column per BF [n_bf]
    float2* tw = nullptr;      // FFT twiddle tables: inverse sign, then forward sign
    int64_t support_entries = 0, columns_written = 0, columns_read = 0;
    // loss / moments workspace
    char* ws = nullptr;
    size_t ws_bytes = 0;
    // object workspace
    char* ows = nullptr;
    size_t ows_bytes = 0;
    // trials every loss call up to this many fits without allocating (ssb_reserve)
    int reserved_trials = 0;
    // host staging of the per-trial constants (capacity = reserved trials)
    std::vector<TrialConst> htc;
    // pinned host landing area for the losses of up to hres_cap trials (the copy back
    // then needs no staging through a pageable buffer)
    double* hres = nullptr;
    int hres_cap = 0;
    // device address of the no-allocation scratch on this handle's device
    char* scratch = nullptr;
    // host copy of the active flags, prefix counts for range queries
    std::vector<int64_t> active_prefix;
    // stage profiling
    struct ProfRec {
        int stage;
        hipEvent_t a, b;
        int64_t units;
    };
    bool prof_on = false;
    std::vector<ProfRec> prof_pending;
    std::vector<hipEvent_t> prof_pool;
    double prof_ms[SSB_NUM_STAGES] = {};
    int64_t prof_n[SSB_NUM_STAGES] = {};
    int64_t prof_units[SSB_NUM_STAGES] = {};
};

namespace {

bool finite_pos(double v) { return std::isfinite(v) && v > 0.0; }

int check_handle(const ssb_handle* h) {
    if (!h) return fail(SSB_EINVAL, "null handle");
    if (h->magic != kMagic) return fail(SSB_EINVAL, "invalid or released handle");
    return SSB_OK;
}

int check_params(const float* p, int n) {
    for (int i = 0; i < 3 * n; ++i)
        if (!std::isfinite(p[i])) return fail(SSB_EINVAL, "parameter %d of trial %d is not finite", i % 3, i / 3);
    return SSB_OK;
}

hipEvent_t prof_event(ssb_handle* h) {
    if (!h->prof_pool.empty()) {
        hipEvent_t e = h->prof_pool.back();
        h->prof_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Records events around one stage's launches when profiling is on.
struct StageTimer {
    ssb_handle* h;
    int stage;
    hipStream_t st;
    int64_t units;
    hipEvent_t a = nullptr, b = nullptr;
    StageTimer(ssb_handle* h_, int stage_, hipStream_t st_, int64_t units_, bool allowed = true)
        : h(h_), stage(stage_), st(st_), units(units_) {
        if (!h->prof_on || !allowed) return;
        a = prof_event(h);
        b = prof_event(h);
        if (a && b) (void)hipEventRecord(a, st);
    }
    ~StageTimer() {
        if (a && b) {
            (void)hipEventRecord(b, st);
            h->prof_pending.push_back({stage, a, b, units});
        } else {
            if (a) h->prof_pool.push_back(a);
            if (b) h->prof_pool.push_back(b);
        }
    }
};

int prof_flush(ssb_handle* h) {
    for (auto& r : h->prof_pending) {
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(r.b);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess) return hip_fail(e, "profile events");
        h->prof_ms[r.stage] += ms;
        h->prof_n[r.stage] += 1;
        h->prof_units[r.stage] += r.units;
        h->prof_pool.push_back(r.a);
        h->prof_pool.push_back(r.b);
    }
    h->prof_pending.clear();
    return SSB_OK;
}

int64_t active_in(const ssb_handle* h, int64_t b0, int64_t b1) {
    return h->active_prefix[b1] - h->active_prefix[b0];
}

TrialConst trial_const(const ssb_handle* h, const float* p) {
    const double c10 = (double)p[0] * 10.0;    // nm -> Angstrom
    const double c12 = (double)p[1] * 10.0;
    const double phi = (double)p[2];
    const double c2 = std::cos(2.0 * phi), s2 = std::sin(2.0 * phi);
    const double k = 0.5 * h->g.wavelength_A * h->g.dk * h->g.dk;   // revolutions per (px^2 Angstrom)
    TrialConst t;
    t.mxx = k * (c10 + c12 * c2);
    t.myy = k * (c10 - c12 * c2);
    t.mxy = k * (c12 * s2);
    t.pad = 0.0;
    return t;
}

// Whether the row pass forms the object sums itself (ssb_loss_object): every scan size in
// the half plane, up to 512 in the full plane (at 1,024 the full plane's sums would not fit
// the row pass's registers).
bool fused_object(const ssb_handle* h, int variant) {
    return pass2_obj_sizes(h->n, variant == SSB_VARIANT_FULL_PLANE);
}

struct LossPlan {
    int cap;       // BF capacity of one chunk (multiple of kGroupBF)
    int gcap;      // groups per chunk
    size_t off_im, off_in, off_ps1, off_ps2, off_s1, off_s2, off_loss, off_lpart, off_tc, off_chm, off_chn;
    size_t off_na, off_nb;   // full-plane variant only (else 0)
    size_t off_po, off_oacc; // object sums of the row pass (fused loss and object; else 0)
    size_t total;
};

LossPlan plan_loss(const ssb_handle* h, int64_t nb, int n_trials, int variant, int64_t chunk_user,
                   bool obj = false) {
    const int64_t n = h->n, hh = h->h;
    const double plane = (double)n * (hh + 1) * sizeof(float2);
    // memory bound on the chunk (intermediate for all trials of the call)
    int64_t budget_cap = (int64_t)(kInterBudget / (plane * n_trials));
    budget_cap = std::max<int64_t>(kGroupBF, (budget_cap / kGroupBF) * kGroupBF);
    int64_t cap = budget_cap;
    if (chunk_user > 0)
        cap = std::min<int64_t>(cap, ((chunk_user + kGroupBF - 1) / kGroupBF) * kGroupBF);
    const int64_t need = ((nb + kGroupBF - 1) / kGroupBF) * kGroupBF;
    if (cap > need) cap = need;
    LossPlan pl;
    pl.cap = (int)cap;
    pl.gcap = (int)(cap / kGroupBF);
    const int rb = pass2_row_blocks(h->n);
    size_t off = 0;
    char* z = nullptr;
    pl.off_im = (size_t)align_up<float2>(z, off, (size_t)n_trials * cap * n * hh);
    pl.off_in = (size_t)align_up<float2>(z, off, (size_t)n_trials * cap * n);
    pl.off_ps1 = (size_t)align_up<float>(z, off, (size_t)n_trials * pl.gcap * n * n);
    pl.off_ps2 = (size_t)align_up<double>(z, off, (size_t)n_trials * pl.gcap * rb);
    pl.off_s1 = (size_t)align_up<double>(z, off, (size_t)n_trials * n * n);
    pl.off_s2 = (size_t)align_up<double>(z, off, (size_t)n_trials);
    pl.off_loss = (size_t)align_up<double>(z, off, (size_t)n_trials);
    pl.off_lpart = (size_t)align_up<double>(z, off, (size_t)n_trials * loss_blocks());
    pl.off_tc = (size_t)align_up<TrialConst>(z, off, (size_t)n_trials);
    pl.off_chm = (size_t)align_up<float2>(z, off, (size_t)n_trials * n * hh);
    pl.off_chn = (size_t)align_up<float2>(z, off, (size_t)n_trials * n);
    pl.off_na = pl.off_nb = 0;
    if (variant == SSB_VARIANT_FULL_PLANE) {
        pl.off_na = (size_t)align_up<float2>(z, off, (size_t)n_trials * cap * n);
        pl.off_nb = (size_t)align_up<float2>(z, off, (size_t)n_trials * cap * n);
    }
    pl.off_po = pl.off_oacc = 0;
    if (obj) {
        const int64_t no = obj_sum_count(h->n, variant == SSB_VARIANT_FULL_PLANE);
        pl.off_po = (size_t)align_up<float>(z, off, (size_t)n_trials * pl.gcap * no);
        pl.off_oacc = (size_t)align_up<double>(z, off, (size_t)n_trials * no);
    }
    pl.total = off + 256;
    return pl;
}

LossPlan plan_loss(const ssb_handle* h, int64_t nb, int n_trials) {
    return plan_loss(h, nb, n_trials, h->variant, h->chunk_user);
}

// Loss workspace that every call with at most n_trials trials fits, on any BF range, in
// either variant and under any chunk cap (a cap only shrinks the chunk; the chunk also
// shrinks as trials grow, so the need is not monotonic in the trial count).
size_t loss_ws_need(const ssb_handle* h, int n_trials) {
    size_t need = 0;
    for (int t = 1; t <= n_trials; ++t)
        for (int var : {SSB_VARIANT_HALF_PLANE, SSB_VARIANT_FULL_PLANE})
            need = std::max(need, plan_loss(h, h->n_bf, t, var, 0).total);
    // the fused loss and object (one trial)
    for (int var : {SSB_VARIANT_HALF_PLANE, SSB_VARIANT_FULL_PLANE})
        if (fused_object(h, var)) need = std::max(need, plan_loss(h, h->n_bf, 1, var, 0, true).total);
    return need;
}

// Object workspace layout (both variants' buffers; the half plane leaves the last two unused).
struct ObjPlan {
    size_t o_part, o_pm, o_pn, o_npart, o_nab, total;
};
ObjPlan plan_object(const ssb_handle* h) {
    const int n = h->n, hh = h->h;
    const int nseg = obj_segments(h->n_bf);
    const size_t ne = (size_t)n * (hh + 1);
    size_t off = 0;
    char* z = nullptr;
    ObjPlan p;
    p.o_part = (size_t)align_up<float2>(z, off, ne * nseg);
    p.o_pm = (size_t)align_up<float2>(z, off, (size_t)n * hh);
    p.o_pn = (size_t)align_up<float2>(z, off, (size_t)n);
    p.o_npart = (size_t)align_up<double2>(z, off, (size_t)2 * n * nseg);
    p.o_nab = (size_t)align_up<float2>(z, off, (size_t)2 * n);
    p.total = off + 256;
    return p;
}

int ensure(char** buf, size_t* have, size_t need, const char* what) {
    if (*have >= need) return SSB_OK;
    if (*buf) {
        hipError_t e = hipFree(*buf);
        *buf = nullptr;
        *have = 0;
        if (e != hipSuccess) return hip_fail(e, what);
    }
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, need);
    if (e != hipSuccess) return hip_fail(e, what);
    *buf = static_cast<char*>(p);
    *have = need;
    return SSB_OK;
}

// Workspaces for calls of up to max_trials trials, so that those calls allocate nothing.
int reserve(ssb_handle* h, int max_trials) {
    int rc = ensure(&h->ws, &h->ws_bytes, loss_ws_need(h, max_trials), "workspace allocation");
    if (rc) return rc;
    if ((rc = ensure(&h->ows, &h->ows_bytes, plan_object(h).total, "object workspace allocation"))) return rc;
    try {
        h->htc.reserve((size_t)max_trials);
    } catch (...) {
        return fail(SSB_ENOMEM, "host staging of %d trial constants", max_trials);
    }
    const int cap = std::max(max_trials, kTrialBlock);
    if (cap > h->hres_cap) {
        double* p = nullptr;
        if (hipHostMalloc(reinterpret_cast<void**>(&p), sizeof(double) * cap, hipHostMallocDefault) != hipSuccess)
            return fail(SSB_ENOMEM, "pinned host buffer for %d losses", cap);
        if (h->hres) (void)hipHostFree(h->hres);
        h->hres = p;
        h->hres_cap = cap;
    }
    h->reserved_trials = std::max(h->reserved_trials, max_trials);
    return SSB_OK;
}

// Phase moments of n_trials trials over BF [b_begin, b_end): leaves S1 (double
// [t][N][N]) and S2 (double [t]) in the workspace ws laid out by pl.
// staged: stage timers run, and batches of more than kTrialBlock trials send their
// constants through a host copy in the handle (h->htc), which must outlive the
// stream's use of it (the caller synchronizes before returning).  Otherwise, and for
// smaller batches in any case, the constants are passed to a small kernel by value (one
// launch instead of a staged pageable copy; nothing allocated).  The first chunk's
// accumulation writes S1 and S2 outright, so they need no clearing launch (with the
// previous change, about 0.015 ms per evaluation).
// obj: the row pass also leaves the object sums of every chunk, accumulated in
// ws + pl.off_oacc (the plan must have them).
int run_moments(ssb_handle* h, char* ws, const LossPlan& pl, const float* params, int n_trials, int64_t b_begin,
                int64_t b_end, hipStream_t st, bool staged, bool obj = false) {
    std::vector<TrialConst>& htc = h->htc;
    float2* im = reinterpret_cast<float2*>(ws + pl.off_im);
    float2* in = reinterpret_cast<float2*>(ws + pl.off_in);
    float* ps1 = reinterpret_cast<float*>(ws + pl.off_ps1);
    double* ps2 = reinterpret_cast<double*>(ws + pl.off_ps2);
    double* s1 = reinterpret_cast<double*>(ws + pl.off_s1);
    double* s2 = reinterpret_cast<double*>(ws + pl.off_s2);
    TrialConst* tc = reinterpret_cast<TrialConst*>(ws + pl.off_tc);
    float2* chm = reinterpret_cast<float2*>(ws + pl.off_chm);
    float2* chn = reinterpret_cast<float2*>(ws + pl.off_chn);
    const bool fp = h->variant == SSB_VARIANT_FULL_PLANE;
    float2* nyq_a = fp ? reinterpret_cast<float2*>(ws + pl.off_na) : nullptr;
    float2* nyq_b = fp ? reinterpret_cast<float2*>(ws + pl.off_nb) : nullptr;
    float* po = obj ? reinterpret_cast<float*>(ws + pl.off_po) : nullptr;
    double* oacc = obj ? reinterpret_cast<double*>(ws + pl.off_oacc) : nullptr;

    if (staged && n_trials > kTrialBlock) {
        if ((size_t)n_trials > htc.capacity()) {      // beyond the reservation: the one host allocation
            try {
                htc.reserve((size_t)n_trials);
            } catch (...) {
                return fail(SSB_ENOMEM, "host staging of %d trial constants", n_trials);
            }
        }
        htc.resize(n_trials);
        for (int t = 0; t < n_trials; ++t) htc[t] = trial_const(h, params + 3 * t);
        SSB_HIP(hipMemcpyAsync(tc, htc.data(), sizeof(TrialConst) * n_trials, hipMemcpyHostToDevice, st),
                "copy trial constants");
    } else {
        for (int t0 = 0; t0 < n_trials; t0 += kTrialBlock) {
            TrialBlock blk;
            const int cnt = std::min(kTrialBlock, n_trials - t0);
            for (int k = 0; k < cnt; ++k) blk.t[k] = trial_const(h, params + 3 * (t0 + k));
            SSB_HIP(launch_set_trials(blk, cnt, tc + t0, st), "trial constants");
        }
    }
    {
        StageTimer tm(h, SSB_STAGE_REDUCE, st, 0, staged);
        if (b_begin >= b_end) {                       // no chunk below writes the sums
            SSB_HIP(launch_fill(s1, (int64_t)n_trials * h->n * h->n, st), "clear S1");
            SSB_HIP(launch_fill(s2, n_trials, st), "clear S2");
            if (obj) SSB_HIP(launch_fill(oacc, (int64_t)n_trials * obj_sum_count(h->n, fp), st), "clear object sums");
        }
        SSB_HIP(launch_chiq(h->n, tc, n_trials, h->geo, chm, chn, st), "phase table launch");
    }

    for (int64_t c0 = b_begin; c0 < b_end; c0 += pl.cap) {
        const int cb = (int)std::min<int64_t>(pl.cap, b_end - c0);
        const int ng = (cb + kGroupBF - 1) / kGroupBF;
        const int64_t units = active_in(h, c0, c0 + cb) * n_trials;
        {
            StageTimer tm(h, SSB_STAGE_PASS1, st, units, staged);
            SSB_HIP(launch_pass1(h->n, h->gm, h->gn, chm, chn, h->kb, h->sup, h->vend, tc, n_trials, h->geo, c0, cb,
                                 pl.cap, im, in, st),
                    "pass 1 launch");
            if (fp)
                SSB_HIP(launch_nyq_lines(h->n, h->gm, h->gn, h->kb, h->active, tc, n_trials, h->geo, c0, cb, pl.cap,
                                         nyq_a, nyq_b, h->tw, st),
                        "Nyquist-line launch");
        }
        {
            StageTimer tm(h, SSB_STAGE_PASS2, st, units, staged);
            SSB_HIP(launch_pass2(h->n, im, in, pl.cap, h->active, h->vend, c0, cb, n_trials, h->dc, ps1, ps2,
                                 pl.gcap, h->tw, nyq_a, nyq_b, po, st),
                    "pass 2 launch");
        }
        {
            StageTimer tm(h, SSB_STAGE_REDUCE, st, 0, staged);
            SSB_HIP(launch_accum(h->n, ps1, ps2, pl.gcap, ng, n_trials, s1, s2, c0 == b_begin, st),
                    "accumulate launch");
            if (obj)
                SSB_HIP(launch_accum_obj(h->n, fp, po, pl.gcap, ng, n_trials, oacc, c0 == b_begin, st),
                        "object-sum accumulate launch");
        }
    }
    return SSB_OK;
}

// The loss of n_trials trials over every BF pixel in the workspace ws (layout pl),
// copied to the host array losses; synchronizes the stream.
// With obj (one trial, a plan that has the object sums) the object's phase (and psi when
// not null) is written as well, from the row pass's object sums.
int run_loss(ssb_handle* h, char* ws, const LossPlan& pl, const float* params, int n_trials, double* losses,
             float* mean_phase, hipStream_t st, bool staged, bool obj = false, float* phase = nullptr,
             float* psi = nullptr) {
    int rc = run_moments(h, ws, pl, params, n_trials, 0, h->n_bf, st, staged, obj);
    if (rc) {
        (void)hipStreamSynchronize(st);
        return rc;
    }
    double* s1 = reinterpret_cast<double*>(ws + pl.off_s1);
    double* s2 = reinterpret_cast<double*>(ws + pl.off_s2);
    double* dl = reinterpret_cast<double*>(ws + pl.off_loss);
    double* lp = reinterpret_cast<double*>(ws + pl.off_lpart);
    {
        StageTimer tm(h, SSB_STAGE_REDUCE, st, 0, staged);
        SSB_HIP(launch_loss(h->n, s1, s2, n_trials, (double)h->n_bf, lp, dl, mean_phase, st), "loss launch");
    }
    if (obj) {
        StageTimer tm(h, SSB_STAGE_OBJ_FFT, st, 0, staged);
        const int n = h->n;
        // the inactive BF pixels add their DC term only
        const double re_extra = h->dc * (double)(h->n_bf - h->n_active);
        const double scale = 1.0 / ((double)h->n_bf * (double)n * (double)n);
        SSB_HIP(launch_obj_from_sums(n, h->variant == SSB_VARIANT_FULL_PLANE,
                                     reinterpret_cast<double*>(ws + pl.off_oacc), re_extra, scale, phase,
                                     reinterpret_cast<float2*>(psi), st),
                "object from sums");
    }
    if (n_trials <= h->hres_cap) {
        SSB_HIP(hipMemcpyAsync(h->hres, dl, sizeof(double) * n_trials, hipMemcpyDeviceToHost, st), "copy losses");
        SSB_HIP(hipStreamSynchronize(st), "loss");
        std::memcpy(losses, h->hres, sizeof(double) * n_trials);
    } else {
        SSB_HIP(hipMemcpyAsync(losses, dl, sizeof(double) * n_trials, hipMemcpyDeviceToHost, st), "copy losses");
        SSB_HIP(hipStreamSynchronize(st), "loss");
    }
    return SSB_OK;
}

}  // namespace

namespace ssb {
// BF rule: (i - cy)^2 + (j - cx)^2 <= bf_r2, squares rounded separately and then
// added (no fused multiply-add), which is also the rounding of the oracle.
bool in_bf_disk(const ssb_geometry* g, int i, int j) {
#pragma clang fp contract(off)
    const double di = i - g->det_cy, dj = j - g->det_cx;
    const double a = di * di, b = dj * dj;
    return a + b <= g->bf_r2;
}

// Shared with the fit driver (ssb_fit.cpp): the thread-local error text.
int set_error(int code, const std::string& msg) {
    g_err = msg;
    return code;
}
void clear_error() { g_err.clear(); }
}  // namespace ssb

extern "C" {

const char* ssb_last_error(void) { return g_err.c_str(); }

int ssb_prepare(const ssb_geometry* g, const uint32_t* counts, int64_t n_bf, void* stream, ssb_handle** out) {
    g_err.clear();
    if (!g || !counts || !out) return fail(SSB_EINVAL, "null argument");
    *out = nullptr;
    const int n = g->scan_n;
    if (n != 32 && n != 64 && n != 128 && n != 256 && n != 512 && n != 1024)
        return fail(SSB_EINVAL, "scan_n must be a power of two in [32, 1024], got %d", n);
    if (g->det_n <= 0) return fail(SSB_EINVAL, "det_n must be positive");
    if (!std::isfinite(g->bf_r2) || g->bf_r2 < 0.0) return fail(SSB_EINVAL, "bf_r2 must be finite and >= 0");
    if (!std::isfinite(g->det_cy) || !std::isfinite(g->det_cx)) return fail(SSB_EINVAL, "non-finite detector center");
    if (!finite_pos(g->q_step_px) || !finite_pos(g->dk) || !finite_pos(g->wavelength_A) ||
        !finite_pos(g->alpha_rad) || !finite_pos(g->edge_px))
        return fail(SSB_EINVAL, "q_step_px, dk, wavelength_A, alpha_rad and edge_px must be finite and > 0");
    if (!std::isfinite(g->rotation_rad)) return fail(SSB_EINVAL, "non-finite rotation");
    if (n_bf <= 0) return fail(SSB_ESHAPE, "n_bf must be positive");

    // BF set (row-major) and per-BF offsets
    const double ra = g->alpha_rad / g->wavelength_A / g->dk;
    const double w = g->edge_px;
    const double hi2 = (ra + 0.5 * w) * (ra + 0.5 * w);
    std::vector<double2> kb;
    std::vector<uint8_t> act;
    for (int i = 0; i < g->det_n; ++i)
        for (int j = 0; j < g->det_n; ++j) {
            const double di = i - g->det_cy, dj = j - g->det_cx;
            if (ssb::in_bf_disk(g, i, j)) {
                kb.push_back(make_double2(dj, di));
                act.push_back(active_pixel(di, dj, hi2) ? 1 : 0);
            }
        }
    if ((int64_t)kb.size() != n_bf)
        return fail(SSB_ESHAPE, "n_bf = %lld but the BF rule selects %zu detector pixels", (long long)n_bf, kb.size());

    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, counts) != hipSuccess || attr.type == hipMemoryTypeHost ||
        attr.type == hipMemoryTypeUnregistered) {
        (void)hipGetLastError();
        return fail(SSB_EINVAL, "counts must be a device pointer");
    }

    ssb_handle* h = new ssb_handle();
    h->magic = kMagic;
    h->g = *g;
    h->n = n;
    h->h = n / 2;
    h->n_bf = n_bf;
    h->n_active = 0;
    h->active_prefix.assign(1, 0);
    for (uint8_t a : act) {
        h->n_active += a;
        h->active_prefix.push_back(h->n_active);
    }
    h->chunk_user = 0;
    h->variant = SSB_VARIANT_HALF_PLANE;
    (void)hipGetDevice(&h->device);
    GeomDev& geo = h->geo;
    geo.n = n;
    geo.h = n / 2;
    geo.s = g->q_step_px;
    geo.crot = std::cos(g->rotation_rad);
    geo.srot = std::sin(g->rotation_rad);
    geo.qvx = g->q_step_px * geo.crot;
    geo.qux = -g->q_step_px * geo.srot;
    geo.qvy = g->q_step_px * geo.srot;
    geo.quy = g->q_step_px * geo.crot;
    geo.inv_w = 1.0 / w;
    geo.ra = ra;
    geo.ra2 = ra * ra;
    geo.w = w;
    geo.lo2 = ra >= 0.5 * w ? (ra - 0.5 * w) * (ra - 0.5 * w) : -1.0;
    geo.hi2 = hi2;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const size_t nm = (size_t)n_bf * n * (n / 2), nn = (size_t)n_bf * n;
    auto cleanup = [&](int rc) {
        ssb_release(h);
        return rc;
    };
    hipError_t e;
    if ((e = hipMalloc(&h->gm, nm * sizeof(float2))) != hipSuccess) return cleanup(hip_fail(e, "spectrum allocation"));
    if ((e = hipMalloc(&h->gn, nn * sizeof(float2))) != hipSuccess) return cleanup(hip_fail(e, "spectrum allocation"));
    if ((e = hipMalloc(&h->kb, kb.size() * sizeof(double2))) != hipSuccess) return cleanup(hip_fail(e, "allocation"));
    if ((e = hipMalloc(&h->active, act.size())) != hipSuccess) return cleanup(hip_fail(e, "allocation"));
    if ((e = hipMalloc(&h->bfsum, n_bf * sizeof(unsigned long long))) != hipSuccess)
        return cleanup(hip_fail(e, "allocation"));
    if ((e = hipMemcpyAsync(h->kb, kb.data(), kb.size() * sizeof(double2), hipMemcpyHostToDevice, st)) != hipSuccess ||
        (e = hipMemcpyAsync(h->active, act.data(), act.size(), hipMemcpyHostToDevice, st)) != hipSuccess ||
        (e = hipMemsetAsync(h->bfsum, 0, n_bf * sizeof(unsigned long long), st)) != hipSuccess)
        return cleanup(hip_fail(e, "prepare upload"));
    const int ntw = twiddle_count(n);
    if ((e = hipMalloc(&h->tw, 2 * (size_t)ntw * sizeof(float2))) != hipSuccess)
        return cleanup(hip_fail(e, "allocation"));
    if ((e = launch_twiddles(n, h->tw, h->tw + ntw, st)) != hipSuccess)
        return cleanup(hip_fail(e, "twiddle tables"));
    if ((e = launch_g_rows(n, counts, n_bf, h->gm, h->gn, h->bfsum, h->tw + ntw, st)) != hipSuccess)
        return cleanup(hip_fail(e, "spectrum row pass"));
    if ((e = launch_g_cols(n, h->gm, h->gn, n_bf, h->tw + ntw, st)) != hipSuccess)
        return cleanup(hip_fail(e, "spectrum column pass"));
    if ((e = hipMalloc(&h->sup, (size_t)n_bf * (n / 2 + 1) * sizeof(uint4))) != hipSuccess ||
        (e = hipMalloc(&h->vend, (size_t)n_bf * sizeof(int))) != hipSuccess)
        return cleanup(hip_fail(e, "allocation"));
    int* nsup = nullptr;
    if ((e = hipMalloc(&nsup, (size_t)n_bf * sizeof(int))) != hipSuccess) return cleanup(hip_fail(e, "allocation"));
    std::vector<int> vend_h(n_bf), nsup_h(n_bf);
    if ((e = launch_support(n, h->kb, h->active, h->geo, n_bf, h->sup, h->vend, nsup, st)) != hipSuccess ||
        (e = hipMemcpyAsync(vend_h.data(), h->vend, n_bf * sizeof(int), hipMemcpyDeviceToHost, st)) != hipSuccess ||
        (e = hipMemcpyAsync(nsup_h.data(), nsup, n_bf * sizeof(int), hipMemcpyDeviceToHost, st)) != hipSuccess ||
        (e = hipStreamSynchronize(st)) != hipSuccess) {
        (void)hipFree(nsup);
        return cleanup(hip_fail(e, "support tables"));
    }
    (void)hipFree(nsup);
    const int tile = pass1_tile(n), hh = n / 2;
    for (int64_t b = 0; b < n_bf; ++b) {
        const int ve = vend_h[b];
        h->support_entries += nsup_h[b];
        if (ve > 0) h->columns_written += std::min(hh, (ve + tile - 1) / tile * tile) + (ve > hh ? 1 : 0);
        h->columns_read += std::min(hh, ve) + (ve > hh ? 1 : 0);
    }
    std::vector<unsigned long long> sums(n_bf);
    if ((e = hipMemcpyAsync(sums.data(), h->bfsum, n_bf * sizeof(unsigned long long), hipMemcpyDeviceToHost, st)) !=
            hipSuccess ||
        (e = hipStreamSynchronize(st)) != hipSuccess)
        return cleanup(hip_fail(e, "prepare"));
    unsigned long long tot = 0;
    for (unsigned long long s : sums) tot += s;
    h->dc = (double)tot / (double)n_bf;
    // single-trial loss and object workspaces now, so that those calls allocate nothing
    int rc = reserve(h, 1);
    if (rc) return cleanup(rc);
    // the no-allocation scratch's address on this device (looked up once per device)
    void* sp = nullptr;
    if ((e = scratch_address(&sp)) != hipSuccess) return cleanup(hip_fail(e, "no-allocation scratch address"));
    h->scratch = static_cast<char*>(sp);
    *out = h;
    return SSB_OK;
}

int ssb_loss(ssb_handle* h, const float* params, int32_t n_trials, double* losses, float* mean_phase,
             void* stream) {
    g_err.clear();
    int rc = check_handle(h);
    if (rc) return rc;
    if (!params || !losses) return fail(SSB_EINVAL, "null params or losses");
    if (n_trials < 1 || n_trials > 65535) return fail(SSB_EINVAL, "n_trials must be in [1, 65535]");
    if ((rc = check_params(params, n_trials))) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const LossPlan pl = plan_loss(h, h->n_bf, n_trials);
    if ((rc = ensure(&h->ws, &h->ws_bytes, pl.total, "workspace allocation"))) return rc;
    return run_loss(h, h->ws, pl, params, n_trials, losses, mean_phase, st, true);
}

int ssb_loss_noalloc(ssb_handle* h, const float* params, int32_t n_trials, double* losses, float* mean_phase,
                     void* stream) {
    g_err.clear();
    int rc = check_handle(h);
    if (rc) return rc;
    if (!params || !losses) return fail(SSB_EINVAL, "null params or losses");
    if (n_trials < 1 || n_trials > 65535) return fail(SSB_EINVAL, "n_trials must be in [1, 65535]");
    if ((rc = check_params(params, n_trials))) return rc;
    if (!h->scratch) return fail(SSB_EDEVICE, "no-allocation scratch not found on this handle's device");
    // the largest chunk (a multiple of the 32-BF group, under the handle's chunk cap)
    // whose buffers fit the scratch; results do not depend on the chunk
    const size_t room = scratch_bytes();
    const int64_t groups = (h->n_bf + kGroupBF - 1) / kGroupBF;
    int64_t lo = 1, hi = groups;
    if (h->chunk_user > 0) hi = std::min<int64_t>(hi, (h->chunk_user + kGroupBF - 1) / kGroupBF);
    if (plan_loss(h, h->n_bf, n_trials, h->variant, kGroupBF).total > room)
        return fail(SSB_EINVAL,
                    "%d trials need %zu bytes of scratch even with %d-BF chunks; the no-allocation scratch holds %zu",
                    (int)n_trials, plan_loss(h, h->n_bf, n_trials, h->variant, kGroupBF).total, kGroupBF, room);
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) / 2;
        if (plan_loss(h, h->n_bf, n_trials, h->variant, mid * kGroupBF).total <= room) lo = mid;
        else hi = mid - 1;
    }
    const LossPlan pl = plan_loss(h, h->n_bf, n_trials, h->variant, lo * kGroupBF);
    return run_loss(h, h->scratch, pl, params, n_trials, losses, mean_phase, static_cast<hipStream_t>(stream),
                    false);
}

int ssb_moments(ssb_handle* h, const float* params3, int64_t bf_begin, int64_t bf_end, double* s1, double* s2,
                void* stream) {
    g_err.clear();
    int rc = check_handle(h);
    if (rc) return rc;
    if (!params3 || !s1 || !s2) return fail(SSB_EINVAL, "null argument");
    if (bf_begin < 0 || bf_end > h->n_bf || bf_begin >= bf_end)
        return fail(SSB_ESHAPE, "BF range [%lld, %lld) outside [0, %lld)", (long long)bf_begin, (long long)bf_end,
                    (long long)h->n_bf);
    if ((rc = check_params(params3, 1))) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const LossPlan pl = plan_loss(h, bf_end - bf_begin, 1);
    if ((rc = ensure(&h->ws, &h->ws_bytes, pl.total, "workspace allocation"))) return rc;
    if ((rc = run_moments(h, h->ws, pl, params3, 1, bf_begin, bf_end, st, true))) {
        (void)hipStreamSynchronize(st);
        return rc;
    }
    SSB_HIP(hipMemcpyAsync(s1, h->ws + pl.off_s1, sizeof(double) * h->n * h->n, hipMemcpyDeviceToDevice, st),
            "copy S1");
    SSB_HIP(hipMemcpyAsync(s2, h->ws + pl.off_s2, sizeof(double), hipMemcpyDeviceToHost, st), "copy S2");
    SSB_HIP(hipStreamSynchronize(st), "moments");
    return SSB_OK;
}

int ssb_object(ssb_handle* h, const float* params3, float* phase, float* psi, void* stream) {
    g_err.clear();
    int rc = check_handle(h);
    if (rc) return rc;
    if (!params3 || !phase) return fail(SSB_EINVAL, "null argument");
    if ((rc = check_params(params3, 1))) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int n = h->n;
    const int nseg = obj_segments(h->n_bf);
    const ObjPlan op = plan_object(h);            // reserved by ssb_prepare: no allocation here
    if ((rc = ensure(&h->ows, &h->ows_bytes, op.total, "object workspace allocation"))) return rc;
    const bool fp = h->variant == SSB_VARIANT_FULL_PLANE;
    const size_t o_npart = op.o_npart;
    float2* part = reinterpret_cast<float2*>(h->ows + op.o_part);
    float2* pm = reinterpret_cast<float2*>(h->ows + op.o_pm);
    float2* pn = reinterpret_cast<float2*>(h->ows + op.o_pn);
    float2* nab = fp ? reinterpret_cast<float2*>(h->ows + op.o_nab) : nullptr;
    const TrialConst tc = trial_const(h, params3);   // kernel argument: no host-staged copy
    {
        StageTimer tm(h, SSB_STAGE_OBJ_SUM, st, h->n_active);
        SSB_HIP(launch_obj_sum(n, h->gm, h->gn, h->kb, h->sup, h->vend, tc, h->geo, h->n_bf, part, nseg, st),
                "object sum");
        if (fp)
            SSB_HIP(launch_obj_nyq(n, h->gm, h->gn, h->kb, h->vend, tc, h->geo, h->n_bf,
                                   reinterpret_cast<double2*>(h->ows + o_npart), nseg, nab, h->tw, st),
                    "object Nyquist lines");
    }
    {
        StageTimer tm(h, SSB_STAGE_OBJ_FFT, st, 0);
        SSB_HIP(launch_obj_reduce(n, part, nseg, pm, pn, st), "object reduce");
        SSB_HIP(launch_obj_cols(n, pm, pn, h->tw, st), "object columns");
        const double dcsum = h->dc * (double)h->n_bf;
        const double scale = 1.0 / ((double)h->n_bf * (double)n * (double)n);
        SSB_HIP(launch_obj_rows(n, pm, pn, dcsum, scale, phase, reinterpret_cast<float2*>(psi), h->tw, nab, st),
                "object rows");
    }
    return SSB_OK;
}

int ssb_loss_object(ssb_handle* h, const float* params3, double* loss, float* phase, float* psi, void* stream) {
    g_err.clear();
    int rc = check_handle(h);
    if (rc) return rc;
    if (!params3 || !loss || !phase) return fail(SSB_EINVAL, "null argument");
    if ((rc = check_params(params3, 1))) return rc;
    if (!fused_object(h, h->variant)) {
        // the full plane at 1,024 points: the loss, then the object's own pass
        if ((rc = ssb_loss(h, params3, 1, loss, nullptr, stream))) return rc;
        if ((rc = ssb_object(h, params3, phase, psi, stream))) return rc;
        SSB_HIP(hipStreamSynchronize(static_cast<hipStream_t>(stream)), "object");
        return SSB_OK;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    const LossPlan pl = plan_loss(h, h->n_bf, 1, h->variant, h->chunk_user, true);
    if ((rc = ensure(&h->ws, &h->ws_bytes, pl.total, "workspace allocation"))) return rc;
    return run_loss(h, h->ws, pl, params3, 1, loss, nullptr, st, true, true, phase, psi);
}

int ssb_spectrum(const ssb_handle* h, int64_t bf, float* out, void* stream) {
    g_err.clear();
    int rc = check_handle(h);
    if (rc) return rc;
    if (!out) return fail(SSB_EINVAL, "null output");
    if (bf < 0 || bf >= h->n_bf) return fail(SSB_ESHAPE, "BF index %lld outside [0, %lld)", (long long)bf,
                                             (long long)h->n_bf);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int n = h->n, hh = h->h;
    float2* o = reinterpret_cast<float2*>(out);
    // the cache is tile-major ([N/2/8][N][8] per BF): one strided copy per 8-column tile
    for (int tile = 0; tile < hh / kTileW; ++tile)
        SSB_HIP(hipMemcpy2DAsync(o + tile * kTileW, sizeof(float2) * (hh + 1),
                                 h->gm + (size_t)bf * n * hh + (size_t)tile * n * kTileW, sizeof(float2) * kTileW,
                                 sizeof(float2) * kTileW, n, hipMemcpyDeviceToDevice, st),
                "copy spectrum");
    SSB_HIP(hipMemcpy2DAsync(o + hh, sizeof(float2) * (hh + 1), h->gn + (size_t)bf * n, sizeof(float2),
                             sizeof(float2), n, hipMemcpyDeviceToDevice, st),
            "copy spectrum");
    return SSB_OK;
}

int ssb_set_chunk(ssb_handle* h, int64_t chunk_bf) {
    g_err.clear();
    int rc = check_handle(h);
    if (rc) return rc;
    if (chunk_bf < 0) return fail(SSB_EINVAL, "chunk_bf must be >= 0");
    h->chunk_user = chunk_bf;
    return SSB_OK;
}

int ssb_set_variant(ssb_handle* h, int32_t variant) {
    g_err.clear();
    int rc = check_handle(h);
    if (rc) return rc;
    if (variant != SSB_VARIANT_HALF_PLANE && variant != SSB_VARIANT_FULL_PLANE)
        return fail(SSB_EINVAL, "variant must be SSB_VARIANT_HALF_PLANE (0) or SSB_VARIANT_FULL_PLANE (1), got %d",
                    (int)variant);
    h->variant = variant;
    return SSB_OK;
}

int ssb_profile(ssb_handle* h, int mode, ssb_profile_data* out) {
    g_err.clear();
    int rc = check_handle(h);
    if (rc) return rc;
    if (mode < 0 || mode > 2) return fail(SSB_EINVAL, "profile mode must be 0, 1 or 2");
    if ((rc = prof_flush(h))) return rc;
    if (out) {
        for (int s = 0; s < SSB_NUM_STAGES; ++s) {
            out->ms[s] = h->prof_ms[s];
            out->launches[s] = h->prof_n[s];
            out->units[s] = h->prof_units[s];
        }
    }
    if (mode == 1) {
        for (int s = 0; s < SSB_NUM_STAGES; ++s) {
            h->prof_ms[s] = 0.0;
            h->prof_n[s] = 0;
            h->prof_units[s] = 0;
        }
        h->prof_on = true;
    } else if (mode == 0) {
        h->prof_on = false;
    }
    return SSB_OK;
}

int ssb_query(const ssb_handle* h, ssb_info* info) {
    g_err.clear();
    int rc = check_handle(h);
    if (rc) return rc;
    if (!info) return fail(SSB_EINVAL, "null info");
    info->n_bf = h->n_bf;
    info->n_active_bf = h->n_active;
    info->scan_n = h->n;
    info->det_n = h->g.det_n;
    info->spectrum_bytes = (int64_t)h->n_bf * h->n * (h->h + 1) * (int64_t)sizeof(float2);
    info->dc = h->dc;
    info->chunk_bf = plan_loss(h, h->n_bf, 1).cap;
    info->support_entries = h->support_entries;
    info->columns_written = h->columns_written;
    info->columns_read = h->columns_read;
    info->variant = h->variant;
    info->pad = 0;
    info->workspace_bytes = (int64_t)(h->ws_bytes + h->ows_bytes);
    info->reserved_trials = h->reserved_trials;
    info->pad2 = 0;
    return SSB_OK;
}

int ssb_reserve(ssb_handle* h, int32_t max_trials) {
    g_err.clear();
    int rc = check_handle(h);
    if (rc) return rc;
    if (max_trials < 1 || max_trials > 65535) return fail(SSB_EINVAL, "max_trials must be in [1, 65535]");
    return reserve(h, max_trials);
}

void ssb_release(ssb_handle* h) {
    if (!h || h->magic != kMagic) return;
    h->magic = kDead;
    (void)hipFree(h->gm);
    (void)hipFree(h->gn);
    (void)hipFree(h->kb);
    (void)hipFree(h->active);
    (void)hipFree(h->bfsum);
    (void)hipFree(h->sup);
    (void)hipFree(h->vend);
    (void)hipFree(h->tw);
    (void)hipFree(h->ws);
    (void)hipFree(h->ows);
    if (h->hres) (void)hipHostFree(h->hres);
    for (auto& r : h->prof_pending) {
        (void)hipEventSynchronize(r.b);
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    for (hipEvent_t e : h->prof_pool) (void)hipEventDestroy(e);
    delete h;
}

}  // extern "C"
