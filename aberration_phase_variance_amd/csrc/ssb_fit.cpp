// Aberration fit on the host: a batch of trials through ssb_loss, then
// Nelder-Mead refinement of the exact loss (declared in ssb.h).
//
// The refinement policy follows the SSB performance notes (Notes page, "MPS wider
// exact-simplex checkpoint": 5% axis steps floored at 2 nm for C12 and 0.04 rad
// for phi12 and rounded to two decimals, loss-spread tolerance 3e-6, reuse of
// evaluations whose float32 inputs repeat; "128 GB Apple M5 Max exact MPS
// checkpoint": coordinate tolerance 0.1).  The simplex itself is the standard
// Nelder-Mead method (Nelder and Mead 1965, in the form analysed by Lagarias,
// Reeds, Wright and Wright 1998): reflection 1, expansion 2, outside and inside
// contraction 1/2, shrink 1/2 towards the best vertex; vertices are kept sorted by
// loss with ties in their previous order (a new vertex goes after equal ones).
#include "../../include/ssb.h"

#include <algorithm>
#include <array>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <vector>

namespace ssb {
// defined in ssb_api.cpp: the thread-local error text of ssb_last_error
int set_error(int code, const std::string& msg);
void clear_error();
}  // namespace ssb

namespace {

constexpr int D = 3;
using Vec = std::array<double, D>;

ssb_fit_options defaults() {
    ssb_fit_options o;
    o.fatol = 3e-6;
    o.xatol = 0.1;
    o.step_frac = 0.05;
    o.step_floor[0] = 0.01;
    o.step_floor[1] = 2.0;
    o.step_floor[2] = 0.04;
    o.max_evals = 0;
    o.max_iter = 0;
    return o;
}

// Evaluations keyed by the float32 triple actually passed to the objective.
struct Memo {
    ssb_objective f;
    void* ctx;
    std::map<std::array<uint32_t, D>, double> seen;
    double* trace;
    int32_t trace_cap;
    int32_t requests = 0, evals = 0;
    int32_t max_evals;
    bool bad = false;

    // Returns false when the evaluation cap forbids a new evaluation.
    bool eval(const Vec& x, double& fx) {
        float p[D];
        std::array<uint32_t, D> key;
        for (int i = 0; i < D; ++i) {
            p[i] = (float)x[i];
            std::memcpy(&key[i], &p[i], sizeof(float));
        }
        ++requests;
        auto it = seen.find(key);
        if (it != seen.end()) {
            fx = it->second;
            return true;
        }
        if (max_evals > 0 && evals >= max_evals) {
            --requests;
            return false;
        }
        fx = f(p, ctx);
        if (!std::isfinite(fx)) {
            bad = true;
            return false;
        }
        if (trace && evals < trace_cap) {
            double* t = trace + 4 * (size_t)evals;
            for (int i = 0; i < D; ++i) t[i] = (double)p[i];
            t[3] = fx;
        }
        ++evals;
        seen.emplace(key, fx);
        return true;
    }
};

double round2(double v) { return std::round(v * 100.0) / 100.0; }

// Initial axis step: 5% of the start value (sign of the value, + for 0), at least
// the floor in magnitude, rounded to two decimals.
double axis_step(double x, double frac, double floor_) {
    double m = std::max(std::fabs(x) * frac, floor_);
    m = round2(m);
    if (m == 0.0) m = 0.01;
    return x < 0.0 ? -m : m;
}

}  // namespace

extern "C" int ssb_nelder_mead(const double* x0, const ssb_fit_options* opt_in, ssb_objective f, void* ctx,
                               ssb_fit_result* res, double* trace, int32_t trace_cap) {
    ssb::clear_error();
    if (!x0 || !f || !res) return ssb::set_error(SSB_EINVAL, "null argument");
    if (trace_cap < 0) return ssb::set_error(SSB_EINVAL, "negative trace capacity");
    const ssb_fit_options opt = opt_in ? *opt_in : defaults();
    for (int i = 0; i < D; ++i)
        if (!std::isfinite(x0[i])) return ssb::set_error(SSB_EINVAL, "non-finite start");
    if (!(opt.fatol >= 0.0) || !(opt.xatol >= 0.0) || !(opt.step_frac >= 0.0) || opt.max_evals < 0 ||
        opt.max_iter < 0)
        return ssb::set_error(SSB_EINVAL, "invalid options");
    const int max_iter = opt.max_iter > 0 ? opt.max_iter : 600;

    Memo memo{f, ctx, {}, trace, trace_cap, 0, 0, opt.max_evals};
    std::array<Vec, D + 1> sim;
    std::array<double, D + 1> fs;
    sim[0] = Vec{x0[0], x0[1], x0[2]};
    for (int k = 0; k < D; ++k) {
        sim[k + 1] = sim[0];
        sim[k + 1][k] += axis_step(x0[k], opt.step_frac, opt.step_floor[k]);
    }
    bool capped = false;
    for (int k = 0; k <= D; ++k) {
        if (!memo.eval(sim[k], fs[k])) {
            if (memo.bad) return ssb::set_error(SSB_EINVAL, "non-finite objective value");
            // the cap left vertices unevaluated: keep the evaluated ones only
            capped = true;
            for (int r = k; r <= D; ++r) fs[r] = INFINITY;
            break;
        }
    }

    // vertices ordered by loss; a stable sort keeps the incoming order of ties
    auto order = [&]() {
        std::array<int, D + 1> idx;
        for (int i = 0; i <= D; ++i) idx[i] = i;
        std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return fs[a] < fs[b]; });
        std::array<Vec, D + 1> s2;
        std::array<double, D + 1> f2;
        for (int i = 0; i <= D; ++i) {
            s2[i] = sim[idx[i]];
            f2[i] = fs[idx[i]];
        }
        sim = s2;
        fs = f2;
    };

    int iter = 0;
    bool converged = false;
    order();
    while (!capped) {
        // termination: simplex small in both coordinates and loss
        double dx = 0.0, df = 0.0;
        for (int k = 1; k <= D; ++k) {
            for (int i = 0; i < D; ++i) dx = std::max(dx, std::fabs(sim[k][i] - sim[0][i]));
            df = std::max(df, std::fabs(fs[k] - fs[0]));
        }
        if (dx <= opt.xatol && df <= opt.fatol) {
            converged = true;
            break;
        }
        if (iter >= max_iter) break;
        ++iter;

        Vec xbar{};
        for (int k = 0; k < D; ++k)
            for (int i = 0; i < D; ++i) xbar[i] += sim[k][i];
        for (int i = 0; i < D; ++i) xbar[i] /= D;
        auto along = [&](double t) {      // xbar + t (xbar - worst)
            Vec y;
            for (int i = 0; i < D; ++i) y[i] = xbar[i] + t * (xbar[i] - sim[D][i]);
            return y;
        };

        const Vec xr = along(1.0);
        double fr;
        if (!memo.eval(xr, fr)) break;
        bool do_shrink = false;
        if (fr < fs[0]) {
            const Vec xe = along(2.0);
            double fe;
            if (!memo.eval(xe, fe)) break;
            if (fe < fr) {
                sim[D] = xe;
                fs[D] = fe;
            } else {
                sim[D] = xr;
                fs[D] = fr;
            }
        } else if (fr < fs[D - 1]) {
            sim[D] = xr;
            fs[D] = fr;
        } else if (fr < fs[D]) {
            const Vec xc = along(0.5);          // outside contraction
            double fc;
            if (!memo.eval(xc, fc)) break;
            if (fc <= fr) {
                sim[D] = xc;
                fs[D] = fc;
            } else {
                do_shrink = true;
            }
        } else {
            const Vec xcc = along(-0.5);        // inside contraction
            double fcc;
            if (!memo.eval(xcc, fcc)) break;
            if (fcc < fs[D]) {
                sim[D] = xcc;
                fs[D] = fcc;
            } else {
                do_shrink = true;
            }
        }
        if (do_shrink) {
            bool ok = true;
            for (int k = 1; k <= D && ok; ++k) {
                for (int i = 0; i < D; ++i) sim[k][i] = sim[0][i] + 0.5 * (sim[k][i] - sim[0][i]);
                ok = memo.eval(sim[k], fs[k]);
                if (!ok)
                    for (int r = k; r <= D; ++r) fs[r] = INFINITY;
            }
            if (!ok) {
                order();
                break;
            }
        }
        order();
    }
    if (memo.bad) return ssb::set_error(SSB_EINVAL, "non-finite objective value");
    order();
    for (int i = 0; i < D; ++i) res->best[i] = sim[0][i];
    res->loss = fs[0];
    res->requests = memo.requests;
    res->evals = memo.evals;
    res->iterations = iter;
    res->converged = converged ? 1 : 0;
    res->batch_best = -1;
    res->pad = 0;
    res->batch_loss = fs[0];
    return SSB_OK;
}

namespace {

struct LossCtx {
    ssb_handle* h;
    void* stream;
    int rc;
};

double loss_objective(const float* p3, void* ctx) {
    LossCtx* c = static_cast<LossCtx*>(ctx);
    double l = NAN;
    const int rc = ssb_loss(c->h, p3, 1, &l, nullptr, c->stream);
    if (rc != SSB_OK) {
        c->rc = rc;
        return NAN;
    }
    return l;
}

}  // namespace

extern "C" int ssb_fit(ssb_handle* h, const float* trials, int32_t n_trials, const ssb_fit_options* opt,
                       ssb_fit_result* res, double* trace, int32_t trace_cap, void* stream) {
    ssb::clear_error();
    if (!trials || !res) return ssb::set_error(SSB_EINVAL, "null argument");
    if (n_trials < 1) return ssb::set_error(SSB_EINVAL, "n_trials must be at least 1");
    std::vector<double> losses((size_t)n_trials);
    int rc = ssb_loss(h, trials, n_trials, losses.data(), nullptr, stream);
    if (rc != SSB_OK) return rc;
    int32_t best = 0;
    for (int32_t t = 1; t < n_trials; ++t)
        if (losses[t] < losses[best]) best = t;
    const double x0[3] = {trials[3 * best], trials[3 * best + 1], trials[3 * best + 2]};
    LossCtx ctx{h, stream, SSB_OK};
    rc = ssb_nelder_mead(x0, opt, loss_objective, &ctx, res, trace, trace_cap);
    if (ctx.rc != SSB_OK) return ctx.rc;     // the loss call's own error text is kept
    if (rc != SSB_OK) return rc;
    res->batch_best = best;
    res->batch_loss = losses[best];
    return SSB_OK;
}
