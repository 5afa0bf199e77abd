// Adaptive draft depth (span-02 spec.rs KPolicy): host-side arithmetic, no GPU work.
// A caller keeps one spec_kpolicy per decoding loop, calls spec_kpolicy_choose before
// drafting and spec_kpolicy_update (or _update_batch with the accept lengths copied
// to the host) after each verify. The verify cost table is the caller's own
// measurement of the verify step against its row count.
#include <cmath>
#include <cstring>

#include "common.h"

namespace {

double accept_prob(const spec_kpolicy* p, int j) {
    return (p->succ[j] + p->prior_p * p->prior_n) / (p->att[j] + p->prior_n);
}

double verify_cost(const spec_kpolicy* p, double r) {
    const double* x = p->cost_rows;
    const double* y = p->cost_us;
    const int n = p->n_points;
    if (r <= x[0]) return y[0] * r / x[0];                       // through the origin
    for (int i = 0; i + 1 < n; ++i)
        if (r <= x[i + 1]) return y[i] + (y[i + 1] - y[i]) * (r - x[i]) / (x[i + 1] - x[i]);
    if (n == 1) return y[0] * r / x[0];
    return y[n - 1] + (y[n - 1] - y[n - 2]) * (r - x[n - 1]) / (x[n - 1] - x[n - 2]);   // last segment extended
}

double expected_tokens(const spec_kpolicy* p, int k) {
    double e = 1.0, prod = 1.0;
    for (int j = 0; j < k; ++j) {
        prod *= accept_prob(p, j);
        e += prod;
    }
    return e;
}

}  // namespace

extern "C" {

int spec_kpolicy_init(spec_kpolicy* p, int32_t kmin, int32_t kmax, double prior_p, double prior_n, double draft_us,
                      const double* cost_rows, const double* cost_us, int32_t n_points) {
    using namespace sv;
    last_error().clear();
    if (!p || !cost_rows || !cost_us) return fail(SPEC_EINVAL, "spec_kpolicy_init: null pointer");
    if (kmin < 0 || kmax < kmin || kmax >= SPEC_KPOLICY_MAXK)
        return fail(SPEC_EINVAL, "spec_kpolicy_init: need 0 <= kmin <= kmax < %d (kmin=%d kmax=%d)", SPEC_KPOLICY_MAXK, kmin, kmax);
    if (!(prior_p > 0.0 && prior_p <= 1.0) || !(prior_n > 0.0) || !std::isfinite(prior_n))
        return fail(SPEC_EINVAL, "spec_kpolicy_init: need 0 < prior_p <= 1 and prior_n > 0");
    if (!(draft_us >= 0.0) || !std::isfinite(draft_us)) return fail(SPEC_EINVAL, "spec_kpolicy_init: draft_us must be >= 0");
    if (n_points < 1 || n_points > SPEC_KPOLICY_MAXPTS)
        return fail(SPEC_EINVAL, "spec_kpolicy_init: n_points=%d outside 1..%d", n_points, SPEC_KPOLICY_MAXPTS);
    for (int i = 0; i < n_points; ++i) {
        if (!(cost_rows[i] > 0.0) || !std::isfinite(cost_rows[i]) || (i && !(cost_rows[i] > cost_rows[i - 1])))
            return fail(SPEC_EINVAL, "spec_kpolicy_init: cost_rows must be positive and strictly increasing");
        if (!(cost_us[i] >= 0.0) || !std::isfinite(cost_us[i])) return fail(SPEC_EINVAL, "spec_kpolicy_init: cost_us must be finite and >= 0");
    }
    std::memset(p, 0, sizeof(*p));
    p->kmin = kmin;
    p->kmax = kmax;
    p->prior_p = prior_p;
    p->prior_n = prior_n;
    p->draft_us = draft_us;
    p->n_points = n_points;
    for (int i = 0; i < n_points; ++i) {
        p->cost_rows[i] = cost_rows[i];
        p->cost_us[i] = cost_us[i];
    }
    return SPEC_OK;
}

double spec_kpolicy_accept_prob(const spec_kpolicy* p, int32_t j) {
    return (p && j >= 0 && j < SPEC_KPOLICY_MAXK) ? accept_prob(p, j) : NAN;
}

double spec_kpolicy_verify_cost(const spec_kpolicy* p, double rows) {
    return (p && p->n_points >= 1) ? verify_cost(p, rows) : NAN;
}

double spec_kpolicy_expected_tokens(const spec_kpolicy* p, int32_t k) {
    return (p && k >= 0 && k <= SPEC_KPOLICY_MAXK) ? expected_tokens(p, k) : NAN;
}

int32_t spec_kpolicy_choose(const spec_kpolicy* p, int32_t B, int32_t row_cap) {
    if (!p || B < 1) return -1;
    int hi = p->kmax;
    if (row_cap > 0) {
        int cap = row_cap / B - 1;
        if (cap < p->kmin) cap = p->kmin;
        if (cap < hi) hi = cap;
    }
    int best = p->kmin;
    double best_cost = INFINITY;
    for (int k = p->kmin; k <= hi; ++k) {
        const double c = (verify_cost(p, (double)B * (k + 1)) + (k > 0 ? k * p->draft_us : 0.0)) / expected_tokens(p, k);
        if (c < best_cost) {
            best = k;
            best_cost = c;
        }
    }
    return best;
}

void spec_kpolicy_update(spec_kpolicy* p, int32_t k, int32_t accepted) {
    if (!p || k < 0 || accepted < 0) return;
    if (k > SPEC_KPOLICY_MAXK) k = SPEC_KPOLICY_MAXK;
    for (int j = 0; j < k; ++j) {
        if (j <= accepted) p->att[j] += 1.0;
        if (j < accepted) p->succ[j] += 1.0;
    }
}

int spec_kpolicy_update_batch(spec_kpolicy* p, const int32_t* k, const int32_t* accept_len, int32_t B) {
    using namespace sv;
    last_error().clear();
    if (!p || !k || !accept_len || B < 0) return fail(SPEC_EINVAL, "spec_kpolicy_update_batch: bad argument");
    for (int s = 0; s < B; ++s)
        if (accept_len[s] >= 0) spec_kpolicy_update(p, k[s], accept_len[s]);   // flagged sequences (-1) skipped
    return SPEC_OK;
}

}  // extern "C"
