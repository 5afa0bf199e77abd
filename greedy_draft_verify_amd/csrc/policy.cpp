// Adaptive draft depth (span-02 spec.rs KPolicy; oxinfer DraftCosts): host-side
// arithmetic on a caller-owned struct, no GPU work. A decoding loop keeps one
// spec_kpolicy, asks spec_kpolicy_choose for the next round's k and feeds the round's
// accept lengths back with spec_kpolicy_update (or _update_batch). The verify cost
// points are the caller's own measurement of the verify step against its rows.
//
// choose tabulates, once per call, the all-kept probabilities S_i = p_0 ... p_{i-1}
// and their running sums E(k) = S_0 + ... + S_k, then scans the candidate depths.
#include <algorithm>
#include <cmath>
#include <cstring>

#include "common.h"

namespace {

constexpr int kMaxK = SPEC_KPOLICY_MAXK;

double smoothed_rate(const spec_kpolicy& pol, int j) {
    const double pseudo_kept = pol.prior_p * pol.prior_n;
    return (pol.kept[j] + pseudo_kept) / (pol.tried[j] + pol.prior_n);
}

// E[0..k]: expected emitted tokens per sequence for every depth up to k.
void expected_table(const spec_kpolicy& pol, int k, double* E) {
    double survive = 1.0;   // S_i
    double running = 0.0;
    for (int i = 0; i <= k; ++i) {
        running += survive;
        E[i] = running;
        if (i < kMaxK) survive *= smoothed_rate(pol, i);
    }
}

// The polyline through the origin and the measured points. The piece used for r is
// the one whose right corner is the first corner at or beyond r; before the origin
// that is the first piece, and past the last point the last piece continues.
double polyline(const spec_kpolicy& pol, double r) {
    const double* xs = pol.cost_rows;
    const double* ys = pol.cost_us;
    const int n = pol.n_points;
    const int right = std::min<int>(static_cast<int>(std::lower_bound(xs, xs + n, r) - xs), n - 1);
    const double xr = xs[right], yr = ys[right];
    const double xl = right > 0 ? xs[right - 1] : 0.0;
    const double yl = right > 0 ? ys[right - 1] : 0.0;
    return yl + (yr - yl) * (r - xl) / (xr - xl);
}

}  // namespace

extern "C" {

int spec_kpolicy_init(spec_kpolicy* p, int32_t kmin, int32_t kmax, double prior_p, double prior_n, double draft_us,
                      const double* cost_rows, const double* cost_us, int32_t n_points) {
    using namespace sv;
    last_error().clear();
    if (!p || !cost_rows || !cost_us) return fail(SPEC_EINVAL, "spec_kpolicy_init: null pointer");
    if (kmin < 0 || kmax < kmin || kmax >= kMaxK)
        return fail(SPEC_EINVAL, "spec_kpolicy_init: need 0 <= kmin <= kmax < %d (kmin=%d kmax=%d)", kMaxK, kmin, kmax);
    if (!(prior_p > 0.0 && prior_p <= 1.0) || !(prior_n > 0.0) || !std::isfinite(prior_n))
        return fail(SPEC_EINVAL, "spec_kpolicy_init: need 0 < prior_p <= 1 and prior_n > 0");
    if (!(draft_us >= 0.0) || !std::isfinite(draft_us)) return fail(SPEC_EINVAL, "spec_kpolicy_init: draft_us must be >= 0");
    if (n_points < 1 || n_points > SPEC_KPOLICY_MAXPTS)
        return fail(SPEC_EINVAL, "spec_kpolicy_init: n_points=%d outside 1..%d", n_points, SPEC_KPOLICY_MAXPTS);
    double prev = 0.0;
    for (int i = 0; i < n_points; ++i) {
        if (!std::isfinite(cost_rows[i]) || !(cost_rows[i] > prev))
            return fail(SPEC_EINVAL, "spec_kpolicy_init: cost_rows must be positive and strictly increasing");
        if (!std::isfinite(cost_us[i]) || !(cost_us[i] >= 0.0))
            return fail(SPEC_EINVAL, "spec_kpolicy_init: cost_us must be finite and >= 0");
        prev = cost_rows[i];
    }
    spec_kpolicy fresh;
    std::memset(&fresh, 0, sizeof(fresh));
    fresh.kmin = kmin;
    fresh.kmax = kmax;
    fresh.prior_p = prior_p;
    fresh.prior_n = prior_n;
    fresh.draft_us = draft_us;
    fresh.n_points = n_points;
    std::copy(cost_rows, cost_rows + n_points, fresh.cost_rows);
    std::copy(cost_us, cost_us + n_points, fresh.cost_us);
    *p = fresh;
    return SPEC_OK;
}

double spec_kpolicy_accept_prob(const spec_kpolicy* p, int32_t j) {
    if (!p || j < 0 || j >= kMaxK) return NAN;
    return smoothed_rate(*p, j);
}

double spec_kpolicy_verify_cost(const spec_kpolicy* p, double rows) {
    if (!p || p->n_points < 1) return NAN;
    return polyline(*p, rows);
}

double spec_kpolicy_expected_tokens(const spec_kpolicy* p, int32_t k) {
    if (!p || k < 0 || k > kMaxK) return NAN;
    double E[kMaxK + 1];
    expected_table(*p, k, E);
    return E[k];
}

int32_t spec_kpolicy_choose(const spec_kpolicy* p, int32_t B, int32_t row_cap) {
    if (!p || B < 1) return -1;
    const int top = row_cap > 0 ? std::min<int>(p->kmax, std::max<int>(row_cap / B - 1, p->kmin)) : p->kmax;
    double E[kMaxK + 1];
    expected_table(*p, top, E);
    int pick = p->kmin;
    double least = INFINITY;
    for (int k = p->kmin; k <= top; ++k) {
        const double per_token = (polyline(*p, (double)B * (k + 1)) + k * p->draft_us) / E[k];
        if (per_token < least) {   // strict: the smaller k keeps a tie
            least = per_token;
            pick = k;
        }
    }
    return pick;
}

void spec_kpolicy_update(spec_kpolicy* p, int32_t k, int32_t accepted) {
    if (!p || k < 0 || accepted < 0) return;
    const int depth = std::min<int>(k, kMaxK);
    const int reached = std::min(depth, accepted + 1);   // positions whose draft was tested
    const int kept = std::min(depth, accepted);          // ... and kept
    for (int j = 0; j < reached; ++j) p->tried[j] += 1.0;
    for (int j = 0; j < kept; ++j) p->kept[j] += 1.0;
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
