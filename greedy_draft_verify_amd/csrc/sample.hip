// spec_sample_accept: the chain walk of speculative sampling (DSSD fast.py
// _sample_verify; oxinfer speculative_accept): draft j of sequence s (row
// r = off_s + j) is kept iff u_r < p_r(x) / q_r(x), with u_r the row's acceptance
// uniform (Philox, counter (0, row_ctr[r], 1), word 0), p_r(x) = exp(z_r(x) - lse_r)
// from spec_lm_head_sample and q_r(x) the draft's mass in its support. At the first
// rejection the row's residual draw is emitted; if every draft is kept, the bonus
// row's draw from p.
//
// One workgroup of 1024 threads: the block scan of the greedy call gives the row
// offsets, then one wave per sequence; lane j tests draft j (64 at a time) and a
// ballot of the rejections gives the first one.
#include "common.h"

namespace sv {

constexpr int kSampleThreads = 1024;
constexpr int kSampleMaxB = 8192;

__global__ __launch_bounds__(kSampleThreads) void sample_accept_kernel(
    const int32_t* __restrict__ drafts, int kmax, const int32_t* __restrict__ k, const int32_t* __restrict__ d2t,
    int n_draft_vocab, int V, int B, int R, const int32_t* __restrict__ q_tok, const float* __restrict__ q_prob,
    int NQ, const float* __restrict__ lse, const float* __restrict__ z_supp, const int32_t* __restrict__ sample_p,
    const int32_t* __restrict__ sample_res, const int32_t* __restrict__ row_ctr, uint32_t key0, uint32_t key1,
    const int32_t* __restrict__ pos_in, int32_t* pos_out, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ n_emit, int32_t* __restrict__ emit, int32_t* __restrict__ next_tok,
    int32_t* __restrict__ status) {
    __shared__ long long s_scan[kSampleThreads];
    __shared__ int s_off[kSampleMaxB];
    __shared__ int s_bad_k;
    const int tid = threadIdx.x;
    const bool packing_ok = block_row_offsets<kSampleThreads>(k, B, R, s_scan, s_off, &s_bad_k);

    const int wave = tid / kWave, lane = tid % kWave;
    constexpr int n_waves = kSampleThreads / kWave;
    for (int s = wave; s < B; s += n_waves) {
        const int ks = k[s];
        const int off = s_off[s];
        int bits = 0;
        if (!packing_ok || ks > kmax) bits |= SPEC_STATUS_BAD_ROWS;
        if (pos_in[s] < 0) bits |= SPEC_STATUS_BAD_POS;
        int32_t* e = emit + (size_t)s * (kmax + 1);
        int a = ks;
        bool bad_tok = false;
        if (!bits) {
            for (int base = 0; base < ks; base += kWave) {
                const int j = base + lane;
                bool rej = false;
                if (j < ks) {
                    const int x = drafts[(size_t)s * kmax + j];
                    int t = x;
                    if (d2t) {
                        if (x < 0 || x >= n_draft_vocab) {
                            bad_tok = true;
                        } else {
                            t = d2t[x];
                            if (t < 0 || t >= V) bad_tok = true;
                        }
                    } else if (x < 0 || x >= V) {
                        bad_tok = true;
                    }
                    const size_t r = (size_t)off + j;
                    int q_e = -1;
                    for (int q = 0; q < NQ && !bad_tok; ++q)
                        if (q_tok[r * NQ + q] == t && q_prob[r * NQ + q] > 0.f) {
                            q_e = q;
                            break;
                        }
                    if (q_e < 0) {
                        bad_tok = true;
                    } else {
                        const float px = __expf(z_supp[r * NQ + q_e] - lse[r]);
                        const uint4 w = philox10(make_uint4(0u, (uint32_t)row_ctr[2 * r], (uint32_t)row_ctr[2 * r + 1], 1u),
                                                 key0, key1);
                        rej = !(u01_23(w.x) < px / q_prob[r * NQ + q_e]);
                    }
                }
                const unsigned long long mm = __ballot(rej);
                if (mm && a == ks) a = base + (int)__builtin_ctzll(mm);
            }
            if (__ballot(bad_tok)) bits |= SPEC_STATUS_BAD_TOKEN;
        }
        if (bits) {
            for (int j = lane; j <= kmax; j += kWave) e[j] = -1;
            if (lane == 0) {
                status[s] = bits;
                accept_len[s] = -1;
                n_emit[s] = 0;
                next_tok[s] = -1;
                pos_out[s] = pos_in[s];
            }
            continue;
        }
        const int tok = a < ks ? sample_res[off + a] : sample_p[off + ks];
        for (int j = lane; j <= kmax; j += kWave) {
            int val = -1;
            if (j < a) {
                const int x = drafts[(size_t)s * kmax + j];
                val = d2t ? d2t[x] : x;
            } else if (j == a) {
                val = tok;
            }
            e[j] = val;
        }
        if (lane == 0) {
            status[s] = 0;
            accept_len[s] = a;
            n_emit[s] = a + 1;
            next_tok[s] = tok;
            pos_out[s] = pos_in[s] + a + 1;
        }
    }
}

}  // namespace sv

extern "C" {

int spec_sample_accept(const int32_t* drafts, int32_t kmax, const int32_t* k, const int32_t* d2t,
                       int32_t n_draft_vocab, int32_t V, int32_t B, int32_t R, const int32_t* q_tok,
                       const float* q_prob, int32_t NQ, const float* lse, const float* z_supp,
                       const int32_t* sample_p, const int32_t* sample_res, const int32_t* row_ctr, uint64_t seed,
                       const int32_t* pos_in, int32_t* pos_out, int32_t* accept_len, int32_t* n_emit,
                       int32_t* emit, int32_t* next_tok, int32_t* seq_status, void* stream) {
    using namespace sv;
    last_error().clear();
    if (B < 1 || B > kSampleMaxB) return fail(SPEC_EINVAL, "spec_sample_accept: B=%d outside 1..%d", B, kSampleMaxB);
    if (kmax < 0 || kmax > 1024) return fail(SPEC_EINVAL, "spec_sample_accept: kmax=%d outside 0..1024", kmax);
    if (R < 1) return fail(SPEC_EINVAL, "spec_sample_accept: R=%d < 1", R);
    if (V < 1) return fail(SPEC_EINVAL, "spec_sample_accept: V=%d < 1", V);
    if (NQ < 0 || NQ > 8) return fail(SPEC_EINVAL, "spec_sample_accept: NQ=%d outside 0..8", NQ);
    if (d2t && n_draft_vocab < 1) return fail(SPEC_EINVAL, "spec_sample_accept: d2t given with n_draft_vocab=%d", n_draft_vocab);
    if (!k || !lse || !sample_p || !sample_res || !row_ctr || !pos_in || !pos_out || !accept_len || !n_emit || !emit ||
        !next_tok || !seq_status || (kmax > 0 && (!drafts || (NQ > 0 && (!q_tok || !q_prob || !z_supp)))))
        return fail(SPEC_EINVAL, "spec_sample_accept: null required pointer");
    hipLaunchKernelGGL(sample_accept_kernel, dim3(1), dim3(kSampleThreads), 0, (hipStream_t)stream, drafts, kmax, k,
                       d2t, n_draft_vocab, V, B, R, q_tok, q_prob, NQ, lse, z_supp, sample_p, sample_res, row_ctr,
                       (uint32_t)seed, (uint32_t)(seed >> 32), pos_in, pos_out, accept_len, n_emit, emit, next_tok,
                       seq_status);
    SV_LAUNCH_CHECK("spec_sample_accept");
    return SPEC_OK;
}

}  // extern "C"
