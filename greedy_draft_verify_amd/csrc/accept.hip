// spec_greedy_accept: greedy acceptance and position rollback, plus the library's
// version and error-string entry points.
//
// One workgroup of 1024 threads: a block scan gives every sequence its row offset
// (ragged packing), then each wave takes sequences in turn. Within a wave, lane j
// compares draft j with the greedy token of row j; a ballot of the mismatches and
// a count of trailing ones give the accepted length in one step (the device-side
// prefix match of flashrt whole_step.py generate_speculative).
#include "common.h"

namespace sv {

std::string& last_error() {
    static thread_local std::string msg;
    return msg;
}

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    last_error() = buf;
    return code;
}

constexpr int kAcceptThreads = 1024;
constexpr int kAcceptMaxB = 8192;
constexpr int kMaxStop = 16;

// STOP: the emitted tokens end after the first stop token and after remaining[s]
// tokens (oxinfer step, DSSD _commit); pos advances by the tokens emitted.
template <bool STOP>
__global__ __launch_bounds__(kAcceptThreads) void accept_kernel(
    const int32_t* __restrict__ g, const int32_t* __restrict__ drafts, int kmax,
    const int32_t* __restrict__ k, const int32_t* __restrict__ d2t, int n_draft_vocab, int V, int B,
    int R, const int32_t* __restrict__ pos_in, int32_t* pos_out, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ n_emit, int32_t* __restrict__ emit, int32_t* __restrict__ next_tok,
    int32_t* __restrict__ status, const int32_t* __restrict__ stop_ids, int n_stop,
    const int32_t* __restrict__ remaining, int32_t* __restrict__ done) {
    __shared__ long long s_scan[kAcceptThreads];
    __shared__ int s_off[kAcceptMaxB];
    __shared__ int s_bad_k;
    const int tid = threadIdx.x;
    // -- row offsets (ragged packing)
    const bool packing_ok = block_row_offsets<kAcceptThreads>(k, B, R, s_scan, s_off, &s_bad_k);

    // -- one wave per sequence
    const int wave = tid / kWave, lane = tid % kWave;
    const int n_waves = kAcceptThreads / kWave;
    for (int s = wave; s < B; s += n_waves) {
        const int ks = k[s];
        const int off = s_off[s];
        int bits = 0;
        if (!packing_ok || ks > kmax) bits |= SPEC_STATUS_BAD_ROWS;
        if (pos_in[s] < 0) bits |= SPEC_STATUS_BAD_POS;
        int lim = 0x7fffffff;
        if constexpr (STOP) {
            if (remaining) {
                lim = remaining[s];
                if (!bits && lim < 1) bits = SPEC_STATUS_BAD_LIMIT;
            }
        }
        int32_t* e = emit + (size_t)s * (kmax + 1);
        if (bits) {
            for (int j = lane; j <= kmax; j += kWave) e[j] = -1;
            if (lane == 0) {
                status[s] = bits;
                accept_len[s] = -1;
                n_emit[s] = 0;
                next_tok[s] = -1;
                pos_out[s] = pos_in[s];
                if constexpr (STOP) done[s] = 0;
            }
            continue;
        }
        // first mismatch, 64 drafts at a time; token range checks over every used draft
        int a = ks;
        bool bad_tok = false;
        for (int base = 0; base < ks; base += kWave) {
            const int j = base + lane;
            bool miss = false;
            if (j < ks) {
                const int x = drafts[(size_t)s * kmax + j];
                int mapped = x;
                if (d2t) {
                    if (x < 0 || x >= n_draft_vocab) {
                        bad_tok = true;
                    } else {
                        mapped = d2t[x];
                        if (mapped < 0 || mapped >= V) bad_tok = true;
                    }
                } else if (x < 0 || x >= V) {
                    bad_tok = true;
                }
                miss = bad_tok || mapped != g[off + j];
            }
            const unsigned long long mm = __ballot(miss);
            if (mm && a == ks) a = base + (int)__builtin_ctzll(mm);
        }
        if (__ballot(bad_tok)) {
            for (int j = lane; j <= kmax; j += kWave) e[j] = -1;
            if (lane == 0) {
                status[s] = SPEC_STATUS_BAD_TOKEN;
                accept_len[s] = -1;
                n_emit[s] = 0;
                next_tok[s] = -1;
                pos_out[s] = pos_in[s];
                if constexpr (STOP) done[s] = 0;
            }
            continue;
        }
        if constexpr (STOP) {
            // out[j] = map(draft j) for j < a, out[a] = g[off + a]; c = up to and including the
            // first stop token, then at most lim tokens
            int c = a + 1;
            for (int base = 0; base <= a; base += kWave) {
                const int j = base + lane;
                bool is_stop = false;
                if (j <= a) {
                    int t;
                    if (j < a) {
                        const int x = drafts[(size_t)s * kmax + j];
                        t = d2t ? d2t[x] : x;
                    } else {
                        t = g[off + a];
                    }
                    for (int q = 0; q < n_stop; ++q) is_stop |= t == stop_ids[q];
                }
                const unsigned long long mm = __ballot(is_stop);
                if (mm && c == a + 1) c = base + (int)__builtin_ctzll(mm) + 1;
            }
            const bool at_lim = c >= lim;
            if (at_lim) c = lim;
            int last = -1;
            for (int j = lane; j <= kmax; j += kWave) {
                int val = -1;
                if (j < c) {
                    if (j < a) {
                        const int x = drafts[(size_t)s * kmax + j];
                        val = d2t ? d2t[x] : x;
                    } else {
                        val = g[off + a];
                    }
                }
                e[j] = val;
                if (j == c - 1) last = val;
            }
            // the last emitted token, from the lane that wrote it
            last = __shfl(last, (c - 1) % kWave);
            if (lane == 0) {
                bool is_stop = false;
                for (int q = 0; q < n_stop; ++q) is_stop |= last == stop_ids[q];
                status[s] = 0;
                accept_len[s] = a < c ? a : c;
                n_emit[s] = c;
                next_tok[s] = last;
                pos_out[s] = pos_in[s] + c;
                done[s] = is_stop || at_lim;
            }
            continue;
        }
        const int bonus = g[off + a];
        for (int j = lane; j <= kmax; j += kWave) {
            int val = -1;
            if (j < a) {
                const int x = drafts[(size_t)s * kmax + j];
                val = d2t ? d2t[x] : x;
            } else if (j == a) {
                val = bonus;
            }
            e[j] = val;
        }
        if (lane == 0) {
            const int p = pos_in[s];
            status[s] = 0;
            accept_len[s] = a;
            n_emit[s] = a + 1;
            next_tok[s] = bonus;
            pos_out[s] = p + a + 1;
        }
    }
}

// The stop rule on its own, applied in place to the outputs of any acceptance walk
// (greedy chain, tree, sampling): one wave per sequence, a ballot over the emitted
// tokens finds the first stop token, the tail of emit (and of the tree path) is
// cleared, and the per-sequence scalars are rewritten. No row offsets are needed,
// so the grid simply covers B with 4 waves per workgroup.
constexpr int kTruncThreads = 256;

__global__ __launch_bounds__(kTruncThreads) void truncate_kernel(
    int B, int kmax, const int32_t* __restrict__ stop_ids, int n_stop, const int32_t* __restrict__ remaining,
    const int32_t* __restrict__ pos_in, int32_t* __restrict__ pos_out, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ n_emit, int32_t* __restrict__ emit, int32_t* __restrict__ next_tok,
    int32_t* __restrict__ path, int32_t* __restrict__ done, int32_t* __restrict__ status) {
    const int lane = threadIdx.x % kWave;
    const int s = blockIdx.x * (kTruncThreads / kWave) + threadIdx.x / kWave;
    if (s >= B) return;
    const int st = status[s];
    const int a_in = accept_len[s];
    int c = n_emit[s];
    int32_t* e = emit + (size_t)s * (kmax + 1);
    int32_t* ph = path ? path + (size_t)s * kmax : nullptr;
    int flag = 0;
    if (st == 0) {
        if (c < 1 || c > kmax + 1 || a_in < 0 || a_in > c)
            flag = SPEC_STATUS_BAD_ROWS;
        else if (remaining && remaining[s] < 1)
            flag = SPEC_STATUS_BAD_LIMIT;
    }
    if (st || flag) {
        if (flag) {
            for (int j = lane; j <= kmax; j += kWave) e[j] = -1;
            if (ph)
                for (int j = lane; j < kmax; j += kWave) ph[j] = -1;
        }
        if (lane == 0) {
            if (flag) {
                status[s] = flag;
                accept_len[s] = -1;
                n_emit[s] = 0;
                next_tok[s] = -1;
                pos_out[s] = pos_in[s];
            }
            done[s] = 0;
        }
        return;
    }
    // first stop token among emit[0 .. c), 64 tokens at a time
    const int n = c;
    for (int base = 0; base < n; base += kWave) {
        const int j = base + lane;
        bool is_stop = false;
        if (j < n) {
            const int t = e[j];
            for (int q = 0; q < n_stop; ++q) is_stop |= t == stop_ids[q];
        }
        const unsigned long long mm = __ballot(is_stop);
        if (mm) {
            c = base + (int)__builtin_ctzll(mm) + 1;
            break;
        }
    }
    const bool at_lim = remaining && c >= remaining[s];
    if (at_lim) c = remaining[s];
    const int last = e[c - 1];
    const int a = a_in < c ? a_in : c;
    for (int j = c + lane; j <= kmax; j += kWave) e[j] = -1;
    if (ph)
        for (int j = a + lane; j < kmax; j += kWave) ph[j] = -1;
    if (lane == 0) {
        bool is_stop = false;
        for (int q = 0; q < n_stop; ++q) is_stop |= last == stop_ids[q];
        accept_len[s] = a;
        n_emit[s] = c;
        next_tok[s] = last;
        pos_out[s] = pos_in[s] + c;
        done[s] = is_stop || at_lim;
    }
}

}  // namespace sv

extern "C" {

int spec_version(void) { return 1; }

const char* spec_last_error(void) { return sv::last_error().c_str(); }

int spec_greedy_accept(const int32_t* argmax, const int32_t* drafts, int32_t kmax, const int32_t* k,
                       const int32_t* d2t, int32_t n_draft_vocab, int32_t V, int32_t B, int32_t R,
                       const int32_t* pos_in, int32_t* pos_out, int32_t* accept_len,
                       int32_t* n_emit, int32_t* emit, int32_t* next_tok, int32_t* seq_status,
                       void* stream) {
    using namespace sv;
    last_error().clear();
    if (B < 1 || B > kAcceptMaxB) return fail(SPEC_EINVAL, "spec_greedy_accept: B=%d outside 1..%d", B, kAcceptMaxB);
    if (kmax < 0 || kmax > 1024) return fail(SPEC_EINVAL, "spec_greedy_accept: kmax=%d outside 0..1024", kmax);
    if (R < 1) return fail(SPEC_EINVAL, "spec_greedy_accept: R=%d < 1", R);
    if (V < 1) return fail(SPEC_EINVAL, "spec_greedy_accept: V=%d < 1", V);
    if (d2t && n_draft_vocab < 1) return fail(SPEC_EINVAL, "spec_greedy_accept: d2t given with n_draft_vocab=%d", n_draft_vocab);
    if (!argmax || !k || !pos_in || !pos_out || !accept_len || !n_emit || !emit || !next_tok || !seq_status || (kmax > 0 && !drafts))
        return fail(SPEC_EINVAL, "spec_greedy_accept: null required pointer");
    hipLaunchKernelGGL(accept_kernel<false>, dim3(1), dim3(kAcceptThreads), 0, (hipStream_t)stream, argmax,
                       drafts, kmax, k, d2t, n_draft_vocab, V, B, R, pos_in, pos_out, accept_len,
                       n_emit, emit, next_tok, seq_status, nullptr, 0, nullptr, nullptr);
    SV_LAUNCH_CHECK("spec_greedy_accept");
    return SPEC_OK;
}

int spec_greedy_accept_stop(const int32_t* argmax, const int32_t* drafts, int32_t kmax, const int32_t* k,
                            const int32_t* d2t, int32_t n_draft_vocab, int32_t V, int32_t B, int32_t R,
                            const int32_t* stop_ids, int32_t n_stop, const int32_t* remaining,
                            const int32_t* pos_in, int32_t* pos_out, int32_t* accept_len, int32_t* n_emit,
                            int32_t* emit, int32_t* next_tok, int32_t* done, int32_t* seq_status, void* stream) {
    using namespace sv;
    last_error().clear();
    if (B < 1 || B > kAcceptMaxB) return fail(SPEC_EINVAL, "spec_greedy_accept_stop: B=%d outside 1..%d", B, kAcceptMaxB);
    if (kmax < 0 || kmax > 1024) return fail(SPEC_EINVAL, "spec_greedy_accept_stop: kmax=%d outside 0..1024", kmax);
    if (R < 1) return fail(SPEC_EINVAL, "spec_greedy_accept_stop: R=%d < 1", R);
    if (V < 1) return fail(SPEC_EINVAL, "spec_greedy_accept_stop: V=%d < 1", V);
    if (n_stop < 0 || n_stop > kMaxStop) return fail(SPEC_EINVAL, "spec_greedy_accept_stop: n_stop=%d outside 0..%d", n_stop, kMaxStop);
    if (d2t && n_draft_vocab < 1) return fail(SPEC_EINVAL, "spec_greedy_accept_stop: d2t given with n_draft_vocab=%d", n_draft_vocab);
    if (!argmax || !k || !pos_in || !pos_out || !accept_len || !n_emit || !emit || !next_tok || !done || !seq_status ||
        (kmax > 0 && !drafts) || (n_stop > 0 && !stop_ids))
        return fail(SPEC_EINVAL, "spec_greedy_accept_stop: null required pointer");
    hipLaunchKernelGGL(accept_kernel<true>, dim3(1), dim3(kAcceptThreads), 0, (hipStream_t)stream, argmax,
                       drafts, kmax, k, d2t, n_draft_vocab, V, B, R, pos_in, pos_out, accept_len,
                       n_emit, emit, next_tok, seq_status, stop_ids, n_stop, remaining, done);
    SV_LAUNCH_CHECK("spec_greedy_accept_stop");
    return SPEC_OK;
}

int spec_truncate_stop(int32_t kmax, int32_t B, const int32_t* stop_ids, int32_t n_stop, const int32_t* remaining,
                       const int32_t* pos_in, int32_t* pos_out, int32_t* accept_len, int32_t* n_emit, int32_t* emit,
                       int32_t* next_tok, int32_t* path, int32_t* done, int32_t* seq_status, void* stream) {
    using namespace sv;
    last_error().clear();
    if (B < 1) return fail(SPEC_EINVAL, "spec_truncate_stop: B=%d < 1", B);
    if (kmax < 0 || kmax > 1024) return fail(SPEC_EINVAL, "spec_truncate_stop: kmax=%d outside 0..1024", kmax);
    if (n_stop < 0 || n_stop > kMaxStop) return fail(SPEC_EINVAL, "spec_truncate_stop: n_stop=%d outside 0..%d", n_stop, kMaxStop);
    if (!pos_in || !pos_out || !accept_len || !n_emit || !emit || !next_tok || !done || !seq_status ||
        (n_stop > 0 && !stop_ids))
        return fail(SPEC_EINVAL, "spec_truncate_stop: null required pointer");
    constexpr int per_wg = kTruncThreads / kWave;
    hipLaunchKernelGGL(truncate_kernel, dim3((B + per_wg - 1) / per_wg), dim3(kTruncThreads), 0, (hipStream_t)stream,
                       B, kmax, stop_ids, n_stop, remaining, pos_in, pos_out, accept_len, n_emit, emit, next_tok,
                       path, done, seq_status);
    SV_LAUNCH_CHECK("spec_truncate_stop");
    return SPEC_OK;
}

}  // extern "C"
