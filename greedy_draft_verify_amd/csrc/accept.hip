// spec_greedy_accept: greedy acceptance and position rollback, plus the library's
// version and error-string entry points.
//
// Workgroups of 1024 threads, each computing every sequence's row offset (ragged
// packing) by a block scan and then taking its sequences, a wave per sequence.
// Within a wave, lane j compares draft j with the greedy token of row j; a ballot
// of the mismatches and a count of trailing ones give the accepted length in one
// step (the device-side prefix match of flashrt whole_step.py generate_speculative).
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
constexpr int kMaxStop = 16;

// STOP: the emitted tokens end after the first stop token and after remaining[s]
// tokens (oxinfer step, DSSD _commit); pos advances by the tokens emitted.
//
// Latency: each workgroup computes the row offsets itself (the scan reads only k)
// and takes every (gridDim.x)-th group of 16 sequences, a wave per sequence. A
// wave's first sequence has its scalars and drafts requested before the scan and
// its greedy tokens right after it; the bonus token and the emitted tokens are then
// taken from registers (draft j and row j live in lane j), so a sequence with
// k < 64 costs two dependent global round trips.
// One sequence's acceptance, by one wave. gs[j] is the greedy token of the sequence's
// row j (j <= ks), in global memory or LDS; ks, p, lim and x (lane j's draft j) are
// loaded and bits holds the flags of the sequence found by the caller.
template <bool STOP>
__device__ __forceinline__ void accept_one(
    int s, int lane, const int32_t* gs, int bits, int ks, int p, int lim, int x, const int32_t* __restrict__ drafts,
    int kmax, const int32_t* __restrict__ d2t, int n_draft_vocab, int V, int32_t* pos_out,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ n_emit, int32_t* __restrict__ emit,
    int32_t* __restrict__ next_tok, int32_t* __restrict__ status, const int* s_stop, int n_stop,
    int32_t* __restrict__ done) {
    int32_t* e = emit + (size_t)s * (kmax + 1);
    auto flag = [&](int why) {
        for (int j = lane; j <= kmax; j += kWave) e[j] = -1;
        if (lane == 0) {
            status[s] = why;
            accept_len[s] = -1;
            n_emit[s] = 0;
            next_tok[s] = -1;
            pos_out[s] = p;
            if constexpr (STOP) done[s] = 0;
        }
    };
    if (bits) {
        flag(bits);
        return;
    }
    // rows off .. off + ks are in range (the packing is defined); lane j < 64 holds
    // draft j mapped (x0) and the greedy token of row j (g0)
    const int g0 = lane <= ks ? gs[lane] : 0;
    bool bad_tok = false;
    auto map_draft = [&](int xv, bool& bad) {
        if (d2t) {
            if (xv < 0 || xv >= n_draft_vocab) {
                bad = true;
                return 0;
            }
            const int m = d2t[xv];
            if (m < 0 || m >= V) bad = true;
            return m;
        }
        if (xv < 0 || xv >= V) bad = true;
        return xv;
    };
    const int x0 = lane < ks ? map_draft(x, bad_tok) : 0;
    // first mismatch; token range checks over every used draft
    int a = ks;
    {
        const unsigned long long mm = __ballot(lane < ks && (bad_tok || x0 != g0));
        if (mm) a = (int)__builtin_ctzll(mm);
    }
    for (int base = kWave; base < ks; base += kWave) {
        const int j = base + lane;
        bool miss = false;
        if (j < ks) {
            const int mj = map_draft(drafts[(size_t)s * kmax + j], bad_tok);
            miss = bad_tok || mj != gs[j];
        }
        const unsigned long long mm = __ballot(miss);
        if (mm && a == ks) a = base + (int)__builtin_ctzll(mm);
    }
    if (__ballot(bad_tok)) {
        flag(SPEC_STATUS_BAD_TOKEN);
        return;
    }
    // token j of the output: mapped draft j for j < a, the greedy token of row a at a
    const int g_a = a < kWave ? __shfl(g0, a) : gs[a];
    auto token = [&](int j) {
        if (j == a) return g_a;
        if (j < kWave) return x0;   // j == lane
        const int xv = drafts[(size_t)s * kmax + j];
        return d2t ? d2t[xv] : xv;
    };
    int c = a + 1;   // tokens emitted
    if constexpr (STOP) {
        // up to and including the first stop token, then at most lim tokens
        for (int base = 0; base <= a; base += kWave) {
            const int j = base + lane;
            bool is_stop = false;
            if (j <= a) {
                const int t = token(j);
                for (int q = 0; q < n_stop; ++q) is_stop |= t == s_stop[q];
            }
            const unsigned long long mm = __ballot(is_stop);
            if (mm && c == a + 1) c = base + (int)__builtin_ctzll(mm) + 1;
        }
    }
    const bool at_lim = c >= lim;
    if (at_lim) c = lim;
    int last = -1;
    for (int j = lane; j <= kmax; j += kWave) {
        const int val = j < c ? token(j) : -1;
        e[j] = val;
        if (j == c - 1) last = val;
    }
    // the last emitted token, from the lane that wrote it
    last = __shfl(last, (c - 1) % kWave);
    if (lane == 0) {
        status[s] = 0;
        accept_len[s] = a < c ? a : c;
        n_emit[s] = c;
        next_tok[s] = last;
        pos_out[s] = p + c;
        if constexpr (STOP) {
            bool is_stop = false;
            for (int q = 0; q < n_stop; ++q) is_stop |= last == s_stop[q];
            done[s] = is_stop || at_lim;
        }
    }
}

template <bool STOP>
__global__ __launch_bounds__(kAcceptThreads) void accept_kernel(
    const int32_t* __restrict__ g, const int32_t* __restrict__ drafts, int kmax,
    const int32_t* __restrict__ k, const int32_t* __restrict__ d2t, int n_draft_vocab, int V, int B,
    int R, const int32_t* __restrict__ pos_in, int32_t* pos_out, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ n_emit, int32_t* __restrict__ emit, int32_t* __restrict__ next_tok,
    int32_t* __restrict__ status, const int32_t* __restrict__ stop_ids, int n_stop,
    const int32_t* __restrict__ remaining, int32_t* __restrict__ done) {
    constexpr int NW = kAcceptThreads / kWave;
    __shared__ long long s_wsum[NW];
    __shared__ int s_wbad[NW];
    __shared__ int s_off[kAcceptMaxB];
    __shared__ int s_stop[kMaxStop];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    if (STOP && tid < n_stop) s_stop[tid] = stop_ids[tid];   // visible after the scan's barriers

    // the first sequence of this wave: requested before the scan
    const int s_first = blockIdx.x * NW + wave;
    int ks = 0, p = 0, lim = 0x7fffffff, x = 0;
    if (s_first < B) {
        ks = k[s_first];
        p = pos_in[s_first];
        if (STOP && remaining) lim = remaining[s_first];
        if (lane < kmax) x = drafts[(size_t)s_first * kmax + lane];
    }
    const bool packing_ok = block_row_offsets<kAcceptThreads>(k, B, R, s_wsum, s_wbad, s_off);

    for (int s = s_first; s < B; s += gridDim.x * NW) {
        if (s != s_first) {
            ks = k[s];
            p = pos_in[s];
            if (STOP && remaining) lim = remaining[s];
            x = lane < kmax ? drafts[(size_t)s * kmax + lane] : 0;
        }
        const int off = s_off[s];
        int bits = 0;
        if (!packing_ok || ks > kmax) bits |= SPEC_STATUS_BAD_ROWS;
        if (p < 0) bits |= SPEC_STATUS_BAD_POS;
        if (STOP && remaining && !bits && lim < 1) bits = SPEC_STATUS_BAD_LIMIT;
        accept_one<STOP>(s, lane, g + off, bits, ks, p, lim, x, drafts, kmax, d2t, n_draft_vocab, V, pos_out,
                         accept_len, n_emit, emit, next_tok, status, s_stop, n_stop, done);
    }
}

// The greedy step's argmax finalize fused with the acceptance (the lm_head's few-row
// path stores one key per (vocabulary workgroup, row); this kernel stands in for its
// finalize and for accept_kernel). One workgroup per sequence: it merges the keys of
// the sequence's own rows into their greedy tokens (the maximum key, as the finalize
// takes it), writes argmax (and maxval) for those rows, writes back as zero every key
// it read, and one wave then takes the sequence's acceptance with the tokens in LDS.
// With an undefined packing (every sequence flagged) workgroup s takes the rows
// s*R/B .. (s+1)*R/B - 1 instead, so argmax is still written and the keys cleared.
__global__ __launch_bounds__(kAcceptThreads) void argmax_accept_kernel(
    unsigned long long* __restrict__ key_rows, int n_vt, int stride, int R, int32_t* __restrict__ argmax,
    float* __restrict__ maxval, const int32_t* __restrict__ drafts, int kmax, const int32_t* __restrict__ k,
    const int32_t* __restrict__ d2t, int n_draft_vocab, int V, int B, const int32_t* __restrict__ pos_in,
    int32_t* pos_out, int32_t* __restrict__ accept_len, int32_t* __restrict__ n_emit,
    int32_t* __restrict__ emit, int32_t* __restrict__ next_tok, int32_t* __restrict__ status) {
    constexpr int NW = kAcceptThreads / kWave;
    __shared__ long long s_wsum[NW];
    __shared__ int s_wbad[NW];
    __shared__ int s_off[kAcceptMaxB];
    __shared__ unsigned long long s_best[kArgmaxAcceptMaxRows];
    __shared__ int s_g[kArgmaxAcceptMaxRows];
    const int tid = threadIdx.x, lane = tid % kWave, s = blockIdx.x;
    // the sequence's scalars and drafts (wave 0 takes the acceptance), requested
    // before the scan
    const int ks = k[s];
    int p = 0, x = 0;
    if (tid < kWave) {
        p = pos_in[s];
        if (lane < kmax) x = drafts[(size_t)s * kmax + lane];
    }
    if (tid < kArgmaxAcceptMaxRows) s_best[tid] = 0ull;   // visible after the scan's barriers
    const bool packing_ok = block_row_offsets<kAcceptThreads>(k, B, R, s_wsum, s_wbad, s_off);
    int r_lo, n_rows;
    if (packing_ok) {
        r_lo = s_off[s];
        n_rows = ks + 1;   // rows r_lo .. r_lo + ks < R
    } else {
        r_lo = (int)((long long)s * R / B);
        n_rows = (int)((long long)(s + 1) * R / B) - r_lo;
    }
    // thread t: row t % n_rows, every (per)-th vocabulary workgroup from t / n_rows, a
    // batch of 8 keys requested before any is used (neighbouring threads read
    // neighbouring keys of one vocabulary workgroup's row block); the maxima meet in
    // LDS. (Measured slower at 16 sequences of 5 rows: whole waves or lane groups per
    // row merged by shuffles, each lane reading its own row block, 14.5 vs 9.4 us;
    // 16-byte loads of the aligned key pairs holding the rows, 11.1 us.)
    if (n_rows > 0) {
        const int per = kAcceptThreads / n_rows;
        const int j = tid % n_rows, v0 = tid / n_rows;
        if (v0 < per) {
            unsigned long long* col = key_rows + r_lo + j;
            unsigned long long best = 0ull;
            for (int i0 = v0; i0 < n_vt; i0 += 8 * per) {
                unsigned long long kk[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int i = i0 + u * per;
                    kk[u] = i < n_vt ? col[(size_t)i * stride] : 0ull;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int i = i0 + u * per;
                    best = kk[u] > best ? kk[u] : best;
                    if (i < n_vt) col[(size_t)i * stride] = 0ull;
                }
            }
            atomicMax(&s_best[j], best);
        }
    }
    __syncthreads();
    if (tid < n_rows) {
        const unsigned long long key = s_best[tid];
        const int gv = (int32_t)~(uint32_t)key;
        s_g[tid] = gv;
        argmax[r_lo + tid] = gv;
        if (maxval) maxval[r_lo + tid] = unpack_value(key);
    }
    __syncthreads();
    if (tid < kWave) {
        int bits = 0;
        if (!packing_ok || ks > kmax) bits |= SPEC_STATUS_BAD_ROWS;
        if (p < 0) bits |= SPEC_STATUS_BAD_POS;
        accept_one<false>(s, lane, s_g, bits, ks, p, 0x7fffffff, x, drafts, kmax, d2t, n_draft_vocab, V, pos_out,
                          accept_len, n_emit, emit, next_tok, status, nullptr, 0, nullptr);
    }
}

int launch_argmax_accept(unsigned long long* key_rows, int n_vt, int stride, int R, int32_t* argmax, float* maxval,
                         const int32_t* drafts, int kmax, const int32_t* k, const int32_t* d2t, int n_draft_vocab,
                         int V, int B, const int32_t* pos_in, int32_t* pos_out, int32_t* accept_len, int32_t* n_emit,
                         int32_t* emit, int32_t* next_tok, int32_t* status, hipStream_t st) {
    hipLaunchKernelGGL(argmax_accept_kernel, dim3(B), dim3(kAcceptThreads), 0, st, key_rows, n_vt, stride, R, argmax,
                       maxval, drafts, kmax, k, d2t, n_draft_vocab, V, B, pos_in, pos_out, accept_len, n_emit, emit,
                       next_tok, status);
    return SPEC_OK;
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
    hipLaunchKernelGGL(accept_kernel<false>, dim3(seq_grid(B, kAcceptThreads)), dim3(kAcceptThreads), 0, (hipStream_t)stream, argmax,
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
    hipLaunchKernelGGL(accept_kernel<true>, dim3(seq_grid(B, kAcceptThreads)), dim3(kAcceptThreads), 0, (hipStream_t)stream, argmax,
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
