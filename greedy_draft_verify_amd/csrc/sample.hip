// spec_sample_accept: the chain walk of speculative sampling (DSSD fast.py
// _sample_verify; oxinfer speculative_accept): draft j of sequence s (row
// r = off_s + j) is kept iff u_r < p_r(x) / q_r(x), with u_r the row's acceptance
// uniform (Philox, counter (0, row_ctr[r], 1), word 0), p_r(x) = exp(z_r(x) - lse_r)
// from spec_lm_head_sample and q_r(x) the draft's mass in its support. At the first
// rejection the row's residual draw is emitted; if every draft is kept, the bonus
// row's draw from p.
//
// Workgroups of 1024 threads, each computing the row offsets by the block scan of
// the greedy call, then a wave per sequence (16 sequences per workgroup); lane j
// tests draft j (64 at a time) and a ballot of the rejections gives the first one.
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
    __shared__ long long s_wsum[kSampleThreads / kWave];
    __shared__ int s_wbad[kSampleThreads / kWave];
    __shared__ int s_off[kSampleMaxB];
    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    constexpr int n_waves = kSampleThreads / kWave;
    // the first sequence of this wave: requested before the scan
    const int s_first = blockIdx.x * n_waves + wave;
    int ks = 0, p = 0, x = 0;
    if (s_first < B) {
        ks = k[s_first];
        p = pos_in[s_first];
        if (lane < kmax) x = drafts[(size_t)s_first * kmax + lane];
    }
    const bool packing_ok = block_row_offsets<kSampleThreads>(k, B, R, s_wsum, s_wbad, s_off);

    for (int s = s_first; s < B; s += gridDim.x * n_waves) {
        if (s != s_first) {
            ks = k[s];
            p = pos_in[s];
            x = lane < kmax ? drafts[(size_t)s * kmax + lane] : 0;
        }
        const int off = s_off[s];
        int bits = 0;
        if (!packing_ok || ks > kmax) bits |= SPEC_STATUS_BAD_ROWS;
        if (p < 0) bits |= SPEC_STATUS_BAD_POS;
        int32_t* e = emit + (size_t)s * (kmax + 1);
        auto flag = [&](int why) {
            for (int jj = lane; jj <= kmax; jj += kWave) e[jj] = -1;
            if (lane == 0) {
                status[s] = why;
                accept_len[s] = -1;
                n_emit[s] = 0;
                next_tok[s] = -1;
                pos_out[s] = p;
            }
        };
        if (bits) {
            flag(bits);
            continue;
        }
        // Rows off .. off + ks are in range (the packing is defined). Draft j (row
        // off + j) maps to t; it is kept iff u_r < p(t) / q(t), where q(t) is the
        // summed mass of the support entries holding t, the q of the residual draw
        // (not positive: the draft is out of its support, BAD_TOKEN); p(t) comes from
        // the z of the first entry holding t. A row's support, masses, z values, lse
        // and counters are requested together.
        auto test = [&](int j, int xv, int& t, bool& bad) {
            t = xv;
            if (d2t) {
                if (xv < 0 || xv >= n_draft_vocab) {
                    bad = true;
                    return false;
                }
                t = d2t[xv];
                if (t < 0 || t >= V) bad = true;
            } else if (xv < 0 || xv >= V) {
                bad = true;
            }
            if (bad) return false;
            const size_t r = (size_t)off + j;
            int qt[8];
            float qp[8], zs[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                qt[q] = q < NQ ? q_tok[r * NQ + q] : -1;
                qp[q] = q < NQ ? q_prob[r * NQ + q] : 0.f;
                zs[q] = q < NQ ? z_supp[r * NQ + q] : 0.f;
            }
            const float lr = lse[r];
            const uint32_t ca = (uint32_t)row_ctr[2 * r], cb = (uint32_t)row_ctr[2 * r + 1];
            // entries in ascending order: the mass summed, the first entry's z kept
            float zq = 0.f, pq = 0.f;
            bool found = false;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (q < NQ && qt[q] == t) {
                    if (!found) zq = zs[q];
                    found = true;
                    pq += qp[q];
                }
            if (!(pq > 0.f)) {
                bad = true;
                return false;
            }
            const float px = __expf(zq - lr);
            const uint4 w = philox10(make_uint4(0u, ca, cb, 1u), key0, key1);
            return !(u01_23(w.x) < px / pq);
        };
        int a = ks;
        bool bad_tok = false;
        int t0 = 0;   // lane j < 64: draft j mapped
        for (int base = 0; base < ks; base += kWave) {
            const int j = base + lane;
            bool rej = false;
            int t = 0;
            if (j < ks) rej = test(j, base == 0 ? x : drafts[(size_t)s * kmax + j], t, bad_tok);
            if (base == 0) t0 = t;
            const unsigned long long mm = __ballot(rej);
            if (mm && a == ks) a = base + (int)__builtin_ctzll(mm);
        }
        if (__ballot(bad_tok)) {
            flag(SPEC_STATUS_BAD_TOKEN);
            continue;
        }
        // the residual draw of the first rejected row, or the bonus row's draw from p
        const int tok = a < ks ? sample_res[off + a] : sample_p[off + ks];
        for (int jj = lane; jj <= kmax; jj += kWave) {
            int val = -1;
            if (jj < a) {
                if (jj < kWave) {
                    val = t0;   // jj == lane
                } else {
                    const int xv = drafts[(size_t)s * kmax + jj];
                    val = d2t ? d2t[xv] : xv;
                }
            } else if (jj == a) {
                val = tok;
            }
            e[jj] = val;
        }
        if (lane == 0) {
            status[s] = 0;
            accept_len[s] = a;
            n_emit[s] = a + 1;
            next_tok[s] = tok;
            pos_out[s] = p + a + 1;
        }
    }
}

// ---------------------------------------------------------------------------
// Dense draft distributions (DSSD _sample_verify with the draft head's full q):
// q [R][V] and z [R][V] (= logit / T, from spec_lm_head_sample_dense). Three launches:
//   dense_walk_kernel      row offsets per workgroup, then a wave per sequence tests
//                          u < p(x) / q(x) for its drafts (a ballot gives the first
//                          rejection) and records (offset, accepted count, status);
//   dense_residual_kernel  (vocabulary chunk, sequence): for a sequence with a
//                          rejection, the chunk's best log(p - q) + G over the entries
//                          with p > q, merged across chunks by a 64-bit atomic maximum;
//   dense_finalize_kernel  a wave per sequence writes the outputs.
// The kernel boundaries order the three; the keys are reset by the walk and read
// back by atomic exchange.
struct DenseRec {
    int32_t off;      // the sequence's first packed row
    int32_t a;        // drafts accepted (k_s: all)
    int32_t status;   // seq_status bits
    int32_t pad;
};

constexpr int kDenseGroupsPerThread = 4;                                  // 4 entries per group
constexpr int kDenseGroupsPerWg = kDenseGroupsPerThread * 256;

__global__ __launch_bounds__(kSampleThreads) void dense_walk_kernel(
    const int32_t* __restrict__ drafts, int kmax, const int32_t* __restrict__ k, const int32_t* __restrict__ d2t,
    int n_draft_vocab, int V, int B, int R, const float* __restrict__ q, const float* __restrict__ z,
    const float* __restrict__ lse, const int32_t* __restrict__ row_ctr, uint32_t key0, uint32_t key1,
    const int32_t* __restrict__ pos_in, DenseRec* __restrict__ rec, unsigned long long* keys) {
    __shared__ long long s_wsum[kSampleThreads / kWave];
    __shared__ int s_wbad[kSampleThreads / kWave];
    __shared__ int s_off[kSampleMaxB];
    const int tid = threadIdx.x;
    const bool packing_ok = block_row_offsets<kSampleThreads>(k, B, R, s_wsum, s_wbad, s_off);
    const int wave = tid / kWave, lane = tid % kWave;
    constexpr int n_waves = kSampleThreads / kWave;
    for (int s = blockIdx.x * n_waves + wave; s < B; s += gridDim.x * n_waves) {
        const int ks = k[s];
        const int off = s_off[s];
        int bits = 0;
        if (!packing_ok || ks > kmax) bits |= SPEC_STATUS_BAD_ROWS;
        if (pos_in[s] < 0) bits |= SPEC_STATUS_BAD_POS;
        int a = ks;
        if (!bits) {
            bool bad_tok = false;
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
                    if (!bad_tok) {
                        const size_t r = (size_t)off + j;
                        const float qx = q[r * V + t];
                        if (!(qx > 0.f)) {
                            bad_tok = true;
                        } else {
                            const float px = __expf(z[r * V + t] - lse[r]);
                            const uint4 w = philox10(
                                make_uint4(0u, (uint32_t)row_ctr[2 * r], (uint32_t)row_ctr[2 * r + 1], 1u), key0, key1);
                            rej = !(u01_23(w.x) < px / qx);
                        }
                    }
                }
                const unsigned long long mm = __ballot(rej);
                if (mm && a == ks) a = base + (int)__builtin_ctzll(mm);
            }
            if (__ballot(bad_tok)) bits |= SPEC_STATUS_BAD_TOKEN;
        }
        if (lane == 0) {
            rec[s] = DenseRec{off, a, bits, 0};
            atomicExch(keys + s, 0ull);
        }
    }
}

__global__ __launch_bounds__(256) void dense_residual_kernel(
    const int32_t* __restrict__ k, int V, const float* __restrict__ q, const float* __restrict__ z,
    const float* __restrict__ lse, const int32_t* __restrict__ row_ctr, uint32_t key0, uint32_t key1,
    const DenseRec* __restrict__ rec, unsigned long long* keys) {
    __shared__ Best s_best[4];
    const int s = blockIdx.y;
    const DenseRec rc = rec[s];
    if (rc.status || rc.a >= k[s]) return;            // flagged, or every draft kept
    const size_t r = (size_t)rc.off + rc.a;           // the rejected row
    const uint32_t ca = (uint32_t)row_ctr[2 * r], cb = (uint32_t)row_ctr[2 * r + 1];
    const float L = lse[r];
    const float* zr = z + r * V;
    const float* qr = q + r * V;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int n_groups = (V + 3) / 4;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int gi = 0; gi < kDenseGroupsPerThread; ++gi) {
        const int g = blockIdx.x * kDenseGroupsPerWg + gi * 256 + tid;
        if (g >= n_groups) break;
        const uint4 w = philox10(make_uint4((uint32_t)g, ca, cb, 0u), key0, key1);
        const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int v = 4 * g + d;
            if (v >= V) break;
            const float wv = __expf(zr[v] - L) - qr[v];
            if (wv > 0.f) {
                const float sc = __logf(wv) + gumbel(words[d]);
                if (better(sc, v, bv, bi)) {
                    bv = sc;
                    bi = v;
                }
            }
        }
    }
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const float ov = __shfl_xor(bv, d);
        const int oi = __shfl_xor(bi, d);
        if (better(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
        }
    }
    if (lane == 0) s_best[wave] = Best{bv, bi};
    __syncthreads();
    if (tid == 0) {
        Best b = s_best[0];
        for (int wv = 1; wv < 4; ++wv)
            if (better(s_best[wv].v, s_best[wv].i, b.v, b.i)) b = s_best[wv];
        if (b.i != 0x7fffffff) atomicMax(keys + s, pack_best(b));
    }
}

__global__ __launch_bounds__(256) void dense_finalize_kernel(
    const int32_t* __restrict__ drafts, int kmax, const int32_t* __restrict__ k, const int32_t* __restrict__ d2t,
    int B, const int32_t* __restrict__ sample_p, const DenseRec* __restrict__ rec, unsigned long long* keys,
    const int32_t* __restrict__ pos_in, int32_t* pos_out, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ n_emit, int32_t* __restrict__ emit, int32_t* __restrict__ next_tok,
    int32_t* __restrict__ status) {
    const int lane = threadIdx.x % kWave;
    const int s = blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
    if (s >= B) return;
    const DenseRec rc = rec[s];
    int32_t* e = emit + (size_t)s * (kmax + 1);
    if (rc.status) {
        for (int j = lane; j <= kmax; j += kWave) e[j] = -1;
        if (lane == 0) {
            status[s] = rc.status;
            accept_len[s] = -1;
            n_emit[s] = 0;
            next_tok[s] = -1;
            pos_out[s] = pos_in[s];
        }
        return;
    }
    const int ks = k[s], a = rc.a;
    // one lane takes (and clears) the key, the wave shares its token
    int tok = 0;
    if (lane == 0) {
        if (a < ks) {
            // the residual's winner; no entry with p > q in fp32 leaves the row's draw from p
            const unsigned long long key = atomicExch(keys + s, 0ull);
            tok = key ? (int)~(uint32_t)key : sample_p[rc.off + a];
        } else {
            tok = sample_p[rc.off + ks];
        }
    }
    tok = __shfl(tok, 0);
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
    hipLaunchKernelGGL(sample_accept_kernel, dim3(seq_grid(B, kSampleThreads)), dim3(kSampleThreads), 0, (hipStream_t)stream, drafts, kmax, k,
                       d2t, n_draft_vocab, V, B, R, q_tok, q_prob, NQ, lse, z_supp, sample_p, sample_res, row_ctr,
                       (uint32_t)seed, (uint32_t)(seed >> 32), pos_in, pos_out, accept_len, n_emit, emit, next_tok,
                       seq_status);
    SV_LAUNCH_CHECK("spec_sample_accept");
    return SPEC_OK;
}

size_t spec_sample_accept_dense_workspace_bytes(int32_t B) {
    if (B < 1) return 0;
    const size_t rec = ((size_t)B * sizeof(sv::DenseRec) + 255) & ~(size_t)255;
    return rec + (size_t)B * sizeof(unsigned long long);
}

int spec_sample_accept_dense(const int32_t* drafts, int32_t kmax, const int32_t* k, const int32_t* d2t,
                             int32_t n_draft_vocab, int32_t V, int32_t B, int32_t R, const float* q, const float* z,
                             const float* lse, const int32_t* sample_p, const int32_t* row_ctr, uint64_t seed,
                             const int32_t* pos_in, int32_t* pos_out, int32_t* accept_len, int32_t* n_emit,
                             int32_t* emit, int32_t* next_tok, int32_t* seq_status, void* workspace,
                             size_t workspace_bytes, void* stream) {
    using namespace sv;
    last_error().clear();
    if (B < 1 || B > kSampleMaxB) return fail(SPEC_EINVAL, "spec_sample_accept_dense: B=%d outside 1..%d", B, kSampleMaxB);
    if (kmax < 0 || kmax > 1024) return fail(SPEC_EINVAL, "spec_sample_accept_dense: kmax=%d outside 0..1024", kmax);
    if (R < 1) return fail(SPEC_EINVAL, "spec_sample_accept_dense: R=%d < 1", R);
    if (V < 1 || V > 0x7ffffff0) return fail(SPEC_EINVAL, "spec_sample_accept_dense: V=%d", V);
    if (d2t && n_draft_vocab < 1) return fail(SPEC_EINVAL, "spec_sample_accept_dense: d2t given with n_draft_vocab=%d", n_draft_vocab);
    if (!k || !q || !z || !lse || !sample_p || !row_ctr || !pos_in || !pos_out || !accept_len || !n_emit || !emit ||
        !next_tok || !seq_status || (kmax > 0 && !drafts))
        return fail(SPEC_EINVAL, "spec_sample_accept_dense: null required pointer");
    const size_t need = spec_sample_accept_dense_workspace_bytes(B);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return fail(SPEC_EWORKSPACE, "spec_sample_accept_dense: workspace %zu bytes < %zu required (or null/misaligned)",
                    workspace_bytes, need);
    char* ws = static_cast<char*>(workspace);
    DenseRec* rec = reinterpret_cast<DenseRec*>(ws);
    unsigned long long* keys =
        reinterpret_cast<unsigned long long*>(ws + (((size_t)B * sizeof(DenseRec) + 255) & ~(size_t)255));
    hipStream_t st = (hipStream_t)stream;
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    hipLaunchKernelGGL(dense_walk_kernel, dim3(seq_grid(B, kSampleThreads)), dim3(kSampleThreads), 0, st, drafts, kmax, k, d2t, n_draft_vocab, V,
                       B, R, q, z, lse, row_ctr, k0, k1, pos_in, rec, keys);
    SV_LAUNCH_CHECK("spec_sample_accept_dense(walk)");
    const int n_chunks = (int)(((V + 3) / 4 + kDenseGroupsPerWg - 1) / kDenseGroupsPerWg);
    hipLaunchKernelGGL(dense_residual_kernel, dim3(n_chunks, B), dim3(256), 0, st, k, V, q, z, lse, row_ctr, k0, k1,
                       rec, keys);
    SV_LAUNCH_CHECK("spec_sample_accept_dense(residual)");
    hipLaunchKernelGGL(dense_finalize_kernel, dim3((B + 3) / 4), dim3(256), 0, st, drafts, kmax, k, d2t, B, sample_p,
                       rec, keys, pos_in, pos_out, accept_len, n_emit, emit, next_tok, seq_status);
    SV_LAUNCH_CHECK("spec_sample_accept_dense(finalize)");
    return SPEC_OK;
}

}  // extern "C"
