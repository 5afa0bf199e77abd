/*
 * Plain fp64 CPU oracle for the greedy draft/verify step.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link or
 * call this file: only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark use it. It shares no code, header or table with the HIP
 * library; the only things both sides agree on are the buffer formats that the
 * public C header documents (bf16 bit patterns, the paged KV layout, the
 * per-sequence status bits).
 *
 * Every function is the definition written out, in fp64, with bf16 inputs
 * widened exactly. Loops run in the order of the definitions; OpenMP only
 * spreads independent units (rows, heads, vocabulary entries) over cores.
 *
 * Sources (the web pages these definitions follow):
 *  - "span-02 engine/crates/model/src/spec.rs", module doc: one verify forward
 *    of B(k+1) rows, KV appended in place at pos..pos+k, greedy acceptance,
 *    rollback = pos advances by the accepted tokens, kv_hi = position;
 *    SpecReq doc: the KV slot of position p is page pages[p / 16].
 *  - "DSSD-dev/dssd/fast.py", _attention: per-row softmax attention over keys
 *    [0, p+1) with grouped query heads; the greedy chain acceptance loop in
 *    generate_spec (first miss stops, then target[len(committed)] is appended).
 *  - "memra-engine src/spec.rs", full_attn_verify: query row r attends to keys
 *    [0 .. base_len + r + 1); attention scale 1/sqrt(head_dim).
 *  - "oxinfer src/qwen_mtp.rs", module doc: Gated DeltaNet states recorded per
 *    token and restored exactly on partial acceptance; DraftHead: draft index i
 *    stands for target token d2t[i]; speculative_accept in the greedy case.
 *  - "flashrt-structures whole_step.py", _gstep / generate_speculative: argmax on
 *    fp32 logits, device prefix match, pos += j + 1.
 *  - The Gated DeltaNet per-token update S_t = a_t S_{t-1} (I - b_t k_t k_t^T)
 *    + b_t v_t k_t^T, o_t = S_t q_t, as the problem statement gives it.
 *  - "DSSD-dev/dssd/fast.py", _set_rows / _tree_cycle / _star_cycle: tree drafts
 *    as rows in creation order, each on its own KV slot, attending to the
 *    committed keys plus the slots of its own path; the verification walk from the
 *    root; compaction of the accepted path's KV to contiguous slots.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_PAGE 16

/* Per-sequence status bits (same meaning as the library's documented bits). */
#define ORC_BAD_PAGE 1  /* a page id the sequence needs is outside [0, n_pages) */
#define ORC_BAD_POS 2   /* pos < 0, or (pos + k) / 16 >= max_pages              */
#define ORC_BAD_ROWS 4  /* packing undefined (some k < 0 or sum(k + 1) != R: all  */
                        /* sequences), or this k > kmax                          */
#define ORC_BAD_TOKEN 8 /* draft id or d2t entry out of range                    */
#define ORC_BAD_TREE 16 /* tree rows: a parent out of creation order             */
#define ORC_BAD_LIMIT 32 /* generation limit below one token                      */

static double bf(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_version(void) { return 1; }

/* ---------------------------------------------------------------------------
 * Row bookkeeping (spec.rs spec_build_verify; fast.py _set_pos): sequence s
 * owns rows off_s .. off_s + k_s, row j of it feeds position pos_s + j.
 * Returns per-sequence status bits in st[B]; fills off[B] (row offsets).
 * ------------------------------------------------------------------------- */
void oracle_validate(const int32_t* page_table, int32_t max_pages, int64_t n_pages,
                     const int32_t* pos, const int32_t* k, int32_t kmax, int32_t B, int32_t R,
                     int32_t* off, int32_t* st) {
    /* The packing r = off_s + j exists only if every k_s >= 0 and the counts add
     * up to R; otherwise no row can be attributed and every sequence is flagged. */
    int64_t total = 0;
    int packing_ok = 1;
    for (int s = 0; s < B; ++s) {
        off[s] = (int32_t)total;
        total += (int64_t)k[s] + 1;
        if (k[s] < 0) packing_ok = 0;
    }
    if (total != R) packing_ok = 0;
    for (int s = 0; s < B; ++s) {
        int bits = 0;
        if (!packing_ok || (kmax >= 0 && k[s] > kmax)) bits |= ORC_BAD_ROWS;
        if (pos[s] < 0) {
            bits |= ORC_BAD_POS;
        } else if (k[s] >= 0) {
            int64_t last = (int64_t)pos[s] + k[s];
            if (last / ORC_PAGE >= max_pages) {
                bits |= ORC_BAD_POS;
            } else if (page_table) {
                for (int64_t pg = 0; pg <= last / ORC_PAGE; ++pg) {
                    int32_t id = page_table[(int64_t)s * max_pages + pg];
                    if (id < 0 || id >= n_pages) bits |= ORC_BAD_PAGE;
                }
            }
        }
        st[s] = bits;
    }
}

/* Offsets of the paged pool format. Both pools hold one 16 * D block per (page,
 * kv head) at ((page * Hkv + hk) * 16 * D); inside a block, token t / channel d
 * sits at
 *   K: (d / 32) * 512 + ((d % 32) / 8) * 128 + t * 8 + d % 8
 *   V: (d / 16) * 256 + (t / 4) * 64 + (d % 16) * 4 + t % 4
 * (the library's documented layout; any permutation inside a block would do for
 * the oracle, which only reads through these two functions). */
static int64_t k_index(int64_t page, int hk, int t, int d, int Hkv, int D) {
    return (page * Hkv + hk) * (int64_t)(ORC_PAGE * D) + (d / 32) * 512 + ((d % 32) / 8) * 128 + t * 8 + d % 8;
}
static int64_t v_index(int64_t page, int hk, int t, int d, int Hkv, int D) {
    return (page * Hkv + hk) * (int64_t)(ORC_PAGE * D) + (d / 16) * 256 + (t / 4) * 64 + (d % 16) * 4 + t % 4;
}

/* ---------------------------------------------------------------------------
 * KV append in place (spec.rs module doc: KV appended at pos..pos+k; fast.py
 * _layers index_copy_ into the cache at the rows' slots). Row r = off_s + j of
 * k_new/v_new [R][Hkv][D] goes to position p = pos_s + j, i.e. page
 * page_table[s][p / 16], in-page token p % 16. Bit-exact copy. Sequences with
 * st[s] != 0 are skipped.
 * ------------------------------------------------------------------------- */
void oracle_append_kv(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_pool,
                      uint16_t* v_pool, const int32_t* page_table, int32_t max_pages,
                      const int32_t* pos, const int32_t* k, const int32_t* off, const int32_t* st,
                      int32_t B, int32_t Hkv, int32_t D) {
    for (int s = 0; s < B; ++s) {
        if (st[s]) continue;
        for (int j = 0; j <= k[s]; ++j) {
            int64_t r = off[s] + j;
            int64_t p = (int64_t)pos[s] + j;
            int64_t page = page_table[(int64_t)s * max_pages + p / ORC_PAGE];
            int t = (int)(p % ORC_PAGE);
            for (int hk = 0; hk < Hkv; ++hk)
                for (int d = 0; d < D; ++d) {
                    int64_t src = (r * Hkv + hk) * D + d;
                    k_pool[k_index(page, hk, t, d, Hkv, D)] = k_new[src];
                    v_pool[v_index(page, hk, t, d, Hkv, D)] = v_new[src];
                }
        }
    }
}

/* ---------------------------------------------------------------------------
 * Verify attention (fast.py _attention reference path; memra full_attn_verify:
 * row r attends to keys [0 .. base_len + r + 1); span-02: kv_hi = position).
 * For row r = (s, j) at position p = pos_s + j and query head h, with kv head
 * hk = h / (Hq / Hkv) (contiguous groups, as grouped-query SDPA does):
 *   z_t = scale * sum_d q[r,h,d] K_t[hk,d]            t = 0..p
 *   w_t = exp(z_t - max z) / sum_u exp(z_u - max z)
 *   o[r,h,:] = sum_t w_t V_t[hk,:]
 * K_t / V_t are read through the page table (after the append). out is fp64
 * [R][Hq][D]; rows of sequences with st[s] != 0 are left untouched.
 * ------------------------------------------------------------------------- */
void oracle_verify_attn(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                        const int32_t* page_table, int32_t max_pages, const int32_t* pos,
                        const int32_t* k, const int32_t* off, const int32_t* st, int32_t B,
                        int32_t R, int32_t Hq, int32_t Hkv, int32_t D, double scale, double* out) {
    int G = Hq / Hkv;
    (void)R;
    for (int s = 0; s < B; ++s) {
        if (st[s]) continue;
        int T = k[s] + 1;
#pragma omp parallel for collapse(2) schedule(dynamic)
        for (int j = 0; j < T; ++j) {
            for (int h = 0; h < Hq; ++h) {
                int64_t r = off[s] + j;
                int64_t p = (int64_t)pos[s] + j;
                int hk = h / G;
                const uint16_t* qr = q + (r * Hq + h) * D;
                double* z = (double*)malloc(sizeof(double) * (size_t)(p + 1));
                double zmax = -INFINITY;
                for (int64_t t = 0; t <= p; ++t) {
                    int64_t page = page_table[(int64_t)s * max_pages + t / ORC_PAGE];
                    int tt = (int)(t % ORC_PAGE);
                    double acc = 0.0;
                    for (int d = 0; d < D; ++d) acc += bf(qr[d]) * bf(k_pool[k_index(page, hk, tt, d, Hkv, D)]);
                    z[t] = scale * acc;
                    if (z[t] > zmax) zmax = z[t];
                }
                double denom = 0.0;
                for (int64_t t = 0; t <= p; ++t) {
                    z[t] = exp(z[t] - zmax);
                    denom += z[t];
                }
                double* o = out + (r * Hq + h) * D;
                for (int d = 0; d < D; ++d) o[d] = 0.0;
                for (int64_t t = 0; t <= p; ++t) {
                    int64_t page = page_table[(int64_t)s * max_pages + t / ORC_PAGE];
                    int tt = (int)(t % ORC_PAGE);
                    double w = z[t] / denom;
                    for (int d = 0; d < D; ++d) o[d] += w * bf(v_pool[v_index(page, hk, tt, d, Hkv, D)]);
                }
                free(z);
            }
        }
    }
}

/* ---------------------------------------------------------------------------
 * lm_head contraction + greedy argmax (span-02 lm_head_argmax; greedy_logprob:
 * the FIRST maximum wins; flashrt: argmax taken on full-precision logits).
 *   logit[r,v] = sum_i W[v,i] h[r,i]      (fp64, i ascending)
 *   g[r]       = lowest v with logit[r,v] == max_v logit[r,v]
 *   top1[r]    = that maximum, top2[r] = the largest logit at any other index
 * (top2 == top1 when the maximum is tied). logits_out (nullable) receives the
 * full [R][V] fp64 matrix.
 * ------------------------------------------------------------------------- */
void oracle_lm_head_argmax(const uint16_t* hidden, const uint16_t* w, int32_t R, int32_t H,
                           int32_t V, int32_t* g, double* top1, double* top2, double* logits_out) {
    double* hd = (double*)malloc(sizeof(double) * (size_t)R * H);
    for (int64_t i = 0; i < (int64_t)R * H; ++i) hd[i] = bf(hidden[i]);
    double* logit = logits_out ? logits_out : (double*)malloc(sizeof(double) * (size_t)R * V);
#pragma omp parallel
    {
        double* acc = (double*)malloc(sizeof(double) * (size_t)R);
        double* wrow = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(static)
        for (int v = 0; v < V; ++v) {
            for (int i = 0; i < H; ++i) wrow[i] = bf(w[(int64_t)v * H + i]);
            for (int r = 0; r < R; ++r) acc[r] = 0.0;
            /* each acc[r] is one dot product summed over i in ascending order */
            for (int i = 0; i < H; ++i)
                for (int r = 0; r < R; ++r) acc[r] += wrow[i] * hd[(int64_t)r * H + i];
            for (int r = 0; r < R; ++r) logit[(int64_t)r * V + v] = acc[r];
        }
        free(acc);
        free(wrow);
    }
    for (int r = 0; r < R; ++r) {
        const double* z = logit + (int64_t)r * V;
        int best = 0;
        for (int v = 1; v < V; ++v)
            if (z[v] > z[best]) best = v;
        double second = -INFINITY;
        for (int v = 0; v < V; ++v)
            if (v != best && z[v] > second) second = z[v];
        g[r] = best;
        if (top1) top1[r] = z[best];
        if (top2) top2[r] = second;
    }
    if (!logits_out) free(logit);
    free(hd);
}

/* First maximum and runner-up of each row of an fp64 logit matrix [R][V]
 * (span-02 greedy_logprob: strict '>' scan from index 0, so the lowest index of
 * the maximum wins). top2 is the largest value at any other index. */
void oracle_argmax_rows(const double* logit, int32_t R, int32_t V, int32_t* g, double* top1,
                        double* top2) {
    for (int r = 0; r < R; ++r) {
        const double* z = logit + (int64_t)r * V;
        int best = 0;
        for (int v = 1; v < V; ++v)
            if (z[v] > z[best]) best = v;
        double second = -INFINITY;
        for (int v = 0; v < V; ++v)
            if (v != best && z[v] > second) second = z[v];
        g[r] = best;
        if (top1) top1[r] = z[best];
        if (top2) top2[r] = second;
    }
}

/* ---------------------------------------------------------------------------
 * Greedy acceptance and rollback bookkeeping (fast.py generate_spec accept loop;
 * oxinfer MtpDecoder::step; flashrt device prefix match; span-02 step_chunk:
 * pos <- pos + a + 1, next token <- last emitted).
 *   map(x) = d2t ? d2t[x] : x
 *   a      = number of leading j < k_s with map(draft[s][j]) == g[off_s + j]
 *   emit   = map(draft[s][0..a)) ++ [g[off_s + a]]        (n_emit = a + 1)
 *   pos_out = pos_in + a + 1, next_tok = g[off_s + a]
 * emit is [B][kmax + 1], unused entries are -1. A sequence with a bad status
 * (from oracle_validate, plus draft ids / d2t entries out of range) gets
 * accept_len = -1, n_emit = 0, next_tok = -1, pos_out = pos_in, emit row -1.
 * ------------------------------------------------------------------------- */
void oracle_greedy_accept(const int32_t* g, const int32_t* drafts, int32_t kmax, const int32_t* k,
                          const int32_t* d2t, int32_t n_draft_vocab, int32_t V, int32_t B,
                          int32_t R, const int32_t* pos_in, int32_t* pos_out, int32_t* accept_len,
                          int32_t* n_emit, int32_t* emit, int32_t* next_tok, int32_t* st) {
    int64_t total = 0;
    int packing_ok = 1;
    for (int s = 0; s < B; ++s) {
        total += (int64_t)k[s] + 1;
        if (k[s] < 0) packing_ok = 0;
    }
    if (total != R) packing_ok = 0;
    int64_t off = 0;
    for (int s = 0; s < B; ++s) {
        int bits = 0;
        int ks = k[s];
        if (!packing_ok || ks > kmax) bits |= ORC_BAD_ROWS;
        if (pos_in[s] < 0) bits |= ORC_BAD_POS;
        if (!bits) {
            for (int j = 0; j < ks; ++j) {
                int32_t x = drafts[(int64_t)s * kmax + j];
                if (d2t) {
                    if (x < 0 || x >= n_draft_vocab || d2t[x] < 0 || d2t[x] >= V) bits |= ORC_BAD_TOKEN;
                } else if (x < 0 || x >= V) {
                    bits |= ORC_BAD_TOKEN;
                }
            }
        }
        int32_t* e = emit + (int64_t)s * (kmax + 1);
        for (int j = 0; j <= kmax; ++j) e[j] = -1;
        if (bits) {
            st[s] = bits;
            accept_len[s] = -1;
            n_emit[s] = 0;
            next_tok[s] = -1;
            pos_out[s] = pos_in[s];
            off += (int64_t)ks + 1;
            continue;
        }
        st[s] = 0;
        int a = 0;
        while (a < ks) {
            int32_t x = drafts[(int64_t)s * kmax + a];
            int32_t mapped = d2t ? d2t[x] : x;
            if (mapped != g[off + a]) break;
            e[a] = mapped;
            ++a;
        }
        e[a] = g[off + a];
        accept_len[s] = a;
        n_emit[s] = a + 1;
        next_tok[s] = g[off + a];
        pos_out[s] = pos_in[s] + a + 1;
        off += ks + 1;
    }
}

/* ---------------------------------------------------------------------------
 * Gated DeltaNet verify with per-token state recording (oxinfer qwen_mtp.rs:
 * states recorded per token during the verify forward; memra: per-column state
 * clones). For each sequence s and head h, starting from S_0 = state[s,h]
 * (dv x dk, row = value channel, column = key channel), for t = 1..T:
 *   M   = I - b_t k_t k_t^T                       (dk x dk)
 *   S_t = a_t S_{t-1} M + b_t v_t k_t^T          (matrix products, fp64)
 *   o_t = S_t (q_scale q_t)
 *   rec[s,t-1,h] = S_t
 * q, k, v: bf16 [B][T][Hd][dk|dv]; a, b: fp32 [B][T][Hd]; state: fp32
 * [B][Hd][dv][dk]; rec: fp64 [B][T][Hd][dv][dk]; o: fp64 [B][T][Hd][dv].
 * ------------------------------------------------------------------------- */
void oracle_delta_verify(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* a,
                         const float* b, double q_scale, const float* state, int32_t B, int32_t T,
                         int32_t Hd, int32_t dk, int32_t dv, double* rec, double* o) {
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int s = 0; s < B; ++s) {
        for (int h = 0; h < Hd; ++h) {
            double* S = (double*)malloc(sizeof(double) * (size_t)dv * dk);
            double* Sn = (double*)malloc(sizeof(double) * (size_t)dv * dk);
            double* M = (double*)malloc(sizeof(double) * (size_t)dk * dk);
            double* kt = (double*)malloc(sizeof(double) * (size_t)dk);
            double* qt = (double*)malloc(sizeof(double) * (size_t)dk);
            double* vt = (double*)malloc(sizeof(double) * (size_t)dv);
            const float* S0 = state + ((int64_t)s * Hd + h) * dv * dk;
            for (int64_t i = 0; i < (int64_t)dv * dk; ++i) S[i] = (double)S0[i];
            for (int t = 0; t < T; ++t) {
                int64_t th = ((int64_t)s * T + t) * Hd + h;
                double at = (double)a[th], bt = (double)b[th];
                for (int i = 0; i < dk; ++i) kt[i] = bf(k[th * dk + i]);
                for (int i = 0; i < dk; ++i) qt[i] = q_scale * bf(q[th * dk + i]);
                for (int i = 0; i < dv; ++i) vt[i] = bf(v[th * dv + i]);
                for (int i = 0; i < dk; ++i)
                    for (int jj = 0; jj < dk; ++jj)
                        M[i * dk + jj] = (i == jj ? 1.0 : 0.0) - bt * kt[i] * kt[jj];
                for (int i = 0; i < dv; ++i)
                    for (int jj = 0; jj < dk; ++jj) {
                        double acc = 0.0;
                        for (int l = 0; l < dk; ++l) acc += S[i * dk + l] * M[l * dk + jj];
                        Sn[i * dk + jj] = at * acc + bt * vt[i] * kt[jj];
                    }
                memcpy(S, Sn, sizeof(double) * (size_t)dv * dk);
                double* ot = o + th * dv;
                for (int i = 0; i < dv; ++i) {
                    double acc = 0.0;
                    for (int jj = 0; jj < dk; ++jj) acc += S[i * dk + jj] * qt[jj];
                    ot[i] = acc;
                }
                memcpy(rec + th * dv * dk, S, sizeof(double) * (size_t)dv * dk);
            }
            free(S); free(Sn); free(M); free(kt); free(qt); free(vt);
        }
    }
}

/* ---------------------------------------------------------------------------
 * DeltaNet rollback (oxinfer: restore the recorded state of the last committed
 * token; flashrt: roll the gated-delta states back). L[s] = committed tokens in
 * 0..T (clamped into that range): the state becomes S_L = rec[s, L-1], or
 * stays S_0 when L = 0.
 * rec and state are fp64 here: [B][T][Hd][dv][dk] and [B][Hd][dv][dk].
 * ------------------------------------------------------------------------- */
void oracle_delta_rollback(const double* rec, const int32_t* L, int32_t B, int32_t T, int32_t Hd,
                           int32_t dk, int32_t dv, double* state) {
    int64_t n = (int64_t)dv * dk;
    for (int s = 0; s < B; ++s) {
        int Ls = L[s] < 0 ? 0 : (L[s] > T ? T : L[s]); /* clamped to 0..T */
        if (Ls == 0) continue;
        int t = Ls - 1;
        for (int h = 0; h < Hd; ++h)
            memcpy(state + ((int64_t)s * Hd + h) * n, rec + (((int64_t)s * T + t) * Hd + h) * n,
                   sizeof(double) * (size_t)n);
    }
}

/* ---------------------------------------------------------------------------
 * Tree (trie) verify rows (fast.py _set_rows, _tree_cycle, _star_cycle). The
 * k_s + 1 rows of sequence s are the nodes of a draft tree in creation order:
 * node 0 is the root (the last committed token, parent -1), every other node i
 * has a parent in [0, i), and the draft token of node i >= 1 is drafts[s][i - 1].
 * Node i sits at position pos + depth(i) and writes its K/V at slot pos + i (its
 * creation index, the ordinary append); it attends to slots 0 .. pos (the
 * committed keys and the root) and then to the slots pos + u of its own path
 * below the root, root's child first, itself last. A chain (parent[i] = i - 1) is
 * the ordinary verify row set. parent is [B][kmax + 1].
 * ------------------------------------------------------------------------- */
void oracle_validate_tree(const int32_t* parent, int32_t kmax, const int32_t* k, int32_t B, int32_t* st) {
    for (int s = 0; s < B; ++s) {
        int ks = k[s];
        if (ks < 0 || ks > kmax) continue;  /* reported by the packing checks */
        const int32_t* par = parent + (int64_t)s * (kmax + 1);
        int bad = par[0] != -1;
        for (int i = 1; i <= ks; ++i)
            if (par[i] < 0 || par[i] >= i) bad = 1;
        if (bad) st[s] |= ORC_BAD_TREE;
    }
}

/* nodes of the path of node j below the root, root's child first, j last */
static int tree_path(const int32_t* par, int j, int* path) {
    int n = 0;
    for (int u = j; u != 0; u = par[u]) path[n++] = u;
    for (int a = 0, b = n - 1; a < b; ++a, --b) {
        int t = path[a];
        path[a] = path[b];
        path[b] = t;
    }
    return n;
}

/* For row r = (s, j) and query head h (kv head h / (Hq / Hkv)), with the key slots
 *   t = 0 .. pos_s, then pos_s + u for u in path(j):
 *   z_t = scale * sum_d q[r,h,d] K[slot t][hk,d],  w = softmax(z),  o = sum_t w_t V[slot t]
 * Rows of sequences with st[s] != 0 are left untouched. */
void oracle_verify_attn_tree(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                             const int32_t* page_table, int32_t max_pages, const int32_t* pos,
                             const int32_t* k, const int32_t* parent, int32_t kmax, const int32_t* off,
                             const int32_t* st, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                             double scale, double* out) {
    int G = Hq / Hkv;
    for (int s = 0; s < B; ++s) {
        if (st[s]) continue;
        int T = k[s] + 1;
        const int32_t* par = parent + (int64_t)s * (kmax + 1);
#pragma omp parallel for collapse(2) schedule(dynamic)
        for (int j = 0; j < T; ++j) {
            for (int h = 0; h < Hq; ++h) {
                int path[1024];
                int np = tree_path(par, j, path);
                int64_t P = pos[s];
                int64_t n_keys = P + 1 + np;
                int64_t* slot = (int64_t*)malloc(sizeof(int64_t) * (size_t)n_keys);
                for (int64_t t = 0; t <= P; ++t) slot[t] = t;
                for (int d = 0; d < np; ++d) slot[P + 1 + d] = P + path[d];
                int64_t r = off[s] + j;
                int hk = h / G;
                const uint16_t* qr = q + (r * Hq + h) * D;
                double* z = (double*)malloc(sizeof(double) * (size_t)n_keys);
                double zmax = -INFINITY;
                for (int64_t t = 0; t < n_keys; ++t) {
                    int64_t page = page_table[(int64_t)s * max_pages + slot[t] / ORC_PAGE];
                    int tt = (int)(slot[t] % ORC_PAGE);
                    double acc = 0.0;
                    for (int d = 0; d < D; ++d) acc += bf(qr[d]) * bf(k_pool[k_index(page, hk, tt, d, Hkv, D)]);
                    z[t] = scale * acc;
                    if (z[t] > zmax) zmax = z[t];
                }
                double denom = 0.0;
                for (int64_t t = 0; t < n_keys; ++t) {
                    z[t] = exp(z[t] - zmax);
                    denom += z[t];
                }
                double* o = out + (r * Hq + h) * D;
                for (int d = 0; d < D; ++d) o[d] = 0.0;
                for (int64_t t = 0; t < n_keys; ++t) {
                    int64_t page = page_table[(int64_t)s * max_pages + slot[t] / ORC_PAGE];
                    int tt = (int)(slot[t] % ORC_PAGE);
                    double w = z[t] / denom;
                    for (int d = 0; d < D; ++d) o[d] += w * bf(v_pool[v_index(page, hk, tt, d, Hkv, D)]);
                }
                free(z);
                free(slot);
            }
        }
    }
}

/* Tree acceptance (fast.py _tree_cycle verification walk), greedy: from the root,
 * move to the child whose mapped draft token equals the greedy token of the
 * current node (the lowest-index such child), as long as one exists.
 *   accepted nodes u_1 .. u_a,  emit = map(tok(u_1 .. u_a)) ++ [g[node_a]]
 *   pos_out = pos_in + a + 1,  next_tok = g[node_a],  path[s] = u_1 .. u_a (-1 after)
 * Checks and the outputs of a rejected sequence as in oracle_greedy_accept; a
 * parent list out of creation order sets ORC_BAD_TREE. */
void oracle_tree_accept(const int32_t* g, const int32_t* drafts, int32_t kmax, const int32_t* k,
                        const int32_t* parent, const int32_t* d2t, int32_t n_draft_vocab, int32_t V,
                        int32_t B, int32_t R, const int32_t* pos_in, int32_t* pos_out, int32_t* accept_len,
                        int32_t* n_emit, int32_t* emit, int32_t* next_tok, int32_t* path, int32_t* st) {
    int64_t total = 0;
    int packing_ok = 1;
    for (int s = 0; s < B; ++s) {
        total += (int64_t)k[s] + 1;
        if (k[s] < 0) packing_ok = 0;
    }
    if (total != R) packing_ok = 0;
    int64_t off = 0;
    for (int s = 0; s < B; ++s) {
        int bits = 0;
        int ks = k[s];
        if (!packing_ok || ks > kmax) bits |= ORC_BAD_ROWS;
        if (pos_in[s] < 0) bits |= ORC_BAD_POS;
        const int32_t* par = parent + (int64_t)s * (kmax + 1);
        if (!bits) {
            if (par[0] != -1) bits |= ORC_BAD_TREE;
            for (int i = 1; i <= ks; ++i)
                if (par[i] < 0 || par[i] >= i) bits |= ORC_BAD_TREE;
            for (int j = 0; j < ks; ++j) {
                int32_t x = drafts[(int64_t)s * kmax + j];
                if (d2t) {
                    if (x < 0 || x >= n_draft_vocab || d2t[x] < 0 || d2t[x] >= V) bits |= ORC_BAD_TOKEN;
                } else if (x < 0 || x >= V) {
                    bits |= ORC_BAD_TOKEN;
                }
            }
        }
        int32_t* e = emit + (int64_t)s * (kmax + 1);
        int32_t* ph = path + (int64_t)s * kmax;
        for (int j = 0; j <= kmax; ++j) e[j] = -1;
        for (int j = 0; j < kmax; ++j) ph[j] = -1;
        if (bits) {
            st[s] = bits;
            accept_len[s] = -1;
            n_emit[s] = 0;
            next_tok[s] = -1;
            pos_out[s] = pos_in[s];
            off += (int64_t)ks + 1;
            continue;
        }
        st[s] = 0;
        int a = 0, u = 0;
        for (;;) {
            int next = -1;
            for (int c = 1; c <= ks && next < 0; ++c) {
                if (par[c] != u) continue;
                int32_t x = drafts[(int64_t)s * kmax + c - 1];
                int32_t mapped = d2t ? d2t[x] : x;
                if (mapped == g[off + u]) next = c;
            }
            if (next < 0) break;
            int32_t x = drafts[(int64_t)s * kmax + next - 1];
            e[a] = d2t ? d2t[x] : x;
            ph[a] = next;
            ++a;
            u = next;
        }
        e[a] = g[off + u];
        accept_len[s] = a;
        n_emit[s] = a + 1;
        next_tok[s] = g[off + u];
        pos_out[s] = pos_in[s] + a + 1;
        off += ks + 1;
    }
}

/* Compaction of the accepted path (fast.py _tree_cycle / _star_cycle): for every
 * sequence with st[s] == 0, the K/V of slot pos + path[s][d] moves to slot
 * pos + 1 + d, d = 0 .. accept_len[s] - 1, in ascending d (a source slot is never
 * below its destination, so no source is overwritten before it is read). Slots
 * past pos + accept_len are left as they are. */
void oracle_kv_compact(uint16_t* k_pool, uint16_t* v_pool, const int32_t* page_table, int32_t max_pages,
                       const int32_t* pos, const int32_t* path, const int32_t* accept_len, int32_t kmax,
                       const int32_t* st, int32_t B, int32_t Hkv, int32_t D) {
    for (int s = 0; s < B; ++s) {
        if (st[s] || accept_len[s] <= 0) continue;
        for (int d = 0; d < accept_len[s]; ++d) {
            int64_t src = (int64_t)pos[s] + path[(int64_t)s * kmax + d];
            int64_t dst = (int64_t)pos[s] + 1 + d;
            if (src == dst) continue;
            int64_t ps = page_table[(int64_t)s * max_pages + src / ORC_PAGE];
            int64_t pd = page_table[(int64_t)s * max_pages + dst / ORC_PAGE];
            for (int hk = 0; hk < Hkv; ++hk)
                for (int c = 0; c < D; ++c) {
                    k_pool[k_index(pd, hk, (int)(dst % ORC_PAGE), c, Hkv, D)] =
                        k_pool[k_index(ps, hk, (int)(src % ORC_PAGE), c, Hkv, D)];
                    v_pool[v_index(pd, hk, (int)(dst % ORC_PAGE), c, Hkv, D)] =
                        v_pool[v_index(ps, hk, (int)(src % ORC_PAGE), c, Hkv, D)];
                }
        }
    }
}

/* ---------------------------------------------------------------------------
 * Speculative-sampling verify (DSSD fast.py _sample_verify; oxinfer
 * speculative_accept; memra's sampled-spec note: counter-based Philox keyed by
 * (seed, event) so that runs are reproducible).
 *
 * Random numbers: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC 2011): a 4-word counter and a 2-word key; each
 * of 10 rounds multiplies words 0 and 2 by the round multipliers, mixes the high
 * halves of the products with the other words and the key, and the key advances by
 * the Weyl constants between rounds. A 32-bit output word w becomes the uniform
 * u = (floor(w / 512) + 1/2) / 2^23, which lies strictly inside (0, 1) and is
 * exactly representable in fp32 (24 significant bits).
 * ------------------------------------------------------------------------- */
void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        const uint32_t n0 = hi1 ^ c1 ^ k0;
        const uint32_t n1 = lo1;
        const uint32_t n2 = hi0 ^ c3 ^ k1;
        const uint32_t n3 = lo0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

static double u01(uint32_t w) { return ((double)(w >> 9) + 0.5) / 8388608.0; }

/* Counter layout (both sides): for a row with counter words (a, b) = row_ctr[r]
 *   Gumbel noise of vocabulary entry v:  ctr = (v / 4, a, b, 0), word v % 4
 *   acceptance uniform of the row:       ctr = (0, a, b, 1), word 0
 * key = (seed low 32 bits, seed high 32 bits). */
static double row_gumbel(uint32_t v, const int32_t* rc, const uint32_t key[2]) {
    const uint32_t ctr[4] = {v >> 2, (uint32_t)rc[0], (uint32_t)rc[1], 0u};
    uint32_t o[4];
    oracle_philox4x32_10(ctr, key, o);
    return -log(-log(u01(o[v & 3])));
}

double oracle_accept_uniform(const int32_t* rc, uint64_t seed) {
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    const uint32_t ctr[4] = {0u, (uint32_t)rc[0], (uint32_t)rc[1], 1u};
    uint32_t o[4];
    oracle_philox4x32_10(ctr, key, o);
    return u01(o[0]);
}

/* Per row r of logits [R][V] (fp64) at temperature T, with the draft distribution's
 * support q_tok[r][0..NQ) (-1 = unused) and masses q_prob[r][..]:
 *   z_v = logit_v / T,  lse = log sum_v exp(z_v),  p_v = exp(z_v - lse)
 *   z_supp[r][e] = z of q_tok[r][e] (NaN for unused entries)
 *   sample_p[r]   = argmax_v (z_v + G_v)                      (a draw from p)
 *   sample_res[r] = argmax_{v: r_v > 0} (log r_v + G_v), r_v = max(p_v - q_v, 0)
 *                   (a draw from norm(max(p - q, 0)); sample_p if every r_v is 0)
 * with G_v the Gumbel noise of the row (Gumbel-max: the argmax of log-weights plus
 * independent standard Gumbel noise is a draw from the normalised weights; ties go
 * to the smaller index). */
void oracle_sample_rows(const double* logits, int32_t R, int32_t V, double T, const int32_t* q_tok,
                        const float* q_prob, int32_t NQ, const int32_t* row_ctr, uint64_t seed, double* lse,
                        double* z_supp, int32_t* sample_p, int32_t* sample_res, double* gap_p, double* gap_res) {
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
#pragma omp parallel for schedule(dynamic)
    for (int r = 0; r < R; ++r) {
        const double* l = logits + (int64_t)r * V;
        double zmax = -INFINITY;
        for (int v = 0; v < V; ++v)
            if (l[v] / T > zmax) zmax = l[v] / T;
        double s = 0.0;
        for (int v = 0; v < V; ++v) s += exp(l[v] / T - zmax);
        const double L = zmax + log(s);
        lse[r] = L;
        const int32_t* qt = q_tok + (int64_t)r * NQ;
        const float* qp = q_prob + (int64_t)r * NQ;
        for (int e = 0; e < NQ; ++e)
            z_supp[(int64_t)r * NQ + e] = (qt[e] >= 0 && qt[e] < V) ? l[qt[e]] / T : NAN;
        /* best and runner-up of each draw (the runner-up only reports how decided the
           draw is: gap = best - runner-up) */
        double bp = -INFINITY, br = -INFINITY, bp2 = -INFINITY, br2 = -INFINITY;
        int ip = -1, ir = -1;
        for (int v = 0; v < V; ++v) {
            const double z = l[v] / T;
            const double g = row_gumbel((uint32_t)v, row_ctr + 2 * (int64_t)r, key);
            if (z + g > bp) {
                bp2 = bp;
                bp = z + g;
                ip = v;
            } else if (z + g > bp2) {
                bp2 = z + g;
            }
            double q = 0.0;
            for (int e = 0; e < NQ; ++e)
                if (qt[e] == v) q += qp[e];
            const double rv = exp(z - L) - q;
            if (rv > 0.0 && log(rv) + g > br) {
                br2 = br;
                br = log(rv) + g;
                ir = v;
            } else if (rv > 0.0 && log(rv) + g > br2) {
                br2 = log(rv) + g;
            }
        }
        sample_p[r] = ip;
        sample_res[r] = ir >= 0 ? ir : ip;
        if (gap_p) gap_p[r] = bp - bp2;
        if (gap_res) gap_res[r] = ir >= 0 ? br - br2 : bp - bp2;
    }
}

/* Chain walk of speculative sampling (DSSD _sample_verify): for j = 0 .. k_s - 1,
 * row r = off_s + j, draft x = drafts[s][j] (a target id, or a draft-vocabulary id
 * mapped through d2t), q(x) = the mass of x in the row's q support:
 *   accept x iff u_r < p_r(x) / q(x)   (u_r the row's acceptance uniform; the
 *                                       probability is min(1, p / q); q(x) is
 *                                       the summed mass of the support entries
 *                                       holding x, the q the residual uses)
 *   else emit sample_res[r], stop.
 * If every draft is accepted, emit sample_p of the bonus row off_s + k_s.
 *   accept_len = accepted drafts, emit = accepted tokens ++ [the sampled token],
 *   pos_out = pos_in + accept_len + 1, next_tok = the sampled token.
 * Status bits as oracle_greedy_accept; a draft whose (mapped) id has no positive
 * summed mass in its row's q support sets ORC_BAD_TOKEN. */
void oracle_sample_accept(const int32_t* drafts, int32_t kmax, const int32_t* k, const int32_t* d2t,
                          int32_t n_draft_vocab, int32_t V, int32_t B, int32_t R, const int32_t* q_tok,
                          const float* q_prob, int32_t NQ, const double* lse, const double* z_supp,
                          const int32_t* sample_p, const int32_t* sample_res, const int32_t* row_ctr,
                          uint64_t seed, const int32_t* pos_in, int32_t* pos_out, int32_t* accept_len,
                          int32_t* n_emit, int32_t* emit, int32_t* next_tok, int32_t* st) {
    int64_t total = 0;
    int packing_ok = 1;
    for (int s = 0; s < B; ++s) {
        total += (int64_t)k[s] + 1;
        if (k[s] < 0) packing_ok = 0;
    }
    if (total != R) packing_ok = 0;
    int64_t off = 0;
    for (int s = 0; s < B; ++s) {
        const int ks = k[s];
        int bits = 0;
        if (!packing_ok || ks > kmax) bits |= ORC_BAD_ROWS;
        if (pos_in[s] < 0) bits |= ORC_BAD_POS;
        int32_t* e = emit + (int64_t)s * (kmax + 1);
        for (int j = 0; j <= kmax; ++j) e[j] = -1;
        int supp_e[1024];
        double supp_q[1024];
        if (!bits) {
            for (int j = 0; j < ks; ++j) {
                const int32_t x = drafts[(int64_t)s * kmax + j];
                int32_t t = x;
                if (d2t) {
                    if (x < 0 || x >= n_draft_vocab || d2t[x] < 0 || d2t[x] >= V) {
                        bits |= ORC_BAD_TOKEN;
                        continue;
                    }
                    t = d2t[x];
                } else if (x < 0 || x >= V) {
                    bits |= ORC_BAD_TOKEN;
                    continue;
                }
                const int64_t r = off + j;
                supp_e[j] = -1;
                supp_q[j] = 0.0;
                for (int q = NQ - 1; q >= 0; --q)
                    if (q_tok[r * NQ + q] == t) {
                        supp_e[j] = q;
                        supp_q[j] += (double)q_prob[r * NQ + q];
                    }
                if (supp_e[j] < 0 || !(supp_q[j] > 0.0)) bits |= ORC_BAD_TOKEN;
            }
        }
        if (bits) {
            st[s] = bits;
            accept_len[s] = -1;
            n_emit[s] = 0;
            next_tok[s] = -1;
            pos_out[s] = pos_in[s];
            off += (int64_t)ks + 1;
            continue;
        }
        int a = 0, tok = -1;
        for (; a < ks; ++a) {
            const int64_t r = off + a;
            const int q = supp_e[a];
            const double px = exp(z_supp[r * NQ + q] - lse[r]);
            const double u = oracle_accept_uniform(row_ctr + 2 * r, seed);
            if (u < px / supp_q[a]) {
                e[a] = q_tok[r * NQ + q];
                continue;
            }
            tok = sample_res[r];
            break;
        }
        if (tok < 0) tok = sample_p[off + ks];
        e[a] = tok;
        st[s] = 0;
        accept_len[s] = a;
        n_emit[s] = a + 1;
        next_tok[s] = tok;
        pos_out[s] = pos_in[s] + a + 1;
        off += ks + 1;
    }
}

/* Speculative sampling with a dense draft distribution (DSSD _sample_verify with the
 * draft head's full distribution): q [R][V] holds q_r(v) for every target entry.
 * With z = logit / T and p_r = softmax(z_r) (fp64), for j = 0 .. k_s - 1, row r =
 * off_s + j, draft x (mapped through d2t when given):
 *   q_r(x) <= 0, or x out of range: ORC_BAD_TOKEN (a draft has positive mass under
 *   the distribution it was drawn from);
 *   accept x iff u_r < p_r(x) / q_r(x);
 *   else the token is a draw from norm(max(p_r - q_r, 0)): the first v maximising
 *   log(p_r(v) - q_r(v)) + G_r(v) over the v with p_r(v) > q_r(v) (the row's
 *   Gumbel noise, as for the draw from p); no such v: the row's draw from p.
 * All kept: the draw from p of the bonus row (first v maximising z + G).
 * Outputs as oracle_sample_accept; margin[s] = the smallest |log u_r - log(p_r(x) /
 * q_r(x))| over the drafts tested (how decided the walk is; +inf if none); gap[s] =
 * how decided the deciding draw is when p is known only to a relative precision
 * rel: for the residual, the winner's lowest possible score log(w - rel p) + G
 * minus the highest possible score log(w + rel p) + G of any other entry (w = p - q;
 * where p and q nearly cancel, a small error in p moves log w a lot); for a draw
 * from p, best - runner-up - 2 log(1 + rel). gap <= 0: not decided at that
 * precision. */
void oracle_sample_accept_dense(const int32_t* drafts, int32_t kmax, const int32_t* k, const int32_t* d2t,
                                int32_t n_draft_vocab, int32_t V, int32_t B, int32_t R, const double* logits,
                                double T, const float* q, const int32_t* row_ctr, uint64_t seed,
                                const int32_t* pos_in, int32_t* pos_out, int32_t* accept_len, int32_t* n_emit,
                                int32_t* emit, int32_t* next_tok, int32_t* st, double rel, double* margin,
                                double* gap) {
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    int64_t total = 0;
    int packing_ok = 1;
    for (int s = 0; s < B; ++s) {
        total += (int64_t)k[s] + 1;
        if (k[s] < 0) packing_ok = 0;
    }
    if (total != R) packing_ok = 0;
    int64_t off = 0;
    for (int s = 0; s < B; ++s) {
        const int ks = k[s];
        int bits = 0;
        if (!packing_ok || ks > kmax) bits |= ORC_BAD_ROWS;
        if (pos_in[s] < 0) bits |= ORC_BAD_POS;
        int32_t* e = emit + (int64_t)s * (kmax + 1);
        for (int j = 0; j <= kmax; ++j) e[j] = -1;
        margin[s] = INFINITY;
        gap[s] = INFINITY;
        if (!bits)
            for (int j = 0; j < ks; ++j) {
                const int32_t x = drafts[(int64_t)s * kmax + j];
                int32_t t = x;
                if (d2t) {
                    if (x < 0 || x >= n_draft_vocab || d2t[x] < 0 || d2t[x] >= V) {
                        bits |= ORC_BAD_TOKEN;
                        continue;
                    }
                    t = d2t[x];
                } else if (x < 0 || x >= V) {
                    bits |= ORC_BAD_TOKEN;
                    continue;
                }
                if (!(q[(off + j) * (int64_t)V + t] > 0.f)) bits |= ORC_BAD_TOKEN;
            }
        if (bits) {
            st[s] = bits;
            accept_len[s] = -1;
            n_emit[s] = 0;
            next_tok[s] = -1;
            pos_out[s] = pos_in[s];
            off += (int64_t)ks + 1;
            continue;
        }
        int a = 0, tok = -1;
        for (; a <= ks; ++a) {
            const int64_t r = off + a;
            const double* l = logits + r * V;
            double zmax = -INFINITY;
            for (int v = 0; v < V; ++v)
                if (l[v] / T > zmax) zmax = l[v] / T;
            double sum = 0.0;
            for (int v = 0; v < V; ++v) sum += exp(l[v] / T - zmax);
            const double L = zmax + log(sum);
            const int32_t* rc = row_ctr + 2 * r;
            int rejected = 0;
            if (a < ks) {
                const int32_t x = drafts[(int64_t)s * kmax + a];
                const int32_t t = d2t ? d2t[x] : x;
                const double px = exp(l[t] / T - L), qx = (double)q[r * V + t];
                const double u = oracle_accept_uniform(rc, seed);
                const double m = fabs(log(u) - log(px / qx));
                if (m < margin[s]) margin[s] = m;
                if (u < px / qx) {
                    e[a] = t;
                    continue;
                }
                rejected = 1;
            }
            /* the deciding draw: residual of the rejected row, or p of the bonus row;
             * hi1/hi2: the two highest upper-bound residual scores (for the gap) */
            double b1 = -INFINITY, p1 = -INFINITY, p2 = -INFINITY, hi1 = -INFINITY, hi2 = -INFINITY;
            int i1 = -1, ip = -1, ih1 = -1;
            for (int v = 0; v < V; ++v) {
                const double g = row_gumbel((uint32_t)v, rc, key);
                const double z = l[v] / T;
                if (z + g > p1) {
                    p2 = p1;
                    p1 = z + g;
                    ip = v;
                } else if (z + g > p2) {
                    p2 = z + g;
                }
                if (!rejected) continue;
                const double pv = exp(z - L);
                const double w = pv - (double)q[r * V + v];
                if (w > 0.0 && log(w) + g > b1) {
                    b1 = log(w) + g;
                    i1 = v;
                }
                const double whi = w + rel * pv;
                if (whi > 0.0) {
                    const double sh = log(whi) + g;
                    if (sh > hi1) {
                        hi2 = hi1;
                        hi1 = sh;
                        ih1 = v;
                    } else if (sh > hi2) {
                        hi2 = sh;
                    }
                }
            }
            if (rejected && i1 >= 0) {
                tok = i1;
                const double pw = exp(l[i1] / T - L);
                const double wlo = pw - (double)q[r * V + i1] - rel * pw;
                const double lo = wlo > 0.0 ? log(wlo) + row_gumbel((uint32_t)i1, rc, key) : -INFINITY;
                gap[s] = lo - (ih1 == i1 ? hi2 : hi1);
            } else {
                tok = ip;
                gap[s] = p1 - p2 - 2.0 * log1p(rel);
            }
            break;
        }
        e[a] = tok;
        st[s] = 0;
        accept_len[s] = a;
        n_emit[s] = a + 1;
        next_tok[s] = tok;
        pos_out[s] = pos_in[s] + a + 1;
        off += ks + 1;
    }
}

/* ---------------------------------------------------------------------------
 * Stop tokens and a generation limit, applied to the outputs of an acceptance walk
 * (oxinfer step: the committed tokens end after the first stop token and the session
 * advances by the number committed; DSSD _commit: truncation at a stop token or at
 * max_new). For every sequence with st[s] == 0, with out = emit[s][0 .. n_emit):
 *   c = the length of out up to and including its first stop token (|out| if none),
 *       then min(c, remaining[s])
 *   n_emit = c, emit = out[0..c) (-1 after), accept_len = min(accept_len, c),
 *   next_tok = out[c - 1], pos_out = pos_in + c,
 *   path (tree walks; NULL otherwise) keeps its first accept_len entries (-1 after),
 *   done = 1 iff out[c - 1] is a stop token or c == remaining[s].
 * remaining == NULL: no limit; remaining[s] < 1 sets ORC_BAD_LIMIT, and walk outputs
 * that are no committed round (n_emit outside 1 .. kmax + 1, accept_len outside
 * 0 .. n_emit) set ORC_BAD_ROWS; both give the outputs of a flagged sequence.
 * Sequences flagged on entry are left as they are, with done = 0. */
void oracle_truncate_stop(int32_t* emit, int32_t* n_emit, int32_t* accept_len, const int32_t* pos_in,
                          int32_t* pos_out, int32_t* next_tok, int32_t* path, int32_t kmax, const int32_t* stop_ids,
                          int32_t n_stop, const int32_t* remaining, int32_t* done, int32_t* st, int32_t B) {
    for (int s = 0; s < B; ++s) {
        done[s] = 0;
        int32_t* e = emit + (int64_t)s * (kmax + 1);
        int32_t* ph = path ? path + (int64_t)s * kmax : NULL;
        /* a walk's output that is not a committed round (no token, more than kmax + 1,
         * or an accepted count outside 0 .. n_emit) has no truncation */
        int flag = 0;
        if (st[s] == 0 && (n_emit[s] < 1 || n_emit[s] > kmax + 1 || accept_len[s] < 0 || accept_len[s] > n_emit[s]))
            flag = ORC_BAD_ROWS;
        else if (st[s] == 0 && remaining && remaining[s] < 1)
            flag = ORC_BAD_LIMIT;
        if (flag) {
            st[s] = flag;
            for (int j = 0; j <= kmax; ++j) e[j] = -1;
            if (ph)
                for (int j = 0; j < kmax; ++j) ph[j] = -1;
            accept_len[s] = -1;
            n_emit[s] = 0;
            next_tok[s] = -1;
            pos_out[s] = pos_in[s];
        }
        if (st[s]) continue;
        const int a = accept_len[s];
        int c = n_emit[s];
        int stopped = 0;
        for (int j = 0; j < c && !stopped; ++j)
            for (int q = 0; q < n_stop; ++q)
                if (e[j] == stop_ids[q]) {
                    c = j + 1;
                    stopped = 1;
                    break;
                }
        if (remaining && c >= remaining[s]) c = remaining[s];
        for (int j = c; j <= kmax; ++j) e[j] = -1;
        n_emit[s] = c;
        accept_len[s] = a < c ? a : c;
        if (ph)
            for (int j = accept_len[s]; j < kmax; ++j) ph[j] = -1;
        next_tok[s] = e[c - 1];
        pos_out[s] = pos_in[s] + c;
        int is_stop = 0;
        for (int q = 0; q < n_stop; ++q)
            if (e[c - 1] == stop_ids[q]) is_stop = 1;
        done[s] = is_stop || (remaining && c == remaining[s]);
    }
}

/* Greedy acceptance with stop tokens and a generation limit: oracle_greedy_accept,
 * then oracle_truncate_stop on its outputs (a flagged sequence gets done = 0). */
void oracle_greedy_accept_stop(const int32_t* g, const int32_t* drafts, int32_t kmax, const int32_t* k,
                               const int32_t* d2t, int32_t n_draft_vocab, int32_t V, int32_t B, int32_t R,
                               const int32_t* stop_ids, int32_t n_stop, const int32_t* remaining,
                               const int32_t* pos_in, int32_t* pos_out, int32_t* accept_len, int32_t* n_emit,
                               int32_t* emit, int32_t* next_tok, int32_t* done, int32_t* st) {
    oracle_greedy_accept(g, drafts, kmax, k, d2t, n_draft_vocab, V, B, R, pos_in, pos_out, accept_len, n_emit, emit,
                         next_tok, st);
    oracle_truncate_stop(emit, n_emit, accept_len, pos_in, pos_out, next_tok, NULL, kmax, stop_ids, n_stop, remaining,
                         done, st, B);
}
