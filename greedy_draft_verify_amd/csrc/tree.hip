// Tree (trie / star) drafts: the acceptance walk and the compaction of the accepted
// path's K/V (DSSD fast.py, _tree_cycle and _star_cycle). Rows are the tree's nodes
// in creation order; node i >= 1 carries draft i - 1 and sits in KV slot pos + i.
//
// spec_tree_accept: workgroups of 1024 threads, each computing every sequence's row
//   offset by a block scan, then walking its 16 sequences, a wave per sequence. Lane l
//   holds nodes l + 1 and l + 65 (parent, mapped draft token) and the greedy tokens
//   of the rows they are; a walk step is one ballot per half ("children of the
//   current node whose token is the current node's greedy token"), the lowest set
//   bit is the next node, and its greedy token comes from its lane by a shuffle.
// spec_kv_compact: a few workgroups per sequence. Each checks the accepted path,
//   then moves the K/V of slot pos + path[d] to slot pos + 1 + d. A thread owns one
//   K chunk (8 channels of one kv head) or one V channel for every token, so no two
//   threads touch the same bytes, and within a thread every source is read before a
//   destination can overwrite it: a destination pos + 1 + d is never the source of
//   a later step (path[d'] > d + 1 for d' > d), and earlier sources are read earlier
//   in program order.
#include "common.h"

namespace sv {

constexpr int kTreeAcceptThreads = 1024;
constexpr int kTreeMaxB = 8192;
constexpr int kTreeMaxK = 127;   // two nodes per lane below the root

__global__ __launch_bounds__(kTreeAcceptThreads) void tree_accept_kernel(
    const int32_t* __restrict__ g, const int32_t* __restrict__ drafts, int kmax,
    const int32_t* __restrict__ k, const int32_t* __restrict__ parent, const int32_t* __restrict__ d2t,
    int n_draft_vocab, int V, int B, int R, const int32_t* __restrict__ pos_in, int32_t* pos_out,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ n_emit, int32_t* __restrict__ emit,
    int32_t* __restrict__ next_tok, int32_t* __restrict__ path, int32_t* __restrict__ status) {
    __shared__ long long s_wsum[kTreeAcceptThreads / kWave];
    __shared__ int s_wbad[kTreeAcceptThreads / kWave];
    __shared__ int s_off[kTreeMaxB];
    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    constexpr int n_waves = kTreeAcceptThreads / kWave;
    // A sequence's scalars, root parent and nodes c = lane + 1, lane + 65 (parent,
    // draft) up to kmax; for a wave's first sequence they are requested before the
    // row-offset scan, the greedy tokens right after it.
    int ks = 0, p = 0, root = -1, par_k[2] = {-2, -2}, x_k[2] = {0, 0};
    auto fetch = [&](int s) {
        ks = k[s];
        p = pos_in[s];
        root = parent[(size_t)s * (kmax + 1)];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int c = lane + 1 + 64 * h;
            par_k[h] = c <= kmax ? parent[(size_t)s * (kmax + 1) + c] : -2;
            x_k[h] = c <= kmax ? drafts[(size_t)s * kmax + c - 1] : 0;
        }
    };
    const int s_first = blockIdx.x * n_waves + wave;
    if (s_first < B) fetch(s_first);
    const bool packing_ok = block_row_offsets<kTreeAcceptThreads>(k, B, R, s_wsum, s_wbad, s_off);

    for (int s = s_first; s < B; s += gridDim.x * n_waves) {
        if (s != s_first) fetch(s);
        const int off = s_off[s];
        int bits = 0;
        if (!packing_ok || ks > kmax) bits |= SPEC_STATUS_BAD_ROWS;
        if (p < 0) bits |= SPEC_STATUS_BAD_POS;
        int32_t* e = emit + (size_t)s * (kmax + 1);
        int32_t* ph = path + (size_t)s * kmax;
        // nodes c0 = lane + 1 and c1 = lane + 65: parent, mapped token, greedy token
        int par[2] = {-2, -2}, tok[2] = {-1, -1}, gn[2] = {0, 0};
        int g_root = 0;
        if (!bits) {
            // rows off .. off + ks are in range (the packing is defined)
            g_root = g[off];
            if (root != -1) bits |= SPEC_STATUS_BAD_TREE;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = lane + 1 + 64 * h;
                if (c > ks) continue;
                par[h] = par_k[h];
                if (par[h] < 0 || par[h] >= c) bits |= SPEC_STATUS_BAD_TREE;
                const int x = x_k[h];
                int mapped = x;
                if (d2t) {
                    if (x < 0 || x >= n_draft_vocab) {
                        bits |= SPEC_STATUS_BAD_TOKEN;
                    } else {
                        mapped = d2t[x];
                        if (mapped < 0 || mapped >= V) bits |= SPEC_STATUS_BAD_TOKEN;
                    }
                } else if (x < 0 || x >= V) {
                    bits |= SPEC_STATUS_BAD_TOKEN;
                }
                tok[h] = mapped;
                gn[h] = g[off + c];
            }
#pragma unroll
            for (int d = 32; d > 0; d >>= 1) bits |= __shfl_xor(bits, d);
        }
        if (bits) {
            for (int j = lane; j <= kmax; j += kWave) e[j] = -1;
            for (int j = lane; j < kmax; j += kWave) ph[j] = -1;
            if (lane == 0) {
                status[s] = bits;
                accept_len[s] = -1;
                n_emit[s] = 0;
                next_tok[s] = -1;
                pos_out[s] = p;
            }
            continue;
        }
        // the walk: u = current node, gu = its greedy token; lane d % 64 keeps step d
        int u = 0, gu = g_root, a = 0;
        int path_lo = -1, path_hi = -1, emit_lo = -1, emit_hi = -1;   // steps lane, lane + 64
        for (;;) {
            const unsigned long long lo = __ballot(par[0] == u && tok[0] == gu);
            const unsigned long long hi = __ballot(par[1] == u && tok[1] == gu);
            if (!lo && !hi) break;
            const int h = lo ? 0 : 1;
            const int src = (int)__builtin_ctzll(lo ? lo : hi);
            const int nxt = src + 1 + 64 * h;
            const int t = h ? __shfl(tok[1], src) : __shfl(tok[0], src);
            const int gv = h ? __shfl(gn[1], src) : __shfl(gn[0], src);
            if (lane == (a & 63)) {
                if (a < 64) {
                    path_lo = nxt;
                    emit_lo = t;
                } else {
                    path_hi = nxt;
                    emit_hi = t;
                }
            }
            ++a;
            u = nxt;
            gu = gv;
        }
        if (lane == (a & 63)) {                      // the bonus token
            if (a < 64) emit_lo = gu;
            else emit_hi = gu;
        }
        if (lane <= kmax) e[lane] = emit_lo;
        if (lane + 64 <= kmax) e[lane + 64] = emit_hi;
        if (lane < kmax) ph[lane] = path_lo;
        if (lane + 64 < kmax) ph[lane + 64] = path_hi;
        if (lane == 0) {
            status[s] = 0;
            accept_len[s] = a;
            n_emit[s] = a + 1;
            next_tok[s] = gu;
            pos_out[s] = p + a + 1;
        }
    }
}

// ---------------------------------------------------------------------------
constexpr int kCompactThreads = 256;
constexpr int kCompactBatch = 8;     // path steps whose sources one thread requests at once
constexpr int kCompactPages = (kPage - 1 + kTreeMaxK) / kPage + 1;   // pages of slots pos+1 .. pos+127

__device__ __forceinline__ int k_blk_off(int t, int d) {
    return (d >> 5) * 512 + ((d & 31) >> 3) * 128 + t * 8 + (d & 7);
}
__device__ __forceinline__ int v_blk_off(int t, int d) {
    return (d >> 4) * 256 + (t >> 2) * 64 + (d & 15) * 4 + (t & 3);
}

// grid (B, item blocks): item = one K chunk (kv head, 8 channels) or one V channel
// (kv head, channel) of the sequence; every workgroup of a sequence checks the path
// on its own (the same reads, from cache) and gives up on the same outcome.
// No __restrict__ on the pools: sources and destinations share them.
__global__ __launch_bounds__(kCompactThreads) void kv_compact_kernel(
    u16* k_pool, u16* v_pool, int64_t n_pages, const int32_t* __restrict__ page_table, int max_pages,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ path, const int32_t* __restrict__ accept_len,
    int kmax, int Hkv, int D, int32_t* __restrict__ status) {
    __shared__ int s_flags;
    __shared__ int s_first;              // first step whose source differs from its destination
    __shared__ int s_pid[kCompactPages]; // page ids of slots pos + 1 .. pos + kmax
    __shared__ int64_t s_src[kTreeMaxK], s_dst[kTreeMaxK];   // block base element of each step
    __shared__ int s_srct[kTreeMaxK], s_dstt[kTreeMaxK];     // in-block token of each step
    const int s = blockIdx.x, tid = threadIdx.x;
    const int st0 = status[s];
    const int a = accept_len[s];
    const int P = pos[s];
    if (st0 != 0 || a <= 0) return;      // flagged upstream, or nothing moves
    // one round of loads: the path and the page ids of every slot a path may touch
    int u = 0, prev = 0;
    if (tid < a && a <= kmax) {
        u = path[(size_t)s * kmax + tid];
        prev = tid ? path[(size_t)s * kmax + tid - 1] : 0;
    }
    const long long pg_first = ((long long)P + 1) / kPage;
    if (tid < kCompactPages && P >= 0) {
        const long long pg = pg_first + tid;
        s_pid[tid] = page_table[(size_t)s * max_pages + (pg < max_pages ? pg : max_pages - 1)];
    }
    if (tid == 0) {
        s_flags = 0;
        s_first = a;
    }
    __syncthreads();
    int flags = 0;
    if (a > kmax) flags |= SPEC_STATUS_BAD_TREE;
    if (P < 0) flags |= SPEC_STATUS_BAD_POS;
    if (!flags && tid < a) {
        if (u <= prev || u > kmax) {
            flags |= SPEC_STATUS_BAD_TREE;
        } else {
            const long long src = (long long)P + u, dst = (long long)P + 1 + tid;
            if (src / kPage >= max_pages) {
                flags |= SPEC_STATUS_BAD_POS;
            } else {
                const int ps = s_pid[src / kPage - pg_first];
                const int pd = s_pid[dst / kPage - pg_first];
                if (ps < 0 || ps >= n_pages || pd < 0 || pd >= n_pages) flags |= SPEC_STATUS_BAD_PAGE;
                s_src[tid] = (int64_t)ps * Hkv * (kPage * D);
                s_dst[tid] = (int64_t)pd * Hkv * (kPage * D);
                s_srct[tid] = (int)(src % kPage);
                s_dstt[tid] = (int)(dst % kPage);
                if (u != tid + 1) atomicMin(&s_first, tid);
            }
        }
    }
    if (flags) atomicOr(&s_flags, flags);
    __syncthreads();
    if (s_flags) {
        if (blockIdx.y == 0 && tid == 0) status[s] = s_flags;
        return;
    }
    const int d0 = s_first;
    const int kch = D / 8;
    const int n_k = Hkv * kch, n_items = n_k + Hkv * D;
    const int it = blockIdx.y * kCompactThreads + tid;
    if (it >= n_items) return;
    if (it < n_k) {
        const int hk = it / kch, dc = it % kch;
        const int64_t col = (int64_t)hk * (kPage * D);
        for (int d = d0; d < a; d += kCompactBatch) {
            uint4 v[kCompactBatch];
#pragma unroll
            for (int i = 0; i < kCompactBatch; ++i)
                if (d + i < a) v[i] = ld16(k_pool + s_src[d + i] + col + k_blk_off(s_srct[d + i], dc * 8));
#pragma unroll
            for (int i = 0; i < kCompactBatch; ++i)
                if (d + i < a) st16(k_pool + s_dst[d + i] + col + k_blk_off(s_dstt[d + i], dc * 8), v[i]);
        }
    } else {
        const int c = it - n_k;
        const int hk = c / D, ch = c % D;
        const int64_t col = (int64_t)hk * (kPage * D);
        for (int d = d0; d < a; d += kCompactBatch) {
            u16 v[kCompactBatch];
#pragma unroll
            for (int i = 0; i < kCompactBatch; ++i)
                if (d + i < a) v[i] = v_pool[s_src[d + i] + col + v_blk_off(s_srct[d + i], ch)];
#pragma unroll
            for (int i = 0; i < kCompactBatch; ++i)
                if (d + i < a) v_pool[s_dst[d + i] + col + v_blk_off(s_dstt[d + i], ch)] = v[i];
        }
    }
}

}  // namespace sv

extern "C" {

int spec_tree_accept(const int32_t* argmax, const int32_t* drafts, int32_t kmax, const int32_t* k,
                     const int32_t* parent, const int32_t* d2t, int32_t n_draft_vocab, int32_t V, int32_t B,
                     int32_t R, const int32_t* pos_in, int32_t* pos_out, int32_t* accept_len,
                     int32_t* n_emit, int32_t* emit, int32_t* next_tok, int32_t* path, int32_t* seq_status,
                     void* stream) {
    using namespace sv;
    last_error().clear();
    if (B < 1 || B > kTreeMaxB) return fail(SPEC_EINVAL, "spec_tree_accept: B=%d outside 1..%d", B, kTreeMaxB);
    if (kmax < 0 || kmax > kTreeMaxK) return fail(SPEC_EINVAL, "spec_tree_accept: kmax=%d outside 0..%d", kmax, kTreeMaxK);
    if (R < 1) return fail(SPEC_EINVAL, "spec_tree_accept: R=%d < 1", R);
    if (V < 1) return fail(SPEC_EINVAL, "spec_tree_accept: V=%d < 1", V);
    if (d2t && n_draft_vocab < 1) return fail(SPEC_EINVAL, "spec_tree_accept: d2t given with n_draft_vocab=%d", n_draft_vocab);
    if (!argmax || !k || !parent || !pos_in || !pos_out || !accept_len || !n_emit || !emit || !next_tok ||
        !seq_status || (kmax > 0 && (!drafts || !path)))
        return fail(SPEC_EINVAL, "spec_tree_accept: null required pointer");
    hipLaunchKernelGGL(tree_accept_kernel, dim3(seq_grid(B, kTreeAcceptThreads)), dim3(kTreeAcceptThreads), 0, (hipStream_t)stream, argmax,
                       drafts, kmax, k, parent, d2t, n_draft_vocab, V, B, R, pos_in, pos_out, accept_len, n_emit,
                       emit, next_tok, path, seq_status);
    SV_LAUNCH_CHECK("spec_tree_accept");
    return SPEC_OK;
}

int spec_kv_compact(spec_bf16* k_pool, spec_bf16* v_pool, int64_t n_pages, const int32_t* page_table,
                    int32_t max_pages, const int32_t* pos, const int32_t* path, const int32_t* accept_len,
                    int32_t kmax, int32_t B, int32_t Hkv, int32_t D, int32_t* seq_status, void* stream) {
    using namespace sv;
    last_error().clear();
    if (D != 64 && D != 128 && D != 256) return fail(SPEC_EINVAL, "spec_kv_compact: D=%d not in {64,128,256}", D);
    if (Hkv < 1 || Hkv > 64) return fail(SPEC_EINVAL, "spec_kv_compact: Hkv=%d outside 1..64", Hkv);
    if (B < 1) return fail(SPEC_EINVAL, "spec_kv_compact: B=%d < 1", B);
    if (kmax < 0 || kmax > kTreeMaxK) return fail(SPEC_EINVAL, "spec_kv_compact: kmax=%d outside 0..%d", kmax, kTreeMaxK);
    if (max_pages < 1 || n_pages < 1) return fail(SPEC_EINVAL, "spec_kv_compact: max_pages=%d n_pages=%lld", max_pages, (long long)n_pages);
    if (!k_pool || !v_pool || !page_table || !pos || !accept_len || !seq_status || (kmax > 0 && !path))
        return fail(SPEC_EINVAL, "spec_kv_compact: null required pointer");
    if (!aligned16(k_pool) || !aligned16(v_pool)) return fail(SPEC_EINVAL, "spec_kv_compact: k_pool and v_pool must be 16-byte aligned");
    if (kmax == 0) return SPEC_OK;   // no draft node: nothing can move
    const int n_items = Hkv * (D / 8) + Hkv * D;
    const dim3 grid(B, (n_items + kCompactThreads - 1) / kCompactThreads);
    hipLaunchKernelGGL(kv_compact_kernel, grid, dim3(kCompactThreads), 0, (hipStream_t)stream, k_pool, v_pool,
                       n_pages, page_table, max_pages, pos, path, accept_len, kmax, Hkv, D, seq_status);
    SV_LAUNCH_CHECK("spec_kv_compact");
    return SPEC_OK;
}

}  // extern "C"
