// spec_verify_attn: KV append in place + paged causal split-KV verify attention.
//
// Three launches on the caller's stream:
//   1. attn_prep_kernel  grid B: validates sequence s (row packing, positions, page
//      ids), records its row offset in the workspace, writes the rows' K/V into
//      their pool slots (span-02 spec.rs: KV appended in place at pos..pos+k).
//   2. attn_split_kernel grid (2 * n_splits, Hkv, B): one workgroup per (sequence,
//      kv head, split of kv_split_tokens positions, half of the query rows). The
//      G*T query rows of a kv head (grouped-query heads x verify rows) share every
//      K/V page: the workgroup streams the split's pages through LDS in tiles of
//      64 tokens (4 pages), each wave turns one 16-row query tile into scores with
//      bf16 MFMA (S^T = K Q^T), runs the online softmax in registers, and
//      accumulates O^T = V^T P^T with MFMA. A key t is kept for row j only if
//      t <= pos + j (kv_hi = position, memra full_attn_verify's per-row bound).
//   3. attn_combine_kernel one wave per (row, q head): merges the row's splits in
//      ascending order (log-sum-exp weights) and writes bf16.
//
// Row invariance: splits sit at absolute multiples of kv_split_tokens, tiles at
// absolute multiples of 64, every reduction runs in a fixed order, and a row reads
// only splits that contain keys <= its position. Tiles past a row's position add
// exact zeros with rescale factor exactly 1, so a row's bytes are the same whatever
// other rows share the launch.
#include "common.h"

namespace sv {

constexpr int kKT = 64;            // keys per LDS tile (4 pages)
constexpr int kAttnThreads = 256;  // 4 waves
constexpr int kMaxRowsPerKvHead = 128;
constexpr int kRowsPerGroup = 64;  // query rows one workgroup handles (4 waves x 16)
constexpr float kLog2e = 1.4426950408889634f;

struct SeqInfo {
    int32_t off;    // first packed row
    int32_t valid;  // 1 if the sequence passed validation
};

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_prep_kernel(
    const u16* __restrict__ k_new, const u16* __restrict__ v_new, u16* __restrict__ k_pool,
    u16* __restrict__ v_pool, int64_t n_pages, const int32_t* __restrict__ page_table, int max_pages,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ k, int B, int R, int Hq, int Hkv,
    int D, SeqInfo* __restrict__ info, int32_t* __restrict__ status) {
    __shared__ long long s_before[256], s_total[256];
    __shared__ int s_flags;
    const int s = blockIdx.x, tid = threadIdx.x;
    if (tid == 0) s_flags = 0;
    __syncthreads();
    long long before = 0, total = 0;
    int neg = 0;
    for (int i = tid; i < B; i += 256) {
        const long long kk = k[i];
        total += kk + 1;
        if (i < s) before += kk + 1;
        if (kk < 0) neg = 1;
    }
    if (neg) atomicOr(&s_flags, SPEC_STATUS_BAD_ROWS);
    s_before[tid] = before;
    s_total[tid] = total;
    __syncthreads();
    for (int d = 128; d > 0; d >>= 1) {
        if (tid < d) {
            s_before[tid] += s_before[tid + d];
            s_total[tid] += s_total[tid + d];
        }
        __syncthreads();
    }
    const int ks = k[s];
    const int P = pos[s];
    if (tid == 0) {
        int bits = 0;
        if (s_total[0] != (long long)R) bits |= SPEC_STATUS_BAD_ROWS;
        if (ks >= 0 && (long long)(Hq / Hkv) * (ks + 1) > kMaxRowsPerKvHead) bits |= SPEC_STATUS_TOO_WIDE;
        if (P < 0) {
            bits |= SPEC_STATUS_BAD_POS;
        } else if (ks >= 0 && ((long long)P + ks) / kPage >= max_pages) {
            bits |= SPEC_STATUS_BAD_POS;
        }
        atomicOr(&s_flags, bits);
    }
    __syncthreads();
    if (!(s_flags & SPEC_STATUS_BAD_POS) && ks >= 0) {
        const int last_page = (int)(((long long)P + ks) / kPage);
        int bad = 0;
        for (int pg = tid; pg <= last_page; pg += 256) {
            const int id = page_table[(size_t)s * max_pages + pg];
            if (id < 0 || id >= n_pages) bad = 1;
        }
        if (bad) atomicOr(&s_flags, SPEC_STATUS_BAD_PAGE);
    }
    __syncthreads();
    const int bits = s_flags;
    const int off = (int)s_before[0];
    if (tid == 0) {
        status[s] = bits;
        info[s].off = off;
        info[s].valid = bits == 0;
    }
    if (bits) return;
    // append: one 16-byte chunk (8 channels) per item
    const int dch = D / 8;
    const int n = (ks + 1) * Hkv * dch;
    for (int i = tid; i < n; i += 256) {
        const int dc = i % dch;
        const int rest = i / dch;
        const int hk = rest % Hkv;
        const int j = rest / Hkv;
        const int p = P + j;
        const int64_t page = page_table[(size_t)s * max_pages + p / kPage];
        const int t = p % kPage;
        const size_t src = ((size_t)(off + j) * Hkv + hk) * D + dc * 8;
        st16(k_pool + ((size_t)(page * Hkv + hk) * kPage + t) * D + dc * 8, ld16(k_new + src));
        const uint4 vv = ld16(v_new + src);
        u16* vdst = v_pool + ((size_t)(page * Hkv + hk) * D + dc * 8) * kPage + t;
        const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vdst[(2 * e) * kPage] = (u16)(w[e] & 0xffffu);
            vdst[(2 * e + 1) * kPage] = (u16)(w[e] >> 16);
        }
    }
}

// ---------------------------------------------------------------------------
template <int D>
struct AttnTile {
    static constexpr int KSTR = D + 8;    // K tile row stride (elements): token-major
    static constexpr int VSTR = kKT + 8;  // V tile row stride (elements): channel-major
    static constexpr int K_ELEMS = kKT * KSTR;
    static constexpr int V_ELEMS = D * VSTR;
    static constexpr int CHUNKS = 16 * D;  // 16-byte chunks per tile (K + V, 4 pages)
    static constexpr int PER_THREAD = CHUNKS / kAttnThreads;
    static constexpr int LDS_BYTES = (K_ELEMS + V_ELEMS) * 2;
};

template <int D>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_split_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k_pool, const u16* __restrict__ v_pool,
    const int32_t* __restrict__ page_table, int max_pages, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ k, const SeqInfo* __restrict__ info, int Hq, int Hkv,
    float scale_log2, int split, int n_splits, float2* __restrict__ part_ml,
    float* __restrict__ part_o) {
    using TL = AttnTile<D>;
    constexpr int NDS = D / 32;  // QK^T k-steps
    constexpr int NDT = D / 16;  // PV output tiles
    __shared__ __attribute__((aligned(16))) u16 smem[TL::K_ELEMS + TL::V_ELEMS];
    u16* Ks = smem;
    u16* Vs = smem + TL::K_ELEMS;

    const int c = blockIdx.x % n_splits;
    const int mgroup = blockIdx.x / n_splits;
    const int hk = blockIdx.y;
    const int s = blockIdx.z;
    const SeqInfo si = info[s];
    if (!si.valid) return;
    const int G = Hq / Hkv;
    const int T = k[s] + 1;
    const int M = G * T;
    const int P0 = pos[s];
    const int last = P0 + T - 1;
    const int c0 = c * split;
    if (c0 > last) return;
    if (mgroup * kRowsPerGroup >= M) return;
    const int c1 = min(c0 + split, last + 1);

    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int l16 = lane % 16, lq = lane / 16;
    const int m_tile0 = mgroup * kRowsPerGroup + wave * 16;
    const bool active = m_tile0 < M;

    // this lane's query row (B operand column / output column)
    const int m = m_tile0 + l16;
    const bool m_ok = m < M;
    const int jrow = m_ok ? m / G : 0;
    const int p_m = m_ok ? P0 + jrow : -1;  // kv_hi of this query row
    bf16x8 qf[NDS];
    if (active) {
        const size_t qoff = ((size_t)(si.off + jrow) * Hq + hk * G + (m_ok ? m % G : 0)) * D;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
            uint4 v = m_ok ? ld16(q + qoff + ds * 32 + lq * 8) : make_uint4(0, 0, 0, 0);
            qf[ds] = as_bf16x8(v);
        }
    }
    f32x4 o[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_lane = 0.f;

    const int32_t* pt = page_table + (size_t)s * max_pages;
    const int last_page = last / kPage;

    // staging registers for the next tile
    uint4 stage[TL::PER_THREAD];
    auto load_tile = [&](int t0) {
#pragma unroll
        for (int it = 0; it < TL::PER_THREAD; ++it) {
            const int cidx = it * kAttnThreads + tid;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (cidx < 8 * D) {  // K chunk: page i, token row, 8-channel chunk
                const int i = cidx / (2 * D), cc = cidx % (2 * D);
                const int row = cc / (D / 8), dc = cc % (D / 8);
                const int pg = t0 / kPage + i;
                if (pg <= last_page) {
                    const int64_t page = pt[pg];
                    v = ld16(k_pool + ((size_t)(page * Hkv + hk) * kPage + row) * D + dc * 8);
                }
            } else {  // V chunk: page i, channel d, 8-token half
                const int c2 = cidx - 8 * D;
                const int i = c2 / (2 * D), cc = c2 % (2 * D);
                const int d = cc / 2, half = cc % 2;
                const int pg = t0 / kPage + i;
                if (pg <= last_page) {
                    const int64_t page = pt[pg];
                    v = ld16(v_pool + ((size_t)(page * Hkv + hk) * D + d) * kPage + half * 8);
                    // tokens past the sequence's last written position may hold anything:
                    // zero them so that a zero softmax weight times V stays zero
                    const int tok0 = pg * kPage + half * 8;
                    if (tok0 + 7 > last) {
                        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (tok0 + e > last) w[e / 2] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
                        v = make_uint4(w[0], w[1], w[2], w[3]);
                    }
                }
            }
            stage[it] = v;
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int it = 0; it < TL::PER_THREAD; ++it) {
            const int cidx = it * kAttnThreads + tid;
            if (cidx < 8 * D) {
                const int i = cidx / (2 * D), cc = cidx % (2 * D);
                const int row = cc / (D / 8), dc = cc % (D / 8);
                st16(Ks + (i * kPage + row) * TL::KSTR + dc * 8, stage[it]);
            } else {
                const int c2 = cidx - 8 * D;
                const int i = c2 / (2 * D), cc = c2 % (2 * D);
                const int d = cc / 2, half = cc % 2;
                st16(Vs + d * TL::VSTR + i * kPage + half * 8, stage[it]);
            }
        }
    };

    load_tile(c0);
    for (int t0 = c0; t0 < c1; t0 += kKT) {
        __syncthreads();  // previous tile's LDS reads are done
        store_tile();
        __syncthreads();
        if (t0 + kKT < c1) load_tile(t0 + kKT);
        if (!active) continue;

        // scores: lane holds, for query row m, keys t0 + 32*g2 + 8*lq + jj (jj = 0..7)
        float sc[2][8];
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
            f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
            // A-operand row l16 <-> key 8*(l16/4) + 4*sub + l16%4 of the 32-key group
            const u16* k0 = Ks + (g2 * 32 + 8 * (l16 / 4) + (l16 % 4)) * TL::KSTR + lq * 8;
            const u16* k1 = k0 + 4 * TL::KSTR;
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) {
                s0 = mfma16x16x32(as_bf16x8(ld16(k0 + ds * 32)), qf[ds], s0);
                s1 = mfma16x16x32(as_bf16x8(ld16(k1 + ds * 32)), qf[ds], s1);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sc[g2][i] = s0[i];
                sc[g2][4 + i] = s1[i];
            }
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int kp = t0 + g2 * 32 + lq * 8 + jj;
                const float x = (kp <= p_m) ? sc[g2][jj] * scale_log2 : -INFINITY;
                sc[g2][jj] = x;
                tmax = fmaxf(tmax, x);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        float psum = 0.f;
        bf16x8 pf[2];
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
            float pv[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                pv[jj] = exp2f(sc[g2][jj] - m_use);
                psum += pv[jj];
            }
            pf[g2] = pack8(pv);
        }
        l_lane = l_lane * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            f32x4 acc = o[dt] * alpha;
            const u16* vrow = Vs + (dt * 16 + l16) * TL::VSTR + lq * 8;
            acc = mfma16x16x32(as_bf16x8(ld16(vrow)), pf[0], acc);
            acc = mfma16x16x32(as_bf16x8(ld16(vrow + 32)), pf[1], acc);
            o[dt] = acc;
        }
    }
    if (!active) return;
    float l_tot = l_lane + __shfl_xor(l_lane, 16);
    l_tot = l_tot + __shfl_xor(l_tot, 32);
    if (!m_ok || p_m < c0) return;
    const size_t idx = ((size_t)(si.off + jrow) * Hq + hk * G + m % G) * n_splits + c;
    if (lq == 0) part_ml[idx] = make_float2(m_run, l_tot);
    float* po = part_o + idx * D + lq * 4;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16) = o[dt];
}

// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(
    const int32_t* __restrict__ pos, const int32_t* __restrict__ k, const SeqInfo* __restrict__ info,
    int B, int R, int Hq, int split, int n_splits, const float2* __restrict__ part_ml,
    const float* __restrict__ part_o, u16* __restrict__ out) {
    constexpr int PER = D / kWave;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const long long item = (long long)blockIdx.x * 4 + wave;
    if (item >= (long long)R * Hq) return;
    const int r = (int)(item / Hq), h = (int)(item % Hq);
    // sequence of row r: last s with off_s <= r (offsets are monotone when valid)
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (info[mid].off <= r) lo = mid; else hi = mid - 1;
    }
    const SeqInfo si = info[lo];
    if (!si.valid) return;
    const int j = r - si.off;
    if (j < 0 || j > k[lo]) return;
    const int p = pos[lo] + j;
    const int nc = p / split + 1;
    const size_t base = ((size_t)r * Hq + h) * n_splits;
    float mx = -INFINITY;
    for (int c = lane; c < nc; c += kWave) mx = fmaxf(mx, part_ml[base + c].x);
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d));
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    float L = 0.f;
    for (int c = 0; c < nc; ++c) {
        const float2 ml = part_ml[base + c];
        const float wgt = exp2f(ml.x - mx);
        L += wgt * ml.y;
        const float* po = part_o + (base + c) * D;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] += wgt * po[e * kWave + lane];
    }
    const float inv = 1.f / L;
    u16* dst = out + ((size_t)r * Hq + h) * D;
#pragma unroll
    for (int e = 0; e < PER; ++e) dst[e * kWave + lane] = f2bf(acc[e] * inv);
}

// ---------------------------------------------------------------------------
static int64_t split_count(int32_t max_pages, int32_t split) {
    return ((int64_t)max_pages * kPage + split - 1) / split;
}

struct AttnWs {
    size_t info_off, ml_off, o_off, total;
};

static AttnWs attn_ws_layout(int32_t B, int32_t R, int32_t Hq, int32_t D, int64_t n_splits) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    AttnWs w;
    w.info_off = 0;
    w.ml_off = up(sizeof(SeqInfo) * (size_t)B);
    w.o_off = w.ml_off + up(sizeof(float2) * (size_t)R * Hq * n_splits);
    w.total = w.o_off + up(sizeof(float) * (size_t)R * Hq * n_splits * D);
    return w;
}

template <int D>
static void launch_attn(const u16* q, const u16* k_pool, const u16* v_pool, const int32_t* pt,
                        int max_pages, const int32_t* pos, const int32_t* k, const SeqInfo* info,
                        int B, int R, int Hq, int Hkv, float scale, int split, int n_splits,
                        float2* ml, float* po, u16* out, hipStream_t st) {
    dim3 grid(2 * n_splits, Hkv, B);
    hipLaunchKernelGGL(attn_split_kernel<D>, grid, dim3(kAttnThreads), 0, st, q, k_pool, v_pool, pt,
                       max_pages, pos, k, info, Hq, Hkv, scale * kLog2e, split, n_splits, ml, po);
    const long long items = (long long)R * Hq;
    hipLaunchKernelGGL(attn_combine_kernel<D>, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, st,
                       pos, k, info, B, R, Hq, split, n_splits, ml, po, out);
}

}  // namespace sv

extern "C" {

int32_t spec_attn_split_tokens(int32_t max_pages) {
    // Capacity-derived: the smallest power of two >= 256 that cuts the page table's
    // capacity into at most 64 splits, capped at 2048 tokens.
    const int64_t cap = (int64_t)(max_pages > 0 ? max_pages : 1) * SPEC_PAGE_TOKENS;
    int32_t s = 256;
    while (s < 2048 && cap > 64 * (int64_t)s) s *= 2;
    return s;
}

size_t spec_verify_attn_workspace_bytes(int32_t B, int32_t R, int32_t Hq, int32_t Hkv, int32_t D,
                                        int32_t max_pages, int32_t kv_split_tokens) {
    (void)Hkv;
    if (B < 1 || R < 1 || Hq < 1 || D < 1 || max_pages < 1) return 0;
    const int32_t split = kv_split_tokens > 0 ? kv_split_tokens : spec_attn_split_tokens(max_pages);
    return sv::attn_ws_layout(B, R, Hq, D, sv::split_count(max_pages, split)).total;
}

int spec_verify_attn(const spec_bf16* q, const spec_bf16* k_new, const spec_bf16* v_new,
                     spec_bf16* k_pool, spec_bf16* v_pool, int64_t n_pages,
                     const int32_t* page_table, int32_t max_pages, const int32_t* pos,
                     const int32_t* k, int32_t B, int32_t R, int32_t Hq, int32_t Hkv, int32_t D,
                     float scale, int32_t kv_split_tokens, spec_bf16* out, void* workspace,
                     size_t workspace_bytes, int32_t* seq_status, void* stream) {
    using namespace sv;
    last_error().clear();
    if (D != 64 && D != 128 && D != 256) return fail(SPEC_EINVAL, "spec_verify_attn: D=%d not in {64,128,256}", D);
    if (Hkv < 1 || Hq < Hkv || Hq % Hkv) return fail(SPEC_EINVAL, "spec_verify_attn: Hq=%d Hkv=%d (need Hq %% Hkv == 0)", Hq, Hkv);
    if (Hq / Hkv > 16) return fail(SPEC_EINVAL, "spec_verify_attn: Hq/Hkv=%d > 16", Hq / Hkv);
    if (B < 1 || B > 4096) return fail(SPEC_EINVAL, "spec_verify_attn: B=%d outside 1..4096", B);
    if (R < 1) return fail(SPEC_EINVAL, "spec_verify_attn: R=%d < 1", R);
    if (max_pages < 1 || n_pages < 1) return fail(SPEC_EINVAL, "spec_verify_attn: max_pages=%d n_pages=%lld", max_pages, (long long)n_pages);
    if (!(scale > 0.f)) return fail(SPEC_EINVAL, "spec_verify_attn: scale must be > 0");
    if (kv_split_tokens < 0 || kv_split_tokens % kKT) return fail(SPEC_EINVAL, "spec_verify_attn: kv_split_tokens=%d not a multiple of 64", kv_split_tokens);
    if (!q || !k_new || !v_new || !k_pool || !v_pool || !page_table || !pos || !k || !out || !seq_status)
        return fail(SPEC_EINVAL, "spec_verify_attn: null required pointer");
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
        return fail(SPEC_EINVAL, "spec_verify_attn: q, k_new, v_new, k_pool, v_pool and out must be 16-byte aligned");
    const int32_t split = kv_split_tokens > 0 ? kv_split_tokens : spec_attn_split_tokens(max_pages);
    const int64_t n_splits = split_count(max_pages, split);
    if (n_splits * 2 > 0x7fffffffLL) return fail(SPEC_ECAPACITY, "spec_verify_attn: too many splits");
    const AttnWs lay = attn_ws_layout(B, R, Hq, D, n_splits);
    if (!workspace || workspace_bytes < lay.total || !aligned16(workspace))
        return fail(SPEC_EWORKSPACE, "spec_verify_attn: workspace %zu bytes < %zu required (or null/misaligned)", workspace_bytes, lay.total);
    char* ws = static_cast<char*>(workspace);
    SeqInfo* info = reinterpret_cast<SeqInfo*>(ws + lay.info_off);
    float2* ml = reinterpret_cast<float2*>(ws + lay.ml_off);
    float* po = reinterpret_cast<float*>(ws + lay.o_off);
    hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL(attn_prep_kernel, dim3(B), dim3(256), 0, st, k_new, v_new, k_pool, v_pool,
                       n_pages, page_table, max_pages, pos, k, B, R, Hq, Hkv, D, info, seq_status);
    SV_LAUNCH_CHECK("spec_verify_attn(prep)");
    switch (D) {
        case 64: launch_attn<64>(q, k_pool, v_pool, page_table, max_pages, pos, k, info, B, R, Hq, Hkv, scale, split, (int)n_splits, ml, po, out, st); break;
        case 128: launch_attn<128>(q, k_pool, v_pool, page_table, max_pages, pos, k, info, B, R, Hq, Hkv, scale, split, (int)n_splits, ml, po, out, st); break;
        default: launch_attn<256>(q, k_pool, v_pool, page_table, max_pages, pos, k, info, B, R, Hq, Hkv, scale, split, (int)n_splits, ml, po, out, st); break;
    }
    SV_LAUNCH_CHECK("spec_verify_attn");
    return SPEC_OK;
}

}  // extern "C"
