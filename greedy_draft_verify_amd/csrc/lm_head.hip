// spec_lm_head_argmax: bf16 MFMA lm_head with the greedy argmax fused into the
// epilogue; the logits never leave registers.
//
// W is consumed in a packed form made once by spec_lm_head_pack. A row-major
// [V][H] matrix read as MFMA fragments touches 16 rows x 64 bytes per wave
// instruction, which caps the stream far below HBM peak. The packed form is
// group-major: a group is 128 vocabulary rows (one workgroup's share), a K-block
// is 128 channels, and the group's 8 tiles of 16 rows store, K-block by K-block,
// their 4 k-steps as the 64 lanes' MFMA B fragments in lane order (1 KB each).
// A workgroup therefore streams one contiguous region, 32 KB per K-block, and
// every wave instruction is one contiguous 1 KB read. The packing is a byte
// permutation, so results are identical.
//
// lm_head_tile_kernel: one workgroup per (group of 128 vocabulary entries, group
// of up to 128 rows). Each wave owns two 16-row tiles of W and streams them from
// HBM straight into MFMA B-operand registers with non-temporal loads (W is read
// once and must not push the hidden rows out of L2) through a ring of one
// K-block: a k-step's fragments are re-requested for the next K-block as soon as
// its MFMAs are issued, and every load is unconditional so the in-order load
// counter never has to drain. The hidden rows are shared by the four waves through
// LDS, one K-block ahead. After the K loop each wave reduces its logits to the best
// (value, index) per row with the order "larger value, then smaller index" (the
// first-maximum rule of span-02 greedy_logprob), the workgroup merges its four
// waves and folds the result into one 64-bit key per row with an atomic maximum
// (the key's unsigned order is that same order). A ticket counter finds the last
// workgroup, which writes argmax/maxval from the keys and resets the workspace to
// zero. The order is total, so the result does not depend on which workgroup
// finishes when; each logit is one MFMA chain over K in a fixed order, so a row's
// result does not depend on R or the row group.
#include <mutex>
#include <type_traits>
#include <utility>

#include "common.h"

namespace sv {

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>): a loop
// whose index is a compile-time constant in every copy of the body.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr int kLmThreads = 256;
constexpr int kLmNT = 2;                  // 16-entry vocabulary tiles per wave
constexpr int kLmTiles = 4 * kLmNT;       // tiles per group (one workgroup)
constexpr int kLmVocabPerWg = 16 * kLmTiles;
constexpr int kLmKB = 128;                // channels per K-block
constexpr int kLmKS = kLmKB / 32;         // MFMA k-steps per K-block
constexpr int kLmMaxMT = 8;               // 16-row tiles per row group
constexpr int kLmHAlign = 256;            // H must be a multiple of this
// Few-row paths. Greedy: one key per (vocabulary workgroup, row) in rows of this
// stride (R rounded up to 8 keys, so a row starts on a 64-byte boundary). Sampling,
// up to kLmSampleRecordsMaxR rows: one 16-byte record per (row, vocabulary group).
__host__ __device__ constexpr int key_rows_stride(int R) { return (R + 7) / 8 * 8; }
constexpr int kLmSampleRecordsMaxR = 64;

// Packed W: fragment f = (((g * H/128 + kb) * 8 + t) * 4 + s) * 64 + lane holds
// W[128 g + 16 t + lane % 16][128 kb + 32 s + 8 (lane / 16) .. + 8] (zero past V).
__global__ __launch_bounds__(256) void lm_head_pack_kernel(const u16* __restrict__ w, int V, int H,
                                                           u16* __restrict__ wp) {
    const size_t nkb = (size_t)(H / kLmKB);
    const size_t nfrag = (size_t)((V + kLmVocabPerWg - 1) / kLmVocabPerWg) * nkb * kLmTiles * kLmKS * 64;
    for (size_t f = (size_t)blockIdx.x * blockDim.x + threadIdx.x; f < nfrag;
         f += (size_t)gridDim.x * blockDim.x) {
        const int lane = (int)(f % 64);
        size_t t = f / 64;
        const int s = (int)(t % kLmKS);
        t /= kLmKS;
        const int tile = (int)(t % kLmTiles);
        t /= kLmTiles;
        const size_t kb = t % nkb, g = t / nkb;
        const size_t v = g * kLmVocabPerWg + (size_t)tile * 16 + lane % 16;
        const size_t k = kb * kLmKB + (size_t)s * 32 + (lane / 16) * 8;
        st16(wp + f * 8, v < (size_t)V ? ld16(w + v * H + k) : make_uint4(0, 0, 0, 0));
    }
}

// Sampling epilogue (speculative-sampling verify): per row, the workgroup's
// softmax partial (max and sum of exp of z = logit / T over its 128 entries), the
// z of the row's draft-support tokens, the best z + Gumbel noise over the entries
// outside that support, and (dense drafts) every entry's z.
struct SampleArgs {
    const int32_t* q_tok;     // [R][NQ] draft support per row (-1: unused)
    const int32_t* row_ctr;   // [R][2] Philox counter words of the row
    float2* part;             // [R][n_vt] (max, sum of exp) per vocabulary group; best keys by atomics
    float4* part4;            // or, at few rows: [R][n_vt] (max, sum of exp, best key's low and high words)
    float* z_supp;            // [R][NQ]
    float* z_out;             // [R][V] z of every entry, or null
    float inv_t;
    int NQ;
    uint32_t key0, key1;
};

__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2) {
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;   // both empty
    s = s * __expf(m - mn) + s2 * __expf(m2 - mn);
    m = mn;
}

// acc[mt][nt][i] = logit of row 16 mt + 4 (lane / 16) + i, entry 16 (tile0 + nt) + lane % 16.
// Gumbel noise of (row, v) is word v % 4 of Philox(ctr = (v / 4, row_ctr[row]), key):
// the four lanes 4c..4c+3 of a 16-lane group hold the same v / 4 and the same four
// rows, so lane 4c + b computes row b's block and a 4x4 transpose by shuffles hands
// every lane the words it needs (one block per lane per (mt, nt)).
template <int MT>
__device__ __forceinline__ void sample_epilogue(const f32x4 (&acc)[MT][kLmNT], const SampleArgs& sa, int r0, int R,
                                                int V, int vt, int n_vt, int tile0, int tid, int wave, int lane,
                                                const uint4* s_sup, float2 (*s_ms)[16 * MT],
                                                Best (*wbest)[16 * MT], unsigned long long* keys) {
    const int l16 = lane % 16, lq = lane / 16, b = lane & 3;
    // The row tiles are expanded at compile time: the body is too large for the
    // unroller at MT = 8, and a loop-carried tile index would put acc in scratch memory.
    static_for<MT>([&](auto mt_c) {
        constexpr int mt = decltype(mt_c)::value;
        // this lane's Philox row: row 16 mt + 4 lq + b
        const int rb = min(r0 + mt * 16 + lq * 4 + b, R - 1);
        const uint32_t ca = (uint32_t)sa.row_ctr[2 * (size_t)rb], cb = (uint32_t)sa.row_ctr[2 * (size_t)rb + 1];
        float g[kLmNT][4];   // g[nt][i]: noise of (row 4 lq + i, entry of this lane)
#pragma unroll
        for (int nt = 0; nt < kLmNT; ++nt) {
            const uint32_t v4 = (uint32_t)(((tile0 + nt) * 16 + l16) >> 2);
            const uint4 w = philox10(make_uint4(v4, ca, cb, 0u), sa.key0, sa.key1);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                // lane b takes word b of lane (b + d) % 4's block (row (b + d) % 4) and
                // gives word (b - d) % 4 of its own
                const int sel = (b - d) & 3;
                const uint32_t send = sel == 0 ? w.x : sel == 1 ? w.y : sel == 2 ? w.z : w.w;
                const int src = (lane & ~3) | ((b + d) & 3);
                const uint32_t got = d == 0 ? send : (uint32_t)__shfl((int)send, src);
                // slot (b + d) % 4 differs per lane: select it with constant indices (a
                // lane-dependent index would put g in scratch memory)
                const float gv = gumbel(got);
                const int slot = (b + d) & 3;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (slot == q) g[nt][q] = gv;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rl = mt * 16 + lq * 4 + i;     // row inside the row group
            const int r = r0 + rl;
            const uint4 sup = s_sup[rl];
            float m = -INFINITY, sm = 0.f;
            float bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int nt = 0; nt < kLmNT; ++nt) {
                const int v = (tile0 + nt) * 16 + l16;
                if (v >= V) continue;
                const float z = acc[mt][nt][i] * sa.inv_t;
                ms_merge(m, sm, z, 1.f);
                const int loc = v - vt * kLmVocabPerWg;
                const uint32_t word = loc < 32 ? sup.x : loc < 64 ? sup.y : loc < 96 ? sup.z : sup.w;
                if ((word >> (loc & 31)) & 1u) {
                    // a support token: its z goes to the finalize (rare path)
                    if (r < R)
                        for (int e = 0; e < sa.NQ; ++e)
                            if (sa.q_tok[(size_t)r * sa.NQ + e] == v) sa.z_supp[(size_t)r * sa.NQ + e] = z;
                } else if (better(z + g[nt][i], v, bv, bi)) {
                    bv = z + g[nt][i];
                    bi = v;
                }
            }
            // the 16 lanes of the row, in a fixed butterfly (every lane ends with the same)
#pragma unroll
            for (int d = 1; d < 16; d <<= 1) {
                const float om = __shfl_xor(m, d), os = __shfl_xor(sm, d);
                ms_merge(m, sm, om, os);
                const float ov = __shfl_xor(bv, d);
                const int oi = __shfl_xor(bi, d);
                if (better(ov, oi, bv, bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
            if (l16 == 0) {
                s_ms[wave][rl] = make_float2(m, sm);
                wbest[wave][rl] = Best{bv, bi};
            }
        }
    });
    __syncthreads();
    if (tid < 16 * MT && r0 + tid < R) {
        const int r = r0 + tid;
        float m = s_ms[0][tid].x, sm = s_ms[0][tid].y;
        Best bb = wbest[0][tid];
#pragma unroll
        for (int wv = 1; wv < 4; ++wv) {   // waves in order
            ms_merge(m, sm, s_ms[wv][tid].x, s_ms[wv][tid].y);
            const Best o = wbest[wv][tid];
            if (better(o.v, o.i, bb.v, bb.i)) bb = o;
        }
        if (sa.part4) {
            // few rows: one 16-byte record per (row, group), merged by the finalize (the
            // atomics would queue at the end of the kernel, as in the greedy pass)
            const unsigned long long key = bb.i != 0x7fffffff ? pack_best(bb) : 0ull;
            sa.part4[(size_t)r * n_vt + vt] =
                make_float4(m, sm, __uint_as_float((uint32_t)key), __uint_as_float((uint32_t)(key >> 32)));
        } else {
            sa.part[(size_t)r * n_vt + vt] = make_float2(m, sm);
            if (bb.i != 0x7fffffff) atomicMax(keys + r, pack_best(bb));
        }
    }
}

// Dense drafts: every entry's z, staged through LDS two 16-row tiles at a time so
// that each row's 128 entries of this group leave as 16-byte row-contiguous stores,
// non-temporal: z is read back by later kernels, not by this one, and streaming it
// past the L2 measured 233 vs 247 us for the b16k4 pass (222 with no z at all).
constexpr int kZStride = kLmVocabPerWg + 4;   // LDS row stride (floats): spreads the 4 row groups over banks

template <int MT>
__device__ __forceinline__ void write_z(const f32x4 (&acc)[MT][kLmNT], const SampleArgs& sa, int r0, int R, int V,
                                        int vt, int tid, int wave, int lane, float* zbuf) {
    const int l16 = lane % 16, lq = lane / 16;
    const bool vec = (V & 3) == 0;
#pragma unroll
    for (int m0 = 0; m0 < MT; m0 += 2) {
        __syncthreads();   // the previous pass's reads of zbuf are done
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
            if (m0 + mm >= MT) break;
#pragma unroll
            for (int nt = 0; nt < kLmNT; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    zbuf[(mm * 16 + lq * 4 + i) * kZStride + (wave * kLmNT + nt) * 16 + l16] =
                        acc[m0 + mm][nt][i] * sa.inv_t;
        }
        __syncthreads();
        const int rows = (m0 + 1 < MT ? 2 : 1) * 16;
        for (int c = tid; c < rows * (kLmVocabPerWg / 4); c += kLmThreads) {
            const int rl = c / (kLmVocabPerWg / 4), q4 = c % (kLmVocabPerWg / 4);
            const int r = r0 + m0 * 16 + rl;
            const int v0 = vt * kLmVocabPerWg + q4 * 4;
            if (r >= R || v0 >= V) continue;
            const float4 val = *reinterpret_cast<const float4*>(zbuf + rl * kZStride + q4 * 4);
            float* dst = sa.z_out + (size_t)r * V + v0;
            if (vec && v0 + 3 < V) {
                __builtin_nontemporal_store(f32x4{val.x, val.y, val.z, val.w}, reinterpret_cast<f32x4*>(dst));
            } else {
                const float e4[4] = {val.x, val.y, val.z, val.w};
                for (int e = 0; e < 4 && v0 + e < V; ++e) dst[e] = e4[e];
            }
        }
    }
}

// NT: 16-entry vocabulary tiles per wave. At NT = 2 a workgroup covers one packed
// group of 128 entries; at NT = 4 it covers two adjacent groups (wave w takes tiles
// 2w, 2w + 1 of each), so every hidden fragment read from LDS feeds twice as many
// MFMAs and the hidden rows are staged once per 256 entries (the packed layout is
// the same). SHARED: other row groups re-read this vocabulary group's W through the
// XCD's L2, so W is loaded with the default cache policy instead of as a stream.
template <int MT, int NT, bool SHARED, bool SAMPLE = false>
__global__ __launch_bounds__(kLmThreads, 2) void lm_head_tile_kernel(
    const u16* __restrict__ hidden, const u16* __restrict__ wp, int R, int H, int V, int n_vt,
    int n_rg, unsigned long long* __restrict__ keys, unsigned int* __restrict__ ticket,
    int32_t* __restrict__ argmax, float* __restrict__ maxval, SampleArgs sa,
    unsigned long long* __restrict__ key_rows) {
    static_assert(NT == 2 || (NT == 4 && !SAMPLE), "the sampling epilogue covers one group per workgroup");
    constexpr int GPW = NT / 2;                                 // packed groups per workgroup
    // LDS row stride (elements): 144 measured 1-2% faster than 136 at 80 rows, and
    // 128 (no padding) 20-35% slower everywhere (bank conflicts of the fragment reads)
    constexpr int HSTR = kLmKB + 16;
    constexpr int HCH = 16 * MT * kLmKB / 8 / kLmThreads;     // hidden chunks per thread per K-block
    static_assert(HCH * kLmThreads * 8 == 16 * MT * kLmKB, "hidden staging must tile evenly");
    __shared__ __attribute__((aligned(16))) u16 hs[16 * MT * HSTR];
    __shared__ Best wbest[4][16 * MT];
    __shared__ uint4 s_sup[SAMPLE ? 16 * MT : 1];   // draft support inside this group, one bit per entry
    __shared__ float2 s_ms[SAMPLE ? 4 : 1][SAMPLE ? 16 * MT : 1];
    __shared__ __attribute__((aligned(16))) float zbuf[SAMPLE ? 32 * kZStride : 4];

    // Logical tile: with several row groups, hardware workgroup i runs on XCD i % 8;
    // give the row groups of one vocabulary group consecutive slots of one XCD so
    // that W is fetched from HBM once and re-read from that XCD's L2.
    int lid = blockIdx.x;
    if (n_rg > 1) {
        const int per_xcd = (int)((gridDim.x + 7) / 8);
        lid = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
        if (lid >= n_vt * n_rg) return;
    }
    const int vt = lid / n_rg, rg = lid % n_rg;
    const int r0 = rg * 16 * MT;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int l16 = lane % 16, lq = lane / 16;
    const int tile0 = (vt * 4 + wave) * kLmNT;       // first 16-row W tile of this wave (NT = 2)
    const int nkb = H / kLmKB;
    const int n_groups = (V + kLmVocabPerWg - 1) / kLmVocabPerWg;
    // vocabulary entry of this lane's column in tile nt
    auto vocab = [&](int nt) { return ((vt * GPW + nt / 2) * kLmTiles + wave * 2 + nt % 2) * 16 + l16; };

    // this wave's fragments of group g (clamped: a workgroup's second group may not
    // exist when the group count is odd; its entries are >= V and never kept)
    auto group_base = [&](int g) {
        return wp + (((size_t)min(g, n_groups - 1) * nkb * kLmTiles + wave * 2) * kLmKS * 64 + lane) * 8;
    };
    const u16* wt[GPW];
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) wt[gi] = group_base(vt * GPW + gi);
    const size_t kb_stride = (size_t)kLmTiles * kLmKS * 512;   // elements per K-block of a group
    uint4 ring[kLmKS][NT], hnext[HCH];
    // Rows past R re-read row R - 1: a row's logits depend on its own hidden row
    // only, and those rows' results are never written.
    auto load_h = [&](int kb) {
#pragma unroll
        for (int it = 0; it < HCH; ++it) {
            const int cidx = it * kLmThreads + tid;
            const int row = cidx / (kLmKB / 8), ch = cidx % (kLmKB / 8);
            hnext[it] = ld16(hidden + (size_t)min(r0 + row, R - 1) * H + kb * kLmKB + ch * 8);
        }
    };
    auto load_slot = [&](int kb, int s, uint4* dst) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const u16* p = wt[nt / 2] + (size_t)kb * kb_stride + s * 512 + (nt % 2) * kLmKS * 512;
            dst[nt] = SHARED ? ld16(p) : ld16_stream(p);
        }
    };

    f32x4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One K-block: publish its hidden rows in LDS, request the next block's hidden
    // rows, then per k-step: MFMAs, and re-request that ring slot for the next block.
    auto block = [&](int kb, auto more_c) {
        constexpr bool more = decltype(more_c)::value;
        __syncthreads();
#pragma unroll
        for (int it = 0; it < HCH; ++it) {
            const int cidx = it * kLmThreads + tid;
            const int row = cidx / (kLmKB / 8), ch = cidx % (kLmKB / 8);
            st16(hs + row * HSTR + ch * 8, hnext[it]);
        }
        if constexpr (more) load_h(kb + 1);
        __syncthreads();
#pragma unroll
        for (int s = 0; s < kLmKS; ++s) {
            bf16x8 a[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) a[mt] = as_bf16x8(ld16(hs + (mt * 16 + l16) * HSTR + s * 32 + lq * 8));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[mt][nt] = mfma16x16x32(a[mt], as_bf16x8(ring[s][nt]), acc[mt][nt]);
            if constexpr (more) {
                // With 14 or more MFMAs per k-step the waves' MFMA issue delays the
                // next K-block's loads; issuing them at raised priority measured
                // 4-7% faster there (112 rows: 222 -> 214 us, 256: 389 -> 361,
                // 1024: 1297 -> 1217) and 1-5 us slower below (16-96 rows).
                if constexpr (MT * NT >= 14) __builtin_amdgcn_s_setprio(3);
                load_slot(kb + 1, s, ring[s]);
                if constexpr (MT * NT >= 14) __builtin_amdgcn_s_setprio(0);
            }
        }
    };
    // sampling: thread t < 16 MT gathers row t's support tokens that fall in this
    // group (its loads are issued before the W stream starts)
    int qt[8];
    if constexpr (SAMPLE) {
        if (tid < 16 * MT) {
            const int r = min(r0 + tid, R - 1);
#pragma unroll
            for (int e = 0; e < 8; ++e) qt[e] = e < sa.NQ ? sa.q_tok[(size_t)r * sa.NQ + e] : -1;
        }
    }
    load_h(0);
#pragma unroll
    for (int s = 0; s < kLmKS; ++s) load_slot(0, s, ring[s]);
    if constexpr (SAMPLE) {
        if (tid < 16 * MT) {
            uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int loc = qt[e] - vt * kLmVocabPerWg;
                if (qt[e] >= 0 && loc >= 0 && loc < kLmVocabPerWg) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)   // constant indices (see the noise transpose)
                        if ((loc >> 5) == q) w[q] |= 1u << (loc & 31);
                }
            }
            s_sup[tid] = make_uint4(w[0], w[1], w[2], w[3]);   // read after the K loop's barriers
        }
    }
    for (int kb = 0; kb + 1 < nkb; ++kb) block(kb, std::true_type{});
    block(nkb - 1, std::false_type{});

    if constexpr (SAMPLE) {
        sample_epilogue<MT>(acc, sa, r0, R, V, vt, n_vt, tile0, tid, wave, lane, s_sup, s_ms, wbest, keys);
        if (sa.z_out) write_z<MT>(acc, sa, r0, R, V, vt, tid, wave, lane, zbuf);
        return;
    }

    // epilogue: C[row = 16 mt + 4 lq + i][vocab = vocab(nt)]
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int v = vocab(nt);
                const float x = acc[mt][nt][i];
                if (v < V && better(x, v, bv, bi)) {
                    bv = x;
                    bi = v;
                }
            }
#pragma unroll
            for (int d = 1; d < 16; d <<= 1) {
                const float ov = __shfl_xor(bv, d);
                const int oi = __shfl_xor(bi, d);
                if (better(ov, oi, bv, bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
            if (l16 == 0) wbest[wave][mt * 16 + lq * 4 + i] = Best{bv, bi};
        }
    }
    __syncthreads();
    if (tid < 16 * MT && r0 + tid < R) {
        Best b = wbest[0][tid];
#pragma unroll
        for (int wv = 1; wv < 4; ++wv) {
            const Best o = wbest[wv][tid];
            if (better(o.v, o.i, b.v, b.i)) b = o;
        }
        if (key_rows) {
            // few rows: this workgroup's row of keys, merged by lm_head_rows_finalize_kernel
            key_rows[(size_t)vt * key_rows_stride(R) + r0 + tid] = pack_best(b);
        } else {
            // the returned value is consumed, so the wave waits until the update is performed
            const unsigned long long prev = atomicMax(keys + r0 + tid, pack_best(b));
            asm volatile("" : : "v"(prev));
        }
    }
    if (key_rows) return;
    // The last workgroup to finish turns the keys into the outputs and leaves the
    // workspace zero for the next call. Keys and ticket are only touched by atomics,
    // which are ordered where they are performed, so no cache flush is needed: every
    // workgroup's key updates are performed before its ticket, and the last
    // workgroup reads the keys after its own ticket.
    __shared__ unsigned int s_last;
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(ticket, 1u) == (unsigned int)(n_vt * n_rg - 1);
    __syncthreads();
    if (!s_last) return;
    for (int r = tid; r < R; r += kLmThreads) {
        const unsigned long long key = atomicExch(keys + r, 0ull);
        argmax[r] = (int32_t)~(uint32_t)key;
        if (maxval) maxval[r] = unpack_value(key);
    }
    if (tid == 0) atomicExch(ticket, 0u);
}

// Few rows (at most kLmKeyRowsMaxR): each workgroup stores its per-row keys as one
// row of a [workgroups][key_rows_stride(R)] array with plain stores, and
// lm_head_rows_finalize_kernel merges them. At these row counts the workgroups end
// close together, and the atomic maxima and ticket of the general path then queue at
// the end of the kernel. Measured at H = 4096, V = 151936 (outputs identical): 1 row
// 203 -> 183 us, 16: 194 -> 183, 32: 195 -> 185, 48: 196 -> 188, 64: 197 -> 195. At 72
// and 80 rows the tile kernel is 6 us faster this way (193 vs 199 us at 80) but the
// finalize launch costs as much, and at 96 rows 1 us more; the general path is kept
// there. The maximum of the keys is the same whichever path takes it.
constexpr int kLmKeyRowsMaxR = 64;
static_assert(kLmKeyRowsMaxR <= 6 * 16 && kArgmaxAcceptMaxRows <= 6 * 16,
              "the dispatch passes the key rows to the tile kernels of up to 6 row tiles");

// Finalize: 8 rows per workgroup of up to 1024 threads (4 per vocabulary workgroup,
// rounded up to whole waves). Thread t reads the keys of rows 2(t%4), 2(t%4)+1 of the
// block (one 16-byte load: the stride is a multiple of 8 keys) from every
// (threads/4)-th vocabulary workgroup, starting at t/4, all of them requested before
// any is used (one round trip up to 2048 vocabulary workgroups); lanes 4 apart then
// merge, then the waves through LDS. Every key read is written back as zero,
// so the workspace is zero after every call, whichever path the call took. (At
// V = 151936: 4.9-5.4 us for 16-64 rows, against 5.8-6.4 for 256 threads reading one
// key at a time in dependent batches.)
constexpr int kLmFinThreads = 1024;
constexpr int kLmFinBatch = 8;

__global__ __launch_bounds__(kLmFinThreads) void lm_head_rows_finalize_kernel(unsigned long long* __restrict__ key_rows,
                                                                              int n_wg, int R, int32_t* __restrict__ argmax,
                                                                              float* __restrict__ maxval) {
    const int kStep = (int)blockDim.x / 4;
    const int q = threadIdx.x % 4, j0 = threadIdx.x / 4;
    const int r0 = blockIdx.x * 8 + 2 * q;
    const size_t stride = (size_t)key_rows_stride(R);
    uint4* base = reinterpret_cast<uint4*>(key_rows + r0);
    unsigned long long b0 = 0ull, b1 = 0ull;
    for (int i0 = j0; i0 < n_wg; i0 += kLmFinBatch * kStep) {
        uint4 k[kLmFinBatch];
#pragma unroll
        for (int u = 0; u < kLmFinBatch; ++u) {
            const int i = i0 + u * kStep;
            k[u] = i < n_wg ? base[(size_t)i * stride / 2] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kLmFinBatch; ++u) {
            const int i = i0 + u * kStep;
            const unsigned long long x0 = ((unsigned long long)k[u].y << 32) | k[u].x;
            const unsigned long long x1 = ((unsigned long long)k[u].w << 32) | k[u].z;
            b0 = x0 > b0 ? x0 : b0;
            b1 = x1 > b1 ? x1 : b1;
            if (i < n_wg) base[(size_t)i * stride / 2] = make_uint4(0, 0, 0, 0);
        }
    }
    // lanes 4 apart hold the same two rows
#pragma unroll
    for (int d = 4; d < kWave; d <<= 1) {
        const unsigned long long o0 = __shfl_xor(b0, d), o1 = __shfl_xor(b1, d);
        b0 = o0 > b0 ? o0 : b0;
        b1 = o1 > b1 ? o1 : b1;
    }
    const int NW = (int)blockDim.x / kWave;
    __shared__ unsigned long long s_b[kLmFinThreads / kWave][8];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    if (lane < 4) {
        s_b[wave][2 * lane] = b0;
        s_b[wave][2 * lane + 1] = b1;
    }
    __syncthreads();
    const int r = blockIdx.x * 8 + threadIdx.x;
    if (threadIdx.x < 8 && r < R) {
        unsigned long long best = s_b[0][threadIdx.x];
        for (int w = 1; w < NW; ++w) best = s_b[w][threadIdx.x] > best ? s_b[w][threadIdx.x] : best;
        argmax[r] = (int32_t)~(uint32_t)best;
        if (maxval) maxval[r] = unpack_value(best);
    }
}

static int n_vtiles(int V) { return (V + kLmVocabPerWg - 1) / kLmVocabPerWg; }

// Four vocabulary tiles per wave (two packed groups per workgroup) for the greedy
// pass when the rows need more than one row group of kLmMaxMT tiles (R > 128):
// measured 5-10% faster there (R = 160: 280 vs 296 us, 256: 388 vs 420, 1024: 1287
// vs 1437 at H = 4096, V = 151936) and slower at one row group (80: 221 vs 201).
// Such row groups hold at most 7 tiles (8 tiles of 4 vocabulary tiles do not fit
// the register file). A row's logits are the same MFMA chain either way, so the
// results do not depend on the choice.
constexpr int kLmMaxMTWide = 7;
static bool lm_wide(int mtiles) { return mtiles > kLmMaxMT; }

// n_vt: workgroups along the vocabulary (packed groups / (NT / 2), rounded up).
// Returns false if no kernel variant fits (MT, n_rg); nothing is launched then.
template <int MT, int NT, bool SAMPLE = false>
static bool launch_tiles(const u16* hidden, const u16* w, int R, int H, int V, int n_vt, int n_rg,
                         unsigned long long* keys, unsigned int* ticket, int32_t* argmax, float* maxval,
                         hipStream_t st, const SampleArgs& sa = SampleArgs{},
                         unsigned long long* key_rows = nullptr) {
    if (n_rg == 1) {
        hipLaunchKernelGGL((lm_head_tile_kernel<MT, NT, false, SAMPLE>), dim3(n_vt), dim3(kLmThreads), 0, st, hidden,
                           w, R, H, V, n_vt, n_rg, keys, ticket, argmax, maxval, sa, key_rows);
        return true;
    }
    // several row groups have >= 5 tiles each (caps of 8), >= 4 (cap of 7)
    if constexpr (MT >= 4) {
        const int grid = (n_vt * n_rg + 7) / 8 * 8;
        hipLaunchKernelGGL((lm_head_tile_kernel<MT, NT, true, SAMPLE>), dim3(grid), dim3(kLmThreads), 0, st, hidden,
                           w, R, H, V, n_vt, n_rg, keys, ticket, argmax, maxval, sa, key_rows);
        return true;
    }
    return false;
}

// One workgroup per row: the row's softmax statistics from the groups' partials (a
// fixed reduction order), then the two draws. Candidates are the best entry outside
// the draft support (from the tile kernel's key, z + G) and each distinct support
// token (z + G recomputed here):
//   draw from p:                    argmax z_v + G_v
//   draw from norm(max(p - q, 0)):  argmax log(max(p_v - q_v, 0)) + G_v, which is
//                                   z_v - lse + G_v outside the support
// with ties to the smaller index. The row's key is reset to zero.
__global__ __launch_bounds__(256) void sample_finalize_kernel(
    const float2* __restrict__ part, const float4* __restrict__ part4, int n_vt, int V,
    unsigned long long* __restrict__ keys,
    const int32_t* __restrict__ q_tok, const float* __restrict__ q_prob, int NQ, const int32_t* __restrict__ row_ctr,
    uint32_t key0, uint32_t key1, float* __restrict__ lse_out, float* __restrict__ z_supp,
    int32_t* __restrict__ sample_p, int32_t* __restrict__ sample_res) {
    __shared__ float2 s_w[4];
    __shared__ unsigned long long s_k[4];
    const int r = blockIdx.x, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    float m = -INFINITY, sm = 0.f;
    unsigned long long key = 0ull;
    if (part4) {
        for (int c = tid; c < n_vt; c += 256) {
            const float4 pm = part4[(size_t)r * n_vt + c];
            ms_merge(m, sm, pm.x, pm.y);
            const unsigned long long k = (unsigned long long)__float_as_uint(pm.w) << 32 | __float_as_uint(pm.z);
            key = k > key ? k : key;
        }
    } else {
        for (int c = tid; c < n_vt; c += 256) {
            const float2 pm = part[(size_t)r * n_vt + c];
            ms_merge(m, sm, pm.x, pm.y);
        }
    }
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) {
        const float om = __shfl_xor(m, d), os = __shfl_xor(sm, d);
        ms_merge(m, sm, om, os);
        const unsigned long long ok = __shfl_xor(key, d);
        key = ok > key ? ok : key;
    }
    if (lane == 0) {
        s_w[wave] = make_float2(m, sm);
        s_k[wave] = key;
    }
    __syncthreads();
    if (tid != 0) return;
    float M = s_w[0].x, S = s_w[0].y;
#pragma unroll
    for (int w = 1; w < 4; ++w) {
        ms_merge(M, S, s_w[w].x, s_w[w].y);
        key = s_k[w] > key ? s_k[w] : key;
    }
    key = s_k[0] > key ? s_k[0] : key;
    if (!part4) key = atomicExch(keys + r, 0ull);   // the atomic maxima; left zero
    const float lse = M + __logf(S);
    lse_out[r] = lse;
    Best bp{-INFINITY, 0x7fffffff}, br{-INFINITY, 0x7fffffff};
    if (key != 0ull) {
        const float zg = unpack_value(key);
        const int idx = (int)~(uint32_t)key;
        bp = Best{zg, idx};
        br = Best{zg - lse, idx};
    }
    const uint32_t ca = (uint32_t)row_ctr[2 * (size_t)r], cb = (uint32_t)row_ctr[2 * (size_t)r + 1];
    for (int e = 0; e < NQ; ++e) {
        const int t = q_tok[(size_t)r * NQ + e];
        if (t < 0 || t >= V) {
            z_supp[(size_t)r * NQ + e] = __int_as_float(0x7fc00000);   // NaN: unused entry
            continue;
        }
        bool dup = false;
        float q = 0.f;
        for (int e2 = 0; e2 < NQ; ++e2) {
            if (q_tok[(size_t)r * NQ + e2] != t) continue;
            if (e2 < e) dup = true;
            q += q_prob[(size_t)r * NQ + e2];
        }
        if (dup) continue;
        const float z = z_supp[(size_t)r * NQ + e];
        const float g = row_gumbel((uint32_t)t, ca, cb, key0, key1);
        if (better(z + g, t, bp.v, bp.i)) bp = Best{z + g, t};
        const float rv = __expf(z - lse) - q;
        if (rv > 0.f && better(__logf(rv) + g, t, br.v, br.i)) br = Best{__logf(rv) + g, t};
    }
    sample_p[r] = bp.i;
    sample_res[r] = br.i != 0x7fffffff ? br.i : bp.i;
}

}  // namespace sv

extern "C" {

size_t spec_lm_head_packed_bytes(int32_t V, int32_t H) {
    if (V < 1 || H < 1) return 0;
    return (size_t)((V + sv::kLmVocabPerWg - 1) / sv::kLmVocabPerWg) * sv::kLmVocabPerWg * (size_t)H * sizeof(spec_bf16);
}

int spec_lm_head_pack(const spec_bf16* w, int32_t V, int32_t H, spec_bf16* w_packed, void* stream) {
    using namespace sv;
    last_error().clear();
    if (V < 1 || V == 0x7fffffff) return fail(SPEC_EINVAL, "spec_lm_head_pack: V=%d", V);
    if (H < kLmHAlign || H % kLmHAlign) return fail(SPEC_EINVAL, "spec_lm_head_pack: H=%d not a positive multiple of %d", H, kLmHAlign);
    if (!w || !w_packed) return fail(SPEC_EINVAL, "spec_lm_head_pack: null pointer");
    if (!aligned16(w) || !aligned16(w_packed)) return fail(SPEC_EINVAL, "spec_lm_head_pack: w and w_packed must be 16-byte aligned");
    hipLaunchKernelGGL(lm_head_pack_kernel, dim3(8192), dim3(256), 0, (hipStream_t)stream, w, V, H, w_packed);
    SV_LAUNCH_CHECK("spec_lm_head_pack");
    return SPEC_OK;
}

size_t spec_lm_head_sample_workspace_bytes(int32_t R, int32_t H, int32_t V) {
    (void)H;
    if (R < 1 || V < 1) return 0;
    // a header and one key per row, then per (row, vocabulary group) (max, sum of exp)
    // or, up to 64 rows, (max, sum of exp, best key)
    return 256 + ((size_t)R * sizeof(unsigned long long) + 15) / 16 * 16 +
           (size_t)R * sv::n_vtiles(V) * (R <= sv::kLmSampleRecordsMaxR ? sizeof(float4) : sizeof(float2));
}

}  // extern "C"

namespace sv {

static int lm_head_sample_impl(const char* name, const spec_bf16* hidden, const spec_bf16* w_packed, int32_t R,
                               int32_t H, int32_t V, float temperature, const int32_t* q_tok, const float* q_prob,
                               int32_t NQ, const int32_t* row_ctr, uint64_t seed, float* lse, float* z_supp,
                               int32_t* sample_p, int32_t* sample_res, float* z_out, void* workspace,
                               size_t workspace_bytes, void* stream) {
    using namespace sv;
    last_error().clear();
    if (R < 1) return fail(SPEC_EINVAL, "%s: R=%d < 1", name, R);
    if (H < kLmHAlign || H % kLmHAlign) return fail(SPEC_EINVAL, "%s: H=%d not a positive multiple of %d", name, H, kLmHAlign);
    if (V < 1 || V == 0x7fffffff) return fail(SPEC_EINVAL, "%s: V=%d", name, V);
    if (!(temperature > 0.f) || !(temperature < INFINITY)) return fail(SPEC_EINVAL, "%s: temperature must be finite and > 0", name);
    if (NQ < 0 || NQ > 8) return fail(SPEC_EINVAL, "%s: NQ=%d outside 0..8", name, NQ);
    if (!hidden || !w_packed || !row_ctr || !lse || !sample_p || !sample_res || (NQ > 0 && (!q_tok || !q_prob || !z_supp)))
        return fail(SPEC_EINVAL, "%s: null required pointer", name);
    if (!aligned16(hidden) || !aligned16(w_packed)) return fail(SPEC_EINVAL, "%s: hidden and w_packed must be 16-byte aligned", name);
    const size_t need = spec_lm_head_sample_workspace_bytes(R, H, V);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return fail(SPEC_EWORKSPACE, "%s: workspace %zu bytes < %zu required (or null/misaligned)", name, workspace_bytes, need);
    const int n_vt = n_vtiles(V);
    unsigned long long* keys = reinterpret_cast<unsigned long long*>(static_cast<char*>(workspace) + 256);
    // the per-(row, group) records, 16-byte aligned after the per-row keys
    char* rec = static_cast<char*>(workspace) + 256 + ((size_t)R * sizeof(unsigned long long) + 15) / 16 * 16;
    const bool records = R <= kLmSampleRecordsMaxR;
    float2* part = records ? nullptr : reinterpret_cast<float2*>(rec);
    float4* part4 = records ? reinterpret_cast<float4*>(rec) : nullptr;
    const int mtiles = (R + 15) / 16;
    const int n_rg = (mtiles + kLmMaxMT - 1) / kLmMaxMT;
    const int MT = (mtiles + n_rg - 1) / n_rg;
    if ((long long)n_vt * n_rg + 8 > 0x7fffffffLL) return fail(SPEC_ECAPACITY, "%s: grid too large", name);
    SampleArgs sa{q_tok, row_ctr, part, part4, z_supp, z_out, 1.f / temperature, NQ, (uint32_t)seed, (uint32_t)(seed >> 32)};
    hipStream_t st = (hipStream_t)stream;
    const spec_bf16* w = w_packed;
    bool ok = false;
    switch (MT) {
        case 1: ok = launch_tiles<1, 2, true>(hidden, w, R, H, V, n_vt, n_rg, keys, nullptr, nullptr, nullptr, st, sa); break;
        case 2: ok = launch_tiles<2, 2, true>(hidden, w, R, H, V, n_vt, n_rg, keys, nullptr, nullptr, nullptr, st, sa); break;
        case 3: ok = launch_tiles<3, 2, true>(hidden, w, R, H, V, n_vt, n_rg, keys, nullptr, nullptr, nullptr, st, sa); break;
        case 4: ok = launch_tiles<4, 2, true>(hidden, w, R, H, V, n_vt, n_rg, keys, nullptr, nullptr, nullptr, st, sa); break;
        case 5: ok = launch_tiles<5, 2, true>(hidden, w, R, H, V, n_vt, n_rg, keys, nullptr, nullptr, nullptr, st, sa); break;
        case 6: ok = launch_tiles<6, 2, true>(hidden, w, R, H, V, n_vt, n_rg, keys, nullptr, nullptr, nullptr, st, sa); break;
        case 7: ok = launch_tiles<7, 2, true>(hidden, w, R, H, V, n_vt, n_rg, keys, nullptr, nullptr, nullptr, st, sa); break;
        default: ok = launch_tiles<8, 2, true>(hidden, w, R, H, V, n_vt, n_rg, keys, nullptr, nullptr, nullptr, st, sa); break;
    }
    if (!ok) return fail(SPEC_EINVAL, "%s: no kernel variant for R=%d", name, R);
    SV_LAUNCH_CHECK(name);
    hipLaunchKernelGGL(sample_finalize_kernel, dim3(R), dim3(256), 0, st, part, part4, n_vt, V, keys, q_tok, q_prob, NQ,
                       row_ctr,
                       sa.key0, sa.key1, lse, z_supp, sample_p, sample_res);
    SV_LAUNCH_CHECK(name);
    return SPEC_OK;
}

}  // namespace sv

namespace sv {

// The greedy lm_head call: argument checks, then the tile kernel for the row count.
// Up to rows_max rows the key-rows path is taken when the workspace holds it (the
// no-allocation entry point passes 0). With rows_out the call stops after the tile
// kernel and hands over the key rows (null after the general path), which the
// caller's own kernel then merges; otherwise the finalize kernel merges them.
static int lm_head_argmax_run(const char* name, const spec_bf16* hidden, const spec_bf16* w_packed, int32_t R,
                              int32_t H, int32_t V, int32_t* argmax, float* maxval, void* workspace,
                              size_t workspace_bytes, int rows_max, hipStream_t st,
                              unsigned long long** rows_out = nullptr) {
    if (R < 1) return fail(SPEC_EINVAL, "%s: R=%d < 1", name, R);
    if (H < kLmHAlign || H % kLmHAlign) return fail(SPEC_EINVAL, "%s: H=%d not a positive multiple of %d", name, H, kLmHAlign);
    if (V < 1 || V == 0x7fffffff) return fail(SPEC_EINVAL, "%s: V=%d", name, V);
    if (!hidden || !w_packed || !argmax) return fail(SPEC_EINVAL, "%s: null required pointer", name);
    if (!aligned16(hidden) || !aligned16(w_packed)) return fail(SPEC_EINVAL, "%s: hidden and w_packed must be 16-byte aligned", name);
    const spec_bf16* w = w_packed;
    const int n_vt = n_vtiles(V);
    const size_t keys_bytes = 256 + (size_t)R * sizeof(unsigned long long);
    if (!workspace || workspace_bytes < keys_bytes || !aligned16(workspace))
        return fail(SPEC_EWORKSPACE, "%s: workspace %zu bytes < %zu required (or null/misaligned)", name, workspace_bytes,
                    keys_bytes);
    // the key-rows path when the workspace holds its key rows too (a workspace sized
    // for more rows may not: then the general path, with the same result); they start
    // 64-byte aligned after the keys (the finalize reads them 16 bytes at a time)
    const size_t rows_at = 256 + (size_t)key_rows_stride(R) * sizeof(unsigned long long);
    const bool rows_path = R <= rows_max &&
                           workspace_bytes >= rows_at + (size_t)n_vt * key_rows_stride(R) * sizeof(unsigned long long);
    unsigned int* ticket = static_cast<unsigned int*>(workspace);
    unsigned long long* keys = reinterpret_cast<unsigned long long*>(static_cast<char*>(workspace) + 256);
    unsigned long long* key_rows =
        rows_path ? reinterpret_cast<unsigned long long*>(static_cast<char*>(workspace) + rows_at) : nullptr;
    // row groups of at most kLmMaxMT 16-row tiles, balanced (160 rows: 2 x 80)
    const int mtiles = (R + 15) / 16;
    const int n_rg = (mtiles + kLmMaxMT - 1) / kLmMaxMT;
    const int MT = (mtiles + n_rg - 1) / n_rg;
    if ((long long)n_vt * n_rg + 8 > 0x7fffffffLL) return fail(SPEC_ECAPACITY, "%s: grid too large", name);
    bool ok = false;
    const SampleArgs no_sa{};
    if (lm_wide(mtiles)) {
        const int n_wg = (n_vt + 1) / 2;
        const int n_rg_w = (mtiles + kLmMaxMTWide - 1) / kLmMaxMTWide;
        const int MT_w = (mtiles + n_rg_w - 1) / n_rg_w;
        switch (MT_w) {
            case 1: ok = launch_tiles<1, 4>(hidden, w, R, H, V, n_wg, n_rg_w, keys, ticket, argmax, maxval, st); break;
            case 2: ok = launch_tiles<2, 4>(hidden, w, R, H, V, n_wg, n_rg_w, keys, ticket, argmax, maxval, st); break;
            case 3: ok = launch_tiles<3, 4>(hidden, w, R, H, V, n_wg, n_rg_w, keys, ticket, argmax, maxval, st); break;
            case 4: ok = launch_tiles<4, 4>(hidden, w, R, H, V, n_wg, n_rg_w, keys, ticket, argmax, maxval, st); break;
            case 5: ok = launch_tiles<5, 4>(hidden, w, R, H, V, n_wg, n_rg_w, keys, ticket, argmax, maxval, st); break;
            case 6: ok = launch_tiles<6, 4>(hidden, w, R, H, V, n_wg, n_rg_w, keys, ticket, argmax, maxval, st); break;
            default: ok = launch_tiles<7, 4>(hidden, w, R, H, V, n_wg, n_rg_w, keys, ticket, argmax, maxval, st); break;
        }
    } else {
        switch (MT) {
            case 1: ok = launch_tiles<1, 2>(hidden, w, R, H, V, n_vt, n_rg, keys, ticket, argmax, maxval, st, no_sa, key_rows); break;
            case 2: ok = launch_tiles<2, 2>(hidden, w, R, H, V, n_vt, n_rg, keys, ticket, argmax, maxval, st, no_sa, key_rows); break;
            case 3: ok = launch_tiles<3, 2>(hidden, w, R, H, V, n_vt, n_rg, keys, ticket, argmax, maxval, st, no_sa, key_rows); break;
            case 4: ok = launch_tiles<4, 2>(hidden, w, R, H, V, n_vt, n_rg, keys, ticket, argmax, maxval, st, no_sa, key_rows); break;
            case 5: ok = launch_tiles<5, 2>(hidden, w, R, H, V, n_vt, n_rg, keys, ticket, argmax, maxval, st, no_sa, key_rows); break;
            case 6: ok = launch_tiles<6, 2>(hidden, w, R, H, V, n_vt, n_rg, keys, ticket, argmax, maxval, st, no_sa, key_rows); break;
            case 7: ok = launch_tiles<7, 2>(hidden, w, R, H, V, n_vt, n_rg, keys, ticket, argmax, maxval, st); break;
            default: ok = launch_tiles<8, 2>(hidden, w, R, H, V, n_vt, n_rg, keys, ticket, argmax, maxval, st); break;
        }
    }
    if (!ok) return fail(SPEC_EINVAL, "%s: no kernel variant for R=%d", name, R);
    if (rows_out)
        *rows_out = key_rows;
    else if (rows_path)
        hipLaunchKernelGGL(lm_head_rows_finalize_kernel, dim3((R + 7) / 8),
                           dim3(std::min(kLmFinThreads, (4 * n_vt + kWave - 1) / kWave * kWave)), 0, st, key_rows, n_vt, R, argmax,
                           maxval);
    SV_LAUNCH_CHECK(name);
    return SPEC_OK;
}

}  // namespace sv

extern "C" {

int spec_lm_head_sample(const spec_bf16* hidden, const spec_bf16* w_packed, int32_t R, int32_t H, int32_t V,
                        float temperature, const int32_t* q_tok, const float* q_prob, int32_t NQ,
                        const int32_t* row_ctr, uint64_t seed, float* lse, float* z_supp, int32_t* sample_p,
                        int32_t* sample_res, void* workspace, size_t workspace_bytes, void* stream) {
    return sv::lm_head_sample_impl("spec_lm_head_sample", hidden, w_packed, R, H, V, temperature, q_tok, q_prob, NQ, row_ctr,
                                   seed, lse, z_supp, sample_p, sample_res, nullptr, workspace, workspace_bytes, stream);
}

int spec_lm_head_sample_dense(const spec_bf16* hidden, const spec_bf16* w_packed, int32_t R, int32_t H, int32_t V,
                              float temperature, const int32_t* row_ctr, uint64_t seed, float* lse, int32_t* sample_p,
                              float* z, void* workspace, size_t workspace_bytes, void* stream) {
    if (!z) {
        sv::last_error().clear();
        return sv::fail(SPEC_EINVAL, "spec_lm_head_sample_dense: null required pointer");
    }
    // no support list: every entry is outside it, so the second draw is the first
    return sv::lm_head_sample_impl("spec_lm_head_sample_dense", hidden, w_packed, R, H, V, temperature, nullptr, nullptr, 0,
                                   row_ctr, seed, lse, nullptr, sample_p, sample_p, z, workspace, workspace_bytes, stream);
}

size_t spec_lm_head_argmax_workspace_bytes(int32_t R, int32_t H, int32_t V) {
    (void)H;
    if (R < 1 || V < 1) return 0;
    // ticket (padded), one key per row; at few rows (the key-rows paths of this call
    // and of spec_lm_head_argmax_accept) the keys padded to key_rows_stride(R) and
    // then the [workgroups][key_rows_stride(R)] key rows
    size_t n = 256 + (size_t)R * sizeof(unsigned long long);
    if (R <= std::max(sv::kLmKeyRowsMaxR, sv::kArgmaxAcceptMaxRows))
        n = 256 + (size_t)(sv::n_vtiles(V) + 1) * sv::key_rows_stride(R) * sizeof(unsigned long long);
    return n;
}

int spec_lm_head_argmax(const spec_bf16* hidden, const spec_bf16* w_packed, int32_t R, int32_t H, int32_t V,
                        int32_t* argmax, float* maxval, void* workspace, size_t workspace_bytes,
                        void* stream) {
    sv::last_error().clear();
    return sv::lm_head_argmax_run("spec_lm_head_argmax", hidden, w_packed, R, H, V, argmax, maxval, workspace,
                                  workspace_bytes, sv::kLmKeyRowsMaxR, (hipStream_t)stream);
}

int spec_lm_head_argmax_accept(const spec_bf16* hidden, const spec_bf16* w_packed, int32_t R, int32_t H, int32_t V,
                               int32_t* argmax, float* maxval, const int32_t* drafts, int32_t kmax, const int32_t* k,
                               const int32_t* d2t, int32_t n_draft_vocab, int32_t B, const int32_t* pos_in,
                               int32_t* pos_out, int32_t* accept_len, int32_t* n_emit, int32_t* emit, int32_t* next_tok,
                               int32_t* seq_status, void* workspace, size_t workspace_bytes, void* stream) {
    using namespace sv;
    last_error().clear();
    const char* name = "spec_lm_head_argmax_accept";
    // the acceptance's checks first, so that a refused call launches nothing
    if (B < 1 || B > kAcceptMaxB) return fail(SPEC_EINVAL, "%s: B=%d outside 1..%d", name, B, kAcceptMaxB);
    if (kmax < 0 || kmax > 1024) return fail(SPEC_EINVAL, "%s: kmax=%d outside 0..1024", name, kmax);
    if (d2t && n_draft_vocab < 1) return fail(SPEC_EINVAL, "%s: d2t given with n_draft_vocab=%d", name, n_draft_vocab);
    if (!k || !pos_in || !pos_out || !accept_len || !n_emit || !emit || !next_tok || !seq_status || (kmax > 0 && !drafts))
        return fail(SPEC_EINVAL, "%s: null required pointer", name);
    hipStream_t st = (hipStream_t)stream;
    unsigned long long* key_rows = nullptr;
    const int rc = lm_head_argmax_run(name, hidden, w_packed, R, H, V, argmax, maxval, workspace, workspace_bytes,
                                      kArgmaxAcceptMaxRows, st, &key_rows);
    if (rc != SPEC_OK) return rc;
    if (key_rows) {
        launch_argmax_accept(key_rows, n_vtiles(V), key_rows_stride(R), R, argmax, maxval, drafts, kmax, k, d2t,
                             n_draft_vocab, V, B, pos_in, pos_out, accept_len, n_emit, emit, next_tok, seq_status, st);
        SV_LAUNCH_CHECK(name);
        return SPEC_OK;
    }
    // the general path: the argmax is complete, the acceptance runs on its own
    return spec_greedy_accept(argmax, drafts, kmax, k, d2t, n_draft_vocab, V, B, R, pos_in, pos_out, accept_len,
                              n_emit, emit, next_tok, seq_status, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// spec_lm_head_argmax_noalloc: the same lm_head with its ticket and keys in a
// library-owned device array instead of a caller workspace.
namespace sv {

constexpr size_t kScratchBytes = SPEC_NOALLOC_SCRATCH_BYTES;
// One copy per GPU the library runs on, held until the process ends. In host code
// this name is only a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ __launch_bounds__(256) void scratch_clear_kernel(uint4* __restrict__ p, int n16) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n16) p[i] = make_uint4(0, 0, 0, 0);
}

constexpr int kMaxDevices = 64;

// The current device's copy of the scratch array (looked up once per device).
static int scratch_for_current_device(void** out) {
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SPEC_EHIP, "spec_lm_head_argmax_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(SPEC_ECAPACITY, "spec_lm_head_argmax_noalloc: device %d >= %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(SPEC_EHIP, "spec_lm_head_argmax_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
        addr[dev] = p;
    }
    *out = addr[dev];
    return SPEC_OK;
}

}  // namespace sv

extern "C" int spec_lm_head_argmax_noalloc(const spec_bf16* hidden, const spec_bf16* w_packed, int32_t R, int32_t H,
                                           int32_t V, int32_t* argmax, float* maxval, void* stream) {
    using namespace sv;
    last_error().clear();
    if (R < 1) return fail(SPEC_EINVAL, "spec_lm_head_argmax_noalloc: R=%d < 1", R);
    if (R > SPEC_NOALLOC_MAX_ROWS)
        return fail(SPEC_ECAPACITY, "spec_lm_head_argmax_noalloc: R=%d exceeds the %d rows its scratch array holds",
                    R, SPEC_NOALLOC_MAX_ROWS);
    // the checks of spec_lm_head_argmax, made before anything is launched
    if (H < kLmHAlign || H % kLmHAlign)
        return fail(SPEC_EINVAL, "spec_lm_head_argmax_noalloc: H=%d not a positive multiple of %d", H, kLmHAlign);
    if (V < 1 || V == 0x7fffffff) return fail(SPEC_EINVAL, "spec_lm_head_argmax_noalloc: V=%d", V);
    if (!hidden || !w_packed || !argmax) return fail(SPEC_EINVAL, "spec_lm_head_argmax_noalloc: null required pointer");
    if (!aligned16(hidden) || !aligned16(w_packed))
        return fail(SPEC_EINVAL, "spec_lm_head_argmax_noalloc: hidden and w_packed must be 16-byte aligned");
    // the ticket and one key per row (the key-rows path of few rows is not used here)
    const size_t need = 256 + (size_t)R * sizeof(unsigned long long);
    if (need > kScratchBytes) return fail(SPEC_EINVAL, "spec_lm_head_argmax_noalloc: R=%d V=%d", R, V);
    void* ws = nullptr;
    const int rc = scratch_for_current_device(&ws);
    if (rc != SPEC_OK) return rc;
    // the ticket and this call's keys start at zero (a fill kernel, so that the call
    // can be captured into a graph)
    const int n16 = (int)((need + 15) / 16);
    hipLaunchKernelGGL(scratch_clear_kernel, dim3((n16 + 255) / 256), dim3(256), 0, (hipStream_t)stream,
                       static_cast<uint4*>(ws), n16);
    SV_LAUNCH_CHECK("spec_lm_head_argmax_noalloc");
    return lm_head_argmax_run("spec_lm_head_argmax_noalloc", hidden, w_packed, R, H, V, argmax, maxval, ws, need,
                              0, (hipStream_t)stream);
}
