// spec_verify_attn: KV append in place + paged causal split-KV verify attention.
//
// Pool format: one 16-token x D block per (page, kv head), stored as MFMA operand
// fragments so that every wave instruction reads contiguous memory:
//   K block: token t, channel d at (d/32)*512 + ((d%32)/8)*128 + t*8 + d%8, i.e. for
//            k-step ds the 64 lanes' A fragments (lane = 16*(d%32/8) + t) are 1 KB;
//   V block: token t, channel d at (d/16)*256 + (t/4)*64 + (d%16)*4 + t%4, i.e. for
//            output tile dt each lane's 4 tokens of one channel are 8 contiguous bytes.
//
// Launches on the caller's stream (two; the row metadata and the append have no
// launch or round trips of their own):
//   1. attn_split_kernel: each workgroup forms the row packing and checks its
//      positions, the parent list (tree rows) and its own page ids with its first
//      metadata loads; a tile that reaches the new rows takes them from k_new/v_new;
//      one workgroup per sequence writes the status and row records, and one per (kv
//      head, split) appends the rows that fall in its split to their pool slots
//      (span-02 spec.rs: KV appended in place at pos..pos+k), both after checking the
//      whole page list, so a flagged sequence writes nothing. Its main work: one
//      workgroup per (sequence, kv head, split of
//      kv_split_tokens positions, group of 64 query rows), kv head fastest in the
//      launch order so that the Hkv blocks of a page (adjacent in the pool) are
//      fetched at about the same time. It stages 64-token tiles
//      (4 K blocks + 4 V blocks, each a contiguous 16*D*2-byte copy) in LDS and
//      gives each wave a 16-row query tile; per 32-token step a wave computes
//      S^T = K Q^T and O^T += V^T P^T with v_mfma_f32_16x16x32_bf16 (the G*T query
//      rows of a kv head are the MFMA columns, so each K/V byte read from HBM serves
//      all of them) and runs the online softmax in registers (row max/sum across
//      the 4 lanes holding a row). A key t is kept for row j only if t <= pos + j
//      (kv_hi = position, memra full_attn_verify's per-row bound). The split's page
//      ids are requested with the sequence metadata, once per wave, and taken with
//      readlane, so tiles never wait on a page-table load.
//   2. attn_combine_kernel one wave per (row, q head): merges the row's splits in
//      ascending order (log-sum-exp weights) and writes bf16.
//
// Tree rows (spec_verify_attn_tree; DSSD fast.py, _set_rows, _tree_cycle and
// _attention): the k+1 rows of a sequence are the nodes of a draft tree in creation
// order; node j still writes slot pos + j, but attends to slots 0..pos and then to the
// nodes of its own path in depth order, exactly as its one-row decode does once the
// accepted path is compacted into slots pos + 1.. (see "Tree rows as chain rows"
// below). Each split workgroup checks the parent list and turns it into one 128-bit
// ancestor mask per node (pointer jumping over the parent links in LDS while its first
// tile's loads are in flight: after r rounds a node's mask covers its 2^r nearest
// ancestors); a node's depth is the mask's population count minus one. A chain (parent
// j - 1) is its own compacted path, so it gives the bytes of spec_verify_attn.
//
// Row invariance: splits sit at absolute multiples of kv_split_tokens and steps at
// absolute multiples of 32; every row's operations run in the same order whichever
// wave, row group or launch serves it; reductions run in a fixed order; a row reads
// only splits that contain keys <= its position; steps past a row's position add
// exact zeros with rescale factor exactly 1. So a row's bytes are the same whatever
// other rows share the launch (kmax only sizes the grid).
#include "common.h"

namespace sv {

constexpr int kKT = 64;            // tokens per LDS tile of attn_split_kernel (4 pages)
constexpr int kAttnThreads = 256;  // 4 waves
constexpr int kMaxK = 127;         // drafts per sequence (the acceptance calls' limit; 128-bit tree masks)
constexpr int kRowsPerGroup = 64;  // query rows one attn_split_kernel workgroup handles
constexpr int kStreamSplit = 1024; // splits of at least this many tokens read the pool non-temporally
constexpr int kMaxSplit = 2048;    // largest kv_split_tokens
constexpr int kRemapMaxB = 256;    // batches up to this size dispatch the workgroups with work first
constexpr float kLog2e = 1.4426950408889634f;

// The tree call's LDS beyond the tile, in u16 units from its start: the K rows and the V
// rows of nodes 1..kmax (row u - 1: D channels), then per node its ancestor mask (16
// bytes) and ancestor link (4 bytes), then per wave one depth-ordered path (kmax + 1
// bytes, rounded to 16).
struct TreeLds {
    int nv, mask, anc, path, path_stride, end;
    __host__ __device__ TreeLds(int kmax, int D) {
        nv = kmax * D;
        mask = 2 * kmax * D;
        anc = mask + 8 * (kmax + 1);
        path_stride = (kmax + 1 + 15) / 16 * 16;
        path = anc + ((2 * (kmax + 1) + 7) / 8) * 8;
        end = path + 2 * path_stride;
    }
    __host__ __device__ size_t bytes() const { return (size_t)end * 2; }
};

// address-space pointer types of global_load_lds (global source, LDS destination)
typedef const __attribute__((address_space(1))) void* global_cptr;
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) uint8_t* lds_u8;
typedef __attribute__((address_space(3))) const u32x4* lds_cu4;
__device__ __forceinline__ uint4 lds_ld16(lds_cu4 p) {
    const u32x4 v = *p;
    return make_uint4(v[0], v[1], v[2], v[3]);
}

struct RowRec {
    int32_t p;      // position of the row
    int32_t nc;     // splits the merge kernel combines for it (0: nothing to merge)
};

// In-block offsets of token t, channel d (see the pool format above).
__device__ __forceinline__ int k_off(int t, int d) {
    return (d >> 5) * 512 + ((d & 31) >> 3) * 128 + t * 8 + (d & 7);
}
__device__ __forceinline__ int v_off(int t, int d) {
    return (d >> 4) * 256 + (t >> 2) * 64 + (d & 15) * 4 + (t & 3);
}

// ---------------------------------------------------------------------------
// Online softmax over one tile of NP pages (NP = 4: 64 tokens, NP = 2: 32 tokens)
// for one 16-row query tile.
//   src.k(p, ds): K A-fragment of the tile's page p, k-step ds
//   src.v(p, dt): V fragment (4 tokens of channel 16 dt + l16) of page p
//   lane l holds query row m = l % 16 of the tile; after the S^T MFMAs it holds
//   the scores of tokens t0 + 16 p + 4 (l / 16) + i, i = 0..3.
// The running maximum is raised only when a row's tile maximum exceeds it by more
// than kRescaleLog2 (a bound on exp2 of the lag); then that row's accumulators
// are scaled by exp2(old - new). The branch is taken by the whole wave, rows that
// do not need it are scaled by exactly 1.0, so a row's arithmetic depends on its
// own scores only.
constexpr float kRescaleLog2 = 8.f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D>
struct TileMath {
    static constexpr int NDS = D / 32;
    static constexpr int NDT = D / 16;

    // p_m: the row's position (it keeps the tile's keys t <= p_m; full: every row keeps
    // every key). A row with p_m < t0 gets only -inf scores, and such a tile leaves its
    // state exactly as it was: no raise, zero weights, zero sum, and zero P in P V.
    template <int NP, class Src>
    __device__ __forceinline__ static void run(const bf16x8 (&qf)[NDS], const Src& src, int t0, int p_m, bool full,
                                               int lq, float scale_log2, float& m_run, float& l_lane,
                                               f32x4 (&o)[NDT]) {
        static_assert(NP == 2 || NP == 4, "tiles of 32 or 64 tokens");
        constexpr int NS = 4 * NP;   // scores per lane
        float sc[NS];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) acc = mfma16x16x32(as_bf16x8(src.k(p, ds)), qf[ds], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[4 * p + i] = acc[i] * scale_log2;
        }
        if (!full) {   // some token of the tile lies past some row's position
#pragma unroll
            for (int jj = 0; jj < NS; ++jj) {
                const int o_t = 16 * (jj >> 2) + 4 * lq + (jj & 3);
                if (t0 + o_t > p_m) sc[jj] = -INFINITY;
            }
        }
        float tmax = sc[0];
#pragma unroll
        for (int jj = 1; jj < NS; ++jj) tmax = fmaxf(tmax, sc[jj]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const bool raise = tmax > m_run + kRescaleLog2;       // also true on a row's first tile
        if (__builtin_amdgcn_ballot_w64(raise)) {
            const float m_new = raise ? tmax : m_run;
            const float alpha = raise ? ((m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new)) : 1.f;
            l_lane *= alpha;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) o[dt] = o[dt] * alpha;
            m_run = m_new;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        float psum = 0.f;
#pragma unroll
        for (int jj = 0; jj < NS; ++jj) {
            sc[jj] = fast_exp2(sc[jj] - m_use);
            psum += sc[jj];
        }
        l_lane += psum;
        // 32-token halves hh: k-slot 8 lq + jj <-> token 32 hh + 16 (jj/4) + 4 lq + jj%4
#pragma unroll
        for (int hh = 0; hh < NP / 2; ++hh) {
            const bf16x8 pf = pack8(sc + 8 * hh);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const uint2 a = src.v(2 * hh, dt), b = src.v(2 * hh + 1, dt);
                o[dt] = mfma16x16x32(as_bf16x8(make_uint4(a.x, a.y, b.x, b.y)), pf, o[dt]);
            }
        }
    }
};


// Fragments of a 64-token tile read from LDS (4 K blocks, then 4 V blocks).
template <int D>
struct LdsTile {
    const u16* kb;   // first K block, offset by this lane's fragment
    const u16* vb;   // first V block, offset by this lane's fragment
    __device__ __forceinline__ uint4 k(int p, int ds) const { return ld16(kb + p * (kPage * D) + ds * 512); }
    __device__ __forceinline__ uint2 v(int p, int dt) const {
        return *reinterpret_cast<const uint2*>(vb + p * (kPage * D) + dt * 256);
    }
};

// Zeroes the V values of tokens past the sequence's last written position in one
// 8-byte fragment (tokens tok0 .. tok0 + 3, token e in half e % 2 of word e / 2): a
// zero softmax weight must not meet whatever those slots hold. Branch-free.
__device__ __forceinline__ uint2 mask_v(uint2 v, int tok0, int last) {
    const uint32_t m0 = (tok0 <= last ? 0x0000ffffu : 0u) | (tok0 + 1 <= last ? 0xffff0000u : 0u);
    const uint32_t m1 = (tok0 + 2 <= last ? 0x0000ffffu : 0u) | (tok0 + 3 <= last ? 0xffff0000u : 0u);
    return make_uint2(v.x & m0, v.y & m1);
}

// Tree rows as chain rows. Node u at depth d_u attends to slots 0..pos and then to the
// nodes of its path in depth order: the keys of a chain row at position pos + d_u
// whose slots pos + i hold the path's node at depth i (its one-row decode once the
// accepted path is compacted). So node u's rows run as that chain row: position
// pos + d_u, the same tiles, splits and merge. Their keys differ from the tile's slots
// only at pos + 1 .. pos + d_u and only when the path is not the nodes 1 .. d_u
// (d_u < u). A tile holding such slots is run once for the other rows; then, per root
// path through such nodes, the workgroup rewrites the tile's slots pos + i with the
// path's node at depth i (the others get node i back) and the waves holding those
// nodes' rows run the tile again. In each run the rows it does not serve get position
// -1: -inf scores only, which leave a row's state as it was. So each row's arithmetic is the
// arithmetic of its chain row (an MFMA column's result depends only on that column's
// operands).

__device__ __forceinline__ int tree_depth(uint4 mk) {   // mk: a node's ancestors and itself
    return __popc(mk.x) + __popc(mk.y) + __popc(mk.z) + __popc(mk.w) - 1;
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// path[i] = the node at depth i on the way to the node whose ancestor set is mk (a
// parent has a smaller index than its child, so depth order is index order).
__device__ __forceinline__ void build_path(uint4 mk, lds_u8 path, int lane) {
    const uint64_t lo = (uint64_t)mk.y << 32 | mk.x, hi = (uint64_t)mk.w << 32 | mk.z;
    const uint64_t below = (1ull << lane) - 1ull;
    wave_sync();
    if ((lo >> lane) & 1ull) path[__popcll(lo & below)] = (uint8_t)lane;
    if ((hi >> lane) & 1ull) path[__popcll(lo) + __popcll(hi & below)] = (uint8_t)(64 + lane);
    wave_sync();
}

// Writes a 16-row query tile's normalised output: lane l holds row l % 16, channels
// 16 dt + 4 (l / 16) + i.
template <int D>
__device__ __forceinline__ void store_out(const f32x4 (&o)[D / 16], float inv, u16* dst) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
        const uint32_t a = (uint32_t)f2bf(o[dt][0] * inv) | ((uint32_t)f2bf(o[dt][1] * inv) << 16);
        const uint32_t b = (uint32_t)f2bf(o[dt][2] * inv) | ((uint32_t)f2bf(o[dt][3] * inv) << 16);
        *reinterpret_cast<uint2*>(dst + dt * 16) = make_uint2(a, b);
    }
}

// ---------------------------------------------------------------------------
// attn_kernel: one workgroup per (sequence, kv head, split, 64-row group), kv head
// fastest. A split's K/V blocks go from HBM straight into LDS (global_load_lds: no
// staging registers), one tile of KT tokens at a time; the register file left free
// lets more workgroups share a CU, so their tiles are in flight while one computes.
// Splits past the sequence's last position leave before any tile work. The rows of a
// sequence that fits one split are final here; otherwise each split writes its
// partial (unnormalised O, running max, sum) for attn_combine_kernel.
// STREAM: pool blocks are read non-temporally (chosen from the split size, i.e. from
// capacity; the cache policy never changes a result).
template <int D>
struct AttnCfg {
    static constexpr int KT = 64;                              // tokens per tile
    static constexpr int NP = KT / kPage;                      // pages per tile
    static constexpr int BLK = kPage * D;                      // elements per block
    static constexpr int CPB = BLK * 2 / 1024;                 // 1 KB chunks per block (>= 2)
    static constexpr int NCH = 2 * NP * (CPB > 0 ? CPB : 1);   // chunks per tile
    static constexpr int WAVE_CH = NCH / 4;                    // chunks per wave
    // workgroups per CU (LDS: one tile, 16 / 32 / 64 KB; at D = 256 32-token tiles at
    // three per CU measured slower, long 441 vs 423 us)
    static constexpr int MINB = D <= 64 ? 5 : D <= 128 ? 4 : 2;
    // tree rows (the node runs' bookkeeping): at D = 64, five per CU spill inside the tile loop
    static constexpr int MINB_TREE = D <= 128 ? 4 : 2;
};

template <int D, bool TREE, bool STREAM>
__global__ __launch_bounds__(kAttnThreads, TREE ? AttnCfg<D>::MINB_TREE : AttnCfg<D>::MINB) void attn_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k_pool, const u16* __restrict__ v_pool,
    const int32_t* __restrict__ page_table, int max_pages, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ k, int Hq, int Hkv, float scale_log2, int split, int n_splits,
    RowRec* __restrict__ rows, int32_t* __restrict__ packing_ok, float2* __restrict__ part_ml, float* __restrict__ part_o,
    const int32_t* __restrict__ parent, int kmax, const u16* __restrict__ k_new, const u16* __restrict__ v_new,
    int64_t n_pages, int B, int R, int32_t* __restrict__ status, u16* __restrict__ out, u16* k_pool_w,
    u16* v_pool_w) {
    using TM = TileMath<D>;
    using C = AttnCfg<D>;
    constexpr int KT = C::KT, NP = C::NP, BLK = C::BLK, NDS = TM::NDS, NDT = TM::NDT;
    static_assert(C::NCH % 4 == 0 && C::CPB >= 2, "a tile must split into whole 1 KB chunks per wave");
    __shared__ __attribute__((aligned(16))) u16 smem[2 * NP * BLK];   // K blocks, then V blocks
    // tree rows, sized at launch from kmax (TreeLds): the new rows 1..k (K, then V), the
    // ancestor masks and links, and a path per wave
    extern __shared__ __attribute__((aligned(16))) u16 s_dyn[];
    const TreeLds tl(kmax, D);
    u16* const s_nk = s_dyn;
    u16* const s_nv = s_dyn + tl.nv;
    uint4* const s_mask = reinterpret_cast<uint4*>(s_dyn + tl.mask);
    int* const s_anc = reinterpret_cast<int*>(s_dyn + tl.anc);
    uint8_t* const s_path = reinterpret_cast<uint8_t*>(s_dyn + tl.path);

    const int tid = threadIdx.x, lane = tid % kWave, l16 = lane % 16, lq = lane / 16;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int G = Hq / Hkv;
    // Row packing (every wave forms it on its own; each k is read by every wave, from
    // cache) and, for batches of at most kRemapMaxB sequences, the work list: the
    // launch's workgroups are numbered in dispatch order and mapped onto the (sequence,
    // row group, split, kv head) items that have work, so that every such workgroup is
    // dispatched before any without (a sequence whose k or pos is invalid counts one
    // item, its status). Larger batches use the launch coordinates directly.
    int hk, c, mgroup, s;
    long long before = 0, total = 0;
    int rowbad = 0;
    if (B <= kRemapMaxB) {
        const long long wid = (long long)blockIdx.x + (long long)gridDim.x * blockIdx.z;
        long long run = 0;            // items before the current chunk of 64 sequences
        int found = -1, f_ks = 0, f_pos = 0;
        long long f_local = 0;
#pragma unroll
        for (int i0 = 0; i0 < kRemapMaxB; i0 += kWave) {
            if (i0 >= B) break;
            const int i = i0 + lane;
            int ki = 0, pi = 0;
            long long ni = 0, nr = 0;
            if (i < B) {
                ki = k[i];
                pi = pos[i];
                const bool valid = ki >= 0 && ki <= kmax && pi >= 0 && ((long long)pi + ki) / kPage < max_pages;
                ni = valid ? (long long)((pi + ki) / split + 1) * Hkv * ((G * (ki + 1) + kRowsPerGroup - 1) / kRowsPerGroup)
                           : 1;
                nr = (long long)ki + 1;
                rowbad |= ki < 0;
            }
            long long incl = ni, rincl = nr;
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const long long o = __shfl_up(incl, d), ro = __shfl_up(rincl, d);
                if (lane >= d) {
                    incl += o;
                    rincl += ro;
                }
            }
            const unsigned long long hit = __ballot(i < B && wid >= run + incl - ni && wid < run + incl);
            if (found < 0 && hit) {
                const int hl = __ffsll((long long)hit) - 1;
                found = i0 + hl;
                f_local = wid - (run + __shfl(incl - ni, hl));
                f_ks = __shfl(ki, hl);
                f_pos = __shfl(pi, hl);
                before = total + __shfl(rincl - nr, hl);
            }
            run += __shfl(incl, kWave - 1);
            total += __shfl(rincl, kWave - 1);
        }
        rowbad = __ballot(rowbad) != 0ull;
        if (found < 0) return;        // past the last item
        s = found;
        const bool valid = f_ks >= 0 && f_ks <= kmax && f_pos >= 0 && ((long long)f_pos + f_ks) / kPage < max_pages;
        const int nsp = valid ? (f_pos + f_ks) / split + 1 : 1;
        hk = (int)(f_local % Hkv);
        // tree rows: a sequence's last splits first (they hold the node runs, the longest work)
        c = (int)((f_local / Hkv) % nsp);
        if (TREE) c = nsp - 1 - c;
        mgroup = (int)(f_local / Hkv / nsp);
    } else {
        hk = blockIdx.x % Hkv;
        c = (blockIdx.x / Hkv) % n_splits;
        mgroup = blockIdx.x / Hkv / n_splits;
        s = blockIdx.z;
    }
    const int c0 = c * split;
    const int pg0 = c0 / kPage;
    // the split's page ids (lane i holds page pg0 + i + 64 r) and the tree parents
    int pid[(kMaxSplit / kPage + kWave - 1) / kWave];
#pragma unroll
    for (int r = 0; r < (int)(sizeof(pid) / sizeof(int)); ++r)
        pid[r] = page_table[(size_t)s * max_pages + min(pg0 + r * kWave + lane, max_pages - 1)];
    int par_i = 0;
    if (TREE) par_i = parent[(size_t)s * (kmax + 1) + min(tid, kmax)];
    const int ks = k[s], P0 = pos[s];
    const int last = P0 + ks;                     // the sequence's last position
    const int T = ks + 1, M = G * T;
    // Splits past the sequence's last position (and row groups past its rows) have no
    // work: they leave now, unless they write the sequence's status.
    const bool lead = hk == 0 && c == 0 && mgroup == 0;
    const bool has_work = ks >= 0 && P0 >= 0 && c0 <= last && mgroup * kRowsPerGroup < M;
    if (!has_work && !lead) return;

    if (B > kRemapMaxB) {
        for (int i = lane; i < B; i += kWave) {
            const long long kk = k[i];
            total += kk + 1;
            if (i < s) before += kk + 1;
            rowbad |= kk < 0;
        }
#pragma unroll
        for (int d = 32; d > 0; d >>= 1) {
            before += __shfl_xor(before, d);
            total += __shfl_xor(total, d);
            rowbad |= __shfl_xor(rowbad, d);
        }
    }
    const bool packed = __builtin_amdgcn_readfirstlane(!rowbad && total == (long long)R);
    const int off = __builtin_amdgcn_readfirstlane((int)before);
    const bool pos_ok = P0 >= 0 && (ks < 0 || ((long long)P0 + ks) / kPage < max_pages);
    int basic = 0;
    if (!packed || ks > kmax) basic |= SPEC_STATUS_BAD_ROWS;
    if (!pos_ok) basic |= SPEC_STATUS_BAD_POS;
    bool tree_bad = false;
    if constexpr (TREE) {
        bool bad = false;
        if (ks >= 0 && ks <= kmax && tid <= ks) bad = tid == 0 ? par_i != -1 : (par_i < 0 || par_i >= tid);
        // workgroup OR through 4 words of LDS (__syncthreads_or would take 256 bytes)
        __shared__ int s_tb[4];
        const bool wave_bad = __builtin_amdgcn_ballot_w64(bad) != 0ull;
        if (lane == 0) s_tb[wave] = wave_bad;
        __syncthreads();
        tree_bad = (s_tb[0] | s_tb[1] | s_tb[2] | s_tb[3]) != 0;
    }
    // this split's own page ids (the whole list is checked by the workgroups that write
    // the status or append rows)
    bool own_bad = false;
    if (!basic) {
        const int hi = min(last / kPage, pg0 + split / kPage - 1);
#pragma unroll
        for (int r = 0; r < (int)(sizeof(pid) / sizeof(int)); ++r) {
            const int pg = pg0 + r * kWave + lane;
            if (pg <= hi && (pid[r] < 0 || (int64_t)pid[r] >= n_pages)) own_bad = true;
        }
    }
    const bool seq_ok = !basic && !tree_bad;      // the same for every workgroup of the sequence
    const bool ok = __builtin_amdgcn_readfirstlane(seq_ok && __ballot(own_bad) == 0ull);
    const bool work = has_work && seq_ok;
    const int nc = last / split + 1;              // splits of the sequence with keys

    const int m_tile0 = mgroup * kRowsPerGroup + wave * 16;
    const bool active = m_tile0 < M;
    const int m = m_tile0 + l16;
    const bool m_ok = m < M;
    const int jrow = m_ok ? m / G : 0;
    const int h = hk * G + (m_ok ? m % G : 0);
    int p_m = m_ok ? P0 + jrow : -1;              // tree rows: P0 + depth, set below
    f32x4 o[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_lane = 0.f;

    if (work && ok) {
        const int c1 = min(c0 + split, last + 1);
        const int last_page = last / kPage;
        auto page_of = [&](int pg) -> int64_t {   // pg: absolute page index, wave-uniform
            const int i = pg - pg0;
            int id = 0;
#pragma unroll
            for (int r = 0; r < (int)(sizeof(pid) / sizeof(int)); ++r)
                if ((i >> 6) == r) id = __builtin_amdgcn_readlane(pid[r], i & 63);
            return id;
        };
        // A tile: chunk qc = it * 4 + wave (1 KB each) of block qc / CPB (K blocks of
        // the tile's pages, then their V blocks) goes to LDS chunk qc. Pages past the
        // sequence read the split's first page instead; their V is zeroed below.
        auto load_tile = [&](int t0) {
            // the tile's page ids first: a read of pid[] waits on the load counter, which
            // must not happen between two of the tile's LDS loads
            int64_t page[NP];
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int pg = t0 / kPage + p;
                page[p] = page_of(pg <= last_page ? pg : pg0);
            }
#pragma unroll
            for (int it = 0; it < C::WAVE_CH; ++it) {
                const int qc = it * 4 + wave;
                const int b = qc / C::CPB, part = qc % C::CPB;
                int64_t pgid = page[0];
#pragma unroll
                for (int p = 1; p < NP; ++p)
                    if ((b % NP) == p) pgid = page[p];
                // the block's address is the same for the whole wave: kept in scalar registers
                const uint64_t blk = (uint64_t)((b < NP ? k_pool : v_pool) + (size_t)(pgid * Hkv + hk) * BLK + part * 512);
                const uint64_t blk_s = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(blk >> 32)) << 32 |
                                       (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)blk);
                const u16* src = reinterpret_cast<const u16*>(blk_s) + lane * 8;
                __builtin_amdgcn_global_load_lds((global_cptr)src, (lds_ptr)(smem + qc * 512), 16, 0,
                                                 STREAM ? 2 : 0);   // 2: non-temporal
            }
        };
        // Tiles that reach the new rows: V slots past the last position are zeroed (a
        // zero softmax weight must not meet what they hold) and the new rows' K and V
        // are taken from k_new / v_new (the bytes the append writes, which this kernel
        // itself may be writing to the pool).
        auto fix_tile = [&](int t0) {
            constexpr int VW = BLK / 4;    // 8-byte V words per block
            for (int i = tid; i < NP * VW; i += kAttnThreads) {
                const int p = i / VW, wi = i % VW;
                const int pg = t0 / kPage + p;
                if (pg * kPage + kPage - 1 <= last) continue;
                const int tok0 = pg * kPage + 4 * ((wi * 4 % 256) / 64);
                uint2* w = reinterpret_cast<uint2*>(smem + (NP + p) * BLK) + wi;
                *w = mask_v(*w, tok0, last);
            }
            // The masking above rewrites whole 8-byte V words, which also hold tokens
            // <= last of the last page (new rows among them): every wave must be done
            // with it before any new row is written below, or a word written back by
            // one wave can undo another wave's new-row value.
            __syncthreads();
            const int r_lo = max(t0, P0), r_hi = min(t0 + KT - 1, last);
            constexpr int dch = D / 8;
            const int n_it = (r_hi - r_lo + 1) * dch;
            for (int i = tid; i < n_it; i += kAttnThreads) {
                const int tp = r_lo + i / dch, dc = i % dch;
                const size_t src = ((size_t)(off + tp - P0) * Hkv + hk) * D + dc * 8;
                const uint4 kv = ld16(k_new + src), vv = ld16(v_new + src);
                const int p = (tp - t0) / kPage, t = tp % kPage;
                st16(smem + p * BLK + k_off(t, dc * 8), kv);
                const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    smem[(NP + p) * BLK + v_off(t, dc * 8 + e)] = (u16)((e & 1) ? (w[e / 2] >> 16) : (w[e / 2] & 0xffffu));
            }
        };
        load_tile(c0);
        bf16x8 qf[NDS];
        if (active) {
            const size_t qoff = ((size_t)(off + jrow) * Hq + h) * D;
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds)
                qf[ds] = as_bf16x8(m_ok ? ld16(q + qoff + ds * 32 + lq * 8) : make_uint4(0, 0, 0, 0));
        }
        if constexpr (TREE) {
            // The new rows' LDS copy (read on tiles past the root), when this split has
            // such tiles.
            if (c1 > P0 + 1) {
                constexpr int dch = D / 8;
                for (int i = tid; i < ks * dch; i += kAttnThreads) {
                    const int u = 1 + i / dch, dc = i % dch;
                    const size_t src = ((size_t)(off + u) * Hkv + hk) * D + dc * 8;
                    st16(s_nk + (u - 1) * D + dc * 8, ld16(k_new + src));
                    st16(s_nv + (u - 1) * D + dc * 8, ld16(v_new + src));
                }
            }
            // Ancestor masks, built while the first tile's loads are in flight (nodes past
            // k_s are never read). Invariant: mask(j) holds the nodes from j up to, not
            // including, anc(j); a round adds mask(anc(j)) and moves anc(j) to anc(anc(j)),
            // doubling the covered distance. The root is its own ancestor (mask {0}), and
            // depth <= ks, so ceil(log2(ks + 1)) rounds reach it from every node.
            uint4 mk = make_uint4(0, 0, 0, 0);
            if (tid <= ks) {
                mk.x = tid < 32 ? 1u << tid : 0u;
                mk.y = tid >= 32 && tid < 64 ? 1u << (tid - 32) : 0u;
                mk.z = tid >= 64 && tid < 96 ? 1u << (tid - 64) : 0u;
                mk.w = tid >= 96 ? 1u << (tid - 96) : 0u;
                s_anc[tid] = tid == 0 ? 0 : par_i;
                s_mask[tid] = mk;
            }
            __syncthreads();
            for (int reach = 1; reach <= ks; reach *= 2) {
                int a2 = 0;
                uint4 m2 = make_uint4(0, 0, 0, 0);
                if (tid <= ks) {
                    const int an = s_anc[tid];
                    a2 = s_anc[an];
                    m2 = s_mask[an];
                }
                __syncthreads();
                if (tid <= ks) {
                    mk.x |= m2.x;
                    mk.y |= m2.y;
                    mk.z |= m2.z;
                    mk.w |= m2.w;
                    s_anc[tid] = a2;
                    s_mask[tid] = mk;
                }
                __syncthreads();
            }
            if (m_ok) p_m = P0 + tree_depth(s_mask[jrow]);
        }
        for (int t0 = c0; t0 < c1; t0 += KT) {
            // this wave's LDS loads of the tile have landed; after the barrier, every wave's
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (t0 + KT > P0) {
                fix_tile(t0);
                __syncthreads();
            }
            // full: every row keeps every key of the tile (chain: the tile ends at or before
            // the first row's position; tree: at or before the root)
            const bool full = t0 + KT - 1 <= P0 + (TREE ? 0 : m_tile0 / G);
            const LdsTile<D> src{smem + lane * 8, smem + NP * BLK + lane * 4};
            // Tree rows: run 0 serves the rows whose keys here are the tile's slots. The
            // nodes of the row group whose paths have slots here are then served in runs of
            // one root path each: the tile's new-row slots are rewritten with the path of the
            // remaining such node of highest index n (no remaining node lies below it), and
            // the run serves n and the remaining such nodes above it, whose paths are
            // prefixes of n's (a row masks the slots past its own depth). One instance of the
            // tile code serves every run.
            const int dep = p_m - P0;
            const bool own = TREE && !full && m_ok && dep < jrow && P0 + dep >= t0 && P0 + 1 <= t0 + KT - 1;
            const int i_lo = max(1, t0 - P0), i_hi = min(ks, t0 + KT - 1 - P0);   // new-row slots pos + i here
            uint32_t rem[4] = {0u, 0u, 0u, 0u};   // nodes still to serve, one bit each
            if (TREE && !full && i_lo <= i_hi) {
                const int g_hi = min((mgroup * kRowsPerGroup + kRowsPerGroup - 1) / G, ks);
#pragma unroll 1
                for (int n = max(mgroup * kRowsPerGroup / G, 1); n <= g_hi; ++n) {
                    const int d = __builtin_amdgcn_readfirstlane(tree_depth(lds_ld16((lds_cu4)s_mask + n)));
                    if (d < n && P0 + d >= t0) rem[n >> 5] |= 1u << (n & 31);
                }
            }
            const lds_u8 path = (lds_u8)(s_path + wave * tl.path_stride);
            bool pending = own;                   // this lane's row still waits for its run
            int p_run = own ? -1 : p_m;           // run 0
            bool first = true;
#pragma unroll 1
            for (;;) {
                if (active && (first || __builtin_amdgcn_ballot_w64(p_run >= 0)))
                    TM::template run<NP>(qf, src, t0, p_run, full && first, lq, scale_log2, m_run, l_lane, o);
                if (!TREE || !(rem[0] | rem[1] | rem[2] | rem[3])) break;
                first = false;
                const int w = rem[3] ? 3 : rem[2] ? 2 : rem[1] ? 1 : 0;
                const int n = 32 * w + 31 - __clz(rem[w]);
                const uint4 mk = lds_ld16((lds_cu4)s_mask + n);
                const int d = __builtin_amdgcn_readfirstlane(tree_depth(mk));
                const uint32_t mw[4] = {(uint32_t)__builtin_amdgcn_readfirstlane(mk.x),
                                        (uint32_t)__builtin_amdgcn_readfirstlane(mk.y),
                                        (uint32_t)__builtin_amdgcn_readfirstlane(mk.z),
                                        (uint32_t)__builtin_amdgcn_readfirstlane(mk.w)};
#pragma unroll
                for (int q = 0; q < 4; ++q) rem[q] &= ~mw[q];
                // this run serves the rows of n and of the waiting nodes above it
                const uint32_t jw = jrow < 32 ? mw[0] : jrow < 64 ? mw[1] : jrow < 96 ? mw[2] : mw[3];
                const bool served = pending && ((jw >> (jrow & 31)) & 1u);
                pending = pending && !served;
                p_run = served ? p_m : -1;
                build_path(mk, path, lane);
                __syncthreads();              // the tile's previous run is done
                constexpr int dch = D / 8;
                for (int it = tid; it < (i_hi - i_lo + 1) * dch; it += kAttnThreads) {
                    const int i = i_lo + it / dch, dc = it % dch;
                    const int u = i <= d ? (int)path[i] : i;
                    const int tp = P0 + i, pp = (tp - t0) / kPage, t = tp % kPage;
                    st16(smem + pp * BLK + k_off(t, dc * 8), ld16(s_nk + (u - 1) * D + dc * 8));
                    const uint4 vv = ld16(s_nv + (u - 1) * D + dc * 8);
                    const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        smem[(NP + pp) * BLK + v_off(t, dc * 8 + e)] = (u16)((e & 1) ? (vw[e / 2] >> 16) : (vw[e / 2] & 0xffffu));
                }
                __syncthreads();
            }
            if (t0 + KT < c1) {
                __syncthreads();              // every wave is done reading the tile
                load_tile(t0 + KT);
            }
        }
    }

    // ---- rows of a single-split sequence are final; otherwise the split partial ----
    if (work && ok && active && m_ok) {
        float l_tot = l_lane + __shfl_xor(l_lane, 16);
        l_tot = l_tot + __shfl_xor(l_tot, 32);
        if (nc == 1) {
            // the merge of one split is the same arithmetic (weight exp2(0) = 1, sum l)
            store_out<D>(o, 1.f / l_tot, out + ((size_t)(off + jrow) * Hq + h) * D + lq * 4);
        } else if (p_m >= c0) {
            // rows whose keys all lie before this split need no partial (the merge reads
            // splits 0 .. p / split of a row at position p)
            const size_t idx = ((size_t)(off + jrow) * Hq + h) * n_splits + c;
            if (lq == 0) part_ml[idx] = make_float2(m_run, l_tot);
            float* po = part_o + idx * D + lq * 4;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16) = o[dt];
        }
    }

    // ---- the sequence's status (one workgroup) and the append of this kv head's
    // new rows that fall in this split (the row-group-0 workgroups) ---------------
    {
        const bool writer = mgroup == 0 && seq_ok && has_work && c0 + split > P0;
        if (!lead && !writer) return;
        int flags = basic | (tree_bad ? SPEC_STATUS_BAD_TREE : 0);
        if (pos_ok && ks >= 0) {
            // 8 page ids per thread requested at once (clamped to the last page), then checked
            const int last_page = last / kPage;
            for (int pgb = tid; pgb <= last_page; pgb += kAttnThreads * 8) {
                int ids[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    ids[u] = page_table[(size_t)s * max_pages + min(pgb + u * kAttnThreads, last_page)];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (pgb + u * kAttnThreads <= last_page && (ids[u] < 0 || (int64_t)ids[u] >= n_pages))
                        flags |= SPEC_STATUS_BAD_PAGE;
            }
        }
        // bitwise OR over the workgroup: across each wave, then across the 4 waves
#pragma unroll
        for (int d = 32; d > 0; d >>= 1) flags |= __shfl_xor(flags, d);
        // the 4 words live in the tile's LDS (so that a chain workgroup's LDS is the tile
        // alone): every wave must be done reading its last tile first
        int* const s_fl = reinterpret_cast<int*>(smem);
        __syncthreads();
        if (lane == 0) s_fl[wave] = flags;
        __syncthreads();
        const int bits = s_fl[0] | s_fl[1] | s_fl[2] | s_fl[3];
        if (lead) {
            if (tid == 0) {
                status[s] = bits;
                if (s == 0) *packing_ok = packed;
            }
            // per-row records for the merge kernel (only when the packing is defined;
            // otherwise it writes nothing): the splits to merge, 0 when the sequence is
            // skipped or its rows were written here
            if (packed)
                for (int j = tid; j <= ks; j += kAttnThreads) {
                    // tree rows: the position of the row's chain row (the masks exist when bits == 0)
                    const int pj = P0 + ((TREE && !bits) ? tree_depth(s_mask[j]) : j);
                    rows[off + j] = RowRec{pj, (bits || nc == 1) ? 0 : pj / split + 1};
                }
        }
        if (!writer || bits) return;
        // 8 channels (one 16-byte chunk of a row) per item
        const int j_lo = max(c0, P0) - P0, j_hi = min(c0 + split - 1, last) - P0;
        constexpr int dch = D / 8;
        const int n_it = (j_hi - j_lo + 1) * dch;
        for (int i = tid; i < n_it; i += kAttnThreads) {
            const int j = j_lo + i / dch, dc = i % dch;
            const size_t src = ((size_t)(off + j) * Hkv + hk) * D + dc * 8;
            const uint4 kv = ld16(k_new + src), vv = ld16(v_new + src);
            const int page = page_table[(size_t)s * max_pages + (P0 + j) / kPage];
            const int t = (P0 + j) % kPage;
            const size_t blk = ((size_t)page * Hkv + hk) * BLK;
            st16(k_pool_w + blk + k_off(t, dc * 8), kv);   // 8 channels contiguous
            const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v_pool_w[blk + v_off(t, dc * 8 + e)] = (u16)((e & 1) ? (w[e / 2] >> 16) : (w[e / 2] & 0xffffu));
        }
    }
}

// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(
    const RowRec* __restrict__ rows, const int32_t* __restrict__ packing_ok, int R, int Hq, int n_splits,
    const float2* __restrict__ part_ml, const float* __restrict__ part_o, u16* __restrict__ out) {
    constexpr int PER = D / kWave;
    constexpr int kGroup = 8;    // splits whose partials are loaded at once
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const long long item = (long long)blockIdx.x * 4 + wave;
    if (item >= (long long)R * Hq) return;
    const int r = (int)(item / Hq), h = (int)(item % Hq);
    const int ok = *packing_ok;
    const RowRec rr = rows[r];
    if (!ok || rr.nc <= 0) return;               // packing undefined, or the sequence is skipped
    const int nc = rr.nc;
    const size_t base = ((size_t)r * Hq + h) * n_splits;
    float2 ml[kGroup];
    float po[kGroup][PER];
    auto load_group = [&](int c0) {
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            const int c = c0 + u < nc ? c0 + u : nc - 1;
            ml[u] = part_ml[base + c];
#pragma unroll
            for (int e = 0; e < PER; ++e) po[u][e] = part_o[(base + c) * D + e * kWave + lane];
        }
    };
    // the first group's partials are requested in the same round as the maxima
    load_group(0);
    float mx = -INFINITY;
    for (int c = lane; c < nc; c += kWave) mx = fmaxf(mx, part_ml[base + c].x);
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d));
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    float L = 0.f;
    // splits merged in ascending order
    for (int c0 = 0; c0 < nc; c0 += kGroup) {
        if (c0 > 0) load_group(c0);
        // consume every loaded value here so that the group's loads are all issued first
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            asm volatile("" : "+v"(ml[u].x), "+v"(ml[u].y));
#pragma unroll
            for (int e = 0; e < PER; ++e) asm volatile("" : "+v"(po[u][e]));
        }
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            if (c0 + u >= nc) break;
            const float wgt = exp2f(ml[u].x - mx);
            L += wgt * ml[u].y;
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] += wgt * po[u][e];
        }
    }
    const float inv = 1.f / L;
    u16* dst = out + ((size_t)r * Hq + h) * D;
#pragma unroll
    for (int e = 0; e < PER; ++e) dst[e * kWave + lane] = f2bf(acc[e] * inv);
}

// ---------------------------------------------------------------------------
// A tree workgroup's whole LDS: the tile (4 K and 4 V blocks), the parent check's
// 4-word flag array and TreeLds. gfx950 gives a workgroup 160 KB.
static size_t tree_lds_bytes(int D, int kmax) {
    return (size_t)2 * kKT * D * sizeof(u16) + 16 + TreeLds(kmax, D).bytes();
}
constexpr size_t kLdsPerWorkgroup = 160 * 1024;

static int64_t split_count(int32_t max_pages, int32_t split) {
    return ((int64_t)max_pages * kPage + split - 1) / split;
}

struct AttnWs {
    size_t flag_off, rows_off, ml_off, o_off, total;
};

static AttnWs attn_ws_layout(int32_t R, int32_t Hq, int32_t D, int64_t n_splits) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    AttnWs w;
    w.flag_off = 0;
    w.rows_off = 256;
    w.ml_off = w.rows_off + up(sizeof(RowRec) * (size_t)R);
    w.o_off = w.ml_off + up(sizeof(float2) * (size_t)R * Hq * n_splits);
    w.total = w.o_off + up(sizeof(float) * (size_t)R * Hq * n_splits * D);
    return w;
}

template <int D>
static void launch_attn(const u16* q, u16* k_pool, u16* v_pool, const int32_t* pt, int max_pages,
                        const int32_t* pos, const int32_t* k, int kmax, RowRec* rows, int32_t* packing_ok, int B,
                        int R, int Hq, int Hkv, float scale, int split, int n_splits, float2* ml, float* po, u16* out,
                        const int32_t* parent, const u16* k_new, const u16* v_new, int64_t n_pages,
                        int32_t* status, hipStream_t st) {
    const int kv_rows = (Hq / Hkv) * (kmax + 1);   // most query rows of one kv head
    const int mgroups = (kv_rows + kRowsPerGroup - 1) / kRowsPerGroup;
    dim3 grid(mgroups * n_splits * Hkv, 1, B);
    // Non-temporal pool reads for long contexts (splits of >= kStreamSplit tokens,
    // i.e. page tables of more than 32K tokens).
    const size_t node_lds = parent ? TreeLds(kmax, D).bytes() : 0;
    auto go = [&](auto tree_c, auto stream_c) {
        constexpr bool T = decltype(tree_c)::value, S = decltype(stream_c)::value;
        hipLaunchKernelGGL((attn_kernel<D, T, S>), grid, dim3(kAttnThreads), node_lds, st, q, k_pool, v_pool, pt, max_pages,
                           pos, k, Hq, Hkv, scale * kLog2e, split, n_splits, rows, packing_ok, ml, po, parent, kmax,
                           k_new, v_new, n_pages, B, R, status, out, k_pool, v_pool);
    };
    const bool stream_kv = split >= kStreamSplit;
    if (parent) {
        if (stream_kv) go(std::true_type{}, std::true_type{});
        else go(std::true_type{}, std::false_type{});
    } else {
        if (stream_kv) go(std::false_type{}, std::true_type{});
        else go(std::false_type{}, std::false_type{});
    }
    const long long items = (long long)R * Hq;
    hipLaunchKernelGGL(attn_combine_kernel<D>, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, st,
                       rows, packing_ok, R, Hq, n_splits, ml, po, out);
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
    return sv::attn_ws_layout(R, Hq, D, sv::split_count(max_pages, split)).total;
}

size_t spec_verify_attn_tree_workspace_bytes(int32_t B, int32_t R, int32_t Hq, int32_t Hkv, int32_t D,
                                             int32_t max_pages, int32_t kv_split_tokens, int32_t kmax) {
    (void)Hkv;
    if (B < 1 || R < 1 || Hq < 1 || D < 1 || max_pages < 1 || kmax < 0) return 0;
    const int32_t split = kv_split_tokens > 0 ? kv_split_tokens : spec_attn_split_tokens(max_pages);
    return sv::attn_ws_layout(R, Hq, D, sv::split_count(max_pages, split)).total;   // as the chain call
}

}  // extern "C"

namespace sv {

// Shared body of the chain and tree entry points (parent == nullptr: chain rows).
static int verify_attn_impl(const char* name, const spec_bf16* q, const spec_bf16* k_new, const spec_bf16* v_new,
                            spec_bf16* k_pool, spec_bf16* v_pool, int64_t n_pages, const int32_t* page_table,
                            int32_t max_pages, const int32_t* pos, const int32_t* k, const int32_t* parent,
                            int32_t kmax, int32_t B, int32_t R, int32_t Hq, int32_t Hkv, int32_t D, float scale,
                            int32_t kv_split_tokens, spec_bf16* out, void* workspace, size_t workspace_bytes,
                            int32_t* seq_status, void* stream) {
    last_error().clear();
    if (D != 64 && D != 128 && D != 256) return fail(SPEC_EINVAL, "%s: D=%d not in {64,128,256}", name, D);
    if (Hkv < 1 || Hq < Hkv || Hq % Hkv) return fail(SPEC_EINVAL, "%s: Hq=%d Hkv=%d (need Hq %% Hkv == 0)", name, Hq, Hkv);
    if (Hq / Hkv > 16) return fail(SPEC_EINVAL, "%s: Hq/Hkv=%d > 16", name, Hq / Hkv);
    if (B < 1 || B > 4096) return fail(SPEC_EINVAL, "%s: B=%d outside 1..4096", name, B);
    if (R < 1) return fail(SPEC_EINVAL, "%s: R=%d < 1", name, R);
    if (kmax < 0 || kmax > kMaxK) return fail(SPEC_EINVAL, "%s: kmax=%d outside 0..%d", name, kmax, kMaxK);
    if (max_pages < 1 || n_pages < 1) return fail(SPEC_EINVAL, "%s: max_pages=%d n_pages=%lld", name, max_pages, (long long)n_pages);
    if (parent && tree_lds_bytes(D, kmax) > kLdsPerWorkgroup)
        return fail(SPEC_EINVAL, "%s: kmax=%d at D=%d needs %zu bytes of LDS per workgroup (> %zu)", name, kmax, D,
                    tree_lds_bytes(D, kmax), kLdsPerWorkgroup);
    if (!(scale > 0.f)) return fail(SPEC_EINVAL, "%s: scale must be > 0", name);
    if (kv_split_tokens < 0 || kv_split_tokens % kKT || kv_split_tokens > kMaxSplit)
        return fail(SPEC_EINVAL, "%s: kv_split_tokens=%d not a multiple of 64 in 0..%d", name, kv_split_tokens, kMaxSplit);
    if (!q || !k_new || !v_new || !k_pool || !v_pool || !page_table || !pos || !k || !out || !seq_status)
        return fail(SPEC_EINVAL, "%s: null required pointer", name);
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
        return fail(SPEC_EINVAL, "%s: q, k_new, v_new, k_pool, v_pool and out must be 16-byte aligned", name);
    const int32_t split = kv_split_tokens > 0 ? kv_split_tokens : spec_attn_split_tokens(max_pages);
    const int64_t n_splits = split_count(max_pages, split);
    if (n_splits * 2 * Hkv > 0x7fffffffLL || (long long)B * Hkv * n_splits > 0x7fffffffLL)
        return fail(SPEC_ECAPACITY, "%s: too many splits", name);
    const AttnWs lay = attn_ws_layout(R, Hq, D, n_splits);
    if (!workspace || workspace_bytes < lay.total || !aligned16(workspace))
        return fail(SPEC_EWORKSPACE, "%s: workspace %zu bytes < %zu required (or null/misaligned)", name, workspace_bytes, lay.total);
    char* ws = static_cast<char*>(workspace);
    int32_t* packing_ok = reinterpret_cast<int32_t*>(ws + lay.flag_off);
    RowRec* rows = reinterpret_cast<RowRec*>(ws + lay.rows_off);
    float2* ml = reinterpret_cast<float2*>(ws + lay.ml_off);
    float* po = reinterpret_cast<float*>(ws + lay.o_off);
    hipStream_t st = (hipStream_t)stream;
    switch (D) {
        case 64: launch_attn<64>(q, k_pool, v_pool, page_table, max_pages, pos, k, kmax, rows, packing_ok, B, R, Hq, Hkv, scale, split, (int)n_splits, ml, po, out, parent, k_new, v_new, n_pages, seq_status, st); break;
        case 128: launch_attn<128>(q, k_pool, v_pool, page_table, max_pages, pos, k, kmax, rows, packing_ok, B, R, Hq, Hkv, scale, split, (int)n_splits, ml, po, out, parent, k_new, v_new, n_pages, seq_status, st); break;
        default: launch_attn<256>(q, k_pool, v_pool, page_table, max_pages, pos, k, kmax, rows, packing_ok, B, R, Hq, Hkv, scale, split, (int)n_splits, ml, po, out, parent, k_new, v_new, n_pages, seq_status, st); break;
    }
    SV_LAUNCH_CHECK(name);
    return SPEC_OK;
}

}  // namespace sv

extern "C" {

int spec_verify_attn(const spec_bf16* q, const spec_bf16* k_new, const spec_bf16* v_new,
                     spec_bf16* k_pool, spec_bf16* v_pool, int64_t n_pages,
                     const int32_t* page_table, int32_t max_pages, const int32_t* pos,
                     const int32_t* k, int32_t kmax, int32_t B, int32_t R, int32_t Hq, int32_t Hkv,
                     int32_t D, float scale, int32_t kv_split_tokens, spec_bf16* out, void* workspace,
                     size_t workspace_bytes, int32_t* seq_status, void* stream) {
    return sv::verify_attn_impl("spec_verify_attn", q, k_new, v_new, k_pool, v_pool, n_pages, page_table, max_pages,
                                pos, k, nullptr, kmax, B, R, Hq, Hkv, D, scale, kv_split_tokens, out, workspace,
                                workspace_bytes, seq_status, stream);
}

int spec_verify_attn_tree(const spec_bf16* q, const spec_bf16* k_new, const spec_bf16* v_new,
                          spec_bf16* k_pool, spec_bf16* v_pool, int64_t n_pages,
                          const int32_t* page_table, int32_t max_pages, const int32_t* pos,
                          const int32_t* k, const int32_t* parent, int32_t kmax, int32_t B, int32_t R,
                          int32_t Hq, int32_t Hkv, int32_t D, float scale, int32_t kv_split_tokens,
                          spec_bf16* out, void* workspace, size_t workspace_bytes, int32_t* seq_status,
                          void* stream) {
    if (!parent) {
        sv::last_error().clear();
        return sv::fail(SPEC_EINVAL, "spec_verify_attn_tree: null parent");
    }
    return sv::verify_attn_impl("spec_verify_attn_tree", q, k_new, v_new, k_pool, v_pool, n_pages, page_table,
                                max_pages, pos, k, parent, kmax, B, R, Hq, Hkv, D, scale, kv_split_tokens, out,
                                workspace, workspace_bytes, seq_status, stream);
}

}  // extern "C"
