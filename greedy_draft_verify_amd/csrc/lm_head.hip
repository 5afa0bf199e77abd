// spec_lm_head_argmax: bf16 MFMA lm_head with the greedy argmax fused into the
// epilogue; the logits never leave registers.
//
// lm_head_tile_kernel: one workgroup per (vocabulary tile of 128 entries, group of
// up to 128 rows). Each wave owns 32 vocabulary rows of W and streams them straight
// from HBM into MFMA B-operand registers (W is read exactly once per row group),
// double-buffered one K-block (128 channels) ahead. The hidden rows are shared by
// the four waves through LDS. After the K loop each wave reduces its logits to the
// best (value, index) per row with the order "larger value, then smaller index"
// (the first-maximum rule of span-02 greedy_logprob), the workgroup merges its four
// waves, and one record per (tile, row) goes to the workspace.
// lm_head_final_kernel: one workgroup per row merges the tiles' records with the
// same order. The order is total, so the result does not depend on how the
// reduction is grouped; each logit is one MFMA chain over K in a fixed order, so a
// row's result does not depend on R.
#include "common.h"

namespace sv {

constexpr int kLmThreads = 256;
constexpr int kLmNT = 2;                  // 16-entry vocabulary tiles per wave
constexpr int kLmVocabPerWg = 4 * 16 * kLmNT;
constexpr int kLmKB = 128;                // K-block (channels) per LDS stage
constexpr int kLmHStr = kLmKB + 8;        // LDS row stride (elements)
constexpr int kLmMaxMT = 8;               // 16-row tiles per row group

struct Best {
    float v;
    int i;
};

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

template <int MT>
__global__ __launch_bounds__(kLmThreads) void lm_head_tile_kernel(
    const u16* __restrict__ hidden, const u16* __restrict__ w, int R, int H, int V, int n_vt,
    int n_rg, float* __restrict__ part_v, int* __restrict__ part_i) {
    __shared__ __attribute__((aligned(16))) u16 hs[16 * MT * kLmHStr];
    __shared__ Best wbest[4][16 * MT];

    // Logical tile: with several row groups, hardware workgroup i runs on XCD i % 8;
    // give the row groups of one vocabulary tile consecutive slots of one XCD so that
    // W is fetched from HBM once and re-read from that XCD's L2.
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
    const int vbase = vt * kLmVocabPerWg + wave * 16 * kLmNT;

    // W rows of this lane (clamped in range; out-of-range entries are masked later)
    const u16* wrow[kLmNT];
#pragma unroll
    for (int nt = 0; nt < kLmNT; ++nt) {
        const int v = min(vbase + nt * 16 + l16, V - 1);
        wrow[nt] = w + (size_t)v * H + lq * 8;
    }
    constexpr int KS = kLmKB / 32;  // MFMA k-steps per K-block
    uint4 wcur[kLmNT][KS], wnext[kLmNT][KS];
    // hidden staging: MT * 256 chunks of 16 bytes per K-block, MT per thread
    uint4 hcur[MT], hnext[MT];
    auto load_h = [&](int kb, uint4* dst) {
#pragma unroll
        for (int it = 0; it < MT; ++it) {
            const int cidx = it * kLmThreads + tid;
            const int row = cidx / (kLmKB / 8), ch = cidx % (kLmKB / 8);
            const int r = r0 + row;
            dst[it] = r < R ? ld16(hidden + (size_t)r * H + kb * kLmKB + ch * 8) : make_uint4(0, 0, 0, 0);
        }
    };
    auto load_w = [&](int kb, uint4 (*dst)[KS]) {
#pragma unroll
        for (int nt = 0; nt < kLmNT; ++nt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) dst[nt][ks] = ld16(wrow[nt] + kb * kLmKB + ks * 32);
    };

    f32x4 acc[MT][kLmNT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < kLmNT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nkb = H / kLmKB;
    load_h(0, hnext);
    load_w(0, wnext);
    for (int kb = 0; kb < nkb; ++kb) {
#pragma unroll
        for (int it = 0; it < MT; ++it) hcur[it] = hnext[it];
#pragma unroll
        for (int nt = 0; nt < kLmNT; ++nt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) wcur[nt][ks] = wnext[nt][ks];
        __syncthreads();
#pragma unroll
        for (int it = 0; it < MT; ++it) {
            const int cidx = it * kLmThreads + tid;
            const int row = cidx / (kLmKB / 8), ch = cidx % (kLmKB / 8);
            st16(hs + row * kLmHStr + ch * 8, hcur[it]);
        }
        __syncthreads();
        if (kb + 1 < nkb) {
            load_h(kb + 1, hnext);
            load_w(kb + 1, wnext);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const bf16x8 a = as_bf16x8(ld16(hs + (mt * 16 + l16) * kLmHStr + ks * 32 + lq * 8));
#pragma unroll
                for (int nt = 0; nt < kLmNT; ++nt)
                    acc[mt][nt] = mfma16x16x32(a, as_bf16x8(wcur[nt][ks]), acc[mt][nt]);
            }
        }
    }

    // epilogue: C[row = 16 mt + 4 lq + i][vocab = vbase + 16 nt + l16]
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int nt = 0; nt < kLmNT; ++nt) {
                const int v = vbase + nt * 16 + l16;
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
        part_v[(size_t)vt * R + r0 + tid] = b.v;
        part_i[(size_t)vt * R + r0 + tid] = b.i;
    }
}

__global__ __launch_bounds__(256) void lm_head_final_kernel(const float* __restrict__ part_v,
                                                            const int* __restrict__ part_i, int R,
                                                            int n_vt, int32_t* __restrict__ argmax,
                                                            float* __restrict__ maxval) {
    __shared__ Best sb[4];
    const int r = blockIdx.x, tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int t = tid; t < n_vt; t += 256) {
        const float v = part_v[(size_t)t * R + r];
        const int i = part_i[(size_t)t * R + r];
        if (better(v, i, bv, bi)) {
            bv = v;
            bi = i;
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
    if (lane == 0) sb[wave] = Best{bv, bi};
    __syncthreads();
    if (tid == 0) {
        Best b = sb[0];
        for (int wv = 1; wv < 4; ++wv)
            if (better(sb[wv].v, sb[wv].i, b.v, b.i)) b = sb[wv];
        argmax[r] = b.i;
        if (maxval) maxval[r] = b.v;
    }
}

static int n_vtiles(int V) { return (V + kLmVocabPerWg - 1) / kLmVocabPerWg; }

template <int MT>
static void launch_tiles(const u16* hidden, const u16* w, int R, int H, int V, int n_vt, int n_rg,
                         float* pv, int* pi, hipStream_t st) {
    int grid = n_vt * n_rg;
    if (n_rg > 1) grid = (grid + 7) / 8 * 8;
    hipLaunchKernelGGL(lm_head_tile_kernel<MT>, dim3(grid), dim3(kLmThreads), 0, st, hidden, w, R, H,
                       V, n_vt, n_rg, pv, pi);
}

}  // namespace sv

extern "C" {

size_t spec_lm_head_argmax_workspace_bytes(int32_t R, int32_t H, int32_t V) {
    (void)H;
    if (R < 1 || V < 1) return 0;
    const size_t n = (size_t)sv::n_vtiles(V) * R;
    return ((n * sizeof(float) + 255) & ~(size_t)255) + n * sizeof(int);
}

int spec_lm_head_argmax(const spec_bf16* hidden, const spec_bf16* w, int32_t R, int32_t H, int32_t V,
                        int32_t* argmax, float* maxval, void* workspace, size_t workspace_bytes,
                        void* stream) {
    using namespace sv;
    last_error().clear();
    if (R < 1) return fail(SPEC_EINVAL, "spec_lm_head_argmax: R=%d < 1", R);
    if (H < kLmKB || H % kLmKB) return fail(SPEC_EINVAL, "spec_lm_head_argmax: H=%d not a positive multiple of %d", H, kLmKB);
    if (V < 1 || V == 0x7fffffff) return fail(SPEC_EINVAL, "spec_lm_head_argmax: V=%d", V);
    if (!hidden || !w || !argmax) return fail(SPEC_EINVAL, "spec_lm_head_argmax: null required pointer");
    if (!aligned16(hidden) || !aligned16(w)) return fail(SPEC_EINVAL, "spec_lm_head_argmax: hidden and w must be 16-byte aligned");
    const size_t need = spec_lm_head_argmax_workspace_bytes(R, H, V);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return fail(SPEC_EWORKSPACE, "spec_lm_head_argmax: workspace %zu bytes < %zu required (or null/misaligned)", workspace_bytes, need);
    const int n_vt = n_vtiles(V);
    const size_t n = (size_t)n_vt * R;
    float* pv = static_cast<float*>(workspace);
    int* pi = reinterpret_cast<int*>(static_cast<char*>(workspace) + ((n * sizeof(float) + 255) & ~(size_t)255));
    const int mtiles = (R + 15) / 16;
    const int MT = mtiles < kLmMaxMT ? mtiles : kLmMaxMT;
    const int n_rg = (mtiles + MT - 1) / MT;
    if ((long long)n_vt * n_rg + 8 > 0x7fffffffLL) return fail(SPEC_ECAPACITY, "spec_lm_head_argmax: grid too large");
    hipStream_t st = (hipStream_t)stream;
    switch (MT) {
        case 1: launch_tiles<1>(hidden, w, R, H, V, n_vt, n_rg, pv, pi, st); break;
        case 2: launch_tiles<2>(hidden, w, R, H, V, n_vt, n_rg, pv, pi, st); break;
        case 3: launch_tiles<3>(hidden, w, R, H, V, n_vt, n_rg, pv, pi, st); break;
        case 4: launch_tiles<4>(hidden, w, R, H, V, n_vt, n_rg, pv, pi, st); break;
        case 5: launch_tiles<5>(hidden, w, R, H, V, n_vt, n_rg, pv, pi, st); break;
        case 6: launch_tiles<6>(hidden, w, R, H, V, n_vt, n_rg, pv, pi, st); break;
        case 7: launch_tiles<7>(hidden, w, R, H, V, n_vt, n_rg, pv, pi, st); break;
        default: launch_tiles<8>(hidden, w, R, H, V, n_vt, n_rg, pv, pi, st); break;
    }
    SV_LAUNCH_CHECK("spec_lm_head_argmax(tiles)");
    hipLaunchKernelGGL(lm_head_final_kernel, dim3(R), dim3(256), 0, st, pv, pi, R, n_vt, argmax, maxval);
    SV_LAUNCH_CHECK("spec_lm_head_argmax(final)");
    return SPEC_OK;
}

}  // extern "C"
