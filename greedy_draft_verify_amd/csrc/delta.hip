// spec_delta_verify_rollback: Gated DeltaNet verify with per-token state recording,
// and rollback to the committed prefix.
//
// delta_scan_kernel: two workgroups (256 threads each) per (sequence, head), one
// per half of the value rows. The fp32 state S [128][128] lives in registers for the
// whole scan: in workgroup w, thread t owns the four key columns 4*(t % 32) .. +3 of
// the eight value rows 64 w + (t / 32) + 8*i, so every row of S is spread over 32
// lanes of one half-wave and each store instruction of a wave writes two whole rows
// (1 KB contiguous). Per token:
//   u  = S k_t                     (half-wave reduce-scatter, then a broadcast per row)
//   S <- a_t S + (b_t v_t - a_t b_t u) k_t^T     (= a_t S (I - b_t k k^T) + b_t v k^T)
//   o_t = S (q_scale q_t)          (half-wave reduce-scatter)
// and S_t is written to the record (modes 1, 3) and, at t = L, to the state (modes 3,
// 5). Mode 4 writes only o; mode 5 runs only tokens 1..L and writes only S_L.
// Iteration t does the same arithmetic whatever T is, so S_L of a T-token scan
// equals the final state of an L-token scan bit for bit (memra linear_attn_verify_t:
// one scan over T tokens equals T chained one-token steps).
// delta_restore_kernel: mode 2, state <- rec[L - 1] (bit-exact copy).
#include "common.h"

namespace sv {

constexpr int kDk = 128, kDv = 128;

// Reduce-scatter of N per-row partial sums over the 32 lanes of a half-wave: at
// distances 16, 8, ... each lane keeps half of its remaining rows and adds the
// partner's partials of those rows; once one row is left, exchanges at the remaining
// distances complete the sum. Lane l of the half-wave ends with the full sum of row
// l / (32 / N) (N = 16: l / 2 after 16 shuffles instead of 5 per row). The order of
// the additions is fixed.
template <int N, int D = 16>
__device__ __forceinline__ float reduce_scatter(const float (&p)[N], int c32) {
    if constexpr (N == 1) {
        float x = p[0];
#pragma unroll
        for (int d = D; d >= 1; d >>= 1) x += __shfl_xor(x, d);
        return x;
    } else {
        float h[N / 2];
        const bool hi = c32 & D;
#pragma unroll
        for (int i = 0; i < N / 2; ++i) h[i] = (hi ? p[N / 2 + i] : p[i]) + __shfl_xor(hi ? p[i] : p[N / 2 + i], D);
        return reduce_scatter<N / 2, D / 2>(h, c32);
    }
}

// Tokens whose q/k/v/a/b are staged in LDS per round (fp32, 24.6 KB), so the scan
// runs without waiting on global loads between tokens.
constexpr int kTokChunk = 16;

// NR value rows per thread: a (sequence, head) is split over 16 / NR workgroups of
// 8 NR rows each (rows are independent: row i of S_t needs only row i of S_{t-1}).
// NR = 8 (two workgroups per (sequence, head), 111 VGPRs, four per CU) against
// NR = 16 (one, 167 VGPRs, three per CU) on the 32 x 32-head workload: verify 28.2 ->
// 25.5 us, re-scan 32.6 -> 29.2, record + rollback 74.2 -> 74.5 (HBM-bound); NR = 4
// was no better. Every row's sums are formed in the same order either way, so the
// results are bit-identical. NR is a constant: every mode must run the same
// arithmetic, so that a re-scan reproduces the recorded states bit for bit.
constexpr int kDeltaNR = 8;
constexpr int kDeltaSplit = 16 / kDeltaNR;
template <int NR>
__global__ __launch_bounds__(256, NR == 16 ? 3 : 4) void delta_scan_kernel(
    int mode, const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const float* __restrict__ a, const float* __restrict__ b, float q_scale, float* state,
    float* __restrict__ rec, const int32_t* __restrict__ L, int T, int Hd, u16* __restrict__ o) {
    __shared__ __attribute__((aligned(16))) float sk[kTokChunk][kDk], sq[kTokChunk][kDk], sv[kTokChunk][kDv];
    __shared__ float sa[kTokChunk], sb[kTokChunk];
    constexpr int SPLIT = 16 / NR, RW = 32 / NR;   // workgroups per (sequence, head); lanes per row sum
    const int sh = blockIdx.x / SPLIT;
    const int s = sh / Hd, h = sh % Hd;
    const int tid = threadIdx.x, c32 = tid % 32, rg = tid / 32;
    const int row0 = (blockIdx.x % SPLIT) * 8 * NR + rg;   // this thread's rows: row0 + 8 i
    const int lane_base = tid % kWave - c32;     // first lane of this half-wave
    const int j0 = 4 * c32;
    const bool record = mode == SPEC_DELTA_RECORD || mode == SPEC_DELTA_BOTH;
    const bool write_o = o && mode != SPEC_DELTA_RESCAN;
    int Ls = -1;
    if (mode == SPEC_DELTA_BOTH || mode == SPEC_DELTA_RESCAN) {
        Ls = L[s];
        Ls = Ls < 0 ? 0 : (Ls > T ? T : Ls);
    }
    if (mode == SPEC_DELTA_RESCAN && Ls == 0) return;   // nothing committed: S_0 stays
    float S[NR][4];
    float* st = state + (size_t)sh * kDv * kDk;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(st + (row0 + 8 * i) * kDk + j0);
        S[i][0] = x[0];
        S[i][1] = x[1];
        S[i][2] = x[2];
        S[i][3] = x[3];
    }
    const int t_run = mode == SPEC_DELTA_RESCAN ? Ls : T;   // re-scan: only the committed tokens
    for (int tc = 0; tc < t_run; tc += kTokChunk) {
        const int nt = min(kTokChunk, t_run - tc);
        __syncthreads();   // the previous round's values are no longer read
        // stage: per token 3 x 16 chunks of 8 bf16 (k, q, v), and a_t, b_t
        for (int c = tid; c < nt * 48; c += 256) {
            const int tok = c / 48, part = c % 48, which = part / 16, off = (part % 16) * 8;
            const size_t th = ((size_t)s * T + tc + tok) * Hd + h;
            const u16* src = (which == 0 ? k : which == 1 ? q : v) + th * kDk + off;
            const uint4 x = ld16(src);
            const uint32_t w[4] = {x.x, x.y, x.z, x.w};
            float f[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = bf2f((u16)((e & 1) ? (w[e / 2] >> 16) : (w[e / 2] & 0xffffu)));
            float* dst = which == 0 ? &sk[tok][off] : which == 1 ? &sq[tok][off] : &sv[tok][off];
            const float sc = which == 1 ? q_scale : 1.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) dst[e] = which == 1 ? sc * f[e] : f[e];
        }
        if (tid < nt) {
            const size_t th = ((size_t)s * T + tc + tid) * Hd + h;
            sa[tid] = a[th];
            sb[tid] = b[th];
        }
        __syncthreads();
        for (int tt = 0; tt < nt; ++tt) {
            const int t = tc + tt;
            const size_t th = ((size_t)s * T + t) * Hd + h;
            const float at = sa[tt], bt = sb[tt];
            float kj[4], qj[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kj[e] = sk[tt][j0 + e];
                qj[e] = sq[tt][j0 + e];
            }
            // u = S k (row i of this half-wave: value row row0 + 8 i)
            float part[NR];
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                float u = S[i][0] * kj[0];
                u = fmaf(S[i][1], kj[1], u);
                u = fmaf(S[i][2], kj[2], u);
                part[i] = fmaf(S[i][3], kj[3], u);
            }
            const float u_mine = reduce_scatter<NR>(part, c32);   // row c32 / RW
            // S <- a S + (b v - a b u) k^T, then the partials of o = S q
            const int hbase = lane_base;
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                const float u = __shfl(u_mine, hbase + RW * i);
                const float wv = bt * (sv[tt][row0 + 8 * i] - at * u);
#pragma unroll
                for (int e = 0; e < 4; ++e) S[i][e] = fmaf(wv, kj[e], at * S[i][e]);
                float ov = S[i][0] * qj[0];
                ov = fmaf(S[i][1], qj[1], ov);
                ov = fmaf(S[i][2], qj[2], ov);
                part[i] = fmaf(S[i][3], qj[3], ov);
            }
            const float o_mine = reduce_scatter<NR>(part, c32);   // row c32 / RW
            if (write_o && c32 % RW == 0) o[th * kDv + row0 + 8 * (c32 / RW)] = f2bf(o_mine);
            if (record) {
                float* dst = rec + th * kDv * kDk;
#pragma unroll
                for (int i = 0; i < NR; ++i)
                    *reinterpret_cast<f32x4*>(dst + (row0 + 8 * i) * kDk + j0) = f32x4{S[i][0], S[i][1], S[i][2], S[i][3]};
            }
            if (Ls == t + 1) {
#pragma unroll
                for (int i = 0; i < NR; ++i)
                    *reinterpret_cast<f32x4*>(st + (row0 + 8 * i) * kDk + j0) = f32x4{S[i][0], S[i][1], S[i][2], S[i][3]};
            }
        }
    }
}

__global__ __launch_bounds__(256) void delta_restore_kernel(float* __restrict__ state,
                                                            const float* __restrict__ rec,
                                                            const int32_t* __restrict__ L, int T,
                                                            int Hd) {
    const int sh = blockIdx.x;
    const int s = sh / Hd, h = sh % Hd;
    int Ls = L[s];
    Ls = Ls < 0 ? 0 : (Ls > T ? T : Ls);
    if (Ls == 0) return;
    const f32x4* src = reinterpret_cast<const f32x4*>(rec + (((size_t)s * T + Ls - 1) * Hd + h) * kDv * kDk);
    f32x4* dst = reinterpret_cast<f32x4*>(state + (size_t)sh * kDv * kDk);
    for (int i = threadIdx.x; i < kDv * kDk / 4; i += 256) dst[i] = src[i];
}

}  // namespace sv

extern "C" {

int spec_delta_verify_rollback(int32_t mode, const spec_bf16* q, const spec_bf16* k,
                               const spec_bf16* v, const float* a, const float* b, float q_scale,
                               float* state, float* rec, const int32_t* L, int32_t B, int32_t T,
                               int32_t Hd, int32_t dk, int32_t dv, spec_bf16* o, void* stream) {
    using namespace sv;
    last_error().clear();
    if (mode < 1 || mode > 5) return fail(SPEC_EINVAL, "spec_delta_verify_rollback: mode=%d not in 1..5", mode);
    if (dk != kDk || dv != kDv) return fail(SPEC_EINVAL, "spec_delta_verify_rollback: dk=%d dv=%d (only 128 x 128)", dk, dv);
    if (B < 1 || Hd < 1 || T < 1 || T > 64) return fail(SPEC_EINVAL, "spec_delta_verify_rollback: B=%d Hd=%d T=%d", B, Hd, T);
    if ((long long)B * Hd * kDeltaSplit > 0x7fffffffLL) return fail(SPEC_ECAPACITY, "spec_delta_verify_rollback: B*Hd too large");
    const bool uses_rec = mode == SPEC_DELTA_RECORD || mode == SPEC_DELTA_ROLLBACK || mode == SPEC_DELTA_BOTH;
    const bool scans = mode != SPEC_DELTA_ROLLBACK;
    const bool needs_L = mode == SPEC_DELTA_ROLLBACK || mode == SPEC_DELTA_BOTH || mode == SPEC_DELTA_RESCAN;
    if (!state || (uses_rec && !rec)) return fail(SPEC_EINVAL, "spec_delta_verify_rollback: null state or rec");
    if (needs_L && !L) return fail(SPEC_EINVAL, "spec_delta_verify_rollback: L required in mode %d", mode);
    if (scans && (!q || !k || !v || !a || !b)) return fail(SPEC_EINVAL, "spec_delta_verify_rollback: null q/k/v/a/b");
    if (!aligned16(state) || (uses_rec && !aligned16(rec)))
        return fail(SPEC_EINVAL, "spec_delta_verify_rollback: state and rec must be 16-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    if (mode == SPEC_DELTA_ROLLBACK) {
        hipLaunchKernelGGL(delta_restore_kernel, dim3(B * Hd), dim3(256), 0, st, state, rec, L, T, Hd);
    } else {
        hipLaunchKernelGGL(delta_scan_kernel<kDeltaNR>, dim3(B * Hd * kDeltaSplit), dim3(256), 0, st, mode, q, k,
                           v, a, b, q_scale, state, rec, L, T, Hd, o);
    }
    SV_LAUNCH_CHECK("spec_delta_verify_rollback");
    return SPEC_OK;
}

}  // extern "C"
