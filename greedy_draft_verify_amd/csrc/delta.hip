// spec_delta_verify_rollback: Gated DeltaNet verify with per-token state recording,
// and rollback to the committed prefix.
//
// delta_scan_kernel: one workgroup (256 threads) per (sequence, head). The fp32
// state S [128][128] lives in registers for the whole scan: thread t owns the four
// key columns 4*(t % 32) .. +3 of the sixteen value rows (t / 32) + 8*i, so every
// row of S is spread over 32 lanes of one half-wave and each store instruction of
// a wave writes two whole rows (1 KB contiguous). Per token:
//   u  = S k_t                     (half-wave reduction)
//   S <- a_t S + (b_t v_t - a_t b_t u) k_t^T     (= a_t S (I - b_t k k^T) + b_t v k^T)
//   o_t = S (q_scale q_t)          (half-wave reduction)
// and S_t is written to the record (mode 1/3) and, at t = L, to the state (mode 3).
// Iteration t does the same arithmetic whatever T is, so S_L of a T-token scan
// equals the final state of an L-token scan bit for bit (memra linear_attn_verify_t:
// one scan over T tokens equals T chained one-token steps).
// delta_restore_kernel: mode 2, state <- rec[L - 1] (bit-exact copy).
#include "common.h"

namespace sv {

constexpr int kDk = 128, kDv = 128;

__device__ __forceinline__ float half_wave_sum(float x) {
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) x += __shfl_xor(x, d);
    return x;
}

__global__ __launch_bounds__(256) void delta_scan_kernel(
    int mode, const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const float* __restrict__ a, const float* __restrict__ b, float q_scale, float* state,
    float* __restrict__ rec, const int32_t* __restrict__ L, int T, int Hd, u16* __restrict__ o) {
    __shared__ float sk[kDk], sq[kDk], sv[kDv];
    const int sh = blockIdx.x;
    const int s = sh / Hd, h = sh % Hd;
    const int tid = threadIdx.x, c32 = tid % 32, rg = tid / 32;
    const int j0 = 4 * c32;
    constexpr int NR = kDv / 8;  // rows per thread
    float S[NR][4];
    float* st = state + (size_t)sh * kDv * kDk;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(st + (rg + 8 * i) * kDk + j0);
        S[i][0] = x[0];
        S[i][1] = x[1];
        S[i][2] = x[2];
        S[i][3] = x[3];
    }
    int Ls = -1;
    if (mode & SPEC_DELTA_ROLLBACK) {
        Ls = L[s];
        Ls = Ls < 0 ? 0 : (Ls > T ? T : Ls);
    }
    for (int t = 0; t < T; ++t) {
        const size_t th = ((size_t)s * T + t) * Hd + h;
        __syncthreads();
        if (tid < kDk) {
            sk[tid] = bf2f(k[th * kDk + tid]);
            sq[tid] = q_scale * bf2f(q[th * kDk + tid]);
        } else if (tid - kDk < kDv) {
            sv[tid - kDk] = bf2f(v[th * kDv + tid - kDk]);
        }
        __syncthreads();
        const float at = a[th], bt = b[th];
        float kj[4], qj[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kj[e] = sk[j0 + e];
            qj[e] = sq[j0 + e];
        }
        float orow = 0.f;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            float u = S[i][0] * kj[0];
            u = fmaf(S[i][1], kj[1], u);
            u = fmaf(S[i][2], kj[2], u);
            u = fmaf(S[i][3], kj[3], u);
            u = half_wave_sum(u);
            const float wv = bt * (sv[rg + 8 * i] - at * u);
#pragma unroll
            for (int e = 0; e < 4; ++e) S[i][e] = fmaf(wv, kj[e], at * S[i][e]);
            float ov = S[i][0] * qj[0];
            ov = fmaf(S[i][1], qj[1], ov);
            ov = fmaf(S[i][2], qj[2], ov);
            ov = fmaf(S[i][3], qj[3], ov);
            ov = half_wave_sum(ov);
            if (c32 == i) orow = ov;
        }
        if (o && c32 < NR) o[th * kDv + rg + 8 * c32] = f2bf(orow);
        if (mode & SPEC_DELTA_RECORD) {
            float* dst = rec + th * kDv * kDk;
#pragma unroll
            for (int i = 0; i < NR; ++i)
                *reinterpret_cast<f32x4*>(dst + (rg + 8 * i) * kDk + j0) = f32x4{S[i][0], S[i][1], S[i][2], S[i][3]};
        }
        if (Ls == t + 1) {
#pragma unroll
            for (int i = 0; i < NR; ++i)
                *reinterpret_cast<f32x4*>(st + (rg + 8 * i) * kDk + j0) = f32x4{S[i][0], S[i][1], S[i][2], S[i][3]};
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
    if (mode < 1 || mode > 3) return fail(SPEC_EINVAL, "spec_delta_verify_rollback: mode=%d not in 1..3", mode);
    if (dk != kDk || dv != kDv) return fail(SPEC_EINVAL, "spec_delta_verify_rollback: dk=%d dv=%d (only 128 x 128)", dk, dv);
    if (B < 1 || Hd < 1 || T < 1 || T > 64) return fail(SPEC_EINVAL, "spec_delta_verify_rollback: B=%d Hd=%d T=%d", B, Hd, T);
    if ((long long)B * Hd > 0x7fffffffLL) return fail(SPEC_ECAPACITY, "spec_delta_verify_rollback: B*Hd too large");
    if (!state || !rec) return fail(SPEC_EINVAL, "spec_delta_verify_rollback: null state or rec");
    if ((mode & SPEC_DELTA_ROLLBACK) && !L) return fail(SPEC_EINVAL, "spec_delta_verify_rollback: L required for rollback");
    if ((mode & SPEC_DELTA_RECORD) && (!q || !k || !v || !a || !b))
        return fail(SPEC_EINVAL, "spec_delta_verify_rollback: null q/k/v/a/b");
    if (!aligned16(state) || !aligned16(rec)) return fail(SPEC_EINVAL, "spec_delta_verify_rollback: state and rec must be 16-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    if (mode == SPEC_DELTA_ROLLBACK) {
        hipLaunchKernelGGL(delta_restore_kernel, dim3(B * Hd), dim3(256), 0, st, state, rec, L, T, Hd);
    } else {
        hipLaunchKernelGGL(delta_scan_kernel, dim3(B * Hd), dim3(256), 0, st, mode, q, k, v, a, b, q_scale,
                           state, rec, L, T, Hd, o);
    }
    SV_LAUNCH_CHECK("spec_delta_verify_rollback");
    return SPEC_OK;
}

}  // extern "C"
