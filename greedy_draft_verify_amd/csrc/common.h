// Shared helpers of the verify-step HIP library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/spec_verify.h"

namespace sv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr int kWave = 64;
constexpr int kPage = SPEC_PAGE_TOKENS;

// ---- numerics -------------------------------------------------------------
__device__ __forceinline__ float bf2f(u16 b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN (quiet bit set).
__device__ __forceinline__ u16 f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u16)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (u16)(u >> 16);
}

// 16x16x32 bf16 MFMA, fp32 accumulate (gfx950). Operand layout, lane l:
//   A[m][k]: m = l % 16, k = 8 * (l / 16) + 0..7
//   B[k][n]: n = l % 16, k = 8 * (l / 16) + 0..7
//   C[m][n]: n = l % 16, m = 4 * (l / 16) + 0..3
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// Non-temporal 16-byte load: for data a call reads once (streamed past the caches).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// Packs 8 fp32 values into bf16x8 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 pack8(const float* x) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (__bf16)x[i];
    return r;
}

// ---- counter-based random numbers ----------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as
// 1, 2, 3", SC 2011): 10 rounds of two 32x32->64 products whose halves are mixed
// with the other words and the key; the key advances by the Weyl constants after
// each round.
__device__ __forceinline__ uint4 philox10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
        const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

// Uniform in (0, 1) from the top 23 bits of a word (exact in fp32), and standard
// Gumbel noise -log(-log u) from it.
__device__ __forceinline__ float u01_23(uint32_t w) { return ((float)(w >> 9) + 0.5f) * (1.0f / 8388608.0f); }
__device__ __forceinline__ float gumbel(uint32_t w) { return -__logf(-__logf(u01_23(w))); }

// Counter layout of the sampling path: for a row with counter words (a, b)
//   Gumbel noise of vocabulary entry v:  ctr (v / 4, a, b, 0), word v % 4
//   acceptance uniform of the row:       ctr (0, a, b, 1), word 0
__device__ __forceinline__ float row_gumbel(uint32_t v, uint32_t a, uint32_t b, uint32_t k0, uint32_t k1) {
    const uint4 w = philox10(make_uint4(v >> 2, a, b, 0u), k0, k1);
    const uint32_t sel = v & 3u;
    return gumbel(sel == 0 ? w.x : sel == 1 ? w.y : sel == 2 ? w.z : w.w);
}

// ---- (value, index) maxima merged across workgroups ----------------------------
// The order: larger value first, then smaller index.
struct Best {
    float v;
    int i;
};

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

// (value, index) as one 64-bit key whose unsigned order is the order above: the high
// half maps the fp32 value monotonically (-0 taken as +0, like the comparison; a
// workgroup's best is never NaN), the low half is ~index. Key 0 is below every key.
__device__ __forceinline__ unsigned long long pack_best(Best b) {
    const uint32_t u = __float_as_uint(b.v == 0.f ? 0.f : b.v);
    const uint32_t hi = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)hi << 32) | (uint32_t)~(uint32_t)b.i;
}

__device__ __forceinline__ float unpack_value(unsigned long long key) {
    const uint32_t hi = (uint32_t)(key >> 32);
    return __uint_as_float((hi & 0x80000000u) ? (hi & 0x7fffffffu) : ~hi);
}

// ---- ragged row packing ------------------------------------------------------
// Exclusive prefix sums of (k_s + 1) over s (the packed row offsets) for B <= the
// size of s_off, by a block of NT threads: each thread sums a contiguous segment of
// sequences, a wave scans its segment sums by shuffles, and the wave totals are
// exchanged once through LDS (s_wsum and s_wbad hold NT / 64 entries). Returns
// whether the packing is defined: every k_s >= 0 and the sum equals R. Every
// thread must call it; it has two workgroup barriers.
template <int NT>
__device__ __forceinline__ bool block_row_offsets(const int32_t* __restrict__ k, int B, int R,
                                                  long long* s_wsum, int* s_wbad, int* s_off) {
    constexpr int NW = NT / kWave;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int per = (B + NT - 1) / NT;
    const int s0 = min(B, tid * per), s1 = min(B, s0 + per);
    long long local = 0;
    bool bad = false;
    for (int s = s0; s < s1; ++s) {
        const int ks = k[s];
        bad |= ks < 0;
        local += (long long)ks + 1;
    }
    long long incl = local;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const long long o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
    }
    const bool wave_bad = __ballot(bad) != 0;
    if (lane == kWave - 1) {
        s_wsum[wave] = incl;
        s_wbad[wave] = wave_bad;
    }
    __syncthreads();
    long long before = 0, total = 0;
    int any_bad = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const long long v = s_wsum[w];
        total += v;
        if (w < wave) before += v;
        any_bad |= s_wbad[w];
    }
    long long run = before + incl - local;
    for (int s = s0; s < s1; ++s) {
        s_off[s] = (int)run;
        if (s + 1 < s1) run += (long long)k[s] + 1;
    }
    __syncthreads();
    return total == (long long)R && !any_bad;
}

// Workgroups for a walk kernel with a wave per sequence: one per NT / 64 sequences,
// at most 64; each computes the row offsets itself (the scan reads only k).
inline int seq_grid(int B, int NT) {
    const int per = NT / kWave, n = (B + per - 1) / per;
    return n < 64 ? n : 64;
}

// ---- host error reporting ---------------------------------------------------
std::string& last_error();
int fail(int code, const char* fmt, ...);

// Acceptance limits, and the greedy step's fused argmax finalize + acceptance
// (accept.hip), launched by spec_lm_head_argmax_accept after the lm_head's pass that
// stores one key per (vocabulary workgroup, row) in rows of `stride` keys.
constexpr int kAcceptMaxB = 8192;
constexpr int kArgmaxAcceptMaxRows = 96;
int launch_argmax_accept(unsigned long long* key_rows, int n_vt, int stride, int R, int32_t* argmax, float* maxval,
                         const int32_t* drafts, int kmax, const int32_t* k, const int32_t* d2t, int n_draft_vocab,
                         int V, int B, const int32_t* pos_in, int32_t* pos_out, int32_t* accept_len, int32_t* n_emit,
                         int32_t* emit, int32_t* next_tok, int32_t* status, hipStream_t st);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define SV_LAUNCH_CHECK(what)                                                              \
    do {                                                                                   \
        hipError_t e_ = hipGetLastError();                                                 \
        if (e_ != hipSuccess) return ::sv::fail(SPEC_EHIP, "%s: %s", what, hipGetErrorString(e_)); \
    } while (0)

}  // namespace sv
