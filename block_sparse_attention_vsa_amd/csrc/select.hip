// Forced + top-k / top-p key-block selection, one wavefront per (b, h, query
// block) row of pooled scores.
//
// USV page, Figure 2 caption: long-range sparse attention over key cubes picked
// by top-k cube selection, next to local attention; Sparse VideoGen2 page,
// Abstract: top-p dynamic budget control.
//
// Each block gets a unique 64-bit rank key [forced:1][order-preserving score
// bits:32][0x7fffffff - index:31]: larger key = better rank (forced first, then
// higher score, then lower index). A row's keys live in the wave's registers
// (lane l holds blocks l, l + 64, ...); nothing needs a workgroup barrier:
//  1. K = min(k_max, nkb): an MSB-first radix select (8-bit digits, 256-bin
//     LDS histograms, a DPP wave scan over the digits) finds the K-th largest
//     key T; the K best blocks are exactly the keys >= T.
//  2. Without top-p (or when forced blocks fill the cap) those K blocks are kept.
//     With top-p, softmax is taken over all nkb scores of the row (fp32). The
//     ranked (non-forced) blocks are kept down to the first one at which the
//     mass ranked at or above it reaches top_p: a second digit walk whose bins
//     weigh mass instead of counting keys finds that key X, and the kept set is
//     the keys >= max(T, X) (the cap wins when X ranks below the K-th key).
//  3. Kept blocks are written in ascending index order (ballot + popcount).
#include <math.h>

#include "vsa_internal.h"

namespace vsa {

constexpr int kSelMax = 4096;   // largest row (key blocks) one wave holds in registers
constexpr int kCopies = 4;      // radix histograms per wave
constexpr int kStride = 257;    // words per histogram copy (odd: copies sit in different banks)
constexpr int kCopyWords = kCopies * kStride + 3 & ~3;   // 16-byte multiple
// LDS words per wave: count copies, weight copies, count totals, weight totals
constexpr int kLdsWords = 2 * kCopyWords + 2 * 256;

__device__ __forceinline__ uint32_t order_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float score_of_key(uint64_t key) {
    uint32_t o = (uint32_t)(key >> 31);
    uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
    return __uint_as_float(u);
}

// LDS operations of one wave complete in issue order; this keeps the compiler
// from moving them across the point and waits for those in flight.
__device__ __forceinline__ void wave_lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t o = __shfl_xor(v, off);
        v = o > v ? o : v;
    }
    return v;
}

// Inclusive scan over the 64 lanes on DPP: shifts by 1, 2, 4, 8 inside each
// row of 16 lanes, then the last lane of rows 0 and 2 is added to rows 1 and 3,
// and lane 31 to rows 2 and 3. Integer adds, so the order does not matter.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);
    return x;
}

// One digit of an MSB-first walk over the wave's keys. Among the keys with
// in[e] set whose bits above `shift + 8` equal `prefix`, bins by the 8-bit digit
// at `shift` and walks the bins from the top digit down, adding each bin's
// weight (its key count, or with WEIGHTED the sum of wt[e]). Returns the digit
// whose bin takes the running total to `need` (-1 if the total stays below),
// the total of the bins above it and the bin's key count.
template <int NPL, bool WEIGHTED>
__device__ __forceinline__ int digit_step(const uint64_t (&key)[NPL], const uint32_t (&wt)[NPL],
                                          const bool (&in)[NPL], uint64_t prefix, uint64_t pmask, int shift,
                                          uint32_t need, uint32_t* lds, int lane, uint32_t& above,
                                          uint32_t& bin_cnt) {
    uint32_t* cnt_h = lds;
    uint32_t* wt_h = lds + kCopyWords;
    uint32_t* cnt_t = lds + 2 * kCopyWords;
    uint32_t* wt_t = cnt_t + 256;
    constexpr int clear_words = WEIGHTED ? 2 * kCopyWords : kCopyWords;
    for (int i = 4 * lane; i < clear_words; i += 256) *reinterpret_cast<u32x4*>(lds + i) = u32x4{0u, 0u, 0u, 0u};
    wave_lds_fence();
    const int copy = (lane % kCopies) * kStride;
#pragma unroll
    for (int e = 0; e < NPL; ++e)
        if (in[e] && (key[e] & pmask) == prefix) {
            const int d = (int)((key[e] >> shift) & 255u);
            atomicAdd(&cnt_h[copy + d], 1u);
            if (WEIGHTED) atomicAdd(&wt_h[copy + d], wt[e]);
        }
    wave_lds_fence();
    // fold the copies: lane t sums digits t, t + 64, t + 128, t + 192
#pragma unroll 1
    for (int q = 0; q < 4; ++q) {
        const int d = lane + 64 * q;
        uint32_t c = 0, w = 0;
#pragma unroll
        for (int k = 0; k < kCopies; ++k) {
            c += cnt_h[k * kStride + d];
            if (WEIGHTED) w += wt_h[k * kStride + d];
        }
        cnt_t[d] = c;
        if (WEIGHTED) wt_t[d] = w;
    }
    wave_lds_fence();
    // lane t takes digits 255 - 4t ... 252 - 4t: lane order is descending
    const u32x4 cv = *reinterpret_cast<const u32x4*>(cnt_t + 252 - 4 * lane);
    const u32x4 wv = WEIGHTED ? *reinterpret_cast<const u32x4*>(wt_t + 252 - 4 * lane) : cv;
    const uint32_t tot = wv[0] + wv[1] + wv[2] + wv[3];
    const uint32_t incl = wave_incl_scan(tot);
    const bool hit = incl - tot < need && incl >= need;      // at most one lane
    const uint64_t bal = __ballot(hit);
    wave_lds_fence();
    if (!bal) return -1;
    const int src = __ffsll((unsigned long long)bal) - 1;
    // inside the lane: digits 255 - 4t - q are elements 3 - q of the vectors
    uint32_t run = incl - tot, ab = 0, bc = 0;
    int q_hit = 0;
    bool done = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (!done && run + wv[3 - q] >= need) { done = true; q_hit = q; ab = run; bc = cv[3 - q]; }
        else if (!done) run += wv[3 - q];
    }
    above = (uint32_t)__shfl((int)ab, src);
    bin_cnt = (uint32_t)__shfl((int)bc, src);
    return 255 - 4 * src - __shfl(q_hit, src);
}

// NPL keys per lane: rows of up to 64 NPL key blocks.
template <int NPL>
__global__ __launch_bounds__(64) void select_kernel(const float* __restrict__ scores, int nqb, int nkb,
                                                    const uint8_t* __restrict__ forced, int k_max, float top_p,
                                                    int32_t* __restrict__ kv_idx, int32_t* __restrict__ kv_cnt) {
    __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsWords];
    const int lane = threadIdx.x;
    const uint64_t lt = (1ull << lane) - 1ull;
    const int64_t row = blockIdx.x;
    const int qb = (int)(row % nqb);
    const float* s = scores + row * (int64_t)nkb;
    const uint8_t* f = forced ? forced + (int64_t)qb * nkb : nullptr;

    uint64_t key[NPL];
    bool in[NPL];
    uint32_t wt[NPL];
    float mx = -INFINITY;
    int nf = 0;
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
        const int j = lane + 64 * e;
        key[e] = 0ull;                                   // below every real key
        in[e] = j < nkb;
        wt[e] = 1u;
        if (j < nkb) {
            const float v = s[j];
            const bool fj = f && f[j];
            mx = fmaxf(mx, v);
            nf += fj;
            key[e] = ((uint64_t)(fj ? 1u : 0u) << 63) | ((uint64_t)order_bits(v) << 31) |
                     (uint64_t)(0x7fffffffu - (uint32_t)j);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) nf += __shfl_xor(nf, off);
    const int nforced = nf;
    const int K = min(k_max, nkb);

    // ---- 1. radix select of the K-th largest key -------------------------------
    uint64_t prefix = 0, pmask = 0;
    uint32_t krem = (uint32_t)K;
#pragma unroll 1
    for (int shift = 56; shift >= 0; shift -= 8) {
        uint32_t above = 0, bc = 0;
        const int d = digit_step<NPL, false>(key, wt, in, prefix, pmask, shift, krem, lds, lane, above, bc);
        prefix |= (uint64_t)d << shift;      // d >= 0: the row holds at least krem matching keys
        pmask |= (uint64_t)0xff << shift;
        krem -= above;
        if (bc == krem) break;               // every key in this bin is taken: the prefix is the threshold
    }
    const uint64_t T = prefix;               // keys >= T are exactly the K best (low bits of T are zero past the stop)

    // ---- 2. how many of the ranked winners to keep -----------------------------
    uint64_t T2 = T;
    if (top_p < 1.f && nforced < k_max) {
        mx = wave_max(mx);
        float z = 0.f;
#pragma unroll
        for (int e = 0; e < NPL; ++e)
            if (lane + 64 * e < nkb) z += expf(score_of_key(key[e]) - mx);
        const float Z = wave_sum(z);
        // Softmax masses of the ranked (non-forced) candidates as fixed-point
        // integers in units of 2^-31: their sums do not depend on the order of
        // the additions, so the walk below is deterministic.
        constexpr float kFix = 2147483648.f;
#pragma unroll
        for (int e = 0; e < NPL; ++e) {
            const float pm = expf(score_of_key(key[e]) - mx) / Z * kFix;
            // a NaN mass (a row of -inf or NaN scores) weighs nothing
            wt[e] = (lane + 64 * e < nkb && !(key[e] >> 63) && pm > 0.f) ? (uint32_t)fminf(pm, kFix) : 0u;
            in[e] = wt[e] != 0u;
        }
        uint32_t mrem = (uint32_t)(top_p * kFix);
        uint64_t xp = 0, xmask = 0;
        bool reached = true;
#pragma unroll 1
        for (int shift = 56; shift >= 0; shift -= 8) {
            uint32_t above = 0, bc = 0;
            const int d = digit_step<NPL, true>(key, wt, in, xp, xmask, shift, mrem, lds, lane, above, bc);
            if (d < 0) { reached = false; break; }   // the ranked mass never reaches top_p
            xp |= (uint64_t)d << shift;
            xmask |= (uint64_t)0xff << shift;
            mrem -= above;
            if (bc == 1) {                           // one key left in the bin: it is the crossing key
                uint64_t x = 0;
#pragma unroll
                for (int e = 0; e < NPL; ++e)
                    if (in[e] && (key[e] & xmask) == xp) x = key[e];
                xp = wave_max_u64(x);
                break;
            }
        }
        if (reached && xp > T2) T2 = xp;             // past the cap (xp < T) every winner stays
    }

    // ---- 3. ascending compaction ------------------------------------------------
    int32_t* out = kv_idx + row * (int64_t)k_max;
    int base = 0;
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
        const int j = lane + 64 * e;
        const bool kj = j < nkb && key[e] >= T2;
        const uint64_t bal = __ballot(kj);
        if (kj) out[base + __popcll(bal & lt)] = j;
        base += __popcll(bal);
    }
    if (lane == 0) kv_cnt[row] = base;
}

}  // namespace vsa

using namespace vsa;

extern "C" int vsa_select_topk(const float* scores, int B, int H, int nqb, int nkb, const uint8_t* forced, int k_max,
                               float top_p, int32_t* kv_idx, int32_t* kv_cnt, void* stream) {
    if (!scores || !kv_idx || !kv_cnt) return fail(VSA_ERR_INVALID, "vsa_select_topk: null pointer");
    if (B <= 0 || H <= 0 || nqb <= 0 || nkb <= 0) return fail(VSA_ERR_INVALID, "vsa_select_topk: sizes must be positive");
    if (nkb > kSelMax) return fail(VSA_ERR_UNSUPPORTED, "vsa_select_topk: nkb must be <= %d", kSelMax);
    if (k_max < 1 || k_max > nkb) return fail(VSA_ERR_INVALID, "vsa_select_topk: k_max must be in [1, nkb]");
    if (!(top_p > 0.f) || !(top_p <= 1.f)) return fail(VSA_ERR_INVALID, "vsa_select_topk: top_p must be in (0, 1]");
    int64_t rows = (int64_t)B * H * nqb;
    if (rows >= (1ll << 31)) return fail(VSA_ERR_INVALID, "vsa_select_topk: too many rows");
    const int npl = (nkb + 63) / 64;
    const dim3 grid((unsigned)rows);
    hipStream_t st = as_stream(stream);
#define VSA_SELECT_LAUNCH(NPL)                                                                                    \
    hipLaunchKernelGGL(select_kernel<NPL>, grid, dim3(64), 0, st, scores, nqb, nkb, forced, k_max, top_p, kv_idx, \
                       kv_cnt)
    if (npl <= 4) VSA_SELECT_LAUNCH(4);
    else if (npl <= 8) VSA_SELECT_LAUNCH(8);
    else if (npl <= 12) VSA_SELECT_LAUNCH(12);
    else if (npl <= 16) VSA_SELECT_LAUNCH(16);
    else if (npl <= 24) VSA_SELECT_LAUNCH(24);
    else if (npl <= 32) VSA_SELECT_LAUNCH(32);
    else if (npl <= 48) VSA_SELECT_LAUNCH(48);
    else VSA_SELECT_LAUNCH(64);
#undef VSA_SELECT_LAUNCH
    return launch_status("vsa_select_topk");
}
