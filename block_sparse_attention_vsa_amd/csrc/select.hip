// Forced + top-k / top-p key-block selection, one workgroup per (b, h, query
// block) row of pooled scores.
//
// USV page, Figure 2 caption: long-range sparse attention over key cubes picked
// by top-k cube selection, next to local attention; Sparse VideoGen2 page,
// Abstract: top-p dynamic budget control.
//
// Each block gets a unique 64-bit rank key [forced:1][order-preserving score
// bits:32][0x7fffffff - index:31]: larger key = better rank (forced first, then
// higher score, then lower index). Per row (256 threads, row state in LDS):
//  1. K = min(k_max, nkb): an MSB-first radix select (8-bit digits, histogram
//     with integer LDS atomics, wave-level scans) finds the K-th largest key T;
//     the K best blocks are exactly the keys >= T.
//  2. Without top-p (or when forced blocks fill the cap) those K blocks are kept.
//     With top-p, the K winners are sorted (bitonic, in LDS) and the softmax mass
//     of the ranked non-forced candidates is accumulated in rank order until it
//     reaches top_p; softmax is over all nkb scores of the row (fp32, Z summed in
//     a fixed tree order).
//  3. Kept blocks are written in ascending index order.
#include <math.h>

#include "vsa_internal.h"

namespace vsa {

constexpr int kSelMax = 4096;   // largest row (key blocks) a workgroup holds

__device__ __forceinline__ uint32_t order_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float score_of_key(uint64_t key) {
    uint32_t o = (uint32_t)(key >> 31);
    uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
    return __uint_as_float(u);
}
__device__ __forceinline__ int index_of_key(uint64_t key) { return 0x7fffffff - (int)(key & 0x7fffffffull); }

// Fixed-order block reduction over 256 threads.
__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
    const int tid = threadIdx.x;
    red[tid] = v;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) red[tid] = is_max ? fmaxf(red[tid], red[tid + s]) : red[tid] + red[tid + s];
        __syncthreads();
    }
    float r = red[0];
    __syncthreads();
    return r;
}

// Inclusive scan of one value per thread over 256 threads (wave scans + totals).
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* wave_tot) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t t = __shfl_up(v, off);
        if (lane >= off) v += t;
    }
    if (lane == 63) wave_tot[w] = v;
    __syncthreads();
    for (int i = 0; i < w; ++i) v += wave_tot[i];
    __syncthreads();
    return v;
}

__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ scores, int nqb, int nkb, int P2K,
                                                     const uint8_t* __restrict__ forced, int k_max, float top_p,
                                                     int32_t* __restrict__ kv_idx, int32_t* __restrict__ kv_cnt) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
    uint64_t* keys = reinterpret_cast<uint64_t*>(dyn);                 // [nkb]
    uint64_t* tops = keys + nkb;                                       // [P2K]
    uint8_t* keep = reinterpret_cast<uint8_t*>(tops + P2K);            // [nkb]
    __shared__ float red[256];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t wave_tot[4];
    __shared__ uint64_t sel_prefix;
    __shared__ uint32_t sel_above, sel_bin;
    __shared__ int n_keep_s, n_top_s;

    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int qb = (int)(row % nqb);
    const float* s = scores + row * (int64_t)nkb;
    const uint8_t* f = forced ? forced + (int64_t)qb * nkb : nullptr;
    const bool use_p = top_p < 1.f;

    float mx = -INFINITY;
    int nf_local = 0;
    for (int j = tid; j < nkb; j += 256) {
        const float v = s[j];
        const bool fj = f && f[j];
        mx = fmaxf(mx, v);
        nf_local += fj;
        keys[j] = ((uint64_t)(fj ? 1u : 0u) << 63) | ((uint64_t)order_bits(v) << 31) |
                  (uint64_t)(0x7fffffffu - (uint32_t)j);
        keep[j] = 0;
    }
    const int nforced = (int)block_reduce((float)nf_local, red, false);
    const int K = min(k_max, nkb);

    // ---- 1. radix select of the K-th largest key -------------------------------
    uint64_t prefix = 0, pmask = 0;
    uint32_t krem = (uint32_t)K;
    for (int shift = 56; shift >= 0; shift -= 8) {
        hist[tid] = 0;
        __syncthreads();
        for (int j = tid; j < nkb; j += 256) {
            const uint64_t key = keys[j];
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        // thread t looks at digit 255 - t (descending), cum = count of digits >= it
        const uint32_t c = hist[255 - tid];
        const uint32_t cum = block_scan(c, wave_tot);
        if (cum >= krem && cum - c < krem) {
            sel_prefix = prefix | ((uint64_t)(255 - tid) << shift);
            sel_above = cum - c;
            sel_bin = c;
        }
        __syncthreads();
        prefix = sel_prefix;
        pmask |= (uint64_t)0xff << shift;
        krem -= sel_above;
        if (sel_bin == krem) break;      // every key in this bin is taken: the prefix is the threshold
        __syncthreads();
    }
    const uint64_t T = prefix;          // keys >= T are exactly the K best (low bits of T are zero past the stop)

    // ---- 2. how many of the ranked winners to keep -----------------------------
    if (!use_p || nforced >= k_max) {
        for (int j = tid; j < nkb; j += 256) keep[j] = keys[j] >= T;
    } else {
        mx = block_reduce(mx, red, true);
        float z_local = 0.f;
        for (int j = tid; j < nkb; j += 256) z_local += expf(s[j] - mx);
        const float Z = block_reduce(z_local, red, false);
        // compact the K winners, then sort them descending
        if (tid == 0) n_top_s = 0;
        for (int i = tid; i < P2K; i += 256) tops[i] = 0ull;
        __syncthreads();
        for (int j = tid; j < nkb; j += 256)
            if (keys[j] >= T) tops[atomicAdd(&n_top_s, 1)] = keys[j];   // order fixed by the sort below
        __syncthreads();
        for (int size = 2; size <= P2K; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int t = tid; t < P2K / 2; t += 256) {
                    const int lo = 2 * t - (t & (stride - 1));
                    const int hi = lo + stride;
                    const bool desc = (lo & size) == 0;
                    const uint64_t a = tops[lo], b = tops[hi];
                    if ((a < b) == desc) { tops[lo] = b; tops[hi] = a; }
                }
                __syncthreads();
            }
        }
        if (tid == 0) {
            // forced blocks (all of them, since nforced < k_max) lead the ranked list
            float cum = 0.f;
            int r = K - nforced;             // every ranked candidate that fits the cap
            for (int i = nforced; i < K; ++i) {
                cum += expf(score_of_key(tops[i]) - mx) / Z;
                if (cum >= top_p) { r = i - nforced + 1; break; }
            }
            n_keep_s = nforced + r;
        }
        __syncthreads();
        for (int i = tid; i < n_keep_s; i += 256) keep[index_of_key(tops[i])] = 1;
    }
    __syncthreads();

    // ---- 3. ascending compaction ------------------------------------------------
    const int lane = tid & 63, w = tid >> 6;
    int32_t* out = kv_idx + row * (int64_t)k_max;
    int base = 0;
    for (int r0 = 0; r0 < nkb; r0 += 256) {
        const int j = r0 + tid;
        const bool kj = j < nkb && keep[j];
        const uint64_t bal = __ballot(kj);
        if (lane == 0) wave_tot[w] = __popcll(bal);
        __syncthreads();
        int before = 0, total = 0;
        for (int i = 0; i < 4; ++i) { before += (i < w) ? (int)wave_tot[i] : 0; total += (int)wave_tot[i]; }
        if (kj) out[base + before + __popcll(bal & ((1ull << lane) - 1ull))] = j;
        base += total;
        __syncthreads();
    }
    if (tid == 0) kv_cnt[row] = base;
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
    int P2K = 512;                       // every thread owns whole compare pairs
    while (P2K < k_max) P2K <<= 1;
    if (top_p >= 1.f) P2K = 0;           // no sort without top-p
    const size_t shm = (size_t)nkb * 8 + (size_t)P2K * 8 + (size_t)((nkb + 15) & ~15);
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)rows), dim3(256), shm, as_stream(stream), scores, nqb, nkb, P2K,
                       forced, k_max, top_p, kv_idx, kv_cnt);
    return launch_status("vsa_select_topk");
}
