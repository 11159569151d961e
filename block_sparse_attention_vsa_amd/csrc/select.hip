// Forced + top-k / top-p key-block selection, one workgroup per (b, h, query
// block) row of pooled scores.
//
// USV page, Figure 2 caption: long-range sparse attention over key cubes picked
// by top-k cube selection, next to local attention; Sparse VideoGen2 page,
// Abstract: top-p dynamic budget control.
//
// Per row (256 threads, row held in LDS):
//  1. row max and Z = sum exp(s - max) by fixed-order tree reductions (fp32);
//  2. a 64-bit key per block: [forced:1][order-preserving score bits:32]
//     [~index:31], so one descending bitonic sort ranks forced blocks first,
//     then by score, then by lower index;
//  3. top-p: inclusive scan of exp(s - max) / Z over the ranked non-forced
//     candidates (per-thread serial segments + a scan of the segment totals);
//  4. kept blocks are flagged and compacted in ascending index order.
#include <math.h>

#include "vsa_internal.h"

namespace vsa {

constexpr int kSelMax = 4096;   // largest row (key blocks) a workgroup holds

__device__ __forceinline__ uint32_t order_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

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

__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ scores, int nqb, int nkb, int P2,
                                                     const uint8_t* __restrict__ forced, int k_max, float top_p,
                                                     int32_t* __restrict__ kv_idx, int32_t* __restrict__ kv_cnt) {
    __shared__ uint64_t keys[kSelMax];
    __shared__ float srow[kSelMax];
    __shared__ float red[256];
    __shared__ int flag_cnt[4];
    __shared__ float seg[256];
    __shared__ int cut;
    __shared__ uint8_t keep[kSelMax];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int qb = (int)(row % nqb);
    const float* s = scores + row * (int64_t)nkb;
    const uint8_t* f = forced ? forced + (int64_t)qb * nkb : nullptr;

    float mx = -INFINITY;
    int nf_local = 0;
    for (int j = tid; j < P2; j += 256) {
        if (j < nkb) {
            float v = s[j];
            bool fj = f && f[j];
            srow[j] = v;
            mx = fmaxf(mx, v);
            nf_local += fj;
            keys[j] = ((uint64_t)(fj ? 1u : 0u) << 63) | ((uint64_t)order_bits(v) << 31) |
                      (uint64_t)(0x7fffffffu - (uint32_t)j);
        } else {
            keys[j] = 0ull;                  // padding sorts last
        }
        if (j < nkb) keep[j] = 0;
    }
    mx = block_reduce(mx, red, true);
    const int nforced = (int)block_reduce((float)nf_local, red, false);
    float z_local = 0.f;
    for (int j = tid; j < nkb; j += 256) z_local += expf(srow[j] - mx);
    const float Z = block_reduce(z_local, red, false);

    // ---- descending bitonic sort of keys[0, P2) ----------------------------
    for (int size = 2; size <= P2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = tid; t < P2 / 2; t += 256) {
                int lo = 2 * t - (t & (stride - 1));
                int hi = lo + stride;
                bool desc = (lo & size) == 0;
                uint64_t a = keys[lo], b = keys[hi];
                if ((a < b) == desc) { keys[lo] = b; keys[hi] = a; }
            }
            __syncthreads();
        }
    }

    // ---- how many ranked entries to keep -----------------------------------
    int n_keep;
    if (nforced >= k_max) {
        n_keep = k_max;
    } else {
        const int n_cand = nkb - nforced;
        const int room = k_max - nforced;
        int r = n_cand;
        if (top_p < 1.f && n_cand > 0) {
            // inclusive scan of candidate probabilities in rank order
            const int per = (n_cand + 255) / 256;
            const int beg = min(tid * per, n_cand), end = min(beg + per, n_cand);
            float acc = 0.f;
            for (int i = beg; i < end; ++i) {
                int j = 0x7fffffff - (int)(keys[nforced + i] & 0x7fffffffull);
                acc += expf(srow[j] - mx) / Z;
            }
            seg[tid] = acc;
            if (tid == 0) cut = n_cand;
            __syncthreads();
            if (tid == 0) {                   // exclusive prefix of segment totals, in order
                float run = 0.f;
                for (int i = 0; i < 256; ++i) { float t = seg[i]; seg[i] = run; run += t; }
            }
            __syncthreads();
            float run = seg[tid];
            int first = n_cand;
            for (int i = beg; i < end; ++i) {
                int j = 0x7fffffff - (int)(keys[nforced + i] & 0x7fffffffull);
                run += expf(srow[j] - mx) / Z;
                if (run >= top_p) { first = i; break; }
            }
            if (first < n_cand) atomicMin(&cut, first);   // integer min: order-independent
            __syncthreads();
            r = max(min(cut + 1, n_cand), 1);
        }
        n_keep = nforced + min(r, room);
    }
    for (int i = tid; i < n_keep; i += 256) {
        int j = 0x7fffffff - (int)(keys[i] & 0x7fffffffull);
        keep[j] = 1;
    }
    __syncthreads();

    // ---- ascending compaction ---------------------------------------------
    const int lane = tid & 63, w = tid >> 6;
    int32_t* out = kv_idx + row * (int64_t)k_max;
    int base = 0;
    for (int r0 = 0; r0 < nkb; r0 += 256) {
        int j = r0 + tid;
        bool kj = j < nkb && keep[j];
        uint64_t bal = __ballot(kj);
        if (lane == 0) flag_cnt[w] = __popcll(bal);
        __syncthreads();
        int before = 0, total = 0;
        for (int i = 0; i < 4; ++i) { before += (i < w) ? flag_cnt[i] : 0; total += flag_cnt[i]; }
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
    int P2 = 2;
    while (P2 < nkb) P2 <<= 1;
    P2 = P2 < 512 ? 512 : P2;                  // every thread owns whole compare pairs
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)rows), dim3(256), 0, as_stream(stream), scores, nqb, nkb, P2,
                       forced, k_max, top_p, kv_idx, kv_cnt);
    return launch_status("vsa_select_topk");
}
