// Semantic-aware permutation on gfx950: k-means of the tokens of every head,
// the stable cluster-major order, row gathers, and size-weighted cluster scores.
//
// Sparse VideoGen2 page, Abstract: tokens are clustered by semantic similarity
// with k-means and reordered so that each cluster is contiguous; a cluster's
// mean represents it when the critical clusters are chosen under a top-p budget.
//
//  * Seeds: the tokens at positions floor(c N / C).
//  * Assignment: token x goes to argmin_c ||m_c||^2 - 2 <x, m_c> with the
//    centroids m rounded to bf16 (the precision of the tokens), ties to the lower
//    index. One workgroup per 128 tokens; the bf16 centroids stream through LDS
//    in 64-row sub-tiles by DMA and the products run on v_mfma_f32_32x32x16_bf16
//    (the accumulator gives each lane one token and 16 centroids per 32-row half).
//  * Update: centroid = mean of its members, an empty cluster keeps its value.
//    Each iteration first puts the tokens in the stable cluster-major order of
//    the new labels (integer work, below), so every cluster's members are one
//    contiguous range; a workgroup per cluster sums its range in 32 fixed
//    streams added in stream order. No floating-point atomics, so the result
//    does not depend on scheduling, and clusters of any size or spatial spread
//    cost the same per member.
//  * Order: stable counting sort by cluster. Chunks of 256 tokens count their
//    clusters, a per-cluster scan over chunks gives each chunk's first slot, and
//    every token's rank among equal clusters in its chunk comes from wave ballots.
#include <math.h>

#include "mfma_tile.h"

namespace vsa {

constexpr int kKmD = 128;                 // token width handled by the k-means kernels
constexpr int kOrdChunk = 256;            // tokens per counting-sort chunk (4 waves)
constexpr int kOrdMaxC = 1024;            // clusters per head for the order kernels

struct KmArgs {
    const uint16_t* x;        // [BH, N, 128] bf16
    float* cent;              // [BH, C, 128] fp32 (in: previous, out: updated)
    uint16_t* cent_bf;        // [BH, C, 128] bf16 rounding of cent
    float* cnorm;             // [BH, C] squared norm of cent_bf, fp32
    int32_t* labels;          // [BH, N]
    int32_t* counts;          // [BH, C]
    int32_t N, C, BH;
};

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Writes centroid row (lane's two channels v0, v1) in fp32 and bf16 and returns
// the lane's part of the bf16 row's squared norm.
__device__ __forceinline__ float put_centroid(const KmArgs& a, int64_t row, int lane, float v0, float v1) {
    const uint16_t b0 = f32_to_bf16_bits(v0), b1 = f32_to_bf16_bits(v1);
    *reinterpret_cast<float2*>(a.cent + row * kKmD + 2 * lane) = make_float2(v0, v1);
    *reinterpret_cast<uint32_t*>(a.cent_bf + row * kKmD + 2 * lane) = (uint32_t)b0 | ((uint32_t)b1 << 16);
    const float r0 = bf16_bits_to_f32(b0), r1 = bf16_bits_to_f32(b1);
    return fmaf(r0, r0, r1 * r1);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// ---- seeds: one wave per (bh, c) -----------------------------------------------
__global__ __launch_bounds__(256) void km_seed_kernel(KmArgs a) {
    const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (g >= (int64_t)a.BH * a.C) return;
    const int64_t bh = g / a.C;
    const int c = (int)(g - bh * a.C);
    const int64_t n = (int64_t)c * a.N / a.C;
    const uint32_t pr = *reinterpret_cast<const uint32_t*>(a.x + (bh * a.N + n) * kKmD + 2 * lane);
    const float nrm = wave_sum(put_centroid(a, g, lane, bf16_bits_to_f32(pr & 0xffffu), bf16_bits_to_f32(pr >> 16)));
    if (lane == 0) a.cnorm[g] = nrm;
}

// ---- assignment: one workgroup per (bh, 128 tokens) -----------------------------
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void km_assign_kernel(KmArgs a,
                                                                                                  int tiles) {
    constexpr int KT = 64, NST = 2, SUBB = KT * kKmD * 2, WAVES = 4;
    __shared__ __attribute__((aligned(1024))) uint8_t c0[SUBB];
    __shared__ __attribute__((aligned(1024))) uint8_t c1[SUBB];
    __shared__ __attribute__((aligned(16))) float n0[KT];
    __shared__ __attribute__((aligned(16))) float n1[KT];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, half = lane >> 5;
    const int item = xcd_remap(blockIdx.x, a.BH * tiles);
    const int bh = item / tiles, tile = item - bh * tiles;
    const int t = tile * 128 + 32 * w + l32;
    const bool ok = t < a.N;
    bf16x8 xf[8];
    load_q_frag<kKmD>(xf, a.x + ((int64_t)bh * a.N + t) * kKmD, ok, half);

    const SubTileDma<WAVES, kVSwz4, KT> dma(lane, w);
    const uint16_t* cb = a.cent_bf + (int64_t)bh * a.C * kKmD;
    const float* cn = a.cnorm + (int64_t)bh * a.C;
    const int cbytes = a.C * kKmD * 2, nbytes = a.C * 4;
    auto issue = [&](int i, uint8_t* cd, float* nd) {
        const int base = i * KT * 256;
#pragma unroll
        for (int u = 0; u < SubTileDma<WAVES, kVSwz4, KT>::IPW; ++u)
            dma16(cb, cbytes, cd + (w + WAVES * u) * 1024, base + dma.voff_k(u), 0);
        if (w == 0 && lane < KT / 4) dma16(cn, nbytes, nd, i * KT * 4 + lane * 16, 0);
    };
    float best = INFINITY;
    int best_c = 0;
    auto compute = [&](int i, const uint8_t* ct, const float* nt) __attribute__((always_inline)) {
        f32x16 s[NST];
        sub_scores<NST>(s, ct, xf, l32, half);
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 n4 = *reinterpret_cast<const f32x4*>(nt + acc_key(st, 4 * j, half));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = i * KT + acc_key(st, 4 * j + e, half);   // ascending within the lane
                    const float d = fmaf(-2.f, s[st][4 * j + e], n4[e]);
                    if (c < a.C && d < best) {
                        best = d;
                        best_c = c;
                    }
                }
            }
    };
    const int n_sub = (a.C + KT - 1) / KT;
    issue(0, c0, n0);
    for (int i = 0; i < n_sub; i += 2) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (i + 1 < n_sub) issue(i + 1, c1, n1);
        compute(i, c0, n0);
        if (i + 1 < n_sub) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (i + 2 < n_sub) issue(i + 2, c0, n0);
            compute(i + 1, c1, n1);
        }
    }
    // lanes l and l ^ 32 hold the same token with interleaved centroid sets
    auto rd = __builtin_amdgcn_permlane32_swap(__float_as_uint(best), __float_as_uint(best), false, false);
    auto rc = __builtin_amdgcn_permlane32_swap((uint32_t)best_c, (uint32_t)best_c, false, false);
    const float d_lo = __uint_as_float(rd[0]), d_hi = __uint_as_float(rd[1]);
    const int c_lo = (int)rc[0], c_hi = (int)rc[1];
    const int pick = (d_hi < d_lo || (d_hi == d_lo && c_hi < c_lo)) ? c_hi : c_lo;
    if (ok && half == 0) a.labels[(int64_t)bh * a.N + t] = pick;
}

// ---- update: one workgroup per (bh, cluster) over its members ------------------
// The members of cluster c are positions [off[c], off[c + 1]) of the stable
// cluster-major order of the current labels. 32 streams (4 per wave, 16 lanes x
// 8 channels each) take every 32nd member, 16 members per stream and pass; the
// streams' partial sums are added in stream order: a fixed order, independent
// of scheduling.
__global__ __launch_bounds__(512) void km_update_kernel(KmArgs a, const int32_t* perm, const int32_t* off) {
    constexpr int STREAMS = 32, UNROLL = 16;
    __shared__ float part[STREAMS][kKmD];
    __shared__ float mb[kKmD];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int item = xcd_remap(blockIdx.x, a.BH * a.C);
    const int64_t bh = item / a.C;
    const int c = item - (int)bh * a.C;
    const int32_t* ofs = off + bh * (a.C + 1);
    const int m0 = ofs[c], m1 = ofs[c + 1];
    const int stream = 4 * w + (lane >> 4), chunk = lane & 15;     // channels 8 chunk .. 8 chunk + 7
    const int32_t* ph = perm + bh * a.N;
    const uint16_t* xh = a.x + bh * a.N * kKmD;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    // the member indices of the next pass are loaded before this pass's rows, so
    // a large cluster waits on one load latency per pass instead of two
    int tok_next[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) tok_next[u] = m0 + stream < m1 ? ph[min(m0 + stream + STREAMS * u, m1 - 1)] : 0;
    for (int p0 = m0 + stream; p0 < m1; p0 += STREAMS * UNROLL) {
        int tok[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) tok[u] = tok_next[u];
        const int pn = p0 + STREAMS * UNROLL;
        if (pn < m1) {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) tok_next[u] = ph[min(pn + STREAMS * u, m1 - 1)];
        }
        u32x4 row[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            row[u] = *reinterpret_cast<const u32x4*>(xh + (int64_t)tok[u] * kKmD + 8 * chunk);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            if (p0 + STREAMS * u >= m1) break;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += bf16_bits_to_f32(row[u][e] & 0xffffu);
                acc[2 * e + 1] += bf16_bits_to_f32(row[u][e] >> 16);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[stream][8 * chunk + e] = acc[e];
    __syncthreads();
    const int64_t row = bh * a.C + c;
    const int n = m1 - m0;
    if (tid < kKmD) {
        float sum = 0.f;
#pragma unroll
        for (int u = 0; u < STREAMS; ++u) sum += part[u][tid];
        mb[tid] = n > 0 ? sum / (float)n : a.cent[row * kKmD + tid];
        if (tid == 0) a.counts[row] = n;
    }
    __syncthreads();
    if (w == 0) {
        const float nrm = wave_sum(put_centroid(a, row, lane, mb[2 * lane], mb[2 * lane + 1]));
        if (lane == 0) a.cnorm[row] = nrm;
    }
}

// ---- stable cluster-major order -------------------------------------------------
struct OrdArgs {
    const int32_t* labels;    // [BH, N]
    int32_t* perm;            // [BH, N]: perm[p] = token at position p
    int32_t* offsets;         // [BH, C + 1]: cluster sizes, then their exclusive prefix
    int32_t* chunk;           // [BH, nch, C]: counts, then each chunk's first slot within its cluster
    int32_t N, C, BH, nch;
};

// per-chunk cluster counts (LDS integer histogram; counts do not depend on order)
__global__ __launch_bounds__(kOrdChunk) void ord_count_kernel(OrdArgs a) {
    __shared__ int hist[kOrdMaxC];
    const int64_t bh = blockIdx.x / a.nch;
    const int ch = (int)(blockIdx.x - bh * a.nch);
    for (int c = threadIdx.x; c < a.C; c += kOrdChunk) hist[c] = 0;
    __syncthreads();
    const int t = ch * kOrdChunk + threadIdx.x;
    if (t < a.N) {
        const int l = a.labels[bh * a.N + t];
        if ((unsigned)l < (unsigned)a.C) atomicAdd(&hist[l], 1);
    }
    __syncthreads();
    int32_t* out = a.chunk + (bh * a.nch + ch) * a.C;
    for (int c = threadIdx.x; c < a.C; c += kOrdChunk) out[c] = hist[c];
}

// each chunk's first slot within its cluster, and the cluster sizes: one wave
// per (bh, c), scanning the chunks
__global__ __launch_bounds__(256) void ord_scan_kernel(OrdArgs a) {
    const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (g >= (int64_t)a.BH * a.C) return;
    const int64_t bh = g / a.C;
    const int c = (int)(g - bh * a.C);
    int run = 0;
    for (int c0 = 0; c0 < a.nch; c0 += 64) {
        const int ch = c0 + lane;
        int32_t* p = a.chunk + (bh * a.nch + ch) * a.C + c;
        const int v = ch < a.nch ? *p : 0;
        int x = v;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(x, d);
            if (lane >= d) x += y;
        }
        if (ch < a.nch) *p = run + x - v;
        run += __shfl(x, 63);
    }
    if (lane == 0) a.offsets[bh * (a.C + 1) + c] = run;
}

// cluster sizes -> offsets, in place: one wave per bh (exclusive scan)
__global__ __launch_bounds__(64) void ord_offsets_kernel(OrdArgs a) {
    const int64_t bh = blockIdx.x;
    const int lane = threadIdx.x;
    int32_t* off = a.offsets + bh * (a.C + 1);
    int run = 0;
    for (int c0 = 0; c0 < a.C; c0 += 64) {
        const int c = c0 + lane;
        const int v = c < a.C ? off[c] : 0;
        int x = v;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(x, d);
            if (lane >= d) x += y;
        }
        if (c < a.C) off[c] = run + x - v;
        run += __shfl(x, 63);
    }
    if (lane == 0) off[a.C] = run;
}

// scatter: position = cluster offset + the chunk's first slot + rank in the chunk
__global__ __launch_bounds__(kOrdChunk) void ord_scatter_kernel(OrdArgs a) {
    constexpr int WAVES = kOrdChunk / 64;
    __shared__ int wcnt[WAVES][kOrdMaxC];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t bh = blockIdx.x / a.nch;
    const int ch = (int)(blockIdx.x - bh * a.nch);
    for (int i = threadIdx.x; i < WAVES * a.C; i += kOrdChunk) wcnt[i / a.C][i % a.C] = 0;
    __syncthreads();
    const int t = ch * kOrdChunk + threadIdx.x;
    const int l = t < a.N ? a.labels[bh * a.N + t] : -1;
    const bool ok = (unsigned)l < (unsigned)a.C;
    // rank among the lower lanes of this wave holding the same cluster
    int rank = 0;
    uint64_t todo = __ballot(ok);
    while (todo) {
        const int leader = __builtin_ctzll(todo);
        const int c = __builtin_amdgcn_readlane(l, leader);
        const uint64_t same = __ballot(ok && l == c);
        if (ok && l == c) rank = __popcll(same & ((1ull << lane) - 1ull));
        if (lane == leader) wcnt[w][c] = __popcll(same);
        todo &= ~same;
    }
    __syncthreads();
    if (ok) {
        int before = 0;
        for (int u = 0; u < w; ++u) before += wcnt[u][l];
        const int pos = a.offsets[bh * (a.C + 1) + l] + a.chunk[(bh * a.nch + ch) * a.C + l] + before + rank;
        if ((unsigned)pos < (unsigned)a.N) a.perm[bh * a.N + pos] = t;
    }
}

static void launch_order(const OrdArgs& a, hipStream_t s) {
    const int64_t BH = a.BH;
    hipLaunchKernelGGL(ord_count_kernel, dim3((unsigned)(BH * a.nch)), dim3(kOrdChunk), 0, s, a);
    hipLaunchKernelGGL(ord_scan_kernel, dim3((unsigned)((BH * a.C + 3) / 4)), dim3(256), 0, s, a);
    hipLaunchKernelGGL(ord_offsets_kernel, dim3((unsigned)BH), dim3(64), 0, s, a);
    hipLaunchKernelGGL(ord_scatter_kernel, dim3((unsigned)(BH * a.nch)), dim3(kOrdChunk), 0, s, a);
}

// ---- row gather / scatter -------------------------------------------------------
// forward: dst[bh, r] = src[bh, perm[bh, r]]; inverse: dst[bh, perm[bh, r]] = src[bh, r]
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* src, uint8_t* dst, const int32_t* perm,
                                                          int N, int row_bytes, int64_t rows, int inverse) {
    const int lpr = row_bytes / 16;                       // lanes per row
    const int64_t g = ((int64_t)blockIdx.x * 256 + threadIdx.x) / lpr;
    const int sub = (threadIdx.x % lpr) * 16;
    if (g >= rows) return;
    const int64_t bh = g / N;
    const int p = perm[g];
    if ((unsigned)p >= (unsigned)N) return;               // malformed entry: leave the row alone
    const int64_t from = inverse ? g : bh * N + p;
    const int64_t to = inverse ? bh * N + p : g;
    *reinterpret_cast<u32x4*>(dst + to * row_bytes + sub) = *reinterpret_cast<const u32x4*>(src + from * row_bytes + sub);
}

// ---- size-weighted cluster scores: one workgroup per (bh, query cluster) --------
__global__ __launch_bounds__(256) void cluster_scores_kernel(const float* cq, const float* ck, const int32_t* kcnt,
                                                             int Cq, int Ck, int D, float scale, float* scores) {
    __shared__ float qrow[128];
    const int64_t g = blockIdx.x;                          // bh * Cq + a
    const int64_t bh = g / Cq;
    if (threadIdx.x < D) qrow[threadIdx.x] = cq[g * D + threadIdx.x];
    __syncthreads();
    for (int b = threadIdx.x; b < Ck; b += 256) {
        const float* kr = ck + (bh * Ck + b) * D;
        float s = 0.f;
        for (int d = 0; d < D; d += 4) {
            const float4 k4 = *reinterpret_cast<const float4*>(kr + d);
            s = fmaf(qrow[d], k4.x, s);
            s = fmaf(qrow[d + 1], k4.y, s);
            s = fmaf(qrow[d + 2], k4.z, s);
            s = fmaf(qrow[d + 3], k4.w, s);
        }
        const int n = kcnt[bh * Ck + b];
        scores[g * Ck + b] = n > 0 ? fmaf(scale, s, logf((float)n)) : -INFINITY;
    }
}

}  // namespace vsa

using namespace vsa;

static size_t km_al(size_t x) { return (x + 255) & ~(size_t)255; }

struct KmPlan {
    size_t off_bf, off_norm, off_perm, off_ofs, off_chunk, total;
};

static KmPlan km_plan(int64_t BH, int N, int C) {
    KmPlan p;
    const int64_t nch = (N + kOrdChunk - 1) / kOrdChunk;
    p.off_bf = 0;
    p.off_norm = km_al((size_t)BH * C * kKmD * 2);
    p.off_perm = p.off_norm + km_al((size_t)BH * C * 4);
    p.off_ofs = p.off_perm + km_al((size_t)BH * N * 4);
    p.off_chunk = p.off_ofs + km_al((size_t)BH * (C + 1) * 4);
    p.total = p.off_chunk + km_al((size_t)BH * nch * C * 4);
    return p;
}

extern "C" size_t vsa_kmeans_workspace_bytes(int B, int H, int N, int C, int D) {
    if (B <= 0 || H <= 0 || N <= 0 || C <= 0 || D != kKmD) return 0;
    return km_plan((int64_t)B * H, N, C).total;
}

extern "C" int vsa_kmeans(const void* x, int B, int H, int N, int D, int dtype, int C, int iters, float* centroids,
                          int32_t* labels, int32_t* counts, void* workspace, size_t ws_bytes, void* stream) {
    const char* fn = "vsa_kmeans";
    if (!x || !centroids || !labels || !counts) return fail(VSA_ERR_INVALID, "%s: null tensor", fn);
    if (!aligned16(x) || !aligned16(centroids)) return fail(VSA_ERR_INVALID, "%s: x and centroids must be 16-byte aligned", fn);
    if (B <= 0 || H <= 0 || N <= 0) return fail(VSA_ERR_INVALID, "%s: B, H, N must be positive", fn);
    if (C < 1 || C > N) return fail(VSA_ERR_INVALID, "%s: need 1 <= C <= N (C = %d, N = %d)", fn, C, N);
    if (C > kOrdMaxC) return fail(VSA_ERR_UNSUPPORTED, "%s: at most %d clusters", fn, kOrdMaxC);
    if (iters < 1) return fail(VSA_ERR_INVALID, "%s: iters must be >= 1", fn);
    if (dtype != VSA_BF16 || D != kKmD) return fail(VSA_ERR_UNSUPPORTED, "%s: needs bf16 with D = %d", fn, kKmD);
    const int64_t BH = (int64_t)B * H;
    const int64_t nch = (N + kOrdChunk - 1) / kOrdChunk;
    if (BH * N >= (1ll << 31) || (int64_t)N * kKmD * 2 >= (1ll << 31) || BH * C >= (1ll << 31) ||
        BH * nch * C >= (1ll << 31))
        return fail(VSA_ERR_INVALID, "%s: problem too large", fn);
    const KmPlan pl = km_plan(BH, N, C);
    if (!workspace || ws_bytes < pl.total)
        return fail(VSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, pl.total, ws_bytes);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    KmArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.cent = centroids;
    a.cent_bf = reinterpret_cast<uint16_t*>(ws + pl.off_bf);
    a.cnorm = reinterpret_cast<float*>(ws + pl.off_norm);
    a.labels = labels;
    a.counts = counts;
    a.N = N; a.C = C; a.BH = (int32_t)BH;
    OrdArgs o{};
    o.labels = labels;
    o.perm = reinterpret_cast<int32_t*>(ws + pl.off_perm);
    o.offsets = reinterpret_cast<int32_t*>(ws + pl.off_ofs);
    o.chunk = reinterpret_cast<int32_t*>(ws + pl.off_chunk);
    o.N = N; o.C = C; o.BH = (int32_t)BH; o.nch = (int32_t)nch;
    hipStream_t s = as_stream(stream);
    hipLaunchKernelGGL(km_seed_kernel, dim3((unsigned)((BH * C + 3) / 4)), dim3(256), 0, s, a);
    int st = launch_status("vsa_kmeans (seeds)");
    if (st) return st;
    const int tiles = (N + 127) / 128;
    for (int it = 0; it < iters; ++it) {
        hipLaunchKernelGGL(km_assign_kernel, dim3((unsigned)(BH * tiles)), dim3(256), 0, s, a, tiles);
        launch_order(o, s);
        hipLaunchKernelGGL(km_update_kernel, dim3((unsigned)(BH * C)), dim3(512), 0, s, a, o.perm, o.offsets);
        st = launch_status(fn);
        if (st) return st;
    }
    return VSA_OK;
}

extern "C" size_t vsa_cluster_order_workspace_bytes(int B, int H, int N, int C) {
    if (B <= 0 || H <= 0 || N <= 0 || C <= 0) return 0;
    const size_t nch = ((size_t)N + kOrdChunk - 1) / kOrdChunk;
    return (size_t)B * H * nch * C * 4;
}

extern "C" int vsa_cluster_order(const int32_t* labels, int B, int H, int N, int C, int32_t* perm, int32_t* offsets,
                                 void* workspace, size_t ws_bytes, void* stream) {
    const char* fn = "vsa_cluster_order";
    if (!labels || !perm || !offsets) return fail(VSA_ERR_INVALID, "%s: null tensor", fn);
    if (B <= 0 || H <= 0 || N <= 0 || C <= 0) return fail(VSA_ERR_INVALID, "%s: B, H, N, C must be positive", fn);
    if (C > kOrdMaxC) return fail(VSA_ERR_UNSUPPORTED, "%s: at most %d clusters", fn, kOrdMaxC);
    const int64_t BH = (int64_t)B * H;
    const int64_t nch = (N + kOrdChunk - 1) / kOrdChunk;
    if (BH * N >= (1ll << 31) || BH * nch * C >= (1ll << 31)) return fail(VSA_ERR_INVALID, "%s: problem too large", fn);
    const size_t need = vsa_cluster_order_workspace_bytes(B, H, N, C);
    if (!workspace || ws_bytes < need)
        return fail(VSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need, ws_bytes);
    OrdArgs a{};
    a.labels = labels; a.perm = perm; a.offsets = offsets;
    a.chunk = static_cast<int32_t*>(workspace);
    a.N = N; a.C = C; a.BH = (int32_t)BH; a.nch = (int32_t)nch;
    launch_order(a, as_stream(stream));
    return launch_status(fn);
}

extern "C" int vsa_gather_rows(const void* src, void* dst, int B, int H, int N, int D, int dtype, const int32_t* perm,
                               int inverse, void* stream) {
    const char* fn = "vsa_gather_rows";
    if (!src || !dst || !perm) return fail(VSA_ERR_INVALID, "%s: null tensor", fn);
    if (!aligned16(src) || !aligned16(dst)) return fail(VSA_ERR_INVALID, "%s: tensors must be 16-byte aligned", fn);
    if (B <= 0 || H <= 0 || N <= 0) return fail(VSA_ERR_INVALID, "%s: B, H, N must be positive", fn);
    if (src == dst) return fail(VSA_ERR_INVALID, "%s: src and dst must differ", fn);
    if (dtype != VSA_BF16 && dtype != VSA_F32) return fail(VSA_ERR_UNSUPPORTED, "%s: dtype must be bf16 or f32", fn);
    if (D != 64 && D != 128) return fail(VSA_ERR_UNSUPPORTED, "%s: D must be 64 or 128", fn);
    const int row_bytes = D * (dtype == VSA_BF16 ? 2 : 4);
    const int64_t rows = (int64_t)B * H * N;
    if (rows * row_bytes >= (1ll << 40)) return fail(VSA_ERR_INVALID, "%s: problem too large", fn);
    const int64_t threads = rows * (row_bytes / 16);
    hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, as_stream(stream),
                       static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), perm, N, row_bytes, rows,
                       inverse ? 1 : 0);
    return launch_status(fn);
}

extern "C" int vsa_cluster_scores(const float* cq, const float* ck, const int32_t* k_counts, int B, int H, int Cq,
                                  int Ck, int D, float scale, float* scores, void* stream) {
    const char* fn = "vsa_cluster_scores";
    if (!cq || !ck || !k_counts || !scores) return fail(VSA_ERR_INVALID, "%s: null tensor", fn);
    if (!aligned16(ck)) return fail(VSA_ERR_INVALID, "%s: ck must be 16-byte aligned", fn);
    if (B <= 0 || H <= 0 || Cq <= 0 || Ck <= 0) return fail(VSA_ERR_INVALID, "%s: B, H, Cq, Ck must be positive", fn);
    if (D != 64 && D != 128) return fail(VSA_ERR_UNSUPPORTED, "%s: D must be 64 or 128", fn);
    if (!(scale > 0.f) || !__builtin_isfinite(scale)) return fail(VSA_ERR_INVALID, "%s: scale must be positive and finite", fn);
    const int64_t rows = (int64_t)B * H * Cq;
    if (rows >= (1ll << 31) || rows * Ck >= (1ll << 40)) return fail(VSA_ERR_INVALID, "%s: problem too large", fn);
    hipLaunchKernelGGL(cluster_scores_kernel, dim3((unsigned)rows), dim3(256), 0, as_stream(stream), cq, ck, k_counts,
                       Cq, Ck, D, scale, scores);
    return launch_status(fn);
}
