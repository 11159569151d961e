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
//    A workgroup owns 8 clusters; each of its 16 waves scans one sixteenth of the
//    tokens in order and accumulates its members in registers; the 16 partial
//    sums are then added in wave order. No floating-point atomics, so the result
//    does not depend on scheduling.
//  * Order: stable counting sort by cluster. Chunks of 256 tokens count their
//    clusters, a per-cluster scan over chunks gives each chunk's first slot, and
//    every token's rank among equal clusters in its chunk comes from wave ballots.
#include <math.h>

#include "mfma_tile.h"

namespace vsa {

constexpr int kKmD = 128;                 // token width handled by the k-means kernels
constexpr int kKmMaxC = 4096;             // clusters per head
constexpr int kOrdChunk = 256;            // tokens per counting-sort chunk (4 waves)
constexpr int kOrdMaxC = 1024;            // clusters per head for the order kernels
constexpr int kUpdWaves = 16, kUpdClusters = 8;

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

// ---- update: one workgroup per (bh, 8 clusters), 16 waves over the tokens --------
__global__ __launch_bounds__(kUpdWaves * 64) void km_update_kernel(KmArgs a, int groups) {
    __shared__ float part[kUpdWaves][kUpdClusters][kKmD];
    __shared__ int pcnt[kUpdWaves][kUpdClusters];
    __shared__ float mb[kUpdClusters][kKmD];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int item = xcd_remap(blockIdx.x, a.BH * groups);
    const int64_t bh = item / groups;
    const int c0 = (item - (int)bh * groups) * kUpdClusters;
    const int per = ((a.N + kUpdWaves - 1) / kUpdWaves + 63) & ~63;
    const int t0 = min(a.N, w * per), t1 = min(a.N, t0 + per);
    const int32_t* lab = a.labels + bh * a.N;
    const uint16_t* xh = a.x + bh * a.N * kKmD;
    float acc[kUpdClusters][2];
#pragma unroll
    for (int k = 0; k < kUpdClusters; ++k) acc[k][0] = acc[k][1] = 0.f;
    int cnt[kUpdClusters];
#pragma unroll
    for (int k = 0; k < kUpdClusters; ++k) cnt[k] = 0;
    for (int base = t0; base < t1; base += 64) {
        const int t = base + lane;
        const int rel = (t < t1) ? lab[t] - c0 : -1;
        uint64_t m = __ballot(rel >= 0 && rel < kUpdClusters);
        while (m) {
            // up to four members at a time: their rows load together
            int j[4], r[4], nm = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                j[u] = 0;
                r[u] = 0;
                if (m) {
                    j[u] = __builtin_ctzll(m);
                    m &= m - 1;
                    r[u] = __builtin_amdgcn_readlane(rel, j[u]);
                    ++nm;
                }
            }
            uint32_t pr[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                pr[u] = u < nm ? *reinterpret_cast<const uint32_t*>(xh + (int64_t)(base + j[u]) * kKmD + 2 * lane) : 0u;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (u >= nm) break;
                const float v0 = bf16_bits_to_f32(pr[u] & 0xffffu), v1 = bf16_bits_to_f32(pr[u] >> 16);
#pragma unroll
                for (int k = 0; k < kUpdClusters; ++k)
                    if (r[u] == k) {
                        acc[k][0] += v0;
                        acc[k][1] += v1;
                        ++cnt[k];
                    }
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kUpdClusters; ++k) {
        part[w][k][2 * lane] = acc[k][0];
        part[w][k][2 * lane + 1] = acc[k][1];
        if (lane == 0) pcnt[w][k] = cnt[k];
    }
    __syncthreads();
    // 8 clusters x 128 channels: thread tid < 1024 takes one value
    {
        const int k = tid >> 7, d = tid & 127;
        const int c = c0 + k;
        float s = 0.f;
        int n = 0;
        for (int u = 0; u < kUpdWaves; ++u) {
            s += part[u][k][d];
            n += pcnt[u][k];
        }
        float v = 0.f;
        if (c < a.C) {
            const int64_t row = bh * a.C + c;
            v = n > 0 ? s / (float)n : a.cent[row * kKmD + d];
            if (d == 0) a.counts[row] = n;
        }
        mb[k][d] = v;
    }
    __syncthreads();
    if (w < kUpdClusters && c0 + w < a.C) {
        const int64_t row = bh * a.C + c0 + w;
        const float nrm = wave_sum(put_centroid(a, row, lane, mb[w][2 * lane], mb[w][2 * lane + 1]));
        if (lane == 0) a.cnorm[row] = nrm;
    }
}

// ---- stable cluster-major order -------------------------------------------------
struct OrdArgs {
    const int32_t* labels;    // [BH, N]
    const int32_t* counts;    // [BH, C]
    int32_t* perm;            // [BH, N]: perm[p] = token at position p
    int32_t* offsets;         // [BH, C + 1]
    int32_t* chunk;           // [BH, nch, C]: counts, then first slots
    int32_t N, C, BH, nch;
};

// cluster offsets: one wave per bh (exclusive scan of the counts)
__global__ __launch_bounds__(64) void ord_offsets_kernel(OrdArgs a) {
    const int64_t bh = blockIdx.x;
    const int lane = threadIdx.x;
    const int32_t* cnt = a.counts + bh * a.C;
    int32_t* off = a.offsets + bh * (a.C + 1);
    int run = 0;
    for (int c0 = 0; c0 < a.C; c0 += 64) {
        const int c = c0 + lane;
        const int v = c < a.C ? cnt[c] : 0;
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

// first slot of every (chunk, cluster): one wave per (bh, c), scanning the chunks
__global__ __launch_bounds__(256) void ord_scan_kernel(OrdArgs a) {
    const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (g >= (int64_t)a.BH * a.C) return;
    const int64_t bh = g / a.C;
    const int c = (int)(g - bh * a.C);
    int run = a.offsets[bh * (a.C + 1) + c];
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
}

// scatter: position = first slot of (chunk, cluster) + rank in the chunk
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
        const int pos = a.chunk[(bh * a.nch + ch) * a.C + l] + before + rank;
        if ((unsigned)pos < (unsigned)a.N) a.perm[bh * a.N + pos] = t;   // counts that disagree with the labels
    }
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

extern "C" size_t vsa_kmeans_workspace_bytes(int B, int H, int C, int D) {
    if (B <= 0 || H <= 0 || C <= 0 || D != kKmD) return 0;
    const size_t rows = (size_t)B * H * C;
    return ((rows * kKmD * 2 + 255) & ~(size_t)255) + ((rows * 4 + 255) & ~(size_t)255);
}

extern "C" int vsa_kmeans(const void* x, int B, int H, int N, int D, int dtype, int C, int iters, float* centroids,
                          int32_t* labels, int32_t* counts, void* workspace, size_t ws_bytes, void* stream) {
    const char* fn = "vsa_kmeans";
    if (!x || !centroids || !labels || !counts) return fail(VSA_ERR_INVALID, "%s: null tensor", fn);
    if (!aligned16(x) || !aligned16(centroids)) return fail(VSA_ERR_INVALID, "%s: x and centroids must be 16-byte aligned", fn);
    if (B <= 0 || H <= 0 || N <= 0) return fail(VSA_ERR_INVALID, "%s: B, H, N must be positive", fn);
    if (C < 1 || C > N) return fail(VSA_ERR_INVALID, "%s: need 1 <= C <= N (C = %d, N = %d)", fn, C, N);
    if (C > kKmMaxC) return fail(VSA_ERR_UNSUPPORTED, "%s: at most %d clusters", fn, kKmMaxC);
    if (iters < 1) return fail(VSA_ERR_INVALID, "%s: iters must be >= 1", fn);
    if (dtype != VSA_BF16 || D != kKmD) return fail(VSA_ERR_UNSUPPORTED, "%s: needs bf16 with D = %d", fn, kKmD);
    const int64_t BH = (int64_t)B * H;
    if (BH * N >= (1ll << 31) || (int64_t)N * kKmD * 2 >= (1ll << 31)) return fail(VSA_ERR_INVALID, "%s: problem too large", fn);
    const size_t need = vsa_kmeans_workspace_bytes(B, H, C, D);
    if (!workspace || ws_bytes < need)
        return fail(VSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need, ws_bytes);
    KmArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.cent = centroids;
    a.cent_bf = static_cast<uint16_t*>(workspace);
    a.cnorm = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                       (((size_t)BH * C * kKmD * 2 + 255) & ~(size_t)255));
    a.labels = labels;
    a.counts = counts;
    a.N = N; a.C = C; a.BH = (int32_t)BH;
    hipStream_t s = as_stream(stream);
    hipLaunchKernelGGL(km_seed_kernel, dim3((unsigned)((BH * C + 3) / 4)), dim3(256), 0, s, a);
    int st = launch_status("vsa_kmeans (seeds)");
    if (st) return st;
    const int tiles = (N + 127) / 128;
    const int groups = (C + kUpdClusters - 1) / kUpdClusters;
    for (int it = 0; it < iters; ++it) {
        hipLaunchKernelGGL(km_assign_kernel, dim3((unsigned)(BH * tiles)), dim3(256), 0, s, a, tiles);
        hipLaunchKernelGGL(km_update_kernel, dim3((unsigned)(BH * groups)), dim3(kUpdWaves * 64), 0, s, a, groups);
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

extern "C" int vsa_cluster_order(const int32_t* labels, const int32_t* counts, int B, int H, int N, int C,
                                 int32_t* perm, int32_t* offsets, void* workspace, size_t ws_bytes, void* stream) {
    const char* fn = "vsa_cluster_order";
    if (!labels || !counts || !perm || !offsets) return fail(VSA_ERR_INVALID, "%s: null tensor", fn);
    if (B <= 0 || H <= 0 || N <= 0 || C <= 0) return fail(VSA_ERR_INVALID, "%s: B, H, N, C must be positive", fn);
    if (C > kOrdMaxC) return fail(VSA_ERR_UNSUPPORTED, "%s: at most %d clusters", fn, kOrdMaxC);
    const int64_t BH = (int64_t)B * H;
    const int64_t nch = (N + kOrdChunk - 1) / kOrdChunk;
    if (BH * N >= (1ll << 31) || BH * nch * C >= (1ll << 31)) return fail(VSA_ERR_INVALID, "%s: problem too large", fn);
    const size_t need = vsa_cluster_order_workspace_bytes(B, H, N, C);
    if (!workspace || ws_bytes < need)
        return fail(VSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need, ws_bytes);
    OrdArgs a{};
    a.labels = labels; a.counts = counts; a.perm = perm; a.offsets = offsets;
    a.chunk = static_cast<int32_t*>(workspace);
    a.N = N; a.C = C; a.BH = (int32_t)BH; a.nch = (int32_t)nch;
    hipStream_t s = as_stream(stream);
    hipLaunchKernelGGL(ord_offsets_kernel, dim3((unsigned)BH), dim3(64), 0, s, a);
    hipLaunchKernelGGL(ord_count_kernel, dim3((unsigned)(BH * nch)), dim3(kOrdChunk), 0, s, a);
    hipLaunchKernelGGL(ord_scan_kernel, dim3((unsigned)((BH * C + 3) / 4)), dim3(256), 0, s, a);
    hipLaunchKernelGGL(ord_scatter_kernel, dim3((unsigned)(BH * nch)), dim3(kOrdChunk), 0, s, a);
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
