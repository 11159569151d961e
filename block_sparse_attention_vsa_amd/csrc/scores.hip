// Block mean-pooling of Q and K and pooled block scores S = scale * Qbar Kbar^T.
//
// USV page, Figure 2 caption: long-range key cubes are chosen by top-k cube
// selection; the score of a (query block, key block) pair is read as the scaled
// inner product of the two blocks' mean vectors over their valid rows.
//
// Pooling reads every Q and K row once (HBM-bound): a workgroup per (b, h, block,
// tensor), 16-byte loads, fp32 sums in a fixed order. The score product is a
// small fp32 GEMM per head (nb x D times D x nb), tiled 64 x 64 in LDS.
#include "vsa_internal.h"

namespace vsa {

template <int D>
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                   const int32_t* __restrict__ blk_len, int N, int bs, int nb,
                                                   float* __restrict__ qpool, float* __restrict__ kpool) {
    constexpr int CPR = D / 8;              // 16-byte chunks per row
    constexpr int RPP = 256 / CPR;          // rows per pass
    __shared__ float part[RPP][D + 1];
    const int64_t item = blockIdx.x;        // (bh, block)
    const int which = blockIdx.y;           // 0 = q, 1 = k
    const int64_t bh = item / nb;
    const int b = (int)(item - bh * nb);
    const uint16_t* src = (which ? k : q) + (bh * N + (int64_t)b * bs) * D;
    int valid = min(bs, N - b * bs);
    if (blk_len) valid = min(valid, blk_len[b]);
    valid = max(valid, 0);
    const int c = threadIdx.x % CPR, r0 = threadIdx.x / CPR;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int r = r0; r < valid; r += RPP) {
        u32x4 t = *reinterpret_cast<const u32x4*>(src + (int64_t)r * D + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += __uint_as_float(t[e] << 16);
            acc[2 * e + 1] += __uint_as_float(t[e] & 0xffff0000u);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[r0][8 * c + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < D) {
        float s = 0.f;
        for (int r = 0; r < RPP; ++r) s += part[r][threadIdx.x];
        float* dst = (which ? kpool : qpool) + item * D;
        dst[threadIdx.x] = valid > 0 ? s / (float)valid : 0.f;
    }
}

// S[bh][i][j] = scale * sum_d qp[bh][i][d] * kp[bh][j][d]; 64 x 64 tile per
// workgroup, each thread a 4 x 4 patch, channels in ascending order.
__global__ __launch_bounds__(256) void pooled_gemm_kernel(const float* __restrict__ qp, const float* __restrict__ kp,
                                                          int nb, int D, float scale, float* __restrict__ S) {
    __shared__ float qs[32][64 + 4];
    __shared__ float ks[32][64 + 4];
    const int bh = blockIdx.z;
    const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
    const float* Q = qp + (int64_t)bh * nb * D;
    const float* K = kp + (int64_t)bh * nb * D;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float acc[4][4] = {};
    for (int d0 = 0; d0 < D; d0 += 32) {
        for (int e = threadIdx.x; e < 64 * 32; e += 256) {
            int r = e / 32, dd = e % 32;
            qs[dd][r] = (i0 + r < nb) ? Q[(int64_t)(i0 + r) * D + d0 + dd] : 0.f;
            ks[dd][r] = (j0 + r < nb) ? K[(int64_t)(j0 + r) * D + d0 + dd] : 0.f;
        }
        __syncthreads();
#pragma unroll 8
        for (int dd = 0; dd < 32; ++dd) {
            float a[4], bv[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) { a[x] = qs[dd][ty * 4 + x]; bv[x] = ks[dd][tx * 4 + x]; }
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(a[x], bv[y], acc[x][y]);
        }
        __syncthreads();
    }
    float* out = S + (int64_t)bh * nb * nb;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        int i = i0 + ty * 4 + x;
        if (i >= nb) continue;
#pragma unroll
        for (int y = 0; y < 4; ++y) {
            int j = j0 + tx * 4 + y;
            if (j < nb) out[(int64_t)i * nb + j] = scale * acc[x][y];
        }
    }
}

}  // namespace vsa

using namespace vsa;

extern "C" int vsa_block_scores(const void* q, const void* k, int B, int H, int N, int D, int dtype, int bs,
                                const int32_t* blk_len, float scale, float* scores, float* qpool, float* kpool,
                                void* stream) {
    if (!q || !k || !scores || !qpool || !kpool) return fail(VSA_ERR_INVALID, "vsa_block_scores: null pointer");
    if (!aligned16(q) || !aligned16(k)) return fail(VSA_ERR_INVALID, "vsa_block_scores: q, k must be 16-byte aligned");
    if (B <= 0 || H <= 0 || N <= 0) return fail(VSA_ERR_INVALID, "vsa_block_scores: B, H, N must be positive");
    if (dtype != VSA_BF16) return fail(VSA_ERR_UNSUPPORTED, "vsa_block_scores: only bf16 inputs");
    if (D != 64 && D != 128) return fail(VSA_ERR_UNSUPPORTED, "vsa_block_scores: D must be 64 or 128");
    if (bs != 64 && bs != 128) return fail(VSA_ERR_UNSUPPORTED, "vsa_block_scores: bs must be 64 or 128");
    if (!(scale > 0.f) || !__builtin_isfinite(scale)) return fail(VSA_ERR_INVALID, "vsa_block_scores: scale must be positive and finite");
    const int64_t nb = (N + (int64_t)bs - 1) / bs;
    if ((int64_t)B * H * nb >= (1ll << 31) || (int64_t)B * H > 65535)
        return fail(VSA_ERR_INVALID, "vsa_block_scores: problem too large");
    hipStream_t s = as_stream(stream);
    dim3 pg((unsigned)((int64_t)B * H * nb), 2);
    const uint16_t* qh = static_cast<const uint16_t*>(q);
    const uint16_t* kh = static_cast<const uint16_t*>(k);
    if (D == 128) hipLaunchKernelGGL(pool_kernel<128>, pg, dim3(256), 0, s, qh, kh, blk_len, N, bs, (int)nb, qpool, kpool);
    else hipLaunchKernelGGL(pool_kernel<64>, pg, dim3(256), 0, s, qh, kh, blk_len, N, bs, (int)nb, qpool, kpool);
    int st = launch_status("vsa_block_scores (pool)");
    if (st) return st;
    dim3 gg((unsigned)((nb + 63) / 64), (unsigned)((nb + 63) / 64), (unsigned)(B * H));
    hipLaunchKernelGGL(pooled_gemm_kernel, gg, dim3(256), 0, s, qpool, kpool, (int)nb, D, scale, scores);
    return launch_status("vsa_block_scores (gemm)");
}
