// Block mean-pooling of Q and K and pooled block scores S = scale * Qbar Kbar^T.
//
// USV page, Figure 2 caption: long-range key cubes are chosen by top-k cube
// selection; the score of a (query block, key block) pair is read as the scaled
// inner product of the two blocks' mean vectors over their valid rows.
//
// Pooling reads every Q and K row once (HBM-bound): a wave per (b, h, block,
// tensor), 16-byte loads all in flight at once, fp32 sums in a fixed order. The
// score product is a small fp32 GEMM per head (nb x D times D x nb) on the fp32
// matrix cores.
#include "vsa_internal.h"

namespace vsa {

// One wave per (b, h, block, tensor), four per workgroup. Lane (g, c) adds
// the 16-byte chunk c of rows g, g + RPI, ... (fp32, ascending rows); the RPI
// partial sums of a chunk are then added by a butterfly over the lanes.
template <int D, int BS>
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                   const int32_t* __restrict__ blk_len, int N, int nb, int64_t items,
                                                   float* __restrict__ qpool, float* __restrict__ kpool) {
    constexpr int CPR = D / 8;              // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;           // rows per wave load
    constexpr int STEPS = BS / RPI;
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // 2 (bh nb + block) + tensor
    if (item >= items) return;
    const int which = (int)(item & 1);
    const int64_t ib = item >> 1;
    const int64_t bh = ib / nb;
    const int b = (int)(ib - bh * nb);
    const uint16_t* src = (which ? k : q) + (bh * N + (int64_t)b * BS) * D;
    int valid = min(BS, N - b * BS);
    if (blk_len) valid = min(valid, blk_len[b]);
    valid = max(valid, 0);
    const int c = lane % CPR, g = lane / CPR;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s0 = 0; s0 < STEPS; s0 += 16) {
        u32x4 t[16];
#pragma unroll
        for (int p = 0; p < 16; ++p) {
            const int r = g + (s0 + p) * RPI;
            t[p] = (s0 + p < STEPS && r < valid) ? *reinterpret_cast<const u32x4*>(src + (int64_t)r * D + 8 * c)
                                                 : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int p = 0; p < 16; ++p) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += __uint_as_float(t[p][e] << 16);
                acc[2 * e + 1] += __uint_as_float(t[p][e] & 0xffff0000u);
            }
        }
    }
#pragma unroll
    for (int off = CPR; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off);
    if (g == 0) {
        const float n = (float)max(valid, 1);    // an empty block has sums 0 and mean 0
        float* dst = (which ? kpool : qpool) + ib * D + 8 * c;
        f32x4 lo = {acc[0] / n, acc[1] / n, acc[2] / n, acc[3] / n};
        f32x4 hi = {acc[4] / n, acc[5] / n, acc[6] / n, acc[7] / n};
        *reinterpret_cast<f32x4*>(dst) = lo;
        *reinterpret_cast<f32x4*>(dst + 4) = hi;
    }
}

// S[bh][i][j] = scale * sum_d qp[bh][i][d] * kp[bh][j][d] on the fp32 matrix
// cores (v_mfma_f32_32x32x2_f32). A workgroup owns 64 x 64 scores, each wave
// 32 x 32. Channels are staged 64 at a time through LDS with full-line loads
// (rows padded by 16 bytes so the operand reads below are conflict-free). The
// dot product's two MFMA k slots take alternate 4-channel groups: lane (r, h)
// reads channels 8 c + 4 h + [0, 4) of its row with one 16-byte LDS read and
// feeds them to four steps. Rows past nb stage row nb - 1: they only reach
// outputs past nb, which are not stored.
template <int D>
__global__ __launch_bounds__(256) void pooled_gemm_kernel(const float* __restrict__ qp, const float* __restrict__ kp,
                                                          int nb, float scale, float* __restrict__ S) {
    constexpr int DC = 64;                  // channels per staged phase
    constexpr int LD = DC + 4;              // padded LDS row, floats
    __shared__ __attribute__((aligned(16))) float As[64 * LD];
    __shared__ __attribute__((aligned(16))) float Bs[64 * LD];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane & 31, h = lane >> 5;
    const int64_t bh = blockIdx.z;
    const int I0 = blockIdx.y * 64, J0 = blockIdx.x * 64;
    const float* Q = qp + bh * nb * D;
    const float* K = kp + bh * nb * D;
    const int wi = w >> 1, wj = w & 1;
    f32x16 acc = {};
#pragma unroll
    for (int ph = 0; ph < D / DC; ++ph) {
        f32x4 va[4], vb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {       // 64 rows x 16 float4 per tensor
            const int idx = tid + 256 * u, row = idx >> 4, ch = idx & 15;
            va[u] = *reinterpret_cast<const f32x4*>(Q + (int64_t)min(I0 + row, nb - 1) * D + DC * ph + 4 * ch);
            vb[u] = *reinterpret_cast<const f32x4*>(K + (int64_t)min(J0 + row, nb - 1) * D + DC * ph + 4 * ch);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int idx = tid + 256 * u, row = idx >> 4, ch = idx & 15;
            *reinterpret_cast<f32x4*>(As + row * LD + 4 * ch) = va[u];
            *reinterpret_cast<f32x4*>(Bs + row * LD + 4 * ch) = vb[u];
        }
        __syncthreads();
        const float* ar = As + (32 * wi + r) * LD + 4 * h;
        const float* br = Bs + (32 * wj + r) * LD + 4 * h;
#pragma unroll
        for (int c = 0; c < DC / 8; ++c) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(ar + 8 * c);
            const f32x4 b = *reinterpret_cast<const f32x4*>(br + 8 * c);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], acc, 0, 0, 0);
        }
        __syncthreads();
    }
    float* out = S + bh * nb * nb;
    const int j = J0 + 32 * wj + r;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int i = I0 + 32 * wi + 8 * (e >> 2) + 4 * h + (e & 3);
        if (i < nb && j < nb) out[(int64_t)i * nb + j] = scale * acc[e];
    }
}

}  // namespace vsa

using namespace vsa;

extern "C" int vsa_block_scores(const void* q, const void* k, int B, int H, int N, int D, int dtype, int bs,
                                const int32_t* blk_len, float scale, float* scores, float* qpool, float* kpool,
                                void* stream) {
    if (!q || !k || !scores || !qpool || !kpool) return fail(VSA_ERR_INVALID, "vsa_block_scores: null pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(qpool) || !aligned16(kpool))
        return fail(VSA_ERR_INVALID, "vsa_block_scores: q, k, qpool, kpool must be 16-byte aligned");
    if (B <= 0 || H <= 0 || N <= 0) return fail(VSA_ERR_INVALID, "vsa_block_scores: B, H, N must be positive");
    if (dtype != VSA_BF16) return fail(VSA_ERR_UNSUPPORTED, "vsa_block_scores: only bf16 inputs");
    if (D != 64 && D != 128) return fail(VSA_ERR_UNSUPPORTED, "vsa_block_scores: D must be 64 or 128");
    if (bs != 64 && bs != 128) return fail(VSA_ERR_UNSUPPORTED, "vsa_block_scores: bs must be 64 or 128");
    if (!(scale > 0.f) || !__builtin_isfinite(scale)) return fail(VSA_ERR_INVALID, "vsa_block_scores: scale must be positive and finite");
    const int64_t nb = (N + (int64_t)bs - 1) / bs;
    if ((int64_t)B * H * nb >= (1ll << 31) || (int64_t)B * H > 65535)
        return fail(VSA_ERR_INVALID, "vsa_block_scores: problem too large");
    hipStream_t s = as_stream(stream);
    const int64_t items = 2 * (int64_t)B * H * nb;
    dim3 pg((unsigned)((items + 3) / 4));
    const uint16_t* qh = static_cast<const uint16_t*>(q);
    const uint16_t* kh = static_cast<const uint16_t*>(k);
    const int nbi = (int)nb;
    if (D == 128 && bs == 128) hipLaunchKernelGGL((pool_kernel<128, 128>), pg, dim3(256), 0, s, qh, kh, blk_len, N, nbi, items, qpool, kpool);
    else if (D == 128) hipLaunchKernelGGL((pool_kernel<128, 64>), pg, dim3(256), 0, s, qh, kh, blk_len, N, nbi, items, qpool, kpool);
    else if (bs == 128) hipLaunchKernelGGL((pool_kernel<64, 128>), pg, dim3(256), 0, s, qh, kh, blk_len, N, nbi, items, qpool, kpool);
    else hipLaunchKernelGGL((pool_kernel<64, 64>), pg, dim3(256), 0, s, qh, kh, blk_len, N, nbi, items, qpool, kpool);
    int st = launch_status("vsa_block_scores (pool)");
    if (st) return st;
    dim3 gg((unsigned)((nb + 63) / 64), (unsigned)((nb + 63) / 64), (unsigned)(B * H));
    if (D == 128) hipLaunchKernelGGL(pooled_gemm_kernel<128>, gg, dim3(256), 0, s, qpool, kpool, nbi, scale, scores);
    else hipLaunchKernelGGL(pooled_gemm_kernel<64>, gg, dim3(256), 0, s, qpool, kpool, nbi, scale, scores);
    return launch_status("vsa_block_scores (gemm)");
}
