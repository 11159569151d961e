// FP8 (OCP e4m3) block-sparse attention on gfx950.
//
// Sparse Video-Gen page, "Key results" (and the speed-ups of the Sparse
// VideoGen2 and USV pages): the attention runs faster still in FP8. Quantised
// inputs: Q and K with one scale per (b, h, 64 positions), V with one scale per
// (b, h, channel); code = e4m3(x * (448 / amax)) in fp32, scale = amax / 448.
// The attention computes softmax attention on code * scale.
//
// Kernel (D = 128, query blocks of 128 rows, 4 waves of 32 rows, 64-key
// sub-tiles), on v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3, unit scales):
//  * S^T = K Q^T: per 32-key half two MFMAs over 64 channels each; every lane
//    reads 32 consecutive bytes of its key row (the k index only has to pair up
//    between the two operands, so the natural order serves). The dequantisation
//    scales of the query rows and of the sub-tile's keys fold into the one FMA
//    that takes the score to the log2 domain.
//  * P = exp2(s - m) in fp32 (lazy offset, so P <= 2^8 < 448), converted to e4m3
//    in registers; the row sum uses the fp32 P.
//  * O^T += V^T P^T: one MFMA per 32 channels; V is stored transposed per 64-key
//    tile with its keys in the order in which the score accumulator holds a lane's
//    keys (key 32 st + 8 g + 4 h + e at column 32 h + 16 st + 4 g + e), so a lane's
//    32 operand bytes are contiguous. V's per-channel scale is applied to O at the
//    end.
//  * K rows (128 B) keep 16-byte chunk c at slot c ^ ((r >> 1) & 7), V^T rows
//    (64 B) at c ^ ((r >> 2) & 3): 16 consecutive rows read at one chunk hit 16
//    distinct 16-byte bank groups.
#include <math.h>

#include "mfma_tile.h"

namespace vsa {

typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kF8Block = 64;             // positions per Q / K scale, keys per V tile
constexpr float kE4M3Max = 448.f;

__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ float clamp448(float y) { return fminf(fmaxf(y, -kE4M3Max), kE4M3Max); }

__device__ __forceinline__ float block_max_256(float v, float* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return v;
}

// ---- Q / K: one workgroup per (bh, 64 rows); thread t takes row t / 4, 32 channels
__global__ __launch_bounds__(256) void fp8_quant_rows_kernel(const uint16_t* x, uint8_t* out, float* scales, int N,
                                                             int nblk) {
    __shared__ float red[4];
    const int64_t bh = blockIdx.x / nblk;
    const int blk = (int)(blockIdx.x - bh * nblk);
    const int row = blk * kF8Block + (threadIdx.x >> 2), c0 = 32 * (threadIdx.x & 3);
    const bool ok = row < N;
    const uint16_t* src = x + (bh * N + row) * 128 + c0;
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        u32x4 w = ok ? *reinterpret_cast<const u32x4*>(src + 8 * i) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[8 * i + 2 * e] = bf16_bits_to_f32(w[e] & 0xffffu);
            v[8 * i + 2 * e + 1] = bf16_bits_to_f32(w[e] >> 16);
        }
    }
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(v[i]));
    am = block_max_256(am, red);
    const float inv = am > 0.f ? kE4M3Max / am : 0.f;
    if (ok) {
        uint8_t* dst = out + (bh * N + row) * 128 + c0;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            u32x4 pk;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float* p = v + 16 * i + 4 * e;
                pk[e] = pack4_fp8(clamp448(p[0] * inv), clamp448(p[1] * inv), clamp448(p[2] * inv),
                                  clamp448(p[3] * inv));
            }
            *reinterpret_cast<u32x4*>(dst + 16 * i) = pk;
        }
    }
    if (threadIdx.x == 0) scales[bh * nblk + blk] = am / kE4M3Max;
}

// ---- V: per-channel amax (integer max of the non-negative float bits: exact and
// order-independent), then quantisation into transposed 64-key tiles -------------
__global__ __launch_bounds__(256) void fp8_fill_u32_kernel(uint32_t* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// A workgroup per (b, h, kAmaxRows rows): 16-byte loads, 16 rows per pass, the
// lanes' maxima folded by shuffles and LDS, then one integer max per channel.
constexpr int kAmaxRows = 512;

__global__ __launch_bounds__(256) void fp8_vamax_kernel(const uint16_t* x, uint32_t* amax_bits, int N, int nchunk) {
    __shared__ float red[4][128];
    const int64_t bh = blockIdx.x / nchunk;
    const int chunk = (int)(blockIdx.x - bh * nchunk);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c = threadIdx.x & 15;                              // channels 8 c .. 8 c + 7
    const int r_end = min(N, (chunk + 1) * kAmaxRows);
    float am[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int r = chunk * kAmaxRows + (threadIdx.x >> 4); r < r_end; r += 16) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(x + (bh * N + r) * 128 + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            am[2 * e] = fmaxf(am[2 * e], fabsf(bf16_bits_to_f32(v[e] & 0xffffu)));
            am[2 * e + 1] = fmaxf(am[2 * e + 1], fabsf(bf16_bits_to_f32(v[e] >> 16)));
        }
    }
#pragma unroll
    for (int off = 16; off < 64; off <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i) am[i] = fmaxf(am[i], __shfl_xor(am[i], off));
    if (lane < 16)
#pragma unroll
        for (int i = 0; i < 8; ++i) red[w][8 * c + i] = am[i];
    __syncthreads();
    if (threadIdx.x < 128) {
        const float m = fmaxf(fmaxf(red[0][threadIdx.x], red[1][threadIdx.x]), fmaxf(red[2][threadIdx.x], red[3][threadIdx.x]));
        atomicMax(&amax_bits[bh * 128 + threadIdx.x], __float_as_uint(m));
    }
}

__global__ __launch_bounds__(256) void fp8_quant_vt_kernel(const uint16_t* x, const uint32_t* amax_bits,
                                                           uint8_t* tiles, int N, int ntile) {
    __shared__ uint8_t tile[128][kF8Block];                     // [channel][column]
    __shared__ float inv_s[128];                                // 448 / amax per channel
    const int64_t bh = blockIdx.x / ntile;
    const int t = (int)(blockIdx.x - bh * ntile);
    if (threadIdx.x < 128) {
        const float am = __uint_as_float(amax_bits[bh * 128 + threadIdx.x]);
        inv_s[threadIdx.x] = am > 0.f ? kE4M3Max / am : 0.f;
    }
    __syncthreads();
    // thread: key k = threadIdx.x / 4, channels 32 (threadIdx.x & 3) + [0, 32)
    const int k = threadIdx.x >> 2, c0 = 32 * (threadIdx.x & 3);
    const int row = t * kF8Block + k;
    const bool ok = row < N;
    const int col = 32 * ((k >> 2) & 1) + 16 * (k >> 5) + 4 * ((k >> 3) & 3) + (k & 3);
    const uint16_t* src = x + (bh * N + row) * 128 + c0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        u32x4 w = ok ? *reinterpret_cast<const u32x4*>(src + 8 * i) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int ch = c0 + 8 * i + 2 * e + hh;
                const float y = bf16_bits_to_f32(hh ? (w[e] >> 16) : (w[e] & 0xffffu)) * inv_s[ch];
                const int code = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(y), 0.f, 0, false) & 0xff;
                tile[ch][col] = ok ? (uint8_t)code : (uint8_t)0;
            }
    }
    __syncthreads();
    // 128 rows x 64 bytes = 8 KiB: thread writes 32 bytes
    const int r = threadIdx.x >> 1, half = threadIdx.x & 1;
    uint8_t* dst = tiles + ((bh * ntile + t) * 128 + r) * kF8Block + 32 * half;
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(&tile[r][32 * half]);
    *reinterpret_cast<u32x4*>(dst + 16) = *reinterpret_cast<const u32x4*>(&tile[r][32 * half + 16]);
}

__global__ __launch_bounds__(256) void fp8_vscale_kernel(const uint32_t* amax_bits, float* scales, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) scales[i] = __uint_as_float(amax_bits[i]) / kE4M3Max;
}

// ---- attention ----------------------------------------------------------------------
struct F8Args {
    const uint8_t* q;          // [BH, N, 128] codes
    const uint8_t* k;
    const uint8_t* vt;         // [BH, ntile, 128, 64] codes
    const float* q_scale;      // [BH, ntile]
    const float* k_scale;
    const float* v_scale;      // [BH, 128]
    uint16_t* o;
    float* lse;
    const int32_t* blk_len;
    const uint8_t* mask;
    const int32_t* kv_idx;
    const int32_t* kv_cnt;
    int32_t max_kv;
    int32_t N, nb, ntile, num_items;
    float scale_log2;
};

__device__ __forceinline__ int f8_block_valid(const int32_t* blk_len, int b, int N) {
    const int exist = min(128, N - b * 128);
    return blk_len ? min(ld_const(blk_len, b), exist) : exist;
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_fwd_fp8_kernel(F8Args a) {
    constexpr int BS = 128, KT = 64, NST = 2, WAVES = 4, THREADS = 256, SUB = BS / KT, TB = KT * 128;
    constexpr float TAU = 8.f;
    __shared__ __attribute__((aligned(1024))) uint8_t k0[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t v0[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t k1[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t v1[TB];
    extern __shared__ __attribute__((aligned(16))) int16_t list_lds[];   // mask form only
    __shared__ int wave_cnt[WAVES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS copy targets stay scalar
    const int l32 = lane & 31, half = lane >> 5;
    const int item = xcd_remap(blockIdx.x, a.num_items);
    const int bh = item / a.nb, qb = item - bh * a.nb;
    const int valid_q = f8_block_valid(a.blk_len, qb, a.N);
    const bool wave_active = 32 * w < valid_q;

    int cnt;
    const int32_t* list_g = nullptr;
    if (a.mask) {
        cnt = compact_mask_row<THREADS>(a.mask + (int64_t)item * a.nb, a.nb, list_lds, wave_cnt);
    } else {
        cnt = min(ld_const(a.kv_cnt, item), a.max_kv);
        list_g = a.kv_idx + (int64_t)item * a.max_kv;
    }
    auto sub_valid = [&](int i, int& kb) -> int {
        kb = a.mask ? (int)list_lds[i / SUB] : ld_const(list_g, i / SUB);
        if ((unsigned)kb >= (unsigned)a.nb) return 0;
        const int v = f8_block_valid(a.blk_len, kb, a.N) - (i % SUB) * KT;
        return v < 0 ? 0 : (v > KT ? KT : v);
    };

    // DMA lanes: K instruction ins covers rows 8 ins + (lane >> 3) (16-byte slot
    // lane & 7); V^T instruction covers channel rows 16 ins + (lane >> 2) (slot lane & 3)
    const int k_row = 8 * w + (lane >> 3), k_slot = lane & 7;
    const int v_row = 16 * w + (lane >> 2), v_slot = lane & 3;
    // rows 8 ins + ... and 16 ins + ... keep their swizzle bits for every ins of a wave
    const int k_voff = k_row * 128 + ((k_slot ^ ((k_row >> 1) & 7)) << 4);
    const int v_voff = v_row * 64 + ((v_slot ^ ((v_row >> 2) & 3)) << 4);
    const int64_t head = (int64_t)bh * a.N * 128;
    const int head_bytes = a.N * 128;
    const uint8_t* vt_head = a.vt + (int64_t)bh * a.ntile * TB;
    const int vt_bytes = a.ntile * TB;
    auto issue = [&](int i, uint8_t* kd, uint8_t* vd) {
        int kb;
        if (sub_valid(i, kb) == 0) return;
        const int row0 = kb * BS + (i % SUB) * KT;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int ins = w + WAVES * u;      // 8 instructions of 1 KiB per tensor
            dma16(a.k + head, head_bytes, kd + ins * 1024, row0 * 128 + 1024 * WAVES * u + k_voff, 0);
            dma16(vt_head, vt_bytes, vd + ins * 1024, (row0 / KT) * TB + 1024 * WAVES * u + v_voff, 0);
        }
    };

    const int q_local = 32 * w + l32;
    const int q_row = qb * BS + q_local;
    const bool q_ok = q_local < valid_q;
    v8i qf[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
        if (q_ok) {
            const uint8_t* src = a.q + head + (int64_t)q_row * 128 + 64 * kk + 32 * half;
            lo = *reinterpret_cast<const u32x4*>(src);
            hi = *reinterpret_cast<const u32x4*>(src + 16);
        }
        qf[kk] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    // the wave's 32 rows lie in one 64-row scale block
    const float sq = q_ok || wave_active ? a.q_scale[(int64_t)bh * a.ntile + (qb * BS + 32 * w) / KT] : 0.f;

    f32x16 o_acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o_acc[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    auto compute = [&](int i, const uint8_t* kt, const uint8_t* vt) __attribute__((always_inline)) {
        int kb;
        const int vs = sub_valid(i, kb);
        if (!wave_active || vs == 0) return;
        // the block index is uniform: a scalar load keeps the key scale off the
        // vector-memory counter, so reading it does not wait for the next stage's copy
        const int kt_idx = (__builtin_amdgcn_readfirstlane(kb) * BS + (i % SUB) * KT) / KT;
        const float sk = ((const __attribute__((address_space(4))) float*)a.k_scale)[(int64_t)bh * a.ntile + kt_idx];
        const float mul = sq * sk * a.scale_log2;
        f32x16 s[NST];
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            s[st] = f32x16{};
            const int r = 32 * st + l32;
            const int sw = (r >> 1) & 7;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int c = 4 * kk + 2 * half;
                const u32x4 lo = *reinterpret_cast<const u32x4*>(kt + r * 128 + ((c ^ sw) << 4));
                const u32x4 hi = *reinterpret_cast<const u32x4*>(kt + r * 128 + (((c + 1) ^ sw) << 4));
                const v8i ka = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                s[st] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qf[kk], s[st], 0, 0, 0, 127, 0, 127);
            }
        }
        if (vs < KT) {
#pragma unroll
            for (int st = 0; st < NST; ++st)
#pragma unroll
                for (int x = 0; x < 16; ++x)
                    if (acc_key(st, x, half) >= vs) s[st][x] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
            for (int x = 0; x < 16; ++x) mx = fmaxf(mx, s[st][x]);
        mx = pair_max(mx);
        const float m_tile = mx * mul;
        const bool upd = m_tile > m_run + TAU;
        const float m_new = upd ? m_tile : m_run;
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        if (__ballot(upd)) {
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int x = 0; x < 16; ++x) o_acc[dt][x] *= alpha;
        }
        m_run = m_new;
        // P: byte 16 st + x of the lane's 32 is the key of accumulator element x of st
        float ps[4] = {0.f, 0.f, 0.f, 0.f};
        uint32_t pw[8];
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float p[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    p[e] = __builtin_amdgcn_exp2f(fmaf(s[st][4 * j + e], mul, -m_use));
                    ps[e] += p[e];
                }
                pw[4 * st + j] = pack4_fp8(p[0], p[1], p[2], p[3]);
            }
        l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
        const v8i pb = v8i{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], (int)pw[4], (int)pw[5], (int)pw[6],
                           (int)pw[7]};
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const int r = 32 * dt + l32;                         // channel row of V^T
            const int sw = (r >> 2) & 3;
            const int c = 2 * half;
            const u32x4 lo = *reinterpret_cast<const u32x4*>(vt + r * 64 + ((c ^ sw) << 4));
            const u32x4 hi = *reinterpret_cast<const u32x4*>(vt + r * 64 + (((c + 1) ^ sw) << 4));
            const v8i va = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2],
                               (int)hi[3]};
            o_acc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, o_acc[dt], 0, 0, 0, 127, 0, 127);
        }
    };

    const int n_sub = cnt * SUB;
    if (n_sub > 0) issue(0, k0, v0);
    for (int i = 0; i < n_sub; i += 2) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (i + 1 < n_sub) issue(i + 1, k1, v1);
        compute(i, k0, v0);
        if (i + 1 < n_sub) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (i + 2 < n_sub) issue(i + 2, k0, v0);
            compute(i + 1, k1, v1);
        }
    }

    const float l_tot = pair_sum(l_run);
    if (q_row < a.N) {
        const bool has = q_ok && l_tot > 0.f;
        const float inv = has ? 1.f / l_tot : 0.f;
        uint16_t* orow = a.o + (int64_t)bh * a.N * 128 + (int64_t)q_row * 128;
        const float* vsc = a.v_scale + (int64_t)bh * 128;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const f32x4 s4 = *reinterpret_cast<const f32x4*>(vsc + 32 * dt + 8 * jj + 4 * half);
                const __bf16 b0 = (__bf16)(o_acc[dt][4 * jj + 0] * s4[0] * inv);
                const __bf16 b1 = (__bf16)(o_acc[dt][4 * jj + 1] * s4[1] * inv);
                const __bf16 b2 = (__bf16)(o_acc[dt][4 * jj + 2] * s4[2] * inv);
                const __bf16 b3 = (__bf16)(o_acc[dt][4 * jj + 3] * s4[3] * inv);
                u32x2 pk;
                pk.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
                pk.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
                *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * jj + 4 * half) = pk;
            }
        if (a.lse && half == 0)
            a.lse[(int64_t)bh * a.N + q_row] = has ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    }
}

}  // namespace vsa

using namespace vsa;

extern "C" int vsa_fp8_quantize(const void* x, int B, int H, int N, int D, int dtype, int kind, uint8_t* out,
                                float* scales, void* stream) {
    const char* fn = "vsa_fp8_quantize";
    if (!x || !out || !scales) return fail(VSA_ERR_INVALID, "%s: null tensor", fn);
    if (!aligned16(x) || !aligned16(out) || !aligned16(scales)) return fail(VSA_ERR_INVALID, "%s: tensors must be 16-byte aligned", fn);
    if (B <= 0 || H <= 0 || N <= 0) return fail(VSA_ERR_INVALID, "%s: B, H, N must be positive", fn);
    if (dtype != VSA_BF16 || D != 128) return fail(VSA_ERR_UNSUPPORTED, "%s: needs bf16 with D = 128", fn);
    if (kind != VSA_FP8_ROWS && kind != VSA_FP8_VT) return fail(VSA_ERR_INVALID, "%s: unknown kind %d", fn, kind);
    const int64_t BH = (int64_t)B * H;
    const int64_t ntile = (N + kF8Block - 1) / kF8Block;
    if (BH * ntile >= (1ll << 31) || (int64_t)N * 128 * 2 >= (1ll << 31)) return fail(VSA_ERR_INVALID, "%s: problem too large", fn);
    hipStream_t s = as_stream(stream);
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    if (kind == VSA_FP8_ROWS) {
        hipLaunchKernelGGL(fp8_quant_rows_kernel, dim3((unsigned)(BH * ntile)), dim3(256), 0, s, xb, out, scales, N,
                           (int)ntile);
    } else {
        // the scales buffer holds the amax bits until the last step
        uint32_t* bits = reinterpret_cast<uint32_t*>(scales);
        const int64_t n = BH * 128;
        hipLaunchKernelGGL(fp8_fill_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, bits, n);
        const int64_t nchunk = (N + kAmaxRows - 1) / kAmaxRows;
        hipLaunchKernelGGL(fp8_vamax_kernel, dim3((unsigned)(BH * nchunk)), dim3(256), 0, s, xb, bits, N, (int)nchunk);
        hipLaunchKernelGGL(fp8_quant_vt_kernel, dim3((unsigned)(BH * ntile)), dim3(256), 0, s, xb, bits, out, N,
                           (int)ntile);
        hipLaunchKernelGGL(fp8_vscale_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, bits, scales, n);
    }
    return launch_status(fn);
}

extern "C" int vsa_block_sparse_attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* vt8,
                                             const float* q_scale, const float* k_scale, const float* v_scale, void* o,
                                             float* lse, int B, int H, int N, int D, int bs, const int32_t* blk_len,
                                             const vsa_blocks* blocks, float scale, void* stream) {
    const char* fn = "vsa_block_sparse_attn_fwd_fp8";
    if (!q8 || !k8 || !vt8 || !q_scale || !k_scale || !v_scale || !o) return fail(VSA_ERR_INVALID, "%s: null tensor", fn);
    if (!aligned16(q8) || !aligned16(k8) || !aligned16(vt8) || !aligned16(o) || !aligned16(v_scale))
        return fail(VSA_ERR_INVALID, "%s: tensors must be 16-byte aligned", fn);
    if (B <= 0 || H <= 0 || N <= 0) return fail(VSA_ERR_INVALID, "%s: B, H, N must be positive", fn);
    if (!blocks) return fail(VSA_ERR_INVALID, "%s: null blocks", fn);
    const bool has_mask = blocks->mask != nullptr;
    const bool has_list = blocks->kv_idx != nullptr || blocks->kv_cnt != nullptr;
    if (has_mask == has_list) return fail(VSA_ERR_INVALID, "%s: give exactly one of mask or (kv_idx, kv_cnt)", fn);
    if (has_list && (!blocks->kv_idx || !blocks->kv_cnt || blocks->max_kv <= 0))
        return fail(VSA_ERR_INVALID, "%s: list form needs kv_idx, kv_cnt and max_kv > 0", fn);
    if (!(scale > 0.f) || !__builtin_isfinite(scale)) return fail(VSA_ERR_INVALID, "%s: scale must be positive and finite", fn);
    if (D != 128 || bs != 128) return fail(VSA_ERR_UNSUPPORTED, "%s: needs D = 128 and bs = 128", fn);
    const int64_t nb = (N + 127) / 128;
    const int64_t BH = (int64_t)B * H;
    if (has_mask && nb > 4096) return fail(VSA_ERR_UNSUPPORTED, "%s: mask form supports at most 4096 blocks", fn);
    if (BH * nb >= (1ll << 31) || (int64_t)N * 128 * 2 >= (1ll << 31)) return fail(VSA_ERR_INVALID, "%s: problem too large", fn);
    F8Args a{};
    a.q = q8; a.k = k8; a.vt = vt8;
    a.q_scale = q_scale; a.k_scale = k_scale; a.v_scale = v_scale;
    a.o = static_cast<uint16_t*>(o);
    a.lse = lse;
    a.blk_len = blk_len;
    a.mask = blocks->mask;
    a.kv_idx = blocks->kv_idx;
    a.kv_cnt = blocks->kv_cnt;
    a.max_kv = has_list ? blocks->max_kv : 0;
    a.N = N; a.nb = (int32_t)nb; a.ntile = (int32_t)((N + kF8Block - 1) / kF8Block);
    a.num_items = (int32_t)(BH * nb);
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    const size_t shm = has_mask ? (((size_t)nb * 2 + 15) & ~(size_t)15) : 0;
    hipLaunchKernelGGL(attn_fwd_fp8_kernel, dim3((unsigned)(BH * nb)), dim3(256), shm, as_stream(stream), a);
    return launch_status(fn);
}
