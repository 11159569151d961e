// Block-sparse attention backward on gfx950: dQ, dK, dV.
//
// USV page, Abstract and Figure 2 caption: the sparse attention is trained end
// to end; OSP-Next page, "Method": sparse fine-tuning. The gradients of
// O_i = sum_j softmax_j(scale <q_i, k_j>) v_j over the kept keys J(i) follow
// from the chain rule (P_ij = exp(S_ij - LSE_i) with the forward's LSE):
//   dV_j = sum_i P_ij dO_i,  dP_ij = <dO_i, v_j>,  dS_ij = P_ij (dP_ij - Delta_i),
//   Delta_i = <dO_i, O_i>,   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,
// every sum over kept (query block, key block) tiles only.
//
// Launches (no floating-point atomics; every sum has a fixed order):
//  1. prep: per row, Delta_i in fp32 and LSE_i * log2(e) (+inf for a row that
//     keeps nothing or is not valid, so its P is 0), both padded to whole blocks.
//  2. lists: the block mask (built from the lists for the list form), then for
//     every key block the ascending list of query blocks that keep it.
//  3. dQ: one workgroup per (b, h, query block), like the forward: per kept
//     64-key sub-tile, S^T = K Q^T and dP^T = V dO^T on MFMA (Q and dO held in
//     registers), P^T and dS^T in fp32 on the VALU, dQ^T += K^T dS^T through
//     transposing LDS reads of the same K tile.
//  4. dK and dV: one workgroup per (b, h, key block), two waves per 32 keys
//     (one forms S and P and adds to dV, the other forms dP, takes P through
//     LDS and adds to dK); consecutive key blocks go to one XCD, where they share
//     most of their query tiles in its L2.
#include <math.h>

#include "mfma_tile.h"

namespace vsa {

// The TileAddr products of mfma_tile.h with each operand read issued one step ahead of
// the MFMA that consumes it (scheduling groups: 0x100 LDS reads, 0x008 MFMA),
// so the MFMAs do not each wait out the LDS latency of their own read.

// Two row-operand chains over the same 32-row half-tile st of two tiles:
// a = tile_a rows x frag_a, b = tile_b rows x frag_b, interleaved.
template <int SWZA, int SWZB>
__device__ __forceinline__ void tile_rows_mma2_ahead(f32x16& a, f32x16& b, const uint8_t* tile_a, const uint8_t* tile_b,
                                                     int st, const bf16x8 (&frag_a)[8], const bf16x8 (&frag_b)[8],
                                                     const TileAddr<SWZA>& ad_a, const TileAddr<SWZB>& ad_b) {
    a = f32x16{};
    b = f32x16{};
    u32x4 ra[2], rb[2];
    ra[0] = *reinterpret_cast<const u32x4*>(tile_a + 8192 * st + ad_a.rows[0]);
    rb[0] = *reinterpret_cast<const u32x4*>(tile_b + 8192 * st + ad_b.rows[0]);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        if (kk + 1 < 8) {
            ra[(kk + 1) & 1] = *reinterpret_cast<const u32x4*>(tile_a + 8192 * st + ad_a.rows[kk + 1]);
            rb[(kk + 1) & 1] = *reinterpret_cast<const u32x4*>(tile_b + 8192 * st + ad_b.rows[kk + 1]);
        }
        a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ra[kk & 1]), frag_a[kk], a, 0, 0, 0);
        b = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, rb[kk & 1]), frag_b[kk], b, 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
#pragma unroll
    for (int kk = 0; kk < 7; ++kk) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
}

// One row-operand chain (tile_rows_mma_at with reads one step ahead).
template <int SWZ>
__device__ __forceinline__ f32x16 tile_rows_mma_ahead(const uint8_t* tile, int st, const bf16x8 (&frag)[8],
                                                      const TileAddr<SWZ>& ad) {
    f32x16 s = f32x16{};
    u32x4 r[2];
    r[0] = *reinterpret_cast<const u32x4*>(tile + 8192 * st + ad.rows[0]);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        if (kk + 1 < 8) r[(kk + 1) & 1] = *reinterpret_cast<const u32x4*>(tile + 8192 * st + ad.rows[kk + 1]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, r[kk & 1]), frag[kk], s, 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
#pragma unroll
    for (int kk = 0; kk < 7; ++kk) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    return s;
}

// acc[dt] += (transposed tile, keys 32 st + [0, 32)) x frag[g] over dt and g, in
// the order dt, g; the operands of dt + 1 are read while dt's MFMAs run.
template <int SWZ>
__device__ __forceinline__ void tile_tr_mma_ahead(f32x16 (&acc)[4], const uint8_t* tile, int st,
                                                  const bf16x8 (&frag)[2], const TileAddr<SWZ>& ad) {
    bf16x8 op[2][2];
#pragma unroll
    for (int g = 0; g < 2; ++g) op[0][g] = tile_tr_operand_at(tile, 0, st, g, ad);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        if (dt + 1 < 4) {
#pragma unroll
            for (int g = 0; g < 2; ++g) op[(dt + 1) & 1][g] = tile_tr_operand_at(tile, dt + 1, st, g, ad);
        }
#pragma unroll
        for (int g = 0; g < 2; ++g)
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[dt & 1][g], frag[g], acc[dt], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 2);
#pragma unroll
    for (int dt = 0; dt < 3; ++dt) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 2);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 2);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 2);
}


constexpr int kBwdMaxMask = 4096;      // key blocks per mask row (mask form)

struct BwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* o;
    const uint16_t* dout;
    const float* lse;
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    const int32_t* blk_len;
    const uint8_t* mask;       // block mask [B, H, nb, nb] (given, or built from the lists)
    const int32_t* kv_idx;     // list form (dQ kernel), or null
    const int32_t* kv_cnt;
    int32_t max_kv;
    float* lse2;               // [B H, nb bs]: LSE log2(e), +inf where P must be 0
    float* delta;              // [B H, nb bs]
    int32_t* qt_idx;           // [B H, nb, nb]: query blocks keeping each key block, ascending
    int32_t* qt_cnt;           // [B H, nb]
    int32_t H, N, nb, bs, BH;
    float scale, scale_log2;
};

__device__ __forceinline__ int bwd_block_valid(const int32_t* blk_len, int b, int BS, int N) {
    const int exist = min(BS, N - b * BS);
    return blk_len ? min(ld_const(blk_len, b), exist) : exist;
}

// ---- 1. prep: Delta and the base-2 LSE, 4 rows per wave (16 lanes x 16 bytes) ----
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
    const int64_t g = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);   // padded row id
    const int sub = threadIdx.x & 15;
    const int64_t rows_pad = (int64_t)a.nb * a.bs;
    if (g >= (int64_t)a.BH * rows_pad) return;
    const int64_t bh = g / rows_pad;
    const int i = (int)(g - bh * rows_pad);
    bool valid = i < a.N;
    if (valid && a.blk_len) valid = (i % a.bs) < a.blk_len[i / a.bs];
    float acc = 0.f;
    if (valid) {
        const int64_t off = (bh * a.N + i) * 128 + 8 * sub;
        const u32x4 ov = *reinterpret_cast<const u32x4*>(a.o + off);
        const u32x4 dv = *reinterpret_cast<const u32x4*>(a.dout + off);
        const bf16x8 ob = __builtin_bit_cast(bf16x8, ov), db = __builtin_bit_cast(bf16x8, dv);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf((float)ob[e], (float)db[e], acc);
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 16);
    if (sub == 0) {
        const float l = valid ? a.lse[bh * a.N + i] : -INFINITY;
        a.lse2[g] = (l == -INFINITY) ? INFINITY : l * 1.4426950408889634f;
        a.delta[g] = valid ? acc : 0.f;
    }
}

// ---- 2. block mask from the lists (list form), then its transpose as lists ----
__global__ __launch_bounds__(256) void bwd_fill_u8_kernel(uint8_t* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0;
}

// One wave per (b h, query block) row of the lists.
__global__ __launch_bounds__(256) void bwd_list_to_mask_kernel(BwdArgs a, uint8_t* mask) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= (int64_t)a.BH * a.nb) return;
    const int cnt = min(a.kv_cnt[row], a.max_kv);
    const int32_t* idx = a.kv_idx + row * a.max_kv;
    for (int c = lane; c < cnt; c += 64) {
        const int kb = idx[c];
        if ((unsigned)kb < (unsigned)a.nb) mask[row * a.nb + kb] = 1;
    }
}

// Transpose of the block mask into ascending per-key-block lists. A workgroup
// takes 64 key blocks (one per lane, so every mask row is read as one 64-byte
// segment) of one (b, h); its 16 waves split the query blocks into 16 ranges,
// count their kept entries, and write them at offsets from a prefix over ranges.
constexpr int kTrWaves = 16;
constexpr int kTrChunk = 8;
__global__ __launch_bounds__(kTrWaves * 64) void bwd_transpose_kernel(BwdArgs a, int col_groups) {
    __shared__ int part[kTrWaves][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t bh = blockIdx.x / col_groups;
    const int kb = (int)(blockIdx.x - bh * col_groups) * 64 + lane;
    const bool col_ok = kb < a.nb;
    const int R = (a.nb + kTrWaves - 1) / kTrWaves;
    const int r0 = min(a.nb, w * R), r1 = min(a.nb, r0 + R);
    const uint8_t* m = a.mask + bh * a.nb * (int64_t)a.nb + kb;
    int c = 0;
    if (col_ok)
        for (int qb = r0; qb < r1; qb += kTrChunk) {
            uint8_t x[kTrChunk];
#pragma unroll
            for (int u = 0; u < kTrChunk; ++u) x[u] = (qb + u < r1) ? m[(int64_t)(qb + u) * a.nb] : 0;
#pragma unroll
            for (int u = 0; u < kTrChunk; ++u) c += x[u] != 0;
        }
    part[w][lane] = c;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int u = 0; u < kTrWaves; ++u) {
        const int x = part[u][lane];
        off += (u < w) ? x : 0;
        tot += x;
    }
    if (!col_ok) return;
    int32_t* out = a.qt_idx + (bh * a.nb + kb) * (int64_t)a.nb + off;
    for (int qb = r0; qb < r1; qb += kTrChunk) {
        uint8_t x[kTrChunk];        // loaded before any store: the stores may alias nothing they read
#pragma unroll
        for (int u = 0; u < kTrChunk; ++u) x[u] = (qb + u < r1) ? m[(int64_t)(qb + u) * a.nb] : 0;
#pragma unroll
        for (int u = 0; u < kTrChunk; ++u)
            if (x[u]) *out++ = qb + u;
    }
    if (w == 0) a.qt_cnt[bh * a.nb + kb] = tot;
}

// Stores a 128-channel accumulator row (channel 32 dt + acc_key(0, x, half) in
// element x of acc[dt]) as bf16, times `mul`; zeros when `ok` is false (a padding
// row: written as 0 whatever its inputs held).
__device__ __forceinline__ void store_row_bf16(uint16_t* dst_row, const f32x16 (&acc)[4], float mul, bool ok,
                                               int half) {
    auto val = [&](float x) { return (__bf16)(ok ? x * mul : 0.f); };
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const __bf16 b0 = val(acc[dt][4 * jj + 0]);
            const __bf16 b1 = val(acc[dt][4 * jj + 1]);
            const __bf16 b2 = val(acc[dt][4 * jj + 2]);
            const __bf16 b3 = val(acc[dt][4 * jj + 3]);
            u32x2 pk;
            pk.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
            pk.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
            *reinterpret_cast<u32x2*>(dst_row + 32 * dt + 8 * jj + 4 * half) = pk;
        }
}

// ---- 3. dQ: one workgroup per (b, h, query block), 32 queries per wave ----------
template <int BS>
__global__ __launch_bounds__(BS * 2) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq_kernel(BwdArgs a) {
    constexpr int D = 128, KT = (BS == 128) ? 64 : 32, NST = KT / 32, SUBB = KT * D * 2;
    constexpr int WAVES = BS / 32, THREADS = WAVES * 64, SUB = BS / KT;
    // K: row operand for S^T and transposed operand for dQ^T (both-ways swizzle);
    // V: row operand for dP^T
    __shared__ __attribute__((aligned(1024))) uint8_t k0[SUBB];
    __shared__ __attribute__((aligned(1024))) uint8_t v0[SUBB];
    __shared__ __attribute__((aligned(1024))) uint8_t k1[SUBB];
    __shared__ __attribute__((aligned(1024))) uint8_t v1[SUBB];
    extern __shared__ __attribute__((aligned(16))) int16_t list_lds[];   // mask form only
    __shared__ int wave_cnt[WAVES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS copy targets stay scalar
    const int l32 = lane & 31, half = lane >> 5;
    const int nkb = a.nb;
    const int item = xcd_remap(blockIdx.x, a.BH * a.nb);
    const int bh = item / a.nb, qb = item - bh * a.nb;
    const int64_t head_off = (int64_t)bh * a.N * D;
    const int valid_q = bwd_block_valid(a.blk_len, qb, BS, a.N);
    const bool wave_active = 32 * w < valid_q;

    int cnt;
    const int32_t* list_g = nullptr;
    if (a.kv_idx) {
        cnt = min(ld_const(a.kv_cnt, item), a.max_kv);
        list_g = a.kv_idx + (int64_t)item * a.max_kv;
    } else {
        cnt = compact_mask_row<THREADS>(a.mask + (int64_t)item * nkb, nkb, list_lds, wave_cnt);
    }
    auto sub_valid = [&](int i, int& kb) -> int {
        kb = list_g ? ld_const(list_g, i / SUB) : (int)list_lds[i / SUB];
        if ((unsigned)kb >= (unsigned)nkb) return 0;
        const int v = bwd_block_valid(a.blk_len, kb, BS, a.N) - (i % SUB) * KT;
        return v < 0 ? 0 : (v > KT ? KT : v);
    };
    const PairTileDma<WAVES, kSwzBoth, kSwzRows, KT> dma(lane, w);
    const TileAddr<kSwzBoth> adk(lane);
    const TileAddr<kSwzRows> adv(lane);
    const int head_bytes = a.N * D * 2;
    auto issue = [&](int i, uint8_t* kd, uint8_t* vd) {
        int kb;
        if (sub_valid(i, kb) == 0) return;
        dma.issue(kd, vd, a.k + head_off, a.v + head_off, head_bytes, kb * BS + (i % SUB) * KT, w);
    };

    const int q_local = 32 * w + l32;
    const int q_row = qb * BS + q_local;
    const bool q_ok = q_local < valid_q;
    bf16x8 qf[8], dof[8];
    load_q_frag<D>(qf, a.q + head_off + (int64_t)q_row * D, q_ok, half);
    load_q_frag<D>(dof, a.dout + head_off + (int64_t)q_row * D, q_ok, half);
    const int64_t prow = (int64_t)bh * a.nb * BS + q_row;      // padded row id
    const float lse2 = a.lse2[prow];                           // +inf: P = 0 for this row
    const float dlt = a.delta[prow];

    f32x16 acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};

    auto compute = [&](int i, const uint8_t* kt, const uint8_t* vt) __attribute__((always_inline)) {
        int kb;
        const int vs = sub_valid(i, kb);
        if (!wave_active || vs == 0) return;
        // one 32-key half at a time keeps the live scores within the register budget
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            f32x16 s, dp;                                            // S^T = K Q^T, dP^T = V dO^T
            tile_rows_mma2_ahead(s, dp, kt, vt, st, qf, dof, adk, adv);
            bf16x8 dsf[2];
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                float p = __builtin_amdgcn_exp2f(fmaf(s[x], a.scale_log2, -lse2));
                if (acc_key(st, x, half) >= vs) p = 0.f;
                dsf[x >> 3][x & 7] = (__bf16)(p * (dp[x] - dlt));
            }
            tile_tr_mma_ahead(acc, kt, st, dsf, adk);                // dQ^T += K^T dS^T
            __builtin_amdgcn_sched_barrier(0);                       // keep each half's read order to itself
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
    if (q_row < a.N) store_row_bf16(a.dq + head_off + (int64_t)q_row * D, acc, a.scale, q_ok, half);
}

// ---- 4. dK and dV: one workgroup per (b, h, key block) -------------------------
// Each 32-key group of the block has two waves: the P wave holds K in registers
// and, per kept query sub-tile, forms S = Q K^T (the Q tile as row operand, so a
// lane holds one key and the accumulator rows are queries), P = exp2(S scale
// log2 e - lse2), hands P (fp32) to its partner through LDS and adds dO^T P to
// dV^T; the dS wave holds V, forms dP = dO V^T meanwhile, then takes P and adds
// Q^T dS, dS = P (dP - Delta), to dK^T. Both tiles are read as row and as
// transposed operand (both-ways swizzle). S is thus formed once per pair for dK
// and dV, and each Q / dO tile is streamed into LDS once for both.
template <int BS>
__global__ __launch_bounds__(BS * 4) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dkv_kernel(BwdArgs a) {
    constexpr int D = 128, KT = (BS == 128) ? 64 : 32, NST = KT / 32, SUBB = KT * D * 2;
    constexpr int G = BS / 32, WAVES = 2 * G, SUB = BS / KT;
    __shared__ __attribute__((aligned(1024))) uint8_t q0[SUBB];
    __shared__ __attribute__((aligned(1024))) uint8_t o0[SUBB];
    __shared__ __attribute__((aligned(1024))) uint8_t q1[SUBB];
    __shared__ __attribute__((aligned(1024))) uint8_t o1[SUBB];
    __shared__ __attribute__((aligned(16))) float ld0[2 * KT];     // lse2 | delta of the sub-tile's queries
    __shared__ __attribute__((aligned(16))) float ld1[2 * KT];
    __shared__ __attribute__((aligned(16))) float pex[G * NST * 1024];   // P, [group][st][x / 4][lane][4]

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int half = lane >> 5;
    // waves w and w + G share a SIMD (waves are placed round-robin), so each
    // SIMD carries one P wave and one dS wave of the same key group
    const bool ds_wave = w >= G;
    const int kg = ds_wave ? w - G : w;
    const int item = xcd_remap(blockIdx.x, a.BH * a.nb);
    const int bh = item / a.nb, kb = item - bh * a.nb;
    const int64_t head_off = (int64_t)bh * a.N * D;
    const int valid_k = bwd_block_valid(a.blk_len, kb, BS, a.N);
    const bool active = 32 * kg < valid_k;
    const int k_local = 32 * kg + (lane & 31);
    const int k_row = kb * BS + k_local;
    const bool k_ok = k_local < valid_k;

    const int cnt = ld_const(a.qt_cnt, item);
    const int32_t* list_g = a.qt_idx + (int64_t)item * a.nb;
    const PairTileDma<WAVES, kSwzBoth, kSwzBoth, KT> dma(lane, w);
    const TileAddr<kSwzBoth> ad(lane);
    const int head_bytes = a.N * D * 2;
    const float* lse2_head = a.lse2 + (int64_t)bh * a.nb * BS;
    const float* delta_head = a.delta + (int64_t)bh * a.nb * BS;
    const int ld_bytes = a.nb * BS * 4;
    auto issue = [&](int i, uint8_t* qd, uint8_t* od, float* ldd) {
        const int qb = ld_const(list_g, i / SUB);
        const int row0 = qb * BS + (i % SUB) * KT;
        dma.issue(qd, od, a.q + head_off, a.dout + head_off, head_bytes, row0, w);
        // lse2 and delta of the KT queries: 4 floats per lane, lanes [0, KT / 4) of wave 0
        if (w == 0 && lane < KT / 4) {
            dma16(lse2_head, ld_bytes, ldd, row0 * 4 + lane * 16, 0);
            dma16(delta_head, ld_bytes, ldd + KT, row0 * 4 + lane * 16, 0);
        }
    };

    bf16x8 kv[8];                                     // K (P wave) or V (dS wave)
    load_q_frag<D>(kv, (ds_wave ? a.v : a.k) + head_off + (int64_t)k_row * D, k_ok, half);
    f32x4* pg = reinterpret_cast<f32x4*>(pex) + kg * NST * 256;

    f32x16 acc[4];                                    // dV^T (P wave) or dK^T (dS wave)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};

    auto compute = [&](const uint8_t* qt, const uint8_t* ot, const float* ldt) __attribute__((always_inline)) {
        bf16x8 pf[NST][2];
        f32x16 dp[NST];
        // phase 1: S and P (P wave) | dP (dS wave)
        if (active) {
            if (!ds_wave) {
#pragma unroll
                for (int st = 0; st < NST; ++st) {
                    const f32x16 s = tile_rows_mma_ahead(qt, st, kv, ad);       // S = Q K^T: lane = key
#pragma unroll
                    for (int xg = 0; xg < 4; ++xg) {
                        // queries 32 st + 8 xg + 4 half + [0, 4) of the sub-tile
                        const f32x4 l4 = *reinterpret_cast<const f32x4*>(ldt + 32 * st + 8 * xg + 4 * half);
                        f32x4 p4;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float p = __builtin_amdgcn_exp2f(fmaf(s[4 * xg + e], a.scale_log2, -l4[e]));
                            p4[e] = k_ok ? p : 0.f;
                            pf[st][xg >> 1][4 * (xg & 1) + e] = (__bf16)p4[e];
                        }
                        pg[(st * 4 + xg) * 64 + lane] = p4;
                    }
                }
            } else {
#pragma unroll
                for (int st = 0; st < NST; ++st) dp[st] = tile_rows_mma_ahead(ot, st, kv, ad);   // dP = dO V^T
            }
        }
        lds_barrier();                                // P visible to the dS waves; the next stage's copy runs on
        // phase 2: dV^T += dO^T P (P wave) | dS, dK^T += Q^T dS (dS wave)
        if (!active) return;
        if (!ds_wave) {
#pragma unroll
            for (int st = 0; st < NST; ++st) {
                tile_tr_mma_ahead(acc, ot, st, pf[st], ad);                    // dV^T += dO^T P
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int st = 0; st < NST; ++st) {
                bf16x8 dsf[2];
#pragma unroll
                for (int xg = 0; xg < 4; ++xg) {
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(ldt + KT + 32 * st + 8 * xg + 4 * half);
                    const f32x4 p4 = pg[(st * 4 + xg) * 64 + lane];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        dsf[xg >> 1][4 * (xg & 1) + e] = (__bf16)(p4[e] * (dp[st][4 * xg + e] - d4[e]));
                }
                tile_tr_mma_ahead(acc, qt, st, dsf, ad);                        // dK^T += Q^T dS
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    const int n_sub = cnt * SUB;
    if (n_sub > 0) issue(0, q0, o0, ld0);
    for (int i = 0; i < n_sub; i += 2) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();                              // stage ready; the previous sub-tile's P consumed
        if (i + 1 < n_sub) issue(i + 1, q1, o1, ld1);
        compute(q0, o0, ld0);
        if (i + 1 < n_sub) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (i + 2 < n_sub) issue(i + 2, q0, o0, ld0);
            compute(q1, o1, ld1);
        }
    }
    if (k_row < a.N) {
        uint16_t* dst = (ds_wave ? a.dk : a.dv) + head_off + (int64_t)k_row * D;
        store_row_bf16(dst, acc, ds_wave ? a.scale : 1.f, k_ok, half);
    }
}

struct BwdPlan {
    size_t off_lse2, off_delta, off_mask, off_qt_idx, off_qt_cnt, total;
};

static size_t bwd_align(size_t x) { return (x + 255) & ~(size_t)255; }

static BwdPlan bwd_plan(int64_t BH, int64_t nb, int bs, bool need_mask) {
    BwdPlan p;
    const size_t rows = (size_t)BH * nb * bs;
    p.off_lse2 = 0;
    p.off_delta = p.off_lse2 + bwd_align(rows * 4);
    p.off_mask = p.off_delta + bwd_align(rows * 4);
    p.off_qt_idx = p.off_mask + (need_mask ? bwd_align((size_t)BH * nb * nb) : 0);
    p.off_qt_cnt = p.off_qt_idx + bwd_align((size_t)BH * nb * nb * 4);
    p.total = p.off_qt_cnt + bwd_align((size_t)BH * nb * 4);
    return p;
}

}  // namespace vsa

using namespace vsa;

extern "C" size_t vsa_attn_bwd_workspace_bytes(int B, int H, int N, int bs, int list_form) {
    if (B <= 0 || H <= 0 || N <= 0 || (bs != 64 && bs != 128)) return 0;
    const int64_t nb = (N + (int64_t)bs - 1) / bs;
    return bwd_plan((int64_t)B * H, nb, bs, list_form != 0).total;
}

extern "C" int vsa_block_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                         const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int D,
                                         int dtype, int bs, const int32_t* blk_len, const vsa_blocks* blocks,
                                         float scale, void* workspace, size_t ws_bytes, void* stream) {
    const char* fn = "vsa_block_sparse_attn_bwd";
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return fail(VSA_ERR_INVALID, "%s: null tensor", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv))
        return fail(VSA_ERR_INVALID, "%s: tensors must be 16-byte aligned", fn);
    if (B <= 0 || H <= 0 || N <= 0) return fail(VSA_ERR_INVALID, "%s: B, H, N must be positive", fn);
    if (!blocks) return fail(VSA_ERR_INVALID, "%s: null blocks", fn);
    const bool has_mask = blocks->mask != nullptr;
    const bool has_list = blocks->kv_idx != nullptr || blocks->kv_cnt != nullptr;
    if (has_mask == has_list) return fail(VSA_ERR_INVALID, "%s: give exactly one of mask or (kv_idx, kv_cnt)", fn);
    if (has_list && (!blocks->kv_idx || !blocks->kv_cnt || blocks->max_kv <= 0))
        return fail(VSA_ERR_INVALID, "%s: list form needs kv_idx, kv_cnt and max_kv > 0", fn);
    if (!(scale > 0.f) || !__builtin_isfinite(scale)) return fail(VSA_ERR_INVALID, "%s: scale must be positive and finite", fn);
    if (dtype != VSA_BF16 || D != 128) return fail(VSA_ERR_UNSUPPORTED, "%s: needs bf16 with D = 128", fn);
    if (bs != 64 && bs != 128) return fail(VSA_ERR_UNSUPPORTED, "%s: bs must be 64 or 128 (got %d)", fn, bs);
    const int64_t nb = (N + (int64_t)bs - 1) / bs;
    const int64_t BH = (int64_t)B * H;
    if (has_mask && nb > kBwdMaxMask) return fail(VSA_ERR_UNSUPPORTED, "%s: mask form supports at most %d blocks", fn, kBwdMaxMask);
    if (BH * nb >= (1ll << 31) || (int64_t)N * D * 2 >= (1ll << 31) || BH * nb * nb >= (1ll << 40))
        return fail(VSA_ERR_INVALID, "%s: problem too large", fn);
    const BwdPlan pl = bwd_plan(BH, nb, bs, has_list);
    if (!workspace || ws_bytes < pl.total)
        return fail(VSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, pl.total, ws_bytes);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    BwdArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.o = static_cast<const uint16_t*>(o);
    a.dout = static_cast<const uint16_t*>(dout);
    a.lse = lse;
    a.dq = static_cast<uint16_t*>(dq);
    a.dk = static_cast<uint16_t*>(dk);
    a.dv = static_cast<uint16_t*>(dv);
    a.blk_len = blk_len;
    a.kv_idx = blocks->kv_idx;
    a.kv_cnt = blocks->kv_cnt;
    a.max_kv = has_list ? blocks->max_kv : 0;
    a.lse2 = reinterpret_cast<float*>(ws + pl.off_lse2);
    a.delta = reinterpret_cast<float*>(ws + pl.off_delta);
    a.qt_idx = reinterpret_cast<int32_t*>(ws + pl.off_qt_idx);
    a.qt_cnt = reinterpret_cast<int32_t*>(ws + pl.off_qt_cnt);
    a.H = H; a.N = N; a.nb = (int32_t)nb; a.bs = bs; a.BH = (int32_t)BH;
    a.scale = scale;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    hipStream_t s = as_stream(stream);

    const int64_t prow = BH * nb * bs;
    hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((prow + 15) / 16)), dim3(256), 0, s, a);
    int st = launch_status("vsa_block_sparse_attn_bwd (prep)");
    if (st) return st;
    if (has_list) {
        uint8_t* m = ws + pl.off_mask;
        const int64_t n = BH * nb * nb;
        hipLaunchKernelGGL(bwd_fill_u8_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, m, n);
        hipLaunchKernelGGL(bwd_list_to_mask_kernel, dim3((unsigned)((BH * nb + 3) / 4)), dim3(256), 0, s, a, m);
        a.mask = m;
    } else {
        a.mask = blocks->mask;
    }
    const int col_groups = (int)((nb + 63) / 64);
    hipLaunchKernelGGL(bwd_transpose_kernel, dim3((unsigned)(BH * col_groups)), dim3(kTrWaves * 64), 0, s, a,
                       col_groups);
    st = launch_status("vsa_block_sparse_attn_bwd (lists)");
    if (st) return st;
    // dQ walks the caller's rows (list, or the mask through compaction)
    BwdArgs aq = a;
    if (!has_list) { aq.kv_idx = nullptr; aq.kv_cnt = nullptr; }
    const dim3 grid((unsigned)(BH * nb));
    const size_t shm = has_list ? 0 : (((size_t)nb * 2 + 15) & ~(size_t)15);
    if (bs == 128) {
        hipLaunchKernelGGL((bwd_dq_kernel<128>), grid, dim3(256), shm, s, aq);
        hipLaunchKernelGGL((bwd_dkv_kernel<128>), grid, dim3(512), 0, s, a);
    } else {
        hipLaunchKernelGGL((bwd_dq_kernel<64>), grid, dim3(128), shm, s, aq);
        hipLaunchKernelGGL((bwd_dkv_kernel<64>), grid, dim3(256), 0, s, a);
    }
    return launch_status(fn);
}
