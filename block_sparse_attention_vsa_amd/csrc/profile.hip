// Per-head pattern choice from sampled query rows.
//
// Sparse Video-Gen page, "Approach" and "Key results": about 1 % of query rows
// are used to compare each candidate sparse pattern's output with dense
// attention; each head takes the lower-error pattern. Here the error of
// candidate p is the sum over sampled rows and channels of (o_p - o_dense)^2.
//
// Launches (no tensor is moved):
//  1. bits: for each candidate p and sampled row r, one bit per natural key n,
//     set iff M_p[L_p(r) / bs][L_p(n) / bs] != 0, where L_p is the identity
//     (mask stated in natural order) or the frame-major map (n -> s*T + t).
//  2. main (one launch for the dense output and up to two candidates):
//     workgroups of 4 waves cover 64 sampled rows, 16 per wave, on the
//     16x16x32 bf16 MFMA (scores and P V), so three output sets over all 128
//     channels fit 2 waves per SIMD and no score is computed twice. Each
//     workgroup walks a contiguous range of 64-key sub-tiles (split-K over
//     keys, so a few hundred rows still fill the chip), with K and V streamed
//     into double-buffered LDS by DMA and the candidates' bit words fetched one
//     sub-tile ahead. Per sub-tile: S^T once on MFMA, the dense online softmax
//     (lazy running offset), and P V for the dense set. A candidate reuses the
//     dense probabilities with its unkept keys zeroed (the same running offset
//     serves every set); its P V products run on every sub-tile, with P zero
//     where the candidate keeps nothing. Each (slot, row, split) writes a
//     partial record (m, l, O).
//  3. merge: one wave per (b, h, sampled row) combines the partial records of
//     every slot (exact log-sum-exp rescaling, the splits' loads in flight
//     together), normalises them and sums each candidate's squared difference
//     to the dense output.
//  4. finish: per (b, h) the row sums are added in a fixed tree order; choice =
//     first argmin.
#include <math.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "mfma_tile.h"

namespace vsa {

constexpr int kProfRows = 64;         // sampled rows per workgroup (2 row groups x 32)
constexpr int kProfMaxP = 4;
constexpr int kProfTargetWG = 512;    // 256 CUs x 2 resident workgroups
constexpr int kProfCandPerLaunch = 2; // candidates sharing one main launch with the dense set

struct ProfPlan {
    int nsub, RT, S, TPS, words;
    int64_t rec;                       // floats per partial record
    size_t off_bits, off_part, off_errp, total;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static ProfPlan prof_plan(int B, int H, int64_t N, int D, int R, int P) {
    ProfPlan p;
    p.nsub = (int)((N + kSubKeys - 1) / kSubKeys);
    p.RT = (R + kProfRows - 1) / kProfRows;
    int64_t per = (int64_t)p.RT * B * H;
    // as many key splits as keep the whole grid resident at once (2 workgroups per CU)
    int S = (int)std::min<int64_t>(32, std::max<int64_t>(1, kProfTargetWG / per));
    S = std::min(S, p.nsub);
    p.TPS = (p.nsub + S - 1) / S;
    p.S = (p.nsub + p.TPS - 1) / p.TPS;
    p.words = 2 * p.nsub;              // 32-key words, whole sub-tiles
    p.rec = D + 4;                     // m, l, 2 pad, O[D]
    size_t bits = (size_t)P * R * p.words * 4;
    size_t part = (size_t)(P + 1) * B * H * R * p.S * p.rec * 4;
    size_t errp = (size_t)B * H * R * kProfMaxP * 4;
    p.off_bits = 0;
    p.off_part = align256(bits);
    p.off_errp = p.off_part + align256(part);
    p.total = p.off_errp + align256(errp);
    return p;
}

struct BitsArgs {
    const int32_t* rows;
    const uint8_t* masks;
    uint32_t* bits;
    int32_t R, N, nb, bs, words, P, T, HW;
    int32_t layout[kProfMaxP];
    FastDiv div_HW, div_bs, div_T;
};

__device__ __forceinline__ uint32_t layout_pos(const BitsArgs& a, int lay, uint32_t n) {
    if (lay == 0) return n;
    uint32_t t = a.div_HW.div(n);
    return (n - t * a.HW) * a.T + t;        // frame-major position of natural token n
}

// One thread per 32-key word; the 32 key positions are computed independently
// (fully unrolled), so the 32 mask-byte loads are in flight together.
// Keep bits of one 32-key word of a row under a mask stated in frame-major
// order: key n = t * HW + s (natural order) sits at frame-major position
// s * T + t, in block (s * T + t) / bs; bit b is set when key 32 wi + b is below
// N and its block is kept in mrow. Consecutive keys of one frame step that
// position by T, so they come in runs of about bs / T keys per block, and the
// word is built run by run: one mask read and two divisions per run instead of
// per key.
__host__ __device__ inline uint32_t fm_word_bits(const uint8_t* mrow, uint32_t wi, uint32_t N, uint32_t T,
                                                 uint32_t HW, uint32_t bs, const FastDiv& div_HW,
                                                 const FastDiv& div_bs, const FastDiv& div_T) {
    const uint32_t n0 = 32u * wi;
    const uint32_t nend = N - n0 > 32u ? n0 + 32u : N;
    if (n0 >= N) return 0u;
    uint32_t word = 0u, n = n0;
    uint32_t t = div_HW.div(n), sp = n - t * HW;
    while (n < nend) {
        const uint32_t seg_end = nend - n < HW - sp ? nend : n + (HW - sp);   // rest of frame t
        while (n < seg_end) {
            const uint32_t pos = sp * T + t;
            const uint32_t blk = div_bs.div(pos);
            const uint32_t run = div_T.div((blk + 1u) * bs - pos + T - 1u);    // keys left in block blk
            const uint32_t end = seg_end - n < run ? seg_end : n + run;
            if (mrow[blk]) word |= (uint32_t)(((1ull << (end - n0)) - 1ull) ^ ((1ull << (n - n0)) - 1ull));
            sp += end - n;
            n = end;
        }
        ++t;
        sp = 0u;
    }
    return word;
}

__global__ __launch_bounds__(256) void prof_bits_kernel(BitsArgs a) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)a.P * a.R * a.words;
    if (e >= total) return;
    const int wi = (int)(e % a.words);
    const int64_t pr = e / a.words;
    const int ri = (int)(pr % a.R);
    const int p = (int)(pr / a.R);
    const int r = a.rows[ri];
    uint32_t word = 0;
    if (r >= 0 && r < a.N && 32 * wi < a.N) {
        const int lay = a.layout[p];
        const uint32_t qblk = a.div_bs.div(layout_pos(a, lay, (uint32_t)r));
        const uint8_t* mrow = a.masks + ((int64_t)p * a.nb + qblk) * a.nb;
        if (lay == 0 && (a.bs & 31) == 0) {
            // natural order, blocks a multiple of 32 keys: the word's keys share one block
            const int valid = min(32, a.N - 32 * wi);
            if (mrow[(32 * wi) / a.bs]) word = valid == 32 ? 0xffffffffu : (1u << valid) - 1u;
        } else if (lay == 0) {
#pragma unroll
            for (int b = 0; b < 32; ++b)
                if (32 * wi + b < a.N && mrow[a.div_bs.div((uint32_t)(32 * wi + b))]) word |= 1u << b;
        } else {
            word = fm_word_bits(mrow, (uint32_t)wi, (uint32_t)a.N, (uint32_t)a.T, (uint32_t)a.HW, (uint32_t)a.bs,
                                a.div_HW, a.div_bs, a.div_T);
        }
    }
    a.bits[e] = word;
}

struct ProfArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* rows;
    const uint32_t* bits;
    float* part;
    int32_t R, N, S, TPS, nsub, words, BH;
    int64_t rec;
    float scale_log2;
    int32_t bits_bytes;                  // size of the bit table
    int32_t write_dense;                 // this launch accumulates and writes slot 0 (dense)
    int32_t cand[kProfCandPerLaunch];    // candidates handled (slot 1 + cand), -1 = none
};

// Sum / max over the four 16-lane groups of a wave (one query per lane n & 15,
// its keys spread over the groups), in a fixed order: every group ends with the
// same bits.
__device__ __forceinline__ float group4_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float group4_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// LDS addressing of the 16x16x32 operands, written as a per-lane base plus
// terms that are immediates or one XOR, so only a few address registers stay
// live across the loop.
//  K (row r at r * 256, chunk c at slot c ^ (r & 15)): the A operand of S^T
//    for key tile tt and channel step kk reads row 16 tt + n, chunk 4 kk + g:
//    byte 4096 tt + ka[kk], ka[kk] = 256 n + 16 (g ^ (n & 3)) + 16 (4 kk ^ (n & 12)).
//  V (pair swizzle: 32-byte pair q of row r at pair q ^ (r & 7)): the V^T
//    operand of P V for channel tile ct (16 channels) and K-step j is two
//    ds_read_b64_tr_b16. The P^T operand of lane group g holds keys
//    32 j + 4 g + [0, 4) (elements 0..3) and 32 j + 16 + 4 g + [0, 4)
//    (elements 4..7), which is how the 16x16 score accumulators hold them; in
//    each 16-lane group, lanes 4 jj .. 4 jj + 3 point at 16 consecutive
//    channels of key jj and lane i receives channel i of the four keys. The
//    byte address is 8192 j + 4096 h + va[ct], va[ct] = vbase ^ 32 ct, with
//    vbase = 256 (4 g + n / 4) + 16 ((n & 3) >> 1) + 8 (n & 1) + 32 ((4 g + n / 4) & 7).
// The per-lane parts are passed through an empty asm so the compiler cannot
// see that their bits are disjoint from the constant parts: it then keeps
// base + constant as an add, which folds into the instruction's offset field,
// instead of an OR that needs a register per address.
struct Op16Addr {
    int ka[4], va[8];               // K: kbase + kx[kk]; V: vbase ^ 32 ct
    __device__ __forceinline__ explicit Op16Addr(int lane) {
        const int g = lane >> 4, n = lane & 15;
        const int kbase = 256 * n + 16 * (g ^ (n & 3));
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            ka[kk] = kbase + 16 * ((4 * kk) ^ (n & 12));
            asm("" : "+v"(ka[kk]));
        }
        const int krow = 4 * g + (n >> 2);     // key row of this lane within a 16-key run
        const int vbase = 256 * krow + 16 * ((n & 3) >> 1) + 8 * (n & 1) + 32 * (krow & 7);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            va[ct] = vbase ^ (32 * ct);
            asm("" : "+v"(va[ct]));
        }
    }
};

__device__ __forceinline__ bf16x8 vt_operand16(const uint8_t* vt, int ct, int j, const Op16Addr& ad) {
    v4i16 part[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint8_t* ptr = vt + 8192 * j + 4096 * h + ad.va[ct];
        part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(ptr));
    }
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int NCAND>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prof_main_kernel(ProfArgs a) {
    constexpr int D = 128, KT = kSubKeys, NS = 1 + NCAND, NCT = D / 16;
    constexpr float TAU = 8.f;
    // two stages as distinct LDS objects, loop unrolled by two: a DMA into one
    // stage is then provably disjoint from reads of the other
    __shared__ __attribute__((aligned(1024))) uint8_t k0[kSubBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t v0[kSubBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t k1[kSubBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t v1[kSubBytes];
    // the workgroup's 64 query rows, K-style swizzle (chunk c of row r at slot c ^ (r & 15)):
    // the Q^T operands are read back just before the scores, so they hold no
    // registers across the P V products
    __shared__ __attribute__((aligned(1024))) uint8_t qs[kProfRows * D * 2];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n16 = lane & 15, g = lane >> 4;     // query of this lane, its key group
    // Workgroups are dealt round-robin over the 8 XCDs; the item order gives
    // each XCD a contiguous range of (b h, split) groups with their row tiles
    // fastest, so the row tiles that stream the same K/V range share one L2.
    const int RTn = (a.R + kProfRows - 1) / kProfRows;
    const int item = xcd_remap((int)blockIdx.x, a.S * RTn * a.BH);
    const int rt = item % RTn, split = (item / RTn) % a.S, bh = item / (RTn * a.S);
    const int64_t head_off = (int64_t)bh * a.N * D;
    const int ri = rt * kProfRows + 16 * w + n16;
    const int r = ri < a.R ? a.rows[ri] : -1;
    const bool row_ok = r >= 0 && r < a.N;
    const bool wave_active = rt * kProfRows + 16 * w < a.R;

    const Op16Addr ad(lane);
    // Q^T operand per 32-channel step kk (channels 32 kk + 8 g .. + 8 of this
    // lane's row) staged in LDS at the same swizzled spot the K operand uses
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        u32x4 t = {0u, 0u, 0u, 0u};
        if (row_ok) t = *reinterpret_cast<const u32x4*>(a.q + head_off + (int64_t)r * D + 32 * kk + 8 * g);
        *reinterpret_cast<u32x4*>(qs + 4096 * w + ad.ka[kk]) = t;
    }

    f32x4 o[NS][NCT];                // O^T tiles: channels 16 ct + 4 g + i, query n16
    float l_run[NS];
    float m_run = -INFINITY;         // running offset shared by all sets
#pragma unroll
    for (int c = 0; c < NS; ++c) {
        l_run[c] = 0.f;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) o[c][ct] = f32x4{};
    }
    const int t0 = split * a.TPS, t1 = min(t0 + a.TPS, a.nsub);
    const SubTileDma<4, kVSwzPair> dma(lane, w);
    const int head_bytes = a.N * D * 2;
    auto issue = [&](int t, uint8_t* kd, uint8_t* vd) {
        dma.issue(kd, vd, a.k + head_off, a.v + head_off, head_bytes, t * KT, w);
    };
    // candidate bit words of this lane's row through a descriptor over the bit
    // table: a 32-bit per-lane row offset (past the table, so reading 0, for a
    // lane without a row) and the sub-tile's word as the scalar offset
    int boff[NCAND];
#pragma unroll
    for (int c = 0; c < NCAND; ++c)
        boff[c] = row_ok ? (int)(((int64_t)a.cand[c] * a.R + ri) * a.words * 4) : a.bits_bytes;
    auto load_bits = [&](int t, uint32_t (&wb)[NCAND][2]) {
#pragma unroll
        for (int c = 0; c < NCAND; ++c)
#pragma unroll
            for (int st = 0; st < 2; ++st) wb[c][st] = buf_load_u32(a.bits, a.bits_bytes, boff[c], (2 * t + st) * 4);
    };
    uint32_t bits_cur[NCAND][2], bits_next[NCAND][2];

    auto compute = [&](int t, const uint8_t* kt, const uint8_t* vt) __attribute__((always_inline)) {
        if (!wave_active) return;
        const int vs = min(KT, a.N - t * KT);
        // S^T tiles: s[tt][i] = score of key 16 tt + 4 g + i for query n16
        bf16x8 qf[D / 32];
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
            qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qs + 4096 * w + ad.ka[kk]));
        f32x4 s[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            s[tt] = f32x4{};
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
                u32x4 kv = *reinterpret_cast<const u32x4*>(kt + 4096 * tt + ad.ka[kk]);
                s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv), qf[kk], s[tt], 0, 0, 0);
            }
        }
        if (vs < KT) {
            const int lim = vs - 4 * g;            // key 16 tt + 4 g + i is valid iff 16 tt + i < lim
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * tt + i >= lim) s[tt][i] = -INFINITY;
        }
        // dense online softmax; its offset serves every set
        float mx = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[tt][i]);
        mx = group4_max(mx);
        const float m_tile = mx * a.scale_log2;
        const bool upd = m_tile > m_run + TAU;
        const float m_new = upd ? m_tile : m_run;
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        if (__ballot(upd)) {
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
#pragma unroll
            for (int c = 0; c < NS; ++c) {
                l_run[c] *= alpha;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) o[c][ct] *= alpha;
            }
        }
        m_run = m_new;
        float ps[2] = {0.f, 0.f};              // per 32-key word: tiles 0, 1 and 2, 3
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s[tt][i] = __builtin_amdgcn_exp2f(fmaf(s[tt][i], a.scale_log2, -m_use));   // p, in place
                ps[tt >> 1] += s[tt][i];
            }
        l_run[0] += ps[0] + ps[1];
        // P^T operands for K-steps j = 0, 1: element e of lane group g is key
        // 32 j + 16 (e >> 2) + 4 g + (e & 3), held in s[2 j + (e >> 2)][e & 3];
        // its bit in the candidate's word j is 16 (e >> 2) + 4 g + (e & 3)
        bool any[NCAND], whole[NCAND];
#pragma unroll
        for (int c = 0; c < NCAND; ++c) {
            const uint32_t b0 = bits_cur[c][0], b1 = bits_cur[c][1];
            any[c] = __ballot((b0 | b1) != 0u) != 0;
            whole[c] = __ballot((b0 + 1u > 1u) || (b1 + 1u > 1u)) == 0;
        }
        bf16x8 pc[NCAND][2];
        // candidates kept key by key first, from the fp32 p
#pragma unroll
        for (int c = 0; c < NCAND; ++c) {
            if (!any[c] || whole[c]) continue;
            float lc = 0.f;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t wb = bits_cur[c][j];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bool keep = (wb >> (16 * (e >> 2) + 4 * g + (e & 3))) & 1u;
                    const float pk = keep ? s[2 * j + (e >> 2)][e & 3] : 0.f;
                    lc += pk;
                    pc[c][j][e] = (__bf16)pk;
                }
            }
            l_run[1 + c] += lc;
        }
        bf16x8 pf[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) pf[j][e] = (__bf16)s[2 * j + (e >> 2)][e & 3];
        // block-aligned candidates: the dense P with dropped lanes zeroed; a
        // candidate no row of the wave keeps here gets P = 0
#pragma unroll
        for (int c = 0; c < NCAND; ++c) {
            if (any[c] && !whole[c]) continue;
            const bf16x8 zero = bf16x8{};
#pragma unroll
            for (int j = 0; j < 2; ++j) pc[c][j] = bits_cur[c][j] ? pf[j] : zero;
            l_run[1 + c] += (bits_cur[c][0] ? ps[0] : 0.f) + (bits_cur[c][1] ? ps[1] : 0.f);
        }
        // P V: each V^T operand feeds every set (a candidate's zero P adds
        // nothing; the matrix cores are not this kernel's bottleneck)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const bf16x8 va = vt_operand16(vt, ct, j, ad);
                if (a.write_dense) o[0][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf[j], o[0][ct], 0, 0, 0);
#pragma unroll
                for (int c = 0; c < NCAND; ++c)
                    o[1 + c][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pc[c][j], o[1 + c][ct], 0, 0, 0);
                // keep at most a few operand reads in flight (registers)

            }
    };
    auto rotate = [&]() {
#pragma unroll
        for (int c = 0; c < NCAND; ++c) {
            bits_cur[c][0] = bits_next[c][0];
            bits_cur[c][1] = bits_next[c][1];
        }
    };
    // the bit words are loaded before the DMA, so waiting for them never waits
    // for the tiles behind them
    if (t0 < t1) {
        load_bits(t0, bits_next);
        issue(t0, k0, v0);
    }
    for (int t = t0; t < t1; t += 2) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        rotate();
        if (t + 1 < t1) {
            load_bits(t + 1, bits_next);
            issue(t + 1, k1, v1);
        }
        compute(t, k0, v0);
        if (t + 1 < t1) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            rotate();
            if (t + 2 < t1) {
                load_bits(t + 2, bits_next);
                issue(t + 2, k0, v0);
            }
            compute(t + 1, k1, v1);
        }
    }
    if (!wave_active) return;
#pragma unroll
    for (int c = 0; c < NS; ++c) {
        if (c == 0 && !a.write_dense) continue;
        const float l_tot = group4_sum(l_run[c]);
        if (ri >= a.R) continue;
        const int slot = c == 0 ? 0 : 1 + a.cand[c - 1];
        float* rec = a.part + ((((int64_t)slot * a.BH + bh) * a.R + ri) * a.S + split) * a.rec;
        if (g == 0) {
            rec[0] = m_run;
            rec[1] = l_tot;
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) *reinterpret_cast<f32x4*>(rec + 4 + 16 * ct + 4 * g) = o[c][ct];
    }
}

struct MergeArgs {
    const float* part;
    float* errp;
    int32_t R, S, BH, P;
    int64_t rec;
};

__device__ __forceinline__ float wave_max_f(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// One wave per (b, h, sampled row), four per workgroup; lane d merges channels
// d and d + 64 of every set. Lane s holds split s's (m, l) (at most 32 splits),
// so the common offset and the weight sum come from one load each; the channel
// loads of the splits are independent of each other. Splits add in split order.
__global__ __launch_bounds__(256) void prof_merge_kernel(MergeArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wv >= (int64_t)a.R * a.BH) return;                 // whole waves leave together
    const int bh = (int)(wv / a.R), ri = (int)(wv % a.R);
    float dense0 = 0.f, dense1 = 0.f;
    for (int slot = 0; slot <= a.P; ++slot) {
        const float* recs = a.part + (((int64_t)slot * a.BH + bh) * a.R + ri) * a.S * a.rec;
        const float ms = lane < a.S ? recs[lane * a.rec] : -INFINITY;
        const float ls = lane < a.S ? recs[lane * a.rec + 1] : 0.f;
        const float m = wave_max_f(ms);
        const float f = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - m);
        const float l = wave_sum_f(ls * f);
        float o0 = 0.f, o1 = 0.f;
#pragma unroll 8
        for (int s = 0; s < a.S; ++s) {
            const float mss = recs[s * a.rec];           // the same address on every lane
            const float fs = (mss == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mss - m);
            o0 += recs[s * a.rec + 4 + lane] * fs;
            o1 += recs[s * a.rec + 68 + lane] * fs;
        }
        const float out0 = l > 0.f ? o0 / l : 0.f, out1 = l > 0.f ? o1 / l : 0.f;
        if (slot == 0) {
            dense0 = out0;
            dense1 = out1;
        } else {
            const float d0 = out0 - dense0, d1 = out1 - dense1;
            const float e = wave_sum_f(d0 * d0 + d1 * d1);
            if (lane == 0) a.errp[((int64_t)bh * a.R + ri) * kProfMaxP + slot - 1] = e;
        }
    }
}

// One workgroup per (b, h): per-row errors summed in a fixed order.
__global__ __launch_bounds__(256) void prof_finish_kernel(const float* errp, int R, int P, float* err,
                                                          int32_t* choice) {
    __shared__ float red[kProfMaxP][256];
    __shared__ float tot[kProfMaxP];
    const int bh = blockIdx.x, t = threadIdx.x;
    for (int p = 0; p < P; ++p) {
        float acc = 0.f;
        for (int ri = t; ri < R; ri += 256) acc += errp[((int64_t)bh * R + ri) * kProfMaxP + p];
        red[p][t] = acc;
    }
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (t < s)
            for (int p = 0; p < P; ++p) red[p][t] += red[p][t + s];
        __syncthreads();
    }
    if (t == 0) {
        int best = 0;
        float best_e = INFINITY;
        for (int p = 0; p < P; ++p) {
            const float e = red[p][0];
            tot[p] = e;
            err[(int64_t)bh * P + p] = e;
            if (e < best_e) { best_e = e; best = p; }
        }
        choice[bh] = best;
    }
}

}  // namespace vsa

using namespace vsa;

extern "C" size_t vsa_profile_workspace_bytes(int B, int H, vsa_grid g, int D, int R, int P) {
    if (B <= 0 || H <= 0 || g.T <= 0 || g.Hh <= 0 || g.W <= 0 || R <= 0 || P <= 0 || P > kProfMaxP || D != 128)
        return 0;
    return prof_plan(B, H, (int64_t)g.T * g.Hh * g.W, D, R, P).total;
}

namespace {

// Host-side checks shared by both entry points; fills the plan.
int profile_check(const char* fn, const void* q, const void* k, const void* v, int B, int H, vsa_grid g, int D,
                  int dtype, int bs, const int32_t* rows, int R, const uint8_t* cand_masks,
                  const int32_t* cand_layout, int P, float scale, const float* err, const int32_t* choice,
                  ProfPlan& pl) {
    if (!q || !k || !v || !rows || !cand_masks || !cand_layout || !err || !choice)
        return fail(VSA_ERR_INVALID, "%s: null pointer", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return fail(VSA_ERR_INVALID, "%s: q, k, v must be 16-byte aligned", fn);
    if (B <= 0 || H <= 0 || g.T <= 0 || g.Hh <= 0 || g.W <= 0) return fail(VSA_ERR_INVALID, "%s: bad sizes", fn);
    if (dtype != VSA_BF16) return fail(VSA_ERR_UNSUPPORTED, "%s: only bf16 inputs", fn);
    if (D != 128) return fail(VSA_ERR_UNSUPPORTED, "%s: D must be 128", fn);
    if (bs < 1 || bs > 1024) return fail(VSA_ERR_INVALID, "%s: bs must be in [1, 1024]", fn);
    if (P < 1 || P > kProfMaxP) return fail(VSA_ERR_INVALID, "%s: P must be in [1, %d]", fn, kProfMaxP);
    if (R < 1) return fail(VSA_ERR_INVALID, "%s: R must be >= 1", fn);
    if (!(scale > 0.f) || !__builtin_isfinite(scale)) return fail(VSA_ERR_INVALID, "%s: scale must be positive and finite", fn);
    for (int p = 0; p < P; ++p)
        if (cand_layout[p] != 0 && cand_layout[p] != 1)
            return fail(VSA_ERR_INVALID, "%s: cand_layout[%d] must be 0 or 1", fn, p);
    const int64_t N = (int64_t)g.T * g.Hh * g.W;
    if (N >= (1ll << 31) || R > N) return fail(VSA_ERR_INVALID, "%s: bad N or R", fn);
    // one head of K or V is addressed through a buffer descriptor of N * D * 2 bytes (32-bit size)
    if (N * D * 2 >= (1ll << 31)) return fail(VSA_ERR_INVALID, "%s: one head exceeds 2 GiB (N too large)", fn);
    if ((int64_t)B * H > 65535 || R > 65535) return fail(VSA_ERR_INVALID, "%s: B*H or R too large", fn);
    pl = prof_plan(B, H, N, D, R, P);
    if ((int64_t)P * R * pl.words * 4 >= (1ll << 31))
        return fail(VSA_ERR_INVALID, "%s: candidate bit table exceeds 2 GiB (R or N too large)", fn);
    return VSA_OK;
}

// The launches of one profile, with the scratch at ws (pl.total bytes). Every
// scratch byte a kernel reads was written earlier in the same sequence, so the
// scratch needs no clearing.
int profile_launch(const void* q, const void* k, const void* v, int B, int H, vsa_grid g, int D, int bs,
                   const int32_t* rows, int R, const uint8_t* cand_masks, const int32_t* cand_layout, int P,
                   float scale, float* err, int32_t* choice, const ProfPlan& pl, uint8_t* ws, hipStream_t s) {
    const int64_t N = (int64_t)g.T * g.Hh * g.W;
    BitsArgs ba;
    ba.rows = rows; ba.masks = cand_masks; ba.bits = reinterpret_cast<uint32_t*>(ws + pl.off_bits);
    ba.R = R; ba.N = (int32_t)N; ba.nb = (int32_t)((N + bs - 1) / bs); ba.bs = bs; ba.words = pl.words; ba.P = P;
    ba.T = g.T; ba.HW = g.Hh * g.W;
    for (int p = 0; p < kProfMaxP; ++p) ba.layout[p] = p < P ? cand_layout[p] : 0;
    ba.div_HW = FastDiv((uint32_t)ba.HW);
    ba.div_bs = FastDiv((uint32_t)bs);
    ba.div_T = FastDiv((uint32_t)ba.T);
    int64_t nbits = (int64_t)P * R * pl.words;
    hipLaunchKernelGGL(prof_bits_kernel, dim3((unsigned)((nbits + 255) / 256)), dim3(256), 0, s, ba);
    int st = launch_status("vsa_profile_heads (bits)");
    if (st) return st;

    ProfArgs pa;
    pa.q = static_cast<const uint16_t*>(q); pa.k = static_cast<const uint16_t*>(k); pa.v = static_cast<const uint16_t*>(v);
    pa.rows = rows; pa.bits = ba.bits; pa.part = reinterpret_cast<float*>(ws + pl.off_part);
    pa.R = R; pa.N = (int32_t)N; pa.S = pl.S; pa.TPS = pl.TPS; pa.nsub = pl.nsub; pa.words = pl.words;
    pa.BH = B * H; pa.rec = pl.rec;
    pa.bits_bytes = (int32_t)((size_t)P * R * pl.words * 4);
    pa.scale_log2 = (float)((double)scale * 1.4426950408889634);
    dim3 grid((unsigned)((int64_t)pl.S * pl.RT * B * H));
    // the dense set and up to two candidates per launch (S recomputed per launch)
    for (int first = 0; first < P; first += kProfCandPerLaunch) {
        const int nc = std::min(kProfCandPerLaunch, P - first);
        pa.write_dense = first == 0;
        for (int c = 0; c < kProfCandPerLaunch; ++c) pa.cand[c] = c < nc ? first + c : -1;
        if (nc == 2) hipLaunchKernelGGL(prof_main_kernel<2>, grid, dim3(256), 0, s, pa);
        else hipLaunchKernelGGL(prof_main_kernel<1>, grid, dim3(256), 0, s, pa);
        st = launch_status("vsa_profile_heads (main)");
        if (st) return st;
    }

    MergeArgs ma;
    ma.part = pa.part; ma.errp = reinterpret_cast<float*>(ws + pl.off_errp);
    ma.R = R; ma.S = pl.S; ma.BH = B * H; ma.P = P; ma.rec = pl.rec;
    hipLaunchKernelGGL(prof_merge_kernel, dim3((unsigned)(((int64_t)R * B * H + 3) / 4)), dim3(256), 0, s, ma);
    st = launch_status("vsa_profile_heads (merge)");
    if (st) return st;
    hipLaunchKernelGGL(prof_finish_kernel, dim3(B * H), dim3(256), 0, s, ma.errp, R, P, err, choice);
    return launch_status("vsa_profile_heads (finish)");
}

}  // namespace

extern "C" int vsa_profile_heads(const void* q, const void* k, const void* v, int B, int H, vsa_grid g, int D,
                                 int dtype, int bs, const int32_t* rows, int R, const uint8_t* cand_masks,
                                 const int32_t* cand_layout, int P, float scale, float* err, int32_t* choice,
                                 void* workspace, size_t ws_bytes, void* stream) {
    const char* fn = "vsa_profile_heads";
    ProfPlan pl;
    const int st = profile_check(fn, q, k, v, B, H, g, D, dtype, bs, rows, R, cand_masks, cand_layout, P, scale, err,
                                 choice, pl);
    if (st != VSA_OK) return st;
    if (!workspace || ws_bytes < pl.total)
        return fail(VSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, pl.total, ws_bytes);
    return profile_launch(q, k, v, B, H, g, D, bs, rows, R, cand_masks, cand_layout, P, scale, err, choice, pl,
                          static_cast<uint8_t*>(workspace), as_stream(stream));
}

// ---------------------------------------------------------------------------
// Allocation-free variant: the profile's scratch (candidate bit table, split-K
// partial records, per-row errors) lives in this static device array instead of
// a caller workspace. The device address of the array is looked up once per
// device (its host-side name is only a stand-in) and kept; every call on a
// device shares that device's copy.
constexpr size_t kProfScratchBytes = (size_t)96 << 20;
static __device__ __align__(256) uint8_t scratch[kProfScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of this device's scratch (looked up on the first call).
int scratch_address(const char* fn, uint8_t** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(VSA_ERR_LAUNCH, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(VSA_ERR_UNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(VSA_ERR_LAUNCH, "%s: hipGetSymbolAddress of the static scratch failed: %s", fn,
                        hipGetErrorString(e));
        g_scratch_dev[dev] = p;
    }
    *out = static_cast<uint8_t*>(g_scratch_dev[dev]);
    return VSA_OK;
}
}  // namespace

extern "C" size_t vsa_profile_scratch_capacity(void) { return kProfScratchBytes; }

extern "C" int vsa_profile_heads_noalloc(const void* q, const void* k, const void* v, int B, int H, vsa_grid g,
                                         int D, int dtype, int bs, const int32_t* rows, int R,
                                         const uint8_t* cand_masks, const int32_t* cand_layout, int P, float scale,
                                         float* err, int32_t* choice, void* stream) {
    const char* fn = "vsa_profile_heads_noalloc";
    ProfPlan pl;
    int st = profile_check(fn, q, k, v, B, H, g, D, dtype, bs, rows, R, cand_masks, cand_layout, P, scale, err,
                           choice, pl);
    if (st != VSA_OK) return st;
    if (pl.total > kProfScratchBytes)
        return fail(VSA_ERR_WORKSPACE,
                    "%s: this problem needs %zu bytes of scratch, more than the %zu bytes of static scratch; "
                    "use vsa_profile_heads with a workspace", fn, pl.total, kProfScratchBytes);
    uint8_t* ws = nullptr;
    st = scratch_address(fn, &ws);
    if (st != VSA_OK) return st;
    return profile_launch(q, k, v, B, H, g, D, bs, rows, R, cand_masks, cand_layout, P, scale, err, choice, pl, ws,
                          as_stream(stream));
}

namespace vsa {

// Host check of fm_word_bits: every word of rows under random masks, against the
// key-by-key rule, on the video grids and small ragged ones.
int profile_selftest_host() {
    const uint32_t shapes[][3] = {{21, 1560, 128}, {33, 3600, 128}, {126, 1560, 128}, {3, 5, 4}, {4, 30, 64},
                                  {7, 9, 8}, {1, 100, 64}, {5, 1, 4}, {2, 33, 64}, {9, 7, 128}};
    uint32_t lcg = 12345u;
    for (const auto& sh : shapes) {
        const uint32_t T = sh[0], HW = sh[1], bs = sh[2], N = T * HW, nb = (N + bs - 1) / bs;
        const FastDiv dH(HW), dB(bs), dT(T);
        std::vector<uint8_t> mrow(nb);
        for (int rep = 0; rep < 2; ++rep) {
            for (auto& m : mrow) {
                lcg = lcg * 1664525u + 1013904223u;
                m = (lcg >> 24) % 5 < 2;
            }
            for (uint32_t wi = 0; 32 * wi < N; ++wi) {
                uint32_t ref = 0;
                for (uint32_t b = 0; b < 32 && 32 * wi + b < N; ++b) {
                    const uint32_t n = 32 * wi + b, t = n / HW, sp = n % HW;
                    if (mrow[(sp * T + t) / bs]) ref |= 1u << b;
                }
                if (fm_word_bits(mrow.data(), wi, N, T, HW, bs, dH, dB, dT) != ref)
                    return fail(VSA_ERR_INVALID, "fm_word_bits wrong at T=%u HW=%u bs=%u word %u", T, HW, bs, wi);
            }
        }
    }
    return VSA_OK;
}

}  // namespace vsa

