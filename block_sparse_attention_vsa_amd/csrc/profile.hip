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
//     workgroups of 4 waves cover 64 sampled rows; waves 0/1 and 2/3 take the
//     two 32-row groups, and within a group each wave owns one half of the
//     output channels, so three output sets fit 2 waves per SIMD. Each
//     workgroup walks a contiguous range of 64-key sub-tiles (split-K over
//     keys, so a few hundred rows still fill the chip), with K and V streamed
//     into double-buffered LDS by DMA and the candidates' bit words fetched one
//     sub-tile ahead. Per sub-tile: S^T once on MFMA, the dense online softmax
//     (lazy running offset), and P V for the dense set. A candidate reuses the
//     dense probabilities with its unkept keys zeroed (the same running offset
//     serves every set), and its softmax and P V are skipped outright when
//     none of the wave's rows keeps a key of the sub-tile. Each (slot, row,
//     split) writes a partial record (m, l, O).
//  3. merge: one workgroup per (b, h, sampled row) combines the partial records
//     in split order (exact log-sum-exp rescaling), normalises every slot and
//     sums each candidate's squared difference to the dense output.
//  4. finish: per (b, h) the row sums are added in a fixed tree order; choice =
//     first argmin.
#include <math.h>

#include <algorithm>

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
    FastDiv div_HW, div_bs;
};

__device__ __forceinline__ uint32_t layout_pos(const BitsArgs& a, int lay, uint32_t n) {
    if (lay == 0) return n;
    uint32_t t = a.div_HW.div(n);
    return (n - t * a.HW) * a.T + t;        // frame-major position of natural token n
}

__global__ __launch_bounds__(256) void prof_bits_kernel(BitsArgs a) {
    int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    int64_t total = (int64_t)a.P * a.R * a.words;
    if (e >= total) return;
    int wi = (int)(e % a.words);
    int64_t pr = e / a.words;
    int ri = (int)(pr % a.R);
    int p = (int)(pr / a.R);
    int r = a.rows[ri];
    uint32_t word = 0;
    if (r >= 0 && r < a.N) {
        int lay = a.layout[p];
        uint32_t qblk = a.div_bs.div(layout_pos(a, lay, (uint32_t)r));
        const uint8_t* mrow = a.masks + ((int64_t)p * a.nb + qblk) * a.nb;
        for (int b = 0; b < 32; ++b) {
            int n = 32 * wi + b;
            if (n < a.N && mrow[a.div_bs.div(layout_pos(a, lay, (uint32_t)n))]) word |= 1u << b;
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

template <int NCAND>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prof_main_kernel(ProfArgs a) {
    constexpr int D = 128, KT = kSubKeys, NS = 1 + NCAND;
    constexpr float TAU = 8.f;
    // two stages as distinct LDS objects, loop unrolled by two: a DMA into one
    // stage is then provably disjoint from reads of the other
    __shared__ __attribute__((aligned(1024))) uint8_t k0[kSubBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t v0[kSubBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t k1[kSubBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t v1[kSubBytes];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, half = lane >> 5;
    const int rg = w & 1, chh = w >> 1;             // row group, channel half
    const int split = blockIdx.x, rt = blockIdx.y, bh = blockIdx.z;
    const int64_t head_off = (int64_t)bh * a.N * D;
    const int ri = rt * kProfRows + 32 * rg + l32;
    const int r = ri < a.R ? a.rows[ri] : -1;
    const bool row_ok = r >= 0 && r < a.N;
    const bool wave_active = rt * kProfRows + 32 * rg < a.R;

    bf16x8 qf[D / 16];
    load_q_frag<D>(qf, a.q + head_off + (int64_t)(row_ok ? r : 0) * D, row_ok, half);

    f32x16 o[NS][2];                 // channel tiles 2 chh, 2 chh + 1 of every set
    float l_run[NS];
    float m_run = -INFINITY;         // running offset shared by all sets
#pragma unroll
    for (int c = 0; c < NS; ++c) {
        l_run[c] = 0.f;
        o[c][0] = f32x16{};
        o[c][1] = f32x16{};
    }
    const int t0 = split * a.TPS, t1 = min(t0 + a.TPS, a.nsub);
    const SubTileDma<4> dma(lane, w);
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
    auto pv = [&](f32x16 (&oc)[2], const bf16x8 (&pf)[2][2], const uint8_t* vt) {
#pragma unroll
        for (int dl = 0; dl < 2; ++dl)
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int g = 0; g < 2; ++g)
                    oc[dl] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sub_vt_operand(vt, 2 * chh + dl, st, g, lane),
                                                                     pf[st][g], oc[dl], 0, 0, 0);
    };
    auto compute = [&](int t, const uint8_t* kt, const uint8_t* vt) {
        if (!wave_active) return;
        const int vs = min(KT, a.N - t * KT);
        f32x16 s[2];
        sub_scores(s, kt, qf, l32, half);
        if (vs < KT) {
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int x = 0; x < 16; ++x)
                    if (acc_key(st, x, half) >= vs) s[st][x] = -INFINITY;
        }
        // dense online softmax; its offset serves every set
        float mx = -INFINITY;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int x = 0; x < 16; ++x) mx = fmaxf(mx, s[st][x]);
        mx = pair_max(mx);
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
                for (int dl = 0; dl < 2; ++dl)
#pragma unroll
                    for (int x = 0; x < 16; ++x) o[c][dl][x] *= alpha;
            }
        }
        m_run = m_new;
        float ps[2] = {0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                s[st][x] = __builtin_amdgcn_exp2f(fmaf(s[st][x], a.scale_log2, -m_use));   // p, in place
                ps[st] += s[st][x];
            }
        l_run[0] += ps[0] + ps[1];
        // Candidates: none of the wave's rows keeps a key here -> skipped; every
        // lane's words all-kept or all-dropped (block-aligned masks) -> the dense
        // bf16 P with dropped lanes zeroed, after the dense P V; otherwise (keys
        // kept one by one) P from the fp32 values first, so that those die
        // before the dense bf16 copy exists.
        bool any[NCAND], whole[NCAND];
#pragma unroll
        for (int c = 0; c < NCAND; ++c) {
            const uint32_t b0 = bits_cur[c][0], b1 = bits_cur[c][1];
            any[c] = __ballot((b0 | b1) != 0u) != 0;
            whole[c] = __ballot((b0 + 1u > 1u) || (b1 + 1u > 1u)) == 0;
        }
#pragma unroll
        for (int c = 0; c < NCAND; ++c) {
            if (!any[c] || whole[c]) continue;
            bf16x8 pc[2][2];
            float lc = 0.f;
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const uint32_t wb = bits_cur[c][st];
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const bool keep = (wb >> (8 * (x >> 2) + 4 * half + (x & 3))) & 1u;
                    const float pk = keep ? s[st][x] : 0.f;
                    lc += pk;
                    pc[st][x >> 3][x & 7] = (__bf16)pk;
                }
            }
            l_run[1 + c] += lc;
            pv(o[1 + c], pc, vt);
        }
        bf16x8 pf[2][2];
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int x = 0; x < 16; ++x) pf[st][x >> 3][x & 7] = (__bf16)s[st][x];
        if (a.write_dense) pv(o[0], pf, vt);
#pragma unroll
        for (int c = 0; c < NCAND; ++c) {
            if (!any[c] || !whole[c]) continue;
            const uint32_t b0 = bits_cur[c][0], b1 = bits_cur[c][1];
            const bf16x8 zero = bf16x8{};
            bf16x8 pc[2][2];
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                pc[0][g] = b0 ? pf[0][g] : zero;
                pc[1][g] = b1 ? pf[1][g] : zero;
            }
            l_run[1 + c] += (b0 ? ps[0] : 0.f) + (b1 ? ps[1] : 0.f);
            pv(o[1 + c], pc, vt);
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
        const float l_tot = pair_sum(l_run[c]);
        if (ri >= a.R) continue;
        const int slot = c == 0 ? 0 : 1 + a.cand[c - 1];
        float* rec = a.part + ((((int64_t)slot * a.BH + bh) * a.R + ri) * a.S + split) * a.rec;
        if (chh == 0 && half == 0) {
            rec[0] = m_run;
            rec[1] = l_tot;
        }
#pragma unroll
        for (int dl = 0; dl < 2; ++dl)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f32x4 v4 = {o[c][dl][4 * j], o[c][dl][4 * j + 1], o[c][dl][4 * j + 2], o[c][dl][4 * j + 3]};
                *reinterpret_cast<f32x4*>(rec + 4 + 32 * (2 * chh + dl) + 8 * j + 4 * half) = v4;
            }
    }
}

struct MergeArgs {
    const float* part;
    float* errp;
    int32_t R, S, BH, P;
    int64_t rec;
};

// One workgroup of D = 128 threads per (b, h, sampled row); thread d merges
// channel d of every slot over the splits in order.
__global__ __launch_bounds__(128) void prof_merge_kernel(MergeArgs a) {
    __shared__ float red[kProfMaxP][128];
    const int ri = blockIdx.x, bh = blockIdx.y, d = threadIdx.x;
    float dense = 0.f;
    for (int slot = 0; slot <= a.P; ++slot) {
        const float* recs = a.part + (((int64_t)slot * a.BH + bh) * a.R + ri) * a.S * a.rec;
        float m = -INFINITY;
        for (int s = 0; s < a.S; ++s) m = fmaxf(m, recs[s * a.rec]);
        float l = 0.f, ov = 0.f;
        if (m != -INFINITY) {
            for (int s = 0; s < a.S; ++s) {
                const float ms = recs[s * a.rec];
                if (ms == -INFINITY) continue;
                const float f = __builtin_amdgcn_exp2f(ms - m);
                l += recs[s * a.rec + 1] * f;
                ov += recs[s * a.rec + 4 + d] * f;
            }
        }
        const float out = l > 0.f ? ov / l : 0.f;
        if (slot == 0) dense = out;
        else red[slot - 1][d] = (out - dense) * (out - dense);
    }
    __syncthreads();
    for (int s = 64; s > 0; s >>= 1) {
        if (d < s)
            for (int p = 0; p < a.P; ++p) red[p][d] += red[p][d + s];
        __syncthreads();
    }
    if (d < a.P) a.errp[((int64_t)bh * a.R + ri) * kProfMaxP + d] = red[d][0];
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

extern "C" int vsa_profile_heads(const void* q, const void* k, const void* v, int B, int H, vsa_grid g, int D,
                                 int dtype, int bs, const int32_t* rows, int R, const uint8_t* cand_masks,
                                 const int32_t* cand_layout, int P, float scale, float* err, int32_t* choice,
                                 void* workspace, size_t ws_bytes, void* stream) {
    if (!q || !k || !v || !rows || !cand_masks || !cand_layout || !err || !choice)
        return fail(VSA_ERR_INVALID, "vsa_profile_heads: null pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return fail(VSA_ERR_INVALID, "vsa_profile_heads: q, k, v must be 16-byte aligned");
    if (B <= 0 || H <= 0 || g.T <= 0 || g.Hh <= 0 || g.W <= 0) return fail(VSA_ERR_INVALID, "vsa_profile_heads: bad sizes");
    if (dtype != VSA_BF16) return fail(VSA_ERR_UNSUPPORTED, "vsa_profile_heads: only bf16 inputs");
    if (D != 128) return fail(VSA_ERR_UNSUPPORTED, "vsa_profile_heads: D must be 128");
    if (bs < 1 || bs > 1024) return fail(VSA_ERR_INVALID, "vsa_profile_heads: bs must be in [1, 1024]");
    if (P < 1 || P > kProfMaxP) return fail(VSA_ERR_INVALID, "vsa_profile_heads: P must be in [1, %d]", kProfMaxP);
    if (R < 1) return fail(VSA_ERR_INVALID, "vsa_profile_heads: R must be >= 1");
    if (!(scale > 0.f) || !__builtin_isfinite(scale)) return fail(VSA_ERR_INVALID, "vsa_profile_heads: scale must be positive and finite");
    for (int p = 0; p < P; ++p)
        if (cand_layout[p] != 0 && cand_layout[p] != 1)
            return fail(VSA_ERR_INVALID, "vsa_profile_heads: cand_layout[%d] must be 0 or 1", p);
    const int64_t N = (int64_t)g.T * g.Hh * g.W;
    if (N >= (1ll << 31) || R > N) return fail(VSA_ERR_INVALID, "vsa_profile_heads: bad N or R");
    if ((int64_t)B * H > 65535 || R > 65535) return fail(VSA_ERR_INVALID, "vsa_profile_heads: B*H or R too large");
    const ProfPlan pl = prof_plan(B, H, N, D, R, P);
    if ((int64_t)P * R * pl.words * 4 >= (1ll << 31))
        return fail(VSA_ERR_INVALID, "vsa_profile_heads: candidate bit table exceeds 2 GiB (R or N too large)");
    if (!workspace || ws_bytes < pl.total)
        return fail(VSA_ERR_WORKSPACE, "vsa_profile_heads: workspace of %zu bytes needed (got %zu)", pl.total, ws_bytes);
    hipStream_t s = as_stream(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);

    BitsArgs ba;
    ba.rows = rows; ba.masks = cand_masks; ba.bits = reinterpret_cast<uint32_t*>(ws + pl.off_bits);
    ba.R = R; ba.N = (int32_t)N; ba.nb = (int32_t)((N + bs - 1) / bs); ba.bs = bs; ba.words = pl.words; ba.P = P;
    ba.T = g.T; ba.HW = g.Hh * g.W;
    for (int p = 0; p < kProfMaxP; ++p) ba.layout[p] = p < P ? cand_layout[p] : 0;
    ba.div_HW = FastDiv((uint32_t)ba.HW);
    ba.div_bs = FastDiv((uint32_t)bs);
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
    dim3 grid(pl.S, pl.RT, B * H);
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
    hipLaunchKernelGGL(prof_merge_kernel, dim3(R, B * H), dim3(128), 0, s, ma);
    st = launch_status("vsa_profile_heads (merge)");
    if (st) return st;
    hipLaunchKernelGGL(prof_finish_kernel, dim3(B * H), dim3(256), 0, s, ma.errp, R, P, err, choice);
    return launch_status("vsa_profile_heads (finish)");
}
