// Per-head pattern choice from sampled query rows.
//
// Sparse Video-Gen page, "Approach" and "Key results": about 1 % of query rows
// are used to compare each candidate sparse pattern's output with dense
// attention; each head takes the lower-error pattern. Here the error of
// candidate p is the sum over sampled rows and channels of (o_p - o_dense)^2.
//
// Four launches, no tensor is moved:
//  1. bits: for each candidate p and sampled row r, one bit per natural key n,
//     set iff M_p[L_p(r) / bs][L_p(n) / bs] != 0, where L_p is the identity
//     (mask stated in natural order) or the frame-major map (n -> s*T + t).
//  2. main, once per output slot (dense, then each candidate): workgroups of 4
//     waves x 32 sampled rows walk a contiguous range of 128-key tiles (split-K
//     over keys, so that a few hundred rows still fill the chip). Per tile the
//     scores S^T come from MFMA, the slot's bits mask them, an online softmax
//     (max, sum) runs and O^T accumulates. Each (slot, row, split) writes a
//     partial record (m, l, O) to the workspace.
//  3. merge: partial records are combined in split order (exact log-sum-exp
//     rescaling), outputs normalised, squared differences to the dense output
//     summed per 32-row chunk in a fixed order.
//  4. finish: chunk sums added in order; choice = first argmin.
#include <math.h>

#include <algorithm>

#include "mfma_tile.h"

namespace vsa {

constexpr int kProfKT = 128;          // keys per tile
constexpr int kProfRows = 128;        // sampled rows per workgroup
constexpr int kProfMaxP = 4;
constexpr int kProfTargetWG = 1024;

struct ProfPlan {
    int ntiles, RT, S, TPS, chunks, words;
    int64_t rec;                       // floats per partial record
    size_t off_bits, off_part, off_errp, total;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static ProfPlan prof_plan(int B, int H, int64_t N, int D, int R, int P) {
    ProfPlan p;
    p.ntiles = (int)((N + kProfKT - 1) / kProfKT);
    p.RT = (R + kProfRows - 1) / kProfRows;
    int64_t per = (int64_t)p.RT * B * H;
    int S = (int)std::min<int64_t>(16, std::max<int64_t>(1, (kProfTargetWG + per - 1) / per));
    S = std::min(S, p.ntiles);
    p.TPS = (p.ntiles + S - 1) / S;
    p.S = (p.ntiles + p.TPS - 1) / p.TPS;
    p.chunks = (R + 31) / 32;
    p.words = p.ntiles * 4;            // 32-key words, padded to whole tiles
    p.rec = D + 4;                     // m, l, 2 pad, O[D]
    size_t bits = (size_t)P * R * p.words * 4;
    size_t part = (size_t)(P + 1) * B * H * R * p.S * p.rec * 4;
    size_t errp = (size_t)B * H * p.chunks * kProfMaxP * 4;
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
    int32_t R, N, S, TPS, ntiles, words, BH;
    int64_t rec;
    float scale_log2;
    int32_t slot_out[1];               // output slot (0 = dense, 1 + p = candidate p)
    int32_t slot_cand[1];              // candidate whose bits apply, -1 = none
};

template <int D, int NC>
__global__ __launch_bounds__(256) void prof_main_kernel(ProfArgs a) {
    constexpr int KT = kProfKT;
    constexpr int NST = KT / 32, NDT = D / 32;
    __shared__ __attribute__((aligned(16))) uint8_t k_lds[KT * D * 2];
    __shared__ __attribute__((aligned(16))) uint8_t v_lds[D * KT * 2];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, half = lane >> 5;
    const int split = blockIdx.x, rt = blockIdx.y, bh = blockIdx.z;
    const int64_t head_off = (int64_t)bh * a.N * D;
    const int ri = rt * kProfRows + 32 * w + l32;
    const int r = ri < a.R ? a.rows[ri] : -1;
    const bool row_ok = r >= 0 && r < a.N;
    const bool wave_active = rt * kProfRows + 32 * w < a.R;

    bf16x8 qf[D / 16];
    load_q_frag<D>(qf, a.q + head_off + (int64_t)(row_ok ? r : 0) * D, row_ok, half);

    f32x16 o[NC][NDT];
    float m_run[NC], l_run[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        m_run[c] = -INFINITY;
        l_run[c] = 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[c][dt] = f32x16{};
    }
    const int t0 = split * a.TPS, t1 = min(t0 + a.TPS, a.ntiles);
    for (int t = t0; t < t1; ++t) {
        const int valid = min(KT, a.N - t * KT);
        __syncthreads();
        stage_k_tile<D, KT, 256>(k_lds, a.k + head_off + (int64_t)t * KT * D, valid, tid);
        stage_v_tile<D, KT, 256>(v_lds, a.v + head_off + (int64_t)t * KT * D, valid, tid);
        __syncthreads();
        if (!wave_active) continue;
        f32x16 s[NST];
        tile_scores<D, KT>(s, k_lds, qf, l32, half);
        if (valid < KT) {
#pragma unroll
            for (int st = 0; st < NST; ++st)
#pragma unroll
                for (int x = 0; x < 16; ++x)
                    if (acc_key(st, x, half) >= valid) s[st][x] = -INFINITY;
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            uint32_t wbits[NST];
            const int cand = a.slot_cand[c];
#pragma unroll
            for (int st = 0; st < NST; ++st) {
                wbits[st] = 0xffffffffu;
                if (cand >= 0)
                    wbits[st] = row_ok ? a.bits[((int64_t)cand * a.R + ri) * a.words + 4 * t + st] : 0u;
            }
            float mx = -INFINITY;
#pragma unroll
            for (int st = 0; st < NST; ++st)
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const int bit = 8 * (x >> 2) + 4 * half + (x & 3);
                    if ((wbits[st] >> bit) & 1u) mx = fmaxf(mx, s[st][x]);
                }
            mx = fmaxf(mx, swap_halves(mx));
            const float m_new = fmaxf(m_run[c], mx * a.scale_log2);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = exp2f(m_run[c] - m_use);
            float psum = 0.f;
            bf16x8 pf[NST][2];
#pragma unroll
            for (int st = 0; st < NST; ++st)
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const int bit = 8 * (x >> 2) + 4 * half + (x & 3);
                    float p = ((wbits[st] >> bit) & 1u) ? exp2f(fmaf(s[st][x], a.scale_log2, -m_use)) : 0.f;
                    psum += p;
                    pf[st][x >> 3][x & 7] = (__bf16)p;
                }
            l_run[c] = l_run[c] * alpha + psum;
            m_run[c] = m_new;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int x = 0; x < 16; ++x) o[c][dt][x] *= alpha;
            tile_pv<D, KT>(o[c], v_lds, pf, l32, half);
        }
    }
    if (!wave_active) return;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const float l_tot = l_run[c] + swap_halves(l_run[c]);
        if (ri >= a.R) continue;
        float* rec = a.part + ((((int64_t)a.slot_out[c] * a.BH + bh) * a.R + ri) * a.S + split) * a.rec;
        if (half == 0) {
            rec[0] = m_run[c];
            rec[1] = l_tot;
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f32x4 v4 = {o[c][dt][4 * j], o[c][dt][4 * j + 1], o[c][dt][4 * j + 2], o[c][dt][4 * j + 3]};
                *reinterpret_cast<f32x4*>(rec + 4 + 32 * dt + 8 * j + 4 * half) = v4;
            }
    }
}

struct MergeArgs {
    const float* part;
    float* errp;
    int32_t R, S, BH, D, P, chunks;
    int64_t rec;
};

// One workgroup per (bh, chunk of 32 rows). Thread t handles channel t % D of
// rows 256 / D apart; partial records are merged in split order.
__global__ __launch_bounds__(256) void prof_merge_kernel(MergeArgs a) {
    __shared__ float red[kProfMaxP][256];
    const int bh = blockIdx.y, chunk = blockIdx.x;
    const int d = threadIdx.x % a.D;
    const int rstep = 256 / a.D;
    float acc[kProfMaxP] = {0.f, 0.f, 0.f, 0.f};
    for (int rr = threadIdx.x / a.D; rr < 32; rr += rstep) {
        const int ri = chunk * 32 + rr;
        if (ri >= a.R) break;
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
                    const float f = exp2f(ms - m);
                    l += recs[s * a.rec + 1] * f;
                    ov += recs[s * a.rec + 4 + d] * f;
                }
            }
            const float out = l > 0.f ? ov / l : 0.f;
            if (slot == 0) dense = out;
            else acc[slot - 1] += (out - dense) * (out - dense);
        }
    }
    for (int p = 0; p < a.P; ++p) red[p][threadIdx.x] = acc[p];
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s)
            for (int p = 0; p < a.P; ++p) red[p][threadIdx.x] += red[p][threadIdx.x + s];
        __syncthreads();
    }
    if ((int)threadIdx.x < a.P) a.errp[((int64_t)bh * a.chunks + chunk) * kProfMaxP + threadIdx.x] = red[threadIdx.x][0];
}

__global__ void prof_finish_kernel(const float* errp, int BH, int chunks, int P, float* err, int32_t* choice) {
    int bh = blockIdx.x * blockDim.x + threadIdx.x;
    if (bh >= BH) return;
    int best = 0;
    float best_e = INFINITY;
    for (int p = 0; p < P; ++p) {
        float e = 0.f;
        for (int c = 0; c < chunks; ++c) e += errp[((int64_t)bh * chunks + c) * kProfMaxP + p];
        err[(int64_t)bh * P + p] = e;
        if (e < best_e) { best_e = e; best = p; }
    }
    choice[bh] = best;
}

}  // namespace vsa

using namespace vsa;

extern "C" size_t vsa_profile_workspace_bytes(int B, int H, vsa_grid g, int D, int R, int P) {
    if (B <= 0 || H <= 0 || g.T <= 0 || g.Hh <= 0 || g.W <= 0 || R <= 0 || P <= 0 || P > kProfMaxP ||
        (D != 64 && D != 128))
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
    if (D != 128 && D != 64) return fail(VSA_ERR_UNSUPPORTED, "vsa_profile_heads: D must be 64 or 128");
    if (bs != 64 && bs != 128) return fail(VSA_ERR_UNSUPPORTED, "vsa_profile_heads: bs must be 64 or 128");
    if (P < 1 || P > kProfMaxP) return fail(VSA_ERR_INVALID, "vsa_profile_heads: P must be in [1, %d]", kProfMaxP);
    if (R < 1) return fail(VSA_ERR_INVALID, "vsa_profile_heads: R must be >= 1");
    if (!(scale > 0.f) || !__builtin_isfinite(scale)) return fail(VSA_ERR_INVALID, "vsa_profile_heads: scale must be positive and finite");
    for (int p = 0; p < P; ++p)
        if (cand_layout[p] != 0 && cand_layout[p] != 1)
            return fail(VSA_ERR_INVALID, "vsa_profile_heads: cand_layout[%d] must be 0 or 1", p);
    const int64_t N = (int64_t)g.T * g.Hh * g.W;
    if (N >= (1ll << 31) || R > N) return fail(VSA_ERR_INVALID, "vsa_profile_heads: bad N or R");
    if ((int64_t)B * H > 65535) return fail(VSA_ERR_INVALID, "vsa_profile_heads: B*H too large");
    const ProfPlan pl = prof_plan(B, H, N, D, R, P);
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
    pa.R = R; pa.N = (int32_t)N; pa.S = pl.S; pa.TPS = pl.TPS; pa.ntiles = pl.ntiles; pa.words = pl.words;
    pa.BH = B * H; pa.rec = pl.rec;
    pa.scale_log2 = (float)((double)scale * 1.4426950408889634);
    dim3 grid(pl.S, pl.RT, B * H);
    // One output slot per pass (dense first, then each candidate): a single set
    // of accumulators keeps the kernel free of register spills.
    for (int slot = 0; slot <= P; ++slot) {
        pa.slot_out[0] = slot;
        pa.slot_cand[0] = slot - 1;
        if (D == 128) hipLaunchKernelGGL((prof_main_kernel<128, 1>), grid, dim3(256), 0, s, pa);
        else hipLaunchKernelGGL((prof_main_kernel<64, 1>), grid, dim3(256), 0, s, pa);
        st = launch_status("vsa_profile_heads (main)");
        if (st) return st;
    }

    MergeArgs ma;
    ma.part = pa.part; ma.errp = reinterpret_cast<float*>(ws + pl.off_errp);
    ma.R = R; ma.S = pl.S; ma.BH = B * H; ma.D = D; ma.P = P; ma.chunks = pl.chunks; ma.rec = pl.rec;
    hipLaunchKernelGGL(prof_merge_kernel, dim3(pl.chunks, B * H), dim3(256), 0, s, ma);
    st = launch_status("vsa_profile_heads (merge)");
    if (st) return st;
    hipLaunchKernelGGL(prof_finish_kernel, dim3((B * H + 63) / 64), dim3(64), 0, s, ma.errp, B * H, pl.chunks, P,
                       err, choice);
    return launch_status("vsa_profile_heads (finish)");
}
