// Attention over variable-size clusters in cluster-major storage, on gfx950.
//
// Sparse VideoGen2 page, Abstract: after the semantic-aware permutation the
// critical tokens are dense, so the kernel computes them without padding. Q is
// stored cluster-major by query cluster (cluster a in rows [q_off[a], q_off[a+1])),
// K and V by key cluster (k_off); every query of cluster a attends to the keys
// of the key clusters kept for a:
//   O_i = sum_{j in kept clusters of a} softmax_j(scale <q_i, k_j>) v_j.
//
// One workgroup per (b, h, query cluster, chunk of at most 128 rows), 4 waves of
// 32 rows, Q in registers; the chunks are launched in descending order of their
// kept-key counts, which vary by two orders of magnitude between clusters. The
// kept key clusters are laid end to end into one packed key sequence, walked in
// 64-key sub-tiles: every DMA lane maps its packed position to a row of K / V
// through a per-workgroup LDS table (row minus position for each 16-key group
// inside one cluster; a short walk over the clusters' packed starts for a group
// that spans two), so clusters of any size share sub-tiles and only the last
// sub-tile of a workgroup is partial. The score / softmax / P V core is the one of the block
// kernel (S^T = K Q^T on v_mfma_f32_32x32x16_bf16, online softmax in the log2
// domain with a lazily moved offset, V^T through transposing LDS reads).
#include <math.h>

#include "mfma_tile.h"

namespace vsa {

constexpr int kVarBS = 128;          // query rows per workgroup
constexpr int kVarKT = 64;           // keys per sub-tile
constexpr int kVarMaxMask = 4096;    // key clusters per mask row (mask form)

struct VarArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    const int32_t* q_off;          // [BH, Cq + 1]
    const int32_t* k_off;          // [BH, Ck + 1]
    const uint8_t* mask;           // [BH, Cq, Ck] or null
    const int32_t* kv_idx;         // [BH, Cq, max_kv] or null
    const int32_t* kv_cnt;         // [BH, Cq]
    int32_t max_kv;
    const int32_t* chunk_start;    // [BH, Cq + 1]: first chunk of each query cluster
    int32_t* work;                 // [BH, Cq]: keys kept by each query cluster
    int32_t* order;                // [BH max_chunks]: launch order of the chunks (heaviest first)
    int32_t* n_items;              // [1]: number of chunks
    int32_t N, Cq, Ck, BH, max_chunks, max_entries, max_subs;
    float scale_log2;
};

// chunks of 128 rows per query cluster, as an exclusive scan: one wave per (b, h)
__global__ __launch_bounds__(64) void varlen_chunks_kernel(VarArgs a, int32_t* chunk_start) {
    const int64_t bh = blockIdx.x;
    const int lane = threadIdx.x;
    const int32_t* off = a.q_off + bh * (a.Cq + 1);
    int32_t* out = chunk_start + bh * (a.Cq + 1);
    int run = 0;
    for (int c0 = 0; c0 < a.Cq; c0 += 64) {
        const int c = c0 + lane;
        int v = 0;
        if (c < a.Cq) {
            const int n = off[c + 1] - off[c];
            v = n > 0 ? (n + kVarBS - 1) / kVarBS : 0;
        }
        int x = v;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(x, d);
            if (lane >= d) x += y;
        }
        if (c < a.Cq) out[c] = run + x - v;
        run += __shfl(x, 63);
    }
    if (lane == 0) out[a.Cq] = run;
}

// keys kept by each query cluster: one wave per (b, h, query cluster)
__global__ __launch_bounds__(256) void varlen_work_kernel(VarArgs a) {
    const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (g >= (int64_t)a.BH * a.Cq) return;
    const int64_t bh = g / a.Cq;
    const int32_t* ko = a.k_off + bh * (a.Ck + 1);
    int64_t keys = 0;
    if (a.mask) {
        const uint8_t* row = a.mask + g * a.Ck;
        for (int c = lane; c < a.Ck; c += 64)
            if (row[c]) keys += ko[c + 1] - ko[c];
    } else {
        const int cnt = min(a.kv_cnt[g], a.max_kv);
        const int32_t* idx = a.kv_idx + g * a.max_kv;
        for (int e = lane; e < cnt; e += 64) {
            const int c = idx[e];
            if ((unsigned)c < (unsigned)a.Ck) keys += ko[c + 1] - ko[c];
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) keys += __shfl_xor(keys, off);
    if (lane == 0) a.work[g] = (int32_t)min<int64_t>(keys, 0x7fffffff);
}

// Launch order: every chunk of every query cluster, by descending kept-key count
// (256 buckets of a counting sort in one workgroup), so that the longest
// workgroups start first. Only the schedule depends on it (the order inside a
// bucket comes from LDS integer atomics); no result does.
__global__ __launch_bounds__(1024) void varlen_order_kernel(VarArgs a) {
    __shared__ int hist[256];
    const int t = threadIdx.x;
    const int pairs = a.BH * a.Cq;
    if (t < 256) hist[t] = 0;
    __syncthreads();
    auto bucket = [&](int g) {
        const int64_t b = (int64_t)a.work[g] * 255 / max(a.N, 1);
        return 255 - (int)min<int64_t>(b, 255);
    };
    auto chunks = [&](int g) {
        const int bh = g / a.Cq, c = g - bh * a.Cq;
        const int32_t* cs = a.chunk_start + (int64_t)bh * (a.Cq + 1);
        return cs[c + 1] - cs[c];
    };
    for (int g = t; g < pairs; g += 1024) atomicAdd(&hist[bucket(g)], chunks(g));
    __syncthreads();
    if (t == 0) {
        int run = 0;
        for (int b = 0; b < 256; ++b) {
            const int h = hist[b];
            hist[b] = run;
            run += h;
        }
        *a.n_items = run;
    }
    __syncthreads();
    for (int g = t; g < pairs; g += 1024) {
        const int n = chunks(g);
        if (n <= 0) continue;
        const int pos = atomicAdd(&hist[bucket(g)], n);
        const int bh = g / a.Cq, c = g - bh * a.Cq;
        const int first = a.chunk_start[(int64_t)bh * (a.Cq + 1) + c];
        for (int u = 0; u < n; ++u) a.order[pos + u] = bh * a.max_chunks + first + u;
    }
}

// Exclusive scan of one value per thread over a 256-thread workgroup; returns
// the prefix and sets `total` (all threads). `tmp` holds 4 ints.
__device__ __forceinline__ int block_scan_256(int v, int* tmp, int& total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    if (lane == 63) tmp[w] = x;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int t = tmp[u];
        before += (u < w) ? t : 0;
        total += t;
    }
    __syncthreads();
    return before + x - v;
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_varlen_kernel(VarArgs a) {
    constexpr int D = 128, KT = kVarKT, NST = KT / 32, SUBB = KT * D * 2, WAVES = 4, THREADS = 256;
    constexpr float TAU = 8.f, TAU_POW = 256.f;
    __shared__ __attribute__((aligned(1024))) uint8_t k0[SUBB];
    __shared__ __attribute__((aligned(1024))) uint8_t v0[SUBB];
    __shared__ __attribute__((aligned(1024))) uint8_t k1[SUBB];
    __shared__ __attribute__((aligned(1024))) uint8_t v1[SUBB];
    __shared__ int scan_tmp[4];
    __shared__ int wave_cnt[WAVES];
    // dynamic: pp[max_entries + 1] | kst[max_entries] | t0[max_subs] | gd[4 max_subs] | list16[Ck] (mask form)
    extern __shared__ __attribute__((aligned(16))) int32_t dyn[];
    int32_t* pp = dyn;
    int32_t* kst = pp + a.max_entries + 1;
    int32_t* t0 = kst + a.max_entries;
    int32_t* gd = t0 + a.max_subs;
    int16_t* list16 = reinterpret_cast<int16_t*>(gd + 4 * a.max_subs);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS copy targets stay scalar
    const int l32 = lane & 31, half = lane >> 5;
    if ((int)blockIdx.x >= ld_const(a.n_items, 0)) return;     // past the last chunk (uniform)
    const int item = ld_const(a.order, (int)blockIdx.x);
    const int bh = item / a.max_chunks, ci = item - bh * a.max_chunks;
    const int32_t* cs = a.chunk_start + (int64_t)bh * (a.Cq + 1);
    int lo = 0, hi = a.Cq;                                      // cs[lo] <= ci < cs[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (ld_const(cs, mid) <= ci) lo = mid;
        else hi = mid;
    }
    const int qa = lo;
    const int32_t* qo = a.q_off + (int64_t)bh * (a.Cq + 1);
    const int q0 = ld_const(qo, qa) + (ci - ld_const(cs, qa)) * kVarBS;
    // rows outside [0, N) (malformed offsets) are never read or written
    const int valid_q = q0 < 0 ? 0 : max(0, min(kVarBS, min(ld_const(qo, qa + 1), a.N) - q0));
    const bool wave_active = 32 * w < valid_q;
    const int64_t head_off = (int64_t)bh * a.N * D;
    const int64_t row_item = (int64_t)bh * a.Cq + qa;

    // ---- kept key clusters and the packed-sequence table --------------------------
    int cnt;
    const int32_t* list_g = nullptr;
    if (a.mask) {
        cnt = compact_mask_row<THREADS>(a.mask + row_item * a.Ck, a.Ck, list16, wave_cnt);
    } else {
        cnt = min(ld_const(a.kv_cnt, row_item), a.max_kv);
        list_g = a.kv_idx + row_item * a.max_kv;
    }
    const int32_t* ko = a.k_off + (int64_t)bh * (a.Ck + 1);
    int L = 0;
    for (int e0 = 0; e0 < cnt; e0 += THREADS) {
        const int e = e0 + tid;
        int len = 0, start = 0;
        if (e < cnt) {
            const int c = list_g ? list_g[e] : (int)list16[e];
            if ((unsigned)c < (unsigned)a.Ck) {
                start = ko[c];
                len = ko[c + 1] - start;
            }
        }
        int tot;
        const int pos = L + block_scan_256(len, scan_tmp, tot);
        if (e < cnt) {
            pp[e] = pos;
            kst[e] = start;
        }
        L += tot;
    }
    L = min(L, a.max_subs * KT);          // repeated clusters cannot overrun the table
    if (tid == 0) pp[cnt] = L;
    __syncthreads();
    // t0: first entry of each sub-tile; gd: row - position for every 16-key group
    // that lies inside one entry, INT_MIN for a group that spans entries
    for (int e = tid; e < cnt; e += THREADS) {
        const int p0 = pp[e], p1 = min(pp[e + 1], L);
        if (p1 <= p0) continue;
        for (int i = (p0 + KT - 1) / KT; i * KT < p1; ++i) t0[i] = e;
        for (int g = p0 >> 4; g <= (p1 - 1) >> 4; ++g)
            gd[g] = (16 * g >= p0 && 16 * g + 16 <= p1) ? kst[e] - p0 : INT_MIN;
    }
    __syncthreads();
    const int n_sub = (L + KT - 1) / KT;

    const SubTileDma<WAVES, kVSwz4, KT> dma(lane, w);
    const SubVtAddr vad(lane);
    const SubKAddr kad(lane);
    const int head_bytes = a.N * D * 2;
    constexpr int IPW = SubTileDma<WAVES, kVSwz4, KT>::IPW;
    static_assert(WAVES == 4 && IPW == 4, "copy instruction u of a wave covers 16-key group u of the sub-tile");
    // copy instruction u of wave w covers keys 4 w + (lane >> 4) of the sub-tile's
    // 16-key group u, so the group, and its entry in gd, are wave-uniform
    const int key_in_group = 4 * w + (lane >> 4);
    auto issue = [&](int i, uint8_t* kd, uint8_t* vd) {
        // every table read comes before the first copy: the compiler cannot tell
        // the tables from the stage buffers, and an LDS read after a copy would
        // wait for that copy to land
        int row[IPW];
#pragma unroll
        for (int u = 0; u < IPW; ++u) {
            const int g16 = 4 * i + u;
            const int p = 16 * g16 + key_in_group;
            const int d = __builtin_amdgcn_readfirstlane(gd[g16]);
            if (d != INT_MIN) {
                row[u] = p < L ? d + p : a.N;                         // past the packed keys: zeros
            } else {                                                  // the group spans entries: walk
                row[u] = a.N;
                if (p < L) {
                    int e = t0[i];
                    while (e + 1 < cnt && pp[e + 1] <= p) ++e;
                    row[u] = kst[e] + (p - pp[e]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < IPW; ++u) {
            const int ins = w + WAVES * u;
            dma16(a.k + head_off, head_bytes, kd + ins * 1024, row[u] * 256 + dma.ck[u % SubTileDma<WAVES, kVSwz4, KT>::NCLS], 0);
            dma16(a.v + head_off, head_bytes, vd + ins * 1024, row[u] * 256 + dma.cv, 0);
        }
    };

    const int q_local = 32 * w + l32;
    const int q_row = q0 + q_local;
    const bool q_ok = q_local < valid_q;
    bf16x8 qf[D / 16];
    load_q_frag<D>(qf, a.q + head_off + (int64_t)q_row * D, q_ok, half);

    f32x16 o_acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o_acc[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    auto compute = [&](int i, const uint8_t* kt, const uint8_t* vt) __attribute__((always_inline)) {
        const int vs = min(KT, L - i * KT);
        if (!wave_active) return;
        f32x16 s[NST];
        sub_scores_ahead<NST>(s, kt, qf, kad);
        bf16x8 vfirst[NST][2];
        sub_pv_first<NST>(vfirst, vt, vad);
        if (vs < KT) {
#pragma unroll
            for (int st = 0; st < NST; ++st)
#pragma unroll
                for (int x = 0; x < 16; ++x)
                    if (acc_key(st, x, half) >= vs) s[st][x] = -INFINITY;
        }
        // p is formed first under the current offset, which only moves when some
        // p exceeds 2^TAU: a lane whose p sum to at most 2^TAU has none, so the
        // row maximum is taken only when some lane's sum passes 2^TAU
        bf16x8 pf[NST][2];
        float lsum;
        auto probs = [&](float m_use) __attribute__((always_inline)) {
            float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < NST; ++st)
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[st][x], a.scale_log2, -m_use));
                    ps[x & 3] += p;
                    pf[st][x >> 3][x & 7] = (__bf16)p;
                }
            lsum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
        };
        probs(m_run == -INFINITY ? 0.f : m_run);
        const bool stays = m_run != -INFINITY && lsum <= TAU_POW;
        if (__ballot(!stays)) {
            float mx = -INFINITY;
#pragma unroll
            for (int st = 0; st < NST; ++st)
#pragma unroll
                for (int x = 0; x < 16; ++x) mx = fmaxf(mx, s[st][x]);
            mx = pair_max(mx);
            const float m_tile = mx * a.scale_log2;
            const bool upd = m_tile > m_run + TAU;
            const float m_new = upd ? m_tile : m_run;
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            if (__ballot(upd)) {
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int x = 0; x < 16; ++x) o_acc[dt][x] *= alpha;
                probs(m_use);
            }
            m_run = m_new;
        }
        l_run += lsum;
        sub_pv_ahead<NST>(o_acc, vt, pf, vfirst, vad);
    };

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
    if (q_ok) {
        const bool has = l_tot > 0.f;
        const float inv = has ? 1.f / l_tot : 0.f;
        uint16_t* orow = a.o + head_off + (int64_t)q_row * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const __bf16 b0 = (__bf16)(o_acc[dt][4 * jj + 0] * inv);
                const __bf16 b1 = (__bf16)(o_acc[dt][4 * jj + 1] * inv);
                const __bf16 b2 = (__bf16)(o_acc[dt][4 * jj + 2] * inv);
                const __bf16 b3 = (__bf16)(o_acc[dt][4 * jj + 3] * inv);
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

struct VarPlan {
    size_t off_cs, off_work, off_order, off_n, total;
};

static VarPlan varlen_plan(int64_t BH, int N, int Cq) {
    VarPlan p;
    const int64_t max_chunks = N / kVarBS + Cq;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    p.off_cs = 0;
    p.off_work = al((size_t)BH * (Cq + 1) * 4);
    p.off_order = p.off_work + al((size_t)BH * Cq * 4);
    p.off_n = p.off_order + al((size_t)BH * max_chunks * 4);
    p.total = p.off_n + 256;
    return p;
}

extern "C" size_t vsa_varlen_attn_workspace_bytes(int B, int H, int N, int Cq) {
    if (B <= 0 || H <= 0 || N <= 0 || Cq <= 0) return 0;
    return varlen_plan((int64_t)B * H, N, Cq).total;
}

extern "C" int vsa_varlen_sparse_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                          int H, int N, int D, int dtype, const int32_t* q_off, int Cq,
                                          const int32_t* k_off, int Ck, const vsa_blocks* blocks, float scale,
                                          void* workspace, size_t ws_bytes, void* stream) {
    const char* fn = "vsa_varlen_sparse_attn_fwd";
    if (!q || !k || !v || !o || !q_off || !k_off) return fail(VSA_ERR_INVALID, "%s: null tensor", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(VSA_ERR_INVALID, "%s: tensors must be 16-byte aligned", fn);
    if (B <= 0 || H <= 0 || N <= 0 || Cq <= 0 || Ck <= 0) return fail(VSA_ERR_INVALID, "%s: B, H, N, Cq, Ck must be positive", fn);
    if (!blocks) return fail(VSA_ERR_INVALID, "%s: null blocks", fn);
    const bool has_mask = blocks->mask != nullptr;
    const bool has_list = blocks->kv_idx != nullptr || blocks->kv_cnt != nullptr;
    if (has_mask == has_list) return fail(VSA_ERR_INVALID, "%s: give exactly one of mask or (kv_idx, kv_cnt)", fn);
    if (has_list && (!blocks->kv_idx || !blocks->kv_cnt || blocks->max_kv <= 0))
        return fail(VSA_ERR_INVALID, "%s: list form needs kv_idx, kv_cnt and max_kv > 0", fn);
    if (!(scale > 0.f) || !__builtin_isfinite(scale)) return fail(VSA_ERR_INVALID, "%s: scale must be positive and finite", fn);
    if (dtype != VSA_BF16 || D != 128) return fail(VSA_ERR_UNSUPPORTED, "%s: needs bf16 with D = 128", fn);
    if (has_mask && Ck > kVarMaxMask) return fail(VSA_ERR_UNSUPPORTED, "%s: mask form supports at most %d key clusters", fn, kVarMaxMask);
    const int64_t BH = (int64_t)B * H;
    const int max_chunks = N / kVarBS + Cq;              // sum over clusters of ceil(n / 128) never exceeds this
    const int max_entries = has_mask ? Ck : blocks->max_kv;
    const int max_subs = (N + kVarKT - 1) / kVarKT;
    const size_t shm = ((size_t)(2 * max_entries + 1 + 5 * max_subs) * 4 + (has_mask ? (size_t)Ck * 2 : 0) + 15) & ~(size_t)15;
    if (shm > 64 * 1024) return fail(VSA_ERR_UNSUPPORTED, "%s: block lists too long for one workgroup", fn);
    if (BH * max_chunks >= (1ll << 31) || (int64_t)N * D * 2 >= (1ll << 31))
        return fail(VSA_ERR_INVALID, "%s: problem too large", fn);
    const size_t need = vsa_varlen_attn_workspace_bytes(B, H, N, Cq);
    if (!workspace || ws_bytes < need)
        return fail(VSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need, ws_bytes);
    VarArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.o = static_cast<uint16_t*>(o);
    a.lse = lse;
    a.q_off = q_off;
    a.k_off = k_off;
    a.mask = blocks->mask;
    a.kv_idx = blocks->kv_idx;
    a.kv_cnt = blocks->kv_cnt;
    a.max_kv = has_list ? blocks->max_kv : 0;
    const VarPlan pl = varlen_plan(BH, N, Cq);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    a.chunk_start = reinterpret_cast<const int32_t*>(ws + pl.off_cs);
    a.work = reinterpret_cast<int32_t*>(ws + pl.off_work);
    a.order = reinterpret_cast<int32_t*>(ws + pl.off_order);
    a.n_items = reinterpret_cast<int32_t*>(ws + pl.off_n);
    a.N = N; a.Cq = Cq; a.Ck = Ck; a.BH = (int32_t)BH;
    a.max_chunks = max_chunks; a.max_entries = max_entries; a.max_subs = max_subs;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    hipStream_t s = as_stream(stream);
    hipLaunchKernelGGL(varlen_chunks_kernel, dim3((unsigned)BH), dim3(64), 0, s, a,
                       reinterpret_cast<int32_t*>(ws + pl.off_cs));
    hipLaunchKernelGGL(varlen_work_kernel, dim3((unsigned)((BH * Cq + 3) / 4)), dim3(256), 0, s, a);
    hipLaunchKernelGGL(varlen_order_kernel, dim3(1), dim3(1024), 0, s, a);
    hipLaunchKernelGGL(attn_varlen_kernel, dim3((unsigned)(BH * max_chunks)), dim3(256), shm, s, a);
    return launch_status(fn);
}
