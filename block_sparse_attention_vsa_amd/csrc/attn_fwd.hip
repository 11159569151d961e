// Block-sparse attention forward on gfx950.
//
// What is computed (machinebrief LVSA article: block-sparse attention; Sparse
// VideoGen2 page, Abstract: compute only the critical tokens; OSP-Next page,
// "Method": sparse attention kept FlashAttention-compatible): for each (b, h)
// and query i, O_i = sum_j softmax_j(scale <q_i, k_j>) v_j over the valid keys j
// of the key blocks kept for i's query block. Masked tiles are never loaded.
//
// bf16 kernels, one workgroup per (b, h, query block of BS rows), BS/32 waves,
// each wave owning 32 query rows with Q in registers for the whole loop:
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: the accumulator gives each lane one
//    query and 16 keys per 32-key sub-tile, so a query's row sum (and, when it
//    is needed, its row max) is lane-local except for one exchange between the
//    two half-waves;
//  * online softmax in fp32 in the log2 domain (scale * log2 e folded into one
//    FMA before v_exp_f32), P rounded to bf16;
//  * O^T += V^T P^T on the same MFMA with P taken straight from the score
//    registers.
// D = 128 (the video shapes): K and V sub-tiles go from HBM straight into
// double-buffered LDS stages by buffer-load-to-LDS copies (XOR-swizzled 16-byte
// chunks), V stays row-major and its transposed operand is read with
// ds_read_b64_tr_b16, whose key order matches the score accumulator's. The
// running offset moves lazily (only when a tile's maximum exceeds it by more
// than TAU), and P is formed first under the current offset: the tile maximum
// is only taken when some lane's P sum past 2^TAU, i.e. when it may move. The
// kernel also reads rows through the frame-major map and per-head candidate
// choices (the fused permutation paths). D = 64: threads stage K and a
// transposed V (keys contiguous per channel) in LDS, and the offset is the
// exact running maximum.
// Work items are dealt to the XCDs (workgroups go round-robin over the 8 XCDs)
// so that consecutive query blocks of a head run on one XCD and share its L2;
// when 8 heads' K and V outgrow the last-level cache, runs of items are dealt
// instead so the XCDs work on one or two heads at a time; when heads read
// different chosen patterns, every XCD takes an equal share of each pattern's
// heads.
#include <math.h>

#include "mfma_tile.h"

namespace vsa {

constexpr int kMaxMaskBlocks = 4096;   // key blocks a mask row may hold (mask form)
constexpr int64_t kLlcBytes = 256ll << 20;   // MI355X last-level (Infinity) cache

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    const int32_t* blk_len;
    const uint8_t* mask;
    const int32_t* kv_idx;
    const int32_t* kv_cnt;
    int32_t max_kv;
    int32_t H, N, nb;
    int32_t num_items;
    float scale_log2;      // scale * log2(e)
    // frame-major heads (D = 128 bf16 kernel only): rows are read and written
    // through the map natural n = t*HW + s <-> permuted r = s*T + t
    int32_t T, HW;
    FastDiv div_T;
    uint32_t fm_bits[32];  // bit h set: head h is in frame-major order; all zero otherwise
    // per-(b, h) candidate choice read on the device (D = 128 bf16 kernel only):
    // the mask rows come from mask[choice[b, h]] ([n_cand, nb, nb]) and the
    // layout from cand_fm[choice[b, h]]; fm_bits is unused then
    const int32_t* head_choice;
    int32_t n_cand;
    int32_t cand_fm[4];
    // D = 128 bf16 kernel: int16 entries of the row's block list held in LDS (nb
    // for the mask form, max_kv for the list form; 0 = the list form reads its
    // row from global memory); with blk_len, as many valid lengths follow them
    int32_t lds_cap;
    // heads grouped by a host-known kind (frame-major or not) for the XCD deal;
    // all zero = no grouping
    uint64_t head_groups[kGroups];
    // D = 128 bf16 kernel without grouping: 1 = deal runs of items (run_remap)
    // instead of contiguous eighths (xcd_remap)
    int32_t head_runs;
};

// Natural row of permuted row r (r < N) for a frame-major head.
__device__ __forceinline__ int fm_natural(const AttnArgs& a, int r) {
    const uint32_t s = a.div_T.div((uint32_t)r);
    return (int)(((uint32_t)r - s * (uint32_t)a.T) * (uint32_t)a.HW + s);
}


__device__ __forceinline__ int block_valid(const int32_t* blk_len, int b, int BS, int N) {
    int exist = min(BS, N - b * BS);
    return blk_len ? min(blk_len[b], exist) : exist;
}

template <int D, int BS>
__global__ __launch_bounds__(BS * 2) void attn_fwd_bf16_kernel(AttnArgs a) {
    constexpr int WAVES = BS / 32;
    constexpr int THREADS = WAVES * 64;
    constexpr int NST = BS / 32;               // 32-key sub-tiles per key block
    constexpr int NDT = D / 32;                // 32-channel tiles of O

    __shared__ __attribute__((aligned(16))) uint8_t k_lds[BS * D * 2];
    __shared__ __attribute__((aligned(16))) uint8_t v_lds[D * BS * 2];
    __shared__ int16_t list_lds[kMaxMaskBlocks];
    __shared__ int wave_cnt[WAVES];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, half = lane >> 5;
    const int nqb = a.nb, nkb = a.nb;
    const int item = xcd_remap(blockIdx.x, a.num_items);
    const int bh = item / nqb, qb = item - bh * nqb;
    const int64_t head_off = (int64_t)bh * a.N * D;
    const int valid_q = block_valid(a.blk_len, qb, BS, a.N);
    const bool wave_active = 32 * w < valid_q;

    // ---- kept key blocks -------------------------------------------------
    int cnt;
    const int32_t* list_g = nullptr;
    if (a.mask) {
        cnt = compact_mask_row<THREADS>(a.mask + (int64_t)item * nkb, nkb, list_lds, wave_cnt);
    } else {
        cnt = min(a.kv_cnt[item], a.max_kv);
        list_g = a.kv_idx + (int64_t)item * a.max_kv;
    }

    // ---- Q fragment (registers for the whole loop) -------------------------
    const int q_local = 32 * w + l32;
    const int q_row = qb * BS + q_local;
    const bool q_ok = q_local < valid_q;
    bf16x8 qf[D / 16];
    load_q_frag<D>(qf, a.q + head_off + (int64_t)q_row * D, q_ok, half);

    f32x16 o_acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o_acc[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    for (int it = 0; it < cnt; ++it) {
        const int kb = a.mask ? (int)list_lds[it] : list_g[it];
        if ((unsigned)kb >= (unsigned)nkb) continue;           // malformed entry: skip
        const int valid_k = block_valid(a.blk_len, kb, BS, a.N);
        const int64_t key0 = head_off + (int64_t)kb * BS * D;

        __syncthreads();   // previous tile fully consumed
        stage_k_tile<D, BS, THREADS>(k_lds, a.k + key0, valid_k, tid);
        stage_v_tile<D, BS, THREADS>(v_lds, a.v + key0, valid_k, tid);
        __syncthreads();

        if (wave_active) {
            f32x16 s[NST];
            tile_scores<D, BS>(s, k_lds, qf, l32, half);
            if (valid_k < BS) {                                   // keys past the block's valid length
#pragma unroll
                for (int st = 0; st < NST; ++st)
#pragma unroll
                    for (int x = 0; x < 16; ++x)
                        if (acc_key(st, x, half) >= valid_k) s[st][x] = -INFINITY;
            }
            // ---- online softmax (log2 domain) ---------------------------------
            float mx = -INFINITY;
#pragma unroll
            for (int st = 0; st < NST; ++st)
#pragma unroll
                for (int x = 0; x < 16; ++x) mx = fmaxf(mx, s[st][x]);
            mx = fmaxf(mx, swap_halves(mx));
            const float m_new = fmaxf(m_run, mx * a.scale_log2);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            float psum = 0.f;
            bf16x8 pf[NST][2];
#pragma unroll
            for (int st = 0; st < NST; ++st) {
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    float p = __builtin_amdgcn_exp2f(fmaf(s[st][x], a.scale_log2, -m_use));
                    psum += p;
                    pf[st][x >> 3][x & 7] = (__bf16)p;
                }
            }
            l_run = l_run * alpha + psum;
            m_run = m_new;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int x = 0; x < 16; ++x) o_acc[dt][x] *= alpha;
            tile_pv<D, BS>(o_acc, v_lds, pf, l32, half);
        }
    }

    // ---- epilogue ----------------------------------------------------------
    const float l_tot = l_run + swap_halves(l_run);
    if (q_row < a.N) {
        const bool has = q_ok && l_tot > 0.f;
        const float inv = has ? 1.f / l_tot : 0.f;
        uint16_t* orow = a.o + head_off + (int64_t)q_row * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                __bf16 b0 = (__bf16)(o_acc[dt][4 * j + 0] * inv);
                __bf16 b1 = (__bf16)(o_acc[dt][4 * j + 1] * inv);
                __bf16 b2 = (__bf16)(o_acc[dt][4 * j + 2] * inv);
                __bf16 b3 = (__bf16)(o_acc[dt][4 * j + 3] * inv);
                u32x2 pk;
                pk.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
                pk.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
                *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * j + 4 * half) = pk;
            }
        if (a.lse && half == 0)
            a.lse[(int64_t)bh * a.N + q_row] = has ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    }
}

// ---------------------------------------------------------------------------
// bf16, D = 128: the main kernel.
//
// Per workgroup one query block (BS rows, BS/32 waves of 32 rows); the kept key
// blocks are walked in 64-key sub-tiles, double-buffered in LDS:
//  * K and V sub-tiles go from HBM straight into LDS with buffer loads carrying
//    the lds flag (lane l of a wave instruction lands at base + 16 l), so no
//    VGPRs or VALU instructions are spent staging tiles, and the next sub-tile
//    streams in while the current one is computed. Each lane picks the global
//    16-byte chunk that belongs at its LDS slot, which realises an XOR swizzle of
//    the chunks: K row r keeps chunk c at slot c ^ (r & 15), V row r at slot
//    c ^ 4 (r & 3). Those per-lane offsets are fixed for the whole loop; the
//    buffer descriptor spans one head, so rows past its end read as zeros.
//  * The two stages are distinct LDS objects and the loop is unrolled by two, so
//    the compiler can see that a DMA into one stage never aliases reads of the
//    other; the list entries and valid lengths are read through the constant
//    address space (scalar loads), so waiting for them never waits for the DMA.
//    Together this keeps the prefetch asynchronous.
//  * K is read with ds_read_b128 (16 consecutive keys hit 16 distinct slots).
//  * V stays row-major; the MFMA operand V^T comes from ds_read_b64_tr_b16: in a
//    16-lane group, lanes 4j..4j+3 point at 16 consecutive channels of key j, and
//    lane i receives channel i of the four keys. Two such reads give a lane the
//    8 keys that the P^T operand holds in the same k slots.
//  * Softmax keeps a running offset m per query that only moves when a tile's
//    max exceeds it by more than 8 (log2 units), so O is rarely rescaled; p stays
//    below 2^8 and the final O / l is unchanged.
// Work item of workgroup `bid` when every head reads its chosen candidate: the
// heads are grouped by choice (an invalid choice is a group of its own) and
// each XCD takes an equal contiguous share of every group (group_remap), so a
// mix of heavy and light patterns loads the XCDs evenly. -1: use xcd_remap
// (more than 64 heads, or a problem too small to share).
__device__ int chosen_item(const AttnArgs& a, int bid) {
    const int BH = a.num_items / a.nb;
    if (BH > 64) return -1;
    uint64_t gm[kGroups] = {0, 0, 0, 0, 0};
    for (int h = 0; h < BH; ++h) {
        const int c = ld_const(a.head_choice, h);
        const int g = (unsigned)c < (unsigned)a.n_cand ? c : kGroups - 1;
#pragma unroll
        for (int gg = 0; gg < kGroups; ++gg)
            if (g == gg) gm[gg] |= 1ull << h;
    }
    return group_remap(bid, a.num_items, a.nb, gm);
}

__device__ __forceinline__ int block_valid_c(const int32_t* blk_len, int b, int BS, int N) {
    int exist = min(BS, N - b * BS);
    return blk_len ? min(ld_const(blk_len, b), exist) : exist;
}

template <int BS, bool GATHER>
__global__ __launch_bounds__(BS * 2) __attribute__((amdgpu_waves_per_eu(2))) void attn_fwd_bf16_d128_kernel(AttnArgs a) {
    // 128-row blocks walk 64-key sub-tiles (2 workgroups per CU); 64-row blocks
    // walk 32-key sub-tiles, so that two stages still fit 4 workgroups per CU
    constexpr int D = 128, KT = (BS == 128) ? 64 : 32, NST = KT / 32, SUBB = KT * D * 2;
    constexpr int WAVES = BS / 32, THREADS = WAVES * 64, SUB = BS / KT;
    constexpr float TAU = 8.f, TAU_POW = 256.f;
    constexpr bool TWO_STAGES = true;
    __shared__ __attribute__((aligned(1024))) uint8_t k0[SUBB];
    __shared__ __attribute__((aligned(1024))) uint8_t v0[SUBB];
    __shared__ __attribute__((aligned(1024))) uint8_t k1[SUBB];
    __shared__ __attribute__((aligned(1024))) uint8_t v1[SUBB];
    // the row's kept blocks (compacted from the mask, or copied from the list)
    // and, with blk_len, their valid lengths: sized at launch
    extern __shared__ __attribute__((aligned(16))) int16_t list_lds[];
    __shared__ int wave_cnt[WAVES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS copy targets stay scalar
    const int l32 = lane & 31, half = lane >> 5;
    const int nqb = a.nb, nkb = a.nb;
    int item = a.head_choice ? chosen_item(a, blockIdx.x)
                             : ((a.head_groups[0] | a.head_groups[1])
                                    ? group_remap(blockIdx.x, a.num_items, a.nb, a.head_groups) : -1);
    if (item < 0) item = a.head_runs ? run_remap(blockIdx.x, a.num_items) : xcd_remap(blockIdx.x, a.num_items);
    const int bh = item / nqb, qb = item - bh * nqb;
    const int64_t head_off = (int64_t)bh * a.N * D;
    const int valid_q = block_valid_c(a.blk_len, qb, BS, a.N);
    const bool wave_active = 32 * w < valid_q;
    // frame-major head (uniform over the workgroup); launches without any such
    // head use the GATHER = false instance, which carries no code for it
    bool fm = false;
    const uint8_t* mask_row = a.mask ? a.mask + (int64_t)item * nkb : nullptr;
    if (a.head_choice) {
        const int c = ld_const(a.head_choice, bh);
        const bool ok = (unsigned)c < (unsigned)a.n_cand;     // otherwise: nothing kept
        mask_row = ok ? a.mask + ((int64_t)c * nqb + qb) * nkb : nullptr;
        if constexpr (GATHER) fm = ok && a.cand_fm[ok ? c : 0] != 0;
    } else if constexpr (GATHER) {
        const int h = bh % a.H;
        fm = (a.fm_bits[h >> 5] >> (h & 31)) & 1u;
    }

    // The row's kept blocks go to LDS once, so the loop reads each entry (and its
    // valid length) from LDS instead of waiting on a global load per sub-tile.
    int cnt;
    const int32_t* list_g = nullptr;
    int16_t* len_lds = list_lds + a.lds_cap;
    const bool in_lds = a.mask != nullptr || a.lds_cap > 0;
    if (a.head_choice && !mask_row) {
        cnt = 0;
    } else if (a.mask) {
        cnt = compact_mask_row<THREADS>(mask_row, nkb, list_lds, wave_cnt);
        if (a.blk_len) {
            for (int e = tid; e < cnt; e += THREADS) len_lds[e] = (int16_t)block_valid(a.blk_len, list_lds[e], BS, a.N);
            lds_barrier();
        }
    } else {
        cnt = min(ld_const(a.kv_cnt, item), a.max_kv);
        list_g = a.kv_idx + (int64_t)item * a.max_kv;
        if (a.lds_cap > 0) {
            for (int e = tid; e < cnt; e += THREADS) {
                const int kb = list_g[e];
                const bool okb = (unsigned)kb < (unsigned)nkb;
                list_lds[e] = okb ? (int16_t)kb : (int16_t)-1;     // a malformed entry is skipped
                if (a.blk_len) len_lds[e] = okb ? (int16_t)block_valid(a.blk_len, kb, BS, a.N) : (int16_t)0;
            }
            lds_barrier();
        }
    }
    // valid keys of sub-tile i (0 when it holds none, or its block entry is malformed)
    auto sub_valid = [&](int i, int& kb) -> int {
        const int e = i / SUB;
        int v;
        if (in_lds) {
            kb = list_lds[e];
            if ((unsigned)kb >= (unsigned)nkb) return 0;
            v = a.blk_len ? (int)len_lds[e] : min(BS, a.N - kb * BS);
        } else {
            kb = ld_const(list_g, e);
            if ((unsigned)kb >= (unsigned)nkb) return 0;
            v = block_valid_c(a.blk_len, kb, BS, a.N);
        }
        v -= (i % SUB) * KT;
        return v < 0 ? 0 : (v > KT ? KT : v);
    };
    const SubTileDma<WAVES, kVSwz4, KT> dma(lane, w);
    const SubVtAddr vad(lane);
    const SubKAddr kad(lane);
    const int head_bytes = a.N * D * 2;
    // natural rows / rows through the frame-major map; the main loop below is
    // instantiated once per form, so a natural head runs no gather code
    auto issue_nat = [&](int i, uint8_t* kd, uint8_t* vd) {
        int kb;
        if (sub_valid(i, kb) == 0) return;
        dma.issue(kd, vd, a.k + head_off, a.v + head_off, head_bytes, kb * BS + (i % SUB) * KT, w);
    };
    auto issue_fm = [&](int i, uint8_t* kd, uint8_t* vd) {
        int kb;
        if (sub_valid(i, kb) == 0) return;
        dma.issue_frame_major(kd, vd, a.k + head_off, a.v + head_off, head_bytes, kb * BS + (i % SUB) * KT, a.N, a.T,
                              a.HW, a.div_T, lane, w);
    };

    const int q_local = 32 * w + l32;
    const int q_row = qb * BS + q_local;
    const bool q_ok = q_local < valid_q;
    // row of this query in memory (natural order)
    const int q_mem = (fm && q_row < a.N) ? fm_natural(a, q_row) : q_row;
    bf16x8 qf[D / 16];
    load_q_frag<D>(qf, a.q + head_off + (int64_t)q_mem * D, q_ok, half);

    f32x16 o_acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o_acc[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    auto compute = [&](int i, const uint8_t* kt, const uint8_t* vt) __attribute__((always_inline)) {
        int kb;
        const int vs = sub_valid(i, kb);
        if (!wave_active || vs == 0) return;
        // ---- S^T = K Q^T (NST x 32 keys) --------------------------------------
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
        // ---- online softmax with a lazily moved offset ---------------------------
        // p is first formed under the current offset. The offset only moves when
        // the tile's maximum exceeds it by more than TAU (log2 units), i.e. when
        // some p exceeds 2^TAU; a lane whose p sum to at most 2^TAU has none, so
        // while every lane's sum stays there the row maximum is never needed.
        // Otherwise the maximum is taken and p formed again where the offset
        // moves. p in fp32 feeds the row sum (so the log-sum-exp keeps fp32
        // accuracy); its bf16 rounding feeds the P V product.
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
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);   // 1 where the offset stays
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
        // ---- O^T += V^T P^T, V^T through transposing LDS reads -------------------
        sub_pv_ahead<NST>(o_acc, vt, pf, vfirst, vad);
    };

    const int n_sub = cnt * SUB;
    auto main_loop = [&](auto issue) __attribute__((always_inline)) {
        if (n_sub > 0) issue(0, k0, v0);
        if constexpr (TWO_STAGES) {
            for (int i = 0; i < n_sub; i += 2) {
                __builtin_amdgcn_s_waitcnt(0);      // this thread's copies of sub-tile i have landed
                __syncthreads();                    // ... and everyone's; stage 1 is free again
                if (i + 1 < n_sub) issue(i + 1, k1, v1);
                compute(i, k0, v0);
                if (i + 1 < n_sub) {
                    __builtin_amdgcn_s_waitcnt(0);
                    __syncthreads();
                    if (i + 2 < n_sub) issue(i + 2, k0, v0);
                    compute(i + 1, k1, v1);
                }
            }
        } else {
            for (int i = 0; i < n_sub; ++i) {
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                compute(i, k0, v0);
                __syncthreads();                    // stage free before the next copy
                if (i + 1 < n_sub) issue(i + 1, k0, v0);
            }
        }
    };
    if (GATHER && fm) main_loop(issue_fm);
    else main_loop(issue_nat);

    const float l_tot = pair_sum(l_run);
    if (q_row < a.N) {
        const bool has = q_ok && l_tot > 0.f;
        const float inv = has ? 1.f / l_tot : 0.f;
        uint16_t* orow = a.o + head_off + (int64_t)q_mem * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                __bf16 b0 = (__bf16)(o_acc[dt][4 * jj + 0] * inv);
                __bf16 b1 = (__bf16)(o_acc[dt][4 * jj + 1] * inv);
                __bf16 b2 = (__bf16)(o_acc[dt][4 * jj + 2] * inv);
                __bf16 b3 = (__bf16)(o_acc[dt][4 * jj + 3] * inv);
                u32x2 pk;
                pk.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
                pk.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
                *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * jj + 4 * half) = pk;
            }
        if (a.lse && half == 0)
            a.lse[(int64_t)bh * a.N + q_mem] = has ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    }
}

// fp32 kernel (block size 64): one thread per query row, K and V tiles in LDS,
// exact fp32 arithmetic with an online softmax per tile.
template <int D>
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(AttnArgs a) {
    constexpr int BS = 64;
    __shared__ __attribute__((aligned(16))) float k_lds[BS * D];
    __shared__ __attribute__((aligned(16))) float v_lds[BS * D];
    __shared__ int16_t list_lds[kMaxMaskBlocks];
    __shared__ int wave_cnt[1];
    const float* Q = reinterpret_cast<const float*>(a.q);
    const float* K = reinterpret_cast<const float*>(a.k);
    const float* V = reinterpret_cast<const float*>(a.v);
    float* O = reinterpret_cast<float*>(a.o);
    const int tid = threadIdx.x;
    const int nkb = a.nb;
    const int item = xcd_remap(blockIdx.x, a.num_items);
    const int bh = item / a.nb, qb = item - bh * a.nb;
    const int64_t head_off = (int64_t)bh * a.N * D;
    const int valid_q = block_valid(a.blk_len, qb, BS, a.N);
    int cnt;
    const int32_t* list_g = nullptr;
    if (a.mask) {
        cnt = compact_mask_row<64>(a.mask + (int64_t)item * nkb, nkb, list_lds, wave_cnt);
    } else {
        cnt = min(a.kv_cnt[item], a.max_kv);
        list_g = a.kv_idx + (int64_t)item * a.max_kv;
    }
    const int q_row = qb * BS + tid;
    const bool q_ok = tid < valid_q;
    float qv[D], ov[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        qv[d] = q_ok ? Q[head_off + (int64_t)q_row * D + d] : 0.f;
        ov[d] = 0.f;
    }
    float m_run = -INFINITY, l_run = 0.f;
    for (int it = 0; it < cnt; ++it) {
        const int kb = a.mask ? (int)list_lds[it] : list_g[it];
        if ((unsigned)kb >= (unsigned)nkb) continue;
        const int valid_k = block_valid(a.blk_len, kb, BS, a.N);
        const int64_t key0 = head_off + (int64_t)kb * BS * D;
        __syncthreads();
        for (int i = tid; i < BS * D / 4; i += 64) {
            int r = (4 * i) / D;
            f32x4 kt = {0.f, 0.f, 0.f, 0.f}, vt = {0.f, 0.f, 0.f, 0.f};
            if (r < valid_k) {
                kt = *reinterpret_cast<const f32x4*>(K + key0 + 4 * i);
                vt = *reinterpret_cast<const f32x4*>(V + key0 + 4 * i);
            }
            *reinterpret_cast<f32x4*>(k_lds + 4 * i) = kt;
            *reinterpret_cast<f32x4*>(v_lds + 4 * i) = vt;
        }
        __syncthreads();
        float s[BS];
        float mx = -INFINITY;
        for (int j = 0; j < BS; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) acc = fmaf(qv[d], k_lds[j * D + d], acc);
            s[j] = (j < valid_k) ? acc * a.scale_log2 : -INFINITY;
            mx = fmaxf(mx, s[j]);
        }
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < D; ++d) ov[d] *= alpha;
        for (int j = 0; j < BS; ++j) {
            float p = __builtin_amdgcn_exp2f(s[j] - m_use);
            l_run += p;
#pragma unroll
            for (int d = 0; d < D; ++d) ov[d] = fmaf(p, v_lds[j * D + d], ov[d]);
        }
        m_run = m_new;
    }
    if (q_row < a.N) {
        const bool has = q_ok && l_run > 0.f;
        const float inv = has ? 1.f / l_run : 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) O[head_off + (int64_t)q_row * D + d] = ov[d] * inv;
        if (a.lse) a.lse[(int64_t)bh * a.N + q_row] = has ? (m_run + log2f(l_run)) * 0.69314718055994531f : -INFINITY;
    }
}

}  // namespace vsa

using namespace vsa;

extern "C" size_t vsa_attn_workspace_bytes(int B, int H, int N, int bs, int max_kv) {
    (void)B; (void)H; (void)N; (void)bs; (void)max_kv;
    return 0;
}

namespace {

// Validates the arguments shared by both entry points and fills `a` (no
// frame-major heads). Returns VSA_OK or the failure status.
int prepare_attn(const char* fn, AttnArgs& a, const void* q, const void* k, const void* v, void* o, float* lse, int B,
                 int H, int N, int D, int dtype, int bs, const int32_t* blk_len, const vsa_blocks* blocks,
                 float scale) {
    if (!q || !k || !v || !o) return fail(VSA_ERR_INVALID, "%s: null tensor", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(VSA_ERR_INVALID, "%s: tensors must be 16-byte aligned", fn);
    if (B <= 0 || H <= 0 || N <= 0) return fail(VSA_ERR_INVALID, "%s: B, H, N must be positive", fn);
    if (!blocks) return fail(VSA_ERR_INVALID, "%s: null blocks", fn);
    const bool has_mask = blocks->mask != nullptr;
    const bool has_list = blocks->kv_idx != nullptr || blocks->kv_cnt != nullptr;
    if (has_mask == has_list) return fail(VSA_ERR_INVALID, "%s: give exactly one of mask or (kv_idx, kv_cnt)", fn);
    if (has_list && (!blocks->kv_idx || !blocks->kv_cnt || blocks->max_kv <= 0))
        return fail(VSA_ERR_INVALID, "%s: list form needs kv_idx, kv_cnt and max_kv > 0", fn);
    if (!(scale > 0.f) || !__builtin_isfinite(scale)) return fail(VSA_ERR_INVALID, "%s: scale must be positive and finite", fn);
    if (D != 64 && D != 128) return fail(VSA_ERR_UNSUPPORTED, "%s: D must be 64 or 128 (got %d)", fn, D);
    if (dtype == VSA_BF16) {
        if (bs != 64 && bs != 128) return fail(VSA_ERR_UNSUPPORTED, "%s: bf16 needs bs 64 or 128 (got %d)", fn, bs);
    } else if (dtype == VSA_F32) {
        if (bs != 64) return fail(VSA_ERR_UNSUPPORTED, "%s: fp32 needs bs 64 (got %d)", fn, bs);
    } else {
        return fail(VSA_ERR_UNSUPPORTED, "%s: dtype %d not supported", fn, dtype);
    }
    const int64_t nb = (N + (int64_t)bs - 1) / bs;
    if (has_mask && nb > kMaxMaskBlocks)
        return fail(VSA_ERR_UNSUPPORTED, "%s: mask form supports at most %d blocks per row (use the list form)", fn,
                    kMaxMaskBlocks);
    const int64_t items = (int64_t)B * H * nb;
    const int64_t elt = dtype == VSA_BF16 ? 2 : 4;
    if (items >= (1ll << 31) || (int64_t)N * D * elt >= (1ll << 31) || (int64_t)B * H * N * D >= (1ll << 40))
        return fail(VSA_ERR_INVALID, "%s: problem too large", fn);
    a = AttnArgs{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.o = static_cast<uint16_t*>(o);
    a.lse = lse;
    a.blk_len = blk_len;
    a.mask = blocks->mask;
    a.kv_idx = blocks->kv_idx;
    a.kv_cnt = blocks->kv_cnt;
    a.max_kv = has_list ? blocks->max_kv : 0;
    a.H = H; a.N = N; a.nb = (int32_t)nb;
    a.num_items = (int32_t)items;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    a.T = 1; a.HW = N; a.div_T = FastDiv(1u);
    // Every query block of a head streams that head's kept K and V blocks. Dealt
    // in contiguous eighths, the 8 XCDs work on 8 different heads at once; when
    // 8 heads' K and V exceed the 256 MB last-level cache, the blocks that miss
    // L2 come from HBM, so runs of items are dealt instead and the XCDs share
    // one or two heads' K and V in that cache. Below that size the eighths keep
    // more of each XCD's neighbours in its L2.
    a.head_runs = 8 * (2 * (int64_t)N * D * elt) > kLlcBytes;
    return VSA_OK;
}

void launch_attn(const AttnArgs& a, int D, int dtype, int bs, hipStream_t s) {
    dim3 grid((unsigned)a.num_items);
    if (dtype == VSA_BF16) {
        bool gather = false;
        for (int i = 0; i < 32; ++i) gather |= a.fm_bits[i] != 0;
        if (a.head_choice)
            for (int c = 0; c < a.n_cand; ++c) gather |= a.cand_fm[c] != 0;
        // LDS for the row's list (and valid lengths): the mask form always keeps
        // it there; the list form when it fits beside the K/V stages without
        // costing a workgroup per CU (2 per CU at bs 128, 4 at bs 64) and the
        // block ids fit int16
        AttnArgs b = a;
        const size_t per_entry = a.blk_len ? 4 : 2;
        const size_t budget = bs == 128 ? 16384 : 8192;
        if (a.mask) b.lds_cap = a.nb;
        else b.lds_cap = ((size_t)a.max_kv * per_entry <= budget && a.nb <= 32767) ? a.max_kv : 0;
        const size_t shm = ((size_t)b.lds_cap * per_entry + 15) & ~(size_t)15;
        if (D == 128 && bs == 128) {
            if (gather) hipLaunchKernelGGL((attn_fwd_bf16_d128_kernel<128, true>), grid, dim3(256), shm, s, b);
            else hipLaunchKernelGGL((attn_fwd_bf16_d128_kernel<128, false>), grid, dim3(256), shm, s, b);
        } else if (D == 128 && bs == 64) {
            if (gather) hipLaunchKernelGGL((attn_fwd_bf16_d128_kernel<64, true>), grid, dim3(128), shm, s, b);
            else hipLaunchKernelGGL((attn_fwd_bf16_d128_kernel<64, false>), grid, dim3(128), shm, s, b);
        }
        else if (D == 64 && bs == 128) hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, 128>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, 64>), grid, dim3(128), 0, s, a);
    } else {
        if (D == 64) hipLaunchKernelGGL((attn_fwd_f32_kernel<64>), grid, dim3(64), 0, s, a);
        else hipLaunchKernelGGL((attn_fwd_f32_kernel<128>), grid, dim3(64), 0, s, a);
    }
}

}  // namespace

extern "C" int vsa_block_sparse_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                         int H, int N, int D, int dtype, int bs, const int32_t* blk_len,
                                         const vsa_blocks* blocks, float scale, void* workspace, size_t ws_bytes,
                                         void* stream) {
    (void)workspace; (void)ws_bytes;
    AttnArgs a;
    const int st = prepare_attn("vsa_block_sparse_attn_fwd", a, q, k, v, o, lse, B, H, N, D, dtype, bs, blk_len,
                                blocks, scale);
    if (st != VSA_OK) return st;
    launch_attn(a, D, dtype, bs, as_stream(stream));
    return launch_status("vsa_block_sparse_attn_fwd");
}

extern "C" int vsa_block_sparse_attn_fwd_permuted(const void* q, const void* k, const void* v, void* o, float* lse,
                                                  int B, int H, vsa_grid g, int D, int dtype, int bs,
                                                  const uint8_t* head_fm, const int32_t* blk_len,
                                                  const vsa_blocks* blocks, float scale, void* stream) {
    const char* fn = "vsa_block_sparse_attn_fwd_permuted";
    if (g.T <= 0 || g.Hh <= 0 || g.W <= 0) return fail(VSA_ERR_INVALID, "%s: grid extents must be positive", fn);
    const int64_t N64 = (int64_t)g.T * g.Hh * g.W;
    if (N64 >= (1ll << 31)) return fail(VSA_ERR_INVALID, "%s: grid too large", fn);
    if (H > 1024) return fail(VSA_ERR_UNSUPPORTED, "%s: at most 1024 heads", fn);
    AttnArgs a;
    const int st = prepare_attn(fn, a, q, k, v, o, lse, B, H, (int)N64, D, dtype, bs, blk_len, blocks, scale);
    if (st != VSA_OK) return st;
    if (dtype != VSA_BF16 || D != 128)
        return fail(VSA_ERR_UNSUPPORTED, "%s: frame-major heads need bf16 with D = 128", fn);
    a.T = g.T;
    a.HW = g.Hh * g.W;
    a.div_T = FastDiv((uint32_t)g.T);
    if (head_fm)
        for (int h = 0; h < H; ++h)
            if (head_fm[h]) a.fm_bits[h >> 5] |= 1u << (h & 31);
    // frame-major and natural heads usually run different patterns: deal each
    // kind evenly over the XCDs (at most 64 heads in all)
    if (head_fm && (int64_t)B * H <= 64) {
        bool any_fm = false, any_nat = false;
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < H; ++h) {
                const int bh = b * H + h;
                a.head_groups[head_fm[h] ? 1 : 0] |= 1ull << bh;
                (head_fm[h] ? any_fm : any_nat) = true;
            }
        if (!(any_fm && any_nat)) a.head_groups[0] = a.head_groups[1] = 0;   // one kind: the plain deal
    }
    launch_attn(a, D, dtype, bs, as_stream(stream));
    return launch_status(fn);
}

extern "C" int vsa_block_sparse_attn_fwd_chosen(const void* q, const void* k, const void* v, void* o, float* lse,
                                                int B, int H, vsa_grid g, int D, int dtype, int bs,
                                                const uint8_t* cand_masks, const int32_t* cand_layout, int P,
                                                const int32_t* choice, const int32_t* blk_len, float scale,
                                                void* stream) {
    const char* fn = "vsa_block_sparse_attn_fwd_chosen";
    if (!cand_masks || !cand_layout || !choice) return fail(VSA_ERR_INVALID, "%s: null pointer", fn);
    if (P < 1 || P > 4) return fail(VSA_ERR_INVALID, "%s: P must be in [1, 4]", fn);
    for (int c = 0; c < P; ++c)
        if (cand_layout[c] != 0 && cand_layout[c] != 1)
            return fail(VSA_ERR_INVALID, "%s: cand_layout[%d] must be 0 or 1", fn, c);
    if (g.T <= 0 || g.Hh <= 0 || g.W <= 0) return fail(VSA_ERR_INVALID, "%s: grid extents must be positive", fn);
    const int64_t N64 = (int64_t)g.T * g.Hh * g.W;
    if (N64 >= (1ll << 31)) return fail(VSA_ERR_INVALID, "%s: grid too large", fn);
    vsa_blocks blocks{cand_masks, nullptr, nullptr, 0};
    AttnArgs a;
    const int st = prepare_attn(fn, a, q, k, v, o, lse, B, H, (int)N64, D, dtype, bs, blk_len, &blocks, scale);
    if (st != VSA_OK) return st;
    if (dtype != VSA_BF16 || D != 128) return fail(VSA_ERR_UNSUPPORTED, "%s: needs bf16 with D = 128", fn);
    a.T = g.T;
    a.HW = g.Hh * g.W;
    a.div_T = FastDiv((uint32_t)g.T);
    a.head_choice = choice;
    a.n_cand = P;
    for (int c = 0; c < P; ++c) a.cand_fm[c] = cand_layout[c];
    launch_attn(a, D, dtype, bs, as_stream(stream));
    return launch_status(fn);
}
