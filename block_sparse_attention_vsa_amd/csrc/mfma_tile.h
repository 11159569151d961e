// Device building blocks shared by the attention and profiler kernels: LDS
// staging of a key/value tile and the two MFMA products of one tile.
//
// Layouts (KT keys per tile, D channels, bf16):
//  * K tile, row-major [KT][D]: the 16-byte chunk c of key r is stored at chunk
//    c ^ (r & 7) of its row, so the 8 lanes of a ds_read_b128 group (8
//    consecutive keys, same chunk) hit 8 distinct bank groups.
//  * V tile, transposed [D][KT]: row d holds the tile's keys; key kappa is stored
//    at position pos(kappa) = kappa with bits 2 and 3 swapped, and 16-byte chunk
//    x of row d at chunk x ^ ((d ^ d >> 3) & 7).
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 channels from
//    LDS, B = 16 channels x 32 queries from registers). Accumulator element x of
//    sub-tile st in lane l holds key 32 st + 8 (x >> 2) + 4 (l >> 5) + (x & 3) of
//    query l & 31.
//  * O^T += V^T P^T: the B operand for keys [32 st + 16 g, +16) is accumulator
//    elements [8 g, 8 g + 8) of sub-tile st converted to bf16; the A operand slot
//    (half h, element e) then needs key 32 st + 16 g + 8 (e >> 2) + 4 h + (e & 3),
//    whose transposed position 32 st + 16 g + 8 h + e makes the 8 values of a
//    lane one contiguous 16-byte chunk.
#pragma once

#include "vsa_internal.h"

namespace vsa {

template <int D, int KT>
__device__ __forceinline__ int k_lds_off(int r, int c) {
    return r * D * 2 + ((c ^ (r & 7)) << 4);
}

template <int D, int KT>
__device__ __forceinline__ int v_lds_off(int d, int chunk) {
    return d * KT * 2 + ((chunk ^ ((d ^ (d >> 3)) & 7)) << 4);
}

// Stage a K tile: rows [0, valid) from global (row stride D), zeros after.
template <int D, int KT, int THREADS>
__device__ __forceinline__ void stage_k_tile(uint8_t* k_lds, const uint16_t* kg, int valid, int tid) {
    constexpr int KCH = D / 8;
    static_assert((KT * KCH) % THREADS == 0, "K tile must split evenly over the threads");
#pragma unroll
    for (int u = 0; u < KT * KCH / THREADS; ++u) {
        int i = tid + THREADS * u;
        int r = i / KCH, c = i % KCH;
        u32x4 t = {0u, 0u, 0u, 0u};
        if (r < valid) t = *reinterpret_cast<const u32x4*>(kg + (int64_t)r * D + 8 * c);
        *reinterpret_cast<u32x4*>(k_lds + k_lds_off<D, KT>(r, c)) = t;
    }
}

// Stage a V tile transposed. Each lane moves 4 consecutive keys x 8 channels:
// four 16-byte row loads, a 4x8 -> 8x4 transpose with byte permutes, eight
// 8-byte LDS writes. The lane -> (key group, chunk) map puts, in every 16-lane
// write group, 8 distinct swizzles x both halves of a 16-byte chunk.
template <int D, int KT, int THREADS>
__device__ __forceinline__ void stage_v_tile(uint8_t* v_lds, const uint16_t* vg, int valid, int tid) {
    constexpr int WAVES = THREADS / 64;
    constexpr int GPW = (D == 128) ? 4 : 8;                 // key groups per wave step
    constexpr int STEPS = (KT / 4) / (GPW * WAVES);
    static_assert(STEPS * GPW * WAVES == KT / 4, "V tile must split evenly over the waves");
    const int lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int u = 0; u < STEPS; ++u) {
        int g4, c;
        if (D == 128) {
            g4 = ((lane >> 5) & 1) + 2 * ((lane >> 3) & 1) + GPW * (w + WAVES * u);
            c = (lane & 7) + 8 * ((lane >> 4) & 1);
        } else {
            g4 = ((lane >> 4) & 1) + 2 * ((lane >> 3) & 1) + 4 * ((lane >> 5) & 1) + GPW * (w + WAVES * u);
            c = lane & 7;
        }
        u32x4 rows[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            int r = 4 * g4 + rr;
            rows[rr] = u32x4{0u, 0u, 0u, 0u};
            if (r < valid) rows[rr] = *reinterpret_cast<const u32x4*>(vg + (int64_t)r * D + 8 * c);
        }
        const int key = 4 * g4;
        const int pos = (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            u32x2 out;
            out.x = __builtin_amdgcn_perm(rows[1][e >> 1], rows[0][e >> 1], sel);
            out.y = __builtin_amdgcn_perm(rows[3][e >> 1], rows[2][e >> 1], sel);
            const int d = 8 * c + e;
            *reinterpret_cast<u32x2*>(v_lds + v_lds_off<D, KT>(d, pos >> 3) + (pos & 7) * 2) = out;
        }
    }
}

// Q fragment of one wave: lane holds channels 16 kk + 8 (lane >> 5) + [0, 8) of
// its query row (zeros when the row is absent).
template <int D>
__device__ __forceinline__ void load_q_frag(bf16x8 (&qf)[D / 16], const uint16_t* qrow, bool ok, int half) {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        u32x4 t = {0u, 0u, 0u, 0u};
        if (ok) t = *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * half);
        qf[kk] = __builtin_bit_cast(bf16x8, t);
    }
}

// S^T for one tile: s[st] accumulators as described above.
template <int D, int KT>
__device__ __forceinline__ void tile_scores(f32x16 (&s)[KT / 32], const uint8_t* k_lds, const bf16x8 (&qf)[D / 16],
                                            int l32, int half) {
#pragma unroll
    for (int st = 0; st < KT / 32; ++st) {
        s[st] = f32x16{};
        const int r = 32 * st + l32;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            u32x4 kv = *reinterpret_cast<const u32x4*>(k_lds + k_lds_off<D, KT>(r, 2 * kk + half));
            s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv), qf[kk], s[st], 0, 0, 0);
        }
    }
}

// O^T += V^T P^T for one tile.
template <int D, int KT>
__device__ __forceinline__ void tile_pv(f32x16 (&o)[D / 32], const uint8_t* v_lds, const bf16x8 (&pf)[KT / 32][2],
                                        int l32, int half) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
        const int d = 32 * dt + l32;
#pragma unroll
        for (int st = 0; st < KT / 32; ++st)
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                u32x4 vv = *reinterpret_cast<const u32x4*>(v_lds + v_lds_off<D, KT>(d, 4 * st + 2 * g + half));
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pf[st][g], o[dt], 0, 0, 0);
            }
    }
}

__device__ __forceinline__ int acc_key(int st, int x, int half) {
    return 32 * st + 8 * (x >> 2) + 4 * half + (x & 3);
}

__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32); }

// Max / sum of the values held by lanes l and l ^ 32, via v_permlane32_swap
// (VALU, no LDS round trip). The swap returns the lower-half value in one result
// and the upper-half value in the other, so both halves add in the same order.
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}


// ---------------------------------------------------------------------------
// 64-key sub-tiles for D = 128 staged by DMA (buffer_load_dwordx4 ... lds).
//
// A wave instruction of a buffer load with the lds flag writes lane l's 16
// bytes to LDS base + 16 l, i.e. 1 KiB = 4 rows of 256 bytes. Lane l of
// instruction ins covers row 4 ins + (l >> 4), LDS slot l & 15 of that row, and
// fetches the global chunk that belongs there:
//   K: slot p of row r holds chunk p ^ (r & 15)  (16 keys of one chunk: 16 slots)
//   V: slot p of row r holds chunk p ^ 4 (r & 3) (the transposing reads below hit
//      every 16-byte slot of a 256-byte row exactly twice per wave)
// These per-lane byte offsets do not depend on the sub-tile, so they are
// computed once; the sub-tile's base is a scalar offset. The buffer descriptor
// covers exactly one head's rows, so rows past the head's end read as zeros
// (masked later) without any per-row clamping.
constexpr int kSubKeys = 64;
constexpr int kSubBytes = kSubKeys * 128 * 2;   // one K or V sub-tile, D = 128

__device__ __forceinline__ void dma16(const void* base, int nbytes, void* lds_dst, int voff, int soff) {
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes,
                                                                 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, voff, soff, 0,
                                             0);
}

// Workgroup barrier for LDS data only: this wave's LDS reads and writes finish,
// then the waves meet. Unlike __syncthreads it does not wait for vector-memory
// loads, so LDS copies of a later stage stay in flight across it. Only for
// exchanging data written with ordinary LDS stores, never for a DMA'd stage.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Load of a wave-uniform int32 through the constant address space: a scalar
// load, waited on with lgkmcnt, so it never waits for vector-memory traffic
// such as the LDS DMA.
__device__ __forceinline__ int32_t ld_const(const int32_t* p, int64_t i) {
    return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// Builds this workgroup's ascending list of kept key blocks from a mask row.
template <int THREADS>
__device__ int compact_mask_row(const uint8_t* row, int nkb, int16_t* list, int* wave_cnt) {
    constexpr int WAVES = THREADS / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int base = 0;
    for (int r0 = 0; r0 < nkb; r0 += THREADS) {
        int e = r0 + threadIdx.x;
        bool keep = e < nkb && row[e] != 0;
        uint64_t bal = __ballot(keep);
        if (lane == 0) wave_cnt[w] = __popcll(bal);
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int i = 0; i < WAVES; ++i) {
            int c = wave_cnt[i];
            before += (i < w) ? c : 0;
            total += c;
        }
        if (keep) list[base + before + __popcll(bal & ((1ull << lane) - 1ull))] = (int16_t)e;
        base += total;
        __syncthreads();
    }
    return base;
}

// One dword through a buffer descriptor spanning nbytes: an offset voff at or
// past nbytes reads 0 (the per-lane offset is range checked).
__device__ __forceinline__ uint32_t buf_load_u32(const void* base, int nbytes, int voff, int soff) {
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes,
                                                                 0x00020000);
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// V swizzles: kVSwz4 puts chunk c of row r at slot c ^ 4 (r & 3) (for the 32x32
// operand reads of the attention kernel); kVSwzPair at slot c ^ 2 (r & 7), i.e.
// 32-byte pair q at pair q ^ (r & 7) (for the 16x16 operand reads of the
// profiler). Either way the transposing reads touch every bank the minimum
// number of times.
enum { kVSwz4 = 0, kVSwzPair = 1 };
__device__ __forceinline__ int v_swizzle(int vswz, int row) {
    return vswz == kVSwz4 ? 4 * (row & 3) : 2 * (row & 7);
}

template <int WAVES, int VSWZ = kVSwz4, int KEYS = kSubKeys>
struct SubTileDma {
    static constexpr int IPW = KEYS * 256 / 1024 / WAVES;   // wave instructions per tensor per sub-tile
    static_assert(IPW >= 1, "every wave issues at least one instruction per tensor");
    // Instruction u covers rows 4 (w + WAVES u) + (lane >> 4). Bits 0..3 of the
    // row, which pick the K swizzle, repeat every NCLS instructions (once for 4
    // waves); the V swizzle's bits (0..1, or 0..2 with 4 waves) never change with u.
    static constexpr int NCLS = (4 * WAVES >= 16) ? 1 : 16 / (4 * WAVES);
    static_assert(VSWZ == kVSwz4 || WAVES >= 2, "pair swizzle needs u-independent row bits 0..2");
    int rowb;                       // byte offset of this lane's row for u = 0
    int ck[NCLS], cv;               // swizzled chunk offsets (bytes)
    __device__ __forceinline__ SubTileDma(int lane, int w) {
        const int p = lane & 15;
        rowb = (4 * w + (lane >> 4)) * 256;
#pragma unroll
        for (int u = 0; u < NCLS; ++u) {
            const int row = 4 * (w + WAVES * u) + (lane >> 4);
            ck[u] = (p ^ (row & 15)) << 4;
        }
        cv = (p ^ v_swizzle(VSWZ, 4 * w + (lane >> 4))) << 4;
    }
    __device__ __forceinline__ int voff_k(int u) const { return rowb + 1024 * WAVES * u + ck[u % NCLS]; }
    __device__ __forceinline__ int voff_v(int u) const { return rowb + 1024 * WAVES * u + cv; }
    // Sub-tile whose first key row inside the head is row0 (natural order). The
    // whole row offset goes into the per-lane offset, so the descriptor's range
    // check (one head's bytes) covers it.
    __device__ __forceinline__ void issue(uint8_t* k_dst, uint8_t* v_dst, const uint16_t* k_head,
                                          const uint16_t* v_head, int head_bytes, int row0, int w) const {
        const int base = row0 * 256;
#pragma unroll
        for (int u = 0; u < IPW; ++u) {
            const int ins = w + WAVES * u;
            dma16(k_head, head_bytes, k_dst + ins * 1024, base + voff_k(u), 0);
            dma16(v_head, head_bytes, v_dst + ins * 1024, base + voff_v(u), 0);
        }
    }
    // Same, for a head read through the frame-major map: sub-tile row r of the
    // permuted order is natural row (r mod T) * HW + r / T; rows >= N land past
    // the head and read as zeros.
    __device__ __forceinline__ void issue_frame_major(uint8_t* k_dst, uint8_t* v_dst, const uint16_t* k_head,
                                                      const uint16_t* v_head, int head_bytes, int row0, int N, int T,
                                                      int HW, const FastDiv& div_T, int lane, int w) const {
#pragma unroll
        for (int u = 0; u < IPW; ++u) {
            const int ins = w + WAVES * u;
            const uint32_t r = (uint32_t)(row0 + 4 * ins + (lane >> 4));
            const uint32_t s = div_T.div(r);
            const uint32_t nat = r < (uint32_t)N ? (r - s * (uint32_t)T) * (uint32_t)HW + s : (uint32_t)N;
            dma16(k_head, head_bytes, k_dst + ins * 1024, (int)(nat * 256u) + ck[u % NCLS], 0);
            dma16(v_head, head_bytes, v_dst + ins * 1024, (int)(nat * 256u) + cv, 0);
        }
    }
};

// S^T for a sub-tile of 32 NST keys: s[st] holds keys 32 st + acc_key(0, x, half).
template <int NST>
__device__ __forceinline__ void sub_scores(f32x16 (&s)[NST], const uint8_t* kt, const bf16x8 (&qf)[8], int l32,
                                           int half) {
    constexpr int D = 128;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
        s[st] = f32x16{};
        const int r = 32 * st + l32;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            u32x4 kv = *reinterpret_cast<const u32x4*>(kt + r * D * 2 + (((2 * kk + half) ^ (r & 15)) << 4));
            s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv), qf[kk], s[st], 0, 0, 0);
        }
    }
}

// V^T operand for channel tile dt and keys [32 st + 16 g, +16) of a sub-tile:
// two ds_read_b64_tr_b16. In a 16-lane group G of the wave, lanes 4j..4j+3
// point at 16 consecutive channels (32 dt + 16 (G & 1) + [0, 16)) of key
// 32 st + 16 g + 8 r + 4 (G >> 1) + j; lane i then holds channel i of those four
// keys, which are the keys of k slots (G >> 1, 4 r + j) of the P^T operand.
//
// The key's swizzle term (key & 3) is j for every st, g, r, so a lane's byte
// offset is one value per dt plus the constant 256 (32 st + 16 g + 8 r).
// SubVtAddr holds those four values, hidden from the optimiser: with the
// swizzle visible it re-associates the address so that the reads lose track of
// which stage array they touch, and every transposed read after the first then
// waits for all LDS copies in flight, the next stage's prefetch included.
struct SubVtAddr {
    int tr[4];
    __device__ __forceinline__ explicit SubVtAddr(int lane) {
        const int G = lane >> 4, gi = lane & 15;
        const int j = gi >> 2, c = gi & 3;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const int chunk = 4 * dt + 2 * (G & 1) + (c >> 1);
            tr[dt] = (4 * (G >> 1) + j) * 256 + ((chunk ^ (4 * j)) << 4) + (c & 1) * 8;
            asm("" : "+v"(tr[dt]));
        }
    }
};

__device__ __forceinline__ bf16x8 sub_vt_operand(const uint8_t* vt, int dt, int st, int g, const SubVtAddr& ad) {
    v4i16 part[2];
#pragma unroll
    for (int r2 = 0; r2 < 2; ++r2) {
        const uint8_t* ptr = vt + (32 * st + 16 * g + 8 * r2) * 256 + ad.tr[dt];
        part[r2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(ptr));
    }
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// Row-operand offsets of a K sub-tile (row 32 st + l32, chunk 2 kk + half at slot
// chunk ^ (row & 15); the st term adds 8192), opaque for the same reason as SubVtAddr.
struct SubKAddr {
    int rows[8];
    __device__ __forceinline__ explicit SubKAddr(int lane) {
        const int l32 = lane & 31, half = lane >> 5;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            rows[kk] = l32 * 256 + (((2 * kk + half) ^ (l32 & 15)) << 4);
            asm("" : "+v"(rows[kk]));
        }
    }
};

// sub_scores with the NST chains side by side and each step's K operands read
// one step ahead: the scheduler is told to issue the reads of step kk + 1 before
// the MFMAs of step kk, so an MFMA does not wait on the LDS latency of its own read.
template <int NST>
__device__ __forceinline__ void sub_scores_ahead(f32x16 (&s)[NST], const uint8_t* kt, const bf16x8 (&qf)[8],
                                                 const SubKAddr& ad) {
#pragma unroll
    for (int st = 0; st < NST; ++st) s[st] = f32x16{};
    u32x4 kb[2][NST];
#pragma unroll
    for (int st = 0; st < NST; ++st) kb[0][st] = *reinterpret_cast<const u32x4*>(kt + 8192 * st + ad.rows[0]);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        if (kk + 1 < 8) {
#pragma unroll
            for (int st = 0; st < NST; ++st)
                kb[(kk + 1) & 1][st] = *reinterpret_cast<const u32x4*>(kt + 8192 * st + ad.rows[kk + 1]);
        }
#pragma unroll
        for (int st = 0; st < NST; ++st)
            s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kb[kk & 1][st]), qf[kk], s[st],
                                                            0, 0, 0);
    }
    // groups: 0x100 = LDS reads, 0x008 = MFMA; sync id 1 keeps this sequence apart
    __builtin_amdgcn_sched_group_barrier(0x100, NST, 1);
#pragma unroll
    for (int kk = 0; kk < 7; ++kk) {
        __builtin_amdgcn_sched_group_barrier(0x100, NST, 1);
        __builtin_amdgcn_sched_group_barrier(0x008, NST, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NST, 1);
}

// V^T operands of channel tile 0: they do not depend on P, so the caller reads
// them before the softmax and the reads overlap it.
template <int NST>
__device__ __forceinline__ void sub_pv_first(bf16x8 (&first)[NST][2], const uint8_t* vt, const SubVtAddr& ad) {
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int g = 0; g < 2; ++g) first[st][g] = sub_vt_operand(vt, 0, st, g, ad);
}

// O^T += V^T P^T over the 4 channel tiles (tile 0's operands from sub_pv_first),
// the V^T operands of tile dt + 1 read while the MFMAs of tile dt run (same
// scheduling hint as above, sync id 2).
template <int NST>
__device__ __forceinline__ void sub_pv_ahead(f32x16 (&o_acc)[4], const uint8_t* vt, const bf16x8 (&pf)[NST][2],
                                             const bf16x8 (&first)[NST][2], const SubVtAddr& ad) {
    bf16x8 vb[2][NST][2];
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int g = 0; g < 2; ++g) vb[0][st][g] = first[st][g];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        if (dt + 1 < 4) {
#pragma unroll
            for (int st = 0; st < NST; ++st)
#pragma unroll
                for (int g = 0; g < 2; ++g) vb[(dt + 1) & 1][st][g] = sub_vt_operand(vt, dt + 1, st, g, ad);
        }
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
            for (int g = 0; g < 2; ++g)
                o_acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[dt & 1][st][g], pf[st][g], o_acc[dt], 0, 0, 0);
    }
    // two transposing reads per operand, 2 NST operands per channel tile
#pragma unroll
    for (int dt = 0; dt < 3; ++dt) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * NST, 2);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * NST, 2);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * NST, 2);
}

}  // namespace vsa

namespace vsa {

// ---------------------------------------------------------------------------
// Generic tile access for kernels that read one staged tile both ways.
//
// A staged tile is rows of 128 bf16 (256 bytes, 16 chunks of 16 bytes); chunk c
// of row r sits at slot c ^ swz(r). Two access patterns read it:
//  * row operand (32x32x16 A operand, or B operand from rows): lane l reads row
//    32 st + (l & 31), chunk 2 kk + (l >> 5), 16 bytes (ds_read_b128);
//  * transposed operand (the V^T pattern above): two ds_read_b64_tr_b16.
// kSwzRows (r & 15) is conflict-free for the first, kSwzTr (4 (r & 3)) for the
// second, and kSwzBoth ((r & 3) << 2 | (r >> 2) & 3, the two 2-bit halves of
// r & 15 swapped) for both; a bank model of 64 four-byte banks with 16 lanes per
// ds_read_b128 phase and 32 per ds_read_b64 phase shows each pass touches
// every bank once.
enum { kSwzRows = 0, kSwzTr = 1, kSwzBoth = 2 };

template <int SWZ>
__device__ __forceinline__ int tile_swizzle(int r) {
    if constexpr (SWZ == kSwzRows) return r & 15;
    else if constexpr (SWZ == kSwzTr) return 4 * (r & 3);
    else return ((r & 3) << 2) | ((r >> 2) & 3);
}

// DMA of a KEYS-row sub-tile of two tensors (A with swizzle SA, B with SB) into
// LDS; same lane/instruction mapping as SubTileDma. Rows past the head's end
// read as zeros (the whole row offset is in the range-checked lane offset).
template <int WAVES, int SA, int SB, int KEYS>
struct PairTileDma {
    static constexpr int IPW = KEYS * 256 / 1024 / WAVES;
    static_assert(IPW >= 1, "every wave issues at least one instruction per tensor");
    static constexpr int NCLS = (4 * WAVES >= 16) ? 1 : 16 / (4 * WAVES);   // swizzle classes over u
    int rowb, ca[NCLS], cb[NCLS];
    __device__ __forceinline__ PairTileDma(int lane, int w) {
        const int p = lane & 15;
        rowb = (4 * w + (lane >> 4)) * 256;
#pragma unroll
        for (int u = 0; u < NCLS; ++u) {
            const int row = 4 * (w + WAVES * u) + (lane >> 4);
            ca[u] = (p ^ tile_swizzle<SA>(row)) << 4;
            cb[u] = (p ^ tile_swizzle<SB>(row)) << 4;
        }
    }
    __device__ __forceinline__ void issue(uint8_t* a_dst, uint8_t* b_dst, const uint16_t* a_head,
                                          const uint16_t* b_head, int head_bytes, int row0, int w) const {
        const int base = row0 * 256;
#pragma unroll
        for (int u = 0; u < IPW; ++u) {
            const int ins = w + WAVES * u;
            const int off = base + rowb + 1024 * WAVES * u;
            dma16(a_head, head_bytes, a_dst + ins * 1024, off + ca[u % NCLS], 0);
            dma16(b_head, head_bytes, b_dst + ins * 1024, off + cb[u % NCLS], 0);
        }
    }
};

// s[st] += A(rows of the tile) x B(frag): for st < NST, the 32x32 products over
// the 128 channels; rows 32 st + (lane & 31) of the tile are the M index and the
// fragment's 32 lanes the N index.
template <int NST, int SWZ>
__device__ __forceinline__ void tile_rows_mma(f32x16 (&s)[NST], const uint8_t* tile, const bf16x8 (&frag)[8],
                                              int l32, int half) {
#pragma unroll
    for (int st = 0; st < NST; ++st) {
        s[st] = f32x16{};
        const int r = 32 * st + l32;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            u32x4 t = *reinterpret_cast<const u32x4*>(tile + r * 256 + (((2 * kk + half) ^ tile_swizzle<SWZ>(r)) << 4));
            s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, t), frag[kk], s[st], 0, 0, 0);
        }
    }
}

// Transposed operand (channels 32 dt + (lane & 31) x the 16 rows of (st, g) in
// the accumulator order) of a tile with swizzle SWZ; see sub_vt_operand.
template <int SWZ>
__device__ __forceinline__ bf16x8 tile_tr_operand(const uint8_t* tile, int dt, int st, int g, int lane) {
    const int G = lane >> 4, gi = lane & 15;
    const int j = gi >> 2, c = gi & 3;
    const int chunk = 4 * dt + 2 * (G & 1) + (c >> 1);
    v4i16 part[2];
#pragma unroll
    for (int r2 = 0; r2 < 2; ++r2) {
        const int row = 32 * st + 16 * g + 8 * r2 + 4 * (G >> 1) + j;
        const uint8_t* ptr = tile + row * 256 + ((chunk ^ tile_swizzle<SWZ>(row)) << 4) + (c & 1) * 8;
        part[r2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(ptr));
    }
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace vsa

namespace vsa {

// Per-lane LDS offsets of the two access patterns for a tile with swizzle SWZ,
// computed once. The row index of both patterns differs from the lane's base
// row by multiples of 16 within a 32-row half, so the swizzle (a function of
// row & 15) is fixed per lane; the 32-row half, the stage buffer and the g step
// are then constants the instruction's offset field absorbs. The values pass
// through an empty asm so the compiler cannot prove their bits disjoint from
// those constants and turn the add into an OR (which would need one register
// per address).
template <int SWZ>
struct TileAddr {
    int rows[8];        // row operand, channel step kk: row l32, chunk 2 kk + half
    int tr[4][2];       // transposed operand, channel tile dt, r2
    __device__ __forceinline__ explicit TileAddr(int lane) {
        const int l32 = lane & 31, half = lane >> 5;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            rows[kk] = l32 * 256 + (((2 * kk + half) ^ tile_swizzle<SWZ>(l32)) << 4);
            asm("" : "+v"(rows[kk]));
        }
        const int G = lane >> 4, gi = lane & 15;
        const int j = gi >> 2, c = gi & 3;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
                const int row = 8 * r2 + 4 * (G >> 1) + j;
                const int chunk = 4 * dt + 2 * (G & 1) + (c >> 1);
                tr[dt][r2] = row * 256 + ((chunk ^ tile_swizzle<SWZ>(row)) << 4) + (c & 1) * 8;
                asm("" : "+v"(tr[dt][r2]));
            }
    }
};

// s = rows 32 st + [0, 32) of the tile (A) times frag (B), over 128 channels.
template <int SWZ>
__device__ __forceinline__ f32x16 tile_rows_mma_at(const uint8_t* tile, int st, const bf16x8 (&frag)[8],
                                                   const TileAddr<SWZ>& ad) {
    f32x16 s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        u32x4 t = *reinterpret_cast<const u32x4*>(tile + 8192 * st + ad.rows[kk]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, t), frag[kk], s, 0, 0, 0);
    }
    return s;
}

template <int SWZ>
__device__ __forceinline__ bf16x8 tile_tr_operand_at(const uint8_t* tile, int dt, int st, int g,
                                                     const TileAddr<SWZ>& ad) {
    v4i16 part[2];
#pragma unroll
    for (int r2 = 0; r2 < 2; ++r2) {
        const uint8_t* ptr = tile + (32 * st + 16 * g) * 256 + ad.tr[dt][r2];
        part[r2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(ptr));
    }
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace vsa
