// Internal helpers shared by the HIP sources of libvsa.so (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/vsa.h"

namespace vsa {

// ---------------------------------------------------------------- status ----
// Records the message of the last failing call of this thread and returns the
// status, so that entry points can `return fail(VSA_ERR_INVALID, "...")`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int launch_status(const char* what);   // VSA_OK or VSA_ERR_LAUNCH after a launch
int permute_selftest_host();           // host check of the layout maps (permute.hip)
int profile_selftest_host();           // host check of the frame-major keep bits (profile.hip)

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ------------------------------------------------------------ bf16 types ----
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// ------------------------------------------------ division by a constant ----
// Unsigned division by a divisor fixed at launch (Granlund and Montgomery,
// "Division by invariant integers using multiplication", 1994, round-up form):
// with l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1,
// q = (t + ((n - t) >> min(l,1))) >> max(l-1,0), t = mulhi(n, m). Exact for
// every 32-bit n.
struct FastDiv {
    uint32_t d, m, sh1, sh2;
    FastDiv() : d(1), m(1), sh1(0), sh2(0) {}
    explicit FastDiv(uint32_t divisor) : d(divisor) {
        uint32_t l = 0;
        while ((1ull << l) < (uint64_t)d) ++l;
        m = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
        sh1 = l ? 1u : 0u;
        sh2 = l ? l - 1 : 0u;
    }
    __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
        uint32_t t = (uint32_t)(((uint64_t)n * m) >> 32);   // mul_hi on the device
        return (t + ((n - t) >> sh1)) >> sh2;
    }
};

// Workgroup `bid` of a G-workgroup grid runs on XCD bid % 8 (round-robin
// dispatch over the 8 XCDs). Returns the item it should process so that each
// XCD owns a contiguous range of items, [x q + min(x, r), ...) with q = G / 8,
// r = G % 8: neighbouring items then share that XCD's L2. A bijection on [0, G).
__host__ __device__ __forceinline__ int xcd_remap(int bid, int G) {
    const int x = bid & 7, j = bid >> 3;
    const int q = G >> 3, r = G & 7;
    return x * q + (x < r ? x : r) + j;
}

// The same round-robin dispatch, with the items cut into runs of kHeadRun
// consecutive items that are dealt to the XCDs in turn: XCD x takes runs x,
// x + 8, x + 16, ..., a run's items in order. Each XCD still walks neighbouring
// items (one run is as many workgroups as an XCD holds at once), but the 8 XCDs
// now work on 8 neighbouring runs, i.e. on one or two heads at a time instead
// of 8 far-apart heads. The items past the last whole group of 8 runs map to
// themselves. A bijection on [0, G).
constexpr int kHeadRun = 64;
__host__ __device__ __forceinline__ int run_remap(int bid, int G) {
    const int full = G / (8 * kHeadRun) * (8 * kHeadRun);
    if (bid >= full) return bid;
    const int x = bid & 7, j = bid >> 3;
    return ((j / kHeadRun) * 8 + x) * kHeadRun + j % kHeadRun;
}

// Work items of heads that run different patterns, dealt evenly over the XCDs.
// Items are (head, block) pairs, item = head * nb + block, G = heads * nb. Heads
// are grouped (gm[g] has bit h set for each head h of group g, heads < 64,
// groups < kGroups); every XCD takes a contiguous 1/8 of every group's items,
// the last non-empty group what the XCD's workgroup count leaves, so each XCD
// does an equal share of every group's work whatever the groups cost. Inside a
// share, items stay in head and block order (neighbouring blocks of a head
// share that XCD's L2). With one group this is xcd_remap. Returns -1 when a
// share would be negative (a tiny problem); callers then use xcd_remap.
constexpr int kGroups = 5;
__host__ __device__ __forceinline__ int group_remap(int bid, int G, int nb, const uint64_t (&gm)[kGroups]) {
    const int x = bid & 7, j = bid >> 3;
    const int q = G >> 3, r = G & 7;
    int last = -1;
    for (int g = 0; g < kGroups; ++g)
        if (gm[g]) last = g;
    if (last < 0) return -1;
    // items of group g (not the last) that XCD xx takes, and where they start
    auto size_of = [&](int g, int xx) -> int {
        const int64_t Gg = (int64_t)__builtin_popcountll(gm[g]) * nb;
        return (int)((((int64_t)xx + 1) * Gg >> 3) - ((int64_t)xx * Gg >> 3));
    };
    auto size_last = [&](int xx) -> int {
        int s = q + (xx < r ? 1 : 0);
        for (int g = 0; g < last; ++g)
            if (gm[g]) s -= size_of(g, xx);
        return s;
    };
    int lo_last = 0;
    for (int xx = 0; xx < 8; ++xx) {
        const int s = size_last(xx);
        if (s < 0) return -1;
        if (xx < x) lo_last += s;
    }
    int off = 0;
    for (int g = 0; g <= last; ++g) {
        if (!gm[g]) continue;
        const int64_t Gg = (int64_t)__builtin_popcountll(gm[g]) * nb;
        const int lo = g == last ? lo_last : (int)((int64_t)x * Gg >> 3);
        const int sz = g == last ? size_last(x) : size_of(g, x);
        if (j < off + sz) {
            const int t = lo + (j - off);
            const int k = t / nb, blk = t - k * nb;
            uint64_t m = gm[g];
            for (int i = 0; i < k; ++i) m &= m - 1;      // k-th head of the group
            return __builtin_ctzll(m) * nb + blk;
        }
        off += sz;
    }
    return -1;
}

}  // namespace vsa
