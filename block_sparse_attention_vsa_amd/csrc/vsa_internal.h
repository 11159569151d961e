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
__device__ __forceinline__ int xcd_remap(int bid, int G) {
    const int x = bid & 7, j = bid >> 3;
    const int q = G >> 3, r = G & 7;
    return x * q + min(x, r) + j;
}

}  // namespace vsa
