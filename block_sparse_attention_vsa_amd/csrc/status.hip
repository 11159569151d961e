// Status codes, per-thread error messages and host-only entry points.
#include <stdarg.h>
#include <stdio.h>

#include "vsa_internal.h"

namespace vsa {

static thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

int launch_status(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(VSA_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return VSA_OK;
}

}  // namespace vsa

extern "C" {

const char* vsa_status_string(int status) {
    switch (status) {
        case VSA_OK: return "ok";
        case VSA_ERR_INVALID: return "invalid argument";
        case VSA_ERR_UNSUPPORTED: return "unsupported configuration";
        case VSA_ERR_LAUNCH: return "HIP launch error";
        case VSA_ERR_WORKSPACE: return "workspace too small";
        default: return "unknown status";
    }
}

const char* vsa_last_error(void) { return vsa::g_last_error; }

int vsa_version(void) { return 10000 * 0 + 100 * 1 + 0; }

int vsa_cube_dims(vsa_grid g, int32_t* n_cubes, int32_t* n_slots) {
    if (g.T <= 0 || g.Hh <= 0 || g.W <= 0)
        return vsa::fail(VSA_ERR_INVALID, "vsa_cube_dims: grid extents must be positive");
    if (!n_cubes || !n_slots) return vsa::fail(VSA_ERR_INVALID, "vsa_cube_dims: null output");
    int64_t c = (int64_t)((g.T + 3) / 4) * ((g.Hh + 3) / 4) * ((g.W + 3) / 4);
    if (c * 64 > INT32_MAX) return vsa::fail(VSA_ERR_INVALID, "vsa_cube_dims: grid too large");
    *n_cubes = (int32_t)c;
    *n_slots = (int32_t)(c * 64);
    return VSA_OK;
}

int vsa_check_block_list_host(const int32_t* kv_idx, const int32_t* kv_cnt, int64_t rows, int nkb,
                              int max_kv) {
    if (!kv_idx || !kv_cnt) return vsa::fail(VSA_ERR_INVALID, "vsa_check_block_list_host: null pointer");
    if (rows < 0 || nkb <= 0 || max_kv <= 0)
        return vsa::fail(VSA_ERR_INVALID, "vsa_check_block_list_host: bad sizes");
    for (int64_t r = 0; r < rows; ++r) {
        int32_t c = kv_cnt[r];
        if (c < 0 || c > max_kv)
            return vsa::fail(VSA_ERR_INVALID, "row %lld: kv_cnt %d outside [0, %d]", (long long)r, c, max_kv);
        const int32_t* row = kv_idx + r * (int64_t)max_kv;
        for (int32_t i = 0; i < c; ++i) {
            if (row[i] < 0 || row[i] >= nkb)
                return vsa::fail(VSA_ERR_INVALID, "row %lld entry %d: block %d outside [0, %d)",
                                 (long long)r, i, row[i], nkb);
            if (i > 0 && row[i] <= row[i - 1])
                return vsa::fail(VSA_ERR_INVALID, "row %lld entry %d: not strictly ascending",
                                 (long long)r, i);
        }
    }
    return VSA_OK;
}

// Host self-check of the constant-divisor helper used by the kernels' index maps.
int vsa_selftest_host(void) {
    const uint32_t divisors[] = {1, 2, 3, 4, 5, 7, 21, 30, 33, 45, 52, 64, 80, 126, 1560, 3600,
                                 4096, 32760, 65535, 65536, 196560, 1000003u, 0x7fffffffu};
    for (uint32_t d : divisors) {
        vsa::FastDiv f(d);
        uint32_t probes[] = {0, 1, d - 1, d, d + 1, 2 * d - 1, 2 * d, 12345678u, 0x7ffffffeu,
                             0x7fffffffu, 0xfffffffeu, 0xffffffffu};
        for (uint32_t n : probes)
            if (f.div(n) != n / d)
                return vsa::fail(VSA_ERR_INVALID, "FastDiv(%u) wrong at %u", d, n);
        for (uint32_t n = 0; n < 300000; n += 7)
            if (f.div(n) != n / d) return vsa::fail(VSA_ERR_INVALID, "FastDiv(%u) wrong at %u", d, n);
    }
    return VSA_OK;
}

}  // extern "C"
