// Status codes, per-thread error messages and host-only entry points.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "vsa_internal.h"

namespace vsa {

static thread_local char g_last_error[512] = "";

// Call log: with VSA_TRACE set to a non-empty value other than "0", every
// launch the library makes and every rejected call is written to stderr, one
// line each ("[vsa] <call>: <outcome>"), in the order they happen on the host.
static bool trace_on() {
    static const bool on = [] {
        const char* v = getenv("VSA_TRACE");
        return v && *v && !(v[0] == '0' && v[1] == 0);
    }();
    return on;
}

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    if (trace_on()) fprintf(stderr, "[vsa] rejected (status %d): %s\n", status, g_last_error);
    return status;
}

int launch_status(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(VSA_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    if (trace_on()) fprintf(stderr, "[vsa] %s: launched\n", what);
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
    const int pst = vsa::permute_selftest_host();
    if (pst != VSA_OK) return pst;
    const int bst = vsa::profile_selftest_host();
    if (bst != VSA_OK) return bst;
    // group_remap: a bijection on [0, G) (or -1 everywhere) for head counts,
    // block counts and group patterns around the video shapes; with one group it
    // is xcd_remap, and every XCD gets an equal share (+-1 item) of each group
    const int nbs[] = {1, 2, 3, 5, 7, 8, 9, 31, 256, 929, 1536};
    const int heads[] = {1, 2, 3, 7, 8, 12, 24, 64};
    std::vector<int> seen;
    for (int nb : nbs)
        for (int BH : heads)
            for (int pat = 0; pat < 6; ++pat) {
                uint64_t gm[vsa::kGroups] = {0, 0, 0, 0, 0};
                for (int h = 0; h < BH; ++h) {
                    int g = 0;
                    if (pat == 1) g = h & 1;
                    if (pat == 2) g = (h % 3 == 1) ? 4 : 0;
                    if (pat == 3) g = (h * 7 + 3) % 5;
                    if (pat == 4) g = h < BH / 2 ? 2 : 1;
                    if (pat == 5) g = (h == BH - 1) ? 3 : 1;
                    gm[g] |= 1ull << h;
                }
                const int G = BH * nb;
                seen.assign(G, 0);
                const int first = vsa::group_remap(0, G, nb, gm);
                int ngroups = 0;
                for (int g = 0; g < vsa::kGroups; ++g) ngroups += gm[g] != 0;
                long share[8][vsa::kGroups] = {};
                for (int bid = 0; bid < G; ++bid) {
                    const int it = vsa::group_remap(bid, G, nb, gm);
                    if ((it < 0) != (first < 0))
                        return vsa::fail(VSA_ERR_INVALID, "group_remap: mixed fallback nb=%d heads=%d", nb, BH);
                    if (it < 0) continue;
                    if (it >= G || seen[it]++)
                        return vsa::fail(VSA_ERR_INVALID, "group_remap: not a bijection nb=%d heads=%d pat=%d", nb,
                                         BH, pat);
                    if (ngroups == 1 && it != vsa::xcd_remap(bid, G))
                        return vsa::fail(VSA_ERR_INVALID, "group_remap: one group differs from xcd_remap");
                    for (int g = 0; g < vsa::kGroups; ++g)
                        if ((gm[g] >> (it / nb)) & 1) share[bid & 7][g]++;
                }
                if (first < 0) {
                    if (nb >= 32) return vsa::fail(VSA_ERR_INVALID, "group_remap: fallback at nb=%d", nb);
                    continue;
                }
                for (int g = 0; g < vsa::kGroups; ++g) {
                    const long Gg = (long)__builtin_popcountll(gm[g]) * nb;
                    for (int x = 0; x < 8; ++x)
                        if (share[x][g] < Gg / 8 - vsa::kGroups || share[x][g] > Gg / 8 + vsa::kGroups)
                            return vsa::fail(VSA_ERR_INVALID, "group_remap: unequal share nb=%d heads=%d", nb, BH);
                }
            }
    // run_remap: a bijection on [0, G) around whole groups of 8 runs and ragged tails
    const int gs[] = {1, 7, 8, 511, 512, 513, 1023, 1024, 1536, 12 * 1536, 24 * 929, 12 * 1536 + 37};
    for (int G : gs) {
        seen.assign(G, 0);
        for (int bid = 0; bid < G; ++bid) {
            const int it = vsa::run_remap(bid, G);
            if (it < 0 || it >= G || seen[it]++)
                return vsa::fail(VSA_ERR_INVALID, "run_remap: not a bijection G=%d", G);
            // inside whole groups, XCD bid % 8 takes runs x, x + 8, ... in order
            if (bid < G / (8 * vsa::kHeadRun) * (8 * vsa::kHeadRun) && (it / vsa::kHeadRun) % 8 != (bid & 7))
                return vsa::fail(VSA_ERR_INVALID, "run_remap: run on the wrong XCD G=%d", G);
        }
    }
    return VSA_OK;
}

}  // extern "C"
