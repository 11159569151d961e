// Token permutations of [B, H, N, D] tensors: natural <-> frame-major, and
// natural <-> 4x4x4 cube layout.
//
// Sparse Video-Gen page, "Approach": a token-major to frame-major layout
// transformation makes the same-position tokens of all frames contiguous, so a
// temporal head's sparse pattern becomes dense tiles. USV page, Figure 2
// caption: the cube layout groups the tokens of Q, K and V into 4x4x4
// spatio-temporal cubes, each stored as one 64-slot block. OSP-Next page,
// "Method": fixed token-wise and group-wise spatial patterns; stored subset by
// subset (each subset padded to whole blocks) they become a block-diagonal mask.
//
// Pure data movement, HBM-bound: every destination row (one token's D values)
// is produced by one group of lanes moving 16 bytes each, so a row of a bf16
// D=128 tensor (256 B) is one fully coalesced 16-lane access on both sides.
// Each thread keeps UNROLL loads in flight before its first store.
#include <algorithm>
#include <vector>

#include "vsa_internal.h"

namespace vsa {

constexpr int kSkipMaxK = 8;    // Skiparse-2D factor k <= 8 (at most 64 subsets)

struct PermArgs {
    int64_t rows_dst_total;     // B*H*rows_dst
    int32_t rows_dst, rows_src; // rows per (b, h) on each side
    int32_t T, Hh, W, HW;
    int32_t cy_n, cx_n;         // cubes along y and x
    FastDiv div_rows_dst, div_H, div_T, div_HW, div_W, div_cyx, div_cx;
    int32_t H;
    uint32_t head_bits[32];     // head_sel as a bitmask (bit h set = head h moves)
    // Skiparse-2D layout: factor k, group-wise flag, per subset c = a k + b its
    // first slot, and per residue a (b) the number of rows (columns) in it
    int32_t sk_k, sk_group, sk_nsub;
    int32_t sk_start[kSkipMaxK * kSkipMaxK + 1];
    int32_t sk_ny[kSkipMaxK], sk_nx[kSkipMaxK];
};

enum { K_FM_FWD = 0, K_FM_INV = 1, K_CUBE_FWD = 2, K_CUBE_INV = 3, K_SKIP_FWD = 4, K_SKIP_INV = 5 };

// Skiparse-2D coordinates along one spatial axis: residue class of coordinate
// y (its subset index along the axis), its rank among the coordinates of that
// class, and the inverse of the rank.
__host__ __device__ __forceinline__ int skip_class(const PermArgs& a, int y) {
    return a.sk_group ? (y / a.sk_k) % a.sk_k : y % a.sk_k;
}
__host__ __device__ __forceinline__ int skip_rank(const PermArgs& a, int y) {
    return a.sk_group ? (y / (a.sk_k * a.sk_k)) * a.sk_k + y % a.sk_k : y / a.sk_k;
}
__host__ __device__ __forceinline__ int skip_coord(const PermArgs& a, int cls, int i) {
    return a.sk_group ? a.sk_k * (cls + a.sk_k * (i / a.sk_k)) + i % a.sk_k : cls + a.sk_k * i;
}

// Source row (within its (b, h) slice) of destination row r, or -1 for a
// zero-filled pad slot.
template <int KIND>
__host__ __device__ __forceinline__ int32_t source_row(const PermArgs& a, uint32_t r, bool moves) {
    if (KIND == K_FM_FWD) {                 // r = s*T + t  <-  n = t*HW + s
        if (!moves) return (int32_t)r;
        uint32_t s = a.div_T.div(r);
        uint32_t t = r - s * a.T;
        return (int32_t)(t * a.HW + s);
    } else if (KIND == K_FM_INV) {          // r = t*HW + s  <-  s*T + t
        if (!moves) return (int32_t)r;
        uint32_t t = a.div_HW.div(r);
        uint32_t s = r - t * a.HW;
        return (int32_t)(s * a.T + t);
    } else if (KIND == K_CUBE_FWD) {        // slot r = 64*c + rank  <-  natural token
        uint32_t c = r >> 6, rank = r & 63u;
        uint32_t ct = a.div_cyx.div(c);
        uint32_t rem = c - ct * (uint32_t)(a.cy_n * a.cx_n);
        uint32_t cy = a.div_cx.div(rem);
        uint32_t cx = rem - cy * a.cx_n;
        int et = min(4, a.T - 4 * (int)ct), ey = min(4, a.Hh - 4 * (int)cy), ex = min(4, a.W - 4 * (int)cx);
        if ((int)rank >= et * ey * ex) return -1;
        int plane = ey * ex;
        int dt = (int)rank / plane;        // small divisors (<= 16)
        int r2 = (int)rank - dt * plane;
        int dy = r2 / ex, dx = r2 - (r2 / ex) * ex;
        int t = 4 * (int)ct + dt, y = 4 * (int)cy + dy, x = 4 * (int)cx + dx;
        return (t * a.Hh + y) * a.W + x;
    } else if (KIND == K_SKIP_FWD) {        // padded subset slot r  <-  natural token
        int c = 0;
        while (c + 1 < a.sk_nsub && (int)r >= a.sk_start[c + 1]) ++c;
        const int ca = c / a.sk_k, cb = c - ca * a.sk_k;
        const int ny = a.sk_ny[ca], nx = a.sk_nx[cb];
        const int rank = (int)r - a.sk_start[c];
        if (rank >= a.T * ny * nx) return -1;
        const int t = rank / (ny * nx), rem = rank - t * (ny * nx);
        const int iy = rem / nx, ix = rem - iy * nx;
        return (t * a.Hh + skip_coord(a, ca, iy)) * a.W + skip_coord(a, cb, ix);
    } else if (KIND == K_SKIP_INV) {        // natural n  <-  its padded subset slot
        uint32_t t = a.div_HW.div(r);
        uint32_t rem = r - t * a.HW;
        int y = (int)a.div_W.div(rem);
        int x = (int)rem - y * a.W;
        const int ca = skip_class(a, y), cb = skip_class(a, x);
        const int rank = ((int)t * a.sk_ny[ca] + skip_rank(a, y)) * a.sk_nx[cb] + skip_rank(a, x);
        return a.sk_start[ca * a.sk_k + cb] + rank;
    } else {                                // natural n  <-  slot 64*c + rank
        uint32_t t = a.div_HW.div(r);
        uint32_t rem = r - t * a.HW;
        uint32_t y = a.div_W.div(rem);
        uint32_t x = rem - y * a.W;
        uint32_t ct = t >> 2, cy = y >> 2, cx = x >> 2;
        uint32_t c = (ct * a.cy_n + cy) * a.cx_n + cx;
        int ey = min(4, a.Hh - 4 * (int)cy), ex = min(4, a.W - 4 * (int)cx);
        int rank = ((int)(t & 3) * ey + (int)(y & 3)) * ex + (int)(x & 3);
        return (int32_t)(c * 64 + rank);
    }
}

template <int CPR, int KIND, int UNROLL>
__global__ __launch_bounds__(256) void permute_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                      PermArgs a) {
    constexpr int RPP = 256 / CPR;                      // rows per pass of the workgroup
    const int chunk = threadIdx.x % CPR;
    const int64_t row0 = (int64_t)blockIdx.x * (RPP * UNROLL) + threadIdx.x / CPR;
    u32x4 val[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        int64_t g = row0 + (int64_t)u * RPP;
        val[u] = u32x4{0u, 0u, 0u, 0u};
        if (g < a.rows_dst_total) {
            uint32_t bh = a.div_rows_dst.div((uint32_t)g);
            uint32_t r = (uint32_t)(g - (int64_t)bh * a.rows_dst);
            bool moves = true;
            if (KIND == K_FM_FWD || KIND == K_FM_INV) {
                uint32_t h = bh - a.div_H.div(bh) * a.H;
                moves = (a.head_bits[h >> 5] >> (h & 31)) & 1u;
            }
            int32_t sr = source_row<KIND>(a, r, moves);
            if (sr >= 0) val[u] = src[((int64_t)bh * a.rows_src + sr) * CPR + chunk];
        }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        int64_t g = row0 + (int64_t)u * RPP;
        if (g < a.rows_dst_total) dst[g * CPR + chunk] = val[u];
    }
}

template <int CPR>
static void launch_permute(int kind_id, const void* src, void* dst, const PermArgs& a, hipStream_t s) {
    constexpr int UNROLL = 4;
    constexpr int RPP = 256 / CPR;
    int64_t blocks = (a.rows_dst_total + RPP * UNROLL - 1) / (RPP * UNROLL);
    const u32x4* sp = static_cast<const u32x4*>(src);
    u32x4* dp = static_cast<u32x4*>(dst);
    switch (kind_id) {
        case K_FM_FWD: hipLaunchKernelGGL((permute_kernel<CPR, K_FM_FWD, UNROLL>), dim3((unsigned)blocks), dim3(256), 0, s, sp, dp, a); break;
        case K_FM_INV: hipLaunchKernelGGL((permute_kernel<CPR, K_FM_INV, UNROLL>), dim3((unsigned)blocks), dim3(256), 0, s, sp, dp, a); break;
        case K_CUBE_FWD: hipLaunchKernelGGL((permute_kernel<CPR, K_CUBE_FWD, UNROLL>), dim3((unsigned)blocks), dim3(256), 0, s, sp, dp, a); break;
        case K_SKIP_FWD: hipLaunchKernelGGL((permute_kernel<CPR, K_SKIP_FWD, UNROLL>), dim3((unsigned)blocks), dim3(256), 0, s, sp, dp, a); break;
        case K_SKIP_INV: hipLaunchKernelGGL((permute_kernel<CPR, K_SKIP_INV, UNROLL>), dim3((unsigned)blocks), dim3(256), 0, s, sp, dp, a); break;
        default: hipLaunchKernelGGL((permute_kernel<CPR, K_CUBE_INV, UNROLL>), dim3((unsigned)blocks), dim3(256), 0, s, sp, dp, a); break;
    }
}

}  // namespace vsa

using namespace vsa;

extern "C" int vsa_permute(const void* src, void* dst, int B, int H, vsa_grid g, int D, int dtype, int kind,
                           int inverse, const uint8_t* head_sel, void* stream) {
    if (!src || !dst) return fail(VSA_ERR_INVALID, "vsa_permute: null tensor");
    if (!aligned16(src) || !aligned16(dst)) return fail(VSA_ERR_INVALID, "vsa_permute: pointers must be 16-byte aligned");
    if (B <= 0 || H <= 0) return fail(VSA_ERR_INVALID, "vsa_permute: B and H must be positive");
    if (g.T <= 0 || g.Hh <= 0 || g.W <= 0) return fail(VSA_ERR_INVALID, "vsa_permute: bad grid");
    if (D != 64 && D != 128) return fail(VSA_ERR_UNSUPPORTED, "vsa_permute: D must be 64 or 128 (got %d)", D);
    int elem;
    if (dtype == VSA_BF16) elem = 2;
    else if (dtype == VSA_F32) elem = 4;
    else return fail(VSA_ERR_UNSUPPORTED, "vsa_permute: dtype %d not supported", dtype);
    if (kind != VSA_PERM_FRAME_MAJOR && kind != VSA_PERM_CUBE4)
        return fail(VSA_ERR_INVALID, "vsa_permute: unknown kind %d", kind);
    if (inverse != 0 && inverse != 1) return fail(VSA_ERR_INVALID, "vsa_permute: inverse must be 0 or 1");
    int64_t N = (int64_t)g.T * g.Hh * g.W;
    if (N >= (1ll << 31)) return fail(VSA_ERR_INVALID, "vsa_permute: grid too large");
    PermArgs a = {};
    a.T = g.T; a.Hh = g.Hh; a.W = g.W; a.HW = g.Hh * g.W; a.H = H;
    a.cy_n = (g.Hh + 3) / 4; a.cx_n = (g.W + 3) / 4;
    int kind_id;
    if (kind == VSA_PERM_FRAME_MAJOR) {
        if (H > 1024) return fail(VSA_ERR_INVALID, "vsa_permute: H must be <= 1024");
        for (int h = 0; h < H; ++h)
            if (!head_sel || head_sel[h]) a.head_bits[h >> 5] |= 1u << (h & 31);
        a.rows_dst = a.rows_src = (int32_t)N;
        kind_id = inverse ? K_FM_INV : K_FM_FWD;
    } else {
        if (head_sel) return fail(VSA_ERR_INVALID, "vsa_permute: cube layout moves every head (head_sel must be NULL)");
        int32_t n_cubes, n_slots;
        int st = vsa_cube_dims(g, &n_cubes, &n_slots);
        if (st) return st;
        a.rows_dst = inverse ? (int32_t)N : n_slots;
        a.rows_src = inverse ? n_slots : (int32_t)N;
        kind_id = inverse ? K_CUBE_INV : K_CUBE_FWD;
    }
    a.rows_dst_total = (int64_t)B * H * a.rows_dst;
    if (a.rows_dst_total >= (1ll << 31)) return fail(VSA_ERR_INVALID, "vsa_permute: B*H*rows exceeds 2^31");
    a.div_rows_dst = FastDiv((uint32_t)a.rows_dst);
    a.div_H = FastDiv((uint32_t)H);
    a.div_T = FastDiv((uint32_t)g.T);
    a.div_HW = FastDiv((uint32_t)a.HW);
    a.div_W = FastDiv((uint32_t)g.W);
    a.div_cyx = FastDiv((uint32_t)(a.cy_n * a.cx_n));
    a.div_cx = FastDiv((uint32_t)a.cx_n);
    int cpr = D * elem / 16;
    hipStream_t s = as_stream(stream);
    if (cpr == 8) launch_permute<8>(kind_id, src, dst, a, s);
    else if (cpr == 16) launch_permute<16>(kind_id, src, dst, a, s);
    else launch_permute<32>(kind_id, src, dst, a, s);
    return launch_status("vsa_permute");
}

// ---------------------------------------------------------------------------
// Skiparse-2D layout (OSP-Next page, "Method").
namespace {

struct SkipPlan {
    int k, group, nsub, bs;
    int32_t ny[kSkipMaxK], nx[kSkipMaxK];
    int32_t start[kSkipMaxK * kSkipMaxK + 1];   // first slot of each subset; [nsub] = n_slots
    int64_t n_slots;
};

// Number of coordinates in [0, n) of residue class `cls` along one axis.
int skip_axis_count(int n, int k, int group, int cls) {
    int cnt = 0;
    for (int y = 0; y < n; ++y) cnt += (group ? (y / k) % k : y % k) == cls;
    return cnt;
}

int skip_plan(const char* fn, vsa_grid g, int mode, int k, int bs, SkipPlan& p) {
    if (g.T <= 0 || g.Hh <= 0 || g.W <= 0) return fail(VSA_ERR_INVALID, "%s: grid extents must be positive", fn);
    if (mode != VSA_SKIPARSE_TOKEN && mode != VSA_SKIPARSE_GROUP)
        return fail(VSA_ERR_INVALID, "%s: unknown mode %d", fn, mode);
    if (k < 1 || k > kSkipMaxK) return fail(VSA_ERR_INVALID, "%s: k must be in [1, %d]", fn, kSkipMaxK);
    if (bs < 1 || bs > 1024) return fail(VSA_ERR_INVALID, "%s: bs must be in [1, 1024]", fn);
    const int64_t N = (int64_t)g.T * g.Hh * g.W;
    if (N >= (1ll << 30)) return fail(VSA_ERR_INVALID, "%s: grid too large", fn);
    p.k = k; p.group = mode == VSA_SKIPARSE_GROUP; p.nsub = k * k; p.bs = bs;
    for (int c = 0; c < kSkipMaxK; ++c) {
        p.ny[c] = c < k ? skip_axis_count(g.Hh, k, p.group, c) : 0;
        p.nx[c] = c < k ? skip_axis_count(g.W, k, p.group, c) : 0;
    }
    int64_t slot = 0;
    for (int c = 0; c < p.nsub; ++c) {
        p.start[c] = (int32_t)slot;
        const int64_t n = (int64_t)g.T * p.ny[c / k] * p.nx[c % k];
        slot += (n + bs - 1) / bs * bs;
    }
    p.start[p.nsub] = (int32_t)slot;
    p.n_slots = slot;
    if (slot >= (1ll << 30)) return fail(VSA_ERR_INVALID, "%s: padded layout too large", fn);
    return VSA_OK;
}

struct SkipBlockArgs {
    int32_t nsub, bs, nb, T;
    int32_t k;
    int32_t start[kSkipMaxK * kSkipMaxK + 1];
    int32_t ny[kSkipMaxK], nx[kSkipMaxK];
};

__device__ __forceinline__ int skip_block_subset(const SkipBlockArgs& a, int b) {
    int c = 0;
    while (c + 1 < a.nsub && b * a.bs >= a.start[c + 1]) ++c;
    return c;
}

// Valid slots of each block: a subset's tokens fill its first slots.
__global__ __launch_bounds__(256) void skip_block_len_kernel(SkipBlockArgs a, int32_t* blk_len) {
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b >= a.nb) return;
    const int c = skip_block_subset(a, b);
    const int n = a.T * a.ny[c / a.k] * a.nx[c % a.k];
    const int v = n - (b * a.bs - a.start[c]);
    blk_len[b] = v < 0 ? 0 : (v > a.bs ? a.bs : v);
}

// Block-diagonal mask: block b attends to the blocks of its own subset.
__global__ __launch_bounds__(256) void skip_mask_kernel(SkipBlockArgs a, uint8_t* mask) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)a.nb * a.nb) return;
    const int qb = (int)(e / a.nb), kb = (int)(e - (int64_t)qb * a.nb);
    mask[e] = skip_block_subset(a, qb) == skip_block_subset(a, kb) ? 1 : 0;
}

SkipBlockArgs block_args(const SkipPlan& p, vsa_grid g) {
    SkipBlockArgs a = {};
    a.nsub = p.nsub; a.bs = p.bs; a.nb = (int32_t)(p.n_slots / p.bs); a.T = g.T; a.k = p.k;
    for (int c = 0; c <= p.nsub; ++c) a.start[c] = p.start[c];
    for (int c = 0; c < kSkipMaxK; ++c) { a.ny[c] = p.ny[c]; a.nx[c] = p.nx[c]; }
    return a;
}

}  // namespace

extern "C" int vsa_skiparse_dims(vsa_grid g, int mode, int k, int bs, int32_t* n_slots, int32_t* n_blocks) {
    SkipPlan p;
    const int st = skip_plan("vsa_skiparse_dims", g, mode, k, bs, p);
    if (st) return st;
    if (n_slots) *n_slots = (int32_t)p.n_slots;
    if (n_blocks) *n_blocks = (int32_t)(p.n_slots / bs);
    return VSA_OK;
}

extern "C" int vsa_skiparse_block_len(vsa_grid g, int mode, int k, int bs, int32_t* blk_len, void* stream) {
    const char* fn = "vsa_skiparse_block_len";
    if (!blk_len) return fail(VSA_ERR_INVALID, "%s: null output", fn);
    SkipPlan p;
    const int st = skip_plan(fn, g, mode, k, bs, p);
    if (st) return st;
    const SkipBlockArgs a = block_args(p, g);
    hipLaunchKernelGGL(skip_block_len_kernel, dim3((unsigned)((a.nb + 255) / 256)), dim3(256), 0, as_stream(stream),
                       a, blk_len);
    return launch_status(fn);
}

extern "C" int vsa_skiparse_mask(vsa_grid g, int mode, int k, int bs, uint8_t* mask, void* stream) {
    const char* fn = "vsa_skiparse_mask";
    if (!mask) return fail(VSA_ERR_INVALID, "%s: null output", fn);
    SkipPlan p;
    const int st = skip_plan(fn, g, mode, k, bs, p);
    if (st) return st;
    const SkipBlockArgs a = block_args(p, g);
    const int64_t total = (int64_t)a.nb * a.nb;
    hipLaunchKernelGGL(skip_mask_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, as_stream(stream), a,
                       mask);
    return launch_status(fn);
}

extern "C" int vsa_skiparse_permute(const void* src, void* dst, int B, int H, vsa_grid g, int D, int dtype, int mode,
                                    int k, int bs, int inverse, void* stream) {
    const char* fn = "vsa_skiparse_permute";
    if (!src || !dst) return fail(VSA_ERR_INVALID, "%s: null tensor", fn);
    if (!aligned16(src) || !aligned16(dst)) return fail(VSA_ERR_INVALID, "%s: pointers must be 16-byte aligned", fn);
    if (B <= 0 || H <= 0) return fail(VSA_ERR_INVALID, "%s: B and H must be positive", fn);
    if (D != 64 && D != 128) return fail(VSA_ERR_UNSUPPORTED, "%s: D must be 64 or 128 (got %d)", fn, D);
    int elem;
    if (dtype == VSA_BF16) elem = 2;
    else if (dtype == VSA_F32) elem = 4;
    else return fail(VSA_ERR_UNSUPPORTED, "%s: dtype %d not supported", fn, dtype);
    if (inverse != 0 && inverse != 1) return fail(VSA_ERR_INVALID, "%s: inverse must be 0 or 1", fn);
    SkipPlan p;
    const int st = skip_plan(fn, g, mode, k, bs, p);
    if (st) return st;
    const int64_t N = (int64_t)g.T * g.Hh * g.W;
    PermArgs a = {};
    a.T = g.T; a.Hh = g.Hh; a.W = g.W; a.HW = g.Hh * g.W; a.H = H;
    a.sk_k = k; a.sk_group = p.group; a.sk_nsub = p.nsub;
    for (int c = 0; c <= p.nsub; ++c) a.sk_start[c] = p.start[c];
    for (int c = 0; c < kSkipMaxK; ++c) { a.sk_ny[c] = p.ny[c]; a.sk_nx[c] = p.nx[c]; }
    a.rows_dst = inverse ? (int32_t)N : (int32_t)p.n_slots;
    a.rows_src = inverse ? (int32_t)p.n_slots : (int32_t)N;
    a.rows_dst_total = (int64_t)B * H * a.rows_dst;
    if (a.rows_dst_total >= (1ll << 31)) return fail(VSA_ERR_INVALID, "%s: B*H*rows exceeds 2^31", fn);
    a.div_rows_dst = FastDiv((uint32_t)a.rows_dst);
    a.div_H = FastDiv((uint32_t)H);
    a.div_T = FastDiv((uint32_t)g.T);
    a.div_HW = FastDiv((uint32_t)a.HW);
    a.div_W = FastDiv((uint32_t)g.W);
    a.div_cyx = FastDiv(1u);
    a.div_cx = FastDiv(1u);
    const int kind_id = inverse ? K_SKIP_INV : K_SKIP_FWD;
    const int cpr = D * elem / 16;
    hipStream_t s = as_stream(stream);
    if (cpr == 8) launch_permute<8>(kind_id, src, dst, a, s);
    else if (cpr == 16) launch_permute<16>(kind_id, src, dst, a, s);
    else launch_permute<32>(kind_id, src, dst, a, s);
    return launch_status(fn);
}

// ---------------------------------------------------------------------------
// Host check of the layout maps the kernels use (the same source_row code): for
// grids with ragged edges, every forward map sends each destination slot to a
// source row in range or to a pad, and the inverse map brings every natural
// token back to the slot that reads it.
namespace vsa {
int permute_selftest_host() {
    const vsa_grid grids[] = {{1, 1, 8}, {2, 9, 7}, {3, 6, 10}, {5, 6, 9}, {4, 8, 8}, {2, 17, 23}, {1, 30, 52}};
    for (const vsa_grid& g : grids) {
        const int N = g.T * g.Hh * g.W;
        PermArgs a = {};
        a.T = g.T; a.Hh = g.Hh; a.W = g.W; a.HW = g.Hh * g.W; a.H = 1;
        a.cy_n = (g.Hh + 3) / 4; a.cx_n = (g.W + 3) / 4;
        a.div_T = FastDiv((uint32_t)g.T);
        a.div_HW = FastDiv((uint32_t)a.HW);
        a.div_W = FastDiv((uint32_t)g.W);
        a.div_cyx = FastDiv((uint32_t)(a.cy_n * a.cx_n));
        a.div_cx = FastDiv((uint32_t)a.cx_n);
        std::vector<int> back(N);
        // frame-major: forward and inverse are inverse bijections
        for (int r = 0; r < N; ++r) {
            const int n = source_row<K_FM_FWD>(a, (uint32_t)r, true);
            if (n < 0 || n >= N || source_row<K_FM_INV>(a, (uint32_t)n, true) != r)
                return fail(VSA_ERR_INVALID, "frame-major map wrong at %d (grid %dx%dx%d)", r, g.T, g.Hh, g.W);
        }
        // cube layout
        int32_t n_cubes, n_slots;
        if (vsa_cube_dims(g, &n_cubes, &n_slots)) return VSA_ERR_INVALID;
        int valid = 0;
        for (int r = 0; r < n_slots; ++r) {
            const int n = source_row<K_CUBE_FWD>(a, (uint32_t)r, true);
            if (n < -1 || n >= N || (n >= 0 && source_row<K_CUBE_INV>(a, (uint32_t)n, true) != r))
                return fail(VSA_ERR_INVALID, "cube map wrong at slot %d", r);
            valid += n >= 0;
        }
        if (valid != N) return fail(VSA_ERR_INVALID, "cube map covers %d of %d tokens", valid, N);
        // Skiparse-2D, both modes, several factors and block sizes
        for (int mode = 0; mode < 2; ++mode)
            for (int k = 1; k <= 4; ++k)
                for (int bs : {1, 3, 8, 64}) {
                    SkipPlan p;
                    if (skip_plan("permute_selftest_host", g, mode, k, bs, p)) return VSA_ERR_INVALID;
                    a.sk_k = k; a.sk_group = p.group; a.sk_nsub = p.nsub;
                    for (int c = 0; c <= p.nsub; ++c) a.sk_start[c] = p.start[c];
                    for (int c = 0; c < kSkipMaxK; ++c) { a.sk_ny[c] = p.ny[c]; a.sk_nx[c] = p.nx[c]; }
                    std::fill(back.begin(), back.end(), -1);
                    for (int r = 0; r < (int)p.n_slots; ++r) {
                        const int n = source_row<K_SKIP_FWD>(a, (uint32_t)r, true);
                        if (n < -1 || n >= N)
                            return fail(VSA_ERR_INVALID, "skiparse slot %d out of range (mode %d k %d bs %d)", r, mode,
                                        k, bs);
                        if (n >= 0) {
                            if (back[n] >= 0) return fail(VSA_ERR_INVALID, "skiparse token %d read twice", n);
                            back[n] = r;
                        }
                    }
                    for (int n = 0; n < N; ++n) {
                        const int r = source_row<K_SKIP_INV>(a, (uint32_t)n, true);
                        if (back[n] < 0 || r != back[n])
                            return fail(VSA_ERR_INVALID, "skiparse inverse wrong at token %d (mode %d k %d bs %d)", n,
                                        mode, k, bs);
                        // subset of the slot's block holds the token's subset
                        const int y = (n / g.W) % g.Hh, x = n % g.W;
                        const int c = skip_class(a, y) * k + skip_class(a, x);
                        if (r < p.start[c] || r >= p.start[c + 1])
                            return fail(VSA_ERR_INVALID, "skiparse token %d outside its subset", n);
                    }
                }
    }
    return VSA_OK;
}
}  // namespace vsa
