// Token permutations of [B, H, N, D] tensors: natural <-> frame-major, and
// natural <-> 4x4x4 cube layout.
//
// Sparse Video-Gen page, "Approach": a token-major to frame-major layout
// transformation makes the same-position tokens of all frames contiguous, so a
// temporal head's sparse pattern becomes dense tiles. USV page, Figure 2
// caption: the cube layout groups the tokens of Q, K and V into 4x4x4
// spatio-temporal cubes, each stored as one 64-slot block.
//
// Pure data movement, HBM-bound: every destination row (one token's D values)
// is produced by one group of lanes moving 16 bytes each, so a row of a bf16
// D=128 tensor (256 B) is one fully coalesced 16-lane access on both sides.
// Each thread keeps UNROLL loads in flight before its first store.
#include "vsa_internal.h"

namespace vsa {

struct PermArgs {
    int64_t rows_dst_total;     // B*H*rows_dst
    int32_t rows_dst, rows_src; // rows per (b, h) on each side
    int32_t T, Hh, W, HW;
    int32_t cy_n, cx_n;         // cubes along y and x
    FastDiv div_rows_dst, div_H, div_T, div_HW, div_W, div_cyx, div_cx;
    int32_t H;
    uint32_t head_bits[32];     // head_sel as a bitmask (bit h set = head h moves)
};

enum { K_FM_FWD = 0, K_FM_INV = 1, K_CUBE_FWD = 2, K_CUBE_INV = 3 };

// Source row (within its (b, h) slice) of destination row r, or -1 for a
// zero-filled pad slot.
template <int KIND>
__device__ __forceinline__ int32_t source_row(const PermArgs& a, uint32_t r, bool moves) {
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
