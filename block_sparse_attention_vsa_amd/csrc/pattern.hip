// Block masks from token patterns, cube valid lengths, and mask -> block list.
//
// Sparse Video-Gen page, "Approach": spatial heads attend within a frame,
// temporal heads attend to the same position across frames once tokens are in
// frame-major order. A (query block, key block) tile is kept iff some token pair
// in it satisfies the pattern. Along either layout the pattern coordinate
// (frame t in natural order, position s = y*W + x in frame-major order) never
// decreases and steps by at most 1, so a block's coordinates are exactly the
// integers between its first and last token's, and the any-rule reduces to an
// interval-overlap test of [first, last] ranges widened by w.
#include "vsa_internal.h"

namespace vsa {

__global__ void pattern_mask_kernel(uint8_t* __restrict__ mask, int nb, int bs, int64_t N,
                                    int64_t coord_div, int64_t w) {
    int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (int64_t)nb * nb) return;
    int64_t qb = e / nb, kb = e - qb * nb;
    int64_t q_lo = (qb * bs) / coord_div;
    int64_t q_hi = (min((qb + 1) * bs, N) - 1) / coord_div;
    int64_t k_lo = (kb * bs) / coord_div;
    int64_t k_hi = (min((kb + 1) * bs, N) - 1) / coord_div;
    mask[e] = (q_lo - w <= k_hi) && (k_lo <= q_hi + w);
}

__global__ void cube_len_kernel(int32_t* __restrict__ blk_len, int n_cubes, int T, int Hh, int W) {
    int c = blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= n_cubes) return;
    int cx_n = (W + 3) / 4, cy_n = (Hh + 3) / 4;
    int ct = c / (cy_n * cx_n);
    int rem = c - ct * cy_n * cx_n;
    int cy = rem / cx_n, cx = rem - cy * cx_n;
    int et = min(4, T - 4 * ct), ey = min(4, Hh - 4 * cy), ex = min(4, W - 4 * cx);
    blk_len[c] = et * ey * ex;
}

struct HeadSel {          // per-head mask index, passed by value (1 KiB of kernel arguments)
    uint8_t idx[1024];
};

// One wavefront per row: ballot over 64 mask bytes at a time, prefix counts give
// each kept block its slot, so the output is ascending.
__global__ __launch_bounds__(256) void mask_to_list_kernel(
        const uint8_t* __restrict__ mask, int B, int H, int nqb, int nkb, int use_sel, int max_kv, int32_t* __restrict__ kv_idx, int32_t* __restrict__ kv_cnt,
        HeadSel sel) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t rows = (int64_t)B * H * nqb;
    if (row >= rows) return;
    const int qb = (int)(row % nqb);
    const int64_t bh = row / nqb;
    const int h = (int)(bh % H);
    const uint8_t* m = use_sel ? mask + ((int64_t)sel.idx[h] * nqb + qb) * nkb
                               : mask + row * (int64_t)nkb;
    int32_t* out = kv_idx + row * (int64_t)max_kv;
    int count = 0;
    for (int base = 0; base < nkb; base += 64) {
        int j = base + lane;
        bool keep = (j < nkb) && m[j] != 0;
        uint64_t bal = __ballot(keep);
        int pos = count + __popcll(bal & ((1ull << lane) - 1ull));
        if (keep && pos < max_kv) out[pos] = j;
        count += __popcll(bal);
    }
    if (lane == 0) kv_cnt[row] = min(count, max_kv);
}

}  // namespace vsa

using namespace vsa;

extern "C" {

int vsa_pattern_mask(vsa_grid g, int bs, int pattern, int w, uint8_t* mask, void* stream) {
    if (g.T <= 0 || g.Hh <= 0 || g.W <= 0) return fail(VSA_ERR_INVALID, "vsa_pattern_mask: bad grid");
    if (bs < 1 || bs > 1024) return fail(VSA_ERR_INVALID, "vsa_pattern_mask: bs must be in [1, 1024]");
    if (w < 0) return fail(VSA_ERR_INVALID, "vsa_pattern_mask: w must be >= 0");
    if (!mask) return fail(VSA_ERR_INVALID, "vsa_pattern_mask: null mask");
    int64_t N = (int64_t)g.T * g.Hh * g.W;
    int64_t nb = (N + bs - 1) / bs;
    if (nb > 65536) return fail(VSA_ERR_INVALID, "vsa_pattern_mask: too many blocks");
    int64_t coord_div;
    if (pattern == VSA_PATTERN_SPATIAL) coord_div = (int64_t)g.Hh * g.W;     // frame of a natural position
    else if (pattern == VSA_PATTERN_TEMPORAL) coord_div = g.T;              // (y, x) of a frame-major position
    else return fail(VSA_ERR_INVALID, "vsa_pattern_mask: unknown pattern %d", pattern);
    int64_t total = nb * nb;
    int threads = 256;
    int blocks = (int)((total + threads - 1) / threads);
    hipLaunchKernelGGL(pattern_mask_kernel, dim3(blocks), dim3(threads), 0, as_stream(stream), mask,
                       (int)nb, bs, N, coord_div, (int64_t)w);
    return launch_status("vsa_pattern_mask");
}

int vsa_cube_block_len(vsa_grid g, int32_t* blk_len, void* stream) {
    int32_t n_cubes, n_slots;
    int st = vsa_cube_dims(g, &n_cubes, &n_slots);
    if (st) return st;
    if (!blk_len) return fail(VSA_ERR_INVALID, "vsa_cube_block_len: null blk_len");
    hipLaunchKernelGGL(cube_len_kernel, dim3((n_cubes + 255) / 256), dim3(256), 0, as_stream(stream),
                       blk_len, n_cubes, g.T, g.Hh, g.W);
    return launch_status("vsa_cube_block_len");
}

int vsa_mask_to_list(const uint8_t* mask, int B, int H, int nqb, int nkb, const int32_t* head_mask_idx,
                     int P, int max_kv, int32_t* kv_idx, int32_t* kv_cnt, void* stream) {
    if (!mask || !kv_idx || !kv_cnt) return fail(VSA_ERR_INVALID, "vsa_mask_to_list: null pointer");
    if (B <= 0 || H <= 0 || nqb <= 0 || nkb <= 0)
        return fail(VSA_ERR_INVALID, "vsa_mask_to_list: sizes must be positive");
    if (max_kv < 1 || max_kv > nkb) return fail(VSA_ERR_INVALID, "vsa_mask_to_list: max_kv must be in [1, nkb]");
    HeadSel sel;
    int use_sel = head_mask_idx != nullptr;
    if (use_sel) {
        if (H > 1024) return fail(VSA_ERR_INVALID, "vsa_mask_to_list: head_mask_idx needs H <= 1024");
        if (P <= 0 || P > 255) return fail(VSA_ERR_INVALID, "vsa_mask_to_list: P must be in [1, 255]");
        for (int h = 0; h < H; ++h) {
            if (head_mask_idx[h] < 0 || head_mask_idx[h] >= P)
                return fail(VSA_ERR_INVALID, "vsa_mask_to_list: head_mask_idx[%d] = %d outside [0, %d)", h,
                            head_mask_idx[h], P);
            sel.idx[h] = (uint8_t)head_mask_idx[h];
        }
    }
    int64_t rows = (int64_t)B * H * nqb;
    int64_t blocks = (rows + 3) / 4;
    if (blocks > INT32_MAX) return fail(VSA_ERR_INVALID, "vsa_mask_to_list: too many rows");
    hipLaunchKernelGGL(mask_to_list_kernel, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream), mask, B,
                       H, nqb, nkb, use_sel, max_kv, kv_idx, kv_cnt, sel);
    return launch_status("vsa_mask_to_list");
}

}  // extern "C"
