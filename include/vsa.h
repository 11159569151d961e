/*
 * vsa.h - block-sparse attention over a 3D (frames x height x width) video token
 * grid, on AMD Instinct MI355X (gfx950).
 *
 * One C-ABI shared library, libvsa.so. Every entry point is extern "C", takes
 * plain pointers and sizes, and returns an int status (enum vsa_status).
 *
 * Conventions shared by every call
 * --------------------------------
 * Ownership   Every tensor pointer is DEVICE memory owned by the caller, except
 *             arguments marked "host". The library never allocates or frees
 *             device memory and keeps no state between calls.
 * Streams     `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *             Calls are asynchronous on that stream; results are valid once the
 *             caller synchronises it.
 * Layout      Q, K, V, O are contiguous [B, H, N, D] row-major (D fastest) with
 *             16-byte-aligned base pointers. Token n of a T x Hh x W grid sits at
 *             n = (t*Hh + y)*W + x in natural order.
 * Blocks      A blocked layout of N positions with block size bs has
 *             nb = ceil(N / bs) blocks; block b covers positions
 *             [b*bs, min((b+1)*bs, N)). An optional blk_len[nb] (device int32)
 *             marks only the first blk_len[b] positions of block b as valid
 *             (cube padding); NULL means every existing position is valid.
 * dtype       VSA_BF16 (bfloat16) everywhere; VSA_F32 additionally accepted by
 *             vsa_block_sparse_attn_fwd and vsa_permute.
 * Errors      Arguments are validated on the host BEFORE any HIP call; a bad
 *             argument returns VSA_ERR_INVALID or VSA_ERR_UNSUPPORTED and leaves
 *             outputs untouched. A failed launch returns VSA_ERR_LAUNCH. The
 *             message of the last non-zero status of the calling thread is
 *             returned by vsa_last_error(). Device-side data (index lists, masks,
 *             blk_len contents) is not validated on the hot path;
 *             vsa_check_block_list_host validates a list copied to the host.
 *             No C++ exception crosses this interface.
 * Determinism Results are bit-reproducible from run to run: no floating-point
 *             atomics; every reduction has a fixed order.
 * Tracing     With the environment variable VSA_TRACE set (not "0"), every
 *             kernel launch ("[vsa] <call>: launched") and every rejected call
 *             ("[vsa] rejected (status s): <message>") is logged to stderr.
 */
#ifndef VSA_H
#define VSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum vsa_status {
    VSA_OK = 0,
    VSA_ERR_INVALID = 1,      /* invalid argument (null pointer, bad size, ...) */
    VSA_ERR_UNSUPPORTED = 2,  /* valid but not implemented (dtype, D, bs)       */
    VSA_ERR_LAUNCH = 3,       /* a HIP launch or runtime call failed            */
    VSA_ERR_WORKSPACE = 4     /* workspace missing or smaller than required     */
};

enum vsa_dtype { VSA_BF16 = 0, VSA_F32 = 1 };

/* Token orders (vsa_permute). */
enum vsa_perm_kind {
    VSA_PERM_FRAME_MAJOR = 0, /* all frames of one (y, x) contiguous, ordered by t */
    VSA_PERM_CUBE4 = 1        /* 4x4x4 cubes, each padded to 64 slots             */
};

/* Token patterns (vsa_pattern_mask). */
enum vsa_pattern {
    VSA_PATTERN_SPATIAL = 0,  /* |t_q - t_k| <= w, stated in natural order          */
    VSA_PATTERN_TEMPORAL = 1  /* |s_q - s_k| <= w, s = y*W + x, in frame-major order */
};

/* Skiparse-2D patterns (vsa_skiparse_*). */
enum vsa_skiparse_mode {
    VSA_SKIPARSE_TOKEN = 0,   /* subset (y mod k, x mod k)                          */
    VSA_SKIPARSE_GROUP = 1    /* subset ((y div k) mod k, (x div k) mod k): k x k patches */
};

/* FP8 layouts (vsa_fp8_quantize). */
enum vsa_fp8_kind {
    VSA_FP8_ROWS = 0,         /* [B, H, N, D] codes, one scale per (b, h, 64 rows)          */
    VSA_FP8_VT = 1            /* [B, H, ceil(N/64), D, 64] transposed 64-key tiles, one
                                 scale per (b, h, channel)                                 */
};

typedef struct { int32_t T, Hh, W; } vsa_grid;

/* Block sets for vsa_block_sparse_attn_fwd: exactly one of `mask` or
 * (`kv_idx`, `kv_cnt`) is non-NULL.
 *   mask    uint8 [B, H, nqb, nkb]: 1 = compute this (query block, key block) tile.
 *   kv_idx  int32 [B, H, nqb, max_kv]: kept key blocks of each query block; the
 *           first kv_cnt entries are used, in the order given (ascending keeps
 *           results identical to the mask form). Entries must lie in [0, nkb).
 *   kv_cnt  int32 [B, H, nqb]; values above max_kv are clamped to max_kv. */
typedef struct {
    const uint8_t* mask;
    const int32_t* kv_idx;
    const int32_t* kv_cnt;
    int32_t max_kv;
} vsa_blocks;

const char* vsa_status_string(int status);
const char* vsa_last_error(void);
/* Library version as 10000*major + 100*minor + patch. */
int vsa_version(void);
/* Host-only self-check of the library's integer index helpers (constant-divisor
 * division used by the layout maps). Returns VSA_OK or VSA_ERR_INVALID. */
int vsa_selftest_host(void);

/* Number of 4x4x4 cubes of a grid and padded slot count (= 64 * cubes). Host only.
 * Cubes: USV page, Figure 2 caption (the tokens of Q, K and V grouped into small
 * spatio-temporal cubes). */
int vsa_cube_dims(vsa_grid g, int32_t* n_cubes, int32_t* n_slots);

/* Any-rule block mask of a token pattern.
 * Sparse Video-Gen page, "Approach": spatial heads attend block-wise inside a
 * frame; temporal heads attend to the same position across frames, made
 * contiguous by the frame-major layout. A (query block, key block) pair is kept
 * iff some token pair in it satisfies the pattern.
 *   g, bs    grid and block size (1 <= bs <= 1024); nb = ceil(T*Hh*W / bs)
 *   pattern  VSA_PATTERN_SPATIAL (natural order) or VSA_PATTERN_TEMPORAL
 *            (frame-major order); w >= 0 is the window half-width
 *   mask     out, device uint8 [nb, nb] */
int vsa_pattern_mask(vsa_grid g, int bs, int pattern, int w, uint8_t* mask, void* stream);

/* Valid token count of each 4x4x4 cube (cube layout of vsa_permute).
 *   blk_len  out, device int32 [n_cubes] (see vsa_cube_dims) */
int vsa_cube_block_len(vsa_grid g, int32_t* blk_len, void* stream);

/* Token permutation of Q, K, V or O.
 * Sparse Video-Gen page, "Approach" (token-major to frame-major layout
 * transformation) and USV page, Figure 2 caption (3D cube partition).
 *   VSA_PERM_FRAME_MAJOR  forward: dst[h, s*T + t] = src[h, (t*Hh + y)*W + x]
 *                         with s = y*W + x; inverse: the reverse move. src and
 *                         dst are [B, H, N, D]. Heads with head_sel[h] == 0 are
 *                         copied unchanged; head_sel is a host uint8 [H] (H <= 1024)
 *                         or NULL for all heads.
 *   VSA_PERM_CUBE4        forward: src [B, H, N, D] -> dst [B, H, n_slots, D];
 *                         token (t, y, x) goes to slot 64*c + r, c the raster
 *                         index of cube (t/4, y/4, x/4), r its rank among the
 *                         cube's valid tokens in (t, y, x) order; pad slots are
 *                         zero-filled. inverse: [B, H, n_slots, D] -> [B, H, N, D].
 *                         head_sel must be NULL.
 *   dtype VSA_BF16 or VSA_F32; D in {64, 128}. src and dst must not overlap.
 *   Bit-exact: pure data movement. */
int vsa_permute(const void* src, void* dst, int B, int H, vsa_grid g, int D, int dtype,
                int kind, int inverse, const uint8_t* head_sel, void* stream);

/* ---- Skiparse-2D fixed spatial patterns -----------------------------------
 * OSP-Next page, "Method": the sparse attention uses fixed token-wise and
 * group-wise patterns along the spatial axes, kept FlashAttention-compatible.
 * Reading (the page gives no more): factor k in [1, 8]; a token (t, y, x)
 * belongs to subset a*k + b with (a, b) = (y mod k, x mod k) (token-wise) or
 * ((y div k) mod k, (x div k) mod k) (group-wise: contiguous k x k patches, k
 * patches apart); a query attends to every key of its subset, in every frame.
 * Stored subset by subset (subsets in id order, each padded to a whole number
 * of bs-slot blocks, its tokens in its first slots in natural order) the pattern
 * is a block-diagonal block mask, so the flow is
 *   vsa_skiparse_permute(Q, K, V) -> vsa_block_sparse_attn_fwd(bs, mask from
 *   vsa_skiparse_mask, blk_len from vsa_skiparse_block_len) ->
 *   vsa_skiparse_permute(O, inverse = 1).
 * mode is VSA_SKIPARSE_TOKEN or VSA_SKIPARSE_GROUP; bs in [1, 1024]. */

/* Padded layout size (host only): n_slots = n_blocks * bs. */
int vsa_skiparse_dims(vsa_grid g, int mode, int k, int bs, int32_t* n_slots, int32_t* n_blocks);
/* Valid slots of each block: out, device int32 [n_blocks]. */
int vsa_skiparse_block_len(vsa_grid g, int mode, int k, int bs, int32_t* blk_len, void* stream);
/* Block-diagonal mask: out, device uint8 [n_blocks, n_blocks], 1 where both
 * blocks belong to the same subset. */
int vsa_skiparse_mask(vsa_grid g, int mode, int k, int bs, uint8_t* mask, void* stream);
/* Move Q, K, V to the padded layout (inverse = 0: [B, H, N, D] -> [B, H, n_slots, D],
 * pad slots zero-filled) or O back (inverse = 1: [B, H, n_slots, D] -> [B, H, N, D]).
 * dtype VSA_BF16 or VSA_F32; D in {64, 128}; src and dst must not overlap.
 * Bit-exact: pure data movement. */
int vsa_skiparse_permute(const void* src, void* dst, int B, int H, vsa_grid g, int D, int dtype, int mode,
                         int k, int bs, int inverse, void* stream);

/* Block mean-pooling and pooled scores.
 * USV page, Figure 2 caption: long-range key cubes are chosen by top-k cube
 * selection; the score is read as scale * <mean of the query block's valid
 * rows, mean of the key block's valid rows>.
 *   q, k      [B, H, N, D] bf16 (blocked layout, block size bs in {64, 128})
 *   blk_len   optional device int32 [nb]
 *   scale     > 0 (1/sqrt(D) for the attention scale)
 *   scores    out, device fp32 [B, H, nb, nb]
 *   qpool, kpool  out, device fp32 [B, H, nb, D] (required, 16-byte aligned; mean
 *             vectors; a block with no valid row pools to 0). Accumulation in fp32;
 *             the score product runs on the fp32 matrix cores. */
int vsa_block_scores(const void* q, const void* k, int B, int H, int N, int D, int dtype, int bs,
                     const int32_t* blk_len, float scale, float* scores, float* qpool,
                     float* kpool, void* stream);

/* Forced + top-k / top-p block selection, one row per (b, h, query block).
 * USV page, Figure 2 caption (top-k cube selection beside local attention) and
 * Sparse VideoGen2 page, Abstract (top-p dynamic budget control).
 * Per row: forced blocks outrank all others; within each group blocks rank by
 * score (higher first, equal scores by lower index). If the forced count is
 * >= k_max the best k_max forced blocks are kept. Otherwise the non-forced
 * candidates are taken in rank order: with top_p < 1 the shortest prefix
 * (length >= 1) whose softmax mass (softmax over all nkb scores of the row)
 * reaches top_p, else all of them, capped at k_max - forced. Output ascending.
 *   scores   device fp32 [B, H, nqb, nkb]   (1 <= nkb <= 4096)
 *   forced   device uint8 [nqb, nkb] shared by all (b, h), or NULL
 *   k_max    1 <= k_max <= nkb;  top_p in (0, 1] (1 = off)
 *   kv_idx   out, device int32 [B, H, nqb, k_max] (entries past kv_cnt unspecified)
 *   kv_cnt   out, device int32 [B, H, nqb]
 * Softmax terms in fp32; the cumulative mass adds them as integers in units of
 * 2^-31 (each term truncated once), so the kept count does not depend on the
 * order of the additions. Ties exact. */
int vsa_select_topk(const float* scores, int B, int H, int nqb, int nkb, const uint8_t* forced,
                    int k_max, float top_p, int32_t* kv_idx, int32_t* kv_cnt, void* stream);

/* Per-head pattern choice from sampled query rows.
 * Sparse Video-Gen page, "Approach" and "Key results": about 1 % of query rows,
 * each candidate pattern's output compared with dense attention, the
 * lower-error pattern chosen per head.
 *   q, k, v     [B, H, N, D] bf16 in NATURAL order, N = T*Hh*W, D = 128
 *   bs          block size of the candidate masks (64 or 128)
 *   rows        device int32 [R]: sampled natural query rows (distinct, < N)
 *   cand_masks  device uint8 [P, nb, nb]; cand_layout host int32 [P]: 0 = the mask
 *               is stated in natural order, 1 = in frame-major order (evaluated
 *               through the layout map, no tensor is moved). 1 <= P <= 4.
 *   err         out, device fp32 [B, H, P]: sum over rows and channels of
 *               (o_candidate - o_dense)^2, outputs in fp32
 *   choice      out, device int32 [B, H]: argmin of err, ties to the lowest index
 *   workspace   device scratch of at least vsa_profile_workspace_bytes(...) bytes */
size_t vsa_profile_workspace_bytes(int B, int H, vsa_grid g, int D, int R, int P);
int vsa_profile_heads(const void* q, const void* k, const void* v, int B, int H, vsa_grid g,
                      int D, int dtype, int bs, const int32_t* rows, int R,
                      const uint8_t* cand_masks, const int32_t* cand_layout, int P, float scale,
                      float* err, int32_t* choice, void* workspace, size_t ws_bytes,
                      void* stream);

/* vsa_profile_heads without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments, results and errors as
 * vsa_profile_heads minus (workspace, ws_bytes); the scratch the profile needs
 * (vsa_profile_workspace_bytes of the same sizes) comes from a static device
 * array of vsa_profile_scratch_capacity() bytes (96 MiB: enough for the
 * Wan 480p and HunyuanVideo 720p shapes at 1 % rows and two candidates) that
 * every GPU the library runs on holds until the process ends. A problem that
 * needs more returns VSA_ERR_WORKSPACE before any HIP call. The library
 * allocates nothing: the first call on a device looks up that device's copy of
 * the array (hipGetSymbolAddress), later calls reuse it. Every call on one GPU
 * shares that GPU's scratch, so calls that overlap on one GPU (other streams,
 * other threads) race; calls in order on one stream do not. The scratch keeps
 * the last call's contents; no result depends on them. */
size_t vsa_profile_scratch_capacity(void);
int vsa_profile_heads_noalloc(const void* q, const void* k, const void* v, int B, int H, vsa_grid g,
                              int D, int dtype, int bs, const int32_t* rows, int R,
                              const uint8_t* cand_masks, const int32_t* cand_layout, int P, float scale,
                              float* err, int32_t* choice, void* stream);

/* Mask -> compacted block list (ascending indices of the 1s of each row).
 *   mask           device uint8: [B, H, nqb, nkb] when head_mask_idx is NULL;
 *                  otherwise [P, nqb, nkb] and head h of every batch uses
 *                  mask[head_mask_idx[h]] (host int32 [H], H <= 1024, each < P)
 *   max_kv         capacity of a row of kv_idx (1 <= max_kv <= nkb); rows with
 *                  more kept blocks keep their first max_kv
 *   kv_idx, kv_cnt out, as in vsa_blocks */
int vsa_mask_to_list(const uint8_t* mask, int B, int H, int nqb, int nkb,
                     const int32_t* head_mask_idx, int P, int max_kv, int32_t* kv_idx,
                     int32_t* kv_cnt, void* stream);

/* Block-sparse attention forward.
 * machinebrief LVSA article (block-sparse attention), Sparse VideoGen2 page,
 * Abstract (compute only the critical tokens), OSP-Next page, "Method"
 * (FlashAttention-compatible sparse attention). For each (b, h) and query i:
 *   O_i = sum_{j in J(i)} softmax_j(scale * <q_i, k_j>) v_j,
 *   J(i) = the valid keys of the key blocks kept for query block i / bs,
 * computed tile by tile with an online (running max and sum) softmax over the
 * kept blocks, skipping every other tile.
 *   q, k, v, o  [B, H, N, D]; dtype VSA_BF16 (D in {64, 128}, bs in {64, 128}) or
 *               VSA_F32 (D in {64, 128}, bs = 64); bf16 uses MFMA with fp32
 *               accumulation, softmax in fp32, P rounded to bf16 for P.V, O
 *               rounded to nearest even
 *   lse         optional out, device fp32 [B, H, N]: log-sum-exp (natural log)
 *               of each query's kept scores
 *   blk_len     optional device int32 [nb]
 *   blocks      host pointer to the block set (nqb = nkb = nb)
 *   scale       > 0, finite
 *   workspace   may be NULL when vsa_attn_workspace_bytes returns 0
 * A query with no kept valid key, or in an invalid (padding) slot, gets O = 0
 * and LSE = -inf. */
size_t vsa_attn_workspace_bytes(int B, int H, int N, int bs, int max_kv);
int vsa_block_sparse_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int H, int N, int D, int dtype, int bs,
                              const int32_t* blk_len, const vsa_blocks* blocks, float scale,
                              void* workspace, size_t ws_bytes, void* stream);

/* Block-sparse attention with the frame-major permutation folded into its
 * loads and stores. Sparse Video-Gen page, "Approach": temporal heads work in
 * the frame-major order (position s*T + t holds natural token t*HW + s) so that
 * their pattern becomes dense tiles. The result equals, bit for bit,
 *   vsa_permute(q, k, v -> FRAME_MAJOR, head_sel = head_fm),
 *   vsa_block_sparse_attn_fwd on the permuted tensors,
 *   vsa_permute(o -> FRAME_MAJOR, inverse, head_fm) (and LSE likewise),
 * without the four copies: a head with head_fm[h] = 1 reads its Q, K, V rows
 * through the map and writes O and LSE at natural positions.
 *   q, k, v, o  [B, H, N, D] in natural order, N = g.T * g.Hh * g.W; bf16 with
 *               D = 128 only (other dtypes or D: VSA_ERR_UNSUPPORTED), bs 64/128
 *   lse         optional out, device fp32 [B, H, N], natural order
 *   head_fm     host uint8 [H] (H <= 1024), 1 = frame-major head; NULL = none
 *   blk_len, blocks, scale as for vsa_block_sparse_attn_fwd; for a frame-major
 *               head, blocks are counted along the frame-major order
 * No workspace; errors as for vsa_block_sparse_attn_fwd. */
int vsa_block_sparse_attn_fwd_permuted(const void* q, const void* k, const void* v, void* o, float* lse,
                                       int B, int H, vsa_grid g, int D, int dtype, int bs,
                                       const uint8_t* head_fm, const int32_t* blk_len,
                                       const vsa_blocks* blocks, float scale, void* stream);

/* Block-sparse attention in which every head uses the candidate pattern chosen
 * for it on the device (Sparse Video-Gen page, "Approach": each head takes the
 * pattern whose output on sampled rows is closest to dense attention). The
 * result equals, bit for bit, vsa_block_sparse_attn_fwd_permuted with head
 * (b, h) using block mask cand_masks[choice[b, h]] and head_fm =
 * cand_layout[choice[b, h]]; the choice is read by the kernel, so no host round
 * trip and no mask -> list step sit between the profiler and the attention.
 *   q, k, v, o   [B, H, N, D] natural order, N = g.T * g.Hh * g.W; bf16, D = 128,
 *                bs 64 or 128 (otherwise VSA_ERR_UNSUPPORTED); nb <= 4096
 *   lse          optional out, device fp32 [B, H, N], natural order
 *   cand_masks   device uint8 [P, nb, nb]; a frame-major candidate's mask counts
 *                blocks along the frame-major order
 *   cand_layout  host int32 [P]: 0 natural, 1 frame-major; P in [1, 4]
 *   choice       device int32 [B, H] (e.g. from vsa_profile_heads); an entry
 *                outside [0, P) keeps nothing: O = 0, LSE = -inf for that head
 *   blk_len, scale as for vsa_block_sparse_attn_fwd. No workspace. */
int vsa_block_sparse_attn_fwd_chosen(const void* q, const void* k, const void* v, void* o, float* lse,
                                     int B, int H, vsa_grid g, int D, int dtype, int bs,
                                     const uint8_t* cand_masks, const int32_t* cand_layout, int P,
                                     const int32_t* choice, const int32_t* blk_len, float scale,
                                     void* stream);

/* Block-sparse attention backward: dQ, dK, dV of vsa_block_sparse_attn_fwd.
 * USV page, Abstract and Figure 2 caption (the sparse attention is trained end
 * to end) and OSP-Next page, "Method" (sparse fine-tuning) need these
 * gradients. With P_ij = exp(scale <q_i, k_j> - LSE_i) for j in J(i), 0 else:
 *   dV_j = sum_i P_ij dO_i,   dS_ij = P_ij (<dO_i, v_j> - Delta_i),
 *   Delta_i = <dO_i, O_i>,    dQ_i = scale sum_j dS_ij k_j,
 *   dK_j = scale sum_i dS_ij q_i,
 * every sum over the kept (query block, key block) tiles only.
 *   q, k, v      [B, H, N, D] forward inputs; bf16, D = 128, bs 64 or 128
 *                (otherwise VSA_ERR_UNSUPPORTED)
 *   o, lse       the forward's O [B, H, N, D] and LSE (device fp32 [B, H, N],
 *                natural log; -inf = a row that keeps nothing)
 *   dout         upstream gradient dO [B, H, N, D], bf16
 *   dq, dk, dv   out [B, H, N, D], bf16, each rounded once from fp32 sums; rows
 *                of invalid (padding) positions and positions with nothing
 *                kept are 0. Must not alias any input.
 *   blk_len, blocks, scale as for the forward (same block set); a list row must
 *                hold distinct entries (a repeated block would count twice in dQ
 *                only); the mask form needs nb <= 4096
 *   workspace    device, >= vsa_attn_bwd_workspace_bytes(B, H, N, bs, list_form)
 *                bytes, 16-byte aligned, list_form = 1 for the (kv_idx, kv_cnt)
 *                form; holds base-2 LSE and Delta per row, and per key block the
 *                ascending list of query blocks that keep it
 * Launch order on `stream`: row statistics, block transpose, dQ (one workgroup
 * per query block), dV and dK (one workgroup per key block each). No atomics:
 * results are bit-reproducible. */
size_t vsa_attn_bwd_workspace_bytes(int B, int H, int N, int bs, int list_form);
int vsa_block_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                              const void* dout, const float* lse, void* dq, void* dk, void* dv,
                              int B, int H, int N, int D, int dtype, int bs,
                              const int32_t* blk_len, const vsa_blocks* blocks, float scale,
                              void* workspace, size_t ws_bytes, void* stream);

/* ---- Semantic-aware permutation ------------------------------------------
 * Sparse VideoGen2 page, Abstract: tokens are clustered by semantic similarity
 * with k-means and reordered so that every cluster is contiguous; cluster means
 * stand for their tokens when a top-p budget picks the critical clusters, and
 * the attention over the kept clusters runs without padding. The flow is
 *   vsa_kmeans (Q, then K) -> vsa_cluster_order -> vsa_gather_rows (Q by the
 *   query order, K and V by the key order) -> vsa_cluster_scores ->
 *   vsa_select_topk (nqb = Cq, nkb = Ck) -> vsa_varlen_sparse_attn_fwd ->
 *   vsa_gather_rows(inverse = 1) on O. */

/* Lloyd's k-means of the N tokens of every (b, h), C clusters, `iters`
 * iterations. Seeds: the tokens at positions floor(c N / C). An iteration sends
 * every token to argmin_c ||m_c||^2 - 2 <x, m_c>, m_c the centroid rounded to
 * bf16 (fp32 accumulation, ties to the lower index), then replaces each
 * centroid by the mean of its members (fp32, summed in a fixed order; an empty
 * cluster keeps its centroid). Deterministic: no floating-point atomics.
 *   x          [B, H, N, D] bf16, D = 128 (otherwise VSA_ERR_UNSUPPORTED)
 *   C          1 <= C <= min(N, 1024)
 *   centroids  out, device fp32 [B, H, C, D]: the means of the final assignment
 *   labels     out, device int32 [B, H, N]: the final assignment
 *   counts     out, device int32 [B, H, C]: cluster sizes of the final assignment
 *   workspace  >= vsa_kmeans_workspace_bytes(B, H, N, C, D) bytes (bf16
 *              centroids and their norms, and each iteration's cluster order) */
size_t vsa_kmeans_workspace_bytes(int B, int H, int N, int C, int D);
int vsa_kmeans(const void* x, int B, int H, int N, int D, int dtype, int C, int iters, float* centroids,
               int32_t* labels, int32_t* counts, void* workspace, size_t ws_bytes, void* stream);

/* Stable cluster-major order of every (b, h): tokens sorted by label, members of
 * a cluster in natural order. Integer work, bit-exact.
 *   labels   device int32 [B, H, N]; a label outside [0, C) leaves its token out
 *            (positions from offsets[C] on are then not written)
 *   C        1 <= C <= 1024
 *   perm     out, device int32 [B, H, N]: perm[p] = token stored at position p
 *   offsets  out, device int32 [B, H, C + 1]: cluster c occupies positions
 *            [offsets[c], offsets[c + 1])
 *   workspace >= vsa_cluster_order_workspace_bytes(B, H, N, C) bytes */
size_t vsa_cluster_order_workspace_bytes(int B, int H, int N, int C);
int vsa_cluster_order(const int32_t* labels, int B, int H, int N, int C, int32_t* perm, int32_t* offsets,
                      void* workspace, size_t ws_bytes, void* stream);

/* Row gather by a per-head index list (bit-exact data movement):
 *   inverse = 0: dst[b, h, r] = src[b, h, perm[b, h, r]]
 *   inverse = 1: dst[b, h, perm[b, h, r]] = src[b, h, r]
 *   src, dst  [B, H, N, D], bf16 or fp32, D in {64, 128}; must not overlap
 *   perm      device int32 [B, H, N], a permutation of [0, N) per head (an entry
 *             outside [0, N) moves nothing) */
int vsa_gather_rows(const void* src, void* dst, int B, int H, int N, int D, int dtype,
                    const int32_t* perm, int inverse, void* stream);

/* Size-weighted cluster-pair scores, fp32:
 *   scores[b, h, a, c] = scale * <cq[b, h, a], ck[b, h, c]> + log(k_counts[b, h, c])
 * and -inf for an empty key cluster. The softmax of a row is the share of query
 * cluster a's attention that key cluster c would take if every key equalled its
 * centroid, so top-p on these scores (vsa_select_topk) weighs clusters by size.
 *   cq [B, H, Cq, D], ck [B, H, Ck, D] device fp32 (ck 16-byte aligned), D in {64, 128}
 *   k_counts device int32 [B, H, Ck]; scores out, device fp32 [B, H, Cq, Ck] */
int vsa_cluster_scores(const float* cq, const float* ck, const int32_t* k_counts, int B, int H,
                       int Cq, int Ck, int D, float scale, float* scores, void* stream);

/* Attention over variable-size clusters in cluster-major storage. Query cluster
 * a is rows [q_off[a], q_off[a + 1]) of q, key cluster c rows [k_off[c],
 * k_off[c + 1]) of k and v; each query of cluster a attends (softmax over all of
 * them) to the keys of the key clusters kept for a. No padding: the kept key
 * clusters are packed end to end into 64-key tiles.
 *   q, k, v, o  [B, H, N, D] bf16, D = 128 (otherwise VSA_ERR_UNSUPPORTED); o is
 *               written for every row of every query cluster
 *   lse         optional out, device fp32 [B, H, N]
 *   q_off       device int32 [B, H, Cq + 1], non-decreasing, q_off[0] = 0,
 *               q_off[Cq] <= N; k_off likewise [B, H, Ck + 1]
 *   blocks      host pointer, the kept key clusters of each query cluster: mask
 *               uint8 [B, H, Cq, Ck] (Ck <= 4096), or kv_idx int32
 *               [B, H, Cq, max_kv] + kv_cnt [B, H, Cq] with distinct entries in
 *               [0, Ck), used in the order given (ascending = the mask form's order)
 *   workspace   >= vsa_varlen_attn_workspace_bytes(B, H, N, Cq) bytes (chunk
 *               table, kept-key counts and the launch order: the chunks with the
 *               most kept keys start first)
 * Precision as vsa_block_sparse_attn_fwd. A query whose kept clusters hold no key
 * gets O = 0, LSE = -inf. No floating-point atomics: results are bit-reproducible. */
size_t vsa_varlen_attn_workspace_bytes(int B, int H, int N, int Cq);
int vsa_varlen_sparse_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int N, int D, int dtype, const int32_t* q_off, int Cq,
                               const int32_t* k_off, int Ck, const vsa_blocks* blocks, float scale,
                               void* workspace, size_t ws_bytes, void* stream);

/* ---- FP8 attention ----------------------------------------------------------
 * Sparse Video-Gen page, "Key results": the attention runs faster still in FP8.
 * Format OCP E4M3 (bias 7, largest finite 448, round to nearest even). */

/* Quantises a bf16 tensor to e4m3: code = e4m3(clamp(x * (448 / amax), +-448)),
 * both products in fp32, scale = amax / 448 (a zero block: scale 0, codes 0).
 *   x       [B, H, N, D] bf16, D = 128 (otherwise VSA_ERR_UNSUPPORTED)
 *   kind    VSA_FP8_ROWS (for Q and K): out [B, H, N, D], scales fp32
 *           [B, H, ceil(N / 64)], amax over each block of 64 rows and all channels;
 *           VSA_FP8_VT (for V): out [B, H, ceil(N / 64), D, 64] with key
 *           k = 32 st + 8 g + 4 h + e (st, h in {0, 1}; g, e < 4) of a tile at
 *           column 32 h + 16 st + 4 g + e and keys past N zero, scales fp32
 *           [B, H, D], amax per channel over all N rows
 * No workspace (VSA_FP8_VT uses `scales` for the amax bits until its last step). */
int vsa_fp8_quantize(const void* x, int B, int H, int N, int D, int dtype, int kind, uint8_t* out,
                     float* scales, void* stream);

/* Block-sparse attention on e4m3 inputs: softmax attention of the dequantised
 * values code * scale (same block rule as vsa_block_sparse_attn_fwd), on the
 * gfx950 e4m3 MFMA. S in fp32 from exact code products; P = exp(S - m) in fp32
 * is rounded to e4m3 for P V (the row sum uses the fp32 P); O rounded to bf16.
 *   q8, k8        codes from vsa_fp8_quantize(VSA_FP8_ROWS), with their scales
 *   vt8, v_scale  codes and scales from vsa_fp8_quantize(VSA_FP8_VT)
 *   o             out [B, H, N, D] bf16; lse optional out fp32 [B, H, N] (natural log)
 *   D = 128, bs = 128 (otherwise VSA_ERR_UNSUPPORTED); blk_len, blocks, scale as for
 *   vsa_block_sparse_attn_fwd. No workspace. */
int vsa_block_sparse_attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* vt8,
                                  const float* q_scale, const float* k_scale, const float* v_scale,
                                  void* o, float* lse, int B, int H, int N, int D, int bs,
                                  const int32_t* blk_len, const vsa_blocks* blocks, float scale,
                                  void* stream);

/* Validates a block list held in HOST memory: every kv_cnt in [0, max_kv], the
 * first kv_cnt entries of each row strictly ascending and inside [0, nkb).
 * Returns VSA_OK or VSA_ERR_INVALID (message names the first bad row). */
int vsa_check_block_list_host(const int32_t* kv_idx, const int32_t* kv_cnt, int64_t rows,
                              int nkb, int max_kv);

#ifdef __cplusplus
}
#endif
#endif /* VSA_H */
