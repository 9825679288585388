/*
 * csa2.h - C ABI of the CSA2 hierarchical sparse attention step on MI355X (gfx950).
 *
 * What the step computes (DeepSeek-V4.1-Flash write-ups):
 *   - fupanwang.com article, section "三个方向一起压小缓存" and the figure caption on
 *     the hierarchical sparse indexer: the first Full layer's FP4 indexer scores
 *     every visible cached position; each 8-position block is represented by its
 *     highest score; the top 2048 blocks (16,384 positions) form a candidate pool
 *     shared with later layers; every layer reads 512 selected KV entries.
 *     Reindex layers score only inside the pool; Reuse layers reuse the latest
 *     selection.  The main KV is OCP MXFP4, the sliding-window KV stays FP8.
 *   - same article, section "后 20 层干脆共用一份 KV": a 128-token sliding window
 *     branch next to the sparse global attention.
 *   - dreamax.pages.dev notes, CSA2 paragraph: the Full / Reindex / Reuse modes.
 *
 * Conventions shared by every entry point
 *   - All tensor arguments are DEVICE pointers to caller-owned memory; the library
 *     allocates nothing and keeps no state between calls.
 *   - Every non-NULL tensor pointer must be 16-byte aligned (device allocations
 *     are): the kernels move codes, queries, outputs and partials in 16-byte
 *     vectors.  A misaligned pointer is an argument error (CSA2_ERR_INVALID).
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the
 *     default stream).  Calls return before the work finishes: results are valid
 *     once the caller synchronises the stream.
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     validation error nothing is launched and a negative status is returned.
 *     A failed launch returns CSA2_ERR_HIP.  Device-side contents (codes, scale
 *     bytes, indices) are not validated unless stated.
 *   - Rows: a call covers B sequences with M query rows each, R = B*M rows;
 *     query row r belongs to sequence r / M (decode: M = 1; prefill: M > 1).
 *   - Storage formats (OCP Microscaling Formats v1.0 / OCP FP8):
 *       MXFP4: blocks of 32 elements, one E8M0 scale byte per block
 *              (value 2^(byte-127); 0xFF must not occur), element codes E2M1,
 *              element 2i in the low nibble of byte i.
 *       FP8:   E4M3 (OCP "E4M3FN": bias 7, max 448, no infinities).
 *   - Layouts (row-major, contiguous):
 *       index query  q_codes u8[R][64],  q_scales u8[R][4]          (128-d MXFP4)
 *       index keys   k_codes u8[B][N_max][64], k_scales u8[B][N_max][4]
 *       latent KV    c_codes u8[B][N_max][256], c_scales u8[B][N_max][16] (512-d)
 *       window KV    win u8[B][Tw][512] (FP8 E4M3)
 *       n_visible    i32[R]: query row r sees cached entries 0 .. n_visible[r]-1
 *                    (0 <= n_visible[r] <= N_max, not checked on the device)
 *       queries/out  f32[R][H][512]
 *   - Scores compare by IEEE-754 total order of their fp32 bits; positions and
 *     blocks rank by (score descending, position ascending): ties go to the
 *     lowest position.  Selected positions/blocks are written in ascending order
 *     and the rest of each output row is padded with -1.
 *   - A block value past the fp32 range is +-inf (ldexp semantics); a score
 *     adding opposite infinities is not a number and is stored as the positive
 *     quiet NaN 0x7FC00000, which ranks above +inf.  (Only scale bytes far from
 *     those of real data, eq + ek > 371, can overflow.)
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_BLOCK 8          /* positions per coarse block */
#define CSA2_INDEX_DIM 128    /* indexer query/key width (4 MXFP4 blocks) */
#define CSA2_LATENT_DIM 512   /* latent KV / window / query width */

enum {
    CSA2_OK = 0,
    CSA2_ERR_INVALID = -1,      /* bad pointer, size or range */
    CSA2_ERR_UNSUPPORTED = -2,  /* valid but not supported by this library */
    CSA2_ERR_WORKSPACE = -3,    /* workspace missing or too small */
    CSA2_ERR_HIP = -4,          /* a HIP launch failed */
    CSA2_ERR_TOO_LARGE = -5     /* needs more than CSA2_STATIC_SCRATCH_BYTES (static-scratch calls) */
};

/* Size of the per-device scratch array behind csa2_index_full_static. */
#define CSA2_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

enum { CSA2_OP_INDEX_FULL = 1, CSA2_OP_SPARSE_ATTN = 2 };

/*
 * csa2_index_scan - the Full layer's indexer scan (first step of the indexer).
 * Defined by: fupanwang.com article, section "三个方向一起压小缓存" - the FP4
 * indexer query and key score every visible cached position, and each block of
 * 8 positions is represented by its highest score.
 * For every row r and visible position j computes the score
 *     s = ((v0 + v1) + v2) + v3,   v_b = sum_{i in block b} q_i k_i   (b = 0..3)
 * where each 32-element block sum is exact and the four adds are fp32
 * round-to-nearest-even in this order; and, per 8-position block
 * [8i, 8i+8) intersected with the visible range, the block maximum.
 *   scores     f32[R][N_max] or NULL; entries j >= n_visible[r] are not written.
 *   block_max  f32[R][nblk_max], nblk_max = ceil(N_max/8); blocks past the
 *              visible range are not written.  Required.
 *   super_max  f32[R][nsup_max] or NULL, nsup_max = ceil(N_max/64): the maximum
 *              of the 8 block maxima [8s, 8s+8) (positions [64s, 64s+64) within
 *              the visible range); entries past the visible range are not
 *              written.  csa2_select_blocks can take it to rank long rows from
 *              one level up without re-reading the block maxima.
 * Returns CSA2_OK, CSA2_ERR_INVALID (NULL input, B<1, M<1, N_max<1),
 * CSA2_ERR_HIP.
 */
int csa2_index_scan(const uint8_t* q_codes, const uint8_t* q_scales,
                    const uint8_t* k_codes, const uint8_t* k_scales,
                    const int32_t* n_visible, int B, int M, int64_t N_max,
                    float* scores, float* block_max, float* super_max, void* stream);

/*
 * csa2_select_blocks - the coarse filter: rank the visible blocks of each row by
 * (defined by: fupanwang.com article, section "三个方向一起压小缓存" and its
 * figure caption on the hierarchical sparse indexer - at most 2048 blocks of 8
 * positions, 16,384 candidates, are kept as the pool shared by later layers)
 * (block max descending, block id ascending) and keep the first
 * min(n_pool, nblk) as the candidate pool, nblk = ceil(n_visible[r]/8).
 *   block_max    f32[R][nblk_stride] (as written by csa2_index_scan)
 *   super_max    f32[R][ceil(nblk_stride/8)] or NULL: the maxima of 8
 *                consecutive blocks, as written by csa2_index_scan with the same
 *                N_max.  Used only to speed up rows longer than 16,384 blocks;
 *                the result is the same with or without it.
 *   pool_blocks  i32[R][n_pool]: kept block ids ascending, -1 padded.
 *   topk_blocks  i32[R][k_blocks] or NULL: the first min(k_blocks, nblk) blocks
 *                of the same ranking (a prefix of the pool when k_blocks <= n_pool).
 * Returns CSA2_OK, CSA2_ERR_INVALID (NULL, R<1, n_pool<1, k_blocks<0,
 * nblk_stride<1), CSA2_ERR_HIP.
 */
int csa2_select_blocks(const float* block_max, const float* super_max, int64_t nblk_stride,
                       const int32_t* n_visible, int R, int n_pool, int32_t* pool_blocks, int k_blocks,
                       int32_t* topk_blocks, void* stream);

/*
 * csa2_index_pool - score only inside a pool (Reindex layers, and the Full
 * layer's own top-k; defined by: fupanwang.com article, section
 * "三个方向一起压小缓存" - later layers score only inside the first Full layer's
 * candidate pool; dreamax.pages.dev notes, CSA2 paragraph - the Reindex mode):
 * for row r, pool block i and t = 0..7 the score of position
 * j = 8*pool_blocks[r][i] + t against the row's own index query, written to
 * pool_scores[r][8i+t]; slots with pool_blocks < 0 or j >= n_visible[r] are
 * written as -inf.  Same score definition as csa2_index_scan.
 *   pool_blocks  i32[R][n_pool], ids in [0, ceil(N_max/8)) or -1.
 *   pool_scores  f32[R][8*n_pool]
 * Returns CSA2_OK, CSA2_ERR_INVALID, CSA2_ERR_HIP.
 */
int csa2_index_pool(const uint8_t* q_codes, const uint8_t* q_scales,
                    const uint8_t* k_codes, const uint8_t* k_scales,
                    const int32_t* pool_blocks, int n_pool, const int32_t* n_visible,
                    int B, int M, int64_t N_max, float* pool_scores, void* stream);

/*
 * csa2_topk - keep the first min(k, #valid) slots of each row by (score desc,
 * position asc) and write their positions ascending, -1 padded, to idx i32[R][k].
 * Defined by: fupanwang.com article, section "三个方向一起压小缓存" and its figure
 * caption - every layer selects its 512 entries inside the pool.
 *   pool layout (pool_blocks != NULL): scores f32[R][8*n_pool]; slot s is position
 *     8*pool_blocks[r][s/8] + s%8, valid when the block id is >= 0 and the
 *     position < n_visible[r].  pool_blocks rows must be ascending (as produced by
 *     csa2_select_blocks) so that slot order is position order.
 *   full layout (pool_blocks == NULL): scores f32[R][n_pool] with slot s =
 *     position s, valid when s < n_visible[r] (n_pool is the row stride).
 * Returns CSA2_OK, CSA2_ERR_INVALID (NULL, R<1, n_pool<1, k<0), CSA2_ERR_HIP.
 */
int csa2_topk(const float* scores, const int32_t* pool_blocks, int64_t n_pool, const int32_t* n_visible,
              int R, int k, int32_t* idx, void* stream);

/*
 * csa2_index_pool_topk - a Reindex layer's indexer in one call (defined by:
 * fupanwang.com article, section "三个方向一起压小缓存" - a later layer scores
 * only the first Full layer's candidate pool with its own index query and keeps
 * its own top 512; dreamax.pages.dev notes, CSA2 paragraph - the Reindex mode).
 * idx equals csa2_index_pool followed by csa2_topk in the pool layout, bit for
 * bit, with no pool-score output: each row's pool positions are scored and
 * ranked in one workgroup, which is faster than the two calls for many rows
 * (about 1,024 and up on MI355X with a 2048-block pool) and slower for few.
 *   pool_blocks  i32[R][n_pool], 1 <= n_pool <= 2048, ids ascending, -1 padded
 *                (as csa2_select_blocks writes them)
 *   idx          i32[R][k]: the first min(k, valid slots) positions by
 *                (score desc, position asc), ascending, -1 padded; k = 0 writes
 *                nothing.
 * Other arguments as csa2_index_pool.  Returns CSA2_OK, CSA2_ERR_INVALID (NULL,
 * misaligned, B<1, M<1, N_max<1, n_pool outside [1, 2048], k<0), CSA2_ERR_HIP.
 */
int csa2_index_pool_topk(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                         const uint8_t* k_scales, const int32_t* pool_blocks, int n_pool, const int32_t* n_visible,
                         int B, int M, int64_t N_max, int k, int32_t* idx, void* stream);

/*
 * csa2_index_full - the whole Full-layer indexer (defined by: fupanwang.com
 * article, section "三个方向一起压小缓存" and its figure caption - the first Full
 * layer scores the whole visible context, builds the pool from the block maxima
 * and picks its own top-512): csa2_index_scan, then
 * csa2_select_blocks (the pool and its first kb = min(k, n_pool) blocks), then
 * csa2_index_pool over those kb blocks and csa2_topk.  The row's top-k over the
 * pool equals its top-k over the pool's kb best blocks (every block ranked ahead
 * of a block holding a selected position contributes its own best position to
 * the selection, so such a block ranks within the first k), which is why only
 * those are rescored.  With fewer than 16 queries per sequence (decode) the scan
 * stores every score instead (into `scores`, else the workspace) and one
 * workgroup per row builds the pool and ranks the stored scores of its first kb
 * blocks; the results are the same.
 *   scores, block_max  optional outputs (NULL to skip; block_max then lives in
 *                      the workspace).
 *   pool_blocks  i32[R][n_pool] required;  idx i32[R][k] or NULL (k = 0 skips).
 *   workspace    device memory of csa2_workspace_bytes(CSA2_OP_INDEX_FULL, ...)
 * Returns CSA2_OK, CSA2_ERR_INVALID, CSA2_ERR_WORKSPACE, CSA2_ERR_HIP.
 */
int csa2_index_full(const uint8_t* q_codes, const uint8_t* q_scales,
                    const uint8_t* k_codes, const uint8_t* k_scales,
                    const int32_t* n_visible, int B, int M, int64_t N_max,
                    int n_pool, int k, float* scores, float* block_max,
                    int32_t* pool_blocks, int32_t* idx,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * csa2_index_full_static - csa2_index_full for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments and results without the
 * workspace.  Its scratch is a static device array of CSA2_STATIC_SCRATCH_BYTES
 * (64 MiB) per device, held from the first such call on a device until the
 * process ends; the call allocates nothing.
 *   - Problems whose csa2_workspace_bytes(CSA2_OP_INDEX_FULL, ...) exceeds
 *     CSA2_STATIC_SCRATCH_BYTES return CSA2_ERR_TOO_LARGE and launch nothing
 *     (every decode shape up to 64 rows of 131,072 entries, or 4 rows of
 *     524,288, fits; a 4,096-query prefill chunk does not).
 *   - All calls on one device share that device's array, and each call's
 *     kernels overwrite it: calls that overlap on one device (on different
 *     streams, or from different threads without ordering) race.  Calls
 *     ordered on one stream are safe.
 *   - The scratch of the stream's device is used (the current device for the
 *     NULL stream); its address is looked up once per device.
 * Returns as csa2_index_full, with CSA2_ERR_TOO_LARGE in place of
 * CSA2_ERR_WORKSPACE.
 */
int csa2_index_full_static(const uint8_t* q_codes, const uint8_t* q_scales,
                           const uint8_t* k_codes, const uint8_t* k_scales,
                           const int32_t* n_visible, int B, int M, int64_t N_max,
                           int n_pool, int k, float* scores, float* block_max,
                           int32_t* pool_blocks, int32_t* idx, void* stream);

/*
 * csa2_sparse_attn - one softmax attention per row and head over the row's k
 * selected latent entries and its window rows (value = key for both):
 *     z_i = (q_h . c_i) * sm_scale,  o_h = sum_i softmax(z)_i c_i
 * over entries c_i = MXFP4-decoded latent rows idx[r][0..k) (entries < 0 or >=
 * N_max are skipped; a repeated entry counts each time) followed by the FP8
 * window rows win[seq][win_start[r] + t], t < min(win_len[r], win_max).
 * An empty entry set gives a zero output row.  fp32 output; the products run on
 * MFMA with bf16 split operands (query and probabilities as hi+lo pairs, the
 * decoded values exact in bf16), accumulation in fp32.
 *   H: 16, 32 or 64.   win_max: 0 <= win_max <= Tw (0: no window;
 *   win, win_start and win_len may then be NULL).
 *   Window rows outside [0, Tw) are skipped like entries outside [0, N_max).
 *   workspace: csa2_workspace_bytes(CSA2_OP_SPARSE_ATTN, B, M, 0, H, k + win_max)
 * Defined by: fupanwang.com article, section "三个方向一起压小缓存" - a layer reads
 * its 512 selected entries of the MXFP4 main KV - and section
 * "后 20 层干脆共用一份 KV" - beside them, a 128-token sliding window kept in FP8.
 * Returns CSA2_OK, CSA2_ERR_INVALID, CSA2_ERR_UNSUPPORTED (H), CSA2_ERR_WORKSPACE,
 * CSA2_ERR_HIP.
 */
int csa2_sparse_attn(const float* q, const uint8_t* c_codes, const uint8_t* c_scales,
                     const int32_t* idx, int k,
                     const uint8_t* win, const int32_t* win_start, const int32_t* win_len, int win_max,
                     int B, int M, int64_t N_max, int H, int Tw, float sm_scale,
                     float* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * csa2_cache_write_mxfp4 - the cache write of a CSA2 layer at compression
 * ratio m (fupanwang.com article, section "三个方向一起压小缓存": every m
 * consecutive tokens become one cached entry, entries do not overlap, the merge
 * is weighted by the layer's compression weights; the main KV and the indexer
 * keys are stored in OCP MXFP4):
 *     entry e = sum_{j=0..m-1} w[m*e + j] * x[m*e + j]
 * in fp32, j ascending, each product rounded and then added (no fused
 * multiply-add), then each 32-element block quantized: E = floor(log2 amax) - 2
 * clamped to [-127, 127], scale byte E + 127, elements x / 2^E rounded to the
 * nearest E2M1 value (ties to the even code, saturating at 6, a negative value
 * that rounds to zero stored as +0).  An all-zero block stores scale byte 0 and
 * zero codes; NaN elements are ignored by amax and stored as +0; an infinite
 * amax takes E = 127 (infinite elements store +-6).
 *   x       f32[n_entries*m][D] token rows (D a power of two, 32 <= D <= 16384:
 *           128 for indexer keys, 512 for the latent)
 *   w       f32[n_entries*m] per-token compression weights (the caller's, e.g.
 *           a softmax over each group of m logits); may be NULL only for m = 1
 *           (weight 1: the row is quantized as is)
 *   codes   u8[n_entries][D/2], scales u8[n_entries][D/32] (the cached layout
 *           of the entries: pass k_codes + e0*64 etc. to write entries from e0)
 *   ratio   m, 1..64
 * Alignment (the exception to the 16-byte rule, so that entries can be written
 * at any offset of a cache): x 16 bytes, w 4 bytes, codes 2 bytes, scales any.
 * Returns CSA2_OK, CSA2_ERR_INVALID (NULL pointer, misaligned pointer, D not a
 * power of two in range, ratio out of range, w NULL with m > 1,
 * n_entries < 0), CSA2_ERR_HIP.  n_entries = 0 returns CSA2_OK without
 * launching or looking at the pointers.
 */
int csa2_cache_write_mxfp4(const float* x, const float* w, int64_t n_entries, int ratio, int D,
                           uint8_t* codes, uint8_t* scales, void* stream);

/*
 * csa2_cache_write_e4m3 - quantize-on-write of sliding-window rows to FP8
 * (same section: the sliding-window KV stays FP8): each of the n fp32 values
 * to OCP E4M3FN, nearest value with ties to the even code, saturating at +-448
 * (infinities too), NaN to 0x7F.
 *   x  f32[n] (16-byte aligned), out u8[n] (4-byte aligned; e.g. window rows:
 *      n = rows * 512), n % 4 == 0.
 * Returns CSA2_OK, CSA2_ERR_INVALID (NULL or misaligned pointer, n < 0,
 * n % 4 != 0), CSA2_ERR_HIP.  n = 0 returns CSA2_OK without launching.
 */
int csa2_cache_write_e4m3(const float* x, int64_t n, uint8_t* out, void* stream);

/*
 * csa2_workspace_bytes - device workspace needed by an entry point.
 *   CSA2_OP_INDEX_FULL:  (B, M, N_max, k) as passed to csa2_index_full (H unused)
 *   CSA2_OP_SPARSE_ATTN: (B, M, -, H, k + win_max)
 * Returns 0 for an unknown op or invalid sizes.
 */
size_t csa2_workspace_bytes(int op, int B, int M, int64_t N_max, int H, int k);

/* Static text for a status code. */
const char* csa2_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
