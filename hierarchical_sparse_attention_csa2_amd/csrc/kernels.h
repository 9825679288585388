// Internal launchers of the CSA2 kernels (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

hipError_t launch_index_scan(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                             const uint8_t* k_scales, const int32_t* n_visible, int B, int M, int64_t N_max,
                             float* scores, float* block_max, int64_t nblk_stride, float* super_max,
                             int64_t nsup_stride, hipStream_t stream);

// Many queries per sequence (M > 1) on the FP4 matrix cores; same outputs as
// launch_index_scan.
hipError_t launch_prefill_scan(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                               const uint8_t* k_scales, const int32_t* n_visible, int B, int M, int64_t N_max,
                               float* scores, float* block_max, int64_t nblk_stride, float* super_max,
                               int64_t nsup_stride, hipStream_t stream);

hipError_t launch_pool_scan(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                            const uint8_t* k_scales, const int32_t* pool_blocks, int n_pool,
                            const int32_t* n_visible, int B, int M, int64_t N_max, float* pool_scores,
                            hipStream_t stream);
// Pool rescoring and top-k in one workgroup per row: pool_blocks [B*M][n_pool]
// (ids ascending, -1 padded), idx [B*M][k]; hipErrorNotSupported when
// 8 * n_pool > 16384 or k <= 0 (nothing launched).
hipError_t launch_pool_topk(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                            const uint8_t* k_scales, const int32_t* pool_blocks, int n_pool,
                            const int32_t* n_visible, int B, int M, int64_t N_max, const uint32_t* floor_in, int k,
                            int32_t* idx, hipStream_t stream);

// Ranked selection.  layout 0: block maxima (row length ceil(n_visible/8),
// stride `stride`); 1: pool slots (8*n_pool per row, positions through
// pool_blocks); 2: full score rows (length min(n_visible, stride)).
enum SelectLayout { kSelBlocks = 0, kSelPool = 1, kSelFull = 2 };

// super_max (blocks layout only, may be null): maxima of 8 consecutive blocks,
// row stride nsup_stride, as written by the indexer scan.
// floor_in (may be null): per row, an order key that every selected item
// reaches (items below it are dropped unexamined); floor_out (may be null):
// per row, the order key of target 2's k2-th item, or 1 when the row has at
// most k2 items.
hipError_t launch_select(int layout, const float* scores, int64_t stride, const int32_t* pool_blocks,
                         int64_t n_pool, const int32_t* n_visible, int R, int k1, int32_t* out1, int k2,
                         int32_t* out2, const float* super_max, int64_t nsup_stride, hipStream_t stream,
                         const uint32_t* floor_in = nullptr, uint32_t* floor_out = nullptr);

// Full layer, decode: pool (n_pool <= 2048) and the top-k over the pool's first
// kb blocks in one workgroup per row, from the scan's block maxima (row stride
// `stride`), super-block maxima and stored scores (row stride n_max).
// hipErrorNotSupported (nothing launched) outside the shapes it covers.
hipError_t launch_select_topk(const float* bmax, int64_t stride, const float* super_max, int64_t nsup_stride,
                              const int32_t* n_visible, int R, int n_pool, int32_t* pool_out, int kb,
                              const float* scores, int64_t n_max, int k, int32_t* idx, hipStream_t stream);

// Full layer, decode, every block of every row in the pool (ceil(n_max/8) <=
// n_pool) and rows of at most 16,384 positions: the pool is every visible block
// and the top-k is taken from the stored score rows (row stride n_max).
// hipErrorNotSupported (nothing launched) outside those shapes.
hipError_t launch_select_short(const float* scores, int64_t n_max, const int32_t* n_visible, int R, int n_pool,
                               int32_t* pool_out, int k, int32_t* idx, hipStream_t stream);

// Cache write: ratio-m weighted merge of fp32 token rows (D a power of two,
// >= 32) quantized to MXFP4 codes and E8M0 scales; and fp32 -> FP8 E4M3 of n
// elements (n % 4 == 0).
hipError_t launch_write_mxfp4(const float* x, const float* w, int64_t n_entries, int ratio, int D, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream);
hipError_t launch_write_e4m3(const float* x, int64_t n, uint8_t* out, hipStream_t stream);

struct AttnLaunch {
  const float* q;
  const uint8_t* c_codes;
  const uint8_t* c_scales;
  const int32_t* idx;
  int k;
  const uint8_t* win;
  const int32_t* win_start;
  const int32_t* win_len;
  int win_max;
  int B, M, H, Tw;
  int64_t N_max;
  float sm_scale;
  float* out;
  void* workspace;
  size_t workspace_bytes;
};

int attn_splits(int R, int H, int k_plus_win);
size_t attn_workspace_bytes(int R, int H, int k_plus_win);
hipError_t launch_sparse_attn(const AttnLaunch& a, hipStream_t stream);

}  // namespace csa2
