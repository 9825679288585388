/*
 * CPU oracle for the CSA2 hierarchical sparse attention step.
 * TEST INFRASTRUCTURE ONLY: loaded by tests, the smoke check and the benchmark's
 * CPU baseline, never by the library.  Shares nothing with the HIP path.
 *
 * Layouts (all host memory, row-major, contiguous):
 *   index query  codes u8[R][64]  scales u8[R][4]        (R = B*M query rows)
 *   index keys   codes u8[B][N_max][64] scales u8[B][N_max][4]
 *   latent       codes u8[B][N_max][256] scales u8[B][N_max][16]
 *   window       u8[B][Tw][512] (FP8 E4M3), rows win_start[r] .. + min(win_len[r], win_max)
 *                (rows outside [0, Tw) and indices outside [0, N_max) are left out)
 *   q, out       f32[R][H][512]
 * Query row r belongs to sequence r / M.  All functions return 0 or -1.
 */
#ifndef CSA2_ORACLE_H
#define CSA2_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

double orc_e2m1_value(unsigned code);
double orc_e8m0_scale(unsigned byte);
double orc_e4m3_value(unsigned code);
void orc_mxfp4_encode_block(const double* x, uint8_t* codes16, uint8_t* scale);
uint8_t orc_e4m3_encode(double x);
int orc_merge_f32(const float* x, const float* w, int64_t n_entries, int ratio, int D, float* out);
int orc_cache_write_mxfp4(const float* x, const float* w, int64_t n_entries, int ratio, int D, uint8_t* codes,
                          uint8_t* scales);
void orc_cache_write_e4m3(const float* x, int64_t n, uint8_t* out);
float orc_score(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks);
uint32_t orc_order_key(float f);

int orc_index_full(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                   const uint8_t* k_scales, const int32_t* n_visible, int B, int M, int64_t N_max,
                   int n_pool, int k, float* scores, float* block_max, int32_t* pool_blocks,
                   int32_t* idx, int global_topk, int threads);
int orc_index_pool(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                   const uint8_t* k_scales, const int32_t* pool_blocks, int n_pool,
                   const int32_t* n_visible, int B, int M, int64_t N_max, float* pool_scores, int threads);
int orc_topk_pool(const float* pool_scores, const int32_t* pool_blocks, int n_pool,
                  const int32_t* n_visible, int64_t R, int k, int32_t* idx, int threads);
int orc_topk_full(const float* scores, const int32_t* n_visible, int64_t R, int64_t N_max, int k,
                  int32_t* idx, int threads);
int orc_sparse_attn(const float* q, const uint8_t* c_codes, const uint8_t* c_scales, const int32_t* idx,
                    int k, const uint8_t* win, const int32_t* win_start, const int32_t* win_len, int win_max,
                    int B, int M, int64_t N_max, int H, int Tw, float sm_scale, float* out, int threads);

#ifdef __cplusplus
}
#endif
#endif
