// Indexer scans: the Full layer's scan over every visible position (with the
// 8-position block max fused in) and the pool scan used by Reindex layers and by
// the Full layer's own top-k.
//
// The score (DeepSeek-V4.1-Flash, fupanwang.com article, section
// 三个方向一起压小缓存: FP4 indexer query and key, scored over the visible
// context): one 128-d dot product of two MXFP4 vectors.  Each 32-element block is
// summed exactly; block b contributes v_b = sum_b * 2^(eq_b + ek_b - 254); the
// score is ((v0+v1)+v2)+v3 in fp32.
//
// One query per sequence (decode) and the pool scan: a streaming pass over the
// index keys.  Lane 16g + c of a wave loads block g of key c of each 16-key group
// with one 16-byte load (so one load instruction reads 1 KiB of contiguous
// codes) and its E8M0 byte, decodes the E2M1 codes in registers, forms the
// block's exact value (v_dot2 into fp32, ldexp with the two scale exponents) and
// meets the key's other three blocks through lane shuffles; the four are added
// in block order, so lane l ends with the score of the wave's key l.  Exact for
// any scale bytes.
//
// Several queries per sequence (a verify step over draft tokens): the keys are
// loaded once and every row's block values come from the FP4 matrix cores.  One
// v_mfma_scale_f32_16x16x128_f8f6f4 scores 16 keys: the keys are the B operand
// (the same lane layout, with the E8M0 byte as the lane's scale), and the A
// operand is block-diagonal in the query: row i holds query block i % 4 in K
// group i % 4 and zeros elsewhere.  Output row i of column c is then the single
// block value v_{i%4} of key c, a sum of 32 exact products at one scale: exact
// while the block exponent eq_b + ek_b - 254 lies in [-124, 114] (the integer
// sum needs 13 bits and every value stays a normal float).  Rows whose keys have
// a block exponent outside that range are scored on the vector ALUs, giving the
// same fixed-order result.
#include "device_common.h"
#include "kernels.h"
#include "score_core.h"

namespace csa2 {

constexpr int kScanThreads = 256;
constexpr int kScanWaves = kScanThreads / 64;
constexpr int kScanChunk = kScanWaves * 64;     // positions per workgroup (64 per wave)
constexpr int kScanXcdRun = 64;                 // consecutive chunks per XCD turn
constexpr int kPrefillMinQueries = 16;          // queries per sequence for the many-query scan

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xF, false);
}

// max over the 8-lane group (lanes 8j..8j+7) of x, in every lane of the group
__device__ __forceinline__ uint32_t group8_max_u32(uint32_t x) {
  uint32_t y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  x = y > x ? y : x;
  y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);            // quad_perm [2,3,0,1]
  x = y > x ? y : x;
  y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false);           // row_half_mirror
  return y > x ? y : x;
}

// Grid (ceil(N_max / 256), M, B): query row r = seq * M + blockIdx.y.  Each wave
// scores 64 consecutive positions; all of its loads are issued before any
// arithmetic.  Chunks go to the XCDs in runs of 64 (c3: scan 24.1 -> 23.6 us
// against launch order; runs of 256 made the step slower).  Outputs: block
// maxima, optional super-block maxima (8 blocks) and optional per-position
// scores.
template <bool kScores, bool kSuper>
__global__ __launch_bounds__(kScanThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void index_scan_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales,
    const int32_t* __restrict__ n_visible, int M, int64_t N_max, int64_t nblk_stride, int64_t nsup_stride,
    float* __restrict__ scores, float* __restrict__ block_max, float* __restrict__ super_max) {
  const int64_t seq = blockIdx.z;
  const int r = (int)seq * M + (int)blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15;   // key within a 16-position group
  const int g = lane >> 4;   // block held by this lane
  int64_t nv = n_visible[r];
  nv = nv < 0 ? 0 : (nv > N_max ? N_max : nv);
  const int64_t p0 = xcd_run_tile<kScanXcdRun>(blockIdx.x, gridDim.x) * kScanChunk + (int64_t)wave * 64;
  if (p0 >= nv) return;   // no barriers below: waves leave independently

  const uint8_t* kc = k_codes + seq * N_max * 64;
  const uint8_t* ks = k_scales + seq * N_max * 4;
  u32x4_t kb[4];
  uint32_t ek[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    int64_t p = p0 + 16 * u + c;
    p = p < nv ? p : nv - 1;   // tail lanes re-read a visible row
    kb[u] = load_codes16(kc + p * 64 + 16 * g);
    ek[u] = ks[p * 4 + g];
  }
  // this lane's query block g, decoded once
  half2_t qh[16];
  load_query_block(q_codes + (int64_t)r * 64 + 16 * g, qh);
  const int eq = q_scales[(int64_t)r * 4 + g];
  const float s = score_groups_valu(qh, eq, kb, ek);
  const int64_t key = p0 + lane;
  const bool vis = key < nv;
  if (kScores && vis) __builtin_nontemporal_store(s, &scores[(int64_t)r * N_max + key]);
  const uint32_t m8 = group8_max_u32(vis ? order_key(s) : 0u);
  if ((lane & 7) == 0 && vis) block_max[(int64_t)r * nblk_stride + (key >> 3)] = key_to_float(m8);
  if (kSuper) {
    const uint32_t m = wave_max_u32(m8);
    if (lane == 0) super_max[(int64_t)r * nsup_stride + (p0 >> 6)] = key_to_float(m);
  }
}

// Several queries per sequence (2 <= M < 16, e.g. a verify step over draft
// tokens).  Grid (ceil(N_max / 256), 1, B); 7 waves per SIMD leave the loop
// over the rows 72 registers (no spills).  Each wave loads 64 consecutive keys
// once and scores them against all M query rows of the sequence, rows
// r = seq * M + m: a multi-token decode reads every key once, not M times.  The
// rows' query blocks travel in registers (lane l holds row l / 4, block l % 4)
// and reach the matrix-core operand layout by lane shuffles, so the loop over
// the rows issues no memory loads.  All loads are issued before any arithmetic.
// Outputs per row: block maxima, optional super-block maxima (8 blocks) and
// optional per-position scores.
template <bool kScores, bool kSuper>
__global__ __launch_bounds__(kScanThreads) __attribute__((amdgpu_waves_per_eu(7, 7))) void index_scan_multi_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales,
    const int32_t* __restrict__ n_visible, int M, int64_t N_max, int64_t nblk_stride, int64_t nsup_stride,
    float* __restrict__ scores, float* __restrict__ block_max, float* __restrict__ super_max) {
  const int64_t seq = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15;   // key within a 16-position group (B column)
  const int g = lane >> 4;   // block held by this lane (B K group)
  // lane m < M: row m's visible count and scale bytes; lane l < 4M: row l / 4's
  // query block l % 4
  int nvl = 0;
  uint32_t qsl = 0u;
  u32x4_t qpiece = {0u, 0u, 0u, 0u};
  if (lane < M) {
    int64_t v = n_visible[seq * M + lane];
    nvl = (int)(v < 0 ? 0 : (v > N_max ? N_max : v));
    qsl = *reinterpret_cast<const uint32_t*>(q_scales + (seq * M + lane) * 4);
  }
  if (lane < 4 * M) qpiece = *reinterpret_cast<const u32x4_t*>(q_codes + (seq * M + (lane >> 2)) * 64 + 16 * (lane & 3));
  const int64_t nv_all = (int64_t)wave_max_u32((uint32_t)nvl);   // the widest row: keys loaded for all rows
  const int64_t p0 = xcd_run_tile<kScanXcdRun>(blockIdx.x, gridDim.x) * kScanChunk + (int64_t)wave * 64;
  if (p0 >= nv_all) return;   // no barriers below: waves leave independently

  const uint8_t* kc = k_codes + seq * N_max * 64;
  const uint8_t* ks = k_scales + seq * N_max * 4;
  u32x4_t kb[4];
  uint32_t ek[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    int64_t p = p0 + 16 * u + c;
    p = p < nv_all ? p : nv_all - 1;   // tail lanes re-read a visible row
    kb[u] = load_codes16(kc + p * 64 + 16 * g);
    ek[u] = ks[p * 4 + g];
  }

  // a row's outputs for this wave's 64 keys
  auto emit = [&](int64_t r, int64_t nv, float s) {
    const int64_t key = p0 + lane;
    const bool vis = key < nv;
    if (kScores && vis) __builtin_nontemporal_store(s, &scores[r * N_max + key]);
    const uint32_t m8 = group8_max_u32(vis ? order_key(s) : 0u);
    if ((lane & 7) == 0 && vis) block_max[r * nblk_stride + (key >> 3)] = key_to_float(m8);
    if (kSuper) {
      const uint32_t mx = wave_max_u32(m8);
      if (lane == 0) super_max[r * nsup_stride + (p0 >> 6)] = key_to_float(mx);
    }
  };
  // rows whose visible block exponents all lie in [-124, 114]: the matrix
  // cores; the others are scored on the vector ALUs after this loop, once the
  // keys' registers are free
  uint32_t valu_rows = 0u;
  for (int m = 0; m < M; ++m) {
    const int64_t nv = __builtin_amdgcn_readlane(nvl, m);
    if (p0 >= nv) continue;   // uniform over the wave
    const int eq = (int)((__builtin_amdgcn_readlane(qsl, m) >> (8 * g)) & 0xFFu);
    bool bad = false;
#pragma unroll
    for (int u = 0; u < 4; ++u) bad |= p0 + 16 * u + c < nv && exponent_out_of_range(eq, ek[u]);
    if (__ballot(bad) != 0ull) {
      valu_rows |= 1u << m;
      continue;
    }
    // A operand: lane 16g + i (row i, K group g) holds query block g when i % 4 == g
    const int src = 4 * m + g;   // the lane holding row m's block g
    u32x4_t qa;
#pragma unroll
    for (int e = 0; e < 4; ++e) qa[e] = (uint32_t)__shfl((int)qpiece[e], src, 64);
    if ((lane & 3) != g) qa = u32x4_t{0u, 0u, 0u, 0u};
    emit(seq * M + m, nv, score_groups_mfma(qa, eq, kb, ek));
  }
  while (valu_rows) {
    const int m = __builtin_ctz(valu_rows);
    valu_rows &= valu_rows - 1u;
    const int64_t r = seq * M + m;
    const int64_t nv = __builtin_amdgcn_readlane(nvl, m);
    int64_t p = p0 + lane;
    p = p < nv ? p : nv - 1;
    emit(r, nv, score_key_valu(q_codes + r * 64, q_scales + r * 4, kc + p * 64, ks + p * 4));
  }
}

// Pool scan: one wave scores 8 pool blocks (64 positions) with the decode scan's
// lane layout (group u = pool blocks 2u and 2u + 1; lane 16g + c holds block g
// of position c & 7 of pool block 2u + (c >> 3)); lane l's result is slot l of
// the wave's 64 output slots.  Grid (ceil(n_pool / 32), M, B), four waves (32
// pool blocks of one row) per workgroup.
constexpr int kPoolWaveBlocks = 8;
constexpr int kPoolWaves = 4;

__global__ __launch_bounds__(64 * kPoolWaves) void pool_scan_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales,
    const int32_t* __restrict__ pool_blocks, int n_pool, const int32_t* __restrict__ n_visible, int M,
    int64_t N_max, float* __restrict__ pool_scores) {
  const int64_t seq = blockIdx.z;
  const int r = (int)seq * M + (int)blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int base = ((int)blockIdx.x * kPoolWaves + (int)(threadIdx.x >> 6)) * kPoolWaveBlocks;
  if (base >= n_pool) return;   // no barriers: waves leave independently
  int64_t nv = n_visible[r];
  nv = nv < 0 ? 0 : (nv > N_max ? N_max : nv);
  const int32_t* pb = pool_blocks + (int64_t)r * n_pool;
  // pool block of group u for this lane's column: base + 2u + (c >> 3); loads at
  // clamped indices, all issued together; ids past the pool are -1
  int32_t blk[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = base + 2 * u + (c >> 3);
    const int32_t v = pb[i < n_pool ? i : n_pool - 1];
    blk[u] = i < n_pool ? v : -1;
  }

  const uint8_t* kc = k_codes + seq * N_max * 64;
  const uint8_t* ks = k_scales + seq * N_max * 4;
  u32x4_t kb[4];
  uint32_t ek[4];
  bool ok[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int32_t b = blk[u];
    int64_t p = 8 * (int64_t)b + (c & 7);
    ok[u] = b >= 0 && p < nv;
    p = ok[u] ? p : 0;   // masked lanes read position 0 (in bounds)
    kb[u] = load_codes16(kc + p * 64 + 16 * g);
    ek[u] = ks[p * 4 + g];
  }
  half2_t qh[16];
  load_query_block(q_codes + (int64_t)r * 64 + 16 * g, qh);
  const int eq = q_scales[(int64_t)r * 4 + g];
  const float s = score_groups_valu(qh, eq, kb, ek);
  // this lane's output slot: group g, column c
  const bool mine_ok = (g & 2) ? ((g & 1) ? ok[3] : ok[2]) : ((g & 1) ? ok[1] : ok[0]);
  if (base + 2 * g + (c >> 3) < n_pool)
    pool_scores[((int64_t)r * n_pool + base) * 8 + lane] = mine_ok ? s : -__builtin_inff();
}

hipError_t launch_index_scan(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                             const uint8_t* k_scales, const int32_t* n_visible, int B, int M, int64_t N_max,
                             float* scores, float* block_max, int64_t nblk_stride, float* super_max,
                             int64_t nsup_stride, hipStream_t stream) {
  // many queries per sequence share every key: the matrix-core scan
  if (M >= kPrefillMinQueries)
    return launch_prefill_scan(q_codes, q_scales, k_codes, k_scales, n_visible, B, M, N_max, scores, block_max,
                               nblk_stride, super_max, nsup_stride, stream);
  if (M > 65535 || B > 65535) return hipErrorInvalidConfiguration;
  const unsigned chunks = (unsigned)((N_max + kScanChunk - 1) / kScanChunk);
  // one query per sequence: one row per workgroup; several: every key once for all rows
  const bool multi = M > 1;
  const dim3 grid(chunks, multi ? 1u : (unsigned)M, (unsigned)B);
#define CSA2_SCAN(S, P)                                                                                          \
  do {                                                                                                           \
    if (multi)                                                                                                   \
      hipLaunchKernelGGL((index_scan_multi_kernel<S, P>), grid, dim3(kScanThreads), 0, stream, q_codes, q_scales, \
                         k_codes, k_scales, n_visible, M, N_max, nblk_stride, nsup_stride, scores, block_max,     \
                         super_max);                                                                             \
    else                                                                                                         \
      hipLaunchKernelGGL((index_scan_kernel<S, P>), grid, dim3(kScanThreads), 0, stream, q_codes, q_scales,      \
                         k_codes, k_scales, n_visible, M, N_max, nblk_stride, nsup_stride, scores, block_max,     \
                         super_max);                                                                             \
  } while (0)
  if (scores && super_max) CSA2_SCAN(true, true);
  else if (scores) CSA2_SCAN(true, false);
  else if (super_max) CSA2_SCAN(false, true);
  else CSA2_SCAN(false, false);
#undef CSA2_SCAN
  return hipGetLastError();
}

hipError_t launch_pool_scan(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                            const uint8_t* k_scales, const int32_t* pool_blocks, int n_pool,
                            const int32_t* n_visible, int B, int M, int64_t N_max, float* pool_scores,
                            hipStream_t stream) {
  if (M > 65535 || B > 65535) return hipErrorInvalidConfiguration;
  constexpr int kPer = kPoolWaveBlocks * kPoolWaves;
  dim3 grid((unsigned)((n_pool + kPer - 1) / kPer), (unsigned)M, (unsigned)B);
  hipLaunchKernelGGL(pool_scan_kernel, grid, dim3(64 * kPoolWaves), 0, stream, q_codes, q_scales, k_codes,
                     k_scales, pool_blocks, n_pool, n_visible, M, N_max, pool_scores);
  return hipGetLastError();
}

}  // namespace csa2
