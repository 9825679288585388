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
// Thread mapping: four lanes per cached position, lane 4p+b owns 32-element
// block b, so one 16-byte load per lane reads one whole block and a wave's load
// instruction covers 16 consecutive positions = 1 KiB of contiguous codes.  The
// E2M1 codes are decoded in registers (v_cvt_scalef32_pk_f16_fp4, exact) and
// multiplied with v_dot2 into an fp32 accumulator (exact, see block_dot); the
// quad's four block values are combined in order with DPP broadcasts and the
// block max of 8 positions (half a wave) is a DPP/permute reduction.
#include "device_common.h"
#include "kernels.h"

namespace csa2 {

constexpr int kScanThreads = 256;
constexpr int kScanWaves = kScanThreads / 64;
constexpr int kSupersPerWave = 2;                               // 64-position super-blocks per wave
constexpr int kScanChunk = kScanWaves * kSupersPerWave * 64;    // positions per workgroup
constexpr int kScanGroups = kSupersPerWave * 4;                  // 16-position groups per wave
constexpr int kPrefillMinQueries = 16;                           // queries per sequence for the MFMA scan

__device__ __forceinline__ u32x4_t load_codes16(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xF, false);
}

// Score of one 16-position group (lane 4p+b holds block b of position p) and
// the maxima of its two 8-position blocks: on return lanes 16..31 hold block
// A's (positions 0-7) maximum key and lanes 48..63 block B's (positions 8-15).
__device__ __forceinline__ uint32_t group_score_max(const u32x4_t c, uint32_t e, const half2_t* qh, int eq, bool vis,
                                                    float* s_out) {
  const float v = __builtin_amdgcn_ldexpf(block_dot(c, qh), eq + (int)e - 254);
  const float s = quad_ordered_sum(v);
  *s_out = s;
  uint32_t k = vis ? order_key(s) : 0u;
  uint32_t y = dpp_u32<0x124, 0xF>(k);   // row_ror:4 -> max of two quads
  k = y > k ? y : k;
  y = dpp_u32<0x128, 0xF>(k);            // row_ror:8 -> max of the row (4 positions)
  k = y > k ? y : k;
  y = dpp_u32<0x142, 0xA>(k);            // row_bcast:15 -> rows 1, 3 take the row before
  return y > k ? y : k;
}

// Each wave scores kSupersPerWave consecutive 64-position super-blocks; all of
// its loads are issued before any arithmetic.  Outputs: block maxima, optional
// super-block maxima (8 blocks) and optional per-position scores.
template <bool kScores, bool kSuper>
__global__ __launch_bounds__(kScanThreads) void index_scan_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales,
    const int32_t* __restrict__ n_visible, int M, int64_t N_max, int64_t nblk_stride, int64_t nsup_stride,
    float* __restrict__ scores, float* __restrict__ block_max, float* __restrict__ super_max) {
  const int r = blockIdx.y;
  const int64_t seq = r / M;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = lane & 3;
  const int pl = lane >> 2;
  int64_t nv = n_visible[r];
  nv = nv < 0 ? 0 : (nv > N_max ? N_max : nv);
  const int64_t p0 = (int64_t)blockIdx.x * kScanChunk + (int64_t)wave * (kSupersPerWave * 64);
  if (p0 >= nv) return;   // no barriers below: waves leave independently

  half2_t qh[16];
  load_query_block(q_codes + (int64_t)r * 64 + 16 * b, qh);
  const int eq = q_scales[(int64_t)r * 4 + b];
  const uint8_t* kc = k_codes + seq * N_max * 64 + 16 * b;
  const uint8_t* ks = k_scales + seq * N_max * 4 + b;

  u32x4_t c[kScanGroups];
  uint32_t e[kScanGroups];
#pragma unroll
  for (int u = 0; u < kScanGroups; ++u) {
    int64_t p = p0 + 16 * u + pl;
    p = p < nv ? p : nv - 1;             // tail lanes re-read a visible row
    c[u] = load_codes16(kc + p * 64);
    e[u] = ks[p * 4];
  }
#pragma unroll
  for (int h = 0; h < kSupersPerWave; ++h) {
    uint32_t smax = 0u;
#pragma unroll
    for (int u = 4 * h; u < 4 * h + 4; ++u) {
      const int64_t gp = p0 + 16 * u;
      const int64_t p = gp + pl;
      float s;
      const uint32_t k = group_score_max(c[u], e[u], qh, eq, p < nv, &s);
      if (kScores && b == 0 && p < nv) scores[(int64_t)r * N_max + p] = s;
      smax = k > smax ? k : smax;
      if (lane == 16 && gp < nv) block_max[(int64_t)r * nblk_stride + (gp >> 3)] = key_to_float(k);
      if (lane == 48 && gp + 8 < nv) block_max[(int64_t)r * nblk_stride + (gp >> 3) + 1] = key_to_float(k);
    }
    if (kSuper) {
      const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)smax, 16);
      const uint32_t bb = (uint32_t)__builtin_amdgcn_readlane((int)smax, 48);
      const int64_t sp = p0 + 64 * h;
      if (lane == 0 && sp < nv) super_max[(int64_t)r * nsup_stride + (sp >> 6)] = key_to_float(a > bb ? a : bb);
    }
  }
}

// Pool scan: each half wave scores one pool block (8 positions x 4 blocks).
constexpr int kPoolBlocksPerWG = 64;

__global__ __launch_bounds__(kScanThreads) void pool_scan_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales,
    const int32_t* __restrict__ pool_blocks, int n_pool, const int32_t* __restrict__ n_visible, int M,
    int64_t N_max, float* __restrict__ pool_scores) {
  const int r = blockIdx.y;
  const int64_t seq = r / M;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = lane & 3;
  const int t = (lane >> 2) & 7;
  const int half = lane >> 5;
  int64_t nv = n_visible[r];
  nv = nv < 0 ? 0 : (nv > N_max ? N_max : nv);

  half2_t qh[16];
  load_query_block(q_codes + (int64_t)r * 64 + 16 * b, qh);
  const int eq = q_scales[(int64_t)r * 4 + b];
  const uint8_t* kc = k_codes + seq * N_max * 64 + 16 * b;
  const uint8_t* ks = k_scales + seq * N_max * 4 + b;
  const int32_t* pb = pool_blocks + (int64_t)r * n_pool;

  const int i_begin = blockIdx.x * kPoolBlocksPerWG;
  const int i_end = min(i_begin + kPoolBlocksPerWG, n_pool);
  // wave-groups of two pool blocks; wave w takes pairs w, w+4, ...
  constexpr int kPairs = kPoolBlocksPerWG / 2 / 4;
  u32x4_t c[kPairs];
  uint32_t e[kPairs];
  bool valid[kPairs];
#pragma unroll
  for (int u = 0; u < kPairs; ++u) {
    const int i = i_begin + 2 * (wave + 4 * u) + half;
    int64_t blk = (i < i_end) ? pb[i] : -1;
    int64_t p = 8 * blk + t;
    valid[u] = (blk >= 0) && (p < nv);
    p = valid[u] ? p : 0;
    c[u] = load_codes16(kc + p * 64);
    e[u] = ks[p * 4];
  }
#pragma unroll
  for (int u = 0; u < kPairs; ++u) {
    const int i = i_begin + 2 * (wave + 4 * u) + half;
    const float v = __builtin_amdgcn_ldexpf(block_dot(c[u], qh), eq + (int)e[u] - 254);
    const float s = quad_ordered_sum(v);
    if (b == 0 && i < i_end) pool_scores[((int64_t)r * n_pool + i) * 8 + t] = valid[u] ? s : -__builtin_inff();
  }
}

hipError_t launch_index_scan(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                             const uint8_t* k_scales, const int32_t* n_visible, int B, int M, int64_t N_max,
                             float* scores, float* block_max, int64_t nblk_stride, float* super_max,
                             int64_t nsup_stride, hipStream_t stream) {
  // many queries per sequence share every key: the matrix-core scan
  if (M >= kPrefillMinQueries)
    return launch_prefill_scan(q_codes, q_scales, k_codes, k_scales, n_visible, B, M, N_max, scores, block_max,
                               nblk_stride, super_max, nsup_stride, stream);
  const int R = B * M;
  dim3 grid((unsigned)((N_max + kScanChunk - 1) / kScanChunk), (unsigned)R);
#define CSA2_SCAN(S, P)                                                                                         \
  hipLaunchKernelGGL((index_scan_kernel<S, P>), grid, dim3(kScanThreads), 0, stream, q_codes, q_scales, k_codes, \
                     k_scales, n_visible, M, N_max, nblk_stride, nsup_stride, scores, block_max, super_max)
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
  const int R = B * M;
  dim3 grid((unsigned)((n_pool + kPoolBlocksPerWG - 1) / kPoolBlocksPerWG), (unsigned)R);
  hipLaunchKernelGGL(pool_scan_kernel, grid, dim3(kScanThreads), 0, stream, q_codes, q_scales, k_codes, k_scales,
                     pool_blocks, n_pool, n_visible, M, N_max, pool_scores);
  return hipGetLastError();
}

}  // namespace csa2
