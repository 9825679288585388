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
constexpr int kScanUnroll = 8;          // 16-position groups in flight per wave

__device__ __forceinline__ u32x4_t load_codes16(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

template <bool kScores>
__global__ __launch_bounds__(kScanThreads) void index_scan_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales,
    const int32_t* __restrict__ n_visible, int M, int64_t N_max, int64_t nblk_stride, int chunk,
    float* __restrict__ scores, float* __restrict__ block_max) {
  const int r = blockIdx.y;
  const int64_t seq = r / M;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = lane & 3;
  const int pl = lane >> 2;
  int64_t nv = n_visible[r];
  nv = nv < 0 ? 0 : (nv > N_max ? N_max : nv);
  const int64_t p0 = (int64_t)blockIdx.x * chunk;
  if (p0 >= nv) return;
  const int64_t pend = (p0 + chunk < nv) ? p0 + chunk : nv;

  half2_t qh[16];
  load_query_block(q_codes + (int64_t)r * 64 + 16 * b, qh);
  const int eq = q_scales[(int64_t)r * 4 + b];

  const uint8_t* kc = k_codes + seq * N_max * 64 + 16 * b;
  const uint8_t* ks = k_scales + seq * N_max * 4 + b;
  const int ngroups = (int)((pend - p0 + 15) >> 4);

  for (int g0 = wave; g0 < ngroups; g0 += 4 * kScanUnroll) {
    u32x4_t c[kScanUnroll];
    uint32_t e[kScanUnroll];
#pragma unroll
    for (int u = 0; u < kScanUnroll; ++u) {
      const int g = g0 + 4 * u;
      int64_t p = p0 + 16 * g + pl;
      p = p < pend ? p : pend - 1;           // tail lanes re-read a visible row
      if (g < ngroups) {
        c[u] = load_codes16(kc + p * 64);
        e[u] = ks[p * 4];
      }
    }
#pragma unroll
    for (int u = 0; u < kScanUnroll; ++u) {
      const int g = g0 + 4 * u;
      if (g >= ngroups) break;
      const int64_t p = p0 + 16 * g + pl;
      const float v = __builtin_amdgcn_ldexpf(block_dot(c[u], qh), eq + (int)e[u] - 254);
      const float s = quad_ordered_sum(v);
      const bool vis = p < pend;
      if (kScores && vis && b == 0) scores[(int64_t)r * N_max + p] = s;
      const uint32_t key = halfwave_quad_max(vis ? order_key(s) : 0u);
      if ((lane & 31) == 0) {
        const int64_t blk = ((p0 + 16 * g) >> 3) + (lane >> 5);
        if (8 * blk < pend) block_max[(int64_t)r * nblk_stride + blk] = key_to_float(key);
      }
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
                             float* scores, float* block_max, int64_t nblk_stride, hipStream_t stream) {
  const int R = B * M;
  const int chunk = scan_chunk_positions(N_max);
  dim3 grid((unsigned)((N_max + chunk - 1) / chunk), (unsigned)R);
  if (scores)
    hipLaunchKernelGGL(index_scan_kernel<true>, grid, dim3(kScanThreads), 0, stream, q_codes, q_scales, k_codes,
                       k_scales, n_visible, M, N_max, nblk_stride, chunk, scores, block_max);
  else
    hipLaunchKernelGGL(index_scan_kernel<false>, grid, dim3(kScanThreads), 0, stream, q_codes, q_scales, k_codes,
                       k_scales, n_visible, M, N_max, nblk_stride, chunk, scores, block_max);
  return hipGetLastError();
}

int scan_chunk_positions(int64_t /*N_max*/) { return 2048; }

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
