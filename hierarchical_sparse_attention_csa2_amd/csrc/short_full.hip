// The Full-layer indexer in one launch for short decode rows (one query per
// sequence, at most 16,384 positions, every 8-position block inside the pool):
// the scan, the pool and the top-k of a row without a second kernel.
//
// DeepSeek-V4.1-Flash, fupanwang.com article, section 三个方向一起压小缓存 and the
// figure caption on the hierarchical sparse indexer: the first Full layer
// scores every visible position with the FP4 indexer, keeps the best 2048
// blocks of 8 positions as the pool and reads its best 512 positions.  When a
// row has at most as many blocks as the pool holds, the pool is every visible
// block, and the pool keeping at least k blocks, its top-k is the top-k over
// every visible position (a block ranked ahead of a block holding a selected
// position contributes its own best position to the selection).
//
// Grid (ceil(N_max / 1024), R), 1024 threads.  Every workgroup scores 1024
// positions of its row (64 per wave, the decode scan's lane layout and exact
// arithmetic), stores the scores, writes its blocks' pool entries and then
// counts itself in at the row's counter.  The workgroup that arrives last
// resets the counter to zero and ranks the row's stored scores (the register
// radix select, ties to the lowest position).  No workgroup waits on another.
#include "device_common.h"
#include "kernels.h"
#include "score_core.h"
#include "select_core.h"

namespace csa2 {

constexpr int kShortMaxPositions = 16384;
constexpr int kShortPositionsPerWg = kSelThreads;   // 64 per wave
constexpr int kShortBlocksPerWg = kShortPositionsPerWg / 8;

template <int J>
__global__ __launch_bounds__(kSelThreads) void index_full_short_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales,
    const int32_t* __restrict__ n_visible, int64_t N_max, int n_pool, int32_t* __restrict__ pool_out, int k,
    int32_t* __restrict__ idx, float* scores, float* __restrict__ block_max, int64_t nblk_stride,
    uint32_t* __restrict__ counters) {
  __shared__ RegShared sh;
  __shared__ int last;
  const int r = blockIdx.y;   // row = sequence (one query each)
  const int b = blockIdx.x;
  const int nwg = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  int64_t nv = n_visible[r];
  nv = nv < 0 ? 0 : (nv > N_max ? N_max : nv);

  const int64_t p0 = (int64_t)b * kShortPositionsPerWg + (int64_t)w * 64;
  if (p0 < nv) {   // uniform over the wave
    const uint8_t* kc = k_codes + (int64_t)r * N_max * 64;
    const uint8_t* ks = k_scales + (int64_t)r * N_max * 4;
    u32x4_t kb[4];
    uint32_t ek[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int64_t p = p0 + 16 * u + c;
      p = p < nv ? p : nv - 1;   // tail lanes re-read a visible row
      kb[u] = load_codes16(kc + p * 64 + 16 * g);
      ek[u] = ks[p * 4 + g];
    }
    half2_t qh[16];
    load_query_block(q_codes + (int64_t)r * 64 + 16 * g, qh);
    const int eq = q_scales[(int64_t)r * 4 + g];
    const float s = score_groups_valu(qh, eq, kb, ek);
    const int64_t pos = p0 + lane;
    const bool vis = pos < nv;
    if (vis) scores[(int64_t)r * N_max + pos] = s;
    if (block_max) {
      const uint32_t m8 = group8_max(vis ? order_key(s) : 0u);
      if ((lane & 7) == 0 && vis) block_max[(int64_t)r * nblk_stride + (pos >> 3)] = key_to_float(m8);
    }
  }

  // the pool is every visible block: this workgroup's blocks, and workgroup 0
  // pads the entries past the last workgroup's blocks
  {
    const int64_t nblk = (nv + 7) >> 3;
    int32_t* po = pool_out + (int64_t)r * n_pool;
    const int p = b * kShortBlocksPerWg + tid;
    if (tid < kShortBlocksPerWg && p < n_pool) po[p] = p < nblk ? p : -1;
    if (b == 0)
      for (int q = nwg * kShortBlocksPerWg + tid; q < n_pool; q += kSelThreads) po[q] = -1;
  }

  // arrival: every thread's stores are released at device scope before the
  // workgroup counts itself in
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = atomicAdd(&counters[r], 1u);
    const int is_last = old == (uint32_t)(nwg - 1);
    if (is_last) atomicExch(&counters[r], 0u);   // every workgroup of the row has counted: reset for the next call
    last = is_last;
  }
  __syncthreads();
  if (!last) return;
  __threadfence();   // acquire: the other workgroups' scores

  // the row's scores into the select's registers: item (w, j, lane) is
  // position (w * Jp + j) * 64 + lane
  const int Jp = (int)((N_max + kSelThreads - 1) / kSelThreads);
  const float* row = scores + (int64_t)r * N_max;
  uint32_t key[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t i = (int64_t)(w * Jp + j) * 64 + lane;
    key[j] = (j < Jp && i < nv) ? order_key(row[i]) : 0u;
  }
  hist_zero(sh.c);
  if (tid == 0) {
    sh.s.cnt[0] = 0;
    sh.s.cnt[1] = 0;
  }
  int valid;
  uint32_t kmin, kmax;
  key_range(sh.s, key, Jp, valid, kmin, kmax);
  Thr th0, th1;
  select_thresholds(sh.c, sh.s, key, Jp, valid, kmin, kmax, k, 0, 0, th0, th1);
  int32_t* out = idx + (int64_t)r * k;
  emit_sel(
      sh.s, key, Jp, th0, th1, [&](int, int pos, int, int i) { out[pos] = i; }, [&](int, int p) { out[p] = -1; });
}

hipError_t launch_index_full_short(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                                   const uint8_t* k_scales, const int32_t* n_visible, int B, int M, int64_t N_max,
                                   int n_pool, int k, int32_t* pool_out, int32_t* idx, float* scores,
                                   float* block_max, uint32_t* counters, hipStream_t stream) {
  if (M != 1 || k < 1 || B > kShortCounterRows || N_max < 1 || N_max > kShortMaxPositions ||
      (N_max + 7) / 8 > n_pool)
    return hipErrorNotSupported;
  const dim3 grid((unsigned)((N_max + kShortPositionsPerWg - 1) / kShortPositionsPerWg), (unsigned)B);
  const dim3 block(kSelThreads);
  const int64_t nblk_stride = (N_max + 7) / 8;
#define CSA2_SHORT(J)                                                                                          \
  hipLaunchKernelGGL((index_full_short_kernel<J>), grid, block, 0, stream, q_codes, q_scales, k_codes, k_scales, \
                     n_visible, N_max, n_pool, pool_out, k, idx, scores, block_max, nblk_stride, counters)
  if (N_max <= 4096)
    CSA2_SHORT(4);
  else if (N_max <= 8192)
    CSA2_SHORT(8);
  else
    CSA2_SHORT(16);
#undef CSA2_SHORT
  return hipGetLastError();
}

}  // namespace csa2
