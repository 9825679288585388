// Ranked selection: the coarse block filter (top-n_pool blocks by block max) and
// the top-k over pool or full score rows.
//
// DeepSeek-V4.1-Flash, fupanwang.com article, section 三个方向一起压小缓存 and the
// figure caption on the hierarchical sparse indexer: blocks are represented by
// their highest score, the top blocks form the candidate pool (at most 2048
// blocks), and each layer selects its top-512 positions.  Ranking is by
// (score desc, id asc): ties go to the lowest position / block id.
//
// One 1024-thread workgroup per row.  An exact radix select on the IEEE total-
// order key of each score (12 + 12 + 8 bits, LDS histograms) finds the k-th key
// T and how many of the elements equal to T are taken; an emit pass in id order
// then takes every key > T and the first r keys == T (prefix sums over the
// workgroup), which writes the selected ids already ascending.  Rows of up to
// 16,384 elements are cached in LDS; longer rows are re-read from memory.
#include "device_common.h"
#include "kernels.h"

namespace csa2 {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelCap = 16384;
constexpr int kSelIPT = kSelCap / kSelThreads;   // items per thread per emit chunk
constexpr int kBins = 4096;

struct SelRow {
  int layout;
  const float* s;          // row base
  const int32_t* pb;       // pool layout: this row's pool block ids
  int64_t n;               // elements in the row
  int64_t nv;              // visible positions
  const uint32_t* cache;   // LDS copy of the keys or nullptr

  __device__ __forceinline__ uint32_t key_mem(int64_t i) const {
    if (layout == kSelPool) {
      const int64_t blk = pb[i >> 3];
      const int64_t p = 8 * blk + (i & 7);
      if (blk < 0 || p >= nv) return 0u;
    }
    return order_key(s[i]);
  }
  __device__ __forceinline__ uint32_t key(int64_t i) const { return cache ? cache[i] : key_mem(i); }
  __device__ __forceinline__ int32_t id(int64_t i) const {
    if (layout == kSelPool) return (int32_t)(8 * (int64_t)pb[i >> 3] + (i & 7));
    return (int32_t)i;
  }
};

// Exclusive scan over the workgroup; *total receives the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wave[w] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int i = 0; i < kSelWaves; ++i) {
      const int t = s_wave[i];
      s_wave[i] = acc;
      acc += t;
    }
    s_wave[kSelWaves] = acc;
  }
  __syncthreads();
  const int res = s_wave[w] + x - v;
  *total = s_wave[kSelWaves];
  __syncthreads();
  return res;
}

// Histogram of digit (key >> shift) & (2^bits - 1) over non-zero keys whose
// bits above the digit equal `prefix` (under `mask`); then the digit t such
// that (#elements with a larger digit) < need <= (# with digit >= t).
__device__ void radix_pass(const SelRow& row, int shift, int bits, uint32_t mask, uint32_t prefix, int need,
                           uint32_t* s_hist, int* s_wave, int* s_res, uint32_t* digit, int* above) {
  for (int i = threadIdx.x; i < kBins; i += kSelThreads) s_hist[i] = 0;
  __syncthreads();
  if (threadIdx.x == 0) {
    s_res[0] = 0;
    s_res[1] = 0;
  }
  const uint32_t dmask = (1u << bits) - 1u;
  for (int64_t i = threadIdx.x; i < row.n; i += kSelThreads) {
    const uint32_t k = row.key(i);
    if (k != 0u && (k & mask) == prefix) atomicAdd(&s_hist[(k >> shift) & dmask], 1u);
  }
  __syncthreads();
  // thread t owns bins 4095-4t .. 4092-4t (descending)
  const int hi = kBins - 1 - 4 * (int)threadIdx.x;
  int local = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) local += (int)s_hist[hi - j];
  int total;
  const int before = block_excl_scan(local, s_wave, &total);
  if (before < need && need <= before + local) {
    int acc = before;
    for (int j = 0; j < 4; ++j) {
      const int c = (int)s_hist[hi - j];
      if (acc + c >= need) {
        s_res[0] = hi - j;
        s_res[1] = acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
  // need is within [1, #matching keys] by construction, so exactly one thread
  // found the digit (s_res is preset so a violated precondition stays in range)
  *digit = (uint32_t)s_res[0];
  *above = s_res[1];
  __syncthreads();
}

// Write the first k_eff elements by (key desc, id asc) in id order, -1 pad to k.
__device__ void emit(const SelRow& row, uint32_t T, int take_ties, int k_eff, int k, int32_t* out, int* s_wave) {
  int carry_tie = 0, carry_sel = 0;
  for (int64_t base = 0; base < row.n && k_eff > 0; base += kSelCap) {
    const int64_t i0 = base + (int64_t)threadIdx.x * kSelIPT;
    uint32_t kk[kSelIPT];
    int ties = 0;
#pragma unroll
    for (int j = 0; j < kSelIPT; ++j) {
      kk[j] = (i0 + j < row.n) ? row.key(i0 + j) : 0u;
      ties += (kk[j] == T);
    }
    int tot_t;
    int rank = block_excl_scan(ties, s_wave, &tot_t) + carry_tie;
    unsigned selmask = 0;
    int nsel = 0;
#pragma unroll
    for (int j = 0; j < kSelIPT; ++j) {
      bool s = kk[j] > T;
      if (kk[j] == T) {
        s = rank < take_ties;
        ++rank;
      }
      if (s) {
        selmask |= 1u << j;
        ++nsel;
      }
    }
    int tot_s;
    int pos = block_excl_scan(nsel, s_wave, &tot_s) + carry_sel;
#pragma unroll
    for (int j = 0; j < kSelIPT; ++j)
      if ((selmask & (1u << j)) && pos < k_eff) out[pos++] = row.id(i0 + j);
    carry_tie += tot_t;
    carry_sel += tot_s;
    if (carry_sel >= k_eff) break;
  }
  for (int i = k_eff + threadIdx.x; i < k; i += kSelThreads) out[i] = -1;
}

// Threshold key T and the number of elements == T to take, for the first k_eff
// of the ranking (1 <= k_eff <= #valid).
__device__ void find_kth(const SelRow& row, int k_eff, int valid, uint32_t* s_hist, int* s_wave, int* s_res,
                         uint32_t* T, int* take_ties) {
  if (k_eff >= valid) {
    *T = 1u;               // every non-zero key
    *take_ties = 0x7FFFFFFF;
    return;
  }
  uint32_t d1, d2, d3;
  int a1, a2, a3;
  int need = k_eff;
  radix_pass(row, 20, 12, 0u, 0u, need, s_hist, s_wave, s_res, &d1, &a1);
  need -= a1;
  uint32_t prefix = d1 << 20;
  radix_pass(row, 8, 12, 0xFFF00000u, prefix, need, s_hist, s_wave, s_res, &d2, &a2);
  need -= a2;
  prefix |= d2 << 8;
  radix_pass(row, 0, 8, 0xFFFFFF00u, prefix, need, s_hist, s_wave, s_res, &d3, &a3);
  need -= a3;
  *T = prefix | d3;
  *take_ties = need;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(int layout, const float* __restrict__ scores,
                                                             int64_t stride, const int32_t* __restrict__ pool_blocks,
                                                             int64_t n_pool, const int32_t* __restrict__ n_visible,
                                                             int k1, int32_t* __restrict__ out1, int k2,
                                                             int32_t* __restrict__ out2) {
  __shared__ uint32_t s_keys[kSelCap];
  __shared__ uint32_t s_hist[kBins];
  __shared__ int s_wave[kSelWaves + 1];
  __shared__ int s_res[2];

  const int r = blockIdx.x;
  SelRow row;
  row.layout = layout;
  row.cache = nullptr;
  row.pb = nullptr;
  int64_t nv = n_visible[r];
  nv = nv < 0 ? 0 : nv;
  if (layout == kSelBlocks) {
    row.s = scores + (int64_t)r * stride;
    row.n = (nv + 7) >> 3;
    if (row.n > stride) row.n = stride;
  } else if (layout == kSelPool) {
    row.s = scores + (int64_t)r * n_pool * 8;
    row.pb = pool_blocks + (int64_t)r * n_pool;
    row.n = 8 * n_pool;
  } else {
    row.s = scores + (int64_t)r * stride;
    row.n = nv < stride ? nv : stride;
  }
  row.nv = nv;

  // count valid elements (and cache the keys when the row fits in LDS)
  const bool cached = row.n <= kSelCap;
  int valid_local = 0;
  for (int64_t i = threadIdx.x; i < row.n; i += kSelThreads) {
    const uint32_t k = row.key_mem(i);
    if (cached) s_keys[i] = k;
    valid_local += (k != 0u);
  }
  int valid;
  block_excl_scan(valid_local, s_wave, &valid);   // also a barrier for s_keys
  if (cached) row.cache = s_keys;

  for (int target = 0; target < 2; ++target) {
    const int k = target == 0 ? k1 : k2;
    int32_t* out = (target == 0 ? out1 : out2);
    if (out == nullptr || k <= 0) continue;
    out += (int64_t)r * k;
    const int k_eff = k < valid ? k : valid;
    uint32_t T = 0xFFFFFFFFu;
    int take = 0;
    if (k_eff > 0) find_kth(row, k_eff, valid, s_hist, s_wave, s_res, &T, &take);
    emit(row, T, take, k_eff, k, out, s_wave);
    __syncthreads();
  }
}

hipError_t launch_select(int layout, const float* scores, int64_t stride, const int32_t* pool_blocks,
                         int64_t n_pool, const int32_t* n_visible, int R, int k1, int32_t* out1, int k2,
                         int32_t* out2, hipStream_t stream) {
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)R), dim3(kSelThreads), 0, stream, layout, scores, stride,
                     pool_blocks, n_pool, n_visible, k1, out1, k2, out2);
  return hipGetLastError();
}

}  // namespace csa2
