// The fused prefill selection: the Full layer's pool and top-k for many queries
// per sequence without storing every query's block maxima.
//
// DeepSeek-V4.1-Flash, fupanwang.com article, section 三个方向一起压小缓存 and the
// figure caption on the hierarchical sparse indexer: the pool is the 2048 blocks
// of 8 positions with the largest block maxima, and the step reads the 512 best
// positions of the pool; the selection rule is the same for a chunk of prefill
// queries as for one decode query.  The result equals ranking all blocks: by
// (block max desc, id asc) for the pool, by (score desc, position asc) for the
// top-k, which lies in the pool's first kb = min(k, n_pool) blocks.
//
// Pass 1 (the prefill scan) stores, per query row and sub-chunk of 16 blocks,
// the sub-chunk's four largest block keys.  For a threshold T these bound the
// number of blocks reaching T from both sides: a sub-chunk whose fourth key is
// below T has exactly as many blocks >= T as it has stored keys >= T; one whose
// fourth key reaches T has at least four and at most 16.  T_pool, the n_pool-th
// largest stored key, thus has at least n_pool blocks at or above it, so every
// pool block does; likewise T_kb (the kb-th) for the first kb blocks.  In each
// of two lists (the pool list for T_pool, the kb list for T_kb) a sub-chunk
// gets 16 slots when its fourth key reaches the list's threshold, else exactly
// as many as its blocks at or above it, at offsets in sub-chunk order: the
// lists are in block order.
//
// Pass 2 (the prefill scan again) writes, in block order inside its key loop,
// every block >= T_pool into the pool list (block max and id) and every block
// >= T_kb into the kb list with its eight position scores.  The final kernel
// ranks the pool list for the pool and, beside it, the kb list for the first
// kb blocks and then their eight positions each for the top-k.  Lists longer
// than the register selection holds (many equal keys) are ranked by the memory
// path first.
#include "device_common.h"
#include "kernels.h"
#include "select_core.h"

namespace csa2 {

constexpr int kPfFinalMaxKb = 2048;

// Grid R, 1024 threads.  Thresholds from the row's 4*nsub stored keys, then
// each sub-chunk's slot count in either list and the exclusive prefix in
// sub-chunk order (thread t takes sub-chunks 4t .. 4t+3).
// (two workgroups per compute unit: one's barriers overlap the other's work)
template <int J>
__global__ __launch_bounds__(kSelThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void pf_thresholds_kernel(
    PfFused f, int n_pool, int kb) {
  __shared__ RegShared sh;
  __shared__ int wtot[2][kSelWaves];
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t n = 4 * f.nsub;
  const int Jp = (int)((n + kSelThreads - 1) / kSelThreads);
  const uint32_t* row = f.summ + (int64_t)r * n;
  uint32_t key[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t i = (int64_t)(w * Jp + j) * 64 + lane;
    key[j] = (j < Jp && i < n) ? row[i] : 0u;
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
  select_thresholds(sh.c, sh.s, key, Jp, valid, kmin, kmax, n_pool, kb, 0, th0, th1);
  // T = 1 when the row stores at most that many keys: every visible block
  const uint32_t Tp = th0.T;
  const uint32_t Tk = kb > 0 ? th1.T : 0xFFFFFFFFu;

  const u32x4_t* srow = reinterpret_cast<const u32x4_t*>(row);
  uint32_t ap[4], ak[4];
  int sp = 0, sk = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t c = 4 * (int64_t)tid + e;
    ap[e] = 0u;
    ak[e] = 0u;
    if (c < f.nsub) {
      const u32x4_t x = srow[c];
      ap[e] = x[3] >= Tp ? (uint32_t)kPfSubBlocks
                         : (uint32_t)(x[0] >= Tp) + (uint32_t)(x[1] >= Tp) + (uint32_t)(x[2] >= Tp);
      ak[e] = x[3] >= Tk ? (uint32_t)kPfSubBlocks
                         : (uint32_t)(x[0] >= Tk) + (uint32_t)(x[1] >= Tk) + (uint32_t)(x[2] >= Tk);
    }
    sp += (int)ap[e];
    sk += (int)ak[e];
  }
  const int ip = wave_incl_scan(sp), ik = wave_incl_scan(sk);
  if (lane == 63) {
    wtot[0][w] = ip;
    wtot[1][w] = ik;
  }
  __syncthreads();
  int bp = 0, bk = 0, tp = 0, tk = 0;
#pragma unroll
  for (int v = 0; v < kSelWaves; ++v) {
    const int x = wtot[0][v], y = wtot[1][v];
    bp += v < w ? x : 0;
    bk += v < w ? y : 0;
    tp += x;
    tk += y;
  }
  uint32_t basep = (uint32_t)(bp + ip - sp), basek = (uint32_t)(bk + ik - sk);
  uint32_t* offp = f.offp + (int64_t)r * f.nsub;
  uint32_t* offk = f.offk + (int64_t)r * f.nsub;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t c = 4 * (int64_t)tid + e;
    if (c < f.nsub) {
      offp[c] = basep;
      offk[c] = basek;
    }
    basep += ap[e];
    basek += ak[e];
  }
  if (tid == 0)
    *reinterpret_cast<u32x4_t*>(f.thr + 4 * (int64_t)r) = u32x4_t{Tp, Tk, (uint32_t)tp, (uint32_t)tk};
}

hipError_t launch_prefill_thresholds(const PfFused& f, int R, int n_pool, int kb, hipStream_t stream) {
  const int64_t n = 4 * f.nsub;
  if (n > kPfSummaryCap) return hipErrorNotSupported;
  const dim3 grid((unsigned)R), block(kSelThreads);
  if (n <= 4096)
    hipLaunchKernelGGL((pf_thresholds_kernel<4>), grid, block, 0, stream, f, n_pool, kb);
  else if (n <= 8192)
    hipLaunchKernelGGL((pf_thresholds_kernel<8>), grid, block, 0, stream, f, n_pool, kb);
  else if (n <= 12288)
    hipLaunchKernelGGL((pf_thresholds_kernel<12>), grid, block, 0, stream, f, n_pool, kb);
  else
    hipLaunchKernelGGL((pf_thresholds_kernel<16>), grid, block, 0, stream, f, n_pool, kb);
  return hipGetLastError();
}

struct PfFinalShared {
  RegShared rs;
  int32_t slots[kPfFinalMaxKb];
};

// The top-k over the eight positions of each listed block (slots ascending):
// item i is position t = i % 8 of the block in slot slots[i / 8].  Positions
// past n_lim and keys below floor are left out.
template <int JT>
__device__ __forceinline__ void pf_topk_from_slots(Core& c, Small& s, const int32_t* slots, int kb,
                                                   const int32_t* __restrict__ ids,
                                                   const float* __restrict__ sc, int64_t n_lim, uint32_t floor,
                                                   int k, int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int cap = 8 * kb;
  const int Jp = (cap + kSelThreads - 1) / kSelThreads;
  int32_t slot[JT];
#pragma unroll
  for (int j = 0; j < JT; ++j) {
    const int i = (w * Jp + j) * 64 + lane;
    slot[j] = (j < Jp && i < cap) ? slots[i >> 3] : -1;
  }
  int32_t pos[JT];
  float x[JT];
#pragma unroll
  for (int j = 0; j < JT; ++j) {
    const int i = (w * Jp + j) * 64 + lane;
    const int32_t b = slot[j] >= 0 ? ids[slot[j]] : -1;
    x[j] = slot[j] >= 0 ? sc[8 * (int64_t)slot[j] + (i & 7)] : 0.0f;
    const int64_t p = 8 * (int64_t)b + (i & 7);
    pos[j] = (b >= 0 && p < n_lim) ? (int32_t)p : -1;
  }
  uint32_t key[JT];
#pragma unroll
  for (int j = 0; j < JT; ++j) {
    const uint32_t kk = order_key(x[j]);
    key[j] = (pos[j] >= 0 && kk >= floor) ? kk : 0u;
  }
  hist_zero(c);
  if (threadIdx.x == 0) {
    s.cnt[0] = 0;
    s.cnt[1] = 0;
  }
  int valid;
  uint32_t kmin, kmax;
  key_range(s, key, Jp, valid, kmin, kmax);
  Thr th0, th1;
  select_thresholds(c, s, key, Jp, valid, kmin, kmax, k, 0, 0, th0, th1);
  emit_sel(
      s, key, Jp, th0, th1, [&](int, int p, int j, int) { out[p] = pos[j]; }, [&](int, int p) { out[p] = -1; });
}

// One list of row r ranked in registers (length U <= 1024*J) for one target:
// K items written to out (ids, or list slots when SLOTS), ascending, -1 padded.
// floor_out (may be null): the K-th key when the list holds more than K items.
template <int J, bool SLOTS>
__device__ __forceinline__ void pf_rank_list(RegShared& sh, const float* __restrict__ kv,
                                             const int32_t* __restrict__ ids, int64_t U, int K, int32_t* out,
                                             uint32_t* floor_out) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int Jp = (int)((U + kSelThreads - 1) / kSelThreads);
  int32_t id[J];
  uint32_t key[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t i = (int64_t)(w * Jp + j) * 64 + lane;
    id[j] = (j < Jp && i < U) ? ids[i] : -1;
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t i = (int64_t)(w * Jp + j) * 64 + lane;
    const float x = id[j] >= 0 ? kv[i] : 0.0f;
    key[j] = id[j] >= 0 ? order_key(x) : 0u;
  }
  hist_zero(sh.c);
  if (threadIdx.x == 0) {
    sh.s.cnt[0] = 0;
    sh.s.cnt[1] = 0;
  }
  int valid;
  uint32_t kmin, kmax;
  key_range(sh.s, key, Jp, valid, kmin, kmax);
  Thr th0, th1;
  select_thresholds(sh.c, sh.s, key, Jp, valid, kmin, kmax, K, 0, 0, th0, th1);
  emit_sel(
      sh.s, key, Jp, th0, th1, [&](int, int p, int j, int i) { out[p] = SLOTS ? i : id[j]; },
      [&](int, int p) { out[p] = -1; });
  if (floor_out) *floor_out = (th0.keff == K && valid > K) ? th0.T : 1u;
}

// Grid 2R, 1024 threads.  Workgroup r: row r's first kb blocks from its kb
// list, then its top-k over their positions (what the attention waits for);
// workgroup R + r: row r's pool from its pool list.  Lists longer than the
// registers hold were ranked by the memory path (pool written, slots left).
template <int J, int JT>
__global__ __launch_bounds__(kSelThreads) __attribute__((amdgpu_waves_per_eu(JT <= 4 ? 8 : 4, JT <= 4 ? 8 : 4))) void
pf_final_kernel(PfFused f, const int32_t* __restrict__ n_visible, int64_t N_max, int n_pool,
                int32_t* __restrict__ pool_out, int kb, int k, int32_t* __restrict__ idx) {
  __shared__ PfFinalShared sh;
  __shared__ uint32_t floor_sh;
  const int R = (int)(gridDim.x >> 1);
  const int tid = threadIdx.x;
  if ((int)blockIdx.x >= R) {
    const int r = (int)blockIdx.x - R;
    const int64_t U = f.thr[4 * (int64_t)r + 2];
    if (U > kPfListRegCap) return;
    pf_rank_list<J, false>(sh.rs, f.pool_key + (int64_t)r * f.cap, f.pool_id + (int64_t)r * f.cap, U, n_pool,
                           pool_out + (int64_t)r * n_pool, nullptr);
    return;
  }
  if (k <= 0) return;
  const int r = blockIdx.x;
  const int64_t U = f.thr[4 * (int64_t)r + 3];
  const int32_t* kid = f.kb_id + (int64_t)r * f.cap;
  uint32_t floor = 1u;
  if (U <= kPfListRegCap) {
    pf_rank_list<J, true>(sh.rs, f.kb_key + (int64_t)r * f.cap, kid, U, kb, sh.slots, &floor_sh);
    __syncthreads();
    // the kb-th block key bounds the k-th position score from below when kb = k
    if (kb == k) floor = floor_sh;
  } else {
    for (int p = tid; p < kb; p += kSelThreads) sh.slots[p] = f.kbslot[(int64_t)r * kb + p];
    __syncthreads();
  }
  int64_t nv = n_visible[r];
  nv = nv < 0 ? 0 : (nv < N_max ? nv : N_max);
  pf_topk_from_slots<JT>(sh.rs.c, sh.rs.s, sh.slots, kb, kid, f.kb_sc + (int64_t)r * f.cap * 8, nv, floor, k,
                         idx + (int64_t)r * k);
}

hipError_t launch_prefill_final(const PfFused& f, const int32_t* n_visible, int64_t N_max, int R, int n_pool,
                                int32_t* pool_out, int kb, int k, int32_t* idx, hipStream_t stream) {
  if (kb > kPfFinalMaxKb || kb > n_pool) return hipErrorNotSupported;
  const dim3 grid(2u * (unsigned)R), block(kSelThreads);
  constexpr int J = kPfListRegCap / kSelThreads;
  if (kb <= 512)
    hipLaunchKernelGGL((pf_final_kernel<J, 4>), grid, block, 0, stream, f, n_visible, N_max, n_pool, pool_out, kb,
                       k, idx);
  else
    hipLaunchKernelGGL((pf_final_kernel<J, 16>), grid, block, 0, stream, f, n_visible, N_max, n_pool, pool_out, kb,
                       k, idx);
  return hipGetLastError();
}

}  // namespace csa2
