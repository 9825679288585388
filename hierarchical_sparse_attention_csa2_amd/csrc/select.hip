// Ranked selection: the coarse block filter (top-n_pool blocks by block max) and
// the top-k over pool or full score rows.
//
// DeepSeek-V4.1-Flash, fupanwang.com article, section 三个方向一起压小缓存 and the
// figure caption on the hierarchical sparse indexer: blocks are represented by
// their highest score, the top blocks form the candidate pool (at most 2048
// blocks), and each layer selects its top-512 positions.  Ranking is by
// (score desc, id asc): ties go to the lowest position / block id.
//
// One 1024-thread workgroup per row; every decision is exact on the IEEE
// total-order key of the fp32 score (0 = no element), and the work is
// VALU-bound on the row's one compute unit, so every pass keeps its items in
// registers and as few passes as possible touch all of them.
//   1. Load (up to 16 items a lane) with the count, minimum and maximum key.
//   2. One 4096-bin histogram of the first 12-bit digit of (key - kmin), spread
//      over the row's own key range; all 16 waves search it for the bin of the
//      K-th key of each target (up to two targets share the passes).
//   3. The members of a threshold bin (usually a handful) are copied out and
//      ranked by counting; a bin with more than 256 members (many equal keys) is
//      narrowed by further 12-bit digits first.
//   4. One counting pass and one ordered writing pass emit, per target, the ids
//      of the keys > T and of the first `take` keys == T, ids ascending.
// Rows of block maxima longer than 16,384 blocks are filtered one level up
// first: super-blocks of 8 consecutive blocks are ranked by their own maximum
// (which the indexer scan can supply), and any set of super-blocks holding the
// first K super-blocks holds every block of the first K blocks (a super-block
// ranked ahead of another contributes its best block ahead of every block of the
// other).  Level 1 keeps the super-blocks at or above the threshold bin when
// they fit (else exactly the first K), which bounds the K-th block key from
// below by that bin's lower edge T1; level 2 gathers only the blocks >= T1 of the
// kept super-blocks (a few thousand), compacts them in id order and selects
// exactly among them.  Anything longer runs a generic selection that re-reads
// the row from memory in every pass.
#include "device_common.h"
#include "kernels.h"
#include "select_core.h"
#include "score_core.h"

namespace csa2 {

constexpr int kSegIters = 20;                      // items per lane per pass
constexpr int kSegItems = 64 * kSegIters;          // 1280 items per wave
constexpr int kSelCap = kSelWaves * kSegItems;     // 20,480 keys in LDS
constexpr int kSuperCap = 8192;                    // super-block keys (level 1)
constexpr int kLevelCap = kSelCap / 8;             // super-blocks kept by level 1 (2560)
constexpr int kMemberCap = 2048;                   // members of a threshold bin kept in LDS

struct SelShared {
  uint32_t hist[kBins];
  union {
    uint32_t keys[kSelCap];
    uint32_t skeys[kSuperCap];
  } u;
  int32_t sbsel[kLevelCap];
  uint32_t members[2][kMemberCap];
  int wave_i[4][kSelWaves];
  uint32_t wave_u[2][kSelWaves];
  int res[8];
};

// ---------------------------------------------------------------------------
// row view (memory) and the LDS working set
// ---------------------------------------------------------------------------
struct RowView {
  int layout;
  const float* s;          // row base
  const int32_t* pb;       // pool layout: this row's pool block ids
  int64_t n;               // elements in the row
  int64_t nv;              // visible positions
  __device__ __forceinline__ uint32_t key_mem(int64_t i) const {
    if (layout == kSelPool) {
      const int64_t blk = pb[i >> 3];
      const int64_t p = 8 * blk + (i & 7);
      if (blk < 0 || p >= nv) return 0u;
    }
    return order_key(s[i]);
  }
  __device__ __forceinline__ int32_t id_mem(int64_t i) const {
    if (layout == kSelPool) return (int32_t)(8 * (int64_t)pb[i >> 3] + (i & 7));
    return (int32_t)i;
  }
};

enum { kSrcKeys = 0, kSrcSuper = 1, kSrcMem = 2, kSrcMembers0 = 3, kSrcMembers1 = 4 };
enum { kIdRow = 0, kIdSuperList = 1, kIdIndex = 2 };

template <int SRC>
__device__ __forceinline__ uint32_t src_key(SelShared& sh, const RowView row, int64_t i) {
  if constexpr (SRC == kSrcKeys) return sh.u.keys[i];
  else if constexpr (SRC == kSrcSuper) return sh.u.skeys[i];
  else if constexpr (SRC == kSrcMembers0) return sh.members[0][i];
  else if constexpr (SRC == kSrcMembers1) return sh.members[1][i];
  else return row.key_mem(i);
}

// ids: through the row view, through the kept super-block list (item j is
// block 8*sbsel[j/8] + j%8), or the item index itself
template <int ID>
__device__ __forceinline__ int32_t src_id(SelShared& sh, const RowView row, int64_t i) {
  if constexpr (ID == kIdSuperList) return 8 * sh.sbsel[i >> 3] + (int32_t)(i & 7);
  else if constexpr (ID == kIdIndex) return (int32_t)i;
  else return row.id_mem(i);
}

// Per-lane running (min, max, count) of non-zero keys, folded over the workgroup
// into res[0] = count, res[1] = kmin, res[2] = kmax.
struct KeyStats {
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  int cnt = 0;
  __device__ __forceinline__ void add(uint32_t k) {
    if (k != 0u) {
      mn = k < mn ? k : mn;
      mx = k > mx ? k : mx;
      ++cnt;
    }
  }
};

__device__ __forceinline__ void reduce_stats(SelShared& sh, KeyStats st) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t mn = wave_min_u32(st.mn), mx = wave_max_u32(st.mx);
  const int cnt = wave_sum(st.cnt);
  if (lane == 0) {
    sh.wave_i[0][w] = cnt;
    sh.wave_u[0][w] = mn;
    sh.wave_u[1][w] = mx;
  }
  __syncthreads();
  if (w == 0) {
    const int c = lane < kSelWaves ? sh.wave_i[0][lane] : 0;
    const uint32_t a = lane < kSelWaves ? sh.wave_u[0][lane] : 0xFFFFFFFFu;
    const uint32_t b = lane < kSelWaves ? sh.wave_u[1][lane] : 0u;
    const int tc = wave_sum(c);
    const uint32_t ta = wave_min_u32(a), tb = wave_max_u32(b);
    if (lane == 0) {
      sh.res[0] = tc;
      sh.res[1] = (int)ta;
      sh.res[2] = (int)tb;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// histograms and the threshold bin
// ---------------------------------------------------------------------------
// Histogram of ((key - kmin) >> shift) & (2^bits - 1) over the non-zero keys
// whose ((key - kmin) >> pshift) equals prefix (pshift >= 32: all of them).
// Clears first; ends synchronised.
template <int SRC>
__device__ __forceinline__ void build_hist(SelShared& sh, const RowView row, int64_t n, uint32_t kmin, int shift,
                                           int bits, int pshift, uint32_t prefix) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t dmask = (1u << bits) - 1u;
  __syncthreads();
  for (int i = threadIdx.x; i < kBins; i += kSelThreads) sh.hist[i] = 0;
  __syncthreads();
  for (int64_t base = 0; base < n; base += kSelCap) {
    const int64_t seg = base + (int64_t)w * kSegItems + lane;
#pragma unroll 10
    for (int j = 0; j < kSegIters; ++j) {
      const int64_t i = seg + 64 * j;
      const uint32_t k = i < n ? src_key<SRC>(sh, row, i) : 0u;
      const uint32_t d = k - kmin;
      if (k != 0u && (pshift >= 32 || (d >> pshift) == prefix)) atomicAdd(&sh.hist[(d >> shift) & dmask], 1u);
    }
  }
  __syncthreads();
}

// One wave finds the bin b with (#keys in bins > b) < need <= (#keys in bins
// >= b), 1 <= need <= #keys: res[4] = b, res[5] = count above b.  Ends
// synchronised.
__device__ __forceinline__ void find_bin(SelShared& sh, int need) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (w == 0) {
    // lane l owns bins [4032-64l, 4096-64l): descending order = lane order
    const int lo = kBins - 64 * (lane + 1);
    int sum = 0;
#pragma unroll 16
    for (int t = 0; t < 64; ++t) sum += (int)sh.hist[lo + ((t + lane) & 63)];   // rotated: no bank conflicts
    const int incl = wave_incl_scan(sum);
    const int excl = incl - sum;
    const unsigned long long hit = __ballot(excl < need && need <= incl);
    const int L = hit ? (int)__builtin_ctzll(hit) : 0;
    const int before = __builtin_amdgcn_readlane(excl, L);
    // the 64 bins of lane L, descending: lane t takes bin (4095 - 64L - t)
    const int b = kBins - 1 - 64 * L - lane;
    const int c = (int)sh.hist[b];
    const int incl2 = wave_incl_scan(c) + before;
    const unsigned long long hit2 = __ballot(incl2 >= need);
    const int L2 = hit2 ? (int)__builtin_ctzll(hit2) : 0;
    if (lane == L2) {
      sh.res[4] = b;
      sh.res[5] = incl2 - c;
    }
  }
  __syncthreads();
}

struct Threshold {
  uint32_t T;     // the k-th key (1 = every non-zero key; 0xFFFFFFFF = none)
  int take;       // keys equal to T that are taken
};

// Remaining `cur` low bits of the k-th key among keys whose (key - kmin) >> cur
// equals `prefix`, need-th largest of them, 12 bits a pass.
template <int SRC>
__device__ __forceinline__ Threshold refine(SelShared& sh, const RowView row, int64_t n, uint32_t kmin, int cur,
                                            uint32_t prefix, int need) {
  while (cur > 0) {
    const int next = cur > 12 ? cur - 12 : 0;
    build_hist<SRC>(sh, row, n, kmin, next, cur - next, cur, prefix);
    find_bin(sh, need);
    need -= sh.res[5];
    prefix = (prefix << (cur - next)) | (uint32_t)sh.res[4];
    cur = next;
    __syncthreads();
  }
  return Threshold{kmin + prefix, need};
}

// Copy the non-zero keys whose first digit equals bin[t] into members[t] (no
// order), for both targets at once.  Counts in res[6], res[7].
template <int SRC>
__device__ __forceinline__ void collect_members(SelShared& sh, const RowView row, int64_t n, uint32_t kmin, int s1,
                                                const uint32_t* bin, const bool* want) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x == 0) {
    sh.res[6] = 0;
    sh.res[7] = 0;
  }
  __syncthreads();
  const int w = threadIdx.x >> 6;
  const unsigned long long lt = lanemask_lt();
  for (int64_t base = 0; base < n; base += kSelCap) {
    const int64_t seg = base + (int64_t)w * kSegItems + lane;
#pragma unroll 4
    for (int j = 0; j < kSegIters; ++j) {
      const int64_t i = seg + 64 * j;
      const uint32_t k = i < n ? src_key<SRC>(sh, row, i) : 0u;
      const uint32_t dg = (k - kmin) >> s1;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bool in = want[t] && k != 0u && dg == bin[t];
        const unsigned long long m = __ballot(in);
        if (m) {
          int basepos = 0;
          if (lane == 0) basepos = atomicAdd(&sh.res[6 + t], __popcll(m));
          basepos = __builtin_amdgcn_readfirstlane(basepos);
          const int p = basepos + __popcll(m & lt);
          if (in && p < kMemberCap) sh.members[t][p] = k;
        }
      }
    }
  }
  __syncthreads();
}

// One ordered pass writing both targets: ids of keys > T[t] and of the first
// take[t] keys == T[t], ascending, then -1 padding up to k[t].  Target 0 may go
// to LDS (sbsel) when OUT0_LDS.
template <int SRC, int ID, bool OUT0_LDS>
__device__ __forceinline__ void emit2(SelShared& sh, const RowView row, int64_t n, const Threshold* th,
                                      const int* keff, const int* ks, int32_t* out0, int32_t* out1) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const unsigned long long lt = lanemask_lt();
  int carry_tie[2] = {0, 0}, carry_sel[2] = {0, 0};
  const bool act0 = keff[0] > 0, act1 = keff[1] > 0;
  for (int64_t base = 0; base < n && (act0 || act1); base += kSelCap) {
    const int64_t seg = base + (int64_t)w * kSegItems + lane;
    int ngt[2] = {0, 0}, ntie[2] = {0, 0};
#pragma unroll 4
    for (int j = 0; j < kSegIters; ++j) {
      const int64_t i = seg + 64 * j;
      const uint32_t k = i < n ? src_key<SRC>(sh, row, i) : 0u;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        ngt[t] += __popcll(__ballot(k > th[t].T));
        ntie[t] += __popcll(__ballot(k == th[t].T));
      }
    }
    if (lane == 0) {
      sh.wave_i[0][w] = ngt[0];
      sh.wave_i[1][w] = ntie[0];
      sh.wave_i[2][w] = ngt[1];
      sh.wave_i[3][w] = ntie[1];
    }
    __syncthreads();
    int tie_rank[2], pos[2], tot_tie[2], tot_sel[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      int tb = carry_tie[t], sb = carry_sel[t], tt = 0, ts = 0;
      for (int v = 0; v < kSelWaves; ++v) {
        const int g = sh.wave_i[2 * t][v], c = sh.wave_i[2 * t + 1][v];
        int taken = th[t].take - (carry_tie[t] + tt);
        taken = taken < 0 ? 0 : (taken > c ? c : taken);
        if (v < w) {
          tb += c;
          sb += g + taken;
        }
        tt += c;
        ts += g + taken;
      }
      tie_rank[t] = tb;
      pos[t] = sb;
      tot_tie[t] = tt;
      tot_sel[t] = ts;
    }
    __syncthreads();
#pragma unroll 4
    for (int j = 0; j < kSegIters; ++j) {
      const int64_t i = seg + 64 * j;
      const uint32_t k = i < n ? src_key<SRC>(sh, row, i) : 0u;
      int32_t id = 0;
      bool have_id = false;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bool tie = k == th[t].T;
        const unsigned long long mt = __ballot(tie);
        const bool sel = k > th[t].T || (tie && tie_rank[t] + __popcll(mt & lt) < th[t].take);
        const unsigned long long ms = __ballot(sel);
        if (sel) {
          const int p = pos[t] + __popcll(ms & lt);
          if (p < keff[t]) {
            if (!have_id) {
              id = src_id<ID>(sh, row, i);
              have_id = true;
            }
            if (t == 0) {
              if constexpr (OUT0_LDS) sh.sbsel[p] = id;
              else out0[p] = id;
            } else {
              out1[p] = id;
            }
          }
        }
        tie_rank[t] += __popcll(mt);
        pos[t] += __popcll(ms);
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      carry_tie[t] += tot_tie[t];
      carry_sel[t] += tot_sel[t];
    }
    if ((!act0 || carry_sel[0] >= keff[0]) && (!act1 || carry_sel[1] >= keff[1])) break;
  }
  for (int i = keff[0] + threadIdx.x; i < ks[0]; i += kSelThreads) {
    if constexpr (OUT0_LDS) sh.sbsel[i] = -1;
    else out0[i] = -1;
  }
  for (int i = keff[1] + threadIdx.x; i < ks[1]; i += kSelThreads) out1[i] = -1;
}

// Exact selection of up to two targets (ks[t], outs) from the working set,
// whose key statistics are in res[0..2].  APPROX0: target 0 may instead keep
// every key of its threshold bin and above when that set has at most `cap0`
// keys (res[6] receives how many target 0 kept).
template <int SRC, int ID, bool OUT0_LDS, bool APPROX0>
__device__ __forceinline__ void select_targets(SelShared& sh, const RowView row, int64_t n, int k0, int32_t* out0,
                                               int k1, int32_t* out1, int cap0 = 0) {
  const int valid = sh.res[0];
  const uint32_t kmin = (uint32_t)sh.res[1];
  const uint32_t span = valid > 0 ? (uint32_t)sh.res[2] - kmin : 0u;
  const int span_bits = span ? 32 - __builtin_clz(span) : 0;
  const int s1 = span_bits > 12 ? span_bits - 12 : 0;
  int ks[2] = {k0, k1}, keff[2];
  bool need_thr[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    keff[t] = ks[t] > 0 ? (ks[t] < valid ? ks[t] : valid) : 0;
    need_thr[t] = keff[t] > 0 && keff[t] < valid;
  }
  Threshold th[2] = {{0xFFFFFFFFu, 0}, {0xFFFFFFFFu, 0}};
#pragma unroll
  for (int t = 0; t < 2; ++t)
    if (keff[t] > 0 && !need_thr[t]) th[t] = Threshold{1u, 0x7FFFFFFF};
  if (need_thr[0] || need_thr[1]) {
    build_hist<SRC>(sh, row, n, kmin, s1, 12, 32, 0u);
    uint32_t bin[2] = {0u, 0u};
    int above[2] = {0, 0};
    int inbin[2] = {0, 0};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (!need_thr[t]) continue;
      find_bin(sh, keff[t]);
      bin[t] = (uint32_t)sh.res[4];
      above[t] = sh.res[5];
      inbin[t] = (int)sh.hist[bin[t]];
      __syncthreads();
    }
    bool done0 = false;
    if (APPROX0 && need_thr[0] && above[0] + inbin[0] <= cap0) {
      // keep the whole threshold bin: every key whose first digit >= bin
      th[0] = Threshold{kmin + (bin[0] << s1), 0x7FFFFFFF};
      keff[0] = above[0] + inbin[0];
      done0 = true;
    }
    bool want[2] = {need_thr[0] && !done0 && s1 > 0 && inbin[0] <= kMemberCap,
                    need_thr[1] && s1 > 0 && inbin[1] <= kMemberCap};
    if (want[0] || want[1]) collect_members<SRC>(sh, row, n, kmin, s1, bin, want);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (!need_thr[t] || (t == 0 && done0)) continue;
      const int need = keff[t] - above[t];
      if (s1 == 0) {
        th[t] = Threshold{kmin + bin[t], need};
      } else if (want[t]) {
        const int m = t == 0 ? sh.res[6] : sh.res[7];
        if (t == 0) th[t] = refine<kSrcMembers0>(sh, row, m, kmin, s1, bin[t], need);
        else th[t] = refine<kSrcMembers1>(sh, row, m, kmin, s1, bin[t], need);
      } else {
        th[t] = refine<SRC>(sh, row, n, kmin, s1, bin[t], need);
      }
    }
    if (APPROX0 && threadIdx.x == 0) sh.res[6] = keff[0];
    __syncthreads();
  } else if (APPROX0) {
    if (threadIdx.x == 0) sh.res[6] = keff[0];
    __syncthreads();
  }
  emit2<SRC, ID, OUT0_LDS>(sh, row, n, th, keff, ks, out0, out1);
  __syncthreads();
}

// Rows of at most 1024*J items (any layout), items in registers.  The lane
// layout follows the row's capacity (stride, or 8*n_pool slots), so the loads
// are issued before n_visible arrives and masked after.
// floor_in (may be null): keys below floor_in[r] cannot be selected and are
// dropped; floor_out (may be null): the key of target 1's K1-th item, or 1 when
// the row has at most K1 items.
// Row r of the register path.  o0 / o1: this row's outputs (may be null);
// floor_out: this row's floor slot (may be null).
template <int J, int LAYOUT>
__device__ __forceinline__ void select_reg_row(RegShared& sh, int r, const float* __restrict__ scores,
                                               int64_t stride, const int32_t* __restrict__ pool_blocks,
                                               int64_t n_pool, const int32_t* __restrict__ n_visible, int K0,
                                               int32_t* o0, int K1, int32_t* o1,
                                               const uint32_t* __restrict__ floor_in, uint32_t* floor_out) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int cap = (int)(LAYOUT == kSelPool ? 8 * n_pool : stride);
  const int Jp = (cap + 1023) >> 10;
  const float* row = scores + (int64_t)r * cap;
  const int32_t* pb = LAYOUT == kSelPool ? pool_blocks + (int64_t)r * n_pool : nullptr;
  float x[J];
  int32_t pbv[LAYOUT == kSelPool ? J : 1];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    x[j] = 0.0f;
    if constexpr (LAYOUT == kSelPool) pbv[j] = -1;
    const int i = (w * Jp + j) * 64 + lane;
    if (j < Jp && i < cap) {
      x[j] = row[i];
      if constexpr (LAYOUT == kSelPool) pbv[j] = pb[i >> 3];
    }
  }
  int64_t nv = n_visible[r];
  nv = nv < 0 ? 0 : nv;
  int64_t n = cap;
  if (LAYOUT == kSelBlocks) n = (nv + 7) >> 3;
  if (LAYOUT == kSelFull) n = nv;
  n = n < cap ? n : cap;
  const uint32_t fl = floor_in ? floor_in[r] : 1u;
  uint32_t k[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = (w * Jp + j) * 64 + lane;
    bool ok = j < Jp && i < n;
    if constexpr (LAYOUT == kSelPool) ok = ok && pbv[j] >= 0 && 8 * (int64_t)pbv[j] + (i & 7) < nv;
    const uint32_t key = order_key(x[j]);
    k[j] = ok && key >= fl ? key : 0u;
  }
  if (!o0) K0 = 0;
  if (!o1) K1 = 0;
  hist_zero(sh.c);
  if (threadIdx.x == 0) {
    sh.s.cnt[0] = 0;
    sh.s.cnt[1] = 0;
  }
  int valid;
  uint32_t kmin, kmax;
  key_range(sh.s, k, Jp, valid, kmin, kmax);
  Thr th0, th1;
  select_thresholds(sh.c, sh.s, k, Jp, valid, kmin, kmax, K0, K1, 0, th0, th1);
  if (floor_out && threadIdx.x == 0) *floor_out = (K1 > 0 && th1.keff == K1 && valid > K1) ? th1.T : 1u;
  emit_sel(
      sh.s, k, Jp, th0, th1,
      [&](int t, int pos, int j, int i) {
        int32_t id = i;
        if constexpr (LAYOUT == kSelPool) id = 8 * pbv[j] + (i & 7);
        (t ? o1 : o0)[pos] = id;
      },
      [&](int t, int p) { (t ? o1 : o0)[p] = -1; });
}

template <int J, int LAYOUT>
__global__ __launch_bounds__(kSelThreads) void select_reg_kernel(const float* __restrict__ scores, int64_t stride,
                                                                 const int32_t* __restrict__ pool_blocks,
                                                                 int64_t n_pool,
                                                                 const int32_t* __restrict__ n_visible, int K0,
                                                                 int32_t* __restrict__ out0, int K1,
                                                                 int32_t* __restrict__ out1,
                                                                 const uint32_t* __restrict__ floor_in,
                                                                 uint32_t* __restrict__ floor_out) {
  __shared__ RegShared sh;
  const int r = blockIdx.x;
  select_reg_row<J, LAYOUT>(sh, r, scores, stride, pool_blocks, n_pool, n_visible, K0,
                            out0 ? out0 + (int64_t)r * K0 : nullptr, K1, out1 ? out1 + (int64_t)r * K1 : nullptr,
                            floor_in, floor_out ? floor_out + r : nullptr);
}

// Block rows of up to 65,536 blocks, targets of at most 2048 blocks.
// Level 1 ranks super-blocks (8 consecutive blocks) by their maximum and keeps
// those at or above the threshold bin of the K-th (or exactly the first K);
// every block of the first K blocks lies in them and scores at least that
// threshold T1.  Level 2 selects exactly among the blocks >= T1 of the kept
// super-blocks.
//
// Thread t owns super-blocks 8t..8t+7 at level 1; the kept super-blocks are
// listed in id order with one workgroup prefix sum.  The gather then reads each
// kept super-block's 8 block maxima as two 16-byte halves, six halves per
// thread, in one of two layouts:
//  - runs (kPairs false): thread t takes kept super-blocks [G t, G t + G),
//    G = ceil(nkept / 1024) <= 3, so its survivors are contiguous in id order
//    and one prefix sum places them;
//  - pairs (kPairs true): in pass p, lanes 2i and 2i+1 take the two halves of
//    kept super-block 512p + i, so a load instruction covers 32 consecutive
//    entries of the kept list, one run of rows when most super-blocks are kept
//    (a prefill row: three quarters pass level 1) instead of 64 lines; id order
//    is then (pass, thread, element) order, placed by per-pass prefix sums.
// The stand-alone filter takes pairs; the fused decode selection keeps runs
// (its top-k side keeps a few percent of a long row's super-blocks, far apart,
// where pairs gain nothing and their extra placement work cost 0.4 us a row).
// The blocks >= T1 (the survivors) are written to LDS in id order and counted
// into level 2's histogram on the way.
constexpr int kB3Items = 8;                          // super-blocks per thread at level 1
constexpr int kB3Pass = 2 * kKeepCap / kSelThreads;  // half super-blocks gathered per thread (6)
static_assert(kB3Pass * kSelThreads / 2 == kKeepCap, "gather passes cover the kept-list capacity");
static_assert(kB3Pass == 6, "three packed prefix sums of two passes each");

struct Blocks3Shared {
  int32_t cids[kCompCap];       // survivors' block ids, id order
  uint32_t ckeys[kCompCap];     // survivors' keys, id order
  Core c;
  int32_t sbsel[kKeepCap];      // kept super-blocks, id order
  int wsum[4][kSelWaves];       // per-wave totals of the prefix sums
  Small s;
  uint32_t floor;               // the fused top-k's floor
};

// Exclusive prefix sum of x over the workgroup in thread order, and the total.
// buf: 16 ints that no other thread reads or writes between the barrier before
// this call and the one inside it.
__device__ __forceinline__ int block_excl_scan(int* buf, int x, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_incl_scan(x);
  if (lane == 63) buf[w] = incl;
  __syncthreads();
  const int wt = lane < kSelWaves ? buf[lane] : 0;
  const int wi = row_incl_scan(wt);
  total = __builtin_amdgcn_readlane(wi, kSelWaves - 1);
  return __builtin_amdgcn_readlane(wi, w) - __builtin_amdgcn_readlane(wt, w) + incl - x;
}

// Exclusive prefix sums of three values over the workgroup in thread order,
// and their totals, with one barrier.  buf: 3 x 16 ints, as block_excl_scan's.
__device__ __forceinline__ void block_excl_scan3(int (*buf)[kSelWaves], const int (&x)[3], int (&excl)[3],
                                                 int (&total)[3]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) incl[i] = wave_incl_scan(x[i]);
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < 3; ++i) buf[i][w] = incl[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int wt = lane < kSelWaves ? buf[i][lane] : 0;
    const int wi = row_incl_scan(wt);
    total[i] = __builtin_amdgcn_readlane(wi, kSelWaves - 1);
    excl[i] = __builtin_amdgcn_readlane(wi, w) - __builtin_amdgcn_readlane(wt, w) + incl[i] - x[i];
  }
}

// Level 2 of the block filter: exact selection among the m2 <= 1024*J
// survivors in sh.ckeys / sh.cids (id order), whose first-digit histogram over
// [T1, kmax1] is already counted.
template <int J>
__device__ __forceinline__ void blocks_level2(Blocks3Shared& sh, int m2, uint32_t T1, uint32_t kmax1, int K0,
                                              int32_t* o0, int K1, int32_t* o1, uint32_t* floor_out) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int Jp2 = (m2 + 1023) >> 10;
  uint32_t k2[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = (w * Jp2 + j) * 64 + lane;
    k2[j] = (j < Jp2 && i < m2) ? sh.ckeys[i] : 0u;
  }
  Thr th0, th1;
  select_thresholds(sh.c, sh.s, k2, Jp2, m2, T1, kmax1, K0, K1, 0, th0, th1, true);
  // the K1-th block of the whole row is the K1-th survivor (every block of the
  // first K1 survives level 1)
  if (floor_out && threadIdx.x == 0) *floor_out = (K1 > 0 && th1.keff == K1 && m2 > K1) ? th1.T : 1u;
  emit_sel(
      sh.s, k2, Jp2, th0, th1, [&](int tg, int pos, int j, int i) { (tg ? o1 : o0)[pos] = sh.cids[i]; },
      [&](int tg, int p) { (tg ? o1 : o0)[p] = -1; });
}

// kVec: super_max rows 16-byte aligned and block rows 32-byte aligned, so a
// thread's 8 super maxima and a super-block's 8 block maxima are two 16-byte
// loads each.
// Row r of the two-level block filter.  o0 / o1: this row's outputs (may be
// null); floor_out: this row's floor slot (may be null).
template <bool kHaveSuper, bool kVec, bool kPairs>
__device__ __forceinline__ void select_blocks3_row(Blocks3Shared& sh, int r, const float* __restrict__ bmax,
                                                   int64_t stride, const float* __restrict__ super_max,
                                                   int64_t nsup_stride, const int32_t* __restrict__ n_visible,
                                                   int K0, int32_t* o0, int K1, int32_t* o1, uint32_t* floor_out) {
  const int t = threadIdx.x;
  const float* row = bmax + (int64_t)r * stride;
  const int nsup_cap = (int)((stride + 7) >> 3);   // <= 8192
  if (!o0) K0 = 0;
  if (!o1) K1 = 0;
  const int kmaxK = K0 > K1 ? K0 : K1;
  if (kmaxK == 0) {
    if (floor_out && t == 0) *floor_out = 1u;
    return;
  }

  // level 1: super-blocks 8t..8t+7 (the scan's maxima are read ahead of n_visible)
  float sv[kB3Items];
  if constexpr (kHaveSuper && kVec) {
    // in bounds: nsup_stride is a multiple of 4 and i < nsup_cap <= nsup_stride
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = kB3Items * t + 4 * h;
      const f32x4_t v = i < nsup_cap ? *reinterpret_cast<const f32x4_t*>(super_max + (int64_t)r * nsup_stride + i)
                                     : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[4 * h + e] = v[e];
    }
  } else {
#pragma unroll
    for (int j = 0; j < kB3Items; ++j) {
      const int i = kB3Items * t + j;
      sv[j] = 0.0f;
      if (kHaveSuper && i < nsup_cap) sv[j] = super_max[(int64_t)r * nsup_stride + i];
    }
  }
  int64_t nv = n_visible[r];
  nv = nv < 0 ? 0 : nv;
  const int nblk = (int)(((nv + 7) >> 3) < stride ? ((nv + 7) >> 3) : stride);
  const int nsuper = (nblk + 7) >> 3;
  uint32_t k1[kB3Items];
#pragma unroll
  for (int j = 0; j < kB3Items; ++j) {
    const int i = kB3Items * t + j;
    uint32_t key = 0u;
    if (i < nsuper) {
      if constexpr (kHaveSuper) {
        key = order_key(sv[j]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int b = 8 * i + e;
          const uint32_t x = b < nblk ? order_key(row[b]) : 0u;
          key = x > key ? x : key;
        }
      }
    }
    k1[j] = key;
  }
  hist_zero(sh.c);
  if (t == 0) {
    sh.s.cnt[0] = 0;
    sh.s.cnt[1] = 0;
  }
  int valid1;
  uint32_t kmin1, kmax1;
  key_range(sh.s, k1, kB3Items, valid1, kmin1, kmax1);

  int approx = kKeepCap;
  uint32_t T1 = 1u;
  int nkept = 0, m2 = 0;
  uint32_t ck[kB3Pass * 4];      // survivors (>= T1) of this thread's gathered blocks, 0 elsewhere
  int cpos2[kB3Pass / 2];        // pairs: LDS positions of passes 2i, 2i+1's first survivors (16 bits each)
  int sbq[kB3Pass / 2];          // runs: this thread's kept super-blocks, -1 when none
  int cpos = 0;                  // runs: LDS position of this thread's first survivor
  for (;;) {
    Thr a0, a1;
    select_thresholds(sh.c, sh.s, k1, kB3Items, valid1, kmin1, kmax1, kmaxK, 0, approx, a0, a1);
    T1 = a0.T;
    // kept super-blocks: > T1, or == T1 within the first `take` ties (id order);
    // at most kKeepCap of them
    int tie_base = 0;
    if (a0.take != 0x7FFFFFFF) {
      int nt = 0;
#pragma unroll
      for (int j = 0; j < kB3Items; ++j) nt += (k1[j] != 0u && k1[j] == T1) ? 1 : 0;
      int unused;
      tie_base = block_excl_scan(sh.wsum[0], nt, unused);
    }
    int nk = 0;
    unsigned keep = 0u;
#pragma unroll
    for (int j = 0; j < kB3Items; ++j) {
      bool kp = k1[j] != 0u && k1[j] >= T1;
      if (a0.take != 0x7FFFFFFF && k1[j] == T1) {
        kp = tie_base < a0.take;
        ++tie_base;
      }
      keep |= kp ? (1u << j) : 0u;
      nk += kp ? 1 : 0;
    }
    const int kbase = block_excl_scan(sh.wsum[1], nk, nkept);
    {
      int pos = kbase;
#pragma unroll
      for (int j = 0; j < kB3Items; ++j)
        if ((keep >> j) & 1u) sh.sbsel[pos++] = kB3Items * t + j;
    }
    // level 1's histogram is no longer read: clear it for level 2
    __syncthreads();
    hist_zero(sh.c);
    if (t == 0) {
      sh.s.cnt[0] = 0;
      sh.s.cnt[1] = 0;
    }
    if constexpr (kPairs) {
      // pass p: lanes 2i, 2i+1 take the halves of kept super-block 512p + i
      float gv[kB3Pass * 4];
      int b0p[kB3Pass];   // first block of this lane's half, -1 when none
#pragma unroll
      for (int p = 0; p < kB3Pass; ++p) {
        const int u = (kSelThreads / 2) * p + (t >> 1);
        const bool on = u < nkept;
        const int b0 = 8 * (on ? sh.sbsel[u] : 0) + 4 * (t & 1);
        b0p[p] = on ? b0 : -1;
        if constexpr (kVec) {
          // b0 + 3 < stride: stride is a multiple of 8 here
          const f32x4_t v = on ? *reinterpret_cast<const f32x4_t*>(row + b0) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < 4; ++e) gv[4 * p + e] = v[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) gv[4 * p + e] = (on && b0 + e < nblk) ? row[b0 + e] : 0.0f;
        }
      }
      int nc[kB3Pass];
#pragma unroll
      for (int p = 0; p < kB3Pass; ++p) {
        nc[p] = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = (b0p[p] >= 0 && b0p[p] + e < nblk) ? order_key(gv[4 * p + e]) : 0u;
          ck[4 * p + e] = key >= T1 ? key : 0u;
          nc[p] += ck[4 * p + e] != 0u ? 1 : 0;
        }
      }
      // positions in (pass, thread) order: two passes per scan, 16 bits each
      // (a pass holds at most 4 * 1024 survivors)
      const int x[3] = {nc[0] | (nc[1] << 16), nc[2] | (nc[3] << 16), nc[4] | (nc[5] << 16)};
      int ex[3], tot[3];
      // wsum rows 0-2: their last reads (the tie and kept-list sums) precede the
      // barrier after the kept list
      block_excl_scan3(sh.wsum, x, ex, tot);
      int base = 0;
#pragma unroll
      for (int i = 0; i < kB3Pass / 2; ++i) {
        // m2 <= 24 * 1024 < 2^16
        const int lo = base + (ex[i] & 0xFFFF);
        base += tot[i] & 0xFFFF;
        const int hi = base + (ex[i] >> 16);
        base += tot[i] >> 16;
        cpos2[i] = lo | (hi << 16);
      }
      m2 = base;
    } else {
      // thread t takes kept super-blocks [G t, G t + G), G = ceil(nkept / 1024)
      const int G = (nkept + kSelThreads - 1) / kSelThreads;   // <= 3
      float gv[kB3Pass * 4];
#pragma unroll
      for (int q = 0; q < kB3Pass / 2; ++q) {
        const int u = G * t + q;
        const bool on = q < G && u < nkept;
        sbq[q] = on ? sh.sbsel[u] : -1;
        const int sb = on ? sbq[q] : 0;
        if constexpr (kVec) {
          // 8 sb + 7 < stride: stride is a multiple of 8 here
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const f32x4_t v =
                on ? *reinterpret_cast<const f32x4_t*>(row + 8 * sb + 4 * h) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) gv[8 * q + 4 * h + e] = v[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int b = 8 * sb + e;
            gv[8 * q + e] = (on && b < nblk) ? row[b] : 0.0f;
          }
        }
      }
      int nc = 0;
#pragma unroll
      for (int q = 0; q < kB3Pass / 2; ++q) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t key = (sbq[q] >= 0 && 8 * sbq[q] + e < nblk) ? order_key(gv[8 * q + e]) : 0u;
          ck[8 * q + e] = key >= T1 ? key : 0u;
          nc += ck[8 * q + e] != 0u ? 1 : 0;
        }
      }
      cpos = block_excl_scan(sh.wsum[2], nc, m2);
    }
    if (m2 > kCompCap && approx > 0) {
      // too many survivors for LDS: redo level 1 exactly (at most 8 * 2048)
      approx = 0;
      continue;   // the histogram is clear and every thread is past the barrier above
    }
    break;
  }
  // survivors to LDS in id order, counted into level 2's first-digit histogram
  {
    const int s2 = first_digit_shift(T1, kmax1);
    if constexpr (kPairs) {
#pragma unroll
      for (int p = 0; p < kB3Pass; ++p) {
        int pos = (cpos2[p >> 1] >> ((p & 1) ? 16 : 0)) & 0xFFFF;
        // the kept list is intact until level 2 emits
        const int b0 = 8 * sh.sbsel[(kSelThreads / 2) * p + (t >> 1)] + 4 * (t & 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = ck[4 * p + e];
          if (key != 0u) {
            sh.ckeys[pos] = key;
            sh.cids[pos] = b0 + e;
            atomicAdd(&sh.c.hist[((key - T1) >> s2) & (kBins - 1)], 1u);
            ++pos;
          }
        }
      }
    } else {
      int pos = cpos;
#pragma unroll
      for (int j = 0; j < kB3Pass * 4; ++j) {
        if (ck[j] != 0u) {
          sh.ckeys[pos] = ck[j];
          sh.cids[pos] = 8 * sbq[j >> 3] + (j & 7);
          atomicAdd(&sh.c.hist[((ck[j] - T1) >> s2) & (kBins - 1)], 1u);
          ++pos;
        }
      }
    }
  }
  __syncthreads();
  // level 2 over the m2 survivors (item order = id order), all within [T1, kmax1];
  // registers sized to the count (a typical row keeps 2,000-3,000)
  if (m2 <= 4 * kSelThreads)
    blocks_level2<4>(sh, m2, T1, kmax1, K0, o0, K1, o1, floor_out);
  else
    blocks_level2<16>(sh, m2, T1, kmax1, K0, o0, K1, o1, floor_out);
}

template <bool kHaveSuper, bool kVec>
__global__ __launch_bounds__(kSelThreads) void select_blocks3_kernel(const float* __restrict__ bmax, int64_t stride,
                                                                     const float* __restrict__ super_max,
                                                                     int64_t nsup_stride,
                                                                     const int32_t* __restrict__ n_visible, int K0,
                                                                     int32_t* __restrict__ out0, int K1,
                                                                     int32_t* __restrict__ out1,
                                                                     uint32_t* __restrict__ floor_out) {
  __shared__ Blocks3Shared sh;
  const int r = blockIdx.x;
  select_blocks3_row<kHaveSuper, kVec, true>(sh, r, bmax, stride, super_max, nsup_stride, n_visible, K0,
                                       out0 ? out0 + (int64_t)r * K0 : nullptr, K1,
                                       out1 ? out1 + (int64_t)r * K1 : nullptr, floor_out ? floor_out + r : nullptr);
}

// ---------------------------------------------------------------------------
// Full layer, decode: the block filter and the top-k in one workgroup per row.
// The filter leaves the row's first kb blocks (ids ascending, -1 padded) and
// its floor in LDS; the top-k then reads the scan's stored scores of those
// blocks' 8*kb positions (the row's top-k lies there: the pool lemma) and
// ranks them by (score desc, position asc).  When kb == k the k-th block key
// is at most the k-th position score (those k block maxima are k positions
// reaching it), so positions below it are dropped unexamined.
// ---------------------------------------------------------------------------
constexpr int kFusedMaxKb = 2048;

template <int JT>
__device__ __forceinline__ void topk_from_blocks(Core& c, Small& s, const int32_t* blk, int kb,
                                                 const float* __restrict__ srow, int64_t n_lim, uint32_t floor,
                                                 int k, int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int cap = 8 * kb;
  const int Jp = (cap + 1023) >> 10;
  int32_t pos[JT];
#pragma unroll
  for (int j = 0; j < JT; ++j) {
    const int i = (w * Jp + j) * 64 + lane;
    const int32_t b = (j < Jp && i < cap) ? blk[i >> 3] : -1;
    const int64_t p = 8 * (int64_t)b + (i & 7);
    pos[j] = (b >= 0 && p < n_lim) ? (int32_t)p : -1;
  }
  float x[JT];
#pragma unroll
  for (int j = 0; j < JT; ++j) x[j] = pos[j] >= 0 ? srow[pos[j]] : 0.0f;
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

struct RegTopkShared {
  RegShared rs;
  int32_t blk[kFusedMaxKb];
  uint32_t floor;
};

// Grid 2R: workgroup r < R selects row r's first kb blocks and then its top-k
// (what the attention waits for); workgroup R + r selects row r's pool beside
// it, on another CU (the pool is read only by later layers).  The first kb
// blocks of the ranking do not depend on the pool size, and ranking for kb
// alone keeps fewer super-blocks and survivors than ranking for the pool.
//
// Block rows of at most 1024*J blocks (register filter), kb <= 128*JT.
template <int J, int JT>
__global__ __launch_bounds__(kSelThreads) void select_reg_topk_kernel(
    const float* __restrict__ bmax, int64_t stride, const int32_t* __restrict__ n_visible, int n_pool,
    int32_t* __restrict__ pool_out, int kb, const float* __restrict__ scores, int64_t n_max, int k,
    int32_t* __restrict__ idx) {
  __shared__ RegTopkShared sh;
  const int R = (int)(gridDim.x >> 1);
  if ((int)blockIdx.x >= R) {
    const int r = (int)blockIdx.x - R;
    select_reg_row<J, kSelBlocks>(sh.rs, r, bmax, stride, nullptr, 0, n_visible, n_pool,
                                  pool_out + (int64_t)r * n_pool, 0, nullptr, nullptr, nullptr);
    return;
  }
  const int r = blockIdx.x;
  select_reg_row<J, kSelBlocks>(sh.rs, r, bmax, stride, nullptr, 0, n_visible, 0, nullptr, kb, sh.blk, nullptr,
                                &sh.floor);
  __syncthreads();
  int64_t nv = n_visible[r];
  nv = nv < 0 ? 0 : (nv < n_max ? nv : n_max);
  topk_from_blocks<JT>(sh.rs.c, sh.rs.s, sh.blk, kb, scores + (int64_t)r * n_max, nv, kb == k ? sh.floor : 1u, k,
                       idx + (int64_t)r * k);
}

// Block rows of up to 65,536 blocks (two-level filter), kb <= 128*JT.  The
// filter's kept-super-block list is free once level 2 runs: it holds the kb
// block ids.
template <bool kVec, int JT>
__global__ __launch_bounds__(kSelThreads) void select_blocks3_topk_kernel(
    const float* __restrict__ bmax, int64_t stride, const float* __restrict__ super_max, int64_t nsup_stride,
    const int32_t* __restrict__ n_visible, int n_pool, int32_t* __restrict__ pool_out, int kb,
    const float* __restrict__ scores, int64_t n_max, int k, int32_t* __restrict__ idx) {
  __shared__ Blocks3Shared sh;
  // grid 2R, as select_reg_topk_kernel
  const int R = (int)(gridDim.x >> 1);
  if ((int)blockIdx.x >= R) {
    const int r = (int)blockIdx.x - R;
    select_blocks3_row<true, kVec, false>(sh, r, bmax, stride, super_max, nsup_stride, n_visible, n_pool,
                                   pool_out + (int64_t)r * n_pool, 0, nullptr, nullptr);
    return;
  }
  const int r = blockIdx.x;
  select_blocks3_row<true, kVec, false>(sh, r, bmax, stride, super_max, nsup_stride, n_visible, 0, nullptr, kb, sh.sbsel,
                                 &sh.floor);
  __syncthreads();
  int64_t nv = n_visible[r];
  nv = nv < 0 ? 0 : (nv < n_max ? nv : n_max);
  topk_from_blocks<JT>(sh.c, sh.s, sh.sbsel, kb, scores + (int64_t)r * n_max, nv, kb == k ? sh.floor : 1u, k,
                       idx + (int64_t)r * k);
}

// ---------------------------------------------------------------------------
// Full layer, decode, rows whose every block fits in the pool: the pool is every
// visible block, and (the pool keeping at least k blocks) the top-k over the
// pool is the top-k over every visible position, taken straight from the
// scan's stored score row.  Grid 2R: workgroup r < R ranks row r's scores,
// workgroup R + r writes its pool.  Rows of at most 1024*J positions.
// ---------------------------------------------------------------------------
template <int J>
__global__ __launch_bounds__(kSelThreads) void select_short_kernel(const float* __restrict__ scores, int64_t n_max,
                                                                   const int32_t* __restrict__ n_visible, int n_pool,
                                                                   int32_t* __restrict__ pool_out, int k,
                                                                   int32_t* __restrict__ idx) {
  __shared__ RegShared sh;
  const int R = (int)(gridDim.x >> 1);
  if ((int)blockIdx.x >= R) {
    const int r = (int)blockIdx.x - R;
    int64_t nv = n_visible[r];
    nv = nv < 0 ? 0 : (nv < n_max ? nv : n_max);
    const int nblk = (int)((nv + 7) >> 3);
    int32_t* po = pool_out + (int64_t)r * n_pool;
    for (int p = threadIdx.x; p < n_pool; p += kSelThreads) po[p] = p < nblk ? p : -1;
    return;
  }
  const int r = blockIdx.x;
  select_reg_row<J, kSelFull>(sh, r, scores, n_max, nullptr, 0, n_visible, k, idx + (int64_t)r * k, 0, nullptr,
                              nullptr, nullptr);
}

// ---------------------------------------------------------------------------
// Top-k over a pool's slots (Reindex layers), by the pool lemma: the k best
// positions of the pool lie in its first kb = min(k, n_pool) blocks ranked by
// (block maximum desc, block position asc), since every block ranked ahead of a
// block holding a selected position contributes its own best position ahead of
// that position.  One workgroup per row ranks the pool's block maxima (taken
// from the row's slot scores), then the 8 kb slots of its first kb blocks; when
// kb == k the kb-th block key bounds the k-th position score from below, so
// slots under it are dropped first.  The result is select_reg_kernel's over
// every slot.
// ---------------------------------------------------------------------------
template <int JT>
__device__ __forceinline__ void topk_from_pool_blocks(Core& c, Small& s, const int32_t* pidx, int kb,
                                                      const float* __restrict__ srow,
                                                      const int32_t* __restrict__ pb, int64_t nv, uint32_t floor,
                                                      int k, int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int cap = 8 * kb;
  const int Jp = (cap + 1023) >> 10;
  int32_t pos[JT];
  uint32_t key[JT];
#pragma unroll
  for (int j = 0; j < JT; ++j) {
    const int i = (w * Jp + j) * 64 + lane;
    const int32_t pi = (j < Jp && i < cap) ? pidx[i >> 3] : -1;   // pool index of the slot's block
    const int32_t b = pi >= 0 ? pb[pi] : -1;
    const int64_t p = 8 * (int64_t)b + (i & 7);
    pos[j] = (b >= 0 && p < nv) ? (int32_t)p : -1;
    const float x = pos[j] >= 0 ? srow[8 * pi + (i & 7)] : 0.0f;
    const uint32_t kk = order_key(x);
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

// JB: pool blocks per thread (n_pool <= 1024 JB); JT: slots per thread (kb <= 128 JT).
template <int JB, int JT>
__global__ __launch_bounds__(kSelThreads) void select_pool_topk_kernel(const float* __restrict__ scores,
                                                                       const int32_t* __restrict__ pool_blocks,
                                                                       int n_pool,
                                                                       const int32_t* __restrict__ n_visible, int k,
                                                                       int32_t* __restrict__ idx) {
  __shared__ RegTopkShared sh;
  const int r = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float* srow = scores + (int64_t)r * 8 * n_pool;
  const int32_t* pb = pool_blocks + (int64_t)r * n_pool;
  int64_t nv = n_visible[r];
  nv = nv < 0 ? 0 : nv;
  // block keys, item (w, j, lane) = pool block (w Jp + j) 64 + lane: the
  // maximum key of its valid slots, 0 when it has none
  const int Jp = (n_pool + 1023) >> 10;
  uint32_t bkey[JB];
#pragma unroll
  for (int j = 0; j < JB; ++j) {
    const int i = (w * Jp + j) * 64 + lane;
    uint32_t m = 0u;
    const int32_t b = (j < Jp && i < n_pool) ? pb[i] : -1;
    if (b >= 0) {
      // 32-byte aligned: rows of 8 n_pool floats from a 16-byte aligned base
      const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(srow + 8 * i);
      const f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(srow + 8 * i + 4);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t kk = order_key(t < 4 ? v0[t] : v1[t - 4]);
        m = (8 * (int64_t)b + t < nv && kk > m) ? kk : m;
      }
    }
    bkey[j] = m;
  }
  hist_zero(sh.rs.c);
  if (threadIdx.x == 0) {
    sh.rs.s.cnt[0] = 0;
    sh.rs.s.cnt[1] = 0;
  }
  int valid;
  uint32_t kmin, kmax;
  key_range(sh.rs.s, bkey, Jp, valid, kmin, kmax);
  const int kb = k < n_pool ? k : n_pool;
  Thr th0, th1;
  select_thresholds(sh.rs.c, sh.rs.s, bkey, Jp, valid, kmin, kmax, 0, kb, 0, th0, th1);
  const uint32_t floor = (kb == k && th1.keff == kb && valid > kb) ? th1.T : 1u;
  emit_sel(
      sh.rs.s, bkey, Jp, th0, th1, [&](int, int p, int, int i) { sh.blk[p] = i; },
      [&](int, int p) { sh.blk[p] = -1; });
  __syncthreads();
  topk_from_pool_blocks<JT>(sh.rs.c, sh.rs.s, sh.blk, kb, srow, pb, nv, floor, k, idx + (int64_t)r * k);
}

// ---------------------------------------------------------------------------
// generic selection: the row stays in memory
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSelThreads) void select_mem_kernel(int layout, const float* __restrict__ scores,
                                                                 int64_t stride,
                                                                 const int32_t* __restrict__ pool_blocks,
                                                                 int64_t n_pool,
                                                                 const int32_t* __restrict__ n_visible, int k1,
                                                                 int32_t* __restrict__ out1, int k2,
                                                                 int32_t* __restrict__ out2,
                                                                 uint32_t* __restrict__ floor_out) {
  __shared__ SelShared sh;
  const int r = blockIdx.x;
  if (floor_out && threadIdx.x == 0) floor_out[r] = 1u;   // no floor from this path
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  RowView row;
  row.layout = layout;
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
  if (!out1) k1 = 0;
  if (!out2) k2 = 0;
  int32_t* o1 = out1 ? out1 + (int64_t)r * k1 : nullptr;
  int32_t* o2 = out2 ? out2 + (int64_t)r * k2 : nullptr;
  KeyStats st;
  for (int64_t base = 0; base < row.n; base += kSelCap) {
#pragma unroll 10
    for (int j = 0; j < kSegIters; ++j) {
      const int64_t i = base + (int64_t)w * kSegItems + 64 * j + lane;
      st.add(i < row.n ? row.key_mem(i) : 0u);
    }
  }
  reduce_stats(sh, st);
  select_targets<kSrcMem, kIdRow, false, false>(sh, row, row.n, k1, o1, k2, o2);
}

// ---------------------------------------------------------------------------
// Pool rescoring and top-k in one workgroup per row (many queries per
// sequence).  In round j wave w scores the row's pool blocks [8 (w Jp + j), +8)
// with the pool scan's lane layout (lane 16g + c holds block g of position
// c & 7 of pool block 2u + (c >> 3) in group u), so lane l's score is item
// (w, j, l) of the register-resident selection: slot order is position order
// (the pool blocks are listed by id).  Keys, validity and floor as
// pool_scan_kernel followed by select_reg_kernel<J, kSelPool>, with no round
// trip of the scores through memory.
// ---------------------------------------------------------------------------
template <int J>
__device__ __forceinline__ void pool_topk_row(RegShared& sh, int32_t* sblk, int r, const uint8_t* __restrict__ q_codes,
                                              const uint8_t* __restrict__ q_scales,
                                              const uint8_t* __restrict__ k_codes,
                                              const uint8_t* __restrict__ k_scales,
                                              const int32_t* __restrict__ pool_blocks, int n_pool,
                                              const int32_t* __restrict__ n_visible, int M, int64_t N_max,
                                              const uint32_t* __restrict__ floor_in, int k,
                                              int32_t* __restrict__ idx) {
  const int64_t seq = r / M;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int cap = 8 * n_pool;
  const int Jp = (cap + 1023) >> 10;
  // the row's pool block ids, staged in LDS with one coalesced pass
  const int32_t* pb = pool_blocks + (int64_t)r * n_pool;
  for (int t = threadIdx.x; t < n_pool; t += kSelThreads) sblk[t] = pb[t];
  int64_t nv_sel = n_visible[r];
  nv_sel = nv_sel < 0 ? 0 : nv_sel;                          // the selection's bound
  const int64_t nv = nv_sel > N_max ? N_max : nv_sel;        // the scan's bound
  const uint8_t* kc = k_codes + seq * N_max * 64;
  const uint8_t* ks = k_scales + seq * N_max * 4;
  half2_t qh[16];
  load_query_block(q_codes + (int64_t)r * 64 + 16 * g, qh);
  const int eq = q_scales[(int64_t)r * 4 + g];
  const uint32_t fl = floor_in ? floor_in[r] : 1u;
  __syncthreads();   // the staged ids visible
  uint32_t key[J];
  int32_t pbv[J];   // pool block of this lane's item in round j
#pragma unroll
  for (int j = 0; j < J; ++j) {
    key[j] = 0u;
    pbv[j] = -1;
    const int base = (w * Jp + j) * 8;
    if (j < Jp && base < n_pool) {   // uniform over the wave
      int32_t blk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = base + 2 * u + (c >> 3);
        const int32_t v = sblk[i < n_pool ? i : n_pool - 1];
        blk[u] = i < n_pool ? v : -1;
      }
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
      const float sc = score_groups_valu(qh, eq, kb, ek);
      // this lane's item: pool block base + 2g + (c >> 3) (group u = g), position c & 7
      const bool mine_ok = (g & 2) ? ((g & 1) ? ok[3] : ok[2]) : ((g & 1) ? ok[1] : ok[0]);
      const int32_t bm = (g & 2) ? ((g & 1) ? blk[3] : blk[2]) : ((g & 1) ? blk[1] : blk[0]);
      const int i = base * 8 + lane;
      if (i < cap) {
        pbv[j] = bm;
        const uint32_t kk = order_key(mine_ok ? sc : -__builtin_inff());
        const bool okk = bm >= 0 && 8 * (int64_t)bm + (c & 7) < nv_sel;
        key[j] = okk && kk >= fl ? kk : 0u;
      }
    }
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
  select_thresholds(sh.c, sh.s, key, Jp, valid, kmin, kmax, k, 0, 0, th0, th1);
  int32_t* out = idx + (int64_t)r * k;
  emit_sel(
      sh.s, key, Jp, th0, th1, [&](int, int pos, int j, int i) { out[pos] = 8 * pbv[j] + (i & 7); },
      [&](int, int p) { out[p] = -1; });
}

// Row of a one-dimensional grid of workgroups, renumbered so that each of the
// 8 XCDs (which take linear workgroup ids round-robin) runs a contiguous run of
// rows: neighbouring rows of a prefill chunk, whose pools overlap, rescore
// through one L2.  Grids of a size not divisible by 8 keep their order.
__device__ __forceinline__ int xcd_row() {
  const unsigned b = blockIdx.x, T = gridDim.x;
  return (int)(T % 8u == 0u ? (b % 8u) * (T / 8u) + b / 8u : b);
}

#define CSA2_POOL_TOPK_ARGS                                                                                     \
  const uint8_t *__restrict__ q_codes, const uint8_t *__restrict__ q_scales, const uint8_t *__restrict__ k_codes, \
      const uint8_t *__restrict__ k_scales, const int32_t *__restrict__ pool_blocks, int n_pool,                 \
      const int32_t *__restrict__ n_visible, int M, int64_t N_max, const uint32_t *__restrict__ floor_in, int k,  \
      int32_t *__restrict__ idx
// pools of up to 512 blocks: two workgroups a compute unit (64 registers)
__global__ __launch_bounds__(kSelThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void pool_topk_kernel4(
    CSA2_POOL_TOPK_ARGS) {
  __shared__ RegShared sh;
  __shared__ int32_t sblk[512];
  pool_topk_row<4>(sh, sblk, xcd_row(), q_codes, q_scales, k_codes, k_scales, pool_blocks, n_pool, n_visible, M, N_max,
                   floor_in, k, idx);
}
template <int J>
__global__ __launch_bounds__(kSelThreads) void pool_topk_kernel(CSA2_POOL_TOPK_ARGS) {
  __shared__ RegShared sh;
  __shared__ int32_t sblk[128 * J];   // n_pool <= 1024 J / 8
  pool_topk_row<J>(sh, sblk, xcd_row(), q_codes, q_scales, k_codes, k_scales, pool_blocks, n_pool, n_visible, M, N_max,
                   floor_in, k, idx);
}
#undef CSA2_POOL_TOPK_ARGS

hipError_t launch_pool_topk(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                            const uint8_t* k_scales, const int32_t* pool_blocks, int n_pool,
                            const int32_t* n_visible, int B, int M, int64_t N_max, const uint32_t* floor_in, int k,
                            int32_t* idx, hipStream_t stream) {
  const int64_t R = (int64_t)B * M;
  if (k <= 0 || n_pool <= 0 || R <= 0 || R > 0x7FFFFFFF) return hipErrorNotSupported;
  const int cap = 8 * n_pool;
  const dim3 grid((unsigned)R), block(kSelThreads);
#define CSA2_PT(J)                                                                                                   \
  hipLaunchKernelGGL((pool_topk_kernel<J>), grid, block, 0, stream, q_codes, q_scales, k_codes, k_scales, pool_blocks, \
                     n_pool, n_visible, M, N_max, floor_in, k, idx)
  if (cap <= 4096)
    hipLaunchKernelGGL(pool_topk_kernel4, grid, block, 0, stream, q_codes, q_scales, k_codes, k_scales, pool_blocks,
                       n_pool, n_visible, M, N_max, floor_in, k, idx);
  else if (cap <= 8192)
    CSA2_PT(8);
  else if (cap <= 16384)
    CSA2_PT(16);
  else
    return hipErrorNotSupported;
#undef CSA2_PT
  return hipGetLastError();
}

hipError_t launch_select(int layout, const float* scores, int64_t stride, const int32_t* pool_blocks,
                         int64_t n_pool, const int32_t* n_visible, int R, int k1, int32_t* out1, int k2,
                         int32_t* out2, const float* super_max, int64_t nsup_stride, hipStream_t stream,
                         const uint32_t* floor_in, uint32_t* floor_out) {
  // the longest possible row decides the path
  const int64_t max_n = layout == kSelPool ? 8 * n_pool : stride;
  const int ka = out1 ? k1 : 0, kb = out2 ? k2 : 0;
  const int kmax = ka > kb ? ka : kb;
  const dim3 grid((unsigned)R), block(kSelThreads);
#define CSA2_REG(J, L)                                                                                      \
  hipLaunchKernelGGL((select_reg_kernel<J, L>), grid, block, 0, stream, scores, stride, pool_blocks, n_pool, \
                     n_visible, k1, out1, k2, out2, floor_in, floor_out)
#define CSA2_REG_J(J)                   \
  if (layout == kSelBlocks)             \
    CSA2_REG(J, kSelBlocks);            \
  else if (layout == kSelPool)          \
    CSA2_REG(J, kSelPool);              \
  else                                  \
    CSA2_REG(J, kSelFull)
  if (layout == kSelPool && n_pool <= 2048 && out1 && k1 > 0 && !out2 && !floor_in && !floor_out) {
    // a pool's top-k through its first min(k, n_pool) blocks
    const int kbk = k1 < n_pool ? k1 : (int)n_pool;
    if (kbk <= 512)
      hipLaunchKernelGGL((select_pool_topk_kernel<2, 4>), grid, block, 0, stream, scores, pool_blocks, (int)n_pool,
                         n_visible, k1, out1);
    else
      hipLaunchKernelGGL((select_pool_topk_kernel<2, 16>), grid, block, 0, stream, scores, pool_blocks, (int)n_pool,
                         n_visible, k1, out1);
  } else if (max_n <= 4096) {
    CSA2_REG_J(4);
  } else if (max_n <= 8192) {
    CSA2_REG_J(8);
  } else if (max_n <= 16384) {
    CSA2_REG_J(16);
  } else if (layout == kSelBlocks && (max_n + 7) / 8 <= 8192 && kmax <= 2048) {
    const bool vec = super_max && reinterpret_cast<uintptr_t>(super_max) % 16 == 0 && nsup_stride % 4 == 0 &&
                     reinterpret_cast<uintptr_t>(scores) % 32 == 0 && stride % 8 == 0;
    if (vec)
      hipLaunchKernelGGL((select_blocks3_kernel<true, true>), grid, block, 0, stream, scores, stride, super_max,
                         nsup_stride, n_visible, k1, out1, k2, out2, floor_out);
    else if (super_max)
      hipLaunchKernelGGL((select_blocks3_kernel<true, false>), grid, block, 0, stream, scores, stride, super_max,
                         nsup_stride, n_visible, k1, out1, k2, out2, floor_out);
    else
      hipLaunchKernelGGL((select_blocks3_kernel<false, false>), grid, block, 0, stream, scores, stride, super_max,
                         nsup_stride, n_visible, k1, out1, k2, out2, floor_out);
  } else {
    hipLaunchKernelGGL(select_mem_kernel, grid, block, 0, stream, layout, scores, stride, pool_blocks, n_pool,
                       n_visible, k1, out1, k2, out2, floor_out);
  }
#undef CSA2_REG_J
#undef CSA2_REG
  return hipGetLastError();
}

hipError_t launch_select_topk(const float* bmax, int64_t stride, const float* super_max, int64_t nsup_stride,
                              const int32_t* n_visible, int R, int n_pool, int32_t* pool_out, int kb,
                              const float* scores, int64_t n_max, int k, int32_t* idx, hipStream_t stream) {
  if (kb < 1 || kb > kFusedMaxKb || k < 1 || n_pool < kb || n_pool > 2048 || !super_max)
    return hipErrorNotSupported;
  const dim3 grid(2u * (unsigned)R), block(kSelThreads);   // top-k workgroups, then pool workgroups
  const bool small_kb = kb <= 512;
#define CSA2_REGT(J)                                                                                          \
  do {                                                                                                        \
    if (small_kb)                                                                                             \
      hipLaunchKernelGGL((select_reg_topk_kernel<J, 4>), grid, block, 0, stream, bmax, stride, n_visible,     \
                         n_pool, pool_out, kb, scores, n_max, k, idx);                                        \
    else                                                                                                      \
      hipLaunchKernelGGL((select_reg_topk_kernel<J, 16>), grid, block, 0, stream, bmax, stride, n_visible,    \
                         n_pool, pool_out, kb, scores, n_max, k, idx);                                        \
  } while (0)
  if (stride <= 4096) {
    CSA2_REGT(4);
  } else if (stride <= 8192) {
    CSA2_REGT(8);
  } else if (stride <= 16384) {
    CSA2_REGT(16);
  } else if ((stride + 7) / 8 <= 8192) {
    const bool vec = reinterpret_cast<uintptr_t>(super_max) % 16 == 0 && nsup_stride % 4 == 0 &&
                     reinterpret_cast<uintptr_t>(bmax) % 32 == 0 && stride % 8 == 0;
    if (vec && small_kb)
      hipLaunchKernelGGL((select_blocks3_topk_kernel<true, 4>), grid, block, 0, stream, bmax, stride, super_max,
                         nsup_stride, n_visible, n_pool, pool_out, kb, scores, n_max, k, idx);
    else if (vec)
      hipLaunchKernelGGL((select_blocks3_topk_kernel<true, 16>), grid, block, 0, stream, bmax, stride, super_max,
                         nsup_stride, n_visible, n_pool, pool_out, kb, scores, n_max, k, idx);
    else if (small_kb)
      hipLaunchKernelGGL((select_blocks3_topk_kernel<false, 4>), grid, block, 0, stream, bmax, stride, super_max,
                         nsup_stride, n_visible, n_pool, pool_out, kb, scores, n_max, k, idx);
    else
      hipLaunchKernelGGL((select_blocks3_topk_kernel<false, 16>), grid, block, 0, stream, bmax, stride, super_max,
                         nsup_stride, n_visible, n_pool, pool_out, kb, scores, n_max, k, idx);
  } else {
    return hipErrorNotSupported;
  }
#undef CSA2_REGT
  return hipGetLastError();
}

hipError_t launch_select_short(const float* scores, int64_t n_max, const int32_t* n_visible, int R, int n_pool,
                               int32_t* pool_out, int k, int32_t* idx, hipStream_t stream) {
  if (k < 1 || n_max > 16384 || (n_max + 7) / 8 > n_pool) return hipErrorNotSupported;
  const dim3 grid(2u * (unsigned)R), block(kSelThreads);
  if (n_max <= 4096)
    hipLaunchKernelGGL((select_short_kernel<4>), grid, block, 0, stream, scores, n_max, n_visible, n_pool, pool_out, k,
                       idx);
  else if (n_max <= 8192)
    hipLaunchKernelGGL((select_short_kernel<8>), grid, block, 0, stream, scores, n_max, n_visible, n_pool, pool_out, k,
                       idx);
  else
    hipLaunchKernelGGL((select_short_kernel<16>), grid, block, 0, stream, scores, n_max, n_visible, n_pool, pool_out,
                       k, idx);
  return hipGetLastError();
}

}  // namespace csa2
