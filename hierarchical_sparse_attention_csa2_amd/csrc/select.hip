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
// total-order key of the fp32 score (0 = no element).  The working set (up to
// 20,480 keys) sits in LDS; wave w holds items [1280w, 1280w + 1280), item
// 64j + lane, so LDS and memory accesses are conflict-free and coalesced, and
// ordered prefix sums come from ballots.  Cross-lane reductions use DPP.
//   1. The load pass also finds the smallest and largest key and the count.
//   2. A histogram of the first digit ((key - kmin) >> s1, 12 bits) -- spread
//      over the row's own key range so same-address LDS atomics stay rare --
//      gives, per target k, the bin holding the k-th key.
//   3. The members of each threshold bin are copied to a short LDS list; the
//      remaining bits of the k-th key T and how many keys equal to T are taken
//      come from histograms over that list only.
//   4. One ordered emit pass writes every target: keys > T and the first
//      `take` keys == T, ids ascending.
// Rows of block maxima longer than 16,384 are filtered one level up first:
// super-blocks of 8 consecutive blocks are ranked by their own maximum, and any
// set of super-blocks holding the first K super-blocks holds every block of the
// first K blocks (a super-block ranked ahead of another contributes its best
// block ahead of every block of the other).  Level 1 keeps the super-blocks at
// or above the threshold bin when they fit (else exactly the first K), level 2
// selects exactly among their blocks.  Anything longer runs the same selection
// with every pass reading the row from memory.
#include "device_common.h"
#include "kernels.h"

namespace csa2 {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSegIters = 20;                      // items per lane per pass
constexpr int kSegItems = 64 * kSegIters;          // 1280 items per wave
constexpr int kSelCap = kSelWaves * kSegItems;     // 20,480 keys in LDS
constexpr int kRowCap = 16384;                     // rows cached whole (ids = index)
constexpr int kBins = 4096;
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

// ---------------------------------------------------------------------------
// DPP wave helpers
// ---------------------------------------------------------------------------
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xF, false);
}

// Inclusive prefix sum over the wave (row shifts, then row broadcasts).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp<0x111>(x);          // row_shr:1
  x += dpp<0x112>(x);          // row_shr:2
  x += dpp<0x114>(x);          // row_shr:4
  x += dpp<0x118>(x);          // row_shr:8
  x += dpp<0x142, 0xA>(x);     // row_bcast:15 into rows 1, 3
  x += dpp<0x143, 0xC>(x);     // row_bcast:31 into rows 2, 3
  return x;
}

__device__ __forceinline__ int wave_sum(int x) { return __builtin_amdgcn_readlane(wave_incl_scan(x), 63); }

// max / min over each row of 16 lanes (every lane of the row gets it), then over the wave
__device__ __forceinline__ uint32_t row16_max(uint32_t x) {
  uint32_t y;
  y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  x = y > x ? y : x;
  y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  x = y > x ? y : x;
  y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false);  // row_half_mirror
  x = y > x ? y : x;
  y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, false);  // row_mirror
  return y > x ? y : x;
}
__device__ __forceinline__ uint32_t row16_min(uint32_t x) {
  uint32_t y;
  y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
  x = y < x ? y : x;
  y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);
  x = y < x ? y : x;
  y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false);
  x = y < x ? y : x;
  y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, false);
  return y < x ? y : x;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = row16_max(x);
  uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  a = a > b ? a : b;
  c = c > d ? c : d;
  return a > c ? a : c;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = row16_min(x);
  uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  a = a < b ? a : b;
  c = c < d ? c : d;
  return a < c ? a : c;
}
// max over each aligned group of 8 lanes
__device__ __forceinline__ uint32_t group8_max(uint32_t x) {
  uint32_t y;
  y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
  x = y > x ? y : x;
  y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);
  x = y > x ? y : x;
  y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false);
  return y > x ? y : x;
}

__device__ __forceinline__ unsigned long long lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane ? (~0ull >> (64 - lane)) : 0ull;
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

enum { kPathLds = 0, kPathSuper = 1, kPathMem = 2 };

template <int PATH>
__global__ __launch_bounds__(kSelThreads) void select_kernel(int layout, const float* __restrict__ scores,
                                                             int64_t stride, const int32_t* __restrict__ pool_blocks,
                                                             int64_t n_pool, const int32_t* __restrict__ n_visible,
                                                             int k1, int32_t* __restrict__ out1, int k2,
                                                             int32_t* __restrict__ out2,
                                                             const float* __restrict__ super_max,
                                                             int64_t nsup_stride) {
  __shared__ SelShared sh;
  const int r = blockIdx.x;
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

  if constexpr (PATH == kPathLds) {
    // the whole row in LDS (the host guarantees row.n <= kRowCap)
    KeyStats st;
#pragma unroll 10
    for (int j = 0; j < kSegIters; ++j) {
      const int i = w * kSegItems + 64 * j + lane;
      const uint32_t k = i < row.n ? row.key_mem(i) : 0u;
      sh.u.keys[i] = k;
      st.add(k);
    }
    reduce_stats(sh, st);
    select_targets<kSrcKeys, kIdRow, false, false>(sh, row, row.n, k1, o1, k2, o2);
  } else if constexpr (PATH == kPathSuper) {
    // block maxima (the host guarantees nsuper <= kSuperCap and k <= 2048)
    const int64_t nsuper = (row.n + 7) >> 3;
    const int kmax = k1 > k2 ? k1 : k2;
    if (super_max) {
      // level 1 from the scan's super-block maxima
      KeyStats st;
      const float* srow = super_max + (int64_t)r * nsup_stride;
#pragma unroll 10
      for (int j = 0; j < kSegIters; ++j) {
        const int i = w * kSegItems + 64 * j + lane;
        if (i < nsuper) {
          const uint32_t k = order_key(srow[i]);
          sh.u.skeys[i] = k;
          st.add(k);
        }
      }
      reduce_stats(sh, st);
    } else {
      // level 1: super-block maxima of 8 consecutive blocks; lanes read
      // consecutive blocks (coalesced) and reduce over groups of 8 lanes
      KeyStats st;
      for (int64_t b0 = 0; b0 < 8 * nsuper; b0 += (int64_t)kSelThreads * 8) {
        uint32_t kk[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int64_t i = b0 + (int64_t)w * 512 + 64 * j + lane;
          kk[j] = i < row.n ? order_key(row.s[i]) : 0u;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t m = group8_max(kk[j]);
          const int64_t i = b0 + (int64_t)w * 512 + 64 * j + lane;
          if ((lane & 7) == 0 && (i >> 3) < nsuper) {
            sh.u.skeys[i >> 3] = m;
            st.add(m);
          }
        }
      }
      reduce_stats(sh, st);
    }
    // keep (at least) the first kmax super-blocks, ascending, in sbsel
    select_targets<kSrcSuper, kIdIndex, true, true>(sh, row, nsuper, kmax, nullptr, 0, nullptr, kLevelCap);
    const int nsel = sh.res[6];
    // level 2: the blocks of the kept super-blocks, gathered into LDS
    {
      KeyStats st;
#pragma unroll 10
      for (int j = 0; j < kSegIters; ++j) {
        const int i = w * kSegItems + 64 * j + lane;
        uint32_t k = 0u;
        if (i < 8 * nsel) {
          const int32_t sb = sh.sbsel[i >> 3];
          const int64_t blk = 8 * (int64_t)sb + (i & 7);
          k = (sb >= 0 && blk < row.n) ? order_key(row.s[blk]) : 0u;
        }
        sh.u.keys[i] = k;
        st.add(k);
      }
      reduce_stats(sh, st);
    }
    select_targets<kSrcKeys, kIdSuperList, false, false>(sh, row, 8 * (int64_t)nsel, k1, o1, k2, o2);
  } else {
    // the row stays in memory
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
}

hipError_t launch_select(int layout, const float* scores, int64_t stride, const int32_t* pool_blocks,
                         int64_t n_pool, const int32_t* n_visible, int R, int k1, int32_t* out1, int k2,
                         int32_t* out2, const float* super_max, int64_t nsup_stride, hipStream_t stream) {
  // the longest possible row decides the path
  const int64_t max_n = layout == kSelPool ? 8 * n_pool : stride;
  const int ka = out1 ? k1 : 0, kb = out2 ? k2 : 0;
  const int kmax = ka > kb ? ka : kb;
  const dim3 grid((unsigned)R), block(kSelThreads);
  if (max_n <= kRowCap)
    hipLaunchKernelGGL(select_kernel<kPathLds>, grid, block, 0, stream, layout, scores, stride, pool_blocks, n_pool,
                       n_visible, k1, out1, k2, out2, super_max, nsup_stride);
  else if (layout == kSelBlocks && (max_n + 7) / 8 <= kSuperCap && kmax <= 2048)
    hipLaunchKernelGGL(select_kernel<kPathSuper>, grid, block, 0, stream, layout, scores, stride, pool_blocks, n_pool,
                       n_visible, k1, out1, k2, out2, super_max, nsup_stride);
  else
    hipLaunchKernelGGL(select_kernel<kPathMem>, grid, block, 0, stream, layout, scores, stride, pool_blocks, n_pool,
                       n_visible, k1, out1, k2, out2, super_max, nsup_stride);
  return hipGetLastError();
}

}  // namespace csa2
