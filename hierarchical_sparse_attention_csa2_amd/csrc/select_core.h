// Register-resident ranked selection for one 1024-thread workgroup per row:
// items live in registers (Jp <= J a lane), every decision is exact on the IEEE
// total-order key of the fp32 score (0 = no item), and ranking is by (score
// desc, id asc) with ids ascending in item order.
#pragma once
#include "device_common.h"

namespace csa2 {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kBins = 4096;

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

// ---------------------------------------------------------------------------
// register-resident selection (rows up to 16,384 items, and the two-level
// block filter)
// ---------------------------------------------------------------------------
// A row of up to n items is held as Jp = ceil(n/1024) <= J items a lane; item
// (w, j, lane) is index (w*Jp + j)*64 + lane, so item order is id order, a
// wave's items are one contiguous range and every pass stops after Jp slots.
constexpr int kRankCap = 128;                      // threshold-bin members resolved by counting
constexpr int kKeepCap = 3072;                     // super-blocks kept by level 1
constexpr int kCompCap = 16384;                    // blocks surviving into level 2

struct Core {
  uint32_t hist[kBins];
  uint32_t mem[2][kRankCap];
};

struct Small {
  int cnt[2];                     // members collected per target
  int wcnt[4][kSelWaves];         // emit: per-wave counts
  int wtot[kSelWaves];            // find: per-wave bin totals
  int wstat[kSelWaves];
  uint32_t wmin[kSelWaves], wmax[kSelWaves];
  int res[16];
};

struct RegShared {
  Core c;
  Small s;
};

__device__ __forceinline__ int mbcnt(unsigned long long m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// inclusive prefix sum over each row of 16 lanes
__device__ __forceinline__ int row_incl_scan(int x) {
  x += dpp<0x111>(x);
  x += dpp<0x112>(x);
  x += dpp<0x114>(x);
  x += dpp<0x118>(x);
  return x;
}

// sum over each aligned group of 4 lanes
__device__ __forceinline__ int quad_sum(int x) {
  x += __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  x += __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  return x;
}

// Count, min and max of the non-zero keys over the workgroup (every thread
// gets them).  One barrier.
template <int J>
__device__ __forceinline__ void key_range(Small& s, const uint32_t (&k)[J], int Jp, int& valid, uint32_t& kmin,
                                          uint32_t& kmax) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int c = 0;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t x = j < Jp ? k[j] : 0u;
    c += x != 0u;
    mn = (x != 0u && x < mn) ? x : mn;
    mx = x > mx ? x : mx;
  }
  c = wave_sum(c);
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  if (lane == 0) {
    s.wstat[w] = c;
    s.wmin[w] = mn;
    s.wmax[w] = mx;
  }
  __syncthreads();
  const bool in = lane < kSelWaves;
  const int c2 = row_incl_scan(in ? s.wstat[lane] : 0);
  valid = __builtin_amdgcn_readlane(c2, kSelWaves - 1);
  kmin = (uint32_t)__builtin_amdgcn_readlane((int)row16_min(in ? s.wmin[lane] : 0xFFFFFFFFu), 0);
  kmax = (uint32_t)__builtin_amdgcn_readlane((int)row16_max(in ? s.wmax[lane] : 0u), 0);
}

__device__ __forceinline__ void hist_zero(Core& c) {
  reinterpret_cast<u32x4_t*>(c.hist)[threadIdx.x] = u32x4_t{0u, 0u, 0u, 0u};   // 1024 x 4 bins
}

// hist[((key - kmin) >> shift) & (2^bits - 1)] += 1 over the non-zero keys with
// ((key - kmin) >> pshift) == prefix (pshift >= 32: every key).
template <int J>
__device__ __forceinline__ void hist_add(Core& c, const uint32_t (&k)[J], int Jp, uint32_t kmin, int shift, int bits,
                                         int pshift, uint32_t prefix) {
  const uint32_t dmask = (1u << bits) - 1u;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t d = k[j] - kmin;
    const bool in = j < Jp && k[j] != 0u && (pshift >= 32 || (d >> pshift) == prefix);
    if (in) atomicAdd(&c.hist[(d >> shift) & dmask], 1u);
  }
}

struct BinHit {
  int bin, above, inbin;
};

// With the histogram complete: for each target with need >= 1, the bin b
// (highest first) with (#keys in bins above b) < need <= (#keys in bins >= b).
// Wave w reads bins [4096 - 256(w+1), 4096 - 256w), lane l four of them, so
// the search is a wave scan, a scan over the 16 wave totals and one lane's
// walk over its four bins.  Two barriers.
__device__ __forceinline__ void find_bins(Core& c, Small& s, int need0, int need1, BinHit& h0, BinHit& h1) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int base = kBins - 256 * w - 4 * (lane + 1);
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&c.hist[base]);
  const int sum = (int)(v[0] + v[1] + v[2] + v[3]);
  const int incl = wave_incl_scan(sum);
  const int tot = __builtin_amdgcn_readlane(incl, 63);
  if (lane == 0) s.wtot[w] = tot;
  __syncthreads();
  const int x = lane < kSelWaves ? s.wtot[lane] : 0;
  const int xi = row_incl_scan(x);
  const int excl_w = __builtin_amdgcn_readlane(xi, w) - tot;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int need = t ? need1 : need0;
    if (need >= 1 && excl_w < need && need <= excl_w + tot) {
      const int hi = excl_w + incl;
      const unsigned long long hit = __ballot(hi - sum < need && need <= hi);
      if (lane == (int)__builtin_ctzll(hit)) {
        int acc = hi - sum, bin = base, c_in = (int)v[0];
#pragma unroll
        for (int e = 3; e >= 0; --e) {
          const int ce = (int)v[e];
          if (acc + ce >= need) {
            bin = base + e;
            c_in = ce;
            break;
          }
          acc += ce;
        }
        s.res[4 * t + 0] = bin;
        s.res[4 * t + 1] = acc;
        s.res[4 * t + 2] = c_in;
      }
    }
  }
  __syncthreads();
  h0 = BinHit{s.res[0], s.res[1], s.res[2]};
  h1 = BinHit{s.res[4], s.res[5], s.res[6]};
}

// Copy the non-zero keys with ((key - kmin) >> cur_t) == prefix_t into mem[t]
// (any order) for the targets with want_t.  Ends synchronised.
template <int J>
__device__ __forceinline__ void collect_bins(Core& c, Small& s, const uint32_t (&k)[J], int Jp, uint32_t kmin,
                                             bool want0, int cur0, uint32_t prefix0, bool want1, int cur1,
                                             uint32_t prefix1) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (j < Jp) {
      const uint32_t d = k[j] - kmin;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bool want = t ? want1 : want0;
        if (!want) continue;
        const bool in = k[j] != 0u && (d >> (t ? cur1 : cur0)) == (t ? prefix1 : prefix0);
        const unsigned long long m = __ballot(in);
        if (m) {
          int b = 0;
          if (lane == 0) b = atomicAdd(&s.cnt[t], __popcll(m));
          b = __builtin_amdgcn_readfirstlane(b);
          if (in) c.mem[t][b + mbcnt(m)] = k[j];
        }
      }
    }
  }
  __syncthreads();
}

// For each wanted target, the need-th largest of its m members (T) and how
// many members equal to T are taken.  Threads [512t, 512t + 512) serve target
// t, four per member: each compares its member with every fourth member and
// the quad adds up the counts above and equal.
__device__ __forceinline__ void rank_members(Core& c, Small& s, bool want0, int m0, int need0, bool want1, int m1,
                                             int need1, uint32_t& T0, int& take0, uint32_t& T1, int& take1) {
  const int t = threadIdx.x >> 9, u = (threadIdx.x & 511) >> 2, part = threadIdx.x & 3;
  const bool want = t ? want1 : want0;
  const int m = t ? m1 : m0, need = t ? need1 : need0;
  const bool mine = want && u < m;
  if (threadIdx.x == 0) {
    s.cnt[0] = 0;
    s.cnt[1] = 0;
  }
  int gt = 0, eq = 0;
  uint32_t x = 0u;
  if (mine) {
    const uint32_t* mem = t ? c.mem[1] : c.mem[0];
    x = mem[u];
    for (int v = part; v < m; v += 4) {
      const uint32_t y = mem[v];
      gt += y > x;
      eq += y == x;
    }
  }
  gt = quad_sum(gt);
  eq = quad_sum(eq);
  if (mine && part == 0 && gt < need && need <= gt + eq) {
    s.res[8 + 2 * t] = (int)x;
    s.res[9 + 2 * t] = need - gt;
  }
  __syncthreads();
  if (want0) {
    T0 = (uint32_t)s.res[8];
    take0 = s.res[9];
  }
  if (want1) {
    T1 = (uint32_t)s.res[10];
    take1 = s.res[11];
  }
}

// A target's selection: the keys > T and the first `take` keys == T (item
// order), keff of them, written to positions [0, keff) of a K-entry output and
// -1 after.
struct Thr {
  uint32_t T;
  int take, keff, K;
  bool on;
};

// Thresholds for up to two targets over the non-zero keys (valid of them, all
// within [kmin, kmax]).  The histogram must be zero on entry.  approx_cap > 0:
// target 0 may instead keep every key of its threshold bin and above when that
// is at most approx_cap keys.
// First-digit shift of a key range: bins of 2^shift keys cover [kmin, kmax] in
// at most 4096 bins.
__device__ __forceinline__ int first_digit_shift(uint32_t kmin, uint32_t kmax) {
  const uint32_t span = kmax - kmin;
  const int bits = span ? 32 - __builtin_clz(span) : 0;
  return bits > 12 ? bits - 12 : 0;
}

// prebuilt: the caller has already counted every key into hist[(key - kmin) >>
// first_digit_shift(kmin, kmax)] and synchronised.
template <int J>
__device__ __forceinline__ void select_thresholds(Core& c, Small& s, const uint32_t (&k)[J], int Jp, int valid,
                                                  uint32_t kmin, uint32_t kmax, int K0, int K1, int approx_cap,
                                                  Thr& th0, Thr& th1, bool prebuilt = false) {
  const int keff0 = K0 > 0 ? (K0 < valid ? K0 : valid) : 0;
  const int keff1 = K1 > 0 ? (K1 < valid ? K1 : valid) : 0;
  th0 = Thr{1u, 0x7FFFFFFF, keff0, K0, keff0 > 0};
  th1 = Thr{1u, 0x7FFFFFFF, keff1, K1, keff1 > 0};
  bool act0 = keff0 > 0 && keff0 < valid, act1 = keff1 > 0 && keff1 < valid;
  if (!act0 && !act1) return;
  const int s1 = first_digit_shift(kmin, kmax);
  if (!prebuilt) {
    hist_add(c, k, Jp, kmin, s1, 12, 32, 0u);
    __syncthreads();
  }
  BinHit h0, h1;
  find_bins(c, s, act0 ? keff0 : 0, act1 ? keff1 : 0, h0, h1);
  int cur0 = s1, cur1 = s1;
  uint32_t pre0 = (uint32_t)h0.bin, pre1 = (uint32_t)h1.bin;
  int need0 = keff0 - h0.above, need1 = keff1 - h1.above;
  int m0 = h0.inbin, m1 = h1.inbin;
  if (approx_cap > 0 && act0 && h0.above + h0.inbin <= approx_cap) {
    th0.T = kmin + (pre0 << s1);
    th0.take = 0x7FFFFFFF;
    th0.keff = h0.above + h0.inbin;
    act0 = false;
  }
  // large threshold bins (many equal or near-equal keys): narrow them with
  // further 12-bit digits
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    bool& act = t ? act1 : act0;
    int& cur = t ? cur1 : cur0;
    uint32_t& pre = t ? pre1 : pre0;
    int& need = t ? need1 : need0;
    int& m = t ? m1 : m0;
    while (act && cur > 0 && m > kRankCap) {
      const int nxt = cur > 12 ? cur - 12 : 0;
      hist_zero(c);
      __syncthreads();
      hist_add(c, k, Jp, kmin, nxt, cur - nxt, cur, pre);
      __syncthreads();
      BinHit g, unused;
      find_bins(c, s, need, 0, g, unused);
      need -= g.above;
      pre = (pre << (cur - nxt)) | (uint32_t)g.bin;
      cur = nxt;
      m = g.inbin;
    }
  }
  if (act0 && cur0 == 0) {
    th0.T = kmin + pre0;
    th0.take = need0;
    act0 = false;
  }
  if (act1 && cur1 == 0) {
    th1.T = kmin + pre1;
    th1.take = need1;
    act1 = false;
  }
  if (act0 || act1) {
    collect_bins(c, s, k, Jp, kmin, act0, cur0, pre0, act1, cur1, pre1);
    rank_members(c, s, act0, m0, need0, act1, m1, need1, th0.T, th0.take, th1.T, th1.take);
  }
}

// Ordered emit of both targets: one counting pass, a barrier, one writing pass.
// store(t, pos, j, i) writes the id of item i (slot j of this lane) at
// position pos of target t; pad(t, p) writes the -1 padding.
template <int J, class Store, class Pad>
__device__ __forceinline__ void emit_sel(Small& s, const uint32_t (&k)[J], int Jp, const Thr& th0, const Thr& th1,
                                         Store store, Pad pad) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // per-lane counts, two 16-bit fields per word (a wave counts at most 64*J)
  uint32_t c0 = 0u, c1 = 0u;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t x = j < Jp ? k[j] : 0u;
    c0 += (th0.on && x > th0.T ? 1u : 0u) + (th0.on && x == th0.T ? 0x10000u : 0u);
    c1 += (th1.on && x > th1.T ? 1u : 0u) + (th1.on && x == th1.T ? 0x10000u : 0u);
  }
  c0 = (uint32_t)wave_sum((int)c0);
  c1 = (uint32_t)wave_sum((int)c1);
  if (lane == 0) {
    s.wcnt[0][w] = (int)(c0 & 0xFFFFu);
    s.wcnt[1][w] = (int)(c0 >> 16);
    s.wcnt[2][w] = (int)(c1 & 0xFFFFu);
    s.wcnt[3][w] = (int)(c1 >> 16);
  }
  __syncthreads();
  int run_sel[2], run_tie[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int g = lane < kSelWaves ? s.wcnt[2 * t][lane] : 0;
    const int e = lane < kSelWaves ? s.wcnt[2 * t + 1][lane] : 0;
    const int gi = row_incl_scan(g), ei = row_incl_scan(e);
    const int gb = __builtin_amdgcn_readlane(gi, w) - __builtin_amdgcn_readlane(g, w);
    const int eb = __builtin_amdgcn_readlane(ei, w) - __builtin_amdgcn_readlane(e, w);
    const int take = t ? th1.take : th0.take;
    run_tie[t] = eb;
    run_sel[t] = gb + (take < eb ? take : eb);
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (j < Jp) {
      const int i = (w * Jp + j) * 64 + lane;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const Thr& th = t ? th1 : th0;
        if (!th.on) continue;
        const bool tie = k[j] == th.T;
        const unsigned long long mt = __ballot(tie);
        const bool sel = k[j] > th.T || (tie && run_tie[t] + mbcnt(mt) < th.take);
        const unsigned long long ms = __ballot(sel);
        const int pos = run_sel[t] + mbcnt(ms);
        if (sel && pos < th.keff) store(t, pos, j, i);
        run_tie[t] += __popcll(mt);
        run_sel[t] += __popcll(ms);
      }
    }
  }
  for (int p = th0.keff + (int)threadIdx.x; p < th0.K; p += kSelThreads) pad(0, p);
  for (int p = th1.keff + (int)threadIdx.x; p < th1.K; p += kSelThreads) pad(1, p);
}

}  // namespace csa2
