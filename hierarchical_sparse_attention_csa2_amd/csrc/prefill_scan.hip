// Prefill indexer scan on the FP4 matrix cores: many queries of one sequence
// against the same index keys (the Full layer's scan when M > 1), with the
// 8-entry block max and the 64-entry super-block max fused in.
//
// The score is the one the decode scan computes (DeepSeek-V4.1-Flash,
// fupanwang.com article, section 三个方向一起压小缓存: FP4 indexer query and key
// over the visible context): four exact 32-element block values v_b =
// sum_b * 2^(eq_b + ek_b - 254), added in order ((v0+v1)+v2)+v3 in fp32.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 multiplies a 32x64 by a 64x32 matrix of E2M1
// values with one E8M0 scale per lane's 32-element K group: lane l holds row
// (or column) l%32 and K group l/32, and the result holds column l%32, rows
// 8(i/4) + 4(l/32) + i%4 in element i of lane l.  Two such products, the second
// accumulating onto the first, give the whole 128-element dot product of 32
// keys (rows) with 32 queries (columns).  Their internal sums round differently
// from the fixed order in general, but not here: with block exponents e_b =
// eq_b + ek_b - 254, every block value is an integer multiple of 2^(min e - 2)
// below 2^13 * 2^(e_b - 2), so when the four e_b span at most 9 and lie in
// [-124, 114] every partial sum, in any order, is an exactly representable normal
// fp32 number (at most 15 + 9 significant bits) or zero.  Then the product equals
// the exact sum, which equals ((v0+v1)+v2)+v3.  A 32-key tile whose scales break
// that condition for some query of the wave (never for N(0,1)-like data, whose
// block exponents differ by a few units) is scored after the key loop on the
// VALU, block by block with ldexp semantics, exactly as the decode scan does.
//
// Work: a wave holds 32 queries (the B operands, built once) and walks the keys
// of its 256-key chunk 32 at a time: two 16-byte loads per lane (the cache's own
// block layout), two MFMAs, then per 8-key block three in-lane max operations and
// one exchange between the half-waves.  Block maxima are staged in LDS and leave
// in row segments after the loop, so the loop holds no global stores and its key
// loads stay in flight across tiles.
#include "device_common.h"
#include "kernels.h"

namespace csa2 {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kPfThreads = 256;
constexpr int kPfWaves = kPfThreads / 64;
constexpr int kPfQueriesPerWave = 32;
constexpr int kPfQueriesPerWG = kPfWaves * kPfQueriesPerWave;   // 128
constexpr int kPfKeyChunk = 256;                                // keys per workgroup
constexpr int kPfTileKeys = 32;
constexpr int kPfTiles = kPfKeyChunk / kPfTileKeys;             // one bit each in a 32-bit mask
static_assert(kPfTiles <= 32, "tile mask");
constexpr int kPfPrefetch = 4;                                  // tiles in flight ahead of use
constexpr int kPfBlocks = kPfKeyChunk / 8;                      // 128 block maxima per query row
constexpr int kPfBmLd = kPfBlocks + 1;                          // padded row: conflict-free column writes

// Per-wave staging of the chunk's block maxima, written back in row segments
// after the key loop (which then holds no global stores).
struct PfStage {
  float bm[kPfQueriesPerWave][kPfBmLd];
};

// Workgroup-wide: the query scale statistics of each wave and the chunk's
// tiles that need the VALU path.
struct PfShared {
  PfStage stage[kPfWaves];
  uint32_t qstat[kPfWaves][3];
  uint32_t bad_tiles;
};

// max of x over lane pairs (l, l^32): v_permlane32_swap exchanges the lower
// half of one register with the upper half of the other
__device__ __forceinline__ uint32_t max_halves(uint32_t x) {
  const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return p[0] > p[1] ? p[0] : p[1];
}
// IEEE maximum (v_maximum3_f32: -0 below +0, no operand canonicalisation)
__device__ __forceinline__ float fmaximum(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float fmaximum_halves(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaximum(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// Exact score of one (query row, key) pair on the VALU, for tiles outside the
// matrix cores' exact range.
__device__ __noinline__ float pair_score_valu(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc,
                                              const uint8_t* ks) {
  float s = 0.0f;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    half2_t qh[16];
    load_query_block(qc + 16 * b, qh);
    const u32x4_t c = *reinterpret_cast<const u32x4_t*>(kc + 16 * b);
    const float v = __builtin_amdgcn_ldexpf(block_dot(c, qh), (int)qs[b] + (int)ks[b] - 254);
    s = b == 0 ? v : s + v;
  }
  return s;
}

template <bool kScores, bool kSuper>
__global__ __launch_bounds__(kPfThreads) void prefill_scan_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales,
    const int32_t* __restrict__ n_visible, int M, int64_t N_max, int64_t nblk_stride, int64_t nsup_stride,
    float* __restrict__ scores, float* __restrict__ block_max, float* __restrict__ super_max) {
  __shared__ PfShared sh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  PfStage& st = sh.stage[wave];
  const int64_t seq = blockIdx.z;
  const int qbase = blockIdx.x * kPfQueriesPerWG + wave * kPfQueriesPerWave;
  const int kbeg = blockIdx.y * kPfKeyChunk;
  const int N = (int)N_max;

  const int col = lane & 31, half = lane >> 5;
  // B operands (queries): lane l is query l%32, K group l/32 = block l/32 (first
  // MFMA) or 2 + l/32 (second)
  const int qi = qbase + col;
  const bool q_ok = qi < M;
  const int64_t r = seq * M + (q_ok ? qi : M - 1);
  i32x8_t qlo = {0, 0, 0, 0, 0, 0, 0, 0}, qhi = {0, 0, 0, 0, 0, 0, 0, 0};
  int sqlo = 127, sqhi = 127;
  uint32_t qsc = 0x7F7F7F7Fu;
  if (q_ok) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(q_codes + r * 64 + 16 * half);
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(q_codes + r * 64 + 32 + 16 * half);
    qlo = i32x8_t{(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
    qhi = i32x8_t{(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
    qsc = *reinterpret_cast<const uint32_t*>(q_scales + r * 4);
    sqlo = (int)((qsc >> (8 * half)) & 0xFFu);
    sqhi = (int)((qsc >> (8 * (2 + half))) & 0xFFu);
  }
  int nv = q_ok ? n_visible[r] : 0;
  nv = nv < 0 ? 0 : (nv > N ? N : nv);
  const int nv_max = (int)wave_max_u32((uint32_t)nv);
  const int nv_min = (int)wave_min_u32(q_ok ? (uint32_t)nv : 0x7FFFFFFFu);
  // the query scale statistics: smallest and largest byte, widest spread
  const uint32_t e0 = qsc & 0xFF, e1 = (qsc >> 8) & 0xFF, e2 = (qsc >> 16) & 0xFF, e3 = qsc >> 24;
  const uint32_t qmn = min(min(e0, e1), min(e2, e3)), qmx = max(max(e0, e1), max(e2, e3));
  {
    const uint32_t a = wave_min_u32(q_ok ? qmn : 255u), b = wave_max_u32(q_ok ? qmx : 0u),
                   c = wave_max_u32(q_ok ? qmx - qmn : 0u);
    if (lane == 0) {
      sh.qstat[wave][0] = a;
      sh.qstat[wave][1] = b;
      sh.qstat[wave][2] = c;
    }
    if (threadIdx.x == 0) sh.bad_tiles = 0u;
  }
  __syncthreads();
  // A key is fit for the matrix cores when, against every query of the
  // workgroup, the four block exponents lie in [-124, 114] and span at most 9.
  // One pass over the chunk's key scales marks the 32-key tiles that are not.
  {
    uint32_t qmin = 255u, qmax = 0u, qspread = 0u;
#pragma unroll
    for (int w = 0; w < kPfWaves; ++w) {
      qmin = min(qmin, sh.qstat[w][0]);
      qmax = max(qmax, sh.qstat[w][1]);
      qspread = max(qspread, sh.qstat[w][2]);
    }
    const int kmin_lo = 130 - (int)qmin, kmax_hi = 368 - (int)qmax, kspread_hi = 9 - (int)qspread;
    for (int key = kbeg + (int)threadIdx.x; key < kbeg + kPfKeyChunk && key < N; key += kPfThreads) {
      const uint32_t sc = *reinterpret_cast<const uint32_t*>(k_scales + (seq * N_max + key) * 4);
      const int b0 = (int)(sc & 0xFF), b1 = (int)((sc >> 8) & 0xFF), b2 = (int)((sc >> 16) & 0xFF),
                b3 = (int)(sc >> 24);
      const int kmn = min(min(b0, b1), min(b2, b3)), kmx = max(max(b0, b1), max(b2, b3));
      if (kmn < kmin_lo || kmx > kmax_hi || kmx - kmn > kspread_hi)
        atomicOr(&sh.bad_tiles, 1u << ((key - kbeg) / kPfTileKeys));
    }
  }
  __syncthreads();
  const uint32_t bad_tiles = sh.bad_tiles;
  if (qbase >= M) return;   // no barriers below: waves leave independently, each with its own staging

  // A operands (keys): lane l is key k0 + l%32, K group l/32
  const uint8_t* kc = k_codes + seq * N_max * 64;
  const uint8_t* ks = k_scales + seq * N_max * 4;
  const int kend = kbeg + kPfKeyChunk < nv_max ? kbeg + kPfKeyChunk : nv_max;
  const int ntiles = kend > kbeg ? (kend - kbeg + kPfTileKeys - 1) / kPfTileKeys : 0;

  struct KeyTile {
    u32x4_t lo, hi;
    uint32_t sc;   // the key's four scale bytes
  };
  auto load_tile = [&](int ti) {
    int key = kbeg + kPfTileKeys * ti + col;
    key = key < N ? key : N - 1;
    const uint8_t* p = kc + (int64_t)key * 64 + 16 * half;
    KeyTile t;
    t.lo = *reinterpret_cast<const u32x4_t*>(p);
    t.hi = *reinterpret_cast<const u32x4_t*>(p + 32);
    t.sc = *reinterpret_cast<const uint32_t*>(ks + (int64_t)key * 4);
    return t;
  };

  uint32_t unsafe_tiles = 0u;
  auto tile = [&](int ti, const KeyTile& kt) {
    const int k0 = kbeg + kPfTileKeys * ti;
    if ((bad_tiles >> ti) & 1u) {
      unsafe_tiles |= 1u << ti;   // scored on the VALU after the loop
      return;
    }
    const int b0 = (int)(kt.sc & 0xFF), b1 = (int)((kt.sc >> 8) & 0xFF), b2 = (int)((kt.sc >> 16) & 0xFF),
              b3 = (int)(kt.sc >> 24);
    const i32x8_t klo = {(int)kt.lo[0], (int)kt.lo[1], (int)kt.lo[2], (int)kt.lo[3], 0, 0, 0, 0};
    const i32x8_t khi = {(int)kt.hi[0], (int)kt.hi[1], (int)kt.hi[2], (int)kt.hi[3], 0, 0, 0, 0};
    const int sklo = half ? b1 : b0, skhi = half ? b3 : b2;
    f32x16_t acc = {};
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(klo, qlo, acc, 4, 4, 0, sklo, 0, sqlo);
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(khi, qhi, acc, 4, 4, 0, skhi, 0, sqhi);
    // lane l: query col; element 4j + t is key k0 + 8j + 4*half + t
    if (kScores) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 8 * (i >> 2) + 4 * half + (i & 3);
        if (key < nv) scores[r * N_max + key] = acc[i] + 0.0f;   // an exact zero sum is +0
      }
    }
    // block j = keys [k0 + 8j, k0 + 8j + 8): four values here, four in the
    // other half-wave.  The values are finite, so the IEEE maximum (v_maximum3,
    // -0 below +0) is the total order, and a zero maximum is made +0 as the
    // exact sum gives.
    float bm[4];
    if (k0 + kPfTileKeys <= nv_min) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float m = fmaximum(fmaximum(acc[4 * j], acc[4 * j + 1]), fmaximum(acc[4 * j + 2], acc[4 * j + 3]));
        bm[j] = fmaximum_halves(m) + 0.0f;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float m = -__builtin_inff();
#pragma unroll
        for (int t = 0; t < 4; ++t) m = k0 + 8 * j + 4 * half + t < nv ? fmaximum(m, acc[4 * j + t]) : m;
        bm[j] = fmaximum_halves(m) + 0.0f;   // -inf: no visible key (that block is not written)
      }
    }
    // lanes of the low half stage blocks 0, 1, the high half blocks 2, 3
    st.bm[col][4 * ti + 2 * half] = half ? bm[2] : bm[0];
    st.bm[col][4 * ti + 2 * half + 1] = half ? bm[3] : bm[1];
  };

  KeyTile cur[kPfPrefetch];
#pragma unroll
  for (int i = 0; i < kPfPrefetch; ++i) cur[i] = load_tile(i < ntiles ? i : 0);
  for (int t0 = 0; t0 < ntiles; t0 += kPfPrefetch) {
#pragma unroll
    for (int i = 0; i < kPfPrefetch; ++i) {
      if (t0 + i < ntiles) tile(t0 + i, cur[i]);
      const int nt = t0 + kPfPrefetch + i;
      cur[i] = load_tile(nt < ntiles ? nt : 0);   // the slot's next tile
    }
  }

  // tiles outside the matrix cores' exact range: VALU scores block by block;
  // the maxima take the total order of the keys (values may be -0, infinite or NaN)
  while (unsafe_tiles) {
    const int ti = __builtin_ctz(unsafe_tiles);
    unsafe_tiles &= unsafe_tiles - 1;
    const int k0 = kbeg + kPfTileKeys * ti;
    uint32_t mk[4] = {0u, 0u, 0u, 0u};
    for (int i = 0; i < 16; ++i) {
      const int key = k0 + 8 * (i >> 2) + 4 * half + (i & 3);
      const int kk = key < N ? key : N - 1;
      const float v = pair_score_valu(q_codes + r * 64, q_scales + r * 4, kc + (int64_t)kk * 64, ks + (int64_t)kk * 4);
      if (key < nv) {
        if (kScores) scores[r * N_max + key] = v;
        const uint32_t k = order_key(v);
        const int j = i >> 2;
        mk[0] = (j == 0 && k > mk[0]) ? k : mk[0];
        mk[1] = (j == 1 && k > mk[1]) ? k : mk[1];
        mk[2] = (j == 2 && k > mk[2]) ? k : mk[2];
        mk[3] = (j == 3 && k > mk[3]) ? k : mk[3];
      }
    }
    float bm[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t m = max_halves(mk[j]);
      bm[j] = m ? key_to_float(m) : -__builtin_inff();
    }
    st.bm[col][4 * ti + 2 * half] = half ? bm[2] : bm[0];
    st.bm[col][4 * ti + 2 * half + 1] = half ? bm[3] : bm[1];
  }
  __builtin_amdgcn_wave_barrier();   // the wave's own staging writes precede these reads

  // block maxima out: each store instruction covers whole rows of the chunk's
  // blocks (several rows when a row has fewer than 64); blocks past a row's
  // visible range are not written
  const int nblk_here = (ntiles * kPfTileKeys) >> 3;
  {
    constexpr int kRowsPer = kPfBlocks >= 64 ? 1 : 64 / kPfBlocks;
    constexpr int kStoresPerRow = kPfBlocks >= 64 ? kPfBlocks / 64 : 1;
    const int rsub = kRowsPer > 1 ? lane / kPfBlocks : 0;
    for (int row0 = 0; row0 < kPfQueriesPerWave; row0 += kRowsPer) {
      if (qbase + row0 >= M) break;
      const int row = row0 + rsub;
      int nvr = 0;
#pragma unroll
      for (int j = 0; j < kRowsPer; ++j) {
        const int v = __builtin_amdgcn_readlane(nv, row0 + j);
        nvr = rsub == j ? v : nvr;
      }
#pragma unroll
      for (int h = 0; h < kStoresPerRow; ++h) {
        const int b = kRowsPer > 1 ? lane % kPfBlocks : 64 * h + lane;
        const int blk = (kbeg >> 3) + b;
        if (qbase + row < M && b < nblk_here && 8 * blk < nvr)
          block_max[(seq * M + qbase + row) * nblk_stride + blk] = st.bm[row][b];
      }
    }
  }
  if (kSuper) {
    // super-block maxima from the staged block maxima (total order of the keys):
    // 64 / (chunk/64) query rows per store instruction
    constexpr int kSupers = kPfKeyChunk / 64;
    constexpr int kRowsPer = 64 / kSupers;
    const int sidx = lane % kSupers, sp = (kbeg >> 6) + sidx;
    for (int row0 = 0; row0 < kPfQueriesPerWave; row0 += kRowsPer) {
      if (qbase + row0 >= M) break;
      const int row = row0 + lane / kSupers;
      int nvr = 0;
#pragma unroll
      for (int j = 0; j < kRowsPer; ++j) {
        const int v = __builtin_amdgcn_readlane(nv, row0 + j);
        nvr = lane / kSupers == j ? v : nvr;
      }
      uint32_t m = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int b = 8 * sidx + e;
        const uint32_t k = (b < nblk_here && 8 * ((kbeg >> 3) + b) < nvr) ? order_key(st.bm[row][b]) : 0u;
        m = k > m ? k : m;
      }
      if (qbase + row < M && 8 * sidx < nblk_here && 64 * sp < nvr)
        super_max[(seq * M + qbase + row) * nsup_stride + sp] = key_to_float(m);
    }
  }
}

hipError_t launch_prefill_scan(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                               const uint8_t* k_scales, const int32_t* n_visible, int B, int M, int64_t N_max,
                               float* scores, float* block_max, int64_t nblk_stride, float* super_max,
                               int64_t nsup_stride, hipStream_t stream) {
  dim3 grid((unsigned)((M + kPfQueriesPerWG - 1) / kPfQueriesPerWG), (unsigned)((N_max + kPfKeyChunk - 1) / kPfKeyChunk),
            (unsigned)B);
#define CSA2_PF(S, P)                                                                                            \
  hipLaunchKernelGGL((prefill_scan_kernel<S, P>), grid, dim3(kPfThreads), 0, stream, q_codes, q_scales, k_codes, \
                     k_scales, n_visible, M, N_max, nblk_stride, nsup_stride, scores, block_max, super_max)
  if (scores && super_max) CSA2_PF(true, true);
  else if (scores) CSA2_PF(true, false);
  else if (super_max) CSA2_PF(false, true);
  else CSA2_PF(false, false);
#undef CSA2_PF
  return hipGetLastError();
}

}  // namespace csa2
