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
// Work: a wave holds 32 queries (the B operands, built once) and walks the 1024
// keys of its workgroup's span 32 at a time: two 16-byte buffer loads per lane at
// scalar tile offsets (the cache's own block layout), two MFMAs whose key scale
// bytes are picked by operand select, then per 8-key block in-lane maxima and one
// exchange between the half-waves.  Block maxima are staged in LDS and leave in
// row lines after every 256 keys, so a round's tiles issue no global stores and
// the key loads stay in flight across tiles; the query operands, visibility
// bounds and exactness test are set up once per span.
#include "device_common.h"
#include "kernels.h"

namespace csa2 {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kPfThreads = 256;
constexpr int kPfWaves = kPfThreads / 64;
constexpr int kPfQueriesPerWave = 32;
constexpr int kPfQueriesPerWG = kPfWaves * kPfQueriesPerWave;   // 128
constexpr int kPfKeyChunk = 256;                                // keys per staging round
constexpr int kPfChunks = 4;                                    // staging rounds per workgroup
constexpr int kPfSpan = kPfKeyChunk * kPfChunks;                // keys per workgroup
constexpr int kPfTileKeys = 32;
constexpr int kPfChunkTiles = kPfKeyChunk / kPfTileKeys;        // 8
constexpr int kPfTiles = kPfSpan / kPfTileKeys;                 // one bit each in a 32-bit mask
static_assert(kPfTiles <= 32, "tile mask");
constexpr int kPfPrefetch = 4;                                  // tiles in flight ahead of use
static_assert(kPfChunkTiles % kPfPrefetch == 0, "a staging round ends on a prefetch round");
constexpr int kPfBlocks = kPfKeyChunk / 8;                      // 32 block maxima per query row
constexpr int kPfBmLd = kPfBlocks + 1;                          // padded row: conflict-free column writes
constexpr int kPfBufferConfig = 0x00020000;                     // gfx9 buffer descriptor word 3, raw dwords

// Per-wave staging of a 256-key round's block maxima, written back in row lines
// at the end of the round.
struct PfStage {
  float bm[kPfQueriesPerWave][kPfBmLd];
};

// Workgroup-wide: the staging, the span's key scales, the query scale
// statistics of each wave and the span's tiles that need the VALU path.
struct PfShared {
  PfStage stage[kPfWaves];
  uint32_t kscale[kPfSpan];   // the span's key scale words (zero past the cache)
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
__device__ __forceinline__ float pair_score_valu(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc,
                                                 const uint8_t* ks) {
  float s = 0.0f;
#pragma unroll 1
  for (int b = 0; b < 4; ++b) {
    half2_t qh[16];
    load_query_block(qc + 16 * b, qh);
    const u32x4_t c = *reinterpret_cast<const u32x4_t*>(kc + 16 * b);
    const float v = __builtin_amdgcn_ldexpf(block_dot(c, qh), (int)qs[b] + (int)ks[b] - 254);
    s = b == 0 ? v : s + v;
  }
  return canonical_nan(s);
}

template <bool kScores, bool kSuper>
__global__ __launch_bounds__(kPfThreads) void prefill_scan_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales,
    const int32_t* __restrict__ n_visible, int M, int64_t N_max, int64_t nblk_stride, int64_t nsup_stride,
    float* __restrict__ scores, float* __restrict__ block_max, float* __restrict__ super_max) {
  __shared__ PfShared sh;
  // the wave index is uniform: in a scalar register, so are the wave's row
  // bases and buffer resources
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  PfStage& st = sh.stage[wave];
  const int64_t seq = blockIdx.z;
  const int qbase = blockIdx.x * kPfQueriesPerWG + wave * kPfQueriesPerWave;
  const int kspan = blockIdx.y * kPfSpan;
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
  // One pass over the span's key scales marks the 32-key tiles that are not,
  // and leaves the scale words in LDS for the tiles.
  {
    uint32_t qmin = 255u, qmax = 0u, qspread = 0u;
#pragma unroll
    for (int w = 0; w < kPfWaves; ++w) {
      qmin = min(qmin, sh.qstat[w][0]);
      qmax = max(qmax, sh.qstat[w][1]);
      qspread = max(qspread, sh.qstat[w][2]);
    }
    const int kmin_lo = 130 - (int)qmin, kmax_hi = 368 - (int)qmax, kspread_hi = 9 - (int)qspread;
#pragma unroll
    for (int j = 0; j < kPfSpan / kPfThreads; ++j) {
      const int key = kspan + (int)threadIdx.x + j * kPfThreads;
      const uint32_t sc = key < N ? *reinterpret_cast<const uint32_t*>(k_scales + (seq * N_max + key) * 4) : 0u;
      sh.kscale[key - kspan] = sc;
      const int b0 = (int)(sc & 0xFF), b1 = (int)((sc >> 8) & 0xFF), b2 = (int)((sc >> 16) & 0xFF),
                b3 = (int)(sc >> 24);
      const int kmn = min(min(b0, b1), min(b2, b3)), kmx = max(max(b0, b1), max(b2, b3));
      if (key < N && (kmn < kmin_lo || kmx > kmax_hi || kmx - kmn > kspread_hi))
        atomicOr(&sh.bad_tiles, 1u << ((key - kspan) / kPfTileKeys));
    }
  }
  __syncthreads();
  const uint32_t bad_tiles = sh.bad_tiles;
  if (qbase >= M) return;   // no barriers below: waves leave independently, each with its own staging

  const int kend = kspan + kPfSpan < nv_max ? kspan + kPfSpan : nv_max;
  if (kend <= kspan) return;   // nothing visible in the span: no block of it is written
  const int ntiles = (kend - kspan + kPfTileKeys - 1) / kPfTileKeys;

  // A operands (keys): lane l is key k0 + l%32, K group l/32.  The span's codes
  // as a buffer resource: the tile offset goes into the per-lane offset, which
  // the range check covers, so the lanes of a ragged last tile past the cache
  // read zeros.  (One form for every tile: a branch between two load forms
  // makes the wait counts of the ring unknowable to the compiler.)
  const uint8_t* kc = k_codes + seq * N_max * 64;
  const uint8_t* ks = k_scales + seq * N_max * 4;
  const int nkeys = N - kspan < kPfSpan ? N - kspan : kPfSpan;   // > 0: kspan < nv_max <= N
  const __amdgpu_buffer_rsrc_t kc_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(kc + (int64_t)kspan * 64), 0, nkeys * 64, kPfBufferConfig);
  const int code_off = col * 64 + 16 * half;
  // the key scale word shifted so that byte 0 is block `half` and byte 2 is
  // block 2 + half, the two this lane's K groups take
  const uint32_t scale_shift = 8u * (uint32_t)half;

  struct KeyTile {
    u32x4_t lo, hi;
  };
  auto load_tile = [&](int ti) {
    KeyTile t;
    const int co = code_off + ti * kPfTileKeys * 64;
    t.lo = __builtin_amdgcn_raw_buffer_load_b128(kc_rs, co, 0, 0);
    t.hi = __builtin_amdgcn_raw_buffer_load_b128(kc_rs, co + 32, 0, 0);
    return t;
  };

  uint32_t unsafe_tiles = 0u;
  auto tile = [&](int ti, const KeyTile& kt) {
    const int k0 = kspan + kPfTileKeys * ti;
    const int tl = ti % kPfChunkTiles;   // staging column group of this tile
    if ((bad_tiles >> ti) & 1u) {
      unsafe_tiles |= 1u << ti;   // scored on the VALU at the end of its staging round
      return;
    }
    const int ksc = (int)(sh.kscale[kPfTileKeys * ti + col] >> scale_shift);
    const i32x8_t klo = {(int)kt.lo[0], (int)kt.lo[1], (int)kt.lo[2], (int)kt.lo[3], 0, 0, 0, 0};
    const i32x8_t khi = {(int)kt.hi[0], (int)kt.hi[1], (int)kt.hi[2], (int)kt.hi[3], 0, 0, 0, 0};
    f32x16_t acc = {};
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(klo, qlo, acc, 4, 4, 0, ksc, 0, sqlo);
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(khi, qhi, acc, 4, 4, 2, ksc, 0, sqhi);
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
      // the halves meet in block pairs (0, 2) and (1, 3): one swap each leaves
      // the low half blocks 0 and 1 and the high half blocks 2 and 3, the two
      // it stages
      float m4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        m4[j] = fmaximum(fmaximum(acc[4 * j], acc[4 * j + 1]), fmaximum(acc[4 * j + 2], acc[4 * j + 3]));
      const auto pa = __builtin_amdgcn_permlane32_swap(__float_as_uint(m4[0]), __float_as_uint(m4[2]), false, false);
      const auto pb = __builtin_amdgcn_permlane32_swap(__float_as_uint(m4[1]), __float_as_uint(m4[3]), false, false);
      const float b0 = fmaximum(__uint_as_float(pa[0]), __uint_as_float(pa[1])) + 0.0f;   // block 0 / block 2
      const float b1 = fmaximum(__uint_as_float(pb[0]), __uint_as_float(pb[1])) + 0.0f;   // block 1 / block 3
      st.bm[col][4 * tl + 2 * half] = b0;
      st.bm[col][4 * tl + 2 * half + 1] = b1;
      return;
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
    st.bm[col][4 * tl + 2 * half] = half ? bm[2] : bm[0];
    st.bm[col][4 * tl + 2 * half + 1] = half ? bm[3] : bm[1];
  };

  // tiles of staging round c outside the matrix cores' exact range: VALU
  // scores block by block; the maxima take the total order of the keys (values
  // may be -0, infinite or NaN)
  auto unsafe_round = [&](uint32_t tiles) {
    while (tiles) {
      const int ti = __builtin_ctz(tiles);
      tiles &= tiles - 1;
      const int k0 = kspan + kPfTileKeys * ti;
      const int tl = ti % kPfChunkTiles;
      uint32_t mk[4] = {0u, 0u, 0u, 0u};
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 8 * (i >> 2) + 4 * half + (i & 3);
        const int kk = key < N ? key : N - 1;
        const float v =
            pair_score_valu(q_codes + r * 64, q_scales + r * 4, kc + (int64_t)kk * 64, ks + (int64_t)kk * 4);
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
      st.bm[col][4 * tl + 2 * half] = half ? bm[2] : bm[0];
      st.bm[col][4 * tl + 2 * half + 1] = half ? bm[3] : bm[1];
    }
  };

  // Block maxima of staging round c out, 8 query rows a pass: lane l takes row
  // row0 + l/8 and the round's blocks 4(l%8) .. 4(l%8)+3, so a row's 32 blocks
  // are one 128-byte line in 8 lanes; a super-block (8 blocks) is a lane pair,
  // whose maxima meet in one lane exchange.  Blocks past a row's visible range
  // are not written.  Rounds seen whole by all 32 rows store 16 bytes a lane
  // with global stores from a uniform row base and a 32-bit lane offset (for a
  // buffer store with a register scalar offset the compiler inserts no wait
  // before a vector write may reuse the store's data registers, which then can
  // be overwritten before the store reads them); the maxima are finite or, from
  // the VALU tiles, canonical NaN, infinite or -0, all ranked by the IEEE
  // maximum as by the total order.
  static_assert(kPfBlocks == 32, "a row's blocks in 8 lanes of 4");
  const int sub = lane >> 3, q4 = lane & 7, b0 = 4 * q4;
  const bool vec = (nblk_stride & 3) == 0;   // a lane's first block is then 16-byte aligned
  const bool fast_rows = vec && qbase + kPfQueriesPerWave <= M &&
                         (int64_t)kPfQueriesPerWave * nblk_stride * 4 < 0x7FFFFFFF &&
                         (int64_t)kPfQueriesPerWave * nsup_stride * 4 < 0x7FFFFFFF;
  const int64_t row_first = seq * M + qbase;
  const uint32_t bm_off = (uint32_t)(sub * nblk_stride + b0) * 4u;
  const uint32_t sm_off = (uint32_t)(sub * nsup_stride + (q4 >> 1)) * 4u;

  auto flush_round = [&](int c) {
    const int kbeg = kspan + kPfKeyChunk * c;
    const int nt = ntiles - kPfChunkTiles * c < kPfChunkTiles ? ntiles - kPfChunkTiles * c : kPfChunkTiles;
    const int nblk_here = (nt * kPfTileKeys) >> 3;
    const int blk0 = (kbeg >> 3) + b0;
    __builtin_amdgcn_wave_barrier();   // the wave's own staging writes precede these reads
    if (fast_rows && kbeg + kPfKeyChunk <= nv_min) {
#pragma unroll
      for (int row0 = 0; row0 < kPfQueriesPerWave; row0 += 8) {
        const int row = row0 + sub;
        f32x4_t v;
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = st.bm[row][b0 + t];
        char* bbase = reinterpret_cast<char*>(block_max + (row_first + row0) * nblk_stride + (kbeg >> 3));
        *reinterpret_cast<f32x4_t*>(bbase + bm_off) = v;
        if (kSuper) {
          float m = fmaximum(fmaximum(v[0], v[1]), fmaximum(v[2], v[3]));
          const float o = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0xB1, 0xF, 0xF, false));
          m = fmaximum(m, o);   // lane l ^ 1
          char* sbase = reinterpret_cast<char*>(super_max + (row_first + row0) * nsup_stride + (kbeg >> 6));
          if ((q4 & 1) == 0) *reinterpret_cast<float*>(sbase + sm_off) = m;
        }
      }
    } else {
      for (int row0 = 0; row0 < kPfQueriesPerWave; row0 += 8) {
        if (qbase + row0 >= M) break;
        const int row = row0 + sub;
        const int nvr = __shfl(nv, row);   // lane `row` holds that row's visible count
        const bool rok = qbase + row < M;
        float v[4];
        bool vis[4];
        uint32_t m = 0u;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[t] = st.bm[row][b0 + t];
          vis[t] = b0 + t < nblk_here && 8 * (blk0 + t) < nvr;
          const uint32_t k = vis[t] ? order_key(v[t]) : 0u;
          m = k > m ? k : m;
        }
        float* dst = block_max + (row_first + row) * nblk_stride + blk0;
        if (rok) {
          if (vec && vis[3]) {   // visibility is a prefix: all four visible
            *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
          } else {
#pragma unroll
            for (int t = 0; t < 4; ++t)
              if (vis[t]) dst[t] = v[t];
          }
        }
        if (kSuper) {
          const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false);   // lane l ^ 1
          m = o > m ? o : m;
          const int sidx = q4 >> 1, sp = (kbeg >> 6) + sidx;
          if ((q4 & 1) == 0 && rok && 8 * sidx < nblk_here && 64 * sp < nvr)
            super_max[(row_first + row) * nsup_stride + sp] = key_to_float(m);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();   // these reads precede the next round's staging writes
  };

  // The ring is filled by the loop's own first pass (t0 = -kPfPrefetch, no
  // tiles scored), so every load of it issues from the same code in slot
  // order and each tile waits only for its own two loads.
  KeyTile cur[kPfPrefetch];
#pragma unroll
  for (int i = 0; i < kPfPrefetch; ++i) cur[i] = KeyTile{};
  const int ntiles_r = (ntiles + kPfPrefetch - 1) / kPfPrefetch * kPfPrefetch;
#pragma unroll 1
  for (int t0 = -kPfPrefetch; t0 < ntiles_r; t0 += kPfPrefetch) {
#pragma unroll
    for (int i = 0; i < kPfPrefetch; ++i) {
      if (t0 >= 0 && t0 + i < ntiles) tile(t0 + i, cur[i]);
      const int nt = t0 + kPfPrefetch + i;
      cur[i] = load_tile(nt < ntiles ? nt : 0);   // the slot's next tile
    }
    const int tend = t0 + kPfPrefetch;
    if (t0 >= 0 && (tend % kPfChunkTiles == 0 || tend >= ntiles)) {
      const int c = (tend - 1) / kPfChunkTiles;   // the staging round just scored
      const uint32_t round_unsafe = (unsafe_tiles >> (kPfChunkTiles * c)) & ((1u << kPfChunkTiles) - 1u);
      if (round_unsafe) {
        unsafe_round(round_unsafe << (kPfChunkTiles * c));
        // the ring is loaded again after the call, so that it is not live across it
#pragma unroll
        for (int i = 0; i < kPfPrefetch; ++i) {
          const int nt = tend + i;
          cur[i] = load_tile(nt < ntiles ? nt : 0);
        }
      }
      flush_round(c);
    }
  }
}

hipError_t launch_prefill_scan(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                               const uint8_t* k_scales, const int32_t* n_visible, int B, int M, int64_t N_max,
                               float* scores, float* block_max, int64_t nblk_stride, float* super_max,
                               int64_t nsup_stride, hipStream_t stream) {
  dim3 grid((unsigned)((M + kPfQueriesPerWG - 1) / kPfQueriesPerWG), (unsigned)((N_max + kPfSpan - 1) / kPfSpan),
            (unsigned)B);
#define CSA2_PF(S, P)                                                                                               \
  hipLaunchKernelGGL((prefill_scan_kernel<S, P>), grid, dim3(kPfThreads), 0, stream, q_codes, q_scales,      \
                     k_codes, k_scales, n_visible, M, N_max, nblk_stride, nsup_stride, scores, block_max, super_max)
  if (scores && super_max) CSA2_PF(true, true);
  else if (scores) CSA2_PF(true, false);
  else if (super_max) CSA2_PF(false, true);
  else CSA2_PF(false, false);
#undef CSA2_PF
  return hipGetLastError();
}

}  // namespace csa2
