// Sparse + sliding-window attention over the selected latent entries.
//
// DeepSeek-V4.1-Flash: every layer reads the 512 selected entries of the shared
// MXFP4 latent KV plus its own 128-token FP8 sliding window (fupanwang.com
// article, sections 后 20 层干脆共用一份 KV and 三个方向一起压小缓存).  One softmax
// runs over both sets with value = key: o_h = sum_i softmax_i(q_h . c_i * scale) c_i.
//
// All heads share each entry, so per row this is a dense contraction
// Q[H x 512] . C^T[512 x E] followed by P[H x E] . C[E x 512]: it runs on the bf16
// MFMA units.  Decoded entry values (E2M1 x 2^e, E4M3) are exact in bf16; the
// query and the probabilities are split into hi + lo bf16 parts, so every
// product carries ~16 mantissa bits and accumulates in fp32.
//
// Workgroup = (split, row, head group of 32): 8 waves.  Four waves own 16 heads;
// each keeps the query (hi/lo) and the output accumulator O^T for its quarter of
// the 512 dims in registers, and the four partial S^T tiles are summed through
// LDS in a fixed order.  Entries stream through LDS in chunks of 32 or 64: each
// chunk's rows are gathered whole (one row per wave load) into registers one
// chunk ahead, then decoded once into a row-major LDS copy.  That copy is
// operand A of S^T = C Q^T as is, and operand A of O^T = C^T P^T through the
// transposing LDS reads of gfx950, so no transposed copy is written.  S^T's
// accumulator layout gives each lane the probabilities of exactly the entries
// it must feed as operand B of the second product, so P never leaves
// registers.  An online softmax (log2 domain) runs across chunks; splits > 1
// write partial (o, m, l) that a combine kernel merges.
#include "device_common.h"
#include "kernels.h"

namespace csa2 {

constexpr int kKLd = 512 + 16;             // bf16 row stride of the row-major copy (two chunks of padding)
constexpr float kLazyRescale = 8.0f;       // log2 growth of a running maximum that forces a rescale

// The row-major copy stores 16-byte chunk c of entry row e at chunk
// c ^ ((e >> 2) & 1) of a row padded by two chunks, so rows 0..3 of an aligned
// four start 0, 2, 4, 6 chunks apart (mod 8) and rows 4..7 one chunk further.
// Row writes (8 lanes: one row, 8 chunks), S^T operand reads (8 lanes: rows
// 0..7 mod 8, one chunk) and transposing reads (16 lanes: 4 rows aligned to 4,
// two adjacent chunks) each touch 32 distinct banks, and a lane's addresses
// differ only by constants across its K steps and dim tiles.
__device__ __forceinline__ int kofs(int e, int dim, int x) { return e * kKLd + (((dim >> 3) ^ x) << 3) + (dim & 7); }
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kAttnTargetWorkgroups = 256;   // one per compute unit
constexpr int kAttnChunk = 32;
constexpr int kIdxCap = 1024;                 // staged indices per workgroup (splits keep within it)
constexpr int kAttnThirdsMinChunks = 16;      // chunks a split needs before three streams share it

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct AttnParams {
  const float* q;
  const uint8_t* c_codes;
  const uint8_t* c_scales;
  const int32_t* idx;
  const uint8_t* win;
  const int32_t* win_start;
  const int32_t* win_len;
  float* out;
  float* part_o;      // [R][splits][H][512]
  float* part_ml;     // [R][splits][H][2]
  int64_t N_max;
  int k, win_max, M, H, Tw;
  int splits, chunks_per_split, n_chunks;
  float qscale;       // sm_scale * log2(e)
};

__device__ __forceinline__ bf16x8_t zero_bf16x8() {
  bf16x8_t z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
  return z;
}

__device__ __forceinline__ bf16x8_t decode_latent8(uint32_t wcode, uint32_t scale_byte) {
  // 2^(e-127): e << 23 for e >= 1, the subnormal 2^-127 = 0x00400000 for e = 0
  const float sc = __uint_as_float(max(scale_byte << 23, 0x00400000u));
  const bf16x2_t p0 = fp4x2_to_bf16<0>(wcode, sc);
  const bf16x2_t p1 = fp4x2_to_bf16<1>(wcode, sc);
  const bf16x2_t p2 = fp4x2_to_bf16<2>(wcode, sc);
  const bf16x2_t p3 = fp4x2_to_bf16<3>(wcode, sc);
  return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ bf16x8_t decode_fp8x8(uint32_t w0, uint32_t w1) {
  const f32x2_t f0 = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false);
  const f32x2_t f1 = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
  const f32x2_t f2 = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false);
  const f32x2_t f3 = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
  return bf16x8_t{(__bf16)f0[0], (__bf16)f0[1], (__bf16)f1[0], (__bf16)f1[1],
                  (__bf16)f2[0], (__bf16)f2[1], (__bf16)f3[0], (__bf16)f3[1]};
}

// Entry rows of a chunk: lane l of every wave resolves entry l % CH (its row
// within the sequence and its validity), so a ballot gives the chunk's
// validity mask and any wave can read an entry's row from that lane.
struct EntryRow {
  int32_t row;   // latent row p in [0, N_max), or window row t in [0, Tw); 0 when invalid
  bool valid;
};

__device__ __forceinline__ EntryRow entry_row(const AttnParams& a, int ws0, int E, int e, int32_t p) {
  EntryRow x;
  if (e < a.k) {
    x.valid = p >= 0 && p < a.N_max;
    x.row = x.valid ? p : 0;
  } else {
    const int64_t t = (int64_t)ws0 + (e - a.k);
    x.valid = e < E && t >= 0 && t < a.Tw;
    x.row = x.valid ? (int32_t)t : 0;
  }
  return x;
}

// A wave gathers whole rows: per tile it takes 4 entries (4*eg .. 4*eg+3, eg
// uniform over the wave) and lane l their dims 8l .. 8l+7, so one load
// instruction reads one 256-byte latent (or 512-byte window) row.  The bytes
// stay in registers until the chunk is decoded, one chunk later.
template <int CH, int NT>
struct Gathered {
  static constexpr int kTPT = CH * 16 / NT;   // 4-entry tiles per thread
  uint32_t w0[kTPT][4], w1[kTPT][4];          // latent: 4 code bytes, scale byte; window: 8 bytes
};

// One gathered row as a buffer resource (scalar registers: the row's base and
// its byte length), read at the lane's 32-bit offset: the per-lane address
// needs no 64-bit register pair, and a read past the row returns zero.
constexpr int kBufferConfig = 0x00020000;   // gfx9 buffer descriptor word 3 for raw dword loads
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const uint8_t* row, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(row), 0, (int)bytes, kBufferConfig);
}

// One sequence's latent codes, latent scales and window as buffer resources:
// a row is then one scalar offset away (row * row bytes), which fits 32 bits
// while the sequence has fewer than 2^24 latent rows.
struct SeqRows {
  __amdgpu_buffer_rsrc_t codes, scales, win;
};
constexpr int64_t kFastRows = 1 << 24;

__device__ __forceinline__ SeqRows seq_rows(const AttnParams& a, int64_t seq) {
  SeqRows s;
  const bool fit = a.N_max < kFastRows;
  s.codes = row_rsrc(a.c_codes + seq * a.N_max * 256, fit ? (uint32_t)(a.N_max * 256) : 0u);
  s.scales = row_rsrc(a.c_scales + seq * a.N_max * 16, fit ? (uint32_t)(a.N_max * 16) : 0u);
  s.win = row_rsrc(a.win + seq * a.Tw * 512, (uint32_t)(a.Tw * 512));
  return s;
}

// Chunks whose entries are all valid and all latent (or all window) take one
// branch per chunk; any other chunk (invalid entries, the latent / window
// boundary, rows past 32-bit offsets) goes entry by entry.
enum ChunkKind { kMixed = 0, kLatent = 1, kWindow = 2 };

template <int CH>
__device__ __forceinline__ int chunk_kind(const AttnParams& a, uint64_t mask, int ebase) {
  constexpr uint64_t kChunkBits = CH == 64 ? ~0ull : ((1ull << CH) - 1ull);
  if (mask != kChunkBits) return kMixed;
  if (ebase + CH <= a.k) return a.N_max < kFastRows ? kLatent : kMixed;
  return ebase >= a.k && a.Tw < (1 << 23) ? kWindow : kMixed;
}

template <int CH, int NT>
__device__ __forceinline__ void gather_chunk(const AttnParams& a, const SeqRows& sr, int64_t seq, int32_t row,
                                             uint64_t mask, int kind, int ebase, int w, int lane,
                                             Gathered<CH, NT>& g) {
  constexpr int kTPT = Gathered<CH, NT>::kTPT;
  if (kind == kLatent) {
#pragma unroll
    for (int j = 0; j < kTPT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t re = (uint32_t)__builtin_amdgcn_readlane(row, 4 * (w + j * (NT / 64)) + i);
        g.w0[j][i] = __builtin_amdgcn_raw_buffer_load_b32(sr.codes, 4 * lane, re << 8, 0);
        g.w1[j][i] = __builtin_amdgcn_raw_buffer_load_b8(sr.scales, lane >> 2, re << 4, 0);
      }
  } else if (kind == kWindow) {
#pragma unroll
    for (int j = 0; j < kTPT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t re = (uint32_t)__builtin_amdgcn_readlane(row, 4 * (w + j * (NT / 64)) + i);
        const u32x2_t wb = __builtin_amdgcn_raw_buffer_load_b64(sr.win, 8 * lane, re << 9, 0);
        g.w0[j][i] = wb[0];
        g.w1[j][i] = wb[1];
      }
  } else {
#pragma unroll
    for (int j = 0; j < kTPT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * (w + j * (NT / 64)) + i;
        const uint32_t re = (uint32_t)__builtin_amdgcn_readlane(row, e);
        uint32_t x0 = 0u, x1 = 0u;
        if ((mask >> e) & 1ull) {
          if (ebase + e < a.k) {
            const int64_t o = seq * a.N_max + re;
            x0 = __builtin_amdgcn_raw_buffer_load_b32(row_rsrc(a.c_codes + o * 256, 256), 4 * lane, 0, 0);
            x1 = __builtin_amdgcn_raw_buffer_load_b8(row_rsrc(a.c_scales + o * 16, 16), lane >> 2, 0, 0);
          } else {
            const int64_t o = seq * a.Tw + re;
            const u32x2_t wb = __builtin_amdgcn_raw_buffer_load_b64(row_rsrc(a.win + o * 512, 512), 8 * lane, 0, 0);
            x0 = wb[0];
            x1 = wb[1];
          }
        }
        g.w0[j][i] = x0;
        g.w1[j][i] = x1;
      }
  }
}

// Decode the gathered bytes (zeros for invalid entries) into the row-major
// LDS copy: lane l writes dims 8l .. 8l+7 of each of its entries.
template <int CH, int NT>
__device__ __forceinline__ void store_chunk(const AttnParams& a, const Gathered<CH, NT>& g, uint64_t mask, int kind,
                                            int ebase, int w, int lane, __bf16* sK) {
  constexpr int kTPT = Gathered<CH, NT>::kTPT;
  if (kind == kLatent) {
#pragma unroll
    for (int j = 0; j < kTPT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * (w + j * (NT / 64)) + i;
        *reinterpret_cast<bf16x8_t*>(&sK[kofs(e, 8 * lane, (e >> 2) & 1)]) = decode_latent8(g.w0[j][i], g.w1[j][i]);
      }
  } else if (kind == kWindow) {
#pragma unroll
    for (int j = 0; j < kTPT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * (w + j * (NT / 64)) + i;
        *reinterpret_cast<bf16x8_t*>(&sK[kofs(e, 8 * lane, (e >> 2) & 1)]) = decode_fp8x8(g.w0[j][i], g.w1[j][i]);
      }
  } else {
#pragma unroll
    for (int j = 0; j < kTPT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * (w + j * (NT / 64)) + i;
        bf16x8_t v = zero_bf16x8();
        if ((mask >> e) & 1ull)
          v = ebase + e < a.k ? decode_latent8(g.w0[j][i], g.w1[j][i]) : decode_fp8x8(g.w0[j][i], g.w1[j][i]);
        *reinterpret_cast<bf16x8_t*>(&sK[kofs(e, 8 * lane, (e >> 2) & 1)]) = v;
      }
  }
}

// Two floats rounded to bf16 (round to nearest even), packed low to high.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2v));
}

// max of x over lanes l and l ^ 16 (kHalf: l ^ 32).  v_permlane16_swap
// exchanges the odd 16-lane rows of one register with the even rows of the
// other (v_permlane32_swap: the upper 32 lanes with the lower), so with both
// operands x every lane receives both values of its pair.  The maximum is one
// v_max_f32, where fmaxf would first quiet both operands: a NaN here can only
// come from a NaN score, which makes the row's output NaN whatever this
// maximum is.
template <bool kHalf>
__device__ __forceinline__ float max_lanes(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto p = kHalf ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                       : __builtin_amdgcn_permlane16_swap(u, u, false, false);
  float m;
  asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(p[0]), "v"(p[1]));
  return m;
}

// Four bf16 of a transposed 16x4 tile: in each 16-lane group, lane i receives
// element i % 4 of the 8 bytes that lane 4x + i / 4 addresses, in slot x.
__device__ __forceinline__ bf16x4_t lds_read_tr4(const __bf16* p) {
  typedef __bf16 bf16v4 __attribute__((vector_size(8)));
  typedef __attribute__((address_space(3))) bf16v4 lds_bf16v4;
  const bf16v4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16v4*)(p));
  return bf16x4_t{v[0], v[1], v[2], v[3]};
}

// NP head groups of 16 per workgroup, ND waves per head group (each 512/ND
// dims), CH entries per chunk.  NH = 2: two halves of NP * ND waves each take
// alternate chunks of the split (their own LDS copies, the same barriers) and
// merge their softmax states at the end, so a grid of one workgroup per CU
// keeps two chunks in flight.
template <int NP, int ND, int CH, int NH>
__device__ __forceinline__ void sparse_attn_body(const AttnParams& a) {
  constexpr int kChunk = CH;
  constexpr int NT = NP * ND * 64;    // threads of one half
  constexpr int kDims = 512 / ND;     // dims per wave
  constexpr int kS = kDims / 32;      // K steps of S^T
  constexpr int kM = kDims / 16;      // dim tiles of O^T
  constexpr int kT = CH / 16;         // entry tiles of S^T
  constexpr int kJ = CH / 32;         // K steps of O^T
  constexpr uint64_t kChunkBits = CH == 64 ? ~0ull : ((1ull << CH) - 1ull);
  static_assert(CH == 32 || CH == 64, "chunk of 32 or 64 entries");
  static_assert(NH >= 1 && NH <= 3, "one to three chunk streams");
  __shared__ __attribute__((aligned(16))) __bf16 sKh[NH][kChunk * kKLd];
  __shared__ f32x4 sXh[NH][NP * ND * 64 * kT];   // partial S^T tiles of the ND waves of each head group
  __shared__ int32_t sIdx[kIdxCap];              // rows of the split's entries after each half's first chunk

  // Workgroups reach the 8 XCDs round-robin by linear id; renumbered so that
  // XCD x runs linear ids [x T/8, (x+1) T/8) in order, head group fastest, then
  // split, then row: neighbouring rows, whose selections overlap in a prefill
  // chunk, gather through one L2.  Grids of a size not divisible by 8 keep
  // their order.
  int split, r, hgrp;
  {
    const unsigned gx = gridDim.x, gy = gridDim.y, gz = gridDim.z, T = gx * gy * gz;
    unsigned b = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
    if (T % 8u == 0u) b = (b % 8u) * (T / 8u) + b / 8u;
    hgrp = (int)(b % gz);
    b /= gz;
    split = (int)(b % gx);
    r = (int)(b / gx);
  }
  const int64_t seq = r / a.M;
  const int tid = threadIdx.x;
  const int hf = NH > 1 ? __builtin_amdgcn_readfirstlane(tid / NT) : 0;   // half
  const int tidh = tid - hf * NT;
  __bf16* sK = sKh[hf];
  f32x4* sX = sXh[hf];
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tidh >> 6);
  const int pr = w % NP;       // head group of 16
  const int part = w / NP;     // dims [kDims * part, kDims * (part + 1))
  const int dbase = kDims * part;
  const int g = lane >> 4;     // lane group 0..3
  const int hl = lane & 15;
  const int h = 16 * NP * hgrp + 16 * pr + hl;   // head groups of 16*NP heads
  const int le = lane % kChunk;                          // this lane's entry of a chunk

  int wl = a.win_max > 0 ? a.win_len[r] : 0;
  wl = wl < 0 ? 0 : (wl > a.win_max ? a.win_max : wl);
  const int E = a.k + wl;
  const int ws0 = a.win_max > 0 ? a.win_start[r] : 0;
  const SeqRows sr = seq_rows(a, seq);

  const int c_begin = split * a.chunks_per_split;
  int c_end = c_begin + a.chunks_per_split;
  c_end = c_end < a.n_chunks ? c_end : a.n_chunks;

  // Half hf takes chunks c_begin + hf, c_begin + hf + NH, ...: n_iter rounds
  // for both halves (a round past the split is empty for that half).
  const int n_iter = c_end > c_begin ? (c_end - c_begin + NH - 1) / NH : 0;
  const int c_first = c_begin + hf;

  // Each half's first chunk's indices load first and its rows are gathered as
  // soon as they arrive; the rows of the split's later chunks (-1 for an
  // invalid entry) are resolved once into LDS (visible after the first round's
  // decode barrier), so no chunk waits on a global index load or re-checks its
  // entries in the loop.  The query loads after the first gathers.
  Gathered<CH, NT> gr;
  uint64_t mask = 0ull;   // validity of the gathered chunk's entries (uniform)
  int kind = kMixed;      // and its kind
  const int staged_c0 = c_begin + NH;                                 // first staged chunk
  int n_staged_ch = c_end - staged_c0;
  const int e_chunks = (E + kChunk - 1) / kChunk;                     // chunks holding entries
  n_staged_ch = n_staged_ch < e_chunks - staged_c0 ? n_staged_ch : e_chunks - staged_c0;
  n_staged_ch = n_staged_ch < kIdxCap / kChunk ? n_staged_ch : kIdxCap / kChunk;   // (a longer split loads the rest)
  n_staged_ch = n_staged_ch > 0 ? n_staged_ch : 0;
  const int n_staged = n_staged_ch * kChunk;
  {
    constexpr int kStage = (kIdxCap + NH * NT - 1) / (NH * NT);
    const int e0 = c_first * kChunk + le;
    const int32_t p0 = (c_first < c_end && e0 < a.k) ? a.idx[(int64_t)r * a.k + e0] : -1;
    int32_t st[kStage];
#pragma unroll
    for (int j = 0; j < kStage; ++j) {
      const int e = staged_c0 * kChunk + tid + j * NH * NT;
      st[j] = tid + j * NH * NT < n_staged && e < a.k ? a.idx[(int64_t)r * a.k + e] : -1;
    }
    __builtin_amdgcn_sched_barrier(0);
    if (c_first < c_end) {
      const EntryRow x = entry_row(a, ws0, E, e0, p0);
      mask = __ballot(x.valid) & kChunkBits;
      kind = chunk_kind<CH>(a, mask, c_first * kChunk);
      gather_chunk<CH, NT>(a, sr, seq, x.row, mask, kind, c_first * kChunk, w, lane, gr);
    }
#pragma unroll
    for (int j = 0; j < kStage; ++j) {
      const int t = tid + j * NH * NT;
      if (t < n_staged) {
        const EntryRow x = entry_row(a, ws0, E, staged_c0 * kChunk + t, st[j]);
        sIdx[t] = x.valid ? x.row : -1;
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // query operands (B of S^T = C Q^T): head h, dims dbase + 32s + 8g .. +8,
  // prescaled and split into bf16 hi + lo
  bf16x8_t qhi[kS], qlo[kS];
  {
    const float* qp = a.q + ((int64_t)r * a.H + h) * 512 + dbase + 8 * g;
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      const f32x4 q0 = *reinterpret_cast<const f32x4*>(qp + 32 * s);
      const f32x4 q1 = *reinterpret_cast<const f32x4*>(qp + 32 * s + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = (e < 4 ? q0[e] : q1[e - 4]) * a.qscale;
        const __bf16 hi = (__bf16)v;
        qhi[s][e] = hi;
        qlo[s][e] = (__bf16)(v - (float)hi);
      }
    }
  }

  f32x4 oacc[kM];
#pragma unroll
  for (int m = 0; m < kM; ++m) oacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  for (int it = 0; it < n_iter; ++it) {
    // Three barriers a round whatever the chunk holds, the same for both
    // halves; a chunk with no valid entry (past E, past the split) does no work.
    const int c = c_first + NH * it;
    const int ebase = c * kChunk;
    const uint64_t cm = mask;   // this chunk's validity
    const int ck = kind;
    __syncthreads();   // the previous round's LDS reads are done
    if (cm != 0ull) store_chunk<CH, NT>(a, gr, cm, ck, ebase, w, lane, sK);
    __syncthreads();   // decoded rows (and, in the first round, the staged indices) visible
    // this half's next chunk's rows: in flight during this chunk's products
    mask = 0ull;
    kind = kMixed;
    const int cn = c + NH;
    if (cn < c_end && cn * kChunk < E) {
      int32_t row;
      if (cn - staged_c0 < n_staged_ch) {
        row = sIdx[(cn - staged_c0) * kChunk + le];
      } else {
        const int e = cn * kChunk + le;
        const EntryRow x = entry_row(a, ws0, E, e, e < a.k ? a.idx[(int64_t)r * a.k + e] : -1);
        row = x.valid ? x.row : -1;
      }
      mask = __ballot(row >= 0) & kChunkBits;
      kind = chunk_kind<CH>(a, mask, cn * kChunk);
      gather_chunk<CH, NT>(a, sr, seq, row, mask, kind, cn * kChunk, w, lane, gr);
    }

    // 3. partial S^T[CH entries x 16 heads] over this wave's kDims dims
    // (row 16t + hl, dims dbase + 32s + 8g .. +8: chunk g of K step s, stored at chunk g ^ x)
    const int s_base = hl * kKLd + dbase + 8 * (g ^ ((hl >> 2) & 1));
    f32x4 sacc[kT];
#pragma unroll
    for (int t = 0; t < kT; ++t) sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (cm != 0ull) {
#pragma unroll
    for (int s = 0; s < kS; ++s) {
#pragma unroll
      for (int t = 0; t < kT; ++t) {
        const bf16x8_t A =
            *reinterpret_cast<const bf16x8_t*>(&sK[s_base + t * 16 * kKLd + 32 * s]);
        sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, qhi[s], sacc[t], 0, 0, 0);
        sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, qlo[s], sacc[t], 0, 0, 0);
      }
    }
    // one operand read ahead of each pair of products
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < kS * kT - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    // the ND waves of a head group add their partial sums in part order
    {
      f32x4* mine = sX + (pr * ND + part) * kT * 64 + lane;
#pragma unroll
      for (int t = 0; t < kT; ++t) mine[64 * t] = sacc[t];
    }
    }   // cm != 0
    __syncthreads();
    if (cm == 0ull) continue;
#pragma unroll
    for (int t = 0; t < kT; ++t) {
      f32x4 acc = sX[((pr * ND + 0) * kT + t) * 64 + lane];
#pragma unroll
      for (int p = 1; p < ND; ++p) acc += sX[((pr * ND + p) * kT + t) * 64 + lane];
      sacc[t] = acc;
    }

    // 4. online softmax (lane holds entries 16t + 4g + i of head h).  The
    // running maximum m_run only moves when a head's chunk maximum exceeds it
    // by more than 2^kLazyRescale (then every lane of the wave rescales): the
    // probabilities stay below 2^kLazyRescale, and l and the partials carry
    // the same m_run, so the result is the same softmax.
    if (cm != kChunkBits) {
      const uint64_t mine = cm >> (4 * g);   // bit 16t + i: entry 16t + 4g + i
#pragma unroll
      for (int t = 0; t < kT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!((mine >> (16 * t + i)) & 1ull)) sacc[t][i] = -__builtin_inff();
    }
    float mloc = -__builtin_inff();
#pragma unroll
    for (int t = 0; t < kT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, sacc[t][i]);
    mloc = max_lanes<false>(mloc);   // lanes l ^ 16
    mloc = max_lanes<true>(mloc);    // lanes l ^ 32
    if (__ballot(mloc > m_run + kLazyRescale) != 0ull) {
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int m = 0; m < kM; ++m) oacc[m] *= alpha;
      m_run = m_new;
    }
    // v_exp_f32 directly: arguments lie in [-inf, kLazyRescale], and a result
    // below 2^-126 (flushed to zero here) is below any weight that can move
    // the output
    float psum;
#pragma unroll
    for (int t = 0; t < kT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(sacc[t][i] - m_run);
        sacc[t][i] = p;
        psum = t == 0 && i == 0 ? p : psum + p;
      }
    l_run += psum;

    // 5. O^T[kDims dims x 16 heads] += C^T P^T, k-steps of 32 entries.  The
    // operand C^T is read from the row-major copy with transposing LDS reads:
    // lane (g, hl) receives dim dbase + 16m + hl of entries 32j + 4g + 0..3
    // (elements 0..3) and 32j + 16 + 4g + 0..3 (elements 4..7), the entries whose
    // probabilities it holds.
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      // hi = bf16(p) two at a time, lo = bf16(p - hi)
      u32x4_t bh, bl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = i < 2 ? sacc[2 * j][2 * i] : sacc[2 * j + 1][2 * i - 4];
        const float p1 = i < 2 ? sacc[2 * j][2 * i + 1] : sacc[2 * j + 1][2 * i - 3];
        const uint32_t h = pack_bf16(p0, p1);
        bh[i] = h;
        bl[i] = pack_bf16(p0 - __uint_as_float(h << 16), p1 - __uint_as_float(h & 0xffff0000u));
      }
      const bf16x8_t bhi = __builtin_bit_cast(bf16x8_t, bh);
      const bf16x8_t blo = __builtin_bit_cast(bf16x8_t, bl);
      // rows e0 and e0 + 16 (both with (e >> 2) & 1 = g & 1), dims dbase + 16m +
      // 4 (hl & 3) .. +4: chunk 2m + ((hl & 3) >> 1), stored at that chunk ^ (g & 1)
      const int e0 = 32 * j + 4 * g + (hl >> 2);
      const int v_base = e0 * kKLd + dbase + 8 * (((hl & 3) >> 1) ^ (g & 1)) + 4 * (hl & 1);
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        const bf16x4_t lo4 = lds_read_tr4(&sK[v_base + 16 * m]);
        const bf16x4_t hi4 = lds_read_tr4(&sK[v_base + 16 * kKLd + 16 * m]);
        const bf16x8_t A = bf16x8_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        oacc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, bhi, oacc[m], 0, 0, 0);
        oacc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, blo, oacc[m], 0, 0, 0);
      }
      // the next dim tile's two transposing reads in flight during each pair of
      // products
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int m = 0; m < kM - 1; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
  }

  if constexpr (NH > 1) {
    // the streams' states meet: thread t of stream q holds the same heads and
    // dims as thread t of stream 0, over the other chunks of the split;
    // streams 1 .. NH-1 leave theirs in the chunk buffers, stream 0 adds them
    // in stream order
    __syncthreads();   // every chunk's LDS reads are done
    float* po = reinterpret_cast<float*>(&sKh[0][0]);   // per stream q >= 1: kM x 4 floats a thread
    float* pml = reinterpret_cast<float*>(&sXh[0][0]);  // per stream q >= 1: m and l a thread
    static_assert((NH - 1) * NT * kM * 4 * sizeof(float) <= sizeof(sKh) &&
                      2 * (NH - 1) * NT * sizeof(float) <= sizeof(sXh),
                  "the merge fits the chunk buffers");
    if (hf >= 1) {
      float* pq = po + (hf - 1) * NT * kM * 4;
#pragma unroll
      for (int m = 0; m < kM; ++m) *reinterpret_cast<f32x4*>(pq + (m * NT + tidh) * 4) = oacc[m];
      pml[2 * (hf - 1) * NT + tidh] = m_run;
      pml[(2 * (hf - 1) + 1) * NT + tidh] = l_run;
    }
    __syncthreads();
    if (hf >= 1) return;   // no barrier follows
    float M = m_run;
#pragma unroll
    for (int q = 1; q < NH; ++q) M = fmaxf(M, pml[2 * (q - 1) * NT + tidh]);
    const float a0 = m_run == -__builtin_inff() ? 0.f : exp2f(m_run - M);
    l_run = l_run * a0;
#pragma unroll
    for (int m = 0; m < kM; ++m) oacc[m] = oacc[m] * a0;
#pragma unroll
    for (int q = 1; q < NH; ++q) {
      const float mq = pml[2 * (q - 1) * NT + tidh], lq = pml[(2 * (q - 1) + 1) * NT + tidh];
      const float aq = mq == -__builtin_inff() ? 0.f : exp2f(mq - M);
      l_run = l_run + lq * aq;
      const float* pq = po + (q - 1) * NT * kM * 4;
#pragma unroll
      for (int m = 0; m < kM; ++m) oacc[m] = oacc[m] + *reinterpret_cast<const f32x4*>(pq + (m * NT + tidh) * 4) * aq;
    }
    m_run = M;
  }
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot = l_tot + __shfl_xor(l_tot, 32, 64);
  if (a.splits == 1) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    float* op = a.out + ((int64_t)r * a.H + h) * 512 + dbase + 4 * g;
#pragma unroll
    for (int m = 0; m < kM; ++m) *reinterpret_cast<f32x4*>(op + 16 * m) = oacc[m] * inv;
  } else {
    const int64_t slot = ((int64_t)r * a.splits + split) * a.H + h;
    float* op = a.part_o + slot * 512 + dbase + 4 * g;
#pragma unroll
    // streaming stores: the partials are read once, by the combine
    for (int m = 0; m < kM; ++m) __builtin_nontemporal_store(oacc[m], reinterpret_cast<f32x4*>(op + 16 * m));
    if (g == 0 && part == 0) {
      __builtin_nontemporal_store(m_run, &a.part_ml[2 * slot]);
      __builtin_nontemporal_store(l_tot, &a.part_ml[2 * slot + 1]);
    }
  }
}

// 8-wave workgroups (32 heads).  With 32-entry chunks two fit a compute unit
// (54 KB of LDS each) when a wave keeps to 128 registers (a few spill), so one
// workgroup's loads overlap the other's products: better once the grid holds
// several workgroups per compute unit, worse for a grid that does not.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4))) void sparse_attn_kernel_h32c32_2wg(
    AttnParams a) {
  sparse_attn_body<2, 4, 32, 1>(a);
}
__global__ __launch_bounds__(512, 1) void sparse_attn_kernel_h32c32(AttnParams a) { sparse_attn_body<2, 4, 32, 1>(a); }
// One workgroup per CU over splits of several chunks: 16 waves, two halves on
// alternate chunks.
__global__ __launch_bounds__(1024, 1) void sparse_attn_kernel_h32c32_halves(AttnParams a) {
  sparse_attn_body<2, 4, 32, 2>(a);
}
__global__ __launch_bounds__(512, 1) void sparse_attn_kernel_h16c32_halves(AttnParams a) {
  sparse_attn_body<1, 4, 32, 2>(a);
}
// Three streams of 4 waves on every third chunk (12 waves, 130 KB of LDS), for
// 16-head grids of one workgroup per CU with long splits: a third stream makes
// each round about 40% longer, which pays only where it saves many rounds
// (64 rows x 20 chunks: 10 -> 7 rounds, 34.0 -> 33.0 us a layer; 10-chunk
// splits: 27 -> 28.5 us, not taken).
__global__ __launch_bounds__(768, 1) void sparse_attn_kernel_h16c32_thirds(AttnParams a) {
  sparse_attn_body<1, 4, 32, 3>(a);
}
__global__ __launch_bounds__(512, 1) void sparse_attn_kernel_h32c64(AttnParams a) { sparse_attn_body<2, 4, 64, 1>(a); }
__global__ __launch_bounds__(256) void sparse_attn_kernel_h16c32(AttnParams a) { sparse_attn_body<1, 4, 32, 1>(a); }
__global__ __launch_bounds__(256, 1) void sparse_attn_kernel_h16c64(AttnParams a) { sparse_attn_body<1, 4, 64, 1>(a); }

// Merge split partials: out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// One workgroup per (row, head), V consecutive output dims per thread (512 / V
// threads).  Wave 0 reads the splits' (m, l) pairs and turns them into weights
// in LDS; every thread's dims of the first 32 / V splits are loaded before
// that, so the weights and the partials arrive in one memory round trip.  Few
// splits take V = 4 (small workgroups: a grid of many rows is resident at
// once), many splits V = 1 (all of them in flight per thread).
constexpr int kMaxSplits = kAttnTargetWorkgroups;   // attn_splits never exceeds it

template <int V>
__global__ __launch_bounds__(512 / V) void attn_combine_kernel(const float* __restrict__ part_o,
                                                               const float* __restrict__ part_ml, int splits,
                                                               int H, float* __restrict__ out) {
  constexpr int kGroup = 32 / V;
  typedef float vec_t __attribute__((ext_vector_type(V)));
  __shared__ float sw[kMaxSplits];   // 2^(m_s - M), 0 for splits that saw nothing
  __shared__ float sL;
  const int r = blockIdx.y;
  const int h = blockIdx.x;
  const int d = V * threadIdx.x;
  const int64_t base = (int64_t)r * splits * H + h;     // slot of split s: base + s*H
  float m[kMaxSplits / 64], l[kMaxSplits / 64];
  if (threadIdx.x < 64) {
#pragma unroll
    for (int j = 0; j < kMaxSplits / 64; ++j) {
      const int sidx = 64 * j + threadIdx.x;
      m[j] = -__builtin_inff();
      l[j] = 0.f;
      if (sidx < splits) {
        m[j] = part_ml[2 * (base + (int64_t)sidx * H)];
        l[j] = part_ml[2 * (base + (int64_t)sidx * H) + 1];
      }
    }
  }
  vec_t ov[kGroup];
#pragma unroll
  for (int j = 0; j < kGroup; ++j)
    ov[j] = j < splits ? *reinterpret_cast<const vec_t*>(part_o + (base + (int64_t)j * H) * 512 + d) : vec_t(0.f);
  if (threadIdx.x < 64) {
    // wave 0: M = max_s m_s, then the weights and L = sum_s w_s l_s in split order
    float M = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < kMaxSplits / 64; ++j) M = fmaxf(M, m[j]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    // L: per lane in j order, then a fixed butterfly
    float L = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxSplits / 64; ++j) {
      const int sidx = 64 * j + threadIdx.x;
      const float w = (M == -__builtin_inff() || m[j] == -__builtin_inff()) ? 0.f : exp2f(m[j] - M);
      if (sidx < splits) sw[sidx] = w;
      L += w * l[j];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off, 64);
    if (threadIdx.x == 0) sL = L;
  }
  __syncthreads();
  vec_t acc = vec_t(0.f);
  for (int s0 = 0; s0 < splits; s0 += kGroup) {
    if (s0 > 0) {
#pragma unroll
      for (int j = 0; j < kGroup; ++j)
        ov[j] = s0 + j < splits ? *reinterpret_cast<const vec_t*>(part_o + (base + (int64_t)(s0 + j) * H) * 512 + d)
                                : vec_t(0.f);
    }
#pragma unroll
    for (int j = 0; j < kGroup; ++j)
      if (s0 + j < splits) acc += sw[s0 + j] * ov[j];
  }
  const float L = sL;
  *reinterpret_cast<vec_t*>(out + ((int64_t)r * H + h) * 512 + d) = L > 0.f ? acc / L : vec_t(0.f);
}

// Head groups of 16 heads per workgroup (32 when H allows).
// (16 where 32-head groups leave compute units idle: at 64 rows x 4 groups
// every compute unit gets a workgroup with one split a row, two halves share
// the row's chunks and no combine runs; with fewer rows the splits, and the
// partials the combine reads, halve; a single row's one-chunk workgroups also
// finish sooner at 16 heads: 4,096-entry decode step 24.3 -> 22.9 us)
static int attn_group_heads(int R, int H) {
  if (H < 32) return 16;
  const int64_t g32 = (int64_t)R * (H / 32);
  return H % 16 == 0 && g32 < kAttnTargetWorkgroups ? 16 : 32;
}

// Entries per chunk: 32 keeps a workgroup's LDS at 54 KB, so two workgroups
// share a compute unit and one's loads overlap the other's products.
static int attn_chunk(int R, int H, int k_plus_win) {
  (void)R;
  (void)H;
  (void)k_plus_win;
  return kAttnChunk;
}

// 16-head grids with fewer head groups than compute units run independent
// 4-wave workgroups, two a compute unit (a target of 512), rather than
// workgroups of two halves: decode at 4 rows x 4 groups 55.4 -> 54.1 us (one
// chunk a workgroup), 20 rows x 4 groups 82.5 -> 80.6 us, 32 rows x 4 groups
// unchanged.
static bool attn_small16(int R, int H) {
  return attn_group_heads(R, H) == 16 && (int64_t)R * (H / 16) < kAttnTargetWorkgroups;
}

// Splits of a row's entry chunks: enough workgroups to give every compute unit
// about one (a workgroup's LDS fills a compute unit), or two for small 16-head
// grids, never more splits than chunks or than the combine takes, and chunks
// spread evenly over the splits.
int attn_splits(int R, int H, int k_plus_win) {
  const int ch = attn_chunk(R, H, k_plus_win);
  const int n_chunks = (k_plus_win + ch - 1) / ch;
  if (n_chunks <= 1) return 1;
  const int gh = attn_group_heads(R, H);
  const int64_t groups = (int64_t)R * (H > 0 ? (H + gh - 1) / gh : 1);
  const int64_t target = attn_small16(R, H) ? 2 * kAttnTargetWorkgroups : kAttnTargetWorkgroups;
  int64_t want = (target + groups - 1) / groups;
  if (want < 1) want = 1;
  if (want > n_chunks) want = n_chunks;
  if (want > kMaxSplits) want = kMaxSplits;
  const int cps = (int)((n_chunks + want - 1) / want);
  return (n_chunks + cps - 1) / cps;
}

size_t attn_workspace_bytes(int R, int H, int k_plus_win) {
  const int splits = attn_splits(R, H, k_plus_win);
  if (splits <= 1) return 0;
  return (size_t)R * splits * H * (512 + 2) * sizeof(float);
}

hipError_t launch_sparse_attn(const AttnLaunch& L, hipStream_t stream) {
  const int R = L.B * L.M;
  AttnParams a;
  a.q = L.q;
  a.c_codes = L.c_codes;
  a.c_scales = L.c_scales;
  a.idx = L.idx;
  a.win = L.win;
  a.win_start = L.win_start;
  a.win_len = L.win_len;
  a.out = L.out;
  a.N_max = L.N_max;
  a.k = L.k;
  a.win_max = L.win_max;
  a.M = L.M;
  a.H = L.H;
  a.Tw = L.Tw;
  a.qscale = L.sm_scale * kLog2e;
  const int ch = attn_chunk(R, L.H, L.k + L.win_max);
  a.n_chunks = (L.k + L.win_max + ch - 1) / ch;
  a.splits = attn_splits(R, L.H, L.k + L.win_max);
  a.chunks_per_split = (a.n_chunks + a.splits - 1) / a.splits;
  if (a.n_chunks == 0) {
    a.splits = 1;
    a.chunks_per_split = 0;
  }
  // Workgroups of 32 heads (8 waves); more heads split over blockIdx.z.  Four
  // waves of 128 dims per 16-head group keep every wave's chain of products
  // short and leave two waves per SIMD to overlap LDS and matrix-core work.
  if (L.H % 16 != 0 || L.H < 16) return hipErrorInvalidValue;
  const int NP = attn_group_heads(R, L.H) / 16;
  if (L.H % (16 * NP) != 0) return hipErrorInvalidValue;
  const int64_t n_wg = (int64_t)a.splits * R * (L.H / (16 * NP));
  const bool many = n_wg > 4 * kAttnTargetWorkgroups;
  // a grid of one workgroup per CU whose splits hold several chunks runs
  // 16-wave workgroups whose halves take alternate chunks (c4: 47 -> 41 us per
  // layer); splits of one chunk keep the 8-wave kernel (more workgroups)
  const bool halves = ch == 32 && !many && a.chunks_per_split >= 2 && !attn_small16(R, L.H);
  a.part_o = nullptr;
  a.part_ml = nullptr;
  if (a.splits > 1) {
    a.part_o = static_cast<float*>(L.workspace);
    a.part_ml = a.part_o + (size_t)R * a.splits * L.H * 512;
  }
  dim3 grid((unsigned)a.splits, (unsigned)R, (unsigned)(L.H / (16 * NP)));
  if (NP == 2 && ch == 32 && many)
    hipLaunchKernelGGL(sparse_attn_kernel_h32c32_2wg, grid, dim3(512), 0, stream, a);
  else if (halves && NP == 2)
    hipLaunchKernelGGL(sparse_attn_kernel_h32c32_halves, grid, dim3(1024), 0, stream, a);
  else if (halves && NP == 1 && a.chunks_per_split >= kAttnThirdsMinChunks)
    hipLaunchKernelGGL(sparse_attn_kernel_h16c32_thirds, grid, dim3(768), 0, stream, a);
  else if (halves)
    hipLaunchKernelGGL(sparse_attn_kernel_h16c32_halves, grid, dim3(512), 0, stream, a);
  else if (NP == 2 && ch == 32)
    hipLaunchKernelGGL(sparse_attn_kernel_h32c32, grid, dim3(512), 0, stream, a);
  else if (NP == 2)
    hipLaunchKernelGGL(sparse_attn_kernel_h32c64, grid, dim3(512), 0, stream, a);
  else if (ch == 32)
    hipLaunchKernelGGL(sparse_attn_kernel_h16c32, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(sparse_attn_kernel_h16c64, grid, dim3(256), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.splits == 1) return err;
  const dim3 cgrid((unsigned)L.H, (unsigned)R);
  if (a.splits <= 8)
    hipLaunchKernelGGL(attn_combine_kernel<4>, cgrid, dim3(128), 0, stream, a.part_o, a.part_ml, a.splits, L.H, L.out);
  else if (a.splits <= 16)
    hipLaunchKernelGGL(attn_combine_kernel<2>, cgrid, dim3(256), 0, stream, a.part_o, a.part_ml, a.splits, L.H, L.out);
  else
    hipLaunchKernelGGL(attn_combine_kernel<1>, cgrid, dim3(512), 0, stream, a.part_o, a.part_ml, a.splits, L.H, L.out);
  return hipGetLastError();
}

}  // namespace csa2
