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
// chunk's rows are gathered into registers one chunk ahead, then decoded once
// into a row-major copy (operand A of S^T = C Q^T) and a transposed copy
// (operand A of O^T = C^T P^T).  S^T's accumulator layout gives each lane the
// probabilities of exactly the entries it must feed as operand B of the second
// product, so P never leaves registers.  An online softmax (log2 domain) runs
// across chunks; splits > 1 write partial (o, m, l) that a combine kernel merges.
#include "device_common.h"
#include "kernels.h"

namespace csa2 {

constexpr int kKLd = 512 + 8;              // bf16 row stride of the row-major copy
template <int CH>
constexpr int vld() { return CH + 8; }     // bf16 row stride of the transposed copy
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kAttnTargetWorkgroups = 256;   // one per compute unit
constexpr int kAttnChunk = 32;

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

enum { kLatentRows = 0, kWindowRows = 1, kMixedRows = 2 };

__device__ __forceinline__ bf16x8_t decode_latent8(uint32_t wcode, uint32_t scale_byte) {
  const float sc = e8m0_to_f32(scale_byte);
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

// A thread covers 4 consecutive entries of a chunk (4*eg .. 4*eg+3, the same
// four in every tile it owns) and 8 dims of each per tile (dims 8*dg .. +8).
// Its entries' raw bytes are gathered into registers one chunk ahead of the
// decode, so a chunk's row loads are in flight during the previous chunk's
// products.
template <int CH, int NT>
struct Gathered {
  static constexpr int kEG = CH / 4;            // entry groups of 4
  static constexpr int kTPT = kEG * 64 / NT;    // tiles per thread
  uint32_t w0[kTPT][4], w1[kTPT][4];            // latent: 4 code bytes, scale byte; window: 8 bytes
};

// Selected indices of this thread's entries of the chunk at ebase (-1 beyond k).
__device__ __forceinline__ void load_entry_ids(const AttnParams& a, int r, int ebase, int eg, int32_t (&ix)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = ebase + 4 * eg + i;
    ix[i] = e < a.k ? a.idx[(int64_t)r * a.k + e] : -1;
  }
}

// Row offsets of this thread's entries (latent row seq*N_max + p, window row
// seq*Tw + t) and their validity bits (bit i: entry 4*eg + i).
__device__ __forceinline__ uint32_t entry_rows(const AttnParams& a, int64_t seq, int ws0, int E, int ebase, int eg,
                                               const int32_t (&ix)[4], int64_t (&off)[4]) {
  uint32_t vb = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = ebase + 4 * eg + i;
    bool valid;
    if (e < a.k) {
      const int64_t p = ix[i];
      valid = p >= 0 && p < a.N_max;
      off[i] = seq * a.N_max + p;
    } else {
      const int64_t t = (int64_t)ws0 + (e - a.k);
      valid = e < E && t >= 0 && t < a.Tw;
      off[i] = seq * a.Tw + t;
    }
    vb |= valid ? 1u << i : 0u;
  }
  return vb;
}

// Issue the loads of this thread's valid entries (invalid ones read nothing).
template <int NT, int KIND, int CH>
__device__ __forceinline__ void gather_chunk(const AttnParams& a, const int64_t (&off)[4], uint32_t vb, int ebase,
                                             int tid, Gathered<CH, NT>& g) {
  constexpr int kEG = Gathered<CH, NT>::kEG;
  const int eg = tid % kEG;
#pragma unroll
  for (int j = 0; j < Gathered<CH, NT>::kTPT; ++j) {
    const int dg = (tid + j * NT) / kEG;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t x0 = 0u, x1 = 0u;
      if ((vb >> i) & 1u) {
        const bool lat = KIND == kLatentRows || (KIND == kMixedRows && ebase + 4 * eg + i < a.k);
        if (lat) {
          x0 = *reinterpret_cast<const uint32_t*>(a.c_codes + off[i] * 256 + 4 * dg);
          x1 = a.c_scales[off[i] * 16 + (dg >> 2)];
        } else {
          const u32x2_t wb = *reinterpret_cast<const u32x2_t*>(a.win + off[i] * 512 + 8 * dg);
          x0 = wb[0];
          x1 = wb[1];
        }
      }
      g.w0[j][i] = x0;
      g.w1[j][i] = x1;
    }
  }
}

// Decode the gathered bytes (zeros for invalid entries) into the row-major and
// the transposed LDS copies.
template <int NT, int KIND, int CH>
__device__ __forceinline__ void store_chunk(const AttnParams& a, const Gathered<CH, NT>& g, uint32_t vb, int ebase,
                                            int tid, __bf16* sK, __bf16* sVt) {
  constexpr int kVLd = vld<CH>();
  constexpr int kEG = Gathered<CH, NT>::kEG;
  const int eg = tid % kEG;
#pragma unroll
  for (int j = 0; j < Gathered<CH, NT>::kTPT; ++j) {
    const int dg = (tid + j * NT) / kEG;
    bf16x8_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * eg + i;
      const bool lat = KIND == kLatentRows || (KIND == kMixedRows && ebase + e < a.k);
      if (!((vb >> i) & 1u))
        v[i] = zero_bf16x8();
      else if (lat)
        v[i] = decode_latent8(g.w0[j][i], g.w1[j][i]);
      else
        v[i] = decode_fp8x8(g.w0[j][i], g.w1[j][i]);
      *reinterpret_cast<bf16x8_t*>(&sK[e * kKLd + 8 * dg]) = v[i];
    }
#pragma unroll
    for (int d = 0; d < 8; ++d)
      *reinterpret_cast<bf16x4_t*>(&sVt[(8 * dg + d) * kVLd + 4 * eg]) = bf16x4_t{v[0][d], v[1][d], v[2][d], v[3][d]};
  }
}

// The chunk's row kind (uniform over the workgroup).
__device__ __forceinline__ int chunk_kind(int ebase, int CHn, int k) {
  return ebase + CHn <= k ? kLatentRows : (ebase >= k ? kWindowRows : kMixedRows);
}

// NP head groups of 16 per workgroup, ND waves per head group (each 512/ND
// dims), CH entries per chunk
template <int NP, int ND, int CH>
__device__ __forceinline__ void sparse_attn_body(const AttnParams& a) {
  constexpr int kChunk = CH;
  constexpr int kVLd = vld<CH>();
  constexpr int NT = NP * ND * 64;
  constexpr int kDims = 512 / ND;     // dims per wave
  constexpr int kS = kDims / 32;      // K steps of S^T
  constexpr int kM = kDims / 16;      // dim tiles of O^T
  constexpr int kT = CH / 16;         // entry tiles of S^T
  constexpr int kJ = CH / 32;         // K steps of O^T
  static_assert(NP * ND * 64 * kT * 16 <= kChunk * kKLd * 2, "S^T partials fit in the row-major copy");
  __shared__ __attribute__((aligned(16))) __bf16 sK[kChunk * kKLd];
  __shared__ __attribute__((aligned(16))) __bf16 sVt[512 * kVLd];

  const int split = blockIdx.x;
  const int r = blockIdx.y;
  const int64_t seq = r / a.M;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int pr = w % NP;       // head group of 16
  const int part = w / NP;     // dims [kDims * part, kDims * (part + 1))
  const int dbase = kDims * part;
  const int g = lane >> 4;     // lane group 0..3
  const int hl = lane & 15;
  const int h = 16 * NP * blockIdx.z + 16 * pr + hl;   // head groups of 16*NP heads across blockIdx.z
  constexpr int kEG = Gathered<CH, NT>::kEG;
  const int eg = tid % kEG;    // this thread's entry group (lanes 0..kEG-1 of every wave: groups 0..kEG-1)

  int wl = a.win_max > 0 ? a.win_len[r] : 0;
  wl = wl < 0 ? 0 : (wl > a.win_max ? a.win_max : wl);
  const int E = a.k + wl;
  const int ws0 = a.win_max > 0 ? a.win_start[r] : 0;

  const int c_begin = split * a.chunks_per_split;
  int c_end = c_begin + a.chunks_per_split;
  c_end = c_end < a.n_chunks ? c_end : a.n_chunks;

  // The first two chunks' selected indices load first, then the query; the
  // first chunk's rows are gathered as soon as its indices arrive.  The query
  // is converted to bf16 hi/lo after that, off the index -> gather -> decode path.
  int32_t ix_next[4];
  Gathered<CH, NT> gr;
  uint32_t vb = 0u;       // validity of this thread's entries of the gathered chunk
  uint32_t bm[4] = {0u, 0u, 0u, 0u};   // bit q of bm[i]: entry 4q + i of the gathered chunk is valid
  {
    int32_t ix0[4];
    load_entry_ids(a, r, c_begin * kChunk, eg, ix0);
    load_entry_ids(a, r, (c_begin + 1) * kChunk, eg, ix_next);
    __builtin_amdgcn_sched_barrier(0);
    if (c_begin < c_end) {
      int64_t off[4];
      const int eb = c_begin * kChunk;
      vb = entry_rows(a, seq, ws0, E, eb, eg, ix0, off);
      const int kind = chunk_kind(eb, kChunk, a.k);
      if (kind == kLatentRows)
        gather_chunk<NT, kLatentRows, CH>(a, off, vb, eb, tid, gr);
      else if (kind == kWindowRows)
        gather_chunk<NT, kWindowRows, CH>(a, off, vb, eb, tid, gr);
      else
        gather_chunk<NT, kMixedRows, CH>(a, off, vb, eb, tid, gr);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x4 qraw[2 * kS];
  {
    const float* qp = a.q + ((int64_t)r * a.H + h) * 512 + dbase + 8 * g;
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      qraw[2 * s] = *reinterpret_cast<const f32x4*>(qp + 32 * s);
      qraw[2 * s + 1] = *reinterpret_cast<const f32x4*>(qp + 32 * s + 4);
    }
  }
  // query operands (B of S^T = C Q^T): head h, dims dbase + 32s + 8g .. +8, prescaled
  bf16x8_t qhi[kS], qlo[kS];
  bool q_ready = false;
  auto convert_query = [&]() {
#pragma unroll
    for (int s = 0; s < kS; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = qraw[2 * s + (e >> 2)][e & 3] * a.qscale;
        const __bf16 hi = (__bf16)v;
        qhi[s][e] = hi;
        qlo[s][e] = (__bf16)(v - (float)hi);
      }
    }
    q_ready = true;
  };

  f32x4 oacc[kM];
#pragma unroll
  for (int m = 0; m < kM; ++m) oacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  for (int c = c_begin; c < c_end; ++c) {
    const int ebase = c * kChunk;
    if (ebase >= E) break;
    // this chunk's validity (the same in every wave: lanes 0..kEG-1 hold groups 0..kEG-1)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      bm[i] = (uint32_t)__ballot((vb >> i) & 1u) & (kEG == 32 ? 0xFFFFFFFFu : ((1u << kEG) - 1u));
    const bool any = (bm[0] | bm[1] | bm[2] | bm[3]) != 0u;
    if (any) {
      __syncthreads();   // previous chunk's LDS reads are done
      const int kind = chunk_kind(ebase, kChunk, a.k);
      if (kind == kLatentRows)
        store_chunk<NT, kLatentRows, CH>(a, gr, vb, ebase, tid, sK, sVt);
      else if (kind == kWindowRows)
        store_chunk<NT, kWindowRows, CH>(a, gr, vb, ebase, tid, sK, sVt);
      else
        store_chunk<NT, kMixedRows, CH>(a, gr, vb, ebase, tid, sK, sVt);
      __syncthreads();
    }
    const uint32_t bmc[4] = {bm[0], bm[1], bm[2], bm[3]};
    // the next chunk's rows, then the indices of the one after
    if (c + 1 < c_end && ebase + kChunk < E) {
      int64_t off[4];
      const int eb = ebase + kChunk;
      vb = entry_rows(a, seq, ws0, E, eb, eg, ix_next, off);
      const int kind = chunk_kind(eb, kChunk, a.k);
      if (kind == kLatentRows)
        gather_chunk<NT, kLatentRows, CH>(a, off, vb, eb, tid, gr);
      else if (kind == kWindowRows)
        gather_chunk<NT, kWindowRows, CH>(a, off, vb, eb, tid, gr);
      else
        gather_chunk<NT, kMixedRows, CH>(a, off, vb, eb, tid, gr);
      if (c + 2 < c_end) load_entry_ids(a, r, eb + kChunk, eg, ix_next);
    } else {
      vb = 0u;
    }
    if (!any) continue;

    if (!q_ready) convert_query();

    // 3. partial S^T[CH entries x 16 heads] over this wave's kDims dims
    f32x4 sacc[kT];
#pragma unroll
    for (int t = 0; t < kT; ++t) sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kS; ++s) {
#pragma unroll
      for (int t = 0; t < kT; ++t) {
        const bf16x8_t A =
            *reinterpret_cast<const bf16x8_t*>(&sK[(16 * t + hl) * kKLd + dbase + 32 * s + 8 * g]);
        sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, qhi[s], sacc[t], 0, 0, 0);
        sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, qlo[s], sacc[t], 0, 0, 0);
      }
    }
    // the ND waves of a head group add their partial sums in part order,
    // through the row-major copy's LDS once every wave is done reading it
    __syncthreads();
    f32x4* slots = reinterpret_cast<f32x4*>(sK);   // [NP][ND][64 lanes][kT]
    {
      f32x4* mine = slots + ((pr * ND + part) * 64 + lane) * kT;
#pragma unroll
      for (int t = 0; t < kT; ++t) mine[t] = sacc[t];
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kT; ++t) {
      f32x4 acc = slots[((pr * ND + 0) * 64 + lane) * kT + t];
#pragma unroll
      for (int p = 1; p < ND; ++p) acc += slots[((pr * ND + p) * 64 + lane) * kT + t];
      sacc[t] = acc;
    }

    // 4. online softmax (lane holds entries 16t + 4g + i of head h)
    float mloc = -__builtin_inff();
#pragma unroll
    for (int t = 0; t < kT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // entry 16t + 4g + i: group 4t + g, member i
        if (!((bmc[i] >> (4 * t + g)) & 1u)) sacc[t][i] = -__builtin_inff();
        mloc = fmaxf(mloc, sacc[t][i]);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < kT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(sacc[t][i] - m_new);
        sacc[t][i] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int m = 0; m < kM; ++m) oacc[m] *= alpha;

    // 5. O^T[kDims dims x 16 heads] += C^T P^T, k-steps of 32 entries
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      bf16x8_t bhi, blo;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = i < 4 ? sacc[2 * j][i] : sacc[2 * j + 1][i - 4];
        const __bf16 hi = (__bf16)p;
        bhi[i] = hi;
        blo[i] = (__bf16)(p - (float)hi);
      }
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        const __bf16* vrow = &sVt[(dbase + 16 * m + hl) * kVLd + 32 * j + 4 * g];
        const bf16x4_t lo4 = *reinterpret_cast<const bf16x4_t*>(vrow);
        const bf16x4_t hi4 = *reinterpret_cast<const bf16x4_t*>(vrow + 16);
        const bf16x8_t A = bf16x8_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        oacc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, bhi, oacc[m], 0, 0, 0);
        oacc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, blo, oacc[m], 0, 0, 0);
      }
    }
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
    for (int m = 0; m < kM; ++m) *reinterpret_cast<f32x4*>(op + 16 * m) = oacc[m];
    if (g == 0 && part == 0) {
      a.part_ml[2 * slot] = m_run;
      a.part_ml[2 * slot + 1] = l_tot;
    }
  }
}

// 8-wave workgroups (32 heads).  With 32-entry chunks two fit a compute unit
// (78 KB of LDS each) when a wave keeps to 128 registers (a few spill), so one
// workgroup's loads overlap the other's products: better once the grid holds
// several workgroups per compute unit, worse for a grid that does not.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4))) void sparse_attn_kernel_h32c32_2wg(
    AttnParams a) {
  sparse_attn_body<2, 4, 32>(a);
}
__global__ __launch_bounds__(512, 1) void sparse_attn_kernel_h32c32(AttnParams a) { sparse_attn_body<2, 4, 32>(a); }
__global__ __launch_bounds__(512, 1) void sparse_attn_kernel_h32c64(AttnParams a) { sparse_attn_body<2, 4, 64>(a); }
__global__ __launch_bounds__(256) void sparse_attn_kernel_h16c32(AttnParams a) { sparse_attn_body<1, 4, 32>(a); }
__global__ __launch_bounds__(256, 1) void sparse_attn_kernel_h16c64(AttnParams a) { sparse_attn_body<1, 4, 64>(a); }

// Merge split partials: out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// One workgroup per (row, head), one thread per output dim.  Wave 0 reads the
// splits' (m, l) pairs and turns them into weights in LDS; every thread's own
// dim of the first kCombineGroup splits' o is loaded before that, so the
// weights and the partials arrive in one memory round trip.
constexpr int kMaxSplits = kAttnTargetWorkgroups;   // attn_splits never exceeds it
constexpr int kCombineGroup = 32;

__global__ __launch_bounds__(512) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml, int splits, int H,
                                                           float* __restrict__ out) {
  __shared__ float sw[kMaxSplits];   // 2^(m_s - M), 0 for splits that saw nothing
  __shared__ float sL;
  const int r = blockIdx.y;
  const int h = blockIdx.x;
  const int d = threadIdx.x;
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
  float ov[kCombineGroup];
#pragma unroll
  for (int j = 0; j < kCombineGroup; ++j) ov[j] = j < splits ? part_o[(base + (int64_t)j * H) * 512 + d] : 0.f;
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
  float acc = 0.f;
  for (int s0 = 0; s0 < splits; s0 += kCombineGroup) {
    if (s0 > 0) {
#pragma unroll
      for (int j = 0; j < kCombineGroup; ++j)
        ov[j] = s0 + j < splits ? part_o[(base + (int64_t)(s0 + j) * H) * 512 + d] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kCombineGroup; ++j)
      if (s0 + j < splits) acc += sw[s0 + j] * ov[j];
  }
  const float L = sL;
  out[((int64_t)r * H + h) * 512 + d] = L > 0.f ? acc / L : 0.f;
}

// Head groups of 16 heads per workgroup (32 when H allows).
static int attn_group_heads(int H) { return H >= 32 ? 32 : 16; }

// Entries per chunk: 32 keeps a workgroup's LDS at 78 KB, so two workgroups
// share a compute unit and one's loads overlap the other's products.
static int attn_chunk(int R, int H, int k_plus_win) {
  (void)R;
  (void)H;
  (void)k_plus_win;
  return kAttnChunk;
}

// Splits of a row's entry chunks: enough workgroups to give every compute unit
// about one (a workgroup's LDS fills a compute unit), never more splits than
// chunks, and chunks spread evenly over the splits.
int attn_splits(int R, int H, int k_plus_win) {
  const int ch = attn_chunk(R, H, k_plus_win);
  const int n_chunks = (k_plus_win + ch - 1) / ch;
  if (n_chunks <= 1) return 1;
  const int64_t groups = (int64_t)R * (H > 0 ? (H + attn_group_heads(H) - 1) / attn_group_heads(H) : 1);
  int64_t want = (kAttnTargetWorkgroups + groups - 1) / groups;
  if (want < 1) want = 1;
  if (want > n_chunks) want = n_chunks;
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
  a.part_o = nullptr;
  a.part_ml = nullptr;
  if (a.splits > 1) {
    a.part_o = static_cast<float*>(L.workspace);
    a.part_ml = a.part_o + (size_t)R * a.splits * L.H * 512;
  }
  // Workgroups of 32 heads (8 waves); more heads split over blockIdx.z.  Four
  // waves of 128 dims per 16-head group keep every wave's chain of products
  // short and leave two waves per SIMD to overlap LDS and matrix-core work.
  if (L.H % 16 != 0 || L.H < 16) return hipErrorInvalidValue;
  const int NP = attn_group_heads(L.H) / 16;
  if (L.H % (16 * NP) != 0) return hipErrorInvalidValue;
  dim3 grid((unsigned)a.splits, (unsigned)R, (unsigned)(L.H / (16 * NP)));
  const bool many = (int64_t)grid.x * grid.y * grid.z > 4 * kAttnTargetWorkgroups;
  if (NP == 2 && ch == 32 && many)
    hipLaunchKernelGGL(sparse_attn_kernel_h32c32_2wg, grid, dim3(512), 0, stream, a);
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
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)L.H, (unsigned)R), dim3(512), 0, stream, a.part_o,
                     a.part_ml, a.splits, L.H, L.out);
  return hipGetLastError();
}

}  // namespace csa2
