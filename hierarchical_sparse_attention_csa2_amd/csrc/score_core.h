// MXFP4 indexer scores of single keys and of 16-key groups (the score as
// defined in the indexer scans: exact block sums, ((v0+v1)+v2)+v3 in fp32),
// shared by the indexer scans: on the vector ALUs (any scales) or on the FP4
// matrix cores (block exponents in the range where their sums are exact).
#pragma once
#include "device_common.h"

namespace csa2 {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4_t load_codes16(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// Score of one key on the vector ALUs, for any scale bytes: each block's exact
// sum (E2M1 codes decoded to f16 with v_cvt_scalef32_pk_f16_fp4, v_dot2 into
// fp32) scaled with ldexp, then ((v0+v1)+v2)+v3 in fp32.
__device__ __forceinline__ float score_key_valu(const uint8_t* qr, const uint8_t* qs, const uint8_t* kr,
                                                const uint8_t* ksr) {
  float s = 0.0f;
#pragma unroll 1
  for (int b = 0; b < 4; ++b) {
    half2_t qh[16];
    load_query_block(qr + 16 * b, qh);
    const u32x4_t c = *reinterpret_cast<const u32x4_t*>(kr + 16 * b);
    const float v = __builtin_amdgcn_ldexpf(block_dot(c, qh), (int)qs[b] + (int)ksr[b] - 254);
    s = b == 0 ? v : s + v;
  }
  return canonical_nan(s);
}

// The four block values of 16 keys on the matrix cores.  kb[u], ek[u]: lane
// 16g + c holds block g of key c of group u (codes, scale byte); qa, eq: the
// block-diagonal query operand (lane 16g + i holds query block g when
// i % 4 == g) and this lane's query scale byte (block g).  Returns the score of
// key c of group g, the wave's key 16g + c, in lane 16g + c.
__device__ __forceinline__ float score_groups_mfma(const u32x4_t qa, int eq, const u32x4_t* kb, const uint32_t* ek) {
  const int g = (threadIdx.x & 63) >> 4;
  const i32x8_t a8 = {(int)qa[0], (int)qa[1], (int)qa[2], (int)qa[3], 0, 0, 0, 0};
  f32x4_t acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const i32x8_t b8 = {(int)kb[u][0], (int)kb[u][1], (int)kb[u][2], (int)kb[u][3], 0, 0, 0, 0};
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
    acc[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, zero, 4, 4, 0, eq, 0, (int)ek[u]);
    // keep the product here, with every lane active: the matrix core reads its
    // operands from all 64 lanes, so it must not be moved into a branch that
    // only some lanes take
    asm volatile("" : "+v"(acc[u]));
  }
  // lane 16g + c: column c, rows 4g..4g+3; element i = row 4g + i = v_i of
  // key c of group u.  Take group u = g.
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = (g & 1) ? acc[1][i] : acc[0][i];
    const float hi = (g & 1) ? acc[3][i] : acc[2][i];
    v[i] = (g & 2) ? hi : lo;
  }
  float s = v[0] + v[1];
  s = s + v[2];
  s = s + v[3];
  return s + 0.0f;   // an exact zero sum is +0
}

// The scores of 4 groups of 16 keys on the vector ALUs, for any scale bytes:
// lane 16g + c holds block g of key c of group u (kb[u] codes, ek[u] scale byte,
// as loaded for score_groups_mfma), qh its query block g as 16 f16 pairs and eq
// that block's scale byte.  Each lane forms its block's exact value (E2M1
// decoded in registers, v_dot2 into fp32, ldexp), the four blocks of a key meet
// through lane shuffles and are added in block order.  Returns the score of the
// wave's key 16g + c in lane 16g + c.
__device__ __forceinline__ float score_groups_valu(const half2_t* qh, int eq, const u32x4_t* kb, const uint32_t* ek) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  float sc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float v = __builtin_amdgcn_ldexpf(block_dot(kb[u], qh), eq + (int)ek[u] - 254);
    const float v0 = __shfl(v, c, 64), v1 = __shfl(v, 16 + c, 64), v2 = __shfl(v, 32 + c, 64),
                v3 = __shfl(v, 48 + c, 64);
    float s = v0 + v1;
    s = s + v2;
    s = s + v3;
    sc[u] = canonical_nan(s);
  }
  return g == 0 ? sc[0] : (g == 1 ? sc[1] : (g == 2 ? sc[2] : sc[3]));
}

// Block exponent e = eq + ek - 254 outside [-124, 114]: the matrix-core value
// may be inexact.  Inside it a block value is an integer of at most 13 bits
// (|sum| <= 4608 quarter-units) times 2^(e - 2): every nonzero value is a normal
// float (>= 2^-126) below 2^125, so the product is exact and cannot overflow.
__device__ __forceinline__ bool exponent_out_of_range(int eq, uint32_t ek) {
  return (uint32_t)(eq + (int)ek - 130) > 238u;
}

}  // namespace csa2
