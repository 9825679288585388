// Device helpers shared by the CSA2 kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// IEEE-754 total order of fp32 bits as an unsigned key (larger key = larger
// score, -0 below +0).  Key 0 (bit pattern 0xFFFFFFFF, a negative NaN) is
// reserved as "no element".
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// A score that is not a number (two block values overflowing to opposite
// infinities) is stored as the positive quiet NaN 0x7FC00000, whatever NaN the
// adder produced, so that its rank in the total order is fixed.
__device__ __forceinline__ float canonical_nan(float s) {
  return s != s ? __uint_as_float(0x7FC00000u) : s;
}

// Two E2M1 codes (byte SEL of w, low nibble first) -> two exact f16 values.
template <int SEL>
__device__ __forceinline__ half2_t fp4x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}
// Two E2M1 codes times a power-of-two scale -> two bf16 values (exact for
// scales 2^-126 .. 2^127 times the E2M1 magnitudes).
template <int SEL>
__device__ __forceinline__ bf16x2_t fp4x2_to_bf16(uint32_t w, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, SEL);
}

// E8M0 byte -> fp32 2^(e-127) (e = 0 gives the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
}

// One 32-element MXFP4 block dot product: 16 bytes of key codes against the
// query block held as 16 pairs of f16.  Products of E2M1 values are multiples
// of 1/4 below 36 in magnitude and the running sum stays below 1152, so every
// f16 value, product and fp32 partial sum is exact: the result equals the
// exact integer block sum / 4.
__device__ __forceinline__ float block_dot(const u32x4_t c, const half2_t* q) {
  float acc = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t w = c[d];
    acc = __builtin_amdgcn_fdot2(fp4x2_to_f16<0>(w), q[4 * d + 0], acc, false);
    acc = __builtin_amdgcn_fdot2(fp4x2_to_f16<1>(w), q[4 * d + 1], acc, false);
    acc = __builtin_amdgcn_fdot2(fp4x2_to_f16<2>(w), q[4 * d + 2], acc, false);
    acc = __builtin_amdgcn_fdot2(fp4x2_to_f16<3>(w), q[4 * d + 3], acc, false);
  }
  return acc;
}

// DPP quad broadcast of lane (quad base + I) to all four lanes of the quad.
template <int I>
__device__ __forceinline__ float quad_bcast(float v) {
  constexpr int ctrl = I | (I << 2) | (I << 4) | (I << 6);
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xF, 0xF, false));
}

// Score of the position held by a quad of lanes (lane 4p+b holds block b's
// scaled sum v_b): ((v0+v1)+v2)+v3 in fp32, identical on all four lanes.
__device__ __forceinline__ float quad_ordered_sum(float v) {
  float v0 = quad_bcast<0>(v), v1 = quad_bcast<1>(v), v2 = quad_bcast<2>(v), v3 = quad_bcast<3>(v);
  float s = v0 + v1;
  s = s + v2;
  s = s + v3;
  return s;
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Max over the 8 quads of a 32-lane half wave (one 8-position block).
__device__ __forceinline__ uint32_t halfwave_quad_max(uint32_t k) {
  k = umax(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, 0x124, 0xF, 0xF, false));  // row_ror:4
  k = umax(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, 0x128, 0xF, 0xF, false));  // row_ror:8
  k = umax(k, (uint32_t)__shfl_xor((int)k, 16, 64));
  return k;
}

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
// Convert a query block of 16 code bytes to 16 f16 pairs.
__device__ __forceinline__ void load_query_block(const uint8_t* codes16, half2_t* q) {
  u32x4_t c = *reinterpret_cast<const u32x4_t*>(codes16);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    q[4 * d + 0] = fp4x2_to_f16<0>(c[d]);
    q[4 * d + 1] = fp4x2_to_f16<1>(c[d]);
    q[4 * d + 2] = fp4x2_to_f16<2>(c[d]);
    q[4 * d + 3] = fp4x2_to_f16<3>(c[d]);
  }
}

// Workgroups of a launch are dealt to the 8 XCDs in turn (workgroup i runs on
// XCD i % 8 when the grid's x extent is a multiple of 8).  For streaming
// kernels, xcd_run_tile<kRun>(blockIdx.x, gridDim.x) gives the tile workgroup
// bid should take so that each XCD streams runs of kRun consecutive tiles:
// within each full group of 8 * kRun tiles, XCD k takes the k-th run; a last
// partial group keeps launch order.  A bijection on [0, grid).
template <int kRun>
__device__ __forceinline__ int64_t xcd_run_tile(int64_t bid, int64_t grid) {
  const int64_t g = bid / (8 * kRun);
  if ((g + 1) * 8 * kRun > grid) return bid;
  const int64_t r = bid - g * 8 * kRun;
  return g * 8 * kRun + (r % 8) * kRun + r / 8;
}

}  // namespace csa2
