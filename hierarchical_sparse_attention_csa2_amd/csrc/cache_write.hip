// Cache write path: the step that produces the cached state the hot path reads.
//
// DeepSeek-V4.1-Flash (fupanwang.com article, section 三个方向一起压小缓存): CSA2
// stores every m consecutive tokens as one entry (ratio m, entries do not
// overlap), a merge of the m token vectors weighted by the layer's compression
// weights; the main KV and the indexer keys are kept in OCP MXFP4 and the
// sliding window in FP8.
//
// write_mxfp4: entry e = sum_{j < m} w[m e + j] * x[m e + j] in fp32, j in order
// (each product rounded, then added; no fused multiply-add), then every
// 32-element block is encoded with the OCP MX rule: shared exponent
// E = floor(log2 amax) - 2 clamped to [-127, 127] (byte E + 127; an all-zero
// block gets byte 0 and zero codes; NaN elements do not count towards amax and
// encode as +0; an infinite amax takes E = 127), elements y = v / 2^E rounded
// to the nearest E2M1 value with ties to the even code, saturating at 6; a
// negative value that rounds to zero keeps the +0 code.
// write_e4m3: OCP E4M3FN, nearest value with ties to the even code, saturating
// at +-448 (infinities too), NaN to 0x7F.
//
// Both are streaming kernels bound by HBM: a lane takes 4 consecutive floats
// (one 16-byte non-temporal load per token), a wave 64 consecutive such quads
// (1 KB per load instruction), and the 8 lanes of one 32-element block meet over
// DPP for the block maximum.  Rows are a power-of-two number of quads long, so a
// quad's row and column come from a shift and a mask.  Workgroups go to the 8
// XCDs round-robin; tiles are handed out so that each XCD streams runs of 64
// consecutive tiles (measured on the 1M-token latent write: 6.3 TB/s, against
// 5.4 TB/s with 4 quads per lane and tiles in launch order).
#include "device_common.h"
#include "kernels.h"

namespace csa2 {

constexpr int kWriteThreads = 256;                 // one quad per lane
constexpr int64_t kWriteTile = kWriteThreads;       // quads per workgroup
constexpr int kXcdRun = 64;                         // consecutive tiles per XCD turn

// max over lanes 8g..8g+7 (DPP: swap neighbours, swap pairs, mirror halves of
// each group of 8)
__device__ __forceinline__ float max8(float v) {
  int b = __float_as_int(v);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(b, 0xB1, 0xF, 0xF, false)));
  b = __float_as_int(v);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x4E, 0xF, 0xF, false)));
  b = __float_as_int(v);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x141, 0xF, 0xF, false)));
  return v;
}

// E2M1 magnitude code (0..7) of a = |y|, a not NaN.  Below 1 the values are
// 0, 0.5, 1: rint(2a) (ties to even = the even code).  From 1 up the code is the
// fp32 exponent and top mantissa bit, rounded to nearest even at that bit,
// saturating at 7 (6.0).
__device__ __forceinline__ uint32_t e2m1_code(float a) {
  const uint32_t u = __float_as_uint(a);
  const uint32_t r = (u + 0x1FFFFFu + ((u >> 22) & 1u)) >> 22;   // (exp << 1 | m) rounded
  const uint32_t hi = r - 252u;                                   // 1.0 -> 2
  const uint32_t lo = (uint32_t)rintf(a + a);
  const uint32_t c = a < 1.0f ? lo : hi;
  return c > 7u ? 7u : c;
}

// E4M3 code of x.  Normal range [2^-6, 448): exponent and three mantissa bits
// of the fp32 pattern rounded to nearest even at bit 20; below 2^-6 the values
// are multiples of 2^-9 (code = rint(a * 512), where code 8 is 2^-6 itself).
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  const uint32_t u = __float_as_uint(a);
  const uint32_t nrm = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - 960u;   // (127 - 7) << 3
  const uint32_t sub = (uint32_t)rintf(a * 512.0f);
  uint32_t c = a < 0.015625f ? sub : nrm;
  c = a >= 448.0f ? 0x7Eu : c;
  c |= sign;
  return a != a ? 0x7Fu : c;
}

// One 4-element quad of a merged entry: codes (4 nibbles) and, from the first
// lane of each 8-lane block group, the scale byte.  Every lane of the wave
// calls this (the block maximum is a cross-lane reduction).
__device__ __forceinline__ void encode_quad(f32x4_t v, bool on, int64_t q, int lane, uint8_t* __restrict__ codes,
                                            uint8_t* __restrict__ scales) {
  // maxNum drops NaN operands; the 0 start makes an all-NaN block a zero block
  float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
  amax = max8(fmaxf(amax, 0.0f));
  const int ebits = (int)(__float_as_uint(amax) >> 23);   // amax >= 0: no sign bit
  int E = ebits - 129;
  E = E < -127 ? -127 : E;
  E = ebits == 255 ? 127 : E;
  uint32_t packed = 0u;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float y = __builtin_amdgcn_ldexpf(v[e], -E);   // a power-of-two scaling
    const float a = fabsf(y);
    uint32_t c = e2m1_code(a);
    c = a != a ? 0u : c;
    c |= (y < 0.0f && c != 0u) ? 8u : 0u;
    packed |= c << (4 * e);
  }
  const bool zero = amax == 0.0f;
  if (zero) packed = 0u;
  if (on) {
    *reinterpret_cast<uint16_t*>(codes + 2 * q) = (uint16_t)packed;
    if ((lane & 7) == 0) scales[q >> 3] = zero ? (uint8_t)0 : (uint8_t)(E + 127);
  }
}

// kRatio > 0: the ratio is a compile-time constant and the lane's loads are all
// issued before the first is used; kRatio == 0: any ratio, a token at a time.
template <int kRatio>
__global__ __launch_bounds__(kWriteThreads) void write_mxfp4_kernel(const float* __restrict__ x,
                                                                    const float* __restrict__ w, int ratio,
                                                                    int64_t n_quads, int row_shift,
                                                                    uint8_t* __restrict__ codes,
                                                                    uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t q = xcd_run_tile<kXcdRun>(blockIdx.x, gridDim.x) * kWriteTile + threadIdx.x;
  // the last tile is ragged: lanes past the end read quad 0 and store nothing
  const bool on = q < n_quads;
  const int64_t qq = on ? q : 0;
  const int64_t row = qq >> row_shift;
  const int64_t col = qq & (((int64_t)1 << row_shift) - 1);
  const int64_t dq = (int64_t)1 << row_shift;   // quads per row
  f32x4_t v;
  if constexpr (kRatio > 0) {
    f32x4_t t[kRatio];
    float wt[kRatio];
#pragma unroll
    for (int j = 0; j < kRatio; ++j) {
      const int64_t tok = row * kRatio + j;
      t[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(x + (tok * dq + col) * 4));
      wt[j] = w ? __builtin_nontemporal_load(w + tok) : 1.0f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float s = t[0][e] * wt[0];
#pragma unroll
      for (int j = 1; j < kRatio; ++j) {
        const float p = t[j][e] * wt[j];
        s = s + p;
      }
      v[e] = s;
    }
  } else {
    for (int j = 0; j < ratio; ++j) {
      const int64_t tok = row * ratio + j;
      const f32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(x + (tok * dq + col) * 4));
      const float wt = __builtin_nontemporal_load(w + tok);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = t[e] * wt;
        v[e] = j == 0 ? p : v[e] + p;
      }
    }
  }
  encode_quad(v, on, q, lane, codes, scales);
}

__global__ __launch_bounds__(kWriteThreads) void write_e4m3_kernel(const float* __restrict__ x, int64_t n_quads,
                                                                   uint8_t* __restrict__ out) {
  const int64_t q = xcd_run_tile<kXcdRun>(blockIdx.x, gridDim.x) * kWriteTile + threadIdx.x;
  if (q >= n_quads) return;
  const f32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(x + 4 * q));
  *reinterpret_cast<uint32_t*>(out + 4 * q) =
      e4m3_code(t[0]) | (e4m3_code(t[1]) << 8) | (e4m3_code(t[2]) << 16) | (e4m3_code(t[3]) << 24);
}

hipError_t launch_write_mxfp4(const float* x, const float* w, int64_t n_entries, int ratio, int D, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream) {
  if (D < 32 || (D & (D - 1)) != 0 || ratio < 1) return hipErrorInvalidValue;
  int shift = 0;
  while ((4 << shift) < D) ++shift;
  const int64_t n_quads = n_entries * (D / 4);
  const int64_t grid = (n_quads + kWriteTile - 1) / kWriteTile;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (grid == 0) return hipSuccess;
  const dim3 g((unsigned)grid), b(kWriteThreads);
  switch (ratio) {
    case 1: hipLaunchKernelGGL(write_mxfp4_kernel<1>, g, b, 0, stream, x, w, 1, n_quads, shift, codes, scales); break;
    case 2: hipLaunchKernelGGL(write_mxfp4_kernel<2>, g, b, 0, stream, x, w, 2, n_quads, shift, codes, scales); break;
    case 4: hipLaunchKernelGGL(write_mxfp4_kernel<4>, g, b, 0, stream, x, w, 4, n_quads, shift, codes, scales); break;
    default:
      hipLaunchKernelGGL(write_mxfp4_kernel<0>, g, b, 0, stream, x, w, ratio, n_quads, shift, codes, scales);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_write_e4m3(const float* x, int64_t n, uint8_t* out, hipStream_t stream) {
  if (n % 4 != 0) return hipErrorInvalidValue;
  const int64_t n_quads = n / 4;
  const int64_t grid = (n_quads + kWriteTile - 1) / kWriteTile;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(write_e4m3_kernel, dim3((unsigned)grid), dim3(kWriteThreads), 0, stream, x, n_quads, out);
  return hipGetLastError();
}

}  // namespace csa2
