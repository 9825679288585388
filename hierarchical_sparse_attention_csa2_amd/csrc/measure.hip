// Measurement kernels for the indexer scan's roofline (not part of the C ABI;
// built into libcsa2_measure.so, which only the benchmark and its tests load):
//   - a read-only probe that fetches exactly the bytes the decode scan reads,
//     in the same grid, wave layout and load instructions, and computes nothing
//     from them: the bandwidth this access pattern can reach on the part;
//   - the decode scan with its block values taken on the FP4 matrix cores
//     instead of the vector ALUs (block-diagonal query operand, keys as the B
//     operand; waves with a block exponent outside [-124, 114] fall back to the
//     vector ALUs), same loads and same outputs, so the two ways of forming the
//     block values can be timed against each other.
#include "device_common.h"
#include "score_core.h"

namespace csa2m {

using namespace csa2;

constexpr int kThreads = 256;
constexpr int kChunk = 256;     // positions per workgroup, 64 per wave (as the decode scan)
constexpr int kXcdRun = 64;

__device__ __forceinline__ uint32_t group8_max(uint32_t x) {
  uint32_t y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
  x = y > x ? y : x;
  y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);
  x = y > x ? y : x;
  y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false);
  return y > x ? y : x;
}

// Grid (ceil(N / 256), 1, B).  Lane 16g + c of a wave loads 16 bytes of codes
// (block g of key 16u + c) and one scale byte for u = 0..3, as the scan does;
// the words are folded together and written only if they equal `magic`
// (never, for the magic the benchmark passes), so no load can be dropped.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void read_probe_kernel(
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales, int64_t N, uint32_t magic,
    uint32_t* __restrict__ sink) {
  const int64_t seq = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int64_t p0 = xcd_run_tile<kXcdRun>(blockIdx.x, gridDim.x) * kChunk + (int64_t)wave * 64;
  if (p0 >= N) return;
  const uint8_t* kc = k_codes + seq * N * 64;
  const uint8_t* ks = k_scales + seq * N * 4;
  u32x4_t kb[4];
  uint32_t ek[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    int64_t p = p0 + 16 * u + c;
    p = p < N ? p : N - 1;
    kb[u] = load_codes16(kc + p * 64 + 16 * g);
    ek[u] = ks[p * 4 + g];
  }
  uint32_t x = 0u;
#pragma unroll
  for (int u = 0; u < 4; ++u) x ^= kb[u][0] ^ kb[u][1] ^ kb[u][2] ^ kb[u][3] ^ (ek[u] << (8 * u));
  if (x == magic) sink[0] = x;
}

// The decode scan (one query row per sequence) with FP4 matrix-core block
// values.  Same grid, loads and outputs as the library's decode scan storing
// scores and super-block maxima.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void index_scan_mfma_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales,
    const int32_t* __restrict__ n_visible, int64_t N_max, int64_t nblk_stride, int64_t nsup_stride,
    float* __restrict__ scores, float* __restrict__ block_max, float* __restrict__ super_max) {
  const int64_t seq = blockIdx.z;
  const int64_t r = seq;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  int64_t nv = n_visible[r];
  nv = nv < 0 ? 0 : (nv > N_max ? N_max : nv);
  const int64_t p0 = xcd_run_tile<kXcdRun>(blockIdx.x, gridDim.x) * kChunk + (int64_t)wave * 64;
  if (p0 >= nv) return;
  const uint8_t* kc = k_codes + seq * N_max * 64;
  const uint8_t* ks = k_scales + seq * N_max * 4;
  u32x4_t kb[4];
  uint32_t ek[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    int64_t p = p0 + 16 * u + c;
    p = p < nv ? p : nv - 1;
    kb[u] = load_codes16(kc + p * 64 + 16 * g);
    ek[u] = ks[p * 4 + g];
  }
  // A operand: lane 16g + i (row i, K group g) holds query block g when i % 4 == g
  const uint8_t* qr = q_codes + r * 64;
  const int eq = q_scales[r * 4 + g];
  u32x4_t qa = {0u, 0u, 0u, 0u};
  if ((lane & 3) == g) qa = *reinterpret_cast<const u32x4_t*>(qr + 16 * g);
  bool bad = false;
#pragma unroll
  for (int u = 0; u < 4; ++u) bad |= p0 + 16 * u + c < nv && exponent_out_of_range(eq, ek[u]);
  float s;
  if (__ballot(bad) == 0ull) {
    s = score_groups_mfma(qa, eq, kb, ek);
  } else {
    int64_t p = p0 + lane;
    p = p < nv ? p : nv - 1;
    s = score_key_valu(qr, q_scales + r * 4, kc + p * 64, ks + p * 4);
  }
  const int64_t key = p0 + lane;
  const bool vis = key < nv;
  if (vis) __builtin_nontemporal_store(s, &scores[r * N_max + key]);
  const uint32_t m8 = group8_max(vis ? order_key(s) : 0u);
  if ((lane & 7) == 0 && vis) block_max[r * nblk_stride + (key >> 3)] = key_to_float(m8);
  const uint32_t m = wave_max_u32(m8);
  if (lane == 0) super_max[r * nsup_stride + (p0 >> 6)] = key_to_float(m);
}

}  // namespace csa2m

extern "C" {

// Read-only probe over B sequences of N index keys (codes u8[B][N][64], scales
// u8[B][N][4]); sink: one device word, written only when the folded bytes
// equal magic.  Returns 0 or a negative value on a bad argument or launch.
int csa2m_read_probe(const uint8_t* k_codes, const uint8_t* k_scales, int B, int64_t N, uint32_t magic,
                     uint32_t* sink, void* stream) {
  if (!k_codes || !k_scales || !sink || B < 1 || B > 65535 || N < 1 || N > ((int64_t)1 << 30)) return -1;
  const dim3 grid((unsigned)((N + csa2m::kChunk - 1) / csa2m::kChunk), 1u, (unsigned)B);
  hipLaunchKernelGGL(csa2m::read_probe_kernel, grid, dim3(csa2m::kThreads), 0, reinterpret_cast<hipStream_t>(stream),
                     k_codes, k_scales, N, magic, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// The decode scan with FP4 matrix-core block values: one query row per
// sequence (M = 1), arguments and outputs as csa2_index_scan with scores and
// super_max.
int csa2m_index_scan_mfma(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                          const uint8_t* k_scales, const int32_t* n_visible, int B, int64_t N_max, float* scores,
                          float* block_max, float* super_max, void* stream) {
  if (!q_codes || !q_scales || !k_codes || !k_scales || !n_visible || !scores || !block_max || !super_max)
    return -1;
  if (B < 1 || B > 65535 || N_max < 1 || N_max > ((int64_t)1 << 30)) return -1;
  const dim3 grid((unsigned)((N_max + csa2m::kChunk - 1) / csa2m::kChunk), 1u, (unsigned)B);
  hipLaunchKernelGGL(csa2m::index_scan_mfma_kernel, grid, dim3(csa2m::kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), q_codes, q_scales, k_codes, k_scales, n_visible, N_max,
                     (N_max + 7) / 8, (N_max + 63) / 64, scores, block_max, super_max);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
