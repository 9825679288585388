// C ABI of the CSA2 hierarchical sparse attention step (see include/csa2.h).
// Every entry point validates its arguments on the host, then enqueues kernels
// on the caller's stream; nothing is allocated and no state is kept.
#include "../../include/csa2.h"
#include "kernels.h"

#include <mutex>

namespace {

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int hip_status(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_ERR_HIP; }

inline size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// Decode calls (fewer than this many queries per sequence) store every score
// and take the top-k from those of the pool's first blocks; prefill calls
// rescore those blocks instead of storing M scores per entry.
constexpr int kStoreScoresBelowM = 16;

// index_full workspace carve-up
struct FullWs {
  size_t block_max, super_max, topk_blocks, topk_scores, key_floor, scores, total;
};

// Super-block maxima per row in the workspace: ceil(N_max / 64) rounded up to
// a multiple of 4, so that each row is 16-byte aligned for the block filter.
inline int64_t super_stride(int64_t N_max) { return ((N_max + 63) / 64 + 3) / 4 * 4; }

inline FullWs full_ws(int64_t R, int M, int64_t N_max, int k) {
  FullWs w;
  const int64_t nblk = (N_max + 7) / 8;
  const int64_t nsup = super_stride(N_max);
  w.block_max = 0;
  w.super_max = align_up(w.block_max + (size_t)R * nblk * sizeof(float));
  w.topk_blocks = align_up(w.super_max + (size_t)R * nsup * sizeof(float));
  w.topk_scores = align_up(w.topk_blocks + (size_t)R * (k > 0 ? k : 0) * sizeof(int32_t));
  w.key_floor = align_up(w.topk_scores + (size_t)R * (k > 0 ? k : 0) * 8 * sizeof(float));
  w.scores = align_up(w.key_floor + (size_t)R * sizeof(uint32_t));
  const bool store = M < kStoreScoresBelowM && k > 0;
  w.total = align_up(w.scores + (store ? (size_t)R * N_max * sizeof(float) : 0));
  return w;
}

// Every tensor pointer the caller passes must be 16-byte aligned (NULL passes).
inline bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }
template <typename... P>
inline bool any_misaligned(const P*... p) {
  return (misaligned(p) || ...);
}

constexpr int64_t kMaxRows = 1 << 24;
constexpr int64_t kMaxN = (int64_t)1 << 30;   // ids are int32; 8*blocks must fit
constexpr int kMaxPool = 1 << 20;
constexpr int kMaxFusedPool = 2048;   // pool blocks csa2_index_pool_topk scores in one workgroup
constexpr int kMaxRatio = 64;                          // tokens merged into one cached entry
constexpr int kMaxWriteDim = 1 << 14;                  // elements per cached row
constexpr int64_t kMaxWriteElems = (int64_t)1 << 40;   // fp32 input elements of one write call

}  // namespace

extern "C" {

const char* csa2_status_string(int status) {
  switch (status) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_INVALID: return "invalid argument";
    case CSA2_ERR_UNSUPPORTED: return "unsupported configuration";
    case CSA2_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA2_ERR_HIP: return "HIP launch failed";
    case CSA2_ERR_TOO_LARGE: return "needs more than the static scratch (CSA2_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int csa2_index_scan(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                    const uint8_t* k_scales, const int32_t* n_visible, int B, int M, int64_t N_max,
                    float* scores, float* block_max, float* super_max, void* stream) {
  if (!q_codes || !q_scales || !k_codes || !k_scales || !n_visible || !block_max) return CSA2_ERR_INVALID;
  if (any_misaligned(q_codes, q_scales, k_codes, k_scales, n_visible, scores, block_max, super_max))
    return CSA2_ERR_INVALID;
  if (B < 1 || M < 1 || N_max < 1 || N_max > kMaxN || (int64_t)B * M > kMaxRows) return CSA2_ERR_INVALID;
  return hip_status(csa2::launch_index_scan(q_codes, q_scales, k_codes, k_scales, n_visible, B, M, N_max, scores,
                                            block_max, (N_max + 7) / 8, super_max, (N_max + 63) / 64,
                                            as_stream(stream)));
}

int csa2_select_blocks(const float* block_max, const float* super_max, int64_t nblk_stride,
                       const int32_t* n_visible, int R, int n_pool, int32_t* pool_blocks, int k_blocks,
                       int32_t* topk_blocks, void* stream) {
  if (!block_max || !n_visible || !pool_blocks) return CSA2_ERR_INVALID;
  if (any_misaligned(block_max, super_max, n_visible, pool_blocks, topk_blocks)) return CSA2_ERR_INVALID;
  if (R < 1 || R > kMaxRows || n_pool < 1 || n_pool > kMaxPool || k_blocks < 0 || k_blocks > kMaxPool ||
      nblk_stride < 1 || nblk_stride > kMaxN / 8)
    return CSA2_ERR_INVALID;
  if (k_blocks > 0 && !topk_blocks) return CSA2_ERR_INVALID;
  return hip_status(csa2::launch_select(csa2::kSelBlocks, block_max, nblk_stride, nullptr, 0, n_visible, R, n_pool,
                                        pool_blocks, k_blocks, topk_blocks, super_max, (nblk_stride + 7) / 8,
                                        as_stream(stream)));
}

int csa2_index_pool(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                    const uint8_t* k_scales, const int32_t* pool_blocks, int n_pool, const int32_t* n_visible,
                    int B, int M, int64_t N_max, float* pool_scores, void* stream) {
  if (!q_codes || !q_scales || !k_codes || !k_scales || !pool_blocks || !n_visible || !pool_scores)
    return CSA2_ERR_INVALID;
  if (any_misaligned(q_codes, q_scales, k_codes, k_scales, pool_blocks, n_visible, pool_scores))
    return CSA2_ERR_INVALID;
  if (B < 1 || M < 1 || N_max < 1 || N_max > kMaxN || (int64_t)B * M > kMaxRows || n_pool < 1 ||
      n_pool > kMaxPool)
    return CSA2_ERR_INVALID;
  return hip_status(csa2::launch_pool_scan(q_codes, q_scales, k_codes, k_scales, pool_blocks, n_pool, n_visible, B,
                                           M, N_max, pool_scores, as_stream(stream)));
}

int csa2_topk(const float* scores, const int32_t* pool_blocks, int64_t n_pool, const int32_t* n_visible, int R,
              int k, int32_t* idx, void* stream) {
  if (!scores || !n_visible || !idx) return CSA2_ERR_INVALID;
  if (any_misaligned(scores, pool_blocks, n_visible, idx)) return CSA2_ERR_INVALID;
  if (R < 1 || R > kMaxRows || n_pool < 1 || k < 0 || k > kMaxPool) return CSA2_ERR_INVALID;
  if (pool_blocks ? n_pool > kMaxPool : n_pool > kMaxN) return CSA2_ERR_INVALID;
  if (k == 0) return CSA2_OK;
  const int layout = pool_blocks ? csa2::kSelPool : csa2::kSelFull;
  return hip_status(csa2::launch_select(layout, scores, pool_blocks ? 8 * n_pool : n_pool, pool_blocks, n_pool,
                                        n_visible, R, k, idx, 0, nullptr, nullptr, 0, as_stream(stream)));
}

int csa2_index_pool_topk(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                         const uint8_t* k_scales, const int32_t* pool_blocks, int n_pool, const int32_t* n_visible,
                         int B, int M, int64_t N_max, int k, int32_t* idx, void* stream) {
  if (!q_codes || !q_scales || !k_codes || !k_scales || !pool_blocks || !n_visible || !idx)
    return CSA2_ERR_INVALID;
  if (any_misaligned(q_codes, q_scales, k_codes, k_scales, pool_blocks, n_visible, idx)) return CSA2_ERR_INVALID;
  if (B < 1 || M < 1 || N_max < 1 || N_max > kMaxN || (int64_t)B * M > kMaxRows || n_pool < 1 ||
      n_pool > kMaxFusedPool || k < 0 || k > kMaxPool)
    return CSA2_ERR_INVALID;
  if (k == 0) return CSA2_OK;
  return hip_status(csa2::launch_pool_topk(q_codes, q_scales, k_codes, k_scales, pool_blocks, n_pool, n_visible, B, M,
                                           N_max, nullptr, k, idx, as_stream(stream)));
}

}  // extern "C"

namespace {

// Argument checks of csa2_index_full, apart from the workspace.
int index_full_args(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                    const uint8_t* k_scales, const int32_t* n_visible, int B, int M, int64_t N_max, int n_pool,
                    int k, const float* scores, const float* block_max, const int32_t* pool_blocks,
                    const int32_t* idx) {
  if (!q_codes || !q_scales || !k_codes || !k_scales || !n_visible || !pool_blocks) return CSA2_ERR_INVALID;
  if (any_misaligned(q_codes, q_scales, k_codes, k_scales, n_visible, scores, block_max, pool_blocks, idx))
    return CSA2_ERR_INVALID;
  if (B < 1 || M < 1 || N_max < 1 || N_max > kMaxN || (int64_t)B * M > kMaxRows || n_pool < 1 ||
      n_pool > kMaxPool || k < 0 || k > kMaxPool)
    return CSA2_ERR_INVALID;
  if (k > 0 && !idx) return CSA2_ERR_INVALID;
  return CSA2_OK;
}

// The Full-layer indexer's launches, with the arguments checked and `ws`
// holding at least full_ws(...).total bytes.
int index_full_run(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes, const uint8_t* k_scales,
                   const int32_t* n_visible, int B, int M, int64_t N_max, int n_pool, int k, float* scores,
                   float* block_max, int32_t* pool_blocks, int32_t* idx, char* ws, hipStream_t s) {
  const int64_t R = (int64_t)B * M;
  const int64_t nblk = (N_max + 7) / 8;
  const FullWs w = full_ws(R, M, N_max, k);
  float* bmax = block_max ? block_max : reinterpret_cast<float*>(ws + w.block_max);
  int32_t* topk_blocks = reinterpret_cast<int32_t*>(ws + w.topk_blocks);
  float* topk_scores = reinterpret_cast<float*>(ws + w.topk_scores);
  float* smax = reinterpret_cast<float*>(ws + w.super_max);
  const int64_t nsup = super_stride(N_max);
  // the pool's top-k lies in the pool's first min(k, n_pool) blocks
  const int kb = k < n_pool ? k : n_pool;
  if (M < kStoreScoresBelowM && k > 0) {
    // decode: the scan stores every score; one workgroup per row then builds the
    // pool and takes the top-k from the stored scores of its first kb blocks
    float* sc = scores ? scores : reinterpret_cast<float*>(ws + w.scores);
    hipError_t e = csa2::launch_index_scan(q_codes, q_scales, k_codes, k_scales, n_visible, B, M, N_max, sc, bmax,
                                           nblk, smax, nsup, s);
    if (e != hipSuccess) return CSA2_ERR_HIP;
    // every block in the pool: the top-k straight from the score rows
    e = csa2::launch_select_short(sc, N_max, n_visible, (int)R, n_pool, pool_blocks, k, idx, s);
    if (e != hipErrorNotSupported) return hip_status(e);
    e = csa2::launch_select_topk(bmax, nblk, smax, nsup, n_visible, (int)R, n_pool, pool_blocks, kb, sc, N_max, k,
                                 idx, s);
    if (e != hipErrorNotSupported) return hip_status(e);
    // shapes the fused kernel does not cover: the staged selection below (the
    // scan's outputs are in place)
  } else {
    const hipError_t e = csa2::launch_index_scan(q_codes, q_scales, k_codes, k_scales, n_visible, B, M, N_max,
                                                 scores, bmax, nblk, smax, nsup, s);
    if (e != hipSuccess) return CSA2_ERR_HIP;
  }
  // rescore only the first kb pool blocks
  // When the first kb = k blocks are the k best of the row, the k-th best block
  // maximum (the selection's floor) is at most the k-th best position score:
  // those k block maxima are k positions reaching it.  The top-k then drops
  // every slot below that floor unexamined.
  uint32_t* key_floor = reinterpret_cast<uint32_t*>(ws + w.key_floor);
  hipError_t e = csa2::launch_select(csa2::kSelBlocks, bmax, nblk, nullptr, 0, n_visible, (int)R, n_pool, pool_blocks,
                          kb, k > 0 ? topk_blocks : nullptr, smax, nsup, s, nullptr, key_floor);
  if (e != hipSuccess) return CSA2_ERR_HIP;
  if (k == 0) return CSA2_OK;
  // rescoring and top-k in one kernel where it covers the shape
  e = csa2::launch_pool_topk(q_codes, q_scales, k_codes, k_scales, topk_blocks, kb, n_visible, B, M, N_max,
                             kb == k ? key_floor : nullptr, k, idx, s);
  if (e != hipErrorNotSupported) return hip_status(e);
  e = csa2::launch_pool_scan(q_codes, q_scales, k_codes, k_scales, topk_blocks, kb, n_visible, B, M, N_max,
                             topk_scores, s);
  if (e != hipSuccess) return CSA2_ERR_HIP;
  e = csa2::launch_select(csa2::kSelPool, topk_scores, 8 * (int64_t)kb, topk_blocks, kb, n_visible, (int)R, k, idx,
                          0, nullptr, nullptr, 0, s, kb == k ? key_floor : nullptr, nullptr);
  return hip_status(e);
}

// The allocation-free entry point's scratch: one copy per device, in the code
// object's device memory, kept until the process ends.  Host code never uses
// the array's name as an address: the device address of each GPU's copy comes
// from hipGetSymbolAddress, taken once per device with that device current.
__device__ __align__(256) uint8_t scratch[CSA2_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of the scratch array (the stream's device).
int scratch_for(hipStream_t stream, char** out) {
  int dev = -1;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess) return CSA2_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return CSA2_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return CSA2_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return CSA2_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return CSA2_ERR_HIP;
    if (e != hipSuccess || !p) return CSA2_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return CSA2_OK;
}

}  // namespace

extern "C" {

int csa2_index_full(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                    const uint8_t* k_scales, const int32_t* n_visible, int B, int M, int64_t N_max, int n_pool,
                    int k, float* scores, float* block_max, int32_t* pool_blocks, int32_t* idx, void* workspace,
                    size_t workspace_bytes, void* stream) {
  const int st = index_full_args(q_codes, q_scales, k_codes, k_scales, n_visible, B, M, N_max, n_pool, k, scores,
                                 block_max, pool_blocks, idx);
  if (st != CSA2_OK) return st;
  if (misaligned(workspace)) return CSA2_ERR_INVALID;
  const FullWs w = full_ws((int64_t)B * M, M, N_max, k);
  if (!workspace || workspace_bytes < w.total) return CSA2_ERR_WORKSPACE;
  return index_full_run(q_codes, q_scales, k_codes, k_scales, n_visible, B, M, N_max, n_pool, k, scores, block_max,
                        pool_blocks, idx, static_cast<char*>(workspace), as_stream(stream));
}

int csa2_index_full_static(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                           const uint8_t* k_scales, const int32_t* n_visible, int B, int M, int64_t N_max,
                           int n_pool, int k, float* scores, float* block_max, int32_t* pool_blocks, int32_t* idx,
                           void* stream) {
  const int st = index_full_args(q_codes, q_scales, k_codes, k_scales, n_visible, B, M, N_max, n_pool, k, scores,
                                 block_max, pool_blocks, idx);
  if (st != CSA2_OK) return st;
  if (full_ws((int64_t)B * M, M, N_max, k).total > (size_t)CSA2_STATIC_SCRATCH_BYTES) return CSA2_ERR_TOO_LARGE;
  hipStream_t s = as_stream(stream);
  char* ws = nullptr;
  const int got = scratch_for(s, &ws);
  if (got != CSA2_OK) return got;
  return index_full_run(q_codes, q_scales, k_codes, k_scales, n_visible, B, M, N_max, n_pool, k, scores, block_max,
                        pool_blocks, idx, ws, s);
}

int csa2_sparse_attn(const float* q, const uint8_t* c_codes, const uint8_t* c_scales, const int32_t* idx, int k,
                     const uint8_t* win, const int32_t* win_start, const int32_t* win_len, int win_max, int B,
                     int M, int64_t N_max, int H, int Tw, float sm_scale, float* out, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!q || !out) return CSA2_ERR_INVALID;
  if (any_misaligned(q, c_codes, c_scales, idx, win, win_start, win_len, out, static_cast<const char*>(workspace)))
    return CSA2_ERR_INVALID;
  if (B < 1 || M < 1 || (int64_t)B * M > kMaxRows || k < 0 || k > kMaxPool || win_max < 0 || Tw < 0 ||
      win_max > Tw || N_max < 0 || N_max > kMaxN)
    return CSA2_ERR_INVALID;
  if (k > 0 && (!idx || !c_codes || !c_scales || N_max < 1)) return CSA2_ERR_INVALID;
  if (win_max > 0 && (!win || !win_start || !win_len)) return CSA2_ERR_INVALID;
  if (!(sm_scale == sm_scale)) return CSA2_ERR_INVALID;
  if (H != 16 && H != 32 && H != 64) return CSA2_ERR_UNSUPPORTED;
  const int R = B * M;
  const size_t need = csa2::attn_workspace_bytes(R, H, k + win_max);
  if (need > 0 && (!workspace || workspace_bytes < need)) return CSA2_ERR_WORKSPACE;
  csa2::AttnLaunch L;
  L.q = q;
  L.c_codes = c_codes;
  L.c_scales = c_scales;
  L.idx = idx;
  L.k = k;
  L.win = win;
  L.win_start = win_start;
  L.win_len = win_len;
  L.win_max = win_max;
  L.B = B;
  L.M = M;
  L.H = H;
  L.Tw = Tw;
  L.N_max = N_max;
  L.sm_scale = sm_scale;
  L.out = out;
  L.workspace = workspace;
  L.workspace_bytes = workspace_bytes;
  return hip_status(csa2::launch_sparse_attn(L, as_stream(stream)));
}

int csa2_cache_write_mxfp4(const float* x, const float* w, int64_t n_entries, int ratio, int D, uint8_t* codes,
                           uint8_t* scales, void* stream) {
  if (n_entries < 0 || ratio < 1 || ratio > kMaxRatio || D < 32 || D > kMaxWriteDim || (D & (D - 1)) != 0)
    return CSA2_ERR_INVALID;
  if (n_entries == 0) return CSA2_OK;   // nothing to write: pointers unused
  if (!x || !codes || !scales) return CSA2_ERR_INVALID;
  // entries are appended at any offset of a cache, so only what the kernel
  // moves in vectors is held to 16 bytes: the fp32 rows (codes go out as
  // 2-byte words, weights as floats, scales as bytes)
  if (misaligned(x) || (reinterpret_cast<uintptr_t>(w) & 3u) != 0 || (reinterpret_cast<uintptr_t>(codes) & 1u) != 0)
    return CSA2_ERR_INVALID;
  if (ratio > 1 && !w) return CSA2_ERR_INVALID;
  if (n_entries > kMaxWriteElems / ((int64_t)ratio * D)) return CSA2_ERR_INVALID;
  return hip_status(csa2::launch_write_mxfp4(x, w, n_entries, ratio, D, codes, scales, as_stream(stream)));
}

int csa2_cache_write_e4m3(const float* x, int64_t n, uint8_t* out, void* stream) {
  if (n < 0 || n % 4 != 0 || n > kMaxWriteElems) return CSA2_ERR_INVALID;
  if (n == 0) return CSA2_OK;
  if (!x || !out) return CSA2_ERR_INVALID;
  if (misaligned(x) || (reinterpret_cast<uintptr_t>(out) & 3u) != 0) return CSA2_ERR_INVALID;
  return hip_status(csa2::launch_write_e4m3(x, n, out, as_stream(stream)));
}

size_t csa2_workspace_bytes(int op, int B, int M, int64_t N_max, int H, int k) {
  if (B < 1 || M < 1 || k < 0) return 0;
  const int64_t R = (int64_t)B * M;
  if (op == CSA2_OP_INDEX_FULL) {
    if (N_max < 1) return 0;
    return full_ws(R, M, N_max, k).total;
  }
  if (op == CSA2_OP_SPARSE_ATTN) {
    if (H != 16 && H != 32 && H != 64) return 0;
    return csa2::attn_workspace_bytes((int)R, H, k);
  }
  return 0;
}

}  // extern "C"
