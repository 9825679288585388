"""MI355X (gfx950) CSA2 hierarchical sparse attention: Python binding of the C ABI.

Every function here marshals torch tensors (device memory) and the current HIP
stream into the C entry points of libcsa2.so with the same names; all of the
step's arithmetic runs in the HIP kernels.  Shapes and dtypes are checked on the
host before any call so that a mis-shaped tensor never reaches a kernel.  There
is no fallback: if the library is missing, importing the functions raises.

The step (DeepSeek-V4.1-Flash, fupanwang.com article, section 三个方向一起压小缓存
and its hierarchical-sparse-indexer figure caption; section 后 20 层干脆共用一份 KV
for the 128-token window; dreamax.pages.dev notes, CSA2 paragraph, for the
Full / Reindex / Reuse modes):
    Full    : csa2_index_full (scan -> 8-position block max -> 2048-block pool ->
              top-512) then csa2_sparse_attn
    Reindex : csa2_index_pool over the Full layer's pool -> csa2_topk -> attention
              (csa2_index_pool_topk, the same in one call, from 1,024 rows up)
    Reuse   : csa2_sparse_attn with the previous layer's indices
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

CSA2_OK = 0
CSA2_ERR_INVALID = -1
CSA2_ERR_UNSUPPORTED = -2
CSA2_ERR_WORKSPACE = -3
CSA2_ERR_HIP = -4
CSA2_ERR_TOO_LARGE = -5
CSA2_STATIC_SCRATCH_BYTES = 64 << 20
CSA2_OP_INDEX_FULL = 1
CSA2_OP_SPARSE_ATTN = 2

EXPORTED = (
    "csa2_index_scan", "csa2_select_blocks", "csa2_index_pool", "csa2_topk", "csa2_index_pool_topk", "csa2_index_full",
    "csa2_index_full_static", "csa2_sparse_attn", "csa2_cache_write_mxfp4", "csa2_cache_write_e4m3",
    "csa2_workspace_bytes", "csa2_status_string",
)

_lib = None


class Csa2Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load libcsa2.so (built by build.py); raises if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with hierarchical_sparse_attention_csa2_amd/build.py "
                           "(there is no CPU fallback)")
    L = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.csa2_index_scan.argtypes = [vp, vp, vp, vp, vp, i32, i32, i64, vp, vp, vp, vp]
    L.csa2_select_blocks.argtypes = [vp, vp, i64, vp, i32, i32, vp, i32, vp, vp]
    L.csa2_index_pool.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i32, i64, vp, vp]
    L.csa2_topk.argtypes = [vp, vp, i64, vp, i32, i32, vp, vp]
    L.csa2_index_pool_topk.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i32, i64, i32, vp, vp]
    L.csa2_index_full.argtypes = [vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    L.csa2_index_full_static.argtypes = [vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, vp, vp, vp, vp, vp]
    L.csa2_sparse_attn.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i64, i32, i32, f32, vp, vp, sz,
                                   vp]
    L.csa2_cache_write_mxfp4.argtypes = [vp, vp, i64, i32, i32, vp, vp, vp]
    L.csa2_cache_write_e4m3.argtypes = [vp, i64, vp, vp]
    L.csa2_workspace_bytes.argtypes = [i32, i32, i32, i64, i32, i32]
    L.csa2_workspace_bytes.restype = sz
    L.csa2_status_string.argtypes = [i32]
    L.csa2_status_string.restype = ctypes.c_char_p
    for f in ("csa2_index_scan", "csa2_select_blocks", "csa2_index_pool", "csa2_topk", "csa2_index_full",
              "csa2_index_full_static", "csa2_sparse_attn", "csa2_cache_write_mxfp4", "csa2_cache_write_e4m3"):
        getattr(L, f).restype = i32
    _lib = L
    return L


def status_string(status: int) -> str:
    return load_library().csa2_status_string(int(status)).decode()


def csa2_status_string(status: int) -> str:
    return status_string(status)


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name, dtype, shape=None, numel=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    if _recording is not None:
        _recording_keep.append(t)   # a recorded call's tensors live as long as its replay
    return ctypes.c_void_p(t.data_ptr())


def _check(fn, status):
    if status != CSA2_OK:
        raise Csa2Error(fn, status)


_recording = None
_recording_keep = None


def _call(name, *args):
    """Call C entry point `name` with marshalled arguments, or, inside
    recording(), append the call for a later replay instead."""
    fn = getattr(load_library(), name)
    if _recording is not None:
        _recording.append((name, fn, args))
        return
    _check(name, fn(*args))


class recording:
    """Context manager: the entry points called inside it are validated and
    marshalled as usual but not run; `launches` then issues them again, in
    order, with the same raw arguments (device pointers and the stream that was
    current when they were recorded), so the tensors they name must stay alive
    and in place.  For tight launch loops where the per-call checks cost more
    host time than the kernels take."""

    def __enter__(self):
        global _recording, _recording_keep
        if _recording is not None:
            raise RuntimeError("recording() does not nest")
        _recording = self.calls = []
        _recording_keep = self.keep = []
        return self

    def __exit__(self, *exc):
        global _recording, _recording_keep
        _recording = _recording_keep = None
        return False

    def launches(self):
        calls, keep = list(self.calls), list(self.keep)

        def issue():
            for name, fn, args in calls:
                st = fn(*args)
                if st != CSA2_OK:
                    raise Csa2Error(name, st)
        issue.tensors = keep   # the recorded tensors (workspaces included) live as long as `issue`
        return issue


U8, I32, F32 = torch.uint8, torch.int32, torch.float32


# ---------------------------------------------------------------------------
# the C entry points
# ---------------------------------------------------------------------------
def csa2_workspace_bytes(op: int, B: int, M: int, N_max: int, H: int, k: int) -> int:
    return int(load_library().csa2_workspace_bytes(op, B, M, N_max, H, k))


def csa2_index_scan(q_codes, q_scales, k_codes, k_scales, n_visible, B, M, N_max, block_max, scores=None,
                    super_max=None, stream=None):
    R = B * M
    nblk = (N_max + 7) // 8
    nsup = (N_max + 63) // 64
    _call("csa2_index_scan", 
        _dev(q_codes, "q_codes", U8, (R, 64)), _dev(q_scales, "q_scales", U8, (R, 4)),
        _dev(k_codes, "k_codes", U8, numel=B * N_max * 64), _dev(k_scales, "k_scales", U8, numel=B * N_max * 4),
        _dev(n_visible, "n_visible", I32, (R,)), B, M, N_max,
        _dev(scores, "scores", F32, (R, N_max), optional=True), _dev(block_max, "block_max", F32, (R, nblk)),
        _dev(super_max, "super_max", F32, (R, nsup), optional=True), _stream(stream))


def csa2_select_blocks(block_max, n_visible, n_pool, pool_blocks, k_blocks=0, topk_blocks=None, super_max=None,
                       stream=None):
    R, stride = block_max.shape
    _call("csa2_select_blocks", 
        _dev(block_max, "block_max", F32), _dev(super_max, "super_max", F32, (R, (stride + 7) // 8), optional=True),
        stride, _dev(n_visible, "n_visible", I32, (R,)), R, n_pool,
        _dev(pool_blocks, "pool_blocks", I32, (R, n_pool)), k_blocks,
        _dev(topk_blocks, "topk_blocks", I32, (R, k_blocks), optional=k_blocks == 0), _stream(stream))


def csa2_index_pool(q_codes, q_scales, k_codes, k_scales, pool_blocks, n_visible, B, M, N_max, pool_scores,
                    stream=None):
    R = B * M
    n_pool = pool_blocks.shape[1]
    _call("csa2_index_pool", 
        _dev(q_codes, "q_codes", U8, (R, 64)), _dev(q_scales, "q_scales", U8, (R, 4)),
        _dev(k_codes, "k_codes", U8, numel=B * N_max * 64), _dev(k_scales, "k_scales", U8, numel=B * N_max * 4),
        _dev(pool_blocks, "pool_blocks", I32, (R, n_pool)), n_pool, _dev(n_visible, "n_visible", I32, (R,)),
        B, M, N_max, _dev(pool_scores, "pool_scores", F32, (R, 8 * n_pool)), _stream(stream))


def csa2_index_pool_topk(q_codes, q_scales, k_codes, k_scales, pool_blocks, n_visible, B, M, N_max, k, idx,
                         stream=None):
    R = B * M
    n_pool = pool_blocks.shape[1]
    _call("csa2_index_pool_topk",
        _dev(q_codes, "q_codes", U8, (R, 64)), _dev(q_scales, "q_scales", U8, (R, 4)),
        _dev(k_codes, "k_codes", U8, numel=B * N_max * 64), _dev(k_scales, "k_scales", U8, numel=B * N_max * 4),
        _dev(pool_blocks, "pool_blocks", I32, (R, n_pool)), n_pool, _dev(n_visible, "n_visible", I32, (R,)),
        B, M, N_max, k, _dev(idx, "idx", I32, (R, k)), _stream(stream))


def csa2_topk(scores, n_visible, k, idx, pool_blocks=None, stream=None):
    R = scores.shape[0]
    if pool_blocks is not None:
        n_pool = pool_blocks.shape[1]
        sc = _dev(scores, "scores", F32, (R, 8 * n_pool))
        pb = _dev(pool_blocks, "pool_blocks", I32, (R, n_pool))
    else:
        n_pool = scores.shape[1]
        sc = _dev(scores, "scores", F32, (R, n_pool))
        pb = None
    _call("csa2_topk", sc, pb, n_pool, _dev(n_visible, "n_visible", I32, (R,)), R, k,
                                  _dev(idx, "idx", I32, (R, k)), _stream(stream))


def csa2_index_full(q_codes, q_scales, k_codes, k_scales, n_visible, B, M, N_max, n_pool, k, pool_blocks,
                    idx=None, workspace=None, scores=None, block_max=None, stream=None):
    R = B * M
    nblk = (N_max + 7) // 8
    need = csa2_workspace_bytes(CSA2_OP_INDEX_FULL, B, M, N_max, 0, k)
    if workspace is None:
        workspace = torch.empty(need, dtype=U8, device=q_codes.device)
    if workspace.numel() < need:
        raise ValueError(f"workspace has {workspace.numel()} bytes, needs {need}")
    _call("csa2_index_full", 
        _dev(q_codes, "q_codes", U8, (R, 64)), _dev(q_scales, "q_scales", U8, (R, 4)),
        _dev(k_codes, "k_codes", U8, numel=B * N_max * 64), _dev(k_scales, "k_scales", U8, numel=B * N_max * 4),
        _dev(n_visible, "n_visible", I32, (R,)), B, M, N_max, n_pool, k,
        _dev(scores, "scores", F32, (R, N_max), optional=True),
        _dev(block_max, "block_max", F32, (R, nblk), optional=True),
        _dev(pool_blocks, "pool_blocks", I32, (R, n_pool)), _dev(idx, "idx", I32, (R, k), optional=k == 0),
        _dev(workspace, "workspace", U8), workspace.numel(), _stream(stream))


def csa2_index_full_static(q_codes, q_scales, k_codes, k_scales, n_visible, B, M, N_max, n_pool, k, pool_blocks,
                           idx=None, scores=None, block_max=None, stream=None):
    """csa2_index_full on the library's static per-device scratch: allocates
    nothing (no workspace tensor either).  Raises Csa2Error with
    CSA2_ERR_TOO_LARGE when the problem needs more than
    CSA2_STATIC_SCRATCH_BYTES of scratch.  Calls that overlap on one device
    race on that scratch; calls ordered on one stream do not."""
    R = B * M
    nblk = (N_max + 7) // 8
    _call("csa2_index_full_static",
        _dev(q_codes, "q_codes", U8, (R, 64)), _dev(q_scales, "q_scales", U8, (R, 4)),
        _dev(k_codes, "k_codes", U8, numel=B * N_max * 64), _dev(k_scales, "k_scales", U8, numel=B * N_max * 4),
        _dev(n_visible, "n_visible", I32, (R,)), B, M, N_max, n_pool, k,
        _dev(scores, "scores", F32, (R, N_max), optional=True),
        _dev(block_max, "block_max", F32, (R, nblk), optional=True),
        _dev(pool_blocks, "pool_blocks", I32, (R, n_pool)), _dev(idx, "idx", I32, (R, k), optional=k == 0),
        _stream(stream))


def csa2_sparse_attn(q, c_codes, c_scales, idx, win, win_start, win_len, win_max, B, M, N_max, sm_scale, out,
                     workspace=None, stream=None):
    R, H, D = q.shape
    if D != 512 or R != B * M:
        raise ValueError("q must be [B*M, H, 512]")
    k = idx.shape[1] if idx is not None else 0
    Tw = win.shape[1] if win is not None else 0
    if win is not None and tuple(win.shape) != (B, Tw, 512):
        raise ValueError("win must be [B, Tw, 512]")
    need = csa2_workspace_bytes(CSA2_OP_SPARSE_ATTN, B, M, 0, H, k + win_max)
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=U8, device=q.device)
    if need > 0 and workspace.numel() < need:
        raise ValueError(f"workspace has {workspace.numel()} bytes, needs {need}")
    _call("csa2_sparse_attn", 
        _dev(q, "q", F32, (R, H, 512)),
        _dev(c_codes, "c_codes", U8, numel=B * N_max * 256, optional=k == 0),
        _dev(c_scales, "c_scales", U8, numel=B * N_max * 16, optional=k == 0),
        _dev(idx, "idx", I32, (R, k), optional=k == 0), k,
        _dev(win, "win", U8, optional=win_max == 0), _dev(win_start, "win_start", I32, (R,), optional=win_max == 0),
        _dev(win_len, "win_len", I32, (R,), optional=win_max == 0), win_max, B, M, N_max, H, Tw, float(sm_scale),
        _dev(out, "out", F32, (R, H, 512)),
        _dev(workspace, "workspace", U8, optional=True) if workspace is not None else None,
        workspace.numel() if workspace is not None else 0, _stream(stream))


def csa2_cache_write_mxfp4(x, w, ratio, codes, scales, stream=None):
    """Merge every `ratio` consecutive token rows of x [n*ratio, D] with weights
    w [n*ratio] (None only for ratio 1) and write the MXFP4 entries into codes
    [n, D/2] and scales [n, D/32] (contiguous views into a cache are fine)."""
    if x.dim() != 2:
        raise ValueError("x must be [tokens, D]")
    T, D = x.shape
    if ratio < 1 or T % ratio:
        raise ValueError(f"{T} token rows do not split into groups of {ratio}")
    n = T // ratio
    _call("csa2_cache_write_mxfp4", 
        _dev(x, "x", F32), _dev(w, "w", F32, (T,), optional=ratio == 1), n, int(ratio), D,
        _dev(codes, "codes", U8, numel=n * (D // 2)), _dev(scales, "scales", U8, numel=n * (D // 32)),
        _stream(stream))


def csa2_cache_write_e4m3(x, out, stream=None):
    """FP8 E4M3 codes of every element of x (e.g. window rows [rows, 512]) into
    out (uint8, same number of elements)."""
    n = x.numel()
    _call("csa2_cache_write_e4m3", _dev(x, "x", F32), n, _dev(out, "out", U8, numel=n), _stream(stream))
