"""CPU oracle for the CSA2 hierarchical sparse attention step (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the benchmark's
CPU-baseline leg.  The library's product path never imports this package.
The arithmetic lives in csa2_oracle.c (plain C, fixed-order fp32 score, full
sorts, double-precision attention); this wrapper only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_HDR = os.path.join(_HERE, "csa2_oracle.h")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-o", _LIB_PATH, _SRC, "-lm", "-lpthread"]
    subprocess.check_call(cmd)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        newest = max(os.path.getmtime(_SRC), os.path.getmtime(_HDR))
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < newest:
            build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        L.orc_e2m1_value.argtypes = [ctypes.c_uint]
        L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_e8m0_scale.argtypes = [ctypes.c_uint]
        L.orc_e8m0_scale.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ctypes.c_uint]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_encode.argtypes = [ctypes.c_double]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_mxfp4_encode_block.argtypes = [vp, vp, vp]
        L.orc_merge_f32.argtypes = [vp, vp, i64, i32, i32, vp]
        L.orc_merge_f32.restype = ctypes.c_int
        L.orc_cache_write_mxfp4.argtypes = [vp, vp, i64, i32, i32, vp, vp]
        L.orc_cache_write_mxfp4.restype = ctypes.c_int
        L.orc_cache_write_e4m3.argtypes = [vp, i64, vp]
        L.orc_cache_write_e4m3.restype = None
        L.orc_score.argtypes = [vp, vp, vp, vp]
        L.orc_score.restype = ctypes.c_float
        L.orc_order_key.argtypes = [ctypes.c_float]
        L.orc_order_key.restype = ctypes.c_uint32
        L.orc_index_full.argtypes = [vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, vp, vp, vp, vp, i32, i32]
        L.orc_index_pool.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i32, i64, vp, i32]
        L.orc_topk_pool.argtypes = [vp, vp, i32, vp, i64, i32, vp, i32]
        L.orc_topk_full.argtypes = [vp, vp, i64, i64, i32, vp, i32]
        L.orc_sparse_attn.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i64, i32, i32, f32, vp, i32]
        for f in ("orc_index_full", "orc_index_pool", "orc_topk_pool", "orc_topk_full", "orc_sparse_attn"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def threads_default() -> int:
    return max(1, os.cpu_count() or 1)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


# ---------------- formats ----------------
def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(code)


def e8m0_scale(byte: int) -> float:
    return lib().orc_e8m0_scale(byte)


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(code)


def e4m3_encode(x: float) -> int:
    return int(lib().orc_e4m3_encode(float(x)))


def mxfp4_encode(x: np.ndarray):
    """Encode the last axis (a multiple of 32) of x; returns (codes, scales)."""
    x = np.ascontiguousarray(x, np.float64)
    n = x.shape[-1]
    assert n % 32 == 0
    flat = x.reshape(-1, 32)
    codes = np.empty((flat.shape[0], 16), np.uint8)
    scales = np.empty(flat.shape[0], np.uint8)
    for i in range(flat.shape[0]):
        lib().orc_mxfp4_encode_block(_p(flat[i]), _p(codes[i]), _p(scales[i:i + 1]))
    return codes.reshape(*x.shape[:-1], n // 2), scales.reshape(*x.shape[:-1], n // 32)


def mxfp4_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, np.uint8)
    lo = codes & 15
    hi = codes >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    table = np.array([e2m1_value(c) for c in range(16)])
    sc = np.array([e8m0_scale(b) for b in range(256)])
    v = table[nib]
    s = np.repeat(sc[np.asarray(scales, np.uint8)], 32, axis=-1)
    return v * s


def score(qc, qs, kc, ks) -> float:
    qc, qs, kc, ks = (_c(a, np.uint8) for a in (qc, qs, kc, ks))
    return float(np.float32(lib().orc_score(_p(qc), _p(qs), _p(kc), _p(ks))))


def order_key(f: float) -> int:
    return int(lib().orc_order_key(float(f)))


# ---------------- cache write ----------------
def merge(x, w, ratio):
    """fp32 ratio-m merge of token rows x [n*ratio, D] with weights w [n*ratio]
    (None: weight 1) -> [n, D] float32."""
    x = _c(x, np.float32)
    T, D = x.shape
    assert T % ratio == 0
    w = None if w is None else _c(w, np.float32)
    out = np.empty((T // ratio, D), np.float32)
    assert lib().orc_merge_f32(_p(x), _p(w), T // ratio, ratio, D, _p(out)) == 0
    return out


def cache_write_mxfp4(x, w, ratio):
    """Merged entries of x [n*ratio, D] stored as MXFP4: (codes [n, D/2], scales [n, D/32])."""
    x = _c(x, np.float32)
    T, D = x.shape
    assert T % ratio == 0
    n = T // ratio
    w = None if w is None else _c(w, np.float32)
    codes = np.empty((n, D // 2), np.uint8)
    scales = np.empty((n, D // 32), np.uint8)
    assert lib().orc_cache_write_mxfp4(_p(x), _p(w), n, ratio, D, _p(codes), _p(scales)) == 0
    return codes, scales


def cache_write_e4m3(x):
    """FP8 E4M3 code of every element of x (float32), same shape, uint8."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().orc_cache_write_e4m3(_p(x), x.size, _p(out))
    return out


# ---------------- the step ----------------
def index_full(q_codes, q_scales, k_codes, k_scales, n_visible, B, M, N_max, n_pool=2048, k=512,
               want_scores=False, want_block_max=False, global_topk=False, threads=None):
    R = B * M
    q_codes, q_scales = _c(q_codes, np.uint8), _c(q_scales, np.uint8)
    k_codes, k_scales = _c(k_codes, np.uint8), _c(k_scales, np.uint8)
    n_visible = _c(n_visible, np.int32)
    assert q_codes.size == R * 64 and k_codes.size == B * N_max * 64
    nblk_max = (N_max + 7) // 8
    scores = np.full((R, N_max), np.nan, np.float32) if want_scores else None
    bmax = np.full((R, nblk_max), np.nan, np.float32) if want_block_max else None
    pool = np.empty((R, n_pool), np.int32)
    idx = np.empty((R, k), np.int32) if k > 0 else None
    rc = lib().orc_index_full(_p(q_codes), _p(q_scales), _p(k_codes), _p(k_scales), _p(n_visible),
                              B, M, N_max, n_pool, k, _p(scores), _p(bmax), _p(pool), _p(idx),
                              1 if global_topk else 0, threads or threads_default())
    assert rc == 0
    out = {"pool_blocks": pool}
    if idx is not None:
        out["idx"] = idx
    if scores is not None:
        out["scores"] = scores
    if bmax is not None:
        out["block_max"] = bmax
    return out


def index_pool(q_codes, q_scales, k_codes, k_scales, pool_blocks, n_visible, B, M, N_max, threads=None):
    R = B * M
    q_codes, q_scales = _c(q_codes, np.uint8), _c(q_scales, np.uint8)
    k_codes, k_scales = _c(k_codes, np.uint8), _c(k_scales, np.uint8)
    pool_blocks = _c(pool_blocks, np.int32)
    n_visible = _c(n_visible, np.int32)
    n_pool = pool_blocks.shape[-1]
    out = np.empty((R, n_pool * 8), np.float32)
    rc = lib().orc_index_pool(_p(q_codes), _p(q_scales), _p(k_codes), _p(k_scales), _p(pool_blocks), n_pool,
                              _p(n_visible), B, M, N_max, _p(out), threads or threads_default())
    assert rc == 0
    return out


def topk_pool(pool_scores, pool_blocks, n_visible, k, threads=None):
    pool_scores = _c(pool_scores, np.float32)
    pool_blocks = _c(pool_blocks, np.int32)
    n_visible = _c(n_visible, np.int32)
    R, n_pool = pool_blocks.shape
    idx = np.empty((R, k), np.int32)
    rc = lib().orc_topk_pool(_p(pool_scores), _p(pool_blocks), n_pool, _p(n_visible), R, k, _p(idx),
                             threads or threads_default())
    assert rc == 0
    return idx


def topk_full(scores, n_visible, k, threads=None):
    scores = _c(scores, np.float32)
    n_visible = _c(n_visible, np.int32)
    R, N_max = scores.shape
    idx = np.empty((R, k), np.int32)
    rc = lib().orc_topk_full(_p(scores), _p(n_visible), R, N_max, k, _p(idx), threads or threads_default())
    assert rc == 0
    return idx


def sparse_attn(q, c_codes, c_scales, idx, win, win_start, win_len, B, M, N_max, sm_scale, threads=None,
                win_max=None):
    """win_max: rows per window at most (None: the window store's length Tw)."""
    q = _c(q, np.float32)
    R, H, D = q.shape
    assert D == 512 and R == B * M
    c_codes, c_scales = _c(c_codes, np.uint8), _c(c_scales, np.uint8)
    idx = _c(idx, np.int32).reshape(R, -1)
    k = idx.shape[1]
    win = _c(win, np.uint8)
    Tw = win.shape[1] if win.size else 0
    win_max = Tw if win_max is None else int(win_max)
    win_start, win_len = _c(win_start, np.int32), _c(win_len, np.int32)
    out = np.empty((R, H, 512), np.float32)
    rc = lib().orc_sparse_attn(_p(q), _p(c_codes), _p(c_scales), _p(idx), k, _p(win), _p(win_start),
                               _p(win_len), win_max, B, M, N_max, H, Tw, float(sm_scale), _p(out),
                               threads or threads_default())
    assert rc == 0
    return out
