"""Seeded synthetic inputs for the CSA2 hierarchical sparse attention step.

Data preparation only (no scoring, selection or attention arithmetic): iid
N(0,1) draws from Philox-4x32-10 + Box-Muller, stored in the formats the pages
give for the cached state (DeepSeek-V4.1-Flash article on fupanwang.com, section
"三个方向一起压小缓存": FP4 indexer query/key, OCP MXFP4 main KV, FP8 sliding
window).  The five workloads below carry the pages' constants: 8-position
blocks, a 2048-block pool (16,384 positions), top-512, a 128-token window and a
1M-token context (same section and its figure caption on the hierarchical
sparse indexer).

Both the HIP path and the oracle consume exactly these bytes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

BASE_SEED = 20260919

# tensor ids of the Philox counter
T_INDEX_KEYS = 1
T_LATENT = 2
T_MERGE_LOGITS = 3
# fp32 token rows before the cache write (latent, indexer key, window)
T_TOKEN_LATENT = 7
T_TOKEN_INDEX = 8
T_TOKEN_WINDOW = 9


def t_index_query(layer: int) -> int:
    return 16 * layer + 4


def t_attn_query(layer: int) -> int:
    return 16 * layer + 5


def t_window(layer: int) -> int:
    return 16 * layer + 6


def build() -> str:
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-o", _LIB_PATH, _SRC, "-lm", "-lpthread"]
    subprocess.check_call(cmd)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        u64, u32, i32, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p
        L.synth_mxfp4.argtypes = [u64, u32, u64, u64, i32, vp, vp, i32]
        L.synth_mxfp4_merged2.argtypes = [u64, u32, u32, u64, u64, i32, vp, vp, i32]
        L.synth_e4m3.argtypes = [u64, u32, u64, u64, i32, vp, i32]
        L.synth_f32.argtypes = [u64, u32, u64, u64, i32, vp, i32]
        L.synth_normals.argtypes = [u64, u32, u64, u64, i32, vp]
        L.synth_merge_weights.argtypes = [u64, u32, u64, vp]
        L.synth_merge_weights_f32.argtypes = [u64, u32, u64, u64, vp]
        L.synth_merge_weights_f32.restype = None
        L.synth_mxfp4_encode_block.argtypes = [vp, vp, vp]
        L.synth_e4m3_encode.argtypes = [ctypes.c_double]
        L.synth_e4m3_encode.restype = ctypes.c_uint8
        L.synth_philox4x32_10.argtypes = [vp, vp, vp]
        for f in ("synth_mxfp4", "synth_mxfp4_merged2", "synth_e4m3", "synth_f32", "synth_normals"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def mxfp4(seed, tensor, row0, nrows, cols, threads=None, merged_logits=None):
    codes = np.empty((nrows, cols // 2), np.uint8)
    scales = np.empty((nrows, cols // 32), np.uint8)
    th = threads or default_threads()
    if merged_logits is None:
        rc = lib().synth_mxfp4(seed, tensor, row0, nrows, cols, _p(codes), _p(scales), th)
    else:
        rc = lib().synth_mxfp4_merged2(seed, tensor, merged_logits, row0, nrows, cols, _p(codes), _p(scales), th)
    assert rc == 0
    return codes, scales


def e4m3(seed, tensor, row0, nrows, cols, threads=None):
    out = np.empty((nrows, cols), np.uint8)
    assert lib().synth_e4m3(seed, tensor, row0, nrows, cols, _p(out), threads or default_threads()) == 0
    return out


def f32(seed, tensor, row0, nrows, cols, threads=None):
    out = np.empty((nrows, cols), np.float32)
    assert lib().synth_f32(seed, tensor, row0, nrows, cols, _p(out), threads or default_threads()) == 0
    return out


def normals(seed, tensor, row0, nrows, cols):
    out = np.empty((nrows, cols), np.float64)
    assert lib().synth_normals(seed, tensor, row0, nrows, cols, _p(out)) == 0
    return out


def merge_weights(seed, logit_tensor, row):
    w = np.empty(2, np.float64)
    lib().synth_merge_weights(seed, logit_tensor, row, _p(w))
    return w


def merge_weights_f32(seed, logit_tensor, row0, nrows):
    """Merge weights of entries [row0, row0+nrows) as float32, flattened per token
    ([2*nrows]: token 2r and 2r+1 of entry row0 + r)."""
    out = np.empty(2 * nrows, np.float32)
    lib().synth_merge_weights_f32(seed, logit_tensor, row0, nrows, _p(out))
    return out


def philox(ctr, key):
    c = np.asarray(ctr, np.uint32)
    k = np.asarray(key, np.uint32)
    o = np.empty(4, np.uint32)
    lib().synth_philox4x32_10(_p(c), _p(k), _p(o))
    return o


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
@dataclass
class Workload:
    """One synthetic workload.

    B sequences, each with its own cache of N entries; M query rows per
    sequence (M=1 decode, M>1 prefill); H attention heads of width 512; a pool
    of n_pool 8-position blocks; top-k; a window of win_len FP8 rows taken from
    a per-sequence window buffer of Tw rows.  ratio 2 builds each cached entry as
    the softmax-weighted mean of two adjacent tokens.
    """
    name: str
    seed: int
    B: int
    N: int
    M: int = 1
    H: int = 64
    n_pool: int = 2048
    k: int = 512
    win_len: int = 128
    ratio: int = 1
    layers: tuple = ("full",)
    prefill_base: int = -1          # >= 0: query m sits at position prefill_base + m
    notes: str = ""

    @property
    def R(self) -> int:
        return self.B * self.M

    @property
    def Tw(self) -> int:
        if self.prefill_base >= 0:
            return self.win_len + self.M - 1
        return self.win_len

    def n_visible(self) -> np.ndarray:
        if self.prefill_base >= 0:
            nv = self.prefill_base + 1 + np.arange(self.M, dtype=np.int64)
            return np.tile(nv, self.B).astype(np.int32)
        return np.full(self.R, self.N, np.int32)

    def win_start(self) -> np.ndarray:
        if self.prefill_base >= 0:
            return np.tile(np.arange(self.M, dtype=np.int32), self.B)
        return np.zeros(self.R, np.int32)

    def win_len_arr(self) -> np.ndarray:
        return np.full(self.R, self.win_len, np.int32)

    def scaled(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "c1": Workload("c1_full_b1_n4096", BASE_SEED + 0, B=1, N=4096,
                   notes="Full layer, 1 decode query, 4,096 cached entries (ratio 1)"),
    "c2": Workload("c2_full_b32_n65536", BASE_SEED + 1, B=32, N=65536,
                   notes="Full layer, 32 decode queries, 65,536 cached entries each"),
    "c3": Workload("c3_full_b4_1m_ratio2", BASE_SEED + 2, B=4, N=524288, ratio=2,
                   notes="Full layer, 4 decode queries, 1,048,576 tokens at ratio 2 = 524,288 entries"),
    "c4": Workload("c4_chain_b64_n131072", BASE_SEED + 3, B=64, N=131072,
                   layers=("full", "reindex", "reindex", "reuse"),
                   notes="Full -> Reindex -> Reindex -> Reuse, 64 decode queries, 131,072 entries"),
    "c5": Workload("c5_prefill_4096_on_262144", BASE_SEED + 4, B=1, N=266240, M=4096,
                   prefill_base=262144,
                   notes="prefill chunk of 4,096 causal queries at positions 262,144..266,239"),
    # multi-token decode (a verify step over the drafter's 5 positions) on the
    # 1M-token cache of c3: the 5 queries of a sequence see entries up to their
    # own positions
    "v3": Workload("v3_verify_b4_m5_1m_ratio2", BASE_SEED + 2, B=4, N=524288, M=5, ratio=2,
                   prefill_base=524288 - 5,
                   notes="Full layer, 4 sequences x 5 causal decode queries (a verify step), 1,048,576 tokens "
                         "at ratio 2 = 524,288 entries"),
}


def gen_cache(w: Workload, threads=None):
    """Index keys and latent for all B sequences: dict of numpy arrays."""
    rows = w.B * w.N
    if w.ratio == 1:
        kc, ks = mxfp4(w.seed, T_INDEX_KEYS, 0, rows, 128, threads)
        cc, cs = mxfp4(w.seed, T_LATENT, 0, rows, 512, threads)
    elif w.ratio == 2:
        kc, ks = mxfp4(w.seed, T_INDEX_KEYS, 0, rows, 128, threads, merged_logits=T_MERGE_LOGITS)
        cc, cs = mxfp4(w.seed, T_LATENT, 0, rows, 512, threads, merged_logits=T_MERGE_LOGITS)
    else:
        raise ValueError("ratio must be 1 or 2")
    return {
        "k_codes": kc.reshape(w.B, w.N, 64), "k_scales": ks.reshape(w.B, w.N, 4),
        "c_codes": cc.reshape(w.B, w.N, 256), "c_scales": cs.reshape(w.B, w.N, 16),
    }


def gen_layer(w: Workload, layer: int = 0, threads=None, need_index_query=True):
    """Per-layer inputs: index query, 64-head queries, window, n_visible, window ranges."""
    d = {}
    if need_index_query:
        qc, qs = mxfp4(w.seed, t_index_query(layer), 0, w.R, 128, threads)
        d["q_codes"], d["q_scales"] = qc, qs
    d["q"] = f32(w.seed, t_attn_query(layer), 0, w.R * w.H, 512, threads).reshape(w.R, w.H, 512)
    d["win"] = e4m3(w.seed, t_window(layer), 0, w.B * w.Tw, 512, threads).reshape(w.B, w.Tw, 512)
    d["n_visible"] = w.n_visible()
    d["win_start"] = w.win_start()
    d["win_len"] = w.win_len_arr()
    return d


# ----------------------------------------------------------------------------
# cache-write workloads
# ----------------------------------------------------------------------------
@dataclass
class CacheWriteWorkload:
    """The cache write of whole contexts: B sequences of T fp32 tokens each are
    merged at ratio m into T/m cached entries of the 512-d latent and of the
    128-d indexer keys (MXFP4), and each sequence's newest win_len tokens are
    written to its FP8 window.  Tokens are iid N(0,1) rows; the ratio-2 merge
    weights are the generator's (softmax over each pair of N(0,1) logits)."""
    name: str
    seed: int
    B: int
    T: int
    ratio: int = 2
    win_len: int = 128
    notes: str = ""

    @property
    def tokens(self) -> int:
        return self.B * self.T

    @property
    def entries(self) -> int:
        return self.tokens // self.ratio

    def latent_rows(self, row0, nrows, threads=None):
        return f32(self.seed, T_TOKEN_LATENT, row0, nrows, 512, threads)

    def index_rows(self, row0, nrows, threads=None):
        return f32(self.seed, T_TOKEN_INDEX, row0, nrows, 128, threads)

    def window_rows(self, threads=None):
        return f32(self.seed, T_TOKEN_WINDOW, 0, self.B * self.win_len, 512, threads)

    def weights(self, tok0, ntok):
        """fp32 merge weights of tokens [tok0, tok0+ntok) (whole entries)."""
        assert self.ratio == 2 and tok0 % 2 == 0 and ntok % 2 == 0
        return merge_weights_f32(self.seed, T_MERGE_LOGITS, tok0 // 2, ntok // 2)


CACHE_WRITES = {
    # the cached state of c3 (4 sequences x 1,048,576 tokens at ratio 2) written
    # from its fp32 tokens
    "w3": CacheWriteWorkload("w3_cache_write_b4_1m_ratio2", BASE_SEED + 2, B=4, T=1048576, ratio=2,
                             notes="cache write of 4 x 1,048,576 tokens at ratio 2: 2,097,152 latent (512-d) and "
                                   "indexer-key (128-d) MXFP4 entries + 4 x 128 FP8 window rows"),
}
