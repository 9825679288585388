"""Layer composition of the CSA2 step over the C ABI, with preallocated buffers.

Modes (dreamax.pages.dev notes, CSA2 paragraph; fupanwang.com DeepSeek-V4.1-Flash
article, section 三个方向一起压小缓存 and its figure caption):
  Full    - own index query over the whole visible cache: 8-position block
            maxima, a pool of the best 2048 blocks (shared with later layers),
            its own top-512, then attention.
  Reindex - the Full layer's index keys and pool, its own index query: scores
            only the pool's positions, own top-512, then attention.
  Reuse   - the latest selection as is, own query and window, attention.
Every layer has its own 64-head query and sliding window and reads the Full
layer's latent KV.  Buffers are allocated once, so a step allocates nothing.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

from . import (CSA2_OP_INDEX_FULL, CSA2_OP_SPARSE_ATTN, csa2_index_full, csa2_index_pool, csa2_index_pool_topk,
               csa2_index_scan, csa2_select_blocks, csa2_sparse_attn, csa2_topk, csa2_workspace_bytes, recording)

FUSED_POOL_BLOCKS = 2048   # pools csa2_index_pool_topk takes (one workgroup scores and ranks a row)
# Rows from which the one-call Reindex beats index_pool + topk (a 2048-block pool
# over 266,240 entries: 64 rows 50.3 vs 29.6 us, 256 rows 63.7 vs 62.8 us, 1,024
# rows 211.4 vs 225.2 us, 4,096 rows 812.1 vs 857.7 us): with fewer rows its
# workgroups leave compute units idle.
FUSED_MIN_ROWS = 1024


@dataclass
class Cache:
    """The Full layer's cached state for B sequences (device tensors)."""
    k_codes: torch.Tensor     # u8 [B, N, 64]
    k_scales: torch.Tensor    # u8 [B, N, 4]
    c_codes: torch.Tensor     # u8 [B, N, 256]
    c_scales: torch.Tensor    # u8 [B, N, 16]

    @property
    def B(self):
        return self.k_codes.shape[0]

    @property
    def N(self):
        return self.k_codes.shape[1]


@dataclass
class LayerInputs:
    """Per-layer inputs (device tensors)."""
    q: torch.Tensor                    # f32 [R, H, 512]
    win: torch.Tensor                  # u8 [B, Tw, 512]
    win_start: torch.Tensor            # i32 [R]
    win_len: torch.Tensor              # i32 [R]
    n_visible: torch.Tensor            # i32 [R]
    q_codes: torch.Tensor = None       # u8 [R, 64]   (Full, Reindex)
    q_scales: torch.Tensor = None      # u8 [R, 4]


class Step:
    """A chain of layers ("full", "reindex", "reuse") over one cache."""

    def __init__(self, modes, B, M, N, H=64, n_pool=2048, k=512, win_max=128, device="cuda",
                 staged=False, keep_scores=False):
        if modes[0] != "full":
            raise ValueError("the chain starts with a Full layer")
        self.modes = tuple(modes)
        self.B, self.M, self.N, self.H = B, M, N, H
        self.R = B * M
        self.n_pool, self.k, self.win_max = n_pool, k, win_max
        self.staged = staged
        self.sm_scale = 1.0 / math.sqrt(512.0)
        dev = torch.device(device)
        R, nblk = self.R, (N + 7) // 8
        self.block_max = torch.empty((R, nblk), dtype=torch.float32, device=dev)
        self.super_max = torch.empty((R, (N + 63) // 64), dtype=torch.float32, device=dev)
        self.scores = torch.empty((R, N), dtype=torch.float32, device=dev) if keep_scores else None
        self.pool = torch.empty((R, n_pool), dtype=torch.int32, device=dev)
        self.kb = min(k, n_pool)     # the pool's top-k lies in its first min(k, n_pool) blocks
        self.topk_blocks = torch.empty((R, self.kb), dtype=torch.int32, device=dev)
        self.topk_scores = torch.empty((R, 8 * self.kb), dtype=torch.float32, device=dev)
        self.pool_scores = torch.empty((R, 8 * n_pool), dtype=torch.float32, device=dev)
        self.idx = [torch.empty((R, k), dtype=torch.int32, device=dev) for _ in self.modes]
        self.out = [torch.empty((R, H, 512), dtype=torch.float32, device=dev) for _ in self.modes]
        self.ws_full = torch.empty(max(1, csa2_workspace_bytes(CSA2_OP_INDEX_FULL, B, M, N, 0, k)),
                                   dtype=torch.uint8, device=dev)
        self.ws_attn = torch.empty(max(1, csa2_workspace_bytes(CSA2_OP_SPARSE_ATTN, B, M, 0, H, k + win_max)),
                                   dtype=torch.uint8, device=dev)

    # the Full layer's indexer, either as the composite call or stage by stage
    def full_index(self, cache: Cache, li: LayerInputs, idx: torch.Tensor):
        B, M, N = self.B, self.M, self.N
        if not self.staged:
            # the block maxima are exported only by a step that keeps its
            # intermediates (keep_scores); otherwise they stay in the workspace,
            # in whichever layout the library's block filter reads fastest
            csa2_index_full(li.q_codes, li.q_scales, cache.k_codes, cache.k_scales, li.n_visible, B, M, N,
                            self.n_pool, self.k, self.pool, idx, self.ws_full, scores=self.scores,
                            block_max=self.block_max if self.scores is not None else None)
            return
        csa2_index_scan(li.q_codes, li.q_scales, cache.k_codes, cache.k_scales, li.n_visible, B, M, N,
                        self.block_max, scores=self.scores, super_max=self.super_max)
        csa2_select_blocks(self.block_max, li.n_visible, self.n_pool, self.pool, self.kb, self.topk_blocks,
                           super_max=self.super_max)
        csa2_index_pool(li.q_codes, li.q_scales, cache.k_codes, cache.k_scales, self.topk_blocks, li.n_visible,
                        B, M, N, self.topk_scores)
        csa2_topk(self.topk_scores, li.n_visible, self.k, idx, pool_blocks=self.topk_blocks)

    def scan_only(self, cache: Cache, li: LayerInputs):
        """The Full layer's scan alone, as csa2_index_full runs it: with fewer than
        16 queries per sequence it also stores every score."""
        scores = self.scores
        if scores is None and self.M < 16:
            if getattr(self, "_scan_scores", None) is None:
                self._scan_scores = torch.empty((self.R, self.N), dtype=torch.float32, device=self.block_max.device)
            scores = self._scan_scores
        csa2_index_scan(li.q_codes, li.q_scales, cache.k_codes, cache.k_scales, li.n_visible, self.B, self.M,
                        self.N, self.block_max, scores=scores, super_max=self.super_max)

    def attend_only(self, cache: Cache, li: LayerInputs):
        """The first layer's attention alone, over its last selection."""
        self.attend(cache, li, self.idx[0], self.out[0])

    def reindex(self, cache: Cache, li: LayerInputs, idx: torch.Tensor):
        if self.k > 0 and self.pool.shape[1] <= FUSED_POOL_BLOCKS and self.B * self.M >= FUSED_MIN_ROWS:
            # scoring and top-k in one workgroup per row
            csa2_index_pool_topk(li.q_codes, li.q_scales, cache.k_codes, cache.k_scales, self.pool, li.n_visible,
                                 self.B, self.M, self.N, self.k, idx)
            return
        csa2_index_pool(li.q_codes, li.q_scales, cache.k_codes, cache.k_scales, self.pool, li.n_visible,
                        self.B, self.M, self.N, self.pool_scores)
        csa2_topk(self.pool_scores, li.n_visible, self.k, idx, pool_blocks=self.pool)

    def attend(self, cache: Cache, li: LayerInputs, idx: torch.Tensor, out: torch.Tensor):
        csa2_sparse_attn(li.q, cache.c_codes, cache.c_scales, idx, li.win, li.win_start, li.win_len, self.win_max,
                         self.B, self.M, self.N, self.sm_scale, out, self.ws_attn)

    def bind(self, cache: Cache, layers):
        """The launches run(cache, layers) makes, checked and marshalled once:
        returns a function that issues them again on the stream current now,
        with no per-call argument checks.  It holds raw device pointers, so the
        cache, the layer inputs and this Step must stay alive and in place."""
        with recording() as rec:
            self.run(cache, layers)
        return rec.launches()

    def run(self, cache: Cache, layers):
        """layers: one LayerInputs per mode.  Returns (pool, [idx per layer], [out per layer])."""
        prev_idx = None
        for li_no, (mode, li) in enumerate(zip(self.modes, layers)):
            idx = self.idx[li_no]
            if mode == "full":
                self.full_index(cache, li, idx)
                cur = idx
            elif mode == "reindex":
                self.reindex(cache, li, idx)
                cur = idx
            elif mode == "reuse":
                cur = prev_idx
            else:
                raise ValueError(mode)
            self.attend(cache, li, cur, self.out[li_no])
            prev_idx = cur
        return self.pool, [self.idx[i] if m != "reuse" else None for i, m in enumerate(self.modes)], self.out


def to_device(arrays: dict, device="cuda"):
    """numpy arrays -> contiguous device tensors (plumbing only)."""
    return {k: torch.from_numpy(v).to(device) for k, v in arrays.items()}


def cache_from(d) -> Cache:
    return Cache(d["k_codes"], d["k_scales"], d["c_codes"], d["c_scales"])


def layer_from(d) -> LayerInputs:
    return LayerInputs(q=d["q"], win=d["win"], win_start=d["win_start"], win_len=d["win_len"],
                       n_visible=d["n_visible"], q_codes=d.get("q_codes"), q_scales=d.get("q_scales"))
