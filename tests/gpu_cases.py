"""Shared case builders for the GPU parity tests: seeded inputs (synth), the same
bytes on the device, and oracle results for chosen rows."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import synth
from synth import Workload

SM_SCALE = np.float32(1.0 / math.sqrt(512.0))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host_inputs(w: Workload, layers=1, kind="normal", seed_offset=0):
    """numpy inputs for a workload: cache + per-layer dicts.

    kind: "normal"  - the workload's own distribution
          "ties"    - a 4-code key alphabet and 2-code queries (scores tie a lot)
          "spread"  - N(0,1) codes with scale bytes spread over [60, 200]
                      (block exponents far apart: fp32 rounding in the score)
          "mixed"   - the workload's own distribution, with 2% of the cached
                      positions given four scale bytes 126 + U[-7, 7] (block
                      exponents spanning 0..14) and 0.3% given one scale byte
                      in {1..4, 250..253} (block exponents outside the range
                      where a matrix-core block sum is exact), so the
                      matrix-core and vector paths meet in one row
          "overflow" - query scale bytes 243 + U[0, 4], so that eq + ek lands
                      on both sides of 368 (the top of the matrix cores' exact
                      range) up to 376; half of the query rows hold +6 in every
                      element of blocks 0 and 1, and 20% of the cached
                      positions hold +-6 in every element of each block (sign
                      per block) with scale bytes 126 + U[-2, 3]: block sums of
                      up to 4608 quarter-units that overflow to +-inf, and NaN
                      scores where two blocks overflow with opposite signs
    """
    cache = synth.gen_cache(w)
    lays = [synth.gen_layer(w, layer=L) for L in range(layers)]
    rng = np.random.default_rng(w.seed + 7919 * (seed_offset + 1))
    if kind == "ties":
        cache["k_codes"] = rng.choice(np.array([0x00, 0x11, 0x22, 0x21], np.uint8), size=cache["k_codes"].shape)
        cache["k_scales"][:] = 127
        for d in lays:
            d["q_codes"] = rng.choice(np.array([0x11, 0x22], np.uint8), size=d["q_codes"].shape)
            d["q_scales"][:] = 127
    elif kind == "spread":
        cache["k_scales"] = rng.integers(60, 201, size=cache["k_scales"].shape).astype(np.uint8)
        for d in lays:
            d["q_scales"] = rng.integers(60, 201, size=d["q_scales"].shape).astype(np.uint8)
    elif kind == "mixed":
        ks = cache["k_scales"]
        hit = rng.random(ks.shape[:-1]) < 0.02
        ks[hit] = (126 + rng.integers(-7, 8, size=(int(hit.sum()), ks.shape[-1]))).astype(np.uint8)
        ext = np.argwhere(rng.random(ks.shape[:-1]) < 0.003)
        extreme = np.array([1, 2, 3, 4, 250, 251, 252, 253], np.uint8)
        for pos in ext:
            ks[tuple(pos) + (int(rng.integers(0, ks.shape[-1])),)] = extreme[int(rng.integers(0, len(extreme)))]
    elif kind == "overflow":
        kc, ks = cache["k_codes"], cache["k_scales"]
        lead = kc.shape[:-1]
        hit = rng.random(lead) < 0.2
        signs = rng.integers(0, 2, size=lead + (4,)).astype(np.uint8)    # per block: +6 or -6
        big = np.repeat(np.where(signs == 1, 0xFF, 0x77).astype(np.uint8), 16, axis=-1)
        kc[hit] = big[hit]
        ks[hit] = (126 + rng.integers(-2, 4, size=(int(hit.sum()), 4))).astype(np.uint8)
        for d in lays:
            R = d["q_scales"].shape[0]
            d["q_scales"] = (243 + rng.integers(0, 5, size=(R, 4))).astype(np.uint8)
            d["q_codes"][::2, :32] = 0x77
    elif kind != "normal":
        raise ValueError(kind)
    return cache, lays


def dev(arrays: dict):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in arrays.items()}


def _by_sequence(w: Workload, rows):
    rows = np.arange(w.R) if rows is None else np.asarray(rows)
    groups = {}
    for j, r in enumerate(rows):
        groups.setdefault(int(r) // w.M, []).append((j, int(r)))
    return rows, groups


def oracle_full(w: Workload, cache, lay, rows=None, want_scores=False, want_block_max=False):
    """Oracle Full-layer indexer for the given query rows (all rows by default),
    one oracle call per sequence, threaded over that sequence's rows."""
    rows, groups = _by_sequence(w, rows)
    out = {}
    for seq, members in groups.items():
        js = [j for j, _ in members]
        rs = [r for _, r in members]
        res = oracle.index_full(lay["q_codes"][rs], lay["q_scales"][rs], cache["k_codes"][seq],
                                cache["k_scales"][seq], lay["n_visible"][rs], 1, len(rs), w.N, n_pool=w.n_pool,
                                k=w.k, want_scores=want_scores, want_block_max=want_block_max)
        for key, val in res.items():
            if key not in out:
                out[key] = np.empty((len(rows),) + val.shape[1:], val.dtype)
            out[key][js] = val
    return out


def oracle_attn(w: Workload, cache, lay, idx_rows, rows=None):
    """Oracle attention for the given rows; idx_rows[j] is the selection of rows[j]."""
    rows, groups = _by_sequence(w, rows)
    out = np.empty((len(rows), w.H, 512), np.float32)
    for seq, members in groups.items():
        js = [j for j, _ in members]
        rs = [r for _, r in members]
        o = oracle.sparse_attn(lay["q"][rs], cache["c_codes"][seq:seq + 1], cache["c_scales"][seq:seq + 1],
                               np.asarray(idx_rows)[js], lay["win"][seq:seq + 1], lay["win_start"][rs],
                               lay["win_len"][rs], 1, len(rs), w.N, SM_SCALE, win_max=w.win_len)
        out[js] = o
    return out


def f32_bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)
