"""Pins of the oracle's sparse + sliding-window attention.

The pages: every layer mode computes its own query and sliding-window KV; a
layer reads the 512 selected global KV entries plus a 128-token sliding window
(fupanwang.com DeepSeek-V4.1-Flash article, sections 后 20 层干脆共用一份 KV and
三个方向一起压小缓存; dreamax.pages.dev notes, CSA2 paragraph).  Read as one
softmax over both sets, value = key.  The pins: (b) when the selection covers
every cached entry the output is dense attention, computed here with torch's
float64 softmax; (c) with k = 0 it is pure window attention; (d) a Reuse layer
given the Full layer's indices reproduces the Full output; closed forms (one
entry, equal logits) and convexity.
"""
import numpy as np
import torch

import oracle
import synth


def _decode_latent(cc, cs):
    return oracle.mxfp4_decode(cc, cs)


def _decode_e4m3(b):
    return torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_attn(q, rows, scale):
    """q [H, D] float32, rows [E, D] float64 -> [H, D] via torch float64 softmax."""
    qt = torch.from_numpy(q.astype(np.float64))
    vt = torch.from_numpy(rows)
    z = (qt @ vt.T) * float(np.float32(scale))
    p = torch.softmax(z, dim=-1)
    return (p @ vt).numpy()


def _case(seed, B, N, H, Tw):
    cc, cs = synth.mxfp4(seed, 2, 0, B * N, 512)
    cc, cs = cc.reshape(B, N, 256), cs.reshape(B, N, 16)
    q = synth.f32(seed, 5, 0, B * H, 512).reshape(B, H, 512)
    win = synth.e4m3(seed, 6, 0, B * Tw, 512).reshape(B, Tw, 512)
    return cc, cs, q, win


def test_dense_equivalence_when_selection_covers_all():          # check (b)
    B, N, H, Tw = 2, 40, 4, 16
    cc, cs, q, win = _case(31, B, N, H, Tw)
    idx = np.tile(np.arange(N, dtype=np.int32), (B, 1))
    ws, wl = np.array([0, 3], np.int32), np.array([16, 13], np.int32)
    scale = np.float32(1 / np.sqrt(512))
    out = oracle.sparse_attn(q, cc, cs, idx, win, ws, wl, B, 1, N, scale)
    for r in range(B):
        rows = np.concatenate([_decode_latent(cc[r], cs[r]), _decode_e4m3(win[r, ws[r]: ws[r] + wl[r]])])
        ref = _torch_attn(q[r], rows, scale)
        assert np.max(np.abs(out[r] - ref)) < 1e-6


def test_window_only_when_k_is_zero():                              # check (c)
    B, N, H, Tw = 2, 20, 3, 128
    cc, cs, q, win = _case(32, B, N, H, Tw)
    ws, wl = np.zeros(B, np.int32), np.full(B, 128, np.int32)
    scale = np.float32(1 / np.sqrt(512))
    out0 = oracle.sparse_attn(q, cc, cs, np.zeros((B, 0), np.int32), win, ws, wl, B, 1, N, scale)
    outm = oracle.sparse_attn(q, cc, cs, np.full((B, 7), -1, np.int32), win, ws, wl, B, 1, N, scale)
    for r in range(B):
        ref = _torch_attn(q[r], _decode_e4m3(win[r]), scale)
        assert np.max(np.abs(out0[r] - ref)) < 1e-6
    assert np.array_equal(out0, outm)


def test_reuse_equals_full_given_same_indices():                    # check (d)
    B, N, H, Tw = 2, 300, 4, 128
    seed = 33
    cc, cs, q, win = _case(seed, B, N, H, Tw)
    kc, ks = synth.mxfp4(seed, 1, 0, B * N, 128)
    qc, qs = synth.mxfp4(seed, 4, 0, B, 128)
    nv = np.full(B, N, np.int32)
    full = oracle.index_full(qc, qs, kc.reshape(B, N, 64), ks.reshape(B, N, 4), nv, B, 1, N, n_pool=16, k=64)
    ws, wl = np.zeros(B, np.int32), np.full(B, 128, np.int32)
    scale = np.float32(1 / np.sqrt(512))
    o_full = oracle.sparse_attn(q, cc, cs, full["idx"], win, ws, wl, B, 1, N, scale)
    # a Reuse layer handed the same indices, query and window
    o_reuse = oracle.sparse_attn(q.copy(), cc, cs, full["idx"].copy(), win.copy(), ws, wl, B, 1, N, scale)
    assert np.array_equal(o_full, o_reuse)
    # and its result is dense attention over exactly the selected rows + window
    for r in range(B):
        sel = full["idx"][r][full["idx"][r] >= 0]
        rows = np.concatenate([_decode_latent(cc[r, sel], cs[r, sel]), _decode_e4m3(win[r])])
        assert np.max(np.abs(o_full[r] - _torch_attn(q[r], rows, scale))) < 1e-6


def test_closed_forms():
    B, N, H, Tw = 1, 10, 2, 4
    cc, cs, q, win = _case(34, B, N, H, Tw)
    scale = np.float32(0.1)
    # a single entry: the output is that entry's value
    out = oracle.sparse_attn(q, cc, cs, np.array([[6]], np.int32), win, np.zeros(1, np.int32),
                             np.zeros(1, np.int32), B, 1, N, scale)
    val = _decode_latent(cc[0, 6], cs[0, 6]).astype(np.float32)
    assert np.array_equal(out[0, 0], val) and np.array_equal(out[0, 1], val)
    # equal logits (q = 0): the mean of the values
    qz = np.zeros_like(q)
    idx = np.array([[1, 2, 5]], np.int32)
    out = oracle.sparse_attn(qz, cc, cs, idx, win, np.zeros(1, np.int32), np.full(1, 4, np.int32), B, 1, N, scale)
    rows = np.concatenate([_decode_latent(cc[0, [1, 2, 5]], cs[0, [1, 2, 5]]), _decode_e4m3(win[0])])
    assert np.max(np.abs(out[0, 0] - rows.mean(axis=0))) < 1e-6
    # the empty set gives zeros
    out = oracle.sparse_attn(q, cc, cs, np.full((1, 3), -1, np.int32), win, np.zeros(1, np.int32),
                             np.zeros(1, np.int32), B, 1, N, scale)
    assert (out == 0).all()


def test_convexity_and_duplicates():
    B, N, H, Tw = 1, 50, 8, 128
    cc, cs, q, win = _case(35, B, N, H, Tw)
    idx = np.array([[0, 3, 3, 9, 49]], np.int32)        # a repeated row counts twice
    scale = np.float32(1 / np.sqrt(512))
    out = oracle.sparse_attn(q, cc, cs, idx, win, np.zeros(1, np.int32), np.full(1, 128, np.int32), B, 1, N, scale)
    rows = np.concatenate([_decode_latent(cc[0, idx[0]], cs[0, idx[0]]), _decode_e4m3(win[0])])
    lo, hi = rows.min(axis=0), rows.max(axis=0)
    assert (out[0] >= lo - 1e-6).all() and (out[0] <= hi + 1e-6).all()
    assert np.max(np.abs(out[0] - _torch_attn(q[0], rows, scale))) < 1e-6


def _ref_row(q, cc, cs, idx_row, win, ws, wl, win_max, N, Tw, scale):
    """Brute-force attention of one row: the entries it names, written out by
    hand (indices in [0, N), window rows ws + t in [0, Tw) for
    t < min(max(wl, 0), win_max)), torch float64 softmax; zeros if empty."""
    sel = [int(p) for p in idx_row if 0 <= p < N]
    n = min(max(int(wl), 0), win_max)
    wrows = [int(ws) + t for t in range(n) if 0 <= int(ws) + t < Tw]
    parts = []
    if sel:
        parts.append(_decode_latent(cc[sel], cs[sel]))
    if wrows:
        parts.append(_decode_e4m3(win[wrows]))
    if not parts:
        return np.zeros_like(q, dtype=np.float64)
    return _torch_attn(q, np.concatenate(parts), scale)


def test_many_queries_per_sequence():
    """M > 1 query rows per sequence: row r reads its sequence's (r // M) latent
    and window store, with its own indices, window start and length."""
    B, M, N, H, Tw = 2, 3, 60, 4, 20
    cc, cs, _, win = _case(36, B, N, H, Tw)
    q = synth.f32(36, 5, 0, B * M * H, 512).reshape(B * M, H, 512)
    rng = np.random.default_rng(36)
    idx = rng.integers(0, N, size=(B * M, 9)).astype(np.int32)
    idx[2, 4:] = -1
    ws = np.array([0, 3, 7, 0, 11, 19], np.int32)
    wl = np.array([5, 8, 13, 0, 9, 1], np.int32)
    scale = np.float32(1 / np.sqrt(512))
    out = oracle.sparse_attn(q, cc, cs, idx, win, ws, wl, B, M, N, scale, win_max=Tw)
    for r in range(B * M):
        seq = r // M
        ref = _ref_row(q[r], cc[seq], cs[seq], idx[r], win[seq], ws[r], wl[r], Tw, N, Tw, scale)
        assert np.max(np.abs(out[r] - ref)) < 1e-6, r


def test_out_of_range_entries_and_window_rows_are_left_out():
    """The interface's rules for names that point nowhere: indices outside
    [0, N_max) and window rows outside [0, Tw) are not part of the set, and a
    row's window has min(win_len, win_max) rows (none for a negative length)."""
    B, N, H, Tw = 1, 30, 3, 16
    cc, cs, _, win = _case(37, B, N, H, Tw)
    rows = 7
    q = synth.f32(37, 5, 0, rows * H, 512).reshape(rows, H, 512)
    cc7, cs7 = np.repeat(cc, rows, 0), np.repeat(cs, rows, 0)
    win7 = np.repeat(win, rows, 0)
    idx = np.array([[0, 29, 30, 31, -1],          # 30 and 31 past the cache
                    [5, 1 << 30, -7, 2, 2],        # huge and negative indices
                    [-1, -1, -1, -1, -1],
                    [3, 4, 5, 6, 7],
                    [30, 30, 30, 30, 30],          # nothing valid
                    [1, 2, 3, 4, 5],
                    [29, 0, 15, 40, 16]], np.int32)
    ws = np.array([12, -3, 14, 0, -10, 0, 15], np.int32)
    wl = np.array([8, 6, 2, 40, 5, -4, 1], np.int32)   # past Tw, before 0, > win_max, empty
    win_max = 12
    scale = np.float32(1 / np.sqrt(512))
    out = oracle.sparse_attn(q, cc7, cs7, idx, win7, ws, wl, rows, 1, N, scale, win_max=win_max)
    for r in range(rows):
        ref = _ref_row(q[r], cc[0], cs[0], idx[r], win[0], ws[r], wl[r], win_max, N, Tw, scale)
        assert np.max(np.abs(out[r] - ref)) < 1e-6, r
    # row 4 names no entry at all: zeros
    assert (out[4] == 0).all()
    # row 3's window is clamped to 12 rows: the same as asking for exactly 12
    wl12 = wl.copy()
    wl12[3] = 12
    out12 = oracle.sparse_attn(q, cc7, cs7, idx, win7, ws, wl12, rows, 1, N, scale, win_max=win_max)
    assert np.array_equal(out[3], out12[3])
