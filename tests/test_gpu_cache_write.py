"""GPU parity of the cache write (ratio-m merge + MXFP4 quantize-on-write, FP8
window quantize-on-write) through the C ABI against the oracle: codes and
scale bytes must be bit-exact.

Cases span several workgroups with ragged tails (a workgroup takes 256
four-element quads; tiles are handed out in groups of 512 so that each XCD
streams 64 consecutive tiles, and a last partial group keeps launch order, so
the larger cases cover full and partial groups), every ratio code path (1, 2
and 4 compiled, others
generic), both row widths the cached state uses (128 index-key elements, 512
latent elements) and edge values: E2M1 midpoints and their neighbours, zero,
subnormal, huge, infinite and NaN blocks, exponent clamps at both ends.
"""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_csa2_amd as csa2
import oracle
import synth

from gpu_cases import say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.load_library()


def _weights(seed, tokens, ratio):
    """Softmax over each group of `ratio` N(0,1) logits (the generator's recipe
    for ratio 2, extended to any ratio), rounded to fp32."""
    l = synth.normals(seed, synth.T_MERGE_LOGITS, 0, (tokens + 3) // 4, 4).reshape(-1)[:tokens]
    l = l.reshape(-1, ratio)
    e = np.exp(l - l.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).reshape(-1).astype(np.float32)


def _gpu_write(x, w, ratio, pad=64):
    """Run the kernel into a sentinel-filled buffer with `pad` spare bytes on both
    sides of each output, and check the spare bytes stay untouched."""
    T, D = x.shape
    n = T // ratio
    cb = torch.full((pad + n * (D // 2) + pad,), 0xA5, dtype=torch.uint8, device="cuda")
    sb = torch.full((pad + n * (D // 32) + pad,), 0x5A, dtype=torch.uint8, device="cuda")
    codes = cb[pad:pad + n * (D // 2)]
    scales = sb[pad:pad + n * (D // 32)]
    xt = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    wt = None if w is None else torch.from_numpy(np.ascontiguousarray(w)).cuda()
    csa2.csa2_cache_write_mxfp4(xt, wt, ratio, codes, scales)
    torch.cuda.synchronize()
    cb, sb = cb.cpu().numpy(), sb.cpu().numpy()
    assert np.all(cb[:pad] == 0xA5) and np.all(cb[pad + n * (D // 2):] == 0xA5)
    assert np.all(sb[:pad] == 0x5A) and np.all(sb[pad + n * (D // 32):] == 0x5A)
    return cb[pad:pad + n * (D // 2)].reshape(n, D // 2), sb[pad:pad + n * (D // 32)].reshape(n, D // 32)


def _check(x, w, ratio):
    codes, scales = _gpu_write(x, w, ratio)
    rc, rs = oracle.cache_write_mxfp4(x, w, ratio)
    bad = np.argwhere(np.any(codes != rc, axis=1))
    assert bad.size == 0, f"first mismatching entry {bad[0][0]}"
    assert np.array_equal(scales, rs)


@pytest.mark.parametrize("n,ratio,D", [
    (1, 1, 32), (3, 2, 128), (37, 2, 512), (1000, 1, 128), (517, 3, 64), (64, 4, 512), (5, 8, 256),
    (2049, 2, 128), (300, 1, 512), (8, 64, 32), (1100, 2, 512), (9000, 1, 128), (1025, 3, 512)])
def test_cache_write_mxfp4_random(n, ratio, D):
    say(f"cache write n={n} ratio={ratio} D={D}")
    x = synth.f32(100 + n, synth.T_TOKEN_LATENT, 0, n * ratio, D)
    w = _weights(100 + n, n * ratio, ratio) if (ratio > 1 or n % 2) else None
    _check(x, w, ratio)


def test_cache_write_empty():
    """Zero entries / zero elements: success, nothing launched or written."""
    x = torch.zeros((0, 128), dtype=torch.float32, device="cuda")
    codes = torch.zeros(0, dtype=torch.uint8, device="cuda")
    csa2.csa2_cache_write_mxfp4(x, torch.zeros(0, device="cuda"), 2, codes, codes)
    csa2.csa2_cache_write_e4m3(torch.zeros(0, device="cuda"), codes)
    torch.cuda.synchronize()


def _edge_rows(D=128):
    """Rows whose values hit the encoder's decision points exactly (ratio 1),
    built as 32-element blocks and grouped D/32 to a row."""
    rng = np.random.default_rng(17)
    blocks = []
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.5, 6.0], np.float32)
    for E in (-127, -126, -100, -3, 0, 1, 20, 100, 125):
        for b in range(4):
            blk = np.zeros(32, np.float32)
            blk[0] = np.float32(np.ldexp(6.0 if b % 2 == 0 else 4.5, E))
            vals = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(10))])
            vals = np.ldexp(vals.astype(np.float64), E).astype(np.float32)
            sign = np.where(rng.random(vals.size) < 0.5, -1, 1).astype(np.float32)
            blk[1:1 + 27] = (vals * sign)[:27]
            blk[28:] = [0.0, -0.0, np.float32(np.ldexp(0.1, E)), -np.float32(np.ldexp(0.2, E))]
            blocks.append(rng.permutation(blk))
    special = [
        [np.inf, 1.0, -np.inf, np.nan],                                              # infinite amax
        [np.nan, -2.0, 3.0, np.nan],                                                 # NaN elements
        [np.nan] * 32,                                                               # all NaN
        [np.float32(2.0 ** -128), -np.float32(2.0 ** -149), np.float32(3 * 2.0 ** -130)],  # subnormal amax
        [np.float32(2.0 ** 127), 2.0, -np.float32(2.0 ** 126)],                      # E = 125
        [-0.0] * 32,
        [],                                                                          # zero block
    ]
    for vals in special:
        blk = np.zeros(32, np.float32)
        blk[:len(vals)] = vals
        blocks.append(blk)
    big = np.full(32, np.finfo(np.float32).max, np.float32)
    big[1::2] *= -0.75
    blocks.append(big)
    for _ in range(4):
        blocks.append((rng.standard_normal(32) * 2.0 ** -135).astype(np.float32))   # subnormal blocks
    per = D // 32
    while len(blocks) % per:
        blocks.append(np.zeros(32, np.float32))
    return np.concatenate(blocks).reshape(-1, D)


@pytest.mark.parametrize("D", [32, 128, 512])
def test_cache_write_mxfp4_edge_values(D):
    x = _edge_rows(D)
    say(f"cache write edges D={D} rows={x.shape[0]}")
    _check(x, None, 1)
    # the same rows merged at ratio 2 with weights 1 and 0 (exact products),
    # then with weights 0.5 (halving: exact unless subnormal)
    pairs = np.repeat(x, 2, axis=0)
    _check(pairs, np.tile(np.array([1.0, 0.0], np.float32), x.shape[0]), 2)
    _check(pairs, np.full(2 * x.shape[0], 0.5, np.float32), 2)


def test_cache_write_mxfp4_into_cache_rows():
    """Writing entries [e0, e0+n) of one sequence's cache leaves the rest alone."""
    N, e0, n, ratio = 1000, 333, 77, 2
    x = synth.f32(5, synth.T_TOKEN_INDEX, 0, n * ratio, 128)
    w = _weights(5, n * ratio, ratio)
    kc = torch.full((N, 64), 0x33, dtype=torch.uint8, device="cuda")
    ks = torch.full((N, 4), 0x44, dtype=torch.uint8, device="cuda")
    csa2.csa2_cache_write_mxfp4(torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda(), ratio, kc[e0:e0 + n],
                                ks[e0:e0 + n])
    torch.cuda.synchronize()
    kc, ks = kc.cpu().numpy(), ks.cpu().numpy()
    rc, rs = oracle.cache_write_mxfp4(x, w, ratio)
    assert np.array_equal(kc[e0:e0 + n], rc) and np.array_equal(ks[e0:e0 + n], rs)
    assert np.all(kc[:e0] == 0x33) and np.all(kc[e0 + n:] == 0x33)
    assert np.all(ks[:e0] == 0x44) and np.all(ks[e0 + n:] == 0x44)


def _e4m3_values():
    table = np.array([oracle.e4m3_value(c) for c in range(256)])
    fin = np.sort(np.unique(table[~np.isnan(table)]))
    pos = fin[fin > 0]
    mids = (pos[:-1] + pos[1:]) / 2
    base = np.concatenate([fin, mids, [pos[0] / 2, 448.0, 464.0, 480.0, 1e30]]).astype(np.float32)
    near = np.concatenate([np.nextafter(base, np.float32(-np.inf)), np.nextafter(base, np.float32(np.inf))])
    rng = np.random.default_rng(23)
    rnd = np.concatenate([rng.standard_normal(20000) * 2.0 ** s for s in range(-14, 11, 3)]).astype(np.float32)
    special = np.array([np.inf, -np.inf, np.nan, -np.nan, 0.0, -0.0, np.finfo(np.float32).max,
                        np.float32(2.0 ** -149), np.float32(2.0 ** -126)], np.float32)
    v = np.concatenate([base, -base, near, -near, rnd, special]).astype(np.float32)
    return v[: len(v) - len(v) % 4]


def test_cache_write_e4m3_all_decision_points():
    x = _e4m3_values()
    say(f"e4m3 write n={x.size}")
    pad = 32
    ob = torch.full((pad + x.size + pad,), 0xC3, dtype=torch.uint8, device="cuda")
    csa2.csa2_cache_write_e4m3(torch.from_numpy(x).cuda(), ob[pad:pad + x.size])
    torch.cuda.synchronize()
    ob = ob.cpu().numpy()
    assert np.all(ob[:pad] == 0xC3) and np.all(ob[pad + x.size:] == 0xC3)
    got = ob[pad:pad + x.size]
    want = oracle.cache_write_e4m3(x)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} mismatches, first x={x[bad[0]]!r} got {got[bad[0]]:#x} want {want[bad[0]]:#x}"


@pytest.mark.parametrize("rows", [1, 3, 128, 1001, 1100])
def test_cache_write_e4m3_window_rows(rows):
    x = synth.f32(7 + rows, synth.T_TOKEN_WINDOW, 0, rows, 512)
    out = torch.empty((rows, 512), dtype=torch.uint8, device="cuda")
    csa2.csa2_cache_write_e4m3(torch.from_numpy(x).cuda(), out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle.cache_write_e4m3(x))


def test_cache_write_then_full_layer():
    """End to end: fp32 tokens -> the GPU cache write (ratio 2, latent, indexer
    keys, window) -> a Full layer (pool, top-512, attention) on the written
    cache, against the oracle doing the same from the same tokens."""
    import math

    from hierarchical_sparse_attention_csa2_amd import pipeline

    B, N, ratio, Tw = 2, 3000, 2, 128
    T = N * ratio
    seed = 4711
    xl = synth.f32(seed, synth.T_TOKEN_LATENT, 0, B * T, 512)
    xi = synth.f32(seed, synth.T_TOKEN_INDEX, 0, B * T, 128)
    wts = synth.merge_weights_f32(seed, synth.T_MERGE_LOGITS, 0, B * N)
    xw = synth.f32(seed, synth.T_TOKEN_WINDOW, 0, B * Tw, 512)
    say("cache write -> full layer")
    cc = torch.empty((B, N, 256), dtype=torch.uint8, device="cuda")
    cs = torch.empty((B, N, 16), dtype=torch.uint8, device="cuda")
    kc = torch.empty((B, N, 64), dtype=torch.uint8, device="cuda")
    ks = torch.empty((B, N, 4), dtype=torch.uint8, device="cuda")
    win = torch.empty((B, Tw, 512), dtype=torch.uint8, device="cuda")
    wt = torch.from_numpy(wts).cuda()
    csa2.csa2_cache_write_mxfp4(torch.from_numpy(xl).cuda(), wt, ratio, cc.view(B * N, 256), cs.view(B * N, 16))
    csa2.csa2_cache_write_mxfp4(torch.from_numpy(xi).cuda(), wt, ratio, kc.view(B * N, 64), ks.view(B * N, 4))
    csa2.csa2_cache_write_e4m3(torch.from_numpy(xw).cuda(), win.view(B * Tw, 512))
    qc, qs = synth.mxfp4(seed, synth.t_index_query(0), 0, B, 128)
    q = synth.f32(seed, synth.t_attn_query(0), 0, B * 64, 512).reshape(B, 64, 512)
    nv = np.array([N, N - 777], np.int32)
    ws0, wl = np.zeros(B, np.int32), np.full(B, Tw, np.int32)
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    st = pipeline.Step(("full",), B, 1, N)
    pool, idxs, outs = st.run(pipeline.Cache(kc, ks, cc, cs),
                              [pipeline.LayerInputs(q=dv(q), win=win, win_start=dv(ws0), win_len=dv(wl),
                                                    n_visible=dv(nv), q_codes=dv(qc), q_scales=dv(qs))])
    torch.cuda.synchronize()
    # the oracle's own cache from the same tokens
    rc_c, rc_s = oracle.cache_write_mxfp4(xl, wts, ratio)
    rk_c, rk_s = oracle.cache_write_mxfp4(xi, wts, ratio)
    r_win = oracle.cache_write_e4m3(xw).reshape(B, Tw, 512)
    ref = oracle.index_full(qc, qs, rk_c, rk_s, nv, B, 1, N, n_pool=2048, k=512)
    assert np.array_equal(pool.cpu().numpy(), ref["pool_blocks"])
    assert np.array_equal(idxs[0].cpu().numpy(), ref["idx"])
    o_ref = oracle.sparse_attn(q, rc_c.reshape(B, N, 256), rc_s.reshape(B, N, 16), ref["idx"], r_win, ws0, wl, B, 1,
                               N, np.float32(1 / math.sqrt(512)))
    err = float(np.max(np.abs(outs[0].cpu().numpy() - o_ref)))
    say(f"  attention max abs err {err:.2e}")
    assert err <= 1e-3
