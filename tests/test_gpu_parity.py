"""GPU parity: the HIP path through the C ABI against the oracle, on the same
seeded bytes.  Scores, block maxima, pools and selected indices must be
bit-exact; attention outputs must be within 1e-3 (max abs) of the fp64 oracle.

Small cases span several workgroups and ragged tails (visible counts that are
not multiples of 8 or of the scan chunk, partial pools, k > pool size), tie-
heavy data and adversarial scale exponents.  The workload-size cases live in
test_gpu_workloads.py.
"""
import math

import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_csa2_amd as csa2
import oracle
from hierarchical_sparse_attention_csa2_amd import pipeline
from synth import Workload

from gpu_cases import SM_SCALE, dev, f32_bits, host_inputs, oracle_attn, oracle_full, say

pytestmark = pytest.mark.gpu

ATOL = 1e-3


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.load_library()


def _run_scan(w, c, l, want_super=False):
    nblk = (w.N + 7) // 8
    scores = torch.full((w.R, w.N), float("nan"), device="cuda")
    bmax = torch.full((w.R, nblk), float("nan"), device="cuda")
    smax = torch.full((w.R, (w.N + 63) // 64), float("nan"), device="cuda") if want_super else None
    csa2.csa2_index_scan(l["q_codes"], l["q_scales"], c["k_codes"], c["k_scales"], l["n_visible"], w.B, w.M, w.N,
                         bmax, scores=scores, super_max=smax)
    torch.cuda.synchronize()
    if want_super:
        return scores.cpu().numpy(), bmax.cpu().numpy(), smax.cpu().numpy()
    return scores.cpu().numpy(), bmax.cpu().numpy()


@pytest.mark.parametrize("kind", ["normal", "ties", "spread", "mixed", "overflow"])
@pytest.mark.parametrize("N,nv", [(3000, [3000, 2995, 1]), (4099, [4099, 2048, 2049]), (40, [0, 40, 17])])
def test_index_scan_bitexact(kind, N, nv):
    w = Workload("scan", 1234 + N, B=3, N=N)
    cache, (lay,) = host_inputs(w, kind=kind)
    lay["n_visible"] = np.array(nv, np.int32)
    say(f"scan N={N} nv={nv} kind={kind}")
    scores, bmax, smax = _run_scan(w, dev(cache), dev(lay), want_super=True)
    ref = oracle_full(w, cache, lay, want_scores=True, want_block_max=True)
    for r in range(w.R):
        n = nv[r]
        assert np.array_equal(f32_bits(scores[r, :n]), f32_bits(ref["scores"][r, :n])), r
        nb = (n + 7) // 8
        assert np.array_equal(f32_bits(bmax[r, :nb]), f32_bits(ref["block_max"][r, :nb])), r
        # super-block maxima: the max of each run of 8 oracle block maxima
        ns = (n + 63) // 64
        want = [np.max(ref["block_max"][r, 8 * s:min(8 * s + 8, nb)]) for s in range(ns)]
        assert np.array_equal(f32_bits(smax[r, :ns]), f32_bits(np.array(want, np.float32))), r


def _same_f32(a, b):
    """Bitwise equality (a NaN score is one fixed bit pattern on both sides)."""
    return bool(np.array_equal(f32_bits(a), f32_bits(b)))


@pytest.mark.parametrize("kind", ["normal", "ties", "spread", "mixed", "overflow"])
@pytest.mark.parametrize("B,M,N", [(1, 40, 3000), (2, 33, 2100), (1, 130, 5000), (3, 5, 2500), (2, 15, 700),
                                   (2, 16, 1900), (1, 2, 1800), (2, 8, 1300)])
def test_prefill_scan_bitexact(kind, B, M, N):
    """Several queries per sequence: scores, block maxima and super-block maxima
    bit-exact for ragged visibility, partial query groups, several key chunks,
    and tiles whose scales need the VALU path (spread, mixed).  M < 16 runs the
    decode scan over a (chunk, query, sequence) grid, M >= 16 the many-query
    matrix-core scan; M = 15 and 16 sit on either side of that switch."""
    w = Workload("pf", 777 + N + M, B=B, N=N, M=M)
    cache, (lay,) = host_inputs(w, kind=kind)
    rng = np.random.default_rng(N + 3 * M)
    nv = rng.integers(1, N + 1, size=w.R).astype(np.int32)
    nv[0], nv[-1], nv[w.R // 2] = N, 1, 0
    lay["n_visible"] = nv
    say(f"prefill scan B={B} M={M} N={N} kind={kind}")
    scores, bmax, smax = _run_scan(w, dev(cache), dev(lay), want_super=True)
    ref = oracle_full(w, cache, lay, want_scores=True, want_block_max=True)
    for r in range(w.R):
        n = nv[r]
        assert _same_f32(scores[r, :n], ref["scores"][r, :n]), r
        nb = (n + 7) // 8
        assert _same_f32(bmax[r, :nb], ref["block_max"][r, :nb]), r
        ns = (n + 63) // 64
        want = [np.max(ref["block_max"][r, 8 * s:min(8 * s + 8, nb)]) for s in range(ns)]
        assert _same_f32(smax[r, :ns], np.array(want, np.float32)), r


@pytest.mark.parametrize("kind", ["normal", "spread", "mixed", "overflow"])
@pytest.mark.parametrize("B,M,N", [(1, 64, 4100), (2, 130, 3000), (1, 32, 1024), (2, 96, 2600), (2, 130, 8192),
                                   (2, 64, 5000), (1, 64, 8190), (2, 33, 4096)])
def test_prefill_scan_bitexact_causal(kind, B, M, N):
    """A causal prefill chunk (query i of M sees the first N - M + i + 1
    entries): whole 256-key rounds seen by every query of a wave (the
    many-query scan's common case, stored 16 bytes a lane when the block rows
    are 16-byte aligned: N = 1024, 4096, 8190, 8192), next to ragged last
    rounds, partial query groups and tiles on the VALU path inside otherwise
    whole rounds.  N = 8190 ends in a tile two keys short of 32 behind 16-byte
    rows; M = 33 leaves a last query group of one row."""
    w = Workload("pfc", 4242 + N + M, B=B, N=N, M=M, prefill_base=N - M)
    cache, (lay,) = host_inputs(w, kind=kind)
    nv = lay["n_visible"]
    say(f"prefill scan causal B={B} M={M} N={N} kind={kind}")
    c, l = dev(cache), dev(lay)
    scores, bmax, smax = _run_scan(w, c, l, want_super=True)
    # the maxima alone (no scores stored), as a Full-layer prefill asks for them
    bmax2 = torch.full((w.R, (N + 7) // 8), float("nan"), device="cuda")
    smax2 = torch.full((w.R, (N + 63) // 64), float("nan"), device="cuda")
    csa2.csa2_index_scan(l["q_codes"], l["q_scales"], c["k_codes"], c["k_scales"], l["n_visible"], w.B, w.M, w.N,
                         bmax2, super_max=smax2)
    torch.cuda.synchronize()
    bmax2, smax2 = bmax2.cpu().numpy(), smax2.cpu().numpy()
    ref = oracle_full(w, cache, lay, want_scores=True, want_block_max=True)
    for r in range(w.R):
        n = nv[r]
        assert n == N - M + r % M + 1
        assert _same_f32(scores[r, :n], ref["scores"][r, :n]), r
        nb = (n + 7) // 8
        assert _same_f32(bmax[r, :nb], ref["block_max"][r, :nb]), r
        ns = (n + 63) // 64
        want = [np.max(ref["block_max"][r, 8 * s:min(8 * s + 8, nb)]) for s in range(ns)]
        assert _same_f32(smax[r, :ns], np.array(want, np.float32)), r
        assert _same_f32(bmax2[r, :nb], ref["block_max"][r, :nb]), r
        assert _same_f32(smax2[r, :ns], np.array(want, np.float32)), r


@pytest.mark.parametrize("kind", ["normal", "ties", "spread", "mixed", "overflow"])
@pytest.mark.parametrize("N,n_pool,k,nv", [
    (4096, 2048, 512, [4096, 4000, 3333]),      # pool covers all blocks
    (20000, 2048, 512, [20000, 19999, 8191]),   # pool smaller than the block count
    (2000, 16, 512, [2000, 1999, 5]),           # pool smaller than k
    (300, 8, 64, [300, 64, 9]),
    (150000, 2048, 512, [150000, 131071, 65537]),
    (40000, 2048, 1000, [40000, 0, 17]),       # first 1000 blocks (wide top-k tile), an empty row
    (196608, 2048, 512, [196608, 196600, 100]),  # two-level filter with 16-byte loads
])
def test_index_full_bitexact(kind, N, n_pool, k, nv):
    w = Workload("full", 99 + N + n_pool, B=3, N=N, n_pool=n_pool, k=k)
    cache, (lay,) = host_inputs(w, kind=kind)
    lay["n_visible"] = np.array(nv, np.int32)
    c, l = dev(cache), dev(lay)
    say(f"index_full N={N} pool={n_pool} k={k} kind={kind}")
    ref = oracle_full(w, cache, lay)
    # composite call
    pool = torch.empty((w.R, n_pool), dtype=torch.int32, device="cuda")
    idx = torch.empty((w.R, k), dtype=torch.int32, device="cuda")
    csa2.csa2_index_full(l["q_codes"], l["q_scales"], c["k_codes"], c["k_scales"], l["n_visible"], w.B, 1, N,
                         n_pool, k, pool, idx)
    torch.cuda.synchronize()
    assert np.array_equal(pool.cpu().numpy(), ref["pool_blocks"])
    assert np.array_equal(idx.cpu().numpy(), ref["idx"])
    # with the scores asked for (written to the caller's rows instead of the
    # workspace): the same pool and top-k
    scores = torch.empty((w.R, N), dtype=torch.float32, device="cuda")
    pool3, idx3 = torch.empty_like(pool), torch.empty_like(idx)
    csa2.csa2_index_full(l["q_codes"], l["q_scales"], c["k_codes"], c["k_scales"], l["n_visible"], w.B, 1, N,
                         n_pool, k, pool3, idx3, scores=scores)
    torch.cuda.synchronize()
    assert torch.equal(pool3, pool) and torch.equal(idx3, idx)
    # staged calls (scan, block select, pool scan, top-k as separate entry points)
    st = pipeline.Step(("full",), w.B, 1, N, H=64, n_pool=n_pool, k=k, staged=True)
    st.full_index(pipeline.cache_from(c), pipeline.layer_from(l), st.idx[0])
    torch.cuda.synchronize()
    assert np.array_equal(st.pool.cpu().numpy(), ref["pool_blocks"])
    assert np.array_equal(st.idx[0].cpu().numpy(), ref["idx"])
    # the block filter without the scan's super-block maxima gives the same pool
    pool2 = torch.empty_like(pool)
    csa2.csa2_select_blocks(st.block_max, l["n_visible"], n_pool, pool2)
    torch.cuda.synchronize()
    assert np.array_equal(pool2.cpu().numpy(), ref["pool_blocks"])


@pytest.mark.parametrize("kind", ["normal", "ties", "mixed", "overflow"])
@pytest.mark.parametrize("N,M,k,nv", [
    (1, 1, 512, [1, 0, 1]),
    (64, 1, 512, [64, 63, 1]),
    (4096, 1, 512, [4096, 4095, 2049]),
    (4097, 1, 512, [4097, 4096, 100]),        # 8 key groups per wave
    (8192, 1, 1000, [8192, 0, 8191]),         # an empty row, k above half the blocks
    (16384, 1, 512, [16384, 16383, 9000]),    # 16 key groups per wave; blocks = pool size
    (9000, 5, 512, None),                     # 5 causal queries per sequence
])
def test_index_full_short_context(kind, N, M, k, nv):
    """Decode over contexts whose blocks all fit in the 2048-block pool (the
    pool is every visible block): the pool, the top-k and the optional score and
    block-max outputs of csa2_index_full are bit-exact."""
    w = Workload("small", 7 + N + M, B=3, N=N, M=M, k=k, prefill_base=(N - M) if M > 1 else -1)
    cache, (lay,) = host_inputs(w, kind=kind)
    if nv is not None:
        lay["n_visible"] = np.array(nv, np.int32)
    c, l = dev(cache), dev(lay)
    say(f"index_full short context N={N} M={M} k={k} kind={kind}")
    ref = oracle_full(w, cache, lay, want_scores=True, want_block_max=True)
    nblk = (N + 7) // 8
    pool = torch.empty((w.R, 2048), dtype=torch.int32, device="cuda")
    idx = torch.empty((w.R, k), dtype=torch.int32, device="cuda")
    scores = torch.full((w.R, N), float("nan"), device="cuda")
    bmax = torch.full((w.R, nblk), float("nan"), device="cuda")
    csa2.csa2_index_full(l["q_codes"], l["q_scales"], c["k_codes"], c["k_scales"], l["n_visible"], w.B, w.M, N,
                         2048, k, pool, idx, scores=scores, block_max=bmax)
    torch.cuda.synchronize()
    assert np.array_equal(pool.cpu().numpy(), ref["pool_blocks"])
    assert np.array_equal(idx.cpu().numpy(), ref["idx"])
    sc, bm = scores.cpu().numpy(), bmax.cpu().numpy()
    for r in range(w.R):
        n = int(lay["n_visible"][r])
        assert np.array_equal(f32_bits(sc[r, :n]), f32_bits(ref["scores"][r, :n])), r
        assert np.all(np.isnan(sc[r, n:])), r   # invisible entries are not written
        nb = (n + 7) // 8
        assert np.array_equal(f32_bits(bm[r, :nb]), f32_bits(ref["block_max"][r, :nb])), r


def test_index_full_short_rows_reuse_one_workspace():
    """One workspace serves short-row decode calls of different shapes in a row
    (what a call leaves in it never leaks into the next), each bit-exact."""
    shapes = [(3, 4096, [4096, 4000, 1]), (7, 16384, [16384, 9001, 0, 5, 16383, 8192, 1024]),
              (2, 100, [100, 37]), (5, 8193, [8193, 8192, 1, 4096, 777])]
    need = max(csa2.csa2_workspace_bytes(csa2.CSA2_OP_INDEX_FULL, B, 1, N, 0, 512) for B, N, _ in shapes)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    for i, (B, N, nv) in enumerate(shapes):
        w = Workload("small", 500 + i, B=B, N=N, k=512)
        cache, (lay,) = host_inputs(w, kind="ties" if i % 2 else "normal")
        lay["n_visible"] = np.array(nv, np.int32)
        c, l = dev(cache), dev(lay)
        say(f"index_full short rows, shared workspace B={B} N={N}")
        ref = oracle_full(w, cache, lay)
        pool = torch.empty((B, 2048), dtype=torch.int32, device="cuda")
        idx = torch.empty((B, 512), dtype=torch.int32, device="cuda")
        csa2.csa2_index_full(l["q_codes"], l["q_scales"], c["k_codes"], c["k_scales"], l["n_visible"], B, 1, N,
                             2048, 512, pool, idx, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(pool.cpu().numpy(), ref["pool_blocks"])
        assert np.array_equal(idx.cpu().numpy(), ref["idx"])


@pytest.mark.parametrize("kind", ["normal", "ties", "mixed", "overflow", "spread"])
@pytest.mark.parametrize("N,M,n_pool,k,nv", [
    (9000, 40, 2048, 512, "causal"),     # every block in the pool
    (40000, 130, 2048, 512, "causal"),   # pool below the block count; two query groups and a tail
    (20000, 16, 64, 512, "random"),      # pool below k (kb = 64); rows of 0 .. N visible entries
    (70000, 33, 2048, 1000, "random"),   # the wide top-k
    (30000, 20, 2048, 1500, "causal"),   # a top-k over more than 8,192 pool positions
    (300, 20, 8, 0, "causal"),           # k = 0: the pool alone
    (140000, 16, 2048, 512, "causal"),   # more than 16,384 blocks a row
    (140000, 130, 2048, 512, "causal"),  # and 260 rows: the one-wave-per-row block filter
    (200000, 128, 1000, 300, "random"),  # the same with a smaller pool and k, rows of 0 .. N visible
])
def test_index_full_prefill(kind, N, M, n_pool, k, nv):
    """Many queries per sequence through csa2_index_full: pool and top-k
    bit-exact against the oracle, with and without block maxima asked for."""
    B = 2
    w = Workload("pff", 3 + N + M + k, B=B, N=N, M=M, n_pool=n_pool, k=max(k, 1), prefill_base=N - M)
    cache, (lay,) = host_inputs(w, kind=kind)
    if nv == "random":
        rng = np.random.default_rng(N + M)
        v = rng.integers(0, N + 1, size=w.R).astype(np.int32)
        v[0], v[1], v[-1] = 0, N, 1
        lay["n_visible"] = v
    c, l = dev(cache), dev(lay)
    say(f"index_full prefill N={N} M={M} pool={n_pool} k={k} nv={nv} kind={kind}")
    ref = oracle.index_full(lay["q_codes"], lay["q_scales"], cache["k_codes"], cache["k_scales"], lay["n_visible"],
                            B, M, N, n_pool=n_pool, k=k)
    pool = torch.full((w.R, n_pool), -7, dtype=torch.int32, device="cuda")
    idx = torch.full((w.R, k), -7, dtype=torch.int32, device="cuda") if k else None
    csa2.csa2_index_full(l["q_codes"], l["q_scales"], c["k_codes"], c["k_scales"], l["n_visible"], B, M, N,
                         n_pool, k, pool, idx)
    torch.cuda.synchronize()
    assert np.array_equal(pool.cpu().numpy(), ref["pool_blocks"])
    if k:
        assert np.array_equal(idx.cpu().numpy(), ref["idx"])
    pool2 = torch.empty_like(pool)
    idx2 = torch.empty_like(idx) if k else None
    bmax = torch.empty((w.R, (N + 7) // 8), dtype=torch.float32, device="cuda")
    csa2.csa2_index_full(l["q_codes"], l["q_scales"], c["k_codes"], c["k_scales"], l["n_visible"], B, M, N,
                         n_pool, k, pool2, idx2, block_max=bmax)
    torch.cuda.synchronize()
    assert torch.equal(pool, pool2)
    if k:
        assert torch.equal(idx, idx2)


@pytest.mark.parametrize("kind", ["normal", "ties"])
@pytest.mark.parametrize("N,nv", [(600000, [600000, 599993]), (4194304, [4194304, 3000001])])
def test_index_full_rows_past_the_two_level_filter(kind, N, nv):
    """Rows of more than 65,536 blocks (the block filter's in-memory path) up to
    4,194,304 entries: pool and top-k bit-exact through csa2_index_full."""
    import synth

    B = len(nv)
    w = Workload("long", 31 + N, B=B, N=N)
    say(f"index_full long rows N={N} kind={kind}")
    if kind == "ties":   # a 4-code key alphabet and 2-code queries: scores tie constantly
        rng = np.random.default_rng(N)
        kc = rng.choice(np.array([0x00, 0x11, 0x22, 0x21], np.uint8), size=(B * N, 64))
        ks = np.full((B * N, 4), 127, np.uint8)
        qc = rng.choice(np.array([0x11, 0x22], np.uint8), size=(B, 64))
        qs = np.full((B, 4), 127, np.uint8)
    else:
        kc, ks = synth.mxfp4(w.seed, synth.T_INDEX_KEYS, 0, B * N, 128)
        qc, qs = synth.mxfp4(w.seed, synth.t_index_query(0), 0, B, 128)
    cache = {"k_codes": kc.reshape(B, N, 64), "k_scales": ks.reshape(B, N, 4)}
    lay = {"q_codes": qc, "q_scales": qs, "n_visible": np.array(nv, np.int32)}
    c, l = dev(cache), dev(lay)
    pool = torch.empty((B, 2048), dtype=torch.int32, device="cuda")
    idx = torch.empty((B, 512), dtype=torch.int32, device="cuda")
    csa2.csa2_index_full(l["q_codes"], l["q_scales"], c["k_codes"], c["k_scales"], l["n_visible"], B, 1, N, 2048,
                         512, pool, idx)
    torch.cuda.synchronize()
    ref = oracle.index_full(qc, qs, kc, ks, lay["n_visible"], B, 1, N, n_pool=2048, k=512)
    assert np.array_equal(pool.cpu().numpy(), ref["pool_blocks"])
    assert np.array_equal(idx.cpu().numpy(), ref["idx"])


def test_select_blocks_and_topk_full_layout():
    """csa2_select_blocks (pool + first k blocks) and csa2_topk over full score
    rows, against the oracle's sorts."""
    w = Workload("sel", 4242, B=4, N=70000, n_pool=2048, k=512)
    cache, (lay,) = host_inputs(w, kind="ties")
    lay["n_visible"] = np.array([70000, 69999, 16385, 12], np.int32)
    c, l = dev(cache), dev(lay)
    scores, bmax = _run_scan(w, c, l)
    ref = oracle_full(w, cache, lay, want_scores=True)
    R = w.R
    pool = torch.empty((R, 2048), dtype=torch.int32, device="cuda")
    tb = torch.empty((R, 300), dtype=torch.int32, device="cuda")
    csa2.csa2_select_blocks(torch.from_numpy(bmax).cuda(), l["n_visible"], 2048, pool, 300, tb)
    torch.cuda.synchronize()
    assert np.array_equal(pool.cpu().numpy(), ref["pool_blocks"])
    # the first 300 blocks = the pool of an oracle run with n_pool = 300
    w300 = Workload("sel", 4242, B=4, N=70000, n_pool=300, k=512)
    assert np.array_equal(tb.cpu().numpy(), oracle_full(w300, cache, lay)["pool_blocks"])
    # top-k over the full score rows (global top-k) equals the oracle's global top-k
    for k in (1, 512, 5000):
        idx = torch.empty((R, k), dtype=torch.int32, device="cuda")
        csa2.csa2_topk(torch.from_numpy(scores).cuda(), l["n_visible"], k, idx)
        torch.cuda.synchronize()
        want = oracle.topk_full(np.nan_to_num(ref["scores"], nan=-np.inf), lay["n_visible"], k)
        assert np.array_equal(idx.cpu().numpy(), want), k


@pytest.mark.parametrize("kind", ["normal", "ties", "spread", "mixed", "overflow"])
def test_reindex_pool_scores_and_topk(kind):
    """A Reindex layer: its own index query scored only inside the Full pool."""
    w = Workload("reidx", 777, B=3, N=50000, n_pool=2048, k=512)
    cache, (lay0, lay1) = host_inputs(w, layers=2, kind=kind)
    nv = np.array([50000, 49999, 10003], np.int32)
    lay0["n_visible"] = nv
    lay1["n_visible"] = nv
    c, l1 = dev(cache), dev(lay1)
    pool_np = oracle_full(w, cache, lay0)["pool_blocks"]
    pool = torch.from_numpy(pool_np).cuda()
    ps = torch.empty((w.R, 8 * 2048), dtype=torch.float32, device="cuda")
    csa2.csa2_index_pool(l1["q_codes"], l1["q_scales"], c["k_codes"], c["k_scales"], pool, l1["n_visible"], w.B, 1,
                         w.N, ps)
    idx = torch.empty((w.R, 512), dtype=torch.int32, device="cuda")
    csa2.csa2_topk(ps, l1["n_visible"], 512, idx, pool_blocks=pool)
    torch.cuda.synchronize()
    ref_ps = oracle.index_pool(lay1["q_codes"], lay1["q_scales"], cache["k_codes"], cache["k_scales"], pool_np, nv,
                               w.B, 1, w.N)
    assert np.array_equal(f32_bits(ps.cpu().numpy()), f32_bits(ref_ps))
    ref_idx = oracle.topk_pool(ref_ps, pool_np, nv, 512)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    # the same layer in one call (scores ranked in the scoring workgroup)
    idx1 = torch.full((w.R, 512), -7, dtype=torch.int32, device="cuda")
    csa2.csa2_index_pool_topk(l1["q_codes"], l1["q_scales"], c["k_codes"], c["k_scales"], pool, l1["n_visible"],
                              w.B, 1, w.N, 512, idx1)
    torch.cuda.synchronize()
    assert np.array_equal(idx1.cpu().numpy(), ref_idx)


@pytest.mark.parametrize("n_pool,k", [(2048, 512), (300, 3000), (1, 5), (2048, 16384)])
def test_reindex_one_call_edges(n_pool, k):
    """csa2_index_pool_topk against the oracle's pool scores and top-k: pools
    with -1 padding and blocks past a row's visible range, k above the valid
    slots (-1 padding), a one-block pool, a top-k over the whole pool."""
    w = Workload("reidx1", 4242 + n_pool + k, B=2, M=2, N=30000, n_pool=n_pool, k=k)
    cache, (lay,) = host_inputs(w)
    nv = np.array([30000, 29993, 17, 12345], np.int32)
    lay["n_visible"] = nv
    rng = np.random.default_rng(n_pool + k)
    nblk = (w.N + 7) // 8
    pool_np = np.full((w.R, n_pool), -1, np.int32)
    for r in range(w.R):
        m = n_pool if r % 2 == 0 else max(1, n_pool // 3)          # odd rows padded with -1
        pool_np[r, :m] = np.sort(rng.choice(nblk, size=m, replace=False))   # some blocks past n_visible
    c, l = dev(cache), dev(lay)
    idx = torch.full((w.R, k), -7, dtype=torch.int32, device="cuda")
    csa2.csa2_index_pool_topk(l["q_codes"], l["q_scales"], c["k_codes"], c["k_scales"],
                              torch.from_numpy(pool_np).cuda(), l["n_visible"], w.B, w.M, w.N, k, idx)
    torch.cuda.synchronize()
    ref_ps = oracle.index_pool(lay["q_codes"], lay["q_scales"], cache["k_codes"], cache["k_scales"], pool_np, nv,
                               w.B, w.M, w.N)
    assert np.array_equal(idx.cpu().numpy(), oracle.topk_pool(ref_ps, pool_np, nv, k))


def _attn_case(w, cache, lay, idx_np, win_max, H=None):
    c, l = dev(cache), dev(lay)
    out = torch.full((w.R, w.H, 512), float("nan"), device="cuda")
    idx = torch.from_numpy(idx_np).cuda() if idx_np.shape[1] else None
    csa2.csa2_sparse_attn(l["q"], c["c_codes"], c["c_scales"], idx, l["win"] if win_max else None,
                          l["win_start"] if win_max else None, l["win_len"] if win_max else None, win_max, w.B, w.M,
                          w.N, SM_SCALE, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("H", [16, 32, 64])
@pytest.mark.parametrize("k,win_lens", [(512, [128, 100, 0, 1]), (0, [128, 7, 128, 64]), (37, [0, 0, 0, 0]),
                                        (1000, [128, 128, 3, 0])])
def test_sparse_attn_vs_oracle(H, k, win_lens):
    w = Workload("attn", 31 + H + k, B=4, N=3000, H=H, k=max(k, 1))
    cache, (lay,) = host_inputs(w)
    lay["win_len"] = np.array(win_lens, np.int32)
    rng = np.random.default_rng(H * 1000 + k)
    idx = np.sort(rng.choice(w.N, size=(w.R, k), replace=True), axis=1).astype(np.int32)
    if k:
        idx[1, k // 2:] = -1          # a padded row
        idx[2, :] = idx[2, 0]         # one entry repeated k times
    win_max = 128
    say(f"attn H={H} k={k} win={win_lens}")
    got = _attn_case(w, cache, lay, idx, win_max)
    ref = oracle_attn(w, cache, lay, idx)
    err = np.max(np.abs(got - ref))
    say(f"  max abs err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= ATOL


@pytest.mark.parametrize("B,M,k,H", [
    (2, 64, 1500, 64),    # one split per row, over 1,024 later-chunk indices (the rest load directly)
    (4, 130, 200, 64),    # more than 1,024 workgroups (two per compute unit), a chunk mixing both row kinds
    (1, 700, 96, 32),     # 700 workgroups of 32 heads
    (1, 1100, 1100, 32),  # more than 1,024 workgroups, over 1,024 later-chunk indices
])
def test_sparse_attn_many_rows_long_rows(B, M, k, H):
    w = Workload("attnR", 1000 + B * M + k, B=B, M=M, N=2500, H=H, k=k)
    cache, (lay,) = host_inputs(w)
    rng = np.random.default_rng(B * M + k)
    lay["win_len"] = rng.integers(0, 129, size=w.R).astype(np.int32)
    idx = np.sort(rng.choice(w.N, size=(w.R, k), replace=True), axis=1).astype(np.int32)
    idx[::7, k // 3:] = -1            # padded rows
    say(f"attn B={B} M={M} k={k} H={H}")
    got = _attn_case(w, cache, lay, idx, 128)
    ref = oracle_attn(w, cache, lay, idx)
    err = np.max(np.abs(got - ref))
    say(f"  max abs err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= ATOL


@pytest.mark.parametrize("B,M,k,H", [
    (64, 1, 512, 64),    # 64 rows x 4 groups of 16 heads, one split of 20 chunks: streams of 7, 7, 6
    (4, 16, 600, 64),    # ragged rows, one split of 23 chunks: 8, 8, 7
    (2, 16, 2000, 32),   # four splits of 17 chunks (the last 16) and their combine
])
def test_sparse_attn_three_streams(B, M, k, H):
    """Grids of 16-head workgroups, one a compute unit, whose splits hold 16 or
    more chunks: the workgroup's three streams take every third chunk and merge
    their softmax states at the end (streams with an empty last round, padded
    and repeated entries, short windows)."""
    w = Workload("attn3", 7000 + B * M + k, B=B, M=M, N=2500, H=H, k=k)
    cache, (lay,) = host_inputs(w)
    rng = np.random.default_rng(B * M + k + H)
    lay["win_len"] = rng.integers(0, 129, size=w.R).astype(np.int32)
    idx = np.sort(rng.choice(w.N, size=(w.R, k), replace=True), axis=1).astype(np.int32)
    idx[::5, k // 3:] = -1            # padded rows
    idx[1, :] = idx[1, 0]             # one entry repeated k times
    say(f"attn three streams B={B} M={M} k={k} H={H}")
    got = _attn_case(w, cache, lay, idx, 128)
    ref = oracle_attn(w, cache, lay, idx)
    err = np.max(np.abs(got - ref))
    say(f"  max abs err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= ATOL


@pytest.mark.parametrize("H,k", [(16, 9000), (32, 16000)])
def test_sparse_attn_more_chunks_than_splits(H, k):
    """One row over more than 256 chunks of entries: the splits stop at the 256
    the combine merges (each split then takes two or more chunks) and every
    split's partial still reaches the output."""
    w = Workload("attnS", 9000 + H, B=1, N=k + 100, H=H, k=k)
    cache, (lay,) = host_inputs(w)
    rng = np.random.default_rng(H + k)
    lay["win_len"] = np.array([128], np.int32)
    idx = np.sort(rng.choice(w.N, size=(w.R, k), replace=False), axis=1).astype(np.int32)
    say(f"attn one row H={H} k={k}")
    got = _attn_case(w, cache, lay, idx, 128)
    ref = oracle_attn(w, cache, lay, idx)
    err = np.max(np.abs(got - ref))
    say(f"  max abs err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= ATOL


@pytest.mark.parametrize("H", [32, 64])
def test_sparse_attn_out_of_range_names(H):
    """Indices outside [0, N_max), window rows outside [0, Tw), window lengths
    above win_max or below zero: the kernels leave out what the oracle leaves
    out (the interface's rule), in every chunk position."""
    B, M, N = 2, 4, 900
    w = Workload("attnX", 4000 + H, B=B, M=M, N=N, H=H, k=100, prefill_base=N - M)
    cache, (lay,) = host_inputs(w)
    Tw = lay["win"].shape[1]
    rng = np.random.default_rng(H)
    idx = np.sort(rng.integers(0, N, size=(w.R, 100)), axis=1).astype(np.int32)
    idx[0, 10:20] = N                  # just past the cache
    idx[1, ::3] = N + 12345
    idx[2, :] = -5
    idx[3, 50:] = 1 << 30
    idx[4, :] = N + 1                  # with its window before row 0: nothing to attend to
    idx[5, 31:33] = -1                 # chunk edges
    idx[6, 60:] = N
    lay["win_start"] = np.array([0, -40, Tw - 60, Tw + 3, -200, 5, Tw - 1, 2], np.int32)
    lay["win_len"] = np.array([128, 100, 128, 50, 128, 500, 7, -3], np.int32)
    win_max = 96
    say(f"attn out-of-range names H={H} Tw={Tw} win_max={win_max}")
    got = _attn_case(w, cache, lay, idx, win_max)
    seqs = np.arange(w.R) // M
    ref = np.stack([oracle.sparse_attn(lay["q"][r:r + 1], cache["c_codes"][s:s + 1], cache["c_scales"][s:s + 1],
                                       idx[r:r + 1], lay["win"][s:s + 1], lay["win_start"][r:r + 1],
                                       lay["win_len"][r:r + 1], 1, 1, N, SM_SCALE, win_max=win_max)[0]
                    for r, s in enumerate(seqs)])
    err = np.max(np.abs(got - ref))
    say(f"  max abs err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= ATOL
    assert (got[4] == 0).all() and (ref[4] == 0).all()


def test_sparse_attn_no_window_and_empty():
    w = Workload("attn0", 5, B=2, N=500, H=64, k=64, win_len=0)
    cache, (lay,) = host_inputs(w)
    idx = np.full((2, 64), -1, np.int32)
    idx[0, :10] = np.arange(10)
    got = _attn_case(w, cache, lay, idx, 0)
    ref = oracle_attn(w, cache, lay, idx)
    assert np.max(np.abs(got - ref)) <= ATOL
    assert (got[1] == 0).all()        # empty set -> zeros


def test_dense_equivalence_on_gpu():
    """Check (b): k covering every entry gives dense attention over cache + window."""
    w = Workload("dense", 8, B=2, N=700, H=64, k=700)
    cache, (lay,) = host_inputs(w)
    idx = np.tile(np.arange(700, dtype=np.int32), (2, 1))
    got = _attn_case(w, cache, lay, idx, 128)
    dec = oracle.mxfp4_decode(cache["c_codes"], cache["c_scales"])
    win = torch.from_numpy(lay["win"]).view(torch.float8_e4m3fn).double().numpy()
    for r in range(2):
        rows = np.concatenate([dec[r], win[r]])
        z = torch.from_numpy(lay["q"][r].astype(np.float64)) @ torch.from_numpy(rows).T * float(SM_SCALE)
        ref = (torch.softmax(z, -1) @ torch.from_numpy(rows)).numpy()
        assert np.max(np.abs(got[r] - ref)) <= ATOL


def test_chain_full_reindex_reindex_reuse():
    """Full -> Reindex -> Reindex -> Reuse: shared pool and latent, own queries and
    windows; check (d): the Reuse layer equals attention with the previous indices."""
    w = Workload("chain", 4321, B=4, N=30000, layers=("full", "reindex", "reindex", "reuse"))
    cache, lays = host_inputs(w, layers=4)
    for d in lays:
        d["n_visible"] = np.array([30000, 29993, 17000, 4096], np.int32)
    c = dev(cache)
    ls = [dev(d) for d in lays]
    st = pipeline.Step(w.layers, w.B, 1, w.N)
    pool, idxs, outs = st.run(pipeline.cache_from(c), [pipeline.layer_from(d) for d in ls])
    torch.cuda.synchronize()
    ref_full = oracle_full(w, cache, lays[0])
    assert np.array_equal(pool.cpu().numpy(), ref_full["pool_blocks"])
    ref_idx = [ref_full["idx"]]
    for L in (1, 2):
        ps = oracle.index_pool(lays[L]["q_codes"], lays[L]["q_scales"], cache["k_codes"], cache["k_scales"],
                               ref_full["pool_blocks"], lays[L]["n_visible"], w.B, 1, w.N)
        ref_idx.append(oracle.topk_pool(ps, ref_full["pool_blocks"], lays[L]["n_visible"], 512))
    ref_idx.append(ref_idx[2])
    for L in range(3):
        assert np.array_equal(idxs[L].cpu().numpy(), ref_idx[L]), L
    for L in range(4):
        ref = oracle_attn(w, cache, lays[L], ref_idx[L])
        err = np.max(np.abs(outs[L].cpu().numpy() - ref))
        say(f"chain layer {L} max abs err {err:.3e}")
        assert err <= ATOL
    # check (d): Reuse output equals attention of its inputs with the previous layer's indices
    again = torch.empty_like(outs[3])
    csa2.csa2_sparse_attn(ls[3]["q"], c["c_codes"], c["c_scales"], idxs[2], ls[3]["win"], ls[3]["win_start"],
                          ls[3]["win_len"], 128, w.B, 1, w.N, SM_SCALE, again)
    torch.cuda.synchronize()
    assert torch.equal(again, outs[3])


@pytest.mark.parametrize("M", [5, 40, 520])
def test_chain_many_queries_per_sequence(M):
    """Full -> Reindex -> Reuse with M causal query rows per sequence: M = 5 is a
    verify step (multi-token decode scan), M = 40 a prefill chunk (the many-query
    scan), M = 520 one whose 1,040 rows take the one-call Reindex; the Reindex
    layer rescores the Full pool of each row with its own query, the Reuse
    layer takes the Reindex indices."""
    N = 20000
    w = Workload("chainM", 97 + M, B=2, N=N, M=M, prefill_base=N - M, layers=("full", "reindex", "reuse"),
                 H=16 if M > 100 else 64)   # 16 heads keep the oracle's attention over 1,040 rows short
    cache, lays = host_inputs(w, layers=3)
    c = dev(cache)
    ls = [dev(d) for d in lays]
    say(f"chain M={M}")
    st = pipeline.Step(w.layers, w.B, w.M, w.N, H=w.H, win_max=w.win_len)
    pool, idxs, outs = st.run(pipeline.cache_from(c), [pipeline.layer_from(d) for d in ls])
    torch.cuda.synchronize()
    ref_full = oracle_full(w, cache, lays[0])
    assert np.array_equal(pool.cpu().numpy(), ref_full["pool_blocks"])
    ps = oracle.index_pool(lays[1]["q_codes"], lays[1]["q_scales"], cache["k_codes"], cache["k_scales"],
                           ref_full["pool_blocks"], lays[1]["n_visible"], w.B, w.M, w.N)
    ref_idx = [ref_full["idx"], oracle.topk_pool(ps, ref_full["pool_blocks"], lays[1]["n_visible"], w.k)]
    ref_idx.append(ref_idx[1])
    for L in range(2):
        assert np.array_equal(idxs[L].cpu().numpy(), ref_idx[L]), L
    for L in range(3):
        ref = oracle_attn(w, cache, lays[L], ref_idx[L])
        err = np.max(np.abs(outs[L].cpu().numpy() - ref))
        say(f"chain M={M} layer {L} max abs err {err:.3e}")
        assert err <= ATOL


def test_deterministic_reruns():
    w = Workload("det", 55, B=4, N=60000)
    cache, (lay,) = host_inputs(w, kind="ties")
    c, l = dev(cache), dev(lay)
    st = pipeline.Step(("full",), w.B, 1, w.N, keep_scores=True)
    res = []
    for _ in range(2):
        pool, idxs, outs = st.run(pipeline.cache_from(c), [pipeline.layer_from(l)])
        torch.cuda.synchronize()
        res.append((pool.clone(), idxs[0].clone(), outs[0].clone(), st.scores.clone(), st.block_max.clone()))
    for a, b in zip(*res):
        assert torch.equal(a, b)
