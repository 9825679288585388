"""Pins of the oracle's selection steps: block max, candidate pool, top-k.

The hierarchical sparse indexer (fupanwang.com DeepSeek-V4.1-Flash article,
section 三个方向一起压小缓存 and its figure caption): the first Full layer
scores the visible context, represents each 8-position block by its highest
score, keeps at most 2048 blocks as the candidate pool and selects its top-512;
later layers select their top-512 inside the pool.  Ranks are (score desc,
position asc).  Check (a): every selection equals a full sort done by brute
force in Python; plus the Full-pool lemma (pool top-k equals the global top-k
when the pool keeps at least k blocks), all-ties data, partial blocks and empty
inputs.
"""
import numpy as np
import pytest

import oracle
import synth


def _brute_blocks(scores, nv):
    nb = (nv + 7) // 8
    bm = []
    for b in range(nb):
        seg = [scores[j] for j in range(8 * b, min(8 * b + 8, nv))]
        bm.append(max(seg, key=lambda v: oracle.order_key(v)))
    return bm


def _brute_first_k(keys_ids, k):
    ranked = sorted(keys_ids, key=lambda t: (-t[0], t[1]))
    return sorted(i for _, i in ranked[:k])


def _pad(ids, n):
    return np.array(list(ids) + [-1] * (n - len(ids)), np.int32)


def _random_case(rng, B, N, M=1, few_values=False):
    R = B * M
    if few_values:
        # tiny alphabet so that many scores tie
        kc = rng.choice(np.array([0x00, 0x11, 0x22, 0x21], np.uint8), size=(B, N, 64))
        qc = rng.choice(np.array([0x11, 0x22], np.uint8), size=(R, 64))
    else:
        kc = rng.integers(0, 256, (B, N, 64), dtype=np.uint8)
        qc = rng.integers(0, 256, (R, 64), dtype=np.uint8)
    ks = (127 + rng.integers(-2, 3, (B, N, 4))).astype(np.uint8)
    qs = (127 + rng.integers(-2, 3, (R, 4))).astype(np.uint8)
    return qc, qs, kc, ks


@pytest.mark.parametrize("few", [False, True])
@pytest.mark.parametrize("N,n_pool,k", [(64, 3, 5), (61, 8, 64), (200, 4, 16), (203, 30, 7), (37, 100, 300)])
def test_index_full_against_brute_force(few, N, n_pool, k):
    rng = np.random.default_rng(N * 7 + n_pool + k + few)
    B = 3
    qc, qs, kc, ks = _random_case(rng, B, N, few_values=few)
    nv = np.array([N, N - 5, 1], np.int32)
    out = oracle.index_full(qc, qs, kc, ks, nv, B, 1, N, n_pool=n_pool, k=k, want_scores=True,
                            want_block_max=True)
    for r in range(B):
        s = [oracle.score(qc[r], qs[r], kc[r, j], ks[r, j]) for j in range(nv[r])]
        assert np.array_equal(np.array(s, np.float32), out["scores"][r, : nv[r]])
        bm = _brute_blocks(s, nv[r])
        assert np.array_equal(np.array(bm, np.float32), out["block_max"][r, : len(bm)])
        pool = _brute_first_k([(oracle.order_key(v), b) for b, v in enumerate(bm)], n_pool)
        assert np.array_equal(out["pool_blocks"][r], _pad(pool, n_pool))
        cand = [(oracle.order_key(s[j]), j) for b in pool for j in range(8 * b, min(8 * b + 8, nv[r]))]
        idx = _brute_first_k(cand, k)
        assert np.array_equal(out["idx"][r], _pad(idx, k))


def test_all_ties_select_first_positions():
    B, N = 2, 100
    kc = np.full((B, N, 64), 0x22, np.uint8)
    ks = np.full((B, N, 4), 127, np.uint8)
    qc = np.full((B, 64), 0x11, np.uint8)
    qs = np.full((B, 4), 127, np.uint8)
    nv = np.array([100, 43], np.int32)
    out = oracle.index_full(qc, qs, kc, ks, nv, B, 1, N, n_pool=4, k=10)
    assert np.array_equal(out["pool_blocks"][0], [0, 1, 2, 3])
    assert np.array_equal(out["idx"][0], np.arange(10))
    assert np.array_equal(out["idx"][1], np.arange(10))


def test_lemma_pool_topk_equals_global_topk():
    rng = np.random.default_rng(21)
    for N, n_pool, k in ((4096, 2048, 512), (4096, 600, 512), (3000, 512, 512), (1000, 100, 100),
                         (999, 125, 100), (60, 8, 100)):
        assert n_pool >= min(k, (N + 7) // 8)
        B = 2
        qc, qs = synth.mxfp4(N, 4, 0, B, 128)
        kc, ks = synth.mxfp4(N, 1, 0, B * N, 128)
        kc, ks = kc.reshape(B, N, 64), ks.reshape(B, N, 4)
        nv = np.array([N, N - 3], np.int32)
        a = oracle.index_full(qc, qs, kc, ks, nv, B, 1, N, n_pool=n_pool, k=k)
        g = oracle.index_full(qc, qs, kc, ks, nv, B, 1, N, n_pool=n_pool, k=k, global_topk=True)
        assert np.array_equal(a["idx"], g["idx"])
        # and the top-k equals the top-k restricted to the first k blocks
        b = oracle.index_full(qc, qs, kc, ks, nv, B, 1, N, n_pool=min(k, n_pool), k=k)
        assert np.array_equal(a["idx"], b["idx"])


def test_lemma_needs_enough_blocks():
    """With fewer kept blocks than k the pool restricts the choice (the
    approximation the pages acknowledge): the result stays inside the pool."""
    rng = np.random.default_rng(22)
    B, N = 1, 512
    qc, qs, kc, ks = _random_case(rng, B, N)
    nv = np.array([N], np.int32)
    a = oracle.index_full(qc, qs, kc, ks, nv, B, 1, N, n_pool=2, k=64)
    pool = a["pool_blocks"][0]
    sel = a["idx"][0]
    assert (sel[:16] // 8 >= 0).all() and set((sel[sel >= 0] // 8).tolist()) <= set(pool.tolist())
    assert (sel[16:] == -1).all()


def test_empty_and_tiny():
    B, N = 2, 16
    qc = np.zeros((B, 64), np.uint8)
    qs = np.full((B, 4), 127, np.uint8)
    kc = np.zeros((B, N, 64), np.uint8)
    ks = np.full((B, N, 4), 127, np.uint8)
    out = oracle.index_full(qc, qs, kc, ks, np.array([0, 3], np.int32), B, 1, N, n_pool=4, k=8)
    assert (out["pool_blocks"][0] == -1).all() and (out["idx"][0] == -1).all()
    assert np.array_equal(out["pool_blocks"][1], [0, -1, -1, -1])
    assert np.array_equal(out["idx"][1], [0, 1, 2, -1, -1, -1, -1, -1])


def test_index_pool_and_topk_pool_against_brute_force():
    rng = np.random.default_rng(23)
    B, N = 3, 300
    qc, qs, kc, ks = _random_case(rng, B, N, few_values=True)
    nv = np.array([300, 297, 150], np.int32)
    pool = np.array([[0, 5, 7, 37, -1], [2, 3, 4, 36, 37], [1, 2, 18, -1, -1]], np.int32)
    ps = oracle.index_pool(qc, qs, kc, ks, pool, nv, B, 1, N)
    for r in range(B):
        for i, b in enumerate(pool[r]):
            for t in range(8):
                j = 8 * b + t
                v = ps[r, 8 * i + t]
                if b < 0 or j >= nv[r]:
                    assert v == -np.inf
                else:
                    assert v == oracle.score(qc[r], qs[r], kc[r, j], ks[r, j])
    for k in (1, 7, 20, 40):
        idx = oracle.topk_pool(ps, pool, nv, k)
        for r in range(B):
            cand = [(oracle.order_key(ps[r, 8 * i + t]), 8 * b + t)
                    for i, b in enumerate(pool[r]) if b >= 0 for t in range(8) if 8 * b + t < nv[r]]
            assert np.array_equal(idx[r], _pad(_brute_first_k(cand, k), k))


def test_topk_full_against_brute_force():
    rng = np.random.default_rng(24)
    R, N = 4, 500
    scores = np.round(rng.normal(size=(R, N)) * 3).astype(np.float32)   # many ties
    nv = np.array([500, 499, 10, 0], np.int32)
    for k in (1, 16, 200):
        idx = oracle.topk_full(scores, nv, k)
        for r in range(R):
            cand = [(oracle.order_key(scores[r, j]), j) for j in range(nv[r])]
            assert np.array_equal(idx[r], _pad(_brute_first_k(cand, k), k))


@pytest.mark.parametrize("few", [False, True])
def test_index_full_many_queries_per_sequence_brute_force(few):
    """M > 1 query rows per sequence: row r belongs to sequence r // M and sees
    its own first n_visible[r] entries of that sequence's cache.  Each sequence
    has its own keys, so a row scored against the wrong cache, or with another
    row's visible count, fails the brute-force sort."""
    rng = np.random.default_rng(41 + few)
    B, M, N = 3, 4, 90
    qc, qs, kc, ks = _random_case(rng, B, N, M=M, few_values=few)
    nv = rng.integers(0, N + 1, size=B * M).astype(np.int32)
    nv[0], nv[5], nv[B * M - 1] = N, 1, 0
    n_pool, k = 5, 13
    out = oracle.index_full(qc, qs, kc, ks, nv, B, M, N, n_pool=n_pool, k=k, want_scores=True,
                            want_block_max=True)
    for r in range(B * M):
        seq = r // M
        s = [oracle.score(qc[r], qs[r], kc[seq, j], ks[seq, j]) for j in range(nv[r])]
        assert np.array_equal(np.array(s, np.float32), out["scores"][r, : nv[r]]), r
        bm = _brute_blocks(s, nv[r])
        assert np.array_equal(np.array(bm, np.float32), out["block_max"][r, : len(bm)]), r
        pool = _brute_first_k([(oracle.order_key(v), b) for b, v in enumerate(bm)], n_pool)
        assert np.array_equal(out["pool_blocks"][r], _pad(pool, n_pool)), r
        cand = [(oracle.order_key(s[j]), j) for b in pool for j in range(8 * b, min(8 * b + 8, nv[r]))]
        assert np.array_equal(out["idx"][r], _pad(_brute_first_k(cand, k), k)), r


def test_index_pool_many_queries_per_sequence_brute_force():
    """Reindex over M > 1 rows per sequence: row r's own query against its
    sequence's (r // M) keys, only inside its own pool row, -inf for slots past
    its own visible count or with no block."""
    rng = np.random.default_rng(43)
    B, M, N = 2, 3, 120
    qc, qs, kc, ks = _random_case(rng, B, N, M=M, few_values=True)
    nv = np.array([120, 77, 9, 64, 0, 119], np.int32)
    pool = np.array([[0, 3, 14, -1], [2, 9, 10, -1], [0, 1, -1, -1],
                     [4, 5, 6, 7], [0, -1, -1, -1], [1, 13, 14, -1]], np.int32)
    ps = oracle.index_pool(qc, qs, kc, ks, pool, nv, B, M, N)
    for r in range(B * M):
        seq = r // M
        for i, b in enumerate(pool[r]):
            for t in range(8):
                j = 8 * b + t
                v = ps[r, 8 * i + t]
                if b < 0 or j >= nv[r]:
                    assert v == -np.inf
                else:
                    assert v == oracle.score(qc[r], qs[r], kc[seq, j], ks[seq, j]), (r, i, t)
    for k in (1, 5, 40):
        idx = oracle.topk_pool(ps, pool, nv, k)
        for r in range(B * M):
            cand = [(oracle.order_key(ps[r, 8 * i + t]), 8 * b + t)
                    for i, b in enumerate(pool[r]) if b >= 0 for t in range(8) if 8 * b + t < nv[r]]
            assert np.array_equal(idx[r], _pad(_brute_first_k(cand, k), k)), (r, k)


def test_nan_scores_rank_first():
    """A NaN score (opposite infinite block values) is the positive quiet NaN and
    ranks ahead of +inf and of every number, in the block max, the pool and the
    top-k; ties among the NaN positions go to the lowest position."""
    B, N = 1, 40
    nib = lambda vals: (np.asarray(vals[0::2], np.uint8) | (np.asarray(vals[1::2], np.uint8) << 4))
    qn = np.full(128, 7, np.uint8)                     # +6 everywhere
    qc = nib(qn)[None, :]
    qs = np.array([[250, 250, 127, 127]], np.uint8)
    kc = np.zeros((B, N, 64), np.uint8)
    ks = np.full((B, N, 4), 127, np.uint8)
    # positions 3 and 17: blocks 0 / 1 at +6 / -6 with overflowing exponents -> NaN
    # position 30: block 0 overflowing alone -> +inf; the rest small finite values
    for p in (3, 17):
        kn = np.zeros(128, np.uint8)
        kn[0:32] = 7
        kn[32:64] = 15
        kc[0, p] = nib(kn)
        ks[0, p] = [124, 124, 127, 127]
    kn = np.zeros(128, np.uint8)
    kn[0:32] = 7
    kc[0, 30] = nib(kn)
    ks[0, 30] = [124, 124, 127, 127]
    for p in (1, 9, 25):
        kn = np.zeros(128, np.uint8)
        kn[100] = 2
        kc[0, p] = nib(kn)
    nv = np.array([N], np.int32)
    out = oracle.index_full(qc, qs, kc, ks, nv, B, 1, N, n_pool=3, k=4, want_scores=True, want_block_max=True)
    s = out["scores"][0]
    assert np.isnan(s[3]) and np.isnan(s[17]) and s[30] == np.inf
    assert s.view(np.uint32)[3] == 0x7FC00000
    assert np.array_equal(out["pool_blocks"][0], [0, 2, 3])     # NaN blocks 0, 2, then +inf block 3
    # NaN, NaN and +inf, then the best finite score inside the pool: positions
    # 1 and 25 tie (9 is in block 1, outside the pool), the lower one wins
    assert np.array_equal(out["idx"][0], [1, 3, 17, 30])


def test_threading_does_not_change_results():
    """Fewer rows than threads splits each row's scoring over position ranges
    (and attention over heads); the results equal a one-thread run bit for bit."""
    rng = np.random.default_rng(44)
    B, M, N = 1, 3, 5000
    qc, qs, kc, ks = _random_case(rng, B, N, M=M)
    nv = np.array([5000, 4321, 17], np.int32)
    one = oracle.index_full(qc, qs, kc, ks, nv, B, M, N, n_pool=64, k=100, want_scores=True, want_block_max=True,
                            threads=1)
    many = oracle.index_full(qc, qs, kc, ks, nv, B, M, N, n_pool=64, k=100, want_scores=True,
                             want_block_max=True, threads=16)
    for key in one:
        assert np.array_equal(np.asarray(one[key]).view(np.uint32), np.asarray(many[key]).view(np.uint32)), key
    cc, cs = synth.mxfp4(44, 2, 0, N, 512)
    q = synth.f32(44, 5, 0, M * 8, 512).reshape(M, 8, 512)
    win = synth.e4m3(44, 6, 0, 16, 512).reshape(1, 16, 512)
    ws, wl = np.zeros(M, np.int32), np.array([16, 3, 0], np.int32)
    args = (q, cc.reshape(1, N, 256), cs.reshape(1, N, 16), one["idx"], win, ws, wl, B, M, N, np.float32(0.04))
    a1 = oracle.sparse_attn(*args, threads=1)
    a16 = oracle.sparse_attn(*args, threads=16)
    assert np.array_equal(a1.view(np.uint32), a16.view(np.uint32))
