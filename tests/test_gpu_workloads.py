"""GPU parity at the five workload sizes, in the launch configuration bench.py
times (pipeline.Step: csa2_index_full, then csa2_sparse_attn).  Pools and indices bit-exact, attention
within 1e-3 of the fp64 oracle, on all rows where the oracle is quick and on
sampled rows otherwise."""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_csa2_amd as csa2
import oracle
import synth
from hierarchical_sparse_attention_csa2_amd import pipeline

from gpu_cases import dev, oracle_attn, oracle_full, say

pytestmark = pytest.mark.gpu
ATOL = 1e-3


def _c5_rows():
    """c5 rows checked against the oracle: both ends of several 128-query
    groups of the many-query scan (the first two and last two rows of groups
    0, 1, 7, 15, 16 and 31) and 40 more drawn at random, 64 in all."""
    edges = [g * 128 + o for g in (0, 1, 7, 15, 16, 31) for o in (0, 1, 126, 127)]
    rng = np.random.default_rng(5)
    rest = [r for r in rng.permutation(4096).tolist() if r not in edges][:40]
    return sorted(edges + rest)


# None: every row
SAMPLES = {"c1": None, "c2": None, "c3": None, "c4": None, "c5": _c5_rows(), "v3": None}


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.load_library()


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5", "v3"])
def test_workload_parity(name):
    w = synth.WORKLOADS[name]
    say(f"workload {name}: {w.notes}")
    cache = synth.gen_cache(w)
    lays = [synth.gen_layer(w, layer=L, need_index_query=(m != "reuse")) for L, m in enumerate(w.layers)]
    c = dev(cache)
    ls = [dev(d) for d in lays]
    st = pipeline.Step(w.layers, w.B, w.M, w.N, H=w.H, n_pool=w.n_pool, k=w.k, win_max=w.win_len)
    pool, idxs, outs = st.run(pipeline.cache_from(c), [pipeline.layer_from(d) for d in ls])
    torch.cuda.synchronize()
    rows = SAMPLES[name]
    rows_np = np.arange(w.R) if rows is None else np.asarray(rows)
    say(f"  GPU done; oracle on {len(rows_np)} rows")
    ref_full = oracle_full(w, cache, lays[0], rows=rows_np)
    assert np.array_equal(pool.cpu().numpy()[rows_np], ref_full["pool_blocks"])
    ref_idx = [ref_full["idx"]]
    prev = ref_full["idx"]
    for L, mode in enumerate(w.layers[1:], start=1):
        if mode == "reindex":
            d = lays[L]
            seqs = rows_np // w.M    # each sampled row against its own sequence's keys
            ps = oracle.index_pool(d["q_codes"][rows_np], d["q_scales"][rows_np], cache["k_codes"][seqs],
                                   cache["k_scales"][seqs], ref_full["pool_blocks"], d["n_visible"][rows_np],
                                   len(rows_np), 1, w.N)
            prev = oracle.topk_pool(ps, ref_full["pool_blocks"], d["n_visible"][rows_np], w.k)
        ref_idx.append(prev)
    for L, mode in enumerate(w.layers):
        if mode != "reuse":
            assert np.array_equal(idxs[L].cpu().numpy()[rows_np], ref_idx[L]), (name, L)
        ref = oracle_attn(w, cache, lays[L], ref_idx[L], rows=rows_np)
        got = outs[L].cpu().numpy()[rows_np]
        err = float(np.max(np.abs(got - ref)))
        say(f"  layer {L} ({mode}) idx ok, attention max abs err {err:.3e}")
        assert err <= ATOL


def test_cache_write_full_size_sampled():
    """The cache write of c3's context (w3: 4 x 1,048,576 fp32 tokens at ratio 2,
    latent and indexer keys, plus the window rows) in bench.py's launch
    configuration; codes and scale bytes bit-exact on sampled entries (the first
    and last, entries around the kernels' tile-group boundaries and random ones)
    and on every window row."""
    cw = synth.CACHE_WRITES["w3"]
    T, E = cw.tokens, cw.entries
    say(f"cache write {cw.name}: {T} tokens -> {E} entries")
    x_lat = torch.empty((T, 512), dtype=torch.float32, device="cuda")
    x_idx = torch.empty((T, 128), dtype=torch.float32, device="cuda")
    wts = torch.empty(T, dtype=torch.float32, device="cuda")
    chunk = 1 << 18
    for r0 in range(0, T, chunk):
        n = min(chunk, T - r0)
        x_lat[r0:r0 + n].copy_(torch.from_numpy(cw.latent_rows(r0, n)))
        x_idx[r0:r0 + n].copy_(torch.from_numpy(cw.index_rows(r0, n)))
        wts[r0:r0 + n].copy_(torch.from_numpy(cw.weights(r0, n)))
    xw = cw.window_rows()
    c_codes = torch.empty((E, 256), dtype=torch.uint8, device="cuda")
    c_scales = torch.empty((E, 16), dtype=torch.uint8, device="cuda")
    k_codes = torch.empty((E, 64), dtype=torch.uint8, device="cuda")
    k_scales = torch.empty((E, 4), dtype=torch.uint8, device="cuda")
    win = torch.empty(xw.shape, dtype=torch.uint8, device="cuda")
    csa2.csa2_cache_write_mxfp4(x_lat, wts, cw.ratio, c_codes, c_scales)
    csa2.csa2_cache_write_mxfp4(x_idx, wts, cw.ratio, k_codes, k_scales)
    csa2.csa2_cache_write_e4m3(torch.from_numpy(xw).cuda(), win)
    torch.cuda.synchronize()
    del x_lat, x_idx, wts
    # a workgroup takes 256 quads: 2 latent entries or 8 key entries; tiles are
    # permuted in groups of 512
    rng = np.random.default_rng(3)
    edges = [0, 1, 2, 3, 7, 8, 1023, 1024, 1025, 4095, 4096, 4097, E // 2, E - 2, E - 1]
    sample = np.unique(np.concatenate([edges, rng.integers(0, E, 48)]))
    cc, cs = c_codes.cpu().numpy(), c_scales.cpu().numpy()
    kc, ks = k_codes.cpu().numpy(), k_scales.cpu().numpy()
    say(f"  GPU done; oracle on {sample.size} entries")
    for e in sample.tolist():
        w2 = cw.weights(2 * e, 2)
        rc, rs = oracle.cache_write_mxfp4(cw.latent_rows(2 * e, 2), w2, 2)
        assert np.array_equal(cc[e], rc[0]) and np.array_equal(cs[e], rs[0]), ("latent", e)
        rc, rs = oracle.cache_write_mxfp4(cw.index_rows(2 * e, 2), w2, 2)
        assert np.array_equal(kc[e], rc[0]) and np.array_equal(ks[e], rs[0]), ("index key", e)
    assert np.array_equal(win.cpu().numpy(), oracle.cache_write_e4m3(xw))
