"""A captured HIP graph of a whole step (csa2_index_full + csa2_sparse_attn,
the launches bench.py replays) gives the eager step's outputs bit for bit on
every replay, with other eager work on the same buffers between replays."""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_csa2_amd as csa2
from hierarchical_sparse_attention_csa2_amd import pipeline
from synth import Workload

from gpu_cases import dev, host_inputs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.load_library()


@pytest.mark.parametrize("modes", [("full",), ("full", "reindex", "reuse")])
def test_graph_replays_match_eager(modes):
    w = Workload("graph", 4321, B=3, N=20000, layers=modes)
    w_other = Workload("graph_other", 8765, B=3, N=20000, layers=modes)
    say(f"graph replay modes={modes}")
    cache_a, lays_a = host_inputs(w, layers=len(modes), kind="normal")
    cache_b, lays_b = host_inputs(w_other, layers=len(modes), kind="mixed")
    for lay in lays_a + lays_b:
        lay["n_visible"] = np.array([20000, 17777, 9001], np.int32)
    ca, la = pipeline.cache_from(dev(cache_a)), [pipeline.layer_from(dev(l)) for l in lays_a]
    cb, lb = pipeline.cache_from(dev(cache_b)), [pipeline.layer_from(dev(l)) for l in lays_b]
    st = pipeline.Step(modes, w.B, 1, w.N, n_pool=256, k=128, win_max=128)

    def snapshot():
        return [st.pool.clone()] + [x.clone() for x in st.idx] + [x.clone() for x in st.out]

    st.run(ca, la)
    torch.cuda.synchronize()
    ref = snapshot()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run(ca, la)
    torch.cuda.synchronize()
    for rep in range(3):
        st.run(cb, lb)        # eager work that overwrites every output buffer
        torch.cuda.synchronize()
        other = snapshot()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
        assert any(not torch.equal(a, b) for a, b in zip(other, ref)), "the eager work did not change the outputs"


@pytest.mark.parametrize("modes", [("full",), ("full", "reindex", "reuse")])
def test_bound_step_matches_run(modes):
    """Step.bind(): the recorded launches give run()'s outputs bit for bit, and
    follow new inputs copied into the same tensors."""
    w = Workload("bound", 1357, B=3, N=20000, layers=modes)
    w_other = Workload("bound_other", 2468, B=3, N=20000, layers=modes)
    cache_a, lays_a = host_inputs(w, layers=len(modes))
    cache_b, lays_b = host_inputs(w_other, layers=len(modes), kind="mixed")
    say(f"bound step modes={modes}")
    ca, la = pipeline.cache_from(dev(cache_a)), [pipeline.layer_from(dev(l)) for l in lays_a]
    st = pipeline.Step(modes, w.B, 1, w.N, n_pool=256, k=128, win_max=128)
    # the buffers a step writes (a Reuse layer keeps the previous indices)
    written = [st.pool] + [x for x, m in zip(st.idx, modes) if m != "reuse"] + st.out

    def snapshot():
        return [x.clone() for x in written]

    st.run(ca, la)
    torch.cuda.synchronize()
    want_a = snapshot()
    step = st.bind(ca, la)
    for t in written:
        t.fill_(-7)
    step()
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(snapshot(), want_a))
    # new inputs in place: the bound launches read them
    cb, lb = pipeline.cache_from(dev(cache_b)), [pipeline.layer_from(dev(l)) for l in lays_b]
    st.run(cb, lb)
    torch.cuda.synchronize()
    want_b = snapshot()
    for dst, src in zip((ca.k_codes, ca.k_scales, ca.c_codes, ca.c_scales), (cb.k_codes, cb.k_scales, cb.c_codes,
                                                                             cb.c_scales)):
        dst.copy_(src)
    for x, y in zip(la, lb):
        for name in ("q", "win", "win_start", "win_len", "n_visible", "q_codes", "q_scales"):
            if getattr(x, name) is not None:
                getattr(x, name).copy_(getattr(y, name))
    step()
    step()
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(snapshot(), want_b))


def test_cache_write_graph_replays_match_eager():
    """The cache write (latent merge, indexer-key merge, window rows) captured in
    one HIP graph: every replay equals the eager result bit for bit, with eager
    writes of other inputs into the same outputs between the replays."""
    import synth

    n, ratio = 1500, 2
    xa = torch.from_numpy(synth.f32(11, synth.T_TOKEN_LATENT, 0, n * ratio, 512)).cuda()
    ia = torch.from_numpy(synth.f32(11, synth.T_TOKEN_INDEX, 0, n * ratio, 128)).cuda()
    wa = torch.from_numpy(synth.merge_weights_f32(11, synth.T_MERGE_LOGITS, 0, n)).cuda()
    ya = torch.from_numpy(synth.f32(11, synth.T_TOKEN_WINDOW, 0, 128, 512)).cuda()
    xb, ib, yb = torch.randn_like(xa), torch.randn_like(ia), torch.randn_like(ya) * 100
    cc = torch.empty((n, 256), dtype=torch.uint8, device="cuda")
    cs = torch.empty((n, 16), dtype=torch.uint8, device="cuda")
    kc = torch.empty((n, 64), dtype=torch.uint8, device="cuda")
    ks = torch.empty((n, 4), dtype=torch.uint8, device="cuda")
    win = torch.empty((128, 512), dtype=torch.uint8, device="cuda")

    def write(x, i, y):
        csa2.csa2_cache_write_mxfp4(x, wa, ratio, cc, cs)
        csa2.csa2_cache_write_mxfp4(i, wa, ratio, kc, ks)
        csa2.csa2_cache_write_e4m3(y, win)

    write(xa, ia, ya)
    torch.cuda.synchronize()
    want = [t.clone() for t in (cc, cs, kc, ks, win)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        write(xa, ia, ya)
    torch.cuda.synchronize()
    for rep in range(3):
        write(xb, ib, yb)   # eager work on the same outputs between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(t, w) for t, w in zip((cc, cs, kc, ks, win), want)), rep
