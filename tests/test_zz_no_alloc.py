"""The allocation-free Full-layer indexer (csa2_index_full_static) through the
C ABI, against csa2_index_full with a caller workspace: the same pool, top-k,
scores and block maxima, bit for bit, on two calls in a row (the second
smaller, so it runs over what the first left in the shared scratch), and the
size limit answered before any launch."""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_csa2_amd as csa2
from synth import Workload

from gpu_cases import dev, host_inputs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.load_library()


def _both(w, kind, nv):
    cache, (lay,) = host_inputs(w, kind=kind)
    if nv is not None:
        lay["n_visible"] = np.asarray(nv, np.int32)
    c, l = dev(cache), dev(lay)
    R, N, nblk = w.R, w.N, (w.N + 7) // 8
    outs = []
    for static in (True, False):
        pool = torch.full((R, w.n_pool), -7, dtype=torch.int32, device="cuda")
        idx = torch.full((R, w.k), -7, dtype=torch.int32, device="cuda")
        scores = torch.full((R, N), float("nan"), device="cuda")
        bmax = torch.full((R, nblk), float("nan"), device="cuda")
        args = (l["q_codes"], l["q_scales"], c["k_codes"], c["k_scales"], l["n_visible"], w.B, w.M, N, w.n_pool,
                w.k, pool, idx)
        if static:
            csa2.csa2_index_full_static(*args, scores=scores, block_max=bmax)
        else:
            csa2.csa2_index_full(*args, scores=scores, block_max=bmax)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in (pool, idx, scores, bmax)])
    return outs


def _same(a, b):
    for x, y in zip(a, b):
        if x.dtype == np.float32:
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
        else:
            assert np.array_equal(x, y)


@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_static_scratch_matches_workspace_call_twice(kind):
    # a long-context decode (two-level block filter, stored scores) and then a
    # smaller one (register filter) over the scratch the first one left
    big = Workload("noalloc1", 71, B=4, N=300000)
    small = Workload("noalloc2", 72, B=3, N=20000, k=300)
    for w, nv in ((big, [300000, 299999, 150001, 8]), (small, [20000, 1, 19993])):
        say(f"static scratch {w.name} kind={kind} R={w.R} N={w.N}")
        a, b = _both(w, kind, nv)
        _same(a, b)


def test_static_scratch_many_queries_and_repeat():
    # 5 queries per sequence (the multi-query scan), then the first call again
    w = Workload("noalloc3", 73, B=2, N=9000, M=5, prefill_base=9000 - 5)
    for _ in range(2):
        a, b = _both(w, "mixed", None)
        _same(a, b)


def test_static_scratch_rejects_oversize_without_launching():
    # a 4,096-query prefill chunk needs more block-maximum scratch than the array
    B, M, N = 1, 4096, 266240
    need = csa2.csa2_workspace_bytes(csa2.CSA2_OP_INDEX_FULL, B, M, N, 0, 512)
    assert need > csa2.CSA2_STATIC_SCRATCH_BYTES
    z = lambda *shape, dt=torch.uint8: torch.zeros(shape, dtype=dt, device="cuda")
    pool = z(M, 2048, dt=torch.int32)
    idx = z(M, 512, dt=torch.int32)
    with pytest.raises(csa2.Csa2Error) as e:
        csa2.csa2_index_full_static(z(M, 64), z(M, 4), z(N, 64), z(N, 4), z(M, dt=torch.int32), B, M, N, 2048, 512,
                                    pool, idx)
    assert e.value.status == csa2.CSA2_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert int(pool.abs().sum()) == 0 and int(idx.abs().sum()) == 0    # nothing was launched
