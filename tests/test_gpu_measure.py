"""The benchmark's measurement kernels (libcsa2_measure.so): the decode scan
with FP4 matrix-core block values must give the library scan's outputs bit for bit
(same scores, block maxima and super-block maxima as the oracle), so that its
timing compares like with like; the read-only probe runs and stores nothing."""
import ctypes
import os

import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_csa2_amd as csa2
from synth import Workload

from gpu_cases import dev, f32_bits, host_inputs, oracle_full, say

pytestmark = pytest.mark.gpu
LIB = os.path.join(os.path.dirname(csa2.LIB_PATH), "libcsa2_measure.so")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.load_library()


def _lib():
    L = ctypes.CDLL(LIB)
    vp, i32, i64, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint32
    L.csa2m_read_probe.argtypes = [vp, vp, i32, i64, u32, vp, vp]
    L.csa2m_index_scan_mfma.argtypes = [vp, vp, vp, vp, vp, i32, i64, vp, vp, vp, vp]
    return L


P = lambda t: ctypes.c_void_p(t.data_ptr())
S = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("kind", ["normal", "spread", "mixed", "overflow"])
def test_mfma_scan_variant_bitexact(kind):
    N = 5000
    w = Workload("mmfma", 5150, B=3, N=N)
    cache, (lay,) = host_inputs(w, kind=kind)
    lay["n_visible"] = np.array([N, 4093, 1], np.int32)
    c, l = dev(cache), dev(lay)
    say(f"matrix-core scan variant kind={kind}")
    sc = torch.full((w.R, N), float("nan"), device="cuda")
    bm = torch.full((w.R, (N + 7) // 8), float("nan"), device="cuda")
    sm = torch.full((w.R, (N + 63) // 64), float("nan"), device="cuda")
    assert _lib().csa2m_index_scan_mfma(P(l["q_codes"]), P(l["q_scales"]), P(c["k_codes"]), P(c["k_scales"]),
                                        P(l["n_visible"]), w.B, N, P(sc), P(bm), P(sm), S()) == 0
    torch.cuda.synchronize()
    ref = oracle_full(w, cache, lay, want_scores=True, want_block_max=True)
    sc, bm, sm = sc.cpu().numpy(), bm.cpu().numpy(), sm.cpu().numpy()
    for r in range(w.R):
        n = int(lay["n_visible"][r])
        assert np.array_equal(f32_bits(sc[r, :n]), f32_bits(ref["scores"][r, :n])), r
        nb = (n + 7) // 8
        assert np.array_equal(f32_bits(bm[r, :nb]), f32_bits(ref["block_max"][r, :nb])), r
        want = [np.max(ref["block_max"][r, 8 * s:min(8 * s + 8, nb)]) for s in range((n + 63) // 64)]
        assert np.array_equal(f32_bits(sm[r, :len(want)]), f32_bits(np.array(want, np.float32))), r


def test_read_probe_runs_and_stores_nothing():
    w = Workload("mprobe", 5151, B=2, N=3000)
    cache, _ = host_inputs(w)
    c = dev(cache)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    assert _lib().csa2m_read_probe(P(c["k_codes"]), P(c["k_scales"]), w.B, w.N, 0x5EEDF00D, P(sink), S()) == 0
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
