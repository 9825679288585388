"""Checks of the seeded input generator (not of the method): Philox known-answer
vectors, the normal distribution, determinism, and the ratio-2 merge used for
the 1M-token workload (each cached entry merges two adjacent tokens, fupanwang.com
DeepSeek-V4.1-Flash article, architecture figure caption: 每 2 个 token 合成一条缓存)."""
import os

import numpy as np

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    for line in open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        v = [int(t, 16) for t in line.split()]
        assert list(synth.philox(v[0:4], v[4:6])) == v[6:10]


def test_normals_distribution_and_determinism():
    z = synth.normals(1, 2, 0, 2000, 512)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    assert np.array_equal(z, synth.normals(1, 2, 0, 2000, 512))
    assert np.array_equal(z[100:200], synth.normals(1, 2, 100, 100, 512))
    assert not np.array_equal(z[:10], synth.normals(2, 2, 0, 10, 512))
    c1, s1 = synth.mxfp4(3, 1, 0, 500, 128, threads=1)
    c2, s2 = synth.mxfp4(3, 1, 0, 500, 128, threads=7)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_ratio2_merge():
    seed = 77
    rows = 40
    codes, scales = synth.mxfp4(seed, 1, 0, rows, 128, merged_logits=3)
    tok = synth.normals(seed, 1, 0, 2 * rows, 128)
    merged = np.empty((rows, 128))
    for r in range(rows):
        w = synth.merge_weights(seed, 3, r)
        assert abs(w.sum() - 1) < 1e-15 and (w > 0).all()
        merged[r] = w[0] * tok[2 * r] + w[1] * tok[2 * r + 1]
    c_o, s_o = oracle.mxfp4_encode(merged)
    assert np.array_equal(c_o, codes) and np.array_equal(s_o, scales)


def test_workload_shapes():
    w = synth.WORKLOADS["c5"]
    assert w.R == 4096 and w.Tw == 128 + 4095
    nv = w.n_visible()
    assert nv[0] == 262145 and nv[-1] == 266240 == w.N
    ws = w.win_start()
    # query at position p sees window rows for positions p-127 .. p
    assert ws[0] == 0 and ws[-1] == 4095
    c3 = synth.WORKLOADS["c3"]
    assert c3.N * c3.ratio == 1 << 20
