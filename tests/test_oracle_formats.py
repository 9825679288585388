"""Pins of the oracle's storage formats (check (e): MXFP4 round trip against the
OCP E2M1 value table; E8M0 scales; OCP FP8 E4M3 for the sliding window).

The pages name OCP MXFP4 for the main KV, FP4 for the indexer query/key and
FP8 for the sliding-window KV (fupanwang.com DeepSeek-V4.1-Flash article,
section 三个方向一起压小缓存).  The encodings themselves are the OCP MX v1.0
definitions; each pin below derives the expected value independently of the
oracle's own tables (field arithmetic, torch's float8 dtype, brute force).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e2m1_from_fields(code):
    s = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        return s * 0.5 * m
    return s * 2.0 ** (e - 1) * (1 + m / 2)


def test_e2m1_table_matches_ocp_golden_and_fields():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_ocp_table.txt")) if l.strip() and l[0] != "#"]
    assert len(rows) == 16
    for code_s, val_s in rows:
        code, val = int(code_s), float(val_s)
        assert oracle.e2m1_value(code) == val
        assert math.copysign(1.0, oracle.e2m1_value(code)) == math.copysign(1.0, val)
        assert _e2m1_from_fields(code) == val


def test_e8m0_scale():
    for b in range(255):
        assert oracle.e8m0_scale(b) == 2.0 ** (b - 127)
    assert math.isnan(oracle.e8m0_scale(255))


def test_e4m3_decode_all_codes_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        v = oracle.e4m3_value(c)
        if math.isnan(ref[c]):
            assert math.isnan(v), c
        else:
            assert v == ref[c], (c, v, ref[c])
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9


def test_e4m3_encode_vs_torch_rne():
    rng = np.random.default_rng(5)
    # every representable value, every midpoint, and random values inside the range
    finite = sorted({oracle.e4m3_value(c) for c in range(256)} - {float("nan")})
    finite = [v for v in finite if not math.isnan(v)]
    mids = [(a + b) / 2 for a, b in zip(finite[:-1], finite[1:])]
    xs = np.concatenate([finite, mids, rng.normal(size=4000), rng.normal(size=2000) * 100,
                         rng.normal(size=2000) * 1e-3])
    xs = xs[np.abs(xs) < 448.0]
    ref = torch.tensor(xs, dtype=torch.float64).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for x, r in zip(xs, ref):
        got = oracle.e4m3_encode(float(x))
        if x == 0.0:
            assert oracle.e4m3_value(got) == 0.0
            continue
        assert got == r, (x, got, r)
        assert synth.lib().synth_e4m3_encode(float(x)) == r


def test_e4m3_encode_saturates():
    for x in (448.0, 449.0, 464.0, 1e6, float("inf")):
        assert oracle.e4m3_encode(x) == 0x7E
        assert oracle.e4m3_encode(-x) == 0xFE
        assert synth.lib().synth_e4m3_encode(x) == 0x7E


def _block(vals):
    x = np.zeros(32)
    x[: len(vals)] = vals
    return x


def test_mxfp4_scale_rule_exact_at_powers_of_two():
    # E = floor(log2 amax) - 2: amax = 4 -> E = 0 (byte 127); amax just below 4 -> E = -1
    _, s = oracle.mxfp4_encode(_block([4.0]))
    assert s[0] == 127
    _, s = oracle.mxfp4_encode(_block([np.nextafter(4.0, 0.0)]))
    assert s[0] == 126
    _, s = oracle.mxfp4_encode(_block([1.0]))
    assert s[0] == 125
    _, s = oracle.mxfp4_encode(np.zeros(32))
    assert s[0] == 0


def test_mxfp4_rne_ties_and_saturation():
    # amax fixed at 4 so E = 0 and the element grid is the E2M1 table itself
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0,
            -0.25: 0.0, -2.5: -2.0, -5.0: -4.0}
    for x, want in ties.items():
        c, s = oracle.mxfp4_encode(_block([4.0, x]))
        assert s[0] == 127
        got = oracle.mxfp4_decode(c, s)[1]
        assert got == want, (x, got, want)
    # saturation: with amax in [4, 8) every element is below 8 so y < 8; 7.9 -> 6
    c, s = oracle.mxfp4_encode(_block([7.9]))
    assert s[0] == 127 and oracle.mxfp4_decode(c, s)[0] == 6.0


def test_mxfp4_round_trip_on_representable_values():
    rng = np.random.default_rng(1)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    for _ in range(200):
        E = int(rng.integers(-20, 20))
        v = rng.choice(mags, size=32) * rng.choice([-1, 1], size=32)
        v[rng.integers(0, 32)] = 6.0 if rng.random() < 0.5 else 4.0   # pins amax -> E
        x = v * 2.0 ** E
        c, s = oracle.mxfp4_encode(x)
        back = oracle.mxfp4_decode(c, s)
        assert np.array_equal(back, x)
        c2, s2 = oracle.mxfp4_encode(back)
        assert np.array_equal(c2, c) and np.array_equal(s2, s)


def test_mxfp4_is_nearest_grid_value_brute_force():
    rng = np.random.default_rng(2)
    x = rng.normal(size=(300, 32)) * np.exp(rng.normal(size=(300, 1)) * 3)
    codes, scales = oracle.mxfp4_encode(x)
    dec = oracle.mxfp4_decode(codes, scales)
    table = np.array([_e2m1_from_fields(c) for c in range(16)])
    for i in range(x.shape[0]):
        amax = np.max(np.abs(x[i]))
        E = math.frexp(amax)[1] - 1 - 2          # floor(log2 amax) - 2 via frexp
        assert scales[i, 0] == E + 127
        grid = table * 2.0 ** E
        for j in range(32):
            y = x[i, j]
            d = np.abs(grid - y)
            best = d.min()
            if abs(y) >= 6 * 2.0 ** E:
                assert dec[i, j] == math.copysign(6 * 2.0 ** E, y)
            else:
                assert abs(dec[i, j] - y) == best


def test_synth_encoder_matches_oracle_encoder():
    raw = synth.normals(7, 99, 0, 64, 512)
    c_o, s_o = oracle.mxfp4_encode(raw)
    c_s = np.empty((64, 256), np.uint8)
    s_s = np.empty((64, 16), np.uint8)
    for r in range(64):
        for b in range(16):
            blk = np.ascontiguousarray(raw[r, 32 * b: 32 * b + 32])
            synth.lib().synth_mxfp4_encode_block(
                blk.ctypes.data, c_s[r, 16 * b:].ctypes.data, s_s[r, b:].ctypes.data)
    assert np.array_equal(c_o, c_s) and np.array_equal(s_o, s_s)
    c_g, s_g = synth.mxfp4(7, 99, 0, 64, 512)
    assert np.array_equal(c_g, c_o) and np.array_equal(s_g, s_o)


def test_order_key_matches_numeric_order():
    rng = np.random.default_rng(3)
    f = np.concatenate([rng.normal(size=2000).astype(np.float32) * 50,
                        np.array([0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45], np.float32)])
    keys = np.array([oracle.order_key(x) for x in f], dtype=np.uint64)
    for _ in range(3000):
        i, j = rng.integers(0, len(f), 2)
        a, b = float(f[i]), float(f[j])
        if a == b and math.copysign(1, a) == math.copysign(1, b):
            assert keys[i] == keys[j]
        elif a == b:          # +0 vs -0: -0 is below
            assert (keys[i] > keys[j]) == (math.copysign(1, a) > 0)
        else:
            assert (keys[i] > keys[j]) == (a > b)
