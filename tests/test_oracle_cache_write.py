"""Pins of the oracle's cache write: the ratio-m merge and the quantize-on-write.

The pages (fupanwang.com DeepSeek-V4.1-Flash article, section 三个方向一起压小缓存)
store every m consecutive tokens as one entry, merged with the layer's
compression weights, entries not overlapping, then keep the main KV and indexer
keys in OCP MXFP4 and the window in FP8.  The merge's precision is not given;
the reading taken is fp32, tokens in order, each product rounded before it is
added.  Each pin below fixes that by values worked out by hand from IEEE-754
single-precision rounding, exact small-integer arithmetic, or the error bound
of a sequential sum, so that a dropped term, a wrong token stride, a different
order or a fused multiply-add fails one of them.
"""
import math

import numpy as np
import pytest

import oracle
import synth


def _merge(x, w, ratio):
    return oracle.merge(np.asarray(x, np.float32), None if w is None else np.asarray(w, np.float32), ratio)


def test_merge_one_hot_weights_pick_each_token():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5 * 3, 64)).astype(np.float32)
    for j in range(3):
        w = np.zeros(15, np.float32)
        w[j::3] = 1.0
        out = _merge(x, w, 3)
        assert np.array_equal(out, x[j::3]), j


def test_merge_exact_small_integers_and_power_of_two_weights():
    # every product and partial sum is an integer multiple of 1/4 below 2^10:
    # exact in fp32, so the result equals the exact sum
    rng = np.random.default_rng(4)
    x = rng.integers(-8, 9, size=(6 * 4, 32)).astype(np.float32)
    w = rng.choice(np.array([0.25, 0.5, -1.0, 2.0, -4.0], np.float32), size=24)
    exact = (x.astype(np.float64) * w[:, None]).reshape(6, 4, 32).sum(axis=1)
    assert np.array_equal(_merge(x, w, 4).astype(np.float64), exact)


def test_merge_adds_tokens_in_order():
    # ((1 + 2^-24) + 2^-24) = 1 under round-to-nearest-even, whereas any other
    # grouping adds 2^-23 to 1 first
    x = np.array([[1.0], [2.0 ** -24], [2.0 ** -24]], np.float32).repeat(32, axis=1)
    out = _merge(x, np.ones(3, np.float32), 3)
    assert np.all(out == 1.0)
    x2 = x[::-1].copy()
    assert np.all(_merge(x2, np.ones(3, np.float32), 3) == np.float32(1.0 + 2.0 ** -23))


def test_merge_rounds_each_product_before_adding():
    # (-1)*1 + fl((1+2^-12)^2): the product 1 + 2^-11 + 2^-24 rounds (a tie, to
    # even) to 1 + 2^-11, so the sum is 2^-11; a fused multiply-add would keep
    # the 2^-24 and give 2^-11 + 2^-24
    a = 1.0 + 2.0 ** -12
    x = np.array([[-1.0], [a]], np.float32).repeat(32, axis=1)
    w = np.array([1.0, a], np.float32)
    out = _merge(x, w, 2)
    assert np.all(out == np.float32(2.0 ** -11))


def test_merge_within_sequential_sum_error_bound():
    # |fl(sum) - sum| <= m u sum |w x| (+ product roundings, also u each) with
    # u = 2^-24; random N(0,1) rows and softmax weights as the generator makes them
    x = synth.normals(11, 7, 0, 4096, 128).astype(np.float32)
    w = synth.merge_weights_f32(11, 3, 0, 2048)
    out = _merge(x, w, 2).astype(np.float64)
    xd, wd = x.astype(np.float64), w.astype(np.float64)
    exact = (xd * wd[:, None]).reshape(2048, 2, 128).sum(axis=1)
    bound = 3 * 2.0 ** -24 * np.abs(xd * wd[:, None]).reshape(2048, 2, 128).sum(axis=1)
    assert np.all(np.abs(out - exact) <= bound)
    # and the merge is not trivially exact: some rounding did happen
    assert np.any(out != exact)


def test_cache_write_is_encoder_of_merge():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((8 * 2, 128)).astype(np.float32)
    w = synth.merge_weights_f32(5, 3, 0, 8)
    codes, scales = oracle.cache_write_mxfp4(x, w, 2)
    c2, s2 = oracle.mxfp4_encode(_merge(x, w, 2).astype(np.float64))
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
    # ratio 1 without weights stores the rows as they are
    c1, s1 = oracle.cache_write_mxfp4(x, None, 1)
    c3, s3 = oracle.mxfp4_encode(x.astype(np.float64))
    assert np.array_equal(c1, c3) and np.array_equal(s1, s3)


def _nib(codes, i):
    return (codes[i // 2] >> (4 * (i % 2))) & 15


def test_encoder_special_values():
    # readings for values the format leaves open: NaN elements are ignored by
    # amax and stored as +0; an infinite amax takes E = 127 and stores +-6
    x = np.zeros((1, 32), np.float32)
    x[0, :4] = [np.inf, 1.0, -np.inf, np.nan]
    c, s = oracle.cache_write_mxfp4(x, None, 1)
    assert s[0, 0] == 254
    assert [_nib(c[0], i) for i in range(4)] == [7, 0, 15, 0]
    # a NaN beside finite values: same bytes as with the NaN replaced by 0
    y = np.linspace(-3, 3, 32).astype(np.float32)[None]
    y2 = y.copy()
    y2[0, 5] = np.nan
    cy, sy = oracle.cache_write_mxfp4(y, None, 1)
    y3 = y.copy()
    y3[0, 5] = 0.0
    c3, s3 = oracle.cache_write_mxfp4(y3, None, 1)
    cn, sn = oracle.cache_write_mxfp4(y2, None, 1)
    assert np.array_equal(cn, c3) and np.array_equal(sn, s3)
    # all NaN: a zero block
    cz, sz = oracle.cache_write_mxfp4(np.full((1, 32), np.nan, np.float32), None, 1)
    assert sz[0, 0] == 0 and not cz.any()
    # a subnormal amax 2^-128: E = floor(log2) - 2 = -130 clamps to -127 (byte
    # 0), the element is 2^-128 / 2^-127 = 0.5 -> code 1
    t = np.zeros((1, 32), np.float32)
    t[0, 0] = np.float32(2.0 ** -128)
    ct, st = oracle.cache_write_mxfp4(t, None, 1)
    assert st[0, 0] == 0 and _nib(ct[0], 0) == 1 and not ct[0, 1:].any()
    # -0 and a negative value that rounds to 0 store +0
    u = np.zeros((1, 32), np.float32)
    u[0, :3] = [4.0, -0.0, -0.2]   # E = 0; -0.2 is below the 0.25 midpoint
    cu, su = oracle.cache_write_mxfp4(u, None, 1)
    assert su[0, 0] == 127 and [_nib(cu[0], i) for i in range(3)] == [6, 0, 0]


def test_encoder_midpoints_tie_to_even_codes():
    # E = 0 (amax 6 -> floor(log2 6) - 2 = 0); the midpoints between adjacent
    # E2M1 values go to the even code, a hair above goes up
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    tie = [0, 2, 2, 4, 4, 6, 6]
    up = [1, 2, 3, 4, 5, 6, 7]
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 6.0
    x[0, 1:8] = mids
    x[0, 8:15] = [np.nextafter(np.float32(m), np.float32(10)) for m in mids]
    x[0, 15:22] = [-m for m in mids]
    c, s = oracle.cache_write_mxfp4(x, None, 1)
    assert s[0, 0] == 127
    assert [_nib(c[0], 1 + i) for i in range(7)] == tie
    assert [_nib(c[0], 8 + i) for i in range(7)] == up
    assert [_nib(c[0], 15 + i) for i in range(7)] == [(t | 8) if t else 0 for t in tie]


def test_e4m3_write_hand_values():
    vals = np.array([1.0, 448.0, 464.0, 1e9, -np.inf, np.nan, -0.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10,
                     1.0625, 1.1875, 432.0, -2.0 ** -6], np.float32)
    want = [0x38, 0x7E, 0x7E, 0x7E, 0xFE, 0x7F, 0x80, 0x01, 0x00, 0x02, 0x38, 0x3A, 0x7E, 0x88]
    assert list(oracle.cache_write_e4m3(vals)) == want


def test_e4m3_write_matches_value_table_nearest():
    # every value of a fine grid lands on a nearest E4M3 value (brute force
    # over the decoded table), ties on the even code
    table = np.array([oracle.e4m3_value(c) for c in range(256)])
    grid = np.concatenate([np.linspace(-470, 470, 4001), np.linspace(-0.03, 0.03, 2001)]).astype(np.float32)
    got = oracle.cache_write_e4m3(grid)
    for v, c in zip(grid.astype(np.float64), got):
        if abs(v) >= 448:
            assert c == (0xFE if v < 0 else 0x7E)
            continue
        same = [k for k in range(256) if not math.isnan(table[k]) and math.copysign(1, table[k]) == math.copysign(1, v)]
        d = min(abs(table[k] - v) for k in same)
        assert abs(table[c] - v) == d
        ties = [k for k in same if abs(table[k] - v) == d]
        if len(ties) > 1:
            assert c % 2 == 0
