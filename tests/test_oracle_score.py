"""Pins of the oracle's indexer score.

The pages say the indexer query and key are FP4 and that the indexer scores
every visible position (fupanwang.com DeepSeek-V4.1-Flash article, section
三个方向一起压小缓存).  The score is read as one 128-d dot product whose four
32-element blocks are summed exactly and then added in fp32 in block order.
The pins: exact rational arithmetic whenever the block exponents are close
(then every fp32 partial sum is exact), an adversarial case whose value depends
on the block order, closed forms, and fp32 subnormal rounding.
"""
from fractions import Fraction

import numpy as np

import oracle
import synth


def _pack(nibbles):
    nibbles = np.asarray(nibbles, np.uint8)
    return (nibbles[0::2] | (nibbles[1::2] << 4)).astype(np.uint8)


def _exact_dot(qc, qs, kc, ks):
    def vals(c, s):
        out = []
        for i in range(128):
            code = (c[i // 2] & 15) if i % 2 == 0 else (c[i // 2] >> 4)
            out.append(Fraction(oracle.e2m1_value(int(code))) * Fraction(2) ** (int(s[i // 32]) - 127))
        return out
    return sum(a * b for a, b in zip(vals(qc, qs), vals(kc, ks)))


def test_score_equals_exact_dot_when_exponents_are_close():
    rng = np.random.default_rng(11)
    for trial in range(300):
        qc = rng.integers(0, 256, 64, dtype=np.uint8)
        kc = rng.integers(0, 256, 64, dtype=np.uint8)
        base = int(rng.integers(60, 190))
        qs = (base + rng.integers(0, 5, 4)).astype(np.uint8)      # spread <= 4
        ks = (127 + rng.integers(-2, 3, 4)).astype(np.uint8)     # spread <= 4
        s = oracle.score(qc, qs, kc, ks)
        exact = _exact_dot(qc, qs, kc, ks)
        assert Fraction(s) == exact, (trial, s, float(exact))


def test_score_on_generated_normal_data_is_exact():
    qc, qs = synth.mxfp4(5, 4, 0, 8, 128)
    kc, ks = synth.mxfp4(5, 1, 0, 64, 128)
    for i in range(8):
        for j in range(64):
            assert Fraction(oracle.score(qc[i], qs[i], kc[j], ks[j])) == _exact_dot(qc[i], qs[i], kc[j], ks[j])


def test_score_block_order_is_fixed():
    # block values v = (2^30, 1, -2^30, 1): ((v0+v1)+v2)+v3 = 1 in fp32, exact sum is 2
    qn = np.zeros(128, np.uint8)
    kn = np.zeros(128, np.uint8)
    for b, neg in ((0, False), (1, False), (2, True), (3, False)):
        qn[32 * b] = 1                      # 0.5 -> half-units 1
        kn[32 * b] = 9 if neg else 1        # -0.5 / 0.5
    qc, kc = _pack(qn), _pack(kn)
    qs = np.array([143, 128, 143, 128], np.uint8)
    ks = np.array([143, 128, 143, 128], np.uint8)
    # isum_b = +-1, exponent qs+ks-256 = 30 or 0
    assert oracle.score(qc, qs, kc, ks) == 1.0
    assert _exact_dot(qc, qs, kc, ks) == 2


def test_score_closed_forms():
    rng = np.random.default_rng(12)
    for _ in range(50):
        c = rng.integers(0, 256, 64, dtype=np.uint8)
        s = np.full(4, 127, np.uint8)
        self_dot = oracle.score(c, s, c, s)
        vals = oracle.mxfp4_decode(c, s)
        assert self_dot == float(np.sum(vals * vals))          # exact: small integers / 4
        assert self_dot >= 0
        # symmetry and a power-of-two scale shift
        c2 = rng.integers(0, 256, 64, dtype=np.uint8)
        assert oracle.score(c, s, c2, s) == oracle.score(c2, s, c, s)
        assert oracle.score(c, s + 1, c2, s) == 2 * oracle.score(c, s, c2, s)
        assert oracle.score(c, s, c2, s - 3) == oracle.score(c, s, c2, s) / 8


def test_score_subnormal_rounding():
    # isum = 3 at exponent -150: 3 * 2^-150 rounds (to even) to 2 * 2^-149 in fp32
    qn = np.zeros(128, np.uint8)
    kn = np.zeros(128, np.uint8)
    qn[0] = 3            # 1.5 -> 3 half-units
    kn[0] = 1            # 0.5 -> 1 half-unit
    qc, kc = _pack(qn), _pack(kn)
    qs = np.array([53, 127, 127, 127], np.uint8)
    ks = np.array([53, 127, 127, 127], np.uint8)   # 53+53-256 = -150
    got = oracle.score(qc, qs, kc, ks)
    assert got == float(np.float32(3 * 2.0 ** -150))
    assert got == 2.0 ** -148


def _block_codes(sign_per_block, code=7):
    """128 nibbles: every element of block b is +-6 (E2M1 code 7) with the given sign."""
    n = np.zeros(128, np.uint8)
    for b, neg in enumerate(sign_per_block):
        n[32 * b:32 * b + 32] = code | (8 if neg else 0)
    return _pack(n)


def test_score_overflow_to_infinity_and_canonical_nan():
    """Block sums of 4608 quarter-units (32 products of 6 x 6) at block exponents
    e = eq + ek - 256 past 2^128 / 4608 overflow: ldexp gives +-inf, and a sum of
    opposite infinities is NaN, stored as the positive quiet NaN 0x7FC00000 (a
    fixed bit pattern, so it ranks above +inf in the total order on every host)."""
    q = _block_codes([False] * 4)
    # key blocks 0 and 1 of opposite signs, blocks 2 and 3 zero
    k = _block_codes([False, True, False, False])
    kz = np.frombuffer(k, np.uint8).copy()
    kz[32:] = 0
    qs = np.array([250, 250, 127, 127], np.uint8)
    ks = np.array([124, 124, 127, 127], np.uint8)     # e = 118: 4608 * 2^118 > 2^130 -> inf
    s = oracle.score(q, qs, kz, ks)
    assert np.isnan(s)
    assert np.float32(s).view(np.uint32) == 0x7FC00000
    assert oracle.order_key(s) == 0xFFC00000 > oracle.order_key(np.inf)
    # one block overflowing, the other finite: +inf, and -inf with the signs swapped
    ks2 = np.array([124, 100, 127, 127], np.uint8)
    assert oracle.score(q, qs, kz, ks2) == np.inf
    kneg = _block_codes([True, False, False, False])
    kn = np.frombuffer(kneg, np.uint8).copy()
    kn[32:] = 0
    assert oracle.score(q, qs, kn, ks2) == -np.inf
    # the largest block exponent whose block values stay finite for any codes:
    # 4608 * 2^e < 2^128 for e <= 115 (e = eq + ek - 256), exact there
    for e, want_inf in ((115, False), (116, True)):
        qs3 = np.array([127 + 64, 127, 127, 127], np.uint8)
        ks3 = np.array([256 + e - (127 + 64), 127, 127, 127], np.uint8)
        kk = np.frombuffer(_block_codes([False] * 4), np.uint8).copy()
        kk[16:] = 0
        s = oracle.score(q, qs3, kk, ks3)
        if want_inf:
            assert s == np.inf
        else:
            assert Fraction(s) == Fraction(4608) * Fraction(2) ** e
