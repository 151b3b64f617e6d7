"""Pins of the oracle's random-number side: Philox4x32-10 against published
known-answer vectors, dropout-mask statistics, and the PLD schedule/gate."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat_rows():
    rows = []
    with open(GOLD) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            w = [int(t, 16) for t in line.split()]
            rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


def test_philox_known_answers():
    rows = _kat_rows()
    assert len(rows) == 3
    for ctr, key, want in rows:
        assert oracle.philox4x32_10(ctr, key) == want


def test_drop_threshold_exact():
    # floor(p * 2^16) in exact rational arithmetic, p as the fp32 value the library receives
    for p in (0.0, 0.1, 0.25, 0.5, 0.9):
        pf = np.float32(p)
        want = math.floor(Fraction(float(pf)) * 2 ** 16)
        assert oracle.drop_threshold(float(pf)) == want
    assert oracle.drop_threshold(float(np.float32(0.1))) == 6553


def test_realised_drop_probability():
    # The drop probability a 16-bit draw realises is q = floor(p * 2^16) / 2^16
    # (q <= p < q + 2^-16).  At p = 1.9 * 2^-16 (threshold 1) q is about half
    # of p, so the oracle's masks over 2^24 elements must match q and be far
    # from p (about 256 drops against the 486 p would give).
    n = 1 << 24
    for p in (1.9 * 2 ** -16, float(np.float32(0.1))):
        thr = oracle.drop_threshold(p)
        q = Fraction(thr, 2 ** 16)
        assert q <= Fraction(p) < q + Fraction(1, 2 ** 16)
        dropped = n - int(oracle.dropout_mask(99, 3, 2, 11, p, 0, n).sum(dtype=np.int64))
        sd = math.sqrt(n * float(q) * (1 - float(q)))
        assert abs(dropped - n * float(q)) < 5 * sd, (p, dropped, n * float(q))
        if p < 1e-4:
            assert abs(dropped - n * p) > 5 * sd
    # p = 0.1f: q = 6553/65536 and the inverted-dropout mean (1-q)/(1-p)
    p = float(np.float32(0.1))
    assert oracle.drop_threshold(p) == 6553
    bias = (1 - 6553 / 65536) / (1 - p) - 1
    assert 1.0e-5 < bias < 1.1e-5


def test_unrealisable_probability_rejected():
    # 0 < p < 2^-16 would realise no dropout at all; the oracle refuses it
    cfg = oracle.LayerCfg(1, 16, 64, 4, 256, attn_p=1e-6, hidden_p=0.1)
    p = {n: np.zeros(s) for n, s in {"w_qkv": (192, 64), "b_qkv": (192,), "w_o": (64, 64), "b_o": (64,),
                                     "ln1_g": (64,), "ln1_b": (64,), "w_1": (256, 64), "b_1": (256,),
                                     "w_2": (64, 256), "b_2": (64,), "ln2_g": (64,), "ln2_b": (64,)}.items()}
    with pytest.raises(ValueError):
        oracle.layer_forward(cfg, p, np.zeros((16, 64)), np.array([16]))


def test_mask_uses_philox_halfwords():
    # element e of a site: 16-bit half (e mod 2) of word (e/2 mod 4) of the
    # Philox4x32-10 block floor(e/8) (counter = (block, 0, site, step),
    # key = (seed, layer)); dropped iff that half < floor(p * 2^16).  The
    # Philox function itself is pinned by the known-answer vectors above.
    seed, layer, site, step = 1234, 5, 2, 77
    p = float(np.float32(0.25))
    thr = oracle.drop_threshold(p)
    e0, n = 8 * 1000 + 3, 64
    mask = oracle.dropout_mask(seed, layer, site, step, p, e0, n)
    for i in range(n):
        e = e0 + i
        words = oracle.philox4x32_10([e >> 3, 0, site, step], [seed, layer])
        half = (words[(e >> 1) & 3] >> (16 * (e & 1))) & 0xFFFF
        assert mask[i] == (1 if half >= thr else 0), e


def test_mask_p0_is_identity():
    m = oracle.dropout_mask(1234, 3, 1, 0, 0.0, 0, 10000)
    assert m.all()


@pytest.mark.parametrize("p", [0.1, 0.5])
def test_mask_keep_fraction(p):
    n = 1 << 20
    pf = float(np.float32(p))
    for site in (0, 1, 2):
        m = oracle.dropout_mask(1234, 5, site, 17, pf, 0, n)
        frac = m.mean()
        sigma = math.sqrt(p * (1 - p) / n)
        assert abs(frac - (1 - p)) < 5 * sigma
        # inverted dropout keeps the mean: E[m / (1-p)] = 1
        assert abs(m.mean() / (1 - pf) - 1.0) < 5 * sigma / (1 - p)


def test_mask_independent_of_key_fields():
    n = 1 << 16
    p = float(np.float32(0.1))
    base = oracle.dropout_mask(1234, 0, 1, 0, p, 0, n)
    again = oracle.dropout_mask(1234, 0, 1, 0, p, 0, n)
    assert np.array_equal(base, again)
    for other in (oracle.dropout_mask(1234, 1, 1, 0, p, 0, n),   # layer
                  oracle.dropout_mask(1234, 0, 2, 0, p, 0, n),   # site
                  oracle.dropout_mask(1234, 0, 1, 1, p, 0, n),   # step
                  oracle.dropout_mask(1235, 0, 1, 0, p, 0, n)):  # seed
        diff = (base != other).mean()
        # two independent Bernoulli(0.9) masks differ with probability 2 p (1-p) = 0.18
        assert abs(diff - 0.18) < 0.02


def test_mask_offset_window_consistent():
    p = float(np.float32(0.1))
    full = oracle.dropout_mask(7, 2, 0, 3, p, 0, 4096)
    part = oracle.dropout_mask(7, 2, 0, 3, p, 1001, 2000)
    assert np.array_equal(full[1001:3001], part)


def test_pld_theta_schedule():
    # theta starts at 1 (no skipping), decays towards theta_bar
    for tb in (0.0, 0.1, 0.9, 1.0):
        assert oracle.pld_theta(0, tb, 0.001) == 1.0
        vals = [oracle.pld_theta(t, tb, 0.001) for t in range(0, 20000, 500)]
        assert all(a >= b for a, b in zip(vals, vals[1:]))
        assert abs(oracle.pld_theta(1e7, tb, 0.001) - tb) < 1e-12
    # theta_bar = 0 reduces to a pure exponential decay
    for t in (1, 10, 1000, 4321):
        assert abs(oracle.pld_theta(t, 0.0, 0.001) - np.exp(-0.001 * t)) < 1e-15
    # theta_bar = 1 disables dropping entirely
    assert all(oracle.pld_theta(t, 1.0, 0.001) == 1.0 for t in range(0, 10000, 777))
    # value for the memory-saving stack: 0.5 + 0.5 * e^-5, e^-5 = 0.006737946999085467
    assert abs(oracle.pld_theta(5000, 0.5, 0.001) - 0.5033689734995427) < 1e-15


def test_pld_gate():
    assert all(oracle.pld_keep(7, l, s, 1.0) for l in range(24) for s in range(50))
    assert not any(oracle.pld_keep(7, l, s, 0.0) for l in range(24) for s in range(50))
    theta = oracle.pld_theta(5000, 0.5, 0.001)
    n = 24 * 2000
    kept = sum(oracle.pld_keep(7, l, s, theta) for l in range(24) for s in range(2000))
    sigma = math.sqrt(theta * (1 - theta) / n)
    assert abs(kept / n - theta) < 5 * sigma
