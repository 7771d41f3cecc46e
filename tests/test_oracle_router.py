"""Pins for the oracle's router: logits, top-k and renormalised softmax weights.

The logit is defined as a binary32 sum in one fixed order (lanes of 8-element
chunks, FMA per lane, xor-butterfly over 64 lanes, then + bias).  Pins:
  * one-hot inputs give the router column plus bias (closed form);
  * hand-built cancellations whose binary32 result depends on exactly that
    order (derived by hand below, not by re-running the formula);
  * an exact rational brute force: every logit lies within the error bound
    of that order, and top-k agrees wherever the exact gap exceeds it;
  * duplicate router rows give exact ties, which go to the lower id;
  * top-k equals a stable argsort; weights equal scipy's softmax over the
    selected logits; k = 1 gives weight 1; equal logits give 1/k.
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch


def bf16_bits(v):
    return torch.tensor(np.asarray(v, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)


def bf16_vals(bits):
    return torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("wdt", [0, 1])
def test_one_hot_gives_column_plus_bias(orc, syn, wdt):
    E, H = 16, 128
    wr, b = syn.router(3, 0, E, H, wdt)
    for i in [0, 7, 8, 63, 64, 127]:
        x = np.zeros((1, H), np.float32)
        x[0, i] = 1.0
        if wdt == 1:
            x = bf16_bits(x)
        lg = orc.router_logits(x, wr, b, wdt)
        col = wr[:, i].astype(np.float32) if wdt == 0 else bf16_vals(wr[:, i]).astype(np.float32)
        assert np.array_equal(lg[0], (col + b).astype(np.float32))


def _one_token(H, entries):
    x = np.ones((1, H), np.float32)
    w = np.zeros((1, H), np.float32)
    for i, v in entries.items():
        w[0, i] = v
    return x, w


def test_order_within_lane_is_sequential_fma(orc):
    # elements 0, 1 are lane 0's first chunk; element 8 starts lane 1's chunk.
    # lane 0: fma(1, 2^24, 0) = 2^24; fma(1, 1, 2^24) = 2^24 + 1 is a tie -> 2^24 (even)
    # lane 1: -2^24.  Combine: 2^24 + (-2^24) = 0.  The exact sum is 1.
    x, w = _one_token(64, {0: 2.0 ** 24, 1: 1.0, 8: -(2.0 ** 24)})
    assert orc.router_logits(x, w, np.zeros(1, np.float32), 0)[0, 0] == 0.0


def test_order_across_lanes_is_butterfly(orc):
    # lanes 0..3 hold 2^24, 1, -2^24, 1 (chunks 0, 1, 2, 3).
    # butterfly o=2: lane0 = 2^24 + -2^24 = 0, lane1 = 1 + 1 = 2; o=1: 0 + 2 = 2 (exact).
    # a left-to-right sum would give ((2^24 + 1) - 2^24) + 1 = 1 instead.
    x, w = _one_token(64, {0: 2.0 ** 24, 8: 1.0, 16: -(2.0 ** 24), 24: 1.0})
    assert orc.router_logits(x, w, np.zeros(1, np.float32), 0)[0, 0] == 2.0


def test_lane_owns_every_64th_chunk(orc):
    # chunk 64 (elements 512..519) belongs to lane 0, after chunk 0:
    # lane 0: 2^24, then +1 (tie -> 2^24), then +1 (tie -> 2^24); lane 1: -2^24 -> result 0.
    x, w = _one_token(1024, {0: 2.0 ** 24, 512: 1.0, 513: 1.0, 8: -(2.0 ** 24)})
    assert orc.router_logits(x, w, np.zeros(1, np.float32), 0)[0, 0] == 0.0
    # the same values with chunk 64 moved to lane 2's position: lane 2 sums 1 + 1 = 2 exactly,
    # lane 0 = 2^24, lane 1 = -2^24; butterfly o=2: lane0 = 2^24 + 2 -> exact; o=1: + (-2^24) -> 2
    x, w = _one_token(1024, {0: 2.0 ** 24, 16: 1.0, 17: 1.0, 8: -(2.0 ** 24)})
    assert orc.router_logits(x, w, np.zeros(1, np.float32), 0)[0, 0] == 2.0


def test_bias_added_after_the_sum(orc):
    # sum = 2^24 exactly (lane 0), bias = 1: 2^24 + 1 rounds to 2^24 (tie to even)
    x, w = _one_token(64, {0: 2.0 ** 24})
    assert orc.router_logits(x, w, np.ones(1, np.float32), 0)[0, 0] == 2.0 ** 24
    # bias = 3: 2^24 + 3 is a tie between 2^24+2 and 2^24+4 -> 2^24 + 4
    assert orc.router_logits(x, w, np.full(1, 3.0, np.float32), 0)[0, 0] == 2.0 ** 24 + 4


@pytest.mark.parametrize("wdt,H", [(0, 64), (1, 64), (1, 512)])
def test_exact_rational_brute_force(orc, syn, wdt, H):
    E, T, k = 8, 4, 2
    wr, b = syn.router(11, 0, E, H, wdt)
    x = syn.tokens(11, 2, T, H, 1, 0.0, wdt)[0]
    lg = orc.router_logits(x, wr, b, wdt)
    xv = x.astype(np.float64) if wdt == 0 else bf16_vals(x)
    wv = wr.astype(np.float64) if wdt == 0 else bf16_vals(wr)
    u = Fraction(1, 2 ** 24)
    n = H // 64 + 7  # longest chain of roundings: H/64 fmas, 6 butterfly adds, bias add
    gamma = n * u / (1 - n * u)
    for t in range(T):
        exact = []
        for e in range(E):
            s = sum(Fraction(float(xv[t, i])) * Fraction(float(wv[e, i])) for i in range(H))
            mag = sum(abs(Fraction(float(xv[t, i])) * Fraction(float(wv[e, i]))) for i in range(H))
            ex = s + Fraction(float(b[e]))
            bound = gamma * (mag + abs(Fraction(float(b[e]))))
            assert abs(Fraction(float(lg[t, e])) - ex) <= bound
            exact.append((ex, bound))
        # top-k agrees with the exact ranking wherever the exact gaps are wider than both bounds
        order = sorted(range(E), key=lambda e: (-exact[e][0], e))
        ids, _ = orc.topk(lg[t:t + 1], k)
        for j in range(k):
            a, c = order[j], order[j + 1]
            if exact[a][0] - exact[c][0] > exact[a][1] + exact[c][1]:
                assert ids[0, j] == a


def test_duplicate_rows_tie_to_lower_id(orc, syn):
    E, H, k = 8, 64, 3
    wr, b = syn.router(5, 0, E, H, 0, zipf_s=0.0)
    wr[6] = wr[2]
    wr[5] = wr[2]
    x = np.zeros((1, H), np.float32)
    x[0] = np.sign(wr[2]) + 0.5 * np.sign(wr[2])  # makes row 2 (and its copies) the clear maximum
    lg = orc.router_logits(x, wr, b, 0)
    assert lg[0, 2] == lg[0, 5] == lg[0, 6]
    ids, w = orc.topk(lg, k)
    assert ids[0].tolist() == [2, 5, 6]
    assert np.allclose(w[0], 1.0 / 3, rtol=0, atol=1e-15)


def test_topk_is_stable_argsort_and_weights_are_softmax(orc):
    rng = np.random.default_rng(4)
    for E, k in [(8, 2), (128, 8), (256, 8), (8, 1)]:
        lg = (rng.standard_normal((64, E)) * 2).astype(np.float32)
        lg[:, 1] = lg[:, 3]  # some exact ties
        ids, w = orc.topk(lg, k)
        ref = np.argsort(-lg, axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, ref)
        sel = np.take_along_axis(lg, ref, axis=1).astype(np.float64)
        assert np.allclose(w, scipy.special.softmax(sel, axis=1), rtol=0, atol=1e-15)
        assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-12)
        if k == 1:
            assert np.all(w == 1.0)


def test_equal_logits_give_uniform_weights(orc):
    lg = np.zeros((3, 16), np.float32)
    ids, w = orc.topk(lg, 4)
    assert ids.tolist() == [[0, 1, 2, 3]] * 3
    assert np.all(w == 0.25)


def test_nan_logit_is_an_error(orc):
    lg = np.zeros((1, 8), np.float32)
    lg[0, 3] = np.nan
    with pytest.raises(ValueError):
        orc.topk(lg, 2)
