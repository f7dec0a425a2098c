"""Pins of the oracle's channel top-k ("Channel Selection for Mixture-of-Experts
Decoding Needs No Calibration Data", section 5.2: each channel of a token's
activated experts is scored by router weight x down-column norm x activation
magnitude, and the top-k over the token's channels are kept; section 2: a
channel owns one gate row, one up row and one down column).

Checked against numpy fp64, a lexicographic sort (brute force), and the
special cases that reduce to the full layer (keep everything) or to nothing
(keep none).  No GPU.
"""
import numpy as np
import pytest

import oracle
from test_oracle_pins import bf16_to_f64, normwise, tiny_layer


def routed_tiny(seed=0, bf16=True, k1=3, k2=5):
    x, Wr, Wg, Wu, Wd = tiny_layer(seed=seed, bf16=bf16)
    lg = oracle.logits(x, Wr)
    ids, w = oracle.route(lg, k1, k2)
    return x, Wg, Wu, Wd, ids, w


def brute_select(s_row, keep):
    order = np.lexsort((np.arange(s_row.size), -s_row.astype(np.float64)))
    kept = np.zeros(s_row.size, bool)
    kept[order[:keep]] = True
    return kept


def test_down_column_norms_match_numpy():
    _, _, _, Wd, _, _ = routed_tiny()
    dn = oracle.down_column_norms(Wd)
    ref = np.sqrt((bf16_to_f64(Wd) ** 2).sum(axis=1))
    assert np.allclose(dn, ref, rtol=1e-6, atol=0)


def test_scores_match_numpy_fp64():
    x, Wg, Wu, Wd, ids, w = routed_tiny()
    dn = oracle.down_column_norms(Wd)
    s = oracle.channel_scores(x, Wg, Wu, ids, w, dn)
    x64 = bf16_to_f64(x)
    T, k1 = ids.shape
    I = Wg.shape[1]
    for t in range(T):
        for r in range(k1):
            e = ids[t, r]
            g = bf16_to_f64(Wg[e]) @ x64[t]
            u = bf16_to_f64(Wu[e]) @ x64[t]
            a = g / (1 + np.exp(-g)) * u
            ref = float(w[t, r]) * dn[e].astype(np.float64) * np.abs(a)
            assert np.allclose(s[t, r * I:(r + 1) * I], ref, rtol=1e-6, atol=1e-30)


@pytest.mark.parametrize("keep", [0, 1, 7, 50, 96])
def test_select_matches_a_lexicographic_sort(keep):
    rng = np.random.default_rng(3)
    s = rng.random((6, 96)).astype(np.float32)
    s[1] = np.round(s[1] * 4) / 4          # many ties
    s[2] = 0.5                              # all tied
    kept = oracle.channel_select(s, keep)
    for t in range(s.shape[0]):
        assert np.array_equal(kept[t], brute_select(s[t], keep)), t


def test_kept_sets_are_nested():
    rng = np.random.default_rng(4)
    s = (np.round(rng.random((3, 64)) * 8) / 8).astype(np.float32)
    prev = oracle.channel_select(s, 0)
    for keep in range(1, 65):
        cur = oracle.channel_select(s, keep)
        assert (cur.sum(1) == keep).all() and not (prev & ~cur).any()
        prev = cur


def test_keeping_every_channel_is_the_full_layer():
    x, Wg, Wu, Wd, ids, w = routed_tiny()
    n = ids.shape[1] * Wg.shape[1]
    y_all = oracle.experts_kept(x, Wg, Wu, Wd, ids, w, np.ones((x.shape[0], n), bool))
    assert normwise(y_all, oracle.experts(x, Wg, Wu, Wd, ids, w)) < 1e-6


def test_keeping_no_channel_gives_zero():
    x, Wg, Wu, Wd, ids, w = routed_tiny()
    n = ids.shape[1] * Wg.shape[1]
    y = oracle.experts_kept(x, Wg, Wu, Wd, ids, w, np.zeros((x.shape[0], n), bool))
    assert not y.any()


def test_kept_layer_matches_numpy_masked_fp64():
    x, Wg, Wu, Wd, ids, w = routed_tiny(seed=2)
    dn = oracle.down_column_norms(Wd)
    s = oracle.channel_scores(x, Wg, Wu, ids, w, dn)
    kept = oracle.channel_select(s, 40)
    y = oracle.experts_kept(x, Wg, Wu, Wd, ids, w, kept)
    x64 = bf16_to_f64(x)
    T, k1 = ids.shape
    I = Wg.shape[1]
    ref = np.zeros((T, x.shape[1]))
    for t in range(T):
        for r in range(k1):
            e = ids[t, r]
            g = bf16_to_f64(Wg[e]) @ x64[t]
            u = bf16_to_f64(Wu[e]) @ x64[t]
            a = g / (1 + np.exp(-g)) * u * float(w[t, r])
            a = np.where(kept[t, r * I:(r + 1) * I], a, 0.0)
            ref[t] += bf16_to_f64(Wd[e]) @ a
    assert normwise(y, ref) < 1e-6
