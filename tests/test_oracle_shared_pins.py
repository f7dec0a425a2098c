"""Pins of the oracle's shared expert: a gated MLP that always runs beside the
routed experts ("Channel Selection for Mixture-of-Experts Decoding Needs No
Calibration Data", appendix B "Experimental setup"), added to the routed sum
with the factor sigmoid(x . sg), or 1 without a gate vector (the reading
taken; the pages do not give the gating).

Checks against numpy fp64, against the oracle's routed-expert code on the
same channels split into experts (a channel owns one gate row, one up row and
one down column, so a wide MLP is the sum of narrower ones: the same page,
section 2 "Background"), and closed forms of the gate.  No GPU.
"""
import numpy as np
import pytest
import torch

import oracle
from decoupled_top_routing_amd import synth
from test_oracle_pins import bf16_to_f64, np_swiglu_expert, normwise


def shared_weights(T=5, H=64, Is=96, bf16=False, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    Sg = (rng.standard_normal((Is, H)) * 0.1).astype(np.float32)
    Su = (rng.standard_normal((Is, H)) * 0.1).astype(np.float32)
    Sd = (rng.standard_normal((H, Is)) * 0.1).astype(np.float32)
    sg = (rng.standard_normal(H) / np.sqrt(H)).astype(np.float32)
    if bf16:
        def cvt(a):
            return synth.to_numpy(torch.from_numpy(a).to(torch.bfloat16))
        x, Sg, Su, Sd = cvt(x), cvt(Sg), cvt(Su), cvt(Sd)
    return x, Sg, Su, Sd, sg


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("gated", [False, True])
def test_shared_matches_numpy_fp64(bf16, gated):
    x, Sg, Su, Sd, sg = shared_weights(bf16=bf16)
    ys = oracle.shared(x, Sg, Su, Sd, sg if gated else None)
    x64 = bf16_to_f64(x)
    ref = np_swiglu_expert(x64, bf16_to_f64(Sg), bf16_to_f64(Su), bf16_to_f64(Sd))
    if gated:
        ref = ref / (1.0 + np.exp(-(x64 @ sg.astype(np.float64))))[:, None]
    assert normwise(ys, ref) < 1e-6


def test_shared_is_the_sum_of_its_channel_blocks():
    """Is = 3 * I channels equal three experts of I channels each with weight 1,
    computed by the oracle's routed-expert code."""
    I = 32
    x, Sg, Su, Sd, _ = shared_weights(Is=3 * I)
    ys = oracle.shared(x, Sg, Su, Sd)
    Wg = np.stack([Sg[j * I:(j + 1) * I] for j in range(3)])
    Wu = np.stack([Su[j * I:(j + 1) * I] for j in range(3)])
    Wd = np.stack([np.ascontiguousarray(Sd[:, j * I:(j + 1) * I]) for j in range(3)])
    T = x.shape[0]
    ids = np.tile(np.arange(3, dtype=np.int32), (T, 1))
    w = np.ones((T, 3), np.float32)
    ref = oracle.experts(x, Wg, Wu, Wd, ids, w)
    assert normwise(ys, ref) < 1e-6


def test_zero_gate_vector_halves_the_expert():
    x, Sg, Su, Sd, sg = shared_weights()
    half = oracle.shared(x, Sg, Su, Sd, np.zeros_like(sg))
    full = oracle.shared(x, Sg, Su, Sd)
    assert np.array_equal(half, full * np.float32(0.5))


def test_saturated_gate_is_one_or_zero():
    x, Sg, Su, Sd, _ = shared_weights(T=1)
    x64 = x[0].astype(np.float64)
    on = (x64 / (x64 @ x64) * 60.0).astype(np.float32)     # x . sg = 60
    full = oracle.shared(x, Sg, Su, Sd)
    assert np.array_equal(oracle.shared(x, Sg, Su, Sd, on), full)
    off = oracle.shared(x, Sg, Su, Sd, -on)                 # sigmoid(-60) ~ 1e-26
    assert np.abs(off).max() <= 1e-20 * np.abs(full).max()


def test_shared_tokens_are_independent():
    x, Sg, Su, Sd, sg = shared_weights(T=6)
    ys = oracle.shared(x, Sg, Su, Sd, sg, nthreads=4)
    for t in range(x.shape[0]):
        assert np.array_equal(oracle.shared(x[t:t + 1], Sg, Su, Sd, sg)[0], ys[t])
