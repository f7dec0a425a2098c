"""Pins of the oracle's bf16 router: the router method of "Paper of the Week #3
- Half the FLOPs Is Not Half the Time" (section "Ship It - Code of the Week")
as it runs on a bf16 model -- the linear layer in bf16, the softmax upcast to
fp32, the weights cast back to bf16.  At k1 = k2 that method is the stock
renormalising router, cast included (section "The Receipt": bit-identical to
stock at k1 = k2 = 8).

Each test checks the oracle against something other than itself: torch's
fp32 -> bf16 cast (a library routine), exact rational arithmetic, numpy fp64
matmuls, and an independently written stock router.  None touches the GPU.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from test_oracle_pins import bf16_to_f64, normwise, numpy_layer_fp64


def torch_bf16(a):
    """float32 array -> float32 array of torch's bf16 cast of it."""
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def bf16_bits(a):
    """float32 array -> uint16 bf16 bit patterns (values must be bf16 already)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    assert not (u & 0xFFFF).any()
    return (u >> 16).astype(np.uint16)


def random_bf16(shape, std, seed):
    rng = np.random.default_rng(seed)
    return bf16_bits(torch_bf16(rng.standard_normal(shape).astype(np.float32) * std))


# ---------------------------------------------------------------- rounding

def test_round_bf16_matches_torch_cast_from_fp32():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    low = np.array([0x8000, 0x7FFF, 0x8001, 0x0000], np.uint32)
    n = 80000  # ties, just below, just above, exact
    bits[:n] = (bits[:n] & 0xFFFF0000) | low[np.arange(n) % 4]
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    got = oracle.round_bf16(f.astype(np.float64))
    assert np.array_equal(got.view(np.uint32), torch_bf16(f).view(np.uint32))


def _bf16_neighbours(g):
    """The bf16 values just below and above the bf16 value g (float)."""
    b = int(np.float32(g).view(np.uint32)) >> 16
    out = []
    for nb in (b - 1, b + 1):
        if 0 <= nb <= 0xFFFF:
            v = np.uint32(nb << 16).view(np.float32)
            if np.isfinite(v):
                out.append(float(v))
    return out


def test_round_bf16_of_doubles_is_nearest_with_ties_to_even():
    rng = np.random.default_rng(8)
    n = 3000
    wide = rng.standard_normal(n) * 10.0 ** rng.integers(-30, 30, n)
    tiny = rng.uniform(-1, 1, 500) * 2.0 ** -124  # around the smallest normal
    # exact midpoints between neighbouring bf16 values
    b = rng.integers(0x0001, 0x7F7F, 1000).astype(np.uint32)
    lo = (b << 16).view(np.float32).astype(np.float64)
    hi = ((b + 1) << 16).view(np.float32).astype(np.float64)
    mids = (lo + hi) / 2 * np.where(rng.random(1000) < 0.5, -1.0, 1.0)
    d = np.concatenate([wide, tiny, mids])
    got = oracle.round_bf16(d)
    for di, gi in zip(d, got):
        assert (int(np.float32(gi).view(np.uint32)) & 0xFFFF) == 0
        dist = abs(Fraction(float(di)) - Fraction(float(gi)))
        for nb in _bf16_neighbours(gi):
            dn = abs(Fraction(float(di)) - Fraction(nb))
            assert dist <= dn, (di, gi, nb)
            if dist == dn:  # a tie: the even bf16 mantissa wins
                assert ((int(np.float32(gi).view(np.uint32)) >> 16) & 1) == 0, (di, gi)


# ---------------------------------------------------------------- logits

def test_bf16_logits_are_the_exact_dot_product_rounded_once():
    x = random_bf16((16, 256), 1.0, 1)
    Wr = random_bf16((64, 256), 256 ** -0.5, 2)
    lg = oracle.logits_bf16(x, Wr)
    exact = bf16_to_f64(x) @ bf16_to_f64(Wr).T  # bf16 products and their sum: exact in fp64
    f32 = exact.astype(np.float32)
    ref = torch_bf16(f32)
    # where the fp32 value lies exactly on a bf16 midpoint, rounding twice
    # (fp64 -> fp32 -> bf16) may differ from rounding once: excluded
    amb = (f32.view(np.uint32) & 0xFFFF) == 0x8000
    assert np.array_equal(lg[~amb].view(np.uint32), ref[~amb].view(np.uint32))
    # torch's own bf16 linear (its accumulation order) within one bf16 step
    tl = torch.nn.functional.linear(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16),
                                    torch.from_numpy(Wr.view(np.int16)).view(torch.bfloat16))
    tl = tl.float().numpy()
    assert np.all(np.abs(lg.astype(np.float64) - tl) <= np.abs(tl) * 2.0 ** -7 + 1e-30)


# ---------------------------------------------------------------- route

def stock_router(p_row, k):
    """The stock renormalising router, written independently: the k most
    probable experts (lower index first on equal p), each p over their
    left-to-right fp32 sum, then cast to bf16."""
    order = sorted(range(len(p_row)), key=lambda e: (-float(p_row[e]), e))[:k]
    vals = [np.float32(p_row[e]) for e in order]
    s = np.float32(0.0)
    for v in vals:
        s = np.float32(s + v)
    w = np.array([np.float32(v / s) for v in vals], np.float32)
    return np.array(order, np.int32), torch_bf16(w)


def bf16_logit_rows(T, E, seed):
    """Logits that are bf16 values (ties between experts are common)."""
    rng = np.random.default_rng(seed)
    lg = torch_bf16((rng.standard_normal((T, E)) * 2.0).astype(np.float32))
    lg[0, :] = lg[0, 0]          # every expert tied
    lg[1, 3::7] = lg[1, 5]        # a block of ties
    return lg


@pytest.mark.parametrize("E,k", [(128, 8), (128, 4), (16, 2), (64, 1)])
def test_bf16_router_at_k1_eq_k2_is_stock_bitwise(E, k):
    lg = bf16_logit_rows(48, E, 3)
    p = oracle.softmax(lg)
    ids, w = oracle.route_bf16w(lg, k, k)
    for t in range(lg.shape[0]):
        sid, sw = stock_router(p[t], k)
        assert np.array_equal(ids[t], sid), t
        assert np.array_equal(w[t].view(np.uint32), sw.view(np.uint32)), t


@pytest.mark.parametrize("k1,k2", [(4, 16), (2, 16), (4, 128), (8, 8), (3, 200)])
def test_bf16_router_weights_are_the_fp32_weights_cast(k1, k2):
    lg = bf16_logit_rows(48, 128, 4)
    ids_h, w_h = oracle.route_bf16w(lg, k1, k2)
    ids, w = oracle.route(lg, k1, k2)
    assert np.array_equal(ids_h, ids)
    assert np.array_equal(w_h.view(np.uint32), torch_bf16(w).view(np.uint32))


def test_bf16_router_layer_matches_numpy_fp64():
    T, H, E, I = 6, 64, 8, 32
    x = random_bf16((T, H), 1.0, 5)
    Wr = random_bf16((E, H), H ** -0.5 * 2, 6)
    Wg, Wu = random_bf16((E, I, H), 0.1, 7), random_bf16((E, I, H), 0.1, 8)
    Wd = random_bf16((E, H, I), 0.1, 9)
    for k1, k2 in ((2, 4), (3, 3), (2, 8)):
        y, lg, ids, w = oracle.forward_bf16_router(x, Wr, Wg, Wu, Wd, k1, k2)
        assert np.array_equal(lg, oracle.logits_bf16(x, Wr))
        ids2, w2 = oracle.route_bf16w(lg, k1, k2)
        assert np.array_equal(ids, ids2) and np.array_equal(w, w2)
        assert not (w.view(np.uint32) & 0xFFFF).any()
        assert normwise(y, numpy_layer_fp64(x, None, None, Wg, Wu, Wd, ids, w)) < 1e-6
