"""moe_route on the GPU against the oracle's route: ids and Eq. 2 weights
bit for bit on identical logits ("Paper of the Week #3 - Half the FLOPs Is
Not Half the Time", section "The Receipt", Eq. 2; section "Ship It - Code of
the Week" for the softmax and the min(k2, E) ranking)."""
import numpy as np
import pytest
import torch

import decoupled_top_routing_amd as moe
from parity import check_route_exact

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run(logits_np, k1, k2):
    l = torch.from_numpy(np.ascontiguousarray(logits_np, np.float32)).to(DEV)
    ids, w = moe.route(l, k1, k2)
    torch.cuda.synchronize()
    return ids, w


PAIRS = {16: [(2, 4), (2, 2), (2, 16), (1, 1), (16, 16), (3, 40)],
         128: [(8, 8), (4, 4), (4, 16), (3, 16), (2, 16), (4, 128), (1, 200), (64, 100)],
         512: [(10, 10), (5, 5), (5, 20), (1, 512), (70, 80)]}


@pytest.mark.parametrize("E", sorted(PAIRS))
def test_route_random_logits(E):
    rng = np.random.default_rng(E)
    for T in (1, 8, 1000, 4099):
        l = (rng.standard_normal((T, E)) * 2).astype(np.float32)
        for k1, k2 in PAIRS[E]:
            print(f"E={E} T={T} k1={k1} k2={k2}", flush=True)
            ids, w = run(l, k1, k2)
            check_route_exact(ids, w, l, k1, k2, f"E={E} T={T} ({k1},{k2})")


@pytest.mark.parametrize("E", [1, 2, 3, 7, 33, 63, 64, 65, 100, 127, 129, 255, 256, 257,
                               511, 513, 1000, 1023, 1024])
def test_route_every_lane_layout(E):
    rng = np.random.default_rng(1000 + E)
    l = (rng.standard_normal((67, E)) * 3).astype(np.float32)
    for k1 in sorted({1, min(2, E), min(8, E), E}):
        for k2 in sorted({k1, min(k1 + 3, E), E, E + 5}):
            ids, w = run(l, k1, k2)
            check_route_exact(ids, w, l, k1, k2, f"E={E} ({k1},{k2})")


def test_route_ties_and_near_ties():
    """Tied probabilities resolve to the lower index; quantised logits make
    many exact ties, including across the k1 and k2 boundaries."""
    rng = np.random.default_rng(5)
    for E in (16, 128, 512, 1024):
        l = np.round(rng.standard_normal((512, E)) * 2).astype(np.float32)
        l[:64] = 0.0                                    # all equal
        l[64:128, ::2] = 1.0                            # half tied at the top
        for k1, k2 in ((1, 1), (2, 4), (4, 16), (8, 8), (5, 20), (70, 80), (3, 1000)):
            if k2 <= E:
                ids, w = run(l, k1, k2)
                check_route_exact(ids, w, l, k1, k2, f"ties E={E}")


def test_route_extreme_logits():
    """Large spreads: most probabilities underflow the -80 cut to exact 0."""
    rng = np.random.default_rng(6)
    for E in (16, 128, 1024):
        l = (rng.standard_normal((256, E)) * 60).astype(np.float32)
        l[:16] = np.linspace(-1e4, 1e4, E, dtype=np.float32)
        for k1, k2 in ((1, 2), (4, 16), (8, E)):
            ids, w = run(l, k1, min(k2, E) if k2 != E else E)
            check_route_exact(ids, w, l, k1, min(k2, E) if k2 != E else E, f"extreme E={E}")


def test_route_exp_sweep():
    """Logit rows (0, d_1, ..., d_127) make d = l - max = l exactly, so the
    weights with k1 = k2 = E expose exp(d)/S for d over a sample of every
    997th float in [-80, 0]; a difference in the GPU's exp shows up as a bit
    mismatch."""
    E = 128
    lo, hi = 0x80000000, 0xC2A00000
    d = np.arange(lo, hi, 997, dtype=np.uint64).astype(np.uint32).view(np.float32)
    rows = (d.size + E - 2) // (E - 1)
    l = np.zeros((rows, E), np.float32)
    flat = np.full(rows * (E - 1), -1.0, np.float32)
    flat[:d.size] = d
    l[:, 1:] = flat.reshape(rows, E - 1)
    ids, w = run(l, E, E)
    check_route_exact(ids, w, l, E, E, "exp sweep")


def test_route_zero_tokens():
    ids, w = run(np.zeros((0, 16), np.float32), 2, 4)
    assert ids.shape == (0, 2)


def test_route_is_deterministic():
    rng = np.random.default_rng(9)
    l = (rng.standard_normal((3000, 128)) * 2).astype(np.float32)
    a = run(l, 4, 16)
    b = run(l, 4, 16)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))
