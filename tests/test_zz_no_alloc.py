"""moe_forward_noalloc (the library's fixed device scratch in place of a
workspace) against moe_forward with a caller's workspace, through the C ABI.

Both run the same kernels, so the route (logits, ids, weights) and y must be
identical bit for bit.  Each case makes two calls of the no-allocation entry
point in a row, the second with a smaller input, so the second finds the
first one's contents in the shared array.  Sizes past the array are refused
before anything is launched.
"""
import pytest
import torch

import decoupled_top_routing_amd as moe
from decoupled_top_routing_amd import synth
from parity import DEV, to_dev

pytestmark = pytest.mark.gpu


def same(a, b):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


def check_pair(g, T, k1, k2, flags=0):
    x = g["x"][:T].contiguous()
    args = (x, g["Wr"], g["Wg"], g["Wu"], g["Wd"], k1, k2)
    ref = moe.forward(*args, br=g["br"], return_route=True, flags=flags,
                      workspace=torch.zeros(64 << 20, dtype=torch.uint8, device=DEV))
    got = moe.forward(*args, br=g["br"], return_route=True, flags=flags, noalloc=True)
    torch.cuda.synchronize()
    for name, a, b in zip(("y", "logits", "ids", "w"), ref, got):
        assert same(a, b), f"T={T} {k1}:{k2}: {name} differs from moe_forward"


@pytest.fixture(scope="module")
def a3b():
    return to_dev(synth.make_layer(synth.DECODE_B8, T=300))


@pytest.fixture(scope="module")
def tiny():
    return to_dev(synth.make_layer(synth.TINY))


@pytest.mark.parametrize("Ts,k1,k2", [
    ((300, 8, 1), 4, 16),     # prefill path, then grouped, then the one-launch kernel
    ((8, 1), 8, 8),           # grouped, then one token
    ((2, 1), 4, 128),         # k2 >= E
])
def test_noalloc_matches_forward_a3b(a3b, Ts, k1, k2):
    for T in Ts:
        print(f"noalloc a3b T={T} {k1}:{k2}", flush=True)
        check_pair(a3b, T, k1, k2)


@pytest.mark.parametrize("Ts,k1,k2", [((8, 3), 2, 4), ((5, 1), 2, 16)])
def test_noalloc_matches_forward_tiny(tiny, Ts, k1, k2):
    for T in Ts:
        print(f"noalloc tiny T={T} {k1}:{k2}", flush=True)
        check_pair(tiny, T, k1, k2)


def test_noalloc_forced_grouped_one_token(a3b):
    check_pair(a3b, 4, 4, 16, flags=moe.FORCE_GROUPED)
    check_pair(a3b, 1, 4, 16, flags=moe.FORCE_GROUPED)


def test_noalloc_refuses_sizes_past_its_array(a3b):
    lib = moe.load_library()
    cap = lib.moe_noalloc_scratch_bytes()
    T = 4096
    assert lib.moe_forward_workspace(T, 2048, 128, 768, 8, 1, 1) > cap
    big = torch.zeros((T, 2048), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.forward(big, a3b["Wr"], a3b["Wg"], a3b["Wu"], a3b["Wd"], 8, 8, noalloc=True)
    assert ei.value.code == 3
    # and a normal call afterwards is still exact
    check_pair(a3b, 1, 4, 16)
