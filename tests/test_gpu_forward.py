"""moe_forward on the GPU against the CPU oracle.

For each workload: (i) the GPU's logits match the oracle's within 1e-5
normwise; (ii) the oracle's route on the GPU's own logits equals the GPU's ids
and weights bit for bit; (iii) y matches the oracle's experts and combine on
that route within the tolerance of the dtype; (iv) an independent oracle run
from x picks the same experts except on near-ties, which are counted, not
failed.
"""
import numpy as np
import pytest
import torch

import decoupled_top_routing_amd as moe
import oracle
from decoupled_top_routing_amd import synth
from parity import DEV, host_layer, run_and_check, to_dev

pytestmark = pytest.mark.gpu
@pytest.fixture(scope="module")
def tiny():
    L = synth.make_layer(synth.TINY)
    return L, host_layer(L)


PATHS = [0, moe.FORCE_GROUPED]


@pytest.mark.parametrize("k1,k2", synth.TINY.k_pairs)
@pytest.mark.parametrize("flags", PATHS)
def test_tiny_fp32(tiny, k1, k2, flags):
    L, Lh = tiny
    run_and_check(synth.TINY, L, Lh, k1, k2, flags)


@pytest.fixture(scope="module")
def a3b():
    L = synth.make_layer(synth.DECODE_B8)
    return L, host_layer(L)


@pytest.mark.parametrize("k1,k2", synth.DECODE_B1.k_pairs)
@pytest.mark.parametrize("T", [1, 8])
def test_a3b_decode(a3b, k1, k2, T):
    L, Lh = a3b
    Lt = dict(L, x=L["x"][:T])
    Lht = dict(Lh, x=Lh["x"][:T])
    cfg = synth.DECODE_B1 if T == 1 else synth.DECODE_B8
    run_and_check(cfg, Lt, Lht, k1, k2)


@pytest.mark.parametrize("flags", [moe.FORCE_GROUPED, moe.FORCE_PREFILL])
@pytest.mark.parametrize("k1,k2", [(8, 8), (4, 16)])
@pytest.mark.parametrize("T", [1, 8])
def test_a3b_decode_each_path(a3b, k1, k2, flags, T):
    L, Lh = a3b
    run_and_check(synth.DECODE_B8, dict(L, x=L["x"][:T]), dict(Lh, x=Lh["x"][:T]), k1, k2, flags)


def test_a3b_workspace_reuse_across_shapes(a3b, tiny):
    """One workspace serves calls of different shapes and paths in a row; the
    synchronisation words must be back at zero after every call, and each of
    these calls (every one hands values over as tagged words) advances the
    epoch that makes the call tags by exactly one."""
    L, Lh = a3b
    tL, tLh = tiny
    g, tg = to_dev(L), to_dev(tL)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    ref = {}
    epoch = 0
    for rep in range(3):
        for name, (lay, T, k1, k2, fl) in {
                "a": (g, 1, 4, 16, 0), "b": (tg, 8, 2, 4, 0), "c": (g, 8, 8, 8, 0),
                "d": (g, 5, 3, 16, moe.FORCE_GROUPED), "e": (tg, 3, 2, 16, 0)}.items():
            y = moe.forward(lay["x"][:T], lay["Wr"], lay["Wg"], lay["Wu"], lay["Wd"], k1, k2,
                            br=lay["br"], flags=fl, workspace=ws)
            torch.cuda.synchronize()
            words = ws[:16384].view(torch.int32).cpu().clone()
            # word 0 is the workspace's epoch; every counter and the error
            # word must be back at zero
            assert int(words[0]) == epoch + 1, name
            epoch = int(words[0])
            assert int(words[1:].abs().sum()) == 0, f"sync words left set ({name})"
            yb = y.float().cpu()
            if rep == 0:
                ref[name] = yb
            else:
                assert torch.equal(ref[name], yb), name


def test_a3b_ragged_batches(a3b):
    L, Lh = a3b
    for T in (2, 3, 5, 7):
        Lt = dict(L, x=L["x"][:T])
        run_and_check(synth.DECODE_B8, Lt, dict(Lh, x=Lh["x"][:T]), 4, 16)


def test_a3b_ids_do_not_depend_on_k2(a3b):
    """P1, The Receipt: k2 changes the weights, never the experts."""
    L, _ = a3b
    g = to_dev(L)
    ref = None
    for k2 in (4, 8, 16, 64, 128):
        _, _, ids, _ = moe.forward(g["x"], g["Wr"], g["Wg"], g["Wu"], g["Wd"], 4, k2,
                                   return_route=True)
        if ref is None:
            ref = ids
        assert torch.equal(ids, ref)


def test_forward_is_deterministic(a3b):
    L, _ = a3b
    g = to_dev(L)
    a = moe.forward(g["x"], g["Wr"], g["Wg"], g["Wu"], g["Wd"], 4, 16, return_route=True)
    b = moe.forward(g["x"], g["Wr"], g["Wg"], g["Wu"], g["Wd"], 4, 16, return_route=True)
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u,
                           v.view(torch.int16) if v.dtype == torch.bfloat16 else v)


def test_zero_tokens(a3b):
    L, _ = a3b
    g = to_dev(L)
    y = moe.forward(g["x"][:0], g["Wr"], g["Wg"], g["Wu"], g["Wd"], 4, 16)
    assert y.shape == (0, synth.DECODE_B1.H)


@pytest.mark.parametrize("E,k1,k2,H,I,T", [
    (1, 1, 1, 8, 8, 3),        # one expert, smallest sizes
    (8, 8, 8, 64, 16, 5),      # every expert active: the dense mixture
    (16, 3, 40, 136, 24, 17),  # k2 > E, ragged sizes
    (1024, 2, 7, 64, 8, 9),    # the most experts
    (16, 2, 4, 256, 64, 64),   # 64 tokens: the route kernel's in-kernel plan limit
    (16, 2, 4, 256, 64, 65),   # the smallest batch past it
    (512, 10, 20, 512, 136, 40),  # many unique experts, down rows of 34 chunks
    (33, 5, 9, 1024, 64, 13),  # router rows of 4 chunks per lane
    (1024, 3, 9, 1024, 64, 20),  # a router block per expert for the most experts, two token groups
])
def test_edge_shapes_fp32(E, k1, k2, H, I, T):
    from dataclasses import replace
    cfg = replace(synth.TINY, name=f"edge-E{E}", T=T, H=H, E=E, I=I)
    L = synth.make_layer(cfg)
    run_and_check(cfg, L, host_layer(L), k1, k2)


@pytest.mark.parametrize("E,k1,k2,H,I,dtype", [
    (1, 1, 1, 256, 64, "f32"),        # one expert: p = 1, w = 1
    (1024, 2, 7, 256, 64, "f32"),     # the most experts: the route block's one-wave route
    (300, 32, 64, 256, 64, "f32"),    # the most slots (k1 = 32): down rounds of 8
    (33, 5, 9, 512, 72, "f32"),       # E and I not multiples of the tiles
    (1024, 4, 16, 512, 64, "bf16"),   # bf16, the most experts
    (128, 8, 8, 2048, 768, "bf16"),   # a full-size expert at 8:8
    (1024, 4, 16, 1024, 64, "f32"),   # a router block per expert (rows of 4 chunks per lane), the most experts
    (256, 6, 24, 4096, 128, "bf16"),  # router rows of 16 chunks per lane, a quarter per wave
])
def test_one_launch_limits(E, k1, k2, H, I, dtype):
    """One token on the single-launch kernel at the edges of the shapes it takes."""
    from dataclasses import replace
    cfg = replace(synth.TINY, name=f"b1-E{E}-k{k1}", T=1, H=H, E=E, I=I, dtype=dtype,
                  rms_norm_x=dtype == "bf16", router_var_times_H=4.0 if dtype == "bf16" else 1.0)
    L = synth.make_layer(cfg)
    g = to_dev(L)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    moe.profile_launch(0, ev[0], ev[1])
    moe.forward(g["x"], g["Wr"], g["Wg"], g["Wu"], g["Wd"], k1, k2)
    torch.cuda.synchronize()
    assert moe.profile_launch_name() == "b1_layer"
    run_and_check(cfg, g, host_layer(L), k1, k2)
