"""The prefill path (bf16 MFMA router and grouped expert GEMMs) against the
oracle, at the 4096-token prefill workload and at small shapes that force it
through partial tiles, ragged tails and many experts."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import decoupled_top_routing_amd as moe
from decoupled_top_routing_amd import synth
from parity import DEV, host_layer, run_and_check, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def prefill():
    L = to_dev(synth.make_layer(synth.PREFILL))
    return L, host_layer(L)


@pytest.mark.parametrize("k1,k2", synth.PREFILL.k_pairs)
def test_prefill_4096(prefill, k1, k2):
    """The default path at 4096 tokens is the prefill path; y is checked on
    every token (every row of the plan's permutation and every M tile)."""
    L, Lh = prefill
    _, _, n = run_and_check(synth.PREFILL, L, Lh, k1, k2)
    assert n == 4096


@pytest.mark.parametrize("T", [1, 63, 300])
@pytest.mark.parametrize("flags", [moe.FORCE_PREFILL, moe.FORCE_GROUPED])
def test_prefill_against_grouped_shapes(prefill, T, flags):
    """Both expert paths on batches below and past one M tile, with bias."""
    L, Lh = prefill
    run_and_check(synth.PREFILL, dict(L, x=L["x"][:T]), dict(Lh, x=Lh["x"][:T]), 4, 16,
                  flags=flags)


def test_prefill_plan_beyond_lds_staging(prefill):
    """4096 tokens at k1 = 9 are 36864 assignments, more than the 32768 the
    plan kernel stages in LDS: its list is then scattered straight to global
    memory (8:8 at 4096 tokens, exactly 32768, takes the staged branch)."""
    L, Lh = prefill
    _, _, n = run_and_check(synth.PREFILL, L, Lh, 9, 12)
    assert n == 4096


def test_prefill_deterministic(prefill):
    """The plan's scatter order varies from call to call; the output may not."""
    L, _ = prefill
    x = L["x"][:1000]
    outs = [moe.forward(x, L["Wr"], L["Wg"], L["Wu"], L["Wd"], 8, 8, br=L["br"],
                        return_route=True, flags=moe.FORCE_PREFILL) for _ in range(2)]
    for u, v in zip(*outs):
        assert torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u,
                           v.view(torch.int16) if v.dtype == torch.bfloat16 else v)


BF16_SMALL = replace(synth.TINY, dtype="bf16", rms_norm_x=True, router_var_times_H=4.0)


@pytest.mark.parametrize("E,k1,k2,H,I,T", [
    (1, 1, 1, 128, 64, 1),         # one expert, one token
    (8, 8, 8, 128, 64, 130),       # dense: every expert gets 130 rows (ragged 2nd tile)
    (16, 2, 4, 256, 64, 64),
    (33, 5, 9, 1024, 192, 257),    # E not a multiple of the router tile
    (512, 10, 20, 512, 128, 40),   # hundreds of experts with one partial tile each
    (1024, 2, 7, 128, 64, 9),      # the most experts (wave route)
])
def test_prefill_edge_shapes(E, k1, k2, H, I, T):
    cfg = replace(BF16_SMALL, name=f"pf-E{E}-H{H}-I{I}", T=T, H=H, E=E, I=I, bias_std=0.5)
    L = synth.make_layer(cfg)
    run_and_check(cfg, L, host_layer(L), k1, k2, flags=moe.FORCE_PREFILL)


def test_prefill_rejects_unsupported_shapes():
    cfg = replace(BF16_SMALL, H=136, I=64)
    L = to_dev(synth.make_layer(cfg))
    with pytest.raises(moe.MoeError):
        moe.forward(L["x"], L["Wr"], L["Wg"], L["Wu"], L["Wd"], 2, 4, flags=moe.FORCE_PREFILL)
    f = to_dev(synth.make_layer(synth.TINY))
    with pytest.raises(moe.MoeError):
        moe.forward(f["x"], f["Wr"], f["Wg"], f["Wu"], f["Wd"], 2, 4, flags=moe.FORCE_PREFILL)
