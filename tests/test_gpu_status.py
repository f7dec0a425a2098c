"""The device status word of a workspace (moe_workspace_status).

The one-token kernel's workgroups hand the route over through tagged words,
and the router + route launch of 2..64 tokens makes its route blocks wait
for every token's logits; every wait is bounded.  The test hook
moe_debug_withhold_route keeps a call's hand-over from happening, so every
wait for it gives up after a few re-reads: the kernels still run to the end
(reading only in-range expert rows), and the status call must report
MOE_EDEVICE once, then reset.  Calls after it must be exact again.
"""
import os
import subprocess
import sys
from pathlib import Path

import pytest
import torch

import decoupled_top_routing_amd as moe
from decoupled_top_routing_amd import synth
from parity import DEV, host_layer, run_and_check, to_dev

pytestmark = pytest.mark.gpu

ROOT = Path(__file__).resolve().parents[1]


@pytest.fixture(scope="module")
def tiny():
    L = synth.make_layer(synth.TINY)
    return to_dev(L), host_layer(L)


def one_token(g, ws):
    return moe.forward(g["x"][:1], g["Wr"], g["Wg"], g["Wu"], g["Wd"], 2, 4, br=g["br"],
                       workspace=ws, return_route=True)


def test_status_is_clear_after_normal_calls(tiny):
    g, _ = tiny
    ws = torch.zeros(8 << 20, dtype=torch.uint8, device=DEV)
    for _ in range(3):
        one_token(g, ws)
    moe.workspace_status(ws)          # raises on MOE_EDEVICE


@pytest.fixture(scope="module")
def a3b():
    L = synth.make_layer(synth.DECODE_B1, T=32)
    return to_dev(L), host_layer(L)


# (layer, tokens): one token runs the one-token kernel; 8 and 32 tokens run
# the router + route launch (8 x 4 assignments without a plan, 32 x 4 with one)
@pytest.mark.parametrize("layer,T", [("tiny", 1), ("tiny", 8), ("a3b", 1), ("a3b", 8),
                                     ("a3b", 32)])
def test_withheld_route_is_reported_once(tiny, a3b, layer, T):
    if layer == "tiny":
        g, Lh = tiny
        cfg, k1, k2 = synth.TINY, 2, 4
    else:
        g, Lh = a3b
        cfg, k1, k2 = synth.DECODE_B1, 4, 16
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    x1 = g["x"][:T]
    args = (x1, g["Wr"], g["Wg"], g["Wu"], g["Wd"], k1, k2)
    y0 = moe.forward(*args, br=g["br"], workspace=ws)
    moe.workspace_status(ws)
    print(f"{cfg.name} T={T}: withholding the route of one call", flush=True)
    moe.debug_withhold_route(1, 64)
    moe.forward(*args, br=g["br"], workspace=ws)
    with pytest.raises(moe.MoeError) as ei:
        moe.workspace_status(ws)
    assert ei.value.code == 6
    moe.workspace_status(ws)          # the status was reset by the read
    # the next calls are exact again, and equal to the call before the hook
    y1 = moe.forward(*args, br=g["br"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16) if y0.dtype == torch.bfloat16 else y0,
                       y1.view(torch.int16) if y1.dtype == torch.bfloat16 else y1)
    moe.workspace_status(ws)
    Lt = dict(g, x=g["x"][:T])
    Lht = dict(Lh, x=Lh["x"][:T])
    run_and_check(cfg, Lt, Lht, k1, k2)


def test_debug_environment_checks_every_call():
    """With MOE_DEBUG=1 a forward call that withheld its route returns
    MOE_EDEVICE itself (the library waits for the call and reads the word)."""
    script = r"""
import torch, decoupled_top_routing_amd as moe
from decoupled_top_routing_amd import synth
L = {k: (None if v is None else v.to("cuda:0")) for k, v in synth.make_layer(synth.TINY).items()}
a = (L["x"][:1], L["Wr"], L["Wg"], L["Wu"], L["Wd"], 2, 4)
moe.forward(*a, br=L["br"])
moe.debug_withhold_route(1, 64)
try:
    moe.forward(*a, br=L["br"])
    print("NO ERROR")
except moe.MoeError as e:
    print("CODE", e.code)
moe.forward(*a, br=L["br"])
print("AFTER OK", flush=True)
"""
    env = dict(os.environ, MOE_DEBUG="1", PYTHONPATH=str(ROOT))
    r = subprocess.run([sys.executable, "-c", script], env=env, capture_output=True, text=True,
                       timeout=300, cwd=str(ROOT))
    assert r.returncode == 0, r.stderr[-2000:]
    assert "CODE 6" in r.stdout and "AFTER OK" in r.stdout, r.stdout + r.stderr[-2000:]
