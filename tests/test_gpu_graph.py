"""Every path under HIP graph capture: one call captured with a caller-owned
workspace and output, replayed several times with other eager calls in
between, each replay equal bit for bit to the eager result.  The library
records no memset and allocates nothing per call, so its launches are the
graph's only nodes."""
import pytest
import torch

import decoupled_top_routing_amd as moe
from decoupled_top_routing_amd import synth
from parity import to_dev

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.fixture(scope="module")
def a3b():
    L = to_dev(synth.make_layer(synth.DECODE_B8))
    S = {k: (None if v is None else v.cuda())
         for k, v in synth.make_shared(synth.DECODE_B8, 768, gate=True).items()}
    return L, S


def run_case(call, x, ws_bytes):
    """call(x, out, ws) enqueues one layer call on the current stream."""
    dev = x.device
    stream = torch.cuda.Stream(device=dev)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    ws_other = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty_like(x)
    other = torch.empty_like(x)
    torch.cuda.synchronize()  # inputs made on the default stream are complete
    with torch.cuda.stream(stream):
        call(x, out, ws)
        torch.cuda.synchronize()
        ref = out.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            call(x, out, ws)
        for rep in range(4):
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(bits(out), bits(ref)), f"replay {rep} differs from eager"
            # eager work between replays, on its own workspace
            call(x.flip(0).contiguous(), other, ws_other)
            torch.cuda.synchronize()
    del g


def ws_size(T, k1, Is=0):
    lib = moe.load_library()
    c = synth.DECODE_B8
    return lib.moe_forward_shared_workspace(T, c.H, c.E, c.I, k1, Is, 1, 1)


@pytest.mark.parametrize("T,flags", [(1, 0), (8, 0), (8, moe.FORCE_GROUPED), (1, moe.FORCE_GROUPED)])
def test_graph_routed(a3b, T, flags):
    L, _ = a3b
    run_case(lambda x, out, ws: moe.forward(x, L["Wr"], L["Wg"], L["Wu"], L["Wd"], 4, 16,
                                            flags=flags, out=out, workspace=ws),
             L["x"][:T].contiguous(), ws_size(T, 4))


def test_graph_prefill(a3b):
    L, _ = a3b
    x = torch.cat([L["x"]] * 75)[:600].contiguous()
    run_case(lambda x, out, ws: moe.forward(x, L["Wr"], L["Wg"], L["Wu"], L["Wd"], 8, 8,
                                            flags=moe.FORCE_PREFILL, out=out, workspace=ws),
             x, ws_size(600, 8))


@pytest.mark.parametrize("T", [1, 8])
def test_graph_bf16_router(a3b, T):
    L, _ = a3b
    Wr = L["Wr"].to(torch.bfloat16)
    run_case(lambda x, out, ws: moe.forward(x, Wr, L["Wg"], L["Wu"], L["Wd"], 4, 16, out=out,
                                            workspace=ws),
             L["x"][:T].contiguous(), ws_size(T, 4))


@pytest.mark.parametrize("T", [1, 8])
def test_graph_shared(a3b, T):
    L, S = a3b
    sh = (S["Sg"], S["Su"], S["Sd"], S["sg"])
    run_case(lambda x, out, ws: moe.forward(x, L["Wr"], L["Wg"], L["Wu"], L["Wd"], 4, 16,
                                            shared=sh, out=out, workspace=ws),
             L["x"][:T].contiguous(), ws_size(T, 4, 768))


def test_graph_channel_topk(a3b):
    L, _ = a3b
    dn = moe.down_column_norms(L["Wd"])
    run_case(lambda x, out, ws: moe.forward_channel_topk(x, L["Wr"], L["Wg"], L["Wu"], L["Wd"],
                                                         4, 16, dn, 553, out=out, workspace=ws),
             L["x"][:8].contiguous(), ws_size(8, 4))
