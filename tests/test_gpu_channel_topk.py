"""Channel top-k inside the activated experts on the GPU against the oracle.

"Channel Selection for Mixture-of-Experts Decoding Needs No Calibration Data",
section 5.2: each channel of a token's activated experts is scored by router
weight x down-column norm x |activation|; the exact top-keep over the token's
k1*I channels are kept.  Checks: (i) the down-column norms and the scores
match the oracle's within fp32 accumulation error; (ii) the oracle's
selection on the GPU's own scores equals the GPU's kept set exactly (integer
work); (iii) y equals the oracle's kept-channel sum on that set within the
dtype's tolerance; (iv) the oracle's independent selection differs only on
channels whose scores lie at the selection boundary; (v) keeping every
channel reproduces the full layer.  Every case runs twice: with the column
copy of the down weights (the down projection reads only the kept columns)
and without it (unkept activations zeroed, every down row read).
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import decoupled_top_routing_amd as moe
import oracle
from decoupled_top_routing_amd import synth
from parity import (TOL_BF16, TOL_F32, check_route_exact, host_layer, normwise_err, to_dev,
                    to_f64)

pytestmark = pytest.mark.gpu


_COLS = {}


def cols_of(Wd):
    """The column copy of a layer's down weights, made once per tensor."""
    key = Wd.data_ptr()
    if key not in _COLS:
        _COLS[key] = (Wd, moe.down_columns(Wd))
    return _COLS[key][1]


def check_topk(cfg, L, Lh, k1, k2, keep, flags=0, bf16_router=False, cols=True):
    g = to_dev(L) if L["Wg"].device.type == "cpu" else L
    T = g["x"].shape[0]
    print(f"{cfg.name} T={T} k1={k1} k2={k2} keep={keep} flags={flags} "
          f"bf16_router={bf16_router} cols={cols}", flush=True)
    Wr = g["Wr"].to(torch.bfloat16) if bf16_router else g["Wr"]
    br = None if bf16_router else g["br"]
    dn = moe.down_column_norms(g["Wd"])
    y, lg, ids, w, sc, kept = moe.forward_channel_topk(
        g["x"], Wr, g["Wg"], g["Wu"], g["Wd"], k1, k2, dn, keep, br=br, return_route=True,
        flags=flags, Wdown_cols=cols_of(g["Wd"]) if cols else None)
    torch.cuda.synchronize()
    dn_ref = oracle.down_column_norms(Lh["Wd"])
    assert np.allclose(dn.cpu().numpy(), dn_ref, rtol=2e-5, atol=0)
    lg_h = lg.cpu().numpy()
    if bf16_router:
        oids, ow = oracle.route_bf16w(lg_h, k1, k2)
        assert np.array_equal(oids, ids.cpu().numpy())
        assert np.array_equal(ow.view(np.int32), w.cpu().numpy().view(np.int32))
    else:
        oids, ow = check_route_exact(ids, w, lg_h, k1, k2, cfg.name)
    x_h = Lh["x"]
    sc_h, kept_h = sc.cpu().numpy(), kept.cpu().numpy()
    sc_ref = oracle.channel_scores(x_h, Lh["Wg"], Lh["Wu"], oids, ow, dn_ref)
    # (i) scores, normwise per token
    assert normwise_err(sc_h, sc_ref) <= 1e-4
    # (ii) the selection on the GPU's scores, exactly
    assert np.array_equal(oracle.channel_select(sc_h, keep), kept_h)
    assert (kept_h.sum(1) == keep).all()
    # (iii) y on that selection
    y_ref = oracle.experts_kept(x_h, Lh["Wg"], Lh["Wu"], Lh["Wd"], oids, ow, kept_h)
    if keep == 0:
        assert not to_f64(y).any()
    else:
        tol = TOL_F32 if cfg.dtype == "f32" else TOL_BF16
        err = normwise_err(to_f64(y), y_ref)
        assert err <= tol, f"normwise error {err} > {tol}"
    # (iv) an independent selection differs only at the boundary
    if 0 < keep < sc_ref.shape[1]:
        ind = oracle.channel_select(sc_ref, keep)
        for t in range(T):
            diff = ind[t] != kept_h[t]
            if diff.any():
                kth = np.sort(sc_ref[t])[::-1][keep - 1]
                assert np.all(np.abs(sc_ref[t][diff] - kth) <= 1e-3 * kth), t
    return y


@pytest.fixture(scope="module")
def a3b():
    L = to_dev(synth.make_layer(synth.DECODE_B8))
    return L, host_layer(L)


@pytest.mark.parametrize("cols", [True, False])
@pytest.mark.parametrize("frac", [1.0, 0.18, 0.5])
@pytest.mark.parametrize("k1,k2", [(4, 16), (8, 8)])
@pytest.mark.parametrize("T", [1, 8])
def test_channel_topk_decode(a3b, T, k1, k2, frac, cols):
    L, Lh = a3b
    keep = int(round(frac * k1 * synth.DECODE_B8.I))
    check_topk(synth.DECODE_B8, dict(L, x=L["x"][:T]), dict(Lh, x=Lh["x"][:T]), k1, k2, keep,
               cols=cols)


@pytest.mark.parametrize("cols", [True, False])
@pytest.mark.parametrize("keep", [0, 1, 3])
def test_channel_topk_extremes(a3b, keep, cols):
    L, Lh = a3b
    check_topk(synth.DECODE_B8, dict(L, x=L["x"][:8]), dict(Lh, x=Lh["x"][:8]), 4, 16, keep,
               cols=cols)


def test_channel_topk_many_tokens():
    """64 tokens: few list groups per token (the one-token case has many)."""
    L = synth.make_layer(synth.DECODE_B8, T=64)
    check_topk(synth.DECODE_B8, L, host_layer(L), 8, 8, 1106)


def test_down_columns_is_the_transpose(a3b):
    L, _ = a3b
    Wd = L["Wd"]
    cols = moe.down_columns(Wd)
    torch.cuda.synchronize()
    assert torch.equal(cols.view(torch.int16), Wd.transpose(1, 2).contiguous().view(torch.int16))
    f = synth.make_layer(synth.TINY)["Wd"].cuda()
    assert torch.equal(moe.down_columns(f), f.transpose(1, 2).contiguous())


@pytest.mark.parametrize("cols", [True, False])
def test_keeping_every_channel_is_the_layer(a3b, cols):
    L, _ = a3b
    x = L["x"][:8]
    dn = moe.down_column_norms(L["Wd"])
    n = 4 * synth.DECODE_B8.I
    y_all = moe.forward_channel_topk(x, L["Wr"], L["Wg"], L["Wu"], L["Wd"], 4, 16, dn, n,
                                     Wdown_cols=cols_of(L["Wd"]) if cols else None)
    y = moe.forward(x, L["Wr"], L["Wg"], L["Wu"], L["Wd"], 4, 16, flags=moe.FORCE_GROUPED)
    assert normwise_err(to_f64(y_all), to_f64(y)) <= 1e-2


def test_channel_topk_with_bf16_router(a3b):
    L, Lh = a3b
    check_topk(synth.DECODE_B8, dict(L, x=L["x"][:8]), dict(Lh, x=Lh["x"][:8]), 4, 16, 553,
               bf16_router=True)


@pytest.mark.parametrize("cols", [True, False])
@pytest.mark.parametrize("keep", [128, 40, 1])
def test_channel_topk_fp32(keep, cols):
    cfg = synth.TINY
    L = synth.make_layer(cfg)
    check_topk(cfg, L, host_layer(L), 2, 4, keep, cols=cols)


@pytest.mark.parametrize("cols", [True, False])
def test_channel_topk_ragged_shape(cols):
    cfg = replace(synth.TINY, name="ck-E40-H264-I72", dtype="bf16", rms_norm_x=True,
                  router_var_times_H=4.0, T=5, H=264, E=40, I=72)
    L = synth.make_layer(cfg)
    check_topk(cfg, L, host_layer(L), 3, 7, 100, cols=cols)


@pytest.mark.parametrize("cols", [True, False])
def test_channel_topk_is_deterministic(a3b, cols):
    L, _ = a3b
    dn = moe.down_column_norms(L["Wd"])
    wc = cols_of(L["Wd"]) if cols else None
    outs = [moe.forward_channel_topk(L["x"][:8], L["Wr"], L["Wg"], L["Wu"], L["Wd"], 8, 8, dn,
                                     1106, return_route=True, Wdown_cols=wc) for _ in range(2)]
    for u, v in zip(*outs):
        assert torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u,
                           v.view(torch.int16) if v.dtype == torch.bfloat16 else v)


def test_channel_topk_rejects_unsupported(a3b):
    L, _ = a3b
    dn = moe.down_column_norms(L["Wd"])
    x = L["x"][:1]
    with pytest.raises(moe.MoeError):       # keep > k1*I
        moe.forward_channel_topk(x, L["Wr"], L["Wg"], L["Wu"], L["Wd"], 4, 16, dn, 4 * 768 + 1)
    with pytest.raises(moe.MoeError):       # grouped path only
        moe.forward_channel_topk(x, L["Wr"], L["Wg"], L["Wu"], L["Wd"], 4, 16, dn, 10,
                                 flags=moe.FORCE_PREFILL)
    with pytest.raises(moe.MoeError):       # k1*I > 8192
        moe.forward_channel_topk(x, L["Wr"], L["Wg"], L["Wu"], L["Wd"], 11, 16, dn, 10)
