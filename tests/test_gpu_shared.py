"""The shared expert (moe_forward_shared) on the GPU against the oracle.

A shared expert always runs beside the routed ones ("Channel Selection for
Mixture-of-Experts Decoding Needs No Calibration Data", appendix B); the
layer is y = (routed sum) + g * S(x) with g = sigmoid(x . sg) or 1.  For each
path: the route is unchanged and equals the oracle's route on the GPU's
logits bit for bit; y matches the oracle's routed experts on that route plus
the oracle's shared term, within the dtype's tolerance.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import decoupled_top_routing_amd as moe
import oracle
from decoupled_top_routing_amd import synth
from parity import (NTHREADS, TOL_BF16, TOL_F32, check_route_exact, host_layer, normwise_err,
                    to_dev, to_f64)

pytestmark = pytest.mark.gpu


def check_shared(cfg, L, Lh, S, k1, k2, flags=0, token_sample=None, bf16_router=False):
    g = to_dev(L) if L["Wg"].device.type == "cpu" else L
    Sd = {k: (None if v is None else v.to(g["x"].device)) for k, v in S.items()}
    Is = Sd["Sg"].shape[0]
    gated = Sd["sg"] is not None
    print(f"{cfg.name} T={g['x'].shape[0]} k1={k1} k2={k2} flags={flags} shared Is={Is} "
          f"gated={gated} bf16_router={bf16_router}", flush=True)
    Wr = g["Wr"].to(torch.bfloat16) if bf16_router else g["Wr"]
    br = None if bf16_router else g["br"]
    shared = (Sd["Sg"], Sd["Su"], Sd["Sd"]) + ((Sd["sg"],) if gated else ())
    y, lg, ids, w = moe.forward(g["x"], Wr, g["Wg"], g["Wu"], g["Wd"], k1, k2, br=br,
                                return_route=True, flags=flags, shared=shared)
    torch.cuda.synchronize()
    lg_h = lg.cpu().numpy()
    T = lg_h.shape[0]
    sel = np.arange(T) if token_sample is None else np.asarray(token_sample)
    if bf16_router:
        oids, ow = oracle.route_bf16w(lg_h, k1, k2)
        assert np.array_equal(oids, ids.cpu().numpy())
        assert np.array_equal(ow.view(np.int32), w.cpu().numpy().view(np.int32))
    else:
        oids, ow = check_route_exact(ids, w, lg_h, k1, k2, cfg.name)
    x_h = Lh["x"][sel]
    Sh = {k: synth.to_numpy(v) for k, v in S.items()}
    y_ref = oracle.experts(x_h, Lh["Wg"], Lh["Wu"], Lh["Wd"], oids[sel], ow[sel],
                           nthreads=NTHREADS)
    y_ref = y_ref.astype(np.float64) + oracle.shared(x_h, Sh["Sg"], Sh["Su"], Sh["Sd"],
                                                     Sh["sg"], nthreads=NTHREADS)
    err = normwise_err(to_f64(y)[sel], y_ref)
    tol = TOL_F32 if cfg.dtype == "f32" else TOL_BF16
    assert err <= tol, f"normwise error {err} > {tol}"
    check_shared.checked = len(sel)
    return y


@pytest.fixture(scope="module")
def a3b():
    L = to_dev(synth.make_layer(synth.DECODE_B8))
    return L, host_layer(L)


def shared_of(cfg, Is, gate):
    return synth.make_shared(cfg, Is, gate=gate)


@pytest.mark.parametrize("Is,gate", [(768, True), (768, False), (1536, True), (512, True)])
@pytest.mark.parametrize("k1,k2", [(4, 16), (8, 8)])
def test_shared_decode_b1(a3b, Is, gate, k1, k2):
    """One token: Is a multiple of I runs inside the one-launch kernel, Is = 512
    on the grouped path."""
    L, Lh = a3b
    check_shared(synth.DECODE_B1, dict(L, x=L["x"][:1]), dict(Lh, x=Lh["x"][:1]),
                 shared_of(synth.DECODE_B8, Is, gate), k1, k2)


@pytest.mark.parametrize("flags", [0, moe.FORCE_GROUPED])
@pytest.mark.parametrize("T", [1, 8])
def test_shared_grouped(a3b, T, flags):
    L, Lh = a3b
    check_shared(synth.DECODE_B8, dict(L, x=L["x"][:T]), dict(Lh, x=Lh["x"][:T]),
                 shared_of(synth.DECODE_B8, 768, True), 4, 16, flags=flags)


def test_shared_with_bf16_router(a3b):
    L, Lh = a3b
    for T in (1, 8):
        check_shared(synth.DECODE_B8, dict(L, x=L["x"][:T]), dict(Lh, x=Lh["x"][:T]),
                     shared_of(synth.DECODE_B8, 1536, True), 4, 16, bf16_router=True)


@pytest.fixture(scope="module")
def prefill():
    L = to_dev(synth.make_layer(synth.PREFILL))
    return L, host_layer(L)


@pytest.mark.parametrize("T,flags", [(300, moe.FORCE_PREFILL), (63, moe.FORCE_PREFILL),
                                     (300, moe.FORCE_GROUPED)])
def test_shared_prefill_paths(prefill, T, flags):
    L, Lh = prefill
    check_shared(synth.PREFILL, dict(L, x=L["x"][:T]), dict(Lh, x=Lh["x"][:T]),
                 shared_of(synth.PREFILL, 1536, True), 4, 16, flags=flags)


@pytest.mark.parametrize("k1,k2", synth.PREFILL.k_pairs)
def test_shared_prefill_4096(prefill, k1, k2):
    L, Lh = prefill
    check_shared(synth.PREFILL, L, Lh, shared_of(synth.PREFILL, 768, True), k1, k2)
    assert check_shared.checked == 4096


@pytest.mark.parametrize("T,Is", [(1, 128), (1, 64), (8, 64), (8, 200)])
def test_shared_fp32(T, Is):
    """fp32 layer: the one-launch kernel (T = 1, Is a multiple of I = 64) and the
    grouped path, to the fp32 tolerance."""
    cfg = synth.TINY
    L = synth.make_layer(cfg)
    Lt = dict(L, x=L["x"][:T])
    check_shared(cfg, Lt, host_layer(Lt), synth.make_shared(cfg, Is, gate=True), 2, 4)


def test_shared_is_deterministic_and_adds_to_the_routed_layer(a3b):
    L, _ = a3b
    S = {k: (None if v is None else v.cuda()) for k, v in
         shared_of(synth.DECODE_B8, 768, False).items()}
    x = L["x"][:1]
    args = (x, L["Wr"], L["Wg"], L["Wu"], L["Wd"], 4, 16)
    y1 = moe.forward(*args, shared=(S["Sg"], S["Su"], S["Sd"]))
    y2 = moe.forward(*args, shared=(S["Sg"], S["Su"], S["Sd"]))
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    # a zero shared expert leaves the routed layer (up to the bf16 rounding of y)
    z = [torch.zeros_like(S[k]) for k in ("Sg", "Su", "Sd")]
    y0 = moe.forward(*args)
    yz = moe.forward(*args, shared=tuple(z))
    assert torch.equal(y0.view(torch.int16), yz.view(torch.int16))


def test_shared_rejects_an_unknown_flag(a3b):
    L, _ = a3b
    S = {k: (None if v is None else v.cuda()) for k, v in
         shared_of(synth.DECODE_B8, 768, False).items()}
    with pytest.raises(moe.MoeError):
        moe.forward(L["x"][:1], L["Wr"], L["Wg"], L["Wu"], L["Wd"], 4, 16,
                    flags=1, shared=(S["Sg"], S["Su"], S["Sd"]))
