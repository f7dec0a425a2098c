"""The bf16 router (MOE_FLAG_ROUTER_BF16) on the GPU against the oracle.

The router method of "Paper of the Week #3 - Half the FLOPs Is Not Half the
Time" (section "Ship It - Code of the Week") on a bf16 model: bf16 logits,
fp32 softmax and Eq. 2, weights cast to bf16.  For every path:
(i) the GPU's logits are bf16 values within one bf16 step plus the fp32
accumulation bound of the oracle's exact-then-rounded logits; (ii) the oracle's bf16-weight route on the GPU's
own logits equals the GPU's ids and weights bit for bit, and at k1 = k2 both
equal the stock renormalising router, cast included; (iii) y matches the
oracle's experts on that route within the bf16 tolerance; (iv) an
independent oracle route picks the same experts on every token whose logits
came out identical.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import decoupled_top_routing_amd as moe
import oracle
from decoupled_top_routing_amd import synth
from parity import NTHREADS, TOL_BF16, bits, host_layer, normwise_err, to_dev, to_f64
from test_oracle_bf16_router_pins import stock_router

pytestmark = pytest.mark.gpu


def bf16_steps(a, b):
    """Distance between float32 arrays of bf16 values, in bf16 steps."""
    def key(v):
        u = (np.ascontiguousarray(v, np.float32).view(np.uint32) >> 16).astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(key(a) - key(b))


def bf16_ulp(v):
    """Spacing of bf16 values at |v| (the normal range; 2^-133 below it)."""
    e = np.floor(np.log2(np.maximum(np.abs(np.asarray(v, np.float64)), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def logit_gate(lg, ref, x, Wr):
    """Per logit, how far the GPU's bf16 logit may lie from the oracle's exact
    dot product rounded once to bf16.  The GPU accumulates the exact bf16
    products in fp32 in its own order, then rounds once, as a bf16 linear
    layer does: any fp32 summation order of H terms is within H * 2^-24 *
    sum_h |x_h w_h| of the exact sum, and each side's rounding to bf16 adds at
    most half a bf16 step.  Returns (allowed distance, accumulation bound)."""
    xf = x.astype(np.uint32) << 16 if x.dtype == np.uint16 else x
    wf = Wr.astype(np.uint32) << 16 if Wr.dtype == np.uint16 else Wr
    xf = np.ascontiguousarray(xf).view(np.float32).astype(np.float64)
    wf = np.ascontiguousarray(wf).view(np.float32).astype(np.float64)
    acc = x.shape[1] * 2.0 ** -24 * (np.abs(xf) @ np.abs(wf).T)
    return np.maximum(bf16_ulp(lg), bf16_ulp(ref)) + acc, acc


def with_bf16_router(L):
    """The layer with its router weight cast to bf16 and no bias."""
    return dict(L, Wr=L["Wr"].to(torch.bfloat16), br=None)


def check_bf16_router(name, L, Lh, k1, k2, flags=0, token_sample=None):
    g = to_dev(L) if L["Wg"].device.type == "cpu" else L
    print(f"{name} T={g['x'].shape[0]} k1={k1} k2={k2} flags={flags} bf16 router", flush=True)
    assert g["Wr"].dtype == torch.bfloat16 and g["br"] is None
    y, lg, ids, w = moe.forward(g["x"], g["Wr"], g["Wg"], g["Wu"], g["Wd"], k1, k2,
                                return_route=True, flags=flags)
    torch.cuda.synchronize()
    lg_h = lg.cpu().numpy()
    T = lg_h.shape[0]
    sel = np.arange(T) if token_sample is None else np.asarray(token_sample)
    # (i) logits: bf16 values, within one bf16 step of the oracle
    assert not (lg_h.view(np.uint32) & 0xFFFF).any(), "logits are not bf16 values"
    x_h = Lh["x"][sel]
    wr_h = synth.to_numpy(g["Wr"].cpu())
    ref_l = oracle.logits_bf16(x_h, wr_h, nthreads=NTHREADS)
    allowed, acc = logit_gate(lg_h[sel], ref_l, x_h, wr_h)
    dist = np.abs(lg_h[sel].astype(np.float64) - ref_l.astype(np.float64))
    steps = bf16_steps(lg_h[sel], ref_l)
    assert (dist <= allowed).all(), f"{int((dist > allowed).sum())} logits outside the bound"
    # past one step only where the accumulation bound itself exceeds a step
    far = steps > 1
    assert (acc[far] > bf16_ulp(ref_l)[far]).all()
    # (ii) route on the GPU's logits, bit for bit
    oids, ow = oracle.route_bf16w(lg_h, k1, k2)
    gi, gw = ids.cpu().numpy(), w.cpu().numpy()
    bad = np.nonzero((gi != oids).any(1) | (bits(gw) != bits(ow)).any(1))[0]
    assert bad.size == 0, f"{bad.size} tokens differ, first {bad[:5]}"
    if k1 == k2:
        p = oracle.softmax(lg_h)
        for t in range(min(T, 64)):
            sid, sw = stock_router(p[t], k1)
            assert np.array_equal(gi[t], sid) and np.array_equal(bits(gw[t]), bits(sw)), t
    # (iii) y on that route
    Wg, Wu, Wd = Lh["Wg"], Lh["Wu"], Lh["Wd"]
    y_ref = oracle.experts(x_h, Wg, Wu, Wd, oids[sel], ow[sel], nthreads=NTHREADS)
    err = normwise_err(to_f64(y)[sel], y_ref)
    assert err <= TOL_BF16, f"normwise error {err} > {TOL_BF16}"
    # (iv) independent route: same experts wherever the logits agree exactly
    iids, _ = oracle.route_bf16w(ref_l, k1, k2)
    same_logits = (bits(lg_h[sel]) == bits(ref_l)).all(1)
    differ = (iids != gi[sel]).any(1)
    assert not (differ & same_logits).any()
    return err, len(sel)


@pytest.fixture(scope="module")
def a3b():
    L = with_bf16_router(to_dev(synth.make_layer(synth.DECODE_B8)))
    return L, host_layer(L)


@pytest.mark.parametrize("k1,k2", [(8, 8), (4, 4), (4, 16), (2, 16), (3, 16), (4, 128)])
@pytest.mark.parametrize("T", [1, 8])
def test_bf16_router_decode(a3b, k1, k2, T):
    """T = 1 runs the one-launch kernel, T = 8 the grouped path."""
    L, Lh = a3b
    check_bf16_router(synth.DECODE_B8.name, dict(L, x=L["x"][:T]), dict(Lh, x=Lh["x"][:T]),
                      k1, k2)


@pytest.mark.parametrize("T", [1, 8])
def test_bf16_router_forced_grouped(a3b, T):
    L, Lh = a3b
    check_bf16_router(synth.DECODE_B8.name, dict(L, x=L["x"][:T]), dict(Lh, x=Lh["x"][:T]),
                      4, 16, flags=moe.FORCE_GROUPED)


@pytest.fixture(scope="module")
def prefill():
    L = with_bf16_router(to_dev(synth.make_layer(synth.PREFILL)))
    return L, host_layer(L)


@pytest.mark.parametrize("k1,k2", synth.PREFILL.k_pairs)
def test_bf16_router_prefill_4096(prefill, k1, k2):
    L, Lh = prefill
    _, n = check_bf16_router(synth.PREFILL.name, L, Lh, k1, k2)
    assert n == 4096


@pytest.mark.parametrize("T", [1, 63, 300])
@pytest.mark.parametrize("flags", [moe.FORCE_PREFILL, moe.FORCE_GROUPED])
def test_bf16_router_paths_on_small_batches(prefill, T, flags):
    L, Lh = prefill
    check_bf16_router(synth.PREFILL.name, dict(L, x=L["x"][:T]), dict(Lh, x=Lh["x"][:T]),
                      4, 16, flags=flags)


SMALL = replace(synth.TINY, dtype="bf16", rms_norm_x=True, router_var_times_H=4.0)


@pytest.mark.parametrize("E,k1,k2,H,I,T,flags", [
    (40, 3, 7, 264, 72, 1, 0),        # no one-launch shape: grouped at T = 1, ragged rows
    (40, 3, 7, 264, 72, 5, 0),
    (300, 6, 12, 512, 64, 1, 0),      # E > 256: the one-launch kernel's wave route
    (300, 6, 12, 512, 64, 8, 0),      # E > 256 on the grouped path
    (300, 6, 12, 1024, 64, 8, 0),     # the small-batch router + route launch, E > 256
    (64, 4, 16, 2048, 128, 40, 0),    # the same launch with three groups of tokens
    (1, 1, 1, 256, 64, 3, 0),         # one expert: p = 1, w = 1
    (33, 5, 9, 1024, 192, 257, moe.FORCE_PREFILL),  # E not a multiple of the router tile
])
def test_bf16_router_edge_shapes(E, k1, k2, H, I, T, flags):
    cfg = replace(SMALL, name=f"hf-E{E}-H{H}-I{I}", T=T, H=H, E=E, I=I)
    L = with_bf16_router(to_dev(synth.make_layer(cfg)))
    check_bf16_router(cfg.name, L, host_layer(L), k1, k2, flags=flags)


def test_bf16_router_is_deterministic(a3b):
    L, _ = a3b
    outs = [moe.forward(L["x"], L["Wr"], L["Wg"], L["Wu"], L["Wd"], 4, 16, return_route=True)
            for _ in range(2)]
    for u, v in zip(*outs):
        assert torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u,
                           v.view(torch.int16) if v.dtype == torch.bfloat16 else v)


def test_bf16_router_rejected_where_unsupported(a3b):
    L, _ = a3b
    with pytest.raises(moe.MoeError):   # bit value 1 is not a flag
        moe.forward(L["x"][:1], L["Wr"], L["Wg"], L["Wu"], L["Wd"], 4, 16, flags=1)
    with pytest.raises(moe.MoeError):   # no bias with the bf16 router
        moe.forward(L["x"][:1], L["Wr"], L["Wg"], L["Wu"], L["Wd"], 4, 16,
                    br=torch.zeros(L["Wr"].shape[0], device=L["x"].device))
