"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: closed forms,
libm / numpy fp64, brute force on tiny inputs, invariants and special cases of
Eq. 2 ("Paper of the Week #3 - Half the FLOPs Is Not Half the Time", section
"The Receipt").  None of these tests touches the GPU.
"""
import ctypes
import itertools
import json
import math
import subprocess
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle
from decoupled_top_routing_amd import synth

GOLDEN = Path(__file__).parent / "golden"
NATIVE = Path(__file__).parent / "native"


def ulp_diff(a, b):
    """|a - b| in units in the last place for float32 arrays of equal sign."""
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ai - bi)


# ---------------------------------------------------------------- exp_spec

def test_exp_spec_special_values():
    e = oracle.exp_spec(np.array([0.0, -0.0, -80.0, -80.00001, -1e30], np.float32))
    assert e[0] == 1.0 and e[1] == 1.0
    assert e[2] > 0.0 and np.isfinite(e[2])
    assert e[3] == 0.0 and e[4] == 0.0
    # every value at or above -80 is a normal float
    assert e[2] >= np.finfo(np.float32).tiny


@pytest.mark.slow
def test_exp_spec_exhaustive(tmp_path):
    """Every binary32 d in [-80, 0]: within 1 ulp of libm's exp (fp64, rounded
    to float) and exp(0) == 1.  A polynomial exp with a 1-ulp error cannot be
    exactly monotone; the sweep bounds every upward step (as d decreases) by
    1 ulp and counts them, so a change in the reduction or the polynomial that
    loosens either shows up here."""
    so = tmp_path / "exp_sweep.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                    str(NATIVE / "exp_sweep.c"), "-o", str(so), "-lm"],
                   check=True)
    lib = oracle._load()
    sw = ctypes.CDLL(str(so))
    res = (ctypes.c_int64 * 5)()
    fn = ctypes.cast(lib.oracle_exp_spec, ctypes.c_void_p)
    sw.sweep.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    sw.sweep(fn, res)
    max_ulp, max_up, n_up, count, one_bits = list(res)
    assert count == 0xC2A00000 - 0x80000000 + 1
    assert max_ulp <= 1, f"max error {max_ulp} ulp"
    assert max_up <= 1, f"steps up by {max_up} ulp"
    assert n_up < 10_000, f"{n_up} upward steps"
    assert one_bits == np.float32(1.0).view(np.int32)


def test_exp_spec_sampled_against_numpy():
    rng = np.random.default_rng(1)
    d = -rng.uniform(0, 80, 200_000).astype(np.float32)
    got = oracle.exp_spec(d)
    want = np.exp(d.astype(np.float64)).astype(np.float32)
    assert ulp_diff(got, want).max() <= 1


# ---------------------------------------------------------------- softmax

@pytest.mark.parametrize("E", [1, 2, 3, 16, 100, 128, 512, 1000, 1024])
def test_softmax_sums_to_one_and_matches_fp64(E):
    rng = np.random.default_rng(E)
    l = (rng.standard_normal((64, E)) * 3).astype(np.float32)
    p = oracle.softmax(l)
    assert np.all(np.abs(p.astype(np.float64).sum(1) - 1.0) <= E * 2.0 ** -23)
    ref = np.exp(l.astype(np.float64) - l.max(1, keepdims=True).astype(np.float64))
    ref /= ref.sum(1, keepdims=True)
    rel = np.abs(p - ref) / ref
    assert rel.max() < 8 * 2.0 ** -24 * math.log2(max(E, 2)) + 4e-7


@pytest.mark.parametrize("E", [1, 2, 4, 16, 64, 128, 512, 1024])
def test_softmax_uniform_power_of_two_is_exact(E):
    for v in (0.0, 1.5, -30.0):
        p = oracle.softmax(np.full((1, E), v, np.float32))
        assert np.all(p == np.float32(1.0 / E))


@pytest.mark.parametrize("E", [2, 5, 16, 128, 1024])
@pytest.mark.parametrize("L", [0.5, 3.0, 10.0, -2.0])
def test_softmax_one_hot_logit_closed_form(E, L):
    """logits (L, 0, ..., 0): p0 = 1 / (1 + (E-1) e^-L), pi = e^-L p0 if L > 0."""
    l = np.zeros((1, E), np.float32)
    l[0, 0] = L
    p = oracle.softmax(l)[0]
    p0 = 1.0 / (1.0 + (E - 1) * math.exp(-L))
    pi = math.exp(-L) * p0
    assert ulp_diff(np.float32(p0), p[0]) <= 4
    assert np.all(ulp_diff(np.full(E - 1, pi, np.float32), p[1:]) <= 4)


def test_softmax_matches_torch_within_8ulp():
    """torch's CPU softmax (its own exp, a reciprocal multiply) is a library
    routine with an unstated error; both sit within a few ulp of the exact
    value, so they agree within 8 ulp.  The tight pin is the fp64 one above."""
    rng = np.random.default_rng(7)
    for E in (16, 128, 512):
        l = (rng.standard_normal((256, E)) * 2).astype(np.float32)
        p = oracle.softmax(l)
        t = torch.softmax(torch.from_numpy(l), dim=-1, dtype=torch.float32).numpy()
        big = t > 1e-30
        assert ulp_diff(p[big], t[big]).max() <= 8


def test_softmax_max_subtraction_is_shift_invariant():
    """Adding a constant that is exact in fp32 to every logit changes nothing:
    the max subtraction makes the result depend only on l - max(l)."""
    rng = np.random.default_rng(3)
    l = np.round(rng.standard_normal((32, 128)) * 256).astype(np.float32) / 256
    p1 = oracle.softmax(l)
    p2 = oracle.softmax(l + np.float32(64.0))
    assert np.array_equal(p1, p2)


def test_softmax_sum_order_and_division():
    """The sum order reading: S is the pairwise (halving) sum of the e values,
    zero-padded to a power of two, and p = e / S with one IEEE division.  The
    e values come from the separately pinned exp; the tree here is built
    bottom-up with numpy float32 pair additions."""
    rng = np.random.default_rng(21)
    for E in (3, 100, 128, 1000):
        l = (rng.standard_normal((16, E)) * 4).astype(np.float32)
        p = oracle.softmax(l)
        for t in range(l.shape[0]):
            d = (l[t] - l[t].max()).astype(np.float32)
            e = oracle.exp_spec(d)
            P = 1 << (E - 1).bit_length()
            level = np.zeros(P, np.float32)
            level[:E] = e
            while level.size > 1:
                level = (level[0::2] + level[1::2]).astype(np.float32)
            ref = (e / level[0]).astype(np.float32)
            assert np.array_equal(p[t].view(np.int32), ref.view(np.int32))


# ---------------------------------------------------------------- top-k

def brute_route(p_row, k1, k2):
    """Full stable sort by (p descending, index ascending); weights per Eq. 2
    with a sequential sum in rank order, or no division when k2 >= E."""
    E = len(p_row)
    order = sorted(range(E), key=lambda e: (-float(p_row[e]), e))
    K2 = min(k2, E)
    ids = order[:k1]
    if k2 >= E:
        w = [np.float32(p_row[e]) for e in ids]
    else:
        M = np.float32(0.0)
        for e in order[:K2]:
            M = np.float32(M + np.float32(p_row[e]))
        w = [np.float32(np.float32(p_row[e]) / M) for e in ids]
    return np.array(ids, np.int32), np.array(w, np.float32)


def _tiny_logit_sets(E, rng):
    sets = [rng.standard_normal(E).astype(np.float32),
            np.zeros(E, np.float32),                        # all equal
            np.round(rng.standard_normal(E)).astype(np.float32)]  # many ties
    if E >= 2:
        v = rng.standard_normal(E).astype(np.float32)
        v[E - 1] = v[0]                                      # tied pair
        sets.append(v)
        # ties straddling every rank boundary: values in pairs of equals
        v = np.repeat(np.arange(E // 2 + 1, dtype=np.float32), 2)[:E][::-1].copy()
        sets.append(rng.permutation(v).astype(np.float32))
    return sets


@pytest.mark.parametrize("E", list(range(1, 9)))
def test_topk_matches_brute_force_on_tiny_E(E):
    rng = np.random.default_rng(100 + E)
    for l in _tiny_logit_sets(E, rng):
        l = l.reshape(1, E)
        p = oracle.softmax(l)[0]
        for k1 in range(1, E + 1):
            for k2 in range(k1, E + 3):
                ids, w = oracle.route(l, k1, k2)
                bids, bw = brute_route(p, k1, k2)
                assert np.array_equal(ids[0], bids), (l, k1, k2)
                assert np.array_equal(w[0].view(np.int32), bw.view(np.int32)), (l, k1, k2)


def test_tie_break_takes_lower_index():
    l = np.array([[1.0, 2.0, 2.0, 0.5, 2.0]], np.float32)
    ids, _ = oracle.route(l, 3, 3)
    assert ids.tolist() == [[1, 2, 4]]
    ids, _ = oracle.route(l, 1, 4)
    assert ids.tolist() == [[1]]


# ---------------------------------------------------------------- Eq. 2

def test_golden_closed_forms():
    g = json.loads((GOLDEN / "eq2_closed_forms.json").read_text())
    for c in g["cases"]:
        l = np.full((1, c["E"]), c["logit"], np.float32)
        ids, w = oracle.route(l, c["k1"], c["k2"])
        assert ids[0].tolist() == c["ids"], c
        assert w[0].tolist() == c["w"], c


def standard_renorm(p_row, k):
    """Standard top-k renormalisation written independently: argsort by
    (-p, index), take k, divide by their sequential fp32 sum."""
    idx = np.lexsort((np.arange(len(p_row)), -p_row.astype(np.float64)))[:k]
    s = np.float32(0)
    for e in idx:
        s = np.float32(s + p_row[e])
    return idx.astype(np.int32), (p_row[idx] / s).astype(np.float32)


@pytest.mark.parametrize("E,k", [(16, 2), (16, 8), (128, 8), (128, 4), (512, 10), (1024, 64)])
def test_k1_equal_k2_is_standard_renormalisation_bitwise(E, k):
    """k2 = k1 reproduces standard renormalisation bit for bit (P1, The
    Receipt: the patch is bit-identical to the stock router at k1 = k2)."""
    rng = np.random.default_rng(E * 31 + k)
    l = (rng.standard_normal((200, E)) * 2).astype(np.float32)
    p = oracle.softmax(l)
    ids, w = oracle.route(l, k, k)
    for t in range(l.shape[0]):
        sid, sw = standard_renorm(p[t], k)
        assert np.array_equal(ids[t], sid)
        assert np.array_equal(w[t].view(np.int32), sw.view(np.int32))


@pytest.mark.parametrize("E,k", [(16, 2), (128, 1), (128, 4), (128, 8), (512, 2), (512, 8)])
def test_k1_equal_k2_matches_the_stock_router_for_small_k(E, k):
    """The page's stock router ("Paper of the Week #3", "Ship It - Code of
    the Week": top-k of the probabilities, then each divided by their sum)
    run with torch's own topk and sum on the oracle's probabilities: at
    k = 1, 2, 4 and 8 its weights equal the oracle's at k1 = k2 bit for bit.
    At other k torch's vectorised sum can add in another order (k = 5 at
    E = 512: the last bit differs on about a third of the tokens, k = 10 and
    64 on more), so "standard renormalisation" is read as the sequential sum
    in rank order, which the pins above fix."""
    rng = np.random.default_rng(E * 7 + k)
    l = (rng.standard_normal((500, E)) * 2).astype(np.float32)
    p = torch.from_numpy(oracle.softmax(l))
    vals, idx = torch.topk(p, k, dim=-1, largest=True, sorted=True)
    w_stock = vals / vals.sum(dim=-1, keepdim=True)
    ids, w = oracle.route(l, k, k)
    # torch.topk breaks exact ties its own way; compare where the k-th and
    # (k+1)-th probabilities differ (a tie at the boundary changes the set)
    srt = torch.sort(p, dim=-1, descending=True).values
    ok = (srt[:, k - 1] != srt[:, k]).numpy() if k < E else np.ones(len(l), bool)
    assert ok.sum() > 0.9 * len(l)
    assert np.array_equal(np.sort(ids[ok], axis=1), np.sort(idx.numpy()[ok], axis=1))
    wo = np.take_along_axis(w[ok], np.argsort(ids[ok], axis=1), axis=1)
    ws = np.take_along_axis(w_stock.numpy()[ok], np.argsort(idx.numpy()[ok], axis=1), axis=1)
    assert np.array_equal(wo.view(np.int32), ws.view(np.int32))


@pytest.mark.parametrize("E,k1", [(16, 2), (128, 4), (128, 8), (512, 10), (1000, 7)])
def test_k2_at_least_E_gives_probabilities_bitwise(E, k1):
    rng = np.random.default_rng(E + k1)
    l = (rng.standard_normal((100, E)) * 2).astype(np.float32)
    p = oracle.softmax(l)
    for k2 in (E, E + 1, 4 * E):
        ids, w = oracle.route(l, k1, k2)
        assert np.array_equal(w.view(np.int32),
                              np.take_along_axis(p, ids, 1).view(np.int32))


@pytest.mark.parametrize("E,k1,k2", [(16, 2, 4), (128, 4, 16), (128, 3, 16),
                                     (128, 2, 16), (512, 5, 20), (1024, 8, 512)])
def test_weight_sum_is_topk1_mass_over_topk2_mass(E, k1, k2):
    rng = np.random.default_rng(E * k1 + k2)
    l = (rng.standard_normal((300, E)) * 2).astype(np.float32)
    p = oracle.softmax(l).astype(np.float64)
    ids, w = oracle.route(l, k1, k2)
    ps = -np.sort(-p, axis=1)
    expect = ps[:, :k1].sum(1) / ps[:, :k2].sum(1)
    got = w.astype(np.float64).sum(1)
    assert np.all(np.abs(got - expect) / expect <= (k1 + 1) * 2.0 ** -24 + 2 * k2 * 2.0 ** -24)


def test_ids_do_not_depend_on_k2_and_weights_shrink_with_k2():
    """P1, The Receipt: k2 changes the weights, never which experts run."""
    rng = np.random.default_rng(11)
    E = 128
    l = (rng.standard_normal((300, E)) * 2).astype(np.float32)
    for k1 in (1, 2, 4, 8):
        prev_ids, prev_w = None, None
        for k2 in sorted({k1, k1 + 1, 8, 16, 64, 127, 128, 1000} - set(range(k1))):
            ids, w = oracle.route(l, k1, k2)
            if prev_ids is not None:
                assert np.array_equal(ids, prev_ids)
                assert np.all(w <= prev_w)
            prev_ids, prev_w = ids, w


def test_invalid_arguments_are_rejected():
    l = np.zeros((2, 8), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.route(l, 3, 2)        # k1 > k2
    with pytest.raises(oracle.OracleError):
        oracle.route(l, 9, 9)        # k1 > E
    bad = l.copy()
    bad[1, 3] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.route(bad, 1, 2)      # non-finite logit


# ---------------------------------------------------------------- experts

def np_swiglu_expert(x64, Wg, Wu, Wd):
    """One gated-MLP expert in numpy fp64: (silu(x Wg^T) * (x Wu^T)) Wd^T."""
    g = x64 @ Wg.T
    u = x64 @ Wu.T
    a = g / (1.0 + np.exp(-g)) * u
    return a @ Wd.T


def bf16_to_f64(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def normwise(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return (np.abs(y - ref).max(axis=1) / np.abs(ref).max(axis=1)).max()


def tiny_layer(seed=0, T=8, H=64, E=8, I=32, bf16=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    Wr = (rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32)
    Wg = (rng.standard_normal((E, I, H)) * 0.1).astype(np.float32)
    Wu = (rng.standard_normal((E, I, H)) * 0.1).astype(np.float32)
    Wd = (rng.standard_normal((E, H, I)) * 0.1).astype(np.float32)
    if bf16:
        def cvt(a):
            return synth.to_numpy(torch.from_numpy(a).to(torch.bfloat16))
        x, Wg, Wu, Wd = cvt(x), cvt(Wg), cvt(Wu), cvt(Wd)
    return x, Wr, Wg, Wu, Wd


@pytest.mark.parametrize("bf16", [False, True])
def test_each_expert_matches_numpy_fp64(bf16):
    x, Wr, Wg, Wu, Wd = tiny_layer(bf16=bf16)
    T, E = x.shape[0], Wg.shape[0]
    x64 = bf16_to_f64(x)
    for e in range(E):
        ids = np.full((T, 1), e, np.int32)
        w = np.ones((T, 1), np.float32)
        y = oracle.experts(x, Wg, Wu, Wd, ids, w)
        ref = np_swiglu_expert(x64, bf16_to_f64(Wg[e]), bf16_to_f64(Wu[e]),
                               bf16_to_f64(Wd[e]))
        assert normwise(y, ref) < 1e-6


def test_dense_mixture_special_case():
    """k1 = E with k2 >= E: y = sum_e p_e SwiGLU_e(x), the dense mixture."""
    x, Wr, Wg, Wu, Wd = tiny_layer(seed=5)
    E = Wg.shape[0]
    y, lg, ids, w = oracle.forward(x, Wr, Wg, Wu, Wd, E, E)
    p = oracle.softmax(lg).astype(np.float64)
    x64 = x.astype(np.float64)
    ref = sum(p[:, e:e + 1] * np_swiglu_expert(x64, Wg[e], Wu[e], Wd[e])
              for e in range(E))
    assert normwise(y, ref) < 1e-6
    # logits against an fp64 matmul
    ref_l = x64 @ Wr.astype(np.float64).T
    assert np.abs(lg - ref_l).max() <= 2.0 ** -23 * np.abs(ref_l).max()


def test_router_bias_is_added():
    x, Wr, Wg, Wu, Wd = tiny_layer(seed=13)
    br = np.random.default_rng(14).standard_normal(Wr.shape[0]).astype(np.float32)
    lg = oracle.logits(x, Wr, br)
    ref = x.astype(np.float64) @ Wr.astype(np.float64).T + br
    assert np.abs(lg - ref).max() <= 2.0 ** -23 * np.abs(ref).max()


def test_single_expert_case():
    x, Wr, Wg, Wu, Wd = tiny_layer(seed=6)
    y, lg, ids, w = oracle.forward(x, Wr, Wg, Wu, Wd, 1, 4)
    x64 = x.astype(np.float64)
    for t in range(x.shape[0]):
        e = ids[t, 0]
        ref = w[t, 0] * np_swiglu_expert(x64[t:t + 1], Wg[e], Wu[e], Wd[e])
        assert normwise(y[t:t + 1], ref) < 1e-6


def test_relabelling_experts_permutes_ids_and_keeps_y():
    x, Wr, Wg, Wu, Wd = tiny_layer(seed=8)
    E = Wg.shape[0]
    perm = np.random.default_rng(9).permutation(E)  # new index of old expert e
    inv = np.argsort(perm)
    y1, lg1, ids1, w1 = oracle.forward(x, Wr, Wg, Wu, Wd, 3, 6)
    y2, lg2, ids2, w2 = oracle.forward(x, Wr[inv], Wg[inv], Wu[inv], Wd[inv], 3, 6)
    p = np.sort(oracle.softmax(lg1), axis=1)
    assert np.all(np.diff(p, axis=1) > 0)  # no ties, so the relabelling is clean
    assert np.array_equal(ids2, perm[ids1])
    assert np.array_equal(w1, w2)
    assert np.array_equal(y1, y2)


def test_tokens_are_independent():
    x, Wr, Wg, Wu, Wd = tiny_layer(seed=10)
    y, *_ = oracle.forward(x, Wr, Wg, Wu, Wd, 2, 4)
    for t in (0, 3, 7):
        yt, *_ = oracle.forward(x[t:t + 1], Wr, Wg, Wu, Wd, 2, 4)
        assert np.array_equal(yt[0], y[t])


def test_threads_do_not_change_results():
    x, Wr, Wg, Wu, Wd = tiny_layer(seed=12, T=16)
    a = oracle.forward(x, Wr, Wg, Wu, Wd, 2, 4, nthreads=1)
    b = oracle.forward(x, Wr, Wg, Wu, Wd, 2, 4, nthreads=4)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_zero_tokens():
    x, Wr, Wg, Wu, Wd = tiny_layer()
    y, lg, ids, w = oracle.forward(x[:0], Wr, Wg, Wu, Wd, 2, 4)
    assert y.shape == (0, x.shape[1]) and ids.shape == (0, 2)


# ------------------------------------------------ whole oracle on the workloads

def numpy_layer_fp64(x, Wr, br, Wg, Wu, Wd, ids, w):
    """The definition in numpy fp64, given the route: sum_r w_r SwiGLU(x)."""
    x64 = bf16_to_f64(x)
    y = np.zeros(x64.shape)
    for t in range(x64.shape[0]):
        for r in range(ids.shape[1]):
            e = ids[t, r]
            y[t] += float(w[t, r]) * np_swiglu_expert(
                x64[t:t + 1], bf16_to_f64(Wg[e]), bf16_to_f64(Wu[e]),
                bf16_to_f64(Wd[e]))[0]
    return y


@pytest.mark.parametrize("cfg,T_sub", [(synth.TINY, None), (synth.DECODE_B1, None),
                                       (synth.DECODE_B8, 4)])
def test_whole_oracle_against_numpy_fp64(cfg, T_sub):
    L = synth.make_layer(cfg)
    x = synth.to_numpy(L["x"])
    if T_sub:
        x = x[:T_sub]
    Wr, br = synth.to_numpy(L["Wr"]), synth.to_numpy(L["br"])
    Wg, Wu, Wd = (synth.to_numpy(L[k]) for k in ("Wg", "Wu", "Wd"))
    for k1, k2 in cfg.k_pairs[:3]:
        y, lg, ids, w = oracle.forward(x, Wr, Wg, Wu, Wd, k1, k2, br=br, nthreads=8)
        ref_l = bf16_to_f64(x) @ Wr.astype(np.float64).T
        if br is not None:
            ref_l += br
        assert np.abs(lg - ref_l).max() <= 4 * 2.0 ** -24 * np.abs(ref_l).max()
        assert normwise(y, numpy_layer_fp64(x, Wr, br, Wg, Wu, Wd, ids, w)) < 1e-6


def test_generator_is_deterministic_and_seeded():
    """Build the same layer twice and compare; a different base seed differs
    (the unseeded-weights defect described on the kozo-lab page, section 3)."""
    a = synth.make_layer(synth.TINY)
    b = synth.make_layer(synth.TINY)
    c = synth.make_layer(synth.TINY, base=1)
    for k in ("x", "Wr", "Wg", "Wu", "Wd"):
        assert torch.equal(a[k], b[k])
        assert not torch.equal(a[k], c[k])
    d = synth.make_layer(synth.TINY, layer=1)
    assert not torch.equal(a["Wg"], d["Wg"])
