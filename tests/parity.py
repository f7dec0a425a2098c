"""Comparison helpers for the GPU parity tests (HIP path against the oracle)."""
import os

import numpy as np
import torch

import oracle
from decoupled_top_routing_amd import synth

DEV = "cuda:0"

# host threads for the oracle (it threads over tokens); at most 16, the CPU
# share of one GPU on the boxes these tests run on
NTHREADS = max(1, min(16, len(os.sched_getaffinity(0))))

# Output tolerances, normwise per token: max_h |y - y_ref| / max_h |y_ref|.
TOL_F32 = 1e-5   # fp32 activations and weights
TOL_BF16 = 2e-2  # bf16 weights (bf16 output rounding alone is about 4e-3)


def normwise_err(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    if y.size == 0:
        return 0.0
    return float((np.abs(y - ref).max(axis=1) / np.abs(ref).max(axis=1)).max())


def to_f64(t):
    """A torch tensor (fp32 or bf16) as numpy fp64 on the host."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.int32)


def check_route_exact(gpu_ids, gpu_w, logits_host, k1, k2, what=""):
    """The GPU route must equal the oracle's route on the same logits, bit for bit."""
    oids, ow = oracle.route(logits_host, k1, k2)
    gi = gpu_ids.cpu().numpy()
    gw = gpu_w.cpu().numpy()
    bad = np.nonzero((gi != oids).any(1) | (bits(gw) != bits(ow)).any(1))[0]
    assert bad.size == 0, (f"{what}: {bad.size} tokens differ, first {bad[:5]}: "
                           f"gpu {gi[bad[0]]} {gw[bad[0]]} oracle {oids[bad[0]]} {ow[bad[0]]}")
    return oids, ow


def near_tie_tokens(p, k1, rel=1e-5):
    """Tokens whose k1-th and (k1+1)-th probabilities are within rel of each other."""
    if p.shape[1] <= k1:
        return np.zeros(p.shape[0], bool)
    s = -np.sort(-p, axis=1)
    return (s[:, k1 - 1] - s[:, k1]) < rel * s[:, k1 - 1]


def host_layer(L):
    """numpy copies of a layer for the oracle (bf16 as uint16 bits)."""
    return {k: synth.to_numpy(v) for k, v in L.items()}


def to_dev(L):
    return {k: (None if v is None else v.to(DEV)) for k, v in L.items()}


def expert_subset(L, Lh, ids):
    """Expert weights for the oracle and ids into them.  With host copies of
    the whole layer these are returned as they are; otherwise (layers too large
    to copy) only the experts named in ids are copied from the device and ids
    are renumbered into that subset."""
    if Lh.get("Wg") is not None:
        return Lh["Wg"], Lh["Wu"], Lh["Wd"], ids
    uniq, inv = np.unique(ids, return_inverse=True)
    idx = torch.as_tensor(uniq, dtype=torch.long, device=L["Wg"].device)
    sub = [synth.to_numpy(L[k].index_select(0, idx)) for k in ("Wg", "Wu", "Wd")]
    return sub[0], sub[1], sub[2], inv.reshape(ids.shape).astype(np.int32)


def run_and_check(cfg, L, Lh, k1, k2, flags=0, token_sample=None, tol=None):
    """One moe_forward call checked against the oracle:
    (i) logits within 1e-5 normwise; (ii) the oracle's route on the GPU's own
    logits equals the GPU's ids and weights bit for bit (all tokens); (iii) y
    against the oracle's experts and combine on that route, within the dtype's
    tolerance; (iv) an independent oracle route from x picks the same experts
    except on near-ties.  token_sample limits (i), (iii) and (iv) to those
    tokens; Lh may omit the expert weights (see expert_subset).  Returns
    (y, error, number of tokens whose y was checked)."""
    import decoupled_top_routing_amd as moe
    g = to_dev(L) if L["Wg"].device.type == "cpu" else L
    print(f"{cfg.name} T={g['x'].shape[0]} k1={k1} k2={k2} flags={flags}", flush=True)
    y, lg, ids, w = moe.forward(g["x"], g["Wr"], g["Wg"], g["Wu"], g["Wd"], k1, k2,
                                br=g["br"], return_route=True, flags=flags)
    torch.cuda.synchronize()
    lg_h = lg.cpu().numpy()
    T = lg_h.shape[0]
    sel = np.arange(T) if token_sample is None else np.asarray(token_sample)
    x_h = Lh["x"][sel]
    ref_l = oracle.logits(x_h, Lh["Wr"], Lh["br"], nthreads=NTHREADS)
    assert normwise_err(lg_h[sel], ref_l) <= 1e-5
    oids, ow = check_route_exact(ids, w, lg_h, k1, k2, f"{cfg.name} ({k1},{k2})")
    Wg, Wu, Wd, sids = expert_subset(g, Lh, oids[sel])
    y_ref = oracle.experts(x_h, Wg, Wu, Wd, sids, ow[sel], nthreads=NTHREADS)
    err = normwise_err(to_f64(y)[sel], y_ref)
    tol = tol if tol is not None else (TOL_F32 if cfg.dtype == "f32" else TOL_BF16)
    assert err <= tol, f"normwise error {err} > {tol}"
    iids, _ = oracle.route(ref_l, k1, k2)
    ties = near_tie_tokens(oracle.softmax(ref_l), k1)
    differ = (np.sort(iids, 1) != np.sort(oids[sel], 1)).any(1)
    assert not (differ & ~ties).any(), "experts differ away from a near-tie"
    return y, err, len(sel)
