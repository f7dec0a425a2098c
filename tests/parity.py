"""Comparison helpers for the GPU parity tests (HIP path against the oracle)."""
import numpy as np
import torch

import oracle
from decoupled_top_routing_amd import synth

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
