"""CPU oracle for the routed MoE layer with decoupled top-k1/k2 weights.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU
library never imports, links or executes anything here, and this package
never touches the GPU library.

What it computes (``oracle.c`` holds the arithmetic):

* router logits  l = x . Wr^T (+ br)  -- "Paper of the Week #3 - Half the
  FLOPs Is Not Half the Time", section "Ship It - Code of the Week" (the
  router method's linear layer);
* fp32 softmax, ranking, and the weights of Eq. 2 of the same page, section
  "The Receipt": w_i = p_i / sum_{j in Top-k2} p_j for i in Top-k1, with
  k2 >= E meaning no division (the router method's ``k2 >= num_experts``
  branch);
* the activated experts as gated MLPs whose channels own a gate row, an up row
  and a down column -- "Channel Selection for Mixture-of-Experts Decoding Needs
  No Calibration Data", section 2 "Background" -- with silu on the gate, and
  their weighted sum.

Readings taken where the pages are silent (each is pinned by a test):

1. softmax: m = max l; d = fl(l - m); e = exp_spec(d) (Cody-Waite reduction,
   degree-7 Taylor, 0 below -80); S = pairwise sum of e zero-padded to a power
   of two; p = fl(e / S);
2. ranking is on probabilities, highest first, lower expert index first on
   equal probability;
3. the top-k2 mass is summed sequentially in rank order;
4. k2 >= E gives w = p exactly; k2 > E is clamped to E;
5. k1 <= k2 (k1 == k2 allowed); k1 > k2 is an argument error;
6. weights stay fp32 (the logits are fp32);
7. experts and combine are accumulated in fp64, rounded to fp32 once.

The bf16 router (``logits_bf16``, ``route_bf16w``, ``forward_bf16_router``)
is the same router method run on a bf16 model, as the page's code does it:
the linear layer in bf16 (the exact dot product rounded once to bf16, to
nearest with ties to even), the softmax upcast to fp32, and the weights cast
back to bf16 (same rounding) before they scale the experts.

The shared expert (``shared``) always runs beside the routed ones ("Channel
Selection for Mixture-of-Experts Decoding Needs No Calibration Data",
appendix B): a gated MLP of Is channels whose output is added to the routed
sum, scaled by sigmoid(x . sg) with a gate vector sg, else by 1 (a reading:
the pages do not give the gating).

Channel top-k (``down_column_norms``, ``channel_scores``, ``channel_select``,
``experts_kept``): "Channel Selection ..." section 5.2 scores each channel of
a token's activated experts by router weight x down-column norm x activation
magnitude, keeps the exact top ``keep`` over the token's k1*I channels (equal
scores: lower flat index r*I + c first, a reading) and sums only those.

The route functions (``softmax``, ``route``) are exact fp32 definitions; the
expert functions are accumulated in fp64.  Arrays are numpy; bf16 tensors are
passed as ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SRC = HERE / "oracle.c"
LIB = HERE / "liboracle.so"

F32 = 0
BF16 = 1

_lib = None


def build(verbose: bool = False, src: Path = SRC, out: Path = LIB) -> Path:
    """Compile ``oracle.c`` with gcc (no fast-math, no FP contraction)."""
    cmd = [
        "gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-ffp-contract=off",
        "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
        str(src), "-o", str(out) + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(str(out) + ".tmp", out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not LIB.exists():
        build()
    _lib = _open(LIB)
    return _lib


def _open(path):
    lib = ctypes.CDLL(str(path))
    P = ctypes.c_void_p
    i64, i32, cint = ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    lib.oracle_abi_version.restype = cint
    lib.oracle_exp_spec.restype = ctypes.c_float
    lib.oracle_exp_spec.argtypes = [ctypes.c_float]
    lib.oracle_exp_spec_n.restype = None
    lib.oracle_exp_spec_n.argtypes = [P, P, i64]
    lib.oracle_softmax.restype = cint
    lib.oracle_softmax.argtypes = [P, i64, i32, P]
    lib.oracle_route.restype = cint
    lib.oracle_route.argtypes = [P, i64, i32, i32, i32, P, P]
    lib.oracle_logits.restype = cint
    lib.oracle_logits.argtypes = [P, cint, i64, i32, P, P, i32, P, cint]
    lib.oracle_experts.restype = cint
    lib.oracle_experts.argtypes = [P, cint, i64, i32, P, P, P, cint, i32, i32,
                                   i32, P, P, P, cint]
    lib.oracle_forward.restype = cint
    lib.oracle_forward.argtypes = [P, cint, i64, i32, P, P, i32, P, P, P, cint,
                                   i32, i32, i32, P, P, P, P, cint]
    lib.oracle_round_bf16_n.restype = None
    lib.oracle_round_bf16_n.argtypes = [P, P, i64]
    lib.oracle_logits_bf16.restype = cint
    lib.oracle_logits_bf16.argtypes = [P, i64, i32, P, i32, P, cint]
    lib.oracle_route_bf16w.restype = cint
    lib.oracle_route_bf16w.argtypes = [P, i64, i32, i32, i32, P, P]
    lib.oracle_forward_bf16_router.restype = cint
    lib.oracle_forward_bf16_router.argtypes = [P, i64, i32, P, i32, P, P, P, i32,
                                               i32, i32, P, P, P, P, cint]
    lib.oracle_shared.restype = cint
    lib.oracle_shared.argtypes = [P, cint, i64, i32, P, P, P, cint, i32, P, P, cint]
    lib.oracle_down_column_norms.restype = cint
    lib.oracle_down_column_norms.argtypes = [P, cint, i32, i32, i32, P]
    lib.oracle_channel_scores.restype = cint
    lib.oracle_channel_scores.argtypes = [P, cint, i64, i32, P, P, cint, i32, i32, i32, P, P,
                                          P, P]
    lib.oracle_channel_select.restype = cint
    lib.oracle_channel_select.argtypes = [P, i64, i32, i32, P]
    lib.oracle_experts_kept.restype = cint
    lib.oracle_experts_kept.argtypes = [P, cint, i64, i32, P, P, P, cint, i32, i32, i32, P, P,
                                        P, P]
    return lib


class using_library:
    """Context manager that points this module at another build of the oracle
    source (the mutation tests build copies with planted mistakes)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = _open(self.path)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


class OracleError(RuntimeError):
    pass


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} failed with status {rc}")


def _dtype_code(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"unsupported dtype {a.dtype} (float32, or uint16 bf16 bits)")


def _c(a, dtype=None):
    a = np.ascontiguousarray(a)
    if dtype is not None and a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def exp_spec(d):
    """exp_spec elementwise over a float32 array (d <= 0)."""
    lib = _load()
    d = _c(np.asarray(d, dtype=np.float32))
    out = np.empty_like(d)
    lib.oracle_exp_spec_n(_ptr(d), _ptr(out), d.size)
    return out


def softmax(logits):
    lib = _load()
    logits = _c(logits, np.float32)
    T, E = logits.shape
    p = np.empty_like(logits)
    _check(lib.oracle_softmax(_ptr(logits), T, E, _ptr(p)), "oracle_softmax")
    return p


def route(logits, k1: int, k2: int):
    """(ids [T,k1] int32, w [T,k1] float32) in rank order."""
    lib = _load()
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k1), np.int32)
    w = np.empty((T, k1), np.float32)
    _check(lib.oracle_route(_ptr(logits), T, E, k1, k2, _ptr(ids), _ptr(w)),
           "oracle_route")
    return ids, w


def logits(x, Wr, br=None, nthreads: int = 1):
    lib = _load()
    x = _c(x)
    Wr = _c(Wr, np.float32)
    br = None if br is None else _c(br, np.float32)
    T, H = x.shape
    E = Wr.shape[0]
    out = np.empty((T, E), np.float32)
    _check(lib.oracle_logits(_ptr(x), _dtype_code(x), T, H, _ptr(Wr), _ptr(br),
                             E, _ptr(out), nthreads), "oracle_logits")
    return out


def experts(x, Wg, Wu, Wd, ids, w, nthreads: int = 1):
    """y [T,H] float32 = sum_r w[t,r] * SwiGLU_{ids[t,r]}(x[t])."""
    lib = _load()
    x = _c(x)
    Wg, Wu, Wd = _c(Wg), _c(Wu), _c(Wd)
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    T, H = x.shape
    E, I, H2 = Wg.shape
    assert H2 == H and Wu.shape == Wg.shape and Wd.shape == (E, H, I)
    wt = _dtype_code(Wg)
    assert _dtype_code(Wu) == wt and _dtype_code(Wd) == wt
    k1 = ids.shape[1]
    y = np.empty((T, H), np.float32)
    _check(lib.oracle_experts(_ptr(x), _dtype_code(x), T, H, _ptr(Wg), _ptr(Wu),
                              _ptr(Wd), wt, E, I, k1, _ptr(ids), _ptr(w), _ptr(y),
                              nthreads), "oracle_experts")
    return y


def forward(x, Wr, Wg, Wu, Wd, k1: int, k2: int, br=None, nthreads: int = 1):
    """Whole layer: returns (y, logits, ids, w)."""
    lib = _load()
    x = _c(x)
    Wr = _c(Wr, np.float32)
    br = None if br is None else _c(br, np.float32)
    Wg, Wu, Wd = _c(Wg), _c(Wu), _c(Wd)
    T, H = x.shape
    E, I, _ = Wg.shape
    wt = _dtype_code(Wg)
    y = np.empty((T, H), np.float32)
    lg = np.empty((T, E), np.float32)
    ids = np.empty((T, k1), np.int32)
    w = np.empty((T, k1), np.float32)
    _check(lib.oracle_forward(_ptr(x), _dtype_code(x), T, H, _ptr(Wr), _ptr(br),
                              E, _ptr(Wg), _ptr(Wu), _ptr(Wd), wt, I, k1, k2,
                              _ptr(y), _ptr(lg), _ptr(ids), _ptr(w), nthreads),
           "oracle_forward")
    return y, lg, ids, w


def round_bf16(d):
    """float64 array -> float32 array of the nearest bf16 values (ties to even)."""
    lib = _load()
    d = _c(np.asarray(d, dtype=np.float64))
    out = np.empty(d.shape, np.float32)
    lib.oracle_round_bf16_n(_ptr(d), _ptr(out), d.size)
    return out


def logits_bf16(x, Wr, nthreads: int = 1):
    """bf16 router logits [T,E] (float32 holding bf16 values); x [T,H] and
    Wr [E,H] as uint16 bf16 bits."""
    lib = _load()
    x = _c(x, np.uint16)
    Wr = _c(Wr, np.uint16)
    T, H = x.shape
    E = Wr.shape[0]
    out = np.empty((T, E), np.float32)
    _check(lib.oracle_logits_bf16(_ptr(x), T, H, _ptr(Wr), E, _ptr(out), nthreads),
           "oracle_logits_bf16")
    return out


def route_bf16w(logits, k1: int, k2: int):
    """``route``, with each weight then cast to bf16 (returned as float32)."""
    lib = _load()
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k1), np.int32)
    w = np.empty((T, k1), np.float32)
    _check(lib.oracle_route_bf16w(_ptr(logits), T, E, k1, k2, _ptr(ids), _ptr(w)),
           "oracle_route_bf16w")
    return ids, w


def forward_bf16_router(x, Wr, Wg, Wu, Wd, k1: int, k2: int, nthreads: int = 1):
    """Whole layer with the bf16 router; every tensor uint16 bf16 bits.
    Returns (y, logits, ids, w)."""
    lib = _load()
    x, Wr = _c(x, np.uint16), _c(Wr, np.uint16)
    Wg, Wu, Wd = _c(Wg, np.uint16), _c(Wu, np.uint16), _c(Wd, np.uint16)
    T, H = x.shape
    E, I, _ = Wg.shape
    y = np.empty((T, H), np.float32)
    lg = np.empty((T, E), np.float32)
    ids = np.empty((T, k1), np.int32)
    w = np.empty((T, k1), np.float32)
    _check(lib.oracle_forward_bf16_router(_ptr(x), T, H, _ptr(Wr), E, _ptr(Wg), _ptr(Wu),
                                          _ptr(Wd), I, k1, k2, _ptr(y), _ptr(lg), _ptr(ids),
                                          _ptr(w), nthreads), "oracle_forward_bf16_router")
    return y, lg, ids, w


def shared(x, Sg, Su, Sd, sg=None, nthreads: int = 1):
    """The shared expert's term [T,H] float32: g * Sd (silu(Sg x) * (Su x)),
    g = sigmoid(x . sg) (sg [H] float32) or 1 without sg."""
    lib = _load()
    x = _c(x)
    Sg, Su, Sd = _c(Sg), _c(Su), _c(Sd)
    T, H = x.shape
    Is = Sg.shape[0]
    assert Sg.shape == (Is, H) and Su.shape == Sg.shape and Sd.shape == (H, Is)
    wt = _dtype_code(Sg)
    assert _dtype_code(Su) == wt and _dtype_code(Sd) == wt
    sg = None if sg is None else _c(sg, np.float32)
    ys = np.empty((T, H), np.float32)
    _check(lib.oracle_shared(_ptr(x), _dtype_code(x), T, H, _ptr(Sg), _ptr(Su), _ptr(Sd), wt,
                             Is, _ptr(sg), _ptr(ys), nthreads), "oracle_shared")
    return ys


def down_column_norms(Wd):
    """dn [E,I] float32: the 2-norm of each down column Wd[e,:,c]."""
    lib = _load()
    Wd = _c(Wd)
    E, H, I = Wd.shape
    dn = np.empty((E, I), np.float32)
    _check(lib.oracle_down_column_norms(_ptr(Wd), _dtype_code(Wd), E, H, I, _ptr(dn)),
           "oracle_down_column_norms")
    return dn


def channel_scores(x, Wg, Wu, ids, w, dn):
    """scores [T, k1*I] float32 = w_r * dn[e_r, c] * |silu(g) * u|."""
    lib = _load()
    x, Wg, Wu = _c(x), _c(Wg), _c(Wu)
    ids, w, dn = _c(ids, np.int32), _c(w, np.float32), _c(dn, np.float32)
    T, H = x.shape
    E, I, _ = Wg.shape
    k1 = ids.shape[1]
    out = np.empty((T, k1 * I), np.float32)
    _check(lib.oracle_channel_scores(_ptr(x), _dtype_code(x), T, H, _ptr(Wg), _ptr(Wu),
                                     _dtype_code(Wg), E, I, k1, _ptr(ids), _ptr(w), _ptr(dn),
                                     _ptr(out)), "oracle_channel_scores")
    return out


def channel_select(scores, keep: int):
    """kept [T, n] bool: the keep highest scores per row, lower index on ties."""
    lib = _load()
    scores = _c(scores, np.float32)
    T, n = scores.shape
    kept = np.zeros((T, n), np.uint8)
    _check(lib.oracle_channel_select(_ptr(scores), T, n, keep, _ptr(kept)),
           "oracle_channel_select")
    return kept.astype(bool)


def experts_kept(x, Wg, Wu, Wd, ids, w, kept):
    """y [T,H] float32 from the kept channels only."""
    lib = _load()
    x, Wg, Wu, Wd = _c(x), _c(Wg), _c(Wu), _c(Wd)
    ids, w = _c(ids, np.int32), _c(w, np.float32)
    kept = _c(np.asarray(kept, np.uint8))
    T, H = x.shape
    E, I, _ = Wg.shape
    k1 = ids.shape[1]
    assert kept.shape == (T, k1 * I)
    y = np.empty((T, H), np.float32)
    _check(lib.oracle_experts_kept(_ptr(x), _dtype_code(x), T, H, _ptr(Wg), _ptr(Wu), _ptr(Wd),
                                   _dtype_code(Wg), E, I, k1, _ptr(ids), _ptr(w), _ptr(kept),
                                   _ptr(y)), "oracle_experts_kept")
    return y
