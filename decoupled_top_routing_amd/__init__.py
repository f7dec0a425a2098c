"""Routed MoE layer with decoupled top-k1/k2 weights on AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libmoe.so`` (declared in
``include/moe.h``).  Every step of the layer runs in the library's HIP
kernels; this module only checks tensors, allocates outputs and workspace with
torch, and passes pointers and the current stream.  There is no CPU fallback:
if the library is missing or cannot be loaded, every call raises.

The method: "Paper of the Week #3 - Half the FLOPs Is Not Half the Time",
section "The Receipt", Eq. 2 -- activate the top-k1 experts, each weighted by
its probability over the probability mass of the top-k2 experts (k2 = k1:
standard renormalisation; k2 >= E: none).
"""
from __future__ import annotations

import ctypes
import threading
from pathlib import Path

import torch

__all__ = ["route", "forward", "forward_channel_topk", "down_column_norms", "down_columns",
           "workspace_status",
           "MoeError", "library_path", "load_library",
           "F32", "BF16", "FORCE_GROUPED", "FORCE_PREFILL", "ROUTER_BF16"]

PKG = Path(__file__).resolve().parent
LIB_PATH = PKG / "libmoe.so"

F32, BF16 = 0, 1
FORCE_GROUPED, FORCE_PREFILL = 2, 4
ROUTER_BF16 = 8
ABI_VERSION = 2

_STATUS = {0: "MOE_OK", 1: "MOE_EINVAL", 2: "MOE_EALIGN", 3: "MOE_EWORKSPACE",
           4: "MOE_ENOTSUP", 5: "MOE_EHIP", 6: "MOE_EDEVICE"}

_lib = None
_lock = threading.Lock()


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_STATUS.get(code, code)}: {msg}")
        self.code = code


def library_path() -> Path:
    return LIB_PATH


def load_library():
    """Load libmoe.so (once); raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not LIB_PATH.exists():
            raise MoeError(-1, f"{LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(str(LIB_PATH))
        P, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
        lib.moe_abi_version.restype = ctypes.c_int
        lib.moe_status_str.restype = ctypes.c_char_p
        lib.moe_status_str.argtypes = [ctypes.c_int]
        lib.moe_last_error_str.restype = ctypes.c_char_p
        lib.moe_route.restype = ctypes.c_int
        lib.moe_route.argtypes = [P, i64, i32, i32, i32, P, P, P]
        lib.moe_forward_workspace.restype = ctypes.c_size_t
        lib.moe_forward_workspace.argtypes = [i64, i32, i32, i32, i32, i32, i32]
        lib.moe_forward.restype = ctypes.c_int
        lib.moe_forward.argtypes = [P, i32, i64, i32, P, P, i32, P, P, P, i32, i32, i32,
                                    i32, P, P, P, P, u32, P, ctypes.c_size_t, P]
        lib.moe_forward_shared.restype = ctypes.c_int
        lib.moe_forward_shared.argtypes = [P, i32, i64, i32, P, P, i32, P, P, P, i32, i32, i32,
                                           i32, P, P, P, i32, P, P, P, P, P, u32, P,
                                           ctypes.c_size_t, P]
        lib.moe_down_column_norms.restype = ctypes.c_int
        lib.moe_down_column_norms.argtypes = [P, i32, i32, i32, i32, P, P]
        lib.moe_forward_channel_topk.restype = ctypes.c_int
        lib.moe_forward_channel_topk.argtypes = [P, i32, i64, i32, P, P, i32, P, P, P, i32, i32,
                                                 i32, i32, P, i32, P, P, P, P, P, P, P, u32, P,
                                                 ctypes.c_size_t, P]
        lib.moe_forward_channel_topk_workspace.restype = ctypes.c_size_t
        lib.moe_forward_channel_topk_workspace.argtypes = [i64, i32, i32, i32, i32, i32, i32]
        lib.moe_down_columns.restype = ctypes.c_int
        lib.moe_down_columns.argtypes = [P, i32, i32, i32, i32, P, P]
        lib.moe_forward_shared_workspace.restype = ctypes.c_size_t
        lib.moe_forward_shared_workspace.argtypes = [i64, i32, i32, i32, i32, i32, i32, i32]
        lib.moe_profile_launch.restype = ctypes.c_int
        lib.moe_profile_launch.argtypes = [i32, P, P]
        lib.moe_profile_launch_name.restype = ctypes.c_char_p
        lib.moe_workspace_status.restype = ctypes.c_int
        lib.moe_workspace_status.argtypes = [P, P]
        lib.moe_debug_withhold_route.restype = ctypes.c_int
        lib.moe_debug_withhold_route.argtypes = [i32, u32]
        lib.moe_forward_noalloc.restype = ctypes.c_int
        lib.moe_forward_noalloc.argtypes = [P, i32, i64, i32, P, P, i32, P, P, P, i32, i32, i32,
                                            i32, P, P, P, P, u32, P]
        lib.moe_noalloc_scratch_bytes.restype = ctypes.c_size_t
        lib.moe_noalloc_scratch_bytes.argtypes = []
        lib.moe_hbm_read_probe.restype = ctypes.c_int
        lib.moe_hbm_read_probe.argtypes = [P, ctypes.c_size_t, P, i32, P]
        if lib.moe_abi_version() != ABI_VERSION:
            raise MoeError(-1, f"libmoe ABI {lib.moe_abi_version()} != {ABI_VERSION}")
        _lib = lib
        return lib


def _check(rc: int):
    if rc != 0:
        lib = load_library()
        raise MoeError(rc, lib.moe_last_error_str().decode(errors="replace"))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_cuda(name, t, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise MoeError(1, f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise MoeError(1, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise MoeError(4, f"{name} must be {dtype}, got {t.dtype}")


def _dtype_code(t) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise MoeError(4, f"unsupported dtype {t.dtype}")


def route(logits: torch.Tensor, k1: int, k2: int):
    """ids [T,k1] int32 and Eq. 2 weights [T,k1] fp32 from fp32 logits [T,E]."""
    lib = load_library()
    _need_cuda("logits", logits, torch.float32)
    T, E = logits.shape
    ids = torch.empty((T, k1), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, k1), dtype=torch.float32, device=logits.device)
    _check(lib.moe_route(_ptr(logits), T, E, k1, k2, _ptr(ids), _ptr(w),
                         _stream(logits.device)))
    return ids, w


def profile_launch(launch: int, start, stop):
    """Arm the next forward() on this thread to record the torch.cuda.Event
    objects start and stop (timing enabled) right before and right after its
    kernel launch number `launch` (moe_profile_launch)."""
    lib = load_library()
    for ev in (start, stop):
        if ev.cuda_event == 0:
            ev.record()  # creates the event; the library records it again
    _check(lib.moe_profile_launch(launch, ctypes.c_void_p(start.cuda_event),
                                  ctypes.c_void_p(stop.cuda_event)))


def profile_launch_name() -> str:
    """Kernel name of the launch bracketed by the last armed forward()."""
    return load_library().moe_profile_launch_name().decode()


# One zero-filled workspace per (device, stream), grown on demand (a new one
# is zero-filled again).  It can serve calls of any shape: the library keeps
# its hand-over words at fixed places with call tags that do not repeat for
# 2^31 calls.
_workspaces: dict = {}


def _workspace(device, stream_ptr: int, nbytes: int) -> torch.Tensor:
    key = (device, stream_ptr)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def workspace_status(workspace=None, device=None):
    """Wait for the current stream and read and reset the device status word of
    ``workspace`` (default: this module's workspace for the current device and
    stream); raises MoeError (MOE_EDEVICE) if a hand-over wait inside a kernel
    gave up since the last check (moe_workspace_status)."""
    lib = load_library()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    stream = _stream(dev)
    if workspace is None:
        workspace = _workspaces.get((dev, stream.value or 0))
        if workspace is None:
            return
    _need_cuda("workspace", workspace, torch.uint8)
    _check(lib.moe_workspace_status(_ptr(workspace), stream))


def debug_withhold_route(calls: int, spin_limit: int = 64):
    """Test hook (moe_debug_withhold_route): the next ``calls`` one-token calls
    on this thread do not publish their route; their waits give up after
    ``spin_limit`` re-reads and set the device status word."""
    _check(load_library().moe_debug_withhold_route(calls, spin_limit))


def hbm_read_probe(buf: torch.Tensor, out: torch.Tensor, blocks: int):
    """Measurement aid (moe_hbm_read_probe): stream-read every byte of the
    contiguous device tensor ``buf`` once; ``out`` is a uint32/int32 device
    tensor of at least ``blocks`` elements."""
    lib = load_library()
    _need_cuda("buf", buf)
    _need_cuda("out", out)
    if out.numel() < blocks or out.element_size() != 4:
        raise MoeError(1, "out needs `blocks` 4-byte elements")
    _check(lib.moe_hbm_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out),
                                  blocks, _stream(buf.device)))


def forward(x, Wr, Wgate, Wup, Wdown, k1: int, k2: int, br=None,
            return_route: bool = False, flags: int = 0, out=None, workspace=None,
            shared=None, noalloc: bool = False):
    """The whole routed MoE layer.

    x [T,H] (fp32 or bf16), Wr [E,H] fp32, br [E] fp32 or None, Wgate and Wup
    [E,I,H], Wdown [E,H,I] in the dtype of x.  Returns y [T,H] in x's dtype,
    or (y, logits, ids, w) with ``return_route=True``.

    A bf16 ``Wr`` selects the bf16 router (``ROUTER_BF16``, the page's router
    method on a bf16 model): bf16 logits, fp32 softmax and Eq. 2, weights
    rounded to bf16; it takes bf16 x and expert weights and no ``br``.

    ``shared`` = (Sgate [Is,H], Sup [Is,H], Sdown [H,Is]) or the same with a
    fourth fp32 gate vector sgate [H] adds the shared expert, which runs on
    every token: y += sigmoid(x . sgate) (or 1) * Sdown(silu(Sgate x) * Sup x).  ``out`` receives y if
    given; ``workspace`` is an optional zero-filled uint8 device tensor of at
    least ``moe_forward_workspace`` bytes (needed under graph capture, where
    nothing may be allocated).
    """
    lib = load_library()
    _need_cuda("x", x)
    act = _dtype_code(x)
    if Wr.dtype == torch.bfloat16:
        flags |= ROUTER_BF16
    _need_cuda("Wr", Wr, torch.bfloat16 if flags & ROUTER_BF16 else torch.float32)
    for n, t in (("Wgate", Wgate), ("Wup", Wup), ("Wdown", Wdown)):
        _need_cuda(n, t, x.dtype)
    if br is not None:
        _need_cuda("br", br, torch.float32)
    T, H = x.shape
    E, I, H2 = Wgate.shape
    if H2 != H or Wup.shape != Wgate.shape or tuple(Wdown.shape) != (E, H, I) \
            or tuple(Wr.shape) != (E, H):
        raise MoeError(1, "shape mismatch between x, Wr, Wgate, Wup and Wdown")
    Is, sgate = 0, None
    if shared is not None:
        Sg, Su, Sd = shared[:3]
        sgate = shared[3] if len(shared) > 3 else None
        for n, t in (("Sgate", Sg), ("Sup", Su), ("Sdown", Sd)):
            _need_cuda(n, t, x.dtype)
        Is = Sg.shape[0]
        if tuple(Sg.shape) != (Is, H) or Su.shape != Sg.shape or tuple(Sd.shape) != (H, Is):
            raise MoeError(1, "shape mismatch between x, Sgate, Sup and Sdown")
        if sgate is not None:
            _need_cuda("sgate", sgate, torch.float32)
            if tuple(sgate.shape) != (H,):
                raise MoeError(1, "sgate must be [H]")
    dev = x.device
    y = out if out is not None else torch.empty((T, H), dtype=x.dtype, device=dev)
    lg = ids = w = None
    if return_route:
        lg = torch.empty((T, E), dtype=torch.float32, device=dev)
        ids = torch.empty((T, k1), dtype=torch.int32, device=dev)
        w = torch.empty((T, k1), dtype=torch.float32, device=dev)
    stream = _stream(dev)
    if noalloc:
        if shared is not None or workspace is not None:
            raise MoeError(1, "noalloc takes neither a shared expert nor a workspace")
        _check(lib.moe_forward_noalloc(_ptr(x), act, T, H, _ptr(Wr), _ptr(br), E, _ptr(Wgate),
                                       _ptr(Wup), _ptr(Wdown), act, I, k1, k2, _ptr(y), _ptr(lg),
                                       _ptr(ids), _ptr(w), flags, stream))
        return (y, lg, ids, w) if return_route else y
    nbytes = lib.moe_forward_shared_workspace(T, H, E, I, k1, Is, act, act)
    if nbytes == 0 and T > 0:
        raise MoeError(1, f"invalid sizes T={T} H={H} E={E} I={I} k1={k1}")
    if workspace is not None:
        _need_cuda("workspace", workspace, torch.uint8)
        ws = workspace
    else:
        ws = _workspace(dev, stream.value or 0, nbytes)
    if shared is None:
        _check(lib.moe_forward(_ptr(x), act, T, H, _ptr(Wr), _ptr(br), E, _ptr(Wgate),
                               _ptr(Wup), _ptr(Wdown), act, I, k1, k2, _ptr(y), _ptr(lg),
                               _ptr(ids), _ptr(w), flags, _ptr(ws), ws.numel(), stream))
    else:
        _check(lib.moe_forward_shared(_ptr(x), act, T, H, _ptr(Wr), _ptr(br), E, _ptr(Wgate),
                                      _ptr(Wup), _ptr(Wdown), act, I, k1, k2, _ptr(Sg), _ptr(Su),
                                      _ptr(Sd), Is, _ptr(sgate), _ptr(y), _ptr(lg), _ptr(ids),
                                      _ptr(w), flags, _ptr(ws), ws.numel(), stream))
    if return_route:
        return y, lg, ids, w
    return y


def down_column_norms(Wdown):
    """dnorm [E, I] fp32: the 2-norm of each down column Wdown[e, :, c]."""
    lib = load_library()
    _need_cuda("Wdown", Wdown)
    E, H, I = Wdown.shape
    dn = torch.empty((E, I), dtype=torch.float32, device=Wdown.device)
    _check(lib.moe_down_column_norms(_ptr(Wdown), _dtype_code(Wdown), E, H, I, _ptr(dn),
                                     _stream(Wdown.device)))
    return dn


def down_columns(Wdown):
    """The column copy [E, I, H] of Wdown [E, H, I] (moe_down_columns): each
    channel's down column as one contiguous row."""
    lib = load_library()
    _need_cuda("Wdown", Wdown)
    E, H, I = Wdown.shape
    cols = torch.empty((E, I, H), dtype=Wdown.dtype, device=Wdown.device)
    _check(lib.moe_down_columns(_ptr(Wdown), _dtype_code(Wdown), E, H, I, _ptr(cols),
                                _stream(Wdown.device)))
    return cols


def forward_channel_topk(x, Wr, Wgate, Wup, Wdown, k1: int, k2: int, dnorm, keep: int,
                         br=None, return_route: bool = False, flags: int = 0, out=None,
                         workspace=None, Wdown_cols=None):
    """The layer with channel top-k inside the activated experts: of each
    token's k1*I channels only the ``keep`` highest-scoring (router weight x
    down-column norm x |activation|) are summed.  ``dnorm`` comes from
    ``down_column_norms``; with ``Wdown_cols`` (from ``down_columns``) the down
    projection reads only the kept channels' columns.  Returns y, or (y,
    logits, ids, w, scores, kept) with ``return_route=True`` (scores [T, k1*I]
    fp32, kept [T, k1*I] bool).  ``out`` and ``workspace`` as for ``forward``."""
    lib = load_library()
    _need_cuda("x", x)
    act = _dtype_code(x)
    if Wr.dtype == torch.bfloat16:
        flags |= ROUTER_BF16
    _need_cuda("Wr", Wr, torch.bfloat16 if flags & ROUTER_BF16 else torch.float32)
    for n, t in (("Wgate", Wgate), ("Wup", Wup), ("Wdown", Wdown)):
        _need_cuda(n, t, x.dtype)
    _need_cuda("dnorm", dnorm, torch.float32)
    if br is not None:
        _need_cuda("br", br, torch.float32)
    T, H = x.shape
    E, I, H2 = Wgate.shape
    if H2 != H or Wup.shape != Wgate.shape or tuple(Wdown.shape) != (E, H, I) \
            or tuple(Wr.shape) != (E, H) or tuple(dnorm.shape) != (E, I):
        raise MoeError(1, "shape mismatch between x, Wr, Wgate, Wup, Wdown and dnorm")
    if Wdown_cols is not None:
        _need_cuda("Wdown_cols", Wdown_cols, x.dtype)
        if tuple(Wdown_cols.shape) != (E, I, H):
            raise MoeError(1, "Wdown_cols must be [E, I, H]")
    dev = x.device
    y = out if out is not None else torch.empty((T, H), dtype=x.dtype, device=dev)
    lg = ids = w = sc = kept = None
    if return_route:
        lg = torch.empty((T, E), dtype=torch.float32, device=dev)
        ids = torch.empty((T, k1), dtype=torch.int32, device=dev)
        w = torch.empty((T, k1), dtype=torch.float32, device=dev)
        sc = torch.empty((T, k1 * I), dtype=torch.float32, device=dev)
        kept = torch.empty((T, k1 * I), dtype=torch.uint8, device=dev)
    nbytes = lib.moe_forward_channel_topk_workspace(T, H, E, I, k1, act, act)
    if nbytes == 0 and T > 0:
        raise MoeError(1, f"invalid sizes T={T} H={H} E={E} I={I} k1={k1}")
    stream = _stream(dev)
    if workspace is not None:
        _need_cuda("workspace", workspace, torch.uint8)
        ws = workspace
    else:
        ws = _workspace(dev, stream.value or 0, nbytes)
    _check(lib.moe_forward_channel_topk(_ptr(x), act, T, H, _ptr(Wr), _ptr(br), E, _ptr(Wgate),
                                        _ptr(Wup), _ptr(Wdown), act, I, k1, k2, _ptr(dnorm), keep,
                                        _ptr(Wdown_cols), _ptr(y), _ptr(lg), _ptr(ids), _ptr(w),
                                        _ptr(sc), _ptr(kept), flags, _ptr(ws), ws.numel(),
                                        stream))
    if return_route:
        return y, lg, ids, w, sc, kept.bool()
    return y
