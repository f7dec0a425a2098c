"""The C ABI library loads and exports what include/moe.h declares, and its
argument checks return before anything is launched (no GPU needed)."""
import ctypes
import re
from pathlib import Path

import pytest

import decoupled_top_routing_amd as moe

HEADER = Path(__file__).resolve().parents[1] / "include" / "moe.h"


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("moe_route", "moe_forward", "moe_forward_workspace", "moe_abi_version",
              "moe_status_str", "moe_last_error_str"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = moe.load_library()
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} not exported"
    assert lib.moe_abi_version() == moe.ABI_VERSION


def test_status_strings():
    lib = moe.load_library()
    for code in range(7):
        assert lib.moe_status_str(code)
    assert lib.moe_status_str(99) == b"unknown status"


def test_workspace_size():
    lib = moe.load_library()
    n1 = lib.moe_forward_workspace(1, 2048, 128, 768, 4, 1, 1)
    n8 = lib.moe_forward_workspace(8, 2048, 128, 768, 4, 1, 1)
    assert n1 > 0 and n1 % 256 == 0 and n8 > n1
    assert lib.moe_forward_workspace(1, 2048, 2000, 768, 4, 1, 1) == 0  # E > 1024
    assert lib.moe_forward_workspace(1, 2048, 128, 768, 0, 1, 1) == 0  # k1 = 0


def _route(lib, T, E, k1, k2, ptr=8):
    p = ctypes.c_void_p(ptr)
    return lib.moe_route(p, T, E, k1, k2, p, p, None)


@pytest.mark.parametrize("T,E,k1,k2,code", [
    (1, 0, 1, 1, 1),          # E < 1
    (1, 1025, 1, 1, 1),       # E > 1024
    (1, 16, 0, 4, 1),         # k1 < 1
    (1, 16, 17, 17, 1),       # k1 > E
    (1, 16, 4, 3, 1),         # k2 < k1
    (-1, 16, 2, 4, 1),        # T < 0
    ((1 << 18) + 1, 16, 2, 4, 1),   # T above the limit that keeps T*256 work-items in range
])
def test_route_rejects_bad_arguments(T, E, k1, k2, code):
    lib = moe.load_library()
    assert _route(lib, T, E, k1, k2) == code
    assert lib.moe_last_error_str()


def test_route_zero_tokens_is_a_no_op():
    lib = moe.load_library()
    assert _route(lib, 0, 16, 2, 4) == 0


def test_route_null_and_misaligned_pointers():
    lib = moe.load_library()
    assert lib.moe_route(None, 1, 16, 2, 4, None, None, None) == 1
    assert _route(lib, 1, 16, 2, 4, ptr=6) == 2


def _fwd(lib, **kw):
    a = dict(x=16, act=1, T=1, H=2048, Wr=16, br=None, E=128, Wg=16, Wu=16, Wd=16, wt=1,
             I=768, k1=4, k2=16, y=16, lo=None, io=None, wo=None, flags=0, ws=256,
             wsb=1 << 30, stream=None)
    a.update(kw)
    v = lambda p: None if p is None else ctypes.c_void_p(p)
    return lib.moe_forward(v(a["x"]), a["act"], a["T"], a["H"], v(a["Wr"]), v(a["br"]),
                           a["E"], v(a["Wg"]), v(a["Wu"]), v(a["Wd"]), a["wt"], a["I"],
                           a["k1"], a["k2"], v(a["y"]), v(a["lo"]), v(a["io"]), v(a["wo"]),
                           a["flags"], v(a["ws"]), a["wsb"], v(a["stream"]))


@pytest.mark.parametrize("kw,code", [
    (dict(k2=3), 1), (dict(H=100), 1), (dict(I=4), 1), (dict(E=2048), 1),
    (dict(act=0, wt=1), 4), (dict(act=1, wt=0), 4), (dict(act=2, wt=2), 4),
    (dict(x=24), 2), (dict(Wd=8), 2), (dict(br=2), 2),
    (dict(ws=None), 3), (dict(ws=128), 3), (dict(wsb=1024), 3),
    (dict(x=None), 1), (dict(flags=3), 1), (dict(flags=16), 1),
    (dict(flags=4, act=0, wt=0), 4), (dict(flags=4, I=776), 4), (dict(flags=4, H=2056), 4),
    # bit value 1 is not a flag (it was a retired path)
    (dict(flags=1), 1), (dict(flags=9), 1),
    # the bf16 router: bf16 pair only, no bias
    (dict(flags=8, act=0, wt=0), 4), (dict(flags=8, br=16), 1),
    (dict(flags=8 | 6), 1), (dict(flags=8 | 32), 1),
    # sizes whose launch grids would pass 2^32 work-items
    (dict(T=(1 << 18) + 1), 1), (dict(T=1 << 18, H=2048), 1), (dict(E=1024, H=65536), 1),
    (dict(E=1024, I=65536), 1),
])
def test_forward_rejects_bad_arguments(kw, code):
    lib = moe.load_library()
    assert _fwd(lib, **kw) == code, lib.moe_last_error_str()


def test_forward_zero_tokens_is_a_no_op():
    lib = moe.load_library()
    assert _fwd(lib, T=0, x=None, y=None, ws=None, wsb=0) == 0


def _fwd_shared(lib, **kw):
    a = dict(x=16, act=1, T=1, H=2048, Wr=16, br=None, E=128, Wg=16, Wu=16, Wd=16, wt=1,
             I=768, k1=4, k2=16, Sg=16, Su=16, Sd=16, Is=768, sg=None, y=16, lo=None,
             io=None, wo=None, flags=0, ws=256, wsb=1 << 30, stream=None)
    a.update(kw)
    v = lambda p: None if p is None else ctypes.c_void_p(p)
    return lib.moe_forward_shared(v(a["x"]), a["act"], a["T"], a["H"], v(a["Wr"]), v(a["br"]),
                                  a["E"], v(a["Wg"]), v(a["Wu"]), v(a["Wd"]), a["wt"], a["I"],
                                  a["k1"], a["k2"], v(a["Sg"]), v(a["Su"]), v(a["Sd"]), a["Is"],
                                  v(a["sg"]), v(a["y"]), v(a["lo"]), v(a["io"]), v(a["wo"]),
                                  a["flags"], v(a["ws"]), a["wsb"], v(a["stream"]))


@pytest.mark.parametrize("kw,code", [
    (dict(Sg=None), 1), (dict(Sd=None), 1), (dict(Is=4), 1), (dict(Is=772), 1),
    (dict(Sg=24), 2), (dict(Sd=8), 2), (dict(sg=2), 2),
    (dict(flags=1), 1),                   # not a flag
    (dict(flags=4, Is=72), 4),            # the prefill path needs Is % 64 == 0
    (dict(T=1 << 17, Is=4096), 1),        # T*Is above 2^28
    (dict(k2=3), 1), (dict(ws=None), 3),
])
def test_forward_shared_rejects_bad_arguments(kw, code):
    lib = moe.load_library()
    assert _fwd_shared(lib, **kw) == code, lib.moe_last_error_str()


def test_forward_shared_workspace_size():
    lib = moe.load_library()
    plain = lib.moe_forward_workspace(8, 2048, 128, 768, 4, 1, 1)
    assert lib.moe_forward_shared_workspace(8, 2048, 128, 768, 4, 0, 1, 1) == plain
    sh = lib.moe_forward_shared_workspace(8, 2048, 128, 768, 4, 1536, 1, 1)
    assert sh > plain and sh % 256 == 0
    assert lib.moe_forward_shared_workspace(8, 2048, 128, 768, 4, 4, 1, 1) == 0


def test_forward_shared_zero_tokens_is_a_no_op():
    lib = moe.load_library()
    assert _fwd_shared(lib, T=0, x=None, y=None, ws=None, wsb=0) == 0


def test_channel_topk_argument_checks():
    lib = moe.load_library()
    v = ctypes.c_void_p
    # down column norms: E out of range, misaligned Wdown, unsupported dtype
    assert lib.moe_down_column_norms(v(16), 1, 0, 2048, 768, v(16), None) == 1
    assert lib.moe_down_column_norms(v(8), 1, 128, 2048, 768, v(16), None) == 2
    assert lib.moe_down_column_norms(v(16), 7, 128, 2048, 768, v(16), None) == 4

    def fwd(**kw):
        a = dict(k1=4, keep=100, dn=16, flags=0, cols=None)
        a.update(kw)
        return lib.moe_forward_channel_topk(v(16), 1, 1, 2048, v(16), None, 128, v(16), v(16),
                                            v(16), 1, 768, a["k1"], 16,
                                            None if a["dn"] is None else v(a["dn"]), a["keep"],
                                            None if a["cols"] is None else v(a["cols"]),
                                            v(16), None, None, None, None, None, a["flags"],
                                            v(256), 1 << 30, None)
    assert fwd(dn=None) == 1
    assert fwd(keep=-1) == 1
    assert fwd(keep=4 * 768 + 1) == 1
    assert fwd(k1=11, keep=10) == 4          # k1*I > 8192
    assert fwd(flags=4) == 4                 # prefill path
    assert fwd(flags=1) == 1                 # not a flag
    assert fwd(dn=2) == 2                    # misaligned dnorm
    assert fwd(dn=20) == 2                   # dnorm needs 16-byte alignment
    assert fwd(cols=24) == 2                 # the column copy needs 16-byte alignment
    # the column copy: E out of range, misaligned, unsupported dtype
    assert lib.moe_down_columns(v(16), 1, 0, 2048, 768, v(16), None) == 1
    assert lib.moe_down_columns(v(16), 1, 128, 2048, 768, v(8), None) == 2
    assert lib.moe_down_columns(v(16), 7, 128, 2048, 768, v(16), None) == 4
    # its workspace holds the kept list and the partial sums beyond the grouped
    # path's buffers: never smaller than moe_forward's, and 0 for invalid sizes
    for T in (1, 8, 64):
        assert lib.moe_forward_channel_topk_workspace(T, 2048, 128, 768, 4, 1, 1) >= \
            lib.moe_forward_workspace(T, 2048, 128, 768, 4, 1, 1)
    assert lib.moe_forward_channel_topk_workspace(1, 2048, 128, 768, 0, 1, 1) == 0


def test_workspace_status_argument_checks():
    lib = moe.load_library()
    assert lib.moe_workspace_status(None, None) == 1
    assert lib.moe_workspace_status(ctypes.c_void_p(128), None) == 3


def test_withhold_route_hook_argument_checks():
    lib = moe.load_library()
    assert lib.moe_debug_withhold_route(-1, 64) == 1
    assert lib.moe_debug_withhold_route(1, 0) == 1
    assert lib.moe_debug_withhold_route(0, 1) == 0     # disarmed


def test_workspace_size_is_the_same_for_calls_of_any_shape_prefix():
    """The sync region and the one-token kernel's tagged region sit at fixed
    places: a workspace for one shape starts with the same fixed part as one
    for any other, so calls of different shapes can share it."""
    lib = moe.load_library()
    small = lib.moe_forward_workspace(1, 256, 16, 64, 2, 0, 0)
    big = lib.moe_forward_workspace(1, 4096, 1024, 1024, 32, 1, 1)
    assert 0 < small < big
