#!/usr/bin/env python3
"""Benchmark of the routed MoE layer with Eq. 2 weights on one MI355X.

A step is one call of the whole layer (router, route, experts, combine) on one
batch.  The headline workload is batch-1 decode on the H=2048, E=128, I=768
bf16 layer with k1:k2 = 4:16, run over a ring of 32 distinct seeded layers
(38.7 GB) so that every layer's weights come from HBM, not from the 256 MB
Infinity Cache.  Each cell's ring is captured once in a HIP graph and
replayed; HIP events on the capture stream time the replays.  The other cells
(batch 1 and 8 at every k1:k2 pair, the 4096-token prefill, the E=512 layer
at 1 and 64 tokens) are reported in "cells".

The timed region of the headline is exactly --steps layer calls (whole ring
replays, then the remaining calls launched one by one), queued behind a short
GPU spin so that it holds the calls back to back and not the host's
submission of them; the spread is reported from at least 10 ring replays
timed one by one the same way.

The roofline object is for the headline's dominant kernel: every launch of
one call is bracketed with HIP events (moe_profile_launch) in an eager pass,
the longest is the dominant one; when a call is that one launch, the timed
region gives its average duration.

The last line of stdout is one compact JSON object (the benchmark contract);
every cell is printed to stderr as a JSON line and, with --cells-out, written
to a file.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
# a GPU spin (torch.cuda._sleep, clock cycles) queued ahead of each timed
# region: about 2 ms, longer than the host takes to queue a ring of calls
GPU_SPIN_CYCLES = 5_000_000
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA, TFLOP/s
RING = 32
PATH_FLAGS = {"auto": 0, "g": 2, "p": 4}
TOPK_FRAC = 0.18  # channel top-k cells keep this share of a token's k1*I channels
DEFAULT_CELLS = ",".join([
    "C2:1:4:16", "C2:1:8:8", "C2:1:4:4", "C2:1:4:128", "C2:1:3:16", "C2:1:2:16",
    "C3:8:4:16", "C3:8:8:8", "C3:8:4:4", "C3:8:4:128", "C3:8:3:16", "C3:8:2:16",
    "C4:4096:4:16", "C4:4096:8:8",
    # batch sweep of the decode layer (the ring's layers, more tokens)
    "C3:2:4:16", "C3:2:8:8", "C3:4:4:16", "C3:4:8:8", "C3:16:4:16", "C3:16:8:8",
    "C3:32:4:16", "C3:32:8:8", "C3:64:4:16", "C3:64:8:8", "C3:128:4:16", "C3:128:8:8",
    "C3:256:4:16", "C3:256:8:8",
    "C5:1:10:10", "C5:1:5:5", "C5:1:5:20", "C5:64:10:10", "C5:64:5:5", "C5:64:5:20",
    # the bf16 router (router weight bf16, bf16 logits and weights), same layers
    "C2h:1:4:16", "C2h:1:8:8", "C3h:8:4:16", "C3h:8:8:8", "C4h:4096:4:16", "C4h:4096:8:8",
    # plus a gated shared expert of I channels, same layers
    "C2s:1:4:16", "C2s:1:8:8", "C3s:8:4:16", "C3s:8:8:8", "C4s:4096:4:16", "C4s:4096:8:8",
    # channel top-k: 18% of each token's k1*I channels kept, same layers
    "C2k:1:4:16", "C2k:1:8:8", "C3k:8:4:16", "C3k:8:8:8",
    # the tiny fp32 layer (latency only)
    "C1:8:2:4", "C1:8:2:2", "C1:8:2:16",
])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=6400,
                    help="timed layer calls of the headline cell")
    ap.add_argument("--warmup", type=int, default=320)
    ap.add_argument("--ring", type=int, default=RING)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cells-out", default=None, help="write every cell as a JSON line here")
    ap.add_argument("--cells", default=DEFAULT_CELLS,
                    help="CONFIG:T:k1:k2[:path] list; the first is the headline; a "
                         "CONFIG ending in h runs that config's layers with the bf16 router, "
                         "one ending in s adds a gated shared expert of I channels, one "
                         "ending in k keeps the top 18%% of each token's channels")
    return ap.parse_args()


# ------------------------------------------------------------------ workloads
def make_sets(synth, torch, names, ring):
    """Device layers per configuration name; NAMEh is NAME's layers with the
    router weight cast to bf16 and no bias (the bf16 router), NAMEs adds a
    gated shared expert of I channels to each layer."""
    sets = {}
    t0 = time.perf_counter()
    base = {n[:2] for n in names}
    if "C1" in base:
        sets["C1"] = (synth.TINY, [synth.make_layer(synth.TINY, layer=i, device="cuda")
                                   for i in range(ring)])
    if base & {"C2", "C3"}:
        # x holds 256 tokens; a cell of T tokens uses the first T
        sets["C2"] = sets["C3"] = (synth.DECODE_B8,
                                   [synth.make_layer(synth.DECODE_B8, layer=i, device="cuda",
                                                     T=256)
                                    for i in range(ring)])
    if "C4" in base:
        # one layer, called 8 times per graph (its 1.2 GB of weights exceed the
        # 256 MB Infinity Cache, so each call reads them from HBM); a graph of
        # one call would time the gap between two graph launches with it
        lay = synth.make_layer(synth.PREFILL, device="cuda")
        sets["C4"] = (synth.PREFILL, [lay] * 8)
    if "C5" in base:
        cfg = synth.LARGE
        sets["C5"] = (cfg, [synth.make_layer(cfg, layer=i, device="cuda", T=64)
                            for i in range(cfg.layers)])
    for n in names:
        if n.endswith("h"):
            cfg, layers = sets[n[:2]]
            sets[n] = (cfg, [dict(lay, Wr=lay["Wr"].to(torch.bfloat16), br=None)
                             for lay in layers])
        elif n.endswith("s"):
            cfg, layers = sets[n[:2]]
            sets[n] = (cfg, [dict(lay, shared=synth.make_shared(cfg, cfg.I, gate=True, layer=i,
                                                                device="cuda"))
                             for i, lay in enumerate(layers)])
        elif n.endswith("k"):
            import decoupled_top_routing_amd as moe
            cfg, layers = sets[n[:2]]
            sets[n] = (cfg, [dict(lay, topk={"dn": moe.down_column_norms(lay["Wd"]),
                                             "cols": moe.down_columns(lay["Wd"]),
                                             "frac": TOPK_FRAC})
                             for lay in layers])
    torch.cuda.synchronize()
    print(f"# generated {sorted(names)} on the device in {time.perf_counter() - t0:.1f} s",
          file=sys.stderr, flush=True)
    return sets


def unique_experts(ids_list):
    return sum(len(set(ids.flatten().tolist())) for ids in ids_list) / len(ids_list)


def expert_bytes(cfg, U):
    return 3 * cfg.I * cfg.H * (2 if cfg.dtype == "bf16" else 4) * U


def shared_bytes(cfg, lay):
    """Weights of the layer's shared expert (gate, up, down, gate vector), or 0."""
    sh = lay.get("shared")
    if not sh:
        return 0
    return sum(sh[k].numel() * sh[k].element_size() for k in ("Sg", "Su", "Sd", "sg")
               if sh[k] is not None)


def layer_bytes(cfg, T, U, bias, wr_elt=4, shared=0):
    """Algorithmic bytes of one call: activated experts, shared expert, router, x, y."""
    elt = 2 if cfg.dtype == "bf16" else 4
    return expert_bytes(cfg, U) + shared + cfg.E * cfg.H * wr_elt + \
        (cfg.E * 4 if bias else 0) + 2 * T * cfg.H * elt


def expert_flops(cfg, T, k1):
    return 6.0 * T * k1 * cfg.H * cfg.I


def kernel_work(name, cfg, T, k1, U, bias, wr_elt=4, shared=0):
    """(algorithmic bytes, flops) of one launch of the named kernel."""
    elt = 2 if cfg.dtype == "bf16" else 4
    H, E, I = cfg.H, cfg.E, cfg.I
    router = E * H * wr_elt + (E * 4 if bias else 0) + T * H * elt
    gu = 2 * U * I * H * elt
    dn = U * I * H * elt
    n = T * k1
    table = {
        "b1_layer": (layer_bytes(cfg, T, U, bias, wr_elt, shared),
                     2.0 * E * H + expert_flops(cfg, T, k1)),
        "router": (router + T * E * 4, 2.0 * T * E * H),
        "router_route": (router, 2.0 * T * E * H),
        "gateup": (gu + T * H * elt, 4.0 * n * I * H),
        "down": (dn, 2.0 * n * I * H),
        "down_one_token": (dn + H * elt, 2.0 * n * I * H),
        "router_mma": (router + T * E * 4, 2.0 * T * E * H),
        "gateup_mma": (gu + T * H * elt, 4.0 * n * I * H),
        "down_mma": (dn, 2.0 * n * I * H),
    }
    return table.get(name, (None, None))


def layer_call(moe, lay, x, k1, k2, cfg, **kw):
    """One moe call on a layer dict: channel top-k layers go through
    forward_channel_topk, the others through forward (with their shared expert)."""
    ck = lay.get("topk")
    if ck:
        keep = int(round(ck["frac"] * k1 * cfg.I))
        rr = kw.pop("return_route", False)
        r = moe.forward_channel_topk(x, lay["Wr"], lay["Wg"], lay["Wu"], lay["Wd"], k1, k2,
                                     ck["dn"], keep, br=lay["br"], return_route=rr,
                                     Wdown_cols=ck["cols"], **kw)
        return r[:4] if rr else r
    return moe.forward(x, lay["Wr"], lay["Wg"], lay["Wu"], lay["Wd"], k1, k2, br=lay["br"],
                       shared=shared_args(lay), **kw)


def shared_args(lay):
    """moe.forward's shared argument for a layer dict (None without one)."""
    sh = lay.get("shared")
    if not sh:
        return None
    return (sh["Sg"], sh["Su"], sh["Sd"]) + ((sh["sg"],) if sh["sg"] is not None else ())


# ------------------------------------------------------------------ timing
def time_cell(moe, torch, cfg, layers, T, k1, k2, path, steps, warmup, min_replays=0):
    """Graph-capture one pass over the layers; time exactly `steps` layer calls
    (whole ring replays, then a graph of the first steps % ring calls), then
    at least `min_replays` whole replays one by one for the spread."""
    dev = layers[0]["Wg"].device
    L = len(layers)
    stream = torch.cuda.Stream(device=dev)
    xs = [lay["x"][:T].contiguous() for lay in layers]
    ys = [torch.empty_like(x) for x in xs]
    lib = moe.load_library()
    act = 1 if cfg.dtype == "bf16" else 0
    Is = layers[0]["shared"]["Sg"].shape[0] if layers[0].get("shared") else 0
    nws = (lib.moe_forward_channel_topk_workspace(T, cfg.H, cfg.E, cfg.I, k1, act, act)
           if layers[0].get("topk") else
           lib.moe_forward_shared_workspace(T, cfg.H, cfg.E, cfg.I, k1, Is, act, act))
    ws = torch.zeros(nws, dtype=torch.uint8, device=dev)
    ids_list = []

    def one_pass(n=L, record_ids=False):
        for i in range(n):
            r = layer_call(moe, layers[i], xs[i], k1, k2, cfg, out=ys[i], workspace=ws,
                           return_route=record_ids, flags=PATH_FLAGS[path])
            if record_ids:
                ids_list.append(r[2].cpu().numpy())

    n_full, rem = divmod(steps, L)
    with torch.cuda.stream(stream):
        one_pass(record_ids=True)           # eager, also collects the routes
        torch.cuda.synchronize()
        y_eager = [y.clone() for y in ys]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            one_pass()
        for _ in range(max(1, -(-warmup // L))):
            g.replay()
        torch.cuda.synchronize()
        for a, b in zip(y_eager, ys):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "graph replay differs"
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        # the GPU spins before the start event while the host queues the
        # replays behind it, so the timed region holds the layer calls back
        # to back and not the host's submission of the first graph
        torch.cuda._sleep(GPU_SPIN_CYCLES)
        start.record(stream)
        for _ in range(n_full):
            g.replay()
        # the remaining calls are launched one by one: each replay of a graph
        # carries about 10 us of its own on the device (measured: 24.2 us per
        # call with one call per graph, 14.7 with 32), which a region of fewer
        # calls than the ring would otherwise hold once
        one_pass(rem)
        stop.record(stream)
        stop.synchronize()
        total_ms = start.elapsed_time(stop)
        per_rep = []
        for _ in range(max(min_replays, min(20, n_full), 1)):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(GPU_SPIN_CYCLES)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            e1.synchronize()
            per_rep.append(e0.elapsed_time(e1) / L * 1e3)
        torch.cuda.synchronize()
        for a, b in zip(y_eager, ys):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "graph replay differs"
    del g
    us = total_ms * 1e3 / steps
    U = unique_experts(ids_list)
    bias = layers[0]["br"] is not None
    per_rep.sort()
    shb = shared_bytes(cfg, layers[0])
    counted = expert_bytes(cfg, U) + shb
    total = layer_bytes(cfg, T, U, bias, layers[0]["Wr"].element_size(), shb)
    flops = expert_flops(cfg, T, k1)
    return {
        "T": T, "k1": k1, "k2": k2, "path": path, "layers": L, "steps": steps,
        "router": "bf16" if layers[0]["Wr"].dtype == torch.bfloat16 else "fp32",
        "shared_expert_channels": Is,
        "us_per_layer": us,
        "replays": len(per_rep),
        "us_median": per_rep[len(per_rep) // 2],
        "us_p10": per_rep[len(per_rep) // 10], "us_p90": per_rep[(9 * len(per_rep)) // 10],
        "tokens_per_s": T / (us * 1e-6),
        "unique_experts": U,
        "counted_bytes": counted,
        "counted_GBps": counted / (us * 1e-6) / 1e9,
        "hbm_frac_counted": counted / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "total_bytes": total,
        "hbm_frac_total": total / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "expert_tflops": flops / (us * 1e-6) / 1e12,
        "mfma_frac": flops / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
        # time at the binding roof (HBM for every byte of the call, or bf16
        # MFMA for the expert FLOPs, whichever is longer) over the measured time
        "roofline_frac": max(total / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12))
                         / (us * 1e-6),
        "_ys": ys,
    }


def profile_launches(moe, torch, cfg, layers, T, k1, k2, path, n_calls):
    """Per-launch HIP-event times of one call; then the longest launch timed
    in every call of an eager pass of n_calls over the layers."""
    stream = torch.cuda.Stream()
    xs = [lay["x"][:T].contiguous() for lay in layers]
    ys = [torch.empty_like(x) for x in xs]
    lib = moe.load_library()
    act = 1 if cfg.dtype == "bf16" else 0
    Is = layers[0]["shared"]["Sg"].shape[0] if layers[0].get("shared") else 0
    nws = (lib.moe_forward_channel_topk_workspace(T, cfg.H, cfg.E, cfg.I, k1, act, act)
           if layers[0].get("topk") else
           lib.moe_forward_shared_workspace(T, cfg.H, cfg.E, cfg.I, k1, Is, act, act))
    ws = torch.zeros(nws, dtype=torch.uint8, device=layers[0]["Wg"].device)

    def call(i):
        j = i % len(layers)
        lay = layers[j]
        layer_call(moe, lay, xs[j], k1, k2, cfg, out=ys[j], workspace=ws,
                   flags=PATH_FLAGS[path])

    launches = []
    with torch.cuda.stream(stream):
        for i in range(3 * len(layers)):
            call(i)
        for j in range(16):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            times = []
            name = ""
            for i in range(min(len(layers), 16)):
                moe.profile_launch(j, ev[0], ev[1])
                call(i)
                stream.synchronize()
                name = moe.profile_launch_name()
                if not name:
                    break
                times.append(ev[0].elapsed_time(ev[1]) * 1e3)
            if not name:
                break
            times.sort()
            launches.append({"launch": j, "kernel": name,
                             "us_median": round(times[len(times) // 2], 3)})
        dom = max(launches, key=lambda d: d["us_median"])
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_calls)]
        torch.cuda.synchronize()
        for i in range(n_calls):
            moe.profile_launch(dom["launch"], evs[i][0], evs[i][1])
            call(i)
        torch.cuda.synchronize()
        per = [a.elapsed_time(b) * 1e3 for a, b in evs]
    return launches, dom, sum(per) / len(per)


# ------------------------------------------------------------------ checks
def check_parity(moe, torch, oracle, synth, layer, T, k1, k2, path, y_dev, n_tok=32):
    """One layer of the cell against the oracle: ids and weights equal the
    oracle's route on the GPU's logits bit for bit; y within the bf16
    tolerance on a token sample (host copies of the activated experts only)."""
    import numpy as np
    x = layer["x"][:T]
    ck = layer.get("topk")
    if ck:
        keep = int(round(ck["frac"] * k1 * layer["Wg"].shape[1]))
        y, lg, ids, w, sc, kept = moe.forward_channel_topk(
            x, layer["Wr"], layer["Wg"], layer["Wu"], layer["Wd"], k1, k2, ck["dn"], keep,
            br=layer["br"], return_route=True, flags=PATH_FLAGS[path], Wdown_cols=ck["cols"])
    else:
        y, lg, ids, w = moe.forward(x, layer["Wr"], layer["Wg"], layer["Wu"], layer["Wd"], k1,
                                    k2, br=layer["br"], return_route=True,
                                    flags=PATH_FLAGS[path], shared=shared_args(layer))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_dev.view(torch.int16)), "timed output differs"
    lg_h = lg.cpu().numpy()
    bf16_router = layer["Wr"].dtype == torch.bfloat16
    oids, ow = (oracle.route_bf16w if bf16_router else oracle.route)(lg_h, k1, k2)
    assert np.array_equal(oids, ids.cpu().numpy()) and \
        np.array_equal(ow.view(np.int32), w.cpu().numpy().view(np.int32)), "route differs"
    sel = np.unique(np.linspace(0, T - 1, min(T, n_tok)).astype(int))
    sids = oids[sel]
    uniq = np.unique(sids)
    idx = torch.as_tensor(uniq, dtype=torch.long, device=x.device)
    n = synth.to_numpy
    Wg, Wu, Wd = (n(layer[k].index_select(0, idx)) for k in ("Wg", "Wu", "Wd"))
    rids = np.searchsorted(uniq, sids).astype(np.int32)
    if ck:
        # the kept set equals the oracle's selection on the GPU's own scores
        sc_h, kept_h = sc.cpu().numpy(), kept.cpu().numpy()
        assert np.array_equal(oracle.channel_select(sc_h, keep), kept_h), "selection differs"
        y_ref = oracle.experts_kept(n(x)[sel], Wg, Wu, Wd, rids, ow[sel], kept_h[sel])
    else:
        y_ref = oracle.experts(n(x)[sel], Wg, Wu, Wd, rids, ow[sel], nthreads=8)
    if layer.get("shared"):
        sh = {k: n(v) for k, v in layer["shared"].items()}
        y_ref = y_ref.astype(np.float64) + oracle.shared(n(x)[sel], sh["Sg"], sh["Su"], sh["Sd"],
                                                         sh["sg"], nthreads=8)
    yd = y.float().cpu().numpy().astype(np.float64)[sel]
    err = float((np.abs(yd - y_ref).max(1) / np.abs(y_ref).max(1)).max())
    tol = 1e-5 if layer["x"].dtype == torch.float32 else 2e-2
    assert err <= tol, f"normwise error {err} > {tol}"
    return err


def host_cores():
    """Cores this process may use: its affinity mask, capped by OMP_NUM_THREADS
    when that is set (the CPU share of the machine)."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(omp))) if omp.isdigit() and int(omp) > 0 else n


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(oracle, synth, layer, k1, k2, budget_s=8.0):
    """The oracle as it stands, on host copies of one ring layer: single-token
    calls on one core, then batches of tokens threaded over every core."""
    n = synth.to_numpy
    host = {k: n(layer[k]) for k in ("Wr", "Wg", "Wu", "Wd")}
    xs = n(layer["x"])

    def run(batch, nthreads):
        done, t0 = 0, time.perf_counter()
        while True:
            i = (done // batch * batch) % (xs.shape[0] - batch + 1)
            oracle.forward(xs[i:i + batch], host["Wr"], host["Wg"], host["Wu"], host["Wd"], k1,
                           k2, nthreads=nthreads)
            done += batch
            el = time.perf_counter() - t0
            if el > budget_s or done >= 20000:
                return done / el, done, el

    one, n1, t1 = run(1, 1)
    cores = host_cores()
    allc, na, ta = run(min(4 * cores, xs.shape[0]), cores)
    return {"value": allc, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "one_core": one, "cpu_model": cpu_model(),
            "precision": "route in exact fp32; logits, experts and combine accumulated in fp64",
            "sample": f"batch-1 decode layer H=2048 E=128 I=768 bf16 k1:k2={k1}:{k2}: "
                      f"{n1} single-token calls on 1 core in {t1:.1f} s, then {na} tokens in "
                      f"batches threaded over {cores} cores in {ta:.1f} s"}


def read_ceiling(moe, torch, nbytes=4 << 30):
    """Read-only streaming rate (moe_hbm_read_probe) over a buffer 16x the
    Infinity Cache: the best of a few grid sizes, 10 launches each."""
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(65536, dtype=torch.int32, device="cuda")
    best = None
    for blocks in (1024, 2048, 4096, 8192):
        moe.hbm_read_probe(buf, out, blocks)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(10):
            moe.hbm_read_probe(buf, out, blocks)
        b.record()
        b.synchronize()
        gbs = nbytes / (a.elapsed_time(b) / 10 * 1e-3) / 1e9
        if best is None or gbs > best[0]:
            best = (gbs, blocks)
    del buf
    return {"GBps": best[0], "blocks": best[1], "bytes": nbytes}


def copy_calibration(torch, nbytes=256 << 20):
    """A plain device copy of known size (the reference kernel for scaling the
    FETCH_SIZE / WRITE_SIZE counters) and its bandwidth."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(10):
        dst.copy_(src)
    b.record()
    b.synchronize()
    ms = a.elapsed_time(b) / 10
    return {"bytes": nbytes, "us": ms * 1e3,
            "GBps_read_plus_write": 2 * nbytes / (ms * 1e-3) / 1e9}


def traffic_record(kernel):
    """HBM bytes per launch measured with rocprofv3 counters, if the stored
    record is for this kernel and its source is unchanged since."""
    rec_path = ROOT / "profiles" / "traffic.json"
    if not rec_path.exists():
        return None
    rec = json.loads(rec_path.read_text())
    if rec.get("kernel") != kernel:
        return None
    h = hashlib.sha256()
    for name in rec["sources"]:
        src = ROOT / name
        if not src.exists():
            return None
        h.update(src.read_bytes())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return rec["bytes_per_launch"]


# ------------------------------------------------------------------ main
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              f"(this build has no multi-GPU path)", file=sys.stderr)
        return 2
    import torch

    import decoupled_top_routing_amd as moe
    from decoupled_top_routing_amd import synth

    specs = []
    for spec in args.cells.split(","):
        parts = spec.split(":")
        specs.append((parts[0], int(parts[1]), int(parts[2]), int(parts[3]),
                      parts[4] if len(parts) > 4 else "auto"))
    sets = make_sets(synth, torch, {s[0] for s in specs}, args.ring)

    cells_out = open(args.cells_out, "w") if args.cells_out else None

    def emit(c):
        line = json.dumps({k: (round(v, 4) if isinstance(v, float) else v) for k, v in c.items()
                           if not k.startswith("_")})
        print(line, file=sys.stderr, flush=True)
        if cells_out:
            cells_out.write(line + "\n")
            cells_out.flush()

    cells = []
    for idx, (name, T, k1, k2, path) in enumerate(specs):
        cfg, layers = sets[name]
        if name.startswith("C4"):
            steps = 6 * len(layers)
        elif name.startswith("C5"):
            steps = len(layers) * (20 if T > 1 else 40)
        else:
            steps = args.steps if idx == 0 else min(args.steps, 50 * len(layers))
        c = time_cell(moe, torch, cfg, layers, T, k1, k2, path, steps,
                      args.warmup if idx == 0 else min(args.warmup, 4 * len(layers)),
                      min_replays=10 if idx == 0 else 0)
        c["config"] = name
        print(f"# {name} b{T} {k1}:{k2} [{path}]: {c['us_per_layer']:.2f} us/layer "
              f"(replays {c['us_p10']:.2f}-{c['us_median']:.2f}-{c['us_p90']:.2f}), "
              f"{c['tokens_per_s']:.0f} tok/s, "
              f"{c['counted_GBps']:.0f} GB/s counted ({100 * c['hbm_frac_counted']:.1f}% of HBM), "
              f"{c['expert_tflops']:.1f} TFLOP/s, U={c['unique_experts']:.1f}",
              file=sys.stderr, flush=True)
        cells.append(c)

    import oracle
    for (name, T, k1, k2, path), c in zip(specs, cells):
        _, layers = sets[name]
        c["parity_normwise_err"] = check_parity(moe, torch, oracle, synth, layers[0], T, k1, k2,
                                                path, c["_ys"][0],
                                                n_tok=4 if name == "C5" else 32)
        emit(c)
    print("# parity: every cell matches the oracle", file=sys.stderr, flush=True)

    head = cells[0]
    hname, hT, hk1, hk2, hpath = specs[0]
    hcfg, hlayers = sets[hname]
    launches, dom, dom_us = profile_launches(moe, torch, hcfg, hlayers, hT, hk1, hk2, hpath,
                                             min(args.steps, 50 * len(hlayers)))
    bias = hlayers[0]["br"] is not None
    dom_bytes, _ = kernel_work(dom["kernel"], hcfg, hT, hk1, head["unique_experts"], bias,
                               hlayers[0]["Wr"].element_size(), shared_bytes(hcfg, hlayers[0]))
    eager_us = dom_us
    if len(launches) == 1:
        # the call is this one launch: the timed region (calls queued back to
        # back behind a GPU spin, HIP events on the launch stream) gives its
        # average duration without the dispatch cost of an eager launch
        # inside an event pair
        dom_us = head["us_per_layer"]
        timing = "timed region: layer calls queued back to back, one launch per call"
    else:
        timing = "HIP events around the launch in an eager pass over the ring"
    print(f"# launches {launches}; dominant {dom['kernel']}: {dom_us:.2f} us per launch "
          f"({timing}; eager event pair {eager_us:.2f} us)",
          file=sys.stderr, flush=True)
    calib = copy_calibration(torch)
    ceiling = read_ceiling(moe, torch)
    print(f"# read-only streaming ceiling {ceiling['GBps']:.0f} GB/s "
          f"({ceiling['blocks']} workgroups); copy {calib['GBps_read_plus_write']:.0f} GB/s",
          file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(oracle, synth, hlayers[0], hk1, hk2)
        print(f"# cpu baseline {json.dumps(cpu)}", file=sys.stderr, flush=True)

    def find(cfgname, T, k1, k2):
        for (n_, T_, a_, b_, p_), c in zip(specs, cells):
            if (n_, T_, a_, b_, p_) == (cfgname, T, k1, k2, "auto"):
                return c
        return None

    ratios = {}
    for cfgname, T in (("C2", 1), ("C3", 2), ("C3", 4), ("C3", 8), ("C3", 16), ("C3", 32),
                       ("C3", 64), ("C4", 4096)):
        a, b = find(cfgname, T, 4, 16), find(cfgname, T, 8, 8)
        if a and b:
            ratios[f"b{T}"] = round(b["us_per_layer"] / a["us_per_layer"], 3)
    c20, c10 = find("C5", 1, 5, 20), find("C5", 1, 10, 10)
    c5 = find("C5", 1, 5, 5)

    us = head["us_per_layer"]
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9 if dom_bytes else None
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1) if achieved else None,
        "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4) if achieved else None,
        "traffic": traffic_record(dom["kernel"]),
        "kernel": dom["kernel"], "algorithmic_bytes": dom_bytes,
        "us_per_launch": round(dom_us, 3), "timing": timing,
        "frac_of_read_ceiling": round(achieved / ceiling["GBps"], 4) if achieved else None,
    }
    if cpu:
        cpu = {k: (round(v, 2) if isinstance(v, float) else v) for k, v in cpu.items()}
    out = {
        "metric": "MoE-layer tokens/s + % HBM peak at batch 1/8, k1:k2 4:16 vs 8:8",
        "value": round(head["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded Gaussian layers generated on the device",
        "config": {
            "workload": f"decode batch {hT}, H={hcfg.H} E={hcfg.E} I={hcfg.I} bf16 experts, "
                        f"k1:k2={hk1}:{hk2}, cold ring of {len(hlayers)} layers (whole-ring "
                        f"HIP graph replays, the rest of the steps launched one by one)",
            "global_batch": hT,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "replays": {"n": head["replays"], "us_median": round(head["us_median"], 3),
                    "us_p10": round(head["us_p10"], 3), "us_p90": round(head["us_p90"], 3)},
        "ratio_8:8_over_4:16": ratios,
        "C5_b1_us": ({"10:10": round(c10["us_per_layer"], 2), "5:5": round(c5["us_per_layer"], 2),
                      "5:20": round(c20["us_per_layer"], 2)} if c10 and c5 and c20 else None),
        "read_ceiling_GBps": round(ceiling["GBps"], 1),
        "cells": len(cells),
        "cells_out": args.cells_out,
    }
    if cells_out:
        cells_out.close()
    line = json.dumps(out, separators=(",", ":"))
    print(f"# summary line {len(line)} bytes", file=sys.stderr, flush=True)
    print(line, flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
