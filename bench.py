#!/usr/bin/env python3
"""Benchmark of the routed MoE layer with Eq. 2 weights on one MI355X.

A step is one call of the whole layer (router, route, experts, combine) on one
batch.  The headline workload is decode at batch 1 on the H=2048, E=128,
I=768 bf16 layer with k1:k2 = 4:16, run over a ring of 32 distinct seeded
layers (38.7 GB) so that every layer's weights come from HBM, not from the
256 MB Infinity Cache.  The ring is captured once in a HIP graph and replayed;
HIP events on the capture stream time the replays.  The same ring is also
timed at 8:8 and at batch 8, and reported in "cells".

Prints one JSON line (see the repository's benchmark contract).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA, TFLOP/s
RING = 32


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=6400)
    ap.add_argument("--warmup", type=int, default=320)
    ap.add_argument("--ring", type=int, default=RING)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cells", default="b1:4:16,b1:8:8,b8:4:16,b8:8:8",
                    help="cells to time; the first is the headline")
    return ap.parse_args()


def counted_bytes(cfg, ids_list):
    """Activated-expert bytes per step, from the actual routes: unique experts
    of each step's batch times 3*I*H weight elements."""
    per_expert = 3 * cfg.I * cfg.H * (2 if cfg.dtype == "bf16" else 4)
    uniq = [len(set(ids.flatten().tolist())) for ids in ids_list]
    return per_expert * sum(uniq) / len(uniq), sum(uniq) / len(uniq)


def total_bytes(cfg, T, counted):
    elt = 2 if cfg.dtype == "bf16" else 4
    return counted + cfg.E * cfg.H * 4 + 2 * T * cfg.H * elt


PATH_FLAGS = {"auto": 0, "f": 1, "g": 2, "p": 4}


def time_cell(moe, torch, layers, cfg, T, k1, k2, steps, warmup, path="auto"):
    """Graph-capture one pass over the ring and time whole replays."""
    dev = layers[0]["Wg"].device
    L = len(layers)
    stream = torch.cuda.Stream(device=dev)
    xs = [lay["x"][:T].contiguous() for lay in layers]
    ys = [torch.empty_like(x) for x in xs]
    lib = moe.load_library()
    nbytes = lib.moe_forward_workspace(T, cfg.H, cfg.E, cfg.I, k1, 1, 1)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    ids_list = []

    def one_pass(record_ids=False):
        for i, lay in enumerate(layers):
            r = moe.forward(xs[i], lay["Wr"], lay["Wg"], lay["Wu"], lay["Wd"], k1, k2,
                            br=lay["br"], out=ys[i], workspace=ws,
                            return_route=record_ids, flags=PATH_FLAGS[path])
            if record_ids:
                ids_list.append(r[2].cpu().numpy())

    with torch.cuda.stream(stream):
        one_pass(record_ids=True)           # eager, also collects the routes
        torch.cuda.synchronize()
        y_eager = [y.clone() for y in ys]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            one_pass()
        n_warm = max(1, warmup // L)
        n_rep = max(1, steps // L)
        for _ in range(n_warm):
            g.replay()
        torch.cuda.synchronize()
        # replays must reproduce the eager outputs bit for bit
        for a, b in zip(y_eager, ys):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "graph replay differs"
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        per_rep = []
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        start.record(stream)
        for _ in range(n_rep):
            g.replay()
        stop.record(stream)
        stop.synchronize()
        t_wall = time.perf_counter() - t_wall
        total_ms = start.elapsed_time(stop)
        # a few individually timed replays for the spread
        for _ in range(min(20, n_rep)):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            e1.synchronize()
            per_rep.append(e0.elapsed_time(e1) / L * 1e3)
        torch.cuda.synchronize()
        for a, b in zip(y_eager, ys):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "graph replay differs"
    n_steps = n_rep * L
    us = total_ms * 1e3 / n_steps
    counted, uniq = counted_bytes(cfg, ids_list)
    per_rep.sort()
    return {
        "T": T, "k1": k1, "k2": k2, "path": path, "steps": n_steps,
        "us_per_layer": us,
        "us_p10": per_rep[len(per_rep) // 10], "us_p90": per_rep[(9 * len(per_rep)) // 10],
        "tokens_per_s": T / (us * 1e-6),
        "unique_experts": uniq,
        "counted_bytes": counted,
        "counted_GBps": counted / (us * 1e-6) / 1e9,
        "hbm_frac_counted": counted / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "total_bytes": total_bytes(cfg, T, counted),
        "wall_s": t_wall,
        "graph": g, "ws": ws, "ys": ys, "y_eager": y_eager, "ids": ids_list,
    }


def check_parity(moe, torch, oracle, synth, layer, cfg, T, k1, k2, y_dev):
    """Oracle check of one ring layer: route bit for bit on the GPU logits,
    y within the bf16 tolerance (host copies of the activated experts only)."""
    import numpy as np
    x = layer["x"][:T]
    y, lg, ids, w = moe.forward(x, layer["Wr"], layer["Wg"], layer["Wu"], layer["Wd"], k1, k2,
                                br=layer["br"], return_route=True)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_dev.view(torch.int16))
    lg_h = lg.cpu().numpy()
    oids, ow = oracle.route(lg_h, k1, k2)
    assert np.array_equal(oids, ids.cpu().numpy()) and \
        np.array_equal(ow.view(np.int32), w.cpu().numpy().view(np.int32)), "route differs"
    uniq = sorted(set(oids.flatten().tolist()))
    remap = {e: i for i, e in enumerate(uniq)}
    sel = torch.tensor(uniq, device=x.device)
    n = synth.to_numpy
    Wg, Wu, Wd = (n(layer[k].index_select(0, sel)) for k in ("Wg", "Wu", "Wd"))
    rids = np.vectorize(remap.get)(oids).astype(np.int32)
    y_ref = oracle.experts(n(x), Wg, Wu, Wd, rids, ow, nthreads=8)
    yd = y.float().cpu().numpy().astype(np.float64)
    err = float((np.abs(yd - y_ref).max(1) / np.abs(y_ref).max(1)).max())
    assert err <= 2e-2, f"normwise error {err}"
    return err


def cpu_baseline(oracle, synth, torch, layer, cfg, k1, k2, budget_s=12.0):
    """The oracle as it stands, on host copies of one ring layer, batch 1."""
    import numpy as np
    n = synth.to_numpy
    host = {k: n(layer[k]) for k in ("Wr", "Wg", "Wu", "Wd")}
    xs = n(layer["x"])
    done, t0 = 0, time.perf_counter()
    while True:
        x = xs[done % xs.shape[0]:done % xs.shape[0] + 1]
        oracle.forward(x, host["Wr"], host["Wg"], host["Wu"], host["Wd"], k1, k2, nthreads=1)
        done += 1
        el = time.perf_counter() - t0
        if el > budget_s or done >= 400:
            break
    return {"value": done / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} single-token calls (batch 1, k1:k2={k1}:{k2}) of the C oracle on "
                      f"host copies of one {cfg.name} layer, {el:.1f} s; the oracle threads over "
                      f"tokens, so a batch of 1 runs on one core"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              f"(no multi-GPU path is built)", file=sys.stderr)
        return 2
    import torch

    import decoupled_top_routing_amd as moe
    from decoupled_top_routing_amd import synth

    dev = torch.device("cuda:0")
    cfg = synth.DECODE_B8        # the batch-1 cells use the first token of each layer
    t0 = time.perf_counter()
    layers = []
    for i in range(args.ring):
        lay = synth.make_layer(cfg, layer=i, device="cuda")
        layers.append(lay)
    torch.cuda.synchronize()
    print(f"# generated {args.ring} layers of {cfg.name} on the device in "
          f"{time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)

    cells = []
    for spec in args.cells.split(","):
        parts = spec.split(":")
        b, k1, k2 = parts[:3]
        path = parts[3] if len(parts) > 3 else "auto"
        T, k1, k2 = int(b[1:]), int(k1), int(k2)
        c = time_cell(moe, torch, layers, cfg, T, k1, k2, args.steps, args.warmup, path)
        print(f"# cell b{T} {k1}:{k2} [{path}]: {c['us_per_layer']:.2f} us/layer "
              f"({c['us_p10']:.2f}-{c['us_p90']:.2f}), {c['tokens_per_s']:.0f} tok/s, "
              f"{c['counted_GBps']:.0f} GB/s counted ({100 * c['hbm_frac_counted']:.1f}% of HBM), "
              f"U={c['unique_experts']:.1f}", file=sys.stderr, flush=True)
        cells.append(c)

    head = cells[0]
    import oracle
    errs = []
    for c in cells:
        errs.append(check_parity(moe, torch, oracle, synth, layers[0], cfg, c["T"], c["k1"],
                                 c["k2"], c["ys"][0]))
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(oracle, synth, torch, layers[0], cfg, head["k1"], head["k2"])

    def find(T, k1, k2):
        for c in cells:
            if (c["T"], c["k1"], c["k2"], c["path"]) == (T, k1, k2, "auto"):
                return c
        return None

    ratios = {}
    for T in (1, 8):
        a, b = find(T, 4, 16), find(T, 8, 8)
        if a and b:
            ratios[f"b{T}_4:16_over_8:8"] = b["us_per_layer"] / a["us_per_layer"]

    us = head["us_per_layer"]
    achieved = head["counted_bytes"] / (us * 1e-6) / 1e9
    out = {
        "metric": "MoE-layer tokens/s + % HBM peak at batch 1/8, k1:k2 4:16 vs 8:8",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": args.warmup,
        "ms_per_step": us / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded Gaussian layers generated on the device",
        "config": {
            "workload": f"decode batch {head['T']}, H={cfg.H} E={cfg.E} I={cfg.I} bf16 "
                        f"experts, k1:k2={head['k1']}:{head['k2']}, cold ring of "
                        f"{args.ring} layers replayed from one HIP graph",
            "global_batch": head["T"], "ring_layers": args.ring,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": None,
            "kernel": "whole layer (all kernels of one moe_forward call)",
        },
        "cpu_baseline": cpu,
        "cells": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in c.items()
                   if k not in ("graph", "ws", "ys", "y_eager", "ids")} for c in cells],
        "ratios": ratios,
        "parity_normwise_err": errs,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
