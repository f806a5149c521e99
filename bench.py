#!/usr/bin/env python3
"""Throughput of the routed-expert MoE layer over a speculative window, one MI355X.

Default workload: the DeepSeek-V2-Lite-shaped draft layer over a K=16 window
(17 tokens): 64 routed experts, softmax top-6, hidden 2048, intermediate 1408,
INT4 group-128 routed weights with fp16 scales, two always-on FP16 shared
experts, and the activation counter (ELB) with a top-32 plan.

One step = one pass of the whole hot path over one window, every stage in the
HIP library: FP16 shared experts, router top-k, alignment by expert, ELB
accumulate + top-M, fused W4A16 routed-expert FFN, weighted combine. The
steps are captured in one HIP graph that runs one step on each of several
weight copies (more than 1 GiB in total, above the 256 MB last-level cache),
so every step streams its weights from HBM, as the layers of a model's
decode step would. Inputs are resident in HBM before the timed region starts.

Printed: one JSON line with tokens/s (whole job), ms per step, the layer's
achieved HBM bandwidth, a roofline entry for the dominant call (the fused
W4A16 expert FFN, timed with HIP events on the stream it runs on) and the CPU
reference timed on this host's cores on a bounded sample.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A16 MoE-layer tokens/sec + achieved HBM GB/s fraction, K=16 window"
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, vendor figure
PEAK_F16_TFLOPS = 2500.0        # MI355X dense fp16 MFMA, vendor figure
MIN_ROTATION_BYTES = 1 << 30    # rotate weight copies over at least this many bytes
FFN_CALLS_PER_GRAPH = 8         # expert-FFN calls per timing graph
PROFILES = os.path.join(ROOT, "profiles")
FFN_SOURCES = [os.path.join(ROOT, "quantized_speculative_expert_amd", "csrc", f)
               for f in ("ffn.hip", "ffn_device.hpp", "ffn_wide.hip", "ffn_wide.hpp",
                         "smoe_internal.hpp")]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000, help="timed steps")
    p.add_argument("--warmup", type=int, default=100, help="untimed warmup steps")
    p.add_argument("--config", default="dsv2", help="workload shape (default dsv2)")
    p.add_argument("--copies", type=int, default=0,
                   help="weight copies to rotate (0 = enough for >= 1 GiB)")
    p.add_argument("--shared", choices=("fused", "separate"), default="fused",
                   help="shared experts inside the routed FFN launches (fused) or as a call "
                        "of their own (separate)")
    p.add_argument("--layer", choices=("one-call", "calls"), default=None,
                   help="the layer step as one library call (smoe_moe_layer_w4a16, whose "
                        "routing launch also reads the shared experts' weights through the "
                        "caches) or as the separate calls; default: one call with the shared "
                        "experts fused and no side stream, else the separate calls")
    p.add_argument("--layout", choices=("tiled", "rows"), default="tiled",
                   help="expert weights in the tiled layout of smoe_tile_weights, tiled once "
                        "before timing (default), or row-major")
    p.add_argument("--side-stream", action="store_true",
                   help="run the ELB update (and a separate shared-expert call) on a side "
                        "stream branch of the step graph instead of in line")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB `steps` times (reads MIB, "
                        "writes MIB): the reference that scales the HBM traffic counters")
    p.add_argument("--eager-steps", type=int, default=400,
                   help="layer steps also timed eagerly, one library call after another (0 = skip)")
    p.add_argument("--compare", action="store_true",
                   help="also time the same routed-expert work as one W4A16 call per active "
                        "expert and as one batched call over FP16 weights")
    p.add_argument("--offload", action="store_true",
                   help="instead of the layer throughput: speculative windows over a stack "
                        "whose FP16 target experts live in pinned host memory (draft with "
                        "ELB-driven prefetch, cached verification), with and without the "
                        "prefetch and with every expert resident")
    p.add_argument("--offload-layers", type=int, default=4,
                   help="layers of the offloaded stack (--offload)")
    p.add_argument("--offload-windows", type=int, default=6,
                   help="timed windows per mode (--offload), after two untimed ones")
    p.add_argument("--stack", action="store_true",
                   help="time every layer of a multi-layer config (batch: 26 layers of 544 "
                        "tokens) as one step: each layer with its own activations, router and "
                        "weights, the activation counter accumulated over the stack and ranked "
                        "once at its end")
    p.add_argument("--specfit", action="store_true",
                   help="instead of the layer throughput: SpecFit subtree selection on the host "
                        "(18-node top-2 pools of depth 5, K = 7, 48 layers x 128 experts, "
                        "top-8), the library's search against the brute-force oracle")
    p.add_argument("--cpu-reps", type=int, default=10,
                   help="full layers the CPU reference runs for cpu_baseline (0 = skip)")
    return p.parse_args()


# ----------------------------------------------------------------------------- bytes

def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def expert_bytes(d) -> int:
    """Bytes of one routed expert's weights as streamed by the kernels."""
    return sum(_nbytes(t) for t in (d.wg_q, d.wg_s, d.wu_q, d.wu_s, d.wd_q, d.wd_s)) // d.cfg.E


def layer_bytes(d, n_active: int) -> dict:
    """Algorithmic HBM bytes of one layer step (each tensor read or written once).

    Routed: the codes and scales of the distinct experts the window touches.
    Shared: the FP16 shared experts. Router: its weight matrix (and bias / gate
    vector). Activations: x read, y written. Routing metadata, the ELB counter
    and intermediates (h, per-slot outputs) are below 0.5 % and not counted.
    """
    c = d.cfg
    routed = n_active * expert_bytes(d)
    shared = sum(_nbytes(t) for t in (d.sg16, d.su16, d.sd16))
    router = sum(_nbytes(t) for t in (d.w_router, d.router_bias, d.shared_gate_w))
    act = 2 * c.T * c.H * 2
    return {"routed": routed, "shared": shared, "router": router, "activations": act,
            "total": routed + shared + router + act}


def ffn_bytes(d, n_active: int, with_shared: bool) -> int:
    """Algorithmic bytes of one W4A16 expert-FFN call: touched experts' codes
    + scales, x read once, per-slot fp32 outputs written once; with the
    shared experts also their FP16 weights and fp32 outputs."""
    c = d.cfg
    b = n_active * expert_bytes(d) + c.T * c.H * 2 + c.S * c.H * 4
    if with_shared and d.shared_out is not None:
        b += sum(_nbytes(t) for t in (d.sg16, d.su16, d.sd16)) + c.T * c.H * 4
    return b


def ffn_flops(d, with_shared: bool) -> int:
    """Useful MFMA flops of one expert-FFN call: gate, up and down for every
    routed slot, and for every token through the shared experts."""
    c = d.cfg
    f = 2 * 3 * c.H * c.I * c.S
    if with_shared and d.shared_out is not None:
        f += 2 * 3 * c.H * d.shared_I * c.T
    return f


# ----------------------------------------------------------------------------- traffic

def source_digest() -> str:
    """Digest of the FFN sources' code: comments, trailing blanks and empty
    lines are left out, so that an edit of the comments alone keeps the
    recorded counters valid."""
    h = hashlib.sha256()
    for f in FFN_SOURCES:
        with open(f, encoding="utf-8") as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        for line in text.splitlines():
            line = re.sub(r"//.*", "", line).rstrip()
            if line:
                h.update(line.encode() + b"\n")
    return h.hexdigest()[:16]


def recorded_traffic(config: str, shared_mode: str, layout: str):
    """HBM bytes per FFN call from the committed rocprofv3 counter summary.

    Returns None when no summary exists for this workload, shared-expert mode
    and weight layout, or when the kernel sources changed since the counters
    were taken.
    """
    path = os.path.join(PROFILES, f"w4a16_expert_ffn_{config}_traffic.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"^TRAFFIC_JSON: (\{.*\})\s*$", open(path).read(), re.M)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if (rec.get("source_digest") != source_digest() or rec.get("shared") != shared_mode
            or rec.get("layout", "rows") != layout):
        return None
    return rec.get("bytes_per_call")


# ----------------------------------------------------------------------------- CPU leg

def cpu_baseline(cfg_name: str, reps: int):
    """The CPU reference (oracle) timed on this host on `reps` full layers."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from workload import get_config, make_layer

    from threadpoolctl import threadpool_limits

    cfg = get_config(cfg_name)
    L = make_layer(cfg, seed=0)

    def layers(n):
        t0 = time.perf_counter()
        for _ in range(n):
            r = oracle.moe_layer(L, "draft")
            if cfg.elb_M:
                cnt = oracle.elb_accumulate(np.zeros((1, cfg.E), np.int32), r["ids"][None], 0)
                oracle.elb_topm(cnt, cfg.elb_M)
        return time.perf_counter() - t0, r

    dt, r = layers(reps)
    blas = [i.get("num_threads", 1) for i in threadpool_info()]
    cores = max(blas) if blas else 1
    # one BLAS thread, on a smaller sample
    reps1 = max(1, reps // 5)
    with threadpool_limits(limits=1):
        dt1, _ = layers(reps1)
    # bytes the layer's algorithm touches, as on the GPU side: the touched
    # experts' codes and scales, the shared experts, the router, x and y
    n_active = int(r["n_active"])
    per_expert = sum(getattr(L, n_)[0].nbytes for n_ in ("wg_q", "wg_s", "wu_q", "wu_s", "wd_q", "wd_s"))
    shared = sum(t.nbytes for t in (L.sg16, L.su16, L.sd16) if t is not None)
    router = sum(t.nbytes for t in (L.w_router, L.router_bias, L.shared_gate_w) if t is not None)
    nbytes = n_active * per_expert + shared + router + 2 * cfg.T * cfg.H * 2
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": cfg.T * reps / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"{reps} full {cfg.name} layers of {cfg.T} tokens (route, align, ELB "
                       f"top-{cfg.elb_M}, INT4 dequantise + float64 SwiGLU of the touched "
                       f"experts, shared experts, combine) in {dt:.1f} s; BLAS matmuls on "
                       f"{cores} threads, the rest single-threaded NumPy; then {reps1} on one "
                       f"BLAS thread ({cfg.T * reps1 / dt1:.2f} tokens/s): the time goes to "
                       f"single-threaded NumPy (the stated-order router dot products and the "
                       f"INT4 dequantisation), so the baseline is effectively single-threaded "
                       f"whatever `cores` says"),
            "ms_per_layer": 1e3 * dt / reps,
            "single_thread_value": cfg.T * reps1 / dt1,
            "gbps": nbytes * reps / dt / 1e9,
            "cpu_model": model, "os_cpu_count": os.cpu_count()}


# ----------------------------------------------------------------------------- GPU leg

def copy_calibration(mib: int, calls: int) -> int:
    """A plain elementwise copy kernel (dst = src * 1) of known size."""
    import torch
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(calls):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": n, "bytes_written": n, "calls": calls}}),
          flush=True)
    return 0


def compare_ffn(base, layers, fused: bool, stream, batched_us: float) -> dict:
    """The routed experts' work of one window done three ways, each cycling
    over the weight copies inside one HIP graph: the batched W4A16 call (all
    active experts in two launches), one W4A16 call per active expert (E = 1
    on that expert's slots, plus one call for the shared experts), and the
    batched call over FP16 weights of the same shapes (the target format)."""
    import torch
    from quantized_speculative_expert_amd import _lib

    c = base.cfg
    off = base.offsets.cpu().tolist()
    act = [e for e in range(c.E) if off[e + 1] > off[e]]
    offs = [torch.tensor([off[e], off[e + 1]], dtype=torch.int32, device=base.device)
            for e in act]
    ws = torch.zeros(_lib.smoe_ffn_workspace_bytes(c.T, c.k, 1, c.H, c.I),
                     dtype=torch.uint8, device=base.device)

    def per_expert(d):
        for e, o in zip(act, offs):
            sl = slice(e, e + 1)
            d._call("smoe_w4a16_expert_ffn")(d.x, c.k, 1, c.I, c.G, d.wg_q[sl], d.wg_s[sl],
                                             d.wu_q[sl], d.wu_s[sl], d.wd_q[sl], d.wd_s[sl],
                                             d.sorted_slots, o, ws, d.slot_out)
        if fused:
            d.shared_ffn()

    def fp16(d):
        d.routed_ffn(target=True, with_shared=fused)

    def time_graph(body, reps: int = 50) -> float:
        cap = torch.cuda.Stream(device=base.device)
        cap.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            for d in layers:
                body(d)  # eager once: every call checked before capture
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=cap):
                for d in layers:
                    body(d)
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        g.replay()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i in range(reps):
            g.replay()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        return percentiles([1e3 * ev[i].elapsed_time(ev[i + 1]) / len(layers)
                            for i in range(reps)])["median"]

    log(f"compare: one W4A16 call per active expert ({len(act)})")
    seq_us = time_graph(per_expert)
    log("compare: batched FP16 call")
    f16_us = time_graph(fp16)
    return {"batched_w4a16_us": round(batched_us, 2),
            "per_expert_w4a16_us": round(seq_us, 2),
            "batched_fp16_us": round(f16_us, 2),
            "active_experts": len(act),
            "shared_experts": "included" if fused else "excluded",
            "note": ("per graph replay over the rotated weight copies; per-expert = "
                     f"{len(act)} W4A16 calls of E = 1 (2 launches each) + the shared call; "
                     "FP16 = the batched call over FP16 routed weights (4x the bytes)")}


def stack_bench(args) -> int:
    """The whole layer stack as one step: every layer is the draft layer
    (routing, alignment, ELB update of its own counter row, W4A16 FFN with the
    shared experts, combine) over its own activations, router, Zipf router
    skew and device copy of the expert weights (the generated experts of
    layer 0, copied once per layer, so that every layer streams distinct
    bytes). The counter rows accumulate over the stack; the last layer ranks
    the top-M plan over all of them. One HIP graph holds the stack."""
    import torch
    from quantized_speculative_expert_amd.layer import DeviceLayer
    from workload import get_config, make_activations, make_layer, make_router
    from workload.gen import zipf_bias

    cfg = get_config(args.config)
    if cfg.layers < 2:
        raise SystemExit(f"--stack needs a multi-layer config ({cfg.name} has one layer)")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"generating {cfg.name} layer 0 (seed 0)")
    inp = make_layer(cfg, seed=0, layer=0)
    base = DeviceLayer(inp, device=dev, elb_layers=cfg.layers, tiled=args.layout == "tiled")
    del inp
    runners = [base]
    for l in range(1, cfg.layers):
        r = base.with_weight_copy()
        r.x = torch.from_numpy(make_activations(cfg, 0, l)).to(dev)
        r.w_router.copy_(torch.from_numpy(make_router(cfg, 0, l)))
        if cfg.zipf_s > 0:
            r.router_bias.copy_(torch.from_numpy(zipf_bias(cfg.E, cfg.zipf_s, 0, l)))
        runners.append(r)
    log(f"{cfg.layers} layers x {base.weight_bytes() / 2**20:.1f} MiB of weights resident")
    L = cfg.layers

    def step():
        for l, r in enumerate(runners):
            r.run(layer=l, rank=l == L - 1)

    # eager once, layer by layer, to count each layer's active experts
    n_active = []
    for l, r in enumerate(runners):
        r.run(layer=l, rank=l == L - 1)
        n_active.append(int(base.n_active.item()))
    torch.cuda.synchronize()
    cap = torch.cuda.Stream(device=dev)
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    log(f"warmup {args.warmup} stack steps")
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    K = args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    log(f"timing {K} stack steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(K):
        g.replay()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_us = [1e3 * ev[i].elapsed_time(ev[i + 1]) for i in range(K)]
    total = sum(layer_bytes(base, n)["total"] for n in n_active)
    gbps = total * K / wall / 1e9
    out = {
        "metric": f"batched {L}-layer stack tokens/sec (one step = every layer once)",
        "value": round(cfg.T * K / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * wall / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": (f"{cfg.name}: {cfg.description}; seed 0; all {L} layers per step, "
                         "each with its own activations, router and weight copy"),
            "T": cfg.T, "E": cfg.E, "k": cfg.k, "H": cfg.H, "I": cfg.I, "G": cfg.G,
            "shared_I": cfg.shared_I, "elb_M": cfg.elb_M, "layers": L,
            "weight_layout": args.layout,
        },
        "stack_us": {k_: round(v, 2) for k_, v in percentiles(step_us).items()},
        "layer_us_mean": round(sum(step_us) / len(step_us) / L, 2),
        "n_active": n_active,
        "stack_bytes": total,
        "hbm_gbps": round(gbps, 1),
        "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
        "roofline": None,
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    return 0


def specfit_bench(args) -> int:
    """Selection time per verification cycle: the library's depth-first search
    against the oracle's brute force on the same seeded pools (Qwen3-30B-A3B
    shape of the SpecFit page: 48 MoE layers, 128 experts, top-8; pools of 18
    nodes from top-2 expansion to depth 5; K = 7), with a half-resident
    expert cache. Both run on this host, one thread."""
    import numpy as np

    from quantized_speculative_expert_amd import _lib
    import oracle.specfit as SF

    L, E, k, n, K = 48, 128, 8, 18, 7
    reps = max(1, min(args.steps, 50))
    rng = np.random.default_rng(0)
    pools = []
    for _ in range(reps):
        parent, depth, prob, kids = [], [], [], {}
        frontier = [(-1, 0, 1.0)]
        while len(parent) < n and frontier:
            i = int(rng.integers(0, len(frontier)))
            v, dv, pv = frontier[i]
            if kids.get(v, 0) >= 2 or dv >= 5:
                frontier.pop(i)
                continue
            kids[v] = kids.get(v, 0) + 1
            q = float(pv * rng.uniform(0.2, 0.95))
            parent.append(v)
            depth.append(dv + 1)
            prob.append(q)
            frontier.append((len(parent) - 1, dv + 1, q))
        sets_ = [[set(rng.choice(E, k, replace=False).tolist()) for _ in range(L)]
                 for _ in range(n + 1)]
        res = [set(rng.choice(E, E // 2, replace=False).tolist()) for _ in range(L)]
        bits = np.zeros((n + 1, L, 2), np.uint64)
        for r, node in enumerate(sets_):
            for l, es in enumerate(node):
                for e in es:
                    bits[r, l, e // 64] |= np.uint64(1) << np.uint64(e % 64)
        rbits = np.zeros((L, 2), np.uint64)
        for l, es in enumerate(res):
            for e in es:
                rbits[l, e // 64] |= np.uint64(1) << np.uint64(e % 64)
        b = np.cumsum(rng.uniform(5.0, 10.0, K + 1))
        pools.append((np.array(parent, np.int32), np.array(prob), bits, rbits, b, sets_, res))
    beta = 0.05
    t_nat, agree, visited = [], 0, 0
    for parent, prob, bits, rbits, b, _, _ in pools:
        t0 = time.perf_counter()
        sel, r, ev = _lib.smoe_specfit_select(parent, prob, bits, K, b, beta, rbits, E=E)
        t_nat.append(time.perf_counter() - t0)
        visited = ev
    n_or = min(3, reps)
    t_or = []
    for parent, prob, bits, rbits, b, sets_, res in pools[:n_or]:
        t0 = time.perf_counter()
        want, wr, legal = SF.select(parent.tolist(), prob.tolist(), sets_[0], sets_[1:], K,
                                    b.tolist(), beta, res)
        t_or.append(time.perf_counter() - t0)
        sel, r, ev = _lib.smoe_specfit_select(parent, prob, bits, K, b, beta, rbits, E=E)
        agree += int(sel == want and r == wr and ev == legal)
    med = float(np.median(t_nat)) * 1e6
    out = {"metric": "SpecFit subtree selection: us per verification cycle (host)",
           "value": round(med, 2), "unit": "us", "higher_is_better": False, "n_gpus": 0,
           "data": "synthetic",
           "config": {"workload": f"{reps} pools of {n} nodes (top-2 expansion, depth <= 5), "
                                  f"K = {K}, {L} layers x {E} experts, top-{k}, half the "
                                  f"experts resident, beta {beta}; seed 0",
                      "legal_subtrees_per_pool": visited},
           "cpu_baseline": {"value": round(float(np.median(t_or)) * 1e6, 1), "unit": "us",
                            "cores": 1, "kind": "oracle",
                            "sample": f"brute force over every subset of <= {K} nodes on the "
                                      f"first {n_or} pools"},
           "oracle_agrees": f"{agree}/{n_or}",
           "pages_reference_ms": 2.82}
    print(json.dumps(out), flush=True)
    return 0


OFFLOAD_ZIPF_S = 0.7  # router skew giving ~32 distinct experts per 16 draft tokens (of 64)


def offload_bench(args) -> int:
    """Speculative windows (K = 16 draft tokens, a 17-token verification) over
    a stack of dsv2-shaped layers whose FP16 target experts (17.3 MB each)
    live in pinned host memory, with M = 32 device slots per layer. Three
    modes on the same seeded windows: the ELB-driven prefetch planner on,
    off (verification loads every miss itself), and every expert resident
    (M = E, no copies). Per window: draft time, verification time, copies,
    hits and misses. The verification's bound is the larger of its copy
    time at the measured host-to-device bandwidth and its compute time."""
    import dataclasses

    import numpy as np
    import torch

    from quantized_speculative_expert_amd.offload import OffloadStack, measure_h2d
    from workload import get_config, make_layer, make_router
    from workload.gen import zipf_bias

    cfg = get_config("dsv2")
    L, M, K, b1 = args.offload_layers, cfg.elb_M, cfg.T - 1, 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"offload: {L} dsv2 layers, {M} slots per layer, K={K}")
    draft_inp = make_layer(dataclasses.replace(cfg, T=1), seed=0, layer=0)
    routers = [make_router(cfg, 0, l) for l in range(L)]
    zipf = [zipf_bias(cfg.E, OFFLOAD_ZIPF_S, 0, l) for l in range(L)]
    rng = np.random.default_rng(0)
    n_win = args.offload_windows + 2
    xd = [(rng.standard_normal((L, K, cfg.H))).astype(np.float16) for _ in range(n_win)]
    xt = [np.concatenate([x + (0.05 * rng.standard_normal(x.shape)).astype(np.float16),
                          rng.standard_normal((L, 1, cfg.H)).astype(np.float16)], axis=1)
          for x in xd]
    gbps = measure_h2d(dev)
    log(f"host-to-device copy: {gbps:.1f} GB/s")

    def run(mode: str):
        st = OffloadStack(cfg, draft_inp, L, cfg.E if mode == "resident" else M, zipf=zipf,
                          routers=routers, seed=0, tiled=True, device=dev)
        if mode == "resident":  # every expert in its slot before the first window
            slots = np.tile(np.arange(cfg.E, dtype=np.int32), (L, 1))
            import quantized_speculative_expert_amd._lib as lib
            lib.smoe_cache_set_state(st.cache, slots, np.zeros((L, cfg.E), np.int64), 0,
                                     copy_stream=st.copy_stream)
            torch.cuda.synchronize(dev)
        # draft time per token (all layers), from the second of two untimed
        # windows without prefetch (the first pays for first launches)
        xdev = torch.from_numpy(xd[0]).to(dev)
        for _ in range(2):
            torch.cuda.synchronize(dev)
            t0 = time.perf_counter()
            st.draft_window(xdev, False, b1, gbps, 1.0)
            torch.cuda.synchronize(dev)
        us_tok = 1e6 * (time.perf_counter() - t0) / K
        compute = torch.cuda.current_stream(dev)
        rows = []
        for w in range(n_win):
            xdev = torch.from_numpy(xd[w]).to(dev)
            xtdev = torch.from_numpy(np.ascontiguousarray(xt[w])).to(dev)
            torch.cuda.synchronize(dev)
            t0 = time.perf_counter()
            plan = st.draft_window(xdev, mode == "planner", b1, gbps, us_tok)
            # the draft is done when its stream is; prefetch copies may still
            # be in flight and the verification starts at once
            compute.synchronize()
            t1 = time.perf_counter()
            scheds = st.verify_window(xtdev)
            torch.cuda.synchronize(dev)
            t2 = time.perf_counter()
            hits = sum(int((s[:, 2] == 0).sum()) for s in scheds)
            misses = sum(int((s[:, 2] == 1).sum()) for s in scheds)
            loads = sum(len(ld) for _, ld in plan["loads"])
            rows.append({"draft_ms": 1e3 * (t1 - t0), "verify_ms": 1e3 * (t2 - t1),
                         "prefetched": loads, "hits": hits, "misses": misses,
                         "chunks": len(plan["chunks"])})
        st.close()
        del st
        torch.cuda.empty_cache()
        timed = rows[2:]
        mean = {k: round(float(np.mean([r[k] for r in timed])), 3) for k in timed[0]}
        mean["draft_us_per_token"] = round(us_tok, 1)
        return mean

    res = {m: run(m) for m in ("planner", "no-prefetch", "resident")}
    eb = 3 * cfg.I * cfg.H * 2
    for m, r in res.items():
        copy_ms = r["misses"] * eb / (gbps * 1e6)
        r["verify_copy_bound_ms"] = round(copy_ms, 3)
        r["window_ms"] = round(r["draft_ms"] + r["verify_ms"], 3)
    comp = res["resident"]["verify_ms"]
    for m, r in res.items():
        bound = max(r["verify_copy_bound_ms"], comp)
        r["verify_bound_frac"] = round(bound / r["verify_ms"], 4) if r["verify_ms"] else None
    out = {
        "metric": "speculative window with offloaded FP16 target experts: window ms",
        "unit": "ms", "higher_is_better": False, "n_gpus": 1, "data": "synthetic",
        "config": {"workload": (f"{L} dsv2-shaped layers (64 experts, top-6, H 2048, I 1408, "
                                f"FP16 target experts 17.3 MB each in pinned host memory), "
                                f"{M} device slots per layer, K={K} draft tokens then a "
                                f"{cfg.T}-token verification; draft INT4 layers resident; "
                                f"router Zipf({OFFLOAD_ZIPF_S}) skew; b_1={b1}; seed 0"),
                   "layers": L, "M": M, "K": K, "windows": args.offload_windows},
        "h2d_gbps": round(gbps, 2),
        "modes": res,
    }
    print(json.dumps(out), flush=True)
    return 0


def percentiles(xs):
    import numpy as np
    a = np.asarray(xs, dtype=float)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "mean": float(a.mean())}


def main() -> int:
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the layer runs on a single MI355X and libsmoe "
              f"has no multi-GPU path (asked for --gpus {args.gpus}, WORLD_SIZE {world})",
              file=sys.stderr)
        return 2

    if args.specfit:
        return specfit_bench(args)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        return 1
    if args.copy_calibration > 0:
        return copy_calibration(args.copy_calibration, args.steps)
    if args.offload:
        return offload_bench(args)
    if args.stack:
        return stack_bench(args)
    from quantized_speculative_expert_amd.layer import DeviceLayer
    from workload import get_config, make_layer

    cfg = get_config(args.config)
    # a stack of several layers is timed on its layer 0, with the ELB
    # counters of every layer (each step ranks all of them)
    log(f"generating {cfg.name} inputs (seed 0)")
    inp = make_layer(cfg, seed=0, layer=0, want_fp16=args.compare)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    base = DeviceLayer(inp, device=dev, with_target=args.compare, elb_layers=cfg.layers,
                       tiled=args.layout == "tiled")
    del inp
    # rotation sized on the draft path's weights (the FP16 routed copies that
    # --compare adds are read only by the comparison)
    wbytes = base.weight_bytes() - sum(_nbytes(t) for t in (base.wg16, base.wu16, base.wd16))
    copies = args.copies or max(2, -(-MIN_ROTATION_BYTES // wbytes))
    layers = [base] + [base.with_weight_copy() for _ in range(copies - 1)]
    log(f"{copies} weight copies x {wbytes / 2**20:.1f} MiB resident")

    fused = args.shared == "fused"
    side = torch.cuda.Stream(device=dev) if args.side_stream else None
    use_elb = cfg.elb_M > 0

    if args.layer is None:
        args.layer = "one-call" if fused and side is None else "calls"
    one_call = args.layer == "one-call"
    if one_call and (not fused or side is not None):
        raise SystemExit("--layer one-call runs the shared experts fused and has no side stream")

    def step(d):
        d.run(elb=use_elb, fuse_shared=fused, side_stream=side, one_call=one_call)

    # eager run once (checks every call), then capture the graphs
    for d in layers:
        step(d)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream(device=dev)
    cap.wait_stream(torch.cuda.current_stream())
    # one graph holds one layer step on each weight copy, as a model's decode
    # step would be captured; every step still runs every call
    steps_per_graph = copies
    step_graph = torch.cuda.CUDAGraph()
    # the FFN alone: FFN_CALLS_PER_GRAPH back-to-back calls cycling over the
    # weight copies in one graph, so the per-call time is that of the two
    # launches and the gap between them, not of a graph launch
    ffn_graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(step_graph, stream=cap):
            for d in layers:
                step(d)
        with torch.cuda.graph(ffn_graph, stream=cap):
            for i in range(FFN_CALLS_PER_GRAPH):
                layers[i % copies].routed_ffn(with_shared=fused)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    log(f"warmup {args.warmup} steps")
    for i in range(-(-args.warmup // steps_per_graph)):
        step_graph.replay()
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` layer steps (rounded up to whole
    # graphs)
    R = -(-args.steps // steps_per_graph)
    K = R * steps_per_graph
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(R + 1)]
    log(f"timing {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(R):
        step_graph.replay()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_us = [1e3 * evs[i].elapsed_time(evs[i + 1]) / steps_per_graph for i in range(R)]
    gpu_total_ms = evs[0].elapsed_time(evs[R])

    n_active = int(base.n_active.item())
    lb = layer_bytes(base, n_active)
    ms_per_step = 1e3 * wall / K
    tokens_per_s = cfg.T * K / wall
    layer_gbps = lb["total"] * K / wall / 1e9

    # ---- dominant call: W4A16 expert FFN (two launches; with the shared
    # experts when fused), HIP events on the stream it runs on
    R = max(1, K // FFN_CALLS_PER_GRAPH)
    log(f"timing {R * FFN_CALLS_PER_GRAPH} W4A16 expert-FFN calls")
    ffn_graph.replay()
    fe = [torch.cuda.Event(enable_timing=True) for _ in range(R + 1)]
    torch.cuda.synchronize()
    fe[0].record(stream)
    for i in range(R):
        ffn_graph.replay()
        fe[i + 1].record(stream)
    torch.cuda.synchronize()
    ffn_us = [1e3 * fe[i].elapsed_time(fe[i + 1]) / FFN_CALLS_PER_GRAPH for i in range(R)]
    ffn_stats = percentiles(ffn_us)
    fb = ffn_bytes(base, n_active, fused)
    achieved = fb / (ffn_stats["mean"] * 1e3)  # bytes/ns = GB/s
    traffic = recorded_traffic(cfg.name, args.shared, args.layout)
    # windows of 1024 to 4096 slots over tiled weights take the long-window kernel
    long_window = args.layout == "tiled" and 1024 <= cfg.T * cfg.k <= 4096
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                "traffic": traffic,
                "kernel": ("smoe_w4a16_expert_ffn ("
                           + ("wide_ffn_kernel" if long_window else "ffn_kernel")
                           + " stage 1 + 2, routed"
                           + (" + shared experts)" if fused else " experts)")),
                "bytes_per_launch": fb, "us_per_launch": round(ffn_stats["mean"], 2)}

    flops = ffn_flops(base, fused)
    mfma = {"flops_per_call": flops,
            "achieved_tflops": round(flops / (ffn_stats["mean"] * 1e6), 2),
            "peak_tflops": PEAK_F16_TFLOPS,
            "frac": round(flops / (ffn_stats["mean"] * 1e6) / PEAK_F16_TFLOPS, 4)}

    # ---- the same layer step enqueued eagerly, call after call
    eager = None
    if args.eager_steps > 0:
        n = args.eager_steps
        log(f"timing {n} eager steps")
        ee = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        ee[0].record(stream)
        for i in range(n):
            step(layers[i % copies])
            ee[i + 1].record(stream)
        torch.cuda.synchronize()
        eager = {k_: round(v, 2) for k_, v in
                 percentiles([1e3 * ee[i].elapsed_time(ee[i + 1]) for i in range(n)]).items()}

    compare = compare_ffn(base, layers, fused, stream, ffn_stats["mean"]) if args.compare else None

    cpu = None
    if args.cpu_reps > 0:
        log(f"CPU reference on {args.cpu_reps} layers")
        cpu = cpu_baseline(cfg.name, args.cpu_reps)

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": (f"{cfg.name}: {cfg.description}; seed 0; "
                         + (f"layer 0 of the {cfg.layers}-layer stack; " if cfg.layers > 1 else "")
                         + f"{steps_per_graph} steps per graph, {copies} rotated weight copies"),
            "T": cfg.T, "E": cfg.E, "k": cfg.k, "H": cfg.H, "I": cfg.I, "G": cfg.G,
            "shared_I": cfg.shared_I, "elb_M": cfg.elb_M, "weights": "int4 g%d + fp16 scales" % cfg.G,
            "shared_experts": args.shared,
            "side_stream": side is not None,
            "layer_call": args.layer,
            "weight_layout": args.layout,
        },
        "hbm_gbps": round(layer_gbps, 1),
        "hbm_frac": round(layer_gbps / PEAK_HBM_GBPS, 4),
        "layer_us": {k_: round(v, 2) for k_, v in percentiles(step_us).items()},
        "layer_us_gpu_mean": round(1e3 * gpu_total_ms / K, 2),
        "layer_eager_us": eager,
        "ffn_us": {k_: round(v, 2) for k_, v in ffn_stats.items()},
        "mfma": mfma,
        "n_active": n_active,
        "layer_bytes": lb,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if compare is not None:
        out["compare"] = compare
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
