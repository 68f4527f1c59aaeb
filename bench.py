#!/usr/bin/env python3
"""Benchmark: per-token decode of one quantized MoE layer on one MI355X.

Default workload ("layer"): H=4096, I=1024, E=512 routed experts + 1 shared,
top-K=4, 4-bit codes with a bf16 scale and bias per 64 weights, one token per
step.  A step is one pass of the whole decode path (router GEMV + softmax/top-K,
fused gate/up dequant-GEMV + SwiGLU over the 5 active experts, down
dequant-GEMV + weighted combine) for a fresh token.

Cold-cache measurement: the layer is replicated at R distinct HBM addresses
(R = --rotate, default 16) and step t uses copy t mod R, so the bytes a step
reads were last touched R-1 steps (>600 MB of traffic) earlier and cannot be
served from the 256 MB Infinity Cache or the L2s.

Timed regions:
  * graph: K steps captured once into a HIP graph (launch-bound loop); each of
    --replays replays is bracketed by GPU events recorded on the replay stream,
    and the median replay gives ms_per_step and the headline tokens/s (host
    launch latency is outside the events, so the figure does not depend on K).
    The same steps replayed on one layer copy give the warm-cache figure.
  * eager: the same K steps launched one by one with start/stop HIP events
    recorded around the router, gate/up and down kernels on their stream;
    gives each kernel's average duration, hence achieved GB/s.
The other workloads (2-bit layer, 64-token batch, 60-layer stack) are timed the
same way with fewer steps and reported under "configs" in the same JSON line.
The float64 oracle is timed on the host cores on a small sample of tokens
(cpu_baseline).  Each workload's first step is checked against the oracle
before timing; a mismatch reports no throughput.

    python bench.py [--steps K] [--warmup W] [--workload layer|layer2|layer3|layer_g128|requant|batched|batched2|batched3|stack]
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "MoE decode tokens/s and achieved expert-weight HBM GB/s (% of MI355X peak)"

WORKLOADS = {
    "layer": dict(H=4096, I=1024, E=512, K=4, bits=4, B=1, layers=1, zipf=None, seed=1001),
    "layer2": dict(H=4096, I=1024, E=512, K=4, bits=2, B=1, layers=1, zipf=None, seed=1002),
    "stack": dict(H=4096, I=1024, E=512, K=4, bits=4, B=1, layers=60, zipf=None, seed=1003),
    "batched": dict(H=4096, I=1024, E=512, K=10, bits=4, B=64, layers=1, zipf=1.1, seed=1004),
    "batched2": dict(H=4096, I=1024, E=512, K=10, bits=2, B=64, layers=1, zipf=1.1, seed=1004),
    # the layer workload's 4-bit experts requantized to 2-bit on the GPU (moe_requant_4to2)
    "requant": dict(H=4096, I=1024, E=512, K=4, bits=2, B=1, layers=1, zipf=None, seed=1001, requant=True),
    # the layer workload's shape with one scale and bias per 128 weights
    "layer_g128": dict(H=4096, I=1024, E=512, K=4, bits=4, B=1, layers=1, zipf=None, seed=1005, group=128),
    # the layer workload's shape with 3-bit codes
    "layer3": dict(H=4096, I=1024, E=512, K=4, bits=3, B=1, layers=1, zipf=None, seed=1006),
    "batched3": dict(H=4096, I=1024, E=512, K=10, bits=3, B=64, layers=1, zipf=1.1, seed=1004),
}
RMS_EPS = 1e-6


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Hip:
    """hipEvent helpers over libamdhip64 (the events the timing hook records)."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        rc = self.h.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError("hipEventCreate failed (%d)" % rc)
        return e.value

    def elapsed_ms(self, a, b):
        f = ctypes.c_float()
        rc = self.h.hipEventElapsedTime(ctypes.byref(f), a, b)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return f.value

    def recorded(self, a, b):
        """True if the pair was recorded (the elapsed time of a never-recorded pair is an error)."""
        f = ctypes.c_float()
        ok = self.h.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        if not ok:
            self.h.hipGetLastError()  # the failed query leaves a sticky error: clear it
        return ok

    def destroy(self, e):
        self.h.hipEventDestroy(e)


def gateup_bytes_per_expert(c):
    return 2 * c["I"] * c["H"] * c["bits"] // 8 + 2 * c["I"] * (c["H"] // c.get("group", 64)) * 4


def down_bytes_per_expert(c):
    return c["H"] * c["I"] * c["bits"] // 8 + c["H"] * (c["I"] // c.get("group", 64)) * 4


def build_layers(c, n_distinct, n_copies, dev):
    import torch
    import synth
    from quantized_expert_dequant_amd.slab import DeviceLayer, upload_experts
    H, I, E, K, bits = c["H"], c["I"], c["E"], c["K"], c["bits"]
    group = c.get("group", 64)
    base = []
    for l in range(n_distinct):
        t0 = time.time()
        if c.get("requant"):
            from quantized_expert_dequant_amd.slab import upload_requantized
            src = lambda first, n, l=l: synth.experts(c["seed"], l, first, n, 4, H, I, group)
            slab = upload_requantized(src, E + 1, H, I, device=dev, group=group)
        else:
            src = lambda first, n, l=l: synth.experts(c["seed"], l, first, n, bits, H, I, group)
            slab = upload_experts(src, E + 1, bits, H, I, device=dev, group=group)
        wr = torch.from_numpy(synth.router(c["seed"], l, E, H)).to(dev)
        bias = torch.from_numpy(synth.zipf_bias(E, c["zipf"])).to(dev) if c["zipf"] else None
        base.append(DeviceLayer(H, I, E, K, bits, slab, wr, bias, group=group))
        log("layer %d packed in %.1fs" % (l, time.time() - t0))
    layers = list(base)
    for r in range(n_distinct, n_copies):
        b = base[r % n_distinct]
        layers.append(DeviceLayer(H, I, E, K, bits, b.slab.clone(), b.w_router.clone(),
                                  None if b.logit_bias is None else b.logit_bias.clone(), group=group))
    torch.cuda.synchronize()
    return layers


def oracle_check(c, x_host, y_dev, idx_dev, layer_id=0):
    """One sampled token of the timed configuration against the float64 oracle."""
    import oracle
    import synth
    E, K = c["E"], c["K"]
    Wr = synth.router(c["seed"], layer_id, E, c["H"])
    prior = synth.zipf_bias(E, c["zipf"]) if c["zipf"] else None
    lg = oracle.router_logits(x_host, Wr, prior)
    need = {E}
    for b in range(x_host.shape[0]):
        need |= {int(e) for e in oracle.topk(lg[b], K)[0]}
    group = c.get("group", 64)
    experts = {e: synth.experts(c["seed"], layer_id, e, 1, 4 if c.get("requant") else c["bits"], c["H"], c["I"],
                                group)
               for e in sorted(need)}
    if c.get("requant"):
        for e, x4 in experts.items():
            g2, u2, d2, s2, b2 = oracle.requant_expert(c["H"], c["I"], x4.gate[0], x4.up[0], x4.down[0],
                                                       x4.scales[0], x4.biases[0], group=group)
            experts[e] = synth.Canonical(2, c["H"], c["I"], group, g2[None], u2[None], d2[None], s2[None], b2[None])
    y_ref, idx_ref, _, _ = oracle.layer_decode(c["bits"], c["H"], c["I"], E, K, x_host, Wr, experts, prior=prior,
                                               group=group)
    # per token max|dy| / max|y_ref|, the denominator floored where fp32 cannot represent the tolerance
    err = max(float(np.max(np.abs(y_dev[b] - y_ref[b])) / max(np.max(np.abs(y_ref[b])), 2.0 ** -126 / 2e-3))
              for b in range(x_host.shape[0]))
    return bool(np.array_equal(idx_dev, idx_ref)) and err <= 2e-3, err


def kernel_source_hash(workload):
    """Hash of the sources the timed gate/up kernels are built from: the single-token
    kernel lives in kernels.hip; the batched phase also runs grouped.hip's kernels."""
    files = ["kernels.hip", "common.h", "topk.h"]
    if WORKLOADS[workload]["B"] > 1:
        files.append("grouped.hip")
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "quantized_expert_dequant_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


# the stack's layers have the layer workload's shape and run the same gate/up kernel,
# so its per-launch traffic is the layer workload's
PMC_RECORD = {"stack": "layer"}


def traffic_from_profile(workload, launches_per_step):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3 PMC results,
    only while the kernel sources still match the ones the counters were taken on."""
    workload = PMC_RECORD.get(workload, workload)
    p = os.path.join(ROOT, "profiles", "pmc_gateup_%s.json" % workload)
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source_hash") != kernel_source_hash(workload):
        return None
    return d.get("traffic_bytes_per_launch")


def _pmc_per_dispatch(path, kernel_prefix, counter):
    """Mean per-dispatch value (KiB) of `counter` for kernels whose name starts with kernel_prefix."""
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
            if r["Counter_Name"] == counter and r["Kernel_Name"].replace("void ", "").startswith(kernel_prefix)]
    if not vals:
        raise SystemExit("no %s values for %s in %s" % (counter, kernel_prefix, path))
    return sum(vals) / len(vals), len(vals)


def write_pmc_summary(workload, kernel_prefix, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_mb):
    """profiles/pmc_gateup_<workload>.json from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of the bench
    and of the plain device copy (--copy-calibration-mb), which scales each counter to bytes."""
    copy_kib = copy_mb * 1024.0
    cf, _ = _pmc_per_dispatch(copy_fetch_csv, "__amd_rocclr_copyBuffer", "FETCH_SIZE")
    cw, _ = _pmc_per_dispatch(copy_write_csv, "__amd_rocclr_copyBuffer", "WRITE_SIZE")
    # "a|b|c": a phase of several kernels, one dispatch of each per step
    f = w = 0.0
    nf, nw = [], []
    for kp in kernel_prefix.split("|"):
        fk, nfk = _pmc_per_dispatch(fetch_csv, kp, "FETCH_SIZE")
        wk, nwk = _pmc_per_dispatch(write_csv, kp, "WRITE_SIZE")
        f, w = f + fk, w + wk
        nf.append(nfk)
        nw.append(nwk)
    kf, kw = copy_kib / cf, copy_kib / cw
    traffic = (f * kf + w * kw) * 1024.0
    c = WORKLOADS[workload]
    algo = gateup_bytes_per_expert(c) * (c["K"] + 1) if c["B"] == 1 else None
    out = {"workload": workload, "kernel": kernel_prefix, "kernel_source_hash": kernel_source_hash(workload),
           "fetch_kib_per_dispatch": round(f, 1), "write_kib_per_dispatch": round(w, 1), "dispatches": [nf, nw],
           "copy_calibration_mib": copy_mb, "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1),
           "fetch_scale": round(kf, 4), "write_scale": round(kw, 4),
           "traffic_bytes_per_launch": round(traffic), "algorithmic_bytes_per_launch": algo,
           "traffic_over_algorithmic": round(traffic / algo, 4) if algo else None}
    path = os.path.join(ROOT, "profiles", "pmc_gateup_%s.json" % workload)
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out))


def _median(v):
    v = sorted(v)
    return v[len(v) // 2]


def expert_dtype(c):
    """The type the expert arithmetic multiplies in: one token's 4- and 2-bit codes as signed 4-bit
    integers against 4-bit digits of the token (v_dot8, int32 sums); 3-bit codes and the batched
    matrix cores as exact fp16 (fp32 sums)."""
    return "i4" if c["B"] == 1 and c["bits"] in (2, 4) else "f16"


def _workload_name(name, c, n_copies, n_distinct, stack):
    return "%s: H=%d I=%d E=%d+1 shared K=%d %d-bit group %d bf16 scale+bias, B=%d%s%s" % (
        name, c["H"], c["I"], c["E"], c["K"], c["bits"], c.get("group", 64), c["B"],
        ", %d layers with RMS renorm" % c["layers"] if stack else "",
        ", experts requantized from the layer workload's 4-bit ones on the GPU" if c.get("requant") else "")


def measure(name, steps, warmup, dev, rotate=16, distinct=0, graph=True, eager=True, warm=False, replays=5,
            lead_ms=30.0):
    """Time one workload: parity spot check, graph replays (GPU events around each replay on
    the replay stream, median over `replays`), optionally the same steps on one layer copy
    (warm caches), and an eager pass with per-kernel events.  Returns a dict of numbers."""
    import torch
    import synth
    import quantized_expert_dequant_amd as moe
    from quantized_expert_dequant_amd.slab import workspace

    c = dict(WORKLOADS[name])
    K, W, B, H = steps, warmup, c["B"], c["H"]
    stack = c["layers"] > 1
    n_distinct = min(distinct or c["layers"], c["layers"]) if stack else 1
    n_copies = c["layers"] if stack else max(1, rotate)
    log("workload %s: building %d layer(s) (%d distinct)" % (name, n_copies, n_distinct))
    layers = build_layers(c, n_distinct, n_copies, dev)

    xs_host = np.stack([synth.tokens(c["seed"], t, B, H) for t in range(W + K)])
    xs = torch.from_numpy(xs_host).to(dev)
    ws, ws_n = workspace(layers[0].desc, B, stack=stack)
    y = torch.empty((W + K, B, H), dtype=torch.float32, device=dev)
    nL = c["layers"]
    idx = torch.empty((W + K, nL, B, c["K"]), dtype=torch.int32, device=dev)
    wts = torch.empty((W + K, nL, B, c["K"]), dtype=torch.float32, device=dev)
    descs = [L.desc for L in layers]

    def step(t, copy=None):
        if stack:
            moe.stack_decode(descs, xs[t], B, RMS_EPS, y[t], idx[t], wts[t], ws, ws_n)
        else:
            L = layers[t % n_copies if copy is None else copy]
            moe.layer_decode(L.desc, xs[t], B, y[t], idx[t, 0], wts[t, 0], ws, ws_n)

    # parity spot check on the first step's tokens (layer copy 0 == distinct layer 0)
    step(0)
    torch.cuda.synchronize()
    if stack:
        y0 = torch.empty((B, H), dtype=torch.float32, device=dev)
        i0 = torch.empty((B, c["K"]), dtype=torch.int32, device=dev)
        w0 = torch.empty((B, c["K"]), dtype=torch.float32, device=dev)
        moe.layer_decode(layers[0].desc, xs[0], B, y0, i0, w0, ws, ws_n)
        torch.cuda.synchronize()
        ok, err = oracle_check(c, xs_host[0], y0.cpu().numpy(), i0.cpu().numpy())
        ok = ok and bool(torch.equal(i0, idx[0, 0]))
    else:
        ok, err = oracle_check(c, xs_host[0], y[0].cpu().numpy(), idx[0, 0].cpu().numpy())
    log("%s parity spot check: ok=%s max rel err %.3e" % (name, ok, err))
    res = {"workload": name, "config": _workload_name(name, c, n_copies, n_distinct, stack), "parity_ok": ok,
           "parity_rel_err": err, "steps": K, "rotation_copies": n_copies}
    if stack:
        res["distinct_layers"] = n_distinct
    if not ok:
        return res

    for t in range(W):
        step(t)
    torch.cuda.synchronize()

    def graph_time(copy=None):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for t in range(W, W + K):
                    step(t, copy)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g.replay()  # one untimed replay, checked against eager
        torch.cuda.synchronize()
        y_graph = y[W + K - 1].clone()
        step(W + K - 1, copy)
        torch.cuda.synchronize()
        if not torch.equal(y_graph, y[W + K - 1]):
            log("graph replay differs from eager: graph timing disabled")
            return None
        times = []
        for _ in range(replays):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b) / K)
        del g
        return times

    graph_ms = None
    if graph:
        times = graph_time()
        if times:
            graph_ms = _median(times)
            res["graph_replays_ms_per_step"] = [round(v, 6) for v in times]
        if warm and not stack:
            wt = graph_time(copy=0)
            if wt:
                res["warm_ms_per_step"] = round(_median(wt), 6)

    kinds = [moe.KERNEL_ROUTER, moe.KERNEL_GATEUP, moe.KERNEL_DOWN]
    dur = {k: None for k in kinds}
    eager_ms = None
    if eager:
        hip = Hip()
        ev = {k: [(hip.event(), hip.event()) for _ in range(K)] for k in kinds}
        torch.cuda.synchronize()
        # a bounded delay kernel first, so the host has enqueued the steps before the
        # GPU reaches them and the kernels run back to back, as they do in the graph
        torch.cuda._sleep(int(lead_ms * 2.4e6))
        for i, t in enumerate(range(W, W + K)):
            for k in kinds:
                moe.set_timing_events(k, *ev[k][i])
            step(t)
        torch.cuda.synchronize()
        for k in kinds:
            moe.set_timing_events(k, None, None)
        # with several layers per step the hook re-records each pair on every layer,
        # so each pair times the step's last launch of that kernel
        # the fused single-token expert kernel (gate/up and down in one launch) records
        # no separate down events: its down time is part of the gate/up launch
        recorded = {k: hip.recorded(*ev[k][0]) for k in kinds}
        dur = {k: (sum(hip.elapsed_ms(a, b) for a, b in ev[k]) / K if recorded[k] else 0.0) for k in kinds}
        last = moe.KERNEL_DOWN if recorded[moe.KERNEL_DOWN] else moe.KERNEL_GATEUP
        res["expert_launches"] = "gate/up + down" if recorded[moe.KERNEL_DOWN] else "fused gate/up + down"
        eager_ms = hip.elapsed_ms(ev[moe.KERNEL_ROUTER][0][0], ev[last][K - 1][1]) / K
        if not stack:
            st = np.array([hip.elapsed_ms(ev[moe.KERNEL_ROUTER][i][0], ev[last][i][1]) * 1e3
                           for i in range(K)])
            res["eager_step_us"] = {"p10": round(float(np.percentile(st, 10)), 3),
                                    "p50": round(float(np.percentile(st, 50)), 3),
                                    "p90": round(float(np.percentile(st, 90)), 3)}
        for k in kinds:
            for a, b in ev[k]:
                hip.destroy(a)
                hip.destroy(b)

    ms_per_step = graph_ms if graph_ms is not None else eager_ms
    res["timing"] = "graph" if graph_ms is not None else "eager"
    idx_h = idx[W:W + K].cpu().numpy()
    if B > 1:
        # the grouped path reads each distinct routed expert once per step, plus the shared one
        uniq = [len(np.unique(idx_h[i, 0][(idx_h[i, 0] >= 0) & (idx_h[i, 0] < c["E"])])) for i in range(K)]
        n_act = float(np.mean(uniq)) + 1
        res["distinct_experts_per_step"] = n_act
    else:
        n_act = c["K"] + 1
    gu_bytes = gateup_bytes_per_expert(c) * n_act
    dn_bytes = down_bytes_per_expert(c) * n_act
    router_bytes = 4 * c["E"] * H
    expert_bytes_step = (gu_bytes + dn_bytes) * nL
    res.update({
        "ms_per_step": round(ms_per_step, 6),
        "tokens_per_s": round(B / (ms_per_step / 1e3), 2),
        "expert_bytes_per_token": round(expert_bytes_step / B),
        "step_frac": round((expert_bytes_step + router_bytes * nL) / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
    })
    if eager_ms is not None:
        rt_us, gu_us, dn_us = (dur[k] * 1e3 for k in kinds)
        res["eager_ms_per_step"] = round(eager_ms, 6)
        res["kernel_us"] = {"router": round(rt_us, 3), "gateup": round(gu_us, 3), "down": round(dn_us, 3)}
        # the dominant launch: the gate/up kernel, or the fused kernel that also does the down phase
        dom_bytes = gu_bytes + (dn_bytes if dn_us == 0.0 else 0.0)
        res["gateup_gbps"] = round(dom_bytes / (gu_us * 1e-6) / 1e9, 1)
        res["gateup_bytes_per_launch"] = round(dom_bytes)
        # expert bytes over the summed time of every kernel that reads expert bytes
        eg = (gu_bytes + dn_bytes) / ((gu_us + dn_us) * 1e-6) / 1e9
        res["expert_weight_gbps"] = round(eg, 1)
        res["expert_weight_frac_of_peak"] = round(eg / PEAK_HBM_GBPS, 4)
    del layers, xs, ws, y, idx, wts, descs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def measure_tiered(dev, steps=200, warmup=20, slots=64, zipf=1.1, replays=3):
    """The layer workload's 4-bit layer with its E + 1 records in pinned host memory and an HBM
    cache of `slots` records (moe_layer_decode_cached), routing biased by a Zipf(zipf) prior so
    that hot experts recur: tokens/s, hit rate, bytes pulled from host memory per second and
    expert bytes per second.  The steps are captured in one HIP graph (the cache state lives on
    the GPU and evolves from call to call inside the replay as it does eagerly); before each
    replay a fresh set of tokens is copied into the graph's input buffer, so every replay routes
    new tokens through the cache the previous ones left.  After one untimed replay, GPU events
    around each of `replays` replays: the median gives the time per step, and the cache's
    counters over the timed replays give the hit rate and the bytes copied."""
    import torch
    import synth
    import quantized_expert_dequant_amd as moe
    from quantized_expert_dequant_amd.slab import DeviceLayer, host_store
    c = dict(WORKLOADS["layer"])
    H, I, E, K, bits, seed = c["H"], c["I"], c["E"], c["K"], c["bits"], c["seed"]
    t0 = time.time()
    store = host_store(lambda f, n: synth.experts(seed, 0, f, n, bits, H, I), E + 1, bits, H, I, device=dev)
    log("tiered: %d records (%.1f GB) in pinned host memory in %.1fs" % (E + 1, store.numel() / 1e9, time.time() - t0))
    wr = torch.from_numpy(synth.router(seed, 0, E, H)).to(dev)
    bias = torch.from_numpy(synth.zipf_bias(E, zipf)).to(dev)
    L = DeviceLayer(H, I, E, K, bits, store, wr, bias)
    rb = moe.record_bytes(bits, H, I)
    slab = torch.empty((slots + 1) * rb, dtype=torch.uint8, device=dev)
    state = torch.empty(moe.cache_state_bytes(E, slots), dtype=torch.uint8, device=dev)
    cache = moe.make_cache(slots, slab, state)
    moe.cache_init(L.desc, cache)
    n = moe.cache_workspace_bytes(L.desc, slots, 1)
    ws = torch.zeros(n, dtype=torch.uint8, device=dev)
    xs = torch.from_numpy(np.stack([synth.tokens(seed, 20_000 + t, 1, H) for t in range(warmup + steps)])).to(dev)
    # token sets for the replays (the untimed one, then the timed ones), each new to the cache
    pools = [torch.from_numpy(np.stack([synth.tokens(seed, 30_000 + p * steps + t, 1, H) for t in range(steps)]))
             .to(dev) for p in range(1 + replays)]
    y = torch.empty((warmup + steps, 1, H), dtype=torch.float32, device=dev)
    idx = torch.empty((warmup + steps, 1, K), dtype=torch.int32, device=dev)
    w = torch.empty((warmup + steps, 1, K), dtype=torch.float32, device=dev)
    for t in range(warmup):
        moe.layer_decode_cached(L.desc, cache, xs[t], 1, y[t], idx[t], w[t], ws, n)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for t in range(warmup, warmup + steps):
                moe.layer_decode_cached(L.desc, cache, xs[t], 1, y[t], idx[t], w[t], ws, n)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    xs[warmup:].copy_(pools[0])
    g.replay()  # untimed
    torch.cuda.synchronize()
    before = state[:32].cpu().numpy().view(np.uint64).copy()
    times = []
    for r in range(replays):
        xs[warmup:].copy_(pools[1 + r])
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) / steps)
    ms = _median(times)
    after = state[:32].cpu().numpy().view(np.uint64).copy()
    hits, misses, copied = (int(after[i] - before[i]) for i in range(3))
    del g
    steps_timed = steps * replays
    # parity: the last token against the oracle (same records, prior on the logits)
    ok, err = oracle_check(dict(c, zipf=zipf), xs[warmup + steps - 1].cpu().numpy(), y[warmup + steps - 1].cpu().numpy(),
                           idx[warmup + steps - 1].cpu().numpy())
    expert_bytes = (gateup_bytes_per_expert(c) + down_bytes_per_expert(c)) * (K + 1)
    res = {"config": "tiered: layer workload (H=%d I=%d E=%d+1 K=%d %d-bit) with a Zipf(%.1f) prior, all records in "
                     "pinned host memory, %d routed slots + the shared expert in HBM, B=1" % (H, I, E, K, bits, zipf,
                                                                                              slots),
           "parity_ok": ok, "parity_rel_err": err, "steps": steps,
           "timing": "graph (median of %d replays, GPU events)" % replays,
           "ms_per_step": round(ms, 6), "tokens_per_s": round(1e3 / ms, 2),
           "hit_rate": round(hits / max(1, hits + misses), 4), "misses_per_token": round(misses / steps_timed, 3),
           "host_gbps": round(copied / (ms * steps_timed * 1e-3) / 1e9, 2),
           "expert_weight_gbps": round(expert_bytes / (ms * 1e-3) / 1e9, 1)}
    del L, store, slab, state, ws, xs, y
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def requant_throughput(dev, n=64, reps=5):
    """GB/s of moe_requant_4to2 over n full-shape experts (4-bit bytes read + 2-bit bytes written),
    GPU events around each call, median."""
    import torch
    import synth
    import quantized_expert_dequant_amd as moe
    H, I = 4096, 1024
    c = synth.experts(1001, 0, 0, n, 4, H, I)
    ins = [torch.from_numpy(np.ascontiguousarray(a.reshape(n, -1))).to(dev)
           for a in (c.gate, c.up, c.down, c.scales, c.biases)]
    g2 = torch.empty((n, I * H // 4), dtype=torch.uint8, device=dev)
    u2 = torch.empty_like(g2)
    d2 = torch.empty((n, H * I // 4), dtype=torch.uint8, device=dev)
    s2, b2 = torch.empty_like(ins[3]), torch.empty_like(ins[4])
    moe.requant_4to2(H, I, n, *ins, g2, u2, d2, s2, b2)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        moe.requant_4to2(H, I, n, *ins, g2, u2, d2, s2, b2)
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    ms = _median(times)
    nbytes = n * (moe.record_bytes(4, H, I) + moe.record_bytes(2, H, I))
    return {"experts": n, "ms": round(ms, 4), "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "bytes_4bit_per_expert": moe.record_bytes(4, H, I), "bytes_2bit_per_expert": moe.record_bytes(2, H, I)}


ATTN_SHAPES = {
    # GatedDeltaNet: heads, key and value dims; full attention: query heads, KV heads, head dim
    "gdn": dict(n=64, dk=128, dv=128),
    "attn": dict(n_q=32, n_kv=2, d=256),
}


def measure_attention(dev, reps=5, calls=48, contexts=(4096, 32768)):
    """Per-call GPU time of the attention half of a decode step at the synthetic shapes
    above: moe_gdn_step over `calls` distinct states (so each call reads its state from
    HBM, not from the previous call's cache lines) and moe_attn_decode over distinct KV
    caches per context length.  The calls are captured in one HIP graph; GPU events
    around a replay, median of `reps` replays, divided by the calls.  Bytes are the
    algorithmic ones: the state read and written, or the cache read once, plus q and o."""
    import torch
    import quantized_expert_dequant_amd as moe
    torch.manual_seed(5)
    out = {}

    def timed(fn, count):
        fn(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(count):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e3 / count)
        del g
        return _median(ts)

    def entry(shape, us, nbytes):
        gbps = nbytes / (us * 1e-6) / 1e9
        return {"shape": shape, "us_per_call": round(us, 3), "bytes_per_call": nbytes, "gbps": round(gbps, 1),
                "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4)}

    gs = ATTN_SHAPES["gdn"]
    n, dk, dv = gs["n"], gs["dk"], gs["dv"]
    states = torch.randn(calls, n, dv, dk, device=dev).mul_(0.05)
    q = torch.randn(n, dk, device=dev).div_(dk ** 0.5)
    k = torch.nn.functional.normalize(torch.randn(n, dk, device=dev), dim=1)
    v = torch.randn(n, dv, device=dev)
    alpha = torch.rand(n, device=dev).mul_(0.2).add_(0.8)
    beta = torch.rand(n, device=dev)
    o = torch.empty(n, dv, device=dev)
    us = timed(lambda i: moe.gdn_step(n, dk, dv, states[i], q, k, v, alpha, beta, o), calls)
    out["gdn_step"] = entry(gs, us, 8 * n * dv * dk + 4 * (2 * n * dk + 2 * n * dv + 2 * n))
    del states
    a = ATTN_SHAPES["attn"]
    n_q, n_kv, d = a["n_q"], a["n_kv"], a["d"]
    qa = torch.randn(n_q, d, device=dev)
    oa = torch.empty(n_q, d, device=dev)
    for T in contexts:
        per = calls if T <= 4096 else max(4, calls // 8)
        K = torch.randn(per, n_kv, T, d, device=dev).to(torch.bfloat16).view(torch.int16)
        V = torch.randn(per, n_kv, T, d, device=dev).to(torch.bfloat16).view(torch.int16)
        wsb = moe.attn_workspace_bytes(n_q, n_kv, d, T)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        us = timed(lambda i: moe.attn_decode(n_q, n_kv, d, T, qa, K[i], V[i], oa, ws, wsb), per)
        out["attn_decode_T%d" % T] = entry(dict(a, T=T), us, 2 * 2 * n_kv * T * d + 4 * 2 * n_q * d)
        del K, V
    return out


def cpu_baseline(c, budget_s=15.0):
    """The float64 oracle as it stands on the host cores, on a bounded sample of tokens of the
    timed layer: tokens decoded on OpenMP threads (oracle_layer_decode_par, each token by the
    serial oracle), and the serial oracle on one thread."""
    import oracle
    import synth
    omp = os.environ.get("OMP_NUM_THREADS", "")
    ncpu = os.cpu_count() or 1
    threads = int(omp) if omp.isdigit() and int(omp) > 0 else ncpu
    E, K, H, I = c["E"], c["K"], c["H"], c["I"]
    Wr = synth.router(c["seed"], 0, E, H)
    prior = synth.zipf_bias(E, c["zipf"]) if c["zipf"] else None

    def batch(first, n):
        x = synth.tokens(c["seed"], 10_000 + first, n, H)
        lg = oracle.router_logits(x, Wr, prior)
        need = {E} | {int(e) for b in range(n) for e in oracle.topk(lg[b], K)[0]}
        ex = {e: synth.experts(c["seed"], 0, e, 1, c["bits"], H, I) for e in sorted(need)}
        return x, ex

    # one thread: the serial oracle on two tokens
    x, ex = batch(0, 2)
    t0 = time.perf_counter()
    oracle.layer_decode(c["bits"], H, I, E, K, x, Wr, ex, prior=prior)
    one = 2 / (time.perf_counter() - t0)
    # all threads: tokens decoded in parallel, until the budget is spent
    n_tok, elapsed, first = 0, 0.0, 2
    while elapsed < budget_s and n_tok < 512:
        x, ex = batch(first, threads)
        t0 = time.perf_counter()
        oracle.layer_decode(c["bits"], H, I, E, K, x, Wr, ex, prior=prior, parallel=True)
        elapsed += time.perf_counter() - t0
        n_tok += threads
        first += threads
    return {"value": round(n_tok / elapsed, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d tokens of the timed layer, %d at a time on %d OpenMP threads (float64 oracle, each token "
                      "decoded by the serial oracle; weight generation excluded); nproc=%d OMP_NUM_THREADS=%s"
                      % (n_tok, threads, threads, ncpu, omp or "unset"),
            "one_thread_tokens_per_s": round(one, 3)}


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--pmc-summary":
        # bench.py --pmc-summary WORKLOAD KERNEL FETCH.csv WRITE.csv COPY_FETCH.csv COPY_WRITE.csv COPY_MIB
        a = sys.argv[2:]
        write_pmc_summary(a[0], a[1], a[2], a[3], a[4], a[5], int(a[6]))
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="layer", choices=sorted(WORKLOADS))
    ap.add_argument("--rotate", type=int, default=16)
    ap.add_argument("--distinct", type=int, default=0,
                    help="stack: generate this many distinct layers and fill the rest with device copies "
                         "(0 = every layer distinct)")
    ap.add_argument("--replays", type=int, default=5, help="graph replays timed (median reported)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-eager", action="store_true", help="skip the per-kernel event pass (profiling runs)")
    ap.add_argument("--no-configs", action="store_true", help="time the named workload only")
    ap.add_argument("--lead-ms", type=float, default=30.0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--attention", action="store_true",
                    help="only time the attention half (GatedDeltaNet step, decode attention) and print its JSON")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB (PMC counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the decode path is built and measured on a single MI355X "
              "(see the sharding notes); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.replays < 1 or args.rotate < 1 or args.distinct < 0:
        ap.error("--steps, --replays and --rotate must be >= 1, --warmup and --distinct >= 0")

    import torch
    import quantized_expert_dequant_amd as moe

    dev = "cuda"
    torch.cuda.init()
    moe.lib()

    if args.copy_calibration_mb:
        n = args.copy_calibration_mb << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return

    if args.attention:
        print(json.dumps({"attention": measure_attention(dev)}), flush=True)
        return

    c = dict(WORKLOADS[args.workload])
    r = measure(args.workload, args.steps, args.warmup, dev, rotate=args.rotate, distinct=args.distinct,
                graph=not args.no_graph, eager=not args.no_eager, warm=True, replays=args.replays,
                lead_ms=args.lead_ms)
    if not r["parity_ok"]:
        print(json.dumps({"metric": METRIC, "value": None, "error": "parity check failed",
                          "rel_err": r["parity_rel_err"]}))
        sys.exit(1)
    if "kernel_us" not in r:
        print(json.dumps({"metric": METRIC, "value": r["tokens_per_s"], "unit": "tokens/s",
                          "ms_per_step": r["ms_per_step"], "note": "kernel event pass skipped"}), flush=True)
        return
    B, stack = c["B"], c["layers"] > 1
    traffic = traffic_from_profile(args.workload, c["layers"])
    gu_us = r["kernel_us"]["gateup"]
    out = {
        "metric": METRIC,
        "value": r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": expert_dtype(c),
        "data": "synthetic",
        "config": {"workload": r["config"], "global_batch": B, "rotation_copies": r["rotation_copies"],
                   "timing": r["timing"] + (" (median of %d replays, GPU events)" % args.replays
                                            if r["timing"] == "graph" else ""),
                   **({"distinct_layers": r["distinct_layers"]} if stack else {})},
        "roofline": {"bound": "hbm", "achieved": r["gateup_gbps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(r["gateup_gbps"] / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "kernel": (("gate/up phase: k_grouped_mfma<0, 4> + k_gemv_gateup" if c["bits"] == 4 else
                                 "gate/up phase: k_grouped_mfma<0, %d> + k_fixup" % c["bits"]) if B > 1
                                else "k_gateup_fast"),
                     "bytes_per_launch": r["gateup_bytes_per_launch"], "avg_us": gu_us,
                     "step_frac": r["step_frac"]},
        "expert_weight_gbps": r["expert_weight_gbps"],
        "expert_weight_frac_of_peak": r["expert_weight_frac_of_peak"],
        "kernel_us": r["kernel_us"],
        "graph_replays_ms_per_step": r.get("graph_replays_ms_per_step"),
        "eager_ms_per_step": r["eager_ms_per_step"],
        **({"warm_ms_per_step": r["warm_ms_per_step"]} if "warm_ms_per_step" in r else {}),
        **({"eager_step_us": r["eager_step_us"]} if "eager_step_us" in r else {}),
        **({"distinct_experts_per_step": r["distinct_experts_per_step"]} if B > 1 else {}),
        "parity_rel_err": r["parity_rel_err"],
    }
    if not args.no_configs:
        # every other workload at its own shape, fewer steps, same measurement
        extra = {"layer2": dict(steps=100, warmup=10), "requant": dict(steps=100, warmup=10),
                 "layer_g128": dict(steps=100, warmup=10), "layer3": dict(steps=100, warmup=10),
                 "batched": dict(steps=40, warmup=5), "batched2": dict(steps=40, warmup=5),
                 "batched3": dict(steps=40, warmup=5),
                 "stack": dict(steps=10, warmup=2, distinct=4),
                 "layer": dict(steps=100, warmup=10)}
        cfgs = {}
        for name, kw in extra.items():
            if name == args.workload:
                continue
            e = measure(name, kw["steps"], kw["warmup"], dev, rotate=args.rotate, distinct=kw.get("distinct", 0),
                        warm=False, replays=3, lead_ms=args.lead_ms)
            keep = ("config", "parity_ok", "parity_rel_err", "steps", "ms_per_step", "tokens_per_s",
                    "expert_bytes_per_token", "expert_weight_gbps", "expert_weight_frac_of_peak", "gateup_gbps",
                    "step_frac", "kernel_us", "distinct_experts_per_step", "distinct_layers")
            e = {k: e[k] for k in keep if k in e}
            if "gateup_gbps" in e:
                e["gateup_frac"] = round(e["gateup_gbps"] / PEAK_HBM_GBPS, 4)
            if name == "requant":
                e["requant_kernel"] = requant_throughput(dev)
            cfgs[name] = e
        cfgs["tiered"] = measure_tiered(dev)
        cfgs["attention"] = measure_attention(dev)
        out["configs"] = cfgs
    if not args.cpu_seconds <= 0:
        log("timing the oracle on the host ...")
        if stack:
            cb = cpu_baseline(dict(c, layers=1), args.cpu_seconds)
            cb["value"] = round(cb["value"] / c["layers"], 4)
            cb["one_thread_tokens_per_s"] = round(cb["one_thread_tokens_per_s"] / c["layers"], 5)
            cb["sample"] += "; per-layer time extrapolated to %d layers (one layer timed)" % c["layers"]
            out["cpu_baseline"] = cb
        else:
            out["cpu_baseline"] = cpu_baseline(c, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
