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
  * graph: K steps captured once into a HIP graph (launch-bound loop) and
    replayed; gives ms_per_step and the headline tokens/s.
  * eager: the same K steps launched one by one with start/stop HIP events
    recorded around the router, gate/up and down kernels on their stream;
    gives each kernel's average duration, hence achieved GB/s.
The float64 oracle is timed on the host cores on a small sample of tokens
(cpu_baseline).  One token is checked against the oracle before timing; a
mismatch reports no throughput.

    python bench.py [--steps K] [--warmup W] [--workload layer|layer2|batched|stack]
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

    def destroy(self, e):
        self.h.hipEventDestroy(e)


def gateup_bytes_per_expert(c):
    return 2 * c["I"] * c["H"] * c["bits"] // 8 + 2 * c["I"] * (c["H"] // 64) * 4


def down_bytes_per_expert(c):
    return c["H"] * c["I"] * c["bits"] // 8 + c["H"] * (c["I"] // 64) * 4


def build_layers(c, n_distinct, n_copies, dev):
    import torch
    import synth
    from quantized_expert_dequant_amd.slab import DeviceLayer, upload_experts
    H, I, E, K, bits = c["H"], c["I"], c["E"], c["K"], c["bits"]
    base = []
    for l in range(n_distinct):
        t0 = time.time()
        src = lambda first, n, l=l: synth.experts(c["seed"], l, first, n, bits, H, I)
        slab = upload_experts(src, E + 1, bits, H, I, device=dev)
        wr = torch.from_numpy(synth.router(c["seed"], l, E, H)).to(dev)
        bias = torch.from_numpy(synth.zipf_bias(E, c["zipf"])).to(dev) if c["zipf"] else None
        base.append(DeviceLayer(H, I, E, K, bits, slab, wr, bias))
        log("layer %d packed in %.1fs" % (l, time.time() - t0))
    layers = list(base)
    for r in range(n_distinct, n_copies):
        b = base[r % n_distinct]
        layers.append(DeviceLayer(H, I, E, K, bits, b.slab.clone(), b.w_router.clone(),
                                  None if b.logit_bias is None else b.logit_bias.clone()))
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
    experts = {e: synth.experts(c["seed"], layer_id, e, 1, c["bits"], c["H"], c["I"]) for e in sorted(need)}
    y_ref, idx_ref, _, _ = oracle.layer_decode(c["bits"], c["H"], c["I"], E, K, x_host, Wr, experts, prior=prior)
    # per token max|dy| / max|y_ref|, the denominator floored where fp32 cannot represent the tolerance
    err = max(float(np.max(np.abs(y_dev[b] - y_ref[b])) / max(np.max(np.abs(y_ref[b])), 2.0 ** -126 / 2e-3))
              for b in range(x_host.shape[0]))
    return bool(np.array_equal(idx_dev, idx_ref)) and err <= 2e-3, err


def cpu_baseline(c, budget_s=15.0):
    """The float64 oracle as it stands, on the host cores, on a bounded sample of tokens."""
    import oracle
    import synth
    cores = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or min(os.cpu_count() or 1, 16)
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    E, K, H = c["E"], c["K"], c["H"]
    Wr = synth.router(c["seed"], 0, E, H)
    prior = synth.zipf_bias(E, c["zipf"]) if c["zipf"] else None
    n_tok, elapsed = 0, 0.0
    while elapsed < budget_s and n_tok < 64:
        x = synth.tokens(c["seed"], 10_000 + n_tok, 1, H)[0]
        lg = oracle.router_logits(x, Wr, prior)[0]
        sel = oracle.topk(lg, K)[0]
        experts = {e: synth.experts(c["seed"], 0, e, 1, c["bits"], H, c["I"]) for e in sorted(set(sel) | {E})}
        t0 = time.perf_counter()
        oracle.layer_decode_mt(c["bits"], H, c["I"], E, K, x, Wr, experts, prior=prior)
        elapsed += time.perf_counter() - t0
        n_tok += 1
    return {"value": n_tok / elapsed, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%d tokens of the timed layer (one token per decode step), float64 oracle with the active "
                      "experts' FFNs spread over OpenMP threads; weight generation excluded" % n_tok}


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
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-eager", action="store_true", help="skip the per-kernel event pass (profiling runs)")
    ap.add_argument("--lead-ms", type=float, default=30.0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB (PMC counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the decode path is built and measured on a single MI355X "
              "(see the sharding notes); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import quantized_expert_dequant_amd as moe
    from quantized_expert_dequant_amd.slab import workspace

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

    c = dict(WORKLOADS[args.workload])
    K, W, B, H = args.steps, args.warmup, c["B"], c["H"]
    stack = c["layers"] > 1
    n_distinct = min(args.distinct or c["layers"], c["layers"]) if stack else 1
    n_copies = c["layers"] if stack else max(1, args.rotate)
    log("workload %s: building %d layer(s) (%d distinct)" % (args.workload, n_copies, n_distinct))
    layers = build_layers(c, n_distinct, n_copies, dev)

    # tokens for every warmup + timed step, resident in HBM before timing
    xs_host = np.stack([synth.tokens(c["seed"], t, B, H) for t in range(W + K)])
    xs = torch.from_numpy(xs_host).to(dev)
    ws, ws_n = workspace(layers[0].desc, B, stack=stack)
    y = torch.empty((W + K, B, H), dtype=torch.float32, device=dev)
    nL = c["layers"]
    idx = torch.empty((W + K, nL, B, c["K"]), dtype=torch.int32, device=dev)
    wts = torch.empty((W + K, nL, B, c["K"]), dtype=torch.float32, device=dev)
    descs = [L.desc for L in layers]

    def step(t):
        if stack:
            moe.stack_decode(descs, xs[t], B, RMS_EPS, y[t], idx[t], wts[t], ws, ws_n)
        else:
            L = layers[t % n_copies]
            moe.layer_decode(L.desc, xs[t], B, y[t], idx[t, 0], wts[t, 0], ws, ws_n)

    # parity spot check on the first token (layer copy 0 == distinct layer 0)
    step(0)
    torch.cuda.synchronize()
    if stack:
        # layer 0 of the first token, decoded on its own, against the oracle (every layer of a
        # short stack is checked teacher-forced in the GPU tests)
        y0 = torch.empty((B, H), dtype=torch.float32, device=dev)
        i0 = torch.empty((B, c["K"]), dtype=torch.int32, device=dev)
        w0 = torch.empty((B, c["K"]), dtype=torch.float32, device=dev)
        moe.layer_decode(layers[0].desc, xs[0], B, y0, i0, w0, ws, ws_n)
        torch.cuda.synchronize()
        ok, err = oracle_check(c, xs_host[0], y0.cpu().numpy(), i0.cpu().numpy())
        ok = ok and bool(torch.equal(i0, idx[0, 0]))
    else:
        ok, err = oracle_check(c, xs_host[0], y[0].cpu().numpy(), idx[0, 0].cpu().numpy())
    log("parity spot check: ok=%s max rel err %.3e" % (ok, err))
    if not ok:
        print(json.dumps({"metric": METRIC, "value": None, "error": "parity check failed", "rel_err": err}))
        sys.exit(1)

    for t in range(W):
        step(t)
    torch.cuda.synchronize()

    # ---- timed region 1: graph replay of K steps -----------------------------
    graph_ms = None
    if not args.no_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for t in range(W, W + K):
                    step(t)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g.replay()                      # one untimed replay, then check it against eager
        torch.cuda.synchronize()
        y_graph = y[W + K - 1].clone()
        step(W + K - 1)
        torch.cuda.synchronize()
        if not torch.equal(y_graph, y[W + K - 1]):
            log("graph replay differs from eager: graph timing disabled")
        else:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            g.replay()
            torch.cuda.synchronize()
            graph_ms = (time.perf_counter() - t0) * 1e3 / K
        del g

    # ---- timed region 2: eager steps with kernel events ------------------------
    kinds = [moe.KERNEL_ROUTER, moe.KERNEL_GATEUP, moe.KERNEL_DOWN]
    dur = {k: None for k in kinds}
    eager_ms = None
    eager_pct = None
    if not args.no_eager:
        hip = Hip()
        ev = {k: [(hip.event(), hip.event()) for _ in range(K)] for k in kinds}
        torch.cuda.synchronize()
        # a bounded delay kernel first, so the host has enqueued the steps before the
        # GPU reaches them and the kernels run back to back, as they do in the graph
        torch.cuda._sleep(int(args.lead_ms * 2.4e6))
        for i, t in enumerate(range(W, W + K)):
            for k in kinds:
                moe.set_timing_events(k, *ev[k][i])
            step(t)
        torch.cuda.synchronize()
        for k in kinds:
            moe.set_timing_events(k, None, None)
        # with several layers per step the hook re-records each pair on every layer,
        # so each pair times the step's last launch of that kernel
        dur = {k: sum(hip.elapsed_ms(a, b) for a, b in ev[k]) / K for k in kinds}
        eager_ms = hip.elapsed_ms(ev[moe.KERNEL_ROUTER][0][0], ev[moe.KERNEL_DOWN][K - 1][1]) / K
        if not stack:  # per-step spread: router start to down end of each step
            st = np.array([hip.elapsed_ms(ev[moe.KERNEL_ROUTER][i][0], ev[moe.KERNEL_DOWN][i][1]) * 1e3
                           for i in range(K)])
            eager_pct = {"p10": round(float(np.percentile(st, 10)), 3), "p50": round(float(np.percentile(st, 50)), 3),
                         "p90": round(float(np.percentile(st, 90)), 3)}
        for k in kinds:
            for a, b in ev[k]:
                hip.destroy(a)
                hip.destroy(b)
    launches = nL

    # ---- numbers ---------------------------------------------------------------
    ms_per_step = graph_ms if graph_ms is not None else eager_ms
    tokens_per_step = B
    value = tokens_per_step / (ms_per_step / 1e3)
    idx_h = idx[W:W + K].cpu().numpy()
    if B > 1:
        # the grouped path reads each distinct routed expert once per step, plus the shared one
        uniq = [len(np.unique(idx_h[i, 0][(idx_h[i, 0] >= 0) & (idx_h[i, 0] < c["E"])])) for i in range(K)]
        n_experts = float(np.mean(uniq)) + 1
    else:
        n_experts = c["K"] + 1
    n_act = n_experts
    gu_bytes = gateup_bytes_per_expert(c) * n_act
    dn_bytes = down_bytes_per_expert(c) * n_act
    if dur[moe.KERNEL_GATEUP] is None:
        print(json.dumps({"metric": METRIC, "value": round(value, 2), "unit": "tokens/s",
                          "ms_per_step": round(ms_per_step, 6), "note": "kernel event pass skipped"}), flush=True)
        return
    gu_us = dur[moe.KERNEL_GATEUP] * 1e3
    dn_us = dur[moe.KERNEL_DOWN] * 1e3
    rt_us = dur[moe.KERNEL_ROUTER] * 1e3
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    expert_gbps = (gu_bytes + dn_bytes) / ((gu_us + dn_us) * 1e-6) / 1e9
    traffic = traffic_from_profile(args.workload, launches)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",  # fp16 x fp16 products (codes turned exactly into fp16), fp32 accumulation
        "data": "synthetic",
        "config": {"workload": "%s: H=%d I=%d E=%d+1 shared K=%d %d-bit group 64 bf16 scale+bias, B=%d%s" % (
            args.workload, H, c["I"], c["E"], c["K"], c["bits"], B,
            ", %d layers with RMS renorm" % nL if stack else ""),
            "global_batch": B, "rotation_copies": n_copies, "timing": "graph" if graph_ms else "eager",
            **({"distinct_layers": n_distinct} if stack else {})},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "kernel": ("gate/up phase: k_grouped_mfma<0> + k_gemv_gateup" if B > 1
                                else "k_gateup_fast"),
                     "bytes_per_launch": round(gu_bytes), "avg_us": round(gu_us, 3)},
        "expert_weight_gbps": round(expert_gbps, 1),
        "expert_weight_frac_of_peak": round(expert_gbps / PEAK_HBM_GBPS, 4),
        "kernel_us": {"router": round(rt_us, 3), "gateup": round(gu_us, 3), "down": round(dn_us, 3)},
        "eager_ms_per_step": round(eager_ms, 6),
        **({"eager_step_us": eager_pct} if eager_pct else {}),
        "parity_rel_err": err,
    }
    if B > 1:
        out["distinct_experts_per_step"] = n_experts
    if not args.cpu_seconds <= 0:
        log("timing the oracle on the host ...")
        if stack:
            # one layer of the stack's shape timed on the host, per token through nL layers
            cb = cpu_baseline(dict(c, layers=1, seed=c["seed"]), args.cpu_seconds)
            cb["value"] = cb["value"] / nL
            cb["sample"] += "; per-layer time extrapolated to %d layers (one layer timed)" % nL
            out["cpu_baseline"] = cb
        else:
            out["cpu_baseline"] = cpu_baseline(c, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
