"""Shared test glue: the synthetic workloads, device layers built from them, and
the oracle run on the same seeded inputs.

Workloads (seed = 1000 + workload number):
  0 tiny layer    H=512  I=128  E=16  K=4  4-bit, 1 token
  1 full layer    H=4096 I=1024 E=512 K=4  4-bit, 1 token
  2 full layer    as 1 with 2-bit codes
  3 layer stack   60 layers of workload-1 shape, RMS renorm between layers
  4 batched       workload-1 layer, B=64, K=10, Zipf(1.1) prior on the logits
"""
import numpy as np

import oracle
import synth

WORKLOADS = {
    0: dict(H=512, I=128, E=16, K=4, bits=4, B=1, layers=1, zipf=None),
    1: dict(H=4096, I=1024, E=512, K=4, bits=4, B=1, layers=1, zipf=None),
    2: dict(H=4096, I=1024, E=512, K=4, bits=2, B=1, layers=1, zipf=None),
    3: dict(H=4096, I=1024, E=512, K=4, bits=4, B=1, layers=60, zipf=None),
    4: dict(H=4096, I=1024, E=512, K=10, bits=4, B=64, layers=1, zipf=1.1),
}
TOL = 2e-3       # max |y - y_ref| / max |y_ref| per token
W_RTOL = 1e-6    # routing weights
RMS_EPS = 1e-6


def seed_of(n):
    return 1000 + n


def build_layer(cfg, seed, layer=0, device="cuda"):
    import torch
    from quantized_expert_dequant_amd.slab import DeviceLayer, upload_experts
    H, I, E, K, bits = cfg["H"], cfg["I"], cfg["E"], cfg["K"], cfg["bits"]
    group = cfg.get("group", 64)
    src = lambda first, n: synth.experts(seed, layer, first, n, bits, H, I, group)
    slab = upload_experts(src, E + 1, bits, H, I, device=device, group=group)
    wr = torch.from_numpy(synth.router(seed, layer, E, H)).to(device)
    bias = None
    if cfg.get("zipf"):
        bias = torch.from_numpy(synth.zipf_bias(E, cfg["zipf"])).to(device)
    return DeviceLayer(H, I, E, K, bits, slab, wr, bias, group=group)


FP32_FLOOR = 2.0 ** -126   # smallest normal fp32: y is delivered in fp32


def rel_err(y, y_ref):
    """max |y - y_ref| / max |y_ref|, with the denominator floored at FP32_FLOOR / TOL.

    rel_err <= TOL then means max|dy| <= max(TOL * max|y_ref|, FP32_FLOOR): a token whose
    exact output lies below the fp32 normal range (a layer whose SiLU saturates everywhere)
    is correct when the fp32 output is that small too.
    """
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    return float(np.max(np.abs(y - y_ref)) / max(np.max(np.abs(y_ref)), FP32_FLOOR / TOL))


def oracle_route(cfg, seed, layer, x):
    """Oracle logits/selection for tokens x [B][H] (float32)."""
    Wr = synth.router(seed, layer, cfg["E"], cfg["H"])
    prior = synth.zipf_bias(cfg["E"], cfg["zipf"]) if cfg.get("zipf") else None
    lg = oracle.router_logits(x, Wr, prior)
    sel = [oracle.topk(lg[b], cfg["K"]) for b in range(x.shape[0])]
    return Wr, prior, lg, sel


def oracle_layer(cfg, seed, layer, x, shared_weight=1.0, parallel=False):
    """Oracle decode of tokens x through one layer, generating only the experts it selects.
    parallel=True decodes the tokens on OpenMP threads (each token by the serial oracle)."""
    x = np.atleast_2d(np.asarray(x, np.float32))
    Wr, prior, lg, sel = oracle_route(cfg, seed, layer, x)
    need = sorted({int(e) for s in sel for e in s[0]} | {cfg["E"]})
    group = cfg.get("group", 64)
    experts = {e: synth.experts(seed, layer, e, 1, cfg["bits"], cfg["H"], cfg["I"], group) for e in need}
    return oracle.layer_decode(cfg["bits"], cfg["H"], cfg["I"], cfg["E"], cfg["K"], x, Wr, experts, prior=prior,
                               shared_weight=shared_weight, group=group, parallel=parallel)


def mfma_tiles(idx, E, info):
    """Gate/up matrix-core tiles of a batch's routing, by the grouping rule the library states
    (moe_grouped_launch_info): the shared expert's B tokens and every routed expert with at
    least gemv_below_tokens tokens are cut into groups of at most group_tokens."""
    B = idx.shape[0]
    counts = np.bincount(idx[(idx >= 0) & (idx < E)].ravel(), minlength=E)
    g, lo = info["group_tokens"], info["gemv_below_tokens"]
    groups = (-(-B // g) if B >= lo else 0) + sum(-(-int(c) // g) for c in counts if c >= lo)
    return groups * info["gateup_tiles_per_group"]
