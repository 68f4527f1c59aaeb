"""GPU parity of the stacked decode (layers in sequence, RMS renorm between them).

Teacher-forced: each layer's input x_l is the GPU's own (read back), the oracle
decodes that layer from it, and the expert indices must match bit-exactly and the
output within the per-token bar.  A free-running comparison over many layers is
not a gate: a last-bit difference in x can flip a near-tie routing many layers
later.  moe_stack_decode must also reproduce the layer-by-layer run bit-exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import quantized_expert_dequant_amd as moe
from quantized_expert_dequant_amd.slab import workspace

from helpers import RMS_EPS, TOL, W_RTOL, WORKLOADS, build_layer, oracle_layer, oracle_route, rel_err, seed_of

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    moe.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _run(cfg, seed, n_layers, B, step):
    layers = [build_layer(cfg, seed, layer=l) for l in range(n_layers)]
    H, K = cfg["H"], cfg["K"]
    x0 = synth.tokens(seed, step, B, H)
    # layer by layer: layer_decode, then rmsnorm, keeping every layer's input
    ws, n = workspace(layers[0].desc, B)
    xs, ys, idxs, wss = [x0], [], [], []
    x = _t(x0)
    for l, L in enumerate(layers):
        y = torch.empty((B, H), dtype=torch.float32, device=DEV)
        idx = torch.empty((B, K), dtype=torch.int32, device=DEV)
        w = torch.empty((B, K), dtype=torch.float32, device=DEV)
        moe.layer_decode(L.desc, x, B, y, idx, w, ws, n)
        ys.append(y.cpu().numpy())
        idxs.append(idx.cpu().numpy())
        wss.append(w.cpu().numpy())
        if l + 1 < n_layers:
            xn = torch.empty((B, H), dtype=torch.float32, device=DEV)
            moe.rmsnorm(y, B, H, RMS_EPS, xn)
            x = xn
            xs.append(xn.cpu().numpy())
    # the whole stack in one call
    ws2, n2 = workspace(layers[0].desc, B, stack=True)
    y_s = torch.empty((B, H), dtype=torch.float32, device=DEV)
    idx_s = torch.empty((n_layers, B, K), dtype=torch.int32, device=DEV)
    w_s = torch.empty((n_layers, B, K), dtype=torch.float32, device=DEV)
    moe.stack_decode([L.desc for L in layers], _t(x0), B, RMS_EPS, y_s, idx_s, w_s, ws2, n2)
    torch.cuda.synchronize()
    return xs, ys, idxs, wss, y_s.cpu().numpy(), idx_s.cpu().numpy(), w_s.cpu().numpy()


# (2, 3, 1): the 2-bit layers saturate SiLU, so layer 1's output is about 1e-22 and the
# renormalized input of layer 2 about 1e-19: the tiny-value end of every path
@pytest.mark.parametrize("n,n_layers,B", [(0, 6, 1), (0, 4, 3), (3, 3, 1), (2, 3, 1)])
def test_stack_teacher_forced(n, n_layers, B):
    cfg = dict(WORKLOADS[n])
    seed = seed_of(n)
    xs, ys, idxs, wss, y_s, idx_s, w_s = _run(cfg, seed, n_layers, B, step=0)
    # the stack call equals the layer-by-layer run, bit for bit
    np.testing.assert_array_equal(y_s, ys[-1])
    np.testing.assert_array_equal(idx_s, np.stack(idxs))
    np.testing.assert_array_equal(w_s, np.stack(wss))
    for l in range(n_layers):
        y_ref, idx_ref, w_ref, margin = oracle_layer(cfg, seed, l, xs[l])
        # a near-tie could flip with the summation order, whose error scales with the logits:
        # the K-th and (K+1)-th logits must differ by more than 1e-9 of the largest |logit|
        # (after a layer whose SiLU saturates, the renormalized input and every logit can be
        # tiny), or tie exactly (every logit 0 once a layer output has underflowed to zero),
        # which resolves to the lower id on both sides
        scale = np.max(np.abs(oracle_route(cfg, seed, l, xs[l])[2]), axis=1)
        assert np.all((margin > 1e-9 * scale) | (margin == 0.0)), "layer %d: routing margin below 1e-9" % l
        np.testing.assert_array_equal(idxs[l], idx_ref, err_msg="layer %d" % l)
        np.testing.assert_allclose(wss[l], w_ref, rtol=W_RTOL, err_msg="layer %d" % l)
        for b in range(B):
            assert rel_err(ys[l][b], y_ref[b]) <= TOL, "layer %d token %d" % (l, b)
        if l + 1 < n_layers:
            # the renorm between layers against the oracle's
            for b in range(B):
                np.testing.assert_allclose(xs[l + 1][b], oracle.rms_renorm(ys[l][b].astype(np.float64), RMS_EPS),
                                           rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("B", [1, 3])
def test_stack_mixed_code_widths(B):
    """A stack whose layers have 4-, 3- and 2-bit experts and groups of 64 and 128 (the tiny
    shape; one token through the straight-line kernels, three through the grouped ones): the
    stack call equals the layer-by-layer run bit for bit, and every layer matches the oracle
    teacher-forced."""
    base = dict(WORKLOADS[0])
    cfgs = [dict(base, bits=4), dict(base, bits=3), dict(base, bits=2, group=128), dict(base, bits=3, group=128)]
    seed = 1900 + B
    H, K = base["H"], base["K"]
    layers = [build_layer(c, seed, layer=l) for l, c in enumerate(cfgs)]
    x0 = synth.tokens(seed, 0, B, H)
    ws, n = workspace(layers[0].desc, B)
    xs, ys, idxs = [x0], [], []
    x = _t(x0)
    for l, L in enumerate(layers):
        y = torch.empty((B, H), dtype=torch.float32, device=DEV)
        idx = torch.empty((B, K), dtype=torch.int32, device=DEV)
        w = torch.empty((B, K), dtype=torch.float32, device=DEV)
        moe.layer_decode(L.desc, x, B, y, idx, w, ws, n)
        ys.append(y.cpu().numpy())
        idxs.append(idx.cpu().numpy())
        if l + 1 < len(layers):
            xn = torch.empty((B, H), dtype=torch.float32, device=DEV)
            moe.rmsnorm(y, B, H, RMS_EPS, xn)
            x = xn
            xs.append(xn.cpu().numpy())
    ws2, n2 = workspace(layers[0].desc, B, stack=True)
    y_s = torch.empty((B, H), dtype=torch.float32, device=DEV)
    idx_s = torch.empty((len(layers), B, K), dtype=torch.int32, device=DEV)
    w_s = torch.empty((len(layers), B, K), dtype=torch.float32, device=DEV)
    moe.stack_decode([L.desc for L in layers], _t(x0), B, RMS_EPS, y_s, idx_s, w_s, ws2, n2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y_s.cpu().numpy(), ys[-1])
    np.testing.assert_array_equal(idx_s.cpu().numpy(), np.stack(idxs))
    for l, c in enumerate(cfgs):
        y_ref, idx_ref, _, margin = oracle_layer(c, seed, l, xs[l])
        assert margin.min() > 1e-9, "layer %d" % l
        np.testing.assert_array_equal(idxs[l], idx_ref, err_msg="layer %d" % l)
        for b in range(B):
            assert rel_err(ys[l][b], y_ref[b]) <= TOL, "layer %d (%d-bit) token %d" % (l, c["bits"], b)

