"""GPU parity with quantization groups of 128 and 256 weights (one scale and bias each).

The packed codes are laid out as with groups of 64; only the scale/bias areas of a
record shrink, and every kernel takes the scale and bias of 64-column unit g from
group g >> log2(group / 64).  Bars as for groups of 64: the packed layout's
dequantized weights bit-exact against the oracle's exact dequantization rounded once
to fp32; requantized codes, scales and biases bit-exact; expert indices bit-exact,
routing weights within 1e-6 relative, each token's output within 2e-3 of its
largest magnitude.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import quantized_expert_dequant_amd as moe
from quantized_expert_dequant_amd.slab import upload_experts, upload_requantized, DeviceLayer, workspace

from helpers import TOL, W_RTOL, build_layer, oracle_layer, oracle_route, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    moe.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("bits,H,I,group", [(4, 512, 128, 128), (2, 512, 128, 128), (4, 512, 256, 256),
                                            (2, 768, 256, 256), (4, 4096, 1024, 128), (2, 4096, 1024, 256)])
def test_pack_dequant_bit_exact(bits, H, I, group):
    n = 3
    c = synth.experts(78, 5, 0, n, bits, H, I, group)
    slab = upload_experts(lambda f, k: synth.experts(78, 5, f, k, bits, H, I, group), n, bits, H, I, chunk=2,
                          group=group)
    rb = moe.record_bytes(bits, H, I, group)
    assert rb == 2 * I * H * bits // 8 + H * I * bits // 8 + 8 * I * (H // group) + 4 * H * (I // group)
    W = torch.empty(3 * I * H, dtype=torch.float32, device=DEV)
    for e in range(n):
        moe.dequant_expert(bits, H, I, slab[e * rb:(e + 1) * rb], W, group=group)
        Wg, Wu, Wd = oracle.dequant_expert(bits, H, I, c.gate[e], c.up[e], c.down[e], c.scales[e], c.biases[e],
                                           group=group)
        ref = np.concatenate([Wg.ravel(), Wu.ravel(), Wd.ravel()]).astype(np.float32)
        np.testing.assert_array_equal(W.cpu().numpy(), ref)


def _decode(layer, x):
    B = x.shape[0]
    ws, n = workspace(layer.desc, B)
    y = torch.empty((B, layer.H), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, layer.K), dtype=torch.int32, device=DEV)
    w = torch.empty((B, layer.K), dtype=torch.float32, device=DEV)
    moe.layer_decode(layer.desc, torch.from_numpy(x).to(DEV), B, y, idx, w, ws, n)
    torch.cuda.synchronize()
    return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def _check_layer(cfg, seed, B, step):
    L = build_layer(cfg, seed)
    x = synth.tokens(seed, step, B, cfg["H"])
    y, idx, w = _decode(L, x)
    y_ref, idx_ref, w_ref, margin = oracle_layer(cfg, seed, 0, x, parallel=B > 1)
    assert margin.min() > 1e-9
    np.testing.assert_array_equal(idx, idx_ref)
    np.testing.assert_allclose(w, w_ref, rtol=W_RTOL)
    for b in range(B):
        assert rel_err(y[b], y_ref[b]) <= TOL, "token %d: %.3e" % (b, rel_err(y[b], y_ref[b]))
    return L


@pytest.mark.parametrize("group", [128, 256])
@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("B", [1, 5, 40])
def test_layer_decode_tiny(group, bits, B):
    """The tiny layer (I = 256 so that 256 divides it): one token (the straight-line
    kernels), five (grouped: GEMV groups and, at 4 bits, matrix-core groups) and forty."""
    cfg = dict(H=512, I=256, E=16, K=4, bits=bits, B=B, layers=1, zipf=None, group=group)
    L = _check_layer(cfg, 1400 + group + bits, B, 3)
    assert moe.grouped_launch_info(L.desc, B)["grouped"] == (1 if B > 1 else 0)


@pytest.mark.parametrize("group,B", [(128, 1), (128, 8), (256, 1)])
def test_layer_decode_full_size(group, B):
    """The workload-1 shape (H = 4096, I = 1024, E = 512, K = 4, 4-bit) with larger groups."""
    cfg = dict(H=4096, I=1024, E=512, K=4, bits=4, B=B, layers=1, zipf=None, group=group)
    _check_layer(cfg, 1500 + group, B, 0)


@pytest.mark.parametrize("group", [128, 256])
def test_requant_bit_exact(group):
    """4-bit -> 2-bit requantization per group of 128 or 256 weights: codes, scales and biases
    equal the oracle's bit for bit."""
    H, I, n = 512, 256, 5
    c = synth.experts(1600 + group, 0, 0, n, 4, H, I, group)
    ins = [torch.from_numpy(np.ascontiguousarray(a.reshape(n, -1))).to(DEV)
           for a in (c.gate, c.up, c.down, c.scales, c.biases)]
    g2 = torch.empty((n, I * H // 4), dtype=torch.uint8, device=DEV)
    u2 = torch.empty_like(g2)
    d2 = torch.empty((n, H * I // 4), dtype=torch.uint8, device=DEV)
    s2, b2 = torch.empty_like(ins[3]), torch.empty_like(ins[4])
    moe.requant_4to2(H, I, n, *ins, g2, u2, d2, s2, b2, group=group)
    torch.cuda.synchronize()
    got = [t.cpu().numpy() for t in (g2, u2, d2, s2, b2)]
    for j in range(n):
        ref = oracle.requant_expert(H, I, c.gate[j], c.up[j], c.down[j], c.scales[j], c.biases[j], group=group)
        for name, g, r in zip(("gate", "up", "down", "scales", "biases"), got, ref):
            np.testing.assert_array_equal(g[j].reshape(-1), r.reshape(-1), err_msg="%s of expert %d" % (name, j))


def test_requantized_layer_decode_group_128():
    """The tiny layer requantized to 2 bits on the GPU with groups of 128, packed and decoded,
    against the oracle's decode of the oracle-requantized experts (one token and a batch)."""
    H, I, E, K, group = 512, 256, 16, 4, 128
    seed = 1700
    src4 = lambda f, k: synth.experts(seed, 0, f, k, 4, H, I, group)
    slab = upload_requantized(src4, E + 1, H, I, group=group)
    wr = torch.from_numpy(synth.router(seed, 0, E, H)).to(DEV)
    L = DeviceLayer(H, I, E, K, 2, slab, wr, group=group)
    c4 = src4(0, E + 1)
    experts = {}
    for e in range(E + 1):
        g2, u2, d2, s2, b2 = oracle.requant_expert(H, I, c4.gate[e], c4.up[e], c4.down[e], c4.scales[e],
                                                   c4.biases[e], group=group)
        experts[e] = synth.Canonical(2, H, I, group, g2[None], u2[None], d2[None], s2[None], b2[None])
    for B in (1, 6):
        x = synth.tokens(seed, 10 + B, B, H)
        y, idx, w = _decode(L, x)
        y_ref, idx_ref, w_ref, margin = oracle.layer_decode(2, H, I, E, K, x, synth.router(seed, 0, E, H), experts,
                                                             group=group)
        assert margin.min() > 1e-9
        np.testing.assert_array_equal(idx, idx_ref)
        np.testing.assert_allclose(w, w_ref, rtol=W_RTOL)
        for b in range(B):
            assert rel_err(y[b], y_ref[b]) <= TOL, "B=%d token %d" % (B, b)
