"""GPU parity of the offline 4-bit -> 2-bit requantization (moe_requant_4to2).

The codes, scales and biases it writes must equal the oracle's bit for bit: the
reading fixes every operation (IEEE double, ties to even), so the integer codes
follow from them.  A whole layer requantized on the GPU, packed as 2-bit records
and decoded must then match the oracle's decode of the oracle-requantized experts
(indices bit-exact, each token's output within 2e-3 relative).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import quantized_expert_dequant_amd as moe
from quantized_expert_dequant_amd.slab import DeviceLayer, upload_requantized, workspace

from helpers import TOL, W_RTOL, WORKLOADS, oracle_route, rel_err, seed_of

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    moe.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _requant_gpu(c, H, I):
    n = c.gate.shape[0]
    ins = [torch.from_numpy(np.ascontiguousarray(a.reshape(n, -1))).to(DEV)
           for a in (c.gate, c.up, c.down, c.scales, c.biases)]
    g2 = torch.empty((n, I * H // 4), dtype=torch.uint8, device=DEV)
    u2 = torch.empty_like(g2)
    d2 = torch.empty((n, H * I // 4), dtype=torch.uint8, device=DEV)
    s2, b2 = torch.empty_like(ins[3]), torch.empty_like(ins[4])
    moe.requant_4to2(H, I, n, *ins, g2, u2, d2, s2, b2)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (g2, u2, d2, s2, b2)]


def _check_bit_exact(c, H, I):
    got = _requant_gpu(c, H, I)
    for j in range(c.gate.shape[0]):
        ref = oracle.requant_expert(H, I, c.gate[j], c.up[j], c.down[j], c.scales[j], c.biases[j])
        for name, g, r in zip(("gate", "up", "down", "scales", "biases"), got, ref):
            np.testing.assert_array_equal(g[j].reshape(-1), r.reshape(-1), err_msg="%s of expert %d" % (name, j))


def test_requant_bit_exact_tiny_layer():
    H, I, E = 512, 128, 16
    _check_bit_exact(synth.experts(seed_of(0), 0, 0, E + 1, 4, H, I), H, I)


def test_requant_bit_exact_full_shape():
    H, I = 4096, 1024
    for first in (0, 511):  # routed experts 0, 1 and the last routed + the shared one
        _check_bit_exact(synth.experts(seed_of(1), 0, first, 2, 4, H, I), H, I)


def test_requant_edge_groups():
    """Hand-picked scales and biases: zero and negative scales (constant and reversed
    groups), ties, bf16 subnormals, magnitudes near the bf16 range ends, signed zeros."""
    H, I, n = 128, 64, 3
    c = synth.experts(seed_of(0), 0, 0, n, 4, H, I)
    rng = np.random.default_rng(9)
    edge = np.array([0x0000, 0x8000, 0x3F00, 0xBF00, 0x3F80, 0xBF80, 0x0001, 0x8001, 0x0080, 0x7F7F,
                     0x7E00, 0x4040, 0x00FF, 0x3C00], np.uint16)
    c.scales[...] = rng.choice(edge, size=c.scales.shape)
    c.biases[...] = rng.choice(edge, size=c.biases.shape)
    _check_bit_exact(c, H, I)


def test_requantized_layer_decode_matches_oracle():
    """The full workload-1 layer requantized on the GPU and packed as 2-bit records: 4 tokens
    decoded against the oracle on the oracle-requantized selected experts."""
    cfg, seed = dict(WORKLOADS[1]), seed_of(1)
    H, I, E, K = cfg["H"], cfg["I"], cfg["E"], cfg["K"]
    slab = upload_requantized(lambda f, n: synth.experts(seed, 0, f, n, 4, H, I), E + 1, H, I, device=DEV)
    wr = torch.from_numpy(synth.router(seed, 0, E, H)).to(DEV)
    L = DeviceLayer(H, I, E, K, 2, slab, wr)
    B = 4
    x = synth.tokens(seed, 70, B, H)
    ws, nb = workspace(L.desc, B)
    y = torch.empty((B, H), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, K), dtype=torch.int32, device=DEV)
    w = torch.empty((B, K), dtype=torch.float32, device=DEV)
    moe.layer_decode(L.desc, torch.from_numpy(x).to(DEV), B, y, idx, w, ws, nb)
    torch.cuda.synchronize()
    Wr, prior, lg, sel = oracle_route(cfg, seed, 0, x)
    need = sorted({int(e) for s in sel for e in s[0]} | {E})
    ex2 = {}
    for e in need:
        c = synth.experts(seed, 0, e, 1, 4, H, I)
        g2, u2, d2, s2, b2 = oracle.requant_expert(H, I, c.gate[0], c.up[0], c.down[0], c.scales[0], c.biases[0])
        ex2[e] = synth.Canonical(2, H, I, 64, g2[None], u2[None], d2[None], s2[None], b2[None])
    y_ref, idx_ref, w_ref, margin = oracle.layer_decode(2, H, I, E, K, x, Wr, ex2)
    assert margin.min() > 1e-9
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_ref)
    np.testing.assert_allclose(w.cpu().numpy(), w_ref, rtol=W_RTOL)
    yh = y.cpu().numpy()
    for b in range(B):
        assert rel_err(yh[b], y_ref[b]) <= TOL, "token %d" % b
    # how far the 2-bit refit moves the layer's output from the 4-bit layer's (informative)
    ex4 = {e: synth.experts(seed, 0, e, 1, 4, H, I) for e in need}
    y4, _, _, _ = oracle.layer_decode(4, H, I, E, K, x, Wr, ex4)
    dev = [float(np.linalg.norm(y_ref[b] - y4[b]) / np.linalg.norm(y4[b])) for b in range(B)]
    print("requantized layer: output deviation from the 4-bit layer %.3f .. %.3f (relative L2)" % (min(dev), max(dev)))
    del L, slab
    torch.cuda.empty_cache()
