"""GPU parity with 3-bit expert codes.

A record holds each 64-column unit's codes as a 16-byte chunk of their low two bits
(the 2-bit chunk order) and two dwords of their high bits, laid out so that one
mask and one OR per code pair build the fp16 pattern 1024 + t*q the dot2 kernels
multiply.  Bars as for the other widths: the packed layout's dequantized weights
bit-exact against the oracle's exact dequantization rounded once to fp32; expert
indices bit-exact, routing weights within 1e-6 relative, each token's output within
2e-3 of its largest magnitude.  A 3-bit batch is grouped by expert like the other widths:
the matrix-core kernels load each lane's 8 bytes of low bits and 4 bytes of high bits
for the 32 columns of a 4-bit chunk and build the exact fp16 operands s * (q - 4).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import quantized_expert_dequant_amd as moe
from quantized_expert_dequant_amd.slab import upload_experts, workspace

from helpers import TOL, W_RTOL, build_layer, mfma_tiles, oracle_layer, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    moe.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("H,I,group", [(512, 128, 64), (704, 256, 64), (4096, 1024, 64), (512, 256, 128),
                                       (64, 128, 64)])
def test_pack_dequant_bit_exact(H, I, group):
    n = 3
    c = synth.experts(79, 5, 0, n, 3, H, I, group)
    slab = upload_experts(lambda f, k: synth.experts(79, 5, f, k, 3, H, I, group), n, 3, H, I, chunk=2, group=group)
    rb = moe.record_bytes(3, H, I, group)
    assert rb == 3 * I * H * 3 // 8 + 8 * I * (H // group) + 4 * H * (I // group)
    W = torch.empty(3 * I * H, dtype=torch.float32, device=DEV)
    for e in range(n):
        moe.dequant_expert(3, H, I, slab[e * rb:(e + 1) * rb], W, group=group)
        Wg, Wu, Wd = oracle.dequant_expert(3, H, I, c.gate[e], c.up[e], c.down[e], c.scales[e], c.biases[e],
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


def _check(cfg, seed, B, step=0):
    L = build_layer(cfg, seed)
    info = moe.grouped_launch_info(L.desc, B)
    assert info["grouped"] == (1 if B > 1 else 0)
    x = synth.tokens(seed, step, B, cfg["H"])
    y, idx, w = _decode(L, x)
    y_ref, idx_ref, w_ref, margin = oracle_layer(cfg, seed, 0, x, parallel=B > 1)
    assert margin.min() > 1e-9
    np.testing.assert_array_equal(idx, idx_ref)
    np.testing.assert_allclose(w, w_ref, rtol=W_RTOL)
    errs = [rel_err(y[b], y_ref[b]) for b in range(B)]
    print("3-bit H=%d I=%d K=%d B=%d: max rel err %.2e" % (cfg["H"], cfg["I"], cfg["K"], B, max(errs)))
    for b in range(B):
        assert errs[b] <= TOL, "token %d: %.3e" % (b, errs[b])
    return L, idx, info


@pytest.mark.parametrize("K,B", [(4, 1), (1, 1), (2, 1), (6, 1), (8, 1), (5, 1), (4, 2), (4, 3), (4, 16), (4, 37),
                                 (4, 256)])
def test_layer_decode_tiny(K, B):
    """The tiny layer in 3-bit: the straight-line kernels at every K they are built for
    (1, 2, 4, 6, 8), the general ones at K = 5, and grouped batches of 2 to 256 tokens
    (several 16-token tiles, a ragged tail, two 32-token groups per expert)."""
    cfg = dict(H=512, I=128, E=16, K=K, bits=3, B=B, layers=1, zipf=None)
    _check(cfg, 1800 + K + B, B)


@pytest.mark.parametrize("step", range(2))
def test_layer_decode_full_size(step):
    """The workload-1 shape (H = 4096, I = 1024, E = 512, K = 4) in 3-bit, one token."""
    cfg = dict(H=4096, I=1024, E=512, K=4, bits=3, B=1, layers=1, zipf=None)
    _check(cfg, 1850, 1, step)


@pytest.mark.parametrize("step", range(2))
def test_batched_full_size(step):
    """B = 64, K = 10 with the Zipf(1.1) prior at full size in 3-bit: every token."""
    cfg = dict(H=4096, I=1024, E=512, K=10, bits=3, B=64, layers=1, zipf=1.1)
    _check(cfg, 1880, 64, step)


def test_batched_largest_batch():
    """B = 256 at full size in 3-bit: the gate/up tiles outnumber the blocks, so they are cut
    into K chunks and finished from partial sums; every token against the oracle."""
    cfg = dict(H=4096, I=1024, E=512, K=10, bits=3, B=256, layers=1, zipf=1.1)
    L, idx, info = _check(cfg, 1890, 256, 0)
    assert info["gateup_k_chunks"] > 1
    assert mfma_tiles(idx, cfg["E"], info) > info["gateup_blocks"], "the K-chunk split is not taken"


def test_layer_decode_wide_rows_and_groups():
    """Rows of 128 units (H = 8192: the general kernels walk a row in two passes) with one
    scale and bias per 128 weights, one token and a batch of 4."""
    cfg = dict(H=8192, I=1024, E=16, K=4, bits=3, B=4, layers=1, zipf=None, group=128)
    _check(cfg, 1860, 4)
    cfg1 = dict(cfg, B=1)
    _check(cfg1, 1861, 1)


def test_expert_ffn_q3_given_routing():
    """moe_expert_ffn_q3 with caller-given routing (duplicate ids in a token, one expert shared
    by every token): each token against the oracle's expert FFNs."""
    H, I, E, K = 512, 128, 16, 4
    seed = 1870
    cfg = dict(H=H, I=I, E=E, K=K, bits=3, B=1, layers=1, zipf=None)
    L = build_layer(cfg, seed)
    ex = synth.experts(seed, 0, 0, E + 1, 3, H, I)
    B = 12
    x = synth.tokens(seed, 7, B, H)
    idx = np.stack([[2, 2, 5 + b % 7, b % 4] for b in range(B)]).astype(np.int32)
    w = np.random.default_rng(5).random((B, K)).astype(np.float32)
    ws, nb = workspace(L.desc, B)
    y = torch.empty((B, H), dtype=torch.float32, device=DEV)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    moe.expert_ffn_q3(L.desc, t(x), B, t(idx), t(w), y, ws, nb)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()

    def ffn(e, xb):
        return oracle.expert_ffn(3, H, I, ex.gate[e], ex.up[e], ex.down[e], ex.scales[e], ex.biases[e], xb)[1]

    for b in range(B):
        ref = ffn(E, x[b]) + sum(float(w[b, k]) * ffn(int(idx[b, k]), x[b]) for k in range(K))
        assert rel_err(yh[b], ref) <= TOL, "token %d: %.3e" % (b, rel_err(yh[b], ref))
    with pytest.raises(moe.MoeError) as e:
        moe.expert_ffn_q2(L.desc, t(x), B, t(idx), t(w), y, ws, nb)
    assert e.value.code == moe.MOE_EINVAL
