"""GPU parity of batched decode with 2-bit experts on the grouped path.

A 2-bit batch groups its tokens by expert like a 4-bit one and runs the same
matrix-core dequant-GEMMs: each lane loads the 8 bytes of a 2-bit chunk that hold
the 32 columns of a 4-bit chunk and turns them into the same exact fp16 operands
s * (q - 8).  Every token is compared with the oracle: expert indices bit-exact,
routing weights within 1e-6 relative, each token's output within 2e-3 of its
largest magnitude.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import quantized_expert_dequant_amd as moe
from quantized_expert_dequant_amd.slab import DeviceLayer, upload_experts, workspace

from helpers import TOL, W_RTOL, WORKLOADS, build_layer, mfma_tiles, oracle_layer, rel_err, seed_of

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    moe.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _decode(layer, x):
    B = x.shape[0]
    ws, n = workspace(layer.desc, B)
    y = torch.empty((B, layer.H), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, layer.K), dtype=torch.int32, device=DEV)
    w = torch.empty((B, layer.K), dtype=torch.float32, device=DEV)
    moe.layer_decode(layer.desc, _t(x), B, y, idx, w, ws, n)
    torch.cuda.synchronize()
    return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def _check_every_token(cfg, seed, L, x, parallel=False):
    y, idx, w = _decode(L, x)
    y_ref, idx_ref, w_ref, margin = oracle_layer(cfg, seed, 0, x, parallel=parallel)
    assert margin.min() > 1e-9
    np.testing.assert_array_equal(idx, idx_ref)
    np.testing.assert_allclose(w, w_ref, rtol=W_RTOL)
    errs = np.array([rel_err(y[b], y_ref[b]) for b in range(x.shape[0])])
    print("2-bit batch B=%d: max rel err %.2e (token %d), median %.2e"
          % (x.shape[0], errs.max(), int(errs.argmax()), np.median(errs)))
    assert errs.max() <= TOL, "token %d" % int(errs.argmax())
    return idx


@pytest.mark.parametrize("B", [2, 16, 37, 256])
def test_q2_batched_tiny_layer(B):
    """The tiny layer in 2-bit: several 16-token tiles, a ragged tail, and at B = 256 two
    32-token MFMA groups per expert."""
    cfg, seed = dict(WORKLOADS[0], bits=2), seed_of(20)
    L = build_layer(cfg, seed)
    assert L.desc.expert_flags is None
    assert moe.grouped_launch_info(L.desc, B)["grouped"] == 1
    _check_every_token(cfg, seed, L, synth.tokens(seed, 300 + B, B, L.H))


@pytest.mark.parametrize("step", range(2))
def test_q2_batched_full_size(step):
    """B = 64, K = 10 with the Zipf(1.1) prior at full size in 2-bit: every token."""
    cfg, seed = dict(WORKLOADS[4], bits=2), seed_of(24)
    L = build_layer(cfg, seed)
    assert moe.grouped_launch_info(L.desc, cfg["B"])["grouped"] == 1
    _check_every_token(cfg, seed, L, synth.tokens(seed, step, cfg["B"], L.H), parallel=True)


def test_q2_batched_largest_batch():
    """B = 256 at full size in 2-bit: the gate/up tiles outnumber the blocks, so they are cut
    into K chunks and finished from partial sums; every token against the oracle."""
    cfg, seed = dict(WORKLOADS[4], bits=2), seed_of(25)
    L = build_layer(cfg, seed)
    B = moe.MOE_MAX_B
    info = moe.grouped_launch_info(L.desc, B)
    assert info["grouped"] == 1 and info["gateup_k_chunks"] > 1
    x = synth.tokens(seed, 41, B, L.H)
    idx = _check_every_token(cfg, seed, L, x, parallel=True)
    assert mfma_tiles(idx, cfg["E"], info) > info["gateup_blocks"], "the K-chunk split is not taken"


def test_q2_expert_ffn_given_routing():
    """moe_expert_ffn_q2 with caller-given routing (duplicate ids in a token, one expert
    shared by every token): each token against the oracle's expert FFNs."""
    cfg = dict(WORKLOADS[0], bits=2)
    H, I, E, K = cfg["H"], cfg["I"], cfg["E"], cfg["K"]
    seed = seed_of(21)
    L = build_layer(cfg, seed)
    ex = synth.experts(seed, 0, 0, E + 1, 2, H, I)
    B = 24
    x = synth.tokens(seed, 77, B, H)
    idx = np.stack([[2, 2, 5 + b % 7, b % 4] for b in range(B)]).astype(np.int32)
    w = np.random.default_rng(3).random((B, K)).astype(np.float32)
    ws, nb = workspace(L.desc, B)
    y = torch.empty((B, H), dtype=torch.float32, device=DEV)
    moe.expert_ffn_q2(L.desc, _t(x), B, _t(idx), _t(w), y, ws, nb)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()

    def ffn(e, xb):
        return oracle.expert_ffn(2, H, I, ex.gate[e], ex.up[e], ex.down[e], ex.scales[e], ex.biases[e], xb)[1]

    for b in range(B):
        ref = ffn(E, x[b]) + sum(float(w[b, k]) * ffn(int(idx[b, k]), x[b]) for k in range(K))
        assert rel_err(yh[b], ref) <= TOL, "token %d: %.3e" % (b, rel_err(yh[b], ref))


def _bf16_scaled(bits16, k):
    b = bits16.astype(np.int32)
    e = (b >> 7) & 0xFF
    ok = (e > 0) & (e + k < 255)
    return np.where(ok, (b & ~(0xFF << 7)) | ((e + k) << 7), b).astype(np.uint16)


def test_q2_batch_with_flagged_expert_runs_token_by_token():
    """Expert 4's scales x 2^14 put it beyond the matrix cores' range: the layer keeps the
    flags, the 2-bit batch takes the token-by-token kernels (launch info says so), and
    every token matches the oracle."""
    cfg, seed = dict(WORKLOADS[0], bits=2), seed_of(22)
    H, I, E, K = cfg["H"], cfg["I"], cfg["E"], cfg["K"]
    ex = synth.experts(seed, 0, 0, E + 1, 2, H, I)
    ex.scales[4] = _bf16_scaled(ex.scales[4], 14)

    def src(first, n):
        return synth.Canonical(2, H, I, 64, ex.gate[first:first + n], ex.up[first:first + n],
                               ex.down[first:first + n], ex.scales[first:first + n], ex.biases[first:first + n])

    slab = upload_experts(src, E + 1, 2, H, I, device=DEV)
    wr = torch.from_numpy(synth.router(seed, 0, E, H)).to(DEV)
    L = DeviceLayer(H, I, E, K, 2, slab, wr)
    assert L.desc.expert_flags is not None and int(L.expert_flags[4]) == 1
    B = 16
    assert moe.grouped_launch_info(L.desc, B)["grouped"] == 0
    x = synth.tokens(seed, 9, B, H)
    idx = np.stack([[4, 1 + b % 9, 10 + b % 5, b % 2 + 14] for b in range(B)]).astype(np.int32)
    w = np.random.default_rng(4).random((B, K)).astype(np.float32)
    ws, nb = workspace(L.desc, B)
    y = torch.empty((B, H), dtype=torch.float32, device=DEV)
    moe.expert_ffn_q2(L.desc, _t(x), B, _t(idx), _t(w), y, ws, nb)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()

    def ffn(e, xb):
        return oracle.expert_ffn(2, H, I, ex.gate[e], ex.up[e], ex.down[e], ex.scales[e], ex.biases[e], xb)[1]

    for b in range(B):
        ref = ffn(E, x[b]) + sum(float(w[b, k]) * ffn(int(idx[b, k]), x[b]) for k in range(K))
        assert np.all(np.isfinite(yh[b])), "token %d" % b
        assert rel_err(yh[b], ref) <= TOL, "token %d: %.3e" % (b, rel_err(yh[b], ref))
