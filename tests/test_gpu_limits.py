"""GPU parity at the limits of the boundary: the largest batch, the most experts and
the largest K the library takes, and K = E (every expert active).

Bars as everywhere: expert indices bit-exact, routing weights within 1e-6
relative, each token's output within max|dy| / max|y_ref| <= 2e-3.
"""
import numpy as np
import pytest
import torch

import synth
import quantized_expert_dequant_amd as moe
from quantized_expert_dequant_amd.slab import workspace

from helpers import TOL, W_RTOL, WORKLOADS, build_layer, mfma_tiles, oracle_layer, oracle_route, rel_err, seed_of

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    moe.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _decode(layer, x):
    B = x.shape[0]
    ws, n = workspace(layer.desc, B)
    y = torch.empty((B, layer.H), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, layer.K), dtype=torch.int32, device=DEV)
    w = torch.empty((B, layer.K), dtype=torch.float32, device=DEV)
    moe.layer_decode(layer.desc, torch.from_numpy(np.ascontiguousarray(x)).to(DEV), B, y, idx, w, ws, n)
    torch.cuda.synchronize()
    return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def test_batched_largest_batch():
    """B = 256 (the most tokens per call) on the full-size batched layer: routing and output
    of every token against the oracle.  Experts shared by dozens of tokens are cut into
    several 32-token groups, and the gate/up tiles outnumber the blocks of the matrix-core
    launch, so tiles are cut into K chunks and the tiles two blocks share are finished by
    adding their partial sums in K order: every output of those tiles is compared here."""
    cfg, seed = dict(WORKLOADS[4]), seed_of(4)
    assert moe.MOE_MAX_B == 256
    L = build_layer(cfg, seed)
    B = moe.MOE_MAX_B
    info = moe.grouped_launch_info(L.desc, B)
    assert info["grouped"] == 1 and info["gateup_k_chunks"] > 1
    x = synth.tokens(seed, 40, B, L.H)
    y, idx, w = _decode(L, x)
    tiles = mfma_tiles(idx, cfg["E"], info)
    assert tiles > info["gateup_blocks"], "the K-chunk split is not taken (%d tiles, %d blocks)" % (
        tiles, info["gateup_blocks"])
    counts = np.bincount(idx.ravel(), minlength=cfg["E"])
    assert counts.max() > 64  # the hottest expert spans more than two MFMA groups
    y_ref, idx_ref, w_ref, margin = oracle_layer(cfg, seed, 0, x, parallel=True)
    assert margin.min() > 1e-9
    np.testing.assert_array_equal(idx, idx_ref)
    np.testing.assert_allclose(w, w_ref, rtol=W_RTOL)
    errs = np.array([rel_err(y[b], y_ref[b]) for b in range(B)])
    print("B=256: %d tiles on %d blocks, max rel err %.2e (token %d)" % (tiles, info["gateup_blocks"], errs.max(),
                                                                       int(errs.argmax())))
    assert errs.max() <= TOL, "token %d" % int(errs.argmax())
    del L
    torch.cuda.empty_cache()


@pytest.mark.parametrize("E,K,B", [(moe.MOE_MAX_E, moe.MOE_MAX_K, 1), (moe.MOE_MAX_E, moe.MOE_MAX_K, 5),
                                   (16, 16, 1), (16, 16, 3)])
def test_most_experts_and_largest_k(E, K, B):
    """E = 1024 with K = 32 (the library's maxima), and K = E = 16 (every expert active),
    through the per-token path (B = 1) and the grouped path (B > 1); every output checked."""
    cfg = dict(H=512, I=128, E=E, K=K, bits=4, B=B, layers=1, zipf=None)
    seed = 1100 + E + K
    L = build_layer(cfg, seed)
    x = synth.tokens(seed, B, B, L.H)
    y, idx, w = _decode(L, x)
    y_ref, idx_ref, w_ref, margin = oracle_layer(cfg, seed, 0, x)
    assert np.all(margin > 1e-9)  # infinite when K = E
    if K == E:  # every expert is selected; the rank order still has to match
        assert np.all(np.sort(idx, axis=1) == np.arange(E))
    np.testing.assert_array_equal(idx, idx_ref)
    np.testing.assert_allclose(w, w_ref, rtol=W_RTOL)
    for b in range(B):
        assert rel_err(y[b], y_ref[b]) <= TOL, "token %d" % b
    del L
    torch.cuda.empty_cache()
