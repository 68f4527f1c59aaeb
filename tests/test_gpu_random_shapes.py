"""GPU parity over a seeded sample of layer shapes.

Thirty layers drawn once from a fixed seed: H and I multiples of the group (I a multiple
of 128 at 3 bits), up to 3072 x 1536 (rows of up to 48 units, odd unit counts among
them), E from 2 to 200, K from 1 to min(E, 12), 4-, 3- and 2-bit codes, groups of 64,
128 and 256, and batches of 1 to 40 tokens (the straight-line, general, GEMV and
matrix-core kernels).  Every token against the oracle: expert indices bit-exact,
routing weights within 1e-6 relative, outputs within 2e-3 of each token's largest
magnitude.
"""
import numpy as np
import pytest
import torch

import synth
import quantized_expert_dequant_amd as moe
from quantized_expert_dequant_amd.slab import workspace

from helpers import TOL, W_RTOL, build_layer, oracle_layer, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _cases(n=30, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        bits = int(rng.choice([4, 3, 2]))
        group = int(rng.choice([64, 128, 256]))
        H = group * int(rng.integers(1, 3072 // group + 1))
        i_unit = max(group, 128) if bits == 3 else group
        I = i_unit * int(rng.integers(1, 1536 // i_unit + 1))
        E = int(rng.integers(2, 201))
        K = int(rng.integers(1, min(E, 12) + 1))
        B = int(rng.choice([1, 1, 2, 3, 7, 16, 40]))
        out.append(dict(H=H, I=I, E=E, K=K, bits=bits, group=group, B=B, layers=1, zipf=None))
    return out


CASES = _cases()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    moe.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n", range(len(CASES)))
def test_random_layer_shape(n):
    cfg = CASES[n]
    seed = 3000 + n
    B = cfg["B"]
    print("case %d: %s" % (n, cfg), flush=True)
    L = build_layer(cfg, seed)
    x = synth.tokens(seed, 1, B, cfg["H"])
    ws, nb = workspace(L.desc, B)
    y = torch.empty((B, L.H), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, L.K), dtype=torch.int32, device=DEV)
    w = torch.empty((B, L.K), dtype=torch.float32, device=DEV)
    moe.layer_decode(L.desc, torch.from_numpy(x).to(DEV), B, y, idx, w, ws, nb)
    torch.cuda.synchronize()
    y, idx, w = y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    y_ref, idx_ref, w_ref, margin = oracle_layer(cfg, seed, 0, x, parallel=B > 1)
    assert margin.min() > 1e-9
    np.testing.assert_array_equal(idx, idx_ref)
    np.testing.assert_allclose(w, w_ref, rtol=W_RTOL)
    for b in range(B):
        assert rel_err(y[b], y_ref[b]) <= TOL, "token %d: %.3e" % (b, rel_err(y[b], y_ref[b]))
    del L
