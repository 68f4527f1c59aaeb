"""GPU parity at the largest shapes the library accepts and past the straight-line kernels.

Rows of more than 64 groups (H or I above 4096) take the general single-token kernels,
which walk a row's groups in passes of 64 lanes, and a batch then has no dot2 GEMV groups:
every expert runs on the matrix cores.  The shapes: H = 8192 (two group passes per gate/up
row, 4- and 2-bit), I = 8192 (the largest intermediate size: two passes per down row, one
expert's h per LDS round), H = 65536 (the largest hidden size: 1024 groups per gate/up row,
a one-group down row, 256 router slices in a batch).  Every token against the oracle:
expert indices bit-exact, routing weights within 1e-6 relative, outputs within 2e-3 of
each token's largest magnitude.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import quantized_expert_dequant_amd as moe
from quantized_expert_dequant_amd.slab import DeviceLayer, upload_experts, workspace

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


def _decode(layer, x):
    B = x.shape[0]
    ws, n = workspace(layer.desc, B)
    y = torch.empty((B, layer.H), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, layer.K), dtype=torch.int32, device=DEV)
    w = torch.empty((B, layer.K), dtype=torch.float32, device=DEV)
    moe.layer_decode(layer.desc, torch.from_numpy(x).to(DEV), B, y, idx, w, ws, n)
    torch.cuda.synchronize()
    return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("H,I,E,K,bits,B", [
    (8192, 1024, 16, 4, 4, 1),
    (8192, 1024, 16, 4, 4, 4),
    (8192, 1024, 16, 4, 2, 1),
    (8192, 1024, 16, 4, 2, 4),
    (4096, 8192, 8, 2, 4, 1),
    (4096, 8192, 8, 2, 4, 3),
    (65536, 64, 8, 2, 4, 1),
    (65536, 64, 8, 2, 4, 2),
])
def test_large_shapes_match_oracle(H, I, E, K, bits, B):
    cfg = dict(H=H, I=I, E=E, K=K, bits=bits, B=B, layers=1, zipf=None)
    seed = 1300 + H // 64 + I // 64 + bits + B
    L = build_layer(cfg, seed)
    info = moe.grouped_launch_info(L.desc, B)
    assert info["grouped"] == (1 if B > 1 else 0)
    assert info["gemv_below_tokens"] == 1  # rows beyond 64 groups: no GEMV groups in a batch
    x = synth.tokens(seed, 5, B, H)
    y, idx, w = _decode(L, x)
    y_ref, idx_ref, w_ref, margin = oracle_layer(cfg, seed, 0, x, parallel=B > 1)
    assert margin.min() > 1e-9
    np.testing.assert_array_equal(idx, idx_ref)
    np.testing.assert_allclose(w, w_ref, rtol=W_RTOL)
    for b in range(B):
        assert np.all(np.isfinite(y[b])), "token %d" % b
        assert rel_err(y[b], y_ref[b]) <= TOL, "token %d: %.3e" % (b, rel_err(y[b], y_ref[b]))
    del L
    torch.cuda.empty_cache()


def _bf16_scaled(bits16, k):
    """bf16 bit patterns times 2^k (exponent raised; zeros and values that would overflow kept)."""
    b = bits16.astype(np.int32)
    e = (b >> 7) & 0xFF
    ok = (e > 0) & (e + k < 255)
    return np.where(ok, (b & ~(0xFF << 7)) | ((e + k) << 7), b).astype(np.uint16)


def test_flagged_expert_beyond_64_groups_runs_token_by_token():
    """A 4-bit batch at H = 8192 whose expert 3 has scales x 2^14 (beyond the matrix cores'
    fp16 operands): with no GEMV groups to move it to, the flagged batch takes the
    token-by-token kernels (launch info says so) and every token, routed through expert 3
    or not, is finite and matches the oracle's FFNs of the same records."""
    H, I, E, K, bits, B = 8192, 1024, 16, 4, 4, 6
    cfg = dict(H=H, I=I, E=E, K=K, bits=bits, B=B, layers=1, zipf=None)
    seed = 1399
    ex = synth.experts(seed, 0, 0, E + 1, bits, H, I)
    ex.scales[3] = _bf16_scaled(ex.scales[3], 14)

    def src(first, n):
        return synth.Canonical(bits, H, I, 64, ex.gate[first:first + n], ex.up[first:first + n],
                               ex.down[first:first + n], ex.scales[first:first + n], ex.biases[first:first + n])

    wr = torch.from_numpy(synth.router(seed, 0, E, H)).to(DEV)
    L = DeviceLayer(H, I, E, K, bits, upload_experts(src, E + 1, bits, H, I, device=DEV), wr)
    assert L.desc.expert_flags is not None and int(L.expert_flags[3]) == 1
    assert moe.grouped_launch_info(L.desc, B)["grouped"] == 0
    # tokens whose top-K holds expert 3: its router row added to a token raises its logit
    x = synth.tokens(seed, 11, B, H)
    Wr = synth.router(seed, 0, E, H)
    x[: B // 2] += 4.0 * Wr[3] / np.linalg.norm(Wr[3])
    x = np.ascontiguousarray(x, np.float32)
    y, idx, w = _decode(L, x)
    _, _, _, sel = oracle_route(cfg, seed, 0, x)
    assert min(s[2] for s in sel) > 1e-9
    idx_ref = np.array([s[0] for s in sel], np.int32)
    w_ref = np.array([s[1] for s in sel], np.float64)
    np.testing.assert_array_equal(idx, idx_ref)
    np.testing.assert_allclose(w, w_ref, rtol=W_RTOL)
    assert (idx == 3).any(axis=1).sum() >= 1, "no token routed through the flagged expert"

    def ffn(e, xb):
        return oracle.expert_ffn(bits, H, I, ex.gate[e], ex.up[e], ex.down[e], ex.scales[e], ex.biases[e], xb)[1]

    for b in range(B):
        ref = ffn(E, x[b]) + sum(float(w_ref[b, k]) * ffn(int(idx_ref[b, k]), x[b]) for k in range(K))
        assert np.all(np.isfinite(y[b])), "token %d" % b
        assert rel_err(y[b], ref) <= TOL, "token %d: %.3e" % (b, rel_err(y[b], ref))
