"""moe_layer_decode_noalloc: the layer decode with the library's per-GPU static
scratch instead of a caller workspace, for callers that cannot allocate.

Checked against moe_layer_decode on the same inputs (expert indices bit-exact,
routing weights within 1e-6 relative, each token's output within
max|dy| / max|y_ref| <= 2e-3), on two calls in a row with the second smaller than
the first, since every call on a GPU shares the one array; and the rejection of a
call whose workspace would not fit.
"""
import numpy as np
import pytest
import torch

import synth
import quantized_expert_dequant_amd as moe
from quantized_expert_dequant_amd.slab import workspace

from helpers import TOL, W_RTOL, WORKLOADS, build_layer, oracle_layer, rel_err, seed_of

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    moe.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _outputs(L, B):
    y = torch.full((B, L.H), float("nan"), dtype=torch.float32, device=DEV)
    idx = torch.full((B, L.K), -7, dtype=torch.int32, device=DEV)
    w = torch.full((B, L.K), float("nan"), dtype=torch.float32, device=DEV)
    return y, idx, w


def _with_workspace(L, x):
    B = x.shape[0]
    ws, n = workspace(L.desc, B)
    y, idx, w = _outputs(L, B)
    moe.layer_decode(L.desc, x, B, y, idx, w, ws, n)
    torch.cuda.synchronize()
    return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def _noalloc(L, x):
    B = x.shape[0]
    y, idx, w = _outputs(L, B)
    moe.layer_decode_noalloc(L.desc, x, B, y, idx, w)
    torch.cuda.synchronize()
    return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def _same(got, ref):
    y, idx, w = got
    y_ref, idx_ref, w_ref = ref
    np.testing.assert_array_equal(idx, idx_ref)
    np.testing.assert_allclose(w, w_ref, rtol=W_RTOL)
    for b in range(y.shape[0]):
        assert rel_err(y[b], y_ref[b]) <= TOL, "token %d" % b


@pytest.mark.parametrize("first,second", [((2, 4), (2, 1)), ((1, 1), (0, 1)), ((1, 8), (1, 2))])
def test_noalloc_matches_layer_decode_twice(first, second):
    """Two calls in a row, the second smaller than the first: workload 2 (2-bit) with 4
    tokens then 1, workload 1 (the full 4-bit layer) then workload 0 (the tiny layer), and
    workload 1 with 8 tokens then 2 (batches whose grouped workspace exceeds the scratch,
    so they run token by token here and grouped with a workspace).  The second call must
    not see the first's leftovers in the shared scratch."""
    layers = {}
    calls = []
    for t, (n, B) in enumerate((first, second)):
        if n not in layers:
            layers[n] = build_layer(dict(WORKLOADS[n]), seed_of(n))
        L = layers[n]
        x = torch.from_numpy(synth.tokens(seed_of(n), 500 + t, B, L.H)).to(DEV)
        calls.append((n, L, x, _noalloc(L, x)))
    for n, L, x, got in calls:
        _same(got, _with_workspace(L, x))
        y_ref, idx_ref, _, _ = oracle_layer(dict(WORKLOADS[n]), seed_of(n), 0, x.cpu().numpy())
        np.testing.assert_array_equal(got[1], idx_ref)
        for b in range(x.shape[0]):
            assert rel_err(got[0][b], y_ref[b]) <= TOL, "workload %d token %d" % (n, b)
    del layers, calls
    torch.cuda.empty_cache()


def test_noalloc_rejects_a_workspace_that_does_not_fit():
    """A batch of 256 tokens with K = 10 exceeds the static scratch on both paths (the
    token-by-token one holds h of 11 experts per token): the call returns
    MOE_EUNSUPPORTED, launches nothing and leaves the outputs alone."""
    cfg, seed = dict(WORKLOADS[0]), seed_of(0)
    cfg["H"], cfg["I"], cfg["E"], cfg["K"] = 4096, 1024, 512, 10
    L = build_layer(dict(cfg, bits=4), seed)
    B = 256
    assert moe.workspace_bytes(L.desc, B) > moe.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.from_numpy(synth.tokens(seed, 502, B, L.H)).to(DEV)
    y, idx, w = _outputs(L, B)
    with pytest.raises(moe.MoeError) as e:
        moe.layer_decode_noalloc(L.desc, x, B, y, idx, w)
    assert e.value.code == moe.MOE_EUNSUPPORTED
    torch.cuda.synchronize()
    assert torch.isnan(y).all() and (idx == -7).all()
    del L
    torch.cuda.empty_cache()
