"""GPU: HIP graph replay of the decode entry points.

Throughput is measured on a graph replay, so a replayed graph must give what the
same call gives when launched eagerly.  Each case captures one call with static
input and output buffers, then replays it several times.  Before each replay a
fresh token is copied into the static input, the outputs are poisoned, and the
same entry point runs eagerly on its own workspace and outputs (the program's
own work between replays).  Every replay must equal that eager call bit for bit
(the same kernels with fixed summation orders) and, for a single routed layer,
the oracle within the bar; the given-routing entry point's parity with the
oracle is tested in test_gpu_parity.py.  The cases cover the fused single-token
path, the grouped path with and without matrix-core groups, the stack on both,
and the given-routing entry point on the grouped path.
"""
import numpy as np
import pytest
import torch

import synth
import quantized_expert_dequant_amd as moe
from quantized_expert_dequant_amd.slab import workspace

from helpers import RMS_EPS, TOL, W_RTOL, WORKLOADS, build_layer, oracle_layer, rel_err, seed_of

pytestmark = pytest.mark.gpu

DEV = "cuda"
REPLAYS = 4
STACK_LAYERS = 3


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    moe.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def layers():
    cache = {}

    def get(n, l):
        if (n, l) not in cache:
            cache[(n, l)] = build_layer(WORKLOADS[n], seed_of(n), layer=l)
        return cache[(n, l)]

    yield get
    cache.clear()


def _capture(fn):
    """Capture fn() on a side stream after one eager warm-up call there."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.synchronize()
    return g


class _Bufs:
    def __init__(self, B, H, nl, K, desc, stack):
        self.x = torch.empty((B, H), dtype=torch.float32, device=DEV)
        self.y = torch.empty((B, H), dtype=torch.float32, device=DEV)
        self.idx = torch.empty((nl, B, K), dtype=torch.int32, device=DEV)
        self.w = torch.empty((nl, B, K), dtype=torch.float32, device=DEV)
        self.ws, self.n = workspace(desc, B, stack=stack)

    def poison(self):
        self.y.fill_(float("nan"))
        self.idx.fill_(-1)
        self.w.fill_(float("nan"))


# (entry point, workload, tokens): workload 1 is the full single-token layer (fused
# selection); workload 0 at B = 16 has experts with >= 2 tokens (matrix-core groups),
# at B = 2 mostly GEMV groups (experts with one token) and the shared expert's group on
# the matrix cores; the stack renormalizes inside the next router at B = 1
# and with the separate renorm kernel on the grouped path; the given-routing entry point
# at B = 16 writes its own token operands (k_prep_tokens) before the grouped FFNs.
CASES = [("layer", 1, 1), ("layer", 0, 16), ("layer", 0, 2), ("stack", 0, 1), ("stack", 0, 3), ("ffn", 0, 16)]


@pytest.mark.parametrize("kind,n,B", CASES)
def test_graph_replay_matches_eager(layers, kind, n, B):
    cfg = WORKLOADS[n]
    seed = seed_of(n)
    H, K = cfg["H"], cfg["K"]
    stack = kind == "stack"
    nl = STACK_LAYERS if stack else 1
    Ls = [layers(n, l) for l in range(nl)]
    descs = [L.desc for L in Ls]

    # fixed routing for the given-routing entry point: K distinct experts per token
    rng = np.random.default_rng(seed)
    idx_in = _t(np.stack([rng.choice(cfg["E"], K, replace=False) for _ in range(B)]).astype(np.int32))
    w_in = _t(rng.dirichlet(np.ones(K), size=B).astype(np.float32))

    def call(b):
        if stack:
            moe.stack_decode(descs, b.x, B, RMS_EPS, b.y, b.idx, b.w, b.ws, b.n)
        elif kind == "ffn":
            moe.expert_ffn(descs[0], b.x, B, idx_in, w_in, b.y, b.ws, b.n)
        else:
            moe.layer_decode(descs[0], b.x, B, b.y, b.idx[0], b.w[0], b.ws, b.n)

    gb = _Bufs(B, H, nl, K, descs[0], stack)  # the graph's static buffers
    eb = _Bufs(B, H, nl, K, descs[0], stack)  # the eager calls' own
    gb.x.copy_(_t(synth.tokens(seed, 100, B, H)))
    g = _capture(lambda: call(gb))
    try:
        for r in range(REPLAYS):
            xh = synth.tokens(seed, 200 + r, B, H)
            gb.x.copy_(_t(xh))
            eb.x.copy_(gb.x)
            call(eb)
            gb.poison()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            case = "replay %d" % r
            if kind != "ffn":  # routing outputs (the given-routing call has none)
                torch.testing.assert_close(gb.idx, eb.idx, rtol=0, atol=0, msg=case)
                torch.testing.assert_close(gb.w, eb.w, rtol=0, atol=0, msg=case)
            torch.testing.assert_close(gb.y, eb.y, rtol=0, atol=0, equal_nan=False, msg=case)
            if kind == "layer":
                y_ref, idx_ref, w_ref, margin = oracle_layer(cfg, seed, 0, xh)
                assert np.all(margin > 1e-9), case + ": routing margin below 1e-9"
                np.testing.assert_array_equal(gb.idx[0].cpu().numpy(), idx_ref, err_msg=case)
                np.testing.assert_allclose(gb.w[0].cpu().numpy(), w_ref, rtol=W_RTOL, err_msg=case)
                y = gb.y.cpu().numpy()
                for b in range(B):
                    assert rel_err(y[b], y_ref[b]) <= TOL, "%s token %d" % (case, b)
    finally:
        del g
        torch.cuda.synchronize()
