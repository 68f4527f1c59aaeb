"""GPU parity of the attention half of a decode step (moe_gdn_step, moe_attn_decode).

Both sides take the same seeded inputs: the gated-delta-rule state, q, k, v and the
per-head gates in fp32, the KV cache as bf16 bit patterns.  The oracle computes in
float64; the kernels accumulate dot products of length dk (or d, or T) in fp32, so
each result is held to 2e-5 (state, GatedDeltaNet output) or 1e-4 (attention, with
its fp32 exponentials) of the largest magnitude of its head's exact result.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_expert_dequant_amd as moe

pytestmark = pytest.mark.gpu

DEV = "cuda"
GDN_TOL = 2e-5
ATTN_TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    moe.lib()
    yield
    torch.cuda.synchronize()


def _head_err(got, ref):
    """max over heads of max |got - ref| / max |ref| within the head."""
    got = np.asarray(got, np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, np.float64).reshape(ref.shape[0], -1)
    scale = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((np.abs(got - ref).max(axis=1) / scale).max())


def _gdn_inputs(seed, n, dk, dv):
    rng = np.random.default_rng(seed)
    S = rng.normal(0, 0.5, (n, dv, dk)).astype(np.float32)
    # unit-norm keys, as the rule assumes (S (I - beta k k^T) then only removes what k reads)
    k = rng.normal(0, 1, (n, dk))
    k = (k / np.linalg.norm(k, axis=1, keepdims=True)).astype(np.float32)
    q = (rng.normal(0, 1, (n, dk)) / np.sqrt(dk)).astype(np.float32)
    v = rng.normal(0, 1, (n, dv)).astype(np.float32)
    alpha = rng.uniform(0.8, 1.0, n).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, n).astype(np.float32)
    return S, q, k, v, alpha, beta


def _gdn_gpu(S, q, k, v, alpha, beta):
    n, dv, dk = S.shape
    t = [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (S, q, k, v, alpha, beta)]
    o = torch.empty((n, dv), dtype=torch.float32, device=DEV)
    moe.gdn_step(n, dk, dv, *t, o)
    torch.cuda.synchronize()
    return t[0].cpu().numpy(), o.cpu().numpy()


@pytest.mark.parametrize("n,dk,dv", [(64, 128, 128), (3, 64, 37), (2, 256, 130), (5, 128, 1), (2, 256, 4096)])
def test_gdn_step_matches_oracle(n, dk, dv):
    S, q, k, v, a, b = _gdn_inputs(100 + dk + dv, n, dk, dv)
    S_ref, o_ref = oracle.gdn_step(S, q, k, v, a, b)
    S_got, o_got = _gdn_gpu(S, q, k, v, a, b)
    assert _head_err(S_got, S_ref) <= GDN_TOL
    assert _head_err(o_got, o_ref) <= GDN_TOL


def test_gdn_eight_steps_in_a_row():
    """The state carries from step to step: eight steps with fresh q, k, v each."""
    n, dk, dv = 16, 128, 128
    S, *_ = _gdn_inputs(7, n, dk, dv)
    S_ref = S.astype(np.float64)
    S_dev = torch.from_numpy(S).to(DEV)
    o_dev = torch.empty((n, dv), dtype=torch.float32, device=DEV)
    for step in range(8):
        _, q, k, v, a, b = _gdn_inputs(1000 + step, n, dk, dv)
        S_ref, o_ref = oracle.gdn_step(S_ref, q, k, v, a, b)
        ins = [torch.from_numpy(x).to(DEV) for x in (q, k, v, a, b)]
        moe.gdn_step(n, dk, dv, S_dev, *ins, o_dev)
        torch.cuda.synchronize()
        assert _head_err(o_dev.cpu().numpy(), o_ref) <= 4 * GDN_TOL, step
    assert _head_err(S_dev.cpu().numpy(), S_ref) <= 4 * GDN_TOL


def _bf16_bits(x):
    """bf16 bit patterns of the float32 values of x, cut toward zero (any bf16 will do as input)."""
    return (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _attn_inputs(seed, n_q, n_kv, d, T):
    rng = np.random.default_rng(seed)
    q = rng.normal(0, 1, (n_q, d)).astype(np.float32)
    K = _bf16_bits(rng.normal(0, 1, (n_kv, T, d)))
    V = _bf16_bits(rng.normal(0, 1, (n_kv, T, d)))
    return q, K, V


def _attn_gpu(q, K, V):
    n_q, d = q.shape
    n_kv, T, _ = K.shape
    qd = torch.from_numpy(q).to(DEV)
    Kd = torch.from_numpy(K.view(np.int16)).to(DEV)
    Vd = torch.from_numpy(V.view(np.int16)).to(DEV)
    o = torch.empty((n_q, d), dtype=torch.float32, device=DEV)
    wsb = moe.attn_workspace_bytes(n_q, n_kv, d, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    moe.attn_decode(n_q, n_kv, d, T, qd, Kd, Vd, o, ws, wsb)
    torch.cuda.synchronize()
    return o.cpu().numpy()


@pytest.mark.parametrize("n_q,n_kv,d,T", [
    (32, 2, 256, 4096),   # 16 query heads per KV head, a 4096-position cache
    (32, 2, 256, 32768),  # four sub-tiles per wave (the running reference carries over)
    (8, 2, 128, 16384),   # two sub-tiles per wave
    (16, 8, 128, 4096),   # 8 KV heads, 2 query heads each
    (12, 3, 128, 1000),   # ragged last slice
    (8, 8, 64, 1),        # one position: o = V[0]
    (16, 1, 128, 65),     # one position past a slice
    (4, 2, 64, 64),       # exactly one slice
])
def test_attention_decode_matches_oracle(n_q, n_kv, d, T):
    q, K, V = _attn_inputs(200 + T, n_q, n_kv, d, T)
    o_ref = oracle.attn_decode(q, K, V)
    assert _head_err(_attn_gpu(q, K, V), o_ref) <= ATTN_TOL


def test_attention_longest_cache():
    """T = 2^22, the longest cache the entry point accepts (two query heads on one KV head,
    d = 64): 256 sub-tiles per wave, the running reference carried through all of them, and
    256 partials per head in the combine."""
    n_q, n_kv, d, T = 2, 1, 64, 1 << 22
    rng = np.random.default_rng(4242)
    q = rng.standard_normal((n_q, d), dtype=np.float32)
    K = _bf16_bits(rng.standard_normal((n_kv, T, d), dtype=np.float32))
    V = _bf16_bits(rng.standard_normal((n_kv, T, d), dtype=np.float32))
    o_ref = oracle.attn_decode(q, K, V)
    assert _head_err(_attn_gpu(q, K, V), o_ref) <= ATTN_TOL


def test_attention_peaked_scores():
    """Large scores (one key aligned with q, scaled up) exercise the running maximum:
    the weights must not overflow and the aligned position dominates."""
    n_q, n_kv, d, T = 4, 1, 128, 700
    q, K, V = _attn_inputs(9, n_q, n_kv, d, T)
    q *= 8.0
    K[0, 611] = _bf16_bits(q[0] / np.linalg.norm(q[0]) * 6.0)
    o_ref = oracle.attn_decode(q, K, V)
    assert _head_err(_attn_gpu(q, K, V), o_ref) <= ATTN_TOL


def test_shape_errors():
    x = torch.zeros(64 * 4, dtype=torch.float32, device=DEV)
    with pytest.raises(moe.MoeError) as e:
        moe.attn_decode(8, 3, 128, 16, x, x, x, x, x, 4096)
    assert e.value.code == moe.MOE_EINVAL
    with pytest.raises(moe.MoeError) as e:
        moe.attn_decode(8, 2, 96, 16, x, x, x, x, x, 4096)
    assert e.value.code == moe.MOE_EUNSUPPORTED
    with pytest.raises(moe.MoeError) as e:
        moe.attn_decode(34, 2, 128, 16, x, x, x, x, x, 1 << 20)
    assert e.value.code == moe.MOE_EUNSUPPORTED
    with pytest.raises(moe.MoeError) as e:
        moe.attn_decode(8, 2, 128, 4096, x, x, x, x, x, 1024)
    assert e.value.code == moe.MOE_EINVAL
    with pytest.raises(moe.MoeError) as e:
        moe.gdn_step(4, 96, 64, x, x, x, x, x, x, x)
    assert e.value.code == moe.MOE_EUNSUPPORTED


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


def test_graph_replays_match_eager_calls():
    """The bench times both entry points as graph replays.  One captured call of each is
    replayed four times, with fresh inputs copied into its static buffers, its outputs
    poisoned and an eager call of the same entry point on other buffers in between:
    every replay equals that eager call bit for bit (fixed summation orders), and the
    attention output the oracle within its bar."""
    n, dk, dv = 8, 128, 64
    n_q, n_kv, d, T = 8, 2, 128, 300
    S0 = torch.empty((n, dv, dk), device=DEV)
    gq, gk, gv, ga, gb = (torch.empty(sh, device=DEV) for sh in ((n, dk), (n, dk), (n, dv), (n,), (n,)))
    go = torch.empty((n, dv), device=DEV)
    aq = torch.empty((n_q, d), device=DEV)
    aK = torch.empty((n_kv, T, d), dtype=torch.int16, device=DEV)
    aV = torch.empty_like(aK)
    ao = torch.empty((n_q, d), device=DEV)
    wsb = moe.attn_workspace_bytes(n_q, n_kv, d, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    g_gdn = _capture(lambda: moe.gdn_step(n, dk, dv, S0, gq, gk, gv, ga, gb, go))
    g_att = _capture(lambda: moe.attn_decode(n_q, n_kv, d, T, aq, aK, aV, ao, ws, wsb))
    ws2 = torch.empty_like(ws)
    for rep in range(4):
        S, q, k, v, a, b = _gdn_inputs(500 + rep, n, dk, dv)
        for dst, src in zip((S0, gq, gk, gv, ga, gb), (S, q, k, v, a, b)):
            dst.copy_(torch.from_numpy(src))
        qa, K, V = _attn_inputs(600 + rep, n_q, n_kv, d, T)
        aq.copy_(torch.from_numpy(qa))
        aK.copy_(torch.from_numpy(K.view(np.int16)))
        aV.copy_(torch.from_numpy(V.view(np.int16)))
        # the eager calls first, on their own buffers
        S_e = S0.clone()
        o_e = torch.empty_like(go)
        moe.gdn_step(n, dk, dv, S_e, gq, gk, gv, ga, gb, o_e)
        ao_e = torch.empty_like(ao)
        moe.attn_decode(n_q, n_kv, d, T, aq, aK, aV, ao_e, ws2, wsb)
        go.fill_(float("nan"))
        ao.fill_(float("nan"))
        g_gdn.replay()
        g_att.replay()
        torch.cuda.synchronize()
        assert torch.equal(S0, S_e) and torch.equal(go, o_e), "gated delta rule, replay %d" % rep
        assert torch.equal(ao, ao_e), "attention, replay %d" % rep
        assert _head_err(ao.cpu().numpy(), oracle.attn_decode(qa, K, V)) <= ATTN_TOL
    del g_gdn, g_att
