"""GPU tests of tiered expert residency: an HBM cache of expert records over a
store in pinned host memory (moe_cache_init, moe_layer_decode_cached).

The policy is checked call by call against a plain model of it written here
(slot of every expert, hit and miss counts, bytes copied); the outputs against
moe_layer_decode on a slab that holds every record in device memory, bit for
bit, since the same kernels multiply the same records; and the first tokens
against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import quantized_expert_dequant_amd as moe
from quantized_expert_dequant_amd.slab import DeviceLayer, host_store, upload_experts, workspace

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


class CacheModel:
    """The policy: hits refresh their slot's stamp; misses, in ascending expert id, each take
    the slot with the smallest (stamp, slot) among those this call has not stamped."""

    def __init__(self, E, slots):
        self.E, self.S = E, slots
        self.slot_of = [-1] * E
        self.expert_of = [-1] * slots
        self.last_use = [0] * slots
        self.clock = 1
        self.hits = self.misses = self.calls = 0

    def call(self, idx):
        sel = sorted({int(e) for e in idx if 0 <= e < self.E})
        for e in sel:
            if self.slot_of[e] >= 0:
                self.last_use[self.slot_of[e]] = self.clock
                self.hits += 1
        for e in [e for e in sel if self.slot_of[e] < 0]:
            _, s = min((self.last_use[s], s) for s in range(self.S) if self.last_use[s] < self.clock)
            if self.expert_of[s] >= 0:
                self.slot_of[self.expert_of[s]] = -1
            self.expert_of[s], self.slot_of[e], self.last_use[s] = e, s, self.clock
            self.misses += 1
        self.calls += 1
        self.clock += 1


def _up256(n):
    return (n + 255) & ~255


def _state(state, E, slots):
    """(counters, clock, slot_of, expert_of) of the device state (layout in cache.hip)."""
    raw = state.cpu().numpy()
    counters = raw[:32].view(np.uint64)
    clock = int(raw[32:36].view(np.uint32)[0])
    slot_of = raw[64:64 + 4 * E].view(np.int32)
    o = 64 + _up256(4 * E)
    expert_of = raw[o:o + 4 * slots].view(np.int32)
    return counters, clock, slot_of, expert_of


class Cached:
    def __init__(self, n, slots, store=None, bits=None, source=None, cfg=None):
        cfg, seed = dict(WORKLOADS[n] if cfg is None else cfg), seed_of(n)
        if bits is not None:
            cfg["bits"] = bits
        self.cfg, self.seed = cfg, seed
        H, I, E, K, bits = cfg["H"], cfg["I"], cfg["E"], cfg["K"], cfg["bits"]
        if source is None:
            source = lambda f, m: synth.experts(seed, 0, f, m, bits, H, I)
        if store is None:
            store = host_store(source, E + 1, bits, H, I, device=DEV)
        self.store = store
        wr = torch.from_numpy(synth.router(seed, 0, E, H)).to(DEV)
        bias = torch.from_numpy(synth.zipf_bias(E, cfg["zipf"])).to(DEV) if cfg.get("zipf") else None
        self.L = DeviceLayer(H, I, E, K, bits, store, wr, bias)  # desc->experts: the pinned store
        rb = moe.record_bytes(bits, H, I)
        self.slots = slots
        self.slab = torch.empty((slots + 1) * rb, dtype=torch.uint8, device=DEV)
        self.state = torch.empty(moe.cache_state_bytes(E, slots), dtype=torch.uint8, device=DEV)
        self.cache = moe.make_cache(slots, self.slab, self.state)
        moe.cache_init(self.L.desc, self.cache)
        self.rb = rb

    def decode(self, x):
        B, L = x.shape[0], self.L
        n = moe.cache_workspace_bytes(L.desc, self.slots, B)
        ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
        y = torch.empty((B, L.H), dtype=torch.float32, device=DEV)
        idx = torch.empty((B, L.K), dtype=torch.int32, device=DEV)
        w = torch.empty((B, L.K), dtype=torch.float32, device=DEV)
        moe.layer_decode_cached(L.desc, self.cache, x, B, y, idx, w, ws, n)
        torch.cuda.synchronize()
        return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def _resident(layer, x):
    B = x.shape[0]
    ws, n = workspace(layer.desc, B)
    y = torch.empty((B, layer.H), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, layer.K), dtype=torch.int32, device=DEV)
    w = torch.empty((B, layer.K), dtype=torch.float32, device=DEV)
    moe.layer_decode(layer.desc, x, B, y, idx, w, ws, n)
    torch.cuda.synchronize()
    return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("B,slots", [(1, 6), (1, 4), (3, 12)])
def test_cache_policy_and_outputs_tiny(B, slots):
    """Workload 0 (E = 16) through a small cache: 30 calls of B tokens; after every call the
    state equals the model's and the outputs equal the resident decode's bit for bit (B = 3
    takes the grouped path on the slot ids)."""
    c = Cached(0, slots)
    E = c.cfg["E"]
    resident = build_layer(c.cfg, c.seed)
    model = CacheModel(E, slots)
    for t in range(30):
        x = torch.from_numpy(synth.tokens(c.seed, 300 + t, B, c.L.H)).to(DEV)
        y, idx, w = c.decode(x)
        yr, idxr, wr = _resident(resident, x)
        np.testing.assert_array_equal(idx, idxr)
        np.testing.assert_array_equal(w, wr)
        np.testing.assert_array_equal(y, yr)
        model.call(idx.reshape(-1))
        counters, clock, slot_of, expert_of = _state(c.state, E, slots)
        assert list(slot_of) == model.slot_of and list(expert_of) == model.expert_of, "call %d" % t
        assert clock == model.clock
        assert (int(counters[0]), int(counters[1]), int(counters[3])) == (model.hits, model.misses, model.calls)
        assert int(counters[2]) == model.misses * c.rb
    assert model.misses > slots  # the cache was too small to hold every expert: evictions happened
    y_ref, idx_ref, _, _ = oracle_layer(c.cfg, c.seed, 0, x.cpu().numpy())
    np.testing.assert_array_equal(idx, idx_ref)
    for b in range(B):
        assert rel_err(y[b], y_ref[b]) <= TOL


@pytest.mark.parametrize("B,slots", [(1, 5), (3, 12)])
def test_cache_3bit_layer(B, slots):
    """The tiny layer with 3-bit codes through a small cache: 20 calls, the state equal to the
    policy model's after every call and the outputs to the resident decode's bit for bit."""
    c = Cached(0, slots, bits=3)
    E = c.cfg["E"]
    resident = build_layer(c.cfg, c.seed)
    model = CacheModel(E, slots)
    for t in range(20):
        x = torch.from_numpy(synth.tokens(c.seed, 950 + t, B, c.L.H)).to(DEV)
        y, idx, w = c.decode(x)
        yr, idxr, wr = _resident(resident, x)
        np.testing.assert_array_equal(idx, idxr)
        np.testing.assert_array_equal(w, wr)
        np.testing.assert_array_equal(y, yr)
        model.call(idx.reshape(-1))
        _, _, slot_of, _ = _state(c.state, E, slots)
        assert list(slot_of) == model.slot_of, "call %d" % t
    assert model.misses > slots
    y_ref, idx_ref, _, _ = oracle_layer(c.cfg, c.seed, 0, x.cpu().numpy())
    np.testing.assert_array_equal(idx, idx_ref)
    for b in range(B):
        assert rel_err(y[b], y_ref[b]) <= TOL


def _bf16_scaled(bits16, k):
    """bf16 bit patterns times 2^k (exponent raised; zeros and values that would overflow kept)."""
    b = bits16.astype(np.int32)
    e = (b >> 7) & 0xFF
    ok = (e > 0) & (e + k < 255)
    return np.where(ok, (b & ~(0xFF << 7)) | ((e + k) << 7), b).astype(np.uint16)


@pytest.mark.parametrize("B,slots", [(3, 12), (5, 16), (16, 16), (17, 16)])
def test_cache_per_token_routing_batches(B, slots):
    """A 2-bit tiny layer whose expert 4 has its scales x 2^14 keeps the range flags, so a
    batch runs the token-by-token kernels: up to 16 tokens the plan kernel selects each
    token's top-K from the router logits itself, past 16 the top-K kernel does it first.
    20 calls of B tokens: the routing, the weights and the outputs equal those of the
    resident decode of the same records bit for bit, and the cache state the model's."""
    cfg, seed = dict(WORKLOADS[0], bits=2), seed_of(0)  # the seed Cached(0, ...) routes with
    H, I, E, K = cfg["H"], cfg["I"], cfg["E"], cfg["K"]
    ex = synth.experts(seed, 0, 0, E + 1, 2, H, I)
    ex.scales[4] = _bf16_scaled(ex.scales[4], 14)

    def src(first, n):
        return synth.Canonical(2, H, I, 64, ex.gate[first:first + n], ex.up[first:first + n],
                               ex.down[first:first + n], ex.scales[first:first + n], ex.biases[first:first + n])

    c = Cached(0, slots, bits=2, source=src)
    assert c.L.desc.expert_flags is not None and int(c.L.expert_flags[4]) == 1
    assert c.seed == seed
    wr = torch.from_numpy(synth.router(seed, 0, E, H)).to(DEV)
    resident = DeviceLayer(H, I, E, K, 2, upload_experts(src, E + 1, 2, H, I, device=DEV), wr)
    assert moe.grouped_launch_info(resident.desc, B)["grouped"] == 0
    model = CacheModel(E, slots)
    routed_to_4 = 0
    for t in range(20):
        x = torch.from_numpy(synth.tokens(seed, 700 + t, B, H)).to(DEV)
        y, idx, w = c.decode(x)
        yr, idxr, wres = _resident(resident, x)
        np.testing.assert_array_equal(idx, idxr, err_msg="call %d" % t)
        np.testing.assert_array_equal(w, wres, err_msg="call %d" % t)
        np.testing.assert_array_equal(y, yr, err_msg="call %d" % t)
        assert np.all(np.isfinite(y))
        routed_to_4 += int((idx == 4).sum())
        model.call(idx.reshape(-1))
        counters, clock, slot_of, expert_of = _state(c.state, E, slots)
        assert list(slot_of) == model.slot_of and list(expert_of) == model.expert_of, "call %d" % t
        assert clock == model.clock
        assert (int(counters[0]), int(counters[1]), int(counters[3])) == (model.hits, model.misses, model.calls)
    assert routed_to_4 > 0, "no token reached the flagged expert"
    if slots < E:
        assert model.misses > slots  # evictions happened

    # the last call against the oracle's routing and expert FFNs on the same records
    xh = x.cpu().numpy()
    _, idx_ref, w_ref, margin = oracle_layer(cfg, seed, 0, xh)
    assert margin.min() > 1e-9
    np.testing.assert_array_equal(idx, idx_ref)
    np.testing.assert_allclose(w, w_ref, rtol=W_RTOL)

    def ffn(e, xb):
        return oracle.expert_ffn(2, H, I, ex.gate[e], ex.up[e], ex.down[e], ex.scales[e], ex.biases[e], xb)[1]

    for b in range(B):
        ref = ffn(E, xh[b]) + sum(float(w_ref[b, k]) * ffn(int(idx_ref[b, k]), xh[b]) for k in range(K))
        assert rel_err(y[b], ref) <= TOL, "token %d" % b


@pytest.mark.parametrize("B,slots", [(1, 40), (2, 70)])
def test_cache_most_experts_and_largest_k(B, slots):
    """E = 1024 and K = 32, the library's maxima, through a cache smaller than the expert set:
    one token per call (the plan kernel selects its 32 experts from 1024 logits itself) and
    two (the grouped path on slot ids).  20 calls: the state equals the policy model's after
    every call and the outputs equal the resident decode's bit for bit."""
    cfg = dict(H=512, I=128, E=1024, K=32, bits=4, B=B, layers=1, zipf=None)
    c = Cached(0, slots, cfg=cfg)
    resident = build_layer(c.cfg, c.seed)
    model = CacheModel(1024, slots)
    for t in range(20):
        x = torch.from_numpy(synth.tokens(c.seed, 900 + t, B, c.L.H)).to(DEV)
        y, idx, w = c.decode(x)
        yr, idxr, wr = _resident(resident, x)
        np.testing.assert_array_equal(idx, idxr, err_msg="call %d" % t)
        np.testing.assert_array_equal(w, wr, err_msg="call %d" % t)
        np.testing.assert_array_equal(y, yr, err_msg="call %d" % t)
        model.call(idx.reshape(-1))
        counters, clock, slot_of, expert_of = _state(c.state, 1024, slots)
        assert list(slot_of) == model.slot_of and list(expert_of) == model.expert_of, "call %d" % t
        assert (int(counters[0]), int(counters[1]), int(counters[3])) == (model.hits, model.misses, model.calls)
    assert model.misses > slots
    y_ref, idx_ref, _, _ = oracle_layer(c.cfg, c.seed, 0, x.cpu().numpy())
    np.testing.assert_array_equal(idx, idx_ref)
    for b in range(B):
        assert rel_err(y[b], y_ref[b]) <= TOL


def test_cache_full_layer_from_pinned_host_memory():
    """The full workload-1 layer (513 records, 3.6 GB) in pinned host memory, 32 HBM slots:
    16 tokens decoded one at a time, each equal to the resident decode; the first against
    the oracle."""
    c = Cached(1, 32)
    resident = build_layer(c.cfg, c.seed)
    model = CacheModel(c.cfg["E"], 32)
    for t in range(16):
        x = torch.from_numpy(synth.tokens(c.seed, 400 + t, 1, c.L.H)).to(DEV)
        y, idx, w = c.decode(x)
        yr, idxr, _ = _resident(resident, x)
        np.testing.assert_array_equal(idx, idxr)
        np.testing.assert_array_equal(y, yr)
        model.call(idx.reshape(-1))
        if t == 0:
            y_ref, idx_ref, _, _ = oracle_layer(c.cfg, c.seed, 0, x.cpu().numpy())
            np.testing.assert_array_equal(idx, idx_ref)
            assert rel_err(y[0], y_ref[0]) <= TOL
    counters, _, slot_of, _ = _state(c.state, c.cfg["E"], 32)
    assert list(slot_of) == model.slot_of
    assert (int(counters[0]), int(counters[1])) == (model.hits, model.misses)
    del resident, c
    torch.cuda.empty_cache()


def test_cache_graph_replay_matches_eager():
    """Cached decodes captured in a HIP graph: three replays of four calls follow the same
    state sequence as twelve eager calls on a second cache from the same start."""
    a, b = Cached(0, 5), None
    b = Cached(0, 5, store=a.store)
    H, K = a.L.H, a.L.K
    xs = [torch.from_numpy(synth.tokens(a.seed, 500 + t, 1, H)).to(DEV) for t in range(4)]
    n = moe.cache_workspace_bytes(a.L.desc, 5, 1)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    ys = [torch.empty((1, H), dtype=torch.float32, device=DEV) for _ in range(4)]
    idx = torch.empty((1, K), dtype=torch.int32, device=DEV)
    w = torch.empty((1, K), dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for t in range(4):
                moe.layer_decode_cached(a.L.desc, a.cache, xs[t], 1, ys[t], idx, w, ws, n)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    moe.cache_init(a.L.desc, a.cache)  # capture recorded no work: start both caches equal
    torch.cuda.synchronize()
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        got = [y.cpu().numpy() for y in ys]
        for t in range(4):
            ye, _, _ = b.decode(xs[t])
            np.testing.assert_array_equal(got[t], ye, err_msg="replay %d call %d" % (r, t))
        ca, _, sa, _ = _state(a.state, a.cfg["E"], 5)
        cb, _, sb, _ = _state(b.state, b.cfg["E"], 5)
        np.testing.assert_array_equal(ca, cb)
        np.testing.assert_array_equal(sa, sb)
