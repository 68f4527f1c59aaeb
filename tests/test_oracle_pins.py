"""Pins of the float64 oracle against facts that do not come from the oracle.

Each test checks the oracle against a closed form, a hand-built example, a
brute-force search, an identity of the method, or an independent encoding
written here, chosen so that a plausible slip (dropped term, wrong sign,
swapped index, transposed operand, wrong group, wrong tie-break) fails one.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

H_T, I_T, E_T = 128, 64, 16   # tiny shapes that still span two groups per gate/up row


# ---------- independent canonical encoder / decoder (test-side only) ----------

def encode_codes(q, bits):
    """Pack an integer matrix [rows][cols] into canonical bytes (low bits = lower element)."""
    q = np.asarray(q, dtype=np.uint8)
    rows, cols = q.shape
    per = 8 // bits
    out = np.zeros((rows, cols // per), np.uint8)
    for t in range(per):
        out |= (q[:, t::per] << (bits * t)).astype(np.uint8)
    return out


def bf16_value(bits16):
    return float(np.array([int(bits16) << 16], np.uint32).view(np.float32)[0])


def random_expert(rng, bits, H, I, group=64):
    """Random expert given as known (q, s, b) plus its canonical encoding."""
    qmax = (1 << bits) - 1
    qg = rng.integers(0, qmax + 1, (I, H))
    qu = rng.integers(0, qmax + 1, (I, H))
    qd = rng.integers(0, qmax + 1, (H, I))
    ng = 2 * I * (H // group) + H * (I // group)
    s = np.array([synth.bf16_from_double(v) for v in np.abs(rng.normal(0, 0.02, ng))], np.uint16)
    b = np.array([synth.bf16_from_double(v) for v in rng.normal(0, 0.01, ng)], np.uint16)
    return dict(qg=qg, qu=qu, qd=qd, s=s, b=b,
                gate=encode_codes(qg, bits), up=encode_codes(qu, bits), down=encode_codes(qd, bits))


def dense_from_known(q, s_bits, b_bits, group):
    rows, cols = q.shape
    s = np.array([bf16_value(v) for v in s_bits]).reshape(rows, cols // group)
    b = np.array([bf16_value(v) for v in b_bits]).reshape(rows, cols // group)
    return np.repeat(s, group, axis=1) * q + np.repeat(b, group, axis=1)


class Stack:
    def __init__(self, experts):
        self.gate = np.stack([e["gate"] for e in experts])
        self.up = np.stack([e["up"] for e in experts])
        self.down = np.stack([e["down"] for e in experts])
        self.scales = np.stack([e["s"] for e in experts])
        self.biases = np.stack([e["b"] for e in experts])


# ---------------------------------- format ------------------------------------

def test_byte_unpack_handbuilt(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "dequant_handbuilt.json")))
    for case in g["byte_unpack"]:
        row = np.array([int(case["byte"], 16)], np.uint8)
        got = [oracle.code_at(row, case["bits"], c) for c in range(len(case["codes"]))]
        assert got == case["codes"], case


def test_dequant_handbuilt(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "dequant_handbuilt.json")))
    for case in g["cases"]:
        bits, codes = case["bits"], case["codes"]
        cols = 64
        q = np.zeros((1, cols), np.int64)
        q[0, :len(codes)] = codes
        W = oracle.dequant_matrix(bits, 1, cols, encode_codes(q, bits),
                                  np.array([int(case["scale_bf16"], 16)], np.uint16),
                                  np.array([int(case["bias_bf16"], 16)], np.uint16))
        assert list(W[0, :len(codes)]) == case["expect"], case["name"]


def test_bf16_widening_exact():
    assert oracle.bf16_to_double(0x3F80) == 1.0
    assert oracle.bf16_to_double(0xC000) == -2.0
    assert oracle.bf16_to_double(0x0001) == 2.0 ** -133
    assert oracle.bf16_to_double(0x7F7F) == (2 - 2 ** -7) * 2.0 ** 127


@pytest.mark.parametrize("bits", [4, 2])
def test_dequant_group_and_row_indexing(bits):
    """Independent encoding of known (q, s, b): catches row/col/group mix-ups."""
    rng = np.random.default_rng(7 + bits)
    rows, cols, group = 5, 256, 64
    q = rng.integers(0, 1 << bits, (rows, cols))
    s = np.array([synth.bf16_from_double(v) for v in rng.normal(0, 1, rows * cols // group)], np.uint16)
    b = np.array([synth.bf16_from_double(v) for v in rng.normal(0, 1, rows * cols // group)], np.uint16)
    W = oracle.dequant_matrix(bits, rows, cols, encode_codes(q, bits), s, b, group)
    np.testing.assert_array_equal(W, dense_from_known(q, s, b, group))


# ---------------------------------- router -------------------------------------

def test_router_integer_exact():
    rng = np.random.default_rng(1)
    Wr = rng.integers(-8, 9, (E_T, H_T)).astype(np.float32)
    x = rng.integers(-8, 9, (3, H_T)).astype(np.float32)
    prior = rng.integers(-4, 5, E_T).astype(np.float32)
    got = oracle.router_logits(x, Wr, prior)
    want = x.astype(np.int64) @ Wr.astype(np.int64).T + prior.astype(np.int64)
    np.testing.assert_array_equal(got, want.astype(np.float64))


# ---------------------------------- top-k -------------------------------------

def _brute_topk(logits, K):
    """The unique K-subset whose members all rank before every outsider."""
    E = len(logits)
    before = lambda a, b: logits[a] > logits[b] or (logits[a] == logits[b] and a < b)
    winners = []
    for S in itertools.combinations(range(E), K):
        inside = set(S)
        if all(before(a, b) for a in S for b in range(E) if b not in inside):
            winners.append(S)
    assert len(winners) == 1
    members = winners[0]
    # rank order inside the subset by the same relation
    return sorted(members, key=lambda a: sum(before(b, a) for b in members))


@pytest.mark.parametrize("seed", range(6))
def test_topk_bruteforce_E16(seed):
    rng = np.random.default_rng(seed)
    if seed % 2:
        logits = rng.integers(-3, 4, E_T).astype(np.float64)   # many exact ties
    else:
        logits = rng.normal(0, 1, E_T)
    for K in (1, 4, 7):
        idx, w, m = oracle.topk(logits, K)
        assert list(idx) == _brute_topk(list(logits), K)


def test_topk_ties_lower_id_wins():
    rng = np.random.default_rng(3)
    Wr = rng.normal(0, 1, (E_T, H_T)).astype(np.float32)
    Wr[9] = Wr[2]     # exact duplicate rows -> bit-identical logits
    Wr[14] = Wr[2]
    x = rng.normal(0, 1, H_T).astype(np.float32)
    lg = oracle.router_logits(x, Wr)[0]
    assert lg[2] == lg[9] == lg[14]
    order = np.argsort(-lg, kind="stable")      # stable: equal keys keep id order
    K = int(np.where(order == 9)[0][0]) + 1     # K that includes id 9 but not 14
    idx, _, _ = oracle.topk(lg, K)
    assert 2 in idx and 9 in idx and 14 not in idx
    assert list(idx).index(2) < list(idx).index(9)


def test_softmax_equal_logits_and_k1():
    idx, w, _ = oracle.topk(np.zeros(E_T), 4)
    assert list(idx) == [0, 1, 2, 3] and all(v == 0.25 for v in w)
    idx, w, _ = oracle.topk(np.random.default_rng(0).normal(size=E_T), 1)
    assert w[0] == 1.0


def test_renormalized_weights_equal_softmax_over_kept():
    """Softmax over all E then renormalize == softmax over the kept logits only."""
    lg = np.random.default_rng(11).normal(0, 2, 512)
    idx, w, m = oracle.topk(lg, 10)
    kept = lg[idx]
    ref = np.exp(kept - kept.max()) / np.exp(kept - kept.max()).sum()
    np.testing.assert_allclose(w, ref, rtol=1e-14)
    full = np.exp(lg - lg.max()) / np.exp(lg - lg.max()).sum()
    _, w_raw, _ = oracle.topk(lg, 10, renormalize=False)
    np.testing.assert_allclose(w_raw, full[idx], rtol=1e-14)
    srt = np.sort(lg)[::-1]
    assert m == srt[9] - srt[10]


# ---------------------------------- FFN ---------------------------------------

def test_ffn_constant_weights_closed_form():
    """s = 0 everywhere: each matrix is its bias; y has a closed form."""
    H, I = 64, 64
    bits = 4
    ng = synth.n_groups(H, I)
    z = np.zeros((I, H * bits // 8), np.uint8)
    zd = np.zeros((H, I * bits // 8), np.uint8)
    s = np.zeros(ng, np.uint16)
    b = np.full(ng, 0x3F80, np.uint16)             # every weight = 1.0
    x = np.full(H, 1.0 / 32)                       # sum x = 2
    h, y = oracle.expert_ffn(bits, H, I, z, z, zd, s, b, x)
    S = 2.0
    h_ref = S / (1 + math.exp(-S)) * S
    np.testing.assert_allclose(h, h_ref, rtol=1e-15)
    np.testing.assert_allclose(y, I * h_ref, rtol=1e-14)


@pytest.mark.parametrize("bits", [4, 2])
def test_ffn_matches_independent_dense(bits):
    """Known (q, s, b) -> dense numpy SwiGLU vs the oracle reading the encoded bytes."""
    rng = np.random.default_rng(21 + bits)
    ex = random_expert(rng, bits, H_T, I_T)
    x = rng.normal(0, 1, H_T)
    ngu = I_T * (H_T // 64)
    Wg = dense_from_known(ex["qg"], ex["s"][:ngu], ex["b"][:ngu], 64)
    Wu = dense_from_known(ex["qu"], ex["s"][ngu:2 * ngu], ex["b"][ngu:2 * ngu], 64)
    Wd = dense_from_known(ex["qd"], ex["s"][2 * ngu:], ex["b"][2 * ngu:], 64)
    g, u = Wg @ x, Wu @ x
    h_ref = g / (1 + np.exp(-g)) * u
    y_ref = Wd @ h_ref
    h, y = oracle.expert_ffn(bits, H_T, I_T, ex["gate"], ex["up"], ex["down"], ex["s"], ex["b"], x)
    np.testing.assert_allclose(h, h_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y, y_ref, rtol=1e-12, atol=1e-11)


def test_silu_zero_gate_gives_zero():
    rng = np.random.default_rng(5)
    ex = random_expert(rng, 4, H_T, I_T)
    ngu = I_T * (H_T // 64)
    ex["s"][:ngu] = 0
    ex["b"][:ngu] = 0
    h, y = oracle.expert_ffn(4, H_T, I_T, ex["gate"], ex["up"], ex["down"], ex["s"], ex["b"],
                             rng.normal(size=H_T))
    assert np.all(h == 0.0) and np.all(y == 0.0)


# ---------------------------------- layer -------------------------------------

def _tiny_layer(seed, bits=4, E=E_T):
    rng = np.random.default_rng(seed)
    experts = [random_expert(rng, bits, H_T, I_T) for _ in range(E + 1)]
    Wr = rng.normal(0, 1 / math.sqrt(H_T), (E, H_T)).astype(np.float32)
    x = rng.normal(0, 1, (2, H_T)).astype(np.float32)
    return experts, Wr, x


def _ffn(ex, bits, x):
    return oracle.expert_ffn(bits, H_T, I_T, ex["gate"], ex["up"], ex["down"], ex["s"], ex["b"], x)[1]


def test_dense_equivalence_K_equals_E():
    """K = E: the layer equals a dense softmax-weighted sum of every expert (no selection)."""
    experts, Wr, x = _tiny_layer(31)
    y, idx, w, _ = oracle.layer_decode(4, H_T, I_T, E_T, E_T, x, Wr, Stack(experts))
    for b in range(x.shape[0]):
        lg = Wr.astype(np.float64) @ x[b].astype(np.float64)
        p = np.exp(lg - lg.max())
        p /= p.sum()
        ref = sum(p[e] * _ffn(experts[e], 4, x[b].astype(np.float64)) for e in range(E_T))
        ref = ref + _ffn(experts[E_T], 4, x[b].astype(np.float64))
        np.testing.assert_allclose(y[b], ref, rtol=1e-11, atol=1e-10 * np.abs(ref).max())


def test_identical_experts_double_the_ffn():
    experts, Wr, x = _tiny_layer(32)
    same = [experts[0]] * (E_T + 1)
    y, _, _, _ = oracle.layer_decode(4, H_T, I_T, E_T, 4, x, Wr, Stack(same))
    for b in range(x.shape[0]):
        ref = 2.0 * _ffn(experts[0], 4, x[b].astype(np.float64))
        np.testing.assert_allclose(y[b], ref, rtol=1e-13, atol=1e-12 * np.abs(ref).max())


def test_permutation_invariance_of_expert_ids():
    experts, Wr, x = _tiny_layer(33)
    perm = np.random.default_rng(0).permutation(E_T)          # new id j holds old expert perm[j]
    experts_p = [experts[perm[j]] for j in range(E_T)] + [experts[E_T]]
    y0, idx0, w0, _ = oracle.layer_decode(4, H_T, I_T, E_T, 4, x, Wr, Stack(experts))
    y1, idx1, w1, _ = oracle.layer_decode(4, H_T, I_T, E_T, 4, x, Wr[perm], Stack(experts_p))
    np.testing.assert_array_equal(perm[idx1], idx0)
    np.testing.assert_allclose(w1, w0, rtol=1e-15)
    np.testing.assert_allclose(y1, y0, rtol=1e-12, atol=1e-12 * np.abs(y0).max())


def test_zero_gate_routed_leaves_shared_only():
    experts, Wr, x = _tiny_layer(34)
    ngu = I_T * (H_T // 64)
    for e in range(E_T):
        experts[e] = dict(experts[e])
        experts[e]["s"] = experts[e]["s"].copy()
        experts[e]["b"] = experts[e]["b"].copy()
        experts[e]["s"][:ngu] = 0
        experts[e]["b"][:ngu] = 0
    y, _, _, _ = oracle.layer_decode(4, H_T, I_T, E_T, 4, x, Wr, Stack(experts), shared_weight=1.0)
    for b in range(x.shape[0]):
        np.testing.assert_array_equal(y[b], _ffn(experts[E_T], 4, x[b].astype(np.float64)))


def test_layer_combines_selected_experts():
    """Layer output == sum over the oracle's own selection of per-expert FFNs (2-bit)."""
    experts, Wr, x = _tiny_layer(35, bits=2)
    prior = synth.zipf_bias(E_T, 1.1)
    y, idx, w, m = oracle.layer_decode(2, H_T, I_T, E_T, 3, x, Wr, Stack(experts), prior=prior,
                                       shared_weight=0.5)
    for b in range(x.shape[0]):
        lg = Wr.astype(np.float64) @ x[b].astype(np.float64) + prior.astype(np.float64)
        assert list(idx[b]) == _brute_topk(list(lg), 3)
        xb = x[b].astype(np.float64)
        ref = sum(w[b, k] * _ffn(experts[idx[b, k]], 2, xb) for k in range(3)) + 0.5 * _ffn(experts[E_T], 2, xb)
        np.testing.assert_allclose(y[b], ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())


def test_missing_expert_is_an_error():
    experts, Wr, x = _tiny_layer(36)
    with pytest.raises(KeyError):
        oracle.layer_decode(4, H_T, I_T, E_T, 4, x[:1], Wr, {E_T: Stack([experts[E_T]])})


# ------------------------------ grouping / stack -------------------------------

def test_group_by_expert_stable_bruteforce():
    rng = np.random.default_rng(8)
    B, K, E = 9, 3, 12
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(B)]).astype(np.int32)
    off, tok, sl, U = oracle.group_by_expert(idx, E)
    assert U == len(set(idx.reshape(-1).tolist()))
    for e in range(E):
        pairs = [(b, b * K + k) for b in range(B) for k in range(K) if idx[b, k] == e]
        got = list(zip(tok[off[e]:off[e + 1]].tolist(), sl[off[e]:off[e + 1]].tolist()))
        assert got == pairs
    assert off[E] == B * K


def test_rms_renorm_closed_form():
    y = np.random.default_rng(2).normal(0, 3, 4096)
    eps = 1e-6
    x = oracle.rms_renorm(y, eps)
    ms = np.mean(y * y)
    assert abs(math.sqrt(np.mean(x * x)) - 1 / math.sqrt(1 + eps / ms)) < 1e-14
    np.testing.assert_allclose(x / y, x[0] / y[0], rtol=1e-15)   # pure rescale, no shift
