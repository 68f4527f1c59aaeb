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
    """Pack an integer matrix [rows][cols] into canonical bytes (low bits = lower element;
    3-bit: each row as one little-endian bit string, element c at bits 3c..3c+2)."""
    q = np.asarray(q, dtype=np.uint8)
    rows, cols = q.shape
    if bits == 3:
        out = np.zeros((rows, cols * 3 // 8), np.uint8)
        for r in range(rows):
            acc = 0
            for c in range(cols):
                acc |= int(q[r, c]) << (3 * c)
            out[r] = np.frombuffer(acc.to_bytes(cols * 3 // 8, "little"), np.uint8)
        return out
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


def test_byte_unpack_3bit_handbuilt(golden_dir):
    """3-bit codes straddle bytes: hand-derived rows of three bytes decode to their eight codes."""
    g = json.load(open(os.path.join(golden_dir, "dequant_handbuilt.json")))
    for case in g["byte_unpack_3bit"]["cases"]:
        row = np.array([int(x, 16) for x in case["bytes"]], np.uint8)
        assert [oracle.code_at(row, 3, c) for c in range(8)] == case["codes"], case
        np.testing.assert_array_equal(encode_codes(np.array([case["codes"]]), 3)[0], row)


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


@pytest.mark.parametrize("bits", [4, 3, 2])
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


@pytest.mark.parametrize("bits", [4, 3, 2])
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


# -------------------- threaded forms of the layer decode ------------------------
# oracle_layer_decode_mt (the timed CPU baseline: router rows and the active experts'
# FFNs over OpenMP threads) and oracle_layer_decode_par (many tokens of a batch at
# once) must give the serial decode's results bit for bit, since every floating-point
# sum keeps its order; a slip in their indexing (w[k], the shared slot, the token
# offsets) would show as a difference.

def _assert_same_decode(a, b):
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    np.testing.assert_array_equal(a[2], b[2])


@pytest.mark.parametrize("bits,K,prior_s,shared_w", [(4, 4, None, 1.0), (2, 3, 1.1, 0.5), (4, 16, None, 1.0)])
def test_layer_decode_mt_and_par_equal_serial(bits, K, prior_s, shared_w):
    experts, Wr, _ = _tiny_layer(40 + K, bits=bits)
    x = np.random.default_rng(K).normal(0, 1, (5, H_T)).astype(np.float32)
    prior = synth.zipf_bias(E_T, prior_s) if prior_s else None
    kw = dict(prior=prior, shared_weight=shared_w)
    ser = oracle.layer_decode(bits, H_T, I_T, E_T, K, x, Wr, Stack(experts), **kw)
    par = oracle.layer_decode(bits, H_T, I_T, E_T, K, x, Wr, Stack(experts), parallel=True, **kw)
    _assert_same_decode(ser, par)
    np.testing.assert_array_equal(ser[3], par[3])
    for b in range(x.shape[0]):
        mt = oracle.layer_decode_mt(bits, H_T, I_T, E_T, K, x[b], Wr, Stack(experts), **kw)
        _assert_same_decode((ser[0][b], ser[1][b], ser[2][b]), mt)


@pytest.mark.slow
def test_layer_decode_mt_and_par_equal_serial_full_shape():
    """One token of the full layer shape (H=4096, I=1024, E=512, K=4), generated experts."""
    H, I, E, K, seed = 4096, 1024, 512, 4, 1001
    Wr = synth.router(seed, 0, E, H)
    x = synth.tokens(seed, 0, 2, H)
    lg = oracle.router_logits(x, Wr)
    need = sorted({int(e) for b in range(2) for e in oracle.topk(lg[b], K)[0]} | {E})
    experts = {e: synth.experts(seed, 0, e, 1, 4, H, I) for e in need}
    ser = oracle.layer_decode(4, H, I, E, K, x, Wr, experts)
    par = oracle.layer_decode(4, H, I, E, K, x, Wr, experts, parallel=True)
    _assert_same_decode(ser, par)
    mt = oracle.layer_decode_mt(4, H, I, E, K, x[1], Wr, experts)
    _assert_same_decode((ser[0][1], ser[1][1], ser[2][1]), mt)


# ------------------------ 4-bit -> 2-bit requantization -------------------------
# Reading (the pages give only the result, 209 GB -> 120 GB): per group of 64, the
# dequantized 4-bit weights are refit by b2 = bf16(min w), s2 = bf16((max - min) / 3),
# q2 = clamp(rint((w - b2) / s2), 0, 3), every step in IEEE double.

from fractions import Fraction


def _bf16_exact(bits16):
    return Fraction(bf16_value(bits16)) if (bits16 & 0x7F80) != 0x7F80 else None


def _nearest_bf16_bruteforce(v):
    """The nearest bf16 to a finite double by exact rational search over the two candidates
    around it (bit patterns are monotone in value for a fixed sign), ties to even."""
    x = Fraction(v)
    sign = 0x8000 if v < 0 or (v == 0 and math.copysign(1, v) < 0) else 0
    a = abs(x)
    lo, hi = 0, 0x7F80  # largest pattern with value <= a, searched by bisection
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if _bf16_exact(mid) <= a:
            lo = mid
        else:
            hi = mid - 1
    below = lo
    above = lo + 1
    vb = _bf16_exact(below)
    if vb == a:
        return sign | below
    va = Fraction(2) ** 128 if above == 0x7F80 else _bf16_exact(above)
    db, da = a - vb, va - a
    pick = below if db < da or (db == da and below % 2 == 0) else above
    return sign | pick


def test_bf16_round_matches_exact_nearest():
    rng = np.random.default_rng(3)
    vals = [0.0, -0.0, 1.0, -1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 3e38, 1e-40, 2 ** -133, 1.5 * 2 ** -133, 2 ** -127]
    vals += list(rng.normal(0, 0.02, 300)) + list(rng.normal(0, 1, 100) * 10.0 ** rng.integers(-30, 30, 100))
    for v in vals:
        assert oracle.bf16_round(v) == _nearest_bf16_bruteforce(v), v
    assert oracle.bf16_round(3.4e38) == 0x7F80  # past the largest bf16: infinity


def test_requant_group_closed_forms():
    # s4 = 0.5, b4 = 0, codes 0..6: w = 0, 0.5, ..., 3 -> b2 = 0, s2 = 1, q2 = rint(w) (ties to even)
    q2, s2, b2 = oracle.requant_group([0, 1, 2, 3, 4, 5, 6], 0x3F00, 0x0000)
    assert (s2, b2) == (0x3F80, 0x0000)
    assert list(q2) == [0, 0, 1, 2, 2, 2, 3]
    # a constant group: s2 = 0, every code 0, b2 = the weight
    q2, s2, b2 = oracle.requant_group([9] * 64, 0x3F00, 0xBF80)  # w = 0.5 * 9 - 1 = 3.5
    assert s2 == 0 and b2 == 0x4060 and not any(q2)
    # s4 = 1, b4 = 0, codes 0..15: b2 = 0, s2 = 5, q2 = rint(w / 5) clamped
    q2, s2, b2 = oracle.requant_group(list(range(16)), 0x3F80, 0x0000)
    assert (s2, b2) == (0x40A0, 0x0000)
    assert list(q2) == [0, 0, 0, 1, 1, 1, 1, 1, 2, 2, 2, 2, 2, 3, 3, 3]
    # a negative scale reverses the order: w = 1 - q, min at q = 15
    q2, s2, b2 = oracle.requant_group([0, 15, 6, 9], 0xBF80, 0x3F80)
    assert (s2, b2) == (0x40A0, 0xC160)  # (1 - (-14)) / 3 = 5, min = -14
    assert list(q2) == [3, 0, 2, 1]


def test_requant_group_nearest_level_property():
    """For random groups: b2, s2 are the exact nearest bf16 of min and of (max - min) / 3 (the
    division rounded once in double), and every code is the nearest of the four levels."""
    rng = np.random.default_rng(11)
    for _ in range(200):
        q4 = rng.integers(0, 16, 64)
        s4 = synth.bf16_from_double(abs(rng.normal(0, 0.02)))
        b4 = synth.bf16_from_double(rng.normal(0, 0.01))
        q2, s2, b2 = oracle.requant_group(q4, s4, b4)
        w = [Fraction(bf16_value(s4)) * int(q) + Fraction(bf16_value(b4)) for q in q4]
        lo, hi = min(w), max(w)
        assert b2 == _nearest_bf16_bruteforce(float(lo))
        assert s2 == _nearest_bf16_bruteforce((float(hi) - float(lo)) / 3.0)
        S, Bv = Fraction(bf16_value(s2)), Fraction(bf16_value(b2))
        for wc, qc in zip(w, q2):
            d = abs(wc - (Bv + S * int(qc)))
            assert all(d <= abs(wc - (Bv + S * j)) for j in range(4)), (wc, qc)


def test_requant_expert_group_and_row_indexing():
    """Every weight of the requantized expert equals b2 + s2 * q2 of its own group as the
    group function gives it (rows, groups and the gate | up | down split all line up)."""
    rng = np.random.default_rng(5)
    H, I = 192, 128
    ex = random_expert(rng, 4, H, I)
    g2, u2, d2, s2, b2 = oracle.requant_expert(H, I, ex["gate"], ex["up"], ex["down"], ex["s"], ex["b"])
    ngu = I * (H // 64)
    for name, q4, codes2, rows, cols, off in (("gate", ex["qg"], g2, I, H, 0), ("up", ex["qu"], u2, I, H, ngu),
                                              ("down", ex["qd"], d2, H, I, 2 * ngu)):
        W2 = oracle.dequant_matrix(2, rows, cols, codes2, s2[off:off + rows * cols // 64], b2[off:off + rows * cols // 64])
        for r in range(0, rows, 7):
            for g in range(cols // 64):
                gi = off + r * (cols // 64) + g
                q2, ss, bb = oracle.requant_group(q4[r, 64 * g:64 * g + 64], ex["s"][gi], ex["b"][gi])
                assert (ss, bb) == (int(s2[gi]), int(b2[gi])), (name, r, g)
                np.testing.assert_array_equal(W2[r, 64 * g:64 * g + 64],
                                              bf16_value(ss) * q2.astype(np.float64) + bf16_value(bb))


# ------------------- the attention half: GatedDeltaNet and full attention -------------------

def _gdn_inputs(rng, n=3, dk=8, dv=6):
    S = rng.normal(0, 1, (n, dv, dk))
    q, k = rng.normal(0, 1, (n, dk)), rng.normal(0, 1, (n, dk))
    v = rng.normal(0, 1, (n, dv))
    return S, q, k, v, rng.uniform(0.5, 1.0, n), rng.uniform(0.0, 1.0, n)


def test_gdn_no_write_decays_the_state():
    """beta = 0: the state is only decayed, S' = alpha S, and o = S' q."""
    S, q, k, v, a, _ = _gdn_inputs(np.random.default_rng(1))
    S1, o = oracle.gdn_step(S, q, k, v, a, np.zeros(3))
    np.testing.assert_array_equal(S1, a[:, None, None] * S)
    for h in range(3):
        np.testing.assert_allclose(o[h], S1[h] @ q[h], rtol=1e-13, atol=1e-13)


def test_gdn_write_into_an_empty_state_is_the_outer_product():
    _, q, k, v, a, b = _gdn_inputs(np.random.default_rng(2))
    S1, o = oracle.gdn_step(np.zeros((3, 6, 8)), q, k, v, a, b)
    for h in range(3):
        np.testing.assert_array_equal(S1[h], np.outer(b[h] * v[h], k[h]))


def test_gdn_delta_rule_fixed_point():
    """alpha = beta = 1 and a unit key: the new state maps k exactly onto v (S' k = v)."""
    rng = np.random.default_rng(3)
    S, q, k, v, _, _ = _gdn_inputs(rng, n=4, dk=16, dv=12)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    S1, _ = oracle.gdn_step(S, q, k, v, np.ones(4), np.ones(4))
    for h in range(4):
        np.testing.assert_allclose(S1[h] @ k[h], v[h], rtol=1e-12, atol=1e-12)
    # a key orthogonal to k keeps its image, decayed: S' u = alpha S u for u . k = 0
    u = rng.normal(0, 1, 16)
    u -= (u @ k[0]) * k[0]
    S2, _ = oracle.gdn_step(S, q, k, v, np.full(4, 0.7), np.full(4, 0.3))
    np.testing.assert_allclose(S2[0] @ u, 0.7 * (S[0] @ u), rtol=1e-12, atol=1e-12)


def test_gdn_heads_are_independent():
    S, q, k, v, a, b = _gdn_inputs(np.random.default_rng(4), n=5)
    p = np.array([3, 0, 4, 1, 2])
    S1, o1 = oracle.gdn_step(S, q, k, v, a, b)
    S2, o2 = oracle.gdn_step(S[p], q[p], k[p], v[p], a[p], b[p])
    np.testing.assert_array_equal(S2, S1[p])
    np.testing.assert_array_equal(o2, o1[p])


def _bf16_bits(x):
    return np.array([synth.bf16_from_double(float(v)) for v in np.ravel(x)], np.uint16).reshape(np.shape(x))


def test_attention_single_position_returns_its_value():
    rng = np.random.default_rng(5)
    K, V = _bf16_bits(rng.normal(0, 1, (2, 1, 8))), _bf16_bits(rng.normal(0, 1, (2, 1, 8)))
    o = oracle.attn_decode(rng.normal(0, 1, (4, 8)), K, V)
    for h in range(4):
        np.testing.assert_array_equal(o[h], [bf16_value(b) for b in V[h // 2, 0]])


def test_attention_two_positions_closed_form():
    """d = 4, q = (1, 2, 0, 0), keys (1, 0, 0, 0) and (0, 1, 0, 0): scores 1/2 and 1, so the
    weights are e^0.5 / (e^0.5 + e^1) and e^1 / (e^0.5 + e^1)."""
    q = np.array([[1.0, 2.0, 0.0, 0.0]])
    K = _bf16_bits(np.array([[[1, 0, 0, 0], [0, 1, 0, 0]]], np.float64))
    V = _bf16_bits(np.array([[[2, 0, 0, 1], [0, 4, 0, 1]]], np.float64))
    o = oracle.attn_decode(q, K, V)
    w0, w1 = math.exp(0.5) / (math.exp(0.5) + math.exp(1.0)), math.exp(1.0) / (math.exp(0.5) + math.exp(1.0))
    np.testing.assert_allclose(o[0], [2 * w0, 4 * w1, 0.0, 1.0], rtol=1e-15, atol=1e-15)


def test_attention_uniform_keys_average_the_values_and_gqa_mapping():
    """Equal keys (or q = 0) give uniform weights: o is the mean of V over the positions;
    query heads 0..3 read KV head 0 and heads 4..7 KV head 1."""
    rng = np.random.default_rng(6)
    T, d = 9, 8
    K = _bf16_bits(np.broadcast_to(rng.normal(0, 1, (2, 1, d)), (2, T, d)))
    V = _bf16_bits(rng.normal(0, 1, (2, T, d)))
    Vd = np.vectorize(bf16_value)(V)
    o = oracle.attn_decode(rng.normal(0, 1, (8, d)), K, V)
    for h in range(8):
        np.testing.assert_allclose(o[h], Vd[h // 4].mean(axis=0), rtol=1e-13, atol=1e-13)


def test_attention_positions_are_a_set():
    """Shuffling the cached positions (keys and values together) leaves o unchanged."""
    rng = np.random.default_rng(7)
    T, d = 33, 16
    q = rng.normal(0, 1, (6, d))
    K, V = _bf16_bits(rng.normal(0, 1, (3, T, d))), _bf16_bits(rng.normal(0, 1, (3, T, d)))
    p = rng.permutation(T)
    np.testing.assert_allclose(oracle.attn_decode(q, K[:, p], V[:, p]), oracle.attn_decode(q, K, V),
                               rtol=1e-13, atol=1e-13)
