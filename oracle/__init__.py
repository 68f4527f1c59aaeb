"""Float64 CPU oracle of the quantized MoE decode layer (ctypes over liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product library.  The arithmetic
lives in ``oracle.c``; this module only marshals numpy arrays.

Expert tensors are passed as any object with attributes ``gate``, ``up``,
``down``, ``scales``, ``biases`` (uint8 / uint16 numpy arrays stacked over
experts, canonical format), or as a mapping {expert_id: such an object holding
one expert} when only some experts are available (e.g. the active ones at full
size).  Expert id E is the shared expert.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose=False):
    import subprocess
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
           os.path.join(_HERE, "oracle.c"), "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        i32, dbl, vp, lng = ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_long
        L.oracle_code_at.restype = i32
        L.oracle_code_at.argtypes = [vp, i32, lng]
        L.oracle_bf16_to_double.restype = dbl
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_dequant_matrix.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp]
        L.oracle_router_logits.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.oracle_topk.restype = i32
        L.oracle_topk.argtypes = [i32, i32, vp, i32, vp, vp, vp]
        L.oracle_expert_ffn.restype = i32
        L.oracle_expert_ffn.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_layer_decode.restype = i32
        L.oracle_layer_decode.argtypes = [i32, i32, i32, i32, i32, i32, i32, dbl, vp, i32, vp, vp,
                                          vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_layer_decode_par.restype = i32
        L.oracle_layer_decode_par.argtypes = list(L.oracle_layer_decode.argtypes)
        L.oracle_layer_decode_mt.restype = i32
        L.oracle_layer_decode_mt.argtypes = [i32, i32, i32, i32, i32, i32, i32, dbl, vp, vp, vp,
                                             vp, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_group_by_expert.restype = i32
        L.oracle_group_by_expert.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.oracle_rms_renorm.argtypes = [i32, vp, dbl, vp]
        L.oracle_bf16_round.restype = ctypes.c_uint16
        L.oracle_bf16_round.argtypes = [dbl]
        L.oracle_requant_group.argtypes = [i32, vp, ctypes.c_uint16, ctypes.c_uint16, vp, vp, vp]
        L.oracle_requant_expert.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_gdn_step.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_attn_decode.restype = i32
        L.oracle_attn_decode.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def code_at(row_bytes, bits, c):
    row = _c(row_bytes, np.uint8)
    return lib().oracle_code_at(_p(row), bits, c)


def bf16_to_double(b):
    return lib().oracle_bf16_to_double(int(b))


def dequant_matrix(bits, rows, cols, codes, scales, biases, group=64):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint16)
    biases = _c(biases, np.uint16)
    W = np.empty((rows, cols), np.float64)
    lib().oracle_dequant_matrix(bits, rows, cols, group, _p(codes), _p(scales), _p(biases), _p(W))
    return W


def dequant_expert(bits, H, I, gate, up, down, scales, biases, group=64):
    """Dense (Wg [I][H], Wu [I][H], Wd [H][I]) of one canonical expert."""
    ngu = I * (H // group)
    s = _c(scales, np.uint16).reshape(-1)
    b = _c(biases, np.uint16).reshape(-1)
    Wg = dequant_matrix(bits, I, H, gate, s[:ngu], b[:ngu], group)
    Wu = dequant_matrix(bits, I, H, up, s[ngu:2 * ngu], b[ngu:2 * ngu], group)
    Wd = dequant_matrix(bits, H, I, down, s[2 * ngu:], b[2 * ngu:], group)
    return Wg, Wu, Wd


def router_logits(x, Wr, prior=None):
    x = _c(np.atleast_2d(x), np.float32)
    Wr = _c(Wr, np.float32)
    B, H = x.shape
    E = Wr.shape[0]
    pr = None if prior is None else _c(prior, np.float32)
    out = np.empty((B, E), np.float64)
    lib().oracle_router_logits(B, H, E, _p(x), _p(Wr), _p(pr), _p(out))
    return out


def topk(logits, K, renormalize=True):
    """(idx int32 [K], w float64 [K], margin) of one token's logits."""
    lg = _c(logits, np.float64)
    E = lg.shape[0]
    idx = np.empty(K, np.int32)
    w = np.empty(K, np.float64)
    m = np.empty(1, np.float64)
    rc = lib().oracle_topk(E, K, _p(lg), int(bool(renormalize)), _p(idx), _p(w), _p(m))
    if rc != 0:
        raise ValueError("oracle_topk: bad arguments")
    return idx, w, float(m[0])


def expert_ffn(bits, H, I, gate, up, down, scales, biases, x, group=64):
    """(h [I], y [H]) of one expert on one token, float64."""
    xd = _c(x, np.float64).reshape(-1)
    h = np.empty(I, np.float64)
    y = np.empty(H, np.float64)
    args = [_c(a, t) for a, t in ((gate, np.uint8), (up, np.uint8), (down, np.uint8),
                                   (scales, np.uint16), (biases, np.uint16))]
    rc = lib().oracle_expert_ffn(bits, H, I, group, *[_p(a) for a in args], _p(xd), _p(h), _p(y))
    if rc != 0:
        raise MemoryError("oracle_expert_ffn")
    return h, y


class _Table:
    """Per-expert pointer arrays for the C expert table (keeps arrays alive)."""

    def __init__(self, experts, E):
        n = E + 1
        self.keep = []
        self.ptrs = {f: (ctypes.c_void_p * n)() for f in ("gate", "up", "down", "scales", "biases")}
        if isinstance(experts, dict):
            for e, ex in experts.items():
                self._set(e, ex, 0)
        else:
            for e in range(min(n, experts.gate.shape[0])):
                self._set(e, experts, e)

    def _set(self, e, ex, j):
        for f, t in (("gate", np.uint8), ("up", np.uint8), ("down", np.uint8),
                     ("scales", np.uint16), ("biases", np.uint16)):
            arr = getattr(ex, f)
            a = _c(arr[j], t)
            self.keep.append(a)
            self.ptrs[f][e] = a.ctypes.data

    def args(self):
        return [ctypes.cast(self.ptrs[f], ctypes.c_void_p)
                for f in ("gate", "up", "down", "scales", "biases")]


def layer_decode(bits, H, I, E, K, x, Wr, experts, prior=None, renormalize=True,
                 shared_weight=1.0, group=64, parallel=False):
    """Decode B tokens through one layer.

    parallel=True spreads the tokens over OpenMP threads (oracle_layer_decode_par:
    each token decoded by the serial function on its own, so the results are the
    serial ones bit for bit).
    Returns (y float64 [B][H], idx int32 [B][K], w float64 [B][K], margin [B]).
    """
    x = _c(np.atleast_2d(x), np.float32)
    B = x.shape[0]
    Wr = _c(Wr, np.float32)
    pr = None if prior is None else _c(prior, np.float32)
    t = _Table(experts, E)
    y = np.empty((B, H), np.float64)
    idx = np.empty((B, K), np.int32)
    w = np.empty((B, K), np.float64)
    m = np.empty(B, np.float64)
    fn = lib().oracle_layer_decode_par if parallel else lib().oracle_layer_decode
    rc = fn(bits, H, I, E, K, group, int(bool(renormalize)), shared_weight,
            _p(x), B, _p(Wr), _p(pr), *t.args(), _p(y), _p(idx), _p(w), _p(m))
    if rc == -2:
        raise KeyError("oracle_layer_decode: a selected expert was not provided")
    if rc != 0:
        raise RuntimeError("oracle_layer_decode failed (%d)" % rc)
    return y, idx, w, m


def layer_decode_mt(bits, H, I, E, K, x, Wr, experts, prior=None, renormalize=True,
                    shared_weight=1.0, group=64):
    """One token, expert FFNs spread over OpenMP threads (CPU baseline timing)."""
    x = _c(np.asarray(x).reshape(-1), np.float32)
    Wr = _c(Wr, np.float32)
    pr = None if prior is None else _c(prior, np.float32)
    t = _Table(experts, E)
    y = np.empty(H, np.float64)
    idx = np.empty(K, np.int32)
    w = np.empty(K, np.float64)
    rc = lib().oracle_layer_decode_mt(bits, H, I, E, K, group, int(bool(renormalize)), shared_weight,
                                      _p(x), _p(Wr), _p(pr), *t.args(), _p(y), _p(idx), _p(w))
    if rc != 0:
        raise RuntimeError("oracle_layer_decode_mt failed (%d)" % rc)
    return y, idx, w


def group_by_expert(idx, E):
    """(offsets [E+1], tokens [B*K], slots [B*K], U) of a [B][K] selection."""
    idx = _c(idx, np.int32)
    B, K = idx.shape
    off = np.empty(E + 1, np.int32)
    tok = np.empty(B * K, np.int32)
    sl = np.empty(B * K, np.int32)
    U = lib().oracle_group_by_expert(B, K, E, _p(idx), _p(off), _p(tok), _p(sl))
    return off, tok, sl, U


def rms_renorm(y, eps=1e-6):
    y = _c(y, np.float64).reshape(-1)
    x = np.empty_like(y)
    lib().oracle_rms_renorm(y.shape[0], _p(y), eps, _p(x))
    return x


def bf16_round(v):
    """Bit pattern of the nearest bf16 value of a double (ties to even)."""
    return int(lib().oracle_bf16_round(float(v)))


def requant_group(q4, s4, b4):
    """(q2 [n], s2 bits, b2 bits) of one group of 4-bit codes with bf16 bit patterns s4, b4."""
    q4 = _c(q4, np.int32)
    q2 = np.empty_like(q4)
    s2 = np.zeros(1, np.uint16)
    b2 = np.zeros(1, np.uint16)
    lib().oracle_requant_group(q4.shape[0], _p(q4), int(s4), int(b4), _p(q2), _p(s2), _p(b2))
    return q2, int(s2[0]), int(b2[0])


def requant_expert(H, I, gate, up, down, scales, biases, group=64):
    """Canonical 4-bit expert -> canonical 2-bit expert: (gate2, up2, down2, scales2, biases2)."""
    g4, u4, d4 = _c(gate, np.uint8), _c(up, np.uint8), _c(down, np.uint8)
    s4, b4 = _c(scales, np.uint16).reshape(-1), _c(biases, np.uint16).reshape(-1)
    g2 = np.empty((I, H // 4), np.uint8)
    u2 = np.empty((I, H // 4), np.uint8)
    d2 = np.empty((H, I // 4), np.uint8)
    s2 = np.empty_like(s4)
    b2 = np.empty_like(b4)
    lib().oracle_requant_expert(H, I, group, _p(g4), _p(u4), _p(d4), _p(s4), _p(b4), _p(g2), _p(u2), _p(d2),
                                _p(s2), _p(b2))
    return g2, u2, d2, s2, b2


def gdn_step(S, q, k, v, alpha, beta):
    """One gated-delta-rule step: (S' [n][dv][dk], o [n][dv]) in float64 (S is not modified)."""
    S = np.array(S, np.float64, copy=True)
    n, dv, dk = S.shape
    q, k = _c(q, np.float64).reshape(n, dk), _c(k, np.float64).reshape(n, dk)
    v = _c(v, np.float64).reshape(n, dv)
    a, b = _c(alpha, np.float64).reshape(n), _c(beta, np.float64).reshape(n)
    o = np.empty((n, dv), np.float64)
    lib().oracle_gdn_step(n, dk, dv, _p(S), _p(q), _p(k), _p(v), _p(a), _p(b), _p(o))
    return S, o


def attn_decode(q, K, V):
    """One grouped-query attention decode step: q [n_q][d] float, K, V bf16 bits [n_kv][T][d] -> o [n_q][d]."""
    q = _c(q, np.float64)
    K, V = _c(K, np.uint16), _c(V, np.uint16)
    n_q, d = q.shape
    n_kv, T, _ = K.shape
    o = np.empty((n_q, d), np.float64)
    if lib().oracle_attn_decode(n_q, n_kv, d, T, _p(q), _p(K), _p(V), _p(o)) != 0:
        raise ValueError("oracle_attn_decode: bad shape")
    return o

