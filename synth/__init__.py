"""Seeded synthetic workload for the MoE decode layer (inputs only).

Thin ctypes binding over ``libsynth.so`` (built from ``synth.c``).  Everything
here is input generation: canonical quantized expert tensors, router weights,
token activations and the Zipf logit prior.  No routing, dequantization or FFN
arithmetic lives here, so both the GPU library's tests/bench and the oracle can
consume the same bytes without sharing any of the method's code.

Canonical expert format (one expert; groups of ``group`` run along each row):
  gate_codes [I][H*bits/8], up_codes [I][H*bits/8], down_codes [H][I*bits/8]
  (4-bit: element 2j is the low nibble of byte j; 2-bit: element 4j+t sits at
  bits 2t..2t+1 of byte j; 3-bit: a row is one little-endian bit string with
  element c at bits 3c..3c+2; the codes are uniform random bits for any width),
  scales/biases: bf16 bit patterns, concatenated
  gate [I][H/group] | up [I][H/group] | down [H][I/group].
"""
import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

SCALE_STD = 0.02
BIAS_STD = 0.01


def build(verbose=False):
    """Compile libsynth.so in place (gcc, OpenMP)."""
    import subprocess
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
           os.path.join(_HERE, "synth.c"), "-o", _LIB_PATH + ".tmp", "-lm"]
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
        u64, i64, i32, sz, dbl = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int,
                                  ctypes.c_size_t, ctypes.c_double)
        vp = ctypes.c_void_p
        L.synth_stream_key.restype = u64
        L.synth_stream_key.argtypes = [u64, i64, i64, i64]
        L.synth_bf16_from_double.restype = ctypes.c_uint16
        L.synth_bf16_from_double.argtypes = [dbl]
        L.synth_bytes.argtypes = [u64, sz, vp]
        L.synth_normal_f64.argtypes = [u64, sz, dbl, dbl, vp]
        L.synth_normal_f32.argtypes = [u64, sz, dbl, dbl, vp]
        L.synth_normal_bf16.argtypes = [u64, sz, dbl, dbl, i32, vp]
        L.synth_expert.argtypes = [u64, i64, i64, i32, i32, i32, i32, dbl, dbl, vp, vp, vp, vp, vp]
        L.synth_experts.argtypes = [u64, i64, i64, i32, i32, i32, i32, i32, dbl, dbl, vp, vp, vp, vp, vp]
        L.synth_router.argtypes = [u64, i64, i32, i32, vp]
        L.synth_tokens.argtypes = [u64, i64, i32, i32, vp]
        L.synth_zipf_bias.argtypes = [i32, dbl, vp]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


@dataclass
class Canonical:
    """Stacked canonical tensors for ``n`` consecutive experts."""
    bits: int
    H: int
    I: int
    group: int
    gate: np.ndarray    # uint8 [n][I][H*bits/8]
    up: np.ndarray      # uint8 [n][I][H*bits/8]
    down: np.ndarray    # uint8 [n][H][I*bits/8]
    scales: np.ndarray  # uint16 [n][ng]
    biases: np.ndarray  # uint16 [n][ng]

    @property
    def n(self):
        return self.gate.shape[0]

    def expert(self, j):
        return Canonical(self.bits, self.H, self.I, self.group, self.gate[j:j + 1], self.up[j:j + 1],
                         self.down[j:j + 1], self.scales[j:j + 1], self.biases[j:j + 1])


def n_groups(H, I, group=64):
    return I * (H // group) * 2 + H * (I // group)


def empty_canonical(n, bits, H, I, group=64):
    ng = n_groups(H, I, group)
    return Canonical(bits, H, I, group,
                     np.empty((n, I, H * bits // 8), np.uint8), np.empty((n, I, H * bits // 8), np.uint8),
                     np.empty((n, H, I * bits // 8), np.uint8), np.empty((n, ng), np.uint16),
                     np.empty((n, ng), np.uint16))


def experts(seed, layer, first, n, bits, H, I, group=64, out=None):
    """Generate experts [first, first+n) of one layer (expert id E is the shared expert)."""
    c = out if out is not None else empty_canonical(n, bits, H, I, group)
    lib().synth_experts(seed, layer, first, n, bits, H, I, group, SCALE_STD, BIAS_STD,
                        _ptr(c.gate), _ptr(c.up), _ptr(c.down), _ptr(c.scales), _ptr(c.biases))
    return c


def router(seed, layer, E, H):
    w = np.empty((E, H), np.float32)
    lib().synth_router(seed, layer, E, H, _ptr(w))
    return w


def tokens(seed, step, B, H):
    x = np.empty((B, H), np.float32)
    lib().synth_tokens(seed, step, B, H, _ptr(x))
    return x


def zipf_bias(E, s=1.1):
    b = np.empty(E, np.float32)
    lib().synth_zipf_bias(E, s, _ptr(b))
    return b


def uniform_bytes(key, n):
    out = np.empty(n, np.uint8)
    lib().synth_bytes(key, n, _ptr(out))
    return out


def normals_f64(key, n, mean=0.0, std=1.0):
    out = np.empty(n, np.float64)
    lib().synth_normal_f64(key, n, mean, std, _ptr(out))
    return out


def bf16_from_double(d):
    return int(lib().synth_bf16_from_double(float(d)))


def stream_key(seed, layer, expert, tensor):
    return int(lib().synth_stream_key(seed, layer, expert, tensor))
