"""Python binding of libmoe.so: quantized MoE decode on AMD Instinct MI355X (gfx950).

Argument marshalling only.  Every step of the decode path runs in the HIP
kernels behind the C ABI declared in ``include/moe.h``; this module turns torch
tensors (device memory allocated by PyTorch) into pointers and passes the
current HIP stream.  There is no CPU fallback: if ``libmoe.so`` is missing the
import of any entry point raises.
"""
import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "moe.h")

MOE_OK = 0
MOE_EINVAL = -1
MOE_EUNSUPPORTED = -2
MOE_EHIP = -3
MOE_MAX_K = 32      # largest top-K (include/moe.h)
MOE_MAX_E = 1024    # most routed experts
MOE_MAX_B = 256     # most tokens per call
MOE_NOALLOC_SCRATCH_BYTES = 8 << 20  # scratch of moe_layer_decode_noalloc per GPU
MOE_MAX_CACHE_SLOTS = 65536  # most slots of an expert cache

KERNEL_ROUTER = 1
KERNEL_GATEUP = 2
KERNEL_DOWN = 3


class MoeError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (code %d)" % (msg, code))
        self.code = code


class ExpertCache(ctypes.Structure):
    """moe_expert_cache (include/moe.h)."""
    _fields_ = [("slots", ctypes.c_int32), ("slab", ctypes.c_void_p), ("state", ctypes.c_void_p)]


class LayerDesc(ctypes.Structure):
    """moe_layer_desc (include/moe.h)."""
    _fields_ = [("H", ctypes.c_int32), ("I", ctypes.c_int32), ("E", ctypes.c_int32),
                ("K", ctypes.c_int32), ("bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("experts", ctypes.c_void_p), ("w_router", ctypes.c_void_p),
                ("logit_bias", ctypes.c_void_p), ("shared_weight", ctypes.c_float),
                ("renormalize", ctypes.c_int32), ("expert_flags", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe.so is not built (%s); run `python -m quantized_expert_dequant_amd.build`"
                               % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        i32, sz, vp, f32 = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
        dp = ctypes.POINTER(LayerDesc)
        sig = {
            "moe_expert_record_bytes": (sz, [i32, i32, i32, i32]),
            "moe_workspace_bytes": (sz, [dp, i32]),
            "moe_route_workspace_bytes": (sz, [i32, i32, i32]),
            "moe_stack_extra_bytes": (sz, [i32, i32]),
            "moe_pack_experts": (i32, [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp]),
            "moe_dequant_expert": (i32, [i32, i32, i32, i32, vp, vp, vp]),
            "moe_expert_ranges": (i32, [i32, i32, i32, i32, vp, i32, vp, vp]),
            "moe_gdn_step": (i32, [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]),
            "moe_attn_workspace_bytes": (sz, [i32, i32, i32, i32]),
            "moe_attn_decode": (i32, [i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
            "moe_requant_4to2": (i32, [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
            "moe_route_topk": (i32, [vp, i32, vp, vp, i32, i32, i32, i32, vp, vp, vp, sz, vp]),
            "moe_expert_ffn_q4": (i32, [dp, vp, i32, vp, vp, vp, vp, sz, vp]),
            "moe_expert_ffn_q2": (i32, [dp, vp, i32, vp, vp, vp, vp, sz, vp]),
            "moe_expert_ffn_q3": (i32, [dp, vp, i32, vp, vp, vp, vp, sz, vp]),
            "moe_layer_decode": (i32, [dp, vp, i32, vp, vp, vp, vp, sz, vp]),
            "moe_layer_decode_noalloc": (i32, [dp, vp, i32, vp, vp, vp, vp]),
            "moe_group_tokens": (i32, [vp, i32, i32, i32, vp, vp, vp, vp]),
            "moe_rmsnorm": (i32, [vp, i32, i32, f32, vp, vp]),
            "moe_stack_decode": (i32, [dp, i32, vp, i32, f32, vp, vp, vp, vp, sz, vp]),
            "moe_set_timing_events": (i32, [i32, vp, vp]),
            "moe_grouped_launch_info": (i32, [dp, i32, vp]),
            "moe_cache_state_bytes": (sz, [i32, i32]),
            "moe_cache_init": (i32, [dp, ctypes.POINTER(ExpertCache), vp]),
            "moe_cache_workspace_bytes": (sz, [dp, i32, i32]),
            "moe_layer_decode_cached": (i32, [dp, ctypes.POINTER(ExpertCache), vp, i32, vp, vp, vp, vp, sz, vp]),
            "moe_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def declared_functions():
    """Names of the functions include/moe.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def last_error():
    return lib().moe_last_error().decode()


def _check(rc):
    if rc != MOE_OK:
        raise MoeError(rc, last_error())
    return rc


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def make_desc(H, I, E, K, bits, experts, w_router, logit_bias=None, shared_weight=1.0, renormalize=True, group=64,
              expert_flags=None):
    return LayerDesc(H, I, E, K, bits, group, _p(experts), _p(w_router), _p(logit_bias), float(shared_weight),
                     int(bool(renormalize)), _p(expert_flags))


def record_bytes(bits, H, I, group=64):
    return lib().moe_expert_record_bytes(bits, H, I, group)


def workspace_bytes(desc, B):
    return lib().moe_workspace_bytes(ctypes.byref(desc), B)


def route_workspace_bytes(B, E, K):
    return lib().moe_route_workspace_bytes(B, E, K)


def stack_extra_bytes(B, H):
    return lib().moe_stack_extra_bytes(B, H)


def pack_experts(bits, H, I, n, gate, up, down, scales, biases, slab, first, stream=None, group=64):
    return _check(lib().moe_pack_experts(bits, H, I, group, n, _p(gate), _p(up), _p(down), _p(scales), _p(biases),
                                         _p(slab), first, _stream(stream)))


def requant_4to2(H, I, n, gate4, up4, down4, scales4, biases4, gate2, up2, down2, scales2, biases2, stream=None,
                 group=64):
    return _check(lib().moe_requant_4to2(H, I, group, n, _p(gate4), _p(up4), _p(down4), _p(scales4), _p(biases4),
                                         _p(gate2), _p(up2), _p(down2), _p(scales2), _p(biases2), _stream(stream)))


def expert_ranges(bits, H, I, slab, n, flags_out, stream=None, group=64):
    return _check(lib().moe_expert_ranges(bits, H, I, group, _p(slab), n, _p(flags_out), _stream(stream)))


def gdn_step(n_heads, dk, dv, state, q, k, v, alpha, beta, o_out, stream=None):
    return _check(lib().moe_gdn_step(n_heads, dk, dv, _p(state), _p(q), _p(k), _p(v), _p(alpha), _p(beta), _p(o_out),
                                     _stream(stream)))


def attn_workspace_bytes(n_q, n_kv, d, T):
    return lib().moe_attn_workspace_bytes(n_q, n_kv, d, T)


def attn_decode(n_q, n_kv, d, T, q, K, V, o_out, ws, ws_bytes, stream=None):
    return _check(lib().moe_attn_decode(n_q, n_kv, d, T, _p(q), _p(K), _p(V), _p(o_out), _p(ws), ws_bytes,
                                        _stream(stream)))


def dequant_expert(bits, H, I, record, W_out, stream=None, group=64):
    return _check(lib().moe_dequant_expert(bits, H, I, group, _p(record), _p(W_out), _stream(stream)))


def route_topk(x, B, w_router, logit_bias, H, E, K, idx_out, w_out, ws, ws_bytes, renormalize=True, stream=None):
    return _check(lib().moe_route_topk(_p(x), B, _p(w_router), _p(logit_bias), H, E, K, int(bool(renormalize)),
                                       _p(idx_out), _p(w_out), _p(ws), ws_bytes, _stream(stream)))


def expert_ffn(desc, x, B, idx, w, y_out, ws, ws_bytes, stream=None):
    fn = {4: lib().moe_expert_ffn_q4, 3: lib().moe_expert_ffn_q3}.get(desc.bits, lib().moe_expert_ffn_q2)
    return _check(fn(ctypes.byref(desc), _p(x), B, _p(idx), _p(w), _p(y_out), _p(ws), ws_bytes, _stream(stream)))


def expert_ffn_q4(desc, x, B, idx, w, y_out, ws, ws_bytes, stream=None):
    return _check(lib().moe_expert_ffn_q4(ctypes.byref(desc), _p(x), B, _p(idx), _p(w), _p(y_out), _p(ws),
                                          ws_bytes, _stream(stream)))


def expert_ffn_q2(desc, x, B, idx, w, y_out, ws, ws_bytes, stream=None):
    return _check(lib().moe_expert_ffn_q2(ctypes.byref(desc), _p(x), B, _p(idx), _p(w), _p(y_out), _p(ws),
                                          ws_bytes, _stream(stream)))


def expert_ffn_q3(desc, x, B, idx, w, y_out, ws, ws_bytes, stream=None):
    return _check(lib().moe_expert_ffn_q3(ctypes.byref(desc), _p(x), B, _p(idx), _p(w), _p(y_out), _p(ws),
                                          ws_bytes, _stream(stream)))


def layer_decode(desc, x, B, y_out, idx_out, w_out, ws, ws_bytes, stream=None):
    return _check(lib().moe_layer_decode(ctypes.byref(desc), _p(x), B, _p(y_out), _p(idx_out), _p(w_out), _p(ws),
                                         ws_bytes, _stream(stream)))


def layer_decode_noalloc(desc, x, B, y_out, idx_out, w_out, stream=None):
    return _check(lib().moe_layer_decode_noalloc(ctypes.byref(desc), _p(x), B, _p(y_out), _p(idx_out), _p(w_out),
                                                 _stream(stream)))


def group_tokens(idx, B, K, E, offsets_out, tokens_out, slots_out, stream=None):
    return _check(lib().moe_group_tokens(_p(idx), B, K, E, _p(offsets_out), _p(tokens_out), _p(slots_out),
                                         _stream(stream)))


def rmsnorm(y, B, H, eps, x_out, stream=None):
    return _check(lib().moe_rmsnorm(_p(y), B, H, eps, _p(x_out), _stream(stream)))


def stack_decode(descs, x, B, eps, y_out, idx_out, w_out, ws, ws_bytes, stream=None):
    arr = (LayerDesc * len(descs))(*descs)
    return _check(lib().moe_stack_decode(arr, len(descs), _p(x), B, eps, _p(y_out), _p(idx_out), _p(w_out), _p(ws),
                                         ws_bytes, _stream(stream)))


def grouped_launch_info(desc, B):
    """Launch shape of the batched path (dict); see moe_grouped_launch_info."""
    info = (ctypes.c_int32 * 8)()
    _check(lib().moe_grouped_launch_info(ctypes.byref(desc), B, info))
    keys = ("grouped", "gateup_blocks", "gateup_tiles_per_group", "gateup_k_chunks", "down_blocks",
            "down_tiles_per_group", "gemv_below_tokens", "group_tokens")
    return dict(zip(keys, list(info)))


def make_cache(slots, slab, state):
    return ExpertCache(slots, _p(slab), _p(state))


def cache_state_bytes(E, slots):
    return lib().moe_cache_state_bytes(E, slots)


def cache_workspace_bytes(desc, slots, B):
    return lib().moe_cache_workspace_bytes(ctypes.byref(desc), slots, B)


def cache_init(desc, cache, stream=None):
    return _check(lib().moe_cache_init(ctypes.byref(desc), ctypes.byref(cache), _stream(stream)))


def layer_decode_cached(desc, cache, x, B, y_out, idx_out, w_out, ws, ws_bytes, stream=None):
    return _check(lib().moe_layer_decode_cached(ctypes.byref(desc), ctypes.byref(cache), _p(x), B, _p(y_out),
                                                _p(idx_out), _p(w_out), _p(ws), ws_bytes, _stream(stream)))


def set_timing_events(kernel, start_event, stop_event):
    """Record raw hipEvent_t handles (ints) around every launch of `kernel`; None, None clears."""
    return _check(lib().moe_set_timing_events(kernel, start_event, stop_event))
