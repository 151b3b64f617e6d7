"""ctypes binding of the C ABI in include/tel.h (argument marshalling only).

Every function here has the name of the C entry point it wraps and forwards
its arguments unchanged; torch tensors are passed as their device pointers.
A non-OK status raises TelError with the library's message.  The library
must have been built (``python -m transformer_encoder_layer_amd.build``);
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtel.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libtel_debug.so")

TEL_F32, TEL_F16, TEL_BF16 = 0, 1, 2
TEL_OK, TEL_ERR_INVALID_ARG, TEL_ERR_UNSUPPORTED, TEL_ERR_STATE, TEL_ERR_HIP = 0, -1, -2, -3, -4
STATUS_NAMES = {0: "TEL_OK", -1: "TEL_ERR_INVALID_ARG", -2: "TEL_ERR_UNSUPPORTED", -3: "TEL_ERR_STATE",
                -4: "TEL_ERR_HIP"}

PARAM_NAMES = ("w_qkv", "b_qkv", "w_o", "b_o", "ln1_g", "ln1_b",
               "w_1", "b_1", "w_2", "b_2", "ln2_g", "ln2_b")

# every symbol declared in include/tel.h
EXPORTS = ("tel_layer_create", "tel_layer_workspace_bytes", "tel_layer_forward", "tel_layer_forward_noalloc",
           "tel_layer_backward", "tel_layer_backward_chain",
           "tel_layer_set_valid_tokens", "tel_layer_destroy", "tel_last_error", "tel_debug_dropout_mask",
           "tel_debug_kernel_events", "tel_debug_attn_keep_bits", "tel_debug_buffer", "tel_check_key_lengths",
           "tel_debug_checks_enabled", "tel_pld_theta", "tel_pld_keep")

# buffer ids (TEL_BUF_*) of include/tel.h
BUFFERS = {"drop1_in": 0, "drop1_out": 1, "drop2_in": 2, "drop2_out": 3, "attn_keep_bits": 4}

# kernel ids (TEL_K_*) of include/tel.h
KERNELS = {"ln1_fwd": 0, "qkv_fwd": 1, "attn_fwd": 2, "out_fwd": 3, "ln2_fwd": 4, "ffn1_fwd": 5, "ffn2_fwd": 6,
           "ffn2_dgrad": 10, "ffn2_wgrad": 11, "ffn1_dgrad": 12, "ffn1_wgrad": 13, "ln2_bwd": 14,
           "out_dgrad": 15, "out_wgrad": 16, "attn_bwd": 17, "qkv_dgrad": 18, "qkv_wgrad": 19, "ln1_bwd": 20,
           "ffn_wgrad_pair": 21, "attn_wgrad_pair": 22, "ffn_wgrad_reduce": 23, "attn_wgrad_reduce": 24}


class TelError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class tel_config(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("attn_dropout", ctypes.c_float), ("hidden_dropout", ctypes.c_float),
                ("pre_ln", ctypes.c_int32), ("seed", ctypes.c_uint64), ("layer_id", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("ln_eps", ctypes.c_float),
                ("attn_dropout_checkpoint", ctypes.c_int32), ("normalize_invertible", ctypes.c_int32),
                ("gelu_checkpoint", ctypes.c_int32), ("pack_tokens", ctypes.c_int32),
                ("stochastic_mode", ctypes.c_int32)]


class tel_params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in PARAM_NAMES]


class tel_grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in PARAM_NAMES]


_libs = {}


def lib(path: str = LIB_PATH):
    """Load libtel.so (or the debug build at DEBUG_LIB_PATH); raises if it has not been built."""
    if path not in _libs:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m transformer_encoder_layer_amd.build`")
        L = ctypes.CDLL(path)
        vp, i32, u64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
        L.tel_layer_create.argtypes = [ctypes.POINTER(tel_config), ctypes.POINTER(vp)]
        L.tel_layer_workspace_bytes.argtypes = [vp, ctypes.POINTER(sz), ctypes.POINTER(sz)]
        L.tel_layer_forward.argtypes = [vp, ctypes.POINTER(tel_params), vp, vp, ctypes.c_int, u64, vp, vp, vp, vp]
        L.tel_layer_backward.argtypes = [vp, ctypes.POINTER(tel_params), vp, vp, ctypes.c_int, u64, vp, vp, vp,
                                         vp, ctypes.POINTER(tel_grads), vp]
        L.tel_layer_backward_chain.argtypes = [vp, ctypes.POINTER(tel_params), vp, vp, ctypes.c_int, u64, vp, vp,
                                               vp, vp, vp, vp, vp, ctypes.POINTER(tel_grads), vp]
        L.tel_layer_forward_noalloc.argtypes = [vp, ctypes.POINTER(tel_params), vp, vp, vp, vp]
        L.tel_layer_set_valid_tokens.argtypes = [vp, ctypes.c_int64]
        L.tel_layer_destroy.argtypes = [vp]
        L.tel_last_error.argtypes = []
        L.tel_last_error.restype = ctypes.c_char_p
        L.tel_debug_dropout_mask.argtypes = [vp, ctypes.c_int, u64, vp, vp]
        L.tel_debug_kernel_events.argtypes = [vp, ctypes.c_int, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                              ctypes.c_int]
        L.tel_pld_theta.argtypes = [ctypes.c_double] * 3
        L.tel_pld_theta.restype = ctypes.c_double
        L.tel_pld_keep.argtypes = [u64, i32, u64, ctypes.c_double]
        L.tel_pld_keep.restype = i32
        L.tel_debug_attn_keep_bits.argtypes = [vp, vp]
        L.tel_debug_buffer.argtypes = [vp, ctypes.c_int, ctypes.POINTER(sz), ctypes.POINTER(sz),
                                       ctypes.POINTER(ctypes.c_int)]
        L.tel_check_key_lengths.argtypes = [ctypes.POINTER(i32), i32, i32]
        L.tel_debug_checks_enabled.argtypes = []
        L.tel_debug_checks_enabled.restype = i32
        for name in ("tel_layer_create", "tel_layer_workspace_bytes", "tel_layer_forward", "tel_layer_forward_noalloc",
                     "tel_layer_backward", "tel_layer_set_valid_tokens", "tel_layer_destroy",
                     "tel_debug_dropout_mask", "tel_debug_kernel_events", "tel_debug_attn_keep_bits",
                     "tel_debug_buffer", "tel_check_key_lengths"):
            getattr(L, name).restype = ctypes.c_int
        _libs[path] = L
    return _libs[path]


def _check(status: int, L=None):
    if status != TEL_OK:
        raise TelError(status, (L or lib()).tel_last_error().decode(errors="replace"))


def ptr(t):
    """Device pointer of a tensor (or None / int passthrough)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def stream_handle(stream=None):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_params(tensors: dict) -> tel_params:
    return tel_params(*[ptr(tensors[n]) for n in PARAM_NAMES])


def make_grads(tensors: dict) -> tel_grads:
    return tel_grads(*[ptr(tensors[n]) for n in PARAM_NAMES])


def tel_layer_create(cfg: tel_config) -> int:
    h = ctypes.c_void_p()
    _check(lib().tel_layer_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h.value


def tel_layer_workspace_bytes(handle: int):
    s, c = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().tel_layer_workspace_bytes(handle, ctypes.byref(s), ctypes.byref(c)))
    return s.value, c.value


def tel_layer_set_valid_tokens(handle: int, valid_tokens: int):
    _check(lib().tel_layer_set_valid_tokens(handle, int(valid_tokens)))


def tel_layer_forward(handle, params: tel_params, x, key_lengths, training, step, y, saved, scratch, stream=None):
    _check(lib().tel_layer_forward(handle, ctypes.byref(params), ptr(x), ptr(key_lengths), int(training),
                                   int(step), ptr(y), ptr(saved), ptr(scratch), stream_handle(stream)))


def tel_layer_forward_noalloc(handle, params: tel_params, x, key_lengths, y, stream=None):
    _check(lib().tel_layer_forward_noalloc(handle, ctypes.byref(params), ptr(x), ptr(key_lengths), ptr(y),
                                           stream_handle(stream)))


def tel_layer_backward(handle, params: tel_params, x, key_lengths, training, step, dy, saved, scratch, dx,
                       grads: tel_grads, stream=None):
    _check(lib().tel_layer_backward(handle, ctypes.byref(params), ptr(x), ptr(key_lengths), int(training),
                                    int(step), ptr(dy), ptr(saved), ptr(scratch), ptr(dx), ctypes.byref(grads),
                                    stream_handle(stream)))


def tel_layer_backward_chain(handle, params: tel_params, x, key_lengths, training, step, dy, dy_dropped, saved,
                             scratch, dx, below, dx_dropped, grads: tel_grads, stream=None):
    """below: handle of the next layer down, or None (then dx_dropped must be None)."""
    _check(lib().tel_layer_backward_chain(handle, ctypes.byref(params), ptr(x), ptr(key_lengths), int(training),
                                          int(step), ptr(dy), ptr(dy_dropped), ptr(saved), ptr(scratch), ptr(dx),
                                          below, ptr(dx_dropped), ctypes.byref(grads), stream_handle(stream)))


def tel_layer_destroy(handle):
    _check(lib().tel_layer_destroy(handle))


def tel_last_error() -> str:
    return lib().tel_last_error().decode(errors="replace")


def tel_debug_dropout_mask(handle, site, step, out, stream=None):
    _check(lib().tel_debug_dropout_mask(handle, int(site), int(step), ptr(out), stream_handle(stream)))


def tel_debug_kernel_events(handle, kernel_id, start_events, stop_events):
    """start_events / stop_events: sequences of hipEvent_t handles (ints), or None to disable."""
    if kernel_id < 0 or not start_events:
        _check(lib().tel_debug_kernel_events(handle, -1, None, None, 0))
        return None
    n = len(start_events)
    a = (ctypes.c_void_p * n)(*start_events)
    b = (ctypes.c_void_p * n)(*stop_events)
    _check(lib().tel_debug_kernel_events(handle, int(kernel_id), a, b, n))
    return (a, b)  # caller keeps these alive while the hook is on


def tel_debug_attn_keep_bits(handle, out):
    """Arm the keep-bit capture of the next training forward (out: uint32 device tensor, or None to disarm)."""
    _check(lib().tel_debug_attn_keep_bits(handle, ptr(out)))


def tel_debug_buffer(handle, which):
    """(offset, bytes, in_saved) of an internal buffer (which: a BUFFERS name or TEL_BUF_* id)."""
    w = BUFFERS[which] if isinstance(which, str) else int(which)
    off, n, sv = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int()
    _check(lib().tel_debug_buffer(handle, w, ctypes.byref(off), ctypes.byref(n), ctypes.byref(sv)))
    return off.value, n.value, bool(sv.value)


def tel_check_key_lengths(lengths, batch, seq, L=None):
    """Host check of a key-length array (sequence of ints) against [1, seq]."""
    L = L or lib()
    arr = (ctypes.c_int32 * len(lengths))(*[int(v) for v in lengths])
    _check(L.tel_check_key_lengths(arr, int(batch), int(seq)), L)


def tel_debug_checks_enabled(L=None) -> bool:
    return bool((L or lib()).tel_debug_checks_enabled())


def tel_pld_theta(t, theta_bar, gamma) -> float:
    return float(lib().tel_pld_theta(float(t), float(theta_bar), float(gamma)))


def tel_pld_keep(seed, layer_id, step, theta) -> bool:
    return bool(lib().tel_pld_keep(int(seed), int(layer_id), int(step), float(theta)))
