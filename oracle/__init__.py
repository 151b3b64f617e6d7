"""fp64 CPU oracle of one Transformer encoder layer -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It loads ``liboracle.so`` built from ``oracle.c`` (plain
C, fp64 loops, OpenMP) and wraps it with numpy arrays.  It imports nothing
from the GPU package and the GPU package imports nothing from it.

What each function computes, and which page passage it follows, is stated in
``oracle.c``.  Pins (tests that tie the oracle to something other than itself)
live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

PARAM_NAMES = ("w_qkv", "b_qkv", "w_o", "b_o", "ln1_g", "ln1_b",
               "w_1", "b_1", "w_2", "b_2", "ln2_g", "ln2_b")

_DP = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (fp64, -O2, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                        "-Wall", "-Wno-unknown-pragmas", _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("ffn", ctypes.c_int32), ("pre_ln", ctypes.c_int32),
                ("training", ctypes.c_int32), ("batch_offset", ctypes.c_int32),
                ("attn_p", ctypes.c_double), ("hidden_p", ctypes.c_double), ("ln_eps", ctypes.c_double),
                ("seed", ctypes.c_uint64), ("step", ctypes.c_uint64),
                ("layer_id", ctypes.c_int32), ("pad_", ctypes.c_int32)]


class _Params(ctypes.Structure):
    _fields_ = [(n, _DP) for n in PARAM_NAMES]


_ACT_NAMES = ("qkv", "ctx", "lse", "attn_proj", "ln1_in", "ln1_out", "mu1", "rstd1",
              "u", "g", "ffn_out", "ln2_in", "ln2_out", "mu2", "rstd2")


class _Acts(ctypes.Structure):
    _fields_ = [(n, _DP) for n in _ACT_NAMES]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        L.orc_philox4x32_10.argtypes = [ctypes.POINTER(ctypes.c_uint32)] * 3
        L.orc_dropout_mask.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64,
                                       ctypes.c_double, ctypes.c_uint64, ctypes.c_uint64,
                                       ctypes.POINTER(ctypes.c_uint8)]
        L.orc_drop_threshold.argtypes = [ctypes.c_double]
        L.orc_drop_threshold.restype = ctypes.c_uint64
        L.orc_omp_threads.argtypes = []
        L.orc_omp_threads.restype = ctypes.c_int
        L.orc_pld_theta.argtypes = [ctypes.c_double] * 3
        L.orc_pld_theta.restype = ctypes.c_double
        L.orc_pld_keep.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_uint64, ctypes.c_double]
        L.orc_pld_keep.restype = ctypes.c_int
        L.orc_gelu.argtypes = [ctypes.c_double]
        L.orc_gelu.restype = ctypes.c_double
        L.orc_gelu_grad.argtypes = [ctypes.c_double]
        L.orc_gelu_grad.restype = ctypes.c_double
        L.orc_ln_forward.argtypes = [ctypes.c_int, ctypes.c_int, _DP, _DP, _DP, ctypes.c_double, _DP, _DP, _DP]
        L.orc_ln_backward.argtypes = [ctypes.c_int, ctypes.c_int, _DP, _DP, ctypes.c_int, _DP, _DP, _DP, _DP,
                                      _DP, _DP, _DP]
        L.orc_attention_forward.argtypes = [ctypes.POINTER(_Cfg), _DP, ctypes.POINTER(ctypes.c_int32),
                                            _DP, _DP, _DP]
        L.orc_layer_forward.argtypes = [ctypes.POINTER(_Cfg), ctypes.POINTER(_Params), _DP,
                                        ctypes.POINTER(ctypes.c_int32), _DP, ctypes.POINTER(_Acts)]
        L.orc_layer_backward.argtypes = [ctypes.POINTER(_Cfg), ctypes.POINTER(_Params), _DP,
                                         ctypes.POINTER(ctypes.c_int32), _DP, ctypes.c_int, _DP,
                                         ctypes.POINTER(_Params), _DP]
        _lib = L
    return _lib


def _dp(a):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_DP)


@dataclass
class LayerCfg:
    batch: int
    seq: int
    hidden: int
    heads: int
    ffn: int
    pre_ln: bool = True
    training: bool = True
    attn_p: float = 0.0
    hidden_p: float = 0.0
    ln_eps: float = 1e-12
    seed: int = 0
    step: int = 0
    layer_id: int = 0
    batch_offset: int = 0

    def c(self) -> _Cfg:
        return _Cfg(self.batch, self.seq, self.hidden, self.heads, self.ffn, int(self.pre_ln),
                    int(self.training), self.batch_offset, float(self.attn_p), float(self.hidden_p),
                    float(self.ln_eps), self.seed, self.step, self.layer_id, 0)


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def philox4x32_10(ctr, key):
    c = (ctypes.c_uint32 * 4)(*[int(v) & 0xFFFFFFFF for v in ctr])
    k = (ctypes.c_uint32 * 2)(*[int(v) & 0xFFFFFFFF for v in key])
    o = (ctypes.c_uint32 * 4)()
    lib().orc_philox4x32_10(c, k, o)
    return [int(v) for v in o]


def dropout_mask(seed, layer, site, step, p, e0, n):
    out = np.empty(n, dtype=np.uint8)
    lib().orc_dropout_mask(seed, layer, site, step, float(p), e0, n,
                           out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)))
    return out


def drop_threshold(p):
    return int(lib().orc_drop_threshold(float(p)))


def omp_threads():
    """Threads the oracle's OpenMP regions run with."""
    return int(lib().orc_omp_threads())


def pld_theta(t, theta_bar=0.5, gamma=0.001):
    return float(lib().orc_pld_theta(float(t), float(theta_bar), float(gamma)))


def pld_keep(seed, layer, step, theta):
    return bool(lib().orc_pld_keep(seed, layer, step, float(theta)))


def gelu(u):
    return float(lib().orc_gelu(float(u)))


def gelu_grad(u):
    return float(lib().orc_gelu_grad(float(u)))


def ln_forward(x, gamma, beta, eps=1e-12):
    x = _f64(x)
    T, H = x.shape
    y = np.empty_like(x)
    mu = np.empty(T)
    rstd = np.empty(T)
    lib().orc_ln_forward(T, H, _dp(x), _dp(_f64(gamma)), _dp(_f64(beta)), eps, _dp(y), _dp(mu), _dp(rstd))
    return y, mu, rstd


def ln_backward(dy, src, from_output, mu, rstd, gamma, beta):
    dy = _f64(dy)
    T, H = dy.shape
    dx = np.empty_like(dy)
    dg = np.empty(H)
    db = np.empty(H)
    lib().orc_ln_backward(T, H, _dp(dy), _dp(_f64(src)), int(from_output), _dp(_f64(mu)), _dp(_f64(rstd)),
                          _dp(_f64(gamma)), _dp(_f64(beta)), _dp(dx), _dp(dg), _dp(db))
    return dx, dg, db


def attention_forward(cfg: LayerCfg, qkv, lengths, want_probs=False):
    qkv = _f64(qkv)
    B, S, H, N = cfg.batch, cfg.seq, cfg.hidden, cfg.heads
    ctx = np.empty((B * S, H))
    lse = np.empty((B, N, S))
    P = np.empty((B, N, S, S)) if want_probs else None
    ln = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32))
    c = cfg.c()
    lib().orc_attention_forward(ctypes.byref(c), _dp(qkv), ln.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                _dp(ctx), _dp(lse), _dp(P))
    return ctx, lse, P


def _params_struct(params, keep):
    arrs = {n: _f64(params[n]) for n in PARAM_NAMES}
    keep.extend(arrs.values())
    return _Params(*[_dp(arrs[n]) for n in PARAM_NAMES])


def layer_forward(cfg: LayerCfg, params: dict, x, lengths, want_acts=False):
    """Returns (y, acts) with y [T,H] fp64 and acts a dict of intermediates (or None)."""
    keep = []
    P = _params_struct(params, keep)
    x = _f64(x).reshape(cfg.batch * cfg.seq, cfg.hidden)
    T, H, F = cfg.batch * cfg.seq, cfg.hidden, cfg.ffn
    y = np.empty((T, H))
    ln = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32))
    acts = None
    ap = None
    if want_acts:
        shapes = {"qkv": (T, 3 * H), "ctx": (T, H), "lse": (cfg.batch, cfg.heads, cfg.seq),
                  "attn_proj": (T, H), "ln1_in": (T, H), "ln1_out": (T, H), "mu1": (T,), "rstd1": (T,),
                  "u": (T, F), "g": (T, F), "ffn_out": (T, H), "ln2_in": (T, H), "ln2_out": (T, H),
                  "mu2": (T,), "rstd2": (T,)}
        acts = {k: np.empty(v) for k, v in shapes.items()}
        ap = ctypes.byref(_Acts(*[_dp(acts[n]) for n in _ACT_NAMES]))
    c = cfg.c()
    rc = lib().orc_layer_forward(ctypes.byref(c), ctypes.byref(P), _dp(x),
                                 ln.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _dp(y), ap)
    if rc != 0:
        raise ValueError("oracle rejected the configuration")
    return y, acts


def layer_backward(cfg: LayerCfg, params: dict, x, lengths, dy, ln_invertible=False, want_y=False):
    """Returns (dx, grads) in fp64; grads keyed like params.  With want_y,
    returns (dx, grads, y): the forward output it recomputes on the way."""
    keep = []
    P = _params_struct(params, keep)
    x = _f64(x).reshape(cfg.batch * cfg.seq, cfg.hidden)
    dy = _f64(dy).reshape(cfg.batch * cfg.seq, cfg.hidden)
    ln = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32))
    grads = {n: np.empty(np.shape(params[n])) for n in PARAM_NAMES}
    G = _Params(*[_dp(grads[n]) for n in PARAM_NAMES])
    dx = np.empty_like(x)
    y = np.empty_like(x) if want_y else None
    c = cfg.c()
    rc = lib().orc_layer_backward(ctypes.byref(c), ctypes.byref(P), _dp(x),
                                  ln.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _dp(dy),
                                  int(ln_invertible), _dp(dx), ctypes.byref(G), _dp(y))
    if rc != 0:
        raise ValueError("oracle rejected the configuration")
    return (dx, grads, y) if want_y else (dx, grads)
