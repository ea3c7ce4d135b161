"""ctypes binding of the CPU oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's CPU-baseline leg use
this; the product path never imports it.  The oracle is plain single-threaded C in fp64
(tsd_oracle.c); this file only marshals arguments.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tsd_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

FORMATS = {"q4_0": 0, "q8_0": 1, "aff8": 2, "q5_0": 3, "aff4_g64": 4, "aff4_g32": 5}
ARCHS = {"gpt2": 0, "llama": 1, "talker_cp": 2}


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (plain -O2, no OpenMP, no intrinsics)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


class _Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("arch", "wfmt", "n_layer", "d_model", "n_head", "n_kv_head",
                                             "head_dim", "d_ff", "vocab", "n_ctx", "batch")] + [
        ("norm_eps", ctypes.c_double), ("rope_theta", ctypes.c_double),
        ("cp_n_layer", ctypes.c_int), ("n_codebooks", ctypes.c_int), ("cp_vocab", ctypes.c_int),
        ("sample_mode", ctypes.c_int), ("top_k", ctypes.c_int), ("temperature", ctypes.c_double),
        ("seed", ctypes.c_uint64), ("top_p", ctypes.c_double), ("min_p", ctypes.c_double),
        ("rep_penalty", ctypes.c_double), ("sample_order", ctypes.c_int), ("cfg", ctypes.c_int),
        ("cfg_weight", ctypes.c_double)]


class _Samp(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int), ("top_k", ctypes.c_int), ("temperature", ctypes.c_double),
                ("top_p", ctypes.c_double), ("min_p", ctypes.c_double), ("rep_penalty", ctypes.c_double),
                ("order", ctypes.c_int)]


ORDERS = {"t3": 0, "mtl": 1}


_lib = None
_P = ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build())
        d, i, sz, u16, u64, u32 = ctypes.c_double, ctypes.c_int, ctypes.c_size_t, ctypes.c_uint16, ctypes.c_uint64, ctypes.c_uint32
        sig = {
            "orc_half_to_double": (d, [u16]),
            "orc_double_to_half": (u16, [d]),
            "orc_philox4x64_10": (None, [_P, _P, _P]),
            "orc_uniform24": (d, [u64, u32, u32, u32]),
            "orc_matrix_bytes": (sz, [i, i, i]),
            "orc_dequant_row": (i, [i, _P, i, i, i, _P]),
            "orc_gemv": (i, [i, _P, i, i, _P, _P, _P]),
            "orc_gemv_f32": (i, [i, _P, i, i, i, _P, _P, _P]),
            "orc_layernorm": (None, [_P, i, _P, _P, d, _P]),
            "orc_rmsnorm": (None, [_P, i, _P, d, _P]),
            "orc_gelu_tanh": (d, [d]),
            "orc_silu": (d, [d]),
            "orc_rope_neox": (None, [_P, i, i, d]),
            "orc_softmax": (None, [_P, i, _P]),
            "orc_attend": (None, [_P, _P, _P, i, i, _P]),
            "orc_argmax": (i, [_P, i]),
            "orc_sample_topk": (i, [_P, i, i, d, d]),
            "orc_sample_chain": (i, [_P, i, _P, _P, i, d, _P]),
            "orc_n_weights": (i, [_P]),
            "orc_model_create": (_P, [_P, _P, _P, i]),
            "orc_last_error": (ctypes.c_char_p, []),
            "orc_model_destroy": (None, [_P]),
            "orc_reset": (None, [_P]),
            "orc_n_past": (i, [_P]),
            "orc_truncate": (i, [_P, i]),
            "orc_step": (i, [_P, _P, _P]),
            "orc_prefill": (i, [_P, _P, i, _P]),
            "orc_get_logits": (i, [_P, _P, sz]),
            "orc_load_kv": (i, [_P, _P, _P, i]),
            "orc_get_kv": (i, [_P, _P, _P, i]),
            "orc_layer_forward": (i, [_P, i, _P, i, _P]),
            "orc_forward_sequence": (i, [_P, _P, i, _P, _P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_P)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ---- scalar / operator wrappers --------------------------------------------------------------

def half_to_double(h: int) -> float:
    return lib().orc_half_to_double(int(h))


def double_to_half(x: float) -> int:
    return lib().orc_double_to_half(float(x))


def philox4x64_10(ctr, key):
    c, k, o = _c(ctr, np.uint64), _c(key, np.uint64), np.zeros(4, np.uint64)
    lib().orc_philox4x64_10(_ptr(c), _ptr(k), _ptr(o))
    return o


def uniform24(seed, row, pos, pss):
    return lib().orc_uniform24(seed, row, pos, pss)


def matrix_bytes(fmt, N, K):
    return lib().orc_matrix_bytes(FORMATS[fmt], N, K)


def dequant(fmt, blob, N, K):
    blob = _c(blob, np.uint8)
    W = np.empty((N, K), np.float64)
    for n in range(N):
        row = W[n]
        if lib().orc_dequant_row(FORMATS[fmt], _ptr(blob), N, K, n, row.ctypes.data_as(_P)):
            raise ValueError("dequant failed")
    return W


def gemv(fmt, blob, N, K, x, bias=None):
    blob, x = _c(blob, np.uint8), _c(x, np.float64)
    b = None if bias is None else _c(bias, np.float64)
    y = np.empty(N, np.float64)
    if lib().orc_gemv(FORMATS[fmt], _ptr(blob), N, K, _ptr(x), _ptr(b), _ptr(y)):
        raise ValueError("gemv failed")
    return y


def gemv_f32(fmt, blob, N, K, x, bias=None):
    """x float32 [B][K] (or [K]) -> y float64 [B][N]."""
    blob = _c(blob, np.uint8)
    x = _c(x, np.float32).reshape(-1, K)
    b = None if bias is None else _c(bias, np.float32)
    y = np.empty((x.shape[0], N), np.float64)
    if lib().orc_gemv_f32(FORMATS[fmt], _ptr(blob), N, K, x.shape[0], _ptr(x), _ptr(b), _ptr(y)):
        raise ValueError("gemv failed")
    return y


def layernorm(x, g=None, b=None, eps=1e-5):
    x = _c(x, np.float64)
    y = np.empty_like(x)
    lib().orc_layernorm(_ptr(x), x.size, _ptr(None if g is None else _c(g, np.float64)),
                        _ptr(None if b is None else _c(b, np.float64)), eps, _ptr(y))
    return y


def rmsnorm(x, g=None, eps=1e-5):
    x = _c(x, np.float64)
    y = np.empty_like(x)
    lib().orc_rmsnorm(_ptr(x), x.size, _ptr(None if g is None else _c(g, np.float64)), eps, _ptr(y))
    return y


def gelu_tanh(x):
    return lib().orc_gelu_tanh(float(x))


def silu(x):
    return lib().orc_silu(float(x))


def rope_neox(v, pos, theta=10000.0):
    v = _c(v, np.float64).copy()
    lib().orc_rope_neox(_ptr(v), v.size, pos, theta)
    return v


def softmax(s):
    s = _c(s, np.float64)
    a = np.empty_like(s)
    lib().orc_softmax(_ptr(s), s.size, _ptr(a))
    return a


def attend(q, kc, vc):
    """q [hd] float, kc/vc [n][hd] uint16 fp16 bit patterns."""
    q = _c(q, np.float64)
    kc, vc = _c(kc, np.uint16), _c(vc, np.uint16)
    o = np.empty(q.size, np.float64)
    lib().orc_attend(_ptr(q), _ptr(kc), _ptr(vc), kc.shape[0], q.size, _ptr(o))
    return o


def argmax(v):
    v = _c(v, np.float64)
    return lib().orc_argmax(_ptr(v), v.size)


def sample_topk(logits, k, temperature, u):
    v = _c(logits, np.float64)
    return lib().orc_sample_topk(_ptr(v), v.size, k, temperature, u)


def sample_chain(logits, u, mode=1, top_k=0, temperature=1.0, top_p=0.0, min_p=0.0, rep_penalty=1.0,
                 order="t3", hist=()):
    """The sampler chain (tsd_oracle.c orc_sample_chain).  Returns (id, margins) with margins =
    {draw, top_p, min_p, top_k, greedy, order} distances to the nearest decision boundary."""
    v = _c(logits, np.float64)
    h = _c(list(hist) if len(hist) else [0], np.int32)
    s = _Samp(mode, top_k, temperature, top_p, min_p, rep_penalty, ORDERS.get(order, order))
    m = np.zeros(6, np.float64)
    i = lib().orc_sample_chain(_ptr(v), v.size, ctypes.byref(s), _ptr(h), len(hist), float(u), _ptr(m))
    return i, dict(zip(("draw", "top_p", "min_p", "top_k", "greedy", "order"), m.tolist()))


# ---- models -----------------------------------------------------------------------------------

# sampler-chain fields a config may leave out: every filter off, the T3 order
CHAIN_DEFAULTS = {"top_p": 0.0, "min_p": 0.0, "rep_penalty": 1.0, "sample_order": "t3", "cfg": 0, "cfg_weight": 0.0}


def _cfg_struct(cfg: dict) -> _Cfg:
    s = _Cfg()
    for name, _ in _Cfg._fields_:
        v = cfg.get(name, CHAIN_DEFAULTS.get(name)) if name in CHAIN_DEFAULTS else cfg[name]
        if name == "arch":
            v = ARCHS[v]
        elif name == "wfmt":
            v = FORMATS[v]
        elif name == "sample_order":
            v = ORDERS.get(v, v)
        setattr(s, name, v)
    return s


class OracleModel:
    """The oracle decoder; weights are the canonical list from quantized_gemv_kv_amd.synth."""

    def __init__(self, cfg: dict, weights):
        self.cfg = dict(cfg)
        self._s = _cfg_struct(cfg)
        arrs = [np.ascontiguousarray(w) for w in weights]
        ptrs = (_P * len(arrs))(*[a.ctypes.data for a in arrs])
        sizes = (ctypes.c_size_t * len(arrs))(*[a.nbytes for a in arrs])
        h = lib().orc_model_create(ctypes.byref(self._s), ptrs, sizes, len(arrs))
        if not h:
            raise ValueError(lib().orc_last_error().decode())
        self._h = h
        self.tok_per_pos = cfg["n_codebooks"] if cfg["arch"] == "talker_cp" else 1
        self.vmax = max(cfg["vocab"], cfg["cp_vocab"]) if cfg["arch"] == "talker_cp" else cfg["vocab"]

    def close(self):
        if getattr(self, "_h", None):
            lib().orc_model_destroy(self._h)
            self._h = None

    __del__ = close

    def _check(self, rc):
        if rc:
            raise ValueError(lib().orc_last_error().decode())

    @property
    def n_past(self):
        return lib().orc_n_past(self._h)

    def reset(self):
        lib().orc_reset(self._h)

    def truncate(self, n):
        self._check(lib().orc_truncate(self._h, n))

    def step(self, tokens=None):
        B, C = self.cfg["batch"], self.tok_per_pos
        out = np.empty((B, C), np.int32)
        t = None if tokens is None else _c(tokens, np.int32).reshape(B, C)
        self._check(lib().orc_step(self._h, _ptr(t), _ptr(out)))
        return out

    def prefill(self, tokens):
        B, C = self.cfg["batch"], self.tok_per_pos
        t = _c(tokens, np.int32).reshape(B, -1, C)
        out = np.empty((B, C), np.int32)
        self._check(lib().orc_prefill(self._h, _ptr(t), t.shape[1], _ptr(out)))
        return out

    def logits(self):
        B, C = self.cfg["batch"], self.tok_per_pos
        out = np.empty((B, C, self.vmax), np.float64)
        self._check(lib().orc_get_logits(self._h, _ptr(out), out.size))
        return out if self.cfg["arch"] == "talker_cp" else out[:, 0, :]

    def load_kv(self, k, v, n_pos):
        k, v = _c(k, np.uint16), _c(v, np.uint16)
        self._check(lib().orc_load_kv(self._h, _ptr(k), _ptr(v), n_pos))

    def get_kv(self, n_pos=None):
        """The cache of positions 0..n_pos-1 as fp16 bit patterns [L][B][Hkv][n_pos][hd]."""
        c = self.cfg
        n = self.n_past if n_pos is None else n_pos
        shape = (c["n_layer"], c["batch"], c["n_kv_head"], n, c["head_dim"])
        k, v = np.empty(shape, np.uint16), np.empty(shape, np.uint16)
        self._check(lib().orc_get_kv(self._h, _ptr(k), _ptr(v), n))
        return k, v

    def layer_forward(self, layer, x, pos):
        x = _c(x, np.float64).reshape(self.cfg["batch"], self.cfg["d_model"])
        out = np.empty_like(x)
        self._check(lib().orc_layer_forward(self._h, layer, _ptr(x), pos, _ptr(out)))
        return out

    def forward_sequence(self, tokens, with_hidden=False):
        t = _c(tokens, np.int32).reshape(-1)
        lg = np.empty((t.size, self.cfg["vocab"]), np.float64)
        hid = np.empty((t.size, self.cfg["d_model"]), np.float64) if with_hidden else None
        self._check(lib().orc_forward_sequence(self._h, _ptr(t), t.size, _ptr(lg), _ptr(hid)))
        return (lg, hid) if with_hidden else lg
