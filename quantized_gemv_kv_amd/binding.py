"""ctypes binding of libtsd.so (include/tsd.h), argument marshalling only.

Every compute step runs in the library's HIP kernels; PyTorch supplies device memory and the
stream.  The functions keep the C names; `Model` is a small convenience that allocates the
workspace and uploads the canonical weights with torch and then calls the same entry points.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtsd.so")

ARCHS = {"gpt2": 0, "llama": 1, "talker_cp": 2}
FORMATS = {"q4_0": 0, "q8_0": 1, "aff8": 2, "q5_0": 3, "aff4_g64": 4, "aff4_g32": 5}
STATUS = {0: "TSD_OK", 1: "TSD_ERR_INVALID_ARGUMENT", 2: "TSD_ERR_UNSUPPORTED", 3: "TSD_ERR_OUT_OF_MEMORY",
          4: "TSD_ERR_CONTEXT_FULL", 5: "TSD_ERR_HIP", 6: "TSD_ERR_STATE", 7: "TSD_ERR_TIMEOUT"}
LAUNCH_MODES = {"persistent": 0, "per_operator": 1}

# symbols declared in include/tsd.h
EXPORTS = ["tsd_workspace_bytes", "tsd_model_create", "tsd_prefill", "tsd_step", "tsd_step_eager", "tsd_reset", "tsd_truncate",
           "tsd_n_past", "tsd_model_destroy", "tsd_last_error", "tsd_get_logits", "tsd_get_tokens", "tsd_load_kv",
           "tsd_layer_forward", "tsd_gemv_packed_bytes", "tsd_gemv_pack", "tsd_gemv",
           "tsd_attention_scratch_bytes", "tsd_attention", "tsd_time_kernel", "tsd_synchronize",
           "tsd_model_info", "tsd_sample_topk", "tsd_sample", "tsd_gemm_rows_packed_bytes", "tsd_gemm_rows_pack",
           "tsd_gemm_rows_scratch_bytes", "tsd_gemm_rows", "tsd_prefill_stepwise", "tsd_gemm_scratch_bytes", "tsd_gemm",
           "tsd_get_kv", "tsd_debug_gemv", "tsd_attention_noalloc", "tsd_debug_set_wait_limit"]
KERNEL_KINDS = {"qkv": 0, "attn": 1, "oproj": 2, "fc": 3, "down": 4, "head": 5, "step": 6}


class TsdError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class tsd_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("arch", "wfmt", "n_layer", "d_model", "n_head", "n_kv_head",
                                               "head_dim", "d_ff", "vocab", "n_ctx", "batch")] + [
        ("norm_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
        ("cp_n_layer", ctypes.c_int32), ("n_codebooks", ctypes.c_int32), ("cp_vocab", ctypes.c_int32),
        ("launch_mode", ctypes.c_int32), ("n_workgroups", ctypes.c_int32)]


class tsd_sampling(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("top_k", ctypes.c_int32), ("temperature", ctypes.c_float),
                ("seed", ctypes.c_uint64), ("top_p", ctypes.c_float), ("min_p", ctypes.c_float),
                ("rep_penalty", ctypes.c_float), ("order", ctypes.c_int32), ("cfg", ctypes.c_int32),
                ("cfg_weight", ctypes.c_float)]


ORDERS = {"t3": 0, "mtl": 1}


def make_sampling(d: dict) -> tsd_sampling:
    """tsd_sampling from a dict (missing fields: greedy, every filter off, the T3 order)."""
    return tsd_sampling(d.get("mode", 0), d.get("top_k", 0), d.get("temperature", 1.0), d.get("seed", 0),
                        d.get("top_p", 0.0), d.get("min_p", 0.0), d.get("rep_penalty", 0.0),
                        ORDERS.get(d.get("order", "t3"), d.get("order", 0)), d.get("cfg", 0), d.get("cfg_weight", 0.0))


class tsd_tensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("bytes", ctypes.c_size_t)]


_lib = None
_P, _I, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t


def lib():
    """Load libtsd.so; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m quantized_gemv_kv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        st = ctypes.c_int
        sig = {
            "tsd_workspace_bytes": [ctypes.POINTER(tsd_config), ctypes.POINTER(_SZ)],
            "tsd_model_create": [ctypes.POINTER(tsd_config), ctypes.POINTER(tsd_tensor), _I, _P, _SZ, _P,
                                 ctypes.POINTER(tsd_sampling), ctypes.POINTER(_P)],
            "tsd_prefill": [_P, _P, _I, _P],
            "tsd_prefill_stepwise": [_P, _P, _I, _P],
            "tsd_step": [_P, _P, _P],
            "tsd_step_eager": [_P, _P, _P],
            "tsd_reset": [_P],
            "tsd_truncate": [_P, _I],
            "tsd_n_past": [_P, ctypes.POINTER(_I)],
            "tsd_model_destroy": [_P],
            "tsd_get_logits": [_P, _P],
            "tsd_get_tokens": [_P, _I, _I, _P],
            "tsd_load_kv": [_P, _P, _P, _I],
            "tsd_get_kv": [_P, _P, _P, _I],
            "tsd_layer_forward": [_P, _I, _P, _I, _P],
            "tsd_gemv_packed_bytes": [_I, _I, _I, ctypes.POINTER(_SZ)],
            "tsd_gemv_pack": [_I, _P, _SZ, _I, _I, _P, _SZ, _P],
            "tsd_gemv": [_I, _P, _I, _I, _I, _P, _P, _P, _P],
            "tsd_attention_scratch_bytes": [_I, _I, _I, _I, ctypes.POINTER(_SZ)],
            "tsd_attention": [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _SZ, _P],
            "tsd_time_kernel": [_P, _I, _I, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(_I)],
            "tsd_synchronize": [_P],
            "tsd_debug_set_wait_limit": [_P, ctypes.c_int64],
            "tsd_model_info": [_P, _P, _P],
            "tsd_sample_topk": [_P, _I, _I, ctypes.c_float, ctypes.c_uint64, _I, _I, _I, _P, _P],
            "tsd_sample": [_P, _I, ctypes.POINTER(tsd_sampling), _P, _I, _I, _I, _I, _P, _P],
            "tsd_gemm_rows_packed_bytes": [_I, _I, ctypes.POINTER(_SZ)],
            "tsd_gemm_rows_pack": [_P, _SZ, _I, _I, _P, _SZ, _P],
            "tsd_gemm_rows_scratch_bytes": [_I, _I, _I, ctypes.POINTER(_SZ)],
            "tsd_gemm_rows": [_P, _I, _I, _I, _P, _P, _I, _P, _SZ, _P],
            "tsd_gemm_scratch_bytes": [_I, _I, ctypes.POINTER(_SZ)],
            "tsd_gemm": [_I, _P, _I, _I, _I, _P, _P, _P, _P, _SZ, _P],
            "tsd_debug_gemv": [_I, _P, _SZ, _P, _P, _I, _I, _I, _P],
            "tsd_attention_noalloc": [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes, f.restype = args, st
        L.tsd_last_error.argtypes, L.tsd_last_error.restype = [_P], ctypes.c_char_p
        _lib = L
    return _lib


def _check(rc, model=None):
    if rc != 0:
        msg = lib().tsd_last_error(model)
        raise TsdError(rc, msg.decode() if msg else "")


def make_config(cfg: dict) -> tsd_config:
    c = tsd_config()
    for name, _ in tsd_config._fields_:
        v = cfg.get(name, 0)
        if name == "arch":
            v = ARCHS[v] if isinstance(v, str) else v
        elif name == "wfmt":
            v = FORMATS[v] if isinstance(v, str) else v
        elif name == "launch_mode":
            v = LAUNCH_MODES[v] if isinstance(v, str) else v
        setattr(c, name, v)
    return c


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


# ---- C-name wrappers -------------------------------------------------------------------------

def tsd_workspace_bytes(cfg: dict) -> int:
    out = _SZ()
    _check(lib().tsd_workspace_bytes(ctypes.byref(make_config(cfg)), ctypes.byref(out)))
    return out.value


def tsd_gemv_packed_bytes(fmt, N, K) -> int:
    out = _SZ()
    _check(lib().tsd_gemv_packed_bytes(FORMATS.get(fmt, fmt), N, K, ctypes.byref(out)))
    return out.value


def tsd_gemv_pack(fmt, w, N, K, packed, stream=None):
    _check(lib().tsd_gemv_pack(FORMATS.get(fmt, fmt), _ptr(w), w.numel() * w.element_size(), N, K, _ptr(packed),
                               packed.numel() * packed.element_size(), _stream(stream)))


def tsd_gemv(fmt, packed, N, K, B, x, bias, y, stream=None):
    _check(lib().tsd_gemv(FORMATS.get(fmt, fmt), _ptr(packed), N, K, B, _ptr(x), _ptr(bias), _ptr(y), _stream(stream)))


def tsd_debug_gemv(fmt, w, x, y, N, K, B, stream=None):
    """w: the canonical blob (device uint8); x [B][K], y [B][N] fp32 device tensors."""
    _check(lib().tsd_debug_gemv(FORMATS.get(fmt, fmt), _ptr(w), w.numel() * w.element_size(), _ptr(x), _ptr(y), N, K, B,
                                _stream(stream)))


def tsd_sample_topk(logits, top_k, temperature, seed, row, pos, pss, out, stream=None):
    _check(lib().tsd_sample_topk(_ptr(logits), logits.numel(), top_k, temperature, seed, row, pos, pss, _ptr(out),
                                 _stream(stream)))


def tsd_sample(logits, sampling: dict, hist, row, pos, pss, out, stream=None):
    """hist: an int32 device tensor of token ids, or None."""
    s = make_sampling(sampling)
    _check(lib().tsd_sample(_ptr(logits), logits.numel(), ctypes.byref(s), _ptr(hist),
                            0 if hist is None else hist.numel(), row, pos, pss, _ptr(out), _stream(stream)))


def tsd_gemm_rows_packed_bytes(N, K) -> int:
    out = _SZ()
    _check(lib().tsd_gemm_rows_packed_bytes(N, K, ctypes.byref(out)))
    return out.value


def tsd_gemm_rows_pack(w, N, K, packed, stream=None):
    _check(lib().tsd_gemm_rows_pack(_ptr(w), w.numel() * w.element_size(), N, K, _ptr(packed),
                                    packed.numel() * packed.element_size(), _stream(stream)))


def tsd_gemm_rows_scratch_bytes(N, K, splits=1) -> int:
    out = _SZ()
    _check(lib().tsd_gemm_rows_scratch_bytes(N, K, splits, ctypes.byref(out)))
    return out.value


def tsd_gemm_rows(packed, N, K, B, x, y, splits, scratch, stream=None):
    _check(lib().tsd_gemm_rows(_ptr(packed), N, K, B, _ptr(x), _ptr(y), splits, _ptr(scratch), scratch.numel(),
                               _stream(stream)))


def tsd_gemm_scratch_bytes(M, K) -> int:
    out = _SZ()
    _check(lib().tsd_gemm_scratch_bytes(M, K, ctypes.byref(out)))
    return out.value


def tsd_gemm(fmt, packed, N, K, M, x, bias, y, scratch, stream=None):
    _check(lib().tsd_gemm(FORMATS.get(fmt, fmt), _ptr(packed), N, K, M, _ptr(x), _ptr(bias), _ptr(y), _ptr(scratch),
                          scratch.numel(), _stream(stream)))


def tsd_attention_scratch_bytes(B, H, n_ctx, hd) -> int:
    out = _SZ()
    _check(lib().tsd_attention_scratch_bytes(B, H, n_ctx, hd, ctypes.byref(out)))
    return out.value


def tsd_attention(q, k, v, B, H, Hkv, hd, n_keys, n_ctx, out, scratch, stream=None):
    _check(lib().tsd_attention(_ptr(q), _ptr(k), _ptr(v), B, H, Hkv, hd, n_keys, n_ctx, _ptr(out), _ptr(scratch),
                               scratch.numel(), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 4 << 20   # TSD_NOALLOC_SCRATCH_BYTES


def tsd_attention_noalloc(q, k, v, B, H, Hkv, hd, n_keys, n_ctx, out, stream=None):
    """tsd_attention with the library's own per-GPU partials array (no scratch argument)."""
    _check(lib().tsd_attention_noalloc(_ptr(q), _ptr(k), _ptr(v), B, H, Hkv, hd, n_keys, n_ctx, _ptr(out),
                                       _stream(stream)))


# ---- convenience: a model whose memory torch owns --------------------------------------------

class Model:
    """Uploads the canonical weights, allocates the workspace, calls tsd_model_create; the
    methods map one-to-one onto tsd_prefill / tsd_step / ... ."""

    def __init__(self, cfg: dict, weights, stream=None, sampling: dict | None = None):
        import torch
        self.torch = torch
        self.cfg = dict(cfg)
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        self.tpp = cfg["n_codebooks"] if cfg["arch"] == "talker_cp" else 1
        self.vmax = max(cfg["vocab"], cfg.get("cp_vocab", 0)) if cfg["arch"] == "talker_cp" else cfg["vocab"]
        self._c = make_config(cfg)
        nbytes = tsd_workspace_bytes(cfg)
        with torch.cuda.stream(self.stream):
            self.workspace = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            dev = [torch.from_numpy(np.ascontiguousarray(w).reshape(-1).view(np.uint8)).to("cuda", non_blocking=False)
                   for w in weights]
        arr = (tsd_tensor * len(dev))(*[tsd_tensor(t.data_ptr(), t.numel()) for t in dev])
        samp = None
        if sampling is not None:
            samp = make_sampling(sampling)
        h = _P()
        torch.cuda.synchronize()
        _check(lib().tsd_model_create(ctypes.byref(self._c), arr, len(dev), _ptr(self.workspace), nbytes,
                                      _stream(self.stream), ctypes.byref(samp) if samp else None, ctypes.byref(h)))
        self.stream.synchronize()
        del dev                                   # the library keeps its own repacked copy
        self.h = h
        B = cfg["batch"]
        self._next = torch.empty((B, self.tpp), dtype=torch.int32, device="cuda")

    def close(self):
        if getattr(self, "h", None) is not None and self.h.value:
            lib().tsd_model_destroy(self.h)
            self.h = None

    __del__ = close

    def _chk(self, rc):
        _check(rc, self.h)

    @property
    def n_past(self):
        out = _I()
        self._chk(lib().tsd_n_past(self.h, ctypes.byref(out)))
        return out.value

    def prefill(self, tokens):
        """tokens: device int32 [batch][n][tokens per position] (or [n] for batch 1)."""
        t = tokens.reshape(self.cfg["batch"], -1, self.tpp).contiguous()
        self._chk(lib().tsd_prefill(self.h, _ptr(t), t.shape[1], _ptr(self._next)))
        return self._next

    def prefill_stepwise(self, tokens):
        """As prefill, by the decode step at every prompt position."""
        t = tokens.reshape(self.cfg["batch"], -1, self.tpp).contiguous()
        self._chk(lib().tsd_prefill_stepwise(self.h, _ptr(t), t.shape[1], _ptr(self._next)))
        return self._next

    def step(self, tokens=None, out=True):
        t = None if tokens is None else tokens.reshape(self.cfg["batch"], self.tpp).contiguous()
        self._chk(lib().tsd_step(self.h, _ptr(t), _ptr(self._next) if out else None))
        return self._next if out else None

    def step_eager(self, tokens=None, out=True):
        t = None if tokens is None else tokens.reshape(self.cfg["batch"], self.tpp).contiguous()
        self._chk(lib().tsd_step_eager(self.h, _ptr(t), _ptr(self._next) if out else None))
        return self._next if out else None

    def reset(self):
        self._chk(lib().tsd_reset(self.h))

    def truncate(self, n):
        self._chk(lib().tsd_truncate(self.h, n))

    def debug_set_wait_limit(self, ticks):
        """Tests of the time-out path: every bounded wait of the persistent step gives up after
        `ticks` of the 100 MHz clock (<= 0: the normal limit)."""
        self._chk(lib().tsd_debug_set_wait_limit(self.h, int(ticks)))

    def synchronize(self):
        """Wait for the model's stream; TsdError(TSD_ERR_TIMEOUT) if a persistent step gave up,
        TsdError(TSD_ERR_INVALID_ARGUMENT) if a call passed an id outside its vocabulary (that call
        and the ones after it did nothing)."""
        self._chk(lib().tsd_synchronize(self.h))

    def logits(self):
        self.synchronize()
        B = self.cfg["batch"]
        out = self.torch.empty((B, self.tpp, self.vmax) if self.tpp > 1 else (B, self.vmax), dtype=self.torch.float32,
                               device="cuda")
        self._chk(lib().tsd_get_logits(self.h, _ptr(out)))
        return out

    def tokens(self, first, n):
        self.synchronize()
        out = self.torch.empty((n, self.cfg["batch"], self.tpp), dtype=self.torch.int32, device="cuda")
        self._chk(lib().tsd_get_tokens(self.h, first, n, _ptr(out)))
        return out

    def info(self):
        """(launch mode name, workgroups) in effect (tsd_model_info)."""
        mode, nwg = ctypes.c_int32(), ctypes.c_int32()
        self._chk(lib().tsd_model_info(self.h, ctypes.byref(mode), ctypes.byref(nwg)))
        return {v: k for k, v in LAUNCH_MODES.items()}[mode.value], nwg.value

    def uses_persistent_step(self):
        return self.info()[0] == "persistent"

    def time_kernel(self, kind, n_steps):
        """(mean duration in us, launches per step) of one kernel kind over n_steps real steps."""
        us, n = ctypes.c_float(), _I()
        self._chk(lib().tsd_time_kernel(self.h, KERNEL_KINDS.get(kind, kind), n_steps, ctypes.byref(us), ctypes.byref(n)))
        return us.value, n.value

    def load_kv(self, k, v, n_pos):
        self._chk(lib().tsd_load_kv(self.h, _ptr(k), _ptr(v), n_pos))

    def get_kv(self, n_pos=None):
        """The cache of positions 0..n_pos-1 as two device fp16 tensors [L][B][Hkv][n_pos][hd]."""
        torch = self.torch
        c = self.cfg
        n = self.n_past if n_pos is None else n_pos
        shape = (c["n_layer"], c["batch"], c["n_kv_head"], n, c["head_dim"])
        k = torch.empty(shape, dtype=torch.float16, device="cuda")
        v = torch.empty(shape, dtype=torch.float16, device="cuda")
        self._chk(lib().tsd_get_kv(self.h, _ptr(k), _ptr(v), n))
        self.stream.synchronize()
        return k, v

    def layer_forward(self, layer, x, pos):
        out = self.torch.empty_like(x)
        self._chk(lib().tsd_layer_forward(self.h, layer, _ptr(x), pos, _ptr(out)))
        return out
