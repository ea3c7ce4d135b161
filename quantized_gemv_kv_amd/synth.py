"""Seeded synthetic inputs for the decode-step workloads.

This module only draws numbers and lays them out in the canonical storage formats; it holds
none of the decode step's arithmetic.  The CPU oracle and the HIP library both consume what it
returns, each with its own decoding code.

Workload shapes follow the pages: the GPT-2-Medium-shaped T3 decoder and its Llama-shaped
multilingual variant ("Chatterbox -> ggml Port: Development Journal", §3.2, §3.19 and appendix
A3), and the Qwen3-TTS Talker + code predictor ("Every Frame Is a Memory Read", §1 and §3).
None of the pages' datasets or checkpoints is available, so every tensor here is random with
the shape, format and value law stated in the workload recipe.

Canonical storage formats (little endian):
  q4_0 : per row, K/32 blocks of 18 bytes = fp16 scale d, then 16 bytes; element j < 16 is the
         low nibble of byte j, element j+16 its high nibble.
  q8_0 : per row, K/32 blocks of 34 bytes = fp16 scale d, then 32 int8.
  aff8 : planar q[N][K] uint8, then scales[N][K/64] fp16, then biases[N][K/64] fp16.
  q5_0 : per row, K/32 blocks of 22 bytes = fp16 scale d, a 32-bit word whose bit j is element
         j's fifth bit, then the 16 nibble bytes ordered as in q4_0; w = (q - 16) d.
  aff4_g64 / aff4_g32 : planar q[N][K/2] bytes (element 2i in the low nibble of byte i, 2i+1 in
         the high one), then scales[N][K/G] fp16, then biases[N][K/G] fp16; w = s q + b.
"""
from __future__ import annotations

import numpy as np

FORMATS = {"q4_0": 0, "q8_0": 1, "aff8": 2, "q5_0": 3, "aff4_g64": 4, "aff4_g32": 5}
ARCHS = {"gpt2": 0, "llama": 1, "talker_cp": 2}


def rng_for(seed: int, *stream: int) -> np.random.Generator:
    """Independent PCG64 stream per (seed, stream ids)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *stream])))


# --------------------------------------------------------------------------------------------
# quantized matrices


def q8_0_matrix(rng, N, K, dscale=0.01):
    """int8 q uniform in [-127, 127], fp16 d = |N(0,1)| * dscale."""
    assert K % 32 == 0
    q = rng.integers(-127, 128, size=(N, K), dtype=np.int16).astype(np.int8)
    d = (np.abs(rng.standard_normal((N, K // 32))) * dscale).astype(np.float16)
    blob = np.empty((N, K // 32, 34), np.uint8)
    blob[:, :, 0:2] = d.view(np.uint8).reshape(N, K // 32, 2)
    blob[:, :, 2:] = q.view(np.uint8).reshape(N, K // 32, 32)
    return blob.reshape(-1), {"q": q, "d": d}


PLANAR = ("aff8", "aff4_g64", "aff4_g32")   # formats stored as planes (q, then s, then b)


def matrix_into(fmt, N, K, seed, out, chunk_rows=65536):
    """A tall matrix in `fmt`, drawn in row chunks (each from its own seeded stream) straight into
    the canonical byte buffer `out` (any array with slice assignment from numpy uint8, e.g. a
    torch uint8 tensor on the device), so that hundreds of MB never sit in host memory at once."""
    import torch
    for r0 in range(0, N, chunk_rows):
        n = min(chunk_rows, N - r0)
        blob = matrix(fmt, rng_for(seed, r0, K), n, K)
        if fmt in PLANAR:
            qb = n * (K if fmt == "aff8" else K // 2)
            g = 64 if fmt in ("aff8", "aff4_g64") else 32
            sb = n * (K // g) * 2
            qrow = qb // n
            Q = N * qrow
            parts = [(r0 * qrow, blob[:qb]), (Q + r0 * (K // g) * 2, blob[qb:qb + sb]),
                     (Q + N * (K // g) * 2 + r0 * (K // g) * 2, blob[qb + sb:])]
        else:
            rowb = blob.size // n
            parts = [(r0 * rowb, blob)]
        for off, part in parts:
            out[off:off + part.size].copy_(torch.from_numpy(part))


def q8_0_row_chunks(N, K, seed, chunk_rows=65536):
    """A tall Q8_0 matrix in row chunks (the lone-GEMV law, each chunk from its own seeded
    stream), so that hundreds of MB never sit in host memory at once: yields (row0, blob)."""
    for r0 in range(0, N, chunk_rows):
        n = min(chunk_rows, N - r0)
        yield r0, q8_0_matrix(rng_for(seed, r0, K), n, K)[0]


def q4_0_matrix(rng, N, K, dscale=0.02):
    """4-bit q uniform in 0..15, fp16 d = |N(0,1)| * dscale."""
    assert K % 32 == 0
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    d = (np.abs(rng.standard_normal((N, K // 32))) * dscale).astype(np.float16)
    qb = q.reshape(N, K // 32, 32)
    blob = np.empty((N, K // 32, 18), np.uint8)
    blob[:, :, 0:2] = d.view(np.uint8).reshape(N, K // 32, 2)
    blob[:, :, 2:] = qb[:, :, :16] | (qb[:, :, 16:] << 4)
    return blob.reshape(-1), {"q": q, "d": d}


def aff8_matrix(rng, N, K, sscale=0.01):
    """uint8 q uniform in 0..255; fp16 scale s = |N(0,1)| * sscale; fp16 bias b drawn around
    -128 s (so that weights are centred) plus 0.01 N(0,1)."""
    assert K % 64 == 0
    q = rng.integers(0, 256, size=(N, K), dtype=np.int16).astype(np.uint8)
    s = (np.abs(rng.standard_normal((N, K // 64))) * sscale).astype(np.float16)
    b = (-128.0 * s.astype(np.float64) + 0.01 * rng.standard_normal((N, K // 64))).astype(np.float16)
    blob = np.concatenate([q.reshape(-1), s.view(np.uint8).reshape(-1), b.view(np.uint8).reshape(-1)])
    return blob, {"q": q, "s": s, "b": b}


def q5_0_matrix(rng, N, K, dscale=0.02):
    """5-bit q uniform in 0..31, fp16 d = |N(0,1)| * dscale."""
    assert K % 32 == 0
    q = rng.integers(0, 32, size=(N, K), dtype=np.uint8)
    d = (np.abs(rng.standard_normal((N, K // 32))) * dscale).astype(np.float16)
    qb = q.reshape(N, K // 32, 32)
    lo = qb & 15
    hbits = ((qb >> 4) & 1).astype(np.uint32)
    qh = (hbits << np.arange(32, dtype=np.uint32)).sum(axis=2).astype(np.uint32)
    blob = np.empty((N, K // 32, 22), np.uint8)
    blob[:, :, 0:2] = d.view(np.uint8).reshape(N, K // 32, 2)
    blob[:, :, 2:6] = qh.astype("<u4").view(np.uint8).reshape(N, K // 32, 4)
    blob[:, :, 6:] = lo[:, :, :16] | (lo[:, :, 16:] << 4)
    return blob.reshape(-1), {"q": q, "d": d}


def aff4_matrix(rng, N, K, group=64, sscale=0.02):
    """4-bit q uniform in 0..15; fp16 scale s = |N(0,1)| * sscale; fp16 bias around -8 s (centred
    weights) plus 0.01 N(0,1)."""
    assert K % group == 0
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    s = (np.abs(rng.standard_normal((N, K // group))) * sscale).astype(np.float16)
    b = (-8.0 * s.astype(np.float64) + 0.01 * rng.standard_normal((N, K // group))).astype(np.float16)
    packed = q[:, 0::2] | (q[:, 1::2] << 4)
    blob = np.concatenate([packed.reshape(-1), s.view(np.uint8).reshape(-1), b.view(np.uint8).reshape(-1)])
    return blob, {"q": q, "s": s, "b": b}


def matrix(fmt, rng, N, K, scale=None):
    if fmt == "q4_0":
        return q4_0_matrix(rng, N, K, *(() if scale is None else (scale,)))[0]
    if fmt == "q8_0":
        return q8_0_matrix(rng, N, K, *(() if scale is None else (scale,)))[0]
    if fmt == "aff8":
        return aff8_matrix(rng, N, K, *(() if scale is None else (scale,)))[0]
    if fmt == "q5_0":
        return q5_0_matrix(rng, N, K, *(() if scale is None else (scale,)))[0]
    if fmt in ("aff4_g64", "aff4_g32"):
        g = 64 if fmt == "aff4_g64" else 32
        return aff4_matrix(rng, N, K, g, *(() if scale is None else (scale,)))[0]
    raise ValueError(fmt)


def normal_f32(rng, shape, std=1.0):
    return (rng.standard_normal(shape) * std).astype(np.float32)


def fp16_cache(rng, shape):
    """fp16 values ~N(0,1), returned as their uint16 bit patterns."""
    return rng.standard_normal(shape).astype(np.float16).view(np.uint16)


# --------------------------------------------------------------------------------------------
# model configurations (the five workloads)

def config(name: str) -> dict:
    base = dict(norm_eps=1e-5, rope_theta=10000.0, cp_n_layer=0, n_codebooks=0, cp_vocab=0, batch=1,
                sample_mode=0, top_k=0, temperature=1.0, seed=42)
    if name == "gpt2_medium_q4_0":      # 24-layer T3 Turbo shape
        base.update(arch="gpt2", wfmt="q4_0", n_layer=24, d_model=1024, n_head=16, n_kv_head=16,
                    head_dim=64, d_ff=4096, vocab=8192, n_ctx=1024)
    elif name == "gpt2_medium_q5_0":    # the same decoder in the journal's Q5_0 (appendix A3)
        base.update(arch="gpt2", wfmt="q5_0", n_layer=24, d_model=1024, n_head=16, n_kv_head=16,
                    head_dim=64, d_ff=4096, vocab=8192, n_ctx=1024)
    elif name == "gpt2_layer_q4_0":     # one GPT-2-Medium layer
        base.update(arch="gpt2", wfmt="q4_0", n_layer=1, d_model=1024, n_head=16, n_kv_head=16,
                    head_dim=64, d_ff=4096, vocab=8192, n_ctx=1024)
    elif name == "llama520m_q8_0":      # 30-layer multilingual T3 shape
        base.update(arch="llama", wfmt="q8_0", n_layer=30, d_model=1024, n_head=16, n_kv_head=16,
                    head_dim=64, d_ff=4096, vocab=8192, n_ctx=1024)
    elif name == "talker_cp_aff8":      # Qwen3-TTS 0.6B Talker + code predictor, batch 16
        base.update(arch="talker_cp", wfmt="aff8", n_layer=28, d_model=1024, n_head=16, n_kv_head=8,
                    head_dim=128, d_ff=3072, vocab=3072, n_ctx=512, cp_n_layer=5, n_codebooks=16,
                    cp_vocab=2048, batch=16)
    else:
        raise KeyError(name)
    return base


def small_config(arch: str, wfmt: str, **kw) -> dict:
    """Tiny shapes for CPU tests: several GEMV tiles and a ragged tail are still present."""
    c = dict(arch=arch, wfmt=wfmt, n_layer=2, d_model=128, n_head=2, n_kv_head=2, head_dim=64,
             d_ff=256, vocab=160, n_ctx=48, batch=1, norm_eps=1e-5,
             rope_theta=10000.0, cp_n_layer=0, n_codebooks=0, cp_vocab=0, sample_mode=0, top_k=0,
             temperature=1.0, seed=42)
    if arch == "talker_cp":
        c.update(n_kv_head=1, cp_n_layer=2, n_codebooks=4, cp_vocab=96, batch=2)
    c.update(kw)
    return c


# --------------------------------------------------------------------------------------------
# weights in canonical order

def model_weights(cfg: dict, seed: int = 42, norm_std: float = 0.02, emb_std: float = 0.02):
    """List of numpy arrays (fp32 tensors or uint8 quantized blobs) in the canonical order:

    gpt2  : wte[V][d], wpe[n_ctx][d], per layer {ln1_g, ln1_b, qkv_w[3d][d], qkv_b[3d], o_w[d][d],
            o_b[d], ln2_g, ln2_b, fc_w[ff][d], fc_b[ff], down_w[d][ff], down_b[d]},
            lnf_g, lnf_b, head_w[V][d]
    llama : emb[V][d], per layer {rms1_g, q_w, k_w, v_w, o_w, rms2_g, gate_w, up_w, down_w},
            rmsf_g, head_w[V][d]
    talker_cp: E_0[V][d], E_1..E_{C-1}[Vcp][d], Talker layers (as llama), rmsf_g, head_w[V][d],
            predictor layers (as llama), predictor rmsf_g, predictor heads 1..C-1 [Vcp][d]

    Norm gains/biases and linear biases ~N(0, norm_std), embeddings ~N(0, emb_std), matrices
    in cfg["wfmt"] with the format's default scale law.
    """
    arch, f = cfg["arch"], cfg["wfmt"]
    d, H, Hk, hd, ff, V = (cfg[k] for k in ("d_model", "n_head", "n_kv_head", "head_dim", "d_ff", "vocab"))
    out = []
    stream = [0]

    def r():
        stream[0] += 1
        return rng_for(seed, stream[0])

    def vec(n, std=norm_std):
        return normal_f32(r(), (n,), std)

    def mat(N, K):
        return matrix(f, r(), N, K)

    if arch == "gpt2":
        out += [normal_f32(r(), (V, d), emb_std), normal_f32(r(), (cfg["n_ctx"], d), emb_std)]
        for _ in range(cfg["n_layer"]):
            out += [vec(d), vec(d), mat(3 * d, d), vec(3 * d), mat(d, d), vec(d),
                    vec(d), vec(d), mat(ff, d), vec(ff), mat(d, ff), vec(d)]
        out += [vec(d), vec(d), mat(V, d)]
        return out

    def llama_layers(n):
        res = []
        for _ in range(n):
            res += [vec(d), mat(H * hd, d), mat(Hk * hd, d), mat(Hk * hd, d), mat(d, H * hd),
                    vec(d), mat(ff, d), mat(ff, d), mat(d, ff)]
        return res

    if arch == "llama":
        out += [normal_f32(r(), (V, d), emb_std)]
        out += llama_layers(cfg["n_layer"])
        out += [vec(d), mat(V, d)]
        return out
    if arch == "talker_cp":
        C, Vc = cfg["n_codebooks"], cfg["cp_vocab"]
        out += [normal_f32(r(), (V, d), emb_std)]
        out += [normal_f32(r(), (Vc, d), emb_std) for _ in range(1, C)]
        out += llama_layers(cfg["n_layer"])
        out += [vec(d), mat(V, d)]
        out += llama_layers(cfg["cp_n_layer"])
        out += [vec(d)]
        out += [mat(Vc, d) for _ in range(1, C)]
        return out
    raise KeyError(arch)


def prompt_tokens(cfg: dict, n: int, seed: int = 42) -> np.ndarray:
    """Prompt ids [batch][n][tokens per position], uniform over each vocabulary."""
    rng = rng_for(seed, 1000)
    B = cfg["batch"]
    if cfg["arch"] == "talker_cp":
        C = cfg["n_codebooks"]
        t = np.empty((B, n, C), np.int32)
        t[:, :, 0] = rng.integers(0, cfg["vocab"], size=(B, n))
        t[:, :, 1:] = rng.integers(0, cfg["cp_vocab"], size=(B, n, C - 1))
        return t
    return rng.integers(0, cfg["vocab"], size=(B, n, 1)).astype(np.int32)


def kv_cache(cfg: dict, n_pos: int, seed: int = 42):
    """Random fp16 K and V caches [n_layer][batch][n_kv_head][n_pos][head_dim] ~N(0,1)."""
    shape = (cfg["n_layer"], cfg["batch"], cfg["n_kv_head"], n_pos, cfg["head_dim"])
    return fp16_cache(rng_for(seed, 2000), shape), fp16_cache(rng_for(seed, 2001), shape)


def hidden(cfg: dict, seed: int = 42, std: float = 1.0) -> np.ndarray:
    """Hidden-state input [batch][d] ~N(0, std)."""
    return normal_f32(rng_for(seed, 3000), (cfg["batch"], cfg["d_model"]), std)
