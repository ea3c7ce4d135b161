"""Algorithmic byte counts of one decode step (the denominator of the roofline).

The decode step reads every quantized weight once and the key/value cache once; its
arithmetic intensity is about 2 flop/byte, so its floor is bytes / HBM bandwidth ("Every Frame
Is a Memory Read", §3 "Predict first: the roofline": time per step is about the bytes read per
step over the sustained bandwidth).  Counted per step:

* weights   - every quantized matrix in its stored format (scales and biases included);
* vectors   - fp32 norm gains/biases and linear biases;
* embedding - the embedding rows gathered (token row, plus the learned position row for GPT-2;
              sixteen code rows per frame for the Talker, one row per predictor pass);
* kv        - the fp16 keys and values of every position the step attends to, the new position
              included (it is written once and read by attention).

Activations (a few KB) are not counted.
"""
from __future__ import annotations

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published


def matrix_bytes(fmt: str, N: int, K: int) -> int:
    if fmt == "q4_0":
        return N * (K // 32) * 18
    if fmt == "q8_0":
        return N * (K // 32) * 34
    if fmt == "aff8":
        return N * K + N * (K // 64) * 4
    if fmt == "q5_0":
        return N * (K // 32) * 22
    if fmt == "aff4_g64":
        return N * K // 2 + N * (K // 64) * 4
    if fmt == "aff4_g32":
        return N * K // 2 + N * (K // 32) * 4
    raise ValueError(fmt)


def _llama_layer_mats(c):
    d, H, Hk, hd, ff = c["d_model"], c["n_head"], c["n_kv_head"], c["head_dim"], c["d_ff"]
    return [(H * hd, d), (Hk * hd, d), (Hk * hd, d), (d, H * hd), (ff, d), (ff, d), (d, ff)]


def _gpt2_layer_mats(c):
    d, ff = c["d_model"], c["d_ff"]
    return [(3 * d, d), (d, d), (ff, d), (d, ff)]


def params_per_layer(c) -> int:
    mats = _gpt2_layer_mats(c) if c["arch"] == "gpt2" else _llama_layer_mats(c)
    return sum(N * K for N, K in mats)


def kv_bytes_per_position(c, n_layer=None) -> int:
    """fp16 K and V of one position over all layers, one batch row."""
    L = c["n_layer"] if n_layer is None else n_layer
    return L * 2 * c["n_kv_head"] * c["head_dim"] * 2


def layer_weight_bytes(c) -> int:
    mats = _gpt2_layer_mats(c) if c["arch"] == "gpt2" else _llama_layer_mats(c)
    return sum(matrix_bytes(c["wfmt"], N, K) for N, K in mats)


def step_bytes(c, pos: int) -> dict:
    """Bytes of one decode step at position pos (keys 0..pos), all batch rows.

    For talker_cp one step is one frame: the Talker step plus the 15 predictor passes."""
    d, f, L, B = c["d_model"], c["wfmt"], c["n_layer"], c["batch"]
    out = {}
    if c["arch"] == "gpt2":
        ff = c["d_ff"]
        out["weights"] = L * layer_weight_bytes(c) + matrix_bytes(f, c["vocab"], d)
        out["vectors"] = 4 * (L * (4 * d + 3 * d + d + ff + d) + 2 * d)
        out["embedding"] = B * 2 * d * 4
        out["kv"] = B * (pos + 1) * kv_bytes_per_position(c)
    elif c["arch"] == "llama":
        out["weights"] = L * layer_weight_bytes(c) + matrix_bytes(f, c["vocab"], d)
        out["vectors"] = 4 * (L * 2 * d + d)
        out["embedding"] = B * d * 4
        out["kv"] = B * (pos + 1) * kv_bytes_per_position(c)
    elif c["arch"] == "talker_cp":
        C, Lc, Vc = c["n_codebooks"], c["cp_n_layer"], c["cp_vocab"]
        passes = C - 1
        talker_w = L * layer_weight_bytes(c) + matrix_bytes(f, c["vocab"], d)
        cp_w = Lc * layer_weight_bytes(c) + matrix_bytes(f, Vc, d)
        out["weights"] = talker_w + passes * cp_w
        out["vectors"] = 4 * (L * 2 * d + d) + passes * 4 * (Lc * 2 * d + d)
        out["embedding"] = B * C * d * 4 + B * passes * d * 4
        cp_positions = sum(j + 1 for j in range(1, C))          # pass j attends to 0..j
        out["kv"] = B * ((pos + 1) * kv_bytes_per_position(c) + cp_positions * kv_bytes_per_position(c, Lc))
    else:
        raise KeyError(c["arch"])
    out["total"] = sum(out.values())
    return out


def mean_step_bytes(c, first_pos: int, n_steps: int) -> float:
    return sum(step_bytes(c, p)["total"] for p in range(first_pos, first_pos + n_steps)) / n_steps


def gemv_bytes(fmt: str, N: int, K: int, B: int = 1, bias: bool = False) -> int:
    """One GEMV launch: the matrix, plus x [B][K] read and y [B][N] written in fp32."""
    return matrix_bytes(fmt, N, K) + 4 * B * (K + N) + (4 * N if bias else 0)


ATTN_CHUNK = 256     # positions per attention workgroup (one partial each)


def kernel_bytes(c, kind: str, pos: int) -> int:
    """Algorithmic bytes of one launch of a step kernel at position pos (batch 1 GPT-2/Llama):
    the matrix in its stored format, the fp32 vectors it reads (bias, norm gain/bias), the
    activations it reads and writes, and for attention the fp16 keys/values of positions
    0..pos plus the query and the per-chunk partials."""
    d, f, H, Hk, hd, ff = c["d_model"], c["wfmt"], c["n_head"], c["n_kv_head"], c["head_dim"], c["d_ff"]
    gpt2 = c["arch"] == "gpt2"
    n_split = (pos + 1 + ATTN_CHUNK - 1) // ATTN_CHUNK
    part = H * n_split * (hd + 4) * 4
    qkv_rows = (H + 2 * Hk) * hd
    if kind == "qkv":
        return (matrix_bytes(f, qkv_rows, d) + 4 * d * (2 if gpt2 else 1) + (4 * qkv_rows if gpt2 else 0)
                + 4 * d + 4 * H * hd + 2 * 2 * Hk * hd)
    if kind == "attn":
        return (pos + 1) * 2 * Hk * hd * 2 + 4 * H * hd + part
    if kind == "oproj":
        return matrix_bytes(f, d, H * hd) + (4 * d if gpt2 else 0) + part + 2 * 4 * d
    if kind == "fc":
        rows = ff if gpt2 else 2 * ff
        return matrix_bytes(f, rows, d) + 4 * d * (2 if gpt2 else 1) + (4 * ff if gpt2 else 0) + 4 * d + 4 * ff
    if kind == "down":
        return matrix_bytes(f, d, ff) + (4 * d if gpt2 else 0) + 4 * ff + 2 * 4 * d
    if kind == "head":
        return matrix_bytes(f, c["vocab"], d) + 4 * d * (2 if gpt2 else 1) + 4 * d + 4 * c["vocab"]
    raise KeyError(kind)


def frame_kernel_bytes(c, kind: str, pos: int) -> float:
    """Mean algorithmic bytes of one launch of a kind in the batched Talker + predictor frame
    at Talker position pos: the matrix in its stored format (the same for Talker and predictor
    layers, which share their widths), the fp16 hi/lo operand of all 16 GEMM rows and its group
    sums, and what the epilogue writes for the batch rows; attention: the fp16 keys and values
    each launch reads (the Talker's 0..pos, the predictor's 0..cpos) averaged over the frame's
    launches, plus queries and partials."""
    d, f, H, Hk, hd, ff, B = (c[k] for k in ("d_model", "wfmt", "n_head", "n_kv_head", "head_dim", "d_ff", "batch"))
    C, L, Lc = c["n_codebooks"], c["n_layer"], c["cp_n_layer"]
    qd, kd, rows = H * hd, Hk * hd, 16

    def operand(K):
        return rows * K * 4 + rows * (K // 64) * 4

    if kind == "qkv":
        return matrix_bytes(f, qd + 2 * kd, d) + operand(d) + B * (qd * 4 + 2 * kd * 2)
    if kind == "oproj":
        return matrix_bytes(f, d, qd) + operand(qd) + B * d * 4 * 4      # up to four K slices
    if kind == "fc":
        return matrix_bytes(f, 2 * ff, d) + operand(d) + B * ff * 4
    if kind == "down":
        return matrix_bytes(f, d, ff) + operand(ff) + B * d * 4 * 4
    if kind == "head":
        mats = matrix_bytes(f, c["vocab"], d) + (C - 1) * matrix_bytes(f, c["cp_vocab"], d)
        return mats / C + operand(d) + B * 4 * (c["vocab"] + (C - 1) * c["cp_vocab"]) / C
    if kind == "qkv_attn":   # the QKV product and the attention in one launch
        return frame_kernel_bytes(c, "qkv", pos) + frame_kernel_bytes(c, "attn", pos)
    if kind == "attn":
        keys = L * (pos + 1) + Lc * sum(j + 1 for j in range(C))
        n_launch = L + Lc * C
        return (B * keys * 2 * kd * 2 + n_launch * B * (qd * 4 + H * 2 * (hd + 4) * 4)) / n_launch
    raise KeyError(kind)


def mean_kernel_bytes(c, kind: str, first_pos: int, n_steps: int) -> float:
    if c["arch"] == "talker_cp":
        return sum(frame_kernel_bytes(c, kind, p) for p in range(first_pos, first_pos + n_steps)) / n_steps
    return sum(kernel_bytes(c, kind, p) for p in range(first_pos, first_pos + n_steps)) / n_steps
