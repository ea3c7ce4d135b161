"""GPU parity of the standalone kernels (fused dequant GEMV, split-KV attention) against the
CPU oracle, through the C ABI.  Tolerance: rel = max|got-ref| / max|ref| <= 2e-3 per output
tensor; the GEMV is also held to the fp32 accumulation bound."""
import sys

import numpy as np
import pytest

import oracle
from parity import REL_TOL, rel_err
from quantized_gemv_kv_amd import synth

pytestmark = pytest.mark.gpu


def _t():
    import torch
    return torch


def dev(a):
    torch = _t()
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


GEMV_CASES = [
    ("q8_0", 1024, 1024, 1),     # the lone Q8_0 GEMV workload (1024 x 1024, batch 1)
    ("q8_0", 1024, 1024, 3),
    ("q8_0", 4096, 1024, 1),
    ("q8_0", 1024, 4096, 1),     # one row spans four loads
    ("q8_0", 8192, 1024, 1),
    ("q4_0", 3072, 1024, 1),     # GPT-2-Medium fused QKV
    ("q4_0", 4096, 1024, 2),
    ("q4_0", 1024, 4096, 1),     # down projection
    ("q4_0", 8192, 1024, 1),     # head
    ("aff8", 4096, 1024, 1),     # Talker fused QKV (2048 + 1024 + 1024)
    ("aff8", 1024, 2048, 1),
    ("aff8", 1024, 3072, 4),     # three loads per row, last one partly idle
    ("q4_0", 40, 128, 1),        # ragged: not a multiple of the rows per block
    ("q8_0", 7, 64, 2),
    ("aff8", 3, 64, 1),
    ("q4_0", 1, 32, 1),          # one slot per row, 128 rows per wave, one real row
    ("q4_0", 130, 256, 1),
    ("q5_0", 3072, 1024, 1),     # the journal's third T3 quantisation
    ("q5_0", 1024, 4096, 2),     # rows spanning two loads
    ("q5_0", 40, 128, 1),
    ("aff4_g64", 4096, 1024, 1), # 4-bit affine, groups of 64
    ("aff4_g64", 1024, 3072, 1),
    ("aff4_g64", 3, 64, 3),
    ("aff4_g32", 4096, 1024, 1), # and of 32
    ("aff4_g32", 1024, 2048, 4),
    ("aff4_g32", 5, 32, 1),
    ("q4_0", 1000, 1024, 2),     # eight rows per lane (rows of 32 lanes), a ragged last tile
    ("aff4_g64", 1000, 1024, 1),
    ("aff4_g32", 70, 1024, 1),
    ("q5_0", 65, 1024, 1),
]


@pytest.mark.parametrize("fmt,N,K,B", GEMV_CASES)
def test_gemv_matches_oracle(fmt, N, K, B):
    torch = _t()
    say(f"[gemv] fmt={fmt} N={N} K={K} B={B}")
    rng = synth.rng_for(11, N, K, B)
    blob = synth.matrix(fmt, rng, N, K)
    x = synth.normal_f32(rng, (B, K))
    bias = synth.normal_f32(rng, (N,), 0.5)
    ref = oracle.gemv_f32(fmt, blob, N, K, x, bias)
    from quantized_gemv_kv_amd import binding as tb
    packed = torch.empty(tb.tsd_gemv_packed_bytes(fmt, N, K), dtype=torch.uint8, device="cuda")
    tb.tsd_gemv_pack(fmt, dev(blob), N, K, packed)
    y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    tb.tsd_gemv(fmt, packed, N, K, B, dev(x), dev(bias), y)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    assert rel_err(got, ref) <= REL_TOL
    # fp32 accumulation bound, row by row: |err| <= 4 K u sum_k |w x| + |b| u
    W = oracle.dequant(fmt, blob, N, K)
    mag = np.abs(x.astype(np.float64)) @ np.abs(W).T + np.abs(bias)
    assert np.all(np.abs(got - ref) <= 4 * K * 2.0 ** -24 * mag + 1e-30)


DEBUG_GEMV_CASES = [(f, N, K, B) for f in ("q4_0", "q8_0", "aff8", "q5_0", "aff4_g64", "aff4_g32")
                    for (N, K, B) in ((37, 128, 3), (300, 1024, 1), (64, 192 if f in ("aff8", "aff4_g64") else 96, 2))]


@pytest.mark.parametrize("fmt,N,K,B", DEBUG_GEMV_CASES)
def test_debug_gemv_on_canonical_blocks(fmt, N, K, B):
    """tsd_debug_gemv decodes the canonical blob itself (no repacking): against the oracle's fp64
    mat-vec, within the fp32 bound of a K-long sequential sum, and equal to the packed kernel's
    result to the same bound."""
    torch = _t()
    from quantized_gemv_kv_amd import binding as tb
    say(f"[debug-gemv] fmt={fmt} N={N} K={K} B={B}")
    rng = synth.rng_for(17, N, K, B)
    blob = synth.matrix(fmt, rng, N, K)
    x = synth.normal_f32(rng, (B, K))
    ref = oracle.gemv_f32(fmt, blob, N, K, x, None)
    y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    tb.tsd_debug_gemv(fmt, dev(blob), dev(x), y, N, K, B)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    W = oracle.dequant(fmt, blob, N, K)
    mag = np.abs(x.astype(np.float64)) @ np.abs(W).T
    assert np.all(np.abs(got - ref) <= 2 * K * 2.0 ** -24 * mag + 1e-30)
    assert rel_err(got, ref) <= 1e-5
    with pytest.raises(tb.TsdError) as e:
        tb.tsd_debug_gemv(fmt, dev(blob[:-1]), dev(x), y, N, K, B)       # not the canonical size
    assert e.value.status == 1


def test_tall_gemv_sampled_rows():
    """The tall Q8_0 GEMV the benchmark times (524288 x 1024, ~570 MB), in the same launch
    configuration; 96 sampled rows checked against the oracle row by row."""
    torch = _t()
    from quantized_gemv_kv_amd import binding as tb
    N, K, seed = 524288, 1024, 42
    say("[gemv] tall q8_0 524288 x 1024")
    row_b = K // 32 * 34
    canon = torch.empty(N * row_b, dtype=torch.uint8, device="cuda")
    rows = np.sort(synth.rng_for(5).choice(N, size=96, replace=False))
    rows = np.concatenate([[0, N - 1], rows])
    blobs = {}
    for r0, blob in synth.q8_0_row_chunks(N, K, seed):
        canon[r0 * row_b: r0 * row_b + blob.size].copy_(torch.from_numpy(blob))
        for r in rows[(rows >= r0) & (rows < r0 + blob.size // row_b)]:
            blobs[int(r)] = blob[(r - r0) * row_b:(r - r0 + 1) * row_b].copy()
    packed = torch.empty(tb.tsd_gemv_packed_bytes("q8_0", N, K), dtype=torch.uint8, device="cuda")
    tb.tsd_gemv_pack("q8_0", canon, N, K, packed)
    del canon
    x = synth.normal_f32(synth.rng_for(seed, 1), (1, K))
    y = torch.full((1, N), float("nan"), dtype=torch.float32, device="cuda")
    tb.tsd_gemv("q8_0", packed, N, K, 1, dev(x), None, y)
    torch.cuda.synchronize()
    got = y.cpu().numpy()[0]
    assert np.all(np.isfinite(got))
    ref = np.array([oracle.gemv_f32("q8_0", blobs[int(r)], 1, K, x, None)[0, 0] for r in rows])
    assert rel_err(got[rows], ref) <= REL_TOL


def test_gemv_rejects_bad_shapes():
    torch = _t()
    from quantized_gemv_kv_amd import binding as tb
    with pytest.raises(tb.TsdError):
        tb.tsd_gemv_packed_bytes("q4_0", 16, 48)                     # K not a multiple of 32
    p = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    x = torch.zeros(8192, dtype=torch.float32, device="cuda")
    with pytest.raises(tb.TsdError):
        tb.tsd_gemv("q8_0", p, 4, 96, 1, x, None, x)                  # 6 slots per row: no lane mapping
    with pytest.raises(tb.TsdError):
        tb.tsd_gemv("q8_0", p, 4, 64, 5, x, None, x)                  # batch > 4


ATTN_CASES = [
    # hd, H, Hkv, B, n_keys, n_ctx, q scale
    (64, 16, 16, 1, 1, 1024, 1.0),
    (64, 16, 16, 1, 63, 1024, 1.0),
    (64, 16, 16, 1, 64, 1024, 1.0),
    (64, 16, 16, 1, 65, 1024, 1.0),
    (64, 16, 16, 1, 513, 1024, 1.0),   # one GPT-2-Medium layer after 512 cached positions
    (64, 16, 16, 1, 757, 1024, 4.0),   # peaked softmax
    (64, 16, 16, 1, 1024, 1024, 1.0),  # full context
    (128, 16, 8, 2, 300, 512, 1.0),    # GQA 16/8, head 128
    (128, 16, 8, 16, 17, 64, 2.0),     # predictor-sized cache, batch 16
    (64, 4, 1, 1, 200, 256, 1.0),      # all heads share one KV head
]


@pytest.mark.parametrize("hd,H,Hkv,B,n_keys,n_ctx,qs", ATTN_CASES)
def test_attention_matches_oracle(hd, H, Hkv, B, n_keys, n_ctx, qs):
    torch = _t()
    from quantized_gemv_kv_amd import binding as tb
    say(f"[attn] hd={hd} H={H} Hkv={Hkv} B={B} n_keys={n_keys} n_ctx={n_ctx}")
    rng = synth.rng_for(5, hd, H, n_keys)
    q = synth.normal_f32(rng, (B, H, hd), qs)
    k = synth.fp16_cache(rng, (B, Hkv, n_ctx, hd))
    v = synth.fp16_cache(rng, (B, Hkv, n_ctx, hd))
    ref = np.empty((B, H, hd))
    for b in range(B):
        for h in range(H):
            g = h // (H // Hkv)
            ref[b, h] = oracle.attend(q[b, h], k[b, g, :n_keys], v[b, g, :n_keys])
    scratch = torch.empty(tb.tsd_attention_scratch_bytes(B, H, n_ctx, hd), dtype=torch.uint8, device="cuda")
    out = torch.full((B, H, hd), float("nan"), dtype=torch.float32, device="cuda")
    dq, dk, dv = dev(q), dev(k), dev(v)
    for rep in range(2):           # the split counters must be left at zero for the next call
        tb.tsd_attention(dq, dk, dv, B, H, Hkv, hd, n_keys, n_ctx, out, scratch)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.all(np.isfinite(got))
        assert rel_err(got, ref) <= REL_TOL, rep
        assert rel_err(got, ref) <= 1e-5, rep
