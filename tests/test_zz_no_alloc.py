"""tsd_attention_noalloc (the split-KV attention with the library's own per-GPU partials array,
for callers that cannot allocate) against tsd_attention (caller scratch), through the C ABI: two
calls in a row, the second on a smaller input, each equal to tsd_attention's output bit for bit
(the same kernels) and within 1e-5 of the oracle; a shape whose partials exceed the array is
rejected on the host before anything is launched."""
import sys

import numpy as np
import pytest

import oracle
from parity import rel_err
from quantized_gemv_kv_amd import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def one_call(hd, H, Hkv, B, n_keys, n_ctx, seed):
    import torch
    from quantized_gemv_kv_amd import binding as tb
    say(f"[noalloc] hd={hd} H={H} Hkv={Hkv} B={B} n_keys={n_keys} n_ctx={n_ctx}")
    assert tb.tsd_attention_scratch_bytes(B, H, n_ctx, hd) <= tb.NOALLOC_SCRATCH_BYTES
    rng = synth.rng_for(seed, hd, H, n_keys)
    q = synth.normal_f32(rng, (B, H, hd))
    k = synth.fp16_cache(rng, (B, Hkv, n_ctx, hd))
    v = synth.fp16_cache(rng, (B, Hkv, n_ctx, hd))
    dq, dk, dv = dev(q), dev(k), dev(v)
    scratch = torch.empty(tb.tsd_attention_scratch_bytes(B, H, n_ctx, hd), dtype=torch.uint8, device="cuda")
    want = torch.full((B, H, hd), float("nan"), dtype=torch.float32, device="cuda")
    got = torch.full((B, H, hd), float("nan"), dtype=torch.float32, device="cuda")
    tb.tsd_attention(dq, dk, dv, B, H, Hkv, hd, n_keys, n_ctx, want, scratch)
    tb.tsd_attention_noalloc(dq, dk, dv, B, H, Hkv, hd, n_keys, n_ctx, got)
    torch.cuda.synchronize()
    want, got = want.cpu().numpy(), got.cpu().numpy()
    assert np.all(np.isfinite(got))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    b, h = B - 1, H - 1
    ref = oracle.attend(q[b, h], k[b, h // (H // Hkv), :n_keys], v[b, h // (H // Hkv), :n_keys])
    assert rel_err(got[b, h], ref) <= 1e-5


def test_attention_noalloc_matches_attention_twice():
    # a 16-row Talker-shaped call over 1,900 keys (eight chunks; 2.2 MB of partials), then a
    # smaller GPT-2-shaped one over 300 keys: the second call reuses the array the first filled
    one_call(128, 16, 8, 16, 1900, 2048, seed=1)
    one_call(64, 16, 16, 1, 300, 512, seed=2)


def test_attention_noalloc_rejects_shapes_beyond_its_array():
    import torch
    from quantized_gemv_kv_amd import binding as tb
    B, H, hd, n_ctx = 16, 32, 128, 8192           # 17.3 MB of partials
    assert tb.tsd_attention_scratch_bytes(B, H, n_ctx, hd) > tb.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(1, dtype=torch.float32, device="cuda")
    with pytest.raises(tb.TsdError) as e:
        tb.tsd_attention_noalloc(x, x, x, B, H, H, hd, 10, n_ctx, x)
    assert e.value.status == 1
