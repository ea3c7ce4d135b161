"""GPU top-k draw (tsd_sample_topk, the kernel the step uses) against the oracle's draw on the
same logits and the same counter-based uniform.  Logits are multiples of 1/64 (exact in fp32 and
fp64), with repeated values so that ties matter; a draw within 1e-4 of a cumulative-mass
boundary may differ between fp32 and fp64 and is skipped."""
import sys

import numpy as np
import pytest

import oracle
from parity import DRAW_MARGIN, topk_draw_margins

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_draw(logits, k, T, seed, row, pos, pss):
    import torch
    from quantized_gemv_kv_amd import binding
    x = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda()
    out = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    binding.tsd_sample_topk(x, k, T, seed, row, pos, pss, out)
    torch.cuda.synchronize()
    return int(out.item())


def crafted_logits(n, seed, spread=3.0):
    rng = np.random.default_rng(seed)
    v = np.round(rng.normal(0.0, spread, n) * 64.0) / 64.0
    # repeated values: copies of the largest few and of a middling one
    idx = rng.choice(n, size=min(n, 12), replace=False)
    v[idx[:4]] = v.max()
    v[idx[4:8]] = np.sort(v)[-10]
    return v.astype(np.float32)


@pytest.mark.parametrize("n,k,T", [(160, 5, 0.8), (160, 160, 1.0), (1000, 50, 0.9), (1000, 1, 1.0),
                                   (8192, 50, 0.9), (8192, 1024, 2.0), (8192, 7, 0.5), (3072, 256, 1.0)])
def test_topk_draw_matches_oracle(n, k, T):
    say(f"[sampler] n={n} k={k} T={T}")
    seed = 1234 + n + k
    v = crafted_logits(n, seed)
    checked = 0
    for pos in range(40):
        u = oracle.uniform24(seed, 0, pos, 0)
        ref = oracle.sample_topk(v, k, T, u)
        got = gpu_draw(v, k, T, seed, 0, pos, 0)
        margin, _ = topk_draw_margins(v, k, T, u)
        if margin < DRAW_MARGIN:
            continue
        assert got == ref, (pos, got, ref, margin)
        checked += 1
    assert checked >= 30


def test_uniform_logits_pin_the_counter_generator():
    """n equal logits, k = n: the draw is floor(u * n) exactly, so the GPU's Philox4x64-10
    uniform must equal the oracle's (its top 10 bits, for n = 1024) at every counter."""
    n = 1024
    v = np.zeros(n, np.float32)
    for seed in (0, 1, 0xDEADBEEFCAFEF00D):
        for row, pos, pss in [(0, p, 0) for p in range(50)] + [(3, 17, 5), (15, 1000, 14), (1, 2, 3)]:
            u = oracle.uniform24(seed, row, pos, pss)
            assert gpu_draw(v, n, 1.0, seed, row, pos, pss) == int(np.floor(u * n)), (seed, row, pos, pss)


def test_ties_go_to_the_lowest_index():
    v = np.zeros(300, np.float32)
    v[[17, 99, 250]] = 5.0
    for pos in range(5):
        assert gpu_draw(v, 1, 1.0, 7, 0, pos, 0) == 17
    # k = 3 keeps exactly the three tied maxima; their order is by index
    seen = {gpu_draw(v, 3, 1.0, 7, 0, pos, 0) for pos in range(60)}
    assert seen <= {17, 99, 250} and len(seen) == 3


def test_rejects_bad_arguments():
    from quantized_gemv_kv_amd import TsdError
    v = np.zeros(64, np.float32)
    with pytest.raises(TsdError) as e:
        gpu_draw(v, 5, 0.0, 1, 0, 0, 0)
    assert e.value.status == 1
    with pytest.raises(TsdError) as e:
        gpu_draw(np.zeros(4096, np.float32), 2000, 1.0, 1, 0, 0, 0)
    assert e.value.status == 2
