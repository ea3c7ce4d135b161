"""GPU top-k draw (tsd_sample_topk, the kernel the step uses) against the oracle's draw on the
same logits and the same counter-based uniform.  Logits are multiples of 1/64 (exact in fp32 and
fp64), with repeated values so that ties matter; a draw within 1e-4 of a cumulative-mass
boundary may differ between fp32 and fp64 and is skipped."""
import sys

import numpy as np
import pytest

import oracle
from parity import DRAW_MARGIN, chain_near_boundary, topk_draw_margins

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


# ---- the sampler chain (tsd_sample) -------------------------------------------------------------

def gpu_chain(logits, samp, hist, row, pos, pss):
    import torch
    from quantized_gemv_kv_amd import binding
    x = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda()
    h = torch.from_numpy(np.ascontiguousarray(hist, np.int32)).cuda() if len(hist) else None
    out = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    binding.tsd_sample(x, samp, h, row, pos, pss, out)
    torch.cuda.synchronize()
    return int(out.item())


CHAIN_CASES = [
    # n, sampling, history length
    (160, dict(mode=1, top_k=50, temperature=0.8, top_p=0.9, rep_penalty=1.3, order="t3"), 30),
    (1000, dict(mode=1, top_k=1000, temperature=0.8, top_p=0.95, rep_penalty=1.2, order="t3"), 200),
    (8192, dict(mode=1, top_k=1000, temperature=0.8, top_p=0.95, rep_penalty=1.2, order="t3"), 700),
    (8192, dict(mode=1, top_k=50, temperature=0.9, top_p=0.95, rep_penalty=1.05, order="t3"), 300),
    (8192, dict(mode=1, top_k=1000, temperature=0.8, min_p=0.05, top_p=0.95, rep_penalty=2.0, order="mtl"), 700),
    (3072, dict(mode=1, top_k=200, temperature=1.1, min_p=0.02, top_p=0.8, rep_penalty=1.3, order="mtl"), 100),
    (2048, dict(mode=1, top_k=300, temperature=0.7, top_p=0.5, order="t3"), 0),
    (2048, dict(mode=1, top_k=1000, temperature=1.0, min_p=0.1, order="mtl"), 0),
    (8192, dict(mode=0, rep_penalty=1.5), 500),
    (12288, dict(mode=1, top_k=64, temperature=0.9, top_p=0.9, rep_penalty=1.1, order="mtl"), 1000),
]


@pytest.mark.parametrize("n,samp,nh", CHAIN_CASES)
def test_chain_draw_matches_oracle(n, samp, nh):
    say(f"[sampler] chain n={n} {samp} history {nh}")
    seed = 4242 + n + nh
    samp = dict(samp, seed=seed)
    rng = np.random.default_rng(seed)
    checked = 0
    for pos in range(30):
        v = crafted_logits(n, seed + 7 * pos)   # fresh logits: a cut near its boundary stays one case
        # a history drawn mostly from the largest logits, so the penalty reorders the top
        top = np.argsort(-v, kind="stable")[:64]
        hist = np.concatenate([rng.choice(top, size=nh // 2), rng.integers(0, n, nh - nh // 2)]).astype(np.int32) \
            if nh else np.zeros(0, np.int32)
        hist[: min(3, nh)] = [-1, n, n + 5][: min(3, nh)]          # out-of-range ids are ignored
        u = oracle.uniform24(seed, 2, pos, 1)
        ref, mg = oracle.sample_chain(v, u, mode=samp["mode"], top_k=samp.get("top_k", 0),
                                      temperature=samp.get("temperature", 1.0), top_p=samp.get("top_p", 0.0),
                                      min_p=samp.get("min_p", 0.0), rep_penalty=samp.get("rep_penalty", 1.0),
                                      order=samp.get("order", "t3"), hist=hist)
        got = gpu_chain(v, samp, hist, 2, pos, 1)
        # identical fp32 inputs on both sides: only fp32 rounding of the scans separates them
        if chain_near_boundary(mg, mass_tol=2e-5, gap_tol=1e-5):
            continue
        assert got == ref, (pos, got, ref, mg)
        checked += 1
    assert checked >= 20


def test_chain_penalty_changes_the_pick():
    """One logit far above the rest: without a history it is always drawn; once it is in the
    history a huge penalty sends its (positive) logit to about 0, below the others."""
    n = 512
    v = np.full(n, 1.0, np.float32)
    v[100] = 40.0
    samp = dict(mode=1, top_k=n, temperature=1.0, rep_penalty=1e4, order="t3", seed=1)
    for pos in range(10):
        assert gpu_chain(v, samp, [], 0, pos, 0) == 100
        assert gpu_chain(v, samp, [100, 100, 7], 0, pos, 0) != 100
    g = dict(mode=0, rep_penalty=1e4)
    assert gpu_chain(v, g, [], 0, 0, 0) == 100
    assert gpu_chain(v, g, [100], 0, 0, 0) == 0       # every other logit ties at 1: lowest index


def test_chain_rejects_bad_arguments():
    from quantized_gemv_kv_amd import TsdError
    v = np.zeros(64, np.float32)
    for bad in (dict(mode=1, top_p=1.5), dict(mode=1, min_p=0.1, order="t3"), dict(mode=1, min_p=1.0, order="mtl"),
                dict(mode=1, rep_penalty=-1.0), dict(mode=1, order=7), dict(mode=2), dict(mode=1, temperature=0.0),
                dict(mode=1, cfg=1, cfg_weight=0.5), dict(mode=1, cfg=2)):
        with pytest.raises(TsdError) as e:
            gpu_chain(v, dict(dict(temperature=1.0), **bad), [], 0, 0, 0)
        assert e.value.status == 1, bad
    with pytest.raises(TsdError) as e:
        gpu_chain(np.zeros(4096, np.float32), dict(mode=1, top_k=2000, temperature=1.0), [], 0, 0, 0)
    assert e.value.status == 2
