"""Pins of the oracle's sampler chain (CPU only).

The chain is temperature, top-k, top-p, repetition penalty in the T3 port's order and
repetition penalty, temperature, min-p, top-p, top-k in the multilingual T3's order ("Chatterbox
-> ggml Port: Development Journal", §3.2 issues 7-8 and §3.19 "Sampling path").  The pins use
distributions whose nucleus, min-p set and penalized weights are known in closed form, the
reduction to the separately pinned top-k draw when every filter is off, and invariants of the
mathematics (the penalty commutes with the temperature; duplicates in the history do not count
twice)."""
import numpy as np
import pytest

import oracle
from quantized_gemv_kv_amd import synth

GRID = (np.arange(4000) + 0.5) / 4000   # u on a fine grid: the fraction mapping to an id is its mass


def freqs(logits, n, **kw):
    ids = [oracle.sample_chain(logits, u, **kw)[0] for u in GRID]
    return np.bincount(ids, minlength=n) / len(GRID)


# probabilities 1/2, 1/4, 1/8, 1/16, 1/16 (the last two tied: the lower index ranks first)
P5 = np.array([0.5, 0.25, 0.125, 0.0625, 0.0625])
L5 = np.log(P5)


def test_every_filter_off_is_the_topk_draw():
    rng = np.random.default_rng(3)
    for n, k, T in [(50, 5, 0.8), (50, 50, 1.0), (300, 1, 1.0), (300, 37, 1.7)]:
        v = np.round(rng.normal(0, 2.0, n) * 32) / 32
        for u in rng.random(60):
            ref = oracle.sample_topk(v, k, T, u)
            for order in ("t3", "mtl"):
                got, _ = oracle.sample_chain(v, u, top_k=k, temperature=T, order=order)
                assert got == ref, (n, k, T, u, order)


@pytest.mark.parametrize("order", ["t3", "mtl"])
def test_top_p_nucleus_in_closed_form(order):
    # p = 0.7: ranks 0 (preceding mass 0) and 1 (0.5) stay, rank 2 (0.75) goes -> masses 2/3, 1/3
    f = freqs(L5, 5, top_p=0.7, order=order)
    assert np.allclose(f, [2 / 3, 1 / 3, 0, 0, 0], atol=1e-3)
    # p = 0.8: rank 2 (preceding 0.75) stays too -> 4/7, 2/7, 1/7
    f = freqs(L5, 5, top_p=0.8, order=order)
    assert np.allclose(f, [4 / 7, 2 / 7, 1 / 7, 0, 0], atol=1e-3)
    # a tiny p keeps only the largest; p = 1 (or 0) switches the filter off
    assert np.allclose(freqs(L5, 5, top_p=1e-6, order=order), [1, 0, 0, 0, 0])
    assert np.allclose(freqs(L5, 5, top_p=1.0, order=order), P5, atol=1e-3)


def test_top_p_acts_on_the_topk_survivors_in_t3_order():
    # T3: top-k (k = 3) first renormalises over {1/2, 1/4, 1/8} (4/7, 2/7, 1/7); top-p 0.8 then
    # sees preceding masses 0, 4/7, 6/7 and drops rank 2 -> 2/3, 1/3
    f = freqs(L5, 5, top_k=3, top_p=0.8, order="t3")
    assert np.allclose(f, [2 / 3, 1 / 3, 0, 0, 0], atol=1e-3)
    # MTL: top-p 0.8 over the whole vocabulary keeps three (preceding 0.75 < 0.8), top-k 3 keeps them
    f = freqs(L5, 5, top_k=3, top_p=0.8, order="mtl")
    assert np.allclose(f, [4 / 7, 2 / 7, 1 / 7, 0, 0], atol=1e-3)


def test_min_p_in_closed_form():
    # keep p_i >= min_p * 1/2
    assert np.allclose(freqs(L5, 5, min_p=0.3, order="mtl"), [2 / 3, 1 / 3, 0, 0, 0], atol=1e-3)
    assert np.allclose(freqs(L5, 5, min_p=0.2, order="mtl"), [4 / 7, 2 / 7, 1 / 7, 0, 0], atol=1e-3)
    assert np.allclose(freqs(L5, 5, min_p=0.1, order="mtl"), P5, atol=1e-3)
    # min-p precedes top-p: over {4/7, 2/7, 1/7}, p = 0.6 keeps ranks with preceding mass < 0.6
    f = freqs(L5, 5, min_p=0.2, top_p=0.6, order="mtl")
    assert np.allclose(f, [2 / 3, 1 / 3, 0, 0, 0], atol=1e-3)


def test_temperature_reshapes_before_the_nucleus():
    # T = 1/2 squares the probabilities: 1/4, 1/16, 1/64, 1/256, 1/256 over their sum
    q = P5 ** 2 / np.sum(P5 ** 2)
    assert np.allclose(freqs(L5, 5, temperature=0.5), q, atol=1e-3)
    # nucleus 0.9 of q: preceding masses 0, 0.7529, 0.9412 -> ranks 0 and 1
    assert np.allclose(freqs(L5, 5, temperature=0.5, top_p=0.9), np.array([4, 1, 0, 0, 0]) / 5, atol=1e-3)


def test_repetition_penalty_divides_positive_and_multiplies_negative():
    v = np.array([2.0, 2.0, -1.0, 0.5])
    hist = [0, 2]
    pen = np.array([1.0, 2.0, -2.0, 0.5])            # 2 / 2, untouched, -1 * 2, untouched
    w = np.exp(pen) / np.exp(pen).sum()
    for order in ("t3", "mtl"):
        assert np.allclose(freqs(v, 4, rep_penalty=2.0, hist=hist, order=order), w, atol=1e-3)
    # greedy with the penalty: the argmax of the penalized logits (index 1, not the tie-winner 0)
    assert oracle.sample_chain(v, 0.5, mode=0, rep_penalty=2.0, hist=hist)[0] == 1
    assert oracle.sample_chain(v, 0.5, mode=0, rep_penalty=1.0, hist=hist)[0] == 0


def test_penalty_position_in_the_chain_matters_only_for_the_filters():
    v = np.array([2.0, 2.0, -1.0, 0.5])
    # top-k 1: T3 keeps the raw maximum (index 0, lower index of the tie) and penalizes it after;
    # MTL penalizes first, so index 1 is the maximum
    for u in (0.1, 0.5, 0.9):
        assert oracle.sample_chain(v, u, top_k=1, rep_penalty=2.0, hist=[0], order="t3")[0] == 0
        assert oracle.sample_chain(v, u, top_k=1, rep_penalty=2.0, hist=[0], order="mtl")[0] == 1
    # with no filter cutting, the two orders are the same distribution: the penalty and the
    # temperature are both multiplicative, so pen(l / T) = pen(l) / T
    rng = np.random.default_rng(5)
    for _ in range(5):
        x = rng.normal(0, 2, 64)
        h = rng.integers(0, 64, 20)
        for u in rng.random(40):
            a = oracle.sample_chain(x, u, temperature=0.7, rep_penalty=1.3, hist=h, order="t3")[0]
            b = oracle.sample_chain(x, u, temperature=0.7, rep_penalty=1.3, hist=h, order="mtl")[0]
            assert a == b


def test_history_counts_each_id_once_and_ignores_out_of_range():
    v = np.array([1.5, -0.5, 0.25, 3.0, -2.0])
    rng = np.random.default_rng(8)
    for u in rng.random(50):
        a = oracle.sample_chain(v, u, rep_penalty=1.7, hist=[3, 1])
        b = oracle.sample_chain(v, u, rep_penalty=1.7, hist=[3, 3, 1, 1, 3, -1, 5, 99])
        assert a[0] == b[0]
    # penalty 1 (or 0) is off whatever the history
    for u in rng.random(20):
        assert oracle.sample_chain(v, u, rep_penalty=1.0, hist=[0, 1, 2, 3, 4])[0] == oracle.sample_chain(v, u)[0]
        assert oracle.sample_chain(v, u, rep_penalty=0.0, hist=[0, 1, 2, 3, 4])[0] == oracle.sample_chain(v, u)[0]


def test_margins_locate_the_boundaries():
    # u exactly on the first cumulative boundary (1/2 of P5) gives a draw margin of ~0
    _, m = oracle.sample_chain(L5, 0.5)
    assert m["draw"] < 1e-12
    # top-p exactly at a preceding mass (0.75) gives a top-p margin of ~0
    _, m = oracle.sample_chain(L5, 0.3, top_p=0.75)
    assert m["top_p"] < 1e-12
    _, m = oracle.sample_chain(L5, 0.3, min_p=0.25, order="mtl")
    assert m["min_p"] < 1e-12
    _, m = oracle.sample_chain(np.array([1.0, 3.0, 2.0]), 0.3, top_k=2)
    assert m["top_k"] == pytest.approx(1.0)
    # the drawn entry's neighbours in the walk: 1.0001 and 1.0 are nearly equal, the crossing
    # lands on rank 1 (index 0, value 1.0) whose neighbours are 1.0001 above and 0 below
    i, m = oracle.sample_chain(np.array([1.0, 1.0001, 0.0]), 0.6)
    assert i == 0 and m["order"] == pytest.approx(1e-4, rel=1e-6)


def test_model_records_the_consumed_tokens_for_the_penalty():
    """Greedy with an overwhelming penalty: a consumed token keeps a tiny positive logit or gets a
    hugely negative one, so the model picks an unconsumed id whenever one has a positive logit."""
    cfg = synth.small_config("llama", "q8_0", sample_mode=0, rep_penalty=1e6)
    w = synth.model_weights(cfg, seed=11)
    m = oracle.OracleModel(cfg, w)
    prompt = np.array([[5, 17, 5, 40]], np.int32)
    nxt = m.prefill(prompt)
    consumed = set(prompt.ravel().tolist())
    checked = 0
    for _ in range(12):
        lg = m.logits()[0]
        unseen_pos = [i for i in range(cfg["vocab"]) if i not in consumed and lg[i] > 1e-3]
        if unseen_pos:
            assert int(nxt.ravel()[0]) not in consumed
            checked += 1
        tok = int(nxt.ravel()[0])
        consumed.add(tok)
        nxt = m.step(np.array([[tok]], np.int32))
    assert checked >= 8
