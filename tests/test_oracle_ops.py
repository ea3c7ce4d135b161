"""Pins of the oracle's operators against closed forms, library routines (torch CPU fp64,
numpy) and invariants (CPU only)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from quantized_gemv_kv_amd import synth


def _blob(fmt, N, K, seed=0):
    return synth.matrix(fmt, synth.rng_for(seed, N, K), N, K)


# ---- GEMV ------------------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", "aff8", "q5_0", "aff4_g64", "aff4_g32"])
@pytest.mark.parametrize("N,K", [(32, 64), (96, 128), (5, 1024), (64, 192)])
def test_gemv_matches_dense_matmul(orc, fmt, N, K):
    if fmt in ("aff8", "aff4_g64") and K % 64:
        pytest.skip("affine groups are 64 wide")
    blob = _blob(fmt, N, K)
    W = orc.dequant(fmt, blob, N, K)
    x = np.random.default_rng(1).standard_normal(K)
    b = np.random.default_rng(2).standard_normal(N)
    y = orc.gemv(fmt, blob, N, K, x, b)
    ref = torch.from_numpy(W) @ torch.from_numpy(x) + torch.from_numpy(b)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12 * np.abs(W).sum())


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", "aff8", "q5_0", "aff4_g64", "aff4_g32"])
def test_gemv_one_hot_selects_a_column_exactly(orc, fmt):
    N, K = 40, 128
    blob = _blob(fmt, N, K, 3)
    W = orc.dequant(fmt, blob, N, K)
    for k in (0, 31, 32, 63, 64, 127):
        x = np.zeros(K)
        x[k] = 1.0
        assert np.array_equal(orc.gemv(fmt, blob, N, K, x), W[:, k])


def test_gemv_single_nonzero_block_and_transpose(orc):
    # only block 2 of row 1 is non-zero: y picks up exactly that block's dot product and
    # nothing leaks into other rows (a transposed operand would spread it)
    N, K = 3, 128
    blob = np.zeros(orc.matrix_bytes("q8_0", N, K), np.uint8).reshape(N, K // 32, 34)
    blob[1, 2, 0:2] = [0x00, 0x38]                           # d = 0.5
    blob[1, 2, 2:] = np.arange(1, 33, dtype=np.int8).view(np.uint8)
    x = np.arange(K, dtype=np.float64)
    y = orc.gemv("q8_0", blob.reshape(-1), N, K, x)
    assert y[0] == 0.0 and y[2] == 0.0
    assert y[1] == 0.5 * float(np.dot(np.arange(1, 33), np.arange(64, 96)))


def test_gemv_f32_batch_rows_independent(orc):
    N, K, B = 24, 96, 3
    blob = _blob("q4_0", N, K, 5)
    x = np.random.default_rng(4).standard_normal((B, K)).astype(np.float32)
    y = orc.gemv_f32("q4_0", blob, N, K, x)
    for r in range(B):
        np.testing.assert_array_equal(y[r], orc.gemv("q4_0", blob, N, K, x[r].astype(np.float64)))


# ---- norms and activations -------------------------------------------------------------------

def test_layernorm_matches_torch_and_normalises(orc):
    rng = np.random.default_rng(7)
    x = rng.standard_normal(1024) * 3 + 1.5
    g, b = rng.standard_normal(1024), rng.standard_normal(1024)
    y = orc.layernorm(x, g, b, 1e-5)
    ref = F.layer_norm(torch.from_numpy(x), (1024,), torch.from_numpy(g), torch.from_numpy(b), 1e-5)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)
    z = orc.layernorm(x, None, None, 0.0)
    assert abs(z.mean()) < 1e-12 and abs(z.var() - 1.0) < 1e-12
    np.testing.assert_allclose(orc.layernorm(7.0 * x, None, None, 0.0), z, atol=1e-12)


def test_rmsnorm_matches_torch_and_normalises(orc):
    rng = np.random.default_rng(8)
    x = rng.standard_normal(1024) * 2 + 0.3
    g = rng.standard_normal(1024)
    y = orc.rmsnorm(x, g, 1e-5)
    ref = F.rms_norm(torch.from_numpy(x), (1024,), torch.from_numpy(g), 1e-5)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)
    z = orc.rmsnorm(x, None, 0.0)
    assert abs(np.sqrt(np.mean(z * z)) - 1.0) < 1e-12
    assert np.all(np.sign(z) == np.sign(x))


def test_gelu_tanh(orc):
    xs = np.linspace(-8, 8, 321)
    got = np.array([orc.gelu_tanh(v) for v in xs])
    ref = F.gelu(torch.from_numpy(xs), approximate="tanh").numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)
    assert orc.gelu_tanh(0.0) == 0.0
    np.testing.assert_allclose(got - got[::-1], xs, atol=1e-13)        # GELU(x) - GELU(-x) = x
    exact = F.gelu(torch.from_numpy(xs)).numpy()                         # erf form: close, not equal
    assert 0 < np.abs(got - exact).max() < 1e-3


def test_silu(orc):
    xs = np.linspace(-30, 30, 241)
    got = np.array([orc.silu(v) for v in xs])
    np.testing.assert_allclose(got, F.silu(torch.from_numpy(xs)).numpy(), rtol=1e-13, atol=1e-300)
    assert orc.silu(0.0) == 0.0


# ---- RoPE -------------------------------------------------------------------------------------

@pytest.mark.parametrize("hd", [64, 128])
def test_rope_is_a_complex_rotation(orc, hd):
    rng = np.random.default_rng(hd)
    v = rng.standard_normal(hd)
    h = hd // 2
    for pos in (0, 1, 17, 511):
        got = orc.rope_neox(v, pos, 10000.0)
        z = (v[:h] + 1j * v[h:]) * np.exp(1j * pos * 10000.0 ** (-np.arange(h) * 2.0 / hd))
        np.testing.assert_allclose(got, np.r_[z.real, z.imag], atol=1e-12)
        # each (i, i+hd/2) pair keeps its norm
        np.testing.assert_allclose(got[:h] ** 2 + got[h:] ** 2, v[:h] ** 2 + v[h:] ** 2, rtol=1e-12)
    assert np.array_equal(orc.rope_neox(v, 0), v)


def test_rope_dot_depends_only_on_offset(orc):
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    base = orc.rope_neox(q, 5) @ orc.rope_neox(k, 2)
    for m, n in [(13, 10), (103, 100), (703, 700)]:
        assert abs(orc.rope_neox(q, m) @ orc.rope_neox(k, n) - base) < 1e-9


# ---- softmax / attention ------------------------------------------------------------------------

def test_softmax(orc):
    s = np.random.default_rng(0).standard_normal(777) * 20
    a = orc.softmax(s)
    np.testing.assert_allclose(a, torch.softmax(torch.from_numpy(s), 0).numpy(), rtol=1e-12, atol=1e-300)
    assert abs(a.sum() - 1.0) < 1e-12
    np.testing.assert_allclose(orc.softmax(s + 1234.5), a, rtol=1e-12, atol=1e-300)


def _h(a):
    return np.asarray(a).astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 300, 757])
def test_attention_matches_torch_sdpa(orc, n):
    rng = np.random.default_rng(n)
    hd = 64
    q = rng.standard_normal(hd)
    kc, vc = _h(rng.standard_normal((n, hd))), _h(rng.standard_normal((n, hd)))
    o = orc.attend(q, kc, vc)
    K = torch.from_numpy(kc.view(np.float16).astype(np.float64))[None, None]
    V = torch.from_numpy(vc.view(np.float16).astype(np.float64))[None, None]
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None, None, None], K, V)[0, 0, 0].numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)


def test_attention_special_cases(orc):
    rng = np.random.default_rng(11)
    hd = 128
    q = rng.standard_normal(hd)
    k1, v1 = _h(rng.standard_normal((1, hd))), _h(rng.standard_normal((1, hd)))
    assert np.array_equal(orc.attend(q, k1, v1), v1.view(np.float16).astype(np.float64)[0])
    keq = np.repeat(k1, 9, axis=0)                                  # equal keys -> mean of V
    vs = _h(rng.standard_normal((9, hd)))
    np.testing.assert_allclose(orc.attend(q, keq, vs), vs.view(np.float16).astype(np.float64).mean(0), atol=1e-12)


# ---- sampler ------------------------------------------------------------------------------------

def test_argmax_lowest_index_on_ties(orc):
    v = np.array([0.1, 3.0, -1.0, 3.0, 3.0])
    assert orc.argmax(v) == 1
    assert orc.argmax(np.zeros(10)) == 0
    v = np.random.default_rng(0).standard_normal(8192)
    assert orc.argmax(v) == int(np.argmax(v))


def test_topk_special_cases(orc):
    lg = np.random.default_rng(1).standard_normal(2048)
    top = int(np.argmax(lg))
    assert orc.sample_topk(lg, 1, 0.9, 0.999) == top           # k = 1 is greedy
    assert orc.sample_topk(lg, 50, 0.9, 0.0) == top            # u = 0 picks the largest
    # u just below 1 picks the k-th largest
    order = np.argsort(-lg, kind="stable")
    assert orc.sample_topk(lg, 50, 0.9, 1 - 2 ** -24) == order[49]
    # ties among the k largest are broken by lower index
    t = np.array([1.0, 5.0, 5.0, 0.0, 5.0])
    assert orc.sample_topk(t, 2, 1.0, 0.0) == 1
    assert orc.sample_topk(t, 2, 1.0, 0.75) == 2


def test_topk_frequencies_follow_softmax(orc):
    lg = np.random.default_rng(2).standard_normal(300) * 2
    k, T = 20, 0.7
    vals, idx = torch.topk(torch.from_numpy(lg / T), k)
    p = torch.softmax(vals, 0).numpy()
    grid = (np.arange(4096) + 0.5) / 4096
    picks = np.array([orc.sample_topk(lg, k, T, u) for u in grid])
    freq = np.array([(picks == i).mean() for i in idx.numpy()])
    assert set(picks) <= set(idx.numpy())
    np.testing.assert_allclose(freq, p, atol=1.5 / 4096)
