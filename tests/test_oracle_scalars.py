"""Pins of the oracle's scalar building blocks: fp16 storage, the counter-based generator and
the byte layout of the three weight formats (CPU only)."""
import numpy as np
import pytest


# ---- fp16 (IEEE binary16) --------------------------------------------------------------------

def test_half_decode_matches_numpy_on_every_pattern(orc):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_half_encode_matches_numpy_rne(orc):
    rng = np.random.default_rng(0)
    xs = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000),   # wide dynamic range
        rng.standard_normal(2000) * 6e-8,                                   # subnormals
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -12), np.inf, -np.inf]),
        # exact ties between neighbours: must go to the even mantissa
        1.0 + (2 * np.arange(64) + 1) * 2.0 ** -11,
        (1024 + 2 * np.arange(64) + 1) * 2.0 ** -25,                        # subnormal ties
    ])
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    got = np.array([orc.double_to_half(float(x)) for x in xs], np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(xs[i], hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_half_encode_nan(orc):
    h = orc.double_to_half(float("nan"))
    assert (h & 0x7C00) == 0x7C00 and (h & 0x3FF) != 0


# ---- Philox4x64-10 ------------------------------------------------------------------------------

@pytest.mark.parametrize("ctr,key", [
    ((0, 0, 0, 0), (0, 0)),
    ((5, 0, 0, 0), (7, 9)),
    ((2 ** 64 - 2, 3, 2 ** 63, 11), (2 ** 64 - 1, 12345)),
    ((123456789, 987654321, 42, 7), (0xDEADBEEF, 0xC0FFEE)),
])
def test_philox_matches_numpy(orc, ctr, key):
    # numpy's Philox bit generator advances its counter by one before each block of 4 words
    bg = np.random.Philox(counter=np.array(ctr, np.uint64), key=np.array(key, np.uint64))
    ref = bg.random_raw(4).astype(np.uint64)
    c1 = list(ctr)
    c1[0] = (c1[0] + 1) % 2 ** 64
    if c1[0] == 0:
        c1[1] = (c1[1] + 1) % 2 ** 64
    got = orc.philox4x64_10(c1, key)
    assert np.array_equal(got, ref)


def _numpy_counter_before(ctr):
    """The counter numpy's Philox must hold so that its next block is generated at `ctr` (it adds
    one, with carry, before each block of 4 words)."""
    c = list(ctr)
    for i in range(4):
        if c[i] > 0:
            c[i] -= 1
            return c
        c[i] = 2 ** 64 - 1
    return c


@pytest.mark.parametrize("seed,row,pos,pss", [
    (42, 0, 256, 0), (42, 1, 256, 0), (42, 0, 257, 0), (42, 15, 3, 7), (7, 3, 15, 1),
    (0, 1, 0, 0), (2 ** 63 + 5, 2, 900, 14), (123456789, 9, 1, 2),
])
def test_uniform24_is_the_top_24_bits_of_word_0(orc, seed, row, pos, pss):
    # the sampler's uniform: counter (position, row, pass, 0), key (seed, 0), top 24 bits of the
    # first output word of Philox4x64-10, recomputed with numpy's independent implementation
    bg = np.random.Philox(counter=np.array(_numpy_counter_before((pos, row, pss, 0)), np.uint64),
                          key=np.array((seed, 0), np.uint64))
    w0 = int(bg.random_raw(4)[0])
    assert orc.uniform24(seed, row, pos, pss) == (w0 >> 40) / 2.0 ** 24
    # the counter words are not interchangeable: a swapped (row, position) draws another value
    if row != pos:
        bg = np.random.Philox(counter=np.array(_numpy_counter_before((row, pos, pss, 0)), np.uint64),
                              key=np.array((seed, 0), np.uint64))
        assert orc.uniform24(seed, row, pos, pss) != (int(bg.random_raw(4)[0]) >> 40) / 2.0 ** 24


def test_uniform24_range_and_granularity(orc):
    us = np.array([orc.uniform24(42, r, p, s) for r in range(4) for p in range(64) for s in range(4)])
    assert us.min() >= 0.0 and us.max() < 1.0
    assert np.all(us * 2 ** 24 == np.floor(us * 2 ** 24))
    assert len(np.unique(us)) == us.size               # distinct counters give distinct draws
    assert abs(us.mean() - 0.5) < 0.05


# ---- weight formats ----------------------------------------------------------------------------

def _fig(name):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "page_figures.txt")
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            parts = [p.strip() for p in line.split("|")]
            if parts[0] == name:
                return parts[1]
    raise KeyError(name)


def test_block_sizes_match_page(orc):
    # a Q4_0 row of K=1024 is 32 blocks of 18 bytes
    assert orc.matrix_bytes("q4_0", 1, 1024) == int(_fig("q4_0_blocks_per_row_k1024")) * int(_fig("q4_0_block_bytes"))
    assert orc.matrix_bytes("q4_0", 1, 32) == 18
    assert orc.matrix_bytes("q8_0", 1, 32) == 34
    assert orc.matrix_bytes("q8_0", 1, 1024) == 1088
    assert orc.matrix_bytes("aff8", 1, 1024) == 1024 + 16 * 4
    # ~8.5 bits per weight for affine group 64
    assert orc.matrix_bytes("aff8", 1, 1024) * 8 / 1024 == float(_fig("q8_bits_per_weight"))
    # K not a multiple of the block: rejected
    assert orc.matrix_bytes("q4_0", 4, 48) == 0
    assert orc.matrix_bytes("aff8", 4, 96) == 0


HALF = {0x3C00: 1.0, 0x3800: 0.5, 0x1400: 2.0 ** -10, 0x7BFF: 65504.0, 0x0001: 2.0 ** -24,
        0xC000: -2.0}


@pytest.mark.parametrize("dbits", sorted(HALF))
def test_q8_0_hand_built_block(orc, dbits):
    q = np.array([-127, 0, 127, 1, -1] + list(range(-13, 14)), np.int8)
    assert q.size == 32
    blk = np.concatenate([np.array([dbits & 0xFF, dbits >> 8], np.uint8), q.view(np.uint8)])
    w = orc.dequant("q8_0", blk, 1, 32)[0]
    assert np.array_equal(w, HALF[dbits] * q.astype(np.float64))


@pytest.mark.parametrize("dbits", sorted(HALF))
def test_q4_0_hand_built_block(orc, dbits):
    lo = np.arange(16, dtype=np.uint8)                 # elements 0..15
    hi = (15 - np.arange(16)).astype(np.uint8)         # elements 16..31
    blk = np.concatenate([np.array([dbits & 0xFF, dbits >> 8], np.uint8), lo | (hi << 4)])
    w = orc.dequant("q4_0", blk, 1, 32)[0]
    expect = HALF[dbits] * (np.concatenate([lo, hi]).astype(np.float64) - 8.0)
    assert np.array_equal(w, expect)
    assert w[8] == 0.0                                  # q = 8 is zero


def test_q4_0_nibble_order_single_element(orc):
    # byte j carries element j in its low nibble and element j+16 in its high nibble
    for j in range(16):
        qs = np.full(16, 0x88, np.uint8)               # all elements q=8 -> 0
        qs[j] = 0x8F                                   # element j -> 15, element j+16 -> 8
        w = orc.dequant("q4_0", np.concatenate([np.array([0x00, 0x3C], np.uint8), qs]), 1, 32)[0]
        nz = np.nonzero(w)[0]
        assert list(nz) == [j] and w[j] == 7.0
        qs[j] = 0xF8                                   # element j+16 -> 15
        w = orc.dequant("q4_0", np.concatenate([np.array([0x00, 0x3C], np.uint8), qs]), 1, 32)[0]
        assert list(np.nonzero(w)[0]) == [j + 16] and w[j + 16] == 7.0


def test_aff8_hand_built_group(orc):
    N, K = 2, 128
    q = np.zeros((N, K), np.uint8)
    q[0, :64] = np.arange(64)
    q[0, 64:] = 255
    q[1, :] = 3
    s = np.array([[0x3800, 0x3C00], [0x1400, 0x0001]], np.uint16)   # 0.5, 1, 2^-10, 2^-24
    b = np.array([[0xC000, 0x0000], [0x3C00, 0x3800]], np.uint16)   # -2, 0, 1, 0.5
    blob = np.concatenate([q.reshape(-1), s.reshape(-1).view(np.uint8), b.reshape(-1).view(np.uint8)])
    W = orc.dequant("aff8", blob, N, K)
    assert np.array_equal(W[0, :64], 0.5 * np.arange(64) - 2.0)
    assert np.array_equal(W[0, 64:], np.full(64, 255.0))
    assert np.array_equal(W[1, :64], np.full(64, 3 * 2.0 ** -10 + 1.0))
    assert np.array_equal(W[1, 64:], np.full(64, 3 * 2.0 ** -24 + 0.5))
    q[1, :] = 0                                                      # q = 0 gives the bias
    blob = np.concatenate([q.reshape(-1), s.reshape(-1).view(np.uint8), b.reshape(-1).view(np.uint8)])
    assert np.array_equal(orc.dequant("aff8", blob, N, K)[1], np.r_[np.full(64, 1.0), np.full(64, 0.5)])


def test_new_format_block_sizes(orc):
    # Q5_0: 2 + 4 + 16 bytes per 32 weights (5.5 bits); 4-bit affine: K/2 bytes plus a scale and
    # a bias per group (4.5 bits at group 64, 5 at group 32, the "~0.5 bit per weight more" of
    # the finer groups)
    assert orc.matrix_bytes("q5_0", 1, 32) == 22
    assert orc.matrix_bytes("q5_0", 1, 1024) == 704
    assert orc.matrix_bytes("aff4_g64", 1, 1024) * 8 / 1024 == 4.5
    assert orc.matrix_bytes("aff4_g32", 1, 1024) * 8 / 1024 == 5.0
    assert orc.matrix_bytes("q5_0", 2, 48) == 0
    assert orc.matrix_bytes("aff4_g64", 2, 96) == 0
    assert orc.matrix_bytes("aff4_g32", 2, 96) == 2 * 48 + 2 * 3 * 4


def _q5_block(dbits, qh, qs):
    return np.concatenate([np.array([dbits & 0xFF, dbits >> 8], np.uint8),
                           np.array([qh & 0xFF, (qh >> 8) & 0xFF, (qh >> 16) & 0xFF, qh >> 24], np.uint8),
                           np.asarray(qs, np.uint8)])


@pytest.mark.parametrize("dbits", sorted(HALF))
def test_q5_0_hand_built_block(orc, dbits):
    lo = np.arange(16, dtype=np.uint8)                 # low nibbles of elements 0..15
    hi = (15 - np.arange(16)).astype(np.uint8)         # of elements 16..31
    qh = 0xA5C3F00F                                    # fifth bits: bit j for element j
    w = orc.dequant("q5_0", _q5_block(dbits, qh, lo | (hi << 4)), 1, 32)[0]
    five = np.array([(qh >> j) & 1 for j in range(32)], np.float64) * 16
    expect = HALF[dbits] * (np.concatenate([lo, hi]).astype(np.float64) + five - 16.0)
    assert np.array_equal(w, expect)
    # all bits clear: -16 d; every bit set: 15 d
    assert np.array_equal(orc.dequant("q5_0", _q5_block(dbits, 0, np.zeros(16)), 1, 32)[0], np.full(32, -16 * HALF[dbits]))
    assert np.array_equal(orc.dequant("q5_0", _q5_block(dbits, 0xFFFFFFFF, np.full(16, 0xFF)), 1, 32)[0],
                          np.full(32, 15 * HALF[dbits]))


def test_q5_0_fifth_bit_order_single_element(orc):
    # q = 16 is zero: nibbles 0 with every fifth bit set; clearing bit j moves element j alone to -16
    for j in range(32):
        w = orc.dequant("q5_0", _q5_block(0x3C00, 0xFFFFFFFF & ~(1 << j), np.zeros(16)), 1, 32)[0]
        assert list(np.nonzero(w)[0]) == [j] and w[j] == -16.0


def test_aff4_nibble_order_and_groups(orc):
    for fmt, G in (("aff4_g64", 64), ("aff4_g32", 32)):
        N, K = 2, 128
        q = np.zeros((N, K), np.uint8)
        q[0, 5] = 9                                    # byte 2's high nibble
        q[0, 6] = 3                                    # byte 3's low nibble
        q[1, :] = np.arange(K) % 16
        ng = K // G
        s = np.full((N, ng), 0x3C00, np.uint16)        # 1
        s[1, :] = 0x3800                               # 0.5
        b = np.zeros((N, ng), np.uint16)
        b[1, -1] = 0xC000                              # -2 on row 1's last group
        packed = q[:, 0::2] | (q[:, 1::2] << 4)
        assert packed[0, 2] == 0x90 and packed[0, 3] == 0x03
        blob = np.concatenate([packed.reshape(-1), s.reshape(-1).view(np.uint8), b.reshape(-1).view(np.uint8)])
        W = orc.dequant(fmt, blob, N, K)
        assert list(np.nonzero(W[0])[0]) == [5, 6] and W[0, 5] == 9.0 and W[0, 6] == 3.0
        expect = 0.5 * (np.arange(K) % 16).astype(np.float64)
        expect[K - G:] -= 2.0
        assert np.array_equal(W[1], expect)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", "aff8", "q5_0", "aff4_g64", "aff4_g32"])
def test_generator_blobs_decode_to_their_draws(orc, fmt):
    """The generator's packing, decoded by the oracle, reproduces the raw draws exactly."""
    from quantized_gemv_kv_amd import synth
    N, K = 7, 192
    rng = synth.rng_for(1, 2)
    if fmt == "q4_0":
        blob, raw = synth.q4_0_matrix(rng, N, K)
        expect = (raw["q"].astype(np.float64) - 8) * np.repeat(raw["d"].astype(np.float64), 32, axis=1)
    elif fmt == "q8_0":
        blob, raw = synth.q8_0_matrix(rng, N, K)
        expect = raw["q"].astype(np.float64) * np.repeat(raw["d"].astype(np.float64), 32, axis=1)
    elif fmt == "q5_0":
        blob, raw = synth.q5_0_matrix(rng, N, K)
        expect = (raw["q"].astype(np.float64) - 16) * np.repeat(raw["d"].astype(np.float64), 32, axis=1)
    elif fmt.startswith("aff4"):
        g = 64 if fmt == "aff4_g64" else 32
        blob, raw = synth.aff4_matrix(rng, N, K, g)
        expect = (raw["q"].astype(np.float64) * np.repeat(raw["s"].astype(np.float64), g, axis=1)
                  + np.repeat(raw["b"].astype(np.float64), g, axis=1))
    else:
        blob, raw = synth.aff8_matrix(rng, N, K)
        expect = (raw["q"].astype(np.float64) * np.repeat(raw["s"].astype(np.float64), 64, axis=1)
                  + np.repeat(raw["b"].astype(np.float64), 64, axis=1))
    assert blob.size == orc.matrix_bytes(fmt, N, K)
    assert np.array_equal(orc.dequant(fmt, blob, N, K), expect)


@pytest.mark.parametrize("fmt", ["q8_0", "q5_0", "aff8", "aff4_g64", "aff4_g32"])
def test_chunked_generator_assembles_the_planes(orc, fmt):
    """The tall-matrix generator writes each row chunk into its place in the canonical layout:
    decoded whole, the matrix is the chunks' own decodes stacked."""
    import torch
    from quantized_gemv_kv_amd import synth
    N, K, ch = 10, 128, 4
    out = torch.zeros(orc.matrix_bytes(fmt, N, K), dtype=torch.uint8)
    synth.matrix_into(fmt, N, K, 5, out, chunk_rows=ch)
    W = orc.dequant(fmt, out.numpy(), N, K)
    for r0 in range(0, N, ch):
        n = min(ch, N - r0)
        part = synth.matrix(fmt, synth.rng_for(5, r0, K), n, K)
        assert np.array_equal(W[r0:r0 + n], orc.dequant(fmt, part, n, K))
