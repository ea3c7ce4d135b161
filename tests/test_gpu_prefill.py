"""GPU parity of the prompt pass (tsd_prefill: matrix-core products over all prompt rows, causal
attention over the cache, the last position through the decode step; the Talker's prompt frames
likewise on its tiled weights) against the CPU oracle, through the C ABI.

* the standalone product tsd_gemm against the oracle's fp64 mat-vec of every row, for every
  weight format, at shapes spanning several 32 x 32 tiles with ragged row and column tails and
  reduction lengths that leave a partial stage: rel <= 1e-5 per tensor, and per element within
  1e-5 of sum_k |w_k x_k| (the scale the rounding works on);
* the cache a prompt writes (every layer, every position) against the oracle's prefill, which
  runs the decode step at every position ([J] §3.2: prompt and decode share one cache): rel <=
  2e-3 per layer for keys and values; then the logits after the prompt and a few teacher-forced
  steps (rel <= 2e-3, ids as in the other model tests);
* the causal mask ([J] §3.11): changing the ids after position i leaves every cached key and
  value at positions <= i bit for bit unchanged;
* prompts longer than one pass (chunks of 4,096 rows), prompts after decoded positions, one-id
  prompts, two batch rows, the Talker at batch 2 and 16, and the prompt pass against the
  stepwise prefill at full size (C3, C4, C5).
"""
import sys

import numpy as np
import pytest

import oracle
from parity import REL_TOL, ids_agree, rel_err, top2_gap
from quantized_gemv_kv_amd import synth

pytestmark = pytest.mark.gpu

GEMM_TOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def dev(a):
    return torch_mod().from_numpy(np.ascontiguousarray(a)).to("cuda")


FORMATS = ["q4_0", "q8_0", "aff8", "q5_0", "aff4_g64", "aff4_g32"]
# (N, K, M): one tile; ragged rows/columns over several tiles with a partial stage of blocks;
# tall K; a single row; a very wide product (64 columns per wave) with a ragged last tile
SHAPES = [(5, 64, 3), (200, 192, 37), (256, 1024, 130), (96, 4096, 65), (130, 320, 1), (6150, 128, 40)]


# the decoders' real widths and pass sizes: GPT-2-Medium / Llama-520M fused QKV (3,072 rows) over
# a 300-row prompt, the 8,192-row head / gate-up width, and a 2,048-row pass through the products
# of 2,048 rows or more (the 64-column-wave tiles of the 8-bit products)
REAL_SHAPES = [(3072, 1024, 300), (8192, 1024, 64), (2048, 1024, 2048), (1024, 4096, 256)]


@pytest.mark.parametrize("N,K,M", SHAPES)
@pytest.mark.parametrize("fmt", FORMATS)
def test_gemm_matches_oracle(fmt, N, K, M):
    gemm_case(fmt, N, K, M)


@pytest.mark.parametrize("N,K,M", REAL_SHAPES)
@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
def test_gemm_real_widths_match_oracle(fmt, N, K, M):
    gemm_case(fmt, N, K, M)


def gemm_case(fmt, N, K, M):
    from quantized_gemv_kv_amd import binding
    torch = torch_mod()
    say(f"[gemm] {fmt} N={N} K={K} M={M}")
    rng = synth.rng_for(11, N, K, M)
    blob = synth.matrix(fmt, rng, N, K)
    x = synth.normal_f32(rng, (M, K))
    bias = synth.normal_f32(rng, (N,), 0.1) if M % 2 else None
    packed = torch.empty(binding.tsd_gemv_packed_bytes(fmt, N, K), dtype=torch.uint8, device="cuda")
    binding.tsd_gemv_pack(fmt, dev(blob), N, K, packed)
    scratch = torch.empty(binding.tsd_gemm_scratch_bytes(M, K), dtype=torch.uint8, device="cuda")
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    binding.tsd_gemm(fmt, packed, N, K, M, dev(x), None if bias is None else dev(bias), y, scratch)
    got = y.cpu().numpy().astype(np.float64)
    ref = np.stack([oracle.gemv(fmt, blob, N, K, x[m].astype(np.float64),
                                None if bias is None else bias.astype(np.float64)) for m in range(M)])
    W = oracle.dequant(fmt, blob, N, K)
    scale = np.abs(x.astype(np.float64)) @ np.abs(W).T + (0 if bias is None else np.abs(bias.astype(np.float64)))
    r = rel_err(got, ref)
    worst = float(np.max(np.abs(got - ref) / np.maximum(scale, 1e-30)))
    say(f"  rel {r:.2e}  elementwise {worst:.2e}")
    assert np.all(np.isfinite(got))
    assert r <= GEMM_TOL
    assert worst <= GEMM_TOL


def test_gemm_rejects_bad_arguments():
    from quantized_gemv_kv_amd import TsdError, binding
    torch = torch_mod()
    packed = torch.zeros(binding.tsd_gemv_packed_bytes("q4_0", 64, 128), dtype=torch.uint8, device="cuda")
    scratch = torch.zeros(binding.tsd_gemm_scratch_bytes(4, 128), dtype=torch.uint8, device="cuda")
    x = torch.zeros((4, 128), dtype=torch.float32, device="cuda")
    y = torch.zeros((4, 64), dtype=torch.float32, device="cuda")
    # K not a block multiple / no rows / K % 64 / scratch too small (it holds one 32-row tile)
    for args in [("q4_0", packed, 64, 100, 4), ("q4_0", packed, 64, 128, 0), ("aff8", packed, 64, 96, 4),
                 ("q4_0", packed, 64, 128, 33)]:
        with pytest.raises(TsdError) as e:
            binding.tsd_gemm(args[0], args[1], args[2], args[3], args[4], x, None, y, scratch)
        assert e.value.status == 1


def kv_rel(gk, gv, ok, ov, n):
    """Worst per-layer rel error of the GPU cache (fp16 tensors) against the oracle's (fp16 bits)."""
    gk = gk.cpu().numpy().astype(np.float64)[:, :, :, :n]
    gv = gv.cpu().numpy().astype(np.float64)[:, :, :, :n]
    ok = ok.view(np.float16).astype(np.float64)[:, :, :, :n]
    ov = ov.view(np.float16).astype(np.float64)[:, :, :, :n]
    return max(max(rel_err(gk[l], ok[l]), rel_err(gv[l], ov[l])) for l in range(gk.shape[0]))


def gpu_model(cfg, w, mode="persistent"):
    from quantized_gemv_kv_amd import Model
    return Model(dict(cfg, launch_mode=mode), w)


def check_prompt(cfg, w, prompts, n_steps=3, mode="persistent", check_ids=True):
    """Prefill each prompt in turn (a later prompt continues after the earlier ones and the
    decoded steps between them), compare the cache and the logits, then n_steps teacher-forced
    steps after each prompt."""
    om = oracle.OracleModel(cfg, w)
    gm = gpu_model(cfg, w, mode)
    worst = 0.0
    for i, n in enumerate(prompts):
        toks = synth.prompt_tokens(cfg, n, seed=30 + i)
        o_ids = om.prefill(toks)
        g_ids = gm.prefill(dev(toks)).cpu().numpy()
        assert gm.n_past == om.n_past
        gk, gv = gm.get_kv()
        ok, ov = om.get_kv()
        r = kv_rel(gk, gv, ok, ov, om.n_past)
        lo, lg = om.logits(), gm.logits().cpu().numpy()
        rl = rel_err(lg, lo)
        say(f"  prompt {n} at {om.n_past - n}: cache rel {r:.2e}, logits rel {rl:.2e}")
        assert r <= REL_TOL and rl <= REL_TOL
        worst = max(worst, r, rl)
        for b in range(cfg["batch"]):
            if check_ids:
                assert ids_agree(g_ids[b, 0], lo[b]), (b, g_ids, o_ids, top2_gap(lo[b]))
        nxt = o_ids
        for s in range(n_steps):
            o_ids = om.step(nxt)
            g_ids = gm.step(dev(nxt)).cpu().numpy()
            lo, lg = om.logits(), gm.logits().cpu().numpy()
            assert rel_err(lg, lo) <= REL_TOL, (s, rel_err(lg, lo))
            for b in range(cfg["batch"]):
                if check_ids:
                    assert ids_agree(g_ids[b, 0], lo[b]), (s, b, g_ids, o_ids, top2_gap(lo[b]))
            nxt = o_ids
    gm.synchronize()
    gm.close()
    return worst


PROMPT_CASES = [("gpt2", "q4_0"), ("gpt2", "q8_0"), ("gpt2", "aff8"), ("gpt2", "q5_0"), ("llama", "q8_0"),
                ("llama", "q4_0"), ("llama", "aff4_g64"), ("llama", "aff4_g32")]


@pytest.mark.parametrize("arch,fmt", PROMPT_CASES)
def test_prompt_pass_matches_oracle(arch, fmt):
    """A 70-id prompt (two 64-row tiles, the second ragged) on a small model."""
    cfg = synth.small_config(arch, fmt, d_ff=256, n_ctx=96)
    say(f"[prefill] {arch} {fmt}")
    w = synth.model_weights(cfg, 42, norm_std=0.5)
    check_prompt(cfg, w, [70])


def test_prompt_pass_gqa_head128():
    cfg = synth.small_config("llama", "q8_0", d_model=256, n_head=4, n_kv_head=2, head_dim=128, d_ff=512, n_ctx=96)
    say("[prefill] llama gqa hd 128")
    w = synth.model_weights(cfg, 42, norm_std=0.5)
    check_prompt(cfg, w, [40])


@pytest.mark.parametrize("mode", ["persistent", "per_operator"])
def test_prompt_continues_after_decoding(mode):
    """A prompt, three decoded steps, a second prompt, three steps, a one-id prompt (only the
    decode step runs), a two-id prompt (one prompt-pass row)."""
    cfg = synth.small_config("gpt2", "q4_0", d_ff=256, n_ctx=160)
    say(f"[prefill] continued prompts {mode}")
    w = synth.model_weights(cfg, 7, norm_std=0.5)
    check_prompt(cfg, w, [33, 45, 1, 2], mode=mode)


def test_prompt_longer_than_one_pass():
    """4,150 ids: a 4,096-row pass, a 53-row pass, the decode step."""
    cfg = synth.small_config("llama", "q4_0", d_ff=256, n_ctx=4160, vocab=500)
    say("[prefill] 4150 ids in two passes")
    w = synth.model_weights(cfg, 3, norm_std=0.5)
    check_prompt(cfg, w, [4150], n_steps=2)


@pytest.mark.parametrize("arch,fmt", [("gpt2", "q4_0"), ("llama", "q8_0")])
def test_prompt_two_rows(arch, fmt):
    """Batch 2, a different prompt per row, 2,100 positions each: 4,200 rows in passes of
    2,048 positions (4,096 rows) and 51."""
    cfg = synth.small_config(arch, fmt, batch=2, d_ff=256, n_ctx=2112, vocab=500)
    say(f"[prefill] batch 2 {arch} {fmt}")
    w = synth.model_weights(cfg, 5, norm_std=0.5)
    check_prompt(cfg, w, [2100], n_steps=2, mode="per_operator")


def test_causal_mask_leaves_earlier_positions_unchanged():
    """Two 90-id prompts that agree on their first 41 ids: the caches agree bit for bit at
    positions 0..40, and differ after."""
    cfg = synth.small_config("llama", "q4_0", d_ff=256, n_ctx=96)
    say("[prefill] causal mask")
    w = synth.model_weights(cfg, 9, norm_std=0.5)
    a = synth.prompt_tokens(cfg, 90, seed=1)
    b = a.copy()
    b[:, 41:, :] = synth.prompt_tokens(cfg, 49, seed=2)
    assert not np.array_equal(a[:, 41:], b[:, 41:])
    caches = []
    for t in (a, b):
        gm = gpu_model(cfg, w)
        gm.prefill(dev(t))
        k, v = gm.get_kv()
        caches.append((k.cpu().numpy().view(np.uint16), v.cpu().numpy().view(np.uint16)))
        gm.close()
    (ka, va), (kb, vb) = caches
    assert np.array_equal(ka[:, :, :, :41], kb[:, :, :, :41]) and np.array_equal(va[:, :, :, :41], vb[:, :, :, :41])
    assert not np.array_equal(ka[:, :, :, 41:], kb[:, :, :, 41:])


def test_prompt_history_and_consumed_ids():
    """The history holds the next prompt id at every prompt position but the last, and the
    sampled id there; the penalty's consumed ids are the prompt."""
    cfg = synth.small_config("gpt2", "q8_0", d_ff=256, n_ctx=64)
    w = synth.model_weights(cfg, 4, norm_std=0.5)
    gm = gpu_model(cfg, w)
    toks = synth.prompt_tokens(cfg, 20, seed=6)
    nxt = gm.prefill(dev(toks)).cpu().numpy()
    hist = gm.tokens(0, 20).cpu().numpy()[:, 0, 0]
    assert list(hist[:19]) == [int(t) for t in toks[0, 1:, 0]]
    assert int(hist[19]) == int(nxt[0, 0])
    gm.close()


@pytest.mark.parametrize("name", ["gpt2_medium_q4_0", "llama520m_q8_0"])
def test_full_size_prompt_pass(name):
    """The benchmark's prompt (256 ids for GPT-2-Medium, 300 for Llama-520M) at the real shapes:
    the prompt pass against the stepwise prefill (cache per layer and logits rel <= 2e-3, same
    next id unless near-tied), and the first layer's cached keys and values at sampled positions
    against the oracle's layer run on the same embedding rows."""
    torch = torch_mod()
    cfg = synth.config(name)
    n = 256 if cfg["arch"] == "gpt2" else 300
    say(f"[prefill-full] {name} {n} ids")
    w = synth.model_weights(cfg, 42)
    toks = synth.prompt_tokens(cfg, n, seed=42)
    gm = gpu_model(cfg, w)
    g_ids = gm.prefill(dev(toks)).cpu().numpy()
    gk, gv = gm.get_kv()
    lg = gm.logits().cpu().numpy()
    gm.close()
    sm = gpu_model(cfg, w)
    s_ids = sm.prefill_stepwise(dev(toks)).cpu().numpy()
    sk, sv = sm.get_kv()
    ls = sm.logits().cpu().numpy()
    sm.close()
    r = max(max(rel_err(gk[l].cpu().numpy(), sk[l].cpu().numpy()), rel_err(gv[l].cpu().numpy(), sv[l].cpu().numpy()))
            for l in range(cfg["n_layer"]))
    say(f"  against stepwise: cache rel {r:.2e}, logits rel {rel_err(lg, ls):.2e}")
    assert r <= REL_TOL and rel_err(lg, ls) <= REL_TOL
    assert ids_agree(g_ids[0, 0], ls[0])
    # layer 0 at sampled positions: the oracle runs the layer on the embedding row and writes its
    # own key and value there (the cache below is the GPU's, loaded so that attention has keys)
    om = oracle.OracleModel(cfg, w)
    om.load_kv(gk.cpu().numpy().view(np.uint16), gv.cpu().numpy().view(np.uint16), n)
    emb = w[0].reshape(cfg["vocab"], cfg["d_model"]).astype(np.float64)
    wpe = w[1].reshape(cfg["n_ctx"], cfg["d_model"]).astype(np.float64) if cfg["arch"] == "gpt2" else None
    for p in (0, 1, 127, n - 2):
        x = emb[int(toks[0, p, 0])] + (wpe[p] if wpe is not None else 0.0)
        om.layer_forward(0, x, p)
    ok, ov = om.get_kv()
    for p in (0, 1, 127, n - 2):
        rk = rel_err(gk[0, :, :, p].cpu().numpy(), ok[0, :, :, p].view(np.float16))
        rv = rel_err(gv[0, :, :, p].cpu().numpy(), ov[0, :, :, p].view(np.float16))
        say(f"  layer 0 position {p}: k rel {rk:.2e} v rel {rv:.2e}")
        assert rk <= REL_TOL and rv <= REL_TOL


def oracle_prefill_with_progress(om, toks, label, chunk=32):
    """The oracle's prefill of toks in chunks of positions (the same sequence of decode steps as
    one call), printing progress so that a long single-threaded run is visibly alive."""
    import time
    t0 = time.perf_counter()
    n = toks.shape[1]
    ids = None
    for a in range(0, n, chunk):
        ids = om.prefill(np.ascontiguousarray(toks[:, a:a + chunk]))
        say(f"  oracle {label}: {min(a + chunk, n)}/{n} positions, {time.perf_counter() - t0:.0f} s")
    return ids


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,n", [("gpt2_medium_q4_0", 256), ("llama520m_q8_0", 48)])
def test_full_size_prompt_pass_matches_oracle(name, n):
    """The prompt pass at the decoders' real widths against the oracle: GPT-2-Medium Q4_0 on the
    benchmark's 256-id prompt, Llama-520M Q8_0 on 48 ids (its 64-column-wave products depend on
    the matrix widths, not on the prompt length).  Every layer's cached keys and values (rel <=
    2e-3 per layer), the logits after the prompt (rel <= 2e-3) and the next id (equal unless the
    oracle's top two are within 1e-3).  The oracle runs the decode step at every position, single
    threaded: about 0.3-0.5 s per position for GPT-2-Medium on these hosts."""
    cfg = synth.config(name)
    say(f"[prefill-full-oracle] {name} {n} ids")
    w = synth.model_weights(cfg, 42)
    toks = synth.prompt_tokens(cfg, n, seed=42)
    gm = gpu_model(cfg, w)
    g_ids = gm.prefill(dev(toks)).cpu().numpy()
    gk, gv = gm.get_kv()
    lg = gm.logits().cpu().numpy()
    gm.close()
    om = oracle.OracleModel(cfg, w)
    o_ids = oracle_prefill_with_progress(om, toks, name)
    ok, ov = om.get_kv()
    lo = om.logits()
    om.close()
    gk = gk.cpu().numpy().astype(np.float64)
    gv = gv.cpu().numpy().astype(np.float64)
    ok = ok.view(np.float16).astype(np.float64)
    ov = ov.view(np.float16).astype(np.float64)
    per_layer = [max(rel_err(gk[l, :, :, :n], ok[l, :, :, :n]), rel_err(gv[l, :, :, :n], ov[l, :, :, :n]))
                 for l in range(cfg["n_layer"])]
    say(f"  cache rel per layer: max {max(per_layer):.2e} (layer {int(np.argmax(per_layer))}), "
        f"logits rel {rel_err(lg, lo):.2e}, top-2 gap {top2_gap(lo[0]):.2e}")
    assert max(per_layer) <= REL_TOL
    assert rel_err(lg, lo) <= REL_TOL
    assert ids_agree(g_ids[0, 0], lo[0]), (g_ids[0, 0], o_ids[0, 0])


@pytest.mark.timeout(600)
def test_talker_widths_prompt_pass_matches_oracle():
    """The Talker's prompt pass at its real widths (d 1024, 16 q / 8 kv heads of 128, SwiGLU
    3072, vocabularies 3072 / 2048, 16 codebooks) with two Talker layers and one predictor layer
    at batch 16: 24 prompt frames (384 rows of the tiled 8-bit products) against the oracle's
    prefill, the cache of every layer and the last frame's code-0 logits."""
    cfg = dict(synth.config("talker_cp_aff8"), n_layer=2, cp_n_layer=1, n_ctx=64)
    n = 24
    say(f"[prefill-oracle] talker widths, batch 16, {n} frames")
    w = synth.model_weights(cfg, 42)
    toks = synth.prompt_tokens(cfg, n, seed=5)
    gm = gpu_model(cfg, w)
    g_ids = gm.prefill(dev(toks)).cpu().numpy()
    gk, gv = gm.get_kv()
    lg = gm.logits().cpu().numpy()
    gm.close()
    om = oracle.OracleModel(cfg, w)
    o_ids = oracle_prefill_with_progress(om, toks, "talker", chunk=8)
    ok, ov = om.get_kv()
    V = cfg["vocab"]
    lo = om.logits()[:, 0, :V]
    om.close()
    r = kv_rel(gk, gv, ok, ov, n)
    say(f"  cache rel {r:.2e}, code-0 logits rel {rel_err(lg[:, 0, :V], lo):.2e}")
    assert r <= REL_TOL and rel_err(lg[:, 0, :V], lo) <= REL_TOL
    for b in range(cfg["batch"]):
        assert ids_agree(g_ids[b, 0], lo[b]), (b, g_ids[b, 0], o_ids[b, 0])


@pytest.mark.parametrize("batch", [2, 16])
def test_talker_prompt_pass_matches_oracle(batch):
    """The Talker's prompt frames (each row's input the sum of its 4 code embeddings) through
    the prompt pass on the tiled 8-bit affine weights: its cache against the oracle's prefill
    (every layer and position) and the last frame's code-0 logits (the predictor's heads follow
    from its own codes, compared in the frame tests)."""
    cfg = synth.small_config("talker_cp", "aff8", batch=batch, n_ctx=64)
    say(f"[prefill] talker batch {batch}")
    w = synth.model_weights(cfg, 42, norm_std=0.1)
    om = oracle.OracleModel(cfg, w)
    gm = gpu_model(cfg, w)
    toks = synth.prompt_tokens(cfg, 37, seed=5)
    o_ids = om.prefill(toks)
    g_ids = gm.prefill(dev(toks)).cpu().numpy()
    gk, gv = gm.get_kv()
    ok, ov = om.get_kv()
    r = kv_rel(gk, gv, ok, ov, 37)
    V = cfg["vocab"]
    lo, lg = om.logits()[:, 0, :V], gm.logits().cpu().numpy()[:, 0, :V]
    say(f"  cache rel {r:.2e}, code-0 logits rel {rel_err(lg, lo):.2e}")
    assert r <= REL_TOL and rel_err(lg, lo) <= REL_TOL
    for b in range(batch):
        assert ids_agree(g_ids[b, 0], lo[b]), (b, g_ids[b, 0], o_ids[b, 0])
    gm.close()


def test_full_size_talker_prompt_pass():
    """The batched frame's 170 prompt frames at batch 16 (2,720 rows in six passes of 32
    positions) at the real Talker shape, against the frame-by-frame prefill: the Talker cache
    per layer and the last frame's code-0 logits at rel <= 2e-3."""
    cfg = synth.config("talker_cp_aff8")
    n = 170
    say(f"[prefill-full] talker_cp_aff8 {n} frames")
    w = synth.model_weights(cfg, 42)
    toks = synth.prompt_tokens(cfg, n, seed=42)
    V = cfg["vocab"]
    out = []
    for kind in ("prefill", "prefill_stepwise"):
        gm = gpu_model(cfg, w)
        ids = getattr(gm, kind)(dev(toks)).cpu().numpy()
        k, v = gm.get_kv()
        out.append((ids, k.cpu().numpy().astype(np.float32), v.cpu().numpy().astype(np.float32),
                    gm.logits().cpu().numpy()[:, 0, :V]))
        gm.close()
    (gi, gk, gv, gl), (si, sk, sv, sl) = out
    r = max(max(rel_err(gk[l], sk[l]), rel_err(gv[l], sv[l])) for l in range(cfg["n_layer"]))
    say(f"  against frame by frame: cache rel {r:.2e}, code-0 logits rel {rel_err(gl, sl):.2e}")
    assert r <= REL_TOL and rel_err(gl, sl) <= REL_TOL
    for b in range(cfg["batch"]):
        assert ids_agree(gi[b, 0], sl[b])


def test_prompt_fills_the_context():
    """A prompt of exactly n_ctx ids (the last position is n_ctx - 1); the next step reports a
    full context and changes nothing."""
    from quantized_gemv_kv_amd import TsdError
    cfg = synth.small_config("llama", "q8_0", d_ff=256, n_ctx=96)
    say("[prefill] whole context")
    w = synth.model_weights(cfg, 8, norm_std=0.5)
    check_prompt(cfg, w, [96], n_steps=0)
    gm = gpu_model(cfg, w)
    gm.prefill(dev(synth.prompt_tokens(cfg, 96, seed=30)))
    with pytest.raises(TsdError) as e:
        gm.step(None)
    assert e.value.status == 4 and gm.n_past == 96
    gm.close()


@pytest.mark.parametrize("launch_mode", ["persistent", "per_operator"])
def test_prompt_ids_outside_the_vocabulary_are_rejected(launch_mode):
    """An id below 0 or past the vocabulary voids the prompt call: the next tsd_synchronize
    reports TSD_ERR_INVALID_ARGUMENT, n_past, the logits, the history and the cache of the earlier
    positions are as before the call (bit for bit), and the model then goes on exactly as one that
    never saw the bad prompt."""
    from quantized_gemv_kv_amd import Model
    from quantized_gemv_kv_amd.binding import TsdError
    cfg = dict(synth.small_config("gpt2", "q4_0", d_ff=256, n_ctx=64), launch_mode=launch_mode)
    say(f"[prefill] bad ids, {launch_mode}")
    w = synth.model_weights(cfg, 9, norm_std=0.5)
    a, c = synth.prompt_tokens(cfg, 20, seed=4), synth.prompt_tokens(cfg, 15, seed=5)

    def state(m):
        k, v = m.get_kv(m.n_past)
        return (m.n_past, m.logits().cpu().numpy(), m.tokens(0, m.n_past).cpu().numpy(),
                k.cpu().numpy().view(np.uint16), v.cpu().numpy().view(np.uint16))

    ref = Model(cfg, w)
    ref.prefill(dev(a))
    ref.prefill(dev(c))
    want = state(ref)
    ref.close()
    for bad_id in (-5, cfg["vocab"], cfg["vocab"] + 7, 1 << 30):
        gm = Model(cfg, w)
        gm.prefill(dev(a))
        before = state(gm)
        bad = synth.prompt_tokens(cfg, 12, seed=6)
        bad[0, 7, 0] = bad_id
        gm.prefill(dev(bad))
        gm.step(None)                      # a call after the rejected one does nothing either
        with pytest.raises(TsdError) as e:
            gm.synchronize()
        assert e.value.status == 1, e.value
        after = state(gm)
        assert after[0] == before[0] == 20
        for x, y in zip(before[1:], after[1:]):
            assert np.array_equal(x, y)
        gm.prefill(dev(c))
        got = state(gm)
        assert got[0] == want[0]
        for x, y in zip(want[1:], got[1:]):
            assert np.array_equal(x, y)
        gm.close()


def test_prompt_after_truncate():
    """40 ids, truncated back to 25, then 30 more: the cache of the 55 positions and the logits
    against the oracle doing the same."""
    cfg = synth.small_config("gpt2", "q8_0", d_ff=256, n_ctx=64)
    say("[prefill] after truncate")
    w = synth.model_weights(cfg, 10, norm_std=0.5)
    om = oracle.OracleModel(cfg, w)
    gm = gpu_model(cfg, w)
    a, b = synth.prompt_tokens(cfg, 40, seed=1), synth.prompt_tokens(cfg, 30, seed=2)
    om.prefill(a)
    gm.prefill(dev(a))
    om.truncate(25)
    gm.truncate(25)
    om.prefill(b)
    g_ids = gm.prefill(dev(b)).cpu().numpy()
    gk, gv = gm.get_kv()
    ok, ov = om.get_kv()
    r = kv_rel(gk, gv, ok, ov, 55)
    lo, lg = om.logits(), gm.logits().cpu().numpy()
    say(f"  cache rel {r:.2e}, logits rel {rel_err(lg, lo):.2e}")
    assert gm.n_past == om.n_past == 55
    assert r <= REL_TOL and rel_err(lg, lo) <= REL_TOL
    assert ids_agree(g_ids[0, 0], lo[0])
    gm.close()
