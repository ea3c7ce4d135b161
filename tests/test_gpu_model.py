"""GPU parity of the whole decode step (captured graph) against the CPU oracle, through the
C ABI, in both launch modes (one persistent launch per step; one launch per operator).
Logits: rel <= 2e-3 per step.  Greedy ids: teacher forced (both sides get the oracle's id as
the next input) and equal except where the oracle's top-2 logits are within 1e-3."""
import sys

import numpy as np
import pytest

import oracle
from parity import (DRAW_MARGIN, REL_TOL, TIE_GAP, chain_margins, chain_near_boundary, ids_agree, rel_err,
                    sampling_of, top2_gap, topk_draw_margins)
from quantized_gemv_kv_amd import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def dev(a):
    return torch_mod().from_numpy(np.ascontiguousarray(a)).to("cuda")


MODES = ["persistent", "per_operator"]


def gpu_model(cfg, w, mode="persistent", n_wg=0):
    from quantized_gemv_kv_amd import Model
    m = Model(dict(cfg, launch_mode=mode, n_workgroups=n_wg), w, sampling=sampling_of(cfg))
    # the launch mode asked for is the one that runs (the step kernel is timed only when it exists)
    assert m.uses_persistent_step() == (mode == "persistent"), "persistent step not built for this shape"
    return m


def teacher_forced(cfg, w, n_prompt, n_steps, kv_pos=None, seed=3, check_ids=True, mode="persistent", n_wg=0):
    """Run both sides n_steps past a prompt (or a loaded random cache) and compare."""
    torch = torch_mod()
    om = oracle.OracleModel(cfg, w)
    gm = gpu_model(cfg, w, mode, n_wg)
    worst = 0.0
    if kv_pos is not None:
        k, v = synth.kv_cache(cfg, kv_pos, seed=seed)
        om.load_kv(k, v, kv_pos)
        gm.load_kv(dev(k), dev(v), kv_pos)
        nxt = np.array([[int(synth.rng_for(seed, 77).integers(0, cfg["vocab"]))]], np.int32)
    else:
        toks = synth.prompt_tokens(cfg, n_prompt, seed=seed)
        o_ids = om.prefill(toks)
        g_ids = gm.prefill(dev(toks)).cpu().numpy()
        lo, lg = om.logits()[0], gm.logits().cpu().numpy()[0]
        worst = max(worst, rel_err(lg, lo))
        assert rel_err(lg, lo) <= REL_TOL
        if check_ids:
            assert ids_agree(g_ids[0, 0], lo), (g_ids, o_ids, top2_gap(lo))
        nxt = o_ids
    for s in range(n_steps):
        o_ids = om.step(nxt)
        g_ids = gm.step(dev(nxt)).cpu().numpy()
        lo, lg = om.logits()[0], gm.logits().cpu().numpy()[0]
        r = rel_err(lg, lo)
        worst = max(worst, r)
        assert r <= REL_TOL, (s, r)
        if check_ids:
            assert ids_agree(g_ids[0, 0], lo), (s, g_ids, o_ids, top2_gap(lo))
        nxt = o_ids
    assert gm.n_past == om.n_past
    gm.synchronize()
    gm.close()
    return worst


SMALL = [("gpt2", "q4_0"), ("gpt2", "q8_0"), ("gpt2", "aff8"), ("llama", "q8_0"), ("llama", "q4_0"),
         ("llama", "aff8"), ("gpt2", "q5_0"), ("llama", "q5_0"), ("gpt2", "aff4_g64"), ("llama", "aff4_g64"),
         ("gpt2", "aff4_g32"), ("llama", "aff4_g32")]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("arch,fmt", SMALL)
def test_small_models_teacher_forced(arch, fmt, mode):
    cfg = synth.small_config(arch, fmt, d_ff=256, n_ctx=64)
    say(f"[model-small] {arch} {fmt} {mode}")
    w = synth.model_weights(cfg, 42, norm_std=0.5)
    worst = teacher_forced(cfg, w, n_prompt=9, n_steps=30, mode=mode)
    say(f"  worst rel {worst:.2e}")


@pytest.mark.parametrize("mode", MODES)
def test_small_llama_gqa_head128(mode):
    cfg = synth.small_config("llama", "q8_0", d_model=256, n_head=4, n_kv_head=2, head_dim=128, d_ff=256, n_ctx=96)
    say(f"[model-small] llama gqa hd128 {mode}")
    w = synth.model_weights(cfg, 7, norm_std=0.5)
    teacher_forced(cfg, w, n_prompt=70, n_steps=20, mode=mode)     # crosses a 64-key tile boundary


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("arch,fmt", [("gpt2", "q4_0"), ("llama", "q8_0")])
def test_small_models_topk_teacher_forced(arch, fmt, mode):
    """Top-k sampling on the device: both sides get the oracle's sampled id as the next input;
    the GPU's draw must equal the oracle's unless the oracle's u * total lies within 1e-4 of a
    cumulative boundary, or the k-th and (k+1)-th logits, or the drawn one and a neighbour in
    the walk, are within 1e-3."""
    k, T, seed = 5, 0.8, 1234
    cfg = synth.small_config(arch, fmt, d_ff=256, n_ctx=64, sample_mode=1, top_k=k, temperature=T, seed=seed)
    say(f"[model-small] top-k {arch} {fmt} {mode}")
    w = synth.model_weights(cfg, 42, norm_std=0.5)
    om = oracle.OracleModel(cfg, w)
    gm = gpu_model(cfg, w, mode)
    toks = synth.prompt_tokens(cfg, 6, seed=2)
    o_ids = om.prefill(toks)
    g_ids = gm.prefill(dev(toks)).cpu().numpy()
    checked = 0
    for s in range(40):
        pos = om.n_past - 1
        lo, lg = om.logits()[0], gm.logits().cpu().numpy()[0]
        assert rel_err(lg, lo) <= REL_TOL, (s, rel_err(lg, lo))
        ref, mg = chain_margins(lo, cfg, oracle.uniform24(seed, 0, pos, 0))
        assert ref == int(o_ids[0, 0])
        if not chain_near_boundary(mg):
            assert int(g_ids[0, 0]) == int(o_ids[0, 0]), (s, g_ids, o_ids, mg)
            checked += 1
        g_ids = gm.step(dev(o_ids)).cpu().numpy()
        o_ids = om.step(o_ids)
    assert checked >= 30
    gm.synchronize()
    gm.close()


CHAINS = {
    "t3": dict(sample_mode=1, top_k=50, temperature=0.8, top_p=0.9, rep_penalty=1.3, sample_order="t3"),
    "mtl": dict(sample_mode=1, top_k=100, temperature=0.9, min_p=0.05, top_p=0.9, rep_penalty=1.2, sample_order="mtl"),
    "greedy-penalty": dict(sample_mode=0, rep_penalty=1.5),
}


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("chain", list(CHAINS))
@pytest.mark.parametrize("arch,fmt", [("gpt2", "q4_0"), ("llama", "q8_0")])
def test_small_models_chain_teacher_forced(arch, fmt, chain, mode):
    """The sampler chain on the device, teacher forced: the repetition penalty's history is every
    token consumed so far (the prompt included); the GPU's id must equal the oracle's unless one
    of the chain's decisions lies within the tolerance of its boundary."""
    cfg = synth.small_config(arch, fmt, d_ff=256, n_ctx=80, seed=4321, **CHAINS[chain])
    say(f"[model-small] chain {chain} {arch} {fmt} {mode}")
    w = synth.model_weights(cfg, 42, norm_std=0.5)
    om = oracle.OracleModel(cfg, w)
    gm = gpu_model(cfg, w, mode)
    toks = synth.prompt_tokens(cfg, 6, seed=2)
    consumed = [int(t) for t in toks.ravel()]
    o_ids = om.prefill(toks)
    g_ids = gm.prefill(dev(toks)).cpu().numpy()
    checked = 0
    for s in range(60):
        pos = om.n_past - 1
        lo, lg = om.logits()[0], gm.logits().cpu().numpy()[0]
        assert rel_err(lg, lo) <= REL_TOL, (s, rel_err(lg, lo))
        ref, mg = chain_margins(lo, cfg, oracle.uniform24(cfg["seed"], 0, pos, 0), consumed)
        assert ref == int(o_ids[0, 0])
        if not chain_near_boundary(mg):
            assert int(g_ids[0, 0]) == int(o_ids[0, 0]), (s, g_ids, o_ids, mg)
            checked += 1
        consumed.append(int(o_ids[0, 0]))
        g_ids = gm.step(dev(o_ids)).cpu().numpy()
        o_ids = om.step(o_ids)
    assert checked >= 30                      # at least half of the steps decide clearly
    gm.synchronize()
    gm.close()


BATCH2 = {
    "greedy": dict(),
    "chain": dict(sample_mode=1, top_k=50, temperature=0.8, top_p=0.9, rep_penalty=1.3, sample_order="t3"),
    "cfg-greedy": dict(cfg=1, cfg_weight=1.5),
    "cfg-chain": dict(cfg=1, cfg_weight=0.5, sample_mode=1, top_k=100, temperature=0.9, min_p=0.05, top_p=0.9,
                      rep_penalty=1.2, sample_order="mtl"),
}


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("variant", list(BATCH2))
@pytest.mark.parametrize("arch,fmt", [("gpt2", "q4_0"), ("llama", "q8_0")])
def test_batch2_teacher_forced(arch, fmt, variant, mode):
    """Two rows in one step (each weight read once for both): two independent streams, or a
    classifier-free-guided pair (row 0 conditioned, row 1 not) whose one draw both rows take.
    Both rows' logits are one tensor at rel <= 2e-3; ids as in the other teacher-forced tests."""
    cfg = synth.small_config(arch, fmt, batch=2, d_ff=256, n_ctx=80, seed=99, **BATCH2[variant])
    say(f"[model-small] batch 2 {variant} {arch} {fmt} {mode}")
    w = synth.model_weights(cfg, 42, norm_std=0.5)
    om = oracle.OracleModel(cfg, w)
    gm = gpu_model(cfg, w, mode)
    toks = synth.prompt_tokens(cfg, 6, seed=2)                  # a different prompt per row
    consumed = [[int(t) for t in toks[b, :, 0]] for b in range(2)]
    o_ids = om.prefill(toks)
    g_ids = gm.prefill(dev(toks)).cpu().numpy()
    guided = cfg.get("cfg", 0) == 1
    checked = 0
    for s in range(40):
        pos = om.n_past - 1
        lo, lg = om.logits(), gm.logits().cpu().numpy()
        assert rel_err(lg, lo) <= REL_TOL, (s, rel_err(lg, lo))
        if guided:
            assert int(g_ids[0, 0]) == int(g_ids[1, 0]) and int(o_ids[0, 0]) == int(o_ids[1, 0])
            gl = lo[0] + cfg["cfg_weight"] * (lo[0] - lo[1])
            cases = [(0, gl)]
        else:
            cases = [(b, lo[b]) for b in range(2)]
        for b, l in cases:
            ref, mg = chain_margins(l, cfg, oracle.uniform24(cfg["seed"], b, pos, 0), consumed[b])
            assert ref == int(o_ids[b, 0])
            if not chain_near_boundary(mg):
                assert int(g_ids[b, 0]) == int(o_ids[b, 0]), (s, b, g_ids, o_ids, mg)
                checked += 1
        for b in range(2):
            consumed[b].append(int(o_ids[b, 0]))
        g_ids = gm.step(dev(o_ids)).cpu().numpy()
        o_ids = om.step(o_ids)
    assert checked >= (20 if guided else 40)
    gm.synchronize()
    gm.close()


@pytest.mark.parametrize("n_wg", [1, 7, 37])
def test_persistent_step_any_grid(n_wg):
    """Grids smaller than the tile counts: workgroups take several tiles of a phase, attention
    items wrap onto workgroups that also hold GEMV tiles, and a single workgroup runs it all."""
    cfg = synth.small_config("gpt2", "q4_0", d_ff=256, n_ctx=320, vocab=1000)
    say(f"[model-small] persistent grid {n_wg}")
    w = synth.model_weights(cfg, 5, norm_std=0.5)
    teacher_forced(cfg, w, n_prompt=0, n_steps=3, kv_pos=300, mode="persistent", n_wg=n_wg)   # two 256-key chunks


def test_gpt2_medium_one_layer_after_512_positions():
    """One GPT-2-Medium-shaped layer (d 1024, 16 x 64, FFN 4096, Q4_0) on a new token at
    position 512 over a random fp16 cache of 512 positions, input x ~ N(0,1)."""
    torch = torch_mod()
    cfg = synth.config("gpt2_layer_q4_0")
    say("[layer] gpt2 medium, 512 prior positions")
    w = synth.model_weights(cfg, 42)
    k, v = synth.kv_cache(cfg, 512, seed=42)
    x = synth.hidden(cfg, seed=42)
    om = oracle.OracleModel(cfg, w)
    om.load_kv(k, v, 512)
    ref = om.layer_forward(0, x, 512)
    gm = gpu_model(cfg, w)
    gm.load_kv(dev(k), dev(v), 512)
    got = gm.layer_forward(0, dev(x), 512).cpu().numpy()
    r = rel_err(got, ref)
    say(f"  rel {r:.2e}")
    assert r <= REL_TOL
    # the same position again (its cache slot is rewritten with the same values)
    got2 = gm.layer_forward(0, dev(x), 512).cpu().numpy()
    assert np.array_equal(got, got2)
    gm.close()


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name,kv_pos", [("gpt2_medium_q4_0", 755), ("llama520m_q8_0", 899), ("gpt2_medium_q4_0", 300),
                                         ("llama520m_q8_0", 511)])
def test_full_size_step_over_long_cache(name, kv_pos, mode):
    """All layers at their real shapes, one teacher-forced step at kv_pos and one more at the next
    position: the last positions of the decode runs (756 / 900 keys, 256-key attention chunks),
    301 keys (three 128-key chunks), and 512 then 513 keys (the persistent step switching from
    four 128-key chunks to three 256-key chunks between the two steps)."""
    cfg = synth.config(name)
    say(f"[model-full] {name} kv_pos={kv_pos} {mode}")
    w = synth.model_weights(cfg, 42)
    worst = teacher_forced(cfg, w, n_prompt=0, n_steps=2, kv_pos=kv_pos, mode=mode)
    say(f"  worst rel {worst:.2e}")


@pytest.mark.parametrize("name,kv_pos,guided", [("gpt2_medium_q4_0", 755, True), ("llama520m_q8_0", 899, True),
                                                 ("llama520m_q8_0", 899, False), ("llama520m_q8_0", 300, False)])
def test_full_size_pair_over_long_cache(name, kv_pos, guided):
    """The persistent pair at the real shapes (each weight read once for both rows): two
    teacher-forced steps over a random cache of kv_pos positions per row, both rows' logits as
    one tensor at rel <= 2e-3; a guided pair (weight 1.5) draws one id from the combined logits
    and both rows take it, two streams pick their own argmax."""
    cfg = dict(synth.config(name), batch=2)
    samp = dict(mode=0, cfg=1, cfg_weight=1.5) if guided else None
    if guided:
        cfg.update(cfg=1, cfg_weight=1.5)
    say(f"[model-full] {name} pair guided={guided} kv_pos={kv_pos}")
    w = synth.model_weights(cfg, 42)
    from quantized_gemv_kv_amd import Model
    gm = Model(dict(cfg, launch_mode="persistent"), w, sampling=samp)
    assert gm.uses_persistent_step()
    om = oracle.OracleModel(cfg, w)
    k, v = synth.kv_cache(cfg, kv_pos, seed=5)
    om.load_kv(k, v, kv_pos)
    gm.load_kv(dev(k), dev(v), kv_pos)
    nxt = synth.prompt_tokens(cfg, 1, seed=6)[:, 0, :]
    for s in range(2):
        o_ids = om.step(nxt)
        g_ids = gm.step(dev(nxt)).cpu().numpy()
        lo, lg = om.logits(), gm.logits().cpu().numpy()
        r = rel_err(lg, lo)
        say(f"  step {s}: rel {r:.2e}")
        assert r <= REL_TOL
        if guided:
            comb = lo[0] + 1.5 * (lo[0] - lo[1])
            assert int(g_ids[0, 0]) == int(g_ids[1, 0])
            assert ids_agree(g_ids[0, 0], comb), (g_ids, o_ids, top2_gap(comb))
        else:
            for b in range(2):
                assert ids_agree(g_ids[b, 0], lo[b]), (b, g_ids, o_ids)
        nxt = o_ids
    gm.synchronize()
    gm.close()


@pytest.mark.parametrize("name,batch,kv_pos", [("gpt2_medium_q4_0", 1, 1300), ("llama520m_q8_0", 2, 1100)])
def test_full_size_step_past_four_chunks(name, batch, kv_pos):
    """A context of more than four 256-key chunks (1,536 positions): the output projection's input
    merges the chunks' partials in rounds of four, which no shorter context reaches; two
    teacher-forced steps over a random cache, every row's logits at rel <= 2e-3."""
    cfg = dict(synth.config(name), n_ctx=1536, batch=batch)
    say(f"[model-full] {name} n_ctx=1536 batch={batch} kv_pos={kv_pos}")
    w = synth.model_weights(cfg, 42)
    from quantized_gemv_kv_amd import Model
    gm = Model(dict(cfg, launch_mode="persistent"), w)
    assert gm.uses_persistent_step()
    om = oracle.OracleModel(cfg, w)
    k, v = synth.kv_cache(cfg, kv_pos, seed=5)
    om.load_kv(k, v, kv_pos)
    gm.load_kv(dev(k), dev(v), kv_pos)
    nxt = synth.prompt_tokens(cfg, 1, seed=6)[:, 0, :]
    for s in range(2):
        o_ids = om.step(nxt)
        g_ids = gm.step(dev(nxt)).cpu().numpy()
        lo, lg = om.logits(), gm.logits().cpu().numpy()
        r = rel_err(lg, lo)
        say(f"  step {s}: rel {r:.2e}")
        assert r <= REL_TOL
        for b in range(batch):
            assert ids_agree(g_ids[b, 0], lo[b]), (b, g_ids, o_ids)
        nxt = o_ids
    gm.synchronize()
    gm.close()


@pytest.mark.parametrize("n_wg,kv_pos", [(208, 100), (208, 300)])
def test_full_size_step_on_a_smaller_grid(n_wg, kv_pos):
    """The GPT-2-Medium-shaped T3 on 208 workgroups: 192 QKV tiles leave 16 workgroups for the
    attention items, one chunk per head (101 keys) or two (301 keys), so the items of a head
    share workgroups with the product's tiles at the longer context."""
    cfg = synth.config("gpt2_medium_q4_0")
    say(f"[model-full] gpt2_medium n_wg={n_wg} kv_pos={kv_pos}")
    w = synth.model_weights(cfg, 42)
    worst = teacher_forced(cfg, w, n_prompt=0, n_steps=2, kv_pos=kv_pos, mode="persistent", n_wg=n_wg)
    say(f"  worst rel {worst:.2e}")


@pytest.mark.parametrize("mode", MODES)
def test_full_size_gpt2_q5_0_step_over_long_cache(mode):
    """The GPT-2-Medium-shaped T3 in Q5_0 (q ~ U{0..31}, d = |N| 0.02) at the decode run's last
    position."""
    cfg = dict(synth.config("gpt2_medium_q4_0"), wfmt="q5_0")
    say(f"[model-full] gpt2_medium q5_0 kv_pos=755 {mode}")
    w = synth.model_weights(cfg, 42)
    worst = teacher_forced(cfg, w, n_prompt=0, n_steps=2, kv_pos=755, mode=mode)
    say(f"  worst rel {worst:.2e}")


def test_full_size_gpt2_prefill_then_decode():
    cfg = synth.config("gpt2_medium_q4_0")
    say("[model-full] gpt2 prefill 6 + 3 steps")
    w = synth.model_weights(cfg, 42)
    teacher_forced(cfg, w, n_prompt=6, n_steps=3)


@pytest.mark.parametrize("mode", MODES)
def test_free_running_greedy_matches_history(mode):
    """The benchmarked path: no input ids, the graph feeds its own samples forward."""
    torch = torch_mod()
    cfg = synth.small_config("gpt2", "q4_0", d_ff=256, n_ctx=64)
    w = synth.model_weights(cfg, 42, norm_std=0.5)
    gm = gpu_model(cfg, w, mode)
    om = oracle.OracleModel(cfg, w)
    toks = synth.prompt_tokens(cfg, 5, seed=1)
    first = gm.prefill(dev(toks)).cpu().numpy()
    o = om.prefill(toks)
    ids = [int(first[0, 0])]
    for _ in range(20):
        ids.append(int(gm.step(None).cpu().numpy()[0, 0]))
    hist = gm.tokens(4, 21).cpu().numpy()[:, 0, 0]
    assert list(hist) == ids
    # oracle free-running from the same prompt: identical while no near-tie occurs
    o_ids = [int(o[0, 0])]
    for _ in range(20):
        lo = om.logits()[0]
        if top2_gap(lo) < 1e-3:
            break
        o_ids.append(int(om.step()[0, 0]))
    assert ids[:len(o_ids)] == o_ids


def test_guidance_needs_a_two_row_model():
    from quantized_gemv_kv_amd import Model, TsdError
    cfg = synth.small_config("llama", "q8_0")
    w = synth.model_weights(cfg, 1)
    with pytest.raises(TsdError) as e:
        Model(cfg, w, sampling=dict(mode=0, cfg=1, cfg_weight=1.0))
    assert e.value.status == 1


def test_errors_leave_state_unchanged():
    torch = torch_mod()
    from quantized_gemv_kv_amd import TsdError, binding
    cfg = synth.small_config("llama", "q8_0", d_ff=256, n_ctx=16)
    w = synth.model_weights(cfg, 1)
    gm = gpu_model(cfg, w)
    gm.prefill(dev(synth.prompt_tokens(cfg, 10)))
    with pytest.raises(TsdError) as e:
        gm.prefill(dev(synth.prompt_tokens(cfg, 7)))
    assert e.value.status == 4                     # TSD_ERR_CONTEXT_FULL
    assert gm.n_past == 10
    with pytest.raises(TsdError) as e:
        gm.prefill_stepwise(dev(synth.prompt_tokens(cfg, 7)))
    assert e.value.status == 4
    assert gm.n_past == 10
    with pytest.raises(TsdError) as e:
        gm.get_kv(11)                              # beyond what the cache holds
    assert e.value.status == 1
    k, v = gm.get_kv(0)
    assert k.shape[3] == 0 and v.shape[3] == 0
    with pytest.raises(TsdError):
        gm.truncate(11)
    gm.truncate(3)
    assert gm.n_past == 3
    for _ in range(13):
        gm.step()
    with pytest.raises(TsdError) as e:
        gm.step()
    assert e.value.status == 4
    gm.close()
    with pytest.raises(TsdError):
        gpu_model(cfg, w[:-1])                     # wrong number of weights
    with pytest.raises(TsdError):
        gpu_model(dict(cfg, d_model=130), w)       # K not a multiple of the block
    with pytest.raises(TsdError) as e:
        gpu_model(cfg, w, n_wg=100000)             # more workgroups than can be resident
    assert e.value.status == 2


@pytest.mark.parametrize("arch,fmt,batch,mode", [
    ("gpt2", "q4_0", 1, "persistent"), ("gpt2", "q4_0", 1, "per_operator"), ("llama", "q8_0", 2, "persistent"),
    ("llama", "q8_0", 1, "per_operator"),
])
def test_step_ids_outside_the_vocabulary_are_rejected(arch, fmt, batch, mode):
    """A step given an id outside [0, vocab) does nothing, and neither does any call after it until
    tsd_synchronize, which reports TSD_ERR_INVALID_ARGUMENT and sets n_past back: the ids, history,
    logits and cache of the earlier positions are unchanged bit for bit, and the model then goes on
    exactly as one that never saw the bad id."""
    from quantized_gemv_kv_amd import TsdError
    torch = torch_mod()
    cfg = synth.small_config(arch, fmt, d_ff=256, n_ctx=64, batch=batch)
    say(f"[step] bad ids, {arch} {fmt} batch {batch} {mode}")
    w = synth.model_weights(cfg, 5, norm_std=0.5)
    prompt = dev(synth.prompt_tokens(cfg, 9, seed=2))
    good = torch.tensor([[3]] * batch, dtype=torch.int32, device="cuda")

    def state(m):
        k, v = m.get_kv(m.n_past)
        return (m.n_past, m.logits().cpu().numpy(), m.tokens(0, m.n_past).cpu().numpy(),
                k.cpu().numpy().view(np.uint16), v.cpu().numpy().view(np.uint16))

    ref = gpu_model(cfg, w, mode)
    ref.prefill(prompt)
    ref.step(good)
    ref.step(None)
    want = state(ref)
    ref.close()
    for bad_id in (-1, cfg["vocab"], 1 << 30):
        gm = gpu_model(cfg, w, mode)
        gm.prefill(prompt)
        before = state(gm)
        bad = good.clone()
        bad[batch - 1, 0] = bad_id
        gm.step(bad)
        gm.step(None)
        gm.step(good)
        assert gm.n_past == 12                     # counted until the device says otherwise
        with pytest.raises(TsdError) as e:
            gm.synchronize()
        assert e.value.status == 1
        after = state(gm)
        assert after[0] == before[0] == 9
        for x, y in zip(before[1:], after[1:]):
            assert np.array_equal(x, y)
        gm.synchronize()                           # reported once
        gm.step(good)
        gm.step(None)
        got = state(gm)
        assert got[0] == want[0]
        for x, y in zip(want[1:], got[1:]):
            assert np.array_equal(x, y)
        gm.close()


def test_step_timing_kinds_follow_launch_mode():
    from quantized_gemv_kv_amd import TsdError
    cfg = synth.small_config("gpt2", "q4_0", d_ff=256, n_ctx=64)
    w = synth.model_weights(cfg, 42, norm_std=0.5)
    for mode, ok, bad in (("persistent", "step", "qkv"), ("per_operator", "qkv", "step")):
        gm = gpu_model(cfg, w, mode)
        gm.prefill(dev(synth.prompt_tokens(cfg, 4)))
        us, n = gm.time_kernel(ok, 3)
        assert us > 0 and n >= 1
        before = gm.n_past
        with pytest.raises(TsdError) as e:
            gm.time_kernel(bad, 3)
        assert e.value.status == 2 and gm.n_past == before
        gm.synchronize()
        gm.close()


def test_persistent_time_out_reruns_lost_steps_per_operator():
    """A persistent step that gives up on a bounded wait (forced from the host: a wait limit of one
    tick, so every workgroup leaves the kernel normally) voids itself and the persistent launches
    after it.  tsd_synchronize then switches the model to one launch per operator and runs the
    lost steps again, since they took their ids from the device: the ids follow the oracle's
    free-running greedy decode as if nothing had happened."""
    cfg = synth.small_config("gpt2", "q4_0", d_ff=256, n_ctx=64)
    w = synth.model_weights(cfg, 42, norm_std=0.5)
    gm = gpu_model(cfg, w, "persistent")
    om = oracle.OracleModel(cfg, w)
    toks = synth.prompt_tokens(cfg, 5, seed=1)
    gm.prefill(dev(toks))
    o = om.prefill(toks)
    for _ in range(3):
        gm.step(None, out=False)
    gm.synchronize()
    gm.debug_set_wait_limit(1)
    for _ in range(4):
        gm.step(None, out=False)
    gm.synchronize()   # the four lost steps run again, one launch per operator
    assert gm.info()[0] == "per_operator"
    for _ in range(3):
        gm.step(None, out=False)
    gm.synchronize()
    assert gm.n_past == 15
    ids = [int(v) for v in gm.tokens(4, 11).cpu().numpy()[:, 0, 0]]
    o_ids = [int(o[0, 0])]
    for _ in range(10):
        if top2_gap(om.logits()[0]) < TIE_GAP:
            break
        o_ids.append(int(om.step()[0, 0]))
    assert ids[:len(o_ids)] == o_ids
    gm.close()
    om.close()


def test_persistent_time_out_with_caller_ids_rolls_back():
    """When the lost steps took ids from a caller buffer, tsd_synchronize reports TSD_ERR_TIMEOUT and
    sets n_past back to the first lost position; the caller submits those positions again, now with
    one launch per operator, and they match the oracle."""
    from quantized_gemv_kv_amd import TsdError
    cfg = synth.small_config("gpt2", "q4_0", d_ff=256, n_ctx=64)
    w = synth.model_weights(cfg, 42, norm_std=0.5)
    gm = gpu_model(cfg, w, "persistent")
    om = oracle.OracleModel(cfg, w)
    toks = synth.prompt_tokens(cfg, 5, seed=2)
    gm.prefill(dev(toks))
    nxt = om.prefill(toks)
    gm.synchronize()
    gm.debug_set_wait_limit(1)
    gm.step(dev(nxt))
    gm.step(dev(nxt))
    with pytest.raises(TsdError) as e:
        gm.synchronize()
    assert e.value.status == 7 and gm.n_past == 5
    assert gm.info()[0] == "per_operator"
    for s in range(3):
        o_ids = om.step(nxt)
        gm.step(dev(nxt))
        lo, lg = om.logits()[0], gm.logits().cpu().numpy()[0]
        assert rel_err(lg, lo) <= REL_TOL, (s, rel_err(lg, lo))
        nxt = o_ids
    assert gm.n_past == om.n_past
    gm.synchronize()
    gm.close()
    om.close()
