"""Decode-step benchmark on one MI355X.

Workload (the pages' T3 decoder at its real shape): a 24-layer GPT-2-Medium-shaped speech-token
decoder, d 1024, 16 heads x 64, FFN 4096, learned positions, vocab 8192 head, Q4_0 weights,
fp32 norms/embeddings ~N(0, 0.02), fp16 KV cache; 256-token prefill, then greedy decode steps at
positions 256 .. 255+K, batch 1.  All inputs are seeded synthetic data.  --workload
llama520m_q8_0 times the 30-layer Llama-shaped Q8_0 decoder instead (300-token prefill), and
--workload talker_cp_aff8 the Qwen3-TTS-shaped Talker (28 layers) + code predictor (5 layers,
15 passes) frame loop with 8-bit affine weights at batch 16 (170 prompt frames, then K frames);
its line also carries "gemm_rows", the batched matrix-core GEMM alone on a matrix larger than
the Infinity Cache.

The line also carries "gemv": the standalone quantized GEMV on one 524288 x 1024 Q8_0 matrix
(~570 MB, more than the Infinity Cache holds), where a launch is amortised; and "prefill": the
prompt (the prompt pass over every prompt position but the last, then one decode step) timed
once under HIP events after an untimed first run.

One step = one replay of the captured decode graph (every layer, the head and the greedy
sampler); by default the graph holds one persistent launch that runs the whole step.  W warm-up
steps run first and the context is then truncated back to 256 positions, so the K timed steps
cover exactly the positions of the configured run.  The timed region is bracketed by stream
synchronisation and hipEvents recorded on the model's stream.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# workload name -> (prompt positions, default steps, description, dtype)
WORKLOADS = {
    "gpt2_medium_q4_0": (256, 500, "GPT-2-Medium-shaped 24-layer speech-token decoder, Q4_0, 256-token prefill then {K} "
                                   "{S} decode steps, batch 1", "q4_0 weights, fp32 accumulate, fp16 kv"),
    "gpt2_medium_q5_0": (256, 500, "GPT-2-Medium-shaped 24-layer speech-token decoder, Q5_0, 256-token prefill then {K} "
                                   "{S} decode steps, batch 1", "q5_0 weights, fp32 accumulate, fp16 kv"),
    "llama520m_q8_0": (300, 600, "Llama-shaped ~520M 30-layer speech-token decoder, Q8_0, 300-token prefill then {K} "
                                 "{S} decode steps, batch 1", "q8_0 weights, fp32 accumulate, fp16 kv"),
    "talker_cp_aff8": (170, 200, "Talker (28 layers, d 1024, 16 q / 8 kv heads of 128, SwiGLU 3072) + code predictor "
                                 "(5 layers, 15 sequential passes, vocab 2048), 8-bit affine group-64 weights, "
                                 "170 prompt frames then {K} {S} frames of 16 codes, batch 16",
                       "aff8 weights, fp16 hi/lo x fp16 weight MFMA with fp32 accumulate, fp16 kv"),
}
WORKLOAD = "gpt2_medium_q4_0"
PROMPT = 256

# sampler presets: greedy (the headline and the parity reference); the T3 port's defaults
# ("Chatterbox -> ggml Port: Development Journal", §3.9 table: top-k 1000, top-p 0.95,
# temperature 0.8, repetition penalty 1.2); the Qwen3-TTS harness's settings ("Every Frame Is a
# Memory Read", the baseline table: temperature 0.9, top-p 0.95, top-k 50, repetition penalty 1.05)
SAMPLERS = {
    "greedy": None,
    "t3": dict(mode=1, top_k=1000, temperature=0.8, top_p=0.95, rep_penalty=1.2, order="t3"),
    "qwen": dict(mode=1, top_k=50, temperature=0.9, top_p=0.95, rep_penalty=1.05, order="t3"),
}


def with_sampler(cfg, samp):
    """The oracle's config fields for a sampling dict (None: greedy)."""
    if samp is None:
        return cfg
    return dict(cfg, sample_mode=samp.get("mode", 0), top_k=samp.get("top_k", 0), temperature=samp.get("temperature", 1.0),
                seed=samp.get("seed", 0), top_p=samp.get("top_p", 0.0), min_p=samp.get("min_p", 0.0),
                rep_penalty=samp.get("rep_penalty", 1.0), sample_order=samp.get("order", "t3"), cfg=samp.get("cfg", 0),
                cfg_weight=samp.get("cfg_weight", 0.0))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", default="gpt2_medium_q4_0", choices=sorted(WORKLOADS),
                    help="the decoder timed (the default is the one the headline metric is quoted on)")
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=42)
    ap.add_argument("--cfg", type=float, default=None, metavar="W",
                    help="classifier-free guidance with weight W: two rows (conditioned, unconditioned prompts) "
                         "per step, one token drawn from cond + W (cond - uncond)")
    ap.add_argument("--sampler", default="greedy", choices=sorted(SAMPLERS),
                    help="greedy, or a sampler-chain preset (t3: the T3 port's defaults; qwen: the Qwen3-TTS settings)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemv", action="store_true", help="skip the standalone tall-GEMV measurement")
    ap.add_argument("--gemv-format", default="q8_0", choices=["q8_0", "q4_0", "q5_0", "aff8", "aff4_g64", "aff4_g32"],
                    help="weight format of the standalone tall GEMV (q8_0: the lone-GEMV workload's)")
    ap.add_argument("--eager", action="store_true",
                    help="enqueue each step kernel by kernel instead of replaying the graph (for counter "
                         "collection, which cannot follow graph launches); prefill is skipped: the cache "
                         "is filled with random values instead")
    ap.add_argument("--launch-mode", default="persistent", choices=["persistent", "per_operator"],
                    help="one persistent launch per step, or one launch per operator")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one plain fp32 device copy of this size (a known-traffic kernel for "
                         "scaling hardware byte counters)")
    return ap.parse_args()


# what the step kernel is compiled from: its sources, and the step-argument block of kernels.h
STEP_SOURCES = ["quantized_gemv_kv_amd/csrc/" + f for f in ("step.hip", "exchange.h", "gemv_core.h", "common.h")]
STEP_DECLS = ("quantized_gemv_kv_amd/csrc/kernels.h", "// ---- persistent decode step", "// ---- sampler chain")


def step_sources_hash():
    import hashlib
    h = hashlib.sha256()
    for f in STEP_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    path, a, b = STEP_DECLS
    with open(os.path.join(ROOT, path)) as fh:
        text = fh.read()
    h.update(text[text.index(a):text.index(b)].encode())
    return h.hexdigest()[:16]
COUNTERS = os.path.join(ROOT, "profiles", "step_gpt2_medium_q4_0_counters.json")


def counted_traffic(kernel, workload="gpt2_medium_q4_0"):
    """HBM-side bytes per launch of the step kernel from the committed FETCH_SIZE / WRITE_SIZE
    summary (scaled by the copy calibration), or None when that summary was taken on other
    kernel sources than the ones built now."""
    if kernel != "step" or workload != "gpt2_medium_q4_0" or not os.path.exists(COUNTERS):
        return None
    with open(COUNTERS) as fh:
        d = json.load(fh)
    return d["traffic_bytes_per_launch"] if d.get("sources_sha256_16") == step_sources_hash() else None


class DeviceState:
    """amd-smi samples (socket power, graphics and memory clocks, temperatures) taken by a
    background thread while the benchmark runs; summary() reports those that fall inside the
    timed region (and the run's maximum power), or null fields where amd-smi is unavailable."""

    def __init__(self):
        import threading
        self.samples, self.stop = [], threading.Event()
        self.thread = threading.Thread(target=self._run, daemon=True)
        self.thread.start()

    @staticmethod
    def _one():
        import subprocess
        out = subprocess.run(["/opt/rocm/bin/amd-smi", "metric", "-g", "0", "-p", "-t", "-c", "--json"],
                             capture_output=True, text=True, timeout=20).stdout
        d = json.loads(out)
        g = d["gpu_data"][0] if isinstance(d, dict) and "gpu_data" in d else d[0]
        num = lambda v: v["value"] if isinstance(v, dict) and isinstance(v.get("value"), (int, float)) else None
        gfx = [num(c["clk"]) for k, c in g["clock"].items() if k.startswith("gfx_")]
        gfx = [v for v in gfx if v is not None]
        return {"power_w": num(g["power"]["socket_power"]), "gfx_mhz_max": max(gfx) if gfx else None,
                "gfx_mhz_mean": sum(gfx) / len(gfx) if gfx else None, "mem_mhz": num(g["clock"]["mem_0"]["clk"]),
                "hotspot_c": num(g["temperature"]["hotspot"]), "mem_c": num(g["temperature"]["mem"])}

    def _run(self):
        while not self.stop.is_set():
            t0 = time.perf_counter()
            try:
                v = self._one()
            except Exception:
                return
            self.samples.append((t0, time.perf_counter(), v))

    LAG = 0.5   # seconds by which amd-smi's metrics trail the device (measured on this board)

    def summary(self, t_begin, t_end):
        self.stop.set()
        inside = [v for a, b, v in self.samples if t_begin + self.LAG <= b <= t_end + self.LAG + 0.1]
        powers = [v["power_w"] for _, _, v in self.samples if v["power_w"] is not None]
        return {"samples_in_timed_region": inside, "samples_total": len(self.samples),
                "max_power_w": max(powers) if powers else None,
                "tool": "amd-smi metric -p -t -c, sampled in a background thread; a reading trails the device by "
                        "about 0.5 s, so the timed region's samples are those read 0.5 s after it"}


def warm(call, seconds=0.25):
    """Back-to-back launches for about `seconds` before a timed measurement: on a GPU that has
    been idle the board's power management first runs a launch at full speed, then slows the
    next ~100 ms while it changes state, so bursts timed straight away are mixed."""
    import time
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            call()
        torch.cuda.synchronize()


TALL_N, TALL_K = 524288, 1024      # one Q8_0 GEMV of ~570 MB, larger than the 256 MB Infinity Cache


def gemv_headline(seed, reps=7, fmt="q8_0"):
    """The quantized GEMV alone at a size where a launch is amortised: y = W x with W a
    524288 x 1024 Q8_0 matrix (the lone-GEMV law), x ~ N(0,1), batch 1; after a quarter second of
    warm-up launches, the median over `reps` bursts of 10 back-to-back launches timed with HIP
    events.  Bytes = the stored matrix + x + y."""
    import torch
    from quantized_gemv_kv_amd import binding, roofline, synth
    N, K = TALL_N, TALL_K
    canon = torch.empty(roofline.matrix_bytes(fmt, N, K), dtype=torch.uint8, device="cuda")
    if fmt == "q8_0":
        row_b = K // 32 * 34
        for r0, blob in synth.q8_0_row_chunks(N, K, seed):
            canon[r0 * row_b: r0 * row_b + blob.size].copy_(torch.from_numpy(blob))
    else:
        synth.matrix_into(fmt, N, K, seed, canon)
    packed = torch.empty(binding.tsd_gemv_packed_bytes(fmt, N, K), dtype=torch.uint8, device="cuda")
    binding.tsd_gemv_pack(fmt, canon, N, K, packed)
    del canon
    x = torch.from_numpy(synth.normal_f32(synth.rng_for(seed, 1), (1, K))).cuda()
    y = torch.empty((1, N), dtype=torch.float32, device="cuda")
    warm(lambda: binding.tsd_gemv(fmt, packed, N, K, 1, x, None, y))
    # median over short bursts of back-to-back launches (about 1 ms each, timed with HIP events
    # around the burst): long runs of full-bandwidth streaming are slowed by the board's power
    # management, which would make the figure depend on the run length
    burst, times = 10, []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(burst):
            binding.tsd_gemv(fmt, packed, N, K, 1, x, None, y)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / burst)
    us = float(np.median(times))
    nbytes = roofline.gemv_bytes(fmt, N, K)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"shape": f"{fmt.upper()} {N}x{K}, batch 1", "bytes": nbytes, "us": us, "gbs": gbs,
            "frac": gbs / roofline.HBM_PEAK_GBS, "timing": f"median over {reps} bursts of {burst} back-to-back launches, after 0.25 s of warm-up launches"}


def cpu_baseline(cfg, weights, seconds, seed):
    """The CPU oracle as it stands (single-threaded C, fp64), timed on this host: decode steps
    from position 256 over a random 256-position fp16 cache, until the time budget is spent."""
    import oracle
    om = oracle.OracleModel(cfg, weights)
    from quantized_gemv_kv_amd import synth
    k, v = synth.kv_cache(cfg, PROMPT, seed=seed)
    om.load_kv(k, v, PROMPT)
    tok = np.array([[1]], np.int32)
    n = 0
    t0 = time.perf_counter()
    while True:
        tok = om.step(tok)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 64:
            break
    om.close()
    return {"value": n / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} decode steps of the same {cfg['n_layer']}-layer model at positions {PROMPT}..{PROMPT + n - 1} "
                      f"over a random {PROMPT}-position fp16 cache, single-threaded fp64 oracle, {el:.1f} s"}


def cpu_baseline_frames(cfg, weights, seconds, seed):
    """The CPU oracle on one batch row of the frame loop (rows are independent, so a 16-row frame
    costs 16 row-frames): frames at positions 170.. over a random 170-position Talker cache."""
    import oracle
    from quantized_gemv_kv_amd import synth
    c1 = dict(cfg, batch=1)
    om = oracle.OracleModel(c1, weights)
    k, v = synth.kv_cache(c1, PROMPT, seed=seed)
    om.load_kv(k, v, PROMPT)
    codes = synth.prompt_tokens(c1, 1, seed=seed)[:, 0, :]
    n = 0
    t0 = time.perf_counter()
    while True:
        codes = om.step(codes)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 16:
            break
    om.close()
    rows = cfg["batch"]
    return {"value": n / el / rows, "unit": "frames/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} frames of one batch row (Talker {cfg['n_layer']} layers + {cfg['n_codebooks'] - 1} predictor "
                      f"passes) at positions {PROMPT}..{PROMPT + n - 1} over a random {PROMPT}-position fp16 cache, "
                      f"single-threaded fp64 oracle, {el:.1f} s; the {rows}-row rate is that rate / {rows}"}


GEMM_N, GEMM_K = 131072, 2048   # one 8-bit affine matrix of ~270 MB, larger than the Infinity Cache


def gemm_rows_headline(seed, reps=7):
    """The batched matrix-core GEMM alone at a size where a launch is amortised: Y = W X for 16
    rows, W 131072 x 2048 in 8-bit affine groups of 64 (the frame's weight law), X ~ N(0,1);
    median over bursts of back-to-back calls (operand interleave, GEMM).  Bytes = the stored
    matrix (tiled: quants, then one scale/bias word per row and group) + X read + Y written."""
    import torch
    from quantized_gemv_kv_amd import binding, roofline, synth
    N, K, B = GEMM_N, GEMM_K, 16
    canon = torch.empty(roofline.matrix_bytes("aff8", N, K), dtype=torch.uint8, device="cuda")
    chunk = 16384
    qs, ss, bs = [], [], []
    for r0 in range(0, N, chunk):
        blob = synth.aff8_matrix(synth.rng_for(seed, r0, K), chunk, K)[0]
        nq, ng = chunk * K, chunk * (K // 64)
        qs.append(torch.from_numpy(blob[:nq]))
        ss.append(torch.from_numpy(blob[nq:nq + 2 * ng]))
        bs.append(torch.from_numpy(blob[nq + 2 * ng:]))
    nq = N * K
    canon[:nq].copy_(torch.cat(qs))
    canon[nq:nq + N * (K // 64) * 2].copy_(torch.cat(ss))
    canon[nq + N * (K // 64) * 2:].copy_(torch.cat(bs))
    del qs, ss, bs
    packed = torch.empty(binding.tsd_gemm_rows_packed_bytes(N, K), dtype=torch.uint8, device="cuda")
    binding.tsd_gemm_rows_pack(canon, N, K, packed)
    del canon
    x = torch.from_numpy(synth.normal_f32(synth.rng_for(seed, 2), (B, K))).cuda()
    y = torch.empty((B, N), dtype=torch.float32, device="cuda")
    scratch = torch.empty(binding.tsd_gemm_rows_scratch_bytes(N, K, 1), dtype=torch.uint8, device="cuda")
    warm(lambda: binding.tsd_gemm_rows(packed, N, K, B, x, y, 1, scratch))
    burst, times = 10, []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(burst):
            binding.tsd_gemm_rows(packed, N, K, B, x, y, 1, scratch)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / burst)
    us = float(np.median(times))
    nbytes = roofline.matrix_bytes("aff8", N, K) + 4 * B * (K + N)   # the tiled layout stores the same bytes
    gbs = nbytes / (us * 1e-6) / 1e9
    flops = 2.0 * N * K * B
    return {"shape": f"aff8 {N}x{K}, 16 rows", "bytes": nbytes, "us": us, "gbs": gbs,
            "frac": gbs / roofline.HBM_PEAK_GBS, "tflops": flops / (us * 1e-6) / 1e12,
            "timing": f"median over {reps} bursts of {burst} back-to-back calls (operand split + GEMM), after 0.25 s of warm-up calls"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library runs the decode step "
              f"on a single GPU and does not shard it.", file=sys.stderr)
        sys.exit(2)
    import torch
    from quantized_gemv_kv_amd import Model, roofline, synth

    global WORKLOAD, PROMPT
    WORKLOAD = args.workload
    PROMPT, default_steps, desc, dtype = WORKLOADS[WORKLOAD]
    if args.steps is None:
        args.steps = default_steps
    cfg = dict(synth.config(WORKLOAD), launch_mode=args.launch_mode)
    frames = cfg["arch"] == "talker_cp"
    if args.cfg is not None:
        if frames:
            print("--cfg applies to the GPT2/LLAMA workloads", file=sys.stderr)
            sys.exit(2)
        cfg["batch"] = 2
    K, W = args.steps, args.warmup
    if PROMPT + max(K, W) > cfg["n_ctx"]:
        print(f"steps/warmup exceed the {cfg['n_ctx']}-position context", file=sys.stderr)
        sys.exit(2)
    weights = synth.model_weights(cfg, args.seed)
    stream = torch.cuda.Stream()
    samp = SAMPLERS[args.sampler]
    if samp is not None:
        samp = dict(samp, seed=args.seed)
    if args.cfg is not None:
        samp = dict(samp or {"mode": 0, "seed": args.seed}, cfg=1, cfg_weight=args.cfg)
    model = Model(cfg, weights, stream=stream, sampling=samp)
    prompt = torch.from_numpy(synth.prompt_tokens(cfg, PROMPT, seed=args.seed)).to("cuda")
    dev_state = DeviceState()
    step = model.step_eager if args.eager else model.step
    with torch.cuda.stream(stream):
        if args.eager:
            k, v = synth.kv_cache(cfg, PROMPT, seed=args.seed)
            model.load_kv(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), PROMPT)
        else:
            # the prompt, once untimed (first launches of its kernels), then again from a reset
            # model under events
            model.prefill(prompt)
            stream.synchronize()
            model.reset()
            p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            p0.record(stream)
            model.prefill(prompt)
            p1.record(stream)
            stream.synchronize()
            prefill_ms = p0.elapsed_time(p1)
        for _ in range(W):
            step(None, out=False)
        stream.synchronize()
        model.truncate(PROMPT)
        stream.synchronize()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(K):
            step(None, out=False)
        e1.record(stream)
        stream.synchronize()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        wall = t1 - t0
    ms = e0.elapsed_time(e1)
    ids = model.tokens(PROMPT, K).cpu().numpy()
    if frames:
        assert ids[..., 1:].max() < cfg["cp_vocab"], "sampled codes out of range"
    ids = ids.reshape(-1)
    assert ids.min() >= 0 and ids.max() < cfg["vocab"], "sampled ids out of range"

    # dominant kernel: every kind timed inside real steps (event records around each launch on
    # the model's stream), then the largest one re-timed over the timed region's positions.
    # With the persistent step there is one kind: the step kernel itself.
    mode, n_wg = model.info()
    kind_list = ("step",) if mode == "persistent" else ("qkv", "attn", "oproj", "fc", "down", "head")
    kinds = {}
    with torch.cuda.stream(stream):
        for kind in kind_list:
            model.truncate(PROMPT)
            kinds[kind] = model.time_kernel(kind, min(K, 100))
        dom = max(kinds, key=lambda k: kinds[k][0] * kinds[k][1])
        model.truncate(PROMPT)
        dom_us, dom_n = model.time_kernel(dom, K)
    model.synchronize()
    dom_bytes = (roofline.mean_step_bytes(cfg, PROMPT, K) if dom == "step"
                 else roofline.mean_kernel_bytes(cfg, dom, PROMPT, K))
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9

    step_bytes = roofline.mean_step_bytes(cfg, PROMPT, K)
    ms_step = ms / K
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    result = {
        "metric": ("Talker + code-predictor frames/sec at batch 16 + achieved HBM GB/s (% of peak) per frame" if frames
                   else "decode tokens/sec at batch 1 + achieved HBM GB/s (% of peak) per step"),
        "value": K / (ms * 1e-3),
        "unit": "frames/s" if frames else "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded random weights, prompt ids and values; no checkpoint)",
        "config": {"workload": desc.format(K=K, S="greedy" if samp is None or samp.get("mode", 0) == 0 else "sampled")
                   + ("" if args.cfg is None else f"; classifier-free guidance: a conditioned and an unconditioned row "
                                                  f"per step (batch 2), one token from cond + {args.cfg} (cond - uncond)"), "d_model": cfg["d_model"], "n_layer": cfg["n_layer"],
                   "n_head": cfg["n_head"], "d_ff": cfg["d_ff"], "vocab": cfg["vocab"],
                   "prompt": PROMPT, "global_batch": cfg["batch"], "launch_mode": mode, "workgroups": n_wg,
                   "sampler": args.sampler if samp is None else dict(samp, preset=args.sampler),
                   "cfg": args.cfg},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": roofline.HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / roofline.HBM_PEAK_GBS, "traffic": counted_traffic(dom, WORKLOAD),
                     "kernel": dom, "launch_us": dom_us, "launches_per_step": dom_n,
                     "bytes_per_launch": dom_bytes},
        "kernel_us": {k: round(v[0], 3) for k, v in kinds.items()},
        "step_gbs": gbs,
        "step_frac_of_hbm_peak": gbs / roofline.HBM_PEAK_GBS,
        "step_bytes": step_bytes,
        "wall_tokens_per_s": K / wall,
    }
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["calibration_copy_bytes"] = 2 * n * 4
    if frames:
        result["codes_per_s"] = result["value"] * cfg["batch"] * cfg["n_codebooks"]
    if not args.no_gemv:
        if frames:
            result["gemm_rows"] = gemm_rows_headline(args.seed)
        else:
            result["gemv"] = gemv_headline(args.seed, fmt=args.gemv_format)
    if not args.eager:
        result["prefill"] = {"positions": PROMPT, "rows": PROMPT * cfg["batch"], "ms": prefill_ms,
                             "positions_per_s": PROMPT / (prefill_ms * 1e-3),
                             "path": "prompt pass (matrix-core products over all prompt rows, causal flash "
                                     "attention), the last position through the decode step"
                                     + (" (the whole frame)" if frames else "")}
    result["device_state"] = dev_state.summary(t0, t1)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = (cpu_baseline_frames if frames else cpu_baseline)(with_sampler(cfg, samp), weights,
                                                                                    args.cpu_seconds, args.seed)
    model.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
