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

# workload name -> (prompt positions, default steps, description, dtype).  The dtype strings
# name every rounding the path makes beyond the weights' own format: the FC / SwiGLU output
# reaches the down projection rounded to a 15-bit mantissa in the persistent step's hand-over.
WORKLOADS = {
    "gpt2_medium_q4_0": (256, 500, "GPT-2-Medium-shaped 24-layer speech-token decoder, Q4_0, 256-token prefill then {K} "
                                   "{S} decode steps, batch 1",
                         "q4_0 weights, fp32 accumulate, fp16 kv; the FC output enters the down projection rounded "
                         "to a 15-bit mantissa"),
    "gpt2_medium_q5_0": (256, 500, "GPT-2-Medium-shaped 24-layer speech-token decoder, Q5_0, 256-token prefill then {K} "
                                   "{S} decode steps, batch 1",
                         "q5_0 weights, fp32 accumulate, fp16 kv; the FC output enters the down projection rounded "
                         "to a 15-bit mantissa"),
    "llama520m_q8_0": (300, 600, "Llama-shaped ~520M 30-layer speech-token decoder, Q8_0, 300-token prefill then {K} "
                                 "{S} decode steps, batch 1",
                       "q8_0 weights, fp32 accumulate, fp16 kv; the SwiGLU output enters the down projection rounded "
                       "to a 15-bit mantissa"),
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
    ap.add_argument("--no-gemv", action="store_true", help="skip the standalone GEMV measurements")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="skip the Llama-520M (c4) and Talker + code predictor (c5) objects of the default line")
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


def _code_only(text):
    """C++ source without its comments and with whitespace collapsed: an edit of comments or
    layout leaves the kernel, and so this text, unchanged."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def step_sources_hash(read=None):
    """Hash of the code the step kernel is compiled from (comments and layout ignored); read(path)
    returns a file's text (default: the working tree)."""
    import hashlib
    if read is None:
        def read(path):
            with open(os.path.join(ROOT, path)) as fh:
                return fh.read()
    h = hashlib.sha256()
    for f in STEP_SOURCES:
        h.update(_code_only(read(f)).encode())
    path, a, b = STEP_DECLS
    text = read(path)
    h.update(_code_only(text[text.index(a):text.index(b)]).encode())
    return h.hexdigest()[:16]
def counted_traffic(kernel, workload, bytes_per_launch):
    """HBM-side bytes per launch of the step kernel from the committed FETCH_SIZE / WRITE_SIZE
    summary of this workload (scaled by the copy calibration), carried over to this run's window
    of positions by the ratio counted / algorithmic bytes the summary measured; (None, reason)
    when there is no summary or it was taken on other kernel sources than the ones built now."""
    path = os.path.join(ROOT, "profiles", f"step_{workload}_counters.json")
    if kernel != "step" or not os.path.exists(path):
        return None, "no counter summary for this kernel and workload"
    with open(path) as fh:
        d = json.load(fh)
    if d.get("sources_sha256_16") != step_sources_hash() or "algorithmic_bytes_per_launch" not in d:
        return None, "the step kernel changed since its counters were taken"
    ratio = d["traffic_bytes_per_launch"] / d["algorithmic_bytes_per_launch"]
    return ratio * bytes_per_launch, (f"FETCH_SIZE + WRITE_SIZE (copy-calibrated) over {d['window']} read {ratio:.3f} x "
                                      f"that window's algorithmic bytes; that ratio times this run's bytes_per_launch")


def under_profiler():
    """True when a rocprofv3 tool library is loaded into this process."""
    return "rocprof" in os.environ.get("LD_PRELOAD", "") or any(k.startswith("ROCPROF") for k in os.environ)


class DeviceState:
    """amd-smi samples (socket power, graphics and memory clocks, temperatures) taken by a
    background thread while the benchmark runs; summary() reports those that fall inside the
    timed region (and the run's maximum power), or null fields where amd-smi is unavailable."""

    def __init__(self):
        import threading
        self.samples, self.stop = [], threading.Event()
        # under a profiler every child process gets its tool library, which initialises the GPU,
        # and amd-smi's launcher would then replace such a process: no sampling there
        self.skipped = under_profiler()
        if not self.skipped:
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
        if self.skipped:
            return {"skipped": "running under a profiler"}
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


C1_N, C1_K, C1_CHAIN = 1024, 1024, 512


def gemv_c1(seed, reps=200):
    """The lone GEMV workload (one 1024 x 1024 Q8_0 matrix, x ~ N(0,1), batch 1): 1.12 MB, which
    HBM streams in 0.14 us, so a single launch measures the launch, not the memory ("Every Frame Is
    a Memory Read", §4: a fixed cost per kernel, and matvec efficiency growing with size).  Two
    readings: the median duration of `reps` single launches, each bracketed by HIP events and
    synchronised (minus the median of as many empty brackets); and the slope, a graph of 512
    launches on 512 distinct matrices (574 MB, more than the Infinity Cache) replayed after a
    warm-up, time per launch."""
    import torch
    from quantized_gemv_kv_amd import binding, roofline, synth
    N, K = C1_N, C1_K
    rng = synth.rng_for(seed, 4)
    x = torch.from_numpy(synth.normal_f32(rng, (1, K))).cuda()
    y = torch.empty((1, N), dtype=torch.float32, device="cuda")
    pb = binding.tsd_gemv_packed_bytes("q8_0", N, K)
    row_b = K // 32 * 34
    packed = torch.empty((C1_CHAIN, pb), dtype=torch.uint8, device="cuda")
    canon = torch.empty(C1_CHAIN * N * row_b, dtype=torch.uint8, device="cuda")
    for r0, blob in synth.q8_0_row_chunks(C1_CHAIN * N, K, seed):
        canon[r0 * row_b: r0 * row_b + blob.size].copy_(torch.from_numpy(blob))
    for i in range(C1_CHAIN):
        binding.tsd_gemv_pack("q8_0", canon[i * N * row_b:(i + 1) * N * row_b], N, K, packed[i])
    del canon
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()

    def bracket(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        fn()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3

    warm(lambda: binding.tsd_gemv("q8_0", packed[0], N, K, 1, x, None, y))
    empty = float(np.median([bracket(lambda: None) for _ in range(reps)]))
    single = float(np.median([bracket(lambda: binding.tsd_gemv("q8_0", packed[0], N, K, 1, x, None, y))
                              for _ in range(reps)])) - empty
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cs):
        for i in range(C1_CHAIN):
            binding.tsd_gemv("q8_0", packed[i], N, K, 1, x, None, y, stream=cs)
    warm(g.replay)
    per = float(np.median([bracket(g.replay) for _ in range(7)])) / C1_CHAIN
    nbytes = roofline.gemv_bytes("q8_0", N, K)
    del packed, g
    return {"shape": f"Q8_0 {N}x{K}, batch 1", "bytes_per_gemv": nbytes,
            "single_launch_us": single, "single_launch_gbs": nbytes / (single * 1e-6) / 1e9,
            "chain_us_per_gemv": per, "chain_gbs": nbytes / (per * 1e-6) / 1e9,
            "chain_frac": nbytes / (per * 1e-6) / 1e9 / roofline.HBM_PEAK_GBS,
            "timing": f"single: median of {reps} synchronised launches under HIP events, minus the median empty "
                      f"bracket ({empty:.1f} us); chain: one graph of {C1_CHAIN} launches on {C1_CHAIN} distinct "
                      f"matrices, median of 7 replays after 0.25 s of warm-up replays, per launch"}


def host_cpu():
    """(CPU model name, logical CPUs of the host, CPUs this process may run on)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count(), len(os.sched_getaffinity(0))


class pinned_thread:
    """Pins the calling thread (Linux: pid 0 is the calling thread) to one CPU it may run on,
    restoring its affinity afterwards; the oracle runs on this thread through ctypes."""

    def __enter__(self):
        self.saved = os.sched_getaffinity(0)
        self.cpu = max(self.saved)
        os.sched_setaffinity(0, {self.cpu})
        return self

    def __exit__(self, *exc):
        os.sched_setaffinity(0, self.saved)


def describe_host(pin):
    model, n, _ = host_cpu()
    return {"cpu_model": model, "nproc": n, "cpus_allowed": len(pin.saved), "pinned_to_cpu": pin.cpu, "threads": 1}


def cpu_baseline(cfg, weights, seconds, seed):
    """The CPU oracle as it stands (single-threaded C, fp64), timed on this host with its thread
    pinned to one CPU: decode steps from position 256 over a random 256-position fp16 cache, until
    the time budget is spent."""
    import oracle
    with pinned_thread() as pin:
        r = _cpu_baseline(oracle, cfg, weights, seconds, seed)
        r["host"] = describe_host(pin)
    return r


def _cpu_baseline(oracle, cfg, weights, seconds, seed):
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
    costs 16 row-frames): frames at positions 170.. over a random 170-position Talker cache, the
    thread pinned to one CPU."""
    import oracle
    with pinned_thread() as pin:
        r = _cpu_baseline_frames(oracle, cfg, weights, seconds, seed)
        r["host"] = describe_host(pin)
    return r


def _cpu_baseline_frames(oracle, cfg, weights, seconds, seed):
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


def measure(workload, K, W, seed, launch_mode="persistent", samp=None, cfg_weight=None, eager=False, time_kinds=True):
    """One workload: the model at its real shape on seeded synthetic weights, its prompt (once
    untimed, then from a reset model under HIP events), W warm-up steps, the context truncated back
    to the prompt, then K timed steps (graph replays) bracketed by stream synchronisation and HIP
    events on the model's stream.  With time_kinds, every kernel kind is then timed inside real
    steps and the dominant one re-timed over the same K positions."""
    import torch
    from quantized_gemv_kv_amd import Model, TsdError, roofline, synth
    UNSUPPORTED = 2
    prompt_n, _, desc, dtype = WORKLOADS[workload]
    cfg = dict(synth.config(workload), launch_mode=launch_mode)
    frames = cfg["arch"] == "talker_cp"
    if cfg_weight is not None:
        cfg["batch"] = 2
    if prompt_n + max(K, W) > cfg["n_ctx"]:
        raise SystemExit(f"steps/warmup exceed the {cfg['n_ctx']}-position context")
    weights = synth.model_weights(cfg, seed)
    stream = torch.cuda.Stream()
    model = Model(cfg, weights, stream=stream, sampling=samp)
    prompt = torch.from_numpy(synth.prompt_tokens(cfg, prompt_n, seed=seed)).to("cuda")
    step = model.step_eager if eager else model.step
    prefill_ms = None
    with torch.cuda.stream(stream):
        if eager:
            k, v = synth.kv_cache(cfg, prompt_n, seed=seed)
            model.load_kv(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), prompt_n)
        else:
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
        model.truncate(prompt_n)
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
    ms = e0.elapsed_time(e1)
    model.synchronize()
    ids = model.tokens(prompt_n, K).cpu().numpy()
    if frames:
        assert ids[..., 1:].max() < cfg["cp_vocab"], "sampled codes out of range"
    ids = ids.reshape(-1)
    assert ids.min() >= 0 and ids.max() < cfg["vocab"], "sampled ids out of range"
    mode, n_wg = model.info()
    out = {"cfg": cfg, "weights": weights, "desc": desc, "prompt": prompt_n, "ms": ms, "wall_s": t1 - t0, "t0": t0, "t1": t1,
           "mode": mode, "n_wg": n_wg, "prefill_ms": prefill_ms,
           "dtype": dtype if mode == "persistent" or frames else dtype.split(";")[0]}
    step_bytes = roofline.mean_step_bytes(cfg, prompt_n, K)
    out["step_bytes"] = step_bytes
    if time_kinds:
        kind_list = ("step",) if mode == "persistent" else ("qkv", "attn", "oproj", "fc", "down", "head")
        kinds = {}
        with torch.cuda.stream(stream):
            for kind in kind_list:
                model.truncate(prompt_n)
                try:
                    kinds[kind] = model.time_kernel(kind, min(K, 100))
                except TsdError as e:   # a kind this step does not launch (the frame's fused attention)
                    if e.status != UNSUPPORTED:
                        raise
            dom = max(kinds, key=lambda k: kinds[k][0] * kinds[k][1])
            model.truncate(prompt_n)
            dom_us, dom_n = model.time_kernel(dom, K)
        model.synchronize()
        dom_kind = "qkv_attn" if frames and dom == "qkv" and "attn" not in kinds else dom
        dom_bytes = step_bytes if dom == "step" else roofline.mean_kernel_bytes(cfg, dom_kind, prompt_n, K)
        out.update(kinds=kinds, dom=dom, dom_us=dom_us, dom_n=dom_n, dom_bytes=dom_bytes)
    model.close()
    return out


def summary_of(m, K, workload):
    """The compact object the default line carries for a second workload."""
    from quantized_gemv_kv_amd import roofline
    ms_step = m["ms"] / K
    gbs = m["step_bytes"] / (ms_step * 1e-3) / 1e9
    frames = m["cfg"]["arch"] == "talker_cp"
    r = {"workload": m["desc"].format(K=K, S="greedy"), "steps": K, "ms_per_step": ms_step,
         "value": K / (m["ms"] * 1e-3), "unit": "frames/s" if frames else "tokens/s",
         "step_bytes": m["step_bytes"], "step_gbs": gbs, "step_frac_of_hbm_peak": gbs / roofline.HBM_PEAK_GBS,
         "launch_mode": m["mode"], "dtype": m["dtype"], "prefill_ms": m["prefill_ms"]}
    if "dom" in m:
        r["kernel"] = m["dom"]
        r["kernel_us"] = m["dom_us"]
        r["kernel_frac_of_hbm_peak"] = m["dom_bytes"] / (m["dom_us"] * 1e-6) / 1e9 / roofline.HBM_PEAK_GBS
        r["kernel_traffic"], r["kernel_traffic_note"] = counted_traffic(m["dom"], workload, m["dom_bytes"])
    if frames:
        r["codes_per_s"] = r["value"] * m["cfg"]["batch"] * m["cfg"]["n_codebooks"]
    return r


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library runs the decode step "
              f"on a single GPU and does not shard it.", file=sys.stderr)
        sys.exit(2)
    import torch
    from quantized_gemv_kv_amd import roofline

    global WORKLOAD, PROMPT
    WORKLOAD = args.workload
    PROMPT, default_steps, _, _ = WORKLOADS[WORKLOAD]
    if args.steps is None:
        args.steps = default_steps
    K, W = args.steps, args.warmup
    frames = WORKLOAD == "talker_cp_aff8"
    if args.cfg is not None and frames:
        print("--cfg applies to the GPT2/LLAMA workloads", file=sys.stderr)
        sys.exit(2)
    samp = SAMPLERS[args.sampler]
    if samp is not None:
        samp = dict(samp, seed=args.seed)
    if args.cfg is not None:
        samp = dict(samp or {"mode": 0, "seed": args.seed}, cfg=1, cfg_weight=args.cfg)
    dev_state = DeviceState()
    m = measure(WORKLOAD, K, W, args.seed, args.launch_mode, samp, args.cfg, args.eager)
    cfg, weights = m["cfg"], m.pop("weights")
    ms = m["ms"]
    dom, dom_us, dom_n, dom_bytes = m["dom"], m["dom_us"], m["dom_n"], m["dom_bytes"]
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    traffic, traffic_note = counted_traffic(dom, WORKLOAD, dom_bytes)
    step_bytes = m["step_bytes"]
    ms_step = ms / K
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": achieved, "peak": roofline.HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / roofline.HBM_PEAK_GBS, "traffic": traffic, "traffic_note": traffic_note,
            "kernel": dom, "launch_us": dom_us, "launches_per_step": dom_n, "bytes_per_launch": dom_bytes}
    if WORKLOAD.startswith("gpt2_medium"):
        roof["cache_note"] = ("the 176 MB of fixed weights fit MI355X's 256 MB Infinity Cache, so part of this 'HBM' "
                              "stream may be served from that memory-side cache")
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
        "dtype": m["dtype"],
        "data": "synthetic (seeded random weights, prompt ids and values; no checkpoint)",
        "config": {"workload": m["desc"].format(K=K, S="greedy" if samp is None or samp.get("mode", 0) == 0 else "sampled")
                   + ("" if args.cfg is None else f"; classifier-free guidance: a conditioned and an unconditioned row "
                                                  f"per step (batch 2), one token from cond + {args.cfg} (cond - uncond)"), "d_model": cfg["d_model"], "n_layer": cfg["n_layer"],
                   "n_head": cfg["n_head"], "d_ff": cfg["d_ff"], "vocab": cfg["vocab"],
                   "prompt": PROMPT, "global_batch": cfg["batch"], "launch_mode": m["mode"], "workgroups": m["n_wg"],
                   "sampler": args.sampler if samp is None else dict(samp, preset=args.sampler),
                   "cfg": args.cfg},
        "roofline": roof,
        "kernel_us": {k: round(v[0], 3) for k, v in m["kinds"].items()},
        "step_gbs": gbs,
        "step_frac_of_hbm_peak": gbs / roofline.HBM_PEAK_GBS,
        "step_bytes": step_bytes,
        "wall_tokens_per_s": K / m["wall_s"],
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
            result["gemv_1024"] = gemv_c1(args.seed)
    if not args.eager:
        result["prefill"] = {"positions": PROMPT, "rows": PROMPT * cfg["batch"], "ms": m["prefill_ms"],
                             "positions_per_s": PROMPT / (m["prefill_ms"] * 1e-3),
                             "path": "prompt pass (matrix-core products over all prompt rows, causal flash "
                                     "attention), the last position through the decode step"
                                     + (" (the whole frame)" if frames else "")}
    # the other two decoders the pages time, at their real shapes, in the same run (greedy)
    if WORKLOAD == "gpt2_medium_q4_0" and not args.no_extra_configs and not args.eager and args.cfg is None \
            and samp is None:
        c4 = measure("llama520m_q8_0", min(K, 100), min(W, 20), args.seed)
        c4.pop("weights")
        result["c4"] = summary_of(c4, min(K, 100), "llama520m_q8_0")
        c5 = measure("talker_cp_aff8", min(K, 50), min(W, 5), args.seed, time_kinds=False)
        c5.pop("weights")
        result["c5"] = summary_of(c5, min(K, 50), "talker_cp_aff8")
    result["device_state"] = dev_state.summary(m["t0"], m["t1"])
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = (cpu_baseline_frames if frames else cpu_baseline)(with_sampler(cfg, samp), weights,
                                                                                    args.cpu_seconds, args.seed)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
