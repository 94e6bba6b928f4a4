"""Decode-step throughput of libqd on one MI355X.

A step is one batched decode step of a Qwen3-style GQA decoder (embedding,
36 x [RMSNorm + QKV, q/k-norm + RoPE + paged KV append + split-KV attention,
O + residual, RMSNorm + gate/up + SwiGLU, down + residual], final RMSNorm, LM
head, on-device argmax) over synthetic seeded weights and paged K/V, run
as the library runs it on a handle sized for the workload (qd_step_path: the
batch-1 weight-streaming kernel, or the per-stage kernels replayed from one
captured hipGraph).  Steps are chained on the device: each step's next-token
ids are the following step's input (two ping-pong id buffers, so the graphs
never change), and the positions advance on the device.

Headline line: Qwen3-4B shape, batch 1, context 512 (value = tokens/s, the
median over --reps repetitions of K timed steps).  The same JSON line also
carries batch 8 / 16 at context 256, batch 1 at 8192 and the Qwen3-8B ragged
batch 8 under "workloads", the live roofline of the dominant kernel, the
measured streaming-read ceiling of the device and the CPU oracle timed on a
bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--reps R]
                       [--workloads a,b] [--no-cpu-baseline] [--no-prefill]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

REPO = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, REPO)

from paged_kv_gqa_qwen3_amd import accounting, binding, synth  # noqa: E402

METRIC = "decode tokens/s + achieved HBM GB/s (% of 8 TB/s), Qwen3-4B shape, bs 1/8/16"
HBM_PEAK_GBPS = 8000.0
HEADLINE = "4b_bs1_ctx512"
DEFAULT_WORKLOADS = ["4b_bs1_ctx512", "4b_bs8_ctx256", "4b_bs16_ctx256", "4b_bs1_ctx8192",
                     "8b_bs8_ragged", "4b_bs8_ctx4096", "4b_bs8_ctx4096_fp8kv", "4b_bs32_ctx256",
                     "4b_bs64_ctx256"]
WEIGHT_SEED = {"qwen3-4b": 2, "qwen3-8b": 6}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


KERNEL_SOURCES = {
    "per_stage": ("qd_device.h", "qd_kernels.hip"),
    "stream_step": ("qd_device.h", "qd_stream_plan.h", "qd_stream.h", "qd_stream.hip"),
}


def kernel_source_sha256(kind="per_stage"):
    """sha256 over the device-code sources of the per-stage kernels, or of the
    batch-1 streaming kernel, in order."""
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        h.update(open(os.path.join(REPO, "paged_kv_gqa_qwen3_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def measured_traffic(kernel_class, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source (else None)."""
    kind = "stream_step" if kernel_class == "stream_step" else "per_stage"
    path = os.path.join(REPO, "profiles", f"traffic_{workload}_{kind}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256") != kernel_source_sha256(kind):
        return None
    return rec.get("traffic_bytes_per_launch", {}).get(kernel_class)


def gemv_bytes(shape, cls):
    """Algorithmic bytes one launch of a projection class reads (bf16 weights)."""
    H, I = shape.hidden, shape.intermediate
    return {
        "qkv": (shape.q_dim + 2 * shape.kv_dim) * H * 2,
        "o_proj": H * shape.q_dim * 2,
        "gate_up": 2 * I * H * 2,
        "down": H * I * 2,
        "lm_head": shape.vocab * H * 2,
    }[cls]


def attention_bytes(shape, ctx, kv_elem_bytes=2):
    """K/V bytes one attention launch (one layer) reads and appends."""
    per_tok_layer = 2 * shape.num_kv_heads * shape.head_dim * kv_elem_bytes
    return sum(int(c) for c in ctx) * per_tok_layer


class Run:
    """One workload on one handle: pool, tables and chained device buffers."""

    def __init__(self, torch, dec, w, batch):
        self.torch, self.dec, self.w, self.batch = torch, dec, w, batch
        B = w.batch
        dev = "cuda"
        pool = np.ascontiguousarray(batch.pool)  # bf16 bits, or E4M3 codes (uint8)
        self.pool = torch.from_numpy(pool if pool.dtype == np.uint8 else pool.view(np.int16)).to(dev)
        self.tab = torch.from_numpy(batch.block_tables).to(dev)
        self.pos0 = torch.from_numpy(batch.positions).to(dev)
        self.pos = self.pos0.clone()
        self.ids = [torch.from_numpy(batch.tokens).to(dev),
                    torch.zeros(B, dtype=torch.int32, device=dev)]
        self.k = 0

    def step(self):
        a, b = self.ids[self.k & 1], self.ids[(self.k + 1) & 1]
        self.dec.step(a, self.pos, self.tab, self.pool, b, None)
        self.pos.add_(1)
        self.k += 1

    def reset(self):
        self.pos.copy_(self.pos0)


def time_workload(torch, dec, w, batch, steps, warmup, reps):
    """`reps` repetitions of `steps` chained steps from the same start
    positions, each bracketed by HIP events on the library's stream (torch's
    current stream here); returns the run, every repetition's milliseconds,
    the wall time of all of them and the algorithmic bytes of one
    repetition."""
    run = Run(torch, dec, w, batch)
    for _ in range(warmup):
        run.step()
    torch.cuda.synchronize()
    times = []
    t0 = time.perf_counter()
    for _ in range(reps):
        run.reset()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps):
            run.step()
        end.record()
        torch.cuda.synchronize()
        times.append(start.elapsed_time(end))
    wall = time.perf_counter() - t0
    flags = dec.device_status()
    if flags:
        raise RuntimeError(f"device input flags {flags} during {w.name}")
    ctx0 = batch.positions.astype(np.int64) + 1
    kvb = 1 if w.kv_fp8 else 2
    total_bytes = sum(accounting.step_bytes(w.shape, ctx0 + s, kvb) for s in range(steps))
    return run, times, wall, total_bytes


def profile_classes(torch, dec, run, reps=5):
    """Per-kernel-class times from HIP events recorded on the library's stream."""
    acc = {c: [0.0, 0] for c in binding.PROF_CLASSES}
    B = run.w.batch
    for _ in range(reps):
        run.reset()
        a, b = run.ids[0], run.ids[1]
        res = binding.qd_profile_step(dec.handle, B, a, run.pos, run.tab, run.pool, b, None)
        for c, (ms, n) in res.items():
            acc[c][0] += ms
            acc[c][1] += n
    return {c: (v[0], v[1]) for c, v in acc.items()}


def cpu_baseline(w, W, batch, budget_s=20.0):
    """The oracle, as it stands, timed on this host on a bounded sample of the
    same workload: consecutive decode steps of the same batch until about
    budget_s seconds have passed (at least one)."""
    import oracle

    orc = oracle.Oracle(w.shape, W)
    pool = batch.pool.copy()
    tokens, positions = batch.tokens.copy(), batch.positions.copy()
    steps = 0
    t0 = time.perf_counter()
    while True:
        _, nxt, _ = orc.decode_step(tokens, positions, batch.block_tables, pool,
                                    want_logits=False)
        steps += 1
        tokens, positions = nxt.astype(np.int32), positions + 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    ncpu = len(os.sched_getaffinity(0))
    cores = min(threads, ncpu) if threads > 0 else ncpu
    return {"value": round(steps * w.batch / dt, 4), "unit": "tokens/s", "cores": cores,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{steps} decode step(s) of {w.name} (batch {w.batch}, context "
                      f"{int(batch.positions[0])}+), {dt:.1f} s, fp64 C oracle with OpenMP"}


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def read_ceiling(torch, gib=2, reps=10):
    """The device's plain streaming-read rate (qd_read_ceiling: 16-byte
    nontemporal loads over a gib GiB buffer, the weight-streaming pattern),
    GB/s: the practical ceiling next to the nominal 8 TB/s."""
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    torch.cuda.synchronize()
    gbps = binding.qd_read_ceiling(buf, buf.numel(), reps,
                                   torch.cuda.current_stream().cuda_stream)
    del buf
    torch.cuda.empty_cache()
    return round(gbps, 1)


def stream_roofline(w, ms, steps, nbytes):
    """The batch-1 step is one kernel launch: its algorithmic bytes (weights
    plus the K/V read and appended) per launch over its mean duration, timed
    with HIP events on the library's stream over the timed steps."""
    avg_us = ms / steps * 1e3
    per_launch = nbytes / steps
    gbps = per_launch / (avg_us * 1e-6) / 1e9
    return {
        "roofline": {"bound": "hbm", "kernel": "stream_step", "achieved": round(gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic("stream_step", w.name),
                     "algorithmic_bytes": int(per_launch), "avg_us": round(avg_us, 3)},
    }


def per_stage_roofline(torch, dec, run, shape, w, batch):
    """Per-stage path: every class's time (projections replayed alone as a
    graph between two events on the library's stream: avg_us; every class,
    attention included, from the step run with an event between kernels:
    events_us, which adds a few us per kernel); the roofline is that of the
    class with the largest share of the step."""
    prof = profile_classes(torch, dec, run)
    ctx_mid = batch.positions.astype(np.int64) + 1
    per_class = {}
    for c, (tot_ms, n) in prof.items():
        if n == 0:
            continue
        ev_us = tot_ms / n * 1e3
        if c in ("qkv", "o_proj", "gate_up", "down", "lm_head"):
            byts = gemv_bytes(shape, c)
            avg_us = binding.qd_profile_class(dec.handle, w.batch, c, reps=20)
        elif c == "attention":
            byts = attention_bytes(shape, ctx_mid, 1 if w.kv_fp8 else 2)
            avg_us = ev_us
        else:
            byts = w.batch * shape.hidden * 2
            avg_us = ev_us
        per_class[c] = {"launches_per_step": n // 5, "avg_us": round(avg_us, 3),
                        "events_us": round(ev_us, 3),
                        "bytes_per_launch": int(byts),
                        "GBps": round(byts / (avg_us * 1e-6) / 1e9, 1),
                        "ms_per_step": round(avg_us * (n // 5) / 1e3, 4)}
    dom = max(per_class, key=lambda c: per_class[c]["ms_per_step"])
    d = per_class[dom]
    return {
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": d["GBps"],
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(d["GBps"] / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(dom, w.name),
                     "algorithmic_bytes": d["bytes_per_launch"],
                     "avg_us": d["avg_us"]},
        "kernel_classes": per_class,
    }


SAMPLING_SETTINGS = (("greedy", 0.0, 0, 1.0), ("T0.6_top_k20_top_p0.95", 0.6, 20, 0.95),
                     ("T1_no_limit", 1.0, 0, 1.0), ("T0.3_top_p0.9", 0.3, 0, 0.9))


def time_sampling(torch, dec, B, V, reps=50):
    """Microseconds per qd_sample call on seeded N(0, 2) logits [B][V] for a few
    settings (HIP events on the library's stream, which is torch's current
    stream here)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    lg = torch.randn(B, V, device="cuda", generator=g) * 2.0
    u = torch.rand(B, device="cuda", generator=g)
    out = torch.zeros(B, dtype=torch.int32, device="cuda")
    res = {}
    for name, T, k, p in SAMPLING_SETTINGS:
        t_ = torch.full((B,), T, device="cuda")
        k_ = torch.full((B,), k, dtype=torch.int32, device="cuda")
        p_ = torch.full((B,), p, device="cuda")
        for _ in range(3):
            dec.sample(lg, t_, k_, p_, u, out)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(reps):
            dec.sample(lg, t_, k_, p_, u, out)
        e.record()
        torch.cuda.synchronize()
        res[name] = round(s.elapsed_time(e) / reps * 1e3, 1)
    return res


def time_prefill(torch, shape, W, n_tokens=512, chunk=32, reps=3):
    """Milliseconds to prefill one n_tokens prompt from an empty pool through
    qd_prefill: chunks of `chunk` rows in position order, logits for the last
    row only (HIP events on the library's stream, torch's current stream).
    Every chunk streams the weights once."""
    from paged_kv_gqa_qwen3_amd.decoder import Decoder
    pages = -(-n_tokens // 16)
    dec = Decoder(shape, chunk, pages, pages, use_graphs=False)
    dec.load_numpy_weights(W)
    pool = torch.zeros(shape.num_layers, pages, 2, shape.num_kv_heads, 16, shape.head_dim,
                       dtype=torch.int16, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    prompt = torch.randint(0, shape.vocab, (n_tokens,), dtype=torch.int32, device="cuda",
                           generator=g)
    table = torch.arange(pages, dtype=torch.int32, device="cuda")
    calls = []
    for c0 in range(0, n_tokens, chunk):
        pos = torch.arange(c0, min(c0 + chunk, n_tokens), dtype=torch.int32, device="cuda")
        last = c0 + chunk >= n_tokens
        if last:  # the prompt's last token first: it gets the logits
            pos = torch.cat([pos[-1:], pos[:-1]])
        calls.append((prompt[pos.long()].contiguous(), pos,
                      table[None].expand(len(pos), pages).contiguous(), 1 if last else 0))
    nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
    lg = torch.zeros(1, shape.vocab, dtype=torch.float32, device="cuda")

    def run():
        for tok, pos, tab, n in calls:
            dec.prefill(tok, pos, tab, pool, n, nxt if n else None, lg if n else None)
    run()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        run()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    assert dec.device_status() == 0
    dec.close()
    del pool
    torch.cuda.empty_cache()
    return {"prompt_tokens": n_tokens, "chunk_rows": chunk, "chunks": len(calls),
            "ms": round(ms, 3), "tokens_per_s": round(n_tokens / (ms / 1e3), 1)}


def time_prefill_prompts(torch, shape, W, n_tokens=512, reps=5):
    """Milliseconds to prefill one n_tokens prompt from an empty pool through
    qd_prefill_prompts: one chunk, projections as GEMMs on the matrix cores,
    tiled causal attention, logits for the last row (HIP events on the
    library's stream, torch's current stream; median of `reps`).  Also the
    projections' algorithmic FLOP rate over the whole prefill time."""
    from paged_kv_gqa_qwen3_amd.decoder import Decoder
    pages = -(-n_tokens // 16)
    dec = Decoder(shape, 1, pages, pages, use_graphs=False, max_prefill_rows=n_tokens)
    dec.load_numpy_weights(W)
    pool = torch.zeros(shape.num_layers, pages, 2, shape.num_kv_heads, 16, shape.head_dim,
                       dtype=torch.int16, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    prompt = torch.randint(0, shape.vocab, (n_tokens,), dtype=torch.int32, device="cuda",
                           generator=g)
    table = torch.arange(pages, dtype=torch.int32, device="cuda")[None].contiguous()
    nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
    lg = torch.zeros(1, shape.vocab, dtype=torch.float32, device="cuda")

    def run():
        dec.prefill_prompts([n_tokens], [0], prompt, table, pool, 1, nxt, lg)
    run()
    times = []
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        run()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    ms = float(np.median(times))
    assert dec.device_status() == 0
    dec.close()
    del pool
    torch.cuda.empty_cache()
    H, I, QD, KD = shape.hidden, shape.intermediate, shape.q_dim, shape.kv_dim
    proj_flop = 2.0 * n_tokens * shape.num_layers * H * (QD + 2 * KD + QD + 3 * I)
    return {"prompt_tokens": n_tokens, "chunk_rows": n_tokens, "chunks": 1,
            "ms": round(ms, 3), "ms_min_max": [round(min(times), 3), round(max(times), 3)],
            "tokens_per_s": round(n_tokens / (ms / 1e3), 1),
            "projection_tflops": round(proj_flop / (ms / 1e3) / 1e12, 1)}


def time_serving(torch, shape, W, n_req=64, max_batch=64, max_new=128, rows=512, seed=17):
    """Offline serving through the continuous-batching engine (qd_engine_*):
    n_req requests queued at once, prompts of 128..1024 tokens (uniform),
    every second one starting with the same 256-token system prompt (or
    its first tokens, for a shorter prompt),
    max_new greedy tokens each, at most max_batch decoding together and
    `rows` prompt rows per iteration.  Graphs for every batch size are
    captured by a warm-up set of requests first.  Reports wall-clock rates
    over the whole queue, the median iteration time while the batch is full
    and no prompt is being prefilled, the GPU time the engine measured (HIP
    events from each iteration's first launch to its last kernel) and the
    rest of the wall time per iteration: the engine's host work."""
    from paged_kv_gqa_qwen3_amd.decoder import Decoder
    V = shape.vocab
    rng = np.random.Generator(np.random.PCG64(seed))
    system = rng.integers(0, V, 256, dtype=np.int32)
    prompts = []
    for i in range(n_req):
        p = rng.integers(0, V, int(rng.integers(128, 1025)), dtype=np.int32)
        if i % 2 == 0:
            p[:min(256, len(p))] = system[:len(p)]
        prompts.append(p)
    mpps = -(-(1024 + max_new) // 16)
    num_pages = max_batch * mpps + 256
    dec = Decoder(shape, max_batch, mpps, num_pages, use_graphs=True, persistent=True,
                  max_prefill_rows=rows)
    dec.load_numpy_weights(W)
    pool = torch.zeros(shape.num_layers, num_pages, 2, shape.num_kv_heads, 16, shape.head_dim,
                       dtype=torch.int16, device="cuda")
    eng = binding.Engine(dec.handle, pool, max_batch)

    def drain():
        per = []
        prev = eng.stats()
        while True:
            t = time.perf_counter()
            eng.step()
            dt = time.perf_counter() - t
            st = eng.stats()
            per.append((dt, st["decode_rows"] - prev["decode_rows"],
                        st["prefill_rows"] - prev["prefill_rows"]))
            prev = st
            if st["waiting"] == 0 and st["running"] == 0:
                return per, st

    # warm-up: requests that leave one by one, so every batch size 1..max_batch
    # captures its graph before the timed queue
    for i in range(max_batch):
        eng.submit(1_000_000 + i, rng.integers(0, V, 16, dtype=np.int32), 2 + i)
    _, st0 = drain()
    for i, p in enumerate(prompts):
        eng.submit(i, p, max_new)
    t0 = time.perf_counter()
    per, st = drain()
    wall = time.perf_counter() - t0
    assert dec.device_status() == 0
    eng.close()
    dec.close()
    del pool
    torch.cuda.empty_cache()
    gen = st["tokens_out"] - st0["tokens_out"]
    n_prompt = int(sum(len(p) for p in prompts))
    full = [dt for dt, b, r in per if b == max_batch and r == 0]
    gpu_s = (st["gpu_us"] - st0["gpu_us"]) / 1e6
    return {"requests": n_req, "prompt_tokens": n_prompt, "generated_tokens": int(gen),
            "max_batch": max_batch, "prefill_rows_per_iteration": rows,
            "max_new_tokens": max_new, "iterations": len(per), "wall_s": round(wall, 3),
            "output_tokens_per_s": round(gen / wall, 1),
            "total_tokens_per_s": round((gen + n_prompt) / wall, 1),
            "prompt_tokens_from_prefix_cache": int(st["cached_rows"] - st0["cached_rows"]),
            "mean_decode_batch": round(float(np.mean([b for _, b, _ in per])), 2),
            "full_batch_iteration_ms_median": round(1e3 * float(np.median(full)), 4) if full else None,
            "full_batch_iterations": len(full),
            "gpu_s": round(gpu_s, 3),
            "host_us_per_iteration": round(1e6 * (wall - gpu_s) / len(per), 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--reps", type=int, default=5,
                    help="timed repetitions of --steps steps per workload (median reported)")
    ap.add_argument("--workloads", default=",".join(DEFAULT_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip timing qd_prefill on a 512-token prompt (profiling runs)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time qd_prefill_prompts on a 512-token prompt of the headline "
                         "model only, print its record and stop (profiling runs)")
    ap.add_argument("--no-serve", action="store_true",
                    help="skip the serving-loop record (qd_engine over 64 queued requests)")
    ap.add_argument("--serve-only", action="store_true",
                    help="only the serving-loop record")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--mode", choices=("auto", "graph"), default="auto",
                    help="auto: a persistent handle, on which the library runs batch 1 as "
                         "the streaming kernel where the handle allows it and every other step "
                         "as the per-stage graph (qd_step_path); graph: the per-stage graph "
                         "only")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (a known-size "
                         "kernel for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested); the decode step "
              "has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.load_library()
    ceiling = read_ceiling(torch)
    log(f"[bench] streaming-read ceiling {ceiling} GB/s")
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.copy_calibration_mib} MiB done")
        del src, dst
    if args.prefill_only:
        shape = synth.WORKLOADS[HEADLINE].shape
        W = synth.make_weights(shape, WEIGHT_SEED[shape.name])
        rec = time_prefill_prompts(torch, shape, W, reps=args.reps)
        log(f"[bench] qd_prefill_prompts of 512 prompt tokens {rec}")
        print(json.dumps({"prefill": rec, "model": shape.name}))
        torch.cuda.synchronize()
        return
    if args.serve_only:
        shape = synth.WORKLOADS[HEADLINE].shape
        W = synth.make_weights(shape, WEIGHT_SEED[shape.name])
        rec = time_serving(torch, shape, W)
        log(f"[bench] serving loop {rec}")
        print(json.dumps({"serve": rec, "model": shape.name}))
        torch.cuda.synchronize()
        return
    names = [n for n in args.workloads.split(",") if n]
    if HEADLINE not in names:
        names.insert(0, HEADLINE)
    wl = [synth.WORKLOADS[n] for n in names]
    results = {}
    headline_extra = {}
    by_shape = {}
    for w in wl:
        by_shape.setdefault(w.shape.name, []).append(w)

    for shape_name, group in by_shape.items():
        shape = group[0].shape
        log(f"[bench] generating {shape_name} weights")
        t0 = time.perf_counter()
        W = synth.make_weights(shape, WEIGHT_SEED[shape_name])
        log(f"[bench] weights ready in {time.perf_counter() - t0:.1f}s")
        from paged_kv_gqa_qwen3_amd.decoder import Decoder

        for w in group:
            # one handle per workload, sized for the positions its timed and
            # warmup steps reach
            span = max(w.steps, args.steps + args.warmup)
            batch = synth.make_paged_batch(shape, synth.context_lengths(w), span, w.seed,
                                           kv_fp8=w.kv_fp8)
            dec = Decoder(shape, w.batch, batch.max_pages, batch.num_pages, use_graphs=True,
                          persistent=(args.mode == "auto"), kv_fp8=w.kv_fp8)
            dec.load_numpy_weights(W)
            path = dec.step_path(w.batch)
            log(f"[bench] {w.name}: {path} path, timing {args.steps} steps after "
                f"{args.warmup} warmup")
            run, times, wall, nbytes = time_workload(torch, dec, w, batch, args.steps,
                                                     args.warmup, args.reps)
            ms = float(np.median(times))
            tok_s = args.steps * w.batch / (ms / 1e3)
            gbps = nbytes / (ms / 1e3) / 1e9
            results[w.name] = {
                "workload": w.name, "batch": w.batch, "path": path,
                "context0": [int(c) for c in batch.positions[:4]] + (["..."] if w.batch > 4 else []),
                "tokens_per_s": round(tok_s, 2), "ms_per_step": round(ms / args.steps, 4),
                "ms_per_step_min_max": [round(min(times) / args.steps, 4),
                                        round(max(times) / args.steps, 4)],
                "reps": args.reps,
                "achieved_GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
                "ceiling_frac": round(gbps / ceiling, 4) if ceiling else None,
                "wall_s": round(wall, 4),
            }
            log(f"[bench] {w.name}: {tok_s:.1f} tok/s, {ms / args.steps:.4f} ms/step, "
                f"{gbps:.0f} GB/s ({100 * gbps / HBM_PEAK_GBPS:.1f}% of 8 TB/s)")
            # on-device sampling of the next token (not part of the step)
            results[w.name]["sampling_us_per_call"] = time_sampling(torch, dec, w.batch, shape.vocab)
            log(f"[bench] {w.name}: qd_sample us per call {results[w.name]['sampling_us_per_call']}")
            if w.name == HEADLINE:
                if path == "stream":
                    headline_extra = stream_roofline(w, ms, args.steps, nbytes)
                else:
                    headline_extra = per_stage_roofline(torch, dec, run, shape, w, batch)
                # prompt processing (qd_prefill) of a 512-token prompt, the
                # headline's context, on a handle of its own
                if not args.no_prefill:
                    results[w.name]["prefill"] = time_prefill_prompts(torch, shape, W)
                    log(f"[bench] {w.name}: qd_prefill_prompts of 512 prompt tokens "
                        f"{results[w.name]['prefill']}")
                    results[w.name]["prefill_decode_kernels"] = time_prefill(torch, shape, W)
                    log(f"[bench] {w.name}: qd_prefill (32-row chunks on the decode "
                        f"kernels) of 512 prompt tokens "
                        f"{results[w.name]['prefill_decode_kernels']}")
                if not args.no_serve:
                    results[w.name]["serve"] = time_serving(torch, shape, W)
                    log(f"[bench] {w.name}: serving loop {results[w.name]['serve']}")
                if not args.no_cpu_baseline:
                    log("[bench] timing the CPU oracle on a bounded sample")
                    headline_extra["cpu_baseline"] = cpu_baseline(w, W, batch, args.cpu_budget)
            del run
            dec.close()
            torch.cuda.empty_cache()
        del W

    h = results[HEADLINE]
    out = {
        "metric": METRIC, "value": h["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": h["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) bf16 weights, N(0,1) bf16 paged K/V)",
        "config": {"workload": "Qwen3-4B-shaped decode, batch 1, context 512, 16-token pages, "
                               "shuffled block table", "name": HEADLINE, "batch": 1,
                   "context0": 512, "parallelism": "single GPU", "mode": args.mode,
                   "path": h["path"]},
        "achieved_GBps": h["achieved_GBps"], "hbm_frac": h["hbm_frac"],
        "reps": args.reps, "ms_per_step_min_max": h["ms_per_step_min_max"],
    }
    out.update(headline_extra)
    if "roofline" in out:
        out["roofline"]["ceiling_GBps"] = ceiling
    out["workloads"] = [results[n] for n in names if n in results]
    print(json.dumps(out), flush=True)
    # every handle is closed above; let the device finish before the
    # interpreter and the runtime tear down
    torch.cuda.synchronize()


if __name__ == "__main__":
    main()
