"""Decoder throughput on one MI355X: prefill and decode tokens/s, the roofline
fraction of the dominant kernel, and the CPU oracle timed as a baseline.

Default workload (one "step" = one whole greedy job): the 28-block
1.7B-shaped stack with random bf16 weights; a 153-row causal prefill of N(0,1)
rows (last-block FFN on the final row only), the tied head's argmax gives the
first token, then 255 decode steps each run the 28 blocks and the head, with
the chosen token's embedding row fed back on the device. Decode steps replay
one captured HIP graph; no host sync per token. Inputs are resident in HBM
before the timed region.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--no-kernel-profile]

Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published (2.5 PFLOP/s)

# HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs, scaled by a plain
# 256 MiB copy (FETCH_SIZE x 1.9998, WRITE_SIZE x 1.0); valid only for the kernel
# sources they were taken on (sha256 of the listed files).
_GEMV_SRC = {"files": ["kernels_gemv.hip", "gemv_ops.h", "common.h"],
             "sha256": "4a9ef155e1b0b895a8b75c409161d378c9d1dcfadbcfa8868d7e479d1951cd19",
             "summary": "profiles/decode_gemv_block_t153_hbm_traffic.md"}
_QA_SRC = {"files": ["kernels_attn.hip", "attn_rows.h", "gemv_ops.h", "common.h"],
           "sha256": "489dfd92a79e7aaaa6db74cc679175c6aaebe43ce03d5e45eb8af3bb055838ab",
           "summary": "profiles/decode_gemv_block_t153_hbm_traffic.md"}
TRAFFIC = {
    "o_gemv": dict(_GEMV_SRC, rows=1, bytes=8676512),
    "gateup_gemv": dict(_GEMV_SRC, rows=1, bytes=50580211),
    "down_gemv": dict(_GEMV_SRC, rows=1, bytes=25508347),
    "qkv_attn": dict(_QA_SRC, rows=1, bytes=18062996),
}


def traffic_bytes(name, rows):
    """Counter-measured HBM bytes per launch, or None if absent, taken at another row
    count, or the kernel changed since."""
    import hashlib
    t = TRAFFIC.get(name)
    if not t or t["rows"] != rows:
        return None
    csrc = os.path.join(ROOT, "speech_text_decoder_amd", "csrc")
    h = hashlib.sha256(b"".join(open(os.path.join(csrc, f), "rb").read() for f in t["files"])).hexdigest()
    return t["bytes"] if h == t["sha256"] else None


KERNEL_NAMES = ["rmsnorm", "qkv_gemv", "qkv_gemm", "qk_rope_kv", "attn_rows", "attn_prefill", "o_gemv", "o_gemm",
                "gateup_gemv", "gateup_gemm", "down_gemv", "down_gemm", "lm_head", "qkv_attn"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_1p7b_stack28_greedy256")
    ap.add_argument("--replicas", type=int, default=8,
                    help="independent weight/KV replicas stacked for single-block workloads (MALL honesty)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-profile", action="store_true")
    ap.add_argument("--act-split", type=int, default=None,
                    help="STTD_OPT_ACT_SPLIT mask (GEMM inputs split into bf16 hi/lo above 512 rows); default: "
                         "the library's (all four) for stacks, 0 for the single-block workloads")
    ap.add_argument("--no-prefill-leg", action="store_true",
                    help="skip the 4096-row single-block prefill figure carried on the default line")
    ap.add_argument("--no-qkv-attn", action="store_true",
                    help="single decode rows: Q|K|V projection and attention as two launches (STTD_OPT_QKV_ATTN 0)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 3 times (scales HBM byte counters)")
    return ap.parse_args()


# ---------------------------------------------------------------- algorithmic cost model (per launch)
def kernel_cost(name, sh, rows, mean_keys=0.0):
    """(bytes, flops) of one launch, algorithmic: each weight byte once, activations in/out once."""
    wb = 2 if sh.wdtype == "bf16" else 4
    kvb = 2 if sh.kvdtype == "f16" else 4
    H, I, qd, kvd = sh.hidden, sh.ffn, sh.q_dim, sh.kv_dim
    qkv = qd + 2 * kvd
    if name in ("qkv_gemv", "qkv_gemm"):
        return qkv * H * wb + H * wb + rows * (H * 4 + qkv * 4), 2.0 * rows * H * qkv
    if name in ("o_gemv", "o_gemm"):
        return H * qd * wb + rows * (qd * 4 + 2 * H * 4), 2.0 * rows * qd * H
    if name in ("gateup_gemv", "gateup_gemm"):
        return 2 * I * H * wb + H * wb + rows * (H * 4 + I * 4), 2.0 * rows * H * 2 * I
    if name in ("down_gemv", "down_gemm"):
        return H * I * wb + rows * (I * 4 + 2 * H * 4), 2.0 * rows * I * H
    if name == "attn_rows":
        return rows * (mean_keys * kvd * 2 * kvb + 2 * qd * 4), rows * 4.0 * qd * mean_keys
    if name == "qk_rope_kv":
        return rows * (qkv * 4 + qd * 4 + 2 * kvd * kvb), 0.0
    if name == "lm_head":
        return sh.vocab * H * wb + rows * H * 4, 2.0 * rows * sh.vocab * H
    if name == "attn_prefill":   # causal: row t attends to t+1 keys; rows = prefill rows
        return rows * (2 * qd * 4 + 2 * kvd * kvb), 4.0 * qd * rows * (rows + 1) / 2
    if name == "rmsnorm":
        return rows * H * (4 + 4) + H * wb, 4.0 * rows * H
    if name == "qkv_attn":       # one decode row: Q|K|V projection and attention in one launch
        parts = [kernel_cost(n, sh, rows, mean_keys) for n in ("qkv_gemv", "attn_rows")]
        return sum(p[0] for p in parts), sum(p[1] for p in parts)
    return 0, 0.0


def decode_step_bytes(sh, n_layers, rows, mean_keys, with_head):
    """Algorithmic HBM bytes of one decode step: weights once, KV rows read, x and the new KV rows."""
    kvb = 2 if sh.kvdtype == "f16" else 4
    wb = 2 if sh.wdtype == "bf16" else 4
    per_block = sh.block_weight_bytes() + rows * (mean_keys * sh.kv_dim * 2 * kvb + 2 * sh.kv_dim * kvb)
    head = (sh.vocab * sh.hidden * wb + sh.hidden * wb) if with_head else 0
    return n_layers * per_block + head + rows * sh.hidden * 4 * 2


# ---------------------------------------------------------------- helpers
def cpu_model():
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads") for i in threadpool_info() if i.get("internal_api") in ("openblas", "mkl")]
        if n:
            return int(max(n))
    except Exception:
        pass
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


CLOCK_SLOTS = 1024
ALL_KERNELS = (1 << len(KERNEL_NAMES)) - 1


def clock_accumulate(binding, totals):
    for k, name in enumerate(KERNEL_NAMES):
        n, us = binding.clock_read(k)
        if n:
            t = totals.setdefault(name, [0, 0.0])
            t[0] += n
            t[1] += us


def clock_profile(binding, torch, stream, eager=None, capture=None, reps=8):
    """Per-kernel device-clock spans (first workgroup start to last workgroup end).

    eager(): launches run once, eagerly; capture(): launches captured into one HIP
    graph, which is then replayed `reps` times with the slots re-armed in between.
    Returns {name: [launches, total_us]}."""
    totals = {}
    if eager is not None:
        binding.clock_enable(ALL_KERNELS, CLOCK_SLOTS)
        with torch.cuda.stream(stream):
            eager()
        torch.cuda.synchronize()
        binding.clock_disable()
        clock_accumulate(binding, totals)
    if capture is not None:
        binding.clock_enable(ALL_KERNELS, CLOCK_SLOTS)
        with torch.cuda.stream(stream):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                capture()
        torch.cuda.synchronize()
        binding.clock_disable()
        for _ in range(reps):
            binding.clock_reset()
            with torch.cuda.stream(stream):
                g.replay()
            torch.cuda.synchronize()
            clock_accumulate(binding, totals)
        del g
    return totals


def event_profile(binding, torch, stream, fn):
    """Per-kernel HIP-event durations: fn() launches eagerly on `stream` with every
    kernel family bracketed by an event pair on that stream (sttd_profile_enable).
    Event pairs cover the dispatch and the end-of-kernel release, as rocprofv3's
    durations do. Returns {name: [launches, total_us]}."""
    binding.profile_enable(ALL_KERNELS)
    with torch.cuda.stream(stream):
        fn()
    torch.cuda.synchronize()
    binding.profile_enable(0)
    out = {}
    for k, name in enumerate(KERNEL_NAMES):
        n, ms = binding.profile_read(k)
        if n:
            out[name] = [n, ms * 1e3]
    return out


def kernel_table(totals, sh, rows_of, keys_of, events=None):
    """Attach algorithmic bytes/flops per launch and the achieved rates to the
    device-clock spans (and to the HIP-event durations, when given)."""
    out = {}
    for name, (n, us) in totals.items():
        avg_us = us / n
        b, f = kernel_cost(name, sh, rows_of(name), keys_of(name))
        e = {"launches": n, "avg_us": round(avg_us, 3), "bytes": int(b), "flops": f,
             "gbs": round(b / (avg_us * 1e-6) / 1e9, 1) if b else None,
             "tflops": round(f / (avg_us * 1e-6) / 1e12, 2) if f else None}
        if events and name in events:
            ev_us = events[name][1] / events[name][0]
            e["event_avg_us"] = round(ev_us, 3)
            e["event_gbs"] = round(b / (ev_us * 1e-6) / 1e9, 1) if b else None
            e["event_tflops"] = round(f / (ev_us * 1e-6) / 1e12, 2) if f else None
        out[name] = e
    return out


def job_roofline(phases):
    """The roofline object of the kernel family that takes the most time over the
    job. phases: [(phase, table, events, launches_per_job_scale, rows_of)], where
    events[name] = [launches, total_us] of the profiled launches and the scale turns
    those into per-job time (e.g. steps per job / steps profiled)."""
    best = None
    total = 0.0
    for phase, table, events, scale, rows_of in phases:
        for name, (n, us) in events.items():
            t = us * scale
            total += t
            if name in table and (best is None or t > best[0]):
                best = (t, phase, table, name, rows_of(name))
    if best is None:
        return None
    t, phase, table, name, rows = best
    r = roofline_entry(table, name, kernel_bound(name, rows), rows)
    r["phase"] = phase
    r["job_share"] = round(t / total, 4) if total else None
    return r


def roofline_entry(table, name, bound, rows=1):
    """The roofline object of one kernel family. achieved = algorithmic bytes (flops)
    per launch / the HIP-event average duration of its launches (the headline; it
    covers what rocprofv3's kernel durations cover); the device-clock span figure
    (first workgroup start to last workgroup end, shorter by the dispatch and the
    end-of-kernel release) is reported beside it."""
    e = table.get(name)
    if not e:
        return None
    ev_us = e.get("event_avg_us", e["avg_us"])
    timing = "hip events" if "event_avg_us" in e else "device clock"
    if bound == "hbm":
        ach = e["bytes"] / (ev_us * 1e-6) / 1e9
        return {"kernel": name, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic_bytes(name, rows), "avg_us": round(ev_us, 3),
                "timing": timing, "bytes_per_launch": e["bytes"], "device_span_avg_us": e["avg_us"],
                "device_span_frac": round(e["gbs"] / HBM_PEAK_GBS, 4)}
    ach = e["flops"] / (ev_us * 1e-6) / 1e12
    return {"kernel": name, "bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": None, "avg_us": round(ev_us, 3), "timing": timing,
            "flops_per_launch": e.get("flops"), "device_span_avg_us": e["avg_us"],
            "device_span_frac": round(e["tflops"] / BF16_PEAK_TFLOPS, 4)}


def kernel_bound(name, rows):
    """Which roof a kernel family is held to at this row count: MFMA for the many-row
    GEMMs and the flash attention (arithmetic intensity above the ~315 FLOP/B ridge),
    HBM for everything that streams weights or the cache."""
    if name == "attn_prefill" or (name.endswith("gemm") and rows >= 1024):
        return "mfma"
    return "hbm"


# ---------------------------------------------------------------- greedy stack (prefill + greedy decode)
def bench_greedy_stack(args, wl):
    import torch
    from speech_text_decoder_amd import binding, synth
    from speech_text_decoder_amd.device import DecoderSession

    sh = wl.shape
    T, n_steps = wl.prefill_rows, wl.steps
    layers = [synth.block_weights(wl.cfg_id, l, sh) for l in range(sh.n_layers)]
    E = synth.embedding(wl.cfg_id, sh)
    g = synth.final_norm(wl.cfg_id, sh)
    x_host = synth.prefill_rows(wl.cfg_id, T, sh.hidden)
    sess = DecoderSession(sh, layers, embed=E, final_norm=g, n_ctx=wl.n_ctx, max_rows=T)
    sess.set_qkv_attn(not args.no_qkv_attn)
    if args.act_split is not None:
        sess.set_act_split(args.act_split)
    x0 = torch.from_numpy(x_host).cuda()
    x = torch.empty_like(x0)
    xs = torch.zeros(1, sh.hidden, device="cuda")
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    pos0 = torch.full((1,), T, dtype=torch.int32, device="cuda")

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            sess.step(xs, pos, pos_bound=wl.n_ctx)
            sess.head(xs, ids, next_x=xs, pos=pos)
    torch.cuda.synchronize()

    def prefill_part(s):
        with torch.cuda.stream(s):
            x.copy_(x0)
            sess.prefill(x, slice_last=True)
            sess.head(x[T - 1:], ids, next_x=xs)
            pos.copy_(pos0)

    def job(ev=None):
        with torch.cuda.stream(stream):
            if ev:
                ev[0].record(stream)
            prefill_part(stream)
            if ev:
                ev[1].record(stream)
            for _ in range(n_steps):
                graph.replay()
            if ev:
                ev[2].record(stream)

    for _ in range(args.warmup):
        job()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        job(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dec_ms = [e[1].elapsed_time(e[2]) for e in evs]
    job_ms = [e[0].elapsed_time(e[2]) for e in evs]
    assert int(pos.item()) == T + n_steps, "step loop did not advance the device position"
    last_token = int(ids.item())

    ms = float(np.median(job_ms))
    new_tokens = n_steps + 1
    mean_keys = T + (n_steps + 1) / 2.0
    step_bytes = decode_step_bytes(sh, sh.n_layers, 1, mean_keys, True)
    dec_step_ms = float(np.median(dec_ms)) / n_steps
    res = {
        "value": round(new_tokens / (ms * 1e-3), 2),
        "ms_per_step": round(ms, 3),
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 3),
        "prefill_ms": round(float(np.median(pre_ms)), 4),
        "prefill_tok_s": round(T / (float(np.median(pre_ms)) * 1e-3), 1),
        "decode_ms_per_token": round(dec_step_ms, 5),
        "decode_tok_s": round(1e3 / dec_step_ms, 2),
        "decode_step_bytes": int(step_bytes),
        "decode_step_hbm_frac": round(step_bytes / (dec_step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "last_token": last_token,
        "config": {"workload": wl.name, "layers": sh.n_layers, "hidden": sh.hidden, "heads": sh.n_heads,
                   "kv_heads": sh.n_kv_heads, "head_dim": sh.head_dim, "ffn": sh.ffn, "vocab": sh.vocab,
                   "prefill_rows": T, "new_tokens": new_tokens, "batch": 1, "kv_dtype": sh.kvdtype,
                   "n_ctx": wl.n_ctx, "parallelism": "none (1 GPU)", "qkv_attn": not args.no_qkv_attn,
                   "act_split_above_512_rows": args.act_split if args.act_split is not None else 15},
    }
    if not args.no_kernel_profile:
        # device-clock spans: the prefill part eagerly, the decode step+head as a replayed
        # graph; HIP-event durations: the same launches eagerly. Each profile starts from a
        # fresh prefill, so the decode steps run at positions T, T + 1, ...
        reps = 16

        def dec_steps():
            for _ in range(reps):
                sess.step(xs, pos, pos_bound=wl.n_ctx)
                sess.head(xs, ids, next_x=xs, pos=pos)

        pre = clock_profile(binding, torch, stream, eager=lambda: prefill_part(stream))
        dec = clock_profile(binding, torch, stream, reps=reps, capture=lambda: (
            sess.step(xs, pos, pos_bound=wl.n_ctx), sess.head(xs, ids, next_x=xs, pos=pos)))
        pre_ev = event_profile(binding, torch, stream, lambda: prefill_part(stream))
        dec_ev = event_profile(binding, torch, stream, dec_steps)
        torch.cuda.synchronize()
        rows = lambda n: T if n.endswith("gemm") or n in ("rmsnorm", "attn_prefill") else 1
        res["kernels"] = {"prefill": kernel_table(pre, sh, rows, lambda n: T, pre_ev),
                          "decode": kernel_table(dec, sh, lambda n: 1, lambda n: T + 1 + reps / 2.0, dec_ev)}
        res["kernel_timing"] = ("avg_us: device clock (s_memrealtime, 100 MHz), first-workgroup start to "
                                "last-workgroup end; event_avg_us: HIP event pair bound to each eager dispatch (hipExtLaunchKernel)")
        res["roofline"] = job_roofline([("prefill", res["kernels"]["prefill"], pre_ev, 1.0, rows),
                                        ("decode", res["kernels"]["decode"], dec_ev, n_steps / reps,
                                         lambda n: 1)])
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_greedy(wl, layers, E, g, x_host, new_tokens)
    sess.close()
    return res


def cpu_baseline_greedy(wl, layers, E, g, x_host, new_tokens):
    """The oracle on the host: prefill + 2 greedy steps of the same stack, extrapolated to the job."""
    import oracle as O
    from speech_text_decoder_amd import synth

    sh = wl.shape
    T = wl.prefill_rows
    ol = [{k: synth.widen(v).astype(np.float64) for k, v in w.items()} for w in layers]
    Ef = synth.widen(E).astype(np.float64)
    gf = synth.widen(g)
    cache = O.KVCache(sh.n_layers, 1, T + 4, sh.n_kv_heads, sh.head_dim)
    t0 = time.perf_counter()
    last = O.prefill_stack(x_host, ol, sh, cache, slice_last=True)
    tok = O.greedy_token(O.final_logits(last, gf, Ef, sh.rms_eps)[0])
    t1 = time.perf_counter()
    n = 2
    for k in range(n):
        xo = O.step_stack(Ef[tok][None], [T + k], [0], ol, sh, cache)
        tok = O.greedy_token(O.final_logits(xo, gf, Ef, sh.rms_eps)[0])
    t2 = time.perf_counter()
    step_s = (t2 - t1) / n
    job_s = (t1 - t0) + (new_tokens - 1) * step_s
    return {"value": round(new_tokens / job_s, 4), "unit": "tokens/s", "cores": cpu_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"fp64 oracle: {T}-row prefill of the 28-block stack + head ({t1 - t0:.1f} s), then {n} greedy "
                      f"steps ({step_s:.2f} s each); job time extrapolated to {new_tokens} new tokens",
            "prefill_tok_s": round(T / (t1 - t0), 2), "decode_tok_s": round(1.0 / step_s, 4)}


# ---------------------------------------------------------------- packed batched prefill
def bench_packed_prefill(args, wl):
    """B prompts: token embeddings with an injected audio block each, packed back to
    back through one prefill call per block of the stack, then every prompt's last row
    through the tied head. value = prompt rows per second of the whole job; the same
    prompts one at a time are timed beside it."""
    import torch
    from speech_text_decoder_amd import binding, synth
    from speech_text_decoder_amd.device import DecoderSession

    sh = wl.shape
    Bn, T = wl.batch, wl.prefill_rows
    pre, n_audio, suf = wl.prompt_split
    assert pre + n_audio + suf == T
    layers = [synth.block_weights(wl.cfg_id, l, sh) for l in range(sh.n_layers)]
    E = synth.embedding(wl.cfg_id, sh)
    g = synth.final_norm(wl.cfg_id, sh)
    ids_h, keep_h, dense_h = synth.injected_prompts(wl.cfg_id, Bn, wl.prompt_split, sh.hidden, sh.vocab)
    sess = DecoderSession(sh, layers, embed=E, final_norm=g, n_ctx=wl.n_ctx, n_seq=Bn, max_rows=Bn * T)
    if args.act_split is not None:
        sess.set_act_split(args.act_split)
    ids_d = torch.from_numpy(ids_h).cuda()
    keep_d = torch.from_numpy(keep_h).cuda()
    dense_d = torch.from_numpy(dense_h).cuda()
    x = torch.empty(Bn * T, sh.hidden, device="cuda")
    out_ids = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    last_rows = torch.arange(1, Bn + 1, dtype=torch.int32, device="cuda") * T - 1
    stream = torch.cuda.Stream()

    def packed_job():
        sess.inject(ids_d, keep_d, dense_d, x, stream=stream)
        sess.prefill_batched(x, [T] * Bn, list(range(Bn)), stream=stream)
        # each prompt's last row, picked on the device by row index
        sess.head(x, out_ids, x_rows=last_rows, stream=stream)

    def separate_job():
        for b in range(Bn):
            r = slice(b * T, (b + 1) * T)
            sess.inject(ids_d[r], keep_d[r], dense_d[r], x[r], stream=stream)
            sess.prefill(x[r], seq=b, stream=stream)
            sess.head(x[(b + 1) * T - 1:(b + 1) * T], out_ids[b:b + 1], stream=stream)

    def timed(job):
        with torch.cuda.stream(stream):
            for _ in range(args.warmup):
                job()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        with torch.cuda.stream(stream):
            for i in range(args.steps):
                evs[i][0].record(stream)
                job()
                evs[i][1].record(stream)
        torch.cuda.synchronize()
        return float(np.median([e[0].elapsed_time(e[1]) for e in evs]))

    t0 = time.perf_counter()
    ms = timed(packed_job)
    wall = time.perf_counter() - t0
    packed_ids = out_ids.cpu().numpy().tolist()
    ms_sep = timed(separate_job)
    assert out_ids.cpu().numpy().tolist() == packed_ids, "packed and one-at-a-time prefills chose different ids"
    rows = Bn * T
    res = {
        "value": round(rows / (ms * 1e-3), 1),
        "ms_per_step": round(ms, 3),
        "wall_ms_per_step": round(wall * 1e3 / (args.steps + args.warmup), 3),
        "prefill_tok_s": round(rows / (ms * 1e-3), 1),
        "one_at_a_time_ms": round(ms_sep, 3),
        "one_at_a_time_tok_s": round(rows / (ms_sep * 1e-3), 1),
        "ids": packed_ids,
        "config": {"workload": wl.name, "layers": sh.n_layers, "hidden": sh.hidden, "heads": sh.n_heads,
                   "kv_heads": sh.n_kv_heads, "head_dim": sh.head_dim, "ffn": sh.ffn, "vocab": sh.vocab,
                   "prompts": Bn, "prompt_rows": T, "prompt_split": list(wl.prompt_split), "kv_dtype": sh.kvdtype,
                   "n_ctx": wl.n_ctx, "parallelism": "none (1 GPU)",
                   "act_split_above_512_rows": args.act_split if args.act_split is not None else 15},
    }
    if not args.no_kernel_profile:
        prof = clock_profile(binding, torch, stream, eager=packed_job)
        ev = event_profile(binding, torch, stream, packed_job)
        torch.cuda.synchronize()
        rws = lambda n: rows if n.endswith("gemm") or n in ("rmsnorm", "qk_rope_kv") else (
            T if n == "attn_prefill" else Bn)
        res["kernels"] = {"prefill": kernel_table(prof, sh, rws, lambda n: T, ev)}
        res["kernel_timing"] = ("avg_us: device clock (s_memrealtime, 100 MHz), first-workgroup start to "
                                "last-workgroup end; event_avg_us: HIP event pair bound to each eager dispatch (hipExtLaunchKernel)")
        res["roofline"] = job_roofline([("prefill", res["kernels"]["prefill"], ev, 1.0, rws)])
    if not args.no_cpu_baseline:
        import oracle as O
        ol = [{k: synth.widen(v).astype(np.float64) for k, v in w.items()} for w in layers]
        Ef = synth.widen(E).astype(np.float64)
        cache = O.KVCache(sh.n_layers, 1, T, sh.n_kv_heads, sh.head_dim)
        t0 = time.perf_counter()
        x0 = O.inject(Ef, ids_h[:T], keep_h[:T], dense_h[:T])
        last = O.prefill_stack(x0, ol, sh, cache)[-1:]
        O.greedy_token(O.final_logits(last, synth.widen(g), Ef, sh.rms_eps)[0])
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(T / dt, 2), "unit": "tokens/s", "cores": cpu_threads(),
                               "kind": "oracle", "cpu_model": cpu_model(),
                               "sample": f"fp64 oracle: one of the {Bn} prompts ({T} rows: "
                               f"injection, 28 blocks, head) in {dt:.1f} s"}
    sess.close()
    return res


# ---------------------------------------------------------------- single-block workloads (replicated)
def bench_block(args, wl):
    """One 1.7B-shaped block, timed as R independent replicas (distinct weights and KV)
    chained per step, so the weights stream from HBM rather than the 256 MB MALL; per-block
    figures are totals / R."""
    import torch
    from speech_text_decoder_amd import binding, synth
    from speech_text_decoder_amd.device import DecoderSession

    sh = wl.shape
    R = max(1, args.replicas)
    T, n_steps = wl.prefill_rows, wl.steps
    layers = [synth.block_weights(wl.cfg_id, r, sh) for r in range(R)]
    x_host = synth.prefill_rows(wl.cfg_id, T, sh.hidden)
    rows_host = np.stack([synth.step_rows(wl.cfg_id, k, 1, sh.hidden)[0] for k in range(n_steps)])
    sess = DecoderSession(sh, layers, n_ctx=wl.n_ctx, max_rows=T)
    sess.set_qkv_attn(not args.no_qkv_attn)
    # one block (the replicas are independent single blocks): plain bf16 activations
    # above 512 rows stay within the parity bound for a single block
    sess.set_act_split(args.act_split if args.act_split is not None else 0)
    x0 = torch.from_numpy(x_host).cuda()
    x = torch.empty_like(x0)
    r0 = torch.from_numpy(rows_host).cuda()
    rows = torch.empty_like(r0)
    pos_all = torch.arange(T, T + n_steps, dtype=torch.int32, device="cuda").view(n_steps, 1)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()

    def decode_loop():
        for k in range(n_steps):
            sess.step(rows[k:k + 1], pos_all[k], pos_bound=T + k + 1)

    with torch.cuda.stream(stream):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            decode_loop()
    torch.cuda.synchronize()

    def job(ev=None):
        with torch.cuda.stream(stream):
            x.copy_(x0)
            rows.copy_(r0)
            if ev:
                ev[0].record(stream)
            sess.prefill(x)
            if ev:
                ev[1].record(stream)
            graph.replay()
            if ev:
                ev[2].record(stream)

    for _ in range(args.warmup):
        job()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        job(evs[i])
    torch.cuda.synchronize()
    pre_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs])) / R
    dec_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evs])) / R / n_steps
    mean_keys = T + (n_steps + 1) / 2.0
    step_bytes = decode_step_bytes(sh, 1, 1, mean_keys, False)
    H, I, qd, kvd = sh.hidden, sh.ffn, sh.q_dim, sh.kv_dim
    gemm_flops = 2.0 * T * H * (qd + 2 * kvd + I * 2) + 2.0 * T * (qd * H + I * H)
    attn_flops = 4.0 * sh.n_heads * sh.head_dim * T * (T + 1) / 2
    pre_flops = gemm_flops + attn_flops
    res = {
        "value": round((T + n_steps) / ((pre_ms + dec_ms * n_steps) * 1e-3), 1),
        "ms_per_step": round((pre_ms + dec_ms * n_steps) * R, 4),
        "prefill_ms_per_block": round(pre_ms, 5),
        "prefill_tok_s_per_block": round(T / (pre_ms * 1e-3), 1),
        "prefill_tflops": round(pre_flops / (pre_ms * 1e-3) / 1e12, 2),
        "prefill_mfma_frac": round(pre_flops / (pre_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "decode_us_per_block_step": round(dec_ms * 1e3, 3),
        "decode_tok_s_per_block": round(1e3 / dec_ms, 1),
        "decode_step_bytes": int(step_bytes),
        "decode_hbm_frac": round(step_bytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "config": {"workload": wl.name, "replicas": R, "hidden": sh.hidden, "heads": sh.n_heads,
                   "kv_heads": sh.n_kv_heads, "head_dim": sh.head_dim, "ffn": sh.ffn, "prefill_rows": T,
                   "decode_steps": n_steps, "batch": 1, "kv_dtype": sh.kvdtype, "wdtype": sh.wdtype,
                   "parallelism": "none (1 GPU)", "qkv_attn": not args.no_qkv_attn,
                   "act_split_above_512_rows": args.act_split if args.act_split is not None else 0},
    }
    if R > 1:
        # the same job on one replica: its 100.7 MB of weights then stay in the 256 MB MALL
        # between steps (labelled separately; the headline uses the replicas above)
        with torch.cuda.stream(stream):
            g1 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g1, stream=stream):
                for k in range(n_steps):
                    sess.step(rows[k:k + 1], pos_all[k], pos_bound=T + k + 1, layers=[0])
        torch.cuda.synchronize()
        ev1 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for i in range(args.warmup + args.steps):
            with torch.cuda.stream(stream):
                x.copy_(x0)
                rows.copy_(r0)
                if i >= args.warmup:
                    ev1[i - args.warmup][0].record(stream)
                sess.prefill(x, layers=[0])
                if i >= args.warmup:
                    ev1[i - args.warmup][1].record(stream)
                g1.replay()
                if i >= args.warmup:
                    ev1[i - args.warmup][2].record(stream)
        torch.cuda.synchronize()
        p1 = float(np.median([e[0].elapsed_time(e[1]) for e in ev1]))
        d1 = float(np.median([e[1].elapsed_time(e[2]) for e in ev1])) / n_steps
        res["mall_resident_one_replica"] = {
            "prefill_ms_per_block": round(p1, 5), "decode_us_per_block_step": round(d1 * 1e3, 3),
            "decode_hbm_frac_equiv": round(step_bytes / (d1 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del g1
    if not args.no_kernel_profile:
        n_prof = min(n_steps, 16)

        def pre_eager():
            x.copy_(x0)
            rows.copy_(r0)
            sess.prefill(x)

        def dec_capture():
            for k in range(n_prof):
                sess.step(rows[k:k + 1], pos_all[k], pos_bound=T + k + 1)

        pre = clock_profile(binding, torch, stream, eager=pre_eager)
        dec = clock_profile(binding, torch, stream, capture=dec_capture, reps=4)
        pre_ev = event_profile(binding, torch, stream, pre_eager)
        dec_ev = event_profile(binding, torch, stream, dec_capture)
        rw = lambda n: T if n.endswith("gemm") or n in ("rmsnorm", "attn_prefill") else 1
        res["kernels"] = {"prefill": kernel_table(pre, sh, rw, lambda n: T, pre_ev),
                          "decode": kernel_table(dec, sh, lambda n: 1, lambda n: T + (n_prof + 1) / 2.0, dec_ev)}
        res["kernel_timing"] = ("avg_us: device clock (s_memrealtime, 100 MHz), first-workgroup start to "
                                "last-workgroup end; event_avg_us: HIP event pair bound to each eager dispatch (hipExtLaunchKernel)")
        res["roofline"] = job_roofline([("prefill", res["kernels"]["prefill"], pre_ev, 1.0, rw),
                                        ("decode", res["kernels"]["decode"], dec_ev, n_steps / n_prof,
                                         lambda n: 1)])
        # the prefill's own dominant kernel (the MFMA roof for long prefills)
        res["prefill_roofline"] = job_roofline([("prefill", res["kernels"]["prefill"], pre_ev, 1.0, rw)])
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_block(wl, layers[0], x_host, rows_host)
    sess.close()
    return res


def cpu_baseline_block(wl, w, x_host, rows_host):
    import oracle as O
    from speech_text_decoder_amd import synth

    sh = wl.shape
    T = wl.prefill_rows
    ow = {k: synth.widen(v).astype(np.float64) for k, v in w.items()}
    cache = O.KVCache(1, 1, T + 8, sh.n_kv_heads, sh.head_dim)
    Ts = min(T, 512)
    t0 = time.perf_counter()
    O.block(x_host[:Ts], np.arange(Ts), np.zeros(Ts, int), ow, sh, cache, 0)
    t1 = time.perf_counter()
    n = 4
    for k in range(n):
        O.block(rows_host[k:k + 1], [Ts + k], [0], ow, sh, cache, 0)
    t2 = time.perf_counter()
    return {"value": round((Ts + n) / (t2 - t0), 3), "unit": "tokens/s", "cores": cpu_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"fp64 oracle, one block: {Ts}-row prefill ({t1 - t0:.2f} s) + {n} decode steps "
                      f"({(t2 - t1) / n:.3f} s each)",
            "prefill_tok_s": round(Ts / (t1 - t0), 2), "decode_tok_s": round(n / (t2 - t1), 3)}


# ---------------------------------------------------------------- batched decode
def bench_batched(args, wl):
    import torch
    from speech_text_decoder_amd import binding, synth
    from speech_text_decoder_amd.device import DecoderSession

    sh = wl.shape
    Bn, n_steps, n_ctx = wl.batch, wl.steps, wl.n_ctx
    lens = synth.context_lengths(wl.cfg_id, Bn, *wl.ctx_len_range)
    layers = [synth.block_weights(wl.cfg_id, l, sh) for l in range(sh.n_layers)]
    E = synth.embedding(wl.cfg_id, sh)
    g = synth.final_norm(wl.cfg_id, sh)
    sess = DecoderSession(sh, layers, embed=E, final_norm=g, n_ctx=n_ctx, n_seq=Bn, max_rows=Bn)
    for l in range(sh.n_layers):
        for b in range(Bn):
            k, v = synth.kv_fill(wl.cfg_id, l, b, int(lens[b]), sh, n_ctx)
            gk, gv = sess.kv_slab(l, b)
            gk[:, :lens[b], :] = torch.from_numpy(synth.kv_stored(k, sh.kvdtype).view(np.int16)).cuda().permute(1, 0, 2)
            gv[:, :lens[b], :] = torch.from_numpy(synth.kv_stored(v, sh.kvdtype).view(np.int16)).cuda().permute(1, 0, 2)
    x0 = torch.from_numpy(synth.step_rows(wl.cfg_id, 0, Bn, sh.hidden)).cuda()
    x = torch.empty_like(x0)
    pos0 = torch.from_numpy(lens.astype(np.int32)).cuda()
    pos = torch.empty_like(pos0)
    ids = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    bound = int(lens.max()) + n_steps + 1
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            sess.step(x, pos, pos_bound=bound)
            sess.head(x, ids, next_x=x, pos=pos)
    torch.cuda.synchronize()

    def job(ev=None):
        with torch.cuda.stream(stream):
            x.copy_(x0)
            pos.copy_(pos0)
            if ev:
                ev[0].record(stream)
            for _ in range(n_steps):
                graph.replay()
            if ev:
                ev[1].record(stream)

    for _ in range(args.warmup):
        job()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        job(evs[i])
    torch.cuda.synchronize()
    ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    mean_keys = float(lens.mean()) + (n_steps + 1) / 2.0
    step_bytes = decode_step_bytes(sh, sh.n_layers, Bn, mean_keys, True)
    step_ms = ms / n_steps
    res = {
        "value": round(Bn * n_steps / (ms * 1e-3), 1),
        "ms_per_step": round(ms, 3),
        "decode_ms_per_step": round(step_ms, 4),
        "decode_step_bytes": int(step_bytes),
        "decode_step_hbm_frac": round(step_bytes / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "config": {"workload": wl.name, "layers": sh.n_layers, "batch": Bn, "steps": n_steps,
                   "ctx_len_range": list(wl.ctx_len_range), "mean_ctx": float(lens.mean()), "n_ctx": n_ctx,
                   "kv_dtype": sh.kvdtype, "parallelism": "none (1 GPU)", "qkv_attn": not args.no_qkv_attn},
    }
    if not args.no_kernel_profile:
        with torch.cuda.stream(stream):
            x.copy_(x0)
            pos.copy_(pos0)
        reps = 8

        def eager_steps():
            x.copy_(x0)
            pos.copy_(pos0)
            for _ in range(reps):
                sess.step(x, pos, pos_bound=bound)
                sess.head(x, ids, next_x=x, pos=pos)

        dec = clock_profile(binding, torch, stream, reps=reps, capture=lambda: (
            sess.step(x, pos, pos_bound=bound), sess.head(x, ids, next_x=x, pos=pos)))
        ev = event_profile(binding, torch, stream, eager_steps)
        table = kernel_table(dec, sh, lambda n: Bn, lambda n: float(lens.mean()) + (reps + 1) / 2.0, ev)
        res["kernels"] = {"decode": table}
        res["kernel_timing"] = ("avg_us: device clock (s_memrealtime, 100 MHz), first-workgroup start to "
                                "last-workgroup end; event_avg_us: HIP event pair bound to each eager dispatch (hipExtLaunchKernel)")
        res["roofline"] = job_roofline([("decode", table, ev, n_steps / reps, lambda n: Bn)])
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_batched(wl, layers, E, g, lens)
    sess.close()
    return res


def cpu_baseline_batched(wl, layers, E, g, lens):
    """The oracle on the host: one decode step of two of the batch's sequences (the
    shortest and the longest context) through the 28 blocks + head, with their
    caches filled as on the GPU; rows per second of that sample."""
    import oracle as O
    from speech_text_decoder_amd import synth

    sh = wl.shape
    sample = [int(np.argmin(lens)), int(np.argmax(lens))]
    ol = [{k: synth.widen(v).astype(np.float64) for k, v in w.items()} for w in layers]
    Ef = synth.widen(E).astype(np.float64)
    gf = synth.widen(g)
    cache = O.KVCache(sh.n_layers, len(sample), int(lens.max()) + 2, sh.n_kv_heads, sh.head_dim)
    for l in range(sh.n_layers):
        for i, b in enumerate(sample):
            k, v = synth.kv_fill(wl.cfg_id, l, b, int(lens[b]), sh, wl.n_ctx)
            cache.k[l, i, :lens[b]] = synth.kv_widen(synth.kv_stored(k, sh.kvdtype))
            cache.v[l, i, :lens[b]] = synth.kv_widen(synth.kv_stored(v, sh.kvdtype))
    x = synth.step_rows(wl.cfg_id, 0, wl.batch, sh.hidden)[sample].astype(np.float64)
    t0 = time.perf_counter()
    xo = O.step_stack(x, lens[sample], list(range(len(sample))), ol, sh, cache)
    [O.greedy_token(r) for r in O.final_logits(xo, gf, Ef, sh.rms_eps)]
    dt = time.perf_counter() - t0
    return {"value": round(len(sample) / dt, 4), "unit": "tokens/s", "cores": cpu_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"fp64 oracle: one decode step of 2 of the {wl.batch} sequences (contexts "
                      f"{int(lens[sample[0]])} and {int(lens[sample[1]])}) through 28 blocks + head in {dt:.2f} s"}


def prefill_leg(args, name="qwen3_1p7b_block_long4096", replicas=8):
    """The long-prefill figure carried on the default line: the causal prefill of one
    1.7B-shaped block over 4096 rows, timed as `replicas` independent replicas chained
    (weights and KV stream from HBM, not the 256 MB MALL), per block = total / replicas;
    bf16 MFMA fraction of the whole prefill and the roofline of its dominant kernel."""
    import torch
    from speech_text_decoder_amd import binding, synth
    from speech_text_decoder_amd.device import DecoderSession
    from speech_text_decoder_amd.workloads import WORKLOADS

    wl = WORKLOADS[name]
    sh = wl.shape
    T = wl.prefill_rows
    layers = [synth.block_weights(wl.cfg_id, r, sh) for r in range(replicas)]
    x_host = synth.prefill_rows(wl.cfg_id, T, sh.hidden)
    sess = DecoderSession(sh, layers, n_ctx=wl.n_ctx, max_rows=T)
    x0 = torch.from_numpy(x_host).cuda()
    x = torch.empty_like(x0)
    stream = torch.cuda.Stream()

    def run():
        x.copy_(x0)
        sess.prefill(x)

    def timed_ms():
        with torch.cuda.stream(stream):
            for _ in range(args.warmup):
                run()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for i in range(args.steps):
                x.copy_(x0)
                evs[i][0].record(stream)
                sess.prefill(x)
                evs[i][1].record(stream)
        torch.cuda.synchronize()
        return float(np.median([e[0].elapsed_time(e[1]) for e in evs])) / replicas

    H, I, qd, kvd = sh.hidden, sh.ffn, sh.q_dim, sh.kv_dim
    flops = 2.0 * T * H * (qd + 2 * kvd + I * 2) + 2.0 * T * (qd * H + I * H) + 4.0 * qd * T * (T + 1) / 2
    sess.set_act_split(binding.SPLIT_ALL)
    ms_split = timed_ms()
    # the headline: one block with plain bf16 GEMM activations (within the parity
    # bound for a single block; its 4096-row parity test runs the same mode)
    sess.set_act_split(0)
    ms = timed_ms()
    out = {"workload": name, "rows": T, "replicas": replicas, "act_split": 0, "prefill_ms_per_block": round(ms, 5),
           "prefill_tok_s_per_block": round(T / (ms * 1e-3), 1),
           "prefill_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
           "prefill_mfma_frac": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
           "split_activations": {"act_split": binding.SPLIT_ALL, "prefill_ms_per_block": round(ms_split, 5),
                                 "prefill_mfma_frac": round(flops / (ms_split * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}}
    if not args.no_kernel_profile:
        pre = clock_profile(binding, torch, stream, eager=run)
        ev = event_profile(binding, torch, stream, run)
        rw = lambda n: T if n.endswith("gemm") or n in ("rmsnorm", "attn_prefill") else 1
        out["kernels"] = kernel_table(pre, sh, rw, lambda n: T, ev)
        out["roofline"] = job_roofline([("prefill", out["kernels"], ev, 1.0, rw)])
    sess.close()
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "one GPU only: the decoder block is not sharded across GPUs; "
                                   "run with --gpus 1", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    from speech_text_decoder_amd import binding
    from speech_text_decoder_amd.workloads import WORKLOADS

    binding.lib()  # fails loudly when the HIP library is missing
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n // 4, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read": n, "bytes_written": n, "launches": 3}}), flush=True)
        return
    wl = WORKLOADS[args.workload]
    if wl.packed:
        res = bench_packed_prefill(args, wl)
        unit = "tokens/s"
    elif wl.greedy and wl.prefill_rows > 0:
        res = bench_greedy_stack(args, wl)
        unit = "tokens/s"
        if args.workload == "qwen3_1p7b_stack28_greedy256" and not args.no_prefill_leg:
            res["long_prefill"] = prefill_leg(args)
    elif wl.batch > 1:
        res = bench_batched(args, wl)
        unit = "tokens/s"
    else:
        res = bench_block(args, wl)
        unit = "tokens/s"
    out = {"metric": "decoder tokens/sec (prefill, decode) + % of MFMA/HBM roofline, 1 MI355X",
           "value": res.pop("value"), "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": res.pop("ms_per_step"), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if wl.shape.wdtype == "bf16" else "f32", "data": "synthetic (seeded N(0,1) rows, "
           "N(0,0.02) weights, 1+N(0,0.02) gains)", "config": res.pop("config")}
    out.update(res)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
