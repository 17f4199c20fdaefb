#!/usr/bin/env python
"""Decoder tokens/s of the RLT recurrent decoder on one MI355X, and its roofline fraction.

One benchmark step is one ``rlt_run_sequence`` call on a fresh state and empty memory: the
token-parallel memory projection of all T tokens, then the T sequential decoder
transitions for all B sequences, recording every s_t. The workload is the ~140M-scale
configuration (d=768, 12 heads x 64, 12 blocks, FFN 3072, W=128, layer-specific memory,
alpha=1, B=256, T=1024) with synthetic N(0,1) encoder outputs and N(0, 0.02) weights.

Printed JSON (one line): value = B*T*steps / timed seconds; ``roofline`` for the dominant
kernel (cross-attention; algorithmic bytes / HIP-event time of its launches over the timed
region, against 8 TB/s HBM); ``step_roofline`` = ideal per-step roofline time over measured
time; ``cpu_baseline`` = the CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12        # MI355X HBM3E, bytes/s
BF16_PEAK = 2.5e15       # MI355X dense bf16 MFMA, flop/s
FP32_PEAK = 157.3e12
METRIC = "RLT decoder tokens/sec (B seqs x T) on 1 MI355X; % of per-step roofline"


def step_roofline_seconds(cfg, B: int, T: int, memory_once: bool = False) -> float:
    """Ideal time of one run: memory projection + T steps, each at max(bytes / HBM peak,
    flops / MFMA peak) with the algorithmic bytes of every step (weights once, the window and
    the memory prefix of every layer once, s read and written). With ``memory_once`` (only
    meaningful for one memory shared by all layers) the shared prefix counts once per step
    instead of once per layer: the floor if the layers' re-reads all hit a cache."""
    d, L, F, W, G = cfg.d, cfg.n_layers, cfg.ffn, cfg.window, cfg.n_groups
    es = 2 if cfg.dtype == "bf16" else 4
    peak = BF16_PEAK if cfg.dtype == "bf16" else FP32_PEAK
    p_step = 2 * d * d + L * (6 * d * d + 3 * d * F)
    mem_reads = 1 if memory_once else L
    total = 0.0
    for t in range(1, T + 1):
        win = min(t, W)
        by = (es * (p_step + B * L * win * 2 * d + B * mem_reads * t * 2 * d)
              + B * d * (es + 8))
        fl = 2 * B * p_step + 4 * B * L * d * (win + t)
        total += max(by / HBM_PEAK, fl / peak)
    mp_bytes = es * (B * T * d + G * B * T * 2 * d + 2 * G * d * d)
    mp_flops = 2 * B * T * 2 * G * d * d
    return total + max(mp_bytes / HBM_PEAK, mp_flops / peak)


def traffic_record(workload: str):
    """HBM bytes per memory-attention launch measured by rocprofv3 (FETCH_SIZE + WRITE_SIZE,
    each scaled by the same counter's reading for a plain copy of known size) on this
    workload, averaged over every launch of one step; None unless the committed record exists
    for this workload and was taken on the current attention source."""
    path = os.path.join(ROOT, "profiles", f"k_attend_memory_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"```traffic-record\n(.*?)```", text, re.S)
    if not m:
        return None
    rec = dict(line.split(": ", 1) for line in m.group(1).strip().splitlines())
    csrc = os.path.join(ROOT, "stateful_decoding_amd", "csrc")
    h = hashlib.sha256()
    for name in ("attention.hip", "internal.h", "common.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    if rec.get("workload") != workload or rec.get("source_sha256_16") != h.hexdigest()[:16]:
        return None
    return int(rec["traffic_per_launch"])


def cpu_baseline(cfg, params, budget_s: float, n_seqs: int = 16) -> dict:
    """The float64 oracle as it stands, on the first n_seqs sequences, token by token from
    t = 1 until the time budget is used (memory projection of those tokens included)."""
    import numpy as np

    import oracle
    from synth import make_encoder_outputs
    try:
        from threadpoolctl import threadpool_info
        threads = max(i["num_threads"] for i in threadpool_info()) or 1
    except Exception:  # pragma: no cover
        threads = 1
    T = cfg.seq_len
    e = make_encoder_outputs(cfg, range(n_seqs)).astype(np.float64)
    t0 = time.perf_counter()
    p = oracle.prepare_params(params)
    t_prep = time.perf_counter() - t0
    t0 = time.perf_counter()
    km, vm = oracle.memory_projection(p, e)
    t_mem = time.perf_counter() - t0
    st = oracle.init_state(p, cfg, n_seqs)
    t0 = time.perf_counter()
    n = 0
    while n < T and (n == 0 or time.perf_counter() - t0 + t_mem * (n + 1) / T < budget_s):
        oracle.decoder_step(p, cfg, st, km, vm, e[:, n])
        n += 1
    wall = time.perf_counter() - t0 + t_mem * n / T  # projection of the n tokens used
    return {"value": n_seqs * n / wall, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"float64 NumPy oracle, first {n_seqs} sequences, tokens 1..{n} of {T} "
                      f"(memory projection pro rata), {wall:.1f} s; early tokens have short "
                      "memory prefixes, so this overstates the oracle's whole-run rate",
            "host_cpus": len(os.sched_getaffinity(0)), "param_prep_s": round(t_prep, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--mode", choices=("recurrent", "parallel", "train", "ragged", "head"),
                    default="recurrent",
                    help="recurrent: rlt_run_sequence (the headline); parallel: the token-parallel "
                         "pass for alpha = 0 (rlt_run_parallel); train: forward + "
                         "backpropagation through time (rlt_bptt); ragged: ready updates "
                         "(rlt_decoder_step_ragged) with a random 75%% of sequences ready per step; "
                         "head: the causal encoder over the prompt (rlt_encode) and the readout "
                         "with sampling (rlt_readout)")
    ap.add_argument("--workload", default=None,
                    help="synth.CONFIGS name (default s140m_bf16, or long_a0_bf16 in parallel mode)")
    ap.add_argument("--seq-len", type=int, default=0,
                    help="tokens per sequence (default: the workload's); for short profiling "
                         "runs only, the headline is the workload's length")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-stride", type=int, default=0,
                    help="time the memory-attention launches of every N-th token (default: "
                         "every token, or every 16th when the attention is split); the launches "
                         "time themselves by the GPU clock, with nothing queued around them")
    ap.add_argument("--copy-calibration", type=int, metavar="MIB", default=0,
                    help="only run 5 plain device copies of MIB MiB (fp32) and exit: the known-size "
                         "kernel that scales the HBM byte counters of a profiler")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}): decoding shards over independent sequences with no exchange, so the "
              "multi-GPU figure is N times the one-GPU figure at B/N sequences per GPU; it is "
              "not run here.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = args.copy_calibration * 2**20 // 4
        src = torch.empty(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"launches": 5, "read_bytes": 4 * n,
                                               "write_bytes": 4 * n}}), flush=True)
        return

    import stateful_decoding_amd as sd
    from synth import CONFIGS, make_encoder_outputs, make_params

    if args.workload is None:
        args.workload = "long_a0_bf16" if args.mode == "parallel" else "s140m_bf16"
    cfg = CONFIGS[args.workload]
    if args.seq_len:
        cfg = cfg.replace(seq_len=args.seq_len)
    B, T = cfg.batch, cfg.seq_len
    torch.cuda.set_device(0)
    dev = "cuda"
    print(f"[bench] workload {cfg.name}: B={B} T={T} d={cfg.d} L={cfg.n_layers} W={cfg.window} "
          f"G={cfg.n_groups}", file=sys.stderr, flush=True)
    params = make_params(cfg)
    e_host = make_encoder_outputs(cfg, range(B))
    c = sd.make_config(cfg)
    model = sd.Model(c, sd.upload_weights(params, c, dev))
    e = torch.from_numpy(e_host).to(dev, model.dtype).contiguous()
    del e_host
    state = sd.State(model, B)
    mem = sd.Memory(model, B, T)
    traj = torch.empty(B, T, cfg.d, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    if args.mode == "parallel":
        return bench_parallel(args, cfg, params, model, state, mem, e, traj, stream)
    if args.mode == "train":
        del state, mem
        return bench_train(args, cfg, params, model, e, traj, stream)
    if args.mode == "ragged":
        return bench_ragged(args, cfg, params, model, state, mem, e, stream)
    if args.mode == "head":
        del state, mem, e, traj
        return bench_head(args, cfg, params, model, stream)

    def one_step():
        state.reset(stream)
        mem.reset()
        sd.rlt_run_sequence(model, state, mem, e, traj, stream)

    for i in range(args.warmup):
        one_step()
        torch.cuda.synchronize()
        print(f"[bench] warmup {i + 1}/{args.warmup} done", file=sys.stderr, flush=True)

    # one clock slot pair per workgroup (sequence, head, and slice of the prefix when fewer
    # than 128 sequence-head pairs split it into up to 16) of every timed memory attention
    per_bh = 1 if B * cfg.n_heads >= 128 else 16
    stride = args.profile_stride or (1 if per_bh == 1 else 16)
    timed_tokens = (T + stride - 1) // stride
    state.profile_clock(args.steps * timed_tokens * cfg.n_layers * B * cfg.n_heads * per_bh)
    state.profile_begin(["cross_attn", "memproj"], token_stride=stride)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        one_step()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = start.elapsed_time(stop)
    prof = state.profile_end()
    assert bool(torch.isfinite(traj).all()), "non-finite decoder output"
    print(f"[bench] timed {args.steps} steps: {ms_total:.1f} ms (host wall {wall:.2f} s)",
          file=sys.stderr, flush=True)

    secs = ms_total / 1e3
    value = B * T * args.steps / secs
    ideal = step_roofline_seconds(cfg, B, T)
    ca = prof["cross_attn"]
    achieved = ca["bytes"] / (ca["total_ms"] / 1e3)
    # the record averages over every launch of a step, so it applies when every token is timed
    traffic = traffic_record(cfg.name) if stride == 1 else None
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_total / args.steps, 2), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "seq_len": T, "d": cfg.d,
                   "heads": cfg.n_heads, "head_dim": cfg.head_dim, "decoder_blocks": cfg.n_layers,
                   "ffn": cfg.ffn, "window": cfg.window, "memory_groups": cfg.n_groups,
                   "alpha": cfg.alpha, "inputs": "e_t ~ N(0,1), weights ~ N(0,0.02), seed 0"},
        "roofline": {"bound": "hbm", "kernel": "k_attend_memory (cross-attention over memory 1..t)",
                     "achieved": round(achieved / 1e9, 1), "peak": HBM_PEAK / 1e9,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK, 4),
                     "traffic": traffic,
                     "launches": ca["launches"],
                     "avg_launch_us": round(ca["total_ms"] * 1e3 / ca["launches"], 2),
                     "bytes_per_launch": round(ca["bytes"] / ca["launches"]),
                     "timed": f"every launch in the steps of tokens t with t % "
                              f"{stride} == 0 (all layers and row groups), each "
                              f"by the kernel's own clock stamps: first wave's start to last "
                              f"wave's end"},
        "step_roofline": {"ideal_s": round(ideal, 4), "measured_s": round(secs / args.steps, 4),
                          "frac": round(ideal / (secs / args.steps), 4),
                          "peaks": "HBM 8.0 TB/s, bf16 MFMA 2.5 PFLOP/s"},
        "memproj_ms": round(prof["memproj"]["total_ms"] / args.steps, 2),
    }
    if cfg.n_groups == 1 and cfg.n_layers > 1:
        # one memory shared by every layer: also against the floor where it is read once a step
        once = step_roofline_seconds(cfg, B, T, memory_once=True)
        out["step_roofline"]["ideal_memory_once_s"] = round(once, 4)
        out["step_roofline"]["frac_memory_once"] = round(once / (secs / args.steps), 4)
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, params, args.cpu_seconds)
    print(json.dumps(out), flush=True)


PAR_KINDS = ("par_gemm", "par_self_attn", "par_cross_attn", "par_other", "memproj")


def bench_parallel(args, cfg, params, model, state, mem, e, traj, stream):
    """The token-parallel pass for alpha = 0: one step is one rlt_run_parallel (memory
    projection + all layers over all B x T tokens) on a reset state and emptied memory."""
    import torch

    import stateful_decoding_amd as sd

    if cfg.alpha != 0.0:
        sys.exit(f"--mode parallel needs an alpha = 0 workload ({cfg.name} has {cfg.alpha})")
    B, T = cfg.batch, cfg.seq_len
    ws = sd.parallel_workspace(model, B, T)

    def one_step():
        state.reset(stream)
        mem.reset()
        sd.rlt_run_parallel(model, state, mem, e, traj, ws, stream)

    for i in range(args.warmup):
        one_step()
        torch.cuda.synchronize()
        print(f"[bench] warmup {i + 1}/{args.warmup} done", file=sys.stderr, flush=True)
    state.profile_begin(list(PAR_KINDS))
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        one_step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    prof = state.profile_end()
    assert bool(torch.isfinite(traj).all()), "non-finite decoder output"
    secs = ms_total / 1e3
    # per kind: ideal time at the HBM or MFMA peak, whichever binds
    ideal = 0.0
    for v in prof.values():
        ideal += max(v["bytes"] / HBM_PEAK, v["flops"] / BF16_PEAK) / args.steps
    dom_name, dom = max(prof.items(), key=lambda kv: kv[1]["total_ms"])
    mfma = dom["flops"] / BF16_PEAK > dom["bytes"] / HBM_PEAK
    rate = (dom["flops"] if mfma else dom["bytes"]) / (dom["total_ms"] / 1e3)
    peak = BF16_PEAK if mfma else HBM_PEAK
    kern = {"par_gemm": "k_gemm_big (all projections)", "par_cross_attn": "k_flash (memory prefix)",
            "par_self_attn": "k_flash (window)", "par_other": "k_norm_rows, k_row_rinv / hand-off",
            "memproj": "k_gemm_big (memory projection)"}[dom_name]
    out = {
        "metric": "RLT token-parallel decoder pass at alpha = 0, tokens/sec (B seqs x T) on 1 "
                  "MI355X; % of the pass roofline",
        "value": round(B * T * args.steps / secs, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_total / args.steps, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "mode": "parallel", "batch": B, "seq_len": T, "d": cfg.d,
                   "heads": cfg.n_heads, "head_dim": cfg.head_dim, "decoder_blocks": cfg.n_layers,
                   "ffn": cfg.ffn, "window": cfg.window, "memory_groups": cfg.n_groups,
                   "alpha": cfg.alpha, "inputs": "e_t ~ N(0,1), weights ~ N(0,0.02), seed 0"},
        "roofline": {"bound": "mfma" if mfma else "hbm", "kernel": kern,
                     "achieved": round(rate / 1e12, 1) if mfma else round(rate / 1e9, 1),
                     "peak": (BF16_PEAK / 1e12) if mfma else (HBM_PEAK / 1e9),
                     "unit": "TFLOP/s" if mfma else "GB/s", "frac": round(rate / peak, 4),
                     "traffic": None, "launches": dom["launches"],
                     "avg_launch_us": round(dom["total_ms"] * 1e3 / dom["launches"], 2)},
        "step_roofline": {"ideal_s": round(ideal, 5), "measured_s": round(secs / args.steps, 5),
                          "frac": round(ideal / (secs / args.steps), 4),
                          "peaks": "HBM 8.0 TB/s, bf16 MFMA 2.5 PFLOP/s, per kernel kind"},
        "kernel_ms_per_step": {k: round(v["total_ms"] / args.steps, 2) for k, v in prof.items()},
    }
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, params, args.cpu_seconds, n_seqs=4)
    print(json.dumps(out), flush=True)


def bench_ragged(args, cfg, params, model, state, mem, e, stream, ready: float = 0.75):
    """Ragged ready updates: one step is the memory projection of all T tokens, then T decoder
    steps in which each sequence is ready with probability `ready` (seeded masks) and, when
    ready, consumes its own next token at its own position. value = tokens actually advanced
    per second. The roofline's bytes are counted on the host from the known positions: every
    row of a launch reads its own memory prefix (rows that are not ready compute along)."""
    import numpy as np
    import torch

    import stateful_decoding_amd as sd

    B, T, d, L = cfg.batch, cfg.seq_len, cfg.d, cfg.n_layers
    es = 2 if cfg.dtype == "bf16" else 4
    rng = np.random.default_rng(0)
    masks = rng.random((T, B)) < ready
    pos = np.zeros(B, np.int64)
    rows = np.empty((T, B), np.int64)
    before = np.empty((T, B), np.int64)
    for s_ in range(T):
        before[s_] = pos
        rows[s_] = np.arange(B) * T + np.minimum(pos, T - 1)
        pos += masks[s_]
    advanced = int(masks.sum())
    e_steps = e.view(B * T, d)[torch.from_numpy(rows.reshape(-1)).to(e.device)].view(T, B, d)
    e_steps = e_steps.contiguous()
    masks_d = torch.from_numpy(masks.astype(np.uint8)).to(e.device).contiguous()

    def one_step():
        state.reset(stream)
        mem.reset()
        sd.rlt_memproj(model, mem, e, 0, stream)
        for s_ in range(T):
            sd.rlt_decoder_step_ragged(model, state, mem, e_steps[s_], masks_d[s_], None, stream)

    for i in range(args.warmup):
        one_step()
        torch.cuda.synchronize()
        print(f"[bench] warmup {i + 1}/{args.warmup} done", file=sys.stderr, flush=True)
    stride = args.profile_stride or 1
    per_bh = 1 if B * cfg.n_heads >= 128 else 16
    state.profile_clock(args.steps * ((T + stride - 1) // stride) * L * B * cfg.n_heads * per_bh)
    state.profile_begin(["cross_attn"], token_stride=stride)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        one_step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    prof = state.profile_end()
    assert state.positions() == pos.tolist(), "positions differ from the schedule"
    secs = ms_total / 1e3
    ca = prof["cross_attn"]
    sampled = [s_ for s_ in range(T) if s_ % stride == 0]
    by = sum(L * (float((before[s_] + 1).sum()) * 2 * d * es + B * d * (4 + es))
             for s_ in sampled) * args.steps
    achieved = by / (ca["total_ms"] / 1e3)
    out = {
        "metric": "RLT decoder ragged ready updates, tokens advanced/sec (B seqs, T steps, 75% "
                  "ready per step) on 1 MI355X",
        "value": round(advanced * args.steps / secs, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_total / args.steps, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "mode": "ragged", "batch": B, "steps": T,
                   "ready_fraction": ready, "tokens_advanced": advanced, "d": d,
                   "decoder_blocks": L, "window": cfg.window, "memory_groups": cfg.n_groups,
                   "inputs": "e_t ~ N(0,1), weights ~ N(0,0.02), ready masks Bernoulli(0.75), "
                             "seed 0"},
        "roofline": {"bound": "hbm", "kernel": "k_attend_memory (cross-attention, per-row "
                                               "prefixes)",
                     "achieved": round(achieved / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK, 4), "traffic": None,
                     "launches": ca["launches"],
                     "avg_launch_us": round(ca["total_ms"] * 1e3 / ca["launches"], 2),
                     "timed": f"every launch in the steps s with s % {stride} == 0, "
                              f"by the kernel's own clock stamps"},
    }
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline ...", file=sys.stderr, flush=True)
        cb = cpu_baseline(cfg, params, args.cpu_seconds)
        cb["sample"] += "; the oracle steps each sequence alone, so readiness does not change its rate"
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


LOSS_SCALE = 2.0 ** -100
TRAIN_KINDS = ("gate", "qkv", "self_attn", "self_out", "cross_q", "cross_attn", "cross_out",
               "ffn_up", "ffn_down", "memproj", "bwd_proj", "bwd_self_attn", "bwd_cross_attn",
               "bwd_memory", "bwd_wgrad", "bwd_other")
TRAIN_KERNEL = "k_xattn_back (memory-prefix attention backward)"


def cpu_baseline_train(cfg, params, budget_s: float, n_seqs: int = 2) -> dict:
    """The float64 oracle's forward + backward (oracle.bptt) as it stands, on the first n_seqs
    sequences and the first n tokens, n doubling from 8 while a run stays within the budget."""
    import numpy as np

    import oracle
    from synth import make_encoder_outputs
    try:
        from threadpoolctl import threadpool_info
        threads = max(i["num_threads"] for i in threadpool_info()) or 1
    except Exception:  # pragma: no cover
        threads = 1
    p = oracle.prepare_params(params)
    e = make_encoder_outputs(cfg, range(n_seqs)).astype(np.float64)
    G = np.random.default_rng(0).standard_normal(e.shape)
    n, wall = 8, 0.0
    while True:
        t0 = time.perf_counter()
        oracle.bptt(p, cfg, e[:, :n], G[:, :n])
        wall = time.perf_counter() - t0
        if n >= cfg.seq_len or wall * 2.5 > budget_s:
            break
        n = min(cfg.seq_len, 2 * n)
    return {"value": n_seqs * n / wall, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"float64 NumPy oracle.bptt (forward + reverse walk), first {n_seqs} "
                      f"sequences, tokens 1..{n} of {cfg.seq_len}, {wall:.1f} s; short prefixes "
                      "overstate the whole-run rate",
            "host_cpus": len(os.sched_getaffinity(0))}


def encoder_flops(cfg, B: int, n: int) -> float:
    """Algorithmic flops of the encoder over n tokens of B sequences: per token and block the
    q/k/v/o, up and down products and causal attention over positions 1..t."""
    d, L, F = cfg.d, cfg.n_layers, cfg.ffn
    per_token = 2 * (4 * d * d + 3 * d * F)
    attn = 4 * d * (n * (n + 1) / 2)  # scores and weighted values, all positions of a sequence
    return L * B * (n * per_token + attn)


def bench_head(args, cfg, params, model, stream):
    """One step: the encoder over the whole prompt (B x T token ids) and one readout with
    sampling of B rows. value = prompt tokens encoded per second."""
    import numpy as np
    import torch

    import stateful_decoding_amd as sd
    from synth import VOCAB, make_head_params, make_tokens, make_uniforms

    B, T, V = cfg.batch, cfg.seq_len, VOCAB
    head = sd.Head(model, V, sd.upload_head_weights(make_head_params(cfg, V), model.cfg))
    tok = torch.from_numpy(make_tokens(range(B), T, V)).cuda()
    e = torch.empty(B, T, cfg.d, dtype=model.dtype, device="cuda")
    ws = torch.empty(model.lib.rlt_encode_ws_bytes(sd.binding.byref(model.cfg), B, T),
                     dtype=torch.uint8, device="cuda")
    s = torch.randn(B, cfg.d, device="cuda", generator=torch.Generator("cuda").manual_seed(0))
    u = torch.from_numpy(make_uniforms(B)).cuda()
    rws = sd.readout_workspace(head, B)
    lg = torch.empty(B, V, device="cuda")

    def encode():
        sd.rlt_encode(head, tok, e, ws, stream)

    def readout():
        return sd.rlt_readout(head, s, u, 0.8, 50, 0.95, logits=lg, ws=rws, stream=stream)

    for _ in range(args.warmup):
        encode()
        readout()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(args.steps):
        encode()
    b.record(stream)
    torch.cuda.synchronize()
    enc_ms = a.elapsed_time(b) / args.steps
    reps = 20
    # the GPU first spins for a few milliseconds while the host enqueues every timed readout,
    # so the events time the readouts back to back on the GPU, not the binding's host cost
    torch.cuda._sleep(int(2e7))
    a.record(stream)
    for _ in range(reps * args.steps):
        readout()
    b.record(stream)
    torch.cuda.synchronize()
    ro_us = a.elapsed_time(b) * 1e3 / (reps * args.steps)
    assert bool(torch.isfinite(e.float()).all()), "non-finite encoder output"
    fl = encoder_flops(cfg, B, T)
    ro_bytes = 2 * V * cfg.d + B * V * 4 + B * cfg.d * 4  # W_out once, logits written once
    out = {
        "metric": "RLT causal encoder prompt tokens/sec (B seqs x T) on 1 MI355X",
        "value": round(B * T / (enc_ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(enc_ms, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "mode": "head", "batch": B, "seq_len": T,
                   "vocab": V, "d": cfg.d, "encoder_blocks": cfg.n_layers,
                   "inputs": "token ids uniform over the vocabulary, weights ~ N(0,0.02), seed 0"},
        "roofline": {"bound": "mfma", "kernel": "whole encoder pass",
                     "achieved": round(fl / (enc_ms / 1e3) / 1e12, 1),
                     "peak": BF16_PEAK / 1e12, "unit": "TFLOP/s",
                     "frac": round(fl / (enc_ms / 1e3) / BF16_PEAK, 4), "traffic": None},
        "readout": {"us_per_call": round(ro_us, 1), "rows": B, "vocab": V,
                    "sampling": "temperature 0.8, top-k 50, top-p 0.95",
                    "hbm_bound_us": round(ro_bytes / HBM_PEAK * 1e6, 2)},
    }
    print(json.dumps(out), flush=True)


def bench_train(args, cfg, params, model, e, traj, stream):
    """Forward + backpropagation through time: one step is one rlt_bptt over all B x T tokens
    (memory projection, the recurrent forward keeping what the walk needs, the reverse walk,
    weight and memory gradients) for seeded N(0, 1) upstream gradients of every s_t."""
    import torch

    import stateful_decoding_amd as sd

    B, T, d = cfg.batch, cfg.seq_len, cfg.d
    ws = sd.bptt_workspace(model, B, T)
    grads = sd.grad_buffers(model)
    gen = torch.Generator(device="cuda").manual_seed(0)
    # Loss scaling: this random-init model's backward grows about 1.1x per token, beyond fp32
    # over 1024 tokens at unit scale; the walk is linear in ds, so the scale changes no work.
    ds = torch.randn(B, T, d, device="cuda", generator=gen, dtype=torch.float32) * LOSS_SCALE
    de = torch.empty(B, T, d, device="cuda", dtype=torch.float32)
    print(f"[bench] train workspace {ws.numel() / 2**30:.1f} GiB", file=sys.stderr, flush=True)

    # the memory-prefix attention backward (the largest kernel of the pass) times itself by
    # clock stamps: one slot pair per workgroup (sequence, head) of every launch
    clock = sd.clock_buffer(T * cfg.n_layers * B * cfg.n_heads)

    def one_step(kernels=None, clk=None):
        return sd.rlt_bptt(model, e, ds, grads, de=de, s_traj=traj, ws=ws, stream=stream,
                           time_kernels=kernels, token_stride=1, clock=clk)

    for i in range(args.warmup):
        one_step()
        torch.cuda.synchronize()
        print(f"[bench] warmup {i + 1}/{args.warmup} done", file=sys.stderr, flush=True)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        one_step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    secs = ms_total / 1e3
    print(f"[bench] timed {args.steps} steps: {ms_total:.1f} ms", file=sys.stderr, flush=True)
    # one more step in which the memory-prefix attention backward times every launch by its
    # own clock (nothing is queued around the launches, so the schedule is the timed steps';
    # reading the 16 * H bytes of stamps per sequence and launch back to the host after the
    # pass is what keeps it out of the timed steps)
    xb = one_step(["bwd_cross_attn"], clock)["bwd_cross_attn"]
    # and one with every launch timed by events: per-kind breakdown and pass roofline
    prof = one_step(list(TRAIN_KINDS))
    ok = all(bool(torch.isfinite(g).all()) for g in grads.values())
    assert ok and bool(torch.isfinite(de).all()), "non-finite gradients"
    ideal = 0.0
    mm_peak = BF16_PEAK if cfg.dtype == "bf16" else FP32_PEAK
    for k, v in prof.items():
        ideal += max(v["bytes"] / HBM_PEAK, v["flops"] / mm_peak)
    timed = {k: v for k, v in prof.items() if v["launches"]}
    rate = xb["bytes"] / (xb["total_ms"] / 1e3)
    kernel_ms = sum(v["total_ms"] for v in timed.values())
    out = {
        "metric": "RLT decoder training tokens/sec (forward + backpropagation through time, "
                  "B seqs x T) on 1 MI355X; % of the pass roofline",
        "value": round(B * T * args.steps / secs, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_total / args.steps, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "mode": "train", "batch": B, "seq_len": T, "d": d,
                   "heads": cfg.n_heads, "head_dim": cfg.head_dim, "decoder_blocks": cfg.n_layers,
                   "ffn": cfg.ffn, "window": cfg.window, "memory_groups": cfg.n_groups,
                   "alpha": cfg.alpha,
                   "inputs": "e_t ~ N(0,1), weights ~ N(0,0.02), upstream dL/ds_t ~ N(0,1) x 2^-100 "
                             "(loss scaling), seed 0"},
        "roofline": {"bound": "hbm", "kernel": TRAIN_KERNEL,
                     "achieved": round(rate / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(rate / HBM_PEAK, 4), "traffic": None,
                     "launches": xb["launches"],
                     "avg_launch_us": round(xb["total_ms"] * 1e3 / xb["launches"], 2),
                     "bytes_per_launch": round(xb["bytes"] / xb["launches"]),
                     "timed": "every launch of one extra step after the timed steps, each by "
                              "the kernel's own clock stamps: first wave's start to last wave's "
                              "end"},
        "pass_roofline": {"ideal_s": round(ideal, 4), "measured_s": round(secs / args.steps, 4),
                          "frac": round(ideal / (secs / args.steps), 4),
                          "peaks": "HBM 8.0 TB/s, bf16 MFMA 2.5 PFLOP/s, per kernel kind; weights "
                                   "charged once per token over the two row groups",
                          "kernel_sum_s": round(kernel_ms / 1e3, 4)},
        "kernel_ms_per_step": {k: round(v["total_ms"], 1) for k, v in timed.items()},
        "kernel_ms_timing": "HIP events around every launch of one extra step",
    }
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_train(cfg, params, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
