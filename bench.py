#!/usr/bin/env python3
"""Benchmark: the stacked batch-1 decode step of a Gemma-4-26B-A4B-shaped
fine-grained MoE on one MI355X.

A step is one pass of the whole hot path over one batch of M tokens: for each of
30 MoE layers the residual add + RMSNorm, the router GEMV with softmax top-8 of 128,
the union of selected experts, the FP8 gate/up GEMVs with the GELU-tanh gate, the
FP8 down GEMV with the weighted combine and the always-on shared expert; then the
final norm, the tied 262,144-row FP8 lm_head GEMV with argmax, and greedy
acceptance of M-1 draft tokens. M=1 is plain decoding, M=5 the verify step of
speculative decoding with 4 drafts.

Weights (23.8 GB of FP8 experts and lm_head, every expert at its own address) and
all step inputs are seeded synthetic data resident in HBM before timing. The default
path launches the single-kernel step (moe_decode_step) directly, one launch per step
(--path layers captures the per-layer entry points of each step in a HIP graph). W
warm-up steps run, then exactly K steps are timed with HIP events on the launch
stream, bracketed by device synchronisations, as five contiguous blocks: `value` is K
over the whole timed span, and the median of the five blocks' rates is reported
beside it. Bytes per step are the algorithmic bytes of the routing the GPU actually
took (each selected expert counted once per step).

Other configurations, each its own JSON line: --layer (one Gemma-shaped layer at M=1
and its M=5 verify step through the per-layer entry points), --zipf (the stack at M=8
with Zipf-skewed routing, FP8 and bf16 experts), --sample (the M=5 verify step's
lm_head with stochastic acceptance at temperature 0.7).

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, vendor figure
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "fine_grained_moe_router_amd", "csrc")
# the sources each persistent kernel is compiled from, and its hardware-counter summary
STEP_SOURCES = [os.path.join(CSRC, f) for f in ("step.hip", "device_common.h", "handoff.h", "internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_step_traffic.txt")
DRAFT_SOURCES = [os.path.join(CSRC, f) for f in ("draft_fused.hip", "device_common.h", "handoff.h", "internal.h")]
DRAFT_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_draft_fused_traffic.txt")


def source_hash(paths=None):
    """sha256 over a kernel's sources, in a fixed order (the fused step's by default)."""
    import hashlib
    h = hashlib.sha256()
    for path in paths or STEP_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_from(path, sources, key):
    """HBM bytes per launch from a committed hardware-counter summary (FETCH_SIZE and
    WRITE_SIZE in KiB, each from its own rocprofv3 --pmc run, scaled by the factors a plain
    copy of known size gives) for the row named `key`, or None when there is no such row or
    the kernel's sources have changed since the counters were taken."""
    if not os.path.exists(path):
        return None
    sha, scale, rows = None, {}, {}
    for line in open(path):
        f = line.split()
        if not f or f[0].startswith("#"):
            continue
        if f[0] == "source_sha256":
            sha = f[1]
        elif f[0] == "scale":
            scale = dict(kv.split("=") for kv in f[1:])
        elif "=" in f[0]:
            rows[f[0]] = dict(kv.split("=") for kv in f[1:])
    if sha != source_hash(sources) or key not in rows or not scale:
        return None
    r = rows[key]
    return int(float(r["fetch_kib"]) * 1024 * float(scale["fetch"]) + float(r["write_kib"]) * 1024 * float(scale["write"]))


def measured_traffic(M):
    """HBM bytes per k_step launch at M tokens (see traffic_from)."""
    return traffic_from(TRAFFIC_FILE, STEP_SOURCES, "M=%d" % M)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--M", type=str, default="1,5", help="tokens per step; the first is the headline")
    ap.add_argument("--layers", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=8, help="oracle sample: layers per step")
    ap.add_argument("--cpu-steps", type=int, default=40, help="oracle sample: steps")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="only run a plain device-to-device copy of MB megabytes 5 times (a known "
                         "byte count for calibrating hardware traffic counters) and exit")
    ap.add_argument("--layer", action="store_true",
                    help="the one-layer configurations instead, through the per-layer entry points: "
                         "a Gemma-shaped MoE layer at M=1, and at M=5 followed by the lm_head, argmax "
                         "and acceptance; --steps fresh inputs each (its own JSON line)")
    ap.add_argument("--layer-configs", type=str, default="m1,m5,m1em",
                    help="--layer: which of m1 (M=1), m5 (M=5 + lm_head + accept), m1em (M=1, expert-major "
                         "router) to run")
    ap.add_argument("--copies", type=int, default=8,
                    help="--layer: weight copies rotated step by step, so that an expert's reuse "
                         "distance exceeds the Infinity Cache")
    ap.add_argument("--zipf", action="store_true",
                    help="the skewed-routing configuration instead: the stack at M=8 with a Zipf(1.1) "
                         "router bias, once with FP8 and once with bf16 expert weights (its own JSON line)")
    ap.add_argument("--sample", action="store_true",
                    help="the verify step's lm_head with stochastic acceptance instead (lm_head_spec_sample, "
                         "M=5, temperature 0.7, 2 rotated lm_head copies; its own JSON line)")
    ap.add_argument("--draft", action="store_true",
                    help="the MTP drafter step instead (moe_draft_step, 4 drafts of the 430M head), timed beside the "
                         "fused verify step, with the drafter tax and modelled tokens/s (its own JSON line)")
    ap.add_argument("--attn", action="store_true",
                    help="the attention half of the decode step instead (moe_attn_decode over the 30 layers, 25 "
                         "sliding + 5 global, with a KV cache) at several contexts, M=1 and M=5, bf16 and FP8 KV "
                         "caches (its own JSON line)")
    ap.add_argument("--ladder", action="store_true",
                    help="the precision ladder instead: the stack at M=1 and M=5 for FP8/bf16 experts x FP8/bf16 "
                         "lm_head, with tokens/s modelled from the acceptance rate (its own JSON line)")
    ap.add_argument("--path", choices=("fused", "layers"), default="fused",
                    help="fused: one moe_decode_step launch per step; layers: per-layer entry points "
                         "captured in a HIP graph per step")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the decode step is a single-GPU kernel path "
              "(see the sharding notes); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 5}), flush=True)
        return
    if args.zipf:
        return zipf_main(args)
    if args.sample:
        return sample_main(args)
    if args.ladder:
        return ladder_main(args)
    if args.draft:
        return draft_main(args)
    if args.attn:
        return attn_main(args)
    if args.layer:
        return layer_main(args)
    import synth
    from fine_grained_moe_router_amd import budget, native
    from fine_grained_moe_router_amd.stack import DecodeStack, FusedDecodeStep

    native.lib()   # fail loudly if the HIP library is missing
    dev = "cuda"
    Ms = [int(m) for m in args.M.split(",")]
    sh = synth.GEMMA4_26B_A4B.with_(layers=args.layers)
    K, W = args.steps, args.warmup

    t0 = time.time()
    layers = [synth.layer_weights(sh, l, dev, seed=args.seed, tag="stack") for l in range(sh.layers)]
    gains = synth.rmsnorm_gains(sh, dev, seed=args.seed)
    Q, s = synth.lm_head(sh, dev, seed=args.seed)
    torch.cuda.synchronize()
    log("weights generated in %.1fs (%.2f GB resident)" % (time.time() - t0, torch.cuda.memory_allocated() / 1e9))
    if args.path == "fused":
        runner = FusedDecodeStep(sh, layers, gains, Q, s, max_M=max(Ms))
    else:
        runner = DecodeStack(sh, layers, gains, Q, s, max_M=max(Ms))

    results = {M: measure(args, runner, sh, M) for M in Ms}

    M0 = Ms[0]
    head = results[M0]
    if args.path == "fused":
        # the step is one kernel launch: its average duration over the timed region
        roofline = {"bound": "hbm", "kernel": "k_step (moe_decode_step, M=%d)" % M0,
                    "achieved": round(head["hbm_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(head["hbm_frac"], 4), "traffic": measured_traffic(M0),
                    "bytes_per_launch": int(head["bytes_per_step"]),
                    "avg_launch_us": round(head["ms_per_step"] * 1e3, 2)}
    else:
        # the largest single launch of the per-layer path, timed alone with HIP events
        lm_bytes = budget.lm_head_bytes(sh.vocab, sh.hidden)
        xs_lm = [synth.hidden_inputs(sh, M0, i, device=dev, tag="bench_lm") for i in range(8)]
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            for i in range(3):
                native.lm_head_argmax(M0, sh.hidden, sh.vocab, xs_lm[i % 8], Q, s, runner.tok[:M0],
                                      runner.max_logit[:M0], runner.lm_ws, runner.lm_ws_bytes)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(K):
                native.lm_head_argmax(M0, sh.hidden, sh.vocab, xs_lm[i % 8], Q, s, runner.tok[:M0],
                                      runner.max_logit[:M0], runner.lm_ws, runner.lm_ws_bytes)
            e1.record(stream)
            torch.cuda.synchronize()
        lm_ms = e0.elapsed_time(e1) / K
        lm_gbs = lm_bytes / (lm_ms / 1e3) / 1e9
        roofline = {"bound": "hbm", "kernel": "k_lmhead (lm_head_argmax, M=%d)" % M0,
                    "achieved": round(lm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(lm_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                    "bytes_per_launch": lm_bytes, "avg_launch_us": round(lm_ms * 1e3, 2)}
        log("lm_head alone: %.1f us, %.1f GB/s" % (lm_ms * 1e3, lm_gbs))

    probe = read_probe()
    log("HBM read probe: %.1f GB/s over %.1f GiB (%.1f%% of 8 TB/s)" % (
        probe["read_gbs"], probe["bytes"] / 2 ** 30, 100 * probe["read_gbs"] / HBM_PEAK_GBS))
    roofline["frac_of_probe"] = round(roofline["achieved"] / probe["read_gbs"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, sh, layers, gains, Q, s, Ms[0])

    line = {
        "metric": "decode steps/s + achieved HBM GB/s (% peak), 26B-A4B MoE stack, M=1 & M=5",
        "value": round(head["steps_per_s"], 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 weights x bf16 activations, fp32 accumulate",
        "data": "synthetic (seeded N(0,.) weights quantised to FP8 E4M3FN, N(0,1) inputs)",
        "config": {"workload": "Gemma-4-26B-A4B-shaped MoE stack: 30 layers x (router 2816x128 bf16, "
                               "top-8 of 128 + shared expert, width 704, FP8) + tied 262144x2816 FP8 "
                               "lm_head + argmax + greedy accept, M=%d tokens/step" % Ms[0],
                   "path": args.path,
                   "M": Ms[0], "layers": sh.layers, "hidden": sh.hidden, "experts": sh.experts,
                   "top_k": sh.top_k, "expert_width": sh.width, "vocab": sh.vocab},
        "hbm_gbs": round(head["hbm_gbs"], 1),
        "hbm_frac": round(head["hbm_frac"], 4),
        "bytes_per_step": int(head["bytes_per_step"]),
        "p50_ms": round(head["p50_ms"], 4),
        "p99_ms": round(head["p99_ms"], 4),
        "per_M": {str(M): {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
                  for M, r in results.items()},
        "roofline": roofline,
        "hbm_probe": probe,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def read_probe(nbytes=4 << 30, reps=10):
    """The practical HBM ceiling beside the nominal peak: the library's streaming-read
    probe (moe_hbm_read_probe) over nbytes of device memory, HIP-event-timed on its stream."""
    import torch
    from fine_grained_moe_router_amd import native
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(native.PROBE_GRID, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for _ in range(3):
            native.moe_hbm_read_probe(src, nbytes, sink, stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            native.moe_hbm_read_probe(src, nbytes, sink, stream)
        e1.record(stream)
        torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    del src, sink
    torch.cuda.empty_cache()
    return {"kernel": "moe_hbm_read_probe", "bytes": nbytes, "avg_launch_us": round(us, 2),
            "read_gbs": round(nbytes / (us / 1e6) / 1e9, 1)}


def measure(args, runner, sh, M, expert_dtype="fp8", bias=False, lm_dtype="fp8", router_dtype="bf16"):
    """Warm up, then time exactly args.steps steps of the runner at M tokens (HIP events
    on the launch stream, bracketed by device synchronisations); then record each timed
    step's routing to count the bytes it needed."""
    import torch
    import synth
    from fine_grained_moe_router_amd import budget, native
    dev = "cuda"
    K, W = args.steps, args.warmup
    n = K + W
    xs = [synth.hidden_inputs(sh, M, i, device=dev, seed=args.seed, tag="bench_x") for i in range(n)]
    noises = [synth.stack_noise(sh, M, i, device=dev, seed=args.seed) for i in range(n)]
    g = torch.Generator().manual_seed(synth.seed_of(args.seed, "bench_drafts", M))
    drafts = [torch.randint(0, sh.vocab, (max(M - 1, 1),), generator=g, dtype=torch.int32).to(dev)
              for _ in range(n)]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    if args.path == "fused":
        def launch(i, outputs=False):
            runner.step(xs[i], noises[i], drafts[i], M, stream=stream, outputs=outputs)
    else:
        graphs = []
        with torch.cuda.stream(stream):
            runner.step(xs[0], noises[0], drafts[0], M)
            torch.cuda.synchronize()
            for i in range(n):
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr, stream=stream):
                    runner.step(xs[i], noises[i], drafts[i], M)
                graphs.append(gr)
        torch.cuda.synchronize()
        log("M=%d: %d step graphs captured" % (M, n))

        def launch(i, outputs=False):
            graphs[i].replay()

    with torch.cuda.stream(stream):
        for i in range(W):
            launch(i)
        torch.cuda.synchronize()
        # exactly K steps, timed as five contiguous blocks (events between blocks do not
        # stall the stream): the whole span gives the rate, the blocks its spread
        bounds = [W + (K * b) // 5 for b in range(6)]
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        w0 = time.perf_counter()
        evs[0].record(stream)
        for b in range(5):
            for i in range(bounds[b], bounds[b + 1]):
                launch(i)
            evs[b + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        ms_total = evs[0].elapsed_time(evs[5])
        block_ms = [evs[b].elapsed_time(evs[b + 1]) / max(1, bounds[b + 1] - bounds[b]) for b in range(5)]

        # per-step latency distribution and the routing each step took
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        ev[0].record(stream)
        for j, i in enumerate(range(W, n)):
            launch(i)
            ev[j + 1].record(stream)
        torch.cuda.synchronize()
        per_step = [ev[j].elapsed_time(ev[j + 1]) for j in range(K)]
        uniq = []
        for i in range(W, n):
            launch(i, outputs=True)
            torch.cuda.synchronize()
            idx = (runner.topk_idx(M) if args.path == "fused" else runner.topk_idx[:, :M]).cpu().numpy()
            uniq.append([len(np.unique(idx[l])) for l in range(sh.layers)])
    if args.path == "fused":
        st_code = runner.status()
        if st_code != native.MOE_OK:
            raise RuntimeError("fused step reported %s" % native.strerror(st_code))

    bytes_steps = [budget.step_bytes(sh, u, M, expert_dtype, bias, lm_dtype, router_dtype) for u in uniq]
    ms = ms_total / K
    bps = float(np.mean(bytes_steps))
    r = {
        "steps_per_s": K / (ms_total / 1e3), "ms_per_step": ms, "wall_s": wall,
        "median_block_ms_per_step": float(np.median(block_ms)), "block_ms_per_step": [round(b, 4) for b in block_ms],
        "p50_ms": float(np.percentile(per_step, 50)), "p99_ms": float(np.percentile(per_step, 99)),
        "bytes_per_step": bps, "hbm_gbs": bps / (ms / 1e3) / 1e9,
        "hbm_frac": bps / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        "mean_unique_experts_per_layer": float(np.mean(uniq)),
    }
    log("M=%d: %.3f ms/step, %.1f steps/s, %.1f GB/s (%.1f%% of 8 TB/s), p50 %.3f p99 %.3f ms" % (
        M, ms, r["steps_per_s"], r["hbm_gbs"], 100 * r["hbm_frac"], r["p50_ms"], r["p99_ms"]))
    if args.path != "fused":
        del graphs
    torch.cuda.synchronize()
    return r


def layer_main(args):
    """The one-layer configurations, through the boundary's per-layer entry points:
    (a) one Gemma-4-26B-A4B-shaped MoE layer at M=1 (moe_decode_layer), and (b) the same
    layer at M=5 followed by lm_head_argmax and spec_accept (the verify step), and (c) (a) with
    the router passed expert-major ([E][H], MOE_ROUTER_EXPERT_MAJOR). Each step
    takes a fresh seeded input; the layer's weights rotate over args.copies copies (8 x
    0.77 GB) and the lm_head over 2, so no step finds its weights in the 256 MB Infinity
    Cache. The timed steps are captured into HIP graphs of 100 steps each (a step is a
    few launches), replayed back to back on one stream and timed with HIP events."""
    import torch
    import synth
    from fine_grained_moe_router_amd import budget, native

    native.lib()   # fail loudly if the HIP library is missing
    dev = "cuda"
    sh = synth.GEMMA4_26B_A4B.with_(layers=1)
    R, K, W = args.copies, args.steps, args.warmup
    desc = native.layer_desc(sh)
    copies = [synth.layer_weights(sh, 0, dev, seed=args.seed + c, tag="layer") for c in range(R)]
    lws = [native.layer_weights(w) for w in copies]
    em_copies = [dict(w, router_w=w["router_w"].t().contiguous()) for w in copies]
    lws_em = [native.layer_weights(w) for w in em_copies]
    desc_em = native.layer_desc(sh, expert_major=True)
    lms = [synth.lm_head(sh, dev, seed=args.seed + c) for c in range(2)]
    torch.cuda.synchronize()
    log("layer copies: %d x %.2f GB, lm_head copies: 2 (%.2f GB resident)" % (
        R, budget.expert_bytes(sh.hidden, sh.width) * sh.experts / 1e9, torch.cuda.memory_allocated() / 1e9))
    out = {}
    configs = {"m1": (1, False, False), "m5": (5, True, False), "m1em": (1, False, True)}
    for M, with_lm, em in [configs[c] for c in args.layer_configs.split(",")]:
        n = K + W
        xs = [synth.hidden_inputs(sh, M, i, device=dev, seed=args.seed, tag="layer_x") for i in range(n)]
        ld, lw = (desc_em, lws_em) if em else (desc, lws)
        wsb = native.moe_decode_layer_workspace(ld, M)
        ws = native.workspace(wsb)
        lwsb = native.lm_head_argmax_workspace(M, sh.hidden, sh.vocab)
        lws_ = native.workspace(lwsb)
        y = torch.empty(M, sh.hidden, dtype=torch.bfloat16, device=dev)
        idx = torch.empty(n, M, sh.top_k, dtype=torch.int32, device=dev)
        wts = torch.empty(M, sh.top_k, dtype=torch.float32, device=dev)
        tok = torch.empty(M, dtype=torch.int32, device=dev)
        acc = torch.empty(4, dtype=torch.int32, device=dev)
        outt = torch.empty(M, dtype=torch.int32, device=dev)
        g = torch.Generator().manual_seed(synth.seed_of(args.seed, "layer_drafts", M))
        drafts = torch.randint(0, sh.vocab, (n, max(M - 1, 1)), generator=g, dtype=torch.int32).to(dev)
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())

        def launch(i):
            native.moe_decode_layer(ld, lw[i % R], M, xs[i], y, idx[i], wts, ws, wsb, stream)
            if with_lm:
                Q, s = lms[i % 2]
                native.lm_head_argmax(M, sh.hidden, sh.vocab, y, Q, s, tok, None, lws_, lwsb, stream)
                native.spec_accept(M - 1, drafts[i], tok, acc, outt, stream)

        with torch.cuda.stream(stream):
            for i in range(W):
                launch(i)
            torch.cuda.synchronize()
            graphs = []
            for c0 in range(W, n, 100):
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr, stream=stream):
                    for i in range(c0, min(n, c0 + 100)):
                        launch(i)
                graphs.append(gr)
            torch.cuda.synchronize()
            graphs[0].replay()   # warm replay
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for gr in graphs:
                gr.replay()
            e1.record(stream)
            torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / K
        del graphs
        ih = idx[W:].cpu().numpy()
        uniq = [len(np.unique(ih[j])) for j in range(K)]
        bps = float(np.mean([budget.layer_bytes(sh, u, M) for u in uniq]))
        if with_lm:
            bps += budget.lm_head_bytes(sh.vocab, sh.hidden) + 16 * M
        name = "verify_m5_lm_head" if with_lm else ("layer_m1_expert_major_router" if em else "layer_m1")
        out[name] = {"us_per_step": round(ms * 1e3, 2), "steps_per_s": round(1e3 / ms, 1),
                     "bytes_per_step": int(bps), "hbm_gbs": round(bps / (ms / 1e3) / 1e9, 1),
                     "hbm_frac": round(bps / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                     "mean_unique_experts": round(float(np.mean(uniq)), 2)}
        log("%s: %.1f us/step, %.1f GB/s (%.1f%% of 8 TB/s), %.2f MB/step, union %.2f" % (
            name, ms * 1e3, out[name]["hbm_gbs"], 100 * out[name]["hbm_frac"], bps / 1e6, np.mean(uniq)))
    head = out["layer_m1"] if "layer_m1" in out else next(iter(out.values()))
    line = {
        "metric": "per-step latency + achieved HBM GB/s, one 26B-A4B MoE layer (M=1) and its verify step "
                  "with lm_head (M=5)",
        "value": head["steps_per_s"], "unit": "steps/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(head["us_per_step"] / 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8 weights x bf16 activations, fp32 accumulate",
        "data": "synthetic (seeded N(0,.) weights quantised to FP8 E4M3FN, N(0,1) inputs), %d layer copies "
                "and 2 lm_head copies rotated" % R,
        "config": {"workload": "one Gemma-4-26B-A4B-shaped MoE layer (router 2816x128, top-8 of 128 + shared, "
                               "width 704, FP8) at M=1; at M=5 + tied 262144x2816 FP8 lm_head + argmax + "
                               "greedy accept", "path": "layers", "hidden": sh.hidden, "experts": sh.experts,
                   "top_k": sh.top_k, "expert_width": sh.width, "vocab": sh.vocab},
        "per_config": out,
        "roofline": {"bound": "hbm", "kernel": "moe_decode_layer (one k_step<1> launch, one-layer mode, M=1)",
                     "achieved": head["hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["hbm_frac"], "traffic": traffic_from(TRAFFIC_FILE, STEP_SOURCES, "layer_M=1"),
                     "bytes_per_launch": head["bytes_per_step"],
                     "avg_launch_us": head["us_per_step"]},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def zipf_main(args):
    """The skewed-routing configuration: the 30-layer stack at M=8 tokens per step with a
    router bias b_e = -1.1 ln(rank_e) (Zipf(1.1) expert popularity), run twice on the
    fused step: FP8 expert weights (5,964,288 B per expert) and bf16 expert weights
    (11,894,784 B per expert, no scales). Reports steps/s, bytes/step and the realised
    union size per layer for each; one JSON line."""
    import torch
    import synth
    from fine_grained_moe_router_amd import native
    from fine_grained_moe_router_amd.stack import FusedDecodeStep

    native.lib()   # fail loudly if the HIP library is missing
    dev = "cuda"
    M = 8
    sh = synth.GEMMA4_26B_A4B.with_(layers=args.layers)
    bias = synth.zipf_router_bias(sh.experts, seed=args.seed)
    gains = synth.rmsnorm_gains(sh, dev, seed=args.seed)
    Q, s = synth.lm_head(sh, dev, seed=args.seed)
    per = {}
    for dt in ("fp8", "bf16"):
        t0 = time.time()
        layers = [synth.layer_weights(sh, l, dev, seed=args.seed, tag="stack", expert_dtype=dt, router_bias=bias)
                  for l in range(sh.layers)]
        torch.cuda.synchronize()
        log("%s experts generated in %.1fs (%.2f GB resident)" % (dt, time.time() - t0,
                                                                 torch.cuda.memory_allocated() / 1e9))
        runner = FusedDecodeStep(sh, layers, gains, Q, s, max_M=M)
        r = measure(args, runner, sh, M, dt, bias=True)
        per[dt] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
        del runner, layers
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    head = per["fp8"]
    line = {
        "metric": "decode steps/s + bytes/step, 26B-A4B MoE stack with Zipf(1.1)-skewed routing, M=8, "
                  "FP8 and bf16 experts",
        "value": round(head["steps_per_s"], 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 (value) and bf16 (per_dtype) expert weights x bf16 activations, fp32 accumulate",
        "data": "synthetic (seeded N(0,.) weights, FP8 E4M3FN or bf16 experts, N(0,1) inputs, Zipf router bias)",
        "config": {"workload": "Gemma-4-26B-A4B-shaped MoE stack, 30 layers, router bias -1.1 ln(rank), "
                               "M=8 tokens/step, + tied 262144x2816 FP8 lm_head + argmax + greedy accept",
                   "path": "fused", "M": M, "layers": sh.layers, "hidden": sh.hidden,
                   "experts": sh.experts, "top_k": sh.top_k, "expert_width": sh.width,
                   "vocab": sh.vocab},
        "bytes_per_step": int(head["bytes_per_step"]),
        "hbm_gbs": round(head["hbm_gbs"], 1),
        "hbm_frac": round(head["hbm_frac"], 4),
        "per_dtype": per,
        "roofline": {"bound": "hbm", "kernel": "k_step (moe_decode_step, M=8, FP8 experts)",
                     "achieved": round(head["hbm_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(head["hbm_frac"], 4), "traffic": None,
                     "bytes_per_launch": int(head["bytes_per_step"]),
                     "avg_launch_us": round(head["ms_per_step"] * 1e3, 2)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def sample_main(args):
    """The verify step's lm_head with stochastic speculative acceptance (lm_head_spec_sample):
    M=5 rows of the Gemma-shaped tied lm_head (262,144 x 2816 FP8) at temperature 0.7, four
    drafts with synthetic drafter distributions q (softmax of seeded N(0,1) logits at the same
    temperature), seeded accept uniforms. The lm_head rotates over 2 copies so that no step
    finds it in the Infinity Cache. Steps are captured into HIP graphs of 100 and replayed."""
    import torch
    import synth
    from fine_grained_moe_router_amd import budget, native

    native.lib()   # fail loudly if the HIP library is missing
    dev = "cuda"
    sh = synth.GEMMA4_26B_A4B
    M, T, K, W = 5, 0.7, args.steps, args.warmup
    H, V, g = sh.hidden, sh.vocab, M - 1
    lms = [synth.lm_head(sh, dev, seed=args.seed + c) for c in range(2)]
    n = K + W
    xs = [synth.hidden_inputs(sh, M, i, device=dev, seed=args.seed, tag="sample_x") for i in range(n)]
    gen = torch.Generator(device=dev).manual_seed(synth.seed_of(args.seed, "sample_q"))
    qs = [torch.softmax(torch.randn(g, V, generator=gen, device=dev) / T, dim=1).contiguous() for _ in range(4)]
    ds = [torch.multinomial(q, 1, generator=gen).view(-1).to(torch.int32).contiguous() for q in qs]
    us = [torch.rand(g, generator=gen, device=dev) for _ in range(n)]
    wsb = native.lm_head_spec_sample_workspace(M, H, V)
    ws = native.workspace(wsb)
    acc = torch.zeros(4, dtype=torch.int32, device=dev)
    out = torch.zeros(M, dtype=torch.int32, device=dev)
    accs = torch.zeros(n, dtype=torch.int32, device=dev)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())

    def launch(i):
        Q, s = lms[i % 2]
        native.lm_head_spec_sample(M, H, V, xs[i], Q, s, T, ds[i % 4], qs[i % 4], us[i], 12345, i, accs[i:i + 1],
                                   out, ws, wsb, stream)

    with torch.cuda.stream(stream):
        for i in range(W):
            launch(i)
        torch.cuda.synchronize()
        graphs = []
        for c0 in range(W, n, 100):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=stream):
                for i in range(c0, min(n, c0 + 100)):
                    launch(i)
            graphs.append(gr)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for gr in graphs:
            gr.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    mean_acc = float(accs[W:].float().mean())
    # algorithmic bytes: the lm_head, the M input rows, the drafter row the draw reads (V fp32)
    # and the drafted ids' probabilities and uniforms; the logits' round trip through memory
    # (M x V fp32 written, one row read back) is this implementation's, not the method's
    bps = budget.lm_head_bytes(V, H) + M * H * 2 + V * 4 + g * 12 + 4 * M
    gbs = bps / (ms / 1e3) / 1e9
    log("sample M=5: %.1f us/step, %.1f GB/s (%.1f%% of 8 TB/s), mean accepted %.2f" % (
        ms * 1e3, gbs, 100 * gbs / HBM_PEAK_GBS, mean_acc))
    line = {
        "metric": "verify-step lm_head + stochastic speculative acceptance (temperature 0.7), steps/s and HBM GB/s",
        "value": round(1e3 / ms, 2), "unit": "steps/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 weights x bf16 activations, fp32 accumulate and softmax",
        "data": "synthetic (seeded FP8 lm_head, N(0,1) inputs, drafter distributions softmax(N(0,1)/T)), "
                "2 lm_head copies rotated",
        "config": {"workload": "tied 262144x2816 FP8 lm_head over M=5 verify rows + temperature-0.7 softmax + "
                               "accept min(1,p/q) + residual/bonus draw (Gumbel-max, Philox4x32-10)",
                   "M": M, "hidden": H, "vocab": V, "temperature": T},
        "bytes_per_step": int(bps), "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "mean_accepted": round(mean_acc, 3),
        "roofline": {"bound": "hbm", "kernel": "lm_head_spec_sample (k_lmhead<true> + 3 sampling kernels, M=5)",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "bytes_per_launch": int(bps),
                     "avg_launch_us": round(ms * 1e3, 2)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def attn_layer_bytes(sh, M, pos) -> int:
    """Algorithmic bytes of one attention layer call: the q/k/o FP8 weights and row scales, the
    cached key rows the M tokens see (each row once: the union of their windows), the M new key
    rows written, and the M input and output rows."""
    H, NQ, NK, dh = sh.hidden, sh.q_heads * sh.head_dim, sh.kv_heads * sh.head_dim, sh.head_dim
    w = 2 * NQ * H + NK * H + 4 * (NQ + NK + H)
    lo = max(0, pos - sh.window + 1) if sh.window else 0
    row = dh * (1 if sh.kv_fp8 else 2) + (4 if sh.kv_fp8 else 0)
    kv = (pos - lo) * sh.kv_heads * row + M * sh.kv_heads * row
    return w + kv + 2 * M * H * 2


def attn_main(args):
    """The attention half of a decode step (page 'LLM decoding', "The exact architecture" and
    "Where the 7.36 GB goes"): moe_attn_decode for each of the 30 layers (25 sliding-window
    layers of 16 x 256 query heads over 8 KV heads with a 1024-position window, 5 global layers
    of 16 x 512 over 2 KV heads), each on its own weights and KV cache, at contexts of 768
    positions (the page's workload: 512 prompt + 256 generated tokens), 8K and 32K, for M = 1
    and M = 5, with bf16 and with FP8 caches. The caches hold seeded synthetic keys of every
    earlier position; each step appends the same M keys again, so replays do not drift. Steps
    are captured into HIP graphs of 20 and replayed; bytes per step are the weights plus the
    KV rows read (attn_layer_bytes). One global layer is also timed alone (global_layer_us)."""
    import torch
    import synth
    from fine_grained_moe_router_amd import native

    native.lib()   # fail loudly if the HIP library is missing
    dev = "cuda"
    K, W = args.steps, args.warmup
    layers = synth.GEMMA4_ATTN_LAYERS
    weights = [synth.attn_weights(sh, dev, seed=args.seed, layer=l) for l, sh in enumerate(layers)]
    wd = [native.attn_weights(w) for w in weights]
    H = layers[0].hidden
    results = {}
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    for ctx in (768, 8192, 32768):
        for fp8 in (False, True):
            shapes = [sh.with_(kv_fp8=fp8, capacity=(sh.capacity if sh.window else ctx + 8)) for sh in layers]
            descs = [native.attn_desc(sh) for sh in shapes]
            caches = []
            for l, (sh, d) in enumerate(zip(shapes, descs)):
                c = native.workspace(native.moe_kv_cache_bytes(d))
                lo = max(0, ctx - sh.window + 1) if sh.window else 0
                for p0 in range(lo, ctx, 8192):
                    n = min(8192, ctx - p0)
                    native.moe_kv_cache_write(d, p0, n, synth.kv_keys(sh, p0, n, dev, seed=args.seed, layer=l), c)
                caches.append(c)
            torch.cuda.synchronize()
            for M in (1, 5):
                us = [synth.hidden_inputs(synth.GEMMA4_26B_A4B, M, l, device=dev, seed=args.seed, tag="attn_u")
                      for l in range(len(layers))]
                outs = [torch.empty(M, H, dtype=torch.bfloat16, device=dev) for _ in layers]
                wsb = max(native.moe_attn_decode_workspace(d, M) for d in descs)
                ws = native.workspace(wsb)

                def step():
                    for l in range(len(layers)):
                        native.moe_attn_decode(descs[l], wd[l], M, ctx, us[l], caches[l], outs[l], None, ws, wsb,
                                               stream)

                with torch.cuda.stream(stream):
                    for _ in range(W):
                        step()
                    torch.cuda.synchronize()
                    gr = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(gr, stream=stream):
                        for _ in range(20):
                            step()
                    torch.cuda.synchronize()
                    blocks = []
                    reps = max(1, K // 20)
                    for b in range(5):
                        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        for _ in range(reps):
                            gr.replay()
                        e1.record(stream)
                        torch.cuda.synchronize()
                        blocks.append(e0.elapsed_time(e1) / (20 * reps))
                    del gr
                    # one global layer alone, the same way
                    gl = next(l for l, sh in enumerate(shapes) if not sh.window)
                    gr = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(gr, stream=stream):
                        for _ in range(20):
                            native.moe_attn_decode(descs[gl], wd[gl], M, ctx, us[gl], caches[gl], outs[gl], None, ws,
                                                   wsb, stream)
                    torch.cuda.synchronize()
                    gblocks = []
                    for b in range(5):
                        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        for _ in range(reps):
                            gr.replay()
                        e1.record(stream)
                        torch.cuda.synchronize()
                        gblocks.append(e0.elapsed_time(e1) / (20 * reps))
                    del gr
                ms = float(np.median(blocks))
                g_us = float(np.median(gblocks)) * 1e3
                bps = sum(attn_layer_bytes(sh, M, ctx) for sh in shapes)
                gbs = bps / (ms / 1e3) / 1e9
                key = "ctx%d_M%d_%s" % (ctx, M, "fp8kv" if fp8 else "bf16kv")
                results[key] = {"ms_per_step": round(ms, 5), "bytes_per_step": int(bps), "hbm_gbs": round(gbs, 1),
                                "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                                "block_ms_per_step": [round(b, 5) for b in blocks],
                                "global_layer_us": round(g_us, 2)}
                log("attention ctx %5d M=%d %s KV: %.1f us/step (%.1f us/layer), %.1f MB, %.1f GB/s (%.1f%%); "
                    "one global layer %.1f us" % (ctx, M, "FP8 " if fp8 else "bf16", ms * 1e3, ms * 1e3 / 30, bps / 1e6,
                                                  gbs, 100 * gbs / HBM_PEAK_GBS, g_us))
            del caches
            torch.cuda.empty_cache()
    head = results["ctx8192_M1_bf16kv"]
    line = {
        "metric": "attention decode (30 layers: 25 sliding + 5 global, GQA) with a KV cache, steps/s and HBM GB/s",
        "value": round(1e3 / head["ms_per_step"], 2), "unit": "steps/s (8K context, M=1, bf16 KV)", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8 weights x bf16 activations, bf16 or FP8 KV cache, fp32 accumulate",
        "data": "synthetic (seeded FP8 q/k/o projections, N(0,1) cached keys and inputs)",
        "config": {"workload": "moe_attn_decode over the 30 layers of a Gemma-4-26B-A4B-shaped step: 25 sliding "
                               "(16x256 q heads, 8 KV heads, window 1024, ring cache) + 5 global (16x512 q heads, "
                               "2 KV heads); contexts 768 / 8K / 32K, M=1 and M=5, bf16 and FP8 KV",
                   "hidden": H, "layers": len(layers), "params": sum(sh.params() for sh in layers)},
        "per_config": results,
        "fp8_kv_over_bf16_kv_ctx32768_M1": round(results["ctx32768_M1_bf16kv"]["ms_per_step"] /
                                                 results["ctx32768_M1_fp8kv"]["ms_per_step"], 3),
        "roofline": {"bound": "hbm", "kernel": "moe_attn_decode x 30 (4 launches each), 8K context, M=1, bf16 KV",
                     "achieved": head["hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["hbm_frac"], "traffic": None, "bytes_per_launch": head["bytes_per_step"],
                     "avg_launch_us": round(head["ms_per_step"] * 1e3, 2)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def draft_bytes(hs) -> int:
    """Weight bytes one draft reads: the FP8 matrices with their row scales, the gains and the
    target embedding row (the head's 262,144-row table dominates)."""
    D, F, H, V, B = hs.width, hs.ffn, hs.hidden, hs.vocab, hs.blocks
    return ((D * 2 * H + 4 * D) + B * (3 * D * F + 4 * (2 * F + D)) + (B + 1) * D * 2 + (V * D + 4 * V) +
            (H * D + 4 * H) + (H + 4))


def draft_main(args):
    """The MTP drafter's step (moe_draft_step): gamma = 4 drafts of the 430M head, each chained on
    the previous one on the device, graph-captured in groups of 10 steps, in the one-launch form
    (the value) and as the chain of launches (for comparison); timed beside the fused
    verify step (M = 5) and plain decoding (M = 1) of the 30-layer stack in the same process.
    Reports the drafter tax (drafter time / verify time) and tokens/s = E[n+1] / (t_verify +
    t_draft) at acceptance rates from the page (39 % on random prompts, 87 % and 94 % on
    coherent text)."""
    import torch
    import synth
    from fine_grained_moe_router_amd import native
    from fine_grained_moe_router_amd.stack import FusedDecodeStep

    native.lib()   # fail loudly if the HIP library is missing
    dev = "cuda"
    hs, gamma, K, W = synth.MTP_HEAD, 4, args.steps, args.warmup
    sh = synth.GEMMA4_26B_A4B.with_(layers=args.layers)
    head = synth.draft_head(hs, dev, seed=args.seed)
    Q, s = synth.lm_head(sh, dev, seed=args.seed)
    dw = native.draft_weights(head)
    n = K + W
    g0 = [synth.hidden_inputs(sh, 1, i, device=dev, seed=args.seed, tag="draft_g")[0].contiguous() for i in range(n)]
    t0 = torch.randint(0, sh.vocab, (n, 1), generator=torch.Generator().manual_seed(args.seed),
                       dtype=torch.int32).to(dev)
    bpd = draft_bytes(hs)

    def time_form(chain):
        """ms per drafter step of one form: W eager warm-up calls, then K calls replayed from
        graphs of 10 (the drafts of every call kept apart)."""
        desc = native.draft_desc(hs, chain=chain)
        wsb = native.moe_draft_step_workspace(desc)
        ws = native.workspace(wsb)
        drafts = torch.zeros(n, gamma, dtype=torch.int32, device=dev)
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())

        def launch(i):
            native.moe_draft_step(desc, dw, gamma, t0[i], g0[i], Q, s, drafts[i], ws, wsb, stream)

        with torch.cuda.stream(stream):
            for i in range(W):
                launch(i)
            torch.cuda.synchronize()
            graphs = []
            for c0 in range(W, n, 10):
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr, stream=stream):
                    for i in range(c0, min(n, c0 + 10)):
                        launch(i)
                graphs.append(gr)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for gr in graphs:
                gr.replay()
            e1.record(stream)
            torch.cuda.synchronize()
        if native.moe_draft_step_status(desc, ws) != native.MOE_OK:
            raise RuntimeError("drafter: a device-side wait gave up")
        ms = e0.elapsed_time(e1) / K
        del graphs
        log("drafter step, %s (%d drafts): %.1f us (%.1f us per draft), %.1f GB/s over %.1f MB per draft" % (
            "chain of launches" if chain else "one launch", gamma, ms * 1e3, ms * 1e3 / gamma,
            gamma * bpd / (ms / 1e3) / 1e9, bpd / 1e6))
        return ms, drafts

    ms_draft, d_fused = time_form(False)
    ms_chain, d_chain = time_form(True)
    # the two forms differ only in the order of fp32 sums; report how often a draft differs
    differ = int((d_fused[W:] != d_chain[W:]).sum())
    log("drafts that differ between the two forms: %d of %d" % (differ, K * gamma))
    gbs = gamma * bpd / (ms_draft / 1e3) / 1e9
    layers = [synth.layer_weights(sh, l, dev, seed=args.seed, tag="stack") for l in range(sh.layers)]
    gains = synth.rmsnorm_gains(sh, dev, seed=args.seed)
    runner = FusedDecodeStep(sh, layers, gains, Q, s, max_M=5)
    ver = {M: measure(args, runner, sh, M) for M in (1, 5)}
    t1, t5 = ver[1]["ms_per_step"], ver[5]["ms_per_step"]
    model = {}
    for alpha in (0.39, 0.87, 0.94):
        e = expected_emitted(alpha, gamma)
        model["alpha%.2f" % alpha] = {"emitted_per_step": round(e, 3), "tokens_per_s": round(e / ((t5 + ms_draft) / 1e3), 1),
                                      "tokens_per_s_without_drafter": round(e / (t5 / 1e3), 1)}
    line = {
        "metric": "MTP drafter step (4 drafts of a 430M head) and the drafter tax beside the verify step",
        "value": round(1e3 / ms_draft, 2), "unit": "drafter steps/s (4 drafts each)", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_draft, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8 weights x bf16 activations, fp32 accumulate",
        "data": "synthetic (seeded FP8 head: pre_projection 5632->1024, 12 GELU-gated blocks 1024->4096->1024, "
                "own 262144x1024 table, post-projection 1024->2816)",
        "config": {"workload": "MTP drafter, 4 chained drafts per step (embedding row + pre_projection + 12 blocks + "
                               "norm + 262144-row argmax + post-projection each)", "hidden": hs.hidden,
                   "width": hs.width, "ffn": hs.ffn, "blocks": hs.blocks, "vocab": hs.vocab, "params": hs.params()},
        "us_per_draft": round(ms_draft * 1e3 / gamma, 2), "bytes_per_draft": bpd, "hbm_gbs": round(gbs, 1),
        "chain_ms_per_step": round(ms_chain, 5), "chain_us_per_draft": round(ms_chain * 1e3 / gamma, 2),
        "drafts_differing_between_forms": differ,
        "verify_step_ms_M5": round(t5, 4), "plain_step_ms_M1": round(t1, 4),
        "drafter_tax": round(ms_draft / t5, 4),
        "tokens_per_s_plain": round(1e3 / t1, 1),
        "tokens_per_s_spec": model,
        "roofline": {"bound": "hbm", "kernel": "k_draft_fused (one launch per step)", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from(DRAFT_TRAFFIC_FILE, DRAFT_SOURCES, "gamma=%d" % gamma),
                     "bytes_per_launch": gamma * bpd, "avg_launch_us": round(ms_draft * 1e3, 2)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def expected_emitted(alpha, gamma):
    """Tokens emitted per verify step when each draft is accepted with probability alpha
    (prefix acceptance, then the bonus or correction token): sum_{j=0..gamma} alpha^j."""
    return sum(alpha ** j for j in range(gamma + 1))


def ladder_main(args):
    """The precision ladder (page "LLM decoding", "Lever 1: fewer bytes" and the table "The
    ladder, every rung"): the 30-layer stack on the fused step at M=1 (plain decoding) and M=5
    (the verify step with 4 drafts), for FP8 or bf16 expert weights (routed and shared) and
    an FP8 or bf16 lm_head with a bf16 router, and the all-FP8 rung (FP8 router too). Per
    rung: bytes/step and
    steps/s at both M, and tokens/s = steps/s(M=1) for plain decoding and steps/s(M=5) x
    E[n+1] for speculative decoding at the page's acceptance rates (E[n+1] = sum_j alpha^j,
    j = 0..4). The drafter's own cost is not in these figures."""
    import torch
    import synth
    from fine_grained_moe_router_amd import native
    from fine_grained_moe_router_amd.stack import FusedDecodeStep

    native.lib()   # fail loudly if the HIP library is missing
    dev = "cuda"
    sh = synth.GEMMA4_26B_A4B.with_(layers=args.layers)
    gains = synth.rmsnorm_gains(sh, dev, seed=args.seed)
    lm = {"fp8": synth.lm_head(sh, dev, seed=args.seed), "bf16": (synth.lm_head_bf16(sh, dev, seed=args.seed), None)}
    rungs = {}
    for edt in ("bf16", "fp8"):
        t0 = time.time()
        layers = [synth.layer_weights(sh, l, dev, seed=args.seed, tag="stack", expert_dtype=edt)
                  for l in range(sh.layers)]
        torch.cuda.synchronize()
        log("%s experts generated in %.1fs (%.2f GB resident)" % (edt, time.time() - t0,
                                                                 torch.cuda.memory_allocated() / 1e9))
        plan = [("bf16", "bf16"), ("fp8", "bf16")] + ([("fp8", "fp8")] if edt == "fp8" else [])
        for ldt, rdt in plan:
            Q, s = lm[ldt]
            if rdt == "fp8":   # the same layers with the router swapped for its FP8 rung
                layers = [dict(w, **synth.router_weights(sh, l, dev, seed=args.seed, tag="stack", router_dtype="fp8"))
                          for l, w in enumerate(layers)]
            runner = FusedDecodeStep(sh, layers, gains, Q, s, max_M=5)
            r = {}
            for M in (1, 5):
                m = measure(args, runner, sh, M, edt, lm_dtype=ldt, router_dtype=rdt)
                r["M%d" % M] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in m.items()
                                if k in ("steps_per_s", "ms_per_step", "bytes_per_step", "hbm_gbs", "hbm_frac",
                                         "median_block_ms_per_step")}
            r["tokens_per_s_plain"] = round(r["M1"]["steps_per_s"], 1)
            for alpha in (0.87, 0.90):
                r["tokens_per_s_spec_alpha%.2f" % alpha] = round(r["M5"]["steps_per_s"] * expected_emitted(alpha, 4), 1)
            name = "experts_%s+lm_head_%s" % (edt, ldt) + ("+router_fp8" if rdt == "fp8" else "")
            rungs[name] = r
            log("%s: M=1 %.3f ms, M=5 %.3f ms, plain %.0f tok/s, spec(0.87) %.0f tok/s" % (
                name, r["M1"]["ms_per_step"], r["M5"]["ms_per_step"], r["tokens_per_s_plain"],
                r["tokens_per_s_spec_alpha0.87"]))
            del runner
            torch.cuda.synchronize()
        del layers
        torch.cuda.empty_cache()
    top, base = rungs["experts_fp8+lm_head_fp8"], rungs["experts_bf16+lm_head_bf16"]
    line = {
        "metric": "precision ladder: decode steps/s and modelled tokens/s, 26B-A4B MoE stack, FP8/bf16 experts x "
                  "FP8/bf16 lm_head (bf16 router), and all-FP8 (FP8 router too), M=1 and M=5",
        "value": top["tokens_per_s_plain"], "unit": "tokens/s (FP8 rung, plain decoding)", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": top["M1"]["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 or bf16 weights (per rung) x bf16 activations, fp32 accumulate",
        "data": "synthetic (seeded N(0,.) weights; FP8 rungs quantise the same draws the bf16 rungs round)",
        "config": {"workload": "Gemma-4-26B-A4B-shaped MoE stack, 30 layers + tied lm_head + argmax + accept, "
                               "fused step, M=1 and M=5", "layers": sh.layers, "hidden": sh.hidden,
                   "experts": sh.experts, "top_k": sh.top_k, "expert_width": sh.width, "vocab": sh.vocab},
        "rungs": rungs,
        "fp8_over_bf16_plain": round(top["tokens_per_s_plain"] / base["tokens_per_s_plain"], 3),
        "fp8_spec_over_bf16_plain_alpha0.87": round(top["tokens_per_s_spec_alpha0.87"] / base["tokens_per_s_plain"], 3),
        "router_fp8_over_bf16_plain": round(rungs["experts_fp8+lm_head_fp8+router_fp8"]["tokens_per_s_plain"] /
                                            top["tokens_per_s_plain"], 3),
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(args, sh, layers, gains, Q, s, M):
    """The oracle (plain fp64 C, OpenMP over output rows) on a bounded sample of the
    same workload: the first cpu_layers layers for cpu_steps step inputs, plus the
    full lm_head once per step; scaled to a whole 30-layer step."""
    import oracle
    import synth
    import torch
    t0 = time.time()
    host = [synth.weights_to_host(layers[l]) for l in range(args.cpu_layers)]
    gh = synth.bits16(gains)
    Qh, sh_ = synth.bytes8(Q), synth.f32(s)
    log("oracle sample: host copies in %.1fs" % (time.time() - t0))
    t_layers = 0.0
    t_lm = 0.0
    for i in range(args.cpu_steps):
        x = synth.bits16(synth.hidden_inputs(sh, M, i, tag="bench_x"))
        noise = synth.bits16(synth.stack_noise(sh, M, i))
        t = time.perf_counter()
        h = x
        y = None
        for l in range(args.cpu_layers):
            h, u = oracle.add_rmsnorm(h, noise[l], y, gh[l])
            y = oracle.moe_layer(u, host[l], sh.top_k)["y_bf16"]
        t_layers += time.perf_counter() - t
        t = time.perf_counter()
        oracle.lm_head_argmax(u, Qh, sh_)
        t_lm += time.perf_counter() - t
    per_step = (t_layers / args.cpu_layers * sh.layers + t_lm) / args.cpu_steps
    threads = oracle.num_threads()
    log("oracle: %.2f s per full step on %d threads (sample %.1f s)" % (per_step, threads, t_layers + t_lm))
    # the same oracle on one thread, over a smaller sample (2 layers + the lm_head, 2 steps)
    oracle.set_num_threads(1)
    t1_layers = t1_lm = 0.0
    for i in range(2):
        x = synth.bits16(synth.hidden_inputs(sh, M, i, tag="bench_x"))
        noise = synth.bits16(synth.stack_noise(sh, M, i))
        t = time.perf_counter()
        h, y = x, None
        for l in range(2):
            h, u = oracle.add_rmsnorm(h, noise[l], y, gh[l])
            y = oracle.moe_layer(u, host[l], sh.top_k)["y_bf16"]
        t1_layers += time.perf_counter() - t
        t = time.perf_counter()
        oracle.lm_head_argmax(u, Qh, sh_)
        t1_lm += time.perf_counter() - t
    oracle.set_num_threads(threads)
    per_step_1 = (t1_layers / 2 * sh.layers + t1_lm) / 2
    log("oracle: %.2f s per full step on 1 thread" % per_step_1)
    return {"value": round(1.0 / per_step, 5), "unit": "steps/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "single_thread": {"value": round(1.0 / per_step_1, 6), "unit": "steps/s", "cores": 1,
                              "sample": "M=%d, 2 step inputs x (layers 0-1 + the full lm_head), scaled to 30 "
                                        "layers; %.1f s of CPU time" % (M, t1_layers + t1_lm)},
            "sample": "M=%d, %d step inputs x (layers 0-%d of the 30-layer stack + the full 262144-row "
                      "lm_head), scaled to 30 layers; %.1f s of CPU time" % (
                          M, args.cpu_steps, args.cpu_layers - 1, t_layers + t_lm)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
