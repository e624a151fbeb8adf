#!/usr/bin/env python3
"""Benchmark of the routed-MoE block with sketch-based top-k channel selection.

One step = one forward of the whole block (route, quantise, sketch scores, top-k
selection, gathered SwiGLU over the selected channels, down projection with the
low-rank compensation, combine) for one batch of decode tokens. The default
workload is the Qwen3-30B-A3B-shaped block (d=2048, 128 experts, top-8, m=768,
r=32) at batch 1 with k=138 (the 18% budget); the 13% budget (k=100) and the
dense-read block over the same inputs are timed in the same run. Inputs are
synthetic (seeded bf16 N(0, 0.02) weights, N(0, 1) tokens and logits) and
already resident in HBM when the timed region starts.

Cold-cache protocol: `--copies` distinct prepared layers (different weights) and
`--tokens` distinct tokens per layer are visited round-robin; the batch-1 tokens
of a layer route to disjoint expert groups (token t to group t mod E / top_e), so
no weight, sketch or map byte is reused within copies*tokens calls (2.7 GB of
traffic for the Qwen3-shaped block, ten times the 256 MB last-level cache). The sequence of forwards is captured
once in a HIP graph and replayed; the timed region is bracketed by
torch.cuda.synchronize() and HIP events recorded on the launch stream.
`--eager` launches every forward directly instead (for profilers). The batch-1
figure is also given as its spread over the graph replays (p10 / median / p90
per forward) and as single-call latency: one forward launched on its own,
event-timed and synchronised, over 200 calls (sparse and dense).

Prints ONE JSON line. Only one GPU is supported (`--gpus 1`).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
# sources whose change invalidates stored counter readings of the single-launch kernel
FUSED_SOURCES = ("activation_sparse_expert_amd/csrc/fused.hip",
                 "activation_sparse_expert_amd/csrc/device_common.h",
                 "activation_sparse_expert_amd/csrc/kernels.h")


def algorithmic_bytes(d, m, n_exp, top_e, r, k, batch, dense=False):
    """Bytes the method must move per forward call when every routed pair reads its
    own k channels. Sparse: per routed expert the 2-bit gate+up sketch (m*d/2), the
    channel statistics (12*m), the selected channels' bf16 gate, up and down vectors
    (6*d*k) and the rank-r map (2*(m+d)*r). Dense: 6*d*m per routed expert. Plus x
    (2d), out (2d) and the logits (4E) per token."""
    pairs = batch * top_e
    per_tok = batch * (4 * d + 4 * n_exp)
    if dense:
        return pairs * 6 * d * m + per_tok
    return pairs * (m * d // 2 + 12 * m + 6 * d * k + 2 * (m + d) * r) + per_tok


def progress(msg):
    """One line on stderr as each stage ends (stdout carries only the result line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def sources_digest(paths=FUSED_SOURCES):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_kernel_avg_us(name, kernel_prefix):
    """Average duration (us) of the first kernel whose name contains
    kernel_prefix in a committed rocprofv3 kernel-statistics summary, or None when
    the summary is missing or was taken on other kernel sources."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    digest, avg = None, None
    with open(path) as f:
        for line in f:
            if line.startswith("sources_digest:"):
                digest = line.split(":", 1)[1].strip()
            cells = [c.strip() for c in line.split("|")]  # name | calls | average_ns | ...
            if avg is None and len(cells) > 2 and kernel_prefix in cells[0]:
                try:
                    avg = float(cells[2]) / 1e3
                except ValueError:
                    pass
    return round(avg, 3) if avg is not None and digest == sources_digest() else None


def stored_traffic(name):
    """HBM bytes per launch from a committed counter summary, or None when the
    summary is missing or was taken on other kernel sources."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None, None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, _, val = line.partition(":")
                vals[key.strip()] = val.strip()
    if vals.get("sources_digest") != sources_digest():
        return None, vals.get("sources_digest")
    try:
        return int(float(vals["fetch_bytes_per_launch"]) + float(vals["write_bytes_per_launch"])), vals["sources_digest"]
    except (KeyError, ValueError):
        return None, None


class Block:
    """`copies` prepared layers of one workload plus `ntok` distinct input batches
    each, at batch 1 (logits N(0, 1)) and at batch 64 (Zipf-skewed logits)."""

    def __init__(self, b, synth, torch, w, copies, ntok, stream, big_batch=0):
        self.b, self.w, self.copies, self.ntok, self.stream = b, w, copies, ntok, stream
        d, m, n_exp, top_e, r = w["d"], w["m"], w["n_experts"], w["top_e"], w["rank"]
        self.ctxs, self.host_layer0 = [], None
        self.inputs = {}  # batch -> (xs, lgs, outs) per layer copy
        batches = [w["batch"]] + ([big_batch] if big_batch else [])
        for l in range(copies):
            wg, wu, wd = synth.layer_weights(w["wid"], l, n_exp, d, m, w["channel_scale"])
            cfg = b.make_config(d, n_exp, m, r, top_e, max(batches))
            self.ctxs.append(b.moe_sel_prepare(cfg, wg, wu, wd, stream=stream.cuda_stream))
            if l == 0:
                self.host_layer0 = (wg, wu, wd)
            del wg, wu, wd
            groups = max(1, n_exp // top_e)
            for bsz in batches:
                wid = w["wid"] if bsz == w["batch"] else synth.WORKLOADS["qwen3_b64"]["wid"]
                xb = np.stack([synth.tokens(wid, l, bsz, d, index=i) for i in range(ntok)])
                if bsz == w["batch"]:  # consecutive visits of a layer route to disjoint experts
                    lb = np.stack([synth.router_logits(wid, l, bsz, n_exp, "disjoint", index=i, group=i % groups,
                                                       group_size=top_e) for i in range(ntok)])
                else:
                    lb = np.stack([synth.router_logits(wid, l, bsz, n_exp, "zipf", index=i) for i in range(ntok)])
                xs, lgs, outs = self.inputs.setdefault(bsz, ([], [], []))
                xs.append(torch.from_numpy(xb.view(np.int16)).to("cuda"))
                lgs.append(torch.from_numpy(lb).to("cuda"))
                outs.append(torch.zeros((bsz, d), dtype=torch.int16, device="cuda"))

    def launch(self, n, k, bsz, thr=None, top_e=None):
        """Enqueue n forwards of `bsz` tokens (k=None: the dense-read block; thr: the
        threshold selector; top_e: routed experts per token, default the trained
        count) on the stream."""
        b, s = self.b, self.stream.cuda_stream
        te = self.w["top_e"] if top_e is None else top_e
        xs, lgs, outs = self.inputs[bsz]
        for i in range(n):
            l, t = i % self.copies, (i // self.copies) % self.ntok
            if thr is not None:
                b.moe_sel_forward_threshold(self.ctxs[l], xs[l][t], lgs[l][t], bsz, te, thr, outs[l], s)
            elif k is None:
                b.moe_sel_forward_dense(self.ctxs[l], xs[l][t], lgs[l][t], bsz, te, outs[l], s)
            else:
                b.moe_sel_forward(self.ctxs[l], xs[l][t], lgs[l][t], bsz, te, k, outs[l], s)

    def destroy(self):
        for c in self.ctxs:
            self.b.moe_sel_destroy(c)


def time_block(torch, blk, k, steps, warmup, eager, bsz, thr=None, top_e=None, spread=None):
    """Milliseconds per forward over `steps` timed forwards after `warmup` untimed ones.
    With a dict `spread` (graph timing only), also fills the p10 / median / p90 of
    the per-forward time of each graph replay, in microseconds."""
    R = blk.copies * blk.ntok
    stream = blk.stream
    with torch.cuda.stream(stream):
        blk.launch(R, k, bsz, thr, top_e)  # eager pass over every (layer, token batch)
    torch.cuda.synchronize()
    for c in blk.ctxs:
        blk.b.moe_sel_check_device(c)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if eager:
        with torch.cuda.stream(stream):
            blk.launch(warmup, k, bsz, thr, top_e)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            ev0.record(stream)
            blk.launch(steps, k, bsz, thr, top_e)
            ev1.record(stream)
        torch.cuda.synchronize()
    else:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            blk.launch(R, k, bsz, thr, top_e)
        rem = steps % R
        g_rem = None
        if rem:
            g_rem = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_rem, stream=stream):
                blk.launch(rem, k, bsz, thr, top_e)
        with torch.cuda.stream(stream):
            for _ in range(max(1, math.ceil(warmup / R))):
                g.replay()
        torch.cuda.synchronize()
        n_rep = steps // R
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_rep + 1)] if spread is not None else None
        with torch.cuda.stream(stream):
            ev0.record(stream)
            if evs:
                evs[0].record(stream)
            for i in range(n_rep):
                g.replay()
                if evs:
                    evs[i + 1].record(stream)
            if g_rem is not None:
                g_rem.replay()
            ev1.record(stream)
        torch.cuda.synchronize()
        if evs and n_rep:
            per = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 / R for i in range(n_rep)])
            spread.update({"replays": n_rep, "forwards_per_replay": R, "p10_us": round(float(np.percentile(per, 10)), 3),
                           "median_us": round(float(np.median(per)), 3),
                           "p90_us": round(float(np.percentile(per, 90)), 3)})
    for c in blk.ctxs:
        blk.b.moe_sel_check_device(c)  # raises if a bounded wait gave up
    return ev0.elapsed_time(ev1) / steps


def single_call_latency(torch, blk, k, bsz, n=200, warmup=20):
    """Latency of one forward launched on its own (eager launch, event-timed,
    synchronised after each call), in microseconds: p10 / median / p90 over n calls."""
    stream = blk.stream
    with torch.cuda.stream(stream):
        blk.launch(warmup, k, bsz)
    torch.cuda.synchronize()
    R = blk.copies * blk.ntok
    xs, lgs, outs = blk.inputs[bsz]
    te = blk.w["top_e"]
    b, s = blk.b, stream.cuda_stream
    times = []
    for i in range(n):
        l, t = i % blk.copies, (i // blk.copies) % blk.ntok
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            ev0.record(stream)
            if k is None:
                b.moe_sel_forward_dense(blk.ctxs[l], xs[l][t], lgs[l][t], bsz, te, outs[l], s)
            else:
                b.moe_sel_forward(blk.ctxs[l], xs[l][t], lgs[l][t], bsz, te, k, outs[l], s)
            ev1.record(stream)
        ev1.synchronize()
        times.append(ev0.elapsed_time(ev1) * 1e3)
    del R
    times = np.array(times)
    return {"calls": n, "p10_us": round(float(np.percentile(times, 10)), 3), "median_us": round(float(np.median(times)), 3),
            "p90_us": round(float(np.percentile(times, 90)), 3)}


def read_ceiling(b, torch, stream, nbytes=4 << 30, reps=8):
    """Measured HBM read ceiling: the library's plain read stream (every 16-byte
    piece of a 4 GiB buffer read once per pass), bytes read / time."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    s = stream.cuda_stream
    b.moe_sel_read_stream(buf, nbytes, sink, s)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for _ in range(reps):
            b.moe_sel_read_stream(buf, nbytes, sink, s)
        ev1.record(stream)
    torch.cuda.synchronize()
    sec = ev0.elapsed_time(ev1) * 1e-3 / reps
    del buf, sink
    return nbytes / sec / 1e9


def batch_bytes(b, torch, blk, k, bsz, ms, ms_dense):
    """Algorithmic bytes of the multi-token calls of the rotation, from the
    selections the calls actually made: per active expert the 2-bit sketch
    (m d / 2), the statistics (12 m), the bf16 gate, up and down vectors of the
    union of its tokens' selected channels (6 d |U_e|) and the rank-r map
    (2 (m + d) r); plus x, out and logits per token. Averaged over every call of
    the rotation; GB/s and roofline fractions against the timed calls."""
    w = blk.w
    d, m, n_exp, top_e, r = w["d"], w["m"], w["n_experts"], w["top_e"], w["rank"]
    xs, lgs, outs = blk.inputs[bsz]
    s = blk.stream.cuda_stream
    per_tok = bsz * (4 * d + 4 * n_exp)
    sparse, dense, active, ufrac = [], [], [], []
    for l in range(blk.copies):
        for t in range(blk.ntok):
            b.moe_sel_forward(blk.ctxs[l], xs[l][t], lgs[l][t], bsz, top_e, k, outs[l], s)
            sel = b.moe_sel_debug_selection(blk.ctxs[l], bsz, top_e, k, m, with_scores=False)
            unions = {}
            for tok in range(bsz):
                for slot in range(top_e):
                    e = int(sel["expert_ids"][tok, slot])
                    unions.setdefault(e, set()).update(sel["chan_idx"][tok, slot].tolist())
            sizes = np.array([len(u) for u in unions.values()])
            sparse.append(len(unions) * (m * d // 2 + 12 * m + 2 * (m + d) * r) + 6 * d * int(sizes.sum()) + per_tok)
            dense.append(len(unions) * 6 * d * m + per_tok)
            active.append(len(unions))
            ufrac.append(sizes.mean() / m)
    torch.cuda.synchronize()
    byt, dbyt = float(np.mean(sparse)), float(np.mean(dense))
    out = {"algorithmic_bytes": round(byt), "active_experts_mean": round(float(np.mean(active)), 2),
           "union_fraction_mean": round(float(np.mean(ufrac)), 4),
           "achieved_GBs": round(byt / (ms * 1e-3) / 1e9, 1),
           "frac": round(byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "dense_algorithmic_bytes": round(dbyt), "byte_ideal_speedup": round(dbyt / byt, 3),
           "bytes_from": f"the selections of all {len(sparse)} calls of the rotation"}
    if ms_dense is not None:
        out["dense_achieved_GBs"] = round(dbyt / (ms_dense * 1e-3) / 1e9, 1)
        out["dense_frac"] = round(dbyt / (ms_dense * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    return out


def cpu_model():
    """(model name, physical cores) of the host, from /proc/cpuinfo."""
    name, cores = None, set()
    try:
        phys = core = None
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key, val = key.strip(), val.strip()
                if key == "model name" and name is None:
                    name = val
                elif key == "physical id":
                    phys = val
                elif key == "core id":
                    core = val
                elif not key and phys is not None:
                    cores.add((phys, core))
                    phys = core = None
    except OSError:
        pass
    return name, (len(cores) or None)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4096)
    ap.add_argument("--warmup", type=int, default=512)
    ap.add_argument("--workload", default="qwen3", choices=("qwen3",))
    ap.add_argument("--k", type=int, default=None, help="channel budget (default: the 18%% budget)")
    ap.add_argument("--copies", type=int, default=8, help="distinct prepared layers rotated")
    ap.add_argument("--tokens", type=int, default=16, help="distinct token batches per layer")
    ap.add_argument("--eager", action="store_true", help="launch every forward directly (no graph)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-extra-budgets", action="store_true")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="also run plain 256 MiB copies (known bytes) for counter scaling")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--big-batch", type=int, default=64,
                    help="also time this many Zipf-routed tokens per call (0: skip)")
    ap.add_argument("--big-steps", type=int, default=512)
    ap.add_argument("--mixtral", type=int, default=1,
                    help="also time the Mixtral-shaped block at batch 1 (0: skip)")
    ap.add_argument("--mixtral-steps", type=int, default=256)
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the Mixtral-shaped block's score-kind ablation (counter runs)")
    ap.add_argument("--decode48", type=int, default=1,
                    help="also time a 48-layer decode step at batch 1, 8 and 32 (0: skip)")
    ap.add_argument("--decode-layers", type=int, default=12, help="distinct prepared layers in the 48-layer stack")
    ap.add_argument("--decode-steps", type=int, default=30)
    ap.add_argument("--expert-sweep", type=int, default=1,
                    help="also sweep routed experts per token below the trained count (0: skip)")
    ap.add_argument("--threshold", type=int, default=1,
                    help="also compare the calibrated threshold selector with top-k (0: skip)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py runs on exactly one GPU: the block is a single-GPU kernel "
                                   "pipeline and no multi-GPU figure is produced; run it with --gpus 1"}))
        sys.exit(2)

    import torch
    from activation_sparse_expert_amd import binding as b
    from activation_sparse_expert_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    w = synth.WORKLOADS[args.workload]
    d, m, n_exp, top_e, r, batch = w["d"], w["m"], w["n_experts"], w["top_e"], w["rank"], w["batch"]
    k = args.k if args.k is not None else w["ks"][-1]

    t0 = time.time()
    stream = torch.cuda.Stream()
    blk = Block(b, synth, torch, w, args.copies, args.tokens, stream, args.big_batch)
    setup_s = time.time() - t0
    progress(f"{args.copies} layers prepared in {setup_s:.1f} s")

    spread = {}
    ms = time_block(torch, blk, k, args.steps, args.warmup, args.eager, batch, spread=spread)
    path = b.moe_sel_last_path(blk.ctxs[0])
    single_call = {"sparse": single_call_latency(torch, blk, k, batch)}
    if not args.no_dense:
        single_call["dense"] = single_call_latency(torch, blk, None, batch)
    single = path == b.MOE_SEL_PATH_SINGLE_LAUNCH
    progress(f"batch {batch}, k={k}: {ms * 1e3:.2f} us per call")
    extra_k = {}
    if not args.no_extra_budgets:
        for k2 in w["ks"]:
            if k2 != k:
                ms2 = time_block(torch, blk, k2, args.steps, args.warmup, args.eager, batch)
                extra_k[str(k2)] = {"tokens_per_s": round(batch / (ms2 * 1e-3), 1), "ms_per_step": round(ms2, 6),
                                    "budget": round(k2 / m, 4),
                                    "achieved_GBs": round(algorithmic_bytes(d, m, n_exp, top_e, r, k2, batch)
                                                          / (ms2 * 1e-3) / 1e9, 1)}
    ms_dense = None if args.no_dense else time_block(torch, blk, None, args.steps, args.warmup, args.eager, batch)
    progress("other budgets and the dense block timed")
    big = None
    if args.big_batch:
        bb = args.big_batch
        ws = args.big_steps // 8
        ms_b = time_block(torch, blk, k, args.big_steps, ws, args.eager, bb)
        ms_bd = None if args.no_dense else time_block(torch, blk, None, args.big_steps, ws, args.eager, bb)
        big = {"batch": bb, "routing": "Zipf(1.1)", "k": k, "steps": args.big_steps,
               "tokens_per_s": round(bb / (ms_b * 1e-3), 1), "ms_per_step": round(ms_b, 6),
               "path": "expert-grouped multi-kernel"}
        if ms_bd is not None:
            big["dense_tokens_per_s"] = round(bb / (ms_bd * 1e-3), 1)
            big["dense_ms_per_step"] = round(ms_bd, 6)
            big["speedup_vs_dense"] = round(ms_bd / ms_b, 3)
    if big is not None:
        big.update(batch_bytes(b, torch, blk, k, args.big_batch, ms_b, ms_bd))
        progress(f"batch {args.big_batch} timed")
    ceiling = read_ceiling(b, torch, stream)
    if args.traffic_probe:
        src = torch.empty(1 << 26, dtype=torch.float32, device="cuda").fill_(2.0)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            for _ in range(4):
                dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    tok_s = batch / (ms * 1e-3)
    bytes_sparse = algorithmic_bytes(d, m, n_exp, top_e, r, k, batch)
    bytes_dense = algorithmic_bytes(d, m, n_exp, top_e, r, k, batch, dense=True)
    # The single-launch path runs the whole block as one kernel per forward: its
    # average launch duration, measured with HIP events on the launch stream, is
    # the timed region over the forwards in it (so it includes the gap between
    # consecutive launches in the graph). The kernel-trace average of the same
    # command, from the committed profile of these sources, is reported beside it.
    kernel_s = ms * 1e-3
    achieved = bytes_sparse / kernel_s / 1e9
    traffic, digest = stored_traffic(f"traffic_k_fused_{args.workload}_b{batch}_k{k}.txt") if single else (None, None)
    prof_us = stored_kernel_avg_us(f"kernel_stats_{args.workload}_b{batch}.txt", "k_fused<false") if single else None
    result = {
        "metric": "MoE-block tokens/s at batch 1; achieved HBM GB/s vs peak on bytes read",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"Qwen3-30B-A3B-shaped MoE block, d={d}, {n_exp} experts, top-{top_e}, m={m}, "
                        f"batch {batch}, k={k} ({k / m:.1%} budget), r={r}",
            "batch": batch, "k": k, "rank": r,
            "cold_rotation": {"layers": args.copies, "token_batches_per_layer": args.tokens},
            "timing": "eager launches" if args.eager else "HIP graph of consecutive block calls",
            "path": "single-launch" if single else "multi-kernel",
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "k_fused<sparse> (whole block in one launch)" if single else "multi-kernel block",
            "algorithmic_bytes_per_launch": bytes_sparse,
            "event_us_per_launch": round(kernel_s * 1e6, 3),
            "rocprof_kernel_avg_us": prof_us,
            "frac_rocprof": (round(bytes_sparse / (prof_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4) if prof_us else None),
            "traffic_sources_digest": digest,
            "measured_read_ceiling_GBs": round(ceiling, 1),
            "frac_of_measured_ceiling": round(achieved / ceiling, 4),
        },
        "setup_s": round(setup_s, 1),
    }
    if spread:
        result["graph_replay_spread"] = spread
    result["single_call"] = single_call
    if extra_k:
        result["other_budgets"] = extra_k
    if big is not None:
        result["batch64" if big["batch"] == 64 else f"batch{big['batch']}"] = big
    if ms_dense is not None:
        dense_gbs = bytes_dense / (ms_dense * 1e-3) / 1e9
        result["dense"] = {
            "tokens_per_s": round(batch / (ms_dense * 1e-3), 1), "ms_per_step": round(ms_dense, 6),
            "algorithmic_bytes": bytes_dense, "achieved_GBs": round(dense_gbs, 1),
            "frac": round(dense_gbs / HBM_PEAK_GBS, 4),
        }
        result["speedup_vs_dense"] = round(ms_dense / ms, 3)

    if args.expert_sweep:
        result["expert_count_sweep"] = expert_sweep(b, synth, torch, blk, args.steps // 2, args.warmup // 2)
        result["score_ablation"] = score_ablation(b, torch, blk, w["ks"])
        progress("expert-count sweep and score ablation done")
    if args.threshold and args.big_batch == 64:
        result["threshold_vs_topk"] = threshold_experiment(b, synth, torch, blk, k, args.steps, args.warmup)
        progress("threshold experiment done")
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(blk.host_layer0, w, k, args.cpu_seconds)
        progress("CPU baseline done")
    blk.destroy()
    del blk
    if args.mixtral:
        result["mixtral"] = time_mixtral(b, synth, torch, stream, args.mixtral_steps, args.eager,
                                         ablation=not args.no_ablation)
        progress("Mixtral-shaped block timed")
    if args.decode48:
        result["decode48"] = time_decode48(b, synth, torch, stream, args.decode_layers, args.decode_steps)
        progress("48-layer decode timed")

    print(json.dumps(result), flush=True)


def expert_sweep(b, synth, torch, blk, steps, warmup, tops=(8, 6, 4, 2), n_dev=16):
    """Routed experts per token below the trained top-8 composed with the channel
    budget: batch-1 tokens/s, and the deviation from the dense top-8 block
    (max over n_dev tokens of ||out - dense||_inf / ||dense||_inf)."""
    w = blk.w
    d, m, n_exp, top_e_trained = w["d"], w["m"], w["n_experts"], w["top_e"]
    ctx, s = blk.ctxs[0], blk.stream.cuda_stream
    x = torch.from_numpy(synth.tokens(w["wid"], 0, n_dev, d, index=2000).view(np.int16)).to("cuda")
    lg = torch.from_numpy(synth.router_logits(w["wid"], 0, n_dev, n_exp, "normal", index=2000)).to("cuda")
    ref = torch.zeros((n_dev, d), dtype=torch.int16, device="cuda")
    b.moe_sel_forward_dense(ctx, x, lg, n_dev, top_e_trained, ref, s)
    torch.cuda.synchronize()
    ref_f = ref.view(torch.bfloat16).float().cpu().numpy()

    def deviation(top_e, k):
        o = torch.zeros((n_dev, d), dtype=torch.int16, device="cuda")
        if k is None:
            b.moe_sel_forward_dense(ctx, x, lg, n_dev, top_e, o, s)
        else:
            b.moe_sel_forward(ctx, x, lg, n_dev, top_e, k, o, s)
        torch.cuda.synchronize()
        of = o.view(torch.bfloat16).float().cpu().numpy()
        return round(float((np.abs(of - ref_f).max(axis=1) / np.abs(ref_f).max(axis=1)).max()), 4)

    rows = []
    for top_e in tops:
        for k in list(w["ks"]) + [None]:
            ms = time_block(torch, blk, k, steps, warmup, False, 1, top_e=top_e)
            rows.append({"top_e": top_e, "k": k if k is not None else m,
                         "selector": "top-k" if k is not None else "dense",
                         "tokens_per_s": round(1 / (ms * 1e-3), 1), "max_rel_dev_vs_dense_top8": deviation(top_e, k)})
    return {"reference": f"dense block with the trained top-{top_e_trained}", "tokens_for_deviation": n_dev,
            "rows": rows}


def threshold_experiment(b, synth, torch, blk, k, steps, warmup):
    """The calibrated threshold selector on the same scores as top-k: threshold set
    on 64 calibration tokens for the 18% mean read, per-token read fractions on 256
    other tokens, and the batch-1 time per call of both selectors."""
    from activation_sparse_expert_amd import threshold as th
    w = blk.w
    d, m, n_exp, top_e = w["d"], w["m"], w["n_experts"], w["top_e"]
    ctx, s = blk.ctxs[0], blk.stream.cuda_stream
    out = torch.zeros((64, d), dtype=torch.int16, device="cuda")

    def batch(i):
        x = torch.from_numpy(synth.tokens(w["wid"], 0, 64, d, index=1000 + i).view(np.int16)).to("cuda")
        lg = torch.from_numpy(synth.router_logits(w["wid"], 0, 64, n_exp, "normal", index=1000 + i)).to("cuda")
        return x, lg

    x, lg = batch(0)
    b.moe_sel_forward(ctx, x, lg, 64, top_e, k, out, s)
    scores = b.moe_sel_debug_selection(ctx, 64, top_e, k, m, with_scores=True)["score"]
    thr = th.calibrate(scores, 0.18)
    fr = []
    for i in range(1, 5):
        x, lg = batch(i)
        b.moe_sel_forward_threshold(ctx, x, lg, 64, top_e, thr, out, s)
        cnt = b.moe_sel_debug_selection(ctx, 64, top_e, m, m, with_scores=False)["chan_count"]
        fr.append(th.read_fractions(cnt, m))
    torch.cuda.synchronize()
    ms_thr = time_block(torch, blk, None, steps // 4, warmup // 4, False, 1, thr=thr)
    return {"calibration": "threshold on the scores of 64 calibration tokens for an 18% mean read",
            "threshold": thr, "test_tokens": 256, "threshold_read_fraction": th.summary(np.concatenate(fr)),
            "topk_read_fraction": round(k / m, 5),
            "batch1_threshold_tokens_per_s": round(1 / (ms_thr * 1e-3), 1),
            "batch1_threshold_path": "expert-grouped multi-kernel (counts vary per pair)"}


def score_ablation(b, torch, blk, ks, n_tok=4):
    """Deviation from the dense block (max over n_tok batch-1 tokens of
    ||out - dense||_inf / ||dense||_inf) for each channel score kind and budget."""
    w = blk.w
    ctx, s = blk.ctxs[0], blk.stream.cuda_stream
    xs, lgs, _ = blk.inputs[1]
    top_e = w["top_e"]
    kinds = {"full": b.MOE_SEL_SCORE_FULL, "gate_only": b.MOE_SEL_SCORE_GATE_ONLY,
             "no_down_norm": b.MOE_SEL_SCORE_NO_DOWN_NORM, "x_int16": b.MOE_SEL_SCORE_X_INT16}

    def run(k, kind=None):
        outs = []
        for t in range(n_tok):
            o = torch.zeros((1, w["d"]), dtype=torch.int16, device="cuda")
            if k is None:
                b.moe_sel_forward_dense(ctx, xs[0][t], lgs[0][t], 1, top_e, o, s)
            else:
                b.moe_sel_forward(ctx, xs[0][t], lgs[0][t], 1, top_e, k, o, s)
            outs.append(o)
        torch.cuda.synchronize()
        return np.concatenate([o.view(torch.bfloat16).float().cpu().numpy() for o in outs])

    dense = run(None)
    res = {}
    for name, code in kinds.items():
        b.moe_sel_set_score(ctx, code)
        for k in ks:
            o = run(k)
            res[f"{name}_k{k}"] = round(float((np.abs(o - dense).max(axis=1) / np.abs(dense).max(axis=1)).max()), 4)
    b.moe_sel_set_score(ctx, b.MOE_SEL_SCORE_FULL)
    return {"max_rel_dev_vs_dense": res, "tokens": n_tok}


def time_mixtral(b, synth, torch, stream, steps, eager, ablation=True):
    """Mixtral-8x7B-shaped block (d=4096, 8 experts, top-2, m=14336, r=64, LogNormal
    channel scales) at batch 1: both budgets and the dense-read block, over two
    rotated layer copies and eight tokens each (16 calls, about 3 GB of weights)."""
    w = synth.WORKLOADS["mixtral"]
    d, m, n_exp, top_e, r = w["d"], w["m"], w["n_experts"], w["top_e"], w["rank"]
    t0 = time.time()
    blk = Block(b, synth, torch, w, 2, 8, stream)
    setup = time.time() - t0
    out = {"workload": f"Mixtral-8x7B-shaped MoE block, d={d}, {n_exp} experts, top-{top_e}, m={m}, batch 1, "
                       f"r={r}", "setup_s": round(setup, 1), "steps": steps,
           "path": "expert-grouped multi-kernel"}
    for k in w["ks"]:
        ms = time_block(torch, blk, k, steps, steps // 8, eager, 1)
        byt = algorithmic_bytes(d, m, n_exp, top_e, r, k, 1)
        out[f"k{k}"] = {"tokens_per_s": round(1 / (ms * 1e-3), 1), "ms_per_step": round(ms, 6),
                        "budget": round(k / m, 4), "algorithmic_bytes": byt,
                        "achieved_GBs": round(byt / (ms * 1e-3) / 1e9, 1)}
    ms_d = time_block(torch, blk, None, steps, steps // 8, eager, 1)
    byt = algorithmic_bytes(d, m, n_exp, top_e, r, 0, 1, dense=True)
    out["dense"] = {"tokens_per_s": round(1 / (ms_d * 1e-3), 1), "ms_per_step": round(ms_d, 6),
                    "algorithmic_bytes": byt, "achieved_GBs": round(byt / (ms_d * 1e-3) / 1e9, 1)}
    for k in w["ks"]:
        out[f"k{k}"]["speedup_vs_dense"] = round(ms_d / out[f"k{k}"]["ms_per_step"], 3)
    if ablation:
        out["score_ablation"] = score_ablation(b, torch, blk, w["ks"])
    blk.destroy()
    return out


def time_decode48(b, synth, torch, stream, distinct, steps, batches=(1, 8, 32), n_layers=48, eps=1e-6):
    """Decode step over 48 stacked Qwen3-shaped layers (k=137, r=32): per layer the
    router logits, the block and the residual renormalisation, all on the GPU. The
    stack cycles `distinct` prepared layers (each with its own router); a step
    touches more weight bytes per cycle than the last-level cache holds."""
    w = synth.WORKLOADS["qwen3_48l"]
    d, m, n_exp, top_e, r, k = w["d"], w["m"], w["n_experts"], w["top_e"], w["rank"], w["ks"][0]
    t0 = time.time()
    ctxs, wrs = [], []
    for l in range(distinct):
        wg, wu, wd = synth.layer_weights(w["wid"], l, n_exp, d, m)
        ctxs.append(b.moe_sel_prepare(b.make_config(d, n_exp, m, r, top_e, max(batches)), wg, wu, wd,
                                      stream=stream.cuda_stream))
        del wg, wu, wd
        wrs.append(torch.from_numpy(synth.router_weights(w["wid"], l, n_exp, d).view(np.int16)).to("cuda"))
    out = {"workload": f"{n_layers} stacked Qwen3-shaped layers (d={d}, {n_exp} experts, top-{top_e}, m={m}), "
                       f"k={k} ({k / m:.1%}), r={r}; router and residual RMS renormalisation per layer "
                       "(one launch between layers)",
           "distinct_layers": distinct, "setup_s": round(time.time() - t0, 1), "steps": steps}
    s = stream.cuda_stream
    for bsz in batches:
        x0 = torch.from_numpy(synth.tokens(w["wid"], 0, bsz, d).view(np.int16)).to("cuda")
        x = x0.clone()
        lg = torch.empty((bsz, n_exp), dtype=torch.float32, device="cuda")
        y = torch.empty((bsz, d), dtype=torch.int16, device="cuda")

        xb = (x, torch.empty_like(x))  # the hidden state alternates between two buffers

        def step(dense):
            # router of layer 0; between layers one launch renormalises the residual
            # stream and applies the next layer's router; the last layer renormalises
            b.moe_sel_router_logits(xb[0], wrs[0], bsz, d, n_exp, lg, s)
            for l in range(n_layers):
                c = ctxs[l % distinct]
                xc, xn = xb[l % 2], xb[(l + 1) % 2]
                if dense:
                    b.moe_sel_forward_dense(c, xc, lg, bsz, top_e, y, s)
                else:
                    b.moe_sel_forward(c, xc, lg, bsz, top_e, k, y, s)
                if l + 1 < n_layers:
                    b.moe_sel_residual_rmsnorm_router(xc, y, wrs[(l + 1) % distinct], bsz, d, n_exp, eps, xn, lg, s)
                else:
                    b.moe_sel_residual_rmsnorm(xc, y, bsz, d, eps, xn, s)

        res = {}
        for dense in (False, True):
            with torch.cuda.stream(stream):
                x.copy_(x0)
                step(dense)
            torch.cuda.synchronize()
            for c in ctxs:
                b.moe_sel_check_device(c)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step(dense)
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                x.copy_(x0)
                g.replay()
                ev0.record(stream)
                for _ in range(steps):
                    g.replay()
                ev1.record(stream)
            torch.cuda.synchronize()
            for c in ctxs:
                b.moe_sel_check_device(c)
            ms = ev0.elapsed_time(ev1) / steps
            res["dense" if dense else "sparse"] = ms
            del g
        out[f"batch{bsz}"] = {"tokens_per_s": round(bsz / (res["sparse"] * 1e-3), 1),
                              "ms_per_step": round(res["sparse"], 4),
                              "dense_tokens_per_s": round(bsz / (res["dense"] * 1e-3), 1),
                              "dense_ms_per_step": round(res["dense"], 4),
                              "speedup_vs_dense": round(res["dense"] / res["sparse"], 3)}
    for c in ctxs:
        b.moe_sel_destroy(c)
    return out


def cpu_baseline(weights, w, k, seconds):
    """The CPU oracle (as it stands) on a bounded sample of the same workload."""
    import oracle
    from activation_sparse_expert_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    wg, wu, wd = weights
    d, m, n_exp, top_e, r = w["d"], w["m"], w["n_experts"], w["top_e"], w["rank"]
    lay = oracle.OracleLayer(lambda e: (wg[e], wu[e], wd[e]), n_exp, d, m, r)
    ntok = 4
    xs = [synth.tokens(w["wid"], 0, 1, d, index=i) for i in range(ntok)]
    lgs = [synth.router_logits(w["wid"], 0, 1, n_exp, "normal", index=i) for i in range(ntok)]
    t0 = time.time()
    for lg in lgs:
        for e in oracle.route(lg[0], top_e)[0]:
            lay.expert(e)
    prep_s = time.time() - t0
    reps, n, t0 = 0, 0, time.time()
    while True:
        for x, lg in zip(xs, lgs):
            lay.forward(x, lg, top_e, k)
            n += 1
        reps += 1
        if time.time() - t0 > seconds or reps >= 200:
            break
    el = time.time() - t0
    model, physical = cpu_model()
    return {"value": round(n / el, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "physical_cores": physical, "logical_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
            "sample": f"{ntok} distinct batch-1 tokens of layer 0 x {reps} repetitions ({n} block forwards, "
                      f"k={k}, {el:.1f} s); preparation of the {len(lay._prep)} routed experts excluded "
                      f"({prep_s:.1f} s)"}


if __name__ == "__main__":
    main()
