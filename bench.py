"""Benchmark: KDA speculative verify + commit on one MI355X.

A step is one decode step of the whole path in serving order over several
layers: every layer's kda_verify (window from the checkpoints, outputs and
records), then every layer's commit (accepted prefix replayed into the
checkpoints) in one kda_commit_layers launch, as the commit runs once per
step for all layers after sampling. Each layer has its own pool, inputs and
records (12 layers by default). The default workload is the decode batch per
layer: B=64 requests, H=32 heads, K=V=128, T=4 tokens each (1 + 3 draft),
bf16 activations, fp32 checkpoints made by 64 random prefill tokens through
the library's own recurrence, num_accepted ~ Binomial(4, 0.7).

Inputs are resident in HBM before the timed region. The layers' checkpoints
(12 x 128 MiB) exceed the 256 MB Infinity Cache (MALL) many times over: at
most the last two layers' checkpoints can still be there when the commit
reads them, and nothing of one step is left for the next.

Printed: one JSON line (metric, value = verified tokens/s per layer call,
per-kernel times, achieved HBM bandwidth against the 8 TB/s peak, the same
step in the deferred flow, the stock speculative step on the same batch, the
CPU oracle's rate on a bounded sample of the same workload). The default run
adds sub-records of the other workloads ("workloads": the decode batch with
the bounded gate, the deep-draft batch, the ragged batch, the 8-layer
deferred workload) and the oracle's rate on samples of the tiny, ragged and
deferred workloads.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak, GB/s
STATE_BYTES = 128 * 128 * 4    # one (slot, head) fp32 state
TOKEN_IN_BYTES = 4 * 128 * 2 + 2   # q, k, v, g (bf16 x 128) + beta, per token and head
OUT_BYTES = 128 * 2                # o per token and head
REC_BYTES = 3 * 128 * 2 + 2        # records k, v, g + beta per token and head


def algorithmic_bytes(T, n_commit, valid, H):
    """Bytes the method must move (each counted once).

    verify: per valid (row, head) the state once, each token's inputs, its
            output and its records: 65,536 + 2,052 * T_i.
    commit: per valid (row, head) with n' > 0 the state read and written and
            n' records read: 131,072 + 770 * n'.
    """
    T = np.asarray(T)[valid]
    n = np.asarray(n_commit)[valid]
    verify = H * np.sum(STATE_BYTES + (TOKEN_IN_BYTES + OUT_BYTES + REC_BYTES) * T)
    commit = H * np.sum(np.where(n > 0, 2 * STATE_BYTES + REC_BYTES * n, 0))
    return float(verify), float(commit)


KERNEL_SOURCE = os.path.join(ROOT, "linear_attention_speculative_kda_amd", "csrc", "kda.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 1 << 30   # the plain copy timed below: 1 GiB read + 1 GiB written


def source_hash(text: str | None = None) -> str:
    """sha256 of the kernel source without its comments and blank lines:
    counter data stays valid across edits that change no code."""
    if text is None:
        with open(KERNEL_SOURCE, encoding="utf-8") as f:
            text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def kernel_key(name: str) -> str:
    """Library kernel -> call name (by template mode); others keep their name."""
    if "kda_kernel<1," in name:
        return "kda_verify"
    for mode, call in (("0", "kda_recurrent"), ("2", "kda_commit"), ("3", "kda_verify_deferred"),
                       ("4", "kda_recurrent_spec")):
        if f"kda_kernel<{mode}," in name:
            return call
    for mode, call in (("2", "kda_commit_layers"), ("3", "kda_flush_layers")):
        if f"kda_kernel_layers<{mode}," in name:
            return call
    if "kda_commit_list" in name:
        return "kda_commit_deferring"     # a commit with pending counts, by row list
    if "conv_compact" in name:
        return "kda_conv_compact"
    return name


def summarize_pmc(fetch_dir: str, write_dir: str, workload: str) -> dict:
    """Per-dispatch HBM traffic of each library kernel from two rocprofv3
    --pmc runs of this benchmark on one workload (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch), merged into the summary file under that
    workload. Each counter is calibrated on the plain 1 GiB copy that the
    benchmark times: its dispatches write exactly 1 GiB, so
    factor = 1 GiB / (what the counter reads for them)."""
    def load(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        return rows
    fetch, write = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    copy_kib = COPY_BYTES / 1024
    # The two runs dispatch the same sequence; pair the copies by dispatch id.
    copy_ids = {i for i, k, v in write if "copyBuffer" in k and abs(v - copy_kib) < 0.01 * copy_kib}
    copy_w = [v for i, k, v in write if i in copy_ids]
    copy_f = [v for i, k, v in fetch if i in copy_ids and "copyBuffer" in k]
    if not copy_w or not copy_f:
        raise SystemExit("no 1 GiB copy dispatches found to calibrate the counters")
    f_scale = copy_kib / float(np.median(copy_f))
    w_scale = copy_kib / float(np.median(copy_w))
    out = {"fetch_scale": f_scale, "write_scale": w_scale,
           "copy_fetch_kib": float(np.median(copy_f)), "copy_write_kib": float(np.median(copy_w)),
           "kernels": {}}
    by = {}
    for _, name, v in fetch:
        by.setdefault(kernel_key(name), {}).setdefault("fetch", []).append(v)
    for _, name, v in write:
        by.setdefault(kernel_key(name), {}).setdefault("write", []).append(v)
    for key, d in by.items():
        if not key.startswith("kda_") or "fetch" not in d or "write" not in d:
            continue
        fk, wk = float(np.median(d["fetch"])), float(np.median(d["write"]))
        out["kernels"][key] = {"fetch_kib": fk, "write_kib": wk, "dispatches": len(d["fetch"]),
                               "traffic_bytes": (fk * f_scale + wk * w_scale) * 1024}
    try:
        with open(TRAFFIC_FILE) as f:
            summary = json.load(f)
    except (OSError, ValueError):
        summary = {}
    if summary.get("source_sha256") != source_hash():
        summary = {"source_sha256": source_hash(), "workloads": {}}
    summary.setdefault("workloads", {})[workload] = out
    return summary


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter summary, or None when there is none or the kernel source changed
    since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_hash():
        return None
    k = t.get("workloads", {}).get(workload, {}).get("kernels", {}).get(kernel)
    return None if k is None else k["traffic_bytes"]


SUB_WORKLOADS = ("decode_bounded", "deep", "ragged", "deferred")
METRIC = "KDA verify+commit tokens/s and achieved HBM GB/s vs peak (B=64,H=32,T=4)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "decode_bounded", "deep", "ragged", "deferred"],
                    help="the workload of the headline line (the default line is the decode "
                         "batch, with the other workloads as sub-records)")
    ap.add_argument("--sets", type=int, default=12,
                    help="layers per step, each with its own pool, inputs and records")
    ap.add_argument("--no-sub", action="store_true",
                    help="headline workload only: no sub-records of the other workloads")
    ap.add_argument("--sub-steps", type=int, default=20, help="timed steps of each sub-record")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--cpu-rows", type=int, default=64, help="rows in the decode CPU oracle sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the decode CPU sample until this much wall time is spent")
    ap.add_argument("--cpu-seconds-other", type=float, default=4.0,
                    help="the same for the CPU samples of the other workloads")
    ap.add_argument("--align", action="store_true",
                    help="commit in align mode: a block table sends each row's state to other "
                         "blocks of the pool (decode/deep/ragged workloads)")
    ap.add_argument("--per-layer-commit", action="store_true",
                    help="one kda_commit per layer instead of one kda_commit_layers per step")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="merge two rocprofv3 --pmc runs of --workload into profiles/traffic.json "
                         "and exit")
    return ap.parse_args()


def main():
    args = parse()
    if args.summarize_pmc:
        out = summarize_pmc(*args.summarize_pmc, args.workload)
        os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(out, f, indent=1)
        print(json.dumps(out, indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path shards by requests and heads with no "
              "exchange between GPUs, so a multi-GPU figure is N independent one-GPU runs.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_attention_speculative_kda_amd as kda

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "deferred":
        print(json.dumps(deferred_leg(args, torch, kda, dev)), flush=True)
        return
    leg = serving_leg(args, torch, kda, dev, args.workload, args.sets, args.steps, args.warmup,
                      headline=True)
    stream = torch.cuda.current_stream()
    copy_gbs = device_copy_gbs(torch, stream)
    dom = leg["dominant"]
    kernels = leg["kernels"]
    result = {
        "metric": METRIC,
        "value": leg["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": leg["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": leg["config"],
        "roofline": {
            "bound": "hbm",
            "kernel": dom,
            "achieved": kernels[dom]["gbs"],
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": kernels[dom]["gbs"] / PEAK_HBM_GBS,
            "traffic": kernels[dom]["traffic"],
        },
    }
    for key in ("kernels", "ms_per_layer_step", "step_gbs", "step_frac_of_peak", "step_timing",
                "ms_per_step_eager", "value_eager", "commit_tokens_per_s", "verify_tokens_per_s",
                "interleaved", "deferred_flow", "stock_spec"):
        if key in leg:
            result[key] = leg[key]
    result["copy_gbs_measured"] = copy_gbs

    if not args.no_sub and args.workload == "decode" and not args.align and not args.per_layer_commit:
        subs = {}
        for name in SUB_WORKLOADS:
            sargs = argparse.Namespace(**vars(args))
            sargs.steps = args.sub_steps
            sargs.warmup = min(args.warmup, 5)
            if name == "deferred":
                d = deferred_leg(sargs, torch, kda, dev)
                subs[name] = {k: d[k] for k in ("config", "roofline", "flows", "deferred_speedup",
                                                "kda_conv_compact", "value", "ms_per_step")}
                subs[name]["value_unit"] = "tokens/s (every layer's verified tokens per second)"
            else:
                sub = serving_leg(sargs, torch, kda, dev, name, args.sets, sargs.steps,
                                  sargs.warmup)
                subs[name] = {k: sub[k] for k in ("config", "value", "ms_per_layer_step", "step_gbs",
                                                  "step_frac_of_peak", "kernels",
                                                  "verify_tokens_per_s", "commit_tokens_per_s")}
            print(f"sub-record {name} done", file=sys.stderr, flush=True)
        result["workloads"] = subs

    if not args.no_cpu:
        batch = make_batch_for(args.workload)
        result["cpu_baseline"] = cpu_baseline(batch, args.cpu_rows, args.cpu_seconds)
        if not args.no_sub and args.workload == "decode":
            result["cpu_baselines_other"] = cpu_baselines_other(args.cpu_seconds_other)

    print(json.dumps(result), flush=True)


def make_batch_for(name):
    from workloads import make_batch
    return make_batch(name)


def serving_leg(args, torch, kda, dev, name, L, K, W, headline=False):
    """One workload's decode step in serving order over L layers: every
    layer's kda_verify (the forward pass), then every layer's commit in one
    kda_commit_layers launch (after sampling). Per-kernel times from HIP
    events around eager launches; the step from a HIP graph of the whole
    step replayed K times. headline: also the interleaved order, the
    deferred flow and the stock speculative step on the same inputs."""
    batch = make_batch_for(name)
    B, H, Q = batch.num_rows, batch.H, batch.Q
    T = batch.seq_lens()
    ntok = batch.tokens.num_tokens
    valid = batch.valid_rows()

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    def up_bf16(bits):
        return up(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)

    layer = kda.Layer(a_log=up(batch.a_log), g_bias=up(batch.g_bias), scale=batch.scale,
                      lower_bound=batch.lower_bound)
    cu = up(batch.cu_seqlens)
    si = up(batch.state_indices)
    nacc = up(batch.num_accepted)
    hk = H * 128

    # ---- checkpoints: the prefill recipe runs the library's recurrence
    pool0 = up(batch.initial_pool())
    if batch.init == "prefill":
        p = batch.prefill
        qkv = up_bf16(p.qkv)
        o_pre = torch.empty((p.num_tokens, H, 128), dtype=torch.bfloat16, device=dev)
        kda.kda_recurrent(layer, qkv[:, :hk].view(-1, H, 128), qkv[:, hk:2 * hk].view(-1, H, 128),
                          qkv[:, 2 * hk:].view(-1, H, 128), up_bf16(p.g), up_bf16(p.beta),
                          up(batch.prefill_cu), pool0, si, o_pre)
        torch.cuda.synchronize()
        del qkv, o_pre

    # ---- one input set per layer: pool, activations, records, outputs
    sets = []
    for _ in range(L):
        qkv = up_bf16(batch.tokens.qkv)
        sets.append(dict(
            pool=pool0.clone(),
            q=qkv[:, :hk].view(ntok, H, 128), k=qkv[:, hk:2 * hk].view(ntok, H, 128),
            v=qkv[:, 2 * hk:].view(ntok, H, 128), g=up_bf16(batch.tokens.g),
            beta=up_bf16(batch.tokens.beta), rec=kda.allocate_records(B, H, Q, dev),
            o=torch.empty((ntok, H, 128), dtype=torch.bfloat16, device=dev), qkv=qkv))
    del pool0
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    # Each input set stands for one layer of the model: a step is the
    # serving order of one decode step, every layer's kda_verify (the forward
    # pass), then every layer's commit in one kda_commit_layers launch (after
    # sampling). With 12 sets the decode step touches 12 x 128 MiB of
    # checkpoints: the 256 MB MALL can carry at most the last two layers'
    # checkpoints from their verify to the commit.
    pools = [s["pool"] for s in sets]
    recs = [s["rec"] for s in sets]

    # the window bound a serving batch knows on the host (1 + num_spec)
    max_seqlen = int(T.max())

    def verify(s, st):
        kda.kda_verify(layer, s["q"], s["k"], s["v"], s["g"], s["beta"], cu, s["pool"], si,
                       s["rec"], s["o"], stream=st, max_seqlen=max_seqlen)

    align = None
    if args.align:
        # rows commit into blocks the sources do not use: c = 2 cached tokens
        # and 4-token blocks, so a row whose n' exceeds 2 crosses the boundary
        # at 2 (boundary store into column 0) and ends in column 1
        free = [b for b in range(1, batch.num_slots) if b not in set(int(x) for x in batch.state_indices)]
        if len(free) < 2 * B:
            raise SystemExit("--align needs two free pool blocks per row")
        bt = np.array(free[:2 * B], np.int32).reshape(B, 2)
        align = kda.Align(up(bt), up(np.full(B, 2, np.int32)), 4)

    def commit_one(s, st):
        if align is None:
            kda.kda_commit(layer, cu, s["pool"], si, s["rec"], nacc, stream=st)
        else:
            kda.kda_commit_layers([layer], cu, [s["pool"]], si, [s["rec"]], nacc, align=align,
                                  stream=st)

    def commit_all(st):
        if args.per_layer_commit:
            for s in sets:
                commit_one(s, st)
        else:
            kda.kda_commit_layers([layer] * L, cu, pools, si, recs, nacc, align=align, stream=st)

    def step(st, ev=None):
        for i, s in enumerate(sets):
            if ev is not None:
                ev[i].record(st)
            verify(s, st)
        if ev is not None:
            ev[L].record(st)
        commit_all(st)
        if ev is not None:
            ev[L + 1].record(st)

    for _ in range(max(1, W // L)):
        step(stream)
    torch.cuda.synchronize()

    # ---- timed region: K steps, events around every launch on the launch stream
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(L + 2)] for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(K):
        step(stream, ev[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    tv = np.array([e[i].elapsed_time(e[i + 1]) for e in ev for i in range(L)])
    tc = np.array([e[L].elapsed_time(e[L + 1]) for e in ev])

    n_commit = np.minimum(np.maximum(batch.num_accepted, 0), np.minimum(T, Q))
    vbytes, cbytes = algorithmic_bytes(T, n_commit, valid, H)
    if align is not None:
        # the boundary store (after 2 of the 4-token block) of rows with n' > 2
        cbytes += float(H * STATE_BYTES * np.sum(n_commit[valid] > 2))
    tok_verify = int(T[valid].sum())
    tok_commit = int(n_commit[valid].sum())
    ms_step = total_ms / K
    v_ms, c_ms = float(tv.mean()), float(tc.mean())
    commit_launches = L if args.per_layer_commit else 1
    commit_name = "kda_commit" if args.per_layer_commit and align is None else "kda_commit_layers"
    c_launch_bytes = cbytes * L / commit_launches
    c_launch_ms = c_ms / commit_launches
    # the counter runs used the default step (12 layers, in-place commit in
    # one launch); other shapes of the commit move other bytes
    default_shape = L == 12 and align is None and not args.per_layer_commit
    kernels = {
        "kda_verify": dict(launches_per_step=L, avg_us=v_ms * 1e3,
                           median_us=float(np.median(tv)) * 1e3, bytes=vbytes,
                           gbs=vbytes / (v_ms * 1e6), tokens_per_s=tok_verify / (v_ms * 1e-3),
                           traffic=measured_traffic("kda_verify", name)),
        commit_name: dict(launches_per_step=commit_launches, layers_per_launch=L // commit_launches,
                          avg_us=c_launch_ms * 1e3, median_us=float(np.median(tc)) / commit_launches * 1e3,
                          bytes=c_launch_bytes, gbs=c_launch_bytes / (c_launch_ms * 1e6),
                          tokens_per_s=tok_commit * L / (c_ms * 1e-3),
                          traffic=measured_traffic(commit_name, name) if default_shape else None),
    }
    for kinfo in kernels.values():
        kinfo["frac_of_peak"] = kinfo["gbs"] / PEAK_HBM_GBS
    # the dominant kernel: the one that takes the larger share of the step
    dom = "kda_verify" if L * v_ms >= c_ms else commit_name

    # ---- the step as a serving loop runs it: captured in one HIP graph
    # (every layer's verify, then the commit), replayed for exactly K steps.
    # The eager loop above gives the per-kernel times; this one the step.
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step(side)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(torch.cuda.current_stream())
    for _ in range(max(1, W // L)):
        graph.replay()
    torch.cuda.synchronize()
    g_start = torch.cuda.Event(enable_timing=True)
    g_end = torch.cuda.Event(enable_timing=True)
    g_start.record(stream)
    for i in range(K):
        graph.replay()
    g_end.record(stream)
    torch.cuda.synchronize()
    ms_step_graph = g_start.elapsed_time(g_end) / K
    ms_layer = ms_step_graph / L
    del graph

    step_bytes = L * (vbytes + cbytes)
    tshape = "ragged 1..8" if name == "ragged" else int(T.max())
    out = {
        "value": L * tok_verify / (ms_step_graph * 1e-3),
        "ms_per_step": ms_step_graph,
        "config": {
            "workload": f"{batch.name}: B={B} H={H} K=V=128 T={tshape} Q={Q}, bf16 activations, fp32 "
                        f"checkpoints, {'bounded gate lb=' + str(batch.lower_bound) if batch.lower_bound is not None else 'unbounded gate'}; "
                        f"a step = {L} layers (own pool, inputs and records each): every layer's "
                        f"kda_verify, then "
                        f"{'one kda_commit per layer' if args.per_layer_commit else 'one kda_commit_layers for all layers'}; "
                        f"value = verified tokens per second per layer call",
            "B": B, "H": H, "K": 128, "V": 128, "T": tshape, "window": Q, "layers_per_step": L,
            "max_seqlen": max_seqlen,
            "verified_tokens_per_layer": tok_verify, "committed_tokens_per_layer": tok_commit,
            "commit": "align mode (block table, destinations other than the sources)" if args.align
                      else "in place",
        },
        "dominant": dom,
        "kernels": kernels,
        "ms_per_layer_step": ms_layer,
        "step_gbs": step_bytes / (ms_step_graph * 1e6),
        "step_frac_of_peak": step_bytes / (ms_step_graph * 1e6) / PEAK_HBM_GBS,
        "step_timing": "HIP graph replay of whole steps; per-kernel times from HIP events around "
                       "eager launches",
        "ms_per_step_eager": ms_step,
        "value_eager": L * tok_verify / (ms_step * 1e-3),
        "commit_tokens_per_s": tok_commit * L / (c_ms * 1e-3),
        "verify_tokens_per_s": tok_verify / (v_ms * 1e-3),
    }
    if headline:
        out["interleaved"] = interleaved_leg(torch, sets, verify, commit_one, stream, K, L,
                                             tok_verify, vbytes + cbytes)
        if align is None:
            out["deferred_flow"] = decode_deferred_flow(
                args, torch, kda, layer, sets, cu, si, nacc, stream, T, n_commit, valid, H, B, Q,
                dev, tok_verify)
            out["stock_spec"] = stock_spec_leg(torch, kda, dev, batch, layer, sets, cu, stream, K,
                                               W, L, (L * v_ms + c_ms) / L, vbytes + cbytes)
    del sets, pools, recs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def interleaved_leg(torch, sets, verify, commit_one, stream, K, L, tok_verify, layer_bytes):
    """Context: one layer's verify then its own commit, back to back
    (kda_commit per layer). The commit then re-reads the checkpoints the
    verify has just read, partly from the MALL, and the next verify streams
    its checkpoints while that commit's new state is written back to HBM."""
    Ki = max(4, min(K, 60))
    evi = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(Ki)]
    for i in range(L):
        verify(sets[i], stream)
        commit_one(sets[i], stream)
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    for i in range(Ki):
        s = sets[i % L]
        evi[i][0].record(stream)
        verify(s, stream)
        evi[i][1].record(stream)
        commit_one(s, stream)
        evi[i][2].record(stream)
    a1.record(stream)
    torch.cuda.synchronize()
    ti_v = float(np.mean([e[0].elapsed_time(e[1]) for e in evi]))
    ti_c = float(np.mean([e[1].elapsed_time(e[2]) for e in evi]))
    ms_inter = a0.elapsed_time(a1) / Ki
    return {
        "ms_per_layer_step": ms_inter,
        "value": tok_verify / (ms_inter * 1e-3),
        "kda_verify_avg_us": ti_v * 1e3,
        "kda_commit_avg_us": ti_c * 1e3,
        "gbs": layer_bytes / (ms_inter * 1e6),
        "note": "each layer's verify followed at once by its own single-layer commit (eager "
                "launches); not the serving order",
    }


def spec_bytes(T, cols, valid, H):
    """Bytes of the stock speculative step (each counted once): per valid
    (row, head) the source state read, one state written per token in a
    column, each token's inputs and its output:
    65,536 (1 + min(T_i, cols)) + 1,282 T_i."""
    T = np.asarray(T)[valid]
    return float(H * np.sum(STATE_BYTES * (1 + np.minimum(T, cols)) + (TOKEN_IN_BYTES + OUT_BYTES) * T))


def stock_spec_leg(torch, kda, dev, batch, layer, sets, cu, stream, K, W, L, recover_ms_per_layer,
                   recover_bytes_per_layer):
    """The stock speculative step that RecoverSSM replaces, on the same
    activations: per layer one kda_recurrent_spec over 1 + num_spec columns
    of distinct blocks per request (its own pool per layer), which stores
    one full state per verified token. The source column of a row is its
    accepted count of the previous step minus one (the workload's counts,
    clamped to 1..cols). Events around every launch, K steps of L layers."""
    B, H = batch.num_rows, batch.H
    T = batch.seq_lens()
    cols = int(T.max())
    nslots = 1 + B * cols
    table = torch.arange(1, nslots, dtype=torch.int32, device=dev).view(B, cols)
    acc = torch.from_numpy(np.clip(batch.num_accepted, 1, cols).astype(np.int32)).to(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    pools = []
    for _ in range(L):
        pool = torch.empty((nslots, H, 128, 128), dtype=torch.float32, device=dev)
        pool.normal_(0.0, 0.02, generator=gen)
        pools.append(pool)

    def run(i, st):
        s = sets[i]
        kda.kda_recurrent_spec(layer, s["q"], s["k"], s["v"], s["g"], s["beta"], cu, pools[i], table,
                               acc, s["o"], stream=st)

    for _ in range(max(1, W // L)):
        for i in range(L):
            run(i, stream)
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(L)] for _ in range(K)]
    for k in range(K):
        for i in range(L):
            ev[k][i][0].record(stream)
            run(i, stream)
            ev[k][i][1].record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for row in ev for a, b in row])
    valid = batch.valid_rows()
    nbytes = spec_bytes(T, cols, valid, H)
    us = float(t.mean()) * 1e3
    del pools
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {
        "kda_recurrent_spec": dict(avg_us=us, median_us=float(np.median(t)) * 1e3, bytes=nbytes,
                                   gbs=nbytes / (us * 1e3), frac_of_peak=nbytes / (us * 1e3) / PEAK_HBM_GBS,
                                   columns=cols),
        "bytes_vs_verify_commit": nbytes / recover_bytes_per_layer,
        "time_vs_verify_commit": (us * 1e-3) / recover_ms_per_layer,
        "verify_commit_ms_per_layer": recover_ms_per_layer,
        "verify_commit_bytes_per_layer": recover_bytes_per_layer,
        "note": "per layer: the stock step (one state stored per verified token) against "
                "RecoverSSM's verify + commit on the same batch (their event times per layer)",
    }


def decode_deferred_flow(args, torch, kda, layer, sets, cu, si, nacc, stream, T, n_commit, valid,
                         H, B, Q, dev, tok_verify):
    """The same step in the deferred flow, in the same serving order: every
    layer's kda_verify_deferred (each folds the records its layer accepted
    in the previous step into the checkpoint, stores it and verifies), then
    one commit for all layers that only records this step's accepted counts
    as pending (no eager rows; the counts are per request, shared by the
    layers). Two record buffers per layer alternate. Timed like the eager
    step: events around eager launches for the kernels, HIP graphs for the
    step."""
    L = len(sets)
    for s in sets:
        s["recs"] = [s["rec"], kda.allocate_records(B, H, Q, dev)]
    pools = [s["pool"] for s in sets]
    rec_by_parity = [[s["recs"][par] for s in sets] for par in range(2)]
    pending = torch.zeros(B, dtype=torch.int32, device=dev)

    def dstep(c, st, ev=None):
        par = c % 2
        for i, s in enumerate(sets):
            if ev is not None:
                ev[i].record(st)
            kda.kda_verify_deferred(layer, s["q"], s["k"], s["v"], s["g"], s["beta"], cu, s["pool"],
                                    si, s["recs"][1 - par], pending, s["recs"][par], s["o"], stream=st)
        if ev is not None:
            ev[L].record(st)
        if args.per_layer_commit:
            for s in sets:
                kda.kda_commit(layer, cu, s["pool"], si, s["recs"][par], nacc, pending=pending,
                               stream=st)
        else:
            kda.kda_commit_layers([layer] * L, cu, pools, si, rec_by_parity[par], nacc,
                                  pending=pending, stream=st)
        if ev is not None:
            ev[L + 1].record(st)

    K = args.steps
    c = 0
    for _ in range(max(2, args.warmup // L)):   # every layer has pending counts
        dstep(c, stream)
        c += 1
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(L + 2)] for _ in range(K)]
    for i in range(K):
        dstep(c, stream, ev[i])
        c += 1
    torch.cuda.synchronize()
    tv = np.array([e[i].elapsed_time(e[i + 1]) for e in ev for i in range(L)])
    tc = np.array([e[L].elapsed_time(e[L + 1]) for e in ev])

    # one graph per record parity, replayed alternately as the eager loop ran
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for j in range(2):
            dstep(c + j, side)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    c += 2
    graphs = {}
    for j in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            dstep(c + j, torch.cuda.current_stream())
        graphs[(c + j) % 2] = g
    for _ in range(max(2, args.warmup // L)):
        graphs[c % 2].replay()
        c += 1
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(K):
        graphs[c % 2].replay()
        c += 1
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / K
    zeros = np.zeros(B, np.uint8)
    _, vdef, _ = deferred_bytes(T, n_commit, zeros, n_commit, zeros, valid, H)
    v_ms = float(tv.mean())
    return {
        "ms_per_step": ms,
        "ms_per_layer_step": ms / L,
        "value": L * tok_verify / (ms * 1e-3),
        "layer_step_bytes": vdef,
        "step_gbs": L * vdef / (ms * 1e6),
        "kda_verify_deferred": dict(avg_us=v_ms * 1e3, median_us=float(np.median(tv)) * 1e3,
                                    bytes=vdef, gbs=vdef / (v_ms * 1e6),
                                    frac_of_peak=vdef / (v_ms * 1e6) / PEAK_HBM_GBS,
                                    traffic=measured_traffic("kda_verify_deferred", "decode")),
        "kda_commit_deferring": dict(launches_per_step=L if args.per_layer_commit else 1,
                                     avg_us=float(tc.mean()) * 1e3,
                                     median_us=float(np.median(tc)) * 1e3),
        "note": "every layer's kda_verify_deferred folds the records its layer accepted in the "
                "previous step (the counts repeat) and stores the checkpoint, then verifies; the "
                "commit then writes only the pending counts",
    }


def device_copy_gbs(torch, stream) -> float:
    """The achievable copy bandwidth on this GPU (context for the peak): a
    plain 1 GiB device copy, timed 10 times; also what the counter
    calibration of --summarize-pmc finds in a profile of this benchmark."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=stream.device)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    gbs = 10 * 2 * src.numel() * 4 / (e0.elapsed_time(e1) * 1e6)
    del src, dst
    return gbs


def deferred_bytes(T, n_prev, eager_prev, n_now, eager_now, valid, H):
    """Bytes of one layer-step of each flow (each counted once).

    eager:    verify (65,536 + 2,052 T) + commit (131,072 + 770 n' when n' > 0).
    deferred: kda_verify_deferred folds the previous step's pending p records
              (p = n' of the previous step unless that row was eager): 65,536
              + [p > 0] 65,536 + 770 p + 2,052 T; then kda_commit writes pending
              and commits the eager rows now: 131,072 + 770 n' for those."""
    T = np.asarray(T)[valid]
    p = np.where(np.asarray(eager_prev)[valid] != 0, 0, np.asarray(n_prev)[valid])
    n = np.asarray(n_now)[valid]
    e = np.asarray(eager_now)[valid] != 0
    per_tok = TOKEN_IN_BYTES + OUT_BYTES + REC_BYTES
    verify = H * np.sum(STATE_BYTES + per_tok * T)
    commit = H * np.sum(np.where(n > 0, 2 * STATE_BYTES + REC_BYTES * n, 0))
    vdef = H * np.sum(STATE_BYTES + np.where(p > 0, STATE_BYTES + REC_BYTES * p, 0) + per_tok * T)
    cdef = H * np.sum(np.where(e & (n > 0), 2 * STATE_BYTES + REC_BYTES * n, 0))
    return float(verify + commit), float(vdef), float(cdef)


def deferred_leg(args, torch, kda, dev):
    """Many layers, many steps: the eager flow (kda_verify for every layer,
    then kda_commit for every layer) against the deferred flow
    (kda_verify_deferred for every layer, folding the previous step's pending
    commit, then kda_commit in deferred mode, which records pending counts and
    commits the eager rows now). B=512, H=32, T=Q=4, 8 layers, each with its
    own pool of 513 slots (1 GiB) and its own records. The checkpoints are
    N(0, 0.02) drawn on the device with torch's seeded generator (the same
    distribution as the parity recipe, drawn faster); tokens are the
    workload's per-layer draws of step 0, reused every step."""
    from workloads import make_deferred
    run = make_deferred()
    B, H, Q, T, L = run.B, run.H, run.Q, run.T, run.layers
    ntok = B * T
    hk = H * 128

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    def up_bf16(bits):
        return up(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)

    gen = torch.Generator(device=dev)
    gen.manual_seed(run.seed)
    si, rr, cu = up(run.state_indices), up(run.record_rows), up(run.cu_seqlens)
    layers, pools, toks, recs = [], [], [], []
    for l in range(L):
        p = run.params[l]
        layers.append(kda.Layer(a_log=up(p.a_log), g_bias=up(p.g_bias), scale=run.scale,
                                lower_bound=run.lower_bound))
        pool = torch.zeros((run.num_slots, H, 128, 128), dtype=torch.float32, device=dev)
        pool[1:].normal_(0.0, 0.02, generator=gen)
        pools.append(pool)
        t = run.tokens(l, 0)
        qkv = up_bf16(t.qkv)
        toks.append((qkv[:, :hk].view(ntok, H, 128), qkv[:, hk:2 * hk].view(ntok, H, 128),
                     qkv[:, 2 * hk:].view(ntok, H, 128), up_bf16(t.g), up_bf16(t.beta), qkv))
        recs.append([kda.allocate_records(B, H, Q, dev), kda.allocate_records(B, H, Q, dev)])
    o = torch.empty((ntok, H, 128), dtype=torch.bfloat16, device=dev)
    pending = torch.zeros(B, dtype=torch.int32, device=dev)
    S = run.steps
    nacc = [up(run.num_accepted(s)) for s in range(S)]
    eag = [up(run.eager(s)) for s in range(S)]
    stream = torch.cuda.current_stream()

    rec0 = [recs[l][0] for l in range(L)]
    rec_by_parity = [[recs[l][c] for l in range(L)] for c in range(2)]

    def eager_step(s, ev=None):
        for l in range(L):
            kda.kda_verify(layers[l], *toks[l][:5], cu, pools[l], si, recs[l][0], o,
                           record_rows=rr, stream=stream, max_seqlen=T)
        if args.per_layer_commit:
            for l in range(L):
                kda.kda_commit(layers[l], cu, pools[l], si, recs[l][0], nacc[s % S],
                               record_rows=rr, stream=stream)
        else:   # every layer's commit in one launch
            kda.kda_commit_layers(layers, cu, pools, si, rec0, nacc[s % S], record_rows=rr,
                                  stream=stream)

    def deferred_step(s, ev=None):
        cur = s % 2
        for l in range(L):
            if ev is not None:
                ev[l][0].record(stream)
            kda.kda_verify_deferred(layers[l], *toks[l][:5], cu, pools[l], si, recs[l][1 - cur],
                                    pending, recs[l][cur], o, record_rows=rr, stream=stream)
            if ev is not None:
                ev[l][1].record(stream)
        if args.per_layer_commit:
            for l in range(L):
                kda.kda_commit(layers[l], cu, pools[l], si, recs[l][cur], nacc[s % S],
                               record_rows=rr, pending=pending, eager=eag[s % S], stream=stream)
        else:
            kda.kda_commit_layers(layers, cu, pools, si, rec_by_parity[cur], nacc[s % S],
                                  record_rows=rr, pending=pending, eager=eag[s % S], stream=stream)

    def timed(fn, K, with_events=False):
        W = args.warmup
        for s in range(W):
            fn(s)
        torch.cuda.synchronize()
        evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(L)]
               for _ in range(K)] if with_events else [None] * K
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(K):
            fn(W + i, evs[i])   # step numbers continue, so the record buffers alternate
        b.record(stream)
        torch.cuda.synchronize()
        kt = None
        if with_events:
            kt = float(np.mean([e[0].elapsed_time(e[1]) for step in evs for e in step]))
        return a.elapsed_time(b) / K, kt

    K = max(4, min(args.steps, 40))
    ms_e, _ = timed(eager_step, K)
    pending.zero_()
    ms_d, kt_vd = timed(deferred_step, K, with_events=True)

    # ---- the conv-state half of the commit for every layer in one launch:
    # the short convolutions before q, k and v (3 H K channels, bf16), kernel
    # 4 (history 3), the token axis holding history - 1 + Q columns
    hist = 3
    conv_dim = 3 * hk
    convs = []
    for _ in range(L):
        cst = torch.empty((run.num_slots, conv_dim, Q + hist - 1), dtype=torch.bfloat16, device=dev)
        cst.normal_(generator=gen)
        convs.append(cst)
    for s in range(args.warmup):
        kda.kda_conv_compact(convs, cu, si, nacc[s % S], Q, hist, stream=stream)
    torch.cuda.synchronize()
    cev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for i in range(K):
        cev[i][0].record(stream)
        kda.kda_conv_compact(convs, cu, si, nacc[i % S], Q, hist, stream=stream)
        cev[i][1].record(stream)
    torch.cuda.synchronize()
    conv_us = float(np.mean([a.elapsed_time(b) for a, b in cev])) * 1e3
    copy_gbs = device_copy_gbs(torch, stream)
    conv_bytes = float(np.mean([
        L * conv_dim * hist * 2 * 2 * np.sum((np.minimum(np.maximum(run.num_accepted(s), 0), Q) > 0)
                                            & (run.state_indices > 0))
        for s in range(S)]))
    del convs

    valid = run.state_indices > 0
    Tv = np.full(B, T)
    be, bvd, bcd = [], [], []
    for s in range(S):
        n_prev = np.minimum(np.maximum(run.num_accepted((s - 1) % S), 0), Q)
        n_now = np.minimum(np.maximum(run.num_accepted(s), 0), Q)
        e_, v_, c_ = deferred_bytes(Tv, n_prev, run.eager((s - 1) % S), n_now, run.eager(s), valid, H)
        be.append(e_); bvd.append(v_); bcd.append(c_)
    b_eager, b_vdef, b_cdef = float(np.mean(be)), float(np.mean(bvd)), float(np.mean(bcd))
    per_layer_e, per_layer_d = ms_e / L, ms_d / L
    gbs_vd = b_vdef / (kt_vd * 1e6)
    return {
        "metric": "KDA verify+commit tokens/s and achieved HBM GB/s vs peak (B=64,H=32,T=4)",
        "value": B * T * L / (ms_d * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_d,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {
            "workload": f"deferred: B={B} H={H} K=V=128 T={T} Q={Q}, {L} layers (own 1 GiB pool and "
                        f"records each); a step = every layer's verify, then every layer's commit "
                        f"({'one launch per layer' if args.per_layer_commit else 'one launch for all layers'})",
            "B": B, "H": H, "K": 128, "V": 128, "T": T, "window": Q, "layers": L,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "kda_verify_deferred",
            "achieved": gbs_vd,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": gbs_vd / PEAK_HBM_GBS,
            "traffic": measured_traffic("kda_verify_deferred", "deferred"),
        },
        "flows": {
            "eager": {"ms_per_layer_step": per_layer_e, "bytes_per_layer_step": b_eager,
                      "gbs": b_eager / (per_layer_e * 1e6)},
            "deferred": {"ms_per_layer_step": per_layer_d,
                         "bytes_per_layer_step": b_vdef + b_cdef,
                         "gbs": (b_vdef + b_cdef) / (per_layer_d * 1e6),
                         "kda_verify_deferred_avg_us": kt_vd * 1e3},
        },
        "deferred_speedup": per_layer_e / per_layer_d,
        "kda_conv_compact": {"layers": L, "channels": conv_dim, "history": hist, "avg_us": conv_us,
                             "bytes": conv_bytes, "gbs": conv_bytes / (conv_us * 1e3)},
        "copy_gbs_measured": copy_gbs,
    }


def cpu_baselines_other(seconds):
    """The oracle on bounded samples of the other workloads, one thread each:
    the tiny batch whole, 32 of the ragged batch's 128 rows, and the
    deferred workload's sequential replay (layer 0, 16 of 512 requests, all
    4 steps: each step's verify, then the commit of the accepted prefix)."""
    from workloads import make_batch
    out = {"tiny": cpu_baseline(make_batch("tiny"), 4, seconds),
           "ragged": cpu_baseline(make_batch("ragged"), 32, seconds),
           "deferred": cpu_replay_deferred(16, seconds)}
    return out


def cpu_replay_deferred(rows, seconds):
    from threadpoolctl import threadpool_limits
    from oracle import kda_ref as ref
    from workloads import make_deferred
    run = make_deferred()
    B, H, Q, K = run.B, run.H, run.Q, 128
    p = run.params[0]
    lay = ref.Layer(p.a_log, p.g_bias, run.scale, run.lower_bound)
    # a compact pool: the sampled requests' checkpoints in slots 1..rows
    si = np.zeros(B, np.int32)
    si[:rows] = np.arange(1, rows + 1)
    pool0 = np.zeros((rows + 1, H, K, K), np.float32)
    for i in range(rows):
        pool0[i + 1] = run.slot_state(0, int(run.state_indices[i]))
    toks = [run.tokens(0, s) for s in range(run.steps)]
    accs = [run.num_accepted(s) for s in range(run.steps)]
    ntok = B * run.T
    n_tok = rows * run.T * run.steps
    walls = []
    with threadpool_limits(1):
        while sum(walls) < seconds or len(walls) < 1:
            pool = pool0.copy()
            t0 = time.perf_counter()
            for s in range(run.steps):
                t = toks[s]
                rec = ref.Records.empty(B, H, Q, K)
                o = np.zeros((ntok, H, K), np.uint16)
                ref.kda_verify(lay, t.q, t.k, t.v, t.g, t.beta, run.cu_seqlens, pool, si, rec, o,
                               record_rows=run.record_rows)
                ref.kda_commit(lay, run.cu_seqlens, ntok, pool, si, rec, accs[s],
                               record_rows=run.record_rows)
            walls.append(time.perf_counter() - t0)
    wall = float(np.median(walls))
    return {"value": n_tok / wall, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"sequential replay of layer 0 for {rows} of {B} requests over {run.steps} "
                      f"steps ({n_tok} tokens, all {H} heads; each step's verify then commit), "
                      f"NumPy fp64 on one thread, median of {len(walls)} runs ({wall:.2f} s each)",
            "host_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline(batch, rows, seconds):
    """The oracle (NumPy fp64), as it stands, on the first `rows` rows of the
    same workload: verify then commit, single-threaded, repeated until
    `seconds` of wall time; scaled to tokens/s."""
    from threadpoolctl import threadpool_limits
    from oracle import kda_ref as ref

    rows = min(rows, batch.num_rows)
    lay = ref.Layer(batch.a_log, batch.g_bias, batch.scale, batch.lower_bound)
    sel = np.zeros(batch.num_rows, bool)
    sel[:rows] = True
    si = np.where(sel, batch.state_indices, 0).astype(np.int32)
    pool0 = batch.initial_pool()
    if batch.init == "prefill":     # the sample's checkpoints, by the oracle (untimed)
        p = batch.prefill
        ref.kda_recurrent(lay, p.q, p.k, p.v, p.g, p.beta, batch.prefill_cu, pool0, si,
                          np.zeros((p.num_tokens, batch.H, 128), np.uint16))
    t = batch.tokens
    T = batch.seq_lens()
    toks = int(T[sel & (batch.state_indices > 0)].sum())
    walls = []
    with threadpool_limits(1):
        while sum(walls) < seconds or len(walls) < 1:
            pool = pool0.copy()
            rec = ref.Records.empty(batch.num_rows, batch.H, batch.Q, 128)
            o = np.zeros((t.num_tokens, batch.H, 128), np.uint16)
            t0 = time.perf_counter()
            ref.kda_verify(lay, t.q, t.k, t.v, t.g, t.beta, batch.cu_seqlens, pool, si, rec, o)
            ref.kda_commit(lay, batch.cu_seqlens, t.num_tokens, pool, si, rec,
                           batch.num_accepted)
            walls.append(time.perf_counter() - t0)
    wall = float(np.median(walls))
    return {"value": toks / wall, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"verify+commit of {rows} of {batch.num_rows} rows ({toks} tokens, all "
                      f"{batch.H} heads), NumPy fp64 on one thread, median of {len(walls)} runs "
                      f"({wall:.2f} s each)",
            "host_cpus": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
