#!/usr/bin/env python3
"""Benchmark of one SparSTAR attention scale on one MI355X.

A step is the whole hot path over one batch of synthetic input already
resident in HBM: block means of Q and K, block scores with clip-aware top-k
selection (the screened route: float16 screened scores in a workspace and
exact scores for the blocks that decide a row; --two-step materialises the
float32 score matrix instead, with the same selection) and block-sparse
attention forward, on one stream.  The default workload is the 72,000-token final scale (16 heads,
D = 128, bf16, keys = 512 text + 72,000 reference + 72,000 current, density
0.09375).

Printed: one JSON line.  `value` is selected-block attention TFLOP/s over the
whole step (selected FLOPs / ms per scale); `ms_per_step` is ms per scale
(score + select + attn).  `roofline` is for the attention kernel (bf16 MFMA
peak), with its duration from HIP events recorded on the launch stream.  By
default every timed step starts with L2 and MALL cold (a 512 MiB overwrite
before it, outside the timed region); `other_cache` holds the warm
(back-to-back) figures, or the cold ones under --warm.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "selected-block attn TFLOP/s + ms per scale (score+select+attn) at 72k tokens"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic.txt")
# the attention kernel's sources and build flags: counters are valid only for
# this exact code
ATTN_SOURCES = [os.path.join(ROOT, "block_sparse_attention_head_amd", "csrc", f)
                for f in ("attn_fwd_bf16.hip", "tile_common.hpp", "common.hpp")] + \
               [os.path.join(ROOT, "include", "sparstar.h")]


def attn_source_sha():
    from block_sparse_attention_head_amd.build import compile_flags
    h = hashlib.sha256()
    for path in ATTN_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    # the flags name the include directory by absolute path; hash it relative
    # to the repository so that a copy elsewhere gives the same key
    from block_sparse_attention_head_amd import build as _build
    flags = " ".join(compile_flags()).replace(os.path.abspath(_build.ROOT), "<root>")
    h.update(flags.encode())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def selected_flops(kv_count, kv_index, Nq, Nk, D, block=128):
    """4*D * sum over rows of valid queries x valid keys of the kept blocks."""
    cnt = kv_count.reshape(-1).astype(np.int64)
    idx = kv_index.reshape(cnt.size, -1).astype(np.int64)
    nqb = -(-Nq // block)
    nkb = -(-Nk // block)
    pos = np.arange(idx.shape[1])[None, :]
    valid = (pos < cnt[:, None]) & (idx >= 0) & (idx < nkb)
    keys = np.where(valid, np.minimum((idx + 1) * block, Nk) - idx * block, 0).sum(axis=1)
    rows_i = np.arange(cnt.size) % nqb
    nq = np.minimum((rows_i + 1) * block, Nq) - rows_i * block
    return int(4 * D * (nq * keys).sum())


def stage_bytes(w, kept, nqb, nkb):
    """Algorithmic bytes of means(Q) + means(K) + scores + select."""
    el = 2 if w.dtype == "bf16" else 4
    BH = w.B * w.H
    qk = BH * (w.Nq + w.Nk) * w.D * el
    means = 2 * BH * (nqb + nkb) * w.D * 4
    index = BH * nqb * (4 * kept + 4)
    return qk + means + index


def traffic_for_attention(workload_name):
    """HBM bytes per attention launch from committed rocprofv3 counter runs
    (calibrated FETCH_SIZE + WRITE_SIZE), or None when they were taken on
    another workload or the kernel source changed since."""
    try:
        rec = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if line.startswith("#") or ":" not in line:
                    continue
                key, val = line.split(":", 1)
                rec[key.strip()] = val.strip()
        if rec.get("source_sha256") != attn_source_sha() or rec.get("workload") != workload_name:
            return None
        return int(float(rec["hbm_bytes_per_launch"]))
    except (OSError, ValueError, KeyError):
        return None


def cpu_model():
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(x, w, kept_F, budget_s):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover
        affinity = None
    F = kept_F
    t0 = time.perf_counter()
    qd = oracle.decode(x["q"][0:1, 0:1], w.dtype)
    kd = oracle.decode(x["k"][0:1, 0:1], w.dtype)
    vd = oracle.decode(x["v"][0:1, 0:1], w.dtype)
    qbar = oracle.block_means(qd)
    kbar = oracle.block_means(kd)
    S = oracle.block_scores(qbar, kbar)
    cnt, idx = oracle.select_blocks(S, F, w.density)
    t_sel = time.perf_counter() - t0
    rows, t_att = [], 0.0
    i = 0
    while i < w.nqb and (t_att + t_sel < budget_s or len(rows) < 2):
        t1 = time.perf_counter()
        oracle.sparse_attention_rows(qd, kd, vd, cnt, idx, [(0, 0, i)])
        t_att += time.perf_counter() - t1
        rows.append(i)
        i += 1
    sub_cnt = cnt[0, 0, rows]
    sub_idx = idx[0, 0, rows]
    fl = 0
    for r, ii in enumerate(rows):
        nq = min((ii + 1) * 128, w.Nq) - ii * 128
        ks = sum(min((int(j) + 1) * 128, w.Nk) - int(j) * 128 for j in sub_idx[r, :sub_cnt[r]])
        fl += 4 * int(w.D) * int(nq) * int(ks)
    t_rows = t_att + t_sel * len(rows) / w.nqb
    per_scale_s = (t_sel + t_att / len(rows) * w.nqb) * w.B * w.H
    return {
        "value": fl / t_rows / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "blas_threads": int(threads),
        "os_cpu_count": os.cpu_count(),
        "cpus_in_affinity": affinity,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"batch 0 head 0 of {w.B}x{w.H}: means+scores+selection for the head "
                   f"({t_sel:.2f} s), attention for the first {len(rows)} of {w.nqb} query "
                   f"blocks ({t_att:.2f} s); value = their selected FLOPs / (attention time + "
                   f"their share of the head's selection time)"),
        "ms_per_scale_extrapolated": per_scale_s * 1e3,
        "seconds": t_sel + t_att,
    }


def mass_diagnostic(sp, torch, x, w, q, k, v, cnt, idx, F, kept, sample_blocks=4):
    """Retained attention mass of the selection and its token-wise Top-K
    bound at the same budget (GPU, every query; bf16 inputs), and on a sample
    of query blocks of head 0 the oracle's mass and bound beside them."""
    import oracle
    mass = sp.selection_retained_mass(q, k, v, cnt, idx)
    torch.cuda.synchronize()
    m = mass.float().cpu().numpy().reshape(-1)
    qd = oracle.decode(x["q"][0:1, 0:1], w.dtype)
    kd = oracle.decode(x["k"][0:1, 0:1], w.dtype)
    blocks = sorted({int(round(j)) for j in np.linspace(0, w.nqb - 1, sample_blocks)})
    rows = [(0, 0, i) for i in blocks]
    c_np, i_np = cnt[0:1, 0:1].cpu().numpy(), idx[0:1, 0:1].cpu().numpy()
    t0 = time.perf_counter()
    om = oracle.retained_mass_rows(qd, kd, c_np, i_np, rows)
    ub = oracle.token_topk_bound_rows(qd, kd, F, kept - F, rows)
    secs = time.perf_counter() - t0
    om_all = np.concatenate([om[r] for r in rows])
    ub_all = np.concatenate([ub[r] for r in rows])
    gm = mass[0, 0].float().cpu().numpy()
    g_rows = np.concatenate([gm[i * 128:i * 128 + om[(0, 0, i)].size] for (_, _, i) in rows])
    out = {
        "retained_mass_mean": round(float(m.mean()), 5),
        "retained_mass_p05": round(float(np.quantile(m, 0.05)), 5),
        "retained_mass_min": round(float(m.min()), 5),
        "sample": f"head 0, query blocks {blocks}: oracle fp64 ({secs:.1f} s)",
        "sample_mass_gpu": round(float(g_rows.mean()), 5),
        "sample_mass_oracle": round(float(om_all.mean()), 5),
        "sample_token_topk_bound": round(float(ub_all.mean()), 5),
        "sample_mass_over_bound": round(float(om_all.mean() / ub_all.mean()), 5),
    }
    if w.dtype == "bf16":
        # the token-wise bound for every query on the GPU (the sample checks it)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        bound = sp.token_topk_bound(q, k, F, kept - F)
        ev[1].record()
        torch.cuda.synchronize()
        b_np = bound.float().cpu().numpy()
        gb_rows = np.concatenate([b_np[0, 0, i * 128:i * 128 + ub[(0, 0, i)].size] for (_, _, i) in rows])
        out.update({
            "sample_bound_gpu_max_abs_diff": float(np.abs(gb_rows - ub_all).max()),
            "token_topk_bound_mean": round(float(b_np.mean()), 5),
            "mass_over_bound": round(float(m.mean() / b_np.mean()), 5),
            "token_topk_bound_ms": round(ev[0].elapsed_time(ev[1]), 1),
        })
    return out


def mask_reuse_diagnostic(sp, torch, w, q, k, v, F, kept, fresh_cnt, fresh_idx):
    """The mask-reuse baseline at this scale: the selection carried over from
    the preceding sparsified scale of the same clip, and from the same scale
    of the preceding clip, against the fresh one (retained attention mass and
    block overlap), plus the transfer kernel's time."""
    import dataclasses
    from workloads import make_inputs
    from workloads.configs import SWEEP_SCALES, SWEEP_DENSITIES
    if w.Nq not in SWEEP_SCALES or SWEEP_SCALES.index(w.Nq) == 0:
        return None
    prev = SWEEP_SCALES[SWEEP_SCALES.index(w.Nq) - 1]
    dev = q.device

    def scores_of(ws):
        xs = make_inputs(ws)
        qs = torch.from_numpy(xs["q"].view(np.int16)).view(torch.bfloat16).to(dev)
        ks = torch.from_numpy(xs["k"].view(np.int16)).view(torch.bfloat16).to(dev)
        return sp.block_scores(sp.block_means(qs), sp.block_means(ks))

    dst = (w.n_text, w.n_ref, w.n_cur)
    sources = {
        # preceding scale of the same clip (its reference scales with it
        # unless it is Clip 1's fixed image reference)
        "previous_scale": dataclasses.replace(
            w, name=f"{w.name}-prev-scale", Nq=prev, n_cur=prev,
            n_ref=w.n_ref if w.ref_forced else prev,
            density=SWEEP_DENSITIES[SWEEP_SCALES.index(prev)]),
        # the same scale of the preceding clip: an independent draw
        "previous_clip": dataclasses.replace(w, name=f"{w.name}-prev-clip", seed=w.seed + 1),
    }
    fresh_mass = sp.selection_retained_mass(q, k, v, fresh_cnt, fresh_idx)
    fc, fi = fresh_cnt.cpu().numpy(), fresh_idx.cpu().numpy()
    out = {"fresh_mass_mean": round(float(fresh_mass.float().mean()), 5)}
    for tag, ws in sources.items():
        S_src = scores_of(ws)
        src = (ws.n_text, ws.n_ref, ws.n_cur)
        S_dst = sp.transfer_scores(S_src, src, dst)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(10):
            sp.transfer_scores(S_src, src, dst, out=S_dst)
        ev[1].record()
        torch.cuda.synchronize()
        t_us = ev[0].elapsed_time(ev[1]) * 100.0
        nbytes = 4 * (S_dst.numel() + S_src.numel())
        rc, ri = sp.select_blocks(S_dst, F, w.density, max_kept=kept)
        m = sp.selection_retained_mass(q, k, v, rc, ri).float().cpu().numpy()
        rc_np, ri_np = rc.cpu().numpy(), ri.cpu().numpy()
        shared = 0
        for r in range(fc.size):
            a = fi.reshape(fc.size, -1)[r, :fc.reshape(-1)[r]]
            b = ri_np.reshape(rc_np.size, -1)[r, :rc_np.reshape(-1)[r]]
            shared += np.intersect1d(a[a >= F], b[b >= F]).size
        ranked = int(np.maximum(fc.reshape(-1) - F, 0).sum())
        out[tag] = {
            "source": f"n_text={src[0]} n_ref={src[1]} n_cur={src[2]} (seed {ws.seed})",
            "reused_mass_mean": round(float(m.mean()), 5),
            "reused_mass_p05": round(float(np.quantile(m, 0.05)), 5),
            "ranked_blocks_shared_with_fresh": round(shared / max(ranked, 1), 4),
            "transfer_us": round(t_us, 2),
            "transfer_gbps": round(nbytes / (t_us * 1e-6) / 1e9, 1),
        }
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="final-72k")
    ap.add_argument("--warm", action="store_true",
                    help="headline from back-to-back steps (warm L2/MALL); by default every "
                         "timed step follows a 512 MiB overwrite (cold L2/MALL), and the other "
                         "mode is reported beside it")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline sample")
    ap.add_argument("--block", type=int, default=128, choices=[32, 64, 128],
                    help="block size in tokens (the pages use 128)")
    ap.add_argument("--two-step", action="store_true",
                    help="scores (float32 S in HBM) then selection, instead of the screened "
                         "route (sparstar_select_blocks_from_means, the same selection)")
    ap.add_argument("--from-means", action="store_true",
                    help="run the selection stage as three calls (means of Q, means of K, "
                         "screened selection) instead of one call from Q and K")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step recorded as one HIP graph and replayed")
    ap.add_argument("--no-diagnostics", action="store_true",
                    help="skip the retained-attention-mass diagnostic (outside the timed region)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the SparSTAR hot path here has no multi-GPU "
              "mode (heads would shard across GPUs with no communication).", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_head_amd as sp
    from workloads import make_inputs, workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}), flush=True)
        return

    w = workload(args.workload)
    log(f"[bench] generating {w.name} inputs")
    x = make_inputs(w)

    def dev_t(a):
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q, k, v = dev_t(x["q"]), dev_t(x["k"]), dev_t(x["v"])
    B, H, D = w.B, w.H, w.D
    blk = args.block
    nqb, nkb = -(-w.Nq // blk), -(-w.Nk // blk)
    F = sp.forced_blocks(w.n_forced_tokens, blk)
    kept = sp.kept_blocks(nkb, F, w.density)
    f32, i32 = torch.float32, torch.int32
    qbar = torch.empty((B, H, nqb, D), dtype=f32, device=dev)
    kbar = torch.empty((B, H, nkb, D), dtype=f32, device=dev)
    fused = not args.two_step and nkb <= sp.FUSED_MAX_NKB
    S = None if fused else torch.empty((B, H, nqb, nkb), dtype=f32, device=dev)
    ws = sp.select_workspace(B, H, nqb, nkb, dev) if fused else None
    cnt = torch.empty((B, H, nqb), dtype=i32, device=dev)
    idx = torch.empty((B, H, nqb, max(1, kept)), dtype=i32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, w.Nq), dtype=f32, device=dev)
    stream = torch.cuda.current_stream()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    if fused and not args.from_means:
        names = ["select_from_qk", "attn"]
        calls = [lambda: sp.select_blocks_from_qk(q, k, F, w.density, block=blk, max_kept=kept,
                                                  qbar=qbar, kbar=kbar, kv_count=cnt,
                                                  kv_index=idx, workspace=ws),
                 lambda: sp.block_sparse_attn_fwd(q, k, v, cnt, idx, block=blk, out=o, lse=lse)]
    elif fused:
        names = ["means_q", "means_k", "screened_select", "attn"]
        calls = [lambda: sp.block_means(q, blk, out=qbar),
                 lambda: sp.block_means(k, blk, out=kbar),
                 lambda: sp.select_blocks_from_means(qbar, kbar, F, w.density, max_kept=kept,
                                                     kv_count=cnt, kv_index=idx,
                                                     workspace=ws),
                 lambda: sp.block_sparse_attn_fwd(q, k, v, cnt, idx, block=blk, out=o, lse=lse)]
    else:
        names = ["means_q", "means_k", "scores", "select", "attn"]
        calls = [lambda: sp.block_means(q, blk, out=qbar),
                 lambda: sp.block_means(k, blk, out=kbar),
                 lambda: sp.block_scores(qbar, kbar, out=S),
                 lambda: sp.select_blocks(S, F, w.density, max_kept=kept, kv_count=cnt,
                                          kv_index=idx),
                 lambda: sp.block_sparse_attn_fwd(q, k, v, cnt, idx, block=blk, out=o, lse=lse)]

    def step(ev=None, per_call=False):
        """One scale.  ev: events recorded on the launch stream before the
        first call, before the attention call and at the end (per_call: also
        before every other call)."""
        last = len(calls) - 1
        for i, c in enumerate(calls):
            if ev and (per_call or i == 0 or i == last):
                ev[i].record(stream)
            c()
        if ev: ev[len(calls)].record(stream)

    def measure(cold, steps):
        """ms per step and mean ms of the selection stage and of attention.
        Cold: each step follows an overwrite of 512 MiB (L2 and MALL hold
        none of its inputs) and is timed on its own; warm: `steps` steps back
        to back between two events.  Stage times come from a second pass
        with events only at the stage boundaries on the launch stream."""
        if cold:
            per = []
            for _ in range(steps):
                flush.fill_(0)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                step()
                b.record(stream)
                b.synchronize()
                per.append(a.elapsed_time(b))
            ms = float(np.mean(per))
        else:
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(steps):
                step()
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / steps
        n = len(calls)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]
        for e in evs:
            if cold:
                flush.fill_(0)
            step(e)
        torch.cuda.synchronize()
        stages = {"selection": float(np.mean([e[0].elapsed_time(e[n - 1]) for e in evs])),
                  "attn": float(np.mean([e[n - 1].elapsed_time(e[n]) for e in evs]))}
        return ms, stages

    def breakdown(cold, steps):
        """Mean ms per selection call, an event before and after every call
        (the events themselves add a few microseconds per call)."""
        n = len(calls)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]
        for e in evs:
            if cold:
                flush.fill_(0)
            step(e, per_call=True)
        torch.cuda.synchronize()
        return {nm: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs]))
                for i, nm in enumerate(names[:-1])}

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    primary_cold = not args.warm
    log(f"[bench] timing {args.steps} steps ({'cold' if primary_cold else 'warm'} cache)")
    ms_per_step, stage_ms = measure(primary_cold, args.steps)
    calls_ms = breakdown(primary_cold, min(args.steps, 10))

    graph_ms = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        graph_ms = a.elapsed_time(b) / args.steps

    # the other cache mode, labelled, beside the headline
    other_steps = min(args.steps, 10)
    log(f"[bench] {'warm' if primary_cold else 'cold'}-cache pass ({other_steps} steps)")
    o_ms, o_stage = measure(not primary_cold, other_steps)
    o_sel = o_stage["selection"]
    other = {"cache": "warm" if primary_cold else "cold",
             "ms_per_step": round(o_ms, 4),
             "selection_us": round(o_sel * 1e3, 2), "attn_us": round(o_stage["attn"] * 1e3, 2),
             "selection_frac_hbm": round(stage_bytes(w, kept, nqb, nkb) / (o_sel * 1e-3) / 1e9
                                         / PEAK_HBM_GBPS, 4),
             "steps": other_steps}
    del flush

    kv_count = cnt.cpu().numpy()
    kv_index = idx.cpu().numpy()
    flops = selected_flops(kv_count, kv_index, w.Nq, w.Nk, D, blk)
    attn_tflops = flops / (stage_ms["attn"] * 1e-3) / 1e12
    value = flops / (ms_per_step * 1e-3) / 1e12
    sel_ms = stage_ms["selection"]
    sbytes = stage_bytes(w, kept, nqb, nkb)
    dense_flops = 4 * D * w.Nq * w.Nk * B * H
    traffic = traffic_for_attention(w.name)

    diag = None
    if not args.no_diagnostics and blk == 128:
        log("[bench] retained-attention-mass diagnostic")
        diag = mass_diagnostic(sp, torch, x, w, q, k, v, cnt, idx, F, kept)
        if w.dtype == "bf16":
            log("[bench] mask-reuse baseline")
            diag["mask_reuse"] = mask_reuse_diagnostic(sp, torch, w, q, k, v, F, kept, cnt, idx)

    cpu = None
    if not args.no_cpu_baseline and blk == 128:
        log(f"[bench] CPU baseline (oracle, ~{args.cpu_budget:.0f} s)")
        cpu = cpu_baseline(x, w, F, args.cpu_budget)

    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) + per-block offsets; see workloads/)",
        "config": {**w.describe(), "block": blk, "kept_blocks": kept, "n_forced_blocks": F,
                   "selected_tflop": flops / 1e12, "dense_tflop": dense_flops / 1e12,
                   "cache": "cold" if primary_cold else "warm",
                   "score_select": ("screened, one call from Q and K"
                                    if fused and not args.from_means else
                                    "screened from the means" if fused else "two-step")},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
        "cpu_baseline": cpu,
        "diagnostics": diag,
        "other_cache": other,
        "stages": {
            "attn_us": round(stage_ms["attn"] * 1e3, 2),
            "selection_calls_us": {n: round(calls_ms[n] * 1e3, 2) for n in names[:-1]},
            "attn_tflops": round(attn_tflops, 2),
            "selection_us": round(sel_ms * 1e3, 2),
            "selection_alg_bytes": sbytes,
            "selection_gbps": round(sbytes / (sel_ms * 1e-3) / 1e9, 1),
            "selection_frac_hbm": round(sbytes / (sel_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "selection_share_of_scale": round(sel_ms / ms_per_step, 4),
            "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 4),
            "means_gbps": (round(B * H * (w.Nq + w.Nk) * D * (2 if w.dtype == "bf16" else 4)
                                 / ((calls_ms["means_q"] + calls_ms["means_k"]) * 1e-3) / 1e9, 1)
                           if "means_q" in calls_ms else None),
        },
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
