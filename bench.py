"""Benchmark of the SAS gated block-sparse attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--part all|train|train32k|decode] [--decode-workloads 4,5]
    python bench.py --calibrate-copy      # plain 256 MiB device copy (counter scale)
    python bench.py --stream-floor        # read floor of cold streams at the decode's sizes

One step is one pass of the training hot path over the Qwen3-4B-shaped 8K
workload (batch 1, 8192 tokens, 32 query / 8 KV heads, head_dim 128, bf16,
block 64, Top-31 + current block, stand-in selector): block pooling of q and k,
stand-in scores, gate normalisation + Top-K, fused gated forward, and the
backward returning dq/dk/dv, the per-block gate gradient and the selector
gradient ds.  `value` is selected-attention TFLOP/s: 12*d FLOP per attended
(query head, query, key) pair (4d forward, 8d backward), divided by the step
time.  The decode part of the path (batch 8 x 64K and batch 1 x 512K contexts)
is measured in the same run and reported under "decode" in GB/s of selected
K/V bytes: each decode call takes a fresh query and the calls rotate over
distinct per-layer K/V caches, so the selected blocks come from HBM rather than
from the last-level cache.  Prints one JSON line.

`ceilings` holds what the chip reaches on plain work in the same run (a large
bf16 GEMM through the vendor BLAS, a 1 GiB device copy); each roofline's
`frac_of_practical` divides its achieved rate by the matching ceiling.

`roofline.traffic` is the HBM bytes per launch of the dominant kernel from the
committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary in profiles/, scaled by the
plain-copy calibration recorded there; it is null when that kernel's sources
have changed since the counters were taken (source hash mismatch).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def selected_pairs_device(idx, n, bs, g):
    """Attended (query head, query, key) pairs, counted on the device from idx:
    selected history blocks count fully, the current block causally."""
    import torch
    b, hkv, T, K = idx.shape
    valid = (idx >= 0).sum().item()
    hist = valid * bs * bs                       # all blocks here are full (n % bs == 0)
    cur = b * hkv * T * bs * (bs + 1) // 2
    return (hist + cur) * g


def train_step_fn(w, x, ws, gate=0, K=None, seq_lens=None):
    """One training step of the stand-in workload.  With seq_lens (every
    sequence at full length, so the results are bitwise those of the dense
    call) the library runs the backward's dQ and dK/dV kernels one after the
    other on one stream, which times each kernel alone."""
    import torch
    from gated_block_sparse_scores_amd import ops
    T = w.nblocks
    K = w.topk if K is None else K
    rl = {} if seq_lens is None else {"seq_lens": seq_lens}
    sel_rl = {} if seq_lens is None else {"seq_lens": seq_lens, "seqlen": w.seqlen,
                                          "block": w.block}

    def step():
        qb = ops.block_pool(x["q"], w.block, w.group, **rl)
        kb = ops.block_pool(x["k"], w.block, 1, **rl)
        idx, logg, lse_s, s = ops.select_topk(w.batch, w.hkv, T, T, K, qbar=qb, kbar=kb,
                                              gate=gate, **sel_rl)
        o, lse = ops.attn_fwd(x["q"], x["k"], x["v"], idx, logg, w.block, gate=gate, **rl)
        gr = ops.attn_bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, idx, logg, s, lse_s,
                          w.block, workspace=ws, gate=gate, **rl)
        return idx, gr, qb, kb
    return step


def bench_gate_variants(args, w, x):
    """The same training step under each gate variant (sas_shape.gate) and under
    the dense scope (K = T - 1: every history block selected and gated); a few
    steps each, every variant through the same MFMA kernels (outer gating as
    their OUTER instantiation)."""
    import torch
    from gated_block_sparse_scores_amd import _lib as L
    from gated_block_sparse_scores_amd import ops
    out = {}
    sh = ops.shape_of(x["q"], x["k"], w.block)
    for name, gate, K in (("sigmoid", L.gate_code("sigmoid"), w.topk),
                          ("raw-logit", L.gate_code("raw"), w.topk),
                          ("ste", L.gate_code("softmax", ste=True), w.topk),
                          ("outer", L.gate_code("softmax", outer=True), w.topk),
                          ("dense-scope", 0, w.nblocks - 1)):
        ws = torch.empty(L.sas_attn_bwd_workspace_size(sh, K), dtype=torch.uint8,
                         device=x["q"].device)
        step = train_step_fn(w, x, ws, gate=gate, K=K)
        idx, _, _, _ = step()
        torch.cuda.synchronize()
        pairs = selected_pairs_device(idx, w.seqlen, w.block, w.group)
        for _ in range(5):
            step()
        torch.cuda.synchronize()
        steps = 5
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        out[name] = {"gate": gate, "topk": K, "ms_per_step": round(ms, 3),
                     "TFLOPs": round(12 * w.head_dim * pairs / (ms * 1e-3) / 1e12, 2),
                     "selected_pairs": int(pairs)}
        del ws
    return out


def kernel_rooflines(kt, pairs, d, workload):
    """Roofline of every MFMA kernel from its average launch time (ms) in kt:
    algorithmic FLOPs (selected pairs only: forward 4d; backward 8d split as
    dK/dV 6d for dP, dV, dK and dQ 2d) over the kernel's own duration."""
    out = {}
    for name, (n, tot) in kt.items():
        kf = kernel_flops(name, pairs, d)
        if kf is None:
            continue
        avg_ms = tot / n
        ach = kf / (avg_ms * 1e-3) / 1e12
        out[name] = {"bound": "mfma", "kernel": name, "achieved": round(ach, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(name, workload),
                     "avg_launch_ms": round(avg_ms, 4), "gflop_per_launch": round(kf / 1e9, 2)}
    return out


def kernel_flops(name, pairs, d):
    """Algorithmic FLOPs of one launch of a kernel (selected pairs only)."""
    if name.startswith("fwd"):
        return 4 * d * pairs
    if name.startswith("bwd_dkdv"):
        return 6 * d * pairs       # dP, dV, dK
    if name.startswith("bwd_dq"):
        return 2 * d * pairs       # dQ
    return None


# Sources of each measured kernel (its file plus the headers it includes): the
# counter summary of a kernel is used only while these hash to the same value.
CSRC = os.path.join(ROOT, "gated_block_sparse_scores_amd", "csrc")
KERNEL_SOURCES = {
    "bwd_dkdv_mfma": ["attn_mfma_bwd.hip", "mfma.h", "common.h", "internal.h"],
    "bwd_dq_mfma": ["attn_mfma_bwd.hip", "mfma.h", "common.h", "internal.h"],
    "fwd_mfma": ["attn_mfma_fwd.hip", "mfma.h", "common.h", "internal.h"],
    "decode_split": ["decode.hip", "common.h", "internal.h"],
}
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash(name):
    files = KERNEL_SOURCES.get(name)
    if not files:
        return None
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(name, workload):
    """HBM bytes per launch of `name` on `workload` from the committed counter
    summary profiles/<name>.<workload>.traffic.txt (key: value lines), or None
    when there is none or the kernel's sources changed since it was taken."""
    path = os.path.join(PROFILES, f"{name}.{workload}.traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith((" ", "#", "$")):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(name):
        return None
    try:
        return int(float(rec["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def stream_floor():
    """Runs the stand-alone stream probe (built next to libsas.so): a plain
    read kernel over buffers rotated through 1 GiB, at the decode's stream
    sizes, over grids of 256..4096 workgroups, then the 8 x 64K decode's gather
    pattern without its arithmetic; prints its lines, the best rate per size
    and the gather rates.  Returns the first failing probe's exit status."""
    import subprocess
    probe = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                         "gated_block_sparse_scores_amd", "stream_probe")
    if not os.path.exists(probe):
        print("stream_probe is not built (python -m gated_block_sparse_scores_amd.build)",
              file=sys.stderr)
        return 1
    res = subprocess.run([probe], capture_output=True, text=True, timeout=300)
    sys.stdout.write(res.stdout)
    sys.stderr.write(res.stderr)
    if res.returncode != 0:
        return res.returncode
    best = {}
    for line in res.stdout.splitlines():
        r = json.loads(line)
        if r["bytes"] not in best or r["us_per_launch"] < best[r["bytes"]]["us_per_launch"]:
            best[r["bytes"]] = r
    # the 8 x 64K decode's gather pattern (random 16 KiB K and V blocks) against
    # adjacent blocks through the same kernel
    res = subprocess.run([probe, "--gather"], capture_output=True, text=True, timeout=300)
    sys.stdout.write(res.stdout)
    sys.stderr.write(res.stderr)
    if res.returncode != 0:
        return res.returncode
    gather = [json.loads(line) for line in res.stdout.splitlines()]
    print(json.dumps({"stream_floor": [best[b] for b in sorted(best)], "gather_floor": gather}),
          flush=True)
    return 0


def practical_ceilings(n=16384, copy_bytes=1 << 30, reps=8):
    """What the chip reaches on plain work in this run, beside the published
    peaks: a large bf16 GEMM through the vendor BLAS (torch.matmul, n x n x n,
    contiguous operands; the first products of a cold GPU run slower, so six
    untimed ones come first) and a device copy of 1 GiB (read + write bytes)."""
    import torch
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    for _ in range(6):
        c = torch.matmul(a, b)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        c = torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    gemm_ms = e0.elapsed_time(e1) / reps
    del a, b, c
    x = torch.empty(copy_bytes, dtype=torch.uint8, device="cuda")
    x.fill_(1)
    y = torch.empty_like(x)
    for _ in range(2):
        y.copy_(x)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    copy_ms = e0.elapsed_time(e1) / reps
    del x, y
    torch.cuda.empty_cache()
    tflops = 2.0 * n ** 3 / (gemm_ms * 1e-3) / 1e12
    gbps = 2.0 * copy_bytes / (copy_ms * 1e-3) / 1e9
    return {"bf16_gemm": {"n": n, "ms": round(gemm_ms, 4), "TFLOPs": round(tflops, 1),
                          "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4)},
            "device_copy": {"bytes": copy_bytes, "ms": round(copy_ms, 4), "GBps": round(gbps, 1),
                            "frac_of_peak": round(gbps / PEAK_HBM_GBS, 4)}}


def calibrate_copy(n_bytes=256 << 20, reps=5):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    a = torch.empty(n_bytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n_bytes, "reps": reps}), flush=True)


def bench_train(args):
    import torch
    import synth
    from gated_block_sparse_scores_amd import _lib as L
    from gated_block_sparse_scores_amd import ops

    w = synth.workload(2)
    dev = "cuda"
    x = synth.train_inputs(w, device=dev)
    sh = ops.shape_of(x["q"], x["k"], w.block)
    ws = torch.empty(L.sas_attn_bwd_workspace_size(sh, w.topk), dtype=torch.uint8, device=dev)
    step = train_step_fn(w, x, ws)
    # The outputs kept for counting and for the selector backward come from a
    # step before the warm-up, so the warm-up steps leave the allocator's cache
    # holding one step's buffers and the timed steps allocate nothing new.
    idx, gr, qb, kb = step()
    # counted before the warm-up: the first steps after a host-side reduction
    # like this one run measurably slower
    pairs = selected_pairs_device(idx, w.seqlen, w.block, w.group)
    flops = 12 * w.head_dim * pairs
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Step time with nothing but the step on the stream.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    tflops = flops / (ms * 1e-3) / 1e12
    # Kernel durations: the same steps again with a HIP event pair recorded
    # around every launch on its stream (the events add a little time between
    # kernels, so this pass is not the step time).  At this size dQ runs on a
    # second stream beside dK/dV, so their event spans overlap.
    L.sas_profiler_reset()
    L.sas_profiler_enable(True)
    t2 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    L.sas_profiler_enable(False)
    kt = L.sas_profiler_read()
    ms_events = (t3 - t2) * 1e3 / args.steps
    # Each kernel alone: the same steps through the ragged-batch entry with
    # every sequence at full length (bitwise the same results), where the
    # backward runs dQ, then dK/dV, on one stream.  The rooflines use these
    # durations; the dominant kernel is the longest one.
    full = torch.full((w.batch,), w.seqlen, dtype=torch.int32, device=dev)
    step_serial = train_step_fn(w, x, ws, seq_lens=full)
    for _ in range(3):
        step_serial()
    torch.cuda.synchronize()
    L.sas_profiler_reset()
    L.sas_profiler_enable(True)
    for _ in range(args.steps):
        step_serial()
    torch.cuda.synchronize()
    L.sas_profiler_enable(False)
    kt_alone = L.sas_profiler_read()
    roofs = kernel_rooflines(kt_alone, pairs, w.head_dim, w.name)
    roof = max(roofs.values(), key=lambda r: r["avg_launch_ms"]) if roofs else None
    kernels = {k: {"launches": v[0], "avg_ms": round(v[1] / v[0], 4)} for k, v in kt.items()}
    kernels_alone = {k: {"launches": v[0], "avg_ms": round(v[1] / v[0], 4)}
                     for k, v in kt_alone.items()}
    return dict(w=w, pairs=pairs, flops=flops, ms=ms, tflops=tflops, roofline=roof,
                kernel_rooflines=roofs, kernels_alone=kernels_alone,
                ms_with_kernel_events=ms_events,
                kernels=kernels, x=x, idx=idx, selector_bwd=bench_selector_bwd(args, w, gr, qb, kb),
                gate_variants=None if args.no_variants else bench_gate_variants(args, w, x),
                ragged=None if args.no_variants else bench_ragged_train(args),
                train_32k=None if args.no_variants else bench_train_32k(args))


def bench_train_32k(args):
    """The 32K-token training workload (32/8 heads, d 128, block 64, Top-15,
    given scores): selection, forward and backward per step, timed like the
    8K step."""
    import torch
    import synth
    from gated_block_sparse_scores_amd import _lib as L
    from gated_block_sparse_scores_amd import ops
    w = synth.workload(3)
    x = synth.train_inputs(w, device="cuda")
    T = w.nblocks
    sh = ops.shape_of(x["q"], x["k"], w.block)
    ws = torch.empty(L.sas_attn_bwd_workspace_size(sh, w.topk), dtype=torch.uint8,
                     device="cuda")

    def step():
        idx, logg, lse_s, _ = ops.select_topk(w.batch, w.hkv, T, T, w.topk, s=x["s"])
        o, lse = ops.attn_fwd(x["q"], x["k"], x["v"], idx, logg, w.block)
        ops.attn_bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, idx, logg, x["s"], lse_s,
                     w.block, workspace=ws)
        return idx

    idx = step()
    pairs = selected_pairs_device(idx, w.seqlen, w.block, w.group)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    steps = max(5, args.steps // 2)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    flops = 12 * w.head_dim * pairs
    # kernel durations (at this size the backward already runs dQ, then dK/dV)
    L.sas_profiler_reset()
    L.sas_profiler_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    L.sas_profiler_enable(False)
    kt = L.sas_profiler_read()
    roofs = kernel_rooflines(kt, pairs, w.head_dim, w.name)
    return {"workload": w.name, "selected_pairs": int(pairs), "steps": steps,
            "ms_per_step": round(ms, 4), "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
            "frac_of_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "roofline": max(roofs.values(), key=lambda r: r["avg_launch_ms"]) if roofs else None,
            "kernel_rooflines": roofs,
            "kernels": {k: {"launches": v[0], "avg_ms": round(v[1] / v[0], 4)}
                        for k, v in kt.items()}}


def bench_ragged_train(args):
    """A ragged training batch in the padded layout: 4 sequences of 8192, 6177,
    3077 and 1024 tokens (padded to 8192), 32/8 heads, d 128, block 64, Top-31,
    stand-in selector; one step = the same path as the 8K workload with
    per-sequence lengths.  FLOPs count the selected pairs of each sequence."""
    import numpy as np
    import torch
    import synth
    from gated_block_sparse_scores_amd import _lib as L
    from gated_block_sparse_scores_amd import ops
    lens = [8192, 6177, 3077, 1024]
    w = synth.workload(2, batch=len(lens))
    x = synth.train_inputs(w, seed=77, device="cuda")
    for bb, nb in enumerate(lens):
        for key in ("q", "k", "v", "dout"):
            x[key][bb, :, nb:] = 0
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    T, bs = w.nblocks, w.block
    sh = ops.shape_of(x["q"], x["k"], bs)
    ws = torch.empty(L.sas_attn_bwd_workspace_size(sh, w.topk), dtype=torch.uint8,
                     device="cuda")

    def step():
        qb = ops.block_pool(x["q"], bs, w.group, seq_lens=sl)
        kb = ops.block_pool(x["k"], bs, 1, seq_lens=sl)
        idx, logg, lse_s, s = ops.select_topk(w.batch, w.hkv, T, T, w.topk, qbar=qb, kbar=kb,
                                              seq_lens=sl, seqlen=w.seqlen, block=bs)
        o, lse = ops.attn_fwd(x["q"], x["k"], x["v"], idx, logg, bs, seq_lens=sl)
        ops.attn_bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, idx, logg, s, lse_s, bs,
                     workspace=ws, seq_lens=sl)
        return idx

    idx = step().cpu().numpy()
    pairs = 0
    for bb, nb in enumerate(lens):
        for t in range(-(-nb // bs)):
            rows = min(bs, nb - t * bs)
            pairs += (int((idx[bb, :, t] >= 0).sum()) * bs * rows
                      + w.hkv * rows * (rows + 1) // 2) * w.group
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    return {"seq_lens": lens, "padded_len": w.seqlen, "selected_pairs": pairs,
            "ms_per_step": round(ms, 4),
            "TFLOPs": round(12 * w.head_dim * pairs / (ms * 1e-3) / 1e12, 2),
            "tokens_per_s": round(sum(lens) / (ms * 1e-3), 1)}


def bench_selector_bwd(args, w, gr, qb, kb):
    """The stand-in selector's backward after a step (not in the step time):
    ds -> pooled summaries, then the pools' adjoints added into dq and dk in
    place.  The spread reads and writes dq and dk once (HBM roofline)."""
    import torch
    from gated_block_sparse_scores_amd import _lib as L
    from gated_block_sparse_scores_amd import ops
    call = lambda: ops.selector_bwd(gr["ds"], qb, kb, w.block, w.seqlen, w.hq, dq=gr["dq"],
                                    dk=gr["dk"])
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    L.sas_profiler_reset()
    L.sas_profiler_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    L.sas_profiler_enable(False)
    kt = L.sas_profiler_read()
    esz = 2 if w.dtype == "bf16" else 4
    spread_bytes = 2 * esz * w.batch * (w.hq + w.hkv) * w.seqlen * w.head_dim
    _, t_sp = kt.get("pool_spread", (1, 0.0))
    spread_us = t_sp * 1e3 / args.steps        # the spread into dq and dk, per call
    n_sb, t_sb = kt.get("selector_bwd", (1, 0.0))
    sb_us = t_sb / n_sb * 1e3
    gbs = spread_bytes / (spread_us * 1e-6) / 1e9 if spread_us > 0 else None
    return {"wall_us_per_call": round((t1 - t0) * 1e6 / args.steps, 2),
            "selector_bwd_us": round(sb_us, 2), "pool_spread_us": round(spread_us, 2),
            "pool_spread_bytes": spread_bytes,
            "pool_spread_GBps": None if gbs is None else round(gbs, 1),
            "pool_spread_frac_of_hbm_peak": None if gbs is None else round(gbs / PEAK_HBM_GBS, 4)}


def oracle_decode_baseline(w, kc, vc, kb, q, Lc):
    """The fp64 oracle, as it stands, on one call of a decode workload: its
    selection from the pooled query and the (device-pooled, bf16) pooled-key
    cache, then its decode over the selected blocks; host cores only."""
    from oracle import sas_oracle as O
    kc, vc, q = kc.cpu(), vc.cpu(), q.cpu()
    kb32 = kb.float().cpu().numpy()
    C = (Lc - 1) // w.block
    t0 = time.perf_counter()
    qb = O.to_f32(O.decode_qbar(q, w.hkv))
    s = O.standin_scores(qb, kb32, O.default_scale(w.head_dim), C, row_offset=C)
    idx, logg, _ = O.select_topk(s, w.topk, row_offset=C, C=C)
    t1 = time.perf_counter()
    O.decode(q, kc, vc, Lc, idx[:, :, 0], logg[:, :, 0], w.block)
    t2 = time.perf_counter()
    sel_bytes = w.batch * w.hkv * (w.topk + 1) * w.block * w.head_dim * 2 * 2
    kbar_bytes = w.batch * w.hkv * C * w.head_dim * 2
    return {"workload": w.name, "selection_s": round(t1 - t0, 3),
            "selection_GBps": round(kbar_bytes / (t1 - t0) / 1e9, 3),
            "decode_s": round(t2 - t1, 3),
            "decode_GBps": round(sel_bytes / (t2 - t1) / 1e9, 3),
            "sample": "one call (batch of one new token per sequence), the same shapes"}


def bench_decode(wl, steps, layers=12, kbar_layers=64, cpu=False):
    """Decode of one new token per sequence.  Each call takes a fresh random
    query (so a new selection) and the calls rotate over `layers` distinct K/V
    caches (K and V 1 GiB each per layer at both workloads) and, independently,
    over `kbar_layers` distinct pooled-key caches (16.8 MB each, 1.07 GB in all,
    four times the 256 MB last-level cache), as consecutive layers of a model
    would, so both the selection's pooled-key stream and the selected blocks
    come from HBM.  Pooled-key cache i is the pool of K/V layer i % layers for
    i < layers, and a perturbed copy of it (bf16, + N(0, 0.01^2)) beyond.
    One call = pool the query over its head group, stand-in scores over the
    pooled-key cache + gate normalisation + Top-K, split-K decode + LSE merge,
    through the separate calls; the same calls are then timed as fused steps
    (sas_decode_step), reported under "fused_step"."""
    import torch
    import synth
    from gated_block_sparse_scores_amd import _lib as L
    from gated_block_sparse_scores_amd import ops

    w = synth.workload(wl)
    dev = "cuda"
    Lc = w.seqlen
    C = (Lc - 1) // w.block
    caches, kbars = [], []
    for layer in range(layers):
        x = synth.decode_inputs(w, seed=w.number * 1000 + layer, device=dev)
        kbars.append(ops.block_pool(x["kcache"], w.block, 1, torch.bfloat16))
        caches.append((x["kcache"], x["vcache"]))
        del x
    gen = torch.Generator(device=dev).manual_seed(1000 + wl)
    for i in range(layers, kbar_layers):
        kb = kbars[i % layers].float()
        kb += 0.01 * torch.randn(kb.shape, generator=gen, device=dev)
        kbars.append(kb.to(torch.bfloat16))
        del kb
    torch.cuda.synchronize()
    qshape = (w.batch, w.hq, w.head_dim)
    calls = max(steps * layers, 2 * kbar_layers)
    qs = [torch.randn(qshape, generator=gen, device=dev).to(torch.bfloat16)
          for _ in range(calls + layers)]
    sh = ops.shape_of(qs[0], caches[0][0], w.block, seqlen=Lc)
    ws = torch.empty(L.sas_decode_workspace_size(sh, w.topk), dtype=torch.uint8, device=dev)

    def one(q, c):
        kc, vc = caches[c % layers]
        kb = kbars[c % kbar_layers]
        qb = ops.block_pool(q.unsqueeze(2), w.block, w.group)
        idx, logg, _, _ = ops.select_topk(w.batch, w.hkv, 1, C, w.topk, row_offset=C, qbar=qb,
                                          kbar=kb)
        return ops.decode(q, kc, vc, Lc, idx[:, :, 0], logg[:, :, 0], w.block, workspace=ws)

    def timed(fn, profile):
        """Wall time per call of the timed calls; with profile, kernel times
        from HIP events around every launch (a separate pass)."""
        if profile:
            L.sas_profiler_reset()
            L.sas_profiler_enable(True)
        t0 = time.perf_counter()
        for c in range(calls):
            fn(qs[c], c)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        kt_ = None
        if profile:
            L.sas_profiler_enable(False)
            kt_ = L.sas_profiler_read()
        return (t1 - t0) * 1e6 / calls, kt_

    for layer in range(layers):               # warm-up: one call per layer
        one(qs[calls + layer], layer)
    torch.cuda.synchronize()
    us_step, _ = timed(one, False)
    _, kt = timed(one, True)
    sel_bytes = w.batch * w.hkv * (w.topk + 1) * w.block * w.head_dim * 2 * 2
    kbar_bytes = w.batch * w.hkv * C * w.head_dim * 2

    def avg_us(name):
        n, tot = kt.get(name, (1, 0.0))
        return tot / n * 1e3

    split_us, merge_us = avg_us("decode_split"), avg_us("decode_merge")
    sel_us = avg_us("block_pool") + sum(avg_us(k) for k in
                                        ("standin_scores", "topk", "select_chunk", "select_merge")
                                        if k in kt)
    split_gbs = sel_bytes / (split_us * 1e-6) / 1e9
    dec_gbs = sel_bytes / ((split_us + merge_us) * 1e-6) / 1e9
    gpu_us = sel_us + split_us + merge_us
    kernels = {k: {"launches": v[0], "avg_us": round(v[1] / v[0] * 1e3, 2)} for k, v in kt.items()}

    # The same calls as one fused step each (sas_decode_step): chunked scores +
    # candidates, then the decode (which merges the candidates itself), then
    # the LSE merge.
    ws_step = torch.empty(L.sas_decode_step_workspace_size(sh, w.topk), dtype=torch.uint8,
                          device=dev)

    def one_step(q, c):
        kc, vc = caches[c % layers]
        kb = kbars[c % kbar_layers]
        return ops.decode_step(q, kb, kc, vc, Lc, w.topk, w.block, with_selection=False,
                               workspace=ws_step)

    for layer in range(layers):
        one_step(qs[calls + layer], layer)
    torch.cuda.synchronize()
    step_wall_us, _ = timed(one_step, False)
    _, kt2 = timed(one_step, True)
    step_gpu_us = sum(v[1] / v[0] * 1e3 for v in kt2.values())
    fused = {
        "gpu_us_per_call": round(step_gpu_us, 2),
        "gpu_GBps_per_call": round((sel_bytes + kbar_bytes) / (step_gpu_us * 1e-6) / 1e9, 1),
        "wall_us_per_call": round(step_wall_us, 2),
        "kernels": {k: {"launches": v[0], "avg_us": round(v[1] / v[0] * 1e3, 2)}
                    for k, v in kt2.items()},
        "graph": graph_replays(one_step, qs, kbar_layers, calls),
    }
    oracle_cpu = (oracle_decode_baseline(w, caches[0][0], caches[0][1], kbars[0], qs[0], Lc)
                  if cpu else None)
    del caches, kbars
    torch.cuda.empty_cache()
    return {
        "cpu_oracle": oracle_cpu,
        "workload": w.name, "batch": w.batch, "context": Lc, "hq": w.hq, "hkv": w.hkv,
        "topk": w.topk, "layers_rotated": layers, "pooled_key_caches_rotated": kbar_layers,
        "calls": calls,
        "selected_kv_bytes": sel_bytes, "pooled_key_bytes": kbar_bytes,
        "decode_GBps": round(dec_gbs, 1),
        "decode_frac_of_hbm_peak": round(dec_gbs / PEAK_HBM_GBS, 4),
        "decode_us": round(split_us + merge_us, 2),
        "selection_us": round(sel_us, 2),
        "gpu_us_per_call": round(gpu_us, 2),
        "gpu_GBps_per_call": round((sel_bytes + kbar_bytes) / (gpu_us * 1e-6) / 1e9, 1),
        "wall_us_per_call": round(us_step, 2),
        "fused_step": fused,
        "roofline": {"bound": "hbm", "kernel": "decode_split", "achieved": round(split_gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(split_gbs / PEAK_HBM_GBS, 4),
                     "traffic": recorded_traffic("decode_split", w.name),
                     "avg_launch_us": round(split_us, 2)},
        "kernels": kernels,
    }


def graph_replays(one_step, qs, ngraphs, calls):
    """The fused step of call i (i < ngraphs: its K/V layer and pooled-key cache)
    captured once in a HIP graph (its query in a static buffer), then the graphs
    replayed round-robin, as a serving loop that launches one graph per layer
    would: wall time per replay.  The caches rotate, so the pooled keys and the
    selected blocks still come from HBM."""
    import torch
    qstat = [q.clone() for q in qs[:ngraphs]]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):              # warm-up outside the captures
        for i in range(ngraphs):
            one_step(qstat[i], i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for i in range(ngraphs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            one_step(qstat[i], i)
        graphs.append(g)
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for c in range(calls):
        graphs[c % ngraphs].replay()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / calls
    del graphs
    return {"wall_us_per_call": round(us, 2), "replays": calls}


def bench_decode_paged(steps=10, layers=12):
    """Serving-style decode: batch 8 of ragged lengths (16K to 64K tokens, 32/8
    heads, d 128, block 64, K 63) over a paged cache (pages of one block, pages
    of each sequence scattered at random), rotating over `layers` caches.  Times
    the fused paged step (sas_decode_step_paged) and the paged decode with the
    selection given (sas_decode_paged)."""
    import numpy as np
    import torch
    from gated_block_sparse_scores_amd import _lib as L
    from gated_block_sparse_scores_amd import ops

    dev = "cuda"
    b, hq, hkv, d, bs, K = 8, 32, 8, 128, 64, 63
    lens = [65536, 61457, 57349, 49152, 40993, 32769, 24585, 16386]
    maxlen = max(lens)
    bt_ld = -(-maxlen // bs)
    nblk = [-(-x // bs) for x in lens]
    npages = sum(nblk)
    rng = np.random.default_rng(8)
    gen = torch.Generator(device=dev).manual_seed(8)
    caches = []
    for layer in range(layers):
        perm = rng.permutation(npages)
        table = np.full((b, bt_ld), -1, dtype=np.int32)
        pos = 0
        for bb in range(b):
            table[bb, :nblk[bb]] = perm[pos:pos + nblk[bb]]
            pos += nblk[bb]
        kp = torch.randn((npages, hkv, bs, d), generator=gen, device=dev).to(torch.bfloat16)
        vp = torch.randn((npages, hkv, bs, d), generator=gen, device=dev).to(torch.bfloat16)
        kbar = torch.randn((b, hkv, bt_ld, d), generator=gen, device=dev).mul_(0.125)
        caches.append((kp, vp, torch.from_numpy(table).to(dev), kbar.to(torch.bfloat16)))
    seq = torch.tensor(lens, dtype=torch.int32, device=dev)
    calls = steps * layers
    qs = [torch.randn((b, hq, d), generator=gen, device=dev).to(torch.bfloat16)
          for _ in range(calls + layers)]
    sh = L.Shape(b, hq, hkv, maxlen, d, bs, L.SAS_DTYPE_BF16)
    ws_step = torch.empty(L.sas_decode_step_workspace_size(sh, K), dtype=torch.uint8, device=dev)
    ws_dec = torch.empty(L.sas_decode_workspace_size(sh, K), dtype=torch.uint8, device=dev)
    sels = []
    for layer in range(layers):   # one selection per layer for the given-selection timing
        kp, vp, tb, kb = caches[layer]
        _, _, idx, logg, _ = ops.decode_step_paged(qs[layer], kb, kp, vp, tb, seq, K, bs,
                                                   max_len=maxlen, workspace=ws_step)
        sels.append((idx, logg))

    def step(q, layer):
        kp, vp, tb, kb = caches[layer]
        return ops.decode_step_paged(q, kb, kp, vp, tb, seq, K, bs, max_len=maxlen,
                                     with_selection=False, workspace=ws_step)

    def dec(q, layer):
        kp, vp, tb, _ = caches[layer]
        idx, logg = sels[layer]
        return ops.decode_paged(q, kp, vp, tb, seq, idx, logg, bs, max_len=maxlen,
                                workspace=ws_dec)

    out = {"workload": "paged-ragged-decode-8x16k-64k", "batch": b, "seq_lens": lens,
           "hq": hq, "hkv": hkv, "topk": K, "layers_rotated": layers, "calls": calls}
    sel_bytes = sum(hkv * (min(K, (x - 1) // bs) + 1) * bs * d * 2 * 2 for x in lens)
    kbar_bytes = sum(hkv * ((x - 1) // bs) * d * 2 for x in lens)
    out["selected_kv_bytes"] = sel_bytes
    for name, fn in (("decode_step_paged", step), ("decode_paged", dec)):
        for layer in range(layers):
            fn(qs[calls + layer], layer)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for c in range(calls):
            fn(qs[c], c % layers)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e6 / calls
        L.sas_profiler_reset()
        L.sas_profiler_enable(True)
        for c in range(calls):
            fn(qs[c], c % layers)
        torch.cuda.synchronize()
        L.sas_profiler_enable(False)
        kt = L.sas_profiler_read()
        kern = {k: round(v[1] / v[0] * 1e3, 2) for k, v in kt.items()}
        gpu = sum(kern.values())
        rec = {"wall_us_per_call": round(wall, 2), "gpu_us_per_call": round(gpu, 2),
               "kernels_avg_us": kern}
        split = kern.get("step_decode_split" if name == "decode_step_paged" else "decode_split")
        if name == "decode_paged" and split:
            gbs = sel_bytes / ((split + kern.get("decode_merge", 0.0)) * 1e-6) / 1e9
            rec["decode_GBps"] = round(gbs, 1)
            rec["decode_frac_of_hbm_peak"] = round(gbs / PEAK_HBM_GBS, 4)
        else:
            rec["step_GBps"] = round((sel_bytes + kbar_bytes) / (gpu * 1e-6) / 1e9, 1)
        out[name] = rec
    del caches
    torch.cuda.empty_cache()
    return out


def cpu_baseline(res, budget_s=15.0):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload:
    its own selection over every row, then forward + backward of sampled
    (KV head, query block) rows until the time budget is spent."""
    import numpy as np
    import torch
    from oracle import sas_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    w = res["w"]
    x = {k: res["x"][k].cpu() for k in ("q", "k", "v", "dout")}
    t0 = time.perf_counter()
    qb = O.to_f32(O.pool_queries(x["q"], w.hkv, w.block))
    kb = O.to_f32(O.pool_keys(x["k"], w.block))
    T = w.nblocks
    s = O.standin_scores(qb, kb, O.default_scale(w.head_dim), T)
    idx, logg, lse_s = O.select_topk(s, w.topk)
    t_sel = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    scale = O.default_scale(w.head_dim)
    done, flops, t_rows = 0, 0, 0.0
    order = rng.permutation(w.hkv * T)
    while t_rows < budget_s and done < len(order):
        kv, t = divmod(int(order[done]), T)
        a = time.perf_counter()
        O.bwd_row_block(x["q"], x["k"], x["v"], x["dout"], idx, logg, w.block, scale, 0, kv, t)
        t_rows += time.perf_counter() - a
        nsel = int((idx[0, kv, t] >= 0).sum())
        pairs = (nsel * w.block * w.block + w.block * (w.block + 1) // 2) * w.group
        flops += 12 * w.head_dim * pairs
        done += 1
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return {"value": round(flops / t_rows / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "cpu_model": model, "host_cpus": os.cpu_count(),
            "selection_s": round(t_sel, 3),
            "sample": f"fp64 numpy oracle: selection over all {w.hkv * T} rows "
                      f"({t_sel:.1f} s), then forward+backward of {done} of the "
                      f"{w.hkv * T} (KV head, query block) rows ({t_rows:.1f} s); value = "
                      f"12*d FLOP per attended pair of those rows / their time"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the first few tens of milliseconds on a fresh GPU run slower (clocks
    # ramping); 25 untimed steps of the 8K workload cover about 40 ms
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the GEMM / copy ceilings (profiling runs)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-paged", action="store_true", help="skip the paged ragged decode")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the gate-variant, dense-scope, ragged-batch and 32K training steps")
    ap.add_argument("--part", choices=("all", "train", "train32k", "decode"), default="all",
                    help="train32k: only the 32K-token training workload (profiling)")
    ap.add_argument("--decode-workloads", default="4,5")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--stream-floor", action="store_true",
                    help="run the HBM stream probe (a child process) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the path is single-GPU by design "
              "(sharding across GPUs is not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.stream_floor:  # before this process touches the GPU
        sys.exit(stream_floor())
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy()
        return
    out = {
        "metric": "gated sparse attn fwd+bwd TFLOP/s, decode GB/s; % of MI355X roofline",
        "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
    }
    res = None
    if args.part == "train32k":
        log("32K training workload ...")
        out["train_32k"] = bench_train_32k(args)
    if args.part in ("all", "train"):
        if not args.no_ceilings:
            log("practical ceilings ...")
            out["ceilings"] = practical_ceilings()
        log("training workload ...")
        res = bench_train(args)
        out.update({
            "value": round(res["tflops"], 3),
            "ms_per_step": round(res["ms"], 4),
            "config": {"workload": res["w"].name, "batch": 1, "seq_len": res["w"].seqlen,
                       "hq": 32, "hkv": 8, "head_dim": 128, "block": 64,
                       "topk": res["w"].topk, "selector": "mean-pooled stand-in",
                       "parallelism": "none"},
            "selected_pairs": int(res["pairs"]),
            "algorithmic_gflop_per_step": round(res["flops"] / 1e9, 2),
            "frac_of_bf16_peak": round(res["tflops"] / PEAK_BF16_TFLOPS, 4),
            "roofline": res["roofline"] if "ceilings" not in out else dict(
                res["roofline"], frac_of_practical=round(
                    res["roofline"]["achieved"] / out["ceilings"]["bf16_gemm"]["TFLOPs"], 4)),
            "kernel_rooflines": res["kernel_rooflines"],
            "kernels": res["kernels"],
            "kernels_alone": res["kernels_alone"],
            "ms_per_step_with_kernel_events": round(res["ms_with_kernel_events"], 4),
            "selector_bwd": res["selector_bwd"],
            "gate_variants": res["gate_variants"],
            "ragged_batch": res["ragged"],
            "train_32k": res["train_32k"],
        })
    if args.part in ("all", "decode") and not args.no_decode:
        log("decode workloads ...")
        steps = {4: 10, 5: 25}
        out["decode"] = [bench_decode(int(wl), steps=steps.get(int(wl), 10),
                                      cpu=int(wl) == 4 and not args.no_cpu_baseline)
                         for wl in args.decode_workloads.split(",") if wl]
        if "ceilings" in out:
            for dec in out["decode"]:
                dec["roofline"]["frac_of_practical"] = round(
                    dec["roofline"]["achieved"] / out["ceilings"]["device_copy"]["GBps"], 4)
        if not args.no_paged:
            log("paged ragged decode ...")
            out["decode_paged"] = bench_decode_paged()
    if res is not None and not args.no_cpu_baseline:
        log("cpu baseline ...")
        out["cpu_baseline"] = cpu_baseline(res)
        for dec in out.get("decode", []):
            if dec.get("cpu_oracle"):
                out["cpu_baseline"]["decode"] = dec["cpu_oracle"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
