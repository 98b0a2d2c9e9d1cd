#!/usr/bin/env python
"""Throughput of the fused DSpark loss (forward + backward) on one MI355X.

One step = dspark_loss_fwd + dspark_loss_bwd over one batch of the
large-batch workload (batch 8 x 256 blocks x block_size 7 = 14336 rows,
vocab 151936, hidden 4096, markov rank 256, bf16 inputs, confidence head on
[hidden ; markov embedding]), with every input already resident in HBM.
Prints one JSON line.  Synthetic, seeded data (workloads package).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def _gpu_leg(args, workload=None):
    import torch

    from speculative_decoding_draft_dspark_amd import (DSparkBatch, HParams, _capi,
                                                       dspark_loss_bwd, dspark_loss_fwd,
                                                       dspark_workspace_size)
    from workloads import get_workload, make_inputs

    _capi.lib()  # fail loudly without the HIP library
    wl = get_workload(workload or args.workload)
    dev = "cuda:0"
    t0 = time.time()
    d = make_inputs(wl, dev)
    torch.cuda.synchronize()
    print(f"[bench] inputs for {wl.name} ready in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)
    b = DSparkBatch.from_workload(d)
    hp = HParams()
    sd = args.store_draft_logits
    ws = torch.empty(dspark_workspace_size(b, store_draft_logits=sd), dtype=torch.uint8,
                     device=dev)
    gs = 1.0 / wl.R
    fwd = dspark_loss_fwd(b, hp, workspace=ws, store_draft_logits=sd)
    grads = dspark_loss_bwd(b, hp, fwd, gs)

    def step():
        f = dspark_loss_fwd(b, hp, workspace=ws, store_draft_logits=sd)
        dspark_loss_bwd(b, hp, f, gs, out=grads)
        return f

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    _capi.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        f = step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stages = _capi.profile_read()
    _capi.profile_enable(False)
    loss = f.loss.item()
    flags = int(f.flags.item())
    print(f"[bench] {wl.name}: {args.steps} steps in {elapsed:.3f}s, loss numerator "
          f"{loss:.4f}, flags {flags}", file=sys.stderr, flush=True)
    del b, d, ws, fwd, grads, f
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return wl, elapsed, stages


def _avg_ms(stages, name, steps):
    """Milliseconds per step of one stage (a stage may be several launches)."""
    ms, n = stages.get(name, (0.0, 0))
    return ms / steps if n else None


def _code_sha256(path: str) -> str:
    """SHA-256 of a C++ source with its comments and blank lines removed and
    runs of whitespace collapsed: a comment edit leaves it unchanged, any
    change to the code does not."""
    import hashlib
    import re
    with open(path) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    lines = (" ".join(l.split()) for l in text.split("\n"))
    return hashlib.sha256("\n".join(l for l in lines if l).encode()).hexdigest()


def _traffic(kernel: str, workload: str):
    """HBM-side bytes per launch from the committed rocprofv3 counter summary.

    None when no summary exists, when none was taken on this workload, or
    when the GEMM code changed since the counters were taken (the hash of
    gemm.hip's code is recorded with them).
    """
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.json")
    src = os.path.join(ROOT, "speculative_decoding_draft_dspark_amd", "csrc", "gemm.hip")
    try:
        with open(path) as fh:
            rec = json.load(fh)
        cur = _code_sha256(src)
    except (OSError, ValueError):
        return None
    if rec.get("gemm_code_sha256") != cur:
        return None
    return rec.get("bytes_per_launch", {}).get(workload)


def _cpu_leg(wl, blocks: int):
    """The FP64 oracle on a bounded sample of the same workload (whole blocks)."""
    import numpy as np
    import torch

    import oracle
    from workloads import make_inputs, to_numpy_f64
    from workloads.synth import subset_blocks

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = torch.get_num_threads()
    d = make_inputs(wl, "cuda:0")
    sub = subset_blocks(d, np.arange(blocks))
    n = to_numpy_f64(sub)
    del d, sub
    torch.cuda.empty_cache()
    swl = wl
    inp = oracle.Inputs(B=1, N=blocks, K=swl.K, z=n["z"], target_ids=n["target_ids"],
                        eval_mask=n["eval_mask"], block_keep=n["block_keep"],
                        prev_ids=n["prev_ids"], W1=n["W1"], W2=n["W2"], H_t=n["H_t"],
                        LM=n["LM"], h_d=n["h_d"], W_c=n["W_c"], b_c=n["b_c"])
    hp = oracle.HParams()
    t0 = time.perf_counter()
    oracle.forward(inp, hp)
    oracle.backward(inp, hp, grad_scale=1.0 / wl.R)
    dt = time.perf_counter() - t0
    rows = blocks * wl.K
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next(l.split(":", 1)[1].strip() for l in fh if l.startswith("model name"))
    except (OSError, StopIteration):  # pragma: no cover
        pass
    return {"value": rows / dt, "unit": "rows/s", "cores": int(cores), "kind": "oracle",
            "cpu": cpu,
            "sample": f"{blocks} whole blocks ({rows} rows) of {wl.name}, fwd+bwd in "
                      f"{dt:.1f}s, numpy float64"}


def _copy_probe(nbytes: int, reps: int = 3):
    """A plain device-to-device copy of a known size (counter calibration and
    the measured HBM reference: read + write bytes over the best copy time)."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    best = float("inf")
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        best = min(best, a.elapsed_time(b))
    print(json.dumps({"copy_probe_bytes": n * 4, "reps": reps, "best_ms": round(best, 4),
                      "read_plus_write_GB/s": round(2 * n * 4 / best / 1e6, 1)}), flush=True)


def _library_gemm(args, reps: int = 5):
    """The vendor library's GEMM (torch.matmul, i.e. hipBLASLt) on the teacher
    projection's shape [R, H] x [V, H]^T of the workload, as a reference point
    for the logits kernel: bf16 output, and fp32 output where torch offers it
    (the logits kernel writes fp32 T plus tile statistics).  Prints one JSON
    line; not the benchmark line."""
    import torch

    from workloads import get_workload

    wl = get_workload(args.workload)
    g = torch.Generator(device="cuda:0").manual_seed(5)
    a = torch.randn(wl.R, wl.H, device="cuda:0", generator=g).to(torch.bfloat16)
    b = (0.02 * torch.randn(wl.Vd, wl.H, device="cuda:0", generator=g)).to(torch.bfloat16)
    flops = 2.0 * wl.R * wl.Vd * wl.H

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = {"mode": "library-gemm", "workload": wl.name, "M": wl.R, "N": wl.Vd, "K": wl.H,
           "reps": reps}
    ms = timed(lambda: torch.matmul(a, b.T))
    out["bf16_out_ms"] = round(ms, 4)
    out["bf16_out_TFLOP/s"] = round(flops / ms / 1e9, 1)
    try:
        ms = timed(lambda: torch.mm(a, b.T, out_dtype=torch.float32))
        out["fp32_out_ms"] = round(ms, 4)
        out["fp32_out_TFLOP/s"] = round(flops / ms / 1e9, 1)
    except (TypeError, RuntimeError) as e:
        out["fp32_out"] = f"unavailable: {type(e).__name__}"
    print(json.dumps(out), flush=True)


def _vocab_shard(args, reps: int = 10):
    """One tensor-parallel rank's share of the loss: the large-batch rows over
    the first of G vocabulary shards (widths multiples of 32, the last shard
    takes the remainder), every shard step timed on this GPU with the
    exchanges left out (a single shard merges with itself).  Prints one JSON
    line; not the benchmark line."""
    import dataclasses

    import torch

    from speculative_decoding_draft_dspark_amd import DSparkBatch, HParams, _capi
    from speculative_decoding_draft_dspark_amd.shard import VocabShard, merge_lse
    from workloads import get_workload, make_inputs

    _capi.lib()
    wl = get_workload(args.workload)
    G = args.vocab_shards
    Vs = wl.Vd // G // 32 * 32
    d = make_inputs(wl, "cuda:0")
    b = DSparkBatch.from_workload(d)
    sb = dataclasses.replace(
        b, draft_logits=b.draft_logits[:, :Vs].contiguous(), markov_w2=b.markov_w2[:Vs].contiguous(),
        lm_head=b.lm_head[:Vs].contiguous())
    del d, b
    sh = VocabShard(sb, HParams())

    def step():
        lse = merge_lse(sh.fwd_stats()[None])
        sh.fwd_finish(sh.fwd_terms(lse), row_outputs=False)
        g = sh.bwd(1.0 / wl.R)
        sh.bwd_finish(g.get("d_embed"), 1.0 / wl.R)

    step()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        step()
    e.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(e) / reps
    print(json.dumps({"mode": "vocab-shard", "workload": wl.name, "shards": G, "shard_vocab": Vs,
                      "rows": wl.R, "ms_per_step_one_shard": round(ms, 4),
                      "rows_per_s_if_exchanges_free": round(wl.R / (ms * 1e-3), 1),
                      "reps": reps}), flush=True)


def _side_ops(args, reps: int = 20):
    """Times the standalone ops beside the loss (head ops at the large-batch
    shapes, batch construction for its rows) and prints one JSON line; not the
    benchmark line."""
    import torch

    from speculative_decoding_draft_dspark_amd import (_capi, build_blocks, confidence_logits,
                                                       markov_logits)
    from workloads import get_workload, make_inputs

    _capi.lib()
    wl = get_workload(args.workload)
    d = make_inputs(wl, "cuda:0")
    R, V, r, Hd = wl.R, wl.Vd, wl.r, wl.Hd
    g = torch.Generator(device="cuda:0").manual_seed(7)
    L = 4096
    ids = torch.randint(0, wl.Vt, (wl.B, L), device="cuda:0", dtype=torch.int32, generator=g)
    lm = torch.ones(wl.B, L, device="cuda:0", dtype=torch.uint8)
    anchors = torch.randint(0, L - 1, (wl.B, wl.N), device="cuda:0", dtype=torch.int32,
                            generator=g)
    valid = d["eval_mask"]
    ops = {
        "markov_logits": (lambda: markov_logits(d["z"], d["prev_ids"], d["W1"], d["W2"], valid),
                          {"flops": 2.0 * R * V * r, "bytes": R * V * (2 + 4)}),
        "confidence_logits": (lambda: confidence_logits(d["h_d"], d["W_c"], d["b_c"], d["prev_ids"],
                                                        d["W1"], valid, with_markov=True),
                              {"bytes": R * (Hd + r) * 2}),
        "build_blocks": (lambda: build_blocks(ids, lm, anchors, wl.K, with_candidates=True),
                         {"bytes": wl.B * L * 6 + R * 10}),
    }
    res = {}
    for name, (fn, work) in ops.items():
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        e = {"avg_ms": round(ms, 4)}
        if "flops" in work:
            e["TFLOP/s"] = round(work["flops"] / (ms * 1e-3) / 1e12, 1)
        e["GB/s"] = round(work["bytes"] / (ms * 1e-3) / 1e9, 1)
        res[name] = e
    print(json.dumps({"side_ops": res, "workload": wl.name, "reps": reps,
                      "note": "host-side allocation of outputs included"}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="large-batch-r14336-v151936")
    ap.add_argument("--cpu-blocks", type=int, default=72)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--also", nargs="*", default=["qwen3-8b-r1792-v151936"],
                    help="further workloads timed after the headline one, reported in "
                         "other_workloads (default: the Qwen3-8B-shaped workload)")
    ap.add_argument("--store-draft-logits", action="store_true",
                    help="DSPARK_OPT_STORE_DRAFT_LOGITS: materialise the fp32 corrected draft "
                         "logits instead of recomputing the Markov bias in each sweep")
    ap.add_argument("--side-ops", action="store_true",
                    help="only time the standalone head ops and batch construction")
    ap.add_argument("--vocab-shards", type=int, default=0, metavar="G",
                    help="only time one of G draft-vocabulary shards of the workload (one "
                         "tensor-parallel rank's share, exchanges excluded)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="only time the vendor library GEMM on the teacher projection's shape "
                         "(reference point for the logits kernel)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (rocprofv3 byte-counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        _copy_probe(args.copy_probe)
        return
    if args.side_ops:
        _side_ops(args)
        return
    if args.library_gemm:
        _library_gemm(args)
        return
    if args.vocab_shards:
        _vocab_shard(args)
        return
    wl, elapsed, stages = _gpu_leg(args)
    summary = _summary(args, wl, elapsed, stages)
    roofline, sweeps, stage_ms = summary["roofline"], summary["sweeps"], summary["stage_ms"]
    ms_step, rows_per_s = summary["ms_per_step"], summary["rows_per_s"]
    R, V, H, r = wl.R, wl.Vd, wl.H, wl.r
    # the other V = 151936 workload the metric names, as an extra block
    others = {}
    for name in args.also:
        owl, oel, ost = _gpu_leg(args, name)
        others[owl.name] = _summary(args, owl, oel, ost)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = _cpu_leg(wl, args.cpu_blocks)

    line = {
        "metric": "DSpark loss fwd+bwd rows/s at V=151936",
        "value": round(rows_per_s, 1), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded workloads package)",
        "config": {"workload": wl.name, "rows": R, "batch": wl.B, "num_blocks": wl.N,
                   "block_size": wl.K, "draft_vocab": V, "target_vocab": wl.Vt, "hidden": H,
                   "markov_rank": r, "confidence_head": "with_markov", "gamma": wl.gamma,
                   "parallelism": "single GPU",
                   "corrected_draft_logits": ("stored fp32" if args.store_draft_logits
                                              else "recomputed per sweep")},
        "roofline": roofline,
        "sweeps": sweeps,
        "stage_ms": stage_ms,
        "other_workloads": others,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def _summary(args, wl, elapsed, stages):
    """rows/s, the teacher projection against the bf16 MFMA peak, the sweeps
    against the HBM peak, and per-stage milliseconds of one workload's run."""
    R, V, H, r = wl.R, wl.Vd, wl.H, wl.r
    ms_step = 1000.0 * elapsed / args.steps
    rows_per_s = R * args.steps / elapsed

    stored = args.store_draft_logits
    gemm_ms = _avg_ms(stages, "logits_gemm", args.steps)
    if stored:  # teacher projection (K = H) + the materialised Markov bias (K = r)
        gemm_flops = 2.0 * R * V * (H + r)
        kname = "logits_gemm (lm_head projection + Markov-corrected draft logits, bf16 MFMA)"
    else:       # the teacher projection alone: the bias is recomputed in the sweeps
        gemm_flops = 2.0 * R * V * H
        kname = "logits_gemm (lm_head projection, bf16 MFMA, tile statistics epilogue)"
    gemm_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": kname,
                "achieved": round(gemm_tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": None if stored else _traffic("logits_gemm", wl.name),
                "flops_per_launch": gemm_flops, "avg_ms": round(gemm_ms, 4)}

    # vocabulary sweeps: algorithmic HBM bytes per (row, column) / average
    # duration.  Stored path: z' and T fp32 in, dz bf16 + G lo bf16 out.
    # Recompute path: z bf16 instead of z' (the bias comes from W2 in L2 and E
    # in registers, not counted); statistics read z alone; the L1 pass reads z
    # and T and writes sign(p - q) as 2-bit fields (0.25 byte), which the
    # gradient pass reads with z before writing dz bf16.
    if stored:
        per_elem = (("l1_sweep", 8), ("grad_sweep", 12))
    else:
        per_elem = (("bias_stats", 2), ("l1_sweep", 6.25), ("grad_sweep", 4.25))
    sweeps = {}
    for name, bytes_per_elem in per_elem:
        ms = _avg_ms(stages, name, args.steps)
        if ms:
            gbs = bytes_per_elem * R * V / (ms * 1e-3) / 1e9
            sweeps[name] = {"avg_ms": round(ms, 4), "GB/s": round(gbs, 1),
                            "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                            "bytes_per_row": bytes_per_elem * V}
    stage_ms = {k: round(v[0] / args.steps, 4) for k, v in stages.items() if v[1]}
    return {"rows": R, "rows_per_s": round(rows_per_s, 1), "ms_per_step": round(ms_step, 4),
            "roofline": roofline, "sweeps": sweeps, "stage_ms": stage_ms}


if __name__ == "__main__":
    main()
