#!/usr/bin/env python3
"""Benchmark of the decoder-block forward on one MI355X.

One step = one prefill of the depth-12 workload (8 sequences x 2048
uniform tokens) through every layer, the LM head over all positions and the
vocabulary softmax (LSE); ``value`` is prefill tokens/s with inputs and
weights resident in HBM.  The same run also reports:

* decode: depth-12, 32 prompts of 512 prefilled, then 256 greedy steps
  (tokens/s over the step loop);
* depth-26 prefill (16 x 2048) and depth-26 serving (64 prompts of
  U[64, 2048] tokens, 512 temperature-0.7 steps), unless --skip-d26;
* roofline: the bf16 GEMM kernel (all block GEMMs + LM head), algorithmic
  FLOPs / kernel time from HIP events the library records on its launch
  stream around every launch, over a second pass of the same timed prefills
  (the first pass, which gives ``value``, carries no events), against the
  2.5 PFLOP/s dense bf16 peak; decode attention bytes / time against 8 TB/s;
* cpu_baseline: the oracle (numpy, fp32 BLAS) on the depth-12 prefill
  workload, timed on the host cores; its logits also give a parity sample.

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

import workloads as wl  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
METRIC = "prefill tokens/s + decode tokens/s (depth 12/26, 1 GPU); % MFMA / HBM roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prof_read(B, names):
    out = {"ms": 0.0, "launches": 0, "flops": 0.0, "bytes": 0.0}
    for n in names:
        r = B.gpt_profile_read(B.PROF_CLASSES[n])
        for k in out:
            out[k] += r[k]
    return out


def bench_prefill(B, torch, dm, w, steps, warmup, prof_mask=0):
    """Time `steps` prefills with nothing else in the timed region, then run
    the same `steps` again with the library's HIP-event timing enabled for
    `prof_mask` (the per-kernel-class figures come from that second pass)."""
    n = w.n_seqs
    cu = w.cu_seqlens
    M = int(cu[-1])
    rows = M if w.logits_rows == "all" else n
    logits = torch.empty((rows, dm.model.vocab), dtype=torch.float32, device="cuda")
    lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    tokens = torch.from_numpy(w.tokens).cuda()
    ws = dm.workspace(M, n)
    mode = B.ROWS_ALL if w.logits_rows == "all" else B.ROWS_LAST
    B.gpt_profile_enable(0)
    for _ in range(warmup):
        dm.prefill(tokens, cu, logits, lse, logits_rows=mode, workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dm.prefill(tokens, cu, logits, lse, logits_rows=mode, workspace=ws)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    dt_prof = None
    if prof_mask:
        B.gpt_profile_enable(prof_mask)
        t0 = time.perf_counter()
        for _ in range(steps):
            dm.prefill(tokens, cu, logits, lse, logits_rows=mode, workspace=ws)
        torch.cuda.synchronize()
        dt_prof = time.perf_counter() - t0
    return dt, dt_prof, logits, lse


def bench_prefill_loss(B, torch, dm, w, steps, warmup):
    """Time `steps` next-token cross-entropy prefills (gpt_prefill_loss: no
    logits written), then the same again with the LM head timed by events."""
    n = w.n_seqs
    cu = w.cu_seqlens
    M = int(cu[-1])
    tokens = torch.from_numpy(w.tokens).cuda()
    targets = torch.from_numpy(w.next_token_targets()).cuda()
    loss = torch.empty(M, dtype=torch.float32, device="cuda")
    mean = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = dm.workspace(M, n)
    B.gpt_profile_enable(0)
    for _ in range(warmup):
        dm.prefill_loss(tokens, targets, cu, loss, None, mean, workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dm.prefill_loss(tokens, targets, cu, loss, None, mean, workspace=ws)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    B.gpt_profile_enable(1 << B.PROF_CLASSES["lmhead"])
    for _ in range(steps):
        dm.prefill_loss(tokens, targets, cu, loss, None, mean, workspace=ws)
    torch.cuda.synchronize()
    lm = prof_read(B, ["lmhead"])
    B.gpt_profile_enable(0)
    return dt, lm, float(mean.cpu().numpy()[0])


def bench_loss_grads(B, torch, dm, w, steps, warmup):
    """Time `steps` loss-gradient passes (gpt_loss_grads: forward, loss and
    the gradient of every weight), then the same again with the backward's
    kernel classes timed by events."""
    n = w.n_seqs
    cu = w.cu_seqlens
    M = int(cu[-1])
    tokens = torch.from_numpy(w.tokens).cuda()
    targets = torch.from_numpy(w.next_token_targets()).cuda()
    loss = torch.empty(M, dtype=torch.float32, device="cuda")
    mean = torch.empty(1, dtype=torch.float32, device="cuda")
    grads = B.DeviceGrads(dm)
    ws = dm.train_workspace(M, n)
    B.gpt_profile_enable(0)
    for _ in range(warmup):
        dm.loss_grads(tokens, targets, cu, grads, loss, mean, workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dm.loss_grads(tokens, targets, cu, grads, loss, mean, workspace=ws)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    names = ["gemm", "lmhead", "attn", "norm", "softmax", "bwd_gemm", "bwd_attn", "bwd_other"]
    B.gpt_profile_enable(sum(1 << B.PROF_CLASSES[k] for k in names))
    for _ in range(steps):
        dm.loss_grads(tokens, targets, cu, grads, loss, mean, workspace=ws)
    torch.cuda.synchronize()
    r = {k: prof_read(B, [k]) for k in names}
    B.gpt_profile_enable(0)
    m = float(mean.cpu().numpy()[0])
    del grads, ws, loss, mean
    torch.cuda.empty_cache()
    return dt, r, m


def bench_adam(B, torch, n, steps, warmup=2):
    """Adam over n fp32 parameters with the bf16 copy: `steps` updates timed
    end to end, then again with the kernel timed by events."""
    gen = torch.Generator(device="cuda").manual_seed(0)
    p = torch.randn(n, device="cuda", generator=gen)
    g = torch.randn(n, device="cuda", generator=gen)
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    pb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    B.gpt_profile_enable(0)
    k = 0
    for _ in range(warmup):
        k += 1
        B.gpt_adam_step(p, g, m, v, pb, n, k, 1e-3, 0.9, 0.95, 1e-8)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        k += 1
        B.gpt_adam_step(p, g, m, v, pb, n, k, 1e-3, 0.9, 0.95, 1e-8)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    B.gpt_profile_enable(1 << B.PROF_CLASSES["optim"])
    for _ in range(steps):
        k += 1
        B.gpt_adam_step(p, g, m, v, pb, n, k, 1e-3, 0.9, 0.95, 1e-8)
    torch.cuda.synchronize()
    r = prof_read(B, ["optim"])
    B.gpt_profile_enable(0)
    del p, g, m, v, pb
    torch.cuda.empty_cache()
    kern_gbs = r["bytes"] / (r["ms"] * 1e-3) / 1e9
    return {"workload": "adam_d12_params", "params": n, "steps": steps,
            "ms_per_step": round(dt / steps * 1e3, 4),
            "bytes_per_param": 30,
            "kernel": {"us_per_launch": round(r["ms"] * 1e3 / max(r["launches"], 1), 1),
                       "achieved_gbs": round(kern_gbs, 1), "frac": round(kern_gbs / PEAK_HBM_GBS, 4)}}


def bench_decode(B, torch, dm, w, steps, temperature, warm_steps=3):
    """Prefill the prompts into a fresh cache, pick the first token, then time
    `steps` decode steps (selection included).  A second identical pass with
    HIP-event timing gives the per-kernel-class figures."""
    n = w.n_seqs
    cu = w.cu_seqlens
    cap = int(w.seqlens.max()) + steps
    kv = B.DeviceKV(dm, n, cap)
    tokens = torch.from_numpy(w.tokens).cuda()
    logits = torch.empty((n, dm.model.vocab), dtype=torch.float32, device="cuda")
    pws = dm.workspace(int(cu[-1]), n)
    dws = dm.workspace(n, n)
    toks = torch.empty(n, dtype=torch.int32, device="cuda")
    U = torch.from_numpy(w.uniforms).cuda() if w.uniforms is not None else None

    def start():
        dm.prefill(tokens, cu, logits, kv=kv.handle, logits_rows=B.ROWS_LAST, workspace=pws)
        B.gpt_select_tokens(logits, n, dm.model.vocab, temperature,
                            U[0] if U is not None else None, toks)

    def run(k):
        for s in range(k):
            dm.decode_step(kv.handle, toks, toks, temperature=temperature,
                           uniforms=U[s + 1] if U is not None else None, workspace=dws)

    B.gpt_profile_enable(0)
    start()
    run(warm_steps)
    start()  # re-prefill resets the cached lengths
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    start()
    torch.cuda.synchronize()
    B.gpt_profile_enable(1 << B.PROF_CLASSES["decode_attn"] | 1 << B.PROF_CLASSES["skinny"]
                         | 1 << B.PROF_CLASSES["lmhead"])
    run(steps)
    torch.cuda.synchronize()
    att = prof_read(B, ["decode_attn"])
    sk = prof_read(B, ["skinny", "lmhead"])
    B.gpt_profile_enable(0)
    kv.close()
    return dt, att, sk


# ---------------------------------------------------------------- HBM traffic of the GEMM kernel
# Two rocprofv3 counter passes over `--traffic-pass` (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch) are reduced by `--summarize-traffic` into
# TRAFFIC_FILE.  Each counter is scaled by what it reads for a plain 1 GiB
# copy in the same process.  The figure is reported only while the GEMM
# sources hash to the value recorded with it.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_d12_prefill.json")
GEMM_SOURCES = ["gpt_block_fwd_amd/csrc/gemm.hip", "gpt_block_fwd_amd/csrc/kernels.h",
                "gpt_block_fwd_amd/csrc/common.h"]
COPY_BYTES = 1 << 30


def gemm_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_pass():
    """One warm-up and one counted depth-12 prefill, then a 1 GiB copy."""
    import torch
    from gpt_block_fwd_amd import binding as B
    B.lib()
    w = wl.d12_prefill()
    dm = B.DeviceModel(w.model, wl.make_weights(w.model))
    M = int(w.cu_seqlens[-1])
    logits = torch.empty((M, dm.model.vocab), dtype=torch.float32, device="cuda")
    lse = torch.empty(M, dtype=torch.float32, device="cuda")
    tokens = torch.from_numpy(w.tokens).cuda()
    ws = dm.workspace(M, w.n_seqs)
    for _ in range(2):
        dm.prefill(tokens, w.cu_seqlens, logits, lse, workspace=ws)
        torch.cuda.synchronize()
    del logits
    torch.cuda.empty_cache()
    # calibration: a plain elementwise copy (fp16 -> fp32: reads COPY_BYTES / 2,
    # writes COPY_BYTES), then the runtime's blit copy (COPY_BYTES each way)
    xh = torch.ones(COPY_BYTES // 4, dtype=torch.float16, device="cuda")
    y = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    y.copy_(xh)
    torch.cuda.synchronize()
    del xh
    x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    log("traffic pass done")


def _counter_rows(path, counter):
    import csv
    rows = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r.get("Counter_Name") == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return rows


def summarize_traffic(fetch_csv, write_csv, out_path):
    """GEMM HBM bytes per launch of the counted prefill (the second of the
    two), each counter scaled by its reading for the final 1 GiB copy."""
    res = {}
    for name, path in (("fetch", fetch_csv), ("write", write_csv)):
        rows = _counter_rows(path, "FETCH_SIZE" if name == "fetch" else "WRITE_SIZE")
        # the elementwise fp16 -> fp32 copy, then the runtime's blit copy
        elem = [r for r in rows if "tofloat32_copy_kernel" in r[1]][-1]
        blit = [r for r in rows if "copyBuffer" in r[1]][-1]
        known = COPY_BYTES / 2 if name == "fetch" else COPY_BYTES
        factor = known / 1024.0 / elem[2]
        gemm = [r for r in rows if "gemm_pp_kernel" in r[1]]
        counted = gemm[len(gemm) // 2:]
        res[name] = {"copy_kernel": elem[1][:80], "copy_kib": elem[2], "copy_known_kib": known / 1024.0,
                     "factor": factor, "blit_kib": blit[2], "blit_known_kib": COPY_BYTES / 1024.0,
                     "launches": len(counted), "kib_per_launch": sum(r[2] for r in counted) / len(counted)}
    per_launch = (res["fetch"]["kib_per_launch"] * res["fetch"]["factor"] +
                  res["write"]["kib_per_launch"] * res["write"]["factor"]) * 1024.0
    out = {"kernel": "gemm_pp_kernel (depth-12 prefill: QKV, O, W1, W2, LM head)",
           "bytes_per_launch": per_launch, "fetch": res["fetch"], "write": res["write"],
           "gemm_sources_sha256": gemm_source_hash()}
    with open(out_path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def measured_traffic():
    """Bytes per GEMM launch from TRAFFIC_FILE, or None if absent or stale."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("gemm_sources_sha256") != gemm_source_hash():
        return None
    return round(float(t["bytes_per_launch"]), 0)


def cpu_baseline(w, W, gpu_logits):
    """Time the oracle (fp32 BLAS) over every sequence of the workload on the
    host cores, and compare its logits with the GPU's (parity sample)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    cu = w.cu_seqlens
    total, maxd, agree, rows = 0.0, 0.0, 0, 0
    for b in range(w.n_seqs):
        t0 = time.perf_counter()
        ref, _ = oracle.prefill(w.model, W, w.tokens, w.seqlens, dtype=np.float32, seqs=[b])
        total += time.perf_counter() - t0
        g = gpu_logits[cu[b]:cu[b + 1]]
        maxd = max(maxd, float(np.max(np.abs(g.astype(np.float64) - ref[0]))))
        agree += int(np.sum(np.argmax(g, -1) == np.argmax(ref[0], -1)))
        rows += len(g)
        del ref
    out = {"value": round(rows / total, 2), "unit": "tokens/s", "cores": int(threads),
           "kind": "oracle",
           "sample": f"all {w.n_seqs} depth-12 sequences ({rows} tokens), numpy fp32 BLAS, "
                     f"{total:.1f} s"}
    parity = {"rows": rows, "max_abs": maxd, "top1": agree / rows}
    return out, parity


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--skip-d26", action="store_true")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--skip-gqa", action="store_true")
    ap.add_argument("--skip-train", action="store_true")
    ap.add_argument("--traffic-pass", action="store_true",
                    help="one counted depth-12 prefill and a 1 GiB copy, for rocprofv3 --pmc")
    ap.add_argument("--summarize-traffic", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_JSON"))
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
        return
    if args.traffic_pass:
        traffic_pass()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decoder-block path has no multi-GPU "
              "sharding (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from gpt_block_fwd_amd import binding as B
    B.lib()
    torch.cuda.set_device(0)

    # ---------------- depth-12 prefill (the headline)
    w2 = wl.d12_prefill()
    log("generating depth-12 weights")
    W12 = wl.make_weights(w2.model)
    dm12 = B.DeviceModel(w2.model, W12)
    gemm_mask = 1 << B.PROF_CLASSES["gemm"] | 1 << B.PROF_CLASSES["lmhead"] | \
        1 << B.PROF_CLASSES["attn"] | 1 << B.PROF_CLASSES["norm"] | 1 << B.PROF_CLASSES["softmax"]
    log("timing depth-12 prefill")
    dt, dt_prof, logits, lse = bench_prefill(B, torch, dm12, w2, args.steps, args.warmup, gemm_mask)
    M = int(w2.cu_seqlens[-1])
    value = args.steps * M / dt
    g = prof_read(B, ["gemm", "lmhead"])
    attn = prof_read(B, ["attn"])
    norm = prof_read(B, ["norm"])
    smx = prof_read(B, ["softmax"])
    gemm_tfs = g["flops"] / (g["ms"] * 1e-3) / 1e12
    attn_tfs = attn["flops"] / (attn["ms"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": "gemm_pp_kernel (block GEMMs + LM head)",
                "achieved": round(gemm_tfs, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(gemm_tfs / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(),
                "avg_launch_us": round(g["ms"] * 1e3 / max(g["launches"], 1), 2),
                "flops_per_launch": g["flops"] / max(g["launches"], 1),
                "algorithmic_bytes_per_launch": round(g["bytes"] / max(g["launches"], 1), 0)}
    breakdown = {
        "gemm_ms_per_step": round(g["ms"] / args.steps, 3),
        "attention": {"ms_per_step": round(attn["ms"] / args.steps, 3),
                      "achieved_tflops": round(attn_tfs, 1),
                      "frac": round(attn_tfs / PEAK_BF16_TFLOPS, 4)},
        "norm_rope_embed_ms_per_step": round(norm["ms"] / args.steps, 3),
        "softmax_ms_per_step": round(smx["ms"] / args.steps, 3),
        "ms_per_step_with_event_timing": round(dt_prof / args.steps * 1e3, 3),
    }
    log(f"d12 prefill: {value:,.0f} tok/s, gemm {gemm_tfs:.0f} TFLOP/s, attn {attn_tfs:.0f} TFLOP/s")

    out = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(dt / args.steps * 1e3, 3), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "d12_prefill", "batch": 8, "seq_len": 2048, "layers": 12,
                      "d_model": 768, "heads": 6, "kv_heads": 1, "vocab": 65536,
                      "logits": "all rows + lse"},
           "roofline": roofline, "prefill_breakdown": breakdown}

    g0 = logits.cpu().numpy() if not args.skip_cpu else None
    del logits, lse
    torch.cuda.empty_cache()

    # ---------------- depth-12 prefill ending in the next-token loss (no logits written)
    log("timing depth-12 prefill with the fused cross-entropy")
    dtl, lml, mean_loss = bench_prefill_loss(B, torch, dm12, w2, args.steps, args.warmup)
    lml_tfs = lml["flops"] / (lml["ms"] * 1e-3) / 1e12
    out["d12_prefill_loss"] = {"workload": "d12_prefill_loss", "batch": 8, "seq_len": 2048,
                               "tokens_per_s": round(args.steps * M / dtl, 1),
                               "ms_per_step": round(dtl / args.steps * 1e3, 3),
                               "lm_head_loss_epilogue": {"us_per_launch": round(lml["ms"] * 1e3 / max(lml["launches"], 1), 1),
                                                         "achieved_tflops": round(lml_tfs, 1),
                                                         "frac": round(lml_tfs / PEAK_BF16_TFLOPS, 4)},
                               "mean_loss": round(mean_loss, 4)}
    log(f"d12 prefill + loss: {out['d12_prefill_loss']['tokens_per_s']:,.0f} tok/s, "
        f"LM head {lml_tfs:.0f} TFLOP/s, mean loss {mean_loss:.4f}")

    # ---------------- depth-12 loss gradient (forward + backward of every weight)
    if not args.skip_train:
        log("timing the depth-12 loss gradient")
        ts = max(2, args.steps // 3)
        dtt, tr, tmean = bench_loss_grads(B, torch, dm12, w2, ts, 1)
        def tf(k):
            return round(tr[k]["flops"] / (tr[k]["ms"] * 1e-3) / 1e12, 1) if tr[k]["ms"] else 0.0
        gm = {k: tr[k] for k in ("gemm", "lmhead", "bwd_gemm")}
        g_fl = sum(v["flops"] for v in gm.values())
        g_ms = sum(v["ms"] for v in gm.values())
        out["d12_loss_grads"] = {
            "workload": "d12_loss_grads", "batch": 8, "seq_len": 2048,
            "tokens_per_s": round(ts * M / dtt, 1), "ms_per_step": round(dtt / ts * 1e3, 3),
            "mean_loss": round(tmean, 4),
            "gemm": {"ms_per_step": round(g_ms / ts, 3),
                     "achieved_tflops": round(g_fl / (g_ms * 1e-3) / 1e12, 1),
                     "frac": round(g_fl / (g_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
            "attention_forward": {"ms_per_step": round(tr["attn"]["ms"] / ts, 3), "achieved_tflops": tf("attn")},
            "attention_backward": {"ms_per_step": round(tr["bwd_attn"]["ms"] / ts, 3),
                                   "achieved_tflops": tf("bwd_attn"),
                                   "frac": round(tf("bwd_attn") / PEAK_BF16_TFLOPS, 4)},
            "elementwise_ms_per_step": round((tr["bwd_other"]["ms"] + tr["norm"]["ms"] + tr["softmax"]["ms"]) / ts, 3)}
        log(f"d12 loss grads: {out['d12_loss_grads']}")

    # ---------------- Adam over every depth-12 parameter (fp32 master copy + bf16 copy)
    n12 = sum(int(np.prod(sh)) for _, sh in wl.weight_shapes(w2.model))
    log("timing the Adam update over the depth-12 parameters")
    out["adam"] = bench_adam(B, torch, n12, args.steps)
    log(f"adam: {out['adam']['kernel']['achieved_gbs']:,.0f} GB/s")

    # ---------------- depth-12 decode
    if not args.skip_decode:
        w3 = wl.d12_decode(steps=args.decode_steps)
        log("timing depth-12 decode")
        ddt, att, sk = bench_decode(B, torch, dm12, w3, args.decode_steps, 0.0)
        att_gbs = att["bytes"] / (att["ms"] * 1e-3) / 1e9 if att["ms"] else 0.0
        sk_gbs = sk["bytes"] / (sk["ms"] * 1e-3) / 1e9 if sk["ms"] else 0.0
        out["decode"] = {"workload": "d12_decode", "batch": 32, "prompt": 512,
                         "steps": args.decode_steps,
                         "tokens_per_s": round(32 * args.decode_steps / ddt, 1),
                         "ms_per_step": round(ddt / args.decode_steps * 1e3, 4),
                         "decode_attention": {"achieved_gbs": round(att_gbs, 1),
                                              "frac": round(att_gbs / PEAK_HBM_GBS, 4),
                                              "us_per_launch": round(att["ms"] * 1e3 / max(att["launches"], 1), 2)},
                         "decode_gemms": {"achieved_gbs": round(sk_gbs, 1),
                                          "frac": round(sk_gbs / PEAK_HBM_GBS, 4)}}
        log(f"d12 decode: {out['decode']['tokens_per_s']:,.0f} tok/s")

    # ---------------- grouped-query attention: the depth-12 shape with 2 K/V heads
    if not args.skip_gqa:
        import dataclasses
        mg = dataclasses.replace(w2.model, n_kv_head=2)
        wg = dataclasses.replace(w2, model=mg, name="d12_gqa2_prefill")
        log("timing depth-12 prefill and decode with 2 K/V heads")
        dmg = B.DeviceModel(mg, wl.make_weights(mg))
        dtg, _, lgg, _ = bench_prefill(B, torch, dmg, wg, args.steps, args.warmup,
                                       1 << B.PROF_CLASSES["attn"])
        del lgg
        torch.cuda.empty_cache()
        ag = prof_read(B, ["attn"])
        ag_tfs = ag["flops"] / (ag["ms"] * 1e-3) / 1e12
        out["d12_gqa2"] = {"workload": "d12 shape, 6 query heads on 2 K/V heads",
                           "prefill_tokens_per_s": round(args.steps * M / dtg, 1),
                           "prefill_attention": {"achieved_tflops": round(ag_tfs, 1),
                                                 "frac": round(ag_tfs / PEAK_BF16_TFLOPS, 4)}}
        if not args.skip_decode:
            w3g = dataclasses.replace(wl.d12_decode(steps=args.decode_steps), model=mg)
            ddg, attg, _ = bench_decode(B, torch, dmg, w3g, args.decode_steps, 0.0)
            gbs = attg["bytes"] / (attg["ms"] * 1e-3) / 1e9 if attg["ms"] else 0.0
            out["d12_gqa2"]["decode_tokens_per_s"] = round(32 * args.decode_steps / ddg, 1)
            out["d12_gqa2"]["decode_attention"] = {"achieved_gbs": round(gbs, 1),
                                                   "frac": round(gbs / PEAK_HBM_GBS, 4)}
        del dmg
        torch.cuda.empty_cache()
        log(f"d12 gqa2: {out['d12_gqa2']}")

    # ---------------- CPU oracle on one sequence
    if not args.skip_cpu:
        log("timing the oracle on the host")
        cb, parity = cpu_baseline(w2, W12, g0)
        out["cpu_baseline"] = cb
        out["parity_sample"] = parity
    del dm12
    torch.cuda.empty_cache()

    # ---------------- depth 26
    if not args.skip_d26:
        w4 = wl.d26_prefill()
        log("generating depth-26 weights")
        W26 = wl.make_weights(w4.model)
        dm26 = B.DeviceModel(w4.model, W26)
        del W26
        log("timing depth-26 prefill")
        s26 = max(2, args.steps // 3)
        dt4, _, lg4, _ = bench_prefill(B, torch, dm26, w4, s26, 1,
                                    1 << B.PROF_CLASSES["gemm"] | 1 << B.PROF_CLASSES["lmhead"]
                                    | 1 << B.PROF_CLASSES["attn"])
        del lg4
        torch.cuda.empty_cache()
        g4 = prof_read(B, ["gemm", "lmhead"])
        a4 = prof_read(B, ["attn"])
        M4 = int(w4.cu_seqlens[-1])
        out["d26_prefill"] = {"workload": "d26_prefill", "batch": 16, "seq_len": 2048,
                              "tokens_per_s": round(s26 * M4 / dt4, 1),
                              "ms_per_step": round(dt4 / s26 * 1e3, 3),
                              "gemm_tflops": round(g4["flops"] / (g4["ms"] * 1e-3) / 1e12, 1),
                              "attn_tflops": round(a4["flops"] / (a4["ms"] * 1e-3) / 1e12, 1)}
        log(f"d26 prefill: {out['d26_prefill']['tokens_per_s']:,.0f} tok/s")
        if not args.skip_decode:
            w5 = wl.d26_serving(steps=512)
            log("timing depth-26 serving decode")
            ddt5, att5, sk5 = bench_decode(B, torch, dm26, w5, 512, 0.7)
            att_gbs = att5["bytes"] / (att5["ms"] * 1e-3) / 1e9 if att5["ms"] else 0.0
            out["d26_serving"] = {"workload": "d26_serving", "batch": 64,
                                  "prompt": "U[64,2048]", "steps": 512, "temperature": 0.7,
                                  "tokens_per_s": round(64 * 512 / ddt5, 1),
                                  "ms_per_step": round(ddt5 / 512 * 1e3, 4),
                                  "decode_attention": {"achieved_gbs": round(att_gbs, 1),
                                                       "frac": round(att_gbs / PEAK_HBM_GBS, 4)}}
            log(f"d26 serving: {out['d26_serving']['tokens_per_s']:,.0f} tok/s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
