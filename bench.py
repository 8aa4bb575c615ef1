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


def gemm_by_shape(B, model, M):
    """Per-shape figures of the prefill GEMMs recorded since the last
    profile enable: each launch of the block-GEMM and LM-head classes is
    matched to the named product whose algorithmic flops and bytes it has
    (W1 and W2 have the same flops and differ in bytes)."""
    d, H, Hkv, F, V = model.d_model, model.n_head, model.n_kv_head, model.d_ff, model.vocab
    dims = {"qkv": ((H + 2 * Hkv) * model.head_dim, d, 2), "o": (d, H * model.head_dim, 8),
            "w1": (F, d, 2), "w2": (d, F, 8), "lm_head": (V, d, 4)}  # N, K, output bytes per element
    expect = {n: (2.0 * M * N * K, 2.0 * (M * K + N * K) + ob * M * N) for n, (N, K, ob) in dims.items()}
    out = {}
    for cls in ("gemm", "lmhead"):
        c = B.PROF_CLASSES[cls]
        for i in range(B.gpt_profile_read(c)["launches"]):
            r = B.gpt_profile_read_launch(c, i)
            name = min(expect, key=lambda n: abs(expect[n][0] - r["flops"]) / expect[n][0] +
                       abs(expect[n][1] - r["bytes"]) / expect[n][1])
            acc = out.setdefault(name, {"M": M, "N": dims[name][0], "K": dims[name][1], "launches": 0,
                                        "ms": 0.0, "flops": 0.0})
            acc["launches"] += 1
            acc["ms"] += r["ms"]
            acc["flops"] += r["flops"]
    for acc in out.values():
        tfs = acc["flops"] / (acc["ms"] * 1e-3) / 1e12
        acc["us_per_launch"] = round(acc.pop("ms") * 1e3 / acc["launches"], 2)
        acc.pop("flops")
        acc["achieved_tflops"] = round(tfs, 1)
        acc["frac"] = round(tfs / PEAK_BF16_TFLOPS, 4)
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


PROF_STRIDE = 8


def bench_decode(B, torch, dm, w, steps, temperature, warm_steps=3):
    """Prefill the prompts into a fresh cache, pick the first token, then time
    `steps` decode steps (selection included).  A second identical pass with
    HIP-event timing on every PROF_STRIDE-th step gives the per-kernel-class
    figures."""
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

    def run(k, mask=0):
        for s in range(k):
            if mask:  # time every PROF_STRIDE-th step: bounded event count, all lengths covered
                B.gpt_profile_mask(mask if s % PROF_STRIDE == 0 else 0)
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
    # host cost of issuing a step: two steps enqueued onto an idle GPU, timed
    # on the host alone (median of up to 5), against the step's GPU time
    start()
    host = []
    for _ in range(min(5, steps // 2)):
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        run(2)
        host.append((time.perf_counter() - h0) / 2)
    torch.cuda.synchronize()
    host_us = sorted(host)[len(host) // 2] * 1e6 if host else None
    start()
    torch.cuda.synchronize()
    mask = 1 << B.PROF_CLASSES["decode_attn"] | 1 << B.PROF_CLASSES["skinny"] | 1 << B.PROF_CLASSES["lmhead"]
    B.gpt_profile_enable(mask)
    run(steps, mask)
    torch.cuda.synchronize()
    att = prof_read(B, ["decode_attn"])
    sk = prof_read(B, ["skinny", "lmhead"])
    B.gpt_profile_enable(0)
    kv.close()
    return dt, att, sk, host_us


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


def code_tokens(text):
    """C++/HIP source without its comments and with whitespace collapsed, so
    that an edit to comments or layout leaves the code's identity unchanged.
    (No source hashed here has comment markers inside string literals.)"""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def gemm_source_hash():
    """Identity of the GEMM kernels' code (comments and layout excluded): the
    traffic figure is reported only for the code it was measured on."""
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(code_tokens(fh.read()).encode())
    return h.hexdigest()


def traffic_pass(decode=True):
    """For rocprofv3 counter passes: one warm-up and one counted depth-12
    prefill, then (decode) the depth-12 decode and depth-26 serving shapes
    for a few steps each, then copies of known size."""
    import torch
    from gpt_block_fwd_amd import binding as B
    B.lib()
    w = wl.d12_prefill()
    W12 = wl.make_weights(w.model)
    dm = B.DeviceModel(w.model, W12)
    M = int(w.cu_seqlens[-1])
    logits = torch.empty((M, dm.model.vocab), dtype=torch.float32, device="cuda")
    lse = torch.empty(M, dtype=torch.float32, device="cuda")
    tokens = torch.from_numpy(w.tokens).cuda()
    ws = dm.workspace(M, w.n_seqs)
    for _ in range(2):
        dm.prefill(tokens, w.cu_seqlens, logits, lse, workspace=ws)
        torch.cuda.synchronize()
    del logits, ws
    torch.cuda.empty_cache()
    log("counted prefill done")
    if decode:
        for wd, dmod, temp in ((wl.d12_decode(steps=4), dm, 0.0), (wl.d26_serving(steps=4), None, 0.7)):
            if dmod is None:
                del dm
                torch.cuda.empty_cache()
                dmod = B.DeviceModel(wd.model, wl.make_weights(wd.model))
            decode_capture(B, torch, dmod, wd, 4, temp, [0])
            torch.cuda.synchronize()
            log(f"counted decode {wd.name} done")
        del dmod
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
        # the first two depth-12 prefills (QKV, O, W1, W2 per layer, then the
        # LM head: 49 GEMM launches each); the second is the counted one
        per = 4 * 12 + 1
        gemm = [r for r in rows if "gemm_pp_kernel" in r[1]][:2 * per]
        counted = gemm[per:]
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


def summarize_counters(paths, out_md, title):
    """Per-kernel means of every counter in rocprofv3 counter_collection CSVs
    (one or more passes), grouped by kernel and grid size, as a markdown
    table; FETCH_SIZE and WRITE_SIZE are also given in MB per dispatch with
    the copy-calibrated factors (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0, see
    summarize_traffic)."""
    import csv
    import collections
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in paths:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"]
                name = name.replace("void ", "").replace("(anonymous namespace)::", "").split("(")[0][:48]
                grid = r.get("Grid_Size", r.get("Grid_Size_X", ""))
                wg = r.get("Workgroup_Size", r.get("Workgroup_Size_X", ""))
                vals[(name, grid, wg)][r["Counter_Name"]].append(float(r["Counter_Value"]))
    counters = sorted({c for v in vals.values() for c in v})
    scale = {"FETCH_SIZE": 2.0 * 1024 / 1e6, "WRITE_SIZE": 1024 / 1e6}
    lines = [f"# {title}", "", "| kernel | grid | wg | dispatches | " +
             " | ".join(c + (" (MB)" if c in scale else "") for c in counters) + " |",
             "|---|---|---|---|" + "---|" * len(counters)]
    for (name, grid, wg), cv in sorted(vals.items(), key=lambda kv: kv[0]):
        n = max(len(v) for v in cv.values())
        cells = []
        for c in counters:
            v = cv.get(c)
            if not v:
                cells.append("")
                continue
            m = sum(v) / len(v)
            cells.append(f"{m * scale[c]:.2f}" if c in scale else f"{m:.4g}")
        lines.append(f"| `{name}` | {grid} | {wg} | {n} | " + " | ".join(cells) + " |")
    text = "\n".join(lines) + "\n"
    with open(out_md, "w") as fh:
        fh.write(text)
    print(text)


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


# ---------------------------------------------------------------- the oracle legs
# Everything below that imports the oracle runs on the host cores after the
# GPU timings: the oracle's own timing (cpu_baseline) and the parity samples
# that compare the GPU's logits with it.

LITERAL_MAX_ABS, LITERAL_TOP1 = 3e-2, 0.999


def host_cores():
    """Cores this process may run on, and BLAS limited to that many threads."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(cores)
    except Exception:  # pragma: no cover
        pass
    return cores


def parity_stats(gpu, ref, chosen=None):
    """max |diff|, std, top-1 agreement of the GPU's choice (or its argmax)
    with the oracle's argmax, and the literal-bar flags.  `gpu` and `ref` may
    be lists of row blocks (kept apart to bound host memory)."""
    if not isinstance(gpu, list):
        gpu, ref = [gpu], [ref]
        chosen = None if chosen is None else [chosen]
    n = s1 = s2 = agree = 0
    maxd = 0.0
    for i, (g, r) in enumerate(zip(gpu, ref)):
        V = np.shape(g)[-1]
        g = np.asarray(g, np.float64).reshape(-1, V)
        r = np.asarray(r, np.float64).reshape(-1, V)
        d = g - r
        maxd = max(maxd, float(np.max(np.abs(d))))
        n += d.size
        s1 += float(np.sum(d))
        s2 += float(np.sum(d * d))
        g1 = np.argmax(g, -1) if chosen is None else np.asarray(chosen[i]).reshape(-1)
        agree += int(np.sum(g1 == np.argmax(r, -1)))
        rows = len(g1) if i == 0 else rows + len(g1)
    top1 = agree / rows
    std = float(np.sqrt(max(s2 / n - (s1 / n) ** 2, 0.0)))
    return {"rows": int(rows), "max_abs": round(maxd, 5), "std": round(std, 6),
            "top1": round(top1, 5), "literal_max_met": maxd <= LITERAL_MAX_ABS,
            "literal_top1_met": top1 >= LITERAL_TOP1}


def parity_entry(stats, floor, what):
    """One parity record: the GPU against the oracle, and the bf16 storage
    floor (the oracle rounding at the bf16 storage points) against it."""
    return {"what": what, "gpu_vs_oracle": stats,
            "bf16_floor_vs_oracle": {k: floor[k] for k in ("max_abs", "std", "top1")},
            "literal_bars": {"max_abs<=3e-2": stats["literal_max_met"],
                             "top1>=0.999": stats["literal_top1_met"]}}


def cpu_baseline(w, W, gpu_logits):
    """Time the oracle (fp32 BLAS) over every sequence of the workload on the
    host cores, and compare its logits with the GPU's; the bf16 storage floor
    on sequence 0."""
    import oracle
    cores = host_cores()
    cu = w.cu_seqlens
    total, g_all, r_all = 0.0, [], []
    for b in range(w.n_seqs):
        t0 = time.perf_counter()
        ref, _ = oracle.prefill(w.model, W, w.tokens, w.seqlens, dtype=np.float32, seqs=[b])
        total += time.perf_counter() - t0
        g_all.append(gpu_logits[cu[b]:cu[b + 1]])
        r_all.append(ref[0])
        del ref
    rows = int(cu[-1])
    out = {"value": round(rows / total, 2), "unit": "tokens/s", "cores": cores,
           "kind": "oracle",
           "sample": f"all {w.n_seqs} depth-12 sequences ({rows} tokens), numpy fp32 BLAS "
                     f"on {cores} threads, {total:.1f} s"}
    st = parity_stats(g_all, r_all)
    flo, _ = oracle.prefill(w.model, W, w.tokens, w.seqlens, dtype=np.float32, seqs=[0], bf16_points=True)
    fl = parity_stats(flo[0], r_all[0])
    return out, parity_entry(st, fl, f"all {rows} rows of the {w.n_seqs} sequences; floor on sequence 0")


def prefill_parity(w, W, g, seq):
    """GPU logits of one sequence of a prefill against the oracle and the floor."""
    import oracle
    ref, _ = oracle.prefill(w.model, W, w.tokens, w.seqlens, dtype=np.float32, seqs=[seq])
    flo, _ = oracle.prefill(w.model, W, w.tokens, w.seqlens, dtype=np.float32, seqs=[seq],
                            bf16_points=True)
    return parity_entry(parity_stats(g, ref[0]), parity_stats(flo[0], ref[0]),
                        f"sequence {seq} ({len(g)} rows)")


def decode_parity(w, W, got_tok, got_lg, sample, steps, greedy):
    """Teacher-forced oracle decode of the sampled sequences over the GPU's
    tokens, against the GPU's per-step logits, and the floor."""
    import oracle
    _, ref = oracle.run_serving(w.model, W, w.tokens, w.seqlens, steps, forced=got_tok,
                                dtype=np.float32, seqs=sample)
    _, flo = oracle.run_serving(w.model, W, w.tokens, w.seqlens, steps, forced=got_tok,
                                dtype=np.float32, seqs=sample, bf16_points=True)
    chosen = got_tok[:, sample] if greedy else None
    return parity_entry(parity_stats(got_lg, ref, chosen), parity_stats(flo, ref),
                        f"sequences {sample}, the first {steps} decode steps and the prompt's "
                        f"last row, teacher-forced")


def decode_capture(B, torch, dm, w, steps, temperature, sample):
    """Prefill, then `steps` decode steps keeping every step's tokens and the
    sampled sequences' logits (for the parity legs; not timed)."""
    n = w.n_seqs
    kv = B.DeviceKV(dm, n, int(w.seqlens.max()) + steps)
    logits = torch.empty((n, dm.model.vocab), dtype=torch.float32, device="cuda")
    dm.prefill(torch.from_numpy(w.tokens).cuda(), w.cu_seqlens, logits, kv=kv.handle,
               logits_rows=B.ROWS_LAST)
    U = torch.from_numpy(w.uniforms).cuda() if w.uniforms is not None else None
    toks = torch.empty(n, dtype=torch.int32, device="cuda")
    B.gpt_select_tokens(logits, n, dm.model.vocab, temperature, U[0] if U is not None else None, toks)
    ws = dm.workspace(n, n)
    got_tok, got_lg = [toks.cpu().numpy().copy()], [logits[sample].cpu().numpy()]
    for s_ in range(steps):
        dm.decode_step(kv.handle, toks, toks, temperature=temperature,
                       uniforms=U[s_ + 1] if U is not None else None, logits=logits, workspace=ws)
        got_tok.append(toks.cpu().numpy().copy())
        got_lg.append(logits[sample].cpu().numpy())
    kv.close()
    del logits, ws
    torch.cuda.empty_cache()
    return np.stack(got_tok), np.stack(got_lg)


# ---------------------------------------------------------------- decode-attention sweep

SWEEP = [(8, 512), (8, 2560), (8, 8192), (32, 512), (32, 2560), (32, 8192), (64, 512), (64, 1024),
         (64, 2560), (64, 4096), (128, 1024), (128, 2048)]


def decode_sweep(B, torch, steps=8):
    """Decode attention of the depth-26 shape (13 query heads on one K/V
    head) over B sequences of L cached positions: a one-layer model keeps the
    cache fill cheap; the kernel's launches are timed by HIP events."""
    import dataclasses
    cfg = dataclasses.replace(wl.depth_model(26), n_layer=1, max_seq=8192 + steps + 1)
    dm = B.DeviceModel(cfg, wl.make_weights(cfg))
    rows = []
    for nb, L in SWEEP:
        w = wl.uniform_prefill(cfg, nb, L, seed=nb + L)
        kv = B.DeviceKV(dm, nb, L + steps + 1)  # the warm-up step, then `steps`
        lg = torch.empty((nb, cfg.vocab), dtype=torch.float32, device="cuda")
        dm.prefill(torch.from_numpy(w.tokens).cuda(), w.cu_seqlens, lg, kv=kv.handle, logits_rows=B.ROWS_LAST)
        toks = torch.zeros(nb, dtype=torch.int32, device="cuda")
        ws = dm.workspace(nb, nb)
        dm.decode_step(kv.handle, toks, toks, workspace=ws)  # warm-up
        torch.cuda.synchronize()
        B.gpt_profile_enable(1 << B.PROF_CLASSES["decode_attn"])
        for _ in range(steps):
            dm.decode_step(kv.handle, toks, toks, workspace=ws)
        torch.cuda.synchronize()
        r = prof_read(B, ["decode_attn"])
        B.gpt_profile_enable(0)
        gbs = r["bytes"] / (r["ms"] * 1e-3) / 1e9
        rows.append({"B": nb, "L": L, "us_per_launch": round(r["ms"] * 1e3 / max(r["launches"], 1), 2),
                     "achieved_gbs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)})
        log(f"sweep B={nb} L={L}: {rows[-1]['us_per_launch']} us, {gbs:,.0f} GB/s")
        kv.close()
        del lg, ws
        torch.cuda.empty_cache()
    del dm
    torch.cuda.empty_cache()
    return {"model": "depth-26 shape, 1 layer (13 query heads, 1 K/V head, head 128)",
            "bytes": "(L + 1) x 512 B per sequence (K and V, bf16) + q and o", "steps": steps,
            "points": rows}


def step_bytes(model, n, mean_len, vocab):
    """Algorithmic HBM bytes of one decode step: every bf16 weight once,
    except the token embedding, of which the step reads only its n rows; the
    cached K/V read (mean length + 1 positions), the new K/V written, and
    the fp32 logits written and read back by the selection."""
    wbytes = 2 * sum(int(np.prod(sh)) for name, sh in wl.weight_shapes(model) if name != "wte")
    wbytes += 2 * n * model.d_model
    kv = model.n_layer * n * (mean_len + 1) * 2 * model.n_kv_head * model.head_dim * 2
    kvw = model.n_layer * n * 2 * model.n_kv_head * model.head_dim * 2
    return wbytes + kv + kvw + 2 * n * vocab * 4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--decode-steps", type=int, default=None,
                    help="decode steps of both decode legs (default: 256 at depth 12, 512 at depth 26)")
    ap.add_argument("--skip-sweep", action="store_true")
    ap.add_argument("--skip-d26", action="store_true")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--skip-gqa", action="store_true")
    ap.add_argument("--skip-train", action="store_true")
    ap.add_argument("--traffic-pass", action="store_true",
                    help="one counted depth-12 prefill and a 1 GiB copy, for rocprofv3 --pmc")
    ap.add_argument("--summarize-traffic", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_JSON"))
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="per-kernel counter means of rocprofv3 counter CSVs into --counters-out")
    ap.add_argument("--counters-out", default="counters.md")
    ap.add_argument("--counters-title", default="rocprofv3 counters per kernel")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.counters_out, args.counters_title)
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
                "algorithmic_bytes_per_launch": round(g["bytes"] / max(g["launches"], 1), 0),
                "by_shape": gemm_by_shape(B, w2.model, M)}
    breakdown = {
        "gemm_ms_per_step": round(g["ms"] / args.steps, 3),
        "attention": {"ms_per_step": round(attn["ms"] / args.steps, 3),
                      "achieved_tflops": round(attn_tfs, 1),
                      "frac": round(attn_tfs / PEAK_BF16_TFLOPS, 4)},
        "norm_rope_embed_ms_per_step": round(norm["ms"] / args.steps, 3),
        "softmax_ms_per_step": round(smx["ms"] / args.steps, 3),
        "ms_per_step_with_event_timing": round(dt_prof / args.steps * 1e3, 3),
        "whole_prefill": {"tflop_per_step": round((g["flops"] + attn["flops"]) / args.steps / 1e12, 4),
                          "achieved_tflops": round((g["flops"] + attn["flops"]) / dt / 1e12, 1),
                          "frac": round((g["flops"] + attn["flops"]) / dt / 1e12 / PEAK_BF16_TFLOPS, 4)},
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
        dsteps = args.decode_steps or 256
        w3 = wl.d12_decode(steps=dsteps)
        log("timing depth-12 decode")
        ddt, att, sk, host_us = bench_decode(B, torch, dm12, w3, dsteps, 0.0)
        sb = step_bytes(w3.model, 32, 512 + (dsteps - 1) / 2, w3.model.vocab)
        att_gbs = att["bytes"] / (att["ms"] * 1e-3) / 1e9 if att["ms"] else 0.0
        sk_gbs = sk["bytes"] / (sk["ms"] * 1e-3) / 1e9 if sk["ms"] else 0.0
        out["decode"] = {"workload": "d12_decode", "batch": 32, "prompt": 512,
                         "steps": dsteps,
                         "tokens_per_s": round(32 * dsteps / ddt, 1),
                         "ms_per_step": round(ddt / dsteps * 1e3, 4),
                         "whole_step": {"algorithmic_bytes": round(sb), "achieved_gbs": round(sb / (ddt / dsteps) / 1e9, 1),
                                        "frac": round(sb / (ddt / dsteps) / 1e9 / PEAK_HBM_GBS, 4)},
                         "decode_attention": {"achieved_gbs": round(att_gbs, 1),
                                              "frac": round(att_gbs / PEAK_HBM_GBS, 4),
                                              "us_per_launch": round(att["ms"] * 1e3 / max(att["launches"], 1), 2)},
                         "decode_gemms": {"achieved_gbs": round(sk_gbs, 1),
                                          "frac": round(sk_gbs / PEAK_HBM_GBS, 4)},
                         "host_enqueue_us_per_step": round(host_us, 1) if host_us else None}
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
            w3g = dataclasses.replace(wl.d12_decode(steps=args.decode_steps or 256), model=mg)
            ddg, attg, _, _ = bench_decode(B, torch, dmg, w3g, args.decode_steps or 256, 0.0)
            gbs = attg["bytes"] / (attg["ms"] * 1e-3) / 1e9 if attg["ms"] else 0.0
            out["d12_gqa2"]["decode_tokens_per_s"] = round(32 * (args.decode_steps or 256) / ddg, 1)
            out["d12_gqa2"]["decode_attention"] = {"achieved_gbs": round(gbs, 1),
                                                   "frac": round(gbs / PEAK_HBM_GBS, 4)}
        del dmg
        torch.cuda.empty_cache()
        log(f"d12 gqa2: {out['d12_gqa2']}")

    # ---------------- the oracle on the host cores: its timing and the parity samples
    parity = {}
    if not args.skip_cpu:
        log("timing the oracle on the host")
        cb, parity["d12_prefill"] = cpu_baseline(w2, W12, g0)
        out["cpu_baseline"] = cb
        del g0
        if not args.skip_decode:
            ps = min(args.decode_steps or 256, 64)
            wp = wl.d12_decode(steps=ps)
            log("depth-12 decode parity sample")
            tk, lg = decode_capture(B, torch, dm12, wp, ps, 0.0, [0, 31])
            parity["d12_decode"] = decode_parity(wp, W12, tk, lg, [0, 31], ps, greedy=True)
        out["parity"] = parity
    del dm12
    torch.cuda.empty_cache()

    # ---------------- depth 26
    if not args.skip_d26:
        w4 = wl.d26_prefill()
        log("generating depth-26 weights")
        W26 = wl.make_weights(w4.model)
        dm26 = B.DeviceModel(w4.model, W26)
        if args.skip_cpu:
            del W26
        log("timing depth-26 prefill")
        s26 = max(2, args.steps // 3)
        dt4, _, lg4, _ = bench_prefill(B, torch, dm26, w4, s26, 1,
                                    1 << B.PROF_CLASSES["gemm"] | 1 << B.PROF_CLASSES["lmhead"]
                                    | 1 << B.PROF_CLASSES["attn"])
        g26 = lg4[:int(w4.cu_seqlens[1])].cpu().numpy() if not args.skip_cpu else None
        del lg4
        torch.cuda.empty_cache()
        g4 = prof_read(B, ["gemm", "lmhead"])
        a4 = prof_read(B, ["attn"])
        M4 = int(w4.cu_seqlens[-1])
        out["d26_prefill"] = {"workload": "d26_prefill", "batch": 16, "seq_len": 2048,
                              "tokens_per_s": round(s26 * M4 / dt4, 1),
                              "ms_per_step": round(dt4 / s26 * 1e3, 3),
                              "gemm_tflops": round(g4["flops"] / (g4["ms"] * 1e-3) / 1e12, 1),
                              "attn_tflops": round(a4["flops"] / (a4["ms"] * 1e-3) / 1e12, 1),
                              "gemm_frac": round(g4["flops"] / (g4["ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                              "attn_frac": round(a4["flops"] / (a4["ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                              "whole_prefill": {"tflop_per_step": round((g4["flops"] + a4["flops"]) / s26 / 1e12, 3),
                                                "frac": round((g4["flops"] + a4["flops"]) / dt4 / 1e12 / PEAK_BF16_TFLOPS, 4)}}
        log(f"d26 prefill: {out['d26_prefill']['tokens_per_s']:,.0f} tok/s")
        if not args.skip_decode:
            s5 = args.decode_steps or 512
            w5 = wl.d26_serving(steps=s5)
            log("timing depth-26 serving decode")
            ddt5, att5, sk5, host5 = bench_decode(B, torch, dm26, w5, s5, 0.7)
            att_gbs = att5["bytes"] / (att5["ms"] * 1e-3) / 1e9 if att5["ms"] else 0.0
            sb5 = step_bytes(w5.model, 64, float(np.mean(w5.seqlens)) + (s5 - 1) / 2, w5.model.vocab)
            out["d26_serving"] = {"workload": "d26_serving", "batch": 64,
                                  "prompt": "U[64,2048]", "steps": s5, "temperature": 0.7,
                                  "tokens_per_s": round(64 * s5 / ddt5, 1),
                                  "ms_per_step": round(ddt5 / s5 * 1e3, 4),
                                  "whole_step": {"algorithmic_bytes": round(sb5),
                                                 "achieved_gbs": round(sb5 / (ddt5 / s5) / 1e9, 1),
                                                 "frac": round(sb5 / (ddt5 / s5) / 1e9 / PEAK_HBM_GBS, 4)},
                                  "decode_attention": {"achieved_gbs": round(att_gbs, 1),
                                                       "frac": round(att_gbs / PEAK_HBM_GBS, 4),
                                                       "us_per_launch": round(att5["ms"] * 1e3 / max(att5["launches"], 1), 2)},
                                  "host_enqueue_us_per_step": round(host5, 1) if host5 else None}
            log(f"d26 serving: {out['d26_serving']['tokens_per_s']:,.0f} tok/s")
            if not args.skip_cpu:
                ps5 = min(s5, 64)
                w5p = wl.d26_serving(steps=ps5)
                b5 = int(np.argmax(w5p.seqlens))
                log("depth-26 serving parity sample")
                tk5, lg5 = decode_capture(B, torch, dm26, w5p, ps5, 0.7, [b5])
                out["parity"]["d26_serving"] = decode_parity(w5p, W26, tk5, lg5, [b5], ps5, greedy=False)
        if not args.skip_cpu:
            log("depth-26 prefill parity sample")
            out["parity"]["d26_prefill"] = prefill_parity(w4, W26, g26, 0)
            del W26, g26
        del dm26
        torch.cuda.empty_cache()
    if not args.skip_decode and not args.skip_sweep:
        log("decode-attention sweep over batch and cached length")
        out["decode_attention_sweep"] = decode_sweep(B, torch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
