#!/usr/bin/env python3
"""Benchmark: paged MLA decode on one MI355X.

One step = one pass of the whole path over one batch: ``mla_plan`` (host
planning, schedule staged for the device) and ``mla_run`` (attention kernel
+ split-KV merge kernel); the plan of step k+1 is made while run k executes.
The workload is the decode batch
of 64 rows, 128 heads, page_size 64, kv lengths uniform in [512, 4096]
(seed 1002), with inputs resident in HBM.  Three independent copies of the KV
cache, queries and outputs are rotated so the 256 MB last-level cache cannot
serve a step from the previous one.

``value`` is decode throughput in GB/s of algorithmic bytes (latent rows read
once, queries read, outputs and LSE written, index arrays) per wall-clock
step.  The JSON line also carries the chunked-prefill throughput (TFLOP/s),
the long-context decode and mixed ragged batch (with its extra segment and
the ``mla_merge_state`` of the two results), each against its roofline, the
kernel roofline and the fp64 CPU oracle's throughput on this host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
ROW_BYTES = 576 * 2
FLOPS_PER_PAIR = 2 * 576 + 2 * 512


def algorithmic(w, return_lse=True, row_bytes=ROW_BYTES):
    """Bytes and flops the method must move/compute for workload w (a latent
    row is 1152 bytes in a bf16 cache, 576 in an fp8 one)."""
    lens = w.kv_lens()
    T, H = w.num_tokens, w.num_heads
    nbytes = row_bytes * int(lens.sum()) + T * H * (576 * 2 + 512 * 2)
    if return_lse:
        nbytes += 4 * T * H
    nbytes += 4 * (2 * (w.batch + 1) + w.batch + int(w.kv_indptr[-1]))
    pairs = 0
    qo = w.qo_indptr
    for b in range(w.batch):
        Q, L = int(qo[b + 1] - qo[b]), int(lens[b])
        if w.causal:
            i = np.arange(Q)
            pairs += int(np.clip(i + L - Q + 1, 0, L).sum())
        else:
            pairs += Q * L
    return nbytes, FLOPS_PER_PAIR * H * pairs


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_mla_attention_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload_name):
    """Counter-derived HBM bytes per launch, if measured on the current
    kernel sources (profiles/traffic.json)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        doc = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = doc.get(workload_name)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def _to_dev_bf16(bits, torch):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def run_steps(w, steps, warmup, copies=3, fp8_scale=None):
    import torch

    import paged_mla_attention_amd as pm
    T, H = w.num_tokens, w.num_heads
    if fp8_scale is None:
        kv0 = _to_dev_bf16(w.kv_cache, torch)
    else:  # an fp8 (E4M3) cache standing for the bf16 one
        kv0 = torch.from_numpy(W.fp8_cache_codes(w.kv_cache, fp8_scale)).cuda()
    qn0, qp0 = _to_dev_bf16(w.q_nope, torch), _to_dev_bf16(w.q_pe, torch)
    kvs = [kv0] + [kv0.clone() for _ in range(copies - 1)]
    qns = [qn0] + [qn0.clone() for _ in range(copies - 1)]
    qps = [qp0] + [qp0.clone() for _ in range(copies - 1)]
    outs = [torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda") for _ in range(copies)]
    lses = [torch.empty((T, H), dtype=torch.float32, device="cuda") for _ in range(copies)]
    plan = pm.MLAPlan(H, w.page_size)
    qo, kvp, idx, last = (np.ascontiguousarray(a, dtype=np.int32) for a in
                          (w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len))

    kv_dtype = None if fp8_scale is None else "fp8_e4m3"

    def do_plan():
        plan.plan(qo, kvp, idx, last, causal=w.causal, sm_scale=w.sm_scale,
                  num_cache_pages=w.num_pages, kv_dtype=kv_dtype)

    # A step is one plan and one run.  As in a serving loop, the plan of the
    # next step is made while this step's kernels run.  One pair of events on
    # the launch stream brackets the timed steps (events between the steps
    # would put their own markers between the kernels).
    def step(k):
        c = k % copies
        plan.run(qns[c], qps[c], kvs[c], out=outs[c], lse=lses[c], kv_scale=fp8_scale)
        do_plan()

    do_plan()
    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # Python's cyclic collector would pause the host loop for tens of ms
    # (with torch loaded) somewhere inside the timed steps.
    gc.collect()
    gc.disable()
    t0 = time.perf_counter()
    e0.record()
    for k in range(steps):
        step(k)
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    gc.enable()
    run_ms = e0.elapsed_time(e1) / steps
    stats = plan.stats()
    # The batch is the same every step, so the plans above hit the plan's
    # cache of its last inputs; a full plan's host time is measured apart,
    # alternating the table with one whose first two page ids are swapped
    # (valid for any table).
    idx2 = idx.copy()
    if idx2.size >= 2:
        idx2[[0, 1]] = idx2[[1, 0]]
    full = []
    for k in range(20):
        t1 = time.perf_counter()
        plan.plan(qo, kvp, idx2 if k % 2 == 0 else idx, last, causal=w.causal,
                  sm_scale=w.sm_scale, num_cache_pages=w.num_pages, kv_dtype=kv_dtype)
        full.append(time.perf_counter() - t1)
    torch.cuda.synchronize()
    stats["full_plan_host_us"] = round(float(np.median(full)) * 1e6, 1)
    # Steps whose every plan is a full one (the two tables alternate), as in
    # serving, where the batch changes each step: the host plans while the
    # previous step's kernels run.
    n_re = min(steps, 50)

    def replan_step(k):
        c = k % copies
        plan.run(qns[c], qps[c], kvs[c], out=outs[c], lse=lses[c], kv_scale=fp8_scale)
        plan.plan(qo, kvp, idx2 if k % 2 == 0 else idx, last, causal=w.causal,
                  sm_scale=w.sm_scale, num_cache_pages=w.num_pages, kv_dtype=kv_dtype)

    for k in range(10):
        replan_step(k)
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()
    t0 = time.perf_counter()
    e0.record()
    for k in range(n_re):
        replan_step(k)
    e1.record()
    torch.cuda.synchronize()
    stats["replan_step_us"] = round((time.perf_counter() - t0) / n_re * 1e6, 1)
    gc.enable()
    stats["replan_run_us"] = round(e0.elapsed_time(e1) / n_re * 1e3, 1)
    plan.close()
    return wall * 1e3, run_ms, stats


def roofline_entry(w, run_ms, nbytes, flops):
    """Throughput of one mla_run against the bound that applies to it."""
    secs = run_ms * 1e-3
    gbs, tfs = nbytes / secs / 1e9, flops / secs / 1e12
    hbm_t, mfma_t = nbytes / (HBM_PEAK_GBS * 1e9), flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    bound = "hbm" if hbm_t >= mfma_t else "mfma"
    return {"workload": w.name, "run_ms": round(run_ms, 4), "GB_s": round(gbs, 1),
            "TFLOP_s": round(tfs, 1), "bound": bound,
            "frac": round((gbs / HBM_PEAK_GBS) if bound == "hbm" else (tfs / MFMA_BF16_PEAK_TFLOPS), 4),
            "algorithmic_bytes": nbytes, "algorithmic_flops": flops}


def other_workloads(steps):
    """The long-context decode and the mixed ragged batch (with its extra
    segment and the LSE merge of the two results), timed the same way."""
    import torch

    import paged_mla_attention_amd as pm
    out = {}
    wl = W.long_decode()
    b, f = algorithmic(wl)
    _, run_ms, stats = run_steps(wl, steps, 50, copies=1)
    out["long_decode"] = dict(roofline_entry(wl, run_ms, b, f), plan=stats)
    print(f"[bench] long decode: mla_run {run_ms * 1e3:.1f} us", file=sys.stderr, flush=True)

    # fp8 (E4M3) caches: GB/s on the fp8 bytes (576 per latent row)
    wd = W.decode_batch()
    b, f = algorithmic(wd, row_bytes=576)
    _, run_ms, _ = run_steps(wd, steps, 50, fp8_scale=1 / 32)
    out["decode_fp8"] = roofline_entry(wd, run_ms, b, f)
    out["decode_fp8"]["workload"] = wd.name + "_fp8"
    b, f = algorithmic(wl, row_bytes=576)
    _, run_ms, _ = run_steps(wl, steps, 50, copies=1, fp8_scale=0.05)
    out["long_decode_fp8"] = roofline_entry(wl, run_ms, b, f)
    out["long_decode_fp8"]["workload"] = wl.name + "_fp8"
    print(f"[bench] fp8 decode and long decode done", file=sys.stderr, flush=True)

    wm = W.mixed()
    b, f = algorithmic(wm)
    _, run_ms, _ = run_steps(wm, max(3, steps // 5), 2, copies=1)
    out["mixed"] = roofline_entry(wm, run_ms, b, f)
    we = wm.extra
    b, f = algorithmic(we)
    _, run_ms, _ = run_steps(we, max(3, steps // 5), 2, copies=1)
    out["mixed_extra_segment"] = roofline_entry(we, run_ms, b, f)
    # mla_merge_state over the two results: bf16 [T, H, 512] x 3 + fp32 LSEs
    T, H = wm.num_tokens, wm.num_heads
    va = torch.randn(T, H, 512, device="cuda").to(torch.bfloat16)
    vb = torch.randn(T, H, 512, device="cuda").to(torch.bfloat16)
    sa, sb = torch.randn(T, H, device="cuda"), torch.randn(T, H, device="cuda")
    vo, so = torch.empty_like(va), torch.empty_like(sa)
    for _ in range(3):
        pm.merge_state(va, sa, vb, sb, vo, so)
    n = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        pm.merge_state(va, sa, vb, sb, vo, so)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    mbytes = T * H * (3 * 1024 + 3 * 4)
    out["merge_state"] = {"workload": f"mla_merge_state T={T} H={H}", "run_ms": round(ms, 4),
                          "GB_s": round(mbytes / (ms * 1e-3) / 1e9, 1), "bound": "hbm",
                          "frac": round(mbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "algorithmic_bytes": mbytes}
    print("[bench] mixed batch, extra segment and merge done", file=sys.stderr, flush=True)
    out["append_kv"] = [append_kv_entry(W.decode_batch()), append_kv_entry(W.chunked_prefill())]
    print("[bench] KV append done", file=sys.stderr, flush=True)
    out["projections"] = [projection_entry(kind, T) for kind in ("absorb", "up_project")
                          for T in (64, 4096)]
    print("[bench] projections done", file=sys.stderr, flush=True)
    return out


def _per_call_ms(fn, n=20, reps=10):
    """Milliseconds per call of ``fn`` (enqueues GPU work on torch's current
    stream): (graph, eager).  graph: ``n`` calls captured once in a HIP graph
    and replayed ``reps`` times, the GPU time per call with the host out of
    the way; eager: ``n`` calls issued from Python, which for a few-
    microsecond kernel measures the binding's call rate instead."""
    import torch
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    eager = e0.elapsed_time(e1) / n
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * n), eager


def projection_entry(kind, T, H=128, n=20):
    """mla_absorb_query ([T,H,128] x [H,128,512]) or mla_up_project
    ([T,H,512] x [H,512,128]) with random bf16 operands; bytes = input +
    weights + output, flops = 2 T H K N."""
    import torch

    import paged_mla_attention_amd as pm
    K, N = (128, 512) if kind == "absorb" else (512, 128)
    x = torch.randn(T, H, K, device="cuda").to(torch.bfloat16)
    w = (torch.randn(H, K, N, device="cuda") * K ** -0.5).to(torch.bfloat16)
    out = torch.empty(T, H, N, device="cuda", dtype=torch.bfloat16)
    fn = pm.absorb_query if kind == "absorb" else pm.up_project
    ms, eager_ms = _per_call_ms(lambda: fn(x, w, out=out), n)
    nbytes = 2 * (T * H * K + H * K * N + T * H * N)
    flops = 2 * T * H * K * N
    gbs, tfs = nbytes / (ms * 1e-3) / 1e9, flops / (ms * 1e-3) / 1e12
    bound = "hbm" if nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) else "mfma"
    return {"workload": f"{kind} T={T} H={H} K={K} N={N}", "run_ms": round(ms, 4),
            "eager_call_ms": round(eager_ms, 4), "timing": f"HIP graph of {n} calls",
            "GB_s": round(gbs, 1), "TFLOP_s": round(tfs, 1), "bound": bound,
            "frac": round(gbs / HBM_PEAK_GBS if bound == "hbm" else tfs / MFMA_BF16_PEAK_TFLOPS, 4),
            "algorithmic_bytes": nbytes, "algorithmic_flops": flops}


def append_kv_entry(w, n=20):
    """mla_append_kv for the workload's tokens: the step's new latent rows
    written into their cache slots (1152 B read + 1152 B written per token,
    plus its 4-byte destination), HBM-bound."""
    import torch

    import paged_mla_attention_amd as pm
    rng = np.random.default_rng(7)
    T = w.num_tokens
    ckv = _to_dev_bf16(W.bf16_normals(rng, (T, 512)), torch)
    kpe = _to_dev_bf16(W.bf16_normals(rng, (T, 64)), torch)
    kv = _to_dev_bf16(w.kv_cache, torch)
    plan = pm.MLAPlan(w.num_heads, w.page_size)
    plan.plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len, causal=w.causal,
              sm_scale=w.sm_scale, num_cache_pages=w.num_pages)
    ms, eager_ms = _per_call_ms(lambda: plan.append_kv(ckv, kpe, kv), n)
    plan.close()
    nbytes = T * (2 * 1152 + 4)
    return {"workload": f"append_kv {w.name} T={T}", "run_ms": round(ms, 4),
            "eager_call_ms": round(eager_ms, 4), "timing": f"HIP graph of {n} calls",
            "GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1), "bound": "hbm",
            "frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes}


def cpu_baseline(w, target_s=10.0):
    """The fp64 oracle on this host's cores over whole repeats of the batch."""
    import oracle
    nbytes, _ = algorithmic(w)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.attention(w.q_nope, w.q_pe, w.kv_cache, w.qo_indptr, w.kv_indptr, w.kv_indices,
                         w.kv_last_page_len, w.page_size, w.causal, w.sm_scale)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count()
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    return {"value": round(nbytes * reps / el / 1e9, 3), "unit": "GB/s", "cores": min(cores, threads),
            "kind": "oracle",
            "sample": f"whole decode batch (64 rows, H=128) x {reps} repeats, {el:.1f} s, fp64 numpy"}


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of known size, profiled beside the
    attention kernel to scale the HBM traffic counters (FETCH_SIZE and
    WRITE_SIZE) to bytes."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": nbytes, "bytes_written": nbytes,
                      "reps": reps}), flush=True)


def _rocpd_counter(db_dir, counter, name_part):
    """Per-dispatch values of one counter for the kernels whose name contains
    name_part, from a rocprofv3 --pmc output directory (rocpd database)."""
    import glob
    import sqlite3
    dbs = glob.glob(os.path.join(db_dir, "**", "*.db"), recursive=True)
    if not dbs:
        raise SystemExit(f"no rocprofv3 database under {db_dir}")
    per = {}
    con = sqlite3.connect(dbs[0])
    for name, did, cn, cv in con.execute(
            "select name, dispatch_id, counter_name, counter_value from pmc_events"):
        if cn == counter and name_part in name:
            per[did] = per.get(did, 0.0) + cv
    con.close()
    return [per[k] for k in sorted(per)]


def record_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """Writes profiles/traffic.json: HBM bytes per mla_run of the decode
    workload from the FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch),
    each scaled by what the same counter reads for a device copy of known size
    (bench.py --copy-calibration).  Input: four rocprofv3 --pmc output
    directories of `bench.py --no-prefill` and `bench.py --copy-calibration`."""
    copy_bytes = float(1 << 30)
    cf = _rocpd_counter(copy_fetch_dir, "FETCH_SIZE", "copy")
    cw = _rocpd_counter(copy_write_dir, "WRITE_SIZE", "copy")
    if not cf or not cw:
        raise SystemExit("copy calibration kernel not found in the profiles")
    f_scale = copy_bytes / (float(np.median(cf)) * 1024.0)
    w_scale = copy_bytes / (float(np.median(cw)) * 1024.0)
    out = {}
    for kern in ("attention_kernel", "split_merge_kernel"):
        fe = _rocpd_counter(fetch_dir, "FETCH_SIZE", kern)
        wr = _rocpd_counter(write_dir, "WRITE_SIZE", kern)
        if fe and wr:
            out[kern] = {"fetch_bytes": float(np.median(fe)) * 1024.0 * f_scale,
                         "write_bytes": float(np.median(wr)) * 1024.0 * w_scale}
    total = sum(v["fetch_bytes"] + v["write_bytes"] for v in out.values())
    doc = {"decode": {"source_hash": kernel_source_hash(), "bytes_per_launch": round(total),
                      "per_kernel": out, "fetch_scale": f_scale, "write_scale": w_scale,
                      "note": "FETCH_SIZE/WRITE_SIZE per dispatch (KiB) x copy-calibrated scale; "
                              "one mla_run = attention_kernel + split_merge_kernel"}}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as fh:
        json.dump(doc, fh, indent=1)
    print(json.dumps(doc))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # (a decode step is ~0.1 ms: 200 warm-up steps let the clocks settle)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the long-decode and mixed-batch workloads")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the chunked-prefill workload (for profiling)")
    ap.add_argument("--long-only", action="store_true",
                    help="run only the long-context decode, bf16 then fp8 cache (for profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 1 GiB device copy (for counter calibration)")
    ap.add_argument("--record-traffic", nargs=4, metavar="DIR",
                    help="write profiles/traffic.json from rocprofv3 --pmc directories: "
                         "decode FETCH_SIZE, decode WRITE_SIZE, copy FETCH_SIZE, copy WRITE_SIZE")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        copy_calibration()
        return

    if args.long_only:
        wl = W.long_decode()
        _, run_ms, _ = run_steps(wl, 50, 50, copies=1)
        _, run8_ms, _ = run_steps(wl, 50, 50, copies=1, fp8_scale=0.05)
        print(f"[bench] long decode: mla_run {run_ms * 1e3:.1f} us (bf16), "
              f"{run8_ms * 1e3:.1f} us (fp8)", file=sys.stderr, flush=True)
        return

    if args.prefill_only:
        wp = W.chunked_prefill()
        p_ms, p_run_ms, _ = run_steps(wp, max(3, min(args.steps // 5, 20)), min(args.warmup, 3), copies=1)
        print(f"[bench] prefill: {p_ms:.3f} ms/step, mla_run {p_run_ms:.3f} ms", file=sys.stderr,
              flush=True)
        return

    w = W.decode_batch()
    nbytes, flops = algorithmic(w)
    print(f"[bench] decode workload ready: T={w.num_tokens} H={w.num_heads} "
          f"keys={int(w.kv_lens().sum())}", file=sys.stderr, flush=True)
    ms_step, run_ms, stats = run_steps(w, args.steps, args.warmup)
    value = nbytes / (ms_step * 1e-3) / 1e9
    achieved = nbytes / (run_ms * 1e-3) / 1e9
    print(f"[bench] decode: {ms_step * 1e3:.1f} us/step, mla_run {run_ms * 1e3:.1f} us",
          file=sys.stderr, flush=True)

    prefill = None
    if not args.no_prefill:
        wp = W.chunked_prefill()
        pbytes, pflops = algorithmic(wp)
        print("[bench] prefill workload ready", file=sys.stderr, flush=True)
        p_ms, p_run_ms, _ = run_steps(wp, max(3, min(args.steps // 5, 20)), 2, copies=1)
        prefill = {"workload": wp.name, "tflops": round(pflops / (p_ms * 1e-3) / 1e12, 2),
                   "run_tflops": round(pflops / (p_run_ms * 1e-3) / 1e12, 2),
                   "ms_per_step": round(p_ms, 4), "run_ms": round(p_run_ms, 4),
                   "frac_mfma_peak": round(pflops / (p_run_ms * 1e-3) / 1e12
                                           / MFMA_BF16_PEAK_TFLOPS, 4),
                   "algorithmic_flops": pflops, "algorithmic_bytes": pbytes}
        print(f"[bench] prefill: {p_ms:.3f} ms/step", file=sys.stderr, flush=True)

    others = None
    if not args.no_prefill and not args.no_others:
        others = other_workloads(max(10, min(args.steps // 2, 50)))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w)

    line = {
        "metric": "paged-MLA decode GB/s & prefill TFLOP/s (% MI355X roofline), B=64 H=128",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode B=64 qo_len=1 H=128 kv_lora_rank=512 rope=64 "
                               "page_size=64 kv~U[512,4096] seed=1002",
                   "global_batch": w.batch, "seq_len": int(w.kv_lens().mean()),
                   "tokens_per_s": round(w.num_tokens / (ms_step * 1e-3), 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic("decode"),
                     "kernel": "mla_run (attention_kernel + split_merge_kernel)",
                     "duration_us": round(run_ms * 1e3, 2), "algorithmic_bytes": nbytes,
                     "algorithmic_flops": flops, "plan": stats},
        "prefill": prefill,
        "other_workloads": others,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
