#!/usr/bin/env python3
"""Benchmark of FP8 MLA context prefill on one MI355X.

One step = the whole hot path over one batch of synthetic input that is already
resident in HBM. For the default 32K-token causal workload (C3, a single segment)
that is the one-launch static quantizer over Q, K and V, then the FP8 varlen
prefill; likewise for C1 (128 tokens), C2 (8 packed sequences) and NC (4096
queries over 65536 context keys, non-causal). For the chunked workloads (C4, C5) it
is the quantizer, then the chunked prefill (one prefill launch per query chunk over
its context segments, with the LSE merges).
The headline value is causal-counted TFLOP/s of the step: 640 FLOP per visible
(query, key) pair and head, with 640 = 2 * (192 + 128).

Prints ONE JSON line on stdout. Everything else goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal TFLOP/s + % FP8 MFMA peak, MLA D192/V128 12-head varlen prefill"
FP8_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 MFMA, published (at 2.4 GHz)
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense BF16 MFMA, published
PEAK_CLOCK_GHZ = 2.4
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
FLOP_PER_PAIR = 2 * (192 + 128)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the FP8 prefill kernel's sources (the kernel file and the headers it
    includes), with // comments and blank lines removed, so that the counter record
    stays valid across comment-only edits and changes to other kernels."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp8_mla_context_amd", "csrc")
    for fn in ("device_common.h", "mla_internal.h", "prefill_fp8.hip"):
        with open(os.path.join(csrc, fn)) as f:
            text = f.read()
        code = [re.sub(r"//.*$", "", line).rstrip() for line in text.splitlines()]
        h.update(fn.encode() + "\n".join(line for line in code if line).encode())
    return h.hexdigest()[:16]


def record_counters(dirs, workload: str, path: str = None) -> dict:
    """Build the per-launch counter record of the prefill from rocprofv3 `--pmc` output
    directories (one per pass, csv format) of a run with --copy-probe-mib 1024, and write
    it to profiles/prefill_<workload>_counters.json. Counter values are summed over their
    dimensions per dispatch and averaged over dispatches; FETCH_SIZE and WRITE_SIZE are
    scaled by what they read for the elementwise probe, which moves 1 GiB each way. `path`
    overrides where the record is written."""
    import csv
    import glob
    import re as _re

    per = {}  # kernel name -> counter -> list of per-dispatch sums
    for d in dirs:
        acc, names = {}, {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    key = (r["Dispatch_Id"], r["Counter_Name"])
                    acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
                    names[r["Dispatch_Id"]] = r["Kernel_Name"]
        for (disp, cn), v in acc.items():
            per.setdefault(names[disp], {}).setdefault(cn, []).append(v)
    mean = {k: {cn: sum(v) / len(v) for cn, v in d.items()} for k, d in per.items()}
    pre = [k for k in mean if _re.search(r"prefill_fp8_kernel<1, 0>", k)]  # default PV mode
    probe = [k for k in mean if "elementwise" in k.lower() and mean[k].get("FETCH_SIZE", 0) > 500000]
    if len(pre) != 1 or len(probe) != 1:
        raise SystemExit(f"expected one prefill kernel and one probe kernel, found {pre} / {probe}")
    v, pv = mean[pre[0]], mean[probe[0]]
    fetch_scale = round(1048576 / pv["FETCH_SIZE"], 2)
    write_scale = round(1048576 / pv["WRITE_SIZE"], 2)
    rec = {
        "kernel_hash": kernel_source_hash(),
        "hbm_bytes_per_launch": int(round(v["FETCH_SIZE"] * 1024 * fetch_scale +
                                          v["WRITE_SIZE"] * 1024 * write_scale)),
        "fetch_size_kib": v["FETCH_SIZE"],
        "write_size_kib": v["WRITE_SIZE"],
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "calibration": f"elementwise kernel over 1 GiB uint8: FETCH_SIZE {pv['FETCH_SIZE']:,.0f} KiB, "
                       f"WRITE_SIZE {pv['WRITE_SIZE']:,.0f} KiB",
    }
    if "GRBM_GUI_ACTIVE" in v:
        rec["gfx_cycles_per_launch"] = int(round(v["GRBM_GUI_ACTIVE"] / 8))
        rec["gfx_cycles_counter"] = "GRBM_GUI_ACTIVE summed over the 8 XCDs, divided by 8"
    for cn, key in (("SQ_INSTS_VALU_MFMA_F8", "mfma_f8_instructions"),
                    ("SQ_INSTS_VALU_MFMA_BF16", "mfma_bf16_instructions"),
                    ("SQ_INSTS_VALU", "valu_instructions"), ("SQ_INSTS_LDS", "lds_instructions")):
        if cn in v:
            rec[key] = v[cn]
    if "SQ_INSTS_VALU_MFMA_MOPS_F8" in v and "SQ_INSTS_VALU_MFMA_MOPS_BF16" in v:
        rec["mfma_executed_flop"] = (v["SQ_INSTS_VALU_MFMA_MOPS_F8"] + v["SQ_INSTS_VALU_MFMA_MOPS_BF16"]) * 512
    for cn, key in (("SQ_VALU_MFMA_BUSY_CYCLES", "mfma_busy_cycles_per_simd"),
                    ("SQ_VALU_MFMA_COEXEC_CYCLES", "valu_mfma_coexec_cycles_per_simd")):
        if cn in v:
            rec[key] = int(round(v[cn] / 1024))  # 256 CUs x 4 SIMDs
    if path is None:
        path = os.path.join(ROOT, "profiles", f"prefill_{workload.lower()}_counters.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def load_counters(kernel_hash: str, workload: str, path: str = None):
    """Per-launch counter record of the prefill (HBM bytes, GPU clock cycles) for this
    workload, if it was taken on the current kernel sources; else an empty dict."""
    if path is None:
        path = os.path.join(ROOT, "profiles", f"prefill_{workload.lower()}_counters.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        rec = json.load(f)
    return rec if rec.get("kernel_hash") == kernel_hash else {}


def cpu_baseline(wl, codes_np, ds, target_s: float, seed: int = 1):
    """The oracle, as it stands, on a bounded sample of the workload's query rows, sized by
    two shorter runs so that the reported run takes about target_s."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    rng = np.random.default_rng(seed)

    def run(n_rows):
        rows = np.sort(rng.choice(wl.total_q, size=n_rows, replace=False))
        t0 = time.perf_counter()
        oracle.attention_rows(codes_np[0], codes_np[1], codes_np[2], wl.cu_seqlens_q,
                              wl.cu_seqlens_k, ds[0], ds[1], ds[2], wl.softmax_scale, wl.causal,
                              rows)
        return rows, time.perf_counter() - t0

    # size the sample in two steps (a short probe, then a third of the target)
    n_rows = 128
    _, dt = run(n_rows)
    for frac in (1.0 / 3.0, 1.0):
        n_rows = int(min(wl.total_q, max(n_rows, n_rows * frac * target_s / max(dt, 1e-3))))
        rows, dt = run(n_rows)
    # visible keys of each sampled row (its sequence's last Lq of Lk tokens)
    cu_q = wl.cu_seqlens_q.astype(np.int64)
    cu_k = wl.cu_seqlens_k.astype(np.int64)
    seq = np.searchsorted(cu_q, rows, side="right") - 1
    lq = cu_q[seq + 1] - cu_q[seq]
    lk = cu_k[seq + 1] - cu_k[seq]
    local = rows - cu_q[seq]
    vis = np.clip(local + (lk - lq) + 1, 0, lk) if wl.causal else lk
    flop = float(np.sum(vis)) * wl.q.shape[1] * FLOP_PER_PAIR
    try:
        host_cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        host_cores = os.cpu_count()
    return {
        "value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
        "blas_threads": int(threads), "host_cores": int(host_cores), "kind": "oracle",
        "sample": f"{n_rows} seeded query rows x {wl.q.shape[1]} heads of {wl.name} "
                  f"({float(np.sum(vis)):.3g} visible pairs per head), fp64 NumPy oracle "
                  f"attention on the dequantized FP8 inputs, {dt:.1f} s",
        "seconds": dt,
    }


def public_plan(torch, B, codes, descales, softmax_scale, seg, lq, lk, out, lse):
    """The segmented plan of one causal sequence (the last lq of lk tokens) through the public
    calls only, without grouping: per query chunk of seg rows, one prefill_varlen per
    context segment of seg keys (non-causal) and one for the diagonal (causal), each into
    its own bf16 partial and LSE, then merge_lse over the chunk's partials. Returns a
    closure that runs the plan and the number of prefill and merge launches."""
    heads = codes[0].shape[1]
    off = lk - lq
    plan = []
    for r0 in range(0, lq, seg):
        r1 = min(lq, r0 + seg)
        parts = [(k0, min(off, k0 + seg), False) for k0 in range(0, off, seg)]
        parts += [(off + c0, off + min(r0, c0 + seg), False) for c0 in range(0, r0, seg)]
        parts.append((off + r0, off + r1, True))
        plan.append((r0, r1, parts))
    n_max = max(len(p) for _, _, p in plan)
    rows_max = min(seg, lq)
    pouts = [torch.empty((rows_max, heads, 128), dtype=torch.bfloat16, device="cuda")
             for _ in range(n_max)]
    plses = [torch.empty((heads, rows_max), dtype=torch.float32, device="cuda")
             for _ in range(n_max)]
    cu = {}

    def cu_of(n):
        if n not in cu:
            cu[n] = torch.tensor([0, n], dtype=torch.int32, device="cuda")
        return cu[n]

    def run():
        for r0, r1, parts in plan:
            rows = r1 - r0
            q = codes[0][r0:r1]
            if len(parts) == 1:
                k0, k1, causal = parts[0]
                B.prefill_varlen(q, codes[1][k0:k1], codes[2][k0:k1], cu_of(rows), cu_of(k1 - k0),
                                 rows, k1 - k0, *descales, softmax_scale, causal,
                                 out=out[r0:r1], lse=lse[:, r0:r1])
                continue
            for i, (k0, k1, causal) in enumerate(parts):
                B.prefill_varlen(q, codes[1][k0:k1], codes[2][k0:k1], cu_of(rows), cu_of(k1 - k0),
                                 rows, k1 - k0, *descales, softmax_scale, causal,
                                 out=pouts[i][:rows], lse=plses[i][:, :rows])
            n = len(parts)
            B.merge_lse([p[:rows] for p in pouts[:n]], [p[:, :rows] for p in plses[:n]],
                        out=out[r0:r1], lse_out=lse[:, r0:r1])

    n_prefill = sum(len(p) for _, _, p in plan)
    n_merge = sum(1 for _, _, p in plan if len(p) > 1)
    return run, n_prefill, n_merge


def event_ms(torch, fn, reps: int, stream):
    """Mean and minimum duration of fn() over reps launches, timed with HIP events recorded
    on the launch stream around each launch."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    t = [a.elapsed_time(b) for a, b in ev]
    return float(np.mean(t)), float(np.min(t))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=15,
                    help="untimed steps first: the clock takes about a dozen 32K-token prefills to settle")
    ap.add_argument("--workload", default="C3", choices=["C1", "C2", "C3", "C4", "C5", "NC"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target duration of the timed oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run an elementwise read+write kernel of this size (counter "
                         "calibration and practical HBM roofline)")
    ap.add_argument("--record-counters", nargs="+", metavar="DIR",
                    help="no run: build profiles/prefill_<workload>_counters.json from these "
                         "rocprofv3 --pmc output directories")
    args = ap.parse_args(argv)

    if args.record_counters:
        print(json.dumps(record_counters(args.record_counters, args.workload), indent=1))
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads or context segments would shard with no or one exchange step).",
              file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1
    from fp8_mla_context_amd import binding as B
    from synth import make_workload

    B.lib()  # fail loudly if the library is missing
    t_gen = time.perf_counter()
    wl = make_workload(args.workload)
    heads = wl.q.shape[1]
    chunked = wl.segment_len > 0
    log(f"[bench] workload {wl.name}: {wl.description}; generated in "
        f"{time.perf_counter() - t_gen:.1f} s")

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    # static scale setup (untimed): device amax over the calibration draw, descale = amax / 448
    descales = []
    for c in wl.calib():
        amax = B.amax_per_head(dev_bf16(c)).cpu().numpy()
        d = B.descale_from_amax_host(amax)
        B.check_descales_host(d)
        descales.append(torch.from_numpy(d).cuda())
    wl._calib = None

    q, k, v = dev_bf16(wl.q), dev_bf16(wl.k), dev_bf16(wl.v)
    codes = [torch.empty(x.shape, dtype=torch.uint8, device="cuda") for x in (q, k, v)]
    cu_q = torch.from_numpy(wl.cu_seqlens_q).cuda()
    cu_k = torch.from_numpy(wl.cu_seqlens_k).cuda()
    out = torch.empty((wl.total_q, heads, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((heads, wl.total_q), dtype=torch.float32, device="cuda")
    workspace = None
    if chunked:
        need = B.chunked_workspace_size(wl.total_q, wl.total_k, heads, wl.segment_len, wl.causal)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

    # The step goes through the checked calls. Per-kernel event timings use the same calls
    # prepared once (prepare=True: arguments checked and marshalled, a callable that only
    # launches), so that the events time the kernels and not the host-side checks.
    def quant(prepare=False):
        return B.quant_static([q, k, v], descales, outs=codes, prepare=prepare)

    def prefill_single(prepare=False):
        return B.prefill_varlen(codes[0], codes[1], codes[2], cu_q, cu_k, wl.max_seqlen_q,
                                wl.max_seqlen_k, descales[0], descales[1], descales[2],
                                wl.softmax_scale, wl.causal, out=out, lse=lse, prepare=prepare)

    def prefill_chunked(prepare=False):
        return B.prefill_chunked(codes[0], codes[1], codes[2], descales[0], descales[1],
                                 descales[2], wl.softmax_scale, wl.segment_len, wl.causal,
                                 out=out, lse=lse, workspace=workspace, prepare=prepare)

    prefill = prefill_chunked if chunked else prefill_single

    def step():
        quant()
        prefill()

    pairs = wl.visible_pairs()
    flop = float(pairs) * heads * FLOP_PER_PAIR
    quant_bytes = 3 * (wl.q.size + wl.k.size + wl.v.size)  # 2 B read + 1 B written per element

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done")

    # timed region: exactly `steps` steps, synchronized on both sides; HIP events on the
    # launch stream (torch's current stream) around each step's prefill give the roofline's
    # launch duration over this same region
    stream = torch.cuda.current_stream()
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a_ev, b_ev in step_ev:
        quant()
        a_ev.record(stream)
        prefill()
        b_ev.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    value = flop / (wall / args.steps) / 1e12
    region_ms = float(np.mean([a_ev.elapsed_time(b_ev) for a_ev, b_ev in step_ev]))
    region_tf = flop / (region_ms * 1e-3) / 1e12
    log(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step, {value:.1f} TFLOP/s; "
        f"prefill in those steps {region_ms:.3f} ms = {region_tf:.1f} TFLOP/s")

    # per-kernel durations with HIP events, launches prepared once and run back to back
    # (the figures the variants and the comparator are measured against)
    reps = max(args.steps, 3)
    quant_ms, _ = event_ms(torch, quant(prepare=True), reps, stream)
    prefill_ms, prefill_min = event_ms(torch, prefill(prepare=True), reps, stream)
    achieved = flop / (prefill_ms * 1e-3) / 1e12
    what = "chunked prefill (all segments + merges)" if chunked else "prefill"
    log(f"[bench] event timing: quant {quant_ms * 1e3:.1f} us ({quant_bytes / quant_ms / 1e6:.0f} GB/s), "
        f"{what} {prefill_ms:.3f} ms (min {prefill_min:.3f}) = {achieved:.1f} TFLOP/s")

    kernels = {
        "quant_static_us": round(quant_ms * 1e3, 2),
        "quant_static_GBps": round(quant_bytes / quant_ms / 1e6, 1),
    }
    # the dynamic per-head quantizer (amax of the data itself, then quantize) for comparison:
    # 5 B per element (the bf16 input read twice, the codes written once)
    dyn_codes = [torch.empty_like(c) for c in codes]
    dyn_desc = torch.empty((3, heads), dtype=torch.float32, device="cuda")
    dyn_ms, _ = event_ms(torch, lambda: B.quant_dynamic([q, k, v], outs=dyn_codes,
                                                        descale_out=dyn_desc), reps, stream)
    dyn_bytes = 5 * (wl.q.size + wl.k.size + wl.v.size)
    kernels["quant_dynamic_us"] = round(dyn_ms * 1e3, 2)
    kernels["quant_dynamic_GBps"] = round(dyn_bytes / dyn_ms / 1e6, 1)
    del dyn_codes
    log(f"[bench] dynamic quant {dyn_ms * 1e3:.1f} us ({dyn_bytes / dyn_ms / 1e6:.0f} GB/s, "
        f"{dyn_ms / quant_ms:.2f}x the static quantizer)")
    if chunked:
        # the same attention as one unsegmented bottom-right causal call, and the plan as the
        # workload states it (every context segment its own call, bf16 partials, one public
        # merge per query chunk) through the public calls. The three are timed once more in
        # the reverse order and each keeps its better mean: the first of a run's timings
        # tends to be the slowest, which would favour whichever comes later.
        single_fn = prefill_single(prepare=True)
        single_ms, _ = event_ms(torch, single_fn, reps, stream)
        p_out = torch.empty_like(out)
        p_lse = torch.empty_like(lse)
        run_plan, n_pf, n_mg = public_plan(torch, B, codes, descales, wl.softmax_scale,
                                           wl.segment_len, wl.total_q, wl.total_k, p_out, p_lse)
        run_plan()
        plan_reps = max(3, reps // 4)
        plan_ms, _ = event_ms(torch, run_plan, plan_reps, stream)
        plan_ms = min(plan_ms, event_ms(torch, run_plan, plan_reps, stream)[0])
        single_ms = min(single_ms, event_ms(torch, single_fn, reps, stream)[0])
        again_ms, again_min = event_ms(torch, prefill(prepare=True), reps, stream)
        if again_ms < prefill_ms:
            prefill_ms, prefill_min = again_ms, again_min
            achieved = flop / (prefill_ms * 1e-3) / 1e12
        log(f"[bench] {what}, best of two timings: {prefill_ms:.3f} ms = {achieved:.1f} TFLOP/s")
        kernels["chunked_prefill_ms"] = round(prefill_ms, 4)
        kernels["pipeline_ms"] = round(quant_ms + prefill_ms, 4)
        kernels["unsegmented_prefill_ms"] = round(single_ms, 4)
        kernels["unsegmented_TFLOPs"] = round(flop / (single_ms * 1e-3) / 1e12, 2)
        kernels["public_segment_plan"] = {
            "ms": round(plan_ms, 4), "TFLOPs": round(flop / (plan_ms * 1e-3) / 1e12, 2),
            "prefill_launches": n_pf, "merge_launches": n_mg}
        del p_out, p_lse
        log(f"[bench] as-specified segment plan through the public calls ({n_pf} prefill + "
            f"{n_mg} merge launches): {plan_ms:.3f} ms = {flop / (plan_ms * 1e-3) / 1e12:.1f} TFLOP/s")
        # the public merge on as many bf16 partials as the last query chunk combines
        seg = wl.segment_len
        n_parts = min(64, (wl.total_k + seg - 1) // seg)
        rows = min(wl.total_q, seg)
        gen = torch.Generator(device="cuda").manual_seed(7)
        parts = [torch.randn((rows, heads, 128), device="cuda", generator=gen).to(torch.bfloat16)
                 for _ in range(n_parts)]
        lses = [torch.randn((heads, rows), device="cuda", generator=gen) for _ in range(n_parts)]
        m_out = torch.empty_like(parts[0])
        m_lse = torch.empty_like(lses[0])
        merge_ms, _ = event_ms(torch, B.merge_lse(parts, lses, out=m_out, lse_out=m_lse,
                                                  prepare=True), reps, stream)
        merge_bytes = (n_parts + 1) * rows * heads * (128 * 2 + 4)
        kernels["merge_lse"] = {"partials": n_parts, "rows": rows, "us": round(merge_ms * 1e3, 2),
                                "bytes": merge_bytes,
                                "GBps": round(merge_bytes / merge_ms / 1e6, 1)}
        log(f"[bench] unsegmented prefill {single_ms:.3f} ms; merge of {n_parts} bf16 partials x "
            f"{rows} rows: {merge_ms * 1e3:.1f} us ({merge_bytes / merge_ms / 1e6:.0f} GB/s)")
    else:
        kernels["prefill_ms"] = round(prefill_ms, 4)
        # the PV build variants of the FP8 prefill (same inputs, one launch each)
        pv = {}
        for mode, variant in ((1, "P in one E4M3 term, FP8 MFMA"),
                              (2, "P in two E4M3 terms, FP8 MFMA")):
            path = B.pv_variant_path(mode)
            if not os.path.exists(path):
                continue
            with B.use_library(path):
                call = prefill_single(prepare=True)
                call()
                v_ms, _ = event_ms(torch, call, reps, stream)
            pv[f"pv{mode}"] = {"what": variant, "prefill_ms": round(v_ms, 4),
                               "TFLOPs": round(flop / (v_ms * 1e-3) / 1e12, 2)}
            log(f"[bench] PV variant {mode} ({variant}): {v_ms:.3f} ms = "
                f"{flop / (v_ms * 1e-3) / 1e12:.1f} TFLOP/s")
        if pv:
            kernels["pv_variants"] = pv
        if not wl.causal and wl.batch == 1:
            # split-KV: the same non-causal chunk through the chunked call, one launch over
            # 16384-key segments that merges its own partials
            seg = 16384
            ws = torch.empty(max(1, B.chunked_workspace_size(wl.total_q, wl.total_k, heads, seg,
                                                             False)),
                             dtype=torch.uint8, device="cuda")
            s_out = torch.empty_like(out)
            s_lse = torch.empty_like(lse)
            split_ms, _ = event_ms(torch, B.prefill_chunked(
                codes[0], codes[1], codes[2], descales[0], descales[1], descales[2],
                wl.softmax_scale, seg, False, out=s_out, lse=s_lse, workspace=ws, prepare=True),
                reps, stream)
            kernels["split_kv_chunked"] = {"segment": seg, "ms": round(split_ms, 4),
                                           "TFLOPs": round(flop / (split_ms * 1e-3) / 1e12, 2)}
            log(f"[bench] split-KV over {seg}-key segments (chunked call, merge in the launch): "
                f"{split_ms:.3f} ms = {flop / (split_ms * 1e-3) / 1e12:.1f} TFLOP/s")
            del ws, s_out, s_lse
        # the 256-row varlen grid: query tiles of the longest sequence x sequences x heads;
        # the workgroups of shorter sequences past their last row exit at once (a grid more
        # than a quarter empty runs as twice as many 128-row workgroups)
        lens = np.diff(wl.cu_seqlens_q)
        grid = int((int(lens.max()) + 255) // 256) * len(lens) * heads
        busy = int(np.sum((lens + 255) // 256)) * heads
        kernels["grid"] = {"workgroups": grid, "empty_frac": round(1.0 - busy / grid, 4)}

    # the BF16 comparator: the same attention on the unquantized bf16 Q/K/V, one launch
    # (unsegmented for the chunked workloads), against the FP8 path of this step
    out16 = torch.empty_like(out)
    lse16 = torch.empty_like(lse)
    bf16_ms, _ = event_ms(torch, lambda: B.prefill_varlen_bf16(
        q, k, v, cu_q, cu_k, wl.max_seqlen_q, wl.max_seqlen_k, wl.softmax_scale, wl.causal,
        out=out16, lse=lse16), reps, stream)
    del out16, lse16
    bf16_tf = flop / (bf16_ms * 1e-3) / 1e12
    kernels["bf16_comparator"] = {
        "prefill_ms": round(bf16_ms, 4),
        "TFLOPs": round(bf16_tf, 2),
        "frac_bf16_peak": round(bf16_tf / BF16_PEAK_TFLOPS, 4),
        "fp8_prefill_speedup": round(bf16_ms / prefill_ms, 3),
        "fp8_pipeline_speedup": round(bf16_ms / (quant_ms + prefill_ms), 3),
    }
    log(f"[bench] bf16 comparator: {bf16_ms:.3f} ms = {bf16_tf:.1f} TFLOP/s "
        f"({100 * bf16_tf / BF16_PEAK_TFLOPS:.1f}% of bf16 peak); FP8 {what} is "
        f"{bf16_ms / prefill_ms:.2f}x, quant + {what} {bf16_ms / (quant_ms + prefill_ms):.2f}x "
        f"as fast")

    # the un-absorbed K/V producer fused with the static quantizer, for this workload's keys
    from synth import make_latent

    cache_bits, w_bits = make_latent(7, wl.total_k, heads)
    d_cache, d_w = dev_bf16(cache_bits), dev_bf16(w_bits)
    del cache_bits, w_bits
    pk8 = torch.empty((wl.total_k, heads, 192), dtype=torch.uint8, device="cuda")
    pv8 = torch.empty((wl.total_k, heads, 128), dtype=torch.uint8, device="cuda")
    prod_call = B.kv_produce(d_cache[:, :512], d_cache[:, 512:], d_w, descales[1], descales[2],
                             k8=pk8, v8=pv8, prepare=True)
    prod_call()
    prod_ms, _ = event_ms(torch, prod_call, reps, stream)
    prod_bytes = wl.total_k * (576 * 2 + heads * 320) + d_w.numel() * 2
    prod_flop = 2.0 * wl.total_k * heads * 256 * 512
    kernels["kv_produce"] = {
        "tokens": wl.total_k, "us": round(prod_ms * 1e3, 2),
        "TFLOPs": round(prod_flop / (prod_ms * 1e-3) / 1e12, 1),
        "frac_bf16_peak": round(prod_flop / (prod_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "GBps": round(prod_bytes / prod_ms / 1e6, 1), "bytes": prod_bytes,
    }
    del d_cache, d_w, pk8, pv8
    log(f"[bench] kv producer ({wl.total_k} tokens): {prod_ms * 1e3:.1f} us, "
        f"{prod_flop / (prod_ms * 1e-3) / 1e12:.0f} TFLOP/s, {prod_bytes / prod_ms / 1e6:.0f} GB/s")

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            # an elementwise kernel (a plain D2D copy may go to the DMA engine, which the
            # kernel counters do not see): reads n bytes, writes n bytes
            torch.mul(src, 1, out=dst)
        probe_ms, _ = event_ms(torch, lambda: torch.mul(src, 1, out=dst), 5, stream)
        kernels["copy_probe_GBps"] = round(2 * n / probe_ms / 1e6, 1)
        log(f"[bench] elementwise probe: {2 * n} B moved in {probe_ms:.3f} ms "
            f"({2 * n / probe_ms / 1e6:.0f} GB/s, the practical HBM roofline)")

    khash = kernel_source_hash()
    rec = load_counters(khash, wl.name)
    # the prefill's mean launch duration over the timed region (events around each step's
    # prefill), as the roofline's `achieved`
    roofline = {
        "bound": "mfma",
        "kernel": "prefill_fp8_kernel" + (" (segment launches, merge inside)" if chunked else ""),
        "achieved": round(region_tf, 2),
        "peak": FP8_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(region_tf / FP8_PEAK_TFLOPS, 4),
        "traffic": rec.get("hbm_bytes_per_launch"),
        "launch_ms": round(region_ms, 4),
    }
    if rec.get("gfx_cycles_per_launch") and not chunked:
        # GPU clock during the launch = counted cycles / live duration
        sclk = rec["gfx_cycles_per_launch"] / (region_ms * 1e-3) / 1e9
        peak_adj = FP8_PEAK_TFLOPS * sclk / PEAK_CLOCK_GHZ
        roofline["sclk_GHz"] = round(sclk, 3)
        roofline["peak_clock_adjusted"] = round(peak_adj, 1)
        roofline["frac_clock_adjusted"] = round(region_tf / peak_adj, 4)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 Q/K/V (S on FP8 MFMA; P and decoded V on bf16 MFMA; fp32 accumulate)",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: {wl.description}",
            "tokens_q": wl.total_q, "tokens_k": wl.total_k, "heads": heads,
            "head_dim_qk": 192, "head_dim_v": 128, "causal": bool(wl.causal),
            "segment": wl.segment_len or None, "causal_flop": flop,
            "step": "quant_static(Q,K,V) + " + ("prefill_chunked" if chunked else "prefill_varlen"),
        },
        "pct_fp8_peak": round(100.0 * value / FP8_PEAK_TFLOPS, 2),
        "kernels": kernels,
        "roofline": roofline,
        "kernel_hash": khash,
    }

    if not args.no_cpu_baseline:
        codes_np = [c.cpu().numpy() for c in codes]
        ds_np = [d.cpu().numpy() for d in descales]
        log("[bench] timing the CPU oracle on a sample ...")
        cb = cpu_baseline(wl, codes_np, ds_np, args.cpu_seconds)
        log(f"[bench] cpu oracle: {cb['value'] * 1e3:.2f} GFLOP/s on {cb['cores']} BLAS threads "
            f"({cb['host_cores']} host cores), {cb['seconds']:.1f} s")
        result["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "blas_threads",
                                                     "host_cores", "kind", "sample")}
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
