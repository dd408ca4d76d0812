"""Benchmark: EAGLE target-verify attention (topk = 1) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--all-configs]
                    [--extensions] [--p3-sweep]

One step = the whole path on one batch: block-table scatter, split-KV pass over
the prefix and the causal draft keys, log-sum-exp combine.  Inputs are seeded synthetic workloads
resident in HBM before timing starts.  Prints ONE JSON line:

  value          KV-read GB/s of the whole step on the headline workload (the
                 long-context batch): algorithmic bytes / step time, K steps between
                 two synchronisations, nothing else on the stream
  us_per_call    verify_attn_fwd + verify_attn_combine, K calls back to back
                 between two HIP events; call_pct_of_peak is its KV-read share of
                 the 8 TB/s HBM peak
  call_us        per call (events around fwd + combine only): median, p10, p90;
                 call_us_flushed the same with a 1 GiB read before each call
  roofline       the split-KV kernel (the dominant one): algorithmic bytes per
                 launch / its mean launch time (K launches back to back between two
                 HIP events on its stream), against the 8 TB/s HBM peak
  event_gap_us   what one recorded event adds to an interval on this stream
  cpu_baseline   the fp64 oracle timed on a bounded sample of the same workload
  per_config     the other two target workloads (sliding-window GQA, MLA share),
                 same protocol and their own roofline; with --all-configs also the
                 two small ones
  p3_sweep       (--p3-sweep) the split-KV page's kernel shape across contexts

Workloads whose read set is not at least twice the 256 MB Infinity Cache run over
several copies of the KV pool in rotation, so every step reads memory at least
512 MB of other reads have passed since.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# dense matrix-core peaks of MI355X (TFLOP/s): the bf16 MFMA serves bf16 KV, the fp8
# MFMA the fp8 MLA kernel
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}
CACHE_BYTES = 256 << 20


def traffic_for(workload: str, src_hash: str):
    """HBM bytes per launch measured by rocprofv3 counters, if recorded for this kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


def kernel_source_hash() -> str:
    """Hash of every kernel source: a recorded traffic figure is valid only for it."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "speculative_decoding_verify_02_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode())
                h.update(f.read())
    return h.hexdigest()


def _counter_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def traffic_from(fetch_csv: str, write_csv: str, copy_mib: int, workload: str,
                 kernel_key: str = "splitkv") -> dict:
    """HBM bytes per split-KV launch from two rocprofv3 --pmc runs (FETCH_SIZE, then
    WRITE_SIZE, in KiB per dispatch).  Each counter is scaled by what it reads for the
    plain device copy of `copy_mib` MiB that --copy-calibration-mib issues last: the
    copy reads and writes exactly that many bytes."""
    out = {"workload": workload, "kernel_source_sha256": kernel_source_hash(),
           "copy_calibration_bytes": copy_mib << 20}
    total = 0.0
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _counter_rows(path) if r["Counter_Name"] == counter]
        per = {}
        for r in rows:
            key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        copies = [(d, v) for (d, name), v in per.items() if "copyBuffer" in name]
        kern = [v for (d, name), v in per.items() if kernel_key in name]
        if not copies or not kern:
            raise SystemExit(f"{path}: no copy or {kernel_key} dispatches")
        copy_kib = max(copies)[1]             # the calibration copy is the last copy issued
        factor = (copy_mib << 20) / (copy_kib * 1024.0)
        mean_kib = sum(kern) / len(kern)
        bytes_per_launch = mean_kib * 1024.0 * factor
        out[counter] = {"kernel_mean_kib": round(mean_kib, 1), "copy_kib": round(copy_kib, 1),
                        "scale": round(factor, 4), "bytes_per_launch": round(bytes_per_launch)}
        total += bytes_per_launch
    out["hbm_bytes_per_launch"] = round(total)
    return out


def kv_copies_for(kv_bytes: int) -> int:
    """KV pool copies to rotate through: enough that at least 2x the Infinity Cache of
    other reads passes between two reads of one copy (1 when the read set is that big)."""
    if kv_bytes >= 2 * CACHE_BYTES:
        return 1
    return min(64, 1 + -(-2 * CACHE_BYTES // max(kv_bytes, 1)))


def kernel_name(p) -> str:
    """The split-KV kernel the library picks for a workload (the dominant one)."""
    from speculative_decoding_verify_02_amd import workloads as W
    if p.kv_dtype == W.KV_FP8_E4M3FN and p.qk_dim == 576 and p.v_aliases_k and \
            (p.hq // p.hkv) * p.draft_len <= 64:
        return "splitkv_mla_fp8_kernel"
    if p.kv_dtype == W.KV_BF16 and p.qk_dim == 256 and (p.hq // p.hkv) * p.draft_len <= 64:
        return "splitkv_tile_kernel"
    return "splitkv_fwd_kernel"


def _dist(xs):
    xs = sorted(xs)
    pick = lambda f: xs[min(len(xs) - 1, int(f * (len(xs) - 1) + 0.5))]
    return {"median": round(pick(0.5), 2), "p10": round(pick(0.1), 2), "p90": round(pick(0.9), 2)}


def measure(p, steps: int, warmup: int, splits=None, log=print, flushed=True):
    """Time one workload (a workloads.Problem) with the passes the JSON line reports."""
    import torch

    from speculative_decoding_verify_02_amd import binding
    from speculative_decoding_verify_02_amd import workloads as W
    from speculative_decoding_verify_02_amd.runner import DeviceProblem

    kv_bytes = W.algorithmic_kv_bytes(p)
    fwd_bytes = kv_bytes  # the split-KV pass reads every visible key, draft keys included
    copies = kv_copies_for(kv_bytes)
    dp = DeviceProblem(p, device="cuda", num_splits=splits, kv_copies=copies)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    new_event = lambda: torch.cuda.Event(enable_timing=True)

    for w in range(warmup):
        dp.step(copy=w % copies)
    torch.cuda.synchronize()

    # pass 1: K whole steps (block table, split-KV pass, combine) between two
    # synchronisations and nothing else on the stream, so no event sits inside a step
    # (a recorded event costs the stream a few microseconds of its own)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(steps):
        dp.step(copy=k % copies)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    # pass 2: the verify call (verify_attn_fwd + verify_attn_combine) K times back to
    # back between two events
    ea, eb = new_event(), new_event()
    torch.cuda.synchronize()
    ea.record(stream)
    for k in range(steps):
        binding.verify_attn_fwd(dp.calls[k % copies])
        binding.verify_attn_combine(dp.calls[k % copies])
    eb.record(stream)
    torch.cuda.synchronize()
    call_b2b_us = ea.elapsed_time(eb) * 1e3 / steps

    # pass 3: the split-KV kernel alone, K launches back to back between two events on
    # its stream: its mean launch time for the roofline (no event inside the interval)
    ea, eb = new_event(), new_event()
    torch.cuda.synchronize()
    ea.record(stream)
    for k in range(steps):
        binding.verify_attn_fwd(dp.calls[k % copies])
    eb.record(stream)
    torch.cuda.synchronize()
    fwd_b2b_us = ea.elapsed_time(eb) * 1e3 / steps

    # pass 4: events around each call (fwd + combine, no event between them): the
    # per-call distribution
    ev = [(new_event(), new_event()) for _ in range(steps)]
    torch.cuda.synchronize()
    for k, (e0, e1) in enumerate(ev):
        e0.record(stream)
        binding.verify_attn_fwd(dp.calls[k % copies])
        binding.verify_attn_combine(dp.calls[k % copies])
        e1.record(stream)
    torch.cuda.synchronize()
    call_us = [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]

    # pass 5: the same with a 1 GiB read before each call, outside the timed interval,
    # so no byte of the call's read set is left in the L2s or the Infinity Cache (a read,
    # not a fill: a fill leaves dirty lines whose write-back would land in the call)
    call_flushed = None
    if flushed:
        flush = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
        ev = [(new_event(), new_event()) for _ in range(steps)]
        torch.cuda.synchronize()
        for k, (e0, e1) in enumerate(ev):
            flush.sum()
            e0.record(stream)
            binding.verify_attn_fwd(dp.calls[k % copies])
            binding.verify_attn_combine(dp.calls[k % copies])
            e1.record(stream)
        torch.cuda.synchronize()
        call_flushed = [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]
        del flush

    # pass 6: events around each kernel of each step, for the per-kernel split (each
    # interval includes one event's own cost, measured below as an empty interval)
    ev = [[new_event() for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        c = k % copies
        e = ev[k]
        e[0].record(stream)
        dp.build_block_table()
        e[1].record(stream)
        binding.verify_attn_fwd(dp.calls[c])
        e[2].record(stream)
        binding.verify_attn_combine(dp.calls[c])
        e[3].record(stream)
    torch.cuda.synchronize()
    gaps = []
    for _ in range(20):
        g0, g1 = new_event(), new_event()
        g0.record(stream)
        g1.record(stream)
        torch.cuda.synchronize()
        gaps.append(g0.elapsed_time(g1) * 1e3)
    event_gap_us = sorted(gaps)[len(gaps) // 2]

    bt_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    fwd_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    comb_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / steps
    ms_per_step = wall * 1e3 / steps
    rec = dict(
        name=p.name, p=p, kv_bytes=kv_bytes, fwd_bytes=fwd_bytes, kernel=kernel_name(p),
        ms_per_step=ms_per_step, bt_us=bt_ms * 1e3, fwd_us=fwd_ms * 1e3, comb_us=comb_ms * 1e3,
        fwd_b2b_us=fwd_b2b_us, splits=dp.splits, copies=copies, call_b2b_us=call_b2b_us,
        event_gap_us=event_gap_us, call_us=_dist(call_us),
        call_us_flushed=None if call_flushed is None else _dist(call_flushed),
        step_gbs=kv_bytes / (ms_per_step * 1e-3) / 1e9,
        fwd_gbs=fwd_bytes / (fwd_b2b_us * 1e-6) / 1e9,
        flops=W.algorithmic_flops(p),
        mfma_dtype="fp8" if kernel_name(p) == "splitkv_mla_fp8_kernel" else "bf16",
    )
    rec["mfma_tflops"] = rec["flops"] / (fwd_b2b_us * 1e-6) / 1e12
    log(f"[bench] {p.name}: {ms_per_step * 1e3:.1f} us/step (events: bt {rec['bt_us']:.1f} + fwd "
        f"{rec['fwd_us']:.1f} + combine {rec['comb_us']:.1f} us), KV {kv_bytes / 1e6:.1f} MB, "
        f"step {rec['step_gbs']:.0f} GB/s, fwd back to back {fwd_b2b_us:.1f} us "
        f"({100 * rec['fwd_gbs'] / HBM_PEAK_GBS:.1f}% of peak), call back to back "
        f"{call_b2b_us:.1f} us ({100 * kv_bytes / (call_b2b_us * 1e-6) / 1e9 / HBM_PEAK_GBS:.1f}% "
        f"of peak), call median {rec['call_us']['median']} us"
        + (f", flushed {rec['call_us_flushed']['median']} us" if call_flushed else "")
        + f", event gap {event_gap_us:.1f} us, splits {dp.splits}, KV copies {copies}")
    del dp
    torch.cuda.empty_cache()
    return rec


def measure_config(idx: int, steps: int, warmup: int, splits=None, log=print, overrides=None,
                   label=None, flushed=True):
    from speculative_decoding_verify_02_amd import workloads as W
    t0 = time.time()
    p = W.make_config(idx, **(overrides or {}))
    if label:
        p.name = label
    log(f"[bench] config {idx} {p.name}: inputs drawn in {time.time() - t0:.1f}s")
    r = measure(p, steps, warmup, splits, log, flushed)
    r["idx"] = idx
    return r


def p3_sweep(steps: int, warmup: int, log=print):
    """The split-KV page's kernel shape (H_Q 16, H_KV 2, head_dim 256, 4 draft tokens,
    bf16, batch 1) across contexts, and the 16k point at batch 16: the page's ~536 MB
    of K + V read in 0.79 ms on MI350X by the prefill-kernel fallback ("Motivation").
    The page's table does not give a page size; the Triton backend's token-level pool
    (page size 1, shuffled slots) is used here."""
    from speculative_decoding_verify_02_amd import workloads as W
    out = {}
    for batch, ctx in [(1, 2048), (1, 4096), (1, 8192), (1, 16384), (1, 32768), (16, 16384)]:
        name = f"p3-b{batch}-ctx{ctx}"
        p = W.make_problem(name=name, batch=batch, prefix_lens=[ctx] * batch, draft_len=4, hq=16,
                           hkv=2, qk_dim=256, v_dim=256, page_size=1, seed=1100 + ctx + batch)
        r = measure(p, steps, warmup, None, log, flushed=False)
        out[name] = {"call_us_back_to_back": round(r["call_b2b_us"], 2),
                     "call_us": r["call_us"], "kv_mb": round(r["kv_bytes"] / 1e6, 2),
                     "call_gbs": round(r["kv_bytes"] / (r["call_b2b_us"] * 1e-6) / 1e9, 1),
                     "call_pct_of_peak": round(100 * r["kv_bytes"] / (r["call_b2b_us"] * 1e-6)
                                               / 1e9 / HBM_PEAK_GBS, 2),
                     "splits": r["splits"], "kv_copies": r["copies"]}
        if batch == 16:
            out[name]["page_figure"] = ("split-KV page, Motivation: ~536 MB of K+V in 0.79 ms "
                                        "(~680 GB/s) on MI350X with the prefill fallback")
    return out


def time_translation(steps: int, log=print):
    """verify_attn_translate_slots + the window pool's block table on the long-context
    batch's token list, through a page-preserving full-to-window map."""
    import numpy as np
    import torch

    from speculative_decoding_verify_02_amd import binding
    from speculative_decoding_verify_02_amd import workloads as W

    p = W.make_config(2)
    rng = np.random.default_rng(7)
    pmap = rng.permutation(p.num_pages)
    full_to_swa = (pmap[np.arange(p.num_slots) // p.page_size] * p.page_size
                   + np.arange(p.num_slots) % p.page_size).astype(np.int32)
    dev = "cuda"
    idx = torch.from_numpy(p.kv_indices).to(dev)
    mp = torch.from_numpy(full_to_swa).to(dev)
    out = torch.empty_like(idx)
    indptr = torch.from_numpy(p.kv_indptr).to(dev)
    bt = torch.empty((p.batch, p.max_pages_per_seq), dtype=torch.int32, device=dev)
    for _ in range(3):
        binding.verify_attn_translate_slots(idx, mp, out)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    stream = torch.cuda.current_stream()
    for e in ev:
        e[0].record(stream)
        binding.verify_attn_translate_slots(idx, mp, out)
        e[1].record(stream)
        binding.verify_attn_build_block_table(indptr, out, p.page_size, p.max_pages_per_seq, bt)
        e[2].record(stream)
    torch.cuda.synchronize()
    tr_us = sorted(e[0].elapsed_time(e[1]) * 1e3 for e in ev)[len(ev) // 2]
    bt_us = sorted(e[1].elapsed_time(e[2]) * 1e3 for e in ev)[len(ev) // 2]
    n = int(idx.numel())
    log(f"[bench] slot translation: {n} slots in {tr_us:.1f} us, window-pool table {bt_us:.1f} us")
    # bytes: read the slot, gather the map entry, write the result
    return {"slots": n, "translate_us": round(tr_us, 2), "block_table_us": round(bt_us, 2),
            "translate_gbs": round(12 * n / (tr_us * 1e-6) / 1e9, 1)}


def cpu_baseline(p, budget_s: float = 12.0, log=print):
    """The oracle as it stands on a bounded prefix of the workload's sequences, with as
    many BLAS threads as this process may run on (the count is reported as `cores`)."""
    from threadpoolctl import threadpool_limits

    import oracle
    from speculative_decoding_verify_02_amd import workloads as W

    cores = len(os.sched_getaffinity(0))
    per_tok = p.hkv * (p.qk_dim + (0 if p.v_aliases_k else p.v_dim)) * p.elem_bytes
    done_bytes, nseq = 0, 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=cores):
        for b in range(p.batch):
            rows = list(range(b * p.draft_len, (b + 1) * p.draft_len))
            oracle.run(p, rows=rows)
            done_bytes += W.visible_token_count(int(p.prefix_lens[b]), p.draft_len,
                                                p.window_left) * per_tok
            nseq += 1
            if time.perf_counter() - t0 > budget_s:
                break
    dt = time.perf_counter() - t0
    log(f"[bench] cpu oracle: {nseq} of {p.batch} sequences in {dt:.1f}s, {cores} BLAS threads")
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{nseq} of {p.batch} sequences of {p.name} (all draft rows and heads), "
                      f"{done_bytes / 1e6:.1f} MB of KV in {dt:.1f}s, fp64 NumPy, BLAS threads = "
                      f"{cores} (len(os.sched_getaffinity(0)))"}


def workload_config(p) -> dict:
    L = p.prefix_lens
    return {"workload": p.name, "batch": p.batch, "prefix_len_min": int(L.min()),
            "prefix_len_max": int(L.max()), "draft_len": p.draft_len, "hq": p.hq, "hkv": p.hkv,
            "qk_dim": p.qk_dim, "v_dim": p.v_dim, "page_size": p.page_size,
            "kv_dtype": "fp8_e4m3fn" if p.kv_dtype == 1 else "bf16",
            "window_left": p.window_left}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="headline workload index")
    ap.add_argument("--only", action="store_true",
                    help="time the headline workload alone (no per_config entries)")
    ap.add_argument("--all-configs", action="store_true",
                    help="also time the two small workloads (launch-bound)")
    ap.add_argument("--extensions", action="store_true",
                    help="also time draft-extend rows, tree verify, sinks + logit cap and the "
                         "window-pool slot translation")
    ap.add_argument("--p3-sweep", action="store_true",
                    help="also time the split-KV page's kernel shape across contexts")
    ap.add_argument("--splits", type=int, default=None, help="override the split heuristic")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true", help="skip the flushed-cache pass")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, issue one plain device copy of this size (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 counter CSVs")
    args = ap.parse_args()

    if args.traffic_from:
        from speculative_decoding_verify_02_amd import workloads as W
        name = W.CONFIG_NAMES[args.config]
        p = W.make_config(args.config)
        rec = traffic_from(args.traffic_from[0], args.traffic_from[1],
                           args.copy_calibration_mib or 1024, name, kernel_key=kernel_name(p))
        rec["algorithmic_kv_bytes"] = W.algorithmic_kv_bytes(p)
        path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path has no multi-GPU mode (asked for "
              f"--gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    name = torch.cuda.get_device_properties(0).gcnArchName
    if not name.startswith("gfx950"):
        print(f"bench.py targets MI355X (gfx950); found {name}", file=sys.stderr)
        sys.exit(1)

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    src_hash = kernel_source_hash()

    def mfma_summary(r):
        # algorithmic matrix flops of the split-KV pass over its mean launch time, against
        # the dense peak of the MFMA type the kernel runs
        peak = MFMA_PEAK_TFLOPS[r["mfma_dtype"]]
        return {"dtype": r["mfma_dtype"], "algorithmic_flops_per_launch": r["flops"],
                "achieved_tflops": round(r["mfma_tflops"], 1), "peak_tflops": peak,
                "frac": round(r["mfma_tflops"] / peak, 4)}

    def roofline(r):
        return {"bound": "hbm", "achieved": round(r["fwd_gbs"], 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(r["fwd_gbs"] / HBM_PEAK_GBS, 4),
                "traffic": traffic_for(r["name"], src_hash), "kernel": r["kernel"],
                "algorithmic_bytes_per_launch": r["fwd_bytes"],
                "mean_launch_us": round(r["fwd_b2b_us"], 2)}

    def call_pct(r):
        return round(100 * r["kv_bytes"] / (r["call_b2b_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)

    def summary(r):
        return {
            "config": workload_config(r["p"]),
            "kv_mb": round(r["kv_bytes"] / 1e6, 2),
            "us_per_step": round(r["ms_per_step"] * 1e3, 2),
            "call_us_back_to_back": round(r["call_b2b_us"], 2),
            "call_pct_of_peak": call_pct(r),
            "call_us": r["call_us"],
            "call_us_flushed": r["call_us_flushed"],
            "kernel_us_with_events": {"block_table": round(r["bt_us"], 2),
                                      "splitkv_fwd": round(r["fwd_us"], 2),
                                      "combine": round(r["comb_us"], 2)},
            "roofline": roofline(r),
            "mfma": mfma_summary(r),
            "splits": r["splits"], "kv_copies": r["copies"]}

    flushed = not args.no_flush
    head = measure_config(args.config, args.steps, args.warmup, args.splits, log, flushed=flushed)
    per_config = {}
    others = [] if args.only else [3, 4]
    if args.all_configs:
        others = [0, 1, 2, 3, 4]
    for idx in others:
        if idx == args.config:
            continue
        r = measure_config(idx, args.steps, args.warmup, None, log, flushed=flushed)
        per_config[r["name"]] = summary(r)
    extensions = {}
    if args.extensions:
        # the version 2 extensions on the long-context batch (and the MLA share)
        for idx, over, label in (
                (2, dict(ragged=True), "long-context-batch+draft-extend-rows"),
                (2, dict(tree=True), "long-context-batch+tree-verify"),
                (2, dict(sinks=True, logit_cap=30.0), "long-context-batch+sinks+logit-cap"),
                (4, dict(tree=True), "mla-fp8-share+tree-verify")):
            r = measure_config(idx, args.steps, args.warmup, None, log, overrides=over,
                               label=label, flushed=False)
            extensions[label] = summary(r)
        extensions["window-pool-slot-translation"] = time_translation(args.steps, log)
    p3 = p3_sweep(args.steps, args.warmup, log) if args.p3_sweep else None

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 19     # bf16 elements
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.copy_calibration_mib} MiB issued")
        del src, dst

    p = head["p"]
    cpu = None if args.no_cpu_baseline else cpu_baseline(p, log=log)

    out = {
        "metric": "verify-attention us/call + KV-read HBM GB/s (% of MI355X peak) at 1 GPU",
        "value": round(head["step_gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        # verify_attn_fwd + verify_attn_combine, K calls back to back between two events
        "us_per_call": round(head["call_b2b_us"], 2),
        "pct_of_peak": round(100 * head["step_gbs"] / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q/k/v, shuffled page table)",
        "config": dict(workload_config(p), splits=head["splits"], kv_copies=head["copies"],
                       kv_mb=round(head["kv_bytes"] / 1e6, 2)),
        # the call's share of peak: algorithmic KV bytes over the back-to-back call time
        "call_pct_of_peak": call_pct(head),
        # per call, events around fwd + combine only (median, p10, p90), and the same
        # with a 1 GiB read before each call (nothing of the read set left in any cache)
        "call_us": head["call_us"],
        "call_us_flushed": head["call_us_flushed"],
        # per kernel, events around each launch (each includes one event's own cost)
        "kernel_us_with_events": {"block_table": round(head["bt_us"], 2),
                                  "splitkv_fwd": round(head["fwd_us"], 2),
                                  "combine": round(head["comb_us"], 2)},
        "event_gap_us": round(head["event_gap_us"], 2),
        "roofline": roofline(head),
        # the same kernel against the matrix cores (an HBM-bound kernel sits far below)
        "mfma": mfma_summary(head),
        "cpu_baseline": cpu,
    }
    if per_config:
        out["per_config"] = per_config
    if extensions:
        out["extensions"] = extensions
    if p3:
        out["p3_sweep"] = p3
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
