#!/usr/bin/env python3
"""Benchmark: paged-attention decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one pass of the hot path over one batch: the KV write of each
sequence's new token into its slot (fp16 copy, or quantising int8 / FP8 write),
then paged decode attention over every sequence's context (split-K partition
kernel, plus the log-sum-exp merge when the context spans several
partitions).  Inputs are seeded synthetic tensors already resident in HBM.

Headline workload: one Llama2-7B-shaped layer - 32 sequences x 4096 tokens,
32 query / 32 kv heads, head_dim 128, fp16, 16-token blocks, block tables 85 %
contiguous.  metric value = ideal KV bytes / step time (GB/s); the other
workloads are measured the same way and reported under "others"; the
shared-prefix workload is measured twice, through pa_decode and through the
shared-prefix entry point (whose "decode call" time covers its three
kernels).  "cold" repeats steps one at a time with L2 and MALL flushed first.

"roofline" describes the dominant kernel (the decode partition kernel):
achieved = its algorithmic bytes (the KV bytes it must read) / its mean
duration, timed with HIP events recorded on the stream it runs on, around
the launch of every fifth timed step (--event-every; an event is a marker in
the stream and costs the step a few microseconds, so the other steps run
without).  "traffic" comes from rocprofv3 counter
summaries committed under profiles/ and is null unless they were taken on
the current kernel source.  "cpu_baseline" times the fp64 CPU oracle on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
METRIC = "paged-attn decode: achieved KV HBM GB/s (% of peak) and sequences/s per layer"
HEADLINE = "llama2_7b"
OTHERS = ["gqa70b_mixed", "prefix_shared", "long128k_int8", "long128k_fp8", "tiny_gqa"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--others", default=",".join(OTHERS),
                    help="comma list of extra workloads to report ('' for none)")
    ap.add_argument("--partition-size", type=int, default=-1,
                    help="override the partition size (-1: the workload's own choice)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--shared-prefix", action="store_true",
                    help="run the workload through the shared-prefix entry point "
                         "(workloads with a shared prefix only)")
    ap.add_argument("--event-every", type=int, default=5,
                    help="bracket the decode kernel of every N-th timed step with HIP events "
                         "(the kernel mean comes from those launches)")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="extra steps timed one by one with L2 and MALL flushed before "
                         "each (reported under 'cold'; 0 to skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (the "
                         "known-size reference for rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--counters-summary", nargs=5, default=None,
                    metavar=("OUT_JSON", "DECODE_FETCH_DIR", "DECODE_WRITE_DIR",
                             "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="host only: summarise rocprofv3 --pmc databases of a decode "
                         "run (FETCH_SIZE, WRITE_SIZE) and of a --copy-calibration run "
                         "into OUT_JSON (uses --workload and --copy-calibration MIB)")
    return ap.parse_args()


def source_hash() -> str:
    """Hash of the library sources (every file under csrc/); counter
    summaries carry the hash they were taken on and are ignored once it
    changes."""
    csrc = os.path.join(ROOT, "paged_kv_cache_238_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def decode_kernel_name(wl) -> str:
    return "decode_valu_kernel" if wl.q_heads // wl.kv_heads <= 2 else "decode_mfma_kernel"


class Case:
    """Device-resident inputs of one workload plus its step."""

    def __init__(self, pa, torch, gen, name, partition_size, dev, shared_prefix=0):
        self.pa, self.torch, self.name = pa, torch, name
        self.shared_prefix = shared_prefix          # > 0: shared-prefix path, prefix tokens
        wl = gen.make(name, poison=False)
        self.wl = wl
        vals = gen.fill_torch(wl, dev)
        self.v = vals
        self.bt = torch.from_numpy(wl.block_table).to(dev)
        self.cl = torch.from_numpy(wl.context_lens).to(dev)
        self.slots = torch.from_numpy(wl.new_slots).to(dev)
        P = wl.partition_size if partition_size < 0 else partition_size
        self.P = pa.partition_size(wl.batch, wl.q_heads, wl.kv_heads, wl.head_dim,
                                   wl.max_context_len, P)
        self.n_part = max(1, -(-wl.max_context_len // self.P))
        need = pa.workspace_size(wl.batch, wl.q_heads, wl.kv_heads, wl.head_dim,
                                 wl.max_context_len, self.P)
        if shared_prefix:
            need = pa.shared_prefix_workspace_size(wl.batch, wl.q_heads, wl.kv_heads,
                                                   wl.head_dim, wl.max_context_len,
                                                   shared_prefix)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        self.out = torch.empty_like(vals["q"])
        self.q8 = wl.kv_dtype in ("int8", "fp8")             # 8-bit codes + scales
        self.kv_bytes = gen.kv_ideal_bytes(wl)                # unique bytes
        self.kv_bytes_logical = gen.kv_ideal_bytes(wl, unique=False)

    def write(self):
        v = self.v
        if self.q8:
            fn = self.pa.write_kv_int8 if self.wl.kv_dtype == "int8" else self.pa.write_kv_fp8
            fn(v["k_new"], v["v_new"], self.slots, v["k_pool"], v["v_pool"], v["k_scale"],
               v["v_scale"])
        else:
            self.pa.write_kv(v["k_new"], v["v_new"], self.slots, v["k_pool"], v["v_pool"])

    def decode_kernel(self):
        """The partition kernel alone: direct output when one partition
        covers the context, else the partition records."""
        v, wl = self.v, self.wl
        if self.shared_prefix:
            # the whole entry point: suffix partition kernel, prefix kernel, merge
            self.pa.decode_shared_prefix(v["q"], v["k_pool"], v["v_pool"], self.bt, self.cl,
                                         self.shared_prefix, scale=wl.scale,
                                         max_context_len=wl.max_context_len, out=self.out,
                                         workspace=self.ws, k_scale=v.get("k_scale"),
                                         v_scale=v.get("v_scale"))
        elif self.n_part == 1:
            if self.q8:
                fn = self.pa.decode_int8 if wl.kv_dtype == "int8" else self.pa.decode_fp8
                fn(v["q"], v["k_pool"], v["v_pool"], v["k_scale"], v["v_scale"], self.bt, self.cl,
                   scale=wl.scale, partition_size=self.P, max_context_len=wl.max_context_len,
                   out=self.out, workspace=self.ws)
            else:
                self.pa.decode(v["q"], v["k_pool"], v["v_pool"], self.bt, self.cl, scale=wl.scale,
                               partition_size=self.P, max_context_len=wl.max_context_len,
                               out=self.out, workspace=self.ws)
        else:
            self.pa.decode_partials(v["q"], v["k_pool"], v["v_pool"], self.bt, self.cl, self.ws,
                                    scale=wl.scale, partition_size=self.P,
                                    max_context_len=wl.max_context_len,
                                    k_scale=v.get("k_scale"), v_scale=v.get("v_scale"))

    def merge(self):
        if self.n_part > 1 and not self.shared_prefix:
            wl = self.wl
            self.pa.merge_partials(self.ws, self.cl, wl.q_heads, wl.head_dim, self.P,
                                   wl.max_context_len, out=self.out)

    def run(self, steps, warmup, event_every=1):
        """Warm-up, then `steps` timed steps.  The decode kernel of every
        `event_every`-th timed step is bracketed by HIP events on its stream
        (each event is a marker in the stream, and the steps between two
        sampled ones run without them)."""
        torch = self.torch
        for _ in range(warmup):
            self.write()
            self.decode_kernel()
            self.merge()
        every = max(1, int(event_every))
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(0, steps, every)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.write()
            if i % every == 0:
                a, b = ev[i // every]
                a.record()
                self.decode_kernel()
                b.record()
            else:
                self.decode_kernel()
            self.merge()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kern_ms = sorted(a.elapsed_time(b) for a, b in ev)
        return wall, kern_ms

    def run_cold(self, steps, flush_bytes=1 << 30):
        """Steps with the caches flushed before each: a 1 GiB buffer (beyond
        the 256 MB MALL and the 8 x 4 MB of L2) is read, outside the timed
        events.  Reading rather than zeroing leaves no dirty lines whose
        write-back would land inside the timed step.  Returns sorted step and
        decode-kernel times (ms)."""
        torch = self.torch
        flush = torch.ones(flush_bytes // 8, dtype=torch.int64, device=self.v["q"].device)
        step_ms, kern_ms = [], []
        for _ in range(steps):
            flush.sum()
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            e[0].record()
            self.write()
            e[1].record()
            self.decode_kernel()
            e[2].record()
            self.merge()
            e[3].record()
            torch.cuda.synchronize()
            step_ms.append(e[0].elapsed_time(e[3]))
            kern_ms.append(e[1].elapsed_time(e[2]))
        del flush
        return sorted(step_ms), sorted(kern_ms)


def cold_summary(case, steps):
    """Median and p10/p90 of cold steps (caches flushed before each)."""
    if steps <= 0:
        return None
    step_ms, kern_ms = case.run_cold(steps)

    def pick(v, q):
        return v[min(len(v) - 1, int(q * len(v)))]
    step_med = pick(step_ms, 0.5) / 1e3
    kern_med = pick(kern_ms, 0.5) / 1e3
    return {
        "steps": steps,
        "step_us_median": round(step_med * 1e6, 2),
        "step_us_p10_p90": [round(pick(step_ms, 0.1) * 1e3, 2), round(pick(step_ms, 0.9) * 1e3, 2)],
        "step_GBps": round(case.kv_bytes / step_med / 1e9, 1),
        "decode_kernel_us_median": round(kern_med * 1e6, 2),
        "decode_kernel_GBps": round(case.kv_bytes / kern_med / 1e9, 1),
    }


def summarize(case, wall, kern_ms, steps):
    wl = case.wl
    step_s = wall / steps
    kmean = sum(kern_ms) / len(kern_ms) / 1e3
    med = kern_ms[len(kern_ms) // 2] / 1e3
    return {
        "workload": wl.name + (" (shared-prefix path)" if case.shared_prefix else ""),
        "batch": wl.batch, "q_heads": wl.q_heads, "kv_heads": wl.kv_heads,
        "head_dim": wl.head_dim, "block_size": 16, "kv_dtype": wl.kv_dtype,
        "max_context_len": wl.max_context_len,
        "mean_context_len": round(float(wl.context_lens.mean()), 1),
        "partition_size": case.P, "n_part": case.n_part,
        "kv_bytes": case.kv_bytes, "kv_bytes_logical": case.kv_bytes_logical,
        "ms_per_step": round(step_s * 1e3, 4),
        "step_GBps": round(case.kv_bytes / step_s / 1e9, 1),
        "seq_per_s": round(wl.batch / step_s, 1),
        "decode_kernel_us_mean": round(kmean * 1e6, 2),
        "decode_kernel_us_median": round(med * 1e6, 2),
        "decode_kernel_GBps": round(case.kv_bytes / kmean / 1e9, 1),
        "decode_kernel_frac_of_peak": round(case.kv_bytes / kmean / 1e9 / PEAK_HBM_GBS, 4),
    }


def traffic_for(name):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"decode_{name}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("source_hash") != source_hash():
        return None
    return c.get("traffic_bytes_per_launch")


def _counter_means(directory, counter):
    """kernel name -> (dispatches, mean value per dispatch) from a rocpd db."""
    import glob
    import sqlite3
    out = {}
    for db in glob.glob(os.path.join(directory, "**", "*.db"), recursive=True):
        con = sqlite3.connect(db)
        rows = con.execute("select kernel_name, value from counters_collection "
                           "where counter_name = ?", (counter,)).fetchall()
        acc = {}
        for name, val in rows:
            acc.setdefault(name, []).append(val)
        for name, vals in acc.items():
            out[name] = (len(vals), sum(vals) / len(vals))
    return out


def counters_summary(args):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the decode kernel,
    scaled by what the same counters read for a plain copy of known size."""
    from workloads import gen
    out_json, dfetch, dwrite, cfetch, cwrite = args.counters_summary
    wl = gen.make(args.workload, poison=False)
    # the shared-prefix entry point's partition work runs in its own kernel
    kname = "shared_prefix_kernel" if args.shared_prefix else decode_kernel_name(wl)
    known = args.copy_calibration << 20

    def pick(table, key):
        hits = {k: v for k, v in table.items() if key in k}
        if not hits:
            raise SystemExit(f"no dispatch of a kernel named like {key!r}")
        return max(hits.items(), key=lambda kv: kv[1][1])

    def copy_kernel(table):     # the copy: the dispatch with the largest counter
        return max(table.items(), key=lambda kv: kv[1][1])

    cf_name, (cf_n, cf) = copy_kernel(_counter_means(cfetch, "FETCH_SIZE"))
    cw_name, (cw_n, cw) = copy_kernel(_counter_means(cwrite, "WRITE_SIZE"))
    df_name, (df_n, df) = pick(_counter_means(dfetch, "FETCH_SIZE"), kname)
    dw_name, (dw_n, dw) = pick(_counter_means(dwrite, "WRITE_SIZE"), kname)
    f_fetch = known / (cf * 1024.0)
    f_write = known / (cw * 1024.0)
    traffic = df * 1024.0 * f_fetch + dw * 1024.0 * f_write
    res = {
        "workload": wl.name + (" (shared-prefix path)" if args.shared_prefix else ""),
        "kernel": df_name, "source_hash": source_hash(),
        "decode_fetch_kib_per_dispatch": df, "decode_write_kib_per_dispatch": dw,
        "decode_dispatches": [df_n, dw_n],
        "copy_kernel": cf_name, "copy_bytes": known,
        "copy_fetch_kib_per_dispatch": cf, "copy_write_kib_per_dispatch": cw,
        "fetch_scale": f_fetch, "write_scale": f_write,
        "traffic_bytes_per_launch": round(traffic),
        "algorithmic_bytes_per_launch": gen.kv_ideal_bytes(wl),
        "traffic_over_algorithmic": round(traffic / gen.kv_ideal_bytes(wl), 4),
    }
    with open(out_json, "w") as f:
        json.dump(res, f, indent=2)
    print(json.dumps(res, indent=2))


def cpu_baseline(case, budget_s):
    """fp64 oracle on the host: whole sequences (all heads) in order until
    the time budget is spent; single thread (BLAS pinned to one)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import ref
    wl = case.wl
    v = case.v
    host = {k: v[k].cpu().numpy() for k in ("q", "k_pool", "v_pool")}
    ks = v["k_scale"].cpu().numpy() if case.q8 else None
    vs = v["v_scale"].cpu().numpy() if case.q8 else None
    done_bytes, done_seqs = 0, 0
    per_tok = case.kv_bytes_logical / max(1, int(wl.context_lens.sum()))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for b in range(wl.batch):
            rows = [(b, h) for h in range(wl.q_heads)]
            ref.ref_decode(host["q"], host["k_pool"], host["v_pool"], wl.block_table,
                           wl.context_lens, wl.scale, ks, vs, rows=rows)
            done_seqs += 1
            done_bytes += int(wl.context_lens[b]) * per_tok
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "seq_per_s": round(done_seqs / dt, 3),
            "sample": f"{done_seqs} of {wl.batch} sequences of {wl.name} (all "
                      f"{wl.q_heads} heads each), fp64 numpy, one thread, {dt:.1f} s"}


def main():
    args = parse()
    if args.counters_summary:
        counters_summary(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path runs on a single device)", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_calibration:
        dev = torch.device("cuda:0")
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)
        return

    import paged_kv_cache_238_amd as pa
    from workloads import gen

    dev = torch.device("cuda:0")
    pre = gen.SPECS[args.workload].get("prefix", 0) if args.shared_prefix else 0
    if args.shared_prefix and not pre:
        raise SystemExit(f"--shared-prefix: workload {args.workload} has no shared prefix")
    head = Case(pa, torch, gen, args.workload, args.partition_size, dev, shared_prefix=pre)
    wall, kern = head.run(args.steps, args.warmup, args.event_every)
    s = summarize(head, wall, kern, args.steps)
    s["cold"] = cold_summary(head, args.cold_steps)
    print(f"[bench] {args.workload}: {s['ms_per_step']} ms/step, decode kernel "
          f"{s['decode_kernel_us_mean']} us = {s['decode_kernel_GBps']} GB/s", file=sys.stderr,
          flush=True)
    if s["cold"]:
        print(f"[bench] {args.workload} cold: step {s['cold']['step_us_median']} us, decode "
              f"kernel {s['cold']['decode_kernel_us_median']} us = "
              f"{s['cold']['decode_kernel_GBps']} GB/s", file=sys.stderr, flush=True)
    others = []
    for name in [n for n in args.others.split(",") if n and n != args.workload]:
        c = Case(pa, torch, gen, name, -1, dev)
        w2, k2 = c.run(max(20, args.steps // 2), max(5, args.warmup // 2), args.event_every)
        o = summarize(c, w2, k2, max(20, args.steps // 2))
        o["cold"] = cold_summary(c, args.cold_steps)
        others.append(o)
        print(f"[bench] {name}: {o['ms_per_step']} ms/step, decode kernel "
              f"{o['decode_kernel_us_mean']} us = {o['decode_kernel_GBps']} GB/s",
              file=sys.stderr, flush=True)
        del c
        torch.cuda.empty_cache()
        if name == "prefix_shared":
            # the same workload through the shared-prefix entry point
            c = Case(pa, torch, gen, name, -1, dev, shared_prefix=gen.SPECS[name]["prefix"])
            w2, k2 = c.run(max(20, args.steps // 2), max(5, args.warmup // 2), args.event_every)
            o = summarize(c, w2, k2, max(20, args.steps // 2))
            o["cold"] = cold_summary(c, args.cold_steps)
            others.append(o)
            print(f"[bench] {o['workload']}: {o['ms_per_step']} ms/step, decode call "
                  f"{o['decode_kernel_us_mean']} us = {o['decode_kernel_GBps']} GB/s",
                  file=sys.stderr, flush=True)
            del c
            torch.cuda.empty_cache()
    cpu = None if args.no_cpu_baseline else cpu_baseline(head, args.cpu_seconds)
    achieved = s["decode_kernel_GBps"]
    line = {
        "metric": METRIC,
        "value": s["step_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": s["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "accumulate": "f32",
        "data": "synthetic (seeded N(0,1) fp16 K/V/Q; block tables per workload recipe)",
        "pct_of_peak": round(100 * s["step_GBps"] / PEAK_HBM_GBS, 2),
        "seq_per_s": s["seq_per_s"],
        "config": {k: s[k] for k in ("workload", "batch", "q_heads", "kv_heads", "head_dim",
                                     "block_size", "kv_dtype", "max_context_len",
                                     "partition_size", "n_part", "kv_bytes")},
        "roofline": {"bound": "hbm", "kernel": decode_kernel_name(head.wl),
                     "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "algorithmic_bytes_per_launch": s["kv_bytes"],
                     "launch_us_mean": s["decode_kernel_us_mean"],
                     "launches_timed": len(kern),
                     "traffic": traffic_for(args.workload),
                     "source_hash": source_hash()},
        "cold": s["cold"],
        "cpu_baseline": cpu,
        "others": others,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
