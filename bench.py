#!/usr/bin/env python3
"""Benchmark: one paged decode step of 4-bit, group-64 affine KV pages at head dim 256.

A step is the whole hot path on one batch, run through the library's decode-step entry points
(paged_decode_step_partial, then paged_decode_merge): quantize-on-append of the B*N new K/V rows
into the slots their positions take in the block table, the copy of q in the codes' order, the
split-K partial kernel over every cached token (block-table reads, dequantize-on-load,
GQA-shared K/V rows, online softmax in f32), and the log-sum-exp merge.  Inputs are seeded
synthetic data resident in HBM before timing starts; the pool holds every cached row but each
sequence's last N, which every step appends again (same rows, same slots).

Default workload ("c3"): 32 sequences with lengths drawn uniformly in [4096, 32768] tokens
(sum 598,835), block size 32 with a shuffled block table, 16 query heads over 2 KV heads
(GQA 8), head dim 256, one query row, K/V N(0,1) with 3 outlier channels per KV head
scaled x8.  Beside it, in "variants": the matrix-core engine on the same inputs, and the
32k-context shape ("diag": 32 sequences of 32768 tokens, 8 query heads over 2 KV heads, head
dim 256, 4-bit pages of 32 tokens), on which the vector engine's per-token work stays below
the HBM time.

Prints one JSON line (stdout, last line): effective K/V GB/s (bytes of codes + scales +
biases of every cached token, per step) with the fraction of the 8 TB/s HBM peak,
microseconds per step (mean of K back-to-back steps; median and p10/p90 of per-step events;
cold steps after a 1 GiB read), the partial kernel's roofline figures, and the CPU oracle
timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import concurrent.futures
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
SETTLE_S = 0.2              # seconds of untimed steps before the warm-up steps (clock ramp-up)
# MI355X published dense fp32 vector peak (256 CUs x 4 SIMDs x 16 lanes x 2 FMA x 2 flop x 2.4 GHz:
# packed FP32).  Code here issues no packed FP32, so the vector path's attainable ceiling is half
# of it for its f32 FMAs (its 16-bit dot2 steps still do 2 MACs per lane-op).
VALU_PEAK_TFLOPS = 157.3
METRIC = "effective KV GB/s (% of HBM peak) + µs per decode step, 4-bit paged D=256"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the sources that decide what the partial kernel reads and writes (its code and the
    host-side launch geometry), comments and blank lines left out: a change of wording keeps the
    counters that were taken on the same code."""
    h = hashlib.sha256()
    for f in ("partial_valu.hip", "partial_valu_impl.hpp", "partial_valu_b4.hip", "device_common.hpp",
              "kernels.hpp", "api.cpp"):
        with open(os.path.join(ROOT, "decode_attention_paged_split_amd", "csrc", f), encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str, src_hash: str):
    """HBM bytes per partial launch from the committed counter summary, if it was taken on the
    current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", f"partial_kernel_pmc_{workload}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source_hash") != src_hash:
        return None
    return d.get("traffic_bytes_per_launch")


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return 1


def cpu_baseline(w, budget_s: float):
    """The oracle's decode step on a bounded sample of sequences: append (quantize) the N new
    rows, gather every cached row through the block table, unpack, dequantize in f64 and
    run the f64 two-pass attention.  The sample grows until ~budget_s of CPU work.  The oracle's
    only parallelism is NumPy's BLAS thread pool (its matrix products), so the threads it uses
    are that pool's size, never more than the cores the process may run on."""
    from oracle import attention, paged
    affinity = len(os.sched_getaffinity(0))
    blas = _blas_threads()
    order = list(range(w.B))
    done, elapsed, eff = [], 0.0, 0
    per = w.effective_bytes() // (int(w.lengths.sum()) * w.HK)          # K + V row bytes of a token
    pool = paged.Pool(w.num_blocks, w.HK, w.BS, w.D, w.bits, w.group, v_head_dim=w.DV)
    while order and elapsed < budget_s:
        b = order.pop(0)
        k, v = w.kv(b)
        L = int(w.lengths[b])
        pool.write(k[: L - w.N], v[: L - w.N], w.slots(b, 0, L - w.N))        # cached before the step
        q = attention.q_f64(w.q_bits[b:b + 1])
        t0 = time.perf_counter()
        pool.write(k[L - w.N:], v[L - w.N:], w.slots(b, L - w.N, L))          # the step's new rows
        kk, vv = pool.dequantized(w.table[b], L)
        attention.decode_attention(q, [kk], [vv], w.lengths[b:b + 1], w.scale)
        elapsed += time.perf_counter() - t0
        done.append(b)
        eff += L * w.HK * per
    return {"value": eff / elapsed / 1e9, "unit": "GB/s", "cores": int(min(blas, affinity)), "kind": "oracle",
            "sample": f"{len(done)} of {w.B} sequences ({sum(int(w.lengths[b]) for b in done)} tokens), "
                      f"{elapsed:.1f} s of f64 NumPy: append-quantize of the new rows, gather, unpack, "
                      f"dequantize, two-pass attention",
            "seconds": round(elapsed, 2), "affinity_cores": affinity, "blas_threads": blas,
            "cpu": _cpu_model()}


def _cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _quantiles_us(ms_list):
    a = np.asarray(ms_list, dtype=np.float64) * 1e3
    return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "n": int(a.size)}


class Bench:
    """One workload's device inputs (pool filled with every cached row but each sequence's last N,
    the N new rows, q, table, lengths) and its timing passes."""

    def __init__(self, kvq, torch, w, dev):
        self.kvq, self.torch, self.w, self.dev = kvq, torch, w, dev
        t_setup = time.time()
        log(f"[bench] workload {w.name}: B={w.B} HQ={w.HQ} HK={w.HK} D={w.D} DV={w.DV} N={w.N} bits={w.bits} "
            f"BS={w.BS} sum(len)={int(w.lengths.sum())} NB={w.num_blocks}")
        self.pool = kvq.Pool(w.num_blocks, w.HK, w.BS, w.D, w.bits, w.group, device=dev, v_head_dim=w.DV)
        new_k, new_v = [], []
        # the draws of each sequence are independent (own seed), so a few threads generate them
        # ahead of the device appends (NumPy's generators release the GIL)
        gen = concurrent.futures.ThreadPoolExecutor(max_workers=8)
        ahead = 16
        futs = [gen.submit(w.kv, b) for b in range(min(ahead, w.B))]
        for b in range(w.B):
            k, v = futs[b].result()
            futs[b] = None
            if b + ahead < w.B:
                futs.append(gen.submit(w.kv, b + ahead))
            L = int(w.lengths[b])
            self.pool.append(torch.from_numpy(k[: L - w.N].view(np.int16)).to(dev),
                             torch.from_numpy(v[: L - w.N].view(np.int16)).to(dev),
                             torch.from_numpy(w.slots(b, 0, L - w.N)).to(dev))
            new_k.append(k[L - w.N:]), new_v.append(v[L - w.N:])
            if b % 8 == 7:
                log(f"[bench] filled {b + 1}/{w.B} sequences ({time.time() - t_setup:.0f} s)")
        gen.shutdown()
        self.kn = torch.from_numpy(np.concatenate(new_k).view(np.int16)).to(dev).view(w.B, w.N, w.HK, w.D)
        self.vn = torch.from_numpy(np.concatenate(new_v).view(np.int16)).to(dev).view(w.B, w.N, w.HK, w.DV)
        self.q = torch.from_numpy(w.q_bits.view(np.int16)).to(dev)
        self.table = torch.from_numpy(w.table).to(dev)
        self.lengths = torch.from_numpy(w.lengths.astype(np.int32)).to(dev)
        self.out = torch.empty((w.B, w.HQ, w.N, w.DV), dtype=torch.bfloat16, device=dev)
        self.sink = torch.zeros(1, dtype=torch.int32, device=dev)        # the cold flush's read probe
        torch.cuda.synchronize()
        log(f"[bench] setup {time.time() - t_setup:.0f} s")

    def config(self, engine, partition_tokens=0):
        kvq, w = self.kvq, self.w
        shp = kvq.make_shape(self.pool, w.B, w.HQ, w.N, w.max_blocks, w.max_len, partition_tokens, False, engine)
        wsp = self.torch.empty(kvq.paged_decode_workspace_bytes(self.pool, shp), dtype=self.torch.uint8,
                               device=self.dev)
        return shp, wsp

    def step(self, shp, wsp, mid=None):
        """one decode step: paged_decode_step_partial (append of the new rows with slots from the
        block table, q copy, partial kernel), then paged_decode_merge"""
        kvq = self.kvq
        kvq.paged_decode_step_partial(self.q, self.kn, self.vn, self.pool, self.table, self.lengths,
                                      self.w.scale, shp, wsp)
        if mid is not None:
            mid.record()
        kvq.paged_decode_merge(self.pool, self.lengths, shp, wsp, self.out)

    def timed(self, nsteps, shp, wsp, flush_buf=None):
        """Warm: nsteps back-to-back steps between two events give the step time; then nsteps
        with an event after the partial pass and after each merge split it (the previous step's
        end opens the next step) and give the per-step distribution; then nsteps under the
        library's launch timing, which brackets each kernel with events on its own stream, give
        the kernels' durations.  Event records between kernels delay the next launch by a few
        microseconds, so each pass gives only its own figure.  Cold: a read of 1 GiB (the
        library's streaming-read probe: it evicts the pool from the L2s and the 256 MB Infinity
        Cache and, unlike a write, leaves no dirty lines to be written back inside the step), an
        event, the step, an event, per step.  Returns a dict: ms per step, per-step / partial-pass /
        merge ms lists, wall s (second pass), and the mean ms of the prep, partial and merge
        kernels."""
        torch, kvq = self.torch, self.kvq
        E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
        ms_plain = None
        if flush_buf is None:
            a0, a1 = E(), E()
            torch.cuda.synchronize()
            a0.record()
            for _ in range(nsteps):
                self.step(shp, wsp)
            a1.record()
            torch.cuda.synchronize()
            ms_plain = a0.elapsed_time(a1) / nsteps
        ev0 = E()
        mids = [E() for _ in range(nsteps)]
        ends = [E() for _ in range(nsteps)]
        starts = [E() for _ in range(nsteps)] if flush_buf is not None else None
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record()
        for i in range(nsteps):
            if flush_buf is not None:
                kvq.kvq_probe_read(flush_buf, self.sink)
                starts[i].record()
            self.step(shp, wsp, mids[i])
            ends[i].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kvq.kvq_timing_enable(True)
        for _ in range(nsteps):
            if flush_buf is not None:
                kvq.kvq_probe_read(flush_buf, self.sink)
            self.step(shp, wsp)
        torch.cuda.synchronize()
        kern = {k: kvq.kvq_timing_read(v)[0] for k, v in
                (("prep", kvq.TIMING_PREP), ("partial", kvq.TIMING_PARTIAL), ("merge", kvq.TIMING_MERGE))}
        kvq.kvq_timing_enable(False)
        opens = starts if starts is not None else [ev0] + ends[:-1]
        par = [o.elapsed_time(m) for o, m in zip(opens, mids)]
        mer = [m.elapsed_time(e) for m, e in zip(mids, ends)]
        tot = [o.elapsed_time(e) for o, e in zip(opens, ends)]
        ms = float(np.mean(tot)) if flush_buf is not None else ms_plain
        return {"ms": ms, "tot": tot, "par": par, "mer": mer, "wall": wall, "kern": kern}

    def measure(self, engine, steps, warmup, partition_tokens=0, cold=True, flush=None, label=""):
        """Warm (and, if asked, cold) timing of one engine / partition choice; returns a record."""
        torch, w = self.torch, self.w
        shp, wsp = self.config(engine, partition_tokens)
        pt = self.kvq.paged_decode_partition_tokens(self.pool, shp)
        # the GPU idles at a low clock and takes some tens of ms of load to reach its working clock
        # (c3: 197 us/step timed after 10 warm-up steps, 180 after 300, 178 after 1000, the kernels
        # themselves unchanged); so before the W warm-up steps, steps run for at least SETTLE_S
        settle = 0
        t0 = time.time()
        while time.time() - t0 < SETTLE_S:
            for _ in range(8):
                self.step(shp, wsp)
            torch.cuda.synchronize()
            settle += 8
        for _ in range(warmup):
            self.step(shp, wsp)
        torch.cuda.synchronize()
        t = self.timed(steps, shp, wsp)
        eff = w.effective_bytes()
        rec = {"us_per_step": round(t["ms"] * 1e3, 2), "value": round(eff / (t["ms"] * 1e-3) / 1e9, 1),
               "pct_hbm_peak": round(100 * eff / (t["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
               "step_us_events": _quantiles_us(t["tot"]),
               "partial_pass_us": round(float(np.mean(t["par"])) * 1e3, 2),
               "merge_us_events": round(float(np.mean(t["mer"])) * 1e3, 2),
               "kernels_us": {k: round(v * 1e3, 2) for k, v in t["kern"].items()},
               "partition_tokens": pt,
               "engine_used": "matrix" if self.kvq.paged_decode_engine(self.pool, shp) == self.kvq.ENGINE_MATRIX
                              else "vector",
               "settle_steps": settle, "_t": t}
        log(f"[bench] {label or w.name}: {t['ms'] * 1e3:.1f} us/step (events: median "
            f"{rec['step_us_events']['median']}, p10 {rec['step_us_events']['p10']}, p90 "
            f"{rec['step_us_events']['p90']}); kernels (library events): prep {t['kern']['prep'] * 1e3:.1f}, "
            f"partial {t['kern']['partial'] * 1e3:.1f}, merge {t['kern']['merge'] * 1e3:.1f} us")
        if cold and flush is not None:
            tc = self.timed(steps, shp, wsp, flush)
            rec["cold"] = {"us_per_step": round(tc["ms"] * 1e3, 2),
                           "GB_per_s": round(eff / (tc["ms"] * 1e-3) / 1e9, 1),
                           "step_us": _quantiles_us(tc["tot"]),
                           "partial_pass_us": round(float(np.mean(tc["par"])) * 1e3, 2),
                           "partial_kernel_us": round(tc["kern"]["partial"] * 1e3, 2),
                           "merge_us": round(float(np.mean(tc["mer"])) * 1e3, 2),
                           "note": "1 GiB read before each step (more than the 256 MB Infinity Cache and the "
                                   "L2s; a read leaves no dirty lines to drain inside the step); step = event "
                                   "after the read to event after the merge"}
            log(f"[bench] {label or w.name} cold: {tc['ms'] * 1e3:.1f} us/step")
        return rec

    def close(self):
        self.pool.close()


def roofline(w, part_ms, engine_name, src_hash):
    """The partial kernel's position against its binding roof: HBM (effective bytes / 8 TB/s) or,
    for the vector engine, the vector ALU (2 * REP * N * (D + DV) flop per cached token and KV
    head / the fp32 vector peak), whichever floor is higher."""
    eff = w.effective_bytes()
    part_s = part_ms * 1e-3
    flops = w.attention_flops()
    hbm_floor = eff / (HBM_PEAK_GBS * 1e9)
    alu_floor = flops / (VALU_PEAK_TFLOPS * 1e12)
    hbm = {"achieved": round(eff / part_s / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(eff / part_s / 1e9 / HBM_PEAK_GBS, 4), "floor_us": round(hbm_floor * 1e6, 2)}
    alu = {"achieved": round(flops / part_s / 1e12, 2), "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
           "frac": round(flops / part_s / 1e12 / VALU_PEAK_TFLOPS, 4), "floor_us": round(alu_floor * 1e6, 2)}
    top = alu if (alu_floor > hbm_floor and engine_name != "matrix") else hbm
    return {"bound": "alu" if top is alu else "hbm", "achieved": top["achieved"], "peak": top["peak"],
            "unit": top["unit"], "frac": top["frac"],
            "traffic": traffic_from_profiles(w.name, src_hash) if src_hash else None,
            "kernel": "partial kernel (library launch events on its stream, mean over the timed steps)",
            "kernel_us": round(part_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": eff, "algorithmic_flops_per_launch": flops,
            "hbm": hbm, "alu": alu, "kernel_source_hash": src_hash}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c3")
    ap.add_argument("--bits", type=int, default=0, help="page format override: 16 (bf16) or 2..8 (affine)")
    ap.add_argument("--group", type=int, default=0, help="scale-group override (32, 64 or 128 head dims)")
    ap.add_argument("--rows", type=int, default=0, help="query rows per sequence override (N)")
    ap.add_argument("--dv", type=int, default=0, help="V head dim override (DV; default the K head dim)")
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--engine", choices=["auto", "vector", "matrix"], default="auto",
                    help="partial-pass engine: vector ALU (the default) or matrix cores (4-bit pages)")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold steps (1 GiB read before each)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the matrix-engine and 32k-context lines beside the headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--probe-copy", type=int, default=0, metavar="BYTES",
                    help="instead: time a plain device copy of BYTES (achievable-bandwidth probe, and the "
                         "known-size kernel that calibrates the HBM byte counters)")
    ap.add_argument("--probe-read", type=int, default=0, metavar="BYTES",
                    help="instead: time a streaming read of BYTES (achievable read bandwidth)")
    ap.add_argument("--probe-pool", action="store_true",
                    help="instead: time the pool-read probe over the workload's filled pool (both load patterns)")
    ap.add_argument("--probe-sweep", action="store_true",
                    help="with --probe-read: every launch shape of the probe (loads in flight, non-temporal, workgroups per CU)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import decode_attention_paged_split_amd as kvq
    from workloads import make_workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.probe_read:
        # achievable streaming-read rate: the library's read probe over BYTES (every byte read once),
        # at the default launch shape or (--probe-sweep) over loads in flight, non-temporal loads
        # and workgroups per compute unit; one JSON line per shape
        buf = torch.ones(args.probe_read // 4, dtype=torch.float32, device=dev)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        shapes = [(4, False, 32)]
        if args.probe_sweep:
            shapes = [(u, nt, bpc) for nt in (False, True) for u in (1, 2, 4, 8, 16) for bpc in (4, 8, 16, 32)]
        for u, nt, bpc in shapes:
            for _ in range(3):
                kvq.kvq_probe_read_ex(buf, sink, u, nt, bpc)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(args.steps):
                kvq.kvq_probe_read_ex(buf, sink, u, nt, bpc)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            print(json.dumps({"probe": "read (kvq_probe_read_ex)", "loads_in_flight": u, "nontemporal": nt,
                              "blocks_per_cu": bpc, "bytes_read": buf.numel() * 4,
                              "us_per_read": round(ms * 1e3, 2),
                              "GB_per_s": round(buf.numel() * 4 / (ms * 1e-3) / 1e9, 1)}), flush=True)
        return

    if args.probe_copy:
        src = torch.ones(args.probe_copy // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        moved = 2 * src.numel() * 4
        print(json.dumps({"probe": "copy", "bytes_read": src.numel() * 4, "bytes_written": src.numel() * 4,
                          "us_per_copy": round(ms * 1e3, 2), "GB_per_s": round(moved / (ms * 1e-3) / 1e9, 1)}))
        return

    over = {k: v for k, v in (("bits", args.bits), ("group", args.group), ("N", args.rows), ("DV", args.dv)) if v}
    w = make_workload(args.workload, **over)
    flush = None if args.no_cold else torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    engines = {"auto": kvq.ENGINE_AUTO, "vector": kvq.ENGINE_VECTOR, "matrix": kvq.ENGINE_MATRIX}
    bench = Bench(kvq, torch, w, dev)
    if args.probe_pool:
        # the pool-read probe over this workload's pool: every cached row's K/V codes and scales
        # read through the block table, no arithmetic; one token per lane and coalesced
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        eff = w.effective_bytes()
        for coalesced in (False, True):
            for _ in range(3):
                kvq.kvq_probe_pool_read(bench.pool, bench.table, bench.lengths, w.max_len, coalesced, sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(args.steps):
                kvq.kvq_probe_pool_read(bench.pool, bench.table, bench.lengths, w.max_len, coalesced, sink)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            print(json.dumps({"probe": "pool read (kvq_probe_pool_read)", "workload": w.name,
                              "pattern": "coalesced" if coalesced else "token per lane", "bytes_read": eff,
                              "us_per_read": round(ms * 1e3, 2), "GB_per_s": round(eff / (ms * 1e-3) / 1e9, 1)}),
                  flush=True)
        bench.close()
        return
    head = bench.measure(engines[args.engine], args.steps, args.warmup, args.partition_tokens,
                         flush=flush, label=f"{w.name} ({args.engine} engine)")
    t = head.pop("_t")
    eff = w.effective_bytes()
    src_hash = kernel_source_hash() if head["engine_used"] == "vector" else None
    roof = roofline(w, t["kern"]["partial"], head["engine_used"], src_hash)

    def matrix_ok(wl):
        return wl.bits == 4 and wl.group == 64 and wl.D in (128, 256) and wl.DV == wl.D

    variants = {}
    if not args.no_variants and args.engine == "auto" and args.partition_tokens <= 0 and matrix_ok(w):
        # the separately flagged matrix-core engine on the same inputs, timed the same way
        rm = bench.measure(kvq.ENGINE_MATRIX, args.steps, 3, cold=False, label=f"{w.name} (matrix engine)")
        km = rm.pop("_t")["kern"]["partial"]
        rm["roofline"] = roofline(w, km, "matrix", None)
        rm["note"] = "engine=2: MFMA q.k and P.V, 4-bit pages; not the default path"
        variants["matrix_engine"] = rm
    bench.close()

    if not args.no_variants and args.workload == "c3" and not over and args.engine == "auto":
        # the 32k-context shape: GQA 8/2, head dim 256, 4-bit pages, 32 x 32768 tokens
        wd = make_workload("diag")
        bd = Bench(kvq, torch, wd, dev)
        rd = bd.measure(kvq.ENGINE_AUTO, args.steps, args.warmup, flush=flush, label="diag (vector engine)")
        kd = rd.pop("_t")["kern"]["partial"]
        rd["roofline"] = roofline(wd, kd, rd["engine_used"],
                                  kernel_source_hash() if rd["engine_used"] == "vector" else None)
        rd["config"] = {"workload": f"diag: 4-bit affine g64 paged KV, B={wd.B} x {wd.max_len} tokens, BS={wd.BS}, "
                                    f"HQ={wd.HQ}, HK={wd.HK}, D={wd.D}, N={wd.N}"}
        rd["effective_bytes"] = wd.effective_bytes()
        variants["diag"] = rd
        if matrix_ok(wd):
            rdm = bd.measure(kvq.ENGINE_MATRIX, args.steps, 3, cold=False, label="diag (matrix engine)")
            kdm = rdm.pop("_t")["kern"]["partial"]
            rdm["roofline"] = roofline(wd, kdm, "matrix", None)
            rdm["note"] = "engine=2: MFMA q.k and P.V, 4-bit pages; not the default path"
            variants["diag_matrix_engine"] = rdm
        bd.close()

    rec = {
        "metric": METRIC, "value": head["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t["ms"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": (f"{w.name}: 4-bit affine g64 paged KV, B={w.B}, lengths U[4096,32768] "
                                f"(sum {int(w.lengths.sum())}), BS={w.BS}, HQ={w.HQ}, HK={w.HK}, D={w.D}, "
                                f"N={w.N}") if (w.name == "c3" and not over) else
                               (w.name + "".join(f" {k}={v}" for k, v in over.items())),
                   "global_batch": w.B, "seq_len": w.max_len, "parallelism": "single GPU",
                   "partition_tokens": head["partition_tokens"], "engine": args.engine,
                   "engine_used": head["engine_used"]},
        "us_per_step": head["us_per_step"], "pct_hbm_peak": head["pct_hbm_peak"],
        "step_us_events": head["step_us_events"], "effective_bytes": eff,
        "kernels_us": head["kernels_us"], "partial_pass_us": head["partial_pass_us"],
        "merge_us_events": head["merge_us_events"],
        "settle": {"seconds_min": SETTLE_S, "steps": head["settle_steps"],
                   "note": "untimed steps before the W warm-up steps, until the GPU clock has left its idle level"},
        "roofline": roof,
    }
    if "cold" in head:
        rec["cold"] = head["cold"]
    if variants:
        rec["variants"] = variants
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample ...")
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        log(f"[bench] oracle {rec['cpu_baseline']['value']:.3f} GB/s on {rec['cpu_baseline']['sample']}")
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
