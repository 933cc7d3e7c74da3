#!/usr/bin/env python3
"""Benchmark of the paged prefix-reuse attention hot path on one MI355X.

One step = one pass of the whole path over one batch, on the largest single-GPU workload
(the ragged multi-turn/RAG mix at head dim 96, fp16: 32 sequences, prefixes U{0..16384},
chunks U{1..512} not multiples of 16, 32 query / 8 KV heads, about half the prefix blocks
shared between random pairs of sequences, pool of 32768 16-token blocks):
  kvb_paged_prefill_write (the chunks over their cached prefixes + causal self part, with
  the chunks' K/V scattered into their pool slots in the same launch) -> kvb_write_kv (one
  decode token per sequence) -> kvb_paged_decode (one query per sequence over its whole
  context), captured once in a HIP graph and replayed.

Prints ONE JSON line.  `value` is algorithmic TFLOP/s of the whole step (prefill plus decode
attention FLOPs over the step time) with every input resident in HBM.  `roofline` is the
step's dominant kernel, the prefill, timed per launch between 1 GiB read flushes of L2 and
the Infinity Cache (mean, median and minimum; back-to-back warm launches as a secondary
figure), against the published and the measured (probe) MFMA peaks.  The same run times the
prefill of the other workloads (shared system prompt, long prefix, ragged mix at head dim
64), the paged-decode workload (64 sequences, contexts 512..4096, first 1024 tokens shared)
and the fp64 oracle on the host cores.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config ragged_d96]
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

METRIC = "paged-prefill TFLOP/s & decode KV GB/s on 1 MI355X, % of MFMA/HBM peak"
PEAK_TFLOPS = 2500.0     # MI355X dense bf16/fp16 MFMA, published
PEAK_GBPS = 8000.0       # MI355X HBM3E, published
ESZ = 2


# ----------------------------------------------------------------- algorithmic counts

def prefill_flops(w) -> float:
    """4*d per visible (query row, key, q-head) pair: QK^T and PV, 2 flops per MAC."""
    C = w.q_lens.astype(np.float64)
    P = w.prefix_lens.astype(np.float64)
    pairs = w.num_q_heads * np.sum(C * P + C * (C + 1) / 2)
    return 4.0 * w.head_dim * pairs


def decode_flops(ctx, w) -> float:
    return 4.0 * w.head_dim * w.num_q_heads * float(np.sum(ctx))


def unique_kv_tokens(tables, lens) -> int:
    """Tokens of distinct physical blocks touched (a shared block counts once)."""
    best = {}
    for b, n in enumerate(lens):
        n = int(n)
        for j in range((n + 15) // 16):
            pb = int(tables[b][j])
            best[pb] = max(best.get(pb, 0), min(16, n - 16 * j))
    return sum(best.values())


def decode_bytes(w, ctx, tables) -> float:
    B = len(ctx)
    kv = unique_kv_tokens(tables, ctx) * w.num_kv_heads * w.head_dim * 2 * ESZ
    qo = 2 * B * w.num_q_heads * w.head_dim * ESZ
    tab = sum((int(n) + 15) // 16 for n in ctx) * 4 + B * 4
    return float(kv + qo + tab)


def decode_bytes_q8(w, ctx, tables, bits: int = 8) -> float:
    """Algorithmic bytes of decode over a quantised pool: bits/8 bytes per K and V element
    plus a float32 V scale per (token, KV head)."""
    B = len(ctx)
    kv = unique_kv_tokens(tables, ctx) * w.num_kv_heads * (2 * w.head_dim * bits // 8 + 4)
    qo = 2 * B * w.num_q_heads * w.head_dim * ESZ
    tab = sum((int(n) + 15) // 16 for n in ctx) * 4 + B * 4
    return float(kv + qo + tab)


def prefill_bytes(w) -> float:
    T = w.total_q
    qo = 2 * T * w.num_q_heads * w.head_dim * ESZ
    kvn = 2 * T * w.num_kv_heads * w.head_dim * ESZ
    kvp = unique_kv_tokens(w.block_tables, w.prefix_lens) * w.num_kv_heads * w.head_dim * 2 * ESZ
    tab = sum((int(p) + 15) // 16 for p in w.prefix_lens) * 4 + (2 * w.batch + 1) * 4
    return float(qo + kvn + kvp + tab)


def write_kv_bytes(T, w) -> float:
    return float(2 * 2 * T * w.num_kv_heads * w.head_dim * ESZ + 8 * T)


# ----------------------------------------------------------------- helpers

def _dev_bits(torch, bits, dtype):
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(tdt)


def _idev(torch, a, dt=None):
    dt = dt or torch.int32
    return torch.as_tensor(np.ascontiguousarray(a)).to(dt).to("cuda:0")


def read_traffic(kernel_key: str):
    """HBM traffic per launch from a committed rocprofv3 counter summary, if it was taken
    on the current kernel source (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel_key}.pmc.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    srcs = fields.get("source_files")
    if not srcs:
        return None
    h = hashlib.sha256()
    for src in srcs.split(","):
        h.update(open(os.path.join(ROOT, src.strip()), "rb").read())
    if h.hexdigest()[:16] != fields.get("source_sha256_16"):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_counters(kernel_key: str):
    """Shader-sequencer counters per launch from a committed rocprofv3 summary
    (profiles/<key>.sq.txt: MFMA utilisation, instruction mix, LDS bank conflicts), if it was
    taken on the current kernel source (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel_key}.sq.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for src in fields.get("source_files", "").split(","):
        h.update(open(os.path.join(ROOT, src.strip()), "rb").read())
    if h.hexdigest()[:16] != fields.get("source_sha256_16"):
        return None
    out = {}
    for k in ("mfma_util_percent", "valu_per_mfma", "lds_per_mfma", "salu_per_mfma",
              "lds_bank_conflicts_per_lds_inst", "l2_hit_rate", "wave_cycles_waiting_frac"):
        try:
            out[k] = float(fields[k])
        except (KeyError, ValueError):
            pass
    return out or None


def cpu_baseline(w, budget_s: float = 12.0):
    """The fp64 oracle, as it stands, on a bounded sample of the same prefill workload:
    whole (sequence, query head) problems in order, repeating the workload until about
    `budget_s` seconds of host time have been spent."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    done_flops = 0.0
    pairs = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        for b in range(w.batch):
            C = int(w.q_lens[b])
            P = int(w.prefix_lens[b])
            for h in range(w.num_q_heads):
                oracle.paged_prefill(w.k_pool, w.v_pool, w.q, w.k_new, w.v_new, w.cu_q_lens,
                                     w.prefix_lens, w.block_tables, w.num_q_heads, w.scale, w.dtype,
                                     select=[(b, h, np.arange(C))])
                done_flops += 4.0 * w.head_dim * (C * P + C * (C + 1) / 2)
                pairs += 1
                if time.perf_counter() - t0 > budget_s:
                    break
            if time.perf_counter() - t0 > budget_s:
                break
    dt = time.perf_counter() - t0
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    return {"value": done_flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "cpu_model": model,
            "kind": "oracle",
            "sample": f"{pairs} (sequence, query head) problems of the same prefill workload "
                      f"({w.batch * w.num_q_heads} per pass), fp64 NumPy, {dt:.1f} s",
            "host_cpus": os.cpu_count()}


# ----------------------------------------------------------------- rocprofv3 summaries

def summarize_rocprof(path: str, kernel: str) -> str:
    """Text summary of rocprofv3 CSV output under `path` for kernels whose name contains
    `kernel`: average duration from a kernel trace (all launches, and the launches that run
    cold, i.e. whose call starts right after the benchmark's 1 GiB read flush), and
    per-dispatch averages of counters."""
    import csv
    import glob
    lines = []
    for f in sorted(glob.glob(os.path.join(path, "**", "*_kernel_stats.csv"), recursive=True)):
        for r in csv.DictReader(open(f)):
            if kernel in r["Name"]:
                lines.append(f"kernel: {r['Name'][:120]}")
                lines.append(f"calls: {r['Calls']}")
                lines.append(f"avg_ns: {float(r['AverageNs']):.1f}")
                lines.append(f"min_ns: {float(r['MinNs']):.1f}")
                lines.append(f"max_ns: {float(r['MaxNs']):.1f}")
    for f in sorted(glob.glob(os.path.join(path, "**", "*_kernel_trace.csv"), recursive=True)):
        rows = sorted(csv.DictReader(open(f)), key=lambda r: int(r["Start_Timestamp"]))
        names = sorted({r["Kernel_Name"] for r in rows if kernel in r["Kernel_Name"]})
        for nm in names:
            cold, call = [], []
            for i, r in enumerate(rows):
                if r["Kernel_Name"] != nm:
                    continue
                # the call's first dispatch: this kernel, or the plan kernel right before it
                j = i - 1
                first = i
                if j >= 0 and "plan_kernel" in rows[j]["Kernel_Name"]:
                    first, j = j, j - 1
                if j >= 0 and "read_kernel" in rows[j]["Kernel_Name"]:
                    cold.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                    call.append(int(r["End_Timestamp"]) - int(rows[first]["Start_Timestamp"]))
            if cold:
                lines.append(f"cold_kernel: {nm[:120]}")
                lines.append(f"cold_launches: {len(cold)}")
                lines.append(f"cold_avg_ns: {np.mean(cold):.1f}")
                lines.append(f"cold_median_ns: {np.median(cold):.1f}")
                lines.append(f"cold_min_ns: {np.min(cold):.1f}")
                lines.append(f"cold_call_avg_ns: {np.mean(call):.1f}")
    for f in sorted(glob.glob(os.path.join(path, "**", "*_counter_collection.csv"), recursive=True)):
        per = {}
        for r in csv.DictReader(open(f)):
            if kernel not in r["Kernel_Name"]:
                continue
            d = per.setdefault(r["Dispatch_Id"], {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        if per:
            names = sorted({k for d in per.values() for k in d})
            lines.append(f"dispatches: {len(per)}")
            for n in names:
                vals = [d.get(n, 0.0) for d in per.values()]
                lines.append(f"{n}_per_dispatch: {sum(vals) / len(vals):.6g}")
    return "\n".join(lines)


# ----------------------------------------------------------------- main

CONFIG_NAMES = {
    "ragged_d96": "ragged multi-turn/RAG mix, head dim 96 fp16 (32 seqs, prefixes U{0..16384}, "
                  "chunks U{1..512}, 32/8 heads): paged prefill with slot scatter + decode step",
    "ragged_d64": "ragged multi-turn/RAG mix, head dim 64 bf16 (32 seqs, prefixes U{0..16384}, "
                  "chunks U{1..512}, 32/8 heads): paged prefill with slot scatter + decode step",
    "long_prefix": "long-prefix prefill, 4 x (8192 cached + 1024 new), 40/8 heads, d128 fp16: "
                   "paged prefill with slot scatter + decode step",
    "shared_prompt": "shared-system-prompt prefill, 8 x (2048 shared + 256 new), 16/2 heads, d128 "
                     "bf16: paged prefill with slot scatter + decode step",
    "tiny": "tiny paged prefill (32 cached + 16 new, 1 head, d64 fp16) + decode step",
}
FLUSH_BYTES = 1 << 30


def progress(msg: str) -> None:
    """One line per finished stage on stderr (the JSON result is the only stdout line)."""
    print(f"bench: {msg} ({time.strftime('%H:%M:%S')})", file=sys.stderr, flush=True)


class Probe:
    """libkvb_probe.so: HBM read stream / cache flush, the 4 KiB gather read and the pure-MFMA
    rate probe."""

    def __init__(self, torch):
        import ctypes
        path = os.path.join(ROOT, "attention_paged_prefix_amd", "libkvb_probe.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build first (python -m attention_paged_prefix_amd.build)")
        lib = ctypes.CDLL(path)
        lib.kvb_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_void_p]
        lib.kvb_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p]
        lib.kvb_probe_gather.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_int, ctypes.c_void_p]
        lib.kvb_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
        lib.kvb_probe_mfma_flops.restype = ctypes.c_double
        lib.kvb_probe_clock_khz.argtypes = []
        lib.kvb_probe_clock_khz.restype = ctypes.c_int
        self.lib = lib
        self.torch = torch
        self.buf = torch.ones(FLUSH_BYTES // 2, dtype=torch.int16, device="cuda:0")
        self.sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
        # MFMA operands: N(0,1) values rounded to bf16 (realistic bit toggling)
        g = torch.Generator().manual_seed(0)
        self.ops = torch.randn(16 * 256 * 8, generator=g).to(torch.bfloat16).to("cuda:0")
        self.cus = torch.cuda.get_device_properties(0).multi_processor_count

    def _stream(self):
        return self.torch.cuda.current_stream().cuda_stream

    def flush(self):
        """Read 1 GiB (more than L2 + Infinity Cache) so the next launch starts cold."""
        rc = self.lib.kvb_probe_read(self.buf.data_ptr(), FLUSH_BYTES, self.sink.data_ptr(),
                                     8 * self.cus, self._stream())
        if rc:
            raise RuntimeError(f"kvb_probe_read failed ({rc})")

    def gather(self, buf, idx, n, blocks):
        """Read the n 4-KiB chunks of device tensor `buf` listed in device int32 `idx`."""
        rc = self.lib.kvb_probe_gather(buf.data_ptr(), idx.data_ptr(), n, self.sink.data_ptr(), blocks,
                                       self._stream())
        if rc:
            raise RuntimeError(f"kvb_probe_gather failed ({rc})")

    def mfma(self, iters, blocks):
        rc = self.lib.kvb_probe_mfma(iters, blocks, self.ops.data_ptr(), self.sink.data_ptr(),
                                     self._stream())
        if rc:
            raise RuntimeError(f"kvb_probe_mfma failed ({rc})")

    def peaks(self, settle_ms):
        """Measured ceilings: dense bf16 MFMA rate (independent 32x32x16 chains, two waves per
        SIMD, ~1 ms per launch, after the clocks settle under that load) and the HBM read
        stream (1 GiB per launch, 16-byte loads)."""
        torch = self.torch
        iters, blocks = 8192, 2 * self.cus
        settle(torch, lambda: self.mfma(iters, blocks), settle_ms)
        ms = time_each(torch, lambda: self.mfma(iters, blocks), 10)
        fl = self.lib.kvb_probe_mfma_flops(iters, blocks)
        # HBM read stream: 4 GiB per launch, 32 work-groups per CU (launch ramp amortised)
        big = torch.ones(2 * FLUSH_BYTES, dtype=torch.int16, device="cuda:0")
        rd = lambda: self.lib.kvb_probe_read(big.data_ptr(), 4 * FLUSH_BYTES, self.sink.data_ptr(),  # noqa: E731
                                             32 * self.cus, self._stream())
        settle(torch, rd, min(settle_ms, 100))
        rms = time_each(torch, rd, 10)
        del big
        tflops = fl / (np.median(ms) * 1e-3) / 1e12
        khz = int(self.lib.kvb_probe_clock_khz())
        return {"mfma_bf16_tflops": tflops,
                "mfma_probe": f"{blocks} work-groups x 4 waves x {iters} x 4 independent "
                              f"v_mfma_f32_32x32x16_bf16 on random N(0,1) bf16 operands, median "
                              f"of 10 launches of {np.median(ms):.3f} ms",
                "hbm_read_gbps": 4 * FLUSH_BYTES / (np.median(rms) * 1e-3) / 1e9,
                "hbm_probe": f"4 GiB read with 16-byte loads (32 work-groups per CU), median of "
                             f"10 launches of {np.median(rms):.3f} ms",
                "compute_units": self.cus,
                # the driver's peak engine clock, and the clock at which the probe's MFMA rate
                # would be the full dense rate (4096 bf16 flop per clock per CU)
                "clock_mhz_peak": khz / 1000.0 if khz > 0 else None,
                "nominal_mfma_tflops_at_peak_clock": self.cus * 4096 * khz * 1e3 / 1e12 if khz > 0 else None,
                "mfma_probe_effective_clock_mhz": tflops * 1e12 / (self.cus * 4096) / 1e6}


def time_each(torch, fn, n: int, before=None):
    """Per-launch ms of `fn`, each bracketed by its own HIP events on the current stream
    (the stream the library launches on); `before` runs outside the events first."""
    evs = []
    for _ in range(n):
        if before is not None:
            before()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def stats(ms_list):
    a = np.asarray(ms_list, dtype=np.float64)
    return {"mean": float(a.mean()), "median": float(np.median(a)), "min": float(a.min()),
            "max": float(a.max()), "n": int(a.size)}


class Uploaded:
    """One prefill workload (plus its decode step when generated with one) on the GPU."""

    def __init__(self, torch, kvb, w):
        dt = w.dtype
        self.w = w
        self.k = _dev_bits(torch, w.k_pool, dt)
        self.v = _dev_bits(torch, w.v_pool, dt)
        self.pool = kvb.Pool.from_tensors(self.k, self.v)
        self.q = _dev_bits(torch, w.q, dt)
        self.kn = _dev_bits(torch, w.k_new, dt)
        self.vn = _dev_bits(torch, w.v_new, dt)
        self.cu = _idev(torch, w.cu_q_lens)
        self.pl = _idev(torch, w.prefix_lens)
        self.bt = _idev(torch, w.block_tables)
        self.slots = _idev(torch, w.slot_mapping, torch.int64)
        self.out = torch.empty_like(self.q)
        self.max_q, self.max_p = int(w.q_lens.max()), int(w.prefix_lens.max())
        n = kvb.paged_prefill_workspace_size(w.batch, w.num_q_heads, w.head_dim, w.total_q, self.max_p)
        self.pws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda:0")
        self.kvb = kvb
        if w.dec_q is not None:
            self.dq = _dev_bits(torch, w.dec_q, dt)
            self.dk = _dev_bits(torch, w.dec_k, dt)
            self.dv = _dev_bits(torch, w.dec_v, dt)
            self.dslots = _idev(torch, w.dec_slots, torch.int64)
            self.dctx = _idev(torch, w.dec_context_lens)
            self.dout = torch.empty_like(self.dq)
            self.max_ctx = int(w.dec_context_lens.max())
            n = kvb.paged_decode_workspace_size(w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim,
                                                self.max_ctx)
            self.dws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda:0")

    def part(self, name):
        kvb, w = self.kvb, self.w
        if name == "write_kv":
            kvb.write_kv(self.pool, self.kn, self.vn, self.slots)
        elif name == "prefill":
            kvb.paged_prefill(self.pool, self.q, self.kn, self.vn, self.cu, self.pl, self.bt, w.scale,
                              self.max_q, self.max_p, out=self.out, workspace=self.pws)
        elif name == "prefill_write":
            kvb.paged_prefill(self.pool, self.q, self.kn, self.vn, self.cu, self.pl, self.bt, w.scale,
                              self.max_q, self.max_p, out=self.out, workspace=self.pws,
                              slot_mapping=self.slots)
        elif name == "write_kv_dec":
            kvb.write_kv(self.pool, self.dk, self.dv, self.dslots)
        elif name == "decode":
            kvb.paged_decode(self.pool, self.dq, self.dctx, self.bt, w.scale, self.max_ctx,
                             out=self.dout, workspace=self.dws)
        else:
            raise KeyError(name)


def time_prefill(torch, up, probe, name, steps, settle_ms):
    """One prefill call timed per launch: cold (after a 1 GiB read flush, outside the events)
    and warm (launched back to back).  The call includes its dispatch-plan kernel."""
    fn = lambda: up.part(name)                     # noqa: E731
    settle(torch, fn, settle_ms)
    cold = time_each(torch, fn, steps, before=probe.flush)
    warm = time_launches(torch, fn, steps)
    return stats(cold), warm


def prefill_entry(w, cold, warm_ms, peaks):
    pf = prefill_flops(w)
    t = cold["mean"] * 1e-3
    ach = pf / t / 1e12
    return {"algorithmic_flops": pf, "algorithmic_bytes": prefill_bytes(w),
            "ms_cold": cold, "ms_warm_back_to_back": warm_ms,
            "tflops_cold_mean": ach, "tflops_cold_median": pf / (cold["median"] * 1e-3) / 1e12,
            "tflops_cold_best": pf / (cold["min"] * 1e-3) / 1e12,
            "tflops_warm": pf / (warm_ms * 1e-3) / 1e12,
            "frac_mfma_peak": ach / PEAK_TFLOPS,
            "frac_measured_mfma_peak": ach / peaks["mfma_bf16_tflops"] if peaks else None,
            "gbps_cold": prefill_bytes(w) / t / 1e9}


def main(argv=None):
    argv = sys.argv[1:] if argv is None else argv
    if argv and argv[0] == "--summarize-rocprof":
        # python bench.py --summarize-rocprof DIR KERNEL_SUBSTRING
        print(summarize_rocprof(argv[1], argv[2]))
        return 0
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-graph", action="store_true",
                    help="time the step from eager launches instead of a captured HIP graph")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed back-to-back runs before timing so clocks reach steady state")
    ap.add_argument("--config", default="ragged_d96", choices=sorted(CONFIG_NAMES))
    ap.add_argument("--other-configs", default="shared_prompt,long_prefix,ragged_d64,tiny",
                    help="comma-separated workloads whose prefill is also timed ('' = none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--split-blocks", type=int, default=0, help="decode split size (0 = auto)")
    ap.add_argument("--no-decode", action="store_true", help="skip the separate decode workload")
    ap.add_argument("--no-q8", action="store_true", help="skip the 8-bit pool prefill")
    ap.add_argument("--separate-write", action="store_true",
                    help="step with kvb_write_kv of the chunk before kvb_paged_prefill instead of "
                         "kvb_paged_prefill_write (prefill and slot scatter in one launch)")
    ap.add_argument("--only", choices=["step", "prefill", "prefill_write", "prefill_q8", "prefill_q4",
                                       "decode_workload", "copy", "copy_blocks", "peaks"],
                    default="step", help="profiling aid: run only one part")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path shards by sequence and KV head but no multi-GPU run is provided.",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    import attention_paged_prefix_amd as kvb
    from workloads import make_config

    if args.only == "copy":
        # calibration kernel for the HBM counters: a plain 1 GiB device copy
        a = torch.empty(1 << 29, dtype=torch.int16, device="cuda:0").fill_(1)
        bb = torch.empty_like(a)
        for _ in range(args.steps):
            bb.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": a.numel() * 2, "copy_bytes_written": a.numel() * 2}))
        return 0
    probe = Probe(torch)
    if args.only == "peaks":
        print(json.dumps(probe.peaks(args.settle_ms)))
        return 0
    if args.only == "decode_workload":
        print(json.dumps(bench_decode(torch, kvb, args, probe)))
        return 0
    if args.only == "copy_blocks":
        print(json.dumps(bench_copy_blocks(torch, kvb, args)))
        return 0

    w = make_config(args.config, with_decode=True)
    up = Uploaded(torch, kvb, w)
    if args.only in ("prefill_q8", "prefill_q4"):
        # profiling aid: the quantised-pool prefill against the 16-bit one, both cold
        cold, _ = time_prefill(torch, up, probe, "prefill", args.steps, args.settle_ms)
        r = bench_prefill_q8(torch, kvb, up, probe, cold["mean"], args, 8 if args.only == "prefill_q8" else 4)
        print(json.dumps({"config": args.config, "part": args.only, **r}))
        return 0
    if args.only in ("prefill", "prefill_write"):
        # profiling aid: the prefill call alone, settled, then launched after flushes
        cold, warm = time_prefill(torch, up, probe, args.only, args.steps, args.settle_ms)
        print(json.dumps({"config": args.config, "part": args.only,
                          **prefill_entry(w, cold, warm, None)}))
        return 0

    peaks = probe.peaks(args.settle_ms)
    progress(f"peaks measured: {peaks['mfma_bf16_tflops']:.0f} TFLOP/s MFMA, "
             f"{peaks['hbm_read_gbps']:.0f} GB/s HBM read")
    parts = (["write_kv", "prefill", "write_kv_dec", "decode"] if args.separate_write
             else ["prefill_write", "write_kv_dec", "decode"])

    def one_step():
        for p_ in parts:
            up.part(p_)

    settle(torch, one_step, args.settle_ms)
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for s in range(args.steps):
        ev[s][0].record()
        for i, p_ in enumerate(parts):
            up.part(p_)
            ev[s][i + 1].record()
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    per_part = {p_: float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)]))
                for i, p_ in enumerate(parts)}
    ms_step_eager = total_ms / args.steps

    # The whole step as one HIP graph, the way a serving loop runs it: one launch per step
    # instead of one per call, so the step time is the kernels' time rather than host gaps.
    ms_step, launch = ms_step_eager, "eager"
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            one_step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_step()
        # the capture leaves the GPU idle: bring the clocks back up before timing
        settle(torch, graph.replay, args.settle_ms)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.steps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        ms_step, launch = g0.elapsed_time(g1) / args.steps, "hip graph"

    progress(f"step timed: {ms_step:.4f} ms per step ({launch})")
    # The dominant kernel alone: the step's prefill call per launch, cold and warm.
    pname = "prefill" if args.separate_write else "prefill_write"
    cold, warm = time_prefill(torch, up, probe, pname, max(args.steps, 20), min(args.settle_ms, 200.0))
    pe = prefill_entry(w, cold, warm, peaks)
    pe["ms_in_eager_step"] = per_part[pname]
    progress(f"{args.config} prefill timed: {pe['tflops_cold_mean']:.0f} TFLOP/s cold")
    kernels = {"paged_" + pname: pe}
    dt_ = time_launches(torch, lambda: up.part("decode"), max(args.steps, 10)) * 1e-3
    db = decode_bytes(w, w.dec_context_lens, w.block_tables)
    kernels["paged_decode"] = {"ms": dt_ * 1e3, "ms_in_eager_step": per_part["decode"],
                               "gbps": db / dt_ / 1e9, "frac_hbm_peak": db / dt_ / 1e9 / PEAK_GBPS}
    for nm, cnt in (("write_kv", w.total_q), ("write_kv_dec", w.batch)):
        ms = time_launches(torch, lambda: up.part(nm), max(args.steps, 10))
        kernels[nm] = {"tokens": cnt, "ms": ms, "gbps": write_kv_bytes(cnt, w) / (ms * 1e-3) / 1e9}

    pf = prefill_flops(w)
    df = decode_flops(w.dec_context_lens, w)
    res = {
        "metric": METRIC,
        "value": (pf + df) / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": ms_step,
        "ms_per_step_eager_launches": ms_step_eager,
        "launch": launch,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": CONFIG_NAMES[args.config], "name": args.config,
                   "batch": w.batch, "prefix_tokens": int(w.prefix_lens.sum()),
                   "chunk_tokens": int(w.q_lens.sum()), "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": 16,
                   "num_blocks": w.num_blocks, "seed": w.seed, "parallelism": "single GPU",
                   "step": " -> ".join(parts)},
        "peaks": {"nominal_mfma_tflops": PEAK_TFLOPS, "nominal_hbm_gbps": PEAK_GBPS, **peaks},
        "kernels": kernels,
    }
    res["roofline"] = {"bound": "mfma", "kernel": "paged_" + pname, "achieved": pe["tflops_cold_mean"],
                       "peak": PEAK_TFLOPS, "unit": "TFLOP/s", "frac": pe["frac_mfma_peak"],
                       "traffic": read_traffic(f"paged_{pname}_{args.config}"),
                       "counters": read_counters(f"paged_{pname}_{args.config}"),
                       "timing": "per-launch HIP events after a 1 GiB read flush; mean of "
                                 f"{cold['n']} launches (dispatch-plan kernel included)",
                       "achieved_median": pe["tflops_cold_median"], "achieved_best": pe["tflops_cold_best"],
                       "achieved_warm_back_to_back": pe["tflops_warm"],
                       "measured_peak": peaks["mfma_bf16_tflops"],
                       "frac_measured_peak": pe["frac_measured_mfma_peak"],
                       "algorithmic_flops_per_launch": pf,
                       "algorithmic_bytes_per_launch": prefill_bytes(w)}
    del up

    others = {}
    for name in [c for c in args.other_configs.split(",") if c and c != args.config]:
        wo = make_config(name)
        uo = Uploaded(torch, kvb, wo)
        c_, w_ = time_prefill(torch, uo, probe, pname, max(args.steps, 20), min(args.settle_ms, 200.0))
        e = prefill_entry(wo, c_, w_, peaks)
        e["traffic"] = read_traffic(f"paged_{pname}_{name}")
        e["counters"] = read_counters(f"paged_{pname}_{name}")
        ms = time_launches(torch, lambda: uo.part("write_kv"), max(args.steps, 10))
        e["write_kv"] = {"tokens": wo.total_q, "ms": ms,
                         "gbps": write_kv_bytes(wo.total_q, wo) / (ms * 1e-3) / 1e9}
        e["workload"] = CONFIG_NAMES[name]
        if name == "tiny":
            e["note"] = "latency-bound correctness case (648 pairs): its time, not a roofline fraction"
        others[name] = e
        progress(f"{name} prefill timed: {e['tflops_cold_mean']:.0f} TFLOP/s cold")
        del uo
        torch.cuda.empty_cache()
    if others:
        res["other_configs"] = others

    if not args.no_decode:
        dw = bench_decode(torch, kvb, args, probe)
        dw["roofline"] = {"bound": "hbm", "kernel": "paged_decode", "achieved": dw["gbps_cold_cache"],
                          "peak": PEAK_GBPS, "unit": "GB/s", "frac": dw["gbps_cold_cache"] / PEAK_GBPS,
                          "measured_peak": peaks["hbm_read_gbps"],
                          "frac_measured_peak": dw["gbps_cold_cache"] / peaks["hbm_read_gbps"],
                          "traffic": read_traffic("paged_decode_decode_workload")}
        res["decode_workload"] = dw
        progress(f"decode workload timed: {dw['gbps_cold_cache']:.0f} GB/s cold")

    if not args.no_q8:
        up = Uploaded(torch, kvb, w)
        res["prefill_q8"] = bench_prefill_q8(torch, kvb, up, probe, pe["ms_cold"]["mean"], args)
        res["prefill_q4"] = bench_prefill_q8(torch, kvb, up, probe, pe["ms_cold"]["mean"], args, 4)
        progress("8-bit and 4-bit pool prefill timed")
        del up

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w)
        res["cpu_baseline"]["gpu_prefill_speedup"] = res["roofline"]["achieved"] / res["cpu_baseline"]["value"]

    print(json.dumps(res))
    return 0


def settle(torch, fn, ms: float) -> None:
    """Run `fn` back to back for about `ms` milliseconds (untimed).  The GPU raises its
    clocks only after some time under load; without this the first timed steps of a short
    run are measured at lower clocks than the steady state the kernels run at when busy."""
    t0 = time.time()
    while (time.time() - t0) * 1e3 < ms:
        for _ in range(16):
            fn()
        torch.cuda.synchronize()


def time_launches(torch, fn, n: int) -> float:
    """Mean ms per launch of `fn` run `n` times back to back.  A spin kernel is queued
    first so that the host has enqueued every launch before the first one starts: the
    events then bracket kernel work only, not the host's launch gaps."""
    fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    if hasattr(torch.cuda, "_sleep"):       # absent: the first launches may wait for the host
        torch.cuda._sleep(20_000_000)
    a.record()
    for _ in range(n):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def _decode_read_pattern(torch, w, k, v, probe, steps):
    """The decode's HBM reads alone: every (block, KV head) K and V slice its block tables
    reach, once each (4 KiB at d = 128 bf16), in the order the decode meets them, read by
    the gather probe after a cache flush.  No compute, no re-reads: the rate this access
    pattern reaches, the practical ceiling of the decode's memory stream."""
    H = w.num_kv_heads
    assert 16 * w.head_dim * ESZ == 4096, "gather chunks are 4 KiB"
    kc = []
    for kvh in range(H):
        seen = set()
        for b in range(w.batch):
            for j in range((int(w.context_lens[b]) + 15) // 16):
                pb = int(w.block_tables[b][j])
                if pb not in seen:
                    seen.add(pb)
                    kc.append(pb * H + kvh)
    idx = torch.as_tensor(np.asarray(kc, dtype=np.int32)).to("cuda:0")
    n = len(kc)
    blocks = 8 * probe.cus

    def run():
        probe.gather(k, idx, n, blocks)
        probe.gather(v, idx, n, blocks)

    for _ in range(3):
        run()
    s = stats(time_each(torch, run, steps, before=probe.flush))
    nbytes = 2.0 * n * 4096
    return {"what": "gather probe over the decode's unique (block, KV head) K and V slices, "
                    "4 KiB each, cold cache, no compute",
            "bytes": nbytes, "ms_cold": s["median"], "gbps_cold": nbytes / (s["median"] * 1e-3) / 1e9}


def _time_warm_cold(torch, run, steps, probe):
    """Per-launch ms of `run` launched back to back (warm caches) and after a 1 GiB read
    that evicts L2 and the Infinity Cache (cold); events bracket the launch only."""
    warm = time_each(torch, run, steps)
    cold = time_each(torch, run, steps, before=probe.flush)
    return stats(warm), stats(cold)


def bench_copy_blocks(torch, kvb, args):
    """Block copies (kvb_copy_blocks) of 1024 random blocks of a 16384-block pool, 8 KV
    heads, d=128, bf16 (64 KiB per block, K and V): inside the device pool (copy-on-write)
    and between the device pool and a pool in pinned host memory (swap out / in)."""
    nb, n, hkv, d = 16384, 1024, 8, 128
    k = torch.empty((nb, hkv, 16, d), dtype=torch.bfloat16, device="cuda:0").normal_()
    v = torch.empty_like(k).normal_()
    dev = kvb.Pool.from_tensors(k, v)
    hk = torch.empty((n, hkv, 16, d), dtype=torch.bfloat16).pin_memory()
    hv = torch.empty_like(hk).pin_memory()
    host = kvb.Pool.from_tensors(hk, hv)
    rng = np.random.default_rng(0)
    perm = rng.permutation(nb)
    src = torch.as_tensor(perm[:n].astype(np.int32)).to("cuda:0")
    dst = torch.as_tensor(perm[n:2 * n].astype(np.int32)).to("cuda:0")
    seq = torch.arange(n, dtype=torch.int32, device="cuda:0")
    nbytes = n * 2 * hkv * 16 * d * 2
    res = {"workload": "1024 random blocks of a 16384-block pool, 8 KV heads, d=128, bf16",
           "bytes_per_call": nbytes}
    for name, fn, moved in (("device_to_device", lambda: kvb.copy_blocks(dev, dev, src, dst), 2 * nbytes),
                            ("device_to_host", lambda: kvb.copy_blocks(dev, host, src, seq), nbytes),
                            ("host_to_device", lambda: kvb.copy_blocks(host, dev, seq, dst), nbytes)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(max(args.steps, 10)):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / max(args.steps, 10)
        res[name] = {"ms": ms, "gbps": moved / (ms * 1e-3) / 1e9}
    res["device_to_device"]["frac_hbm_peak"] = res["device_to_device"]["gbps"] / PEAK_GBPS
    return res


def bench_prefill_q8(torch, kvb, up, probe, ms16_cold, args, bits=8):
    """The step's prefill with the cached prefix in the 8-bit (or 4-bit) pool: the prefix
    tokens written by kvb_write_kv_q8 (K scales from their per-channel maxima), then
    kvb_paged_prefill_q8, timed cold like the 16-bit prefill."""
    w = up.w
    slot_list = []
    for b in range(w.batch):
        j = np.arange(int(w.prefix_lens[b]))
        slot_list.append(w.block_tables[b][j // 16].astype(np.int64) * 16 + j % 16)
    slots = torch.from_numpy(np.unique(np.concatenate(slot_list))).to("cuda:0")
    kt = up.k[slots // 16, :, slots % 16, :].contiguous()
    vt = up.v[slots // 16, :, slots % 16, :].contiguous()
    k_scale = (kt.float().abs().amax(dim=0) / (127.0 if bits == 8 else 7.0)).contiguous()
    p8 = kvb.PoolQ8.empty(w.k_pool.shape[0], w.num_kv_heads, w.head_dim, k_scale, bits=bits)
    kvb.write_kv_q8(p8, kt, vt, slots)
    del kt, vt
    out = torch.empty_like(up.q)
    n = kvb.paged_prefill_q8_workspace_size(w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim,
                                            w.total_q, up.max_p)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda:0")

    def run():
        kvb.paged_prefill_q8(p8, up.q, up.kn, up.vn, up.cu, up.pl, up.bt, w.scale, up.max_q, up.max_p,
                             out=out, workspace=ws)

    settle(torch, run, min(args.settle_ms, 200))
    cold = stats(time_each(torch, run, max(args.steps, 10), before=probe.flush))
    pf = prefill_flops(w)
    return {"pool": f"{bits}-bit codes, per-channel K scales, per-token V scales",
            "ms_cold": cold, "tflops_cold": pf / (cold["mean"] * 1e-3) / 1e12,
            "ms_cold_16bit_pool": ms16_cold, "time_vs_16bit": cold["mean"] / ms16_cold}


def bench_decode(torch, kvb, args, probe):
    """The paged-decode workload: 64 sequences, contexts U{512..4096} (seed 3), first 1024
    tokens shared, 32/8 heads, d=128, bf16, pool of 16384 blocks.  Timed as the plain split
    decode, as the shared-prefix (cascade) decode, which reads the 1024 shared tokens
    once for all sequences (both produce the same output up to rounding), and as decode
    over the same tokens in the 8-bit pool."""
    from workloads import make_config
    w = make_config("decode")
    k = _dev_bits(torch, w.k_pool, w.dtype)
    v = _dev_bits(torch, w.v_pool, w.dtype)
    pool = kvb.Pool.from_tensors(k, v)
    q = _dev_bits(torch, w.q, w.dtype)
    ctx = _idev(torch, w.context_lens)
    bt = _idev(torch, w.block_tables)
    out = torch.empty_like(q)
    max_ctx = int(w.context_lens.max())
    sb = args.split_blocks
    n = kvb.paged_decode_workspace_size(w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim, max_ctx, sb)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda:0")
    members, shared_ids = w.notes["first_group"]
    shared = _idev(torch, np.asarray(shared_ids, dtype=np.int32))
    shared_len = 16 * len(shared_ids)
    nc = kvb.paged_decode_cascade_workspace_size(w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim,
                                                 max_ctx, shared_len, sb)
    wsc = torch.empty(max(nc, 16), dtype=torch.uint8, device="cuda:0")

    def run():
        kvb.paged_decode(pool, q, ctx, bt, w.scale, max_ctx, split_blocks=sb, out=out, workspace=ws)

    def run_cascade():
        kvb.paged_decode_cascade(pool, q, ctx, bt, shared, shared_len, w.scale, max_ctx,
                                 split_blocks=sb, out=out, workspace=wsc)

    # The same context tokens in the 8-bit pool (kvb_write_kv_q8); the pool's per-channel
    # K scales are the context tokens' absolute maxima / 127.
    slot_list = []
    for b in range(w.batch):
        j = np.arange(int(w.context_lens[b]))
        slot_list.append(w.block_tables[b][j // 16].astype(np.int64) * 16 + j % 16)
    slots = torch.from_numpy(np.unique(np.concatenate(slot_list))).to("cuda:0")
    kt = k[slots // 16, :, slots % 16, :].contiguous()
    vt = v[slots // 16, :, slots % 16, :].contiguous()
    amax = kt.float().abs().amax(dim=0)
    p8 = kvb.PoolQ8.empty(w.k_pool.shape[0], w.num_kv_heads, w.head_dim, (amax / 127.0).contiguous())
    kvb.write_kv_q8(p8, kt, vt, slots)
    p4 = kvb.PoolQ8.empty(w.k_pool.shape[0], w.num_kv_heads, w.head_dim, (amax / 7.0).contiguous(),
                          bits=4)
    kvb.write_kv_q4(p4, kt, vt, slots)
    del kt, vt, amax

    def run_q8():
        kvb.paged_decode_q8(p8, q, ctx, bt, w.scale, max_ctx, split_blocks=sb, out=out, workspace=ws)

    def run_q4():
        kvb.paged_decode_q4(p4, q, ctx, bt, w.scale, max_ctx, split_blocks=sb, out=out, workspace=ws)

    settle(torch, lambda: (run(), run_cascade(), run_q8(), run_q4()), args.settle_ms)
    for _ in range(args.warmup):
        run()
        run_cascade()
        run_q8()
        run_q4()
    torch.cuda.synchronize()
    steps = max(args.steps, 10)
    sw, sc = _time_warm_cold(torch, run, steps, probe)
    scw, scc = _time_warm_cold(torch, run_cascade, steps, probe)
    sqw, sqc = _time_warm_cold(torch, run_q8, steps, probe)
    sq4w, sq4c = _time_warm_cold(torch, run_q4, steps, probe)
    tw, tc, cw, cc = sw["mean"], sc["mean"], scw["mean"], scc["mean"]
    qw, qc, q4w, q4c = sqw["mean"], sqc["mean"], sq4w["mean"], sq4c["mean"]
    pattern = _decode_read_pattern(torch, w, k, v, probe, steps)
    by8 = decode_bytes_q8(w, w.context_lens, w.block_tables)
    by4 = decode_bytes_q8(w, w.context_lens, w.block_tables, 4)
    by = decode_bytes(w, w.context_lens, w.block_tables)
    logical = float(np.sum(w.context_lens)) * w.num_kv_heads * w.head_dim * 2 * ESZ
    return {"workload": "paged decode, 64 sequences, contexts 512..4096, first 1024 tokens shared",
            "algorithmic_bytes": by, "ms_back_to_back": tw, "ms_cold_cache": tc,
            "ms_cold_stats": sc, "gbps_cold_median": by / (sc["median"] * 1e-3) / 1e9,
            "gbps_cold_best": by / (sc["min"] * 1e-3) / 1e9,
            "gbps_back_to_back": by / (tw * 1e-3) / 1e9, "gbps_cold_cache": by / (tc * 1e-3) / 1e9,
            "frac_hbm_peak_cold": by / (tc * 1e-3) / 1e9 / PEAK_GBPS,
            "logical_kv_gbps_cold": logical / (tc * 1e-3) / 1e9,
            "tflops_cold": decode_flops(w.context_lens, w) / (tc * 1e-3) / 1e12,
            "read_pattern": dict(pattern, decode_time_vs_pattern_cold=tc / pattern["ms_cold"]),
            "cascade": {"shared_tokens": shared_len, "ms_back_to_back": cw, "ms_cold_cache": cc,
                        "gbps_back_to_back": by / (cw * 1e-3) / 1e9,
                        "gbps_cold_cache": by / (cc * 1e-3) / 1e9,
                        "frac_hbm_peak_cold": by / (cc * 1e-3) / 1e9 / PEAK_GBPS},
            "q8": {"pool": "8-bit codes, per-channel K scales, per-token V scales",
                   "algorithmic_bytes": by8, "ms_back_to_back": qw, "ms_cold_cache": qc,
                   "gbps_cold_cache": by8 / (qc * 1e-3) / 1e9,
                   "frac_hbm_peak_cold": by8 / (qc * 1e-3) / 1e9 / PEAK_GBPS,
                   "speedup_vs_16bit_cold": tc / qc},
            "q4": {"pool": "4-bit codes (two per byte), per-channel K scales, per-token V scales",
                   "algorithmic_bytes": by4, "ms_back_to_back": q4w, "ms_cold_cache": q4c,
                   "gbps_cold_cache": by4 / (q4c * 1e-3) / 1e9,
                   "frac_hbm_peak_cold": by4 / (q4c * 1e-3) / 1e9 / PEAK_GBPS,
                   "speedup_vs_16bit_cold": tc / q4c}}


if __name__ == "__main__":
    sys.exit(main())
