"""Decode-attention benchmark: KV-read GB/s (fraction of HBM peak) and µs per decode step.

Default workload (3): paged GQA, bf16, batch 64, 32 q / 8 KV heads, head dim 128, page 16, ragged
seq lens uniform in [128, 8192] over a randomly permuted page pool (seeded, synthetic). The other
workloads (--workload 1..8) are the tiny fp32 MHA step, contiguous GQA, block-sparse speculative
decode, MLA, and workload 3 with an fp8 cache, with draft-token trees, and with an int4 cache;
every one runs the same way.

One step = the whole hot path on inputs already resident in HBM: split planning (host, done once),
the partial split-KV pass, and the LSE merge, launched through the C ABI on torch's current
stream. The step first runs untimed for SETTLE_S seconds (a fresh process runs its first few
hundred steps a few percent slower), then W untimed warm-up steps, then exactly K timed steps
bracketed by synchronisation; the streaming calibration runs after the timed regions.
Consecutive steps rotate over enough copies of the KV cache to exceed the 256 MB last-level cache,
so every step reads its KV from HBM.

`value` = algorithmic KV bytes per step (keys inside each sequence, inside listed blocks and
visible to some query row; K and V once per KV head, the MLA latent + rotary rows once) / step
time. `roofline` prices the dominant kernel (the partial pass) alone: the same algorithmic bytes
over its average duration, measured with HIP events recorded on its launch stream around every
timed launch; the MLA line adds the matrix-core rate of the same launches. `cpu_baseline` times
the fp64 oracle on a bounded sample of the same workload on the host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload N] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
METRIC = "KV-read GB/s (% of HBM peak) and µs per decode step, GQA bf16 paged"
LLC_BYTES = 256 << 20

# dominant kernel of each workload: (traffic record tag, kernel name)
KERNELS = {  # traffic tag, the launches attn_decode makes for the workload (timed together per step)
    1: ("partial_valu_contiguous_f32", "partial_valu_kernel, merge fused in (one launch per step)"),
    2: ("partial_valu_contiguous", "partial_valu_kernel, merge fused in (one launch per step)"),
    3: ("partial_valu_paged", "partial_valu_kernel + merge_kernel (two launches per step)"),
    4: ("partial_mfma_sparse", "partial_mfma_kernel + merge_kernel (two launches per step)"),
    5: ("mla_partial", "mla_partial_kernel + merge_kernel (two launches per step)"),
    6: ("partial_mfma16_paged_fp8", "partial_mfma16_kernel, fp8 cache, 16-row units + merge_kernel (two launches per step)"),
    7: ("partial_mfma_paged_spec", "partial_mfma_kernel, whole-row loads, draft trees + merge_kernel (two launches per step)"),
    8: ("partial_mfma16_paged_int4", "partial_mfma16_kernel, int4 cache, 16-row units + merge_kernel (two launches per step)"),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Step:
    """The hot path of one workload, prepared once; run(i) enqueues step i on the current stream."""

    def __init__(self, w, copies):
        import torch

        from attention_decode_amd import _abi

        self.w = w
        self.abi = _abi
        dev = w.q.device
        B, Q, Hq, Dv = w.batch, w.q_len, w.num_q_heads, w.head_dim_v
        rows = (w.q.shape[0],) if w.q_starts is not None else (B, Q)  # packed variable-length queries
        self.out = torch.empty(*rows, Hq, Dv, dtype=w.dtype, device=dev)
        self.lse = torch.empty(*rows, Hq, dtype=torch.float32, device=dev)
        common = dict(scale=w.scale, seq_lens=w.seq_lens, kv_len_max=w.kv_len_max, causal=w.causal,
                      window=w.window, out=self.out, lse=self.lse)
        if w.q_starts is not None or w.tree_mask is not None:
            common.update(q_starts=w.q_starts, q_len=Q if w.q_starts is not None else None, tree_mask=w.tree_mask)
        self.sets = []
        for c in range(copies):
            # .clone() of a strided view keeps its strides
            if w.kind == "mla":
                ckv = w.k if c == 0 else w.k.clone()
                kpe = w.kpe if c == 0 else w.kpe.clone()
                a = _abi.make_args(w.q, ckv, None, head_dim_qk=w.head_dim_qk, **common)
                self.sets.append((a, ckv, kpe))
            else:
                k = w.k if c == 0 else w.k.clone()
                v = w.v if c == 0 else w.v.clone()
                ks, vs = w.k_scale, w.v_scale  # an fp8 cache's row scales rotate with it
                if c and ks is not None and ks.stride() != (0, 0, 0):
                    ks, vs = ks.clone(), vs.clone()
                self.sets.append((_abi.make_args(w.q, k, v, k_scale=ks, v_scale=vs, **common), k, v, ks, vs))
        self.paged = _abi.make_paged(w.block_table, w.page_size) if w.kind in ("paged", "mla") else None
        self.sparse = _abi.make_sparse(w.num_blocks, w.block_idx, w.block_size) if w.num_blocks is not None else None
        self.splits, self.chunk = _abi.attn_decode_plan(self.sets[0][0], self.paged, self.sparse)
        if w.num_splits:
            self.splits = w.num_splits
        # The whole step through its entry point (attn_decode; attn_decode_mla), in a workspace
        # zero-filled once: one launch where the merge runs inside the partial pass, else the
        # partial pass and the merge kernel.
        self.mla = w.kind == "mla"
        nbytes = _abi.attn_decode_workspace_size(self.sets[0][0], self.paged, self.splits, self.sparse)
        self.workspace = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        self.launches = _abi.attn_decode_launches(self.sets[0][0], self.paged, self.sparse, self.splits)
        kid = _abi.attn_decode_kernel(self.sets[0][0])
        kind = _abi.KERNEL_NAMES[kid]
        if w.kv_format == "int4" and kid == _abi.AD_KERNEL_VECTOR:  # the vector kernel's int4 form has a symbol of its own
            kind += "_int4"
        if self.launches == 1:
            self.kernel_name = f"{kind} (merge inside; the whole step)"
        else:  # the partial pass alone, into buffers of its own
            self.kernel_name = f"{kind} (partial pass alone; the merge kernel follows it in a step)"
            self.kpart_o = torch.empty(B, Q, Hq, self.splits, Dv, dtype=torch.float32, device=dev)
            self.kpart_lse = torch.empty(B, Q, Hq, self.splits, dtype=torch.float32, device=dev)

    def step(self, i):
        """One whole decode step on cache copy i."""
        a, k, x = self.sets[i % len(self.sets)][:3]
        if self.mla:
            self.abi.attn_decode_mla(a, x, self.w.q_pe, self.paged, self.splits, self.workspace)
        else:
            self.abi.attn_decode(a, self.paged, self.sparse, self.splits, self.workspace)

    def kernel(self, i):
        """The step's dominant kernel alone: the partial pass (the whole step where the merge runs
        inside it)."""
        a, k, x = self.sets[i % len(self.sets)][:3]
        if self.launches == 1:
            self.step(i)
        elif self.mla:
            self.abi.attn_decode_mla_splitkv(a, x, self.w.q_pe, self.paged, self.splits, self.kpart_o, self.kpart_lse)
        else:
            self.abi.attn_decode_splitkv(a, self.paged, self.sparse, self.splits, self.kpart_o, self.kpart_lse)


def oracle_kwargs(w):
    """Arguments of the oracle call for a CPU workload (everything but the row selection)."""
    kw = dict(scale=w.scale, seq_lens=w.seq_lens, causal=w.causal, window=w.window)
    if w.kind in ("paged", "mla"):
        kw.update(block_table=w.block_table, page_size=w.page_size)
    if w.num_blocks is not None:
        kw.update(num_blocks=w.num_blocks, block_idx=w.block_idx, block_size=w.block_size)
    if w.kind == "mla":
        kw.update(q2=w.q_pe, k2=w.kpe)
    if w.kv_format == "fp8":
        kw.update(k_scale=w.k_scale, v_scale=w.v_scale)
    if w.kv_format == "int4":
        kw.update(int4_groups=w.kv_groups)
    if w.q_starts is not None:
        kw.update(q_starts=w.q_starts, q_len=w.q_len)
    if w.tree_mask is not None:
        kw.update(tree_mask=w.tree_mask)
    return kw


def cpu_baseline(w_cpu, budget_s=24.0):
    """The fp64 oracle, as it stands, on whole (sequence, KV head) groups of the workload (all their
    query rows), reported in the metric's unit (algorithmic KV GB/s). A fixed sample of groups is
    timed three times with every host thread and a smaller prefix of it three times with one
    thread; each figure is the median of its three runs. About budget_s seconds in all."""
    import oracle

    orc = oracle.load()
    Hq = w_cpu.num_q_heads
    counts = w_cpu.q_counts()
    first = [int(x) for x in w_cpu.q_starts] if w_cpu.q_starts is not None else [b * w_cpu.q_len for b in range(w_cpu.batch)]
    Hkv = 1 if w_cpu.kind == "mla" else w_cpu.num_kv_heads
    G = Hq // Hkv
    by_group = w_cpu.kv_bytes_by_group()
    kw = oracle_kwargs(w_cpu)
    v = w_cpu.k if w_cpu.kind == "mla" else w_cpu.v
    order = [(b, h) for b in range(w_cpu.batch) for h in range(Hkv)]

    def run(groups):
        sel = [order[i % len(order)] for i in range(groups)]
        rows = [(first[b] + t) * Hq + h * G + g for (b, h) in sel for t in range(counts[b]) for g in range(G)]
        t0 = time.perf_counter()
        orc.attend(w_cpu.q, w_cpu.k, v, rows=rows, **kw)
        return time.perf_counter() - t0, sum(by_group[b][h] for (b, h) in sel)

    def sample_for(seconds):
        """Groups (in order, wrapping) that take about `seconds` at the current thread count."""
        n = 1
        while True:
            t, _ = run(n)
            if t >= seconds / 8 or n >= 1 << 20:
                return max(1, int(n * seconds / max(t, 1e-6)))
            n *= 2

    def median3(groups):
        runs = sorted(run(groups) for _ in range(3))
        t, nbytes = runs[1]
        return nbytes / t / 1e9, nbytes, t

    threads = os.cpu_count() or 1
    orc.set_threads(threads)
    used = orc.threads()
    n_all = sample_for(budget_s / 6)
    gbps, nbytes, t = median3(n_all)
    orc.set_threads(1)
    n_one = min(n_all, sample_for(budget_s / 6))
    gbps1, nbytes1, t1 = median3(n_one)
    orc.set_threads(used)
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": used, "kind": "oracle",
            "sample": f"{n_all} (sequence, KV head) groups of the {len(order)} in the workload (in order, "
                      f"wrapping), all {G} x (query tokens) rows each: {nbytes / 1e6:.1f} MB of KV, median of 3 "
                      f"runs on {used} threads ({t:.2f} s)",
            "single_thread": {"value": round(gbps1, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"the first {n_one} of those groups: {nbytes1 / 1e6:.1f} MB of KV, median "
                                        f"of 3 runs on 1 thread ({t1:.2f} s)"}}


TRAFFIC_SOURCES = ["attention_decode_amd/csrc/api.cpp", "attention_decode_amd/csrc/ad_internal.h"]


def sources_sha256(paths):
    """One sha256 over the named files, in order (the kernel's source, the planner, the parameter block)."""
    import hashlib

    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(hashlib.sha256(f.read()).digest())
    return h.hexdigest()


def load_traffic(kernel_tag):
    """HBM traffic of the dominant kernel from committed rocprofv3 counter runs, or None when the
    kernel's source, the split planner or the parameter block changed since the counters were
    taken (a planner change moves splits, and with them the traffic)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_tag}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    srcs = rec.get("sources")
    if not srcs or any(not os.path.exists(os.path.join(ROOT, x)) for x in srcs):
        return None
    if sources_sha256(srcs) != rec.get("sources_sha256"):
        return None
    return rec.get("bytes_per_launch")


# Seconds the step runs untimed before the warm-up steps. A fresh process runs its first few
# hundred steps slower: workload 3 from a cold start, 20-step averages 352 (first touches), 204,
# 196, then 193-194 us per step from about the 60th step on; right after the streaming calibration
# (2 GiB read for a quarter second) it stayed near 199 us for about 280 steps. So the calibration
# runs after the timed regions, and the step settles for SETTLE_S first.
SETTLE_S = 0.15


def stream_peak(stream):
    """Same-process streaming calibration, after the timed regions: the library's read probe
    (attn_decode_read_probe: the partial passes' load form, every work group streaming its own
    region) over 2 GiB, and a torch device copy of 1 GiB for context; 5 launches each after 2
    warm-ups, timed with events on `stream`. GB/s of bytes moved (read for the probe; read + written
    for the copy)."""
    import torch

    from attention_decode_amd import _abi

    out = {}
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    x = torch.zeros(512 << 20, dtype=torch.int32, device="cuda")   # 2 GiB
    sink = torch.empty(_abi.AD_PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
    for _ in range(2):
        _abi.attn_decode_read_probe(x, sink)
    a.record(stream)
    for _ in range(5):
        _abi.attn_decode_read_probe(x, sink)
    b.record(stream)
    torch.cuda.synchronize()
    out["read_probe"] = round(x.numel() * 4 * 5 / (a.elapsed_time(b) * 1e-3) / 1e9, 1)
    del x
    y = torch.ones(256 << 20, device="cuda")             # 1 GiB
    z = torch.empty_like(y)
    for _ in range(2):
        z.copy_(y)
    a.record(stream)
    for _ in range(5):
        z.copy_(y)
    b.record(stream)
    torch.cuda.synchronize()
    out["torch_copy"] = round(2 * y.numel() * 4 * 5 / (a.elapsed_time(b) * 1e-3) / 1e9, 1)
    del y, z
    torch.cuda.empty_cache()
    return out


def pct(xs, q):
    """The q-quantile (0..1) of sorted xs, nearest rank."""
    return xs[min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3, choices=sorted(KERNELS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run 3 device copies of 256 MiB (reads and writes 268,435,456 B each): the "
                         "reference dispatch that scales the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch

        x = torch.ones(64 << 20, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": x.numel() * 4, "bytes_written": y.numel() * 4}))
        return

    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; run it with --gpus 1"}))
        log("bench.py: only --gpus 1 is supported (the decode step runs on a single GPU)")
        sys.exit(2)

    import torch

    from attention_decode_amd import inputs

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    torch.cuda.set_device(int(os.environ.get("LOCAL_RANK", "0")))

    log(f"generating workload {args.workload} ...")
    w_cpu = inputs.make(args.workload)
    w = w_cpu.to("cuda")
    kv_bytes = w_cpu.kv_bytes()
    flops = w_cpu.flops()
    footprint = sum(t.untyped_storage().nbytes() for name, t in w.storage.items() if name != "q" and name != "q_pe")
    copies = max(1, math.ceil((1 << 30) / footprint) + 1) if footprint < (1 << 30) else 2
    step = Step(w, copies)
    log(f"workload {w.name}: {kv_bytes / 1e6:.1f} MB KV/step, splits {step.splits} x {step.chunk} keys, "
        f"{copies} cache copies ({footprint / 1e6:.0f} MB each)")

    stream = torch.cuda.current_stream()
    log(f"settling ({SETTLE_S} s of untimed steps) ...")
    t_settle, n_settle = time.perf_counter(), 0
    while time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(8):
            step.step(n_settle)
            n_settle += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step.step(i)
        step.kernel(i)
    torch.cuda.synchronize()

    K = args.steps
    # 1) the headline: K whole steps back to back, one pair of events around them all
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        step.step(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / K
    # 2) the dominant kernel: K launches of it alone back to back (its average duration)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for i in range(K):
        step.kernel(i)
    k1.record(stream)
    torch.cuda.synchronize()
    kern_avg = k0.elapsed_time(k1) / K
    # 3) its spread: the same launches, each between its own events (which add their own time)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        step.kernel(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    kern_ms = sorted(a.elapsed_time(b) for a, b in ev)
    # 4) the step's spread: whole steps, each between its own events
    for i in range(K):
        ev[i][0].record(stream)
        step.step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    step_ms = sorted(a.elapsed_time(b) for a, b in ev)
    log("streaming calibration ...")
    peak = stream_peak(stream)
    gbps = kv_bytes / (ms_step * 1e-3) / 1e9
    achieved = kv_bytes / (kern_avg * 1e-3) / 1e9
    tflops = flops / (kern_avg * 1e-3) / 1e12
    log(f"step {ms_step * 1e3:.1f} us ({gbps:.0f} GB/s, {gbps / HBM_PEAK_GBPS:.1%} of 8 TB/s); {step.kernel_name} "
        f"alone {kern_avg * 1e3:.1f} us -> {achieved:.0f} GB/s, {tflops:.0f} TFLOP/s (one launch between events: "
        f"p10 {pct(kern_ms, .1) * 1e3:.1f}, p50 {pct(kern_ms, .5) * 1e3:.1f}, p90 {pct(kern_ms, .9) * 1e3:.1f} us); "
        f"streaming calibration {peak}")

    tag, kname = KERNELS[args.workload]
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": load_traffic(tag),
                "kernel": step.kernel_name, "kernel_avg_us": round(kern_avg * 1e3, 3),
                "kernel_event_us_p10_p50_p90": [round(pct(kern_ms, q) * 1e3, 2) for q in (.1, .5, .9)],
                "measured_stream_GBps": peak,
                "frac_of_measured_stream": round(achieved / peak["read_probe"], 4)}
    if w.kind == "mla":
        roofline["mfma_tflops"] = round(tflops, 1)
        roofline["mfma_frac"] = round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)
    config = {"workload": w.name, "batch": w.batch, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
              "head_dim_qk": w.head_dim_qk, "head_dim_v": w.head_dim_v, "q_len": w.q_len,
              "kv_tokens": int(w_cpu.seq_lens.sum()), "kv_bytes_per_step": kv_bytes, "flops_per_step": flops,
              "splits": step.splits, "split_keys": step.chunk, "cache_copies_rotated": copies}
    if w.q_starts is not None:
        config["query_tokens"] = int(w.q.shape[0])  # packed variable-length queries, q_len at most
    if w.tree_mask is not None:
        config["tree_mask"] = True
    if w.page_size:
        config["page_size"] = w.page_size
    config["kv_bytes_convention"] = ("each key once per KV head (K and V rows; MLA: latent + rotary row once) if "
                                     "it is inside its sequence, inside a listed block and visible to at least "
                                     "one query row")
    if w.num_blocks is not None:
        config["sparse_block"] = w.block_size
        listed = w_cpu.kv_bytes_listed()
        config["kv_bytes_listed_blocks"] = listed
        config["value_on_listed_blocks_GBps"] = round(listed / (ms_step * 1e-3) / 1e9, 2)
    if w.causal or w.window:
        config.update(causal=bool(w.causal), window=w.window)
    result = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 2),
        "step_event_us_p10_p50_p90": [round(pct(step_ms, q) * 1e3, 2) for q in (.1, .5, .9)],
        "frac_of_measured_stream": round(gbps / peak["read_probe"], 4),
        "hbm_peak_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic (seeded N(0,1) Q/K/V, seeded ragged lengths, page permutations and block lists)",
        "config": config,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(w_cpu, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
