"""Benchmark of the paged-attention hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input already
resident in HBM: the varlen paged prefill of a 2048-token causal chunk after
150,000 cached tokens (Hq 24, Hkv 4, D 256, page 64, fp16; the shape of the
pages' D256 chunked-prefill measurement, at the full head count of the model),
followed by the split-KV decode of a q=1 row over the same 152,048-token cache
(pass 1 + merge).

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload long_chunk|mixed_step|mixed_step_fp8|mixed_step_e4m3|decode_batch|varlen]
    python bench.py --mode copy|traffic|ceilings|crossover|sequences|operands|options

Prints ONE JSON line.  `value` is the step's algorithmic FLOPs (causal-exact:
4 * D * Hq per attended pair) divided by the step time; the prefill TFLOPS and
the decode GB/s are reported beside it, each from HIP events recorded on the
stream the kernels run on.  `roofline` prices the prefill call (its attention
kernel plus, when the keys are split, the merge of the parts; a split prefill
runs as pass 1 and the merge with an event between them, so the kernel alone
is reported beside it) against the MFMA fp16 dense peak; `decode_roofline`
prices the decode call, with the caches flushed before each call, against
the HBM peak (the warm figure beside it).  `cpu_baseline` times the fp64
oracle on a bounded sample of the same workload on the host cores, and the
whole oracle on the tiny, decode-batch and varlen workloads on all threads and
on one.
"""

import argparse
import copy
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from paged_attention_prefill_amd import inputs as gen  # noqa: E402
from paged_attention_prefill_amd import ops, workload  # noqa: E402

MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16/bf16 matrix peak
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_sources_hash():
    """sha256 over the HIP sources: counters taken on other sources no longer apply."""
    import hashlib
    d = os.path.join(ROOT, "paged_attention_prefill_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()


def measured_traffic(workload_name, part, key="hbm_bytes_per_call"):
    """HBM bytes per call (or, key="hbm_bytes_kernel", of its attention kernel alone) from the
    rocprofv3 counter runs, if taken on these sources."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("sources_sha256") != kernel_sources_hash():
        return None
    e = t.get("workloads", {}).get(workload_name, {}).get(part)
    return None if e is None else e.get(key)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Call:
    """One library call with preallocated outputs and workspace, timed by events."""

    def __init__(self, kind, case, d, splits, max_q=None):
        self.kind, self.case, self.d, self.splits = kind, case, d, splits
        # the case's attention options (sliding window, softcap, ALiBi slopes)
        self.opts = dict(window_left=case.meta.get("window_left", -1), softcap=case.meta.get("softcap", 0.0))
        if case.meta.get("alibi"):
            self.opts["alibi_slopes"] = torch.from_numpy(gen.geometric_alibi_slopes(case.num_q_heads)).to(d["q"].device)
        self.max_q = max_q or max(1, case.max_seqlen_q)
        self.out = torch.empty_like(d["q"])
        self.lse = torch.empty(d["q"].shape[:2], dtype=torch.float32, device=d["q"].device)
        D = case.head_dim
        if kind == "mixed":  # splits = (prefill parts, decode parts); the rows are routed by the library
            nb = ops.mixed_workspace_bytes(case.q_lens, case.max_pages_per_seq, case.num_q_heads, D,
                                           ops._TORCH_TO_PA[d["q"].dtype], 0, splits[1], splits[0])
        elif kind == "prefill":
            nb = ops.prefill_workspace_bytes(case.total_q, case.num_q_heads, D, splits)
        else:
            nb = ops.decode_workspace_bytes(case.total_q, case.num_q_heads, D, splits)
        self.ws = torch.empty(max(1, (nb + 3) // 4), dtype=torch.float32, device=d["q"].device)
        self.times = []
        self.pass1 = []  # (start, end of the attention kernel) of a split prefill

    def __call__(self, stream, record=False):
        c, d = self.case, self.d
        if record:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        if self.kind == "mixed":
            ops.mixed_step(d["q"], d["k"], d["v"], d["cu"], c.q_lens, d["seq_lens"], d["bt"], c.scale,
                           decode_splits=self.splits[1], prefill_splits=self.splits[0], k_scale=c.k_scale,
                           v_scale=c.v_scale, out=self.out, lse=self.lse, workspace=self.ws, stream=stream,
                           **self.opts)
        elif self.kind == "prefill" and self.splits > 1:
            # the two passes apart, so that the attention kernel is timed alone
            parts = ops.paged_prefill(d["q"], d["k"], d["v"], d["cu"], d["seq_lens"], d["bt"], c.max_seqlen_q,
                                      c.scale, k_scale=c.k_scale, v_scale=c.v_scale, num_kv_splits=self.splits,
                                      workspace=self.ws, stream=stream, merge=False, **self.opts)
            if record:
                em = torch.cuda.Event(enable_timing=True)
                em.record(stream)
                self.pass1.append((e0, em))
            ops.merge_states(parts, self.out.dtype, out=self.out, lse=self.lse, stream=stream)
        elif self.kind == "prefill":
            ops.paged_prefill(d["q"], d["k"], d["v"], d["cu"], d["seq_lens"], d["bt"], c.max_seqlen_q, c.scale,
                              k_scale=c.k_scale, v_scale=c.v_scale, num_kv_splits=self.splits, out=self.out,
                              lse=self.lse, workspace=self.ws, stream=stream, **self.opts)
        else:
            ops.split_kv_decode(d["q"], d["k"], d["v"], d["cu"], d["seq_lens"], d["bt"], self.max_q, c.scale,
                                num_splits=self.splits, k_scale=c.k_scale, v_scale=c.v_scale, out=self.out,
                                lse=self.lse, workspace=self.ws, stream=stream, **self.opts)
        if record:
            e1.record(stream)
            self.times.append((e0, e1))

    def ms(self):
        return float(np.mean([a.elapsed_time(b) for a, b in self.times])) if self.times else float("nan")

    def ms_median(self):
        return float(np.median([a.elapsed_time(b) for a, b in self.times])) if self.times else float("nan")

    def kernel_ms(self):
        """Mean duration of the attention kernel alone (the whole call when it is one kernel)."""
        if not self.pass1:
            return self.ms()
        return float(np.mean([a.elapsed_time(b) for a, b in self.pass1]))


# The calls of one step of each workload, in launch order.
WORKLOAD_CALLS = {"long_chunk": ["prefill", "decode"], "long_chunk_window": ["prefill", "decode"],
                  "mixed_step_fused": ["mixed"],
                  "long_chunk_softcap": ["prefill", "decode"], "long_chunk_alibi": ["prefill", "decode"],
                  "mixed_step": ["prefill", "decode"],
                  "mixed_step_fp8": ["prefill", "decode"], "mixed_step_e4m3": ["prefill", "decode"],
                  "decode_batch": ["decode"], "varlen": ["prefill"]}


def build_workload(name):
    """Returns (description, [Call specs]) for one step."""
    if name == "long_chunk":
        c = gen.long_chunk()
        pre = gen.select_seqs(c, [0], name="prefill 2048 after 150000")
        dec = gen.select_seqs(c, [1], name="decode q=1 at 152048")
        desc = {"workload": "paged prefill of a 2048-token causal chunk after 150,000 cached tokens + split-KV "
                            "decode of a q=1 row over the same cache",
                "num_q_heads": 24, "num_kv_heads": 4, "head_dim": 256, "page_size": 64, "q_len": 2048,
                "seq_len": 152048, "kv_dtype": "f16"}
        return desc, [("prefill", pre, "auto"), ("decode", dec, 64)]
    if name == "long_chunk_window":
        c = gen.long_chunk()
        c.meta["window_left"] = 8191
        pre = gen.select_seqs(c, [0], name="prefill 2048 after 150000, window 8192")
        dec = gen.select_seqs(c, [1], name="decode q=1 at 152048, window 8192")
        desc = {"workload": "the long chunk with a left sliding window of 8192 keys (prefill + q=1 decode)",
                "num_q_heads": 24, "num_kv_heads": 4, "head_dim": 256, "page_size": 64, "q_len": 2048,
                "seq_len": 152048, "kv_dtype": "f16", "window_left": 8191}
        return desc, [("prefill", pre, "auto"), ("decode", dec, 16)]
    if name in ("long_chunk_softcap", "long_chunk_alibi"):
        c = gen.long_chunk()
        if name == "long_chunk_softcap":
            c.meta["softcap"], what, opt = 50.0, "logit softcap 50", {"softcap": 50.0}
        else:
            c.meta["alibi"], what, opt = True, "ALiBi slopes 2^(-8 h / 24)", {"alibi": "geometric"}
        pre = gen.select_seqs(c, [0], name=f"prefill 2048 after 150000, {what}")
        dec = gen.select_seqs(c, [1], name=f"decode q=1 at 152048, {what}")
        desc = {"workload": f"the long chunk with {what} (prefill + q=1 decode)",
                "num_q_heads": 24, "num_kv_heads": 4, "head_dim": 256, "page_size": 64, "q_len": 2048,
                "seq_len": 152048, "kv_dtype": "f16", **opt}
        return desc, [("prefill", pre, "auto"), ("decode", dec, 64)]
    if name == "mixed_step_fused":
        c = gen.mixed_step(kv_kind="f16")  # sequence 0: the verify row, 1: the chunk
        c.meta.update(decode_rows=1)
        desc = {"workload": "the mixed step as one pa_mixed_step call (rows routed by q on the device, one attention "
                            "launch): the verify row q=5 at 240,000 keys and the 784-token chunk after 104,000, "
                            "fp16, D 256, page 816",
                "num_q_heads": 24, "num_kv_heads": 4, "head_dim": 256, "page_size": 816, "kv_dtype": "f16"}
        return desc, [("mixed", c, "auto")]
    if name == "mixed_step":
        c = gen.mixed_step(kv_kind="f16")
        ver = gen.select_seqs(c, [0], name="verify q=5 at 240000")
        chunk = gen.select_seqs(c, [1], name="prefill 784 after 104000")
        desc = {"workload": "mixed step: 784-token chunk after 104,000 cached tokens (prefill) + MTP verify row "
                            "q=5 at 240,000 (split-KV decode)", "num_q_heads": 24, "num_kv_heads": 4,
                "head_dim": 256, "page_size": 816, "kv_dtype": "f16"}
        return desc, [("prefill", chunk, "auto"), ("decode", ver, 64)]
    if name == "mixed_step_fp8":
        c = gen.mixed_step(kv_kind="e5m2")
        ver = gen.select_seqs(c, [0], name="verify q=5 at 240000 (fp8)")
        chunk = gen.select_seqs(c, [1], name="prefill 784 after 104000 (fp8)")
        desc = {"workload": "mixed step, fp8_e5m2 KV", "num_q_heads": 24, "num_kv_heads": 4, "head_dim": 256,
                "page_size": 816, "kv_dtype": "e5m2"}
        return desc, [("prefill", chunk, "auto"), ("decode", ver, 64)]
    if name == "mixed_step_e4m3":
        c = gen.mixed_step(kv_kind="e4m3")
        ver = gen.select_seqs(c, [0], name="verify q=5 at 240000 (e4m3)")
        chunk = gen.select_seqs(c, [1], name="prefill 784 after 104000 (e4m3)")
        desc = {"workload": "mixed step, fp8 E4M3 KV", "num_q_heads": 24, "num_kv_heads": 4, "head_dim": 256,
                "page_size": 816, "kv_dtype": "e4m3"}
        return desc, [("prefill", chunk, "auto"), ("decode", ver, 64)]
    if name == "decode_batch":
        c = gen.decode_batch(kind="bf16")
        desc = {"workload": "split-KV decode batch: 32 rows q=1, lengths 0..10000, MHA 16 heads, D 128, page 16",
                "num_q_heads": 16, "num_kv_heads": 16, "head_dim": 128, "page_size": 16, "kv_dtype": "bf16"}
        return desc, [("decode", c, 16)]
    if name == "varlen":
        c = gen.varlen_prefill(kind="bf16")
        desc = {"workload": "varlen paged prefill: q 64/300/1024/2048 after 0/777/4096/8192, Hq 32, Hkv 8, D 128, "
                            "page 32", "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128, "page_size": 32,
                "kv_dtype": "bf16"}
        return desc, [("prefill", c, "auto")]
    raise SystemExit(f"unknown workload {name}")


def prefill_kernel_name(desc):
    """Pass-1 kernel that serves the prefill of this workload."""
    if desc.get("kv_dtype") in ("e5m2", "e4m3") and desc.get("head_dim", 0) <= 128:
        return "attn_mfma_kernel"
    return "attn_prefill_w4_kernel" if desc.get("head_dim", 0) > 128 else "attn_mfma_dma_kernel"


def call_flops(kind, case):
    return workload.prefill_flops(case.cu_seqlens_q, case.seq_lens, case.num_q_heads, case.head_dim,
                                  case.meta.get("window_left", -1))


def call_bytes(kind, case, splits):
    return workload.decode_bytes(case.cu_seqlens_q, case.seq_lens, case.num_q_heads, case.num_kv_heads,
                                 case.head_dim, case.page_size, case.q_kind, case.kv_kind, splits,
                                 case.meta.get("window_left", -1))


def cpu_baseline(case, budget_rows, seed=0):
    """Time the fp64 oracle on a sample of the prefill rows; returns the baseline dict."""
    import oracle
    from threadpoolctl import threadpool_info
    rng = np.random.default_rng(seed)
    toks = np.sort(rng.choice(case.total_q, size=min(budget_rows, case.total_q), replace=False))
    rows = np.array([(t, h) for t in toks for h in range(case.num_q_heads)], dtype=np.int64)
    kind = case.kv_kind if case.kv_kind in ("e5m2", "e4m3") else "float"
    k = oracle.dequantize_pool(gen.to_numpy64(case.k_pool, case.kv_kind), kind, case.k_scale)
    v = oracle.dequantize_pool(gen.to_numpy64(case.v_pool, case.kv_kind), kind, case.v_scale)
    q64 = gen.to_numpy64(case.q)
    t0 = time.perf_counter()
    m = case.meta
    oracle.paged_attention(q64, k, v, case.cu_seqlens_q, case.seq_lens, case.block_tables, case.scale, rows=rows,
                           window_left=m.get("window_left", -1), softcap=m.get("softcap", 0.0),
                           alibi_slopes=gen.geometric_alibi_slopes(case.num_q_heads) if m.get("alibi") else None)
    dt = time.perf_counter() - t0
    # attended pairs of the sampled rows
    L = int(case.seq_lens[0])
    Q = case.total_q
    pairs = int(sum(max(0, L - Q + int(t) + 1) for t in toks)) * case.num_q_heads
    flops = 4 * case.head_dim * pairs
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOPS", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(toks)} of {Q} query tokens x {case.num_q_heads} heads of the prefill "
                      f"({pairs} attended pairs, {dt:.1f} s, numpy fp64)",
            "seconds": dt, "machine": host_machine(), "other_workloads": oracle_workload_timings()}


def host_machine():
    """The host the oracle ran on: logical CPUs, the CPU model, the CPUs this
    process may use and the BLAS threads numpy's matmul runs."""
    from threadpoolctl import threadpool_info
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"os_cpu_count": os.cpu_count(), "cpu_model": model,
            "usable_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
            "blas_threads": max([i.get("num_threads", 1) for i in threadpool_info()] or [1])}


def oracle_workload_timings():
    """The whole oracle on the tiny fp32 case, the 32-row decode batch and the
    varlen prefill, on all BLAS threads and on one (wall clock of the oracle
    call alone), each priced in its own unit: attended-pair FLOPs per second
    for the prefills, K/V bytes per second for the decode batch."""
    import oracle
    from threadpoolctl import threadpool_limits
    out = {}
    for name, make, unit in (("tiny_fp32", gen.tiny_fp32, "flops"),
                             ("decode_batch_bf16", lambda: gen.decode_batch(kind="bf16"), "bytes"),
                             ("varlen_bf16", lambda: gen.varlen_prefill(kind="bf16"), "flops")):
        c = make()
        kind = c.kv_kind if c.kv_kind in ("e5m2", "e4m3") else "float"
        k = oracle.dequantize_pool(gen.to_numpy64(c.k_pool, c.kv_kind), kind, c.k_scale)
        v = oracle.dequantize_pool(gen.to_numpy64(c.v_pool, c.kv_kind), kind, c.v_scale)
        q = gen.to_numpy64(c.q)

        def once():
            t0 = time.perf_counter()
            oracle.paged_attention(q, k, v, c.cu_seqlens_q, c.seq_lens, c.block_tables, c.scale)
            return time.perf_counter() - t0
        t_all = once()
        with threadpool_limits(1):
            t_one = once()
        if unit == "flops":
            work = workload.prefill_flops(c.cu_seqlens_q, c.seq_lens, c.num_q_heads, c.head_dim)
            rate = lambda t: work / t / 1e12  # noqa: E731
            runit = "TFLOPS"
        else:
            work = workload.decode_bytes(c.cu_seqlens_q, c.seq_lens, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                         c.page_size, c.q_kind, c.kv_kind, c.num_splits)
            rate = lambda t: work / t / 1e9  # noqa: E731
            runit = "GB/s"
        out[name] = {"all_threads_s": t_all, "one_thread_s": t_one, unit: work, "unit": runit,
                     "all_threads": rate(t_all), "one_thread": rate(t_one)}
        log(f"  oracle {name}: {t_all:.2f} s on all threads, {t_one:.2f} s on one")
    return out


def kv_write_timing(case, d, reps):
    """Writes the prefill chunk's K and V (fp16 / bf16 rows) into the case's cache
    at the chunk's positions, and into an fp8_e5m2 cache of the same geometry;
    HIP events on the current stream, median over reps, priced in HBM GB/s."""
    stream = torch.cuda.current_stream()
    g = torch.Generator(device="cuda").manual_seed(7)
    shape = (case.total_q, case.num_kv_heads, case.head_dim)
    kn = torch.randn(shape, generator=g, device="cuda").to(d["q"].dtype)
    vn = torch.randn(shape, generator=g, device="cuda").to(d["q"].dtype)
    out = {}
    targets = [(case.kv_kind, d["k"], d["v"])]
    if case.kv_kind != "e5m2" and case.q_kind == "f16":
        k8 = torch.zeros(d["k"].shape, dtype=torch.uint8, device="cuda")
        targets.append(("e5m2", k8, torch.zeros_like(k8)))
    src = "f16" if d["q"].dtype == torch.float16 else "bf16"
    for kv_kind, kp, vp in targets:
        times = []
        for i in range(reps + 3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            ops.write_kv(kn, vn, kp, vp, d["cu"], d["seq_lens"], d["bt"], max(1, case.max_seqlen_q), stream=stream)
            e1.record(stream)
            times.append((e0, e1))
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in times[3:]]))
        b = workload.kv_write_bytes(case.cu_seqlens_q, case.seq_lens, case.num_kv_heads, case.head_dim,
                                    case.page_size, src, kv_kind)
        out[kv_kind] = {"ms_median": ms, "bytes": b, "gbs": b / (ms * 1e-3) / 1e9,
                        "frac_of_hbm_peak": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    out["what"] = (f"write of the chunk's {case.total_q} new K and V rows ({case.num_kv_heads} kv heads, "
                   f"D {case.head_dim}) into its pages; not part of the step's value")
    return out


def copy_reference(steps):
    """A plain device copy of 1 GiB: reads and writes exactly 2^30 bytes per launch."""
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy", "bytes_read_per_launch": n * 4, "bytes_written_per_launch": n * 4,
                      "launches": steps}), flush=True)
    return 0


def _counter_rows(path):
    """(dispatch id, kernel name, value) of every dispatch in a rocprofv3 counter CSV tree."""
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)):
        for r in csv.DictReader(open(f)):
            rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return rows


def write_traffic(workload_name, pmc_dir):
    """Turns the FETCH_SIZE / WRITE_SIZE runs of `workload_name` (and of --mode copy)
    into per-call HBM bytes in profiles/traffic.json, tagged with the kernel sources."""
    per = {}
    factors = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        copy = _counter_rows(os.path.join(pmc_dir, "pmccopy_" + counter))
        if not copy:
            raise SystemExit(f"no copy-reference dispatches under {pmc_dir}/pmccopy_{counter}")
        kib = max(v for _, _, v in copy)
        factors[counter] = float(1 << 30) / (kib * 1024.0)
        # group this workload's dispatches into calls: a pass-1 kernel and the merges after it
        calls = []
        for _, name, v in _counter_rows(os.path.join(pmc_dir, "pmc_" + counter)):
            if "attn_" in name:
                calls.append([(name, v)])
            elif "merge" in name and calls:
                calls[-1].append((name, v))
        per[counter] = calls
    kinds = WORKLOAD_CALLS[workload_name]

    def kind_of(call):  # a call's kind by its pass-1 kernel (the run also holds extra decode repetitions)
        if len(kinds) == 1:
            return kinds[0]
        return "decode" if "attn_decode" in call[0][0] else "prefill"
    out = {"sources_sha256": kernel_sources_hash(),
           "about": "HBM bytes per call from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch), scaled by "
                    "the factors that make the same counters read 2^30 bytes for a 1 GiB device copy "
                    "(bench.py --mode copy).",
           "fetch_factor": factors["FETCH_SIZE"], "write_factor": factors["WRITE_SIZE"], "workloads": {}}
    try:
        old = json.load(open(TRAFFIC_FILE))
        if old.get("sources_sha256") == out["sources_sha256"]:
            out["workloads"] = old.get("workloads", {})
    except (OSError, ValueError):
        pass
    entry = {}
    for kind in kinds:
        f_calls = [c for c in per["FETCH_SIZE"] if kind_of(c) == kind]
        w_calls = [c for c in per["WRITE_SIZE"] if kind_of(c) == kind]
        names = [n for n, _ in f_calls[0]]
        fetch = [float(np.mean([c[j][1] for c in f_calls])) for j in range(len(names))]
        write = [float(np.mean([c[j][1] for c in w_calls])) for j in range(len(names))]
        total = 1024.0 * (sum(fetch) * factors["FETCH_SIZE"] + sum(write) * factors["WRITE_SIZE"])
        first = 1024.0 * (fetch[0] * factors["FETCH_SIZE"] + write[0] * factors["WRITE_SIZE"])
        entry[kind] = {"kernels": names, "fetch_kib": fetch, "write_kib": write, "hbm_bytes_per_call": total,
                       "hbm_bytes_kernel": first}
    out["workloads"][workload_name] = entry
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps({"mode": "traffic", "workload": workload_name, "factors": factors,
                      "bytes_per_call": {k: v["hbm_bytes_per_call"] for k, v in entry.items()}}), flush=True)
    return 0


def ceilings(seed=0):
    """Measured chip ceilings beside the published peaks: a pure MFMA loop on
    random and on zero fp16 operands (with the shader clock it ran at), the same
    loop fed a fresh random A fragment from LDS for every pair of MFMAs, the
    same loop with 0-8 fma or exp instructions after every MFMA (shader-clock
    cycles per MFMA: how much vector work one wave hides behind its own MFMAs),
    and a streaming read of 4 GiB."""
    import ctypes
    L = ops.lib()
    P, I = ctypes.c_void_p, ctypes.c_int32
    L.pa_ceiling_mfma.argtypes = [P, P, I, I, P, P]
    L.pa_ceiling_mfma_lds.argtypes = [P, P, I, I, P, P]
    L.pa_ceiling_stream_read.argtypes = [P, ctypes.c_int64, P, I, P]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    res = {"mode": "ceilings", "cus": cus}

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    g = torch.Generator().manual_seed(seed)
    blocks, iters = cus, 20000
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
    for kind in ("random", "zero"):
        a = torch.randn(128 * 8, generator=g) if kind == "random" else torch.zeros(128 * 8)
        a = a.half().cuda()

        def run():
            st = L.pa_ceiling_mfma(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(sink.data_ptr()), blocks, iters,
                                   ctypes.c_void_p(clocks.data_ptr()), sp)
            assert st == 0, st
        ms = timed(run, 3)
        c = clocks.view(-1, 2).cpu().double()
        ghz = float(torch.median(c[:, 0] / c[:, 1]) * 0.1)
        flops = blocks * 4 * iters * 4 * 32768
        res[f"mfma_f16_{kind}_tflops"] = flops / (ms * 1e-3) / 1e12
        res[f"mfma_f16_{kind}_clock_ghz"] = ghz
        res[f"mfma_f16_{kind}_cycles_per_mfma"] = float(torch.median(c[:, 0])) / (iters * 4)
    # fresh A fragments from LDS for every pair of MFMAs (attention's operand traffic)
    ops_lds = torch.randn((2048 + 256) * 8, generator=g).half().cuda()

    def run_lds():
        st = L.pa_ceiling_mfma_lds(ctypes.c_void_p(ops_lds.data_ptr()), ctypes.c_void_p(sink.data_ptr()), blocks,
                                   iters, ctypes.c_void_p(clocks.data_ptr()), sp)
        assert st == 0, st
    ms = timed(run_lds, 3)
    c = clocks.view(-1, 2).cpu().double()
    res["mfma_f16_lds_random_tflops"] = blocks * 4 * iters * 4 * 32768 / (ms * 1e-3) / 1e12
    res["mfma_f16_lds_random_clock_ghz"] = float(torch.median(c[:, 0] / c[:, 1]) * 0.1)
    res["mfma_f16_lds_random_cycles_per_mfma"] = float(torch.median(c[:, 0])) / (iters * 4)
    # vector-ALU work after every MFMA (one wave per SIMD): how much of it the wave hides
    L.pa_ceiling_mfma_valu.argtypes = [P, P, I, I, I, I, P, P]
    a = torch.randn(128 * 8, generator=g).half().cuda()
    coissue = {}
    for kind, kname in ((0, "fma"), (1, "exp")):
        for nv in (0, 2, 4, 6, 8):
            def run_v():
                st = L.pa_ceiling_mfma_valu(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(sink.data_ptr()), blocks,
                                            iters // 4, nv, kind, ctypes.c_void_p(clocks.data_ptr()), sp)
                assert st == 0, st
            timed(run_v, 1)
            c = clocks.view(-1, 2).cpu().double()
            coissue[f"{kname}_{nv}"] = round(float(torch.median(c[:, 0])) / (iters // 4 * 4), 2)
    res["mfma_cycles_with_valu_per_mfma"] = coissue
    nbytes = 4 << 30
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(1)
    rsink = torch.empty(cus * 8 * 256, dtype=torch.float32, device="cuda")

    def rd():
        st = L.pa_ceiling_stream_read(ctypes.c_void_p(src.data_ptr()), nbytes, ctypes.c_void_p(rsink.data_ptr()),
                                      cus * 8, sp)
        assert st == 0, st
    ms = timed(rd, 5)
    res["stream_read_gbs"] = nbytes / (ms * 1e-3) / 1e9
    res["published"] = {"mfma_f16_dense_tflops": MFMA_F16_PEAK_TFLOPS, "hbm_gbs": HBM_PEAK_GBS}
    print(json.dumps(res), flush=True)
    return 0


def crossover(reps=20):
    """Time one small-q row (q = 1..16 tokens) through the split-KV decode and
    through the prefill kernel, at the shapes of the mixed step (D 256, GQA 6,
    fp16) and of the varlen prefill (D 128, GQA 4, bf16), short and long
    contexts: the q at which the prefill call overtakes the decode call is the
    routing threshold of a mixed step.  One JSON line per (shape, q)."""
    stream = torch.cuda.current_stream()
    shapes = [("D256 GQA 24:4 f16 page 816", 24, 4, 256, 816, "f16"),
              ("D128 GQA 32:8 bf16 page 32", 32, 8, 128, 32, "bf16")]
    for name, hq, hkv, D, P, kind in shapes:
        for L in (2048, 32768, 131072):
            for q in (1, 2, 3, 4, 5, 6, 8, 10, 12, 16):
                case = gen.make_case("crossover", q_lens=[q], seq_lens=[L], num_q_heads=hq, num_kv_heads=hkv,
                                     head_dim=D, page_size=P, q_kind=kind, seed=q + L)
                d = gen.to_device(case)
                dec = Call("decode", case, d, 64 if L > 8192 else 16, max_q=q)
                sp = ops.auto_splits(case.total_q, 1, q, hq, hkv, D, ops._TORCH_TO_PA[case.q.dtype],
                                     ops._TORCH_TO_PA[case.q.dtype])
                pre = Call("prefill", case, d, sp)
                res = {"mode": "crossover", "shape": name, "seq_len": L, "q": q}
                for tag, c in (("decode", dec), ("prefill", pre)):
                    for _ in range(3):
                        c(stream)
                    torch.cuda.synchronize()
                    c.times = []
                    for _ in range(reps):
                        c(stream, record=True)
                    torch.cuda.synchronize()
                    res[f"{tag}_us"] = c.ms_median() * 1e3
                    res[f"{tag}_splits"] = c.splits
                res["faster"] = "decode" if res["decode_us"] <= res["prefill_us"] else "prefill"
                print(json.dumps(res), flush=True)
                del d, dec, pre
    return 0


def sequences(reps=20):
    """The varlen prefill and subsets of its sequences, each launched alone
    (one key part; the longest sequence also with 2): how much of the batch's
    time its longest sequence takes by itself, i.e. whether the batch is bound
    by the kernel's rate per compute unit or by the groups left over at the
    end.  One JSON line per launch, kernel time from HIP events."""
    stream = torch.cuda.current_stream()
    v = gen.varlen_prefill(kind="bf16")
    runs = [("all four", list(range(v.num_seqs)), 1), ("2048 after 8192", [3], 1), ("1024 after 4096", [2], 1),
            ("the three shorter", [0, 1, 2], 1), ("the two longest", [2, 3], 1), ("2048 after 8192", [3], 2)]
    for name, idx, splits in runs:
        case = v if len(idx) == v.num_seqs else gen.select_seqs(v, idx)
        c = Call("prefill", case, gen.to_device(case), splits)
        for _ in range(5):
            c(stream)
        torch.cuda.synchronize()
        c.times, c.pass1 = [], []
        for _ in range(reps):
            c(stream, record=True)
        torch.cuda.synchronize()
        f = call_flops("prefill", case)
        print(json.dumps({"mode": "sequences", "launch": name, "seqs": idx, "splits": splits, "gflop": f / 1e9,
                          "call_us": c.ms_median() * 1e3, "kernel_us": c.kernel_ms() * 1e3,
                          "kernel_tflops": f / (c.kernel_ms() * 1e-3) / 1e12}), flush=True)
        del c
    return 0


def operands(reps=20):
    """The long-chunk prefill call with its real (random) operands and with Q,
    K or V replaced by zeros: the same launch, the same instructions and the
    same memory traffic, only the values the matrix cores multiply differ.  A
    call that gets faster with zero operands is held back by the chip's power
    (its clock drops with the switching activity of the MFMA data), not by its
    instruction schedule.  One JSON line per operand set."""
    stream = torch.cuda.current_stream()
    case = gen.select_seqs(gen.long_chunk(), [0])
    d = gen.to_device(case)
    sp = ops.auto_splits(case.total_q, case.num_seqs, case.max_seqlen_q, case.num_q_heads, case.num_kv_heads,
                         case.head_dim, ops._TORCH_TO_PA[case.q.dtype], ops._TORCH_TO_PA[case.q.dtype])
    c = Call("prefill", case, d, sp)
    f = call_flops("prefill", case)
    keep = {k: d[k].clone() for k in ("q", "k", "v")}
    for zeroed in ((), ("q",), ("k",), ("v",), ("k", "v"), ()):
        for k in ("q", "k", "v"):
            d[k].copy_(keep[k])
            if k in zeroed:
                d[k].zero_()
        for _ in range(5):
            c(stream)
        torch.cuda.synchronize()
        c.times, c.pass1 = [], []
        for _ in range(reps):
            c(stream, record=True)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "operands", "zero": list(zeroed), "splits": c.splits, "call_ms": c.ms_median(),
                          "kernel_ms": c.kernel_ms(), "call_tflops": f / (c.ms_median() * 1e-3) / 1e12}),
              flush=True)
    return 0


def options(reps=8):
    """What the score options cost each kernel: the long-chunk prefill (4
    parts) and q=1 decode row at D 256, the varlen prefill and the decode
    batch at D 128, each plain, with a logit softcap of 30, with ALiBi and
    with both, the four calls of one case interleaved in one process.  One
    JSON line per case with the median call time of each option set (µs)."""
    stream = torch.cuda.current_stream()
    lc = gen.long_chunk()
    cases = [("long chunk prefill, D 256", "prefill", gen.select_seqs(lc, [0]), 4),
             ("long-chunk decode row q=1, D 256", "decode", gen.select_seqs(lc, [1]), 64),
             ("varlen prefill, D 128", "prefill", gen.varlen_prefill(kind="bf16"), 1),
             ("decode batch, 32 rows, D 128", "decode", gen.decode_batch(kind="bf16"), 16)]
    sets = {"plain": {}, "softcap 30": {"softcap": 30.0}, "ALiBi": {"alibi": True},
            "both": {"softcap": 30.0, "alibi": True}}
    for label, kind, case, splits in cases:
        d = gen.to_device(case)
        calls = {}
        for name, o in sets.items():
            c = copy.copy(case)
            c.meta = {**case.meta, **o}
            calls[name] = Call(kind, c, d, splits)
        for c in calls.values():
            for _ in range(2):
                c(stream)
        torch.cuda.synchronize()
        for c in calls.values():
            c.times, c.pass1 = [], []
        for _ in range(reps):
            for c in calls.values():
                c(stream, record=True)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "options", "call": label, "splits": splits,
                          "median_us": {n: c.ms_median() * 1e3 for n, c in calls.items()}}), flush=True)
        del d, calls
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_chunk")
    ap.add_argument("--prefill-splits", default=None, help="override: 0 = auto, or a count")
    ap.add_argument("--decode-splits", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=640, help="query tokens in the oracle sample")
    ap.add_argument("--mode", default="bench", choices=["bench", "copy", "traffic", "ceilings", "crossover", "sequences", "operands",
                                                      "options"],
                    help="copy: a plain 1 GiB device copy, the reference for the HBM traffic counters; "
                         "traffic: write profiles/traffic.json from the counter runs under --pmc-dir (no GPU); "
                         "ceilings: a pure MFMA loop and a streaming read, measured; "
                         "crossover: one small-q row through the decode and the prefill calls, q = 1..16; "
                         "sequences: the varlen prefill and its sequences launched alone; "
                         "operands: the long-chunk prefill with Q, K or V zeroed; "
                         "options: the softcap / ALiBi cost on each kernel")
    ap.add_argument("--pmc-dir", default="pmc",
                    help="--mode traffic: directory holding pmc_<COUNTER>/ and pmccopy_<COUNTER>/ runs")
    a = ap.parse_args()
    if a.mode == "traffic":
        return write_traffic(a.workload, a.pmc_dir)
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1 "
                                   "(the multi-GPU sharding is a design note, not built)"}))
        return 2
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if a.mode == "copy":
        return copy_reference(a.steps)
    if a.mode == "ceilings":
        return ceilings()
    if a.mode == "crossover":
        return crossover()
    if a.mode == "operands":
        return operands()
    if a.mode == "sequences":
        return sequences()
    if a.mode == "options":
        return options()
    ops.lib()

    log(f"building workload {a.workload} ...")
    desc, specs = build_workload(a.workload)
    calls = []
    for kind, case, splits in specs:
        if kind == "mixed":
            chunk = gen.select_seqs(case, range(case.meta["decode_rows"], case.num_seqs))
            sp = a.prefill_splits if a.prefill_splits is not None else splits
            sp = 0 if sp == "auto" else int(sp)
            if sp == 0:
                sp = ops.auto_splits(chunk.total_q, chunk.num_seqs, chunk.max_seqlen_q, case.num_q_heads,
                                     case.num_kv_heads, case.head_dim, ops._TORCH_TO_PA[case.q.dtype],
                                     {"e5m2": ops.PA_FP8_E5M2, "e4m3": ops.PA_FP8_E4M3}.get(
                                         case.kv_kind, ops._TORCH_TO_PA[case.q.dtype]))
            s = (sp, a.decode_splits or 64)
        elif kind == "prefill":
            s = a.prefill_splits if a.prefill_splits is not None else splits
            s = 0 if s == "auto" else int(s)
            if s == 0:
                s = ops.auto_splits(case.total_q, case.num_seqs, case.max_seqlen_q, case.num_q_heads,
                                    case.num_kv_heads, case.head_dim, ops._TORCH_TO_PA[case.q.dtype],
                                    {"e5m2": ops.PA_FP8_E5M2, "e4m3": ops.PA_FP8_E4M3}.get(
                                        case.kv_kind, ops._TORCH_TO_PA[case.q.dtype]))
        else:
            s = a.decode_splits or splits
        log(f"  {kind}: {case.name}, splits {s}")
        calls.append(Call(kind, case, gen.to_device(case), s))
    stream = torch.cuda.current_stream()

    for _ in range(a.warmup):
        for c in calls:
            c(stream)
    torch.cuda.synchronize()
    log(f"warmup done; timing {a.steps} steps")
    t0 = time.perf_counter()
    for _ in range(a.steps):
        for c in calls:
            c(stream, record=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / a.steps * 1e3

    step_flops = 0
    parts = {}
    for c in calls:
        ms = c.ms()
        if c.kind == "prefill":
            f = call_flops(c.kind, c.case)
            step_flops += f
            kms = c.kernel_ms()
            parts["prefill"] = {"ms": ms, "ms_median": c.ms_median(), "tflops": f / (ms * 1e-3) / 1e12, "flops": f,
                                "kernel_ms": kms, "kernel_tflops": f / (kms * 1e-3) / 1e12,
                                "splits": c.splits, "name": c.case.name}
        elif c.kind == "mixed":
            nd = c.case.meta["decode_rows"]
            rows = gen.select_seqs(c.case, range(nd))
            chunk = gen.select_seqs(c.case, range(nd, c.case.num_seqs))
            f = call_flops("prefill", chunk) + call_flops("decode", rows)
            step_flops += f
            parts["mixed"] = {"ms": ms, "ms_median": c.ms_median(), "tflops": f / (ms * 1e-3) / 1e12, "flops": f,
                              "prefill_splits": c.splits[0], "decode_splits": c.splits[1], "name": c.case.name,
                              "what": "one pa_mixed_step call: the fused attention launch and the two merges"}
        else:
            b = call_bytes(c.kind, c.case, c.splits)
            f = call_flops(c.kind, c.case)
            step_flops += f
            parts["decode"] = {"ms": ms, "ms_median": c.ms_median(), "gbs": b / (ms * 1e-3) / 1e9, "bytes": b,
                               "splits": c.splits, "name": c.case.name}
    value = step_flops / (ms_step * 1e-3) / 1e12
    res = {"metric": "paged-prefill TFLOPS (2K chunk @150K ctx, D256); split-KV decode HBM GB/s",
           "value": value, "unit": "TFLOPS", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
           "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": specs[0][1].q_kind, "data": "synthetic", "config": desc}
    res.update(parts)
    if "prefill" in parts:
        # the prefill call: its attention kernel and, when the keys are split,
        # the merge of the parts (both timed; the kernel alone beside them)
        pf = parts["prefill"]
        split = pf["splits"] > 1
        res["roofline"] = {"bound": "mfma", "achieved": pf["tflops"], "peak": MFMA_F16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": pf["tflops"] / MFMA_F16_PEAK_TFLOPS,
                           "traffic": measured_traffic(a.workload, "prefill"),
                           "kernel": prefill_kernel_name(desc) + (" + merge_rows_kernel" if split else ""),
                           "call_ms": pf["ms"], "kernel_ms": pf["kernel_ms"],
                           "merge_ms": pf["ms"] - pf["kernel_ms"] if split else 0.0,
                           "kernel_alone_tflops": pf["kernel_tflops"]}
    if "decode" in parts:
        dc = parts["decode"]
        res["decode_roofline"] = {"bound": "hbm", "achieved": dc["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": dc["gbs"] / HBM_PEAK_GBS,
                                  "traffic": measured_traffic(a.workload, "decode"),
                                  "kernel": "attn_decode_kernel + merge_kernel"}
    # decode with the caches flushed: reading 1 GiB between repetitions evicts
    # the K/V left in the 256 MB Infinity Cache and the L2s by the step (a read,
    # not a write: evicting dirty lines would put their write-back traffic on
    # the decode's HBM time)
    dec = [c for c in calls if c.kind == "decode"]
    if dec:
        c = dec[0]
        scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        c.times = []
        for _ in range(max(5, min(a.steps, 20))):
            scratch.sum()
            c(stream, record=True)
        torch.cuda.synchronize()
        del scratch
        ms = c.ms_median()
        b = parts["decode"]["bytes"]
        res["decode_cold"] = {"ms_median": ms, "gbs": b / (ms * 1e-3) / 1e9, "reps": len(c.times),
                              "note": "1 GiB scratch read before each repetition"}
        if "decode_roofline" in res:
            # the decode roofline is priced on the cache-flushed calls (no K/V
            # left in the Infinity Cache by the step), the warm figure beside it
            dr = res["decode_roofline"]
            dr["achieved_warm"] = dr["achieved"]
            dr["achieved"] = res["decode_cold"]["gbs"]
            dr["frac"] = dr["achieved"] / HBM_PEAK_GBS
            dr["timing"] = "median of the cache-flushed calls"
    pre = [c for c in calls if c.kind == "prefill"]
    if pre:
        res["kv_write"] = kv_write_timing(pre[0].case, pre[0].d, max(5, min(a.steps, 20)))
    if not a.no_cpu_baseline and "prefill" in parts:
        pre = [c for c in calls if c.kind == "prefill"][0].case
        if pre.num_seqs == 1:
            log("timing the oracle on a sample ...")
            res["cpu_baseline"] = cpu_baseline(pre, a.cpu_rows)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
