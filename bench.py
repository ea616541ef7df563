"""Benchmark of the GQA forward hot path on one MI355X.

One step = one pass of the whole hot path over resident, seeded synthetic inputs: one call on
each of the five workloads (workloads.py), largest first:
  1. gqa_prefill, Llama-shaped causal prefill (B 4, S 4096, 32 query heads over 8, d 128, bf16)
     -- the headline: `value` and `roofline` are this call's TFLOP/s;
  2. gqa_decode, uniform decode (B 64, 64 query heads over 8, d 128, 8192-key caches, bf16)
     -- `decode_roofline`;
  3. gqa_prefill, BERT-base-shaped bidirectional prefill (B 32, S 1024, 12 over 3, d 64,
     key lengths U[512, 1024]);
  4. gqa_decode, multi-query ragged decode with split-KV and the log-sum-exp merge (B 32,
     32 over 1, d 128, cache lengths U[1024, 32768]);
  5. gqa_prefill, tiny fp32 prefill (B 1, S 64, 4 over 2, d 32).
Every call is bracketed by HIP events on the stream it is launched on (torch's current
stream). Cache state is controlled for every timed call: before it, a read-only pass over a
768 MiB buffer (three times the 256 MB last-level cache) leaves every cache full of clean
lines that belong to nothing the call touches, and each workload rotates over independently
allocated copies of its inputs and outputs (4, or 2 for the 2 GiB uniform-decode caches).
Before the --warmup steps a time-based settle (--settle-s seconds of steps) brings the clocks
to their sustained level. Each workload's block reports mean / median / min / p90 of its call
time over the timed steps; `achieved` uses the mean, as the rocprofv3 --stats summaries do.

    python bench.py [--steps K] [--warmup W] [--settle-s S] [--no-cpu-baseline] [--no-extra]
                    [--no-probes] [--no-seeds]
    python bench.py --only WORKLOAD --steps K      (work for rocprofv3 runs: flush + call, K times)
    python bench.py --power SECONDS   (power and clock under sustained load, per workload)
    python bench.py --summarize-kernels DIR | --summarize-pmc DIR
    python bench.py --traffic-summary WORKLOAD DIR_FETCH DIR_WRITE DIR_COPY_FETCH DIR_COPY_WRITE
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GQA prefill TFLOP/s (% MFMA peak) + decode KV-cache GB/s (% HBM) on 1 MI355X"
STEP_ORDER = ["llama_causal_prefill", "gqa_decode_8k", "bert_base_prefill", "mqa_ragged_decode",
              "tiny_f32_prefill"]
HEADLINE_PREFILL = "llama_causal_prefill"
HEADLINE_DECODE = "gqa_decode_8k"
FLUSH_BYTES = 768 << 20
COPY_BYTES = 256 << 20
GEMM_N = 8192
CSRC = os.path.join(ROOT, "grouped_query_attention_02_amd", "csrc")

# Kernels each workload launches (names as in rocprofv3 traces) and the sources they are built
# from (a recorded traffic figure is void once any of them changes).
KERNELS = {
    "tiny_f32_prefill": (["prefill_f32_kernel<32, false>"], ["prefill_f32.hip"]),
    "bert_base_prefill": (["prefill_bf16_kernel<64, false, false, false, false>"], ["prefill_bf16.hip"]),
    "llama_causal_prefill": (["prefill_bf16_kernel<128, true, false, false, false>"],
                             ["prefill_bf16.hip"]),
    "gqa_decode_8k": (["decode_split_kernel<128, false, false>", "decode_combine_kernel<128>"],
                      ["decode_bf16.hip"]),
    "mqa_ragged_decode": (["decode_split_kernel<128, false, false>",
                           "decode_combine_kernel<128>"], ["decode_bf16.hip"]),
}
TRAFFIC_FILE = {
    "tiny_f32_prefill": "prefill_tiny_f32_traffic.md",
    "bert_base_prefill": "prefill_bert_base_traffic.md",
    "llama_causal_prefill": "prefill_llama_causal_traffic.md",
    "gqa_decode_8k": "decode_gqa_8k_traffic.md",
    "mqa_ragged_decode": "decode_mqa_ragged_traffic.md",
}


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _pct(xs, p):
    s = sorted(xs)
    k = (len(s) - 1) * p
    lo, hi = math.floor(k), math.ceil(k)
    return s[lo] + (s[hi] - s[lo]) * (k - lo)


def _stats_us(ms):
    us = [x * 1e3 for x in ms]
    return {"n": len(us), "us_mean": round(statistics.mean(us), 3),
            "us_median": round(statistics.median(us), 3), "us_min": round(min(us), 3),
            "us_p90": round(_pct(us, 0.9), 3)}


# ---------------------------------------------------------------- cache flush

class Flusher:
    """Read-only pass over FLUSH_BYTES with the probe library's streaming-read kernel: every
    cache level ends up holding clean lines of this buffer, and dirty lines left by earlier
    calls are written back here rather than inside the next timed call."""

    def __init__(self, dev):
        import ctypes
        import torch
        from grouped_query_attention_02_amd import build as gbuild
        if not os.path.exists(gbuild.PROBES_LIB):
            raise RuntimeError(f"{gbuild.PROBES_LIB} is missing: run __graft_entry__.build()")
        self.lib = ctypes.CDLL(gbuild.PROBES_LIB, mode=ctypes.RTLD_LOCAL)
        self.lib.gqa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                            ctypes.c_int, ctypes.c_void_p]
        self.buf = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        self.blocks = 8 * torch.cuda.get_device_properties(dev).multi_processor_count
        self.out = torch.empty(self.blocks * 256, dtype=torch.int32, device=dev)

    def __call__(self):
        import torch
        st = torch.cuda.current_stream().cuda_stream
        if self.lib.gqa_probe_read(self.buf.data_ptr(), FLUSH_BYTES // 16, self.out.data_ptr(),
                                   self.blocks, st) != 0:
            raise RuntimeError("flush launch failed")


# ---------------------------------------------------------------- workloads

class Case:
    """One workload: rotated copies of its device inputs/outputs, its algorithmic work and
    how to call it."""

    def __init__(self, w, dev, copies, seed=None, host=None, gen_device="cpu"):
        import torch
        import workloads as W
        from grouped_query_attention_02_amd import perfmodel
        import grouped_query_attention_02_amd as gqa
        self.w, self.name = w, w.name
        self.seed = w.seed if seed is None else seed
        if host is None:
            host = (W.make_prefill if w.kind == "prefill" else W.make_decode)(
                w, self.seed, device=gen_device)
        self.host = host if gen_device == "cpu" else None
        self.copies = []
        if w.kind == "prefill":
            lens = host["seqlens"]
            self.lens_host = None if lens is None else lens.cpu().tolist()
            self.work = perfmodel.prefill_flops(w.B, w.S, w.Hq, w.d, w.causal, self.lens_host)
            self.bound, self.unit = "mfma", "TFLOP/s"
            self.peak = (perfmodel.PEAK_BF16_TFLOPS if w.dtype == "bf16"
                         else perfmodel.PEAK_FP32_MFMA_TFLOPS)
            for i in range(copies):
                c = {k: host[k].to(dev) if i == 0 else self.copies[0][k].clone()
                     for k in ("q", "k", "v")}
                c["lens"] = None if lens is None else lens.to(dev)
                c["out"] = torch.empty_like(c["q"])
                self.copies.append(c)
        else:
            lens = host["lens"]
            self.lens_host = lens.cpu().tolist()
            self.work = perfmodel.decode_bytes(w.B, w.Hq, w.Hkv, w.d, self.lens_host,
                                               w.max_len, 2)
            self.bound, self.unit, self.peak = "hbm", "GB/s", perfmodel.PEAK_HBM_GBPS
            need = gqa.decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.max_len, 0)
            for i in range(copies):
                c = {k: host[k].to(dev) if i == 0 else self.copies[0][k].clone()
                     for k in ("q", "k_cache", "v_cache")}
                c["lens"] = lens.to(dev)
                c["out"] = torch.empty_like(c["q"])
                c["ws"] = torch.empty(max(16, need), dtype=torch.uint8, device=dev)
                self.copies.append(c)
        self.ms = []

    def rate(self, ms):
        """Algorithmic work per second in the block's unit for a call of `ms` milliseconds."""
        scale = 1e12 if self.unit == "TFLOP/s" else 1e9
        return self.work / (ms * 1e-3) / scale

    def run(self, i):
        import grouped_query_attention_02_amd as gqa
        c, w = self.copies[i % len(self.copies)], self.w
        if w.kind == "prefill":
            gqa.prefill(c["q"], c["k"], c["v"], causal=w.causal, softmax_scale=w.softmax_scale,
                        seqlens=c["lens"], out=c["out"])
        else:
            gqa.decode(c["q"], c["k_cache"], c["v_cache"], c["lens"],
                       softmax_scale=w.softmax_scale, workspace=c["ws"], out=c["out"])

    def block(self, achievable=None):
        import grouped_query_attention_02_amd as gqa
        st = _stats_us(self.ms)
        mean_ms = statistics.mean(self.ms)
        ach = self.rate(mean_ms)
        w = self.w
        b = {"bound": self.bound, "achieved": round(ach, 3), "peak": self.peak,
             "unit": self.unit, "frac": round(ach / self.peak, 4),
             "traffic": recorded_traffic(self.name),
             "kernel": " + ".join(KERNELS[self.name][0]),
             ("flops_per_launch" if self.bound == "mfma" else "bytes_per_call"): self.work,
             "rate_at_median": round(self.rate(st["us_median"] * 1e-3), 3),
             "rate_at_min": round(self.rate(st["us_min"] * 1e-3), 3), **st,
             "seed": self.seed, "copies_rotated": len(self.copies)}
        if achievable:
            key = "mfma_bf16_tflops" if self.bound == "mfma" else "hbm_read_gbps"
            if self.bound == "hbm" or w.dtype == "bf16":
                b["frac_of_achievable"] = round(ach / achievable[key], 4)
            if self.bound == "mfma" and w.dtype == "bf16":
                for k, f in (("mfma_bf16_random_operands_tflops", "frac_of_mfma_random_operands"),
                             ("gemm_bf16_tflops", "frac_of_gemm")):
                    if achievable.get(k):
                        b[f] = round(ach / achievable[k], 4)
        if w.kind == "prefill":
            b["sum_key_len"] = None if self.lens_host is None else sum(self.lens_host)
        else:
            b["sum_cache_len"] = sum(self.lens_host)
            b["split_workgroups"] = gqa.decode_num_workgroups(w.B, w.Hq, w.Hkv, w.max_len, 0)
        return b


def _shape(w):
    d = {"B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "dtype": w.dtype, "seed": w.seed}
    if w.kind == "prefill":
        d.update(S=w.S, causal=w.causal, key_lengths=list(w.lens) if w.lens else None,
                 value_scale=w.value_scale)
    else:
        d.update(max_len=w.max_len, cache_lengths=list(w.lens) if w.lens else None)
    return d


def _events(n):
    import torch
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)]


def time_calls(fn, reps, flush, ncopies=1):
    """Per-call ms of `reps` calls fn(i), each after a flush, each bracketed by events."""
    import torch
    evs = _events(reps)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        flush()
        a.record()
        fn(i % ncopies)
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


# ---------------------------------------------------------------- traffic records

def _sha256(path):
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def _read_fields(path):
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(("#", " ", "`", "|", "-")):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    return fields


def recorded_traffic(name):
    """HBM bytes per call recorded in profiles/, or None when any source of the workload's
    kernels has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", TRAFFIC_FILE[name])
    if not os.path.exists(path):
        return None
    f = _read_fields(path)
    for src in KERNELS[name][1]:
        if f.get(f"sha256 {src}") != _sha256(os.path.join(CSRC, src)):
            return None
    try:
        return int(float(f["hbm_bytes_per_call"]))
    except (KeyError, ValueError):
        return None


def _csv_rows(d, name):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", name), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _kernel_stats(d):
    """Durations (us) per (kernel name, grid size): one kernel launched with different grids
    (the decode on its two workloads) is listed once per grid."""
    rows = _csv_rows(d, "*kernel_trace.csv")
    acc = {}
    for r in rows:
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        grid = int(r.get("Grid_Size_X", 0) or 0) * int(r.get("Grid_Size_Y", 1) or 1)
        acc.setdefault((r["Kernel_Name"], grid), []).append(dur)
    return acc


def _summarize_kernels(d):
    """Per-kernel call count and mean/median/min duration (us) from rocprofv3 kernel traces."""
    for (name, grid), v in sorted(_kernel_stats(d).items(), key=lambda kv: -sum(kv[1])):
        print(f"{len(v):5d} calls  mean {statistics.mean(v):9.2f} us  median "
              f"{statistics.median(v):9.2f} us  min {min(v):9.2f} us  grid {grid:8d}  "
              f"{name[:100]}")
    return 0


def _pmc_means(d):
    """Per (kernel, counter) mean over dispatches of the counter summed over its instances."""
    per = {}
    for r in _csv_rows(d, "*counter_collection.csv"):
        key = (r["Kernel_Name"], r["Counter_Name"], r["Dispatch_Id"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    agg = {}
    for (kname, cname, _), v in per.items():
        agg.setdefault((kname, cname), []).append(v)
    return {k: (statistics.mean(v), len(v)) for k, v in agg.items()}


def _summarize_pmc(d):
    for (kname, cname), (m, n) in sorted(_pmc_means(d).items()):
        print(f"{cname:28s} mean {m:14.6g}  n={n:3d}  {kname[:100]}")
    return 0


def _match(kname, short):
    return short.replace(" ", "") in kname.replace(" ", "")


def _copy_counter(means, counter):
    """The copy kernel's reading of `counter` in a `--only copy` run (the copy is the dispatch
    named like a copy; else the largest reading)."""
    vals = {k: m for (k, c), (m, n) in means.items() if c == counter}
    named = [m for k, m in vals.items() if "opy" in k]
    return max(named) if named else max(vals.values())


def _traffic_summary(name, d_fetch, d_write, d_cfetch, d_cwrite):
    """Markdown record of one workload's HBM traffic per call: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) of its kernels, scaled by what the same counters read for a device copy of
    COPY_BYTES bytes, next to the algorithmic bytes."""
    import workloads as W
    from grouped_query_attention_02_amd import perfmodel
    w = W.WORKLOADS[name]
    kernels, srcs = KERNELS[name]
    f, wr = _pmc_means(d_fetch), _pmc_means(d_write)
    cf, cw = _pmc_means(d_cfetch), _pmc_means(d_cwrite)
    copy_f, copy_w = _copy_counter(cf, "FETCH_SIZE"), _copy_counter(cw, "WRITE_SIZE")
    sf, sw = COPY_BYTES / (copy_f * 1024), COPY_BYTES / (copy_w * 1024)
    fetch = write = 0.0
    raw = []
    for kn in kernels:
        fk = [m for (k, c), (m, n) in f.items() if c == "FETCH_SIZE" and _match(k, kn)]
        wk = [m for (k, c), (m, n) in wr.items() if c == "WRITE_SIZE" and _match(k, kn)]
        fk, wk = (fk[0] if fk else 0.0), (wk[0] if wk else 0.0)
        raw.append(f"- {kn}: FETCH_SIZE {fk:.1f} KiB, WRITE_SIZE {wk:.1f} KiB per dispatch")
        fetch += fk * 1024 * sf
        write += wk * 1024 * sw
    host = W.make_prefill if w.kind == "prefill" else W.make_decode
    x = host(w)
    if w.kind == "prefill":
        lens = None if x["seqlens"] is None else x["seqlens"].tolist()
        L = [w.S] * w.B if lens is None else lens
        esz = 2 if w.dtype == "bf16" else 4
        algo = 2 * w.B * w.S * w.Hq * w.d * esz + 2 * sum(L) * w.Hkv * w.d * esz
        algo_txt = "Q read + O written + valid K and V rows read once"
    else:
        algo = perfmodel.decode_bytes(w.B, w.Hq, w.Hkv, w.d, x["lens"].tolist(), w.max_len, 2)
        algo_txt = "valid K/V cache rows + q + o (perfmodel.decode_bytes)"
    hbm = fetch + write
    print(f"# HBM traffic: {' + '.join(kernels)} on {name}\n")
    print(f"Workload: {w.description}.\n")
    print("Commands (repository root on an MI355X; one counter per pass; each call of the "
          "workload follows a 768 MiB read-only flush, as in the benchmark):\n")
    print("```")
    for what, cnt in ((name, "FETCH_SIZE"), (name, "WRITE_SIZE"), ("copy", "FETCH_SIZE"),
                      ("copy", "WRITE_SIZE")):
        print(f"cd /tmp && export TMPDIR=/tmp && timeout -s KILL 120 rocprofv3 --pmc {cnt} "
              f"--output-format csv -d $REPO/gpurun_out/pmc/{what}_{cnt} -o run -- python3 "
              f"$REPO/bench.py --only {what} --steps 3")
    print(f"python3 bench.py --traffic-summary {name} gpurun_out/pmc/{name}_FETCH_SIZE "
          f"gpurun_out/pmc/{name}_WRITE_SIZE gpurun_out/pmc/copy_FETCH_SIZE "
          f"gpurun_out/pmc/copy_WRITE_SIZE")
    print("```\n")
    print(f"Calibration: `bench.py --only copy` copies {COPY_BYTES} bytes per launch; its "
          f"FETCH_SIZE reads {copy_f:.0f} KiB and WRITE_SIZE {copy_w:.0f} KiB, so the scale "
          f"factors are fetch x{sf:.3f} and write x{sw:.3f}.\n")
    print("Raw per dispatch (mean of 3):")
    print("\n".join(raw) + "\n")
    print(f"Algorithmic bytes: {algo_txt} = {algo} bytes.\n")
    print(f"workload: {name}")
    print(f"kernels: {' + '.join(kernels)}")
    for s in srcs:
        print(f"sha256 {s}: {_sha256(os.path.join(CSRC, s))}")
    print(f"fetch_bytes_per_call: {fetch:.0f}")
    print(f"write_bytes_per_call: {write:.0f}")
    print(f"hbm_bytes_per_call: {hbm:.0f}")
    print(f"algorithmic_bytes_per_call: {algo}")
    print(f"traffic_over_algorithmic: {hbm / algo:.3f}")
    return 0


# ---------------------------------------------------------------- extra rows

def _alibi_slopes(H):
    return [2.0 ** (-8.0 * (k + 1) / H) for k in range(H)]


def _extended_rows(reps, dev, flush, cases):
    """The optional paths, each timed (flush before every call) on its full-size workload:
    causal Llama-shaped prefill with a 1024-key sliding window and ALiBi; the MQA ragged decode
    read from a paged cache (256-key pages scattered over the pool); the MHA -> GQA conversion
    of a Llama-2-70B-shaped K projection (64 -> 8 heads)."""
    import numpy as np
    import torch
    import grouped_query_attention_02_amd as gqa
    from grouped_query_attention_02_amd import perfmodel
    out = {}
    lc = cases["llama_causal_prefill"]
    w, window = lc.w, 1024
    slopes = torch.tensor(_alibi_slopes(w.Hq), device=dev)
    flops = perfmodel.prefill_flops(w.B, w.S, w.Hq, w.d, True, None, window)

    def run_win(i):
        c = lc.copies[i % len(lc.copies)]
        gqa.prefill(c["q"], c["k"], c["v"], causal=True, softmax_scale=w.softmax_scale,
                    window=window, alibi_slopes=slopes, out=c["out"])
    ms = time_calls(run_win, 3, flush, len(lc.copies))
    ms = time_calls(run_win, reps, flush, len(lc.copies))
    st = _stats_us(ms)
    out["llama_causal_prefill_window1024_alibi"] = {
        "bound": "mfma", "achieved": round(flops / (statistics.mean(ms) * 1e-3) / 1e12, 3),
        "peak": perfmodel.PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(flops / (statistics.mean(ms) * 1e-3) / 1e12 / perfmodel.PEAK_BF16_TFLOPS,
                      4), "flops_per_launch": flops, "window": window, **st}

    dc = cases["mqa_ragged_decode"]
    wd, page = dc.w, 256
    mb = wd.max_len // page
    n_pages = wd.B * mb + 7
    perm = np.random.default_rng(12).permutation(n_pages)
    table = torch.tensor(perm[: wd.B * mb].reshape(wd.B, mb), dtype=torch.int32, device=dev)
    src = dc.copies[0]

    def to_pool(c):
        pool = torch.zeros((n_pages, wd.Hkv, page, wd.d), dtype=c.dtype, device=dev)
        pool[table.view(-1).long()] = c.view(wd.B, wd.Hkv, mb, page, wd.d) \
            .permute(0, 2, 1, 3, 4).reshape(wd.B * mb, wd.Hkv, page, wd.d)
        return pool
    kp, vp = to_pool(src["k_cache"]), to_pool(src["v_cache"])

    def run_paged(i):
        gqa.decode(src["q"], kp, vp, src["lens"], softmax_scale=wd.softmax_scale,
                   block_table=table, page_size=page, workspace=src["ws"], out=src["out"])
    time_calls(run_paged, 3, flush)
    ms = time_calls(run_paged, reps, flush)
    st = _stats_us(ms)
    gb = dc.work / (statistics.mean(ms) * 1e-3) / 1e9
    out["mqa_ragged_decode_paged256"] = {
        "bound": "hbm", "achieved": round(gb, 2), "peak": perfmodel.PEAK_HBM_GBPS,
        "unit": "GB/s", "frac": round(gb / perfmodel.PEAK_HBM_GBPS, 4),
        "bytes_per_call": dc.work, "page_size": page, **st}
    del kp, vp
    torch.cuda.empty_cache()

    H, G, per_head = 64, 8, 128 * 8192
    g = torch.Generator(device=dev).manual_seed(70)
    wk = (torch.randn((H, per_head), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    pooled = torch.empty((G, per_head), dtype=torch.bfloat16, device=dev)
    fn = lambda i: gqa.mean_pool_heads(wk, G, out=pooled)
    time_calls(fn, 3, flush)
    ms = time_calls(fn, reps, flush)
    nb = perfmodel.mean_pool_bytes(H, G, per_head, 2)
    gb = nb / (statistics.mean(ms) * 1e-3) / 1e9
    out["mean_pool_llama70b_kproj"] = {
        "bound": "hbm", "achieved": round(gb, 2), "peak": perfmodel.PEAK_HBM_GBPS,
        "unit": "GB/s", "frac": round(gb / perfmodel.PEAK_HBM_GBPS, 4), "bytes_per_call": nb,
        **_stats_us(ms)}
    return out


# ---------------------------------------------------------------- extra seeds

def _extra_seeds(dev, flush, reps, n_seeds=2):
    """Each bf16 workload on `n_seeds` further seeds (inputs drawn on the GPU with the same
    recipe): call time (median of `reps`, flushed, after half a second of calls to bring the
    clocks back up) and the max error against the oracle on sampled rows / (b, h) pairs, for
    the spread of both over inputs."""
    import numpy as np
    import torch
    import workloads as W
    import oracle
    out = {}
    for name in STEP_ORDER:
        w = W.WORKLOADS[name]
        if w.dtype != "bf16":
            continue
        rows_out = []
        for k in range(1, n_seeds + 1):
            seed = w.seed + 1000 * k
            host = (W.make_prefill if w.kind == "prefill" else W.make_decode)(
                w, seed, device="cuda")
            c = Case(w, dev, 1, seed=seed, host=host, gen_device="cuda")
            # the clocks drop while the host works between these runs: settle them first
            t_end = time.perf_counter() + 0.5
            while time.perf_counter() < t_end:
                time_calls(c.run, 4, flush)
            ms = time_calls(c.run, reps, flush)
            torch.cuda.synchronize()
            rng = np.random.default_rng(seed)
            if w.kind == "prefill":
                lens = host["seqlens"]
                n = 256
                rows = np.stack([rng.integers(w.B, size=n), rng.integers(w.Hq, size=n),
                                 rng.integers(w.S, size=n)], 1).astype(np.int64)
                qh, kh, vh = (host[t].cpu() for t in ("q", "k", "v"))
                ref_o, _ = oracle.prefill_rows(qh, kh, vh, rows, scale=w.softmax_scale,
                                               causal=w.causal,
                                               seqlens=None if lens is None else lens.cpu())
                o = c.copies[0]["out"].cpu()
                got = torch.stack([o[b, i, h] for b, h, i in rows]).double().numpy()
            else:
                n = 128
                pairs = np.stack([rng.integers(w.B, size=n), rng.integers(w.Hq, size=n)],
                                 1).astype(np.int64)
                qh, kh, vh = (host[t].cpu() for t in ("q", "k_cache", "v_cache"))
                ref_o, _ = oracle.decode_pairs(qh, kh, vh, pairs, scale=w.softmax_scale,
                                               lens=host["lens"].cpu())
                o = c.copies[0]["out"].cpu()
                got = torch.stack([o[b, h] for b, h in pairs]).double().numpy()
            err = float(np.abs(got - ref_o).max())
            st = _stats_us(ms)
            rows_out.append({"seed": seed, "us_median": st["us_median"],
                             "rate_at_median": round(c.rate(st["us_median"] * 1e-3), 3),
                             "unit": c.unit, "max_abs_err_sampled": err,
                             "sampled": f"{n} random {'rows' if w.kind == 'prefill' else '(b, h) pairs'}"})
            del c, host, qh, kh, vh
            torch.cuda.empty_cache()
        out[name] = rows_out
        _log(f"extra seeds {name}: " + ", ".join(
            f"seed {r['seed']} {r['us_median']:.1f} us err {r['max_abs_err_sampled']:.2e}"
            for r in rows_out))
    return out


# ---------------------------------------------------------------- CPU baseline

def _cpu_baseline(case, target_s: float):
    """The fp64 oracle, as it stands (OpenMP, all host threads), on random (b, head, query) rows
    of the headline prefill workload: a pilot sizes the sample to about target_s seconds. Also,
    single-threaded: the whole tiny fp32 prefill, and sampled (b, head) pairs of the uniform
    decode."""
    import numpy as np
    import torch
    import workloads as W
    import oracle
    w, x = case.w, case.host
    lens = np.full(w.B, w.S) if x["seqlens"] is None else x["seqlens"].numpy()
    lens = np.asarray(lens, dtype=np.int64)
    rng = np.random.default_rng(0)

    def sample(n):
        return np.stack([rng.integers(w.B, size=n), rng.integers(w.Hq, size=n),
                         rng.integers(w.S, size=n)], 1).astype(np.int64)

    def flops(rows):
        keys = lens[rows[:, 0]]
        if w.causal:
            keys = np.minimum(rows[:, 2] + 1, keys)
        return 4.0 * w.d * float(keys.sum())

    def run(rows, threads=0):
        t = time.perf_counter()
        oracle.prefill_rows(x["q"], x["k"], x["v"], rows, scale=w.softmax_scale,
                            causal=w.causal, seqlens=x["seqlens"], n_threads=threads)
        return time.perf_counter() - t

    pilot = sample(1000)
    rate = flops(pilot) / max(run(pilot), 1e-6)
    per_row = 4 * w.d * float(np.mean(lens)) * (0.5 if w.causal else 1.0)
    goal = int(max(1000, rate * target_s / per_row))
    done, fl, dt = 0, 0.0, 0.0
    total_rows = w.B * w.S * w.Hq
    while done < goal:
        rows = sample(min(200000, goal - done))
        dt += run(rows)
        fl += flops(rows)
        done += len(rows)
    res = {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
           "kind": "oracle",
           "sample": f"{done} random (b, head, query) rows of {w.name} ({done / total_rows:.4f} "
                     f"of its {total_rows} rows), fp64, {dt:.1f} s wall"}
    st = {}
    wt = W.WORKLOADS["tiny_f32_prefill"]
    xt = W.make_prefill(wt)
    t = time.perf_counter()
    oracle.prefill(xt["q"], xt["k"], xt["v"], scale=wt.softmax_scale, causal=False, n_threads=1)
    tt = time.perf_counter() - t
    ft = 4 * wt.d * wt.Hq * wt.B * wt.S * wt.S
    st["tiny_f32_prefill"] = {"value": ft / tt / 1e9, "unit": "GFLOP/s", "cores": 1,
                              "sample": f"whole workload, {tt * 1e3:.2f} ms"}
    wd = W.WORKLOADS["gqa_decode_8k"]
    xd = W.make_decode(wd.with_(B=4))   # 4 sequences of the uniform-decode shape
    pairs = np.array([(b, h) for b in range(4) for h in range(0, wd.Hq, 4)], dtype=np.int64)
    t = time.perf_counter()
    oracle.decode_pairs(xd["q"], xd["k_cache"], xd["v_cache"], pairs, scale=wd.softmax_scale,
                        lens=xd["lens"], n_threads=1)
    td = time.perf_counter() - t
    nbytes = len(pairs) * 2 * wd.max_len * wd.d * 2
    st["gqa_decode_8k"] = {"value": nbytes / td / 1e9, "unit": "GB/s (K/V bytes per head)",
                           "cores": 1,
                           "sample": f"{len(pairs)} (b, head) pairs of a 4-sequence instance "
                                     f"of the uniform-decode shape (8192 keys each), {td:.2f} s"}
    res["single_thread"] = st
    return res


# ---------------------------------------------------------------- achievable peaks

def _achievable(dev) -> dict:
    """Achievable peaks on this GPU from libgqa_probes.so: back-to-back bf16 32x32x16 MFMAs
    (four independent chains per wave, four waves per SIMD) and a read of a 4 GiB buffer
    (16 x the last-level cache) with plain and with non-temporal loads, each the best of
    several timed launches."""
    import ctypes
    import torch
    from grouped_query_attention_02_amd import build as gbuild
    lib = ctypes.CDLL(gbuild.PROBES_LIB, mode=ctypes.RTLD_LOCAL)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.gqa_probe_mfma_flops.argtypes = [i32, i32]
    lib.gqa_probe_mfma_flops.restype = ctypes.c_double
    lib.gqa_probe_mfma_bf16.argtypes = [i32, i32, vp, vp]
    lib.gqa_probe_read.argtypes = [vp, ctypes.c_size_t, vp, i32, vp]
    lib.gqa_probe_read_nt.argtypes = lib.gqa_probe_read.argtypes
    stream = torch.cuda.current_stream().cuda_stream
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks, iters = 4 * cus, 1000
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)

    def best(fn, reps):
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if fn() != 0:
                raise RuntimeError("probe launch failed")
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return min(ts)

    def mfma():
        return lib.gqa_probe_mfma_bf16(blocks, iters, out.data_ptr(), stream)

    best(mfma, 3)
    ms = best(mfma, 8)
    tflops = lib.gqa_probe_mfma_flops(blocks, iters) / (ms * 1e-3) / 1e12
    # The same products on random operands (the multipliers toggle as on real data), after
    # a second of back-to-back launches so that the clock has settled at its power limit.
    lib.gqa_probe_mfma_bf16_rand.argtypes = lib.gqa_probe_mfma_bf16.argtypes

    def mfma_rand():
        return lib.gqa_probe_mfma_bf16_rand(blocks, iters, out.data_ptr(), stream)

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 1.0:
        for _ in range(8):
            mfma_rand()
        torch.cuda.synchronize()
    rand_tflops = lib.gqa_probe_mfma_flops(blocks, iters) / (best(mfma_rand, 8) * 1e-3) / 1e12
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.zero_()
    rates = {}
    for name, fn in (("plain", lib.gqa_probe_read), ("nt", lib.gqa_probe_read_nt)):
        g = 0.0
        for per_cu in (4, 8, 16):
            rblocks = per_cu * cus
            rout = torch.empty(rblocks * 256, dtype=torch.int32, device=dev)

            def rd():
                return fn(buf.data_ptr(), nbytes // 16, rout.data_ptr(), rblocks, stream)
            best(rd, 2)
            g = max(g, nbytes / (best(rd, 5) * 1e-3) / 1e9)
        rates[name] = g
    gbps = max(rates.values())
    del buf, out
    torch.cuda.empty_cache()
    gemm = _gemm_reference(dev, best)
    return {"mfma_bf16_tflops": round(tflops, 1), "hbm_read_gbps": round(gbps, 1),
            "hbm_read_plain_gbps": round(rates["plain"], 1),
            "hbm_read_nt_gbps": round(rates["nt"], 1),
            "mfma_bf16_random_operands_tflops": round(rand_tflops, 1),
            "gemm_bf16_tflops": round(gemm, 1),
            "source": "probes/probes.hip: back-to-back bf16 MFMA on fixed operands, and on "
                      "random operands after 1 s at the power limit; 4 GiB streaming read with "
                      "plain and with non-temporal loads (hbm_read_gbps: the better); "
                      f"gemm: torch.matmul (the vendor BLAS) on {GEMM_N}^3 bf16, a reference "
                      "for the dense matrix-core rate reachable under the board's power limit"}


def _gemm_reference(dev, best=None):
    """TFLOP/s of a 2-D bf16 GEMM through torch.matmul (contiguous operands), the best of
    several launches after one second of back-to-back calls: what the vendor's tuned GEMM
    reaches on this board, to set the prefill fractions beside. Not part of the library."""
    import torch
    n = GEMM_N
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 1.0:
        for _ in range(4):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
    ts = []
    for _ in range(8):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.matmul(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del a, b, c
    torch.cuda.empty_cache()
    return 2.0 * n ** 3 / (min(ts) * 1e-3) / 1e12


# ---------------------------------------------------------------- power and clock

def _smi_sample():
    """(socket power W, mean graphics clock over the XCDs in MHz) from one `amd-smi metric
    -p -c` reading, or None where the tool or the fields are missing."""
    import re
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True, text=True,
                           timeout=10)
    except (OSError, subprocess.TimeoutExpired):
        return None
    pw = re.search(r"SOCKET_POWER: (\d+(?:\.\d+)?) W", r.stdout)
    clks = [int(x) for x in re.findall(r"GFX_\d+:\s*\n\s*CLK: (\d+) MHz", r.stdout)]
    if not pw or not clks:
        return None
    return float(pw.group(1)), statistics.mean(clks)


def _power_cap():
    import re
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showmaxpower"], capture_output=True, text=True,
                           timeout=20)
    except (OSError, subprocess.TimeoutExpired):
        return None
    m = re.search(r"Max Graphics Package Power \(W\): ([\d.]+)", r.stdout)
    return float(m.group(1)) if m else None


def _power(seconds, dev):
    """Power and clock under sustained load: each headline workload, then the bf16 GEMM
    reference and the matrix-core probe, called back to back (no flush) for `seconds` while a
    thread samples socket power and graphics clock; one JSON line with, per row, the rate and
    the medians of the samples taken after the first second."""
    import threading
    import torch
    import workloads as W
    cap = _power_cap()
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            s = _smi_sample()
            if s:
                samples.append((time.time(), *s))
            time.sleep(0.05)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    rows = {}

    def sustain(name, call, ncopies, work, unit):
        for i in range(4):
            call(i)
        torch.cuda.synchronize()
        t0, k = time.time(), 0
        while time.time() - t0 < seconds:
            for _ in range(8):
                call(k % ncopies)
                k += 1
            torch.cuda.synchronize()
        t1 = time.time()
        sel = [x for x in samples if t0 + 1.0 <= x[0] <= t1]
        scale = 1e12 if unit == "TFLOP/s" else 1e9
        rows[name] = {
            "rate": round(work * k / (t1 - t0) / scale, 1), "unit": unit,
            "us_per_call": round((t1 - t0) / k * 1e6, 2), "calls": k,
            "power_w_median": statistics.median(x[1] for x in sel) if sel else None,
            "power_w_max": max(x[1] for x in sel) if sel else None,
            "gfx_mhz_median": round(statistics.median(x[2] for x in sel)) if sel else None,
            "samples": len(sel)}
        _log(f"power: {name} {rows[name]}")
        time.sleep(2.0)

    for name in (HEADLINE_PREFILL, "bert_base_prefill", HEADLINE_DECODE, "mqa_ragged_decode"):
        n = 2 if name == HEADLINE_DECODE else 4
        c = Case(W.WORKLOADS[name], dev, n)
        sustain(name, c.run, n, c.work, c.unit)
        del c
        torch.cuda.empty_cache()
    n = GEMM_N
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    out = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    sustain(f"gemm_bf16_{n}", lambda i: torch.matmul(a, b, out=out), 1, 2.0 * n ** 3,
            "TFLOP/s")
    del a, b, out
    torch.cuda.empty_cache()
    # The matrix-core probe alone (no memory traffic): what the matrix cores sustain at the cap.
    import ctypes
    from grouped_query_attention_02_amd import build as gbuild
    lib = ctypes.CDLL(gbuild.PROBES_LIB, mode=ctypes.RTLD_LOCAL)
    lib.gqa_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.gqa_probe_mfma_flops.restype = ctypes.c_double
    lib.gqa_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p]
    blocks, iters = 4 * torch.cuda.get_device_properties(dev).multi_processor_count, 1000
    pout = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream

    def probe(i):
        if lib.gqa_probe_mfma_bf16(blocks, iters, pout.data_ptr(), stream) != 0:
            raise RuntimeError("probe launch failed")
    sustain("mfma_probe_bf16", probe, 1, lib.gqa_probe_mfma_flops(blocks, iters), "TFLOP/s")
    lib.gqa_probe_mfma_bf16_rand.argtypes = lib.gqa_probe_mfma_bf16.argtypes

    def probe_rand(i):
        if lib.gqa_probe_mfma_bf16_rand(blocks, iters, pout.data_ptr(), stream) != 0:
            raise RuntimeError("probe launch failed")
    sustain("mfma_probe_bf16_random_operands", probe_rand, 1,
            lib.gqa_probe_mfma_flops(blocks, iters), "TFLOP/s")
    stop.set()
    th.join()
    print(json.dumps({"power_cap_w": cap, "seconds_per_row": seconds,
                      "method": "calls back to back without the flush; amd-smi metric -p -c "
                                "sampled in a thread; medians over samples after the first "
                                "second", "rows": rows}), flush=True)
    return 0


# ---------------------------------------------------------------- profiling runs

def _only(what, steps, dev):
    """Run one workload (or a device copy of COPY_BYTES) `steps` times, each call after the
    cache flush, as in the benchmark; for rocprofv3 runs."""
    import torch
    import workloads as W
    if what == "copy":
        src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(steps):
            dst.copy_(src)
    else:
        flush = Flusher(dev)
        c = Case(W.WORKLOADS[what], dev, 1)
        for i in range(steps):
            flush()
            c.run(i)
    torch.cuda.synchronize()
    _log(f"ran {what} x{steps}")
    return 0


# ---------------------------------------------------------------- main

def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10, help="untimed steps after the settle")
    ap.add_argument("--settle-s", type=float, default=2.0,
                    help="seconds of untimed steps before the warm-up (sustained clocks)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the optional-path rows")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the achievable-peak microbenchmarks (achievable = null)")
    ap.add_argument("--no-seeds", action="store_true", help="skip the extra-seed runs")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--power", type=float, metavar="SECONDS",
                    help="power and clock under sustained load, SECONDS per row, then exit")
    ap.add_argument("--only", choices=list(STEP_ORDER) + ["copy"],
                    help="profiling run: execute just this work --steps times and exit")
    ap.add_argument("--summarize-kernels", metavar="DIR")
    ap.add_argument("--summarize-pmc", metavar="DIR")
    ap.add_argument("--traffic-summary", nargs=5,
                    metavar=("WORKLOAD", "FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"))
    args = ap.parse_args(argv)

    if args.summarize_kernels:
        return _summarize_kernels(args.summarize_kernels)
    if args.summarize_pmc:
        return _summarize_pmc(args.summarize_pmc)
    if args.traffic_summary:
        return _traffic_summary(*args.traffic_summary)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    import workloads as W
    import grouped_query_attention_02_amd as gqa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    gqa.load()
    dev = torch.device("cuda:0")
    _log(f"device {torch.cuda.get_device_name(0)}")
    if args.only:
        return _only(args.only, args.steps, dev)
    if args.power:
        return _power(args.power, dev)

    flush = Flusher(dev)
    cases = {}
    for name in STEP_ORDER:
        t = time.perf_counter()
        w = W.WORKLOADS[name]
        ncopies = 2 if name == "gqa_decode_8k" else (1 if name == "tiny_f32_prefill" else 4)
        cases[name] = Case(w, dev, ncopies)
        if name != HEADLINE_PREFILL:
            cases[name].host = None   # only the headline's host copy is kept (CPU baseline)
        _log(f"{name}: inputs ready in {time.perf_counter() - t:.1f} s ({ncopies} copies)")

    def step(i, timed):
        for name in STEP_ORDER:
            c = cases[name]
            flush()
            if timed:
                a, b = timed[name][i]
                a.record()
                c.run(i)
                b.record()
            else:
                c.run(i)

    t0 = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t0 < args.settle_s:
        for _ in range(4):
            step(n_settle, None)
            n_settle += 1
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t0
    for i in range(args.warmup):
        step(i, None)
    torch.cuda.synchronize()
    _log(f"settled {settle_s:.2f} s ({n_settle} steps), warm-up {args.warmup} steps")

    evs = {name: _events(args.steps) for name in STEP_ORDER}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for name in STEP_ORDER:
        cases[name].ms = [a.elapsed_time(b) for a, b in evs[name]]
    _log(f"timed {args.steps} steps in {wall:.3f} s")

    also = {}
    if not args.no_extra:
        also = _extended_rows(max(10, args.steps // 2), dev, flush, cases)
    ach = None
    if not args.no_probes:
        ach = _achievable(dev)
        _log(f"achievable: {ach['mfma_bf16_tflops']} TFLOP/s bf16 MFMA "
             f"({ach['mfma_bf16_random_operands_tflops']} on random operands), "
             f"{ach['hbm_read_gbps']} GB/s HBM read, {ach['gemm_bf16_tflops']} TFLOP/s "
             "bf16 GEMM")
    blocks = {name: cases[name].block(ach) for name in STEP_ORDER}
    for name, b in blocks.items():
        _log(f"{name}: mean {b['us_mean']:.2f} us median {b['us_median']:.2f} us -> "
             f"{b['achieved']} {b['unit']} ({b['frac']:.3f} of peak)")

    cpu = None
    if not args.no_cpu_baseline:
        _log("timing the oracle on the host")
        cpu = _cpu_baseline(cases[HEADLINE_PREFILL], args.cpu_seconds)

    seeds = None
    keep_ms_per_step = sum(statistics.mean(cases[n].ms) for n in STEP_ORDER)
    if not args.no_seeds:
        for name in STEP_ORDER:  # free the rotated copies first
            cases[name].copies = cases[name].copies[:1]
        torch.cuda.empty_cache()
        seeds = _extra_seeds(dev, flush, 10)

    hp, hd = blocks[HEADLINE_PREFILL], blocks[HEADLINE_DECODE]
    line = {
        "metric": METRIC,
        "value": hp["achieved"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(keep_ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) inputs (bf16; fp32 for the tiny case), uniform random "
                "lengths",
        "config": {
            "workload": " + ".join(STEP_ORDER),
            "headline_prefill": HEADLINE_PREFILL,
            "headline_decode": HEADLINE_DECODE,
            **{name: _shape(cases[name].w) for name in STEP_ORDER},
        },
        "roofline": hp,
        "decode_roofline": hd,
        "configs": blocks,
        "timing": {
            "method": "HIP events on the launch stream around each call; before each call a "
                      f"{FLUSH_BYTES >> 20} MiB read-only flush, inputs rotated over copies",
            "settle_s": round(settle_s, 2), "settle_steps": n_settle,
            "wall_s_timed_steps": round(wall, 4),
            "ms_per_step_is": "sum over the five workloads of the mean call time",
        },
        "cpu_baseline": cpu,
        "achievable": ach,
        "extra_seeds": seeds,
        "also": also,
        "context": "pages: ~980 tokens/s for a whole BERT-base model on A100 at seq 1024, "
                   "batch 32, precision unstated; not comparable to an attention-kernel rate. "
                   "Attention-core-only equivalent of the BERT-base prefill here: "
                   f"{cases['bert_base_prefill'].w.B * cases['bert_base_prefill'].w.S / (12 * blocks['bert_base_prefill']['us_mean'] * 1e-6):.0f}"
                   " tokens/s for 12 layers (not comparable)",
        "host": platform.node(),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
