"""Benchmark of the GQA forward hot path on one MI355X.

One step = one pass of the whole hot path on resident, seeded synthetic inputs:
  1. gqa_prefill on the BERT-base-shaped bidirectional workload (batch 32, seq 1024,
     12 query heads over 3 K/V heads, d 64, bf16, key lengths uniform in [512, 1024]);
  2. gqa_decode on the multi-query ragged workload (32 sequences, 32 query heads over
     1 K/V head, d 128, bf16, cache lengths uniform in [1024, 32768], split-KV + combine).
`value` is the prefill rate in TFLOP/s (algorithmic FLOPs / measured launch time) and
the line's `decode` object carries the decode KV-cache GB/s; both are timed with HIP
events on the stream the kernels run on, inside the K timed steps. After the timed
steps, the causal Llama-style prefill and the uniform 8k decode are timed the same way
and reported under `also` (not part of `value`), and two microbenchmarks give the rates
this GPU reaches (`achievable`: bf16 MFMA loop, streaming HBM read).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra] [--no-probes]
    python bench.py --only prefill|prefill_causal|decode|copy --steps K   (work for rocprofv3 runs)
    python bench.py --summarize-kernels DIR | --summarize-pmc DIR
"""
from __future__ import annotations

import argparse
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


def _events(n):
    import torch
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)]


def _ms(evs):
    return [a.elapsed_time(b) for a, b in evs]


def _prefill_case(w, dev):
    import torch
    import workloads as W
    from grouped_query_attention_02_amd import perfmodel
    x = W.make_prefill(w, device="cpu")
    q, k, v = x["q"].to(dev), x["k"].to(dev), x["v"].to(dev)
    lens = None if x["seqlens"] is None else x["seqlens"].to(dev)
    lens_host = None if x["seqlens"] is None else x["seqlens"].tolist()
    flops = perfmodel.prefill_flops(w.B, w.S, w.Hq, w.d, w.causal, lens_host)
    out = torch.empty_like(q)
    return dict(w=w, q=q, k=k, v=v, lens=lens, lens_host=lens_host, flops=flops, out=out,
                host=x)


def _decode_case(w, dev):
    import torch
    import workloads as W
    import grouped_query_attention_02_amd as gqa
    from grouped_query_attention_02_amd import perfmodel
    x = W.make_decode(w, device="cpu")
    q, kc, vc, lens = (x["q"].to(dev), x["k_cache"].to(dev), x["v_cache"].to(dev),
                       x["lens"].to(dev))
    lens_host = x["lens"].tolist()
    nbytes = perfmodel.decode_bytes(w.B, w.Hq, w.Hkv, w.d, lens_host, w.max_len, 2)
    ws = torch.empty(max(16, gqa.decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.max_len, 0)),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    del x
    return dict(w=w, q=q, kc=kc, vc=vc, lens=lens, lens_host=lens_host, bytes=nbytes, ws=ws,
                out=out)


def _run_prefill(c):
    import grouped_query_attention_02_amd as gqa
    w = c["w"]
    gqa.prefill(c["q"], c["k"], c["v"], causal=w.causal, softmax_scale=w.softmax_scale,
                seqlens=c["lens"], out=c["out"])


def _run_decode(c):
    import grouped_query_attention_02_amd as gqa
    w = c["w"]
    gqa.decode(c["q"], c["kc"], c["vc"], c["lens"], softmax_scale=w.softmax_scale,
               workspace=c["ws"], out=c["out"])


def _time_queued(fn, c, n, hold_fn, hold_c):
    """Mean device time of n back-to-back calls: a long call (hold_fn) is enqueued first so that
    all n calls are queued before the GPU reaches them, and the events bracket only the n calls
    (each call's own launch gaps included, the host's per-call overhead not)."""
    import torch
    a, b = _events(1)[0]
    torch.cuda.synchronize()
    hold_fn(hold_c)
    a.record()
    for _ in range(n):
        fn(c)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def _time_loop(fn, c, reps, warm, warm_s=1.0):
    """Mean of `reps` timed calls after `warm` calls and at least warm_s
    seconds of untimed work (so the clocks are at their sustained level)."""
    import torch
    t_end = time.perf_counter() + warm_s
    n = 0
    while n < warm or time.perf_counter() < t_end:
        fn(c)
        n += 1
        if n % 64 == 0:
            torch.cuda.synchronize()
    evs = _events(reps)
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        fn(c)
        b.record()
    torch.cuda.synchronize()
    return _ms(evs)


def _alibi_slopes(H):
    return [2.0 ** (-8.0 * (k + 1) / H) for k in range(H)]


def _extended_rows(steps, dev):
    """The optional paths, each timed on its full-size workload:
    causal Llama-shaped prefill with a 1024-key sliding window and ALiBi; the MQA ragged
    decode read from a paged cache (256-key pages scattered over the pool); and the
    MHA -> GQA conversion of a Llama-2-70B-shaped K projection (64 -> 8 heads)."""
    import numpy as np
    import torch
    import workloads as W
    import grouped_query_attention_02_amd as gqa
    from grouped_query_attention_02_amd import perfmodel
    out = {}
    reps = max(10, steps // 2)

    lc = _prefill_case(W.WORKLOADS["llama_causal_prefill"], dev)
    w, window, slopes = lc["w"], 1024, torch.tensor(_alibi_slopes(32), device=dev)
    flops = perfmodel.prefill_flops(w.B, w.S, w.Hq, w.d, True, None, window)

    def run_win(c):
        gqa.prefill(c["q"], c["k"], c["v"], causal=True, softmax_scale=w.softmax_scale,
                    window=window, alibi_slopes=slopes, out=c["out"])
    ms = _time_loop(run_win, lc, reps, 3)
    out["llama_causal_prefill_window1024_alibi"] = {
        "tflops": flops / (statistics.mean(ms) * 1e-3) / 1e12,
        "frac_mfma_peak": flops / (statistics.mean(ms) * 1e-3) / 1e12 / perfmodel.PEAK_BF16_TFLOPS,
        "ms_mean": statistics.mean(ms), "flops": flops, "window": window}
    del lc
    torch.cuda.empty_cache()

    dc = _decode_case(W.WORKLOADS["mqa_ragged_decode"], dev)
    wd, page = dc["w"], 256
    mb = wd.max_len // page
    n_pages = wd.B * mb + 7
    perm = np.random.default_rng(12).permutation(n_pages)
    table = torch.tensor(perm[: wd.B * mb].reshape(wd.B, mb), dtype=torch.int32, device=dev)
    def to_pool(c):
        pool = torch.zeros((n_pages, wd.Hkv, page, wd.d), dtype=c.dtype, device=dev)
        pool[table.view(-1).long()] = c.view(wd.B, wd.Hkv, mb, page, wd.d) \
            .permute(0, 2, 1, 3, 4).reshape(wd.B * mb, wd.Hkv, page, wd.d)
        return pool
    dc["kp"], dc["vp"] = to_pool(dc["kc"]), to_pool(dc["vc"])
    del dc["kc"], dc["vc"]

    def run_paged(c):
        gqa.decode(c["q"], c["kp"], c["vp"], c["lens"], softmax_scale=wd.softmax_scale,
                   block_table=table, page_size=page, workspace=c["ws"], out=c["out"])
    ms = _time_loop(run_paged, dc, reps, 3)
    out["mqa_ragged_decode_paged256"] = {
        "gbps": dc["bytes"] / (statistics.mean(ms) * 1e-3) / 1e9,
        "frac_hbm_peak": dc["bytes"] / (statistics.mean(ms) * 1e-3) / 1e9 / perfmodel.PEAK_HBM_GBPS,
        "ms_mean": statistics.mean(ms), "bytes": dc["bytes"], "page_size": page}
    del dc
    torch.cuda.empty_cache()

    H, G, per_head = 64, 8, 128 * 8192
    g = torch.Generator(device=dev).manual_seed(70)
    wk = (torch.randn((H, per_head), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    pooled = torch.empty((G, per_head), dtype=torch.bfloat16, device=dev)
    ms = _time_loop(lambda c: gqa.mean_pool_heads(wk, G, out=pooled), None, reps, 3)
    nb = perfmodel.mean_pool_bytes(H, G, per_head, 2)
    out["mean_pool_llama70b_kproj"] = {
        "gbps": nb / (statistics.mean(ms) * 1e-3) / 1e9,
        "frac_hbm_peak": nb / (statistics.mean(ms) * 1e-3) / 1e9 / perfmodel.PEAK_HBM_GBPS,
        "ms_mean": statistics.mean(ms), "bytes": nb}
    return out


def _cpu_baseline(pc, target_s: float):
    """The fp64 oracle, as it stands, on random rows of the prefill workload: a 2000-row pilot
    sizes the sample to about target_s seconds, run in chunks of at most one workload's worth
    of rows (drawn with replacement, so a fast host may see each row more than once)."""
    import numpy as np
    import oracle
    w = pc["w"]
    x = pc["host"]
    lens = x["seqlens"].numpy() if x["seqlens"] is not None else np.full(w.B, w.S)
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

    def run(rows):
        t = time.perf_counter()
        oracle.prefill_rows(x["q"], x["k"], x["v"], rows, scale=w.softmax_scale,
                            causal=w.causal, seqlens=x["seqlens"])
        return time.perf_counter() - t

    pilot = sample(2000)
    rate = flops(pilot) / max(run(pilot), 1e-6)
    total_rows = w.B * w.S * w.Hq
    goal = int(max(2000, rate * target_s / (4 * w.d * float(np.mean(lens)))))
    done, fl, dt = 0, 0.0, 0.0
    while done < goal:
        rows = sample(min(total_rows, goal - done))
        dt += run(rows)
        fl += flops(rows)
        done += len(rows)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"{done} random (b, head, query) rows of {w.name}, drawn with replacement "
                      f"({done / total_rows:.2f} x its {total_rows} rows), fp64, {dt:.1f} s wall"}


def _only(what, steps, dev):
    """Run one piece of work `steps` times (for rocprofv3 runs) and exit."""
    import torch
    import workloads as W
    if what in ("prefill", "prefill_causal"):
        name = "bert_base_prefill" if what == "prefill" else "llama_causal_prefill"
        c = _prefill_case(W.WORKLOADS[name], dev)
        fn = lambda: _run_prefill(c)
    elif what == "decode":
        c = _decode_case(W.WORKLOADS["mqa_ragged_decode"], dev)
        fn = lambda: _run_decode(c)
    else:  # a plain device copy of known size, to calibrate the HBM byte counters
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        fn = lambda: dst.copy_(src)
        print(f"[bench] copy of {n} bytes per launch", file=sys.stderr)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    print(f"[bench] ran {what} x{steps}", file=sys.stderr, flush=True)
    return 0


def _csv_rows(d, name):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", name), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _summarize_kernels(d):
    """Per-kernel call count and mean/min duration (us) from rocprofv3 kernel traces."""
    rows = _csv_rows(d, "*kernel_trace.csv")
    acc = {}
    for r in rows:
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        acc.setdefault(r["Kernel_Name"], []).append(dur)
    for name, v in sorted(acc.items(), key=lambda kv: -sum(kv[1])):
        print(f"{len(v):5d} calls  mean {statistics.mean(v):10.2f} us  min {min(v):10.2f} us"
              f"  total {sum(v):11.1f} us  {name[:110]}")
    return 0


def _summarize_pmc(d):
    """Per-kernel mean of each counter (summed over its instances) from rocprofv3 --pmc."""
    rows = _csv_rows(d, "*counter_collection.csv")
    per = {}
    for r in rows:
        key = (r["Kernel_Name"], r["Counter_Name"], r["Dispatch_Id"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    agg = {}
    for (kname, cname, _), v in per.items():
        agg.setdefault((kname, cname), []).append(v)
    for (kname, cname), v in sorted(agg.items()):
        print(f"{cname:28s} mean {statistics.mean(v):14.6g}  n={len(v):3d}  {kname[:100]}")
    return 0


def _recorded_traffic(summary_name, source_name):
    """HBM bytes per launch recorded in profiles/<summary_name>, or None when the kernel
    source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", summary_name)
    src = os.path.join(ROOT, "grouped_query_attention_02_amd", "csrc", source_name)
    if not (os.path.exists(path) and os.path.exists(src)):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(("#", " ", "`")):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    with open(src, "rb") as fh:
        digest = hashlib.sha256(fh.read()).hexdigest()
    if fields.get("kernel_source_sha256") != digest:
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def _achievable(dev) -> dict:
    """Achievable peaks on this GPU from libgqa_probes.so: back-to-back bf16 32x32x16 MFMAs
    (four independent chains per wave, four waves per SIMD) and a read of a 4 GiB buffer
    (16 x the last-level cache), each the best of several timed launches."""
    import ctypes
    import torch
    from grouped_query_attention_02_amd import build as gbuild
    if not os.path.exists(gbuild.PROBES_LIB):
        raise RuntimeError(f"{gbuild.PROBES_LIB} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(gbuild.PROBES_LIB, mode=ctypes.RTLD_LOCAL)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.gqa_probe_mfma_flops.argtypes = [i32, i32]
    lib.gqa_probe_mfma_flops.restype = ctypes.c_double
    lib.gqa_probe_mfma_bf16.argtypes = [i32, i32, vp, vp]
    lib.gqa_probe_read.argtypes = [vp, ctypes.c_size_t, vp, i32, vp]
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
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.zero_()
    rblocks = 16 * cus
    rout = torch.empty(rblocks * 256, dtype=torch.int32, device=dev)

    def rd():
        return lib.gqa_probe_read(buf.data_ptr(), nbytes // 16, rout.data_ptr(), rblocks, stream)

    gbps = 0.0
    for per_cu in (4, 8, 16):  # the best of a few grid sizes
        rblocks = per_cu * cus
        best(rd, 2)
        gbps = max(gbps, nbytes / (best(rd, 5) * 1e-3) / 1e9)
    del buf, rout, out
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(tflops, 1), "hbm_read_gbps": round(gbps, 1),
            "source": "probes/probes.hip: back-to-back bf16 MFMA; 4 GiB streaming read"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10000,
                    help="untimed steps before timing; the default (~2 s of work) lets the "
                         "GPU clocks settle at their sustained level")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the extra workloads")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the achievable-peak microbenchmarks (achievable = null)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--only", choices=["prefill", "prefill_causal", "decode", "copy"],
                    help="profiling run: execute just this work --steps times and exit")
    ap.add_argument("--summarize-kernels", metavar="DIR",
                    help="print per-kernel mean durations from rocprofv3 --kernel-trace CSV output")
    ap.add_argument("--summarize-pmc", metavar="DIR",
                    help="print per-kernel mean counter values from rocprofv3 --pmc CSV output")
    args = ap.parse_args(argv)

    if args.summarize_kernels:
        return _summarize_kernels(args.summarize_kernels)
    if args.summarize_pmc:
        return _summarize_pmc(args.summarize_pmc)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    import workloads as W
    import grouped_query_attention_02_amd as gqa
    from grouped_query_attention_02_amd import perfmodel

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    gqa.load()
    dev = torch.device("cuda:0")
    print(f"[bench] device {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)

    if args.only:
        return _only(args.only, args.steps, dev)

    pc = _prefill_case(W.WORKLOADS["bert_base_prefill"], dev)
    dc = _decode_case(W.WORKLOADS["mqa_ragged_decode"], dev)
    print(f"[bench] inputs ready: prefill {pc['flops'] / 1e9:.2f} GFLOP, decode "
          f"{dc['bytes'] / 1e6:.2f} MB (sum of cache lengths {sum(dc['lens_host'])})",
          file=sys.stderr, flush=True)

    # warmup steps (untimed)
    for _ in range(args.warmup):
        _run_prefill(pc)
        _run_decode(dc)
    torch.cuda.synchronize()

    pev, dev_ev = _events(args.steps), _events(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        pev[i][0].record()
        _run_prefill(pc)
        pev[i][1].record()
        dev_ev[i][0].record()
        _run_decode(dc)
        dev_ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    p_ms, d_ms = _ms(pev), _ms(dev_ev)
    print(f"[bench] timed {args.steps} steps in {wall:.3f} s", file=sys.stderr, flush=True)

    p_avg = statistics.mean(p_ms)
    d_avg = statistics.mean(d_ms)
    p_tflops = pc["flops"] / (p_avg * 1e-3) / 1e12
    d_gbps = dc["bytes"] / (d_avg * 1e-3) / 1e9

    also = {}
    if not args.no_extra:
        lc = _prefill_case(W.WORKLOADS["llama_causal_prefill"], dev)
        ms = _time_loop(_run_prefill, lc, max(10, args.steps // 2), 3)
        also["llama_causal_prefill"] = {
            "tflops": lc["flops"] / (statistics.mean(ms) * 1e-3) / 1e12,
            "frac_mfma_peak": lc["flops"] / (statistics.mean(ms) * 1e-3) / 1e12
            / perfmodel.PEAK_BF16_TFLOPS,
            "ms_mean": statistics.mean(ms), "ms_min": min(ms), "flops": lc["flops"]}
        del lc
        torch.cuda.empty_cache()
        gc = _decode_case(W.WORKLOADS["gqa_decode_8k"], dev)
        ms = _time_loop(_run_decode, gc, max(10, args.steps // 2), 3)
        also["gqa_decode_8k"] = {
            "gbps": gc["bytes"] / (statistics.mean(ms) * 1e-3) / 1e9,
            "frac_hbm_peak": gc["bytes"] / (statistics.mean(ms) * 1e-3) / 1e9
            / perfmodel.PEAK_HBM_GBPS,
            "ms_mean": statistics.mean(ms), "ms_min": min(ms), "bytes": gc["bytes"]}
        del gc
        torch.cuda.empty_cache()
        tc = _prefill_case(W.WORKLOADS["tiny_f32_prefill"], dev)
        ms = _time_loop(_run_prefill, tc, 20, 3)
        # one call at a time is bound by the host (binding + launch); queued behind a long
        # prefill the same calls show the device time per call
        hold = _prefill_case(W.WORKLOADS["llama_causal_prefill"], dev)
        qd = statistics.median(_time_queued(_run_prefill, tc, 20, _run_prefill, hold)
                               for _ in range(5))
        del hold
        also["tiny_f32_prefill"] = {"us_per_call": statistics.mean(ms) * 1e3,
                                    "us_device_queued": qd * 1e3,
                                    "tflops_device": tc["flops"] / (qd * 1e-3) / 1e12}
        also.update(_extended_rows(args.steps, dev))

    ach = None
    if not args.no_probes:
        ach = _achievable(dev)
        print(f"[bench] achievable: {ach['mfma_bf16_tflops']} TFLOP/s bf16 MFMA, "
              f"{ach['hbm_read_gbps']} GB/s HBM read", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        cpu = _cpu_baseline(pc, args.cpu_seconds)

    wp = pc["w"]
    wd = dc["w"]
    line = {
        "metric": METRIC,
        "value": round(p_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round((p_avg + d_avg), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16 inputs, uniform random lengths",
        "config": {
            "workload": "bert_base_prefill + mqa_ragged_decode",
            "prefill": {"name": wp.name, "B": wp.B, "S": wp.S, "Hq": wp.Hq, "Hkv": wp.Hkv,
                        "d": wp.d, "causal": wp.causal, "key_lengths": list(wp.lens),
                        "seed": wp.seed, "sum_key_len": sum(pc["lens_host"])},
            "decode": {"name": wd.name, "B": wd.B, "Hq": wd.Hq, "Hkv": wd.Hkv, "d": wd.d,
                       "max_len": wd.max_len, "cache_lengths": list(wd.lens), "seed": wd.seed,
                       "sum_cache_len": sum(dc["lens_host"]),
                       "split_workgroups": gqa.decode_num_workgroups(wd.B, wd.Hq, wd.Hkv,
                                                                     wd.max_len, 0)},
        },
        "roofline": {
            "bound": "mfma", "achieved": round(p_tflops, 3),
            "peak": perfmodel.PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(p_tflops / perfmodel.PEAK_BF16_TFLOPS, 4),
            "traffic": _recorded_traffic("prefill_bert_base_traffic.md", "prefill_bf16.hip"),
            "kernel": "prefill_bf16_kernel<64, false, false, false>",
            "launch_us_mean": round(p_avg * 1e3, 2), "flops_per_launch": pc["flops"],
            "frac_of_achievable": round(p_tflops / ach["mfma_bf16_tflops"], 4) if ach else None,
        },
        "decode": {
            "gbps": round(d_gbps, 2), "frac_hbm_peak": round(d_gbps / perfmodel.PEAK_HBM_GBPS, 4),
            "peak_gbps": perfmodel.PEAK_HBM_GBPS, "call_us_mean": round(d_avg * 1e3, 2),
            "call_us_min": round(min(d_ms) * 1e3, 2), "bytes_per_call": dc["bytes"],
            "frac_of_achievable_read": round(d_gbps / ach["hbm_read_gbps"], 4) if ach else None,
            "kernels": "decode_split_kernel<128, false, false> + decode_combine_kernel<128>",
        },
        "cpu_baseline": cpu,
        "achievable": ach,
        "also": also,
        "context": "pages: ~980 tokens/s for a whole BERT-base model on A100 at seq 1024, "
                   "batch 32, precision unstated; not comparable to an attention-kernel rate",
        "host": platform.node(),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
