"""Paged-KV decode benchmark: one JSON line on stdout.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--splits S] [--no-cpu-baseline]

A step is one decode call (run + reduce) over one seeded synthetic batch of
the workload, with every input already resident in HBM. The default
workload is the long-context bf16 GQA decode (batch 4, 64 q / 8 kv heads,
D 128, 64-token pages, contexts uniform in [32768, 131072]). Its 1.0 GB of
KV is several times the last-level cache, so back-to-back calls stream from
HBM. Smaller workloads rotate through enough input copies to exceed 1 GiB.

value = algorithmic KV bytes per call / time per call (GB/s, 1e9 B/s), the
call (run + reduce) replayed from a captured HIP graph, which is how a decode
step runs in serving (graph-first timing is what the pages' own review asks
for); the eager per-call rate is reported beside it.
roofline.achieved = the same bytes / the decode kernel's own average
duration, from HIP events recorded around each eager launch on the stream it
runs on.
read_ceiling = a plain streaming read of the same K/V page pools on the same
box (libpd_probe.so, best of several launch shapes): the achievable read
rate the kernel's is compared with (roofline.frac_of_read_ceiling).
cpu_baseline = the fp64 CPU oracle timed over whole calls of the same batch
on the host's cores (a process pool over the (sequence, kv head) units, one
BLAS thread per process, at most 16), with the CPU model and core count.
secondary = the fp8-KV workload (batch 64, 16 q / 1 kv head, D 256, e4m3fn
pages with per-token scales) timed the same way after the headline one.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "paged-decode µs/call and achieved HBM GB/s (% of peak), bf16 GQA + fp8 KV"


def kernel_source_hash() -> str:
    """Hash of the decode sources with comments and whitespace removed, so a
    traffic record stays valid across edits that change no code."""
    h = hashlib.sha256()
    for name in ("decode_kernels.hip", "paged_decode_abi.cpp", "decode_launch.h"):
        with open(os.path.join(ROOT, "paged_kv_attention_14_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def read_ceiling(dev, steps: int, warmup: int) -> dict:
    """Time a plain streaming read of the same K/V page pools on the same box:
    the achievable-bandwidth context for the decode kernel.

    Each step reads every pool tensor of one input copy (copies rotate, as in
    the decode timing) with the probe in libpd_probe.so: 16 contiguous bytes
    per lane in workgroup-contiguous chunks, grid-stride; the best of fifteen
    launch shapes (grid size x loads in flight per lane) is reported.
    """
    import ctypes

    import torch
    from paged_kv_attention_14_amd import build as _build

    if not os.path.exists(_build.PROBE_PATH):
        raise ImportError(f"{_build.PROBE_PATH} is missing: run the build first")
    lib = ctypes.CDLL(_build.PROBE_PATH)
    fn = lib.pd_probe_stream_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p]
    shapes = [(g, u) for u in (1, 2, 4) for g in (512, 1024, 2048, 4096, 8192)]
    grids = [g for g, _ in shapes]
    sink = torch.zeros(max(grids), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    tensors = [[d["k_pages"], d["v_pages"]] for d in dev]
    nbytes = sum(t.numel() * t.element_size() for t in tensors[0])

    def one(i, grid, unroll):
        for t in tensors[i % len(tensors)]:
            rc = fn(t.data_ptr(), t.numel() * t.element_size(), sink.data_ptr(), grid, unroll,
                    stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"stream-read probe launch failed (hipError {rc})")

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    best = None
    for grid, unroll in shapes:
        for i in range(warmup):
            one(i, grid, unroll)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(steps):
            one(i, grid, unroll)
        end.record(stream)
        torch.cuda.synchronize()
        t = start.elapsed_time(end) * 1e3 / steps
        if best is None or t < best[0]:
            best = (t, grid, unroll)
    us, grid, unroll = best
    return {"GBps": round(nbytes / (us * 1e-6) / 1e9, 2), "us": round(us, 2),
            "bytes": nbytes,
            "grid": grid, "loads_per_lane": unroll,
            "what": "plain coalesced read (16 B per lane, workgroup-contiguous chunks, "
                    "grid-stride) of the same K/V page pools, HIP events, input copies "
                    "rotated, best of 512-8192 workgroups x 1, 2 or 4 loads in flight per lane"}


def measured_traffic(workload: str, splits: int):
    """HBM bytes per decode launch from the committed counter summary, or None.

    The summary records the kernel-source hash it was taken with; once the
    kernels change it no longer applies and traffic is reported as null.
    """
    path = os.path.join(ROOT, "profiles", f"traffic_decode_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash() or rec.get("num_splits") != splits:
        return None
    return rec.get("hbm_bytes_per_launch")


def _rocprof_rows(directory: str, suffix: str):
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    return rows


def ingest_pmc(fetch_dir: str, write_dir: str, workload: str, splits: int, command: str) -> dict:
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) into HBM bytes per launch.

    Each run also holds one device copy of a known size (--copy-calibration-mib);
    the counter value of that copy gives the counter-to-bytes factor.
    """
    out = {"workload": workload, "num_splits": splits, "kernel_source_hash": kernel_source_hash(),
           "command": command}
    for name, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = [r for r in _rocprof_rows(d, "counter_collection.csv") if r["Counter_Name"] == counter]
        dec = [float(r["Counter_Value"]) for r in rows if "paged_decode_split_kernel" in r["Kernel_Name"]]
        cpy = [r for r in rows if "copyBuffer" in r["Kernel_Name"]]
        big = max(cpy, key=lambda r: float(r["Counter_Value"]))
        logs = glob_json_lines(d)
        known = logs.get("copy_calibration_bytes")
        factor = known / (float(big["Counter_Value"]) * 1024.0)
        out[name] = {"counter": counter, "decode_dispatches": len(dec),
                     "decode_kib_mean": sum(dec) / len(dec), "copy_bytes": known,
                     "copy_kib": float(big["Counter_Value"]), "bytes_per_kib_unit": factor,
                     "decode_bytes_per_launch": sum(dec) / len(dec) * 1024.0 * factor}
    out["kv_bytes_per_launch"] = logs.get("config", {}).get("kv_bytes_per_call")
    out["hbm_bytes_per_launch"] = round(out["fetch"]["decode_bytes_per_launch"] +
                                        out["write"]["decode_bytes_per_launch"])
    return out


def glob_json_lines(directory: str) -> dict:
    """The bench JSON line a counter run printed into <directory>/bench.json."""
    path = os.path.join(directory, "bench.json")
    with open(path) as f:
        lines = [l for l in f.read().splitlines() if l.startswith("{")]
    return json.loads(lines[-1])


def summarize_trace(directory: str, command: str) -> str:
    """Markdown summary of a rocprofv3 --kernel-trace --stats run."""
    stats = _rocprof_rows(directory, "kernel_stats.csv")
    lines = ["# rocprofv3 kernel trace", "", "Command (run from the repository root on an MI355X):",
             "", "```", command, "```", "",
             "| kernel | calls | average us | min us | max us | share % |",
             "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
    return "\n".join(lines) + "\n"


# The oracle's inputs for the worker processes of cpu_baseline. Set before the
# pool forks (and before the GPU is touched), so workers read them
# copy-on-write instead of receiving them through pickles.
_ORACLE_INPUT = None


def _limit_blas() -> None:
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:  # pragma: no cover
        pass


def _oracle_unit(unit) -> int:
    """The unmodified oracle on one (sequence b, kv head h) unit: the query
    heads of h against pools viewed at kv head h. Returns its KV bytes."""
    import oracle
    b, h = unit
    d = _ORACLE_INPUT
    g = d["g"]
    head = d["kv_layout"] == "head"
    pick = (lambda t: t[:, h:h + 1]) if head else (lambda t: t[:, :, h:h + 1])
    oracle.paged_attention(
        d["q"][b:b + 1, :, h * g:(h + 1) * g], pick(d["kp"]), pick(d["vp"]),
        d["bt"][b:b + 1], d["ctx"][b:b + 1], d["scale"],
        k_scale=None if d["ks"] is None else pick(d["ks"]),
        v_scale=None if d["vs"] is None else pick(d["vs"]),
        scratch_k=None if d["sk"] is None else d["sk"][b:b + 1, :, h:h + 1],
        scratch_v=None if d["sv"] is None else d["sv"][b:b + 1, :, h:h + 1],
        scratch_mask=d["scratch_mask"], kv_layout=d["kv_layout"], kv_format=d["kv_format"])
    return int(d["ctx"][b]) * d["per_token_head"] + d["scratch_head_bytes"]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(case, budget_s: float = 20.0, min_s: float = 8.0, max_workers: int = 16):
    """Time the fp64 CPU oracle on the host's cores over whole decode calls.

    The (sequence, kv head) units of one call are independent, so a process
    pool (one BLAS thread each) runs the unmodified oracle on one unit per
    task, longest context first; whole calls are repeated until at least
    min_s seconds of wall time (at most about budget_s). Workers = the cores
    in the process's affinity mask, capped at max_workers (the CPU share of
    one GPU on a shared host). Must run before the GPU is initialised: the
    pool forks.
    """
    global _ORACLE_INPUT
    import multiprocessing

    import numpy as np

    fp8 = case.kv_dtype == "fp8"
    elem = 1 if fp8 else 2
    _ORACLE_INPUT = dict(
        q=case.q.double().numpy(),
        kp=case.k_pages.numpy() if fp8 else case.k_pages.float().numpy(),
        vp=case.v_pages.numpy() if fp8 else case.v_pages.float().numpy(),
        ks=None if case.k_scale is None else case.k_scale.float().numpy(),
        vs=None if case.v_scale is None else case.v_scale.float().numpy(),
        sk=None if case.scratch_k is None else case.scratch_k.double().numpy(),
        sv=None if case.scratch_v is None else case.scratch_v.double().numpy(),
        bt=case.block_table.numpy(), ctx=case.context_lens.numpy().astype(np.int64),
        scale=case.scale, g=case.num_q_heads // case.num_kv_heads,
        kv_layout=case.kv_layout, scratch_mask=case.scratch_mask,
        kv_format="fp8" if fp8 else "dense",
        per_token_head=case.head_dim * 2 * elem + (2 * (2 if case.scale_dtype == "f16" else 4)
                                                    if fp8 else 0),
        scratch_head_bytes=case.scratch_tokens * case.head_dim * 2 * 2)
    ctx = _ORACLE_INPUT["ctx"]
    units = sorted(((b, h) for b in range(case.batch) for h in range(case.num_kv_heads)),
                   key=lambda u: -int(ctx[u[0]]))
    visible = len(os.sched_getaffinity(0))
    workers = max(1, min(visible, max_workers, len(units)))

    pool = multiprocessing.get_context("fork").Pool(workers, initializer=_limit_blas)
    try:
        pool.map(_oracle_unit, units[:workers], chunksize=1)   # workers up
        calls, nbytes = 0, 0
        t0 = time.perf_counter()
        while True:
            nbytes += sum(pool.map(_oracle_unit, units, chunksize=1))
            calls += 1
            wall = time.perf_counter() - t0
            if wall >= min_s or wall * (calls + 1) / calls > budget_s:
                break
        # One thread in this process, a few units, for context.
        _limit_blas()
        t0 = time.perf_counter()
        one_bytes = 0
        for u in units:
            one_bytes += _oracle_unit(u)
            if time.perf_counter() - t0 >= 2.0:
                break
        one_s = time.perf_counter() - t0
    finally:
        pool.close()
        pool.join()
        _ORACLE_INPUT = None
    return {
        "value": round(nbytes / wall / 1e9, 4),
        "unit": "GB/s",
        "cores": workers,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "cores_visible": visible,
        "us_per_call": round(wall / calls * 1e6, 1),
        "sample": f"fp64 numpy oracle, {calls} whole call(s) of the same seeded batch "
                  f"({len(units)} (sequence, kv head) units each, {nbytes / calls / 1e9:.3f} GB "
                  f"of KV per call) in {wall:.1f} s wall on a {workers}-process pool, one BLAS "
                  f"thread per process",
        "single_thread_GBps": round(one_bytes / one_s / 1e9, 4),
    }


def bench_kv_write(args) -> int:
    """Time paged_decode_write_kv on 16384 new tokens (8 kv heads, D128).

    Bytes per call = the new rows read (bf16) + the rows and scales written;
    the slots are a seeded permutation of a 1024-page pool (16-token pages).
    """
    import torch
    from paged_kv_attention_14_amd import DecodeConfig, PagedDecoder

    N, H, D, bs = 16384, 8, 128, 16
    fp8 = args.kv_write == "fp8"
    gen = torch.Generator().manual_seed(106)
    P = N // bs
    dec = PagedDecoder(DecodeConfig(num_q_heads=4 * H, num_kv_heads=H, head_dim=D,
                                    block_size=bs, kv_dtype="fp8" if fp8 else "bf16",
                                    max_batch=1, max_blocks_per_seq=1))
    k = torch.randn(N, H, D, generator=gen).to(torch.bfloat16).cuda()
    v = torch.randn(N, H, D, generator=gen).to(torch.bfloat16).cuda()
    slots = torch.randperm(P * bs, generator=gen)[:N].to(torch.int64).cuda()
    pool_dtype = torch.uint8 if fp8 else torch.bfloat16
    kp = torch.empty(P, bs, H, D, dtype=pool_dtype, device="cuda")
    vp = torch.empty_like(kp)
    ks = torch.empty(P, bs, H, device="cuda") if fp8 else None
    vs = torch.empty_like(ks) if fp8 else None
    for _ in range(args.warmup):
        dec.write_kv(k, v, slots, kp, vp, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st.record()
    for _ in range(args.steps):
        dec.write_kv(k, v, slots, kp, vp, k_scale=ks, v_scale=vs)
    en.record()
    torch.cuda.synchronize()
    ms = st.elapsed_time(en) / args.steps
    nbytes = N * H * D * 2 * 2 + N * H * D * 2 * (1 if fp8 else 2) + (N * H * 8 if fp8 else 0)
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "paged KV-cache write GB/s (read new rows + write cache)", "value": round(gbs, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "us_per_call": round(ms * 1e3, 2),
        "higher_is_better": True, "dtype": "bf16->fp8e4m3" if fp8 else "bf16",
        "data": "synthetic (seeded N(0,1) bf16 rows, permuted slots)",
        "config": {"workload": "kv_write_16k_tokens", "tokens": N, "num_kv_heads": H,
                   "head_dim": D, "block_size": bs, "bytes_per_call": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)},
    }), flush=True)
    dec.close()
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long_context_splitk")
    ap.add_argument("--splits", type=int, default=0, help="0 = the library's choice")
    ap.add_argument("--scratch-mask", choices=("none", "causal"), default="none",
                    help="visibility of scratch tokens (workloads with scratch tokens)")
    ap.add_argument("--kv-layout", choices=("token", "head"), default="token",
                    help="page layout: [P, bs, Hkv, D] (token) or [P, Hkv, bs, D] (head)")
    ap.add_argument("--scale-dtype", choices=("f32", "f16"), default="f32",
                    help="storage type of the fp8 scales (fp8 workloads)")
    ap.add_argument("--timing", choices=("graph", "eager"), default="graph",
                    help="how the headline per-call time is measured")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--secondary", default="fp8_mqa_d256",
                    help="workload timed after the headline one and reported in the "
                         "line's 'secondary' list ('none' to skip)")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the streaming-read ceiling measured after the decode timing")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB so a "
                         "counter run can scale FETCH_SIZE/WRITE_SIZE to bytes")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_decode_<workload>.json from two counter runs "
                         "(no GPU work)")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="print a markdown summary of a rocprofv3 kernel-trace run (no GPU work)")
    ap.add_argument("--command", default="", help="the command recorded in a summary")
    ap.add_argument("--kv-write", choices=("fp8", "bf16"), default=None,
                    help="measure the KV-cache write step instead of decode: 16384 new "
                         "tokens x 8 kv heads x D128 (bf16 in) into a shuffled page pool")
    args = ap.parse_args(argv)

    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.command), end="")
        return 0
    if args.ingest_pmc:
        rec = ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], args.workload, args.splits,
                         args.command)
        path = os.path.join(ROOT, "profiles", f"traffic_decode_{args.workload}.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec, indent=1))
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the decode path is single-GPU; sharding is described, not run)",
              file=sys.stderr, flush=True)
        return 2

    import torch
    from workloads import CONFIGS, VARIANT_CONFIGS, make_config_case

    if args.kv_write:
        return bench_kv_write(args)

    cfg = CONFIGS[args.workload] if args.workload in CONFIGS else VARIANT_CONFIGS[args.workload]
    t0 = time.time()
    case = make_config_case(cfg, kv_layout=args.kv_layout, scale_dtype=args.scale_dtype)
    case.scratch_mask = args.scratch_mask
    print(f"[bench] generated {cfg.name} in {time.time() - t0:.1f}s, "
          f"kv_bytes={case.kv_bytes()}", file=sys.stderr, flush=True)
    # The CPU leg forks a process pool, so it runs before the GPU is touched.
    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        cpu = cpu_baseline(case, args.cpu_budget)
        print(f"[bench] cpu baseline {cpu['value']} GB/s on {cpu['cores']} cores "
              f"in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    r = time_decode(case, args, args.splits, args.scratch_mask, args.kv_layout,
                    not args.no_read_ceiling, args.copy_calibration_mib)
    kv_bytes = case.kv_bytes()
    traffic = measured_traffic(cfg.name, args.splits)
    line = {
        "metric": METRIC,
        "value": round(r["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "us_per_call": round(r["ms_per_step"] * 1e3, 2),
        "timing": r["timing"],
        "call_us_p10_p50_p90": r["call_pct"],
        "eager_us_per_call": round(r["eager_ms"] * 1e3, 2),
        "eager_GBps": round(kv_bytes / (r["eager_ms"] * 1e-3) / 1e9, 2),
        "pct_of_peak": round(100.0 * r["value"] / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3+bf16" if case.kv_dtype == "fp8" else case.q_dtype,
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, shuffled page pool)",
        "config": {
            "workload": cfg.name,
            "description": cfg.description,
            "batch": case.batch, "q_tokens": case.q_tokens,
            "num_q_heads": case.num_q_heads, "num_kv_heads": case.num_kv_heads,
            "head_dim": case.head_dim, "block_size": case.block_size,
            "context_tokens": int(case.context_lens.sum()),
            "scratch_tokens": case.scratch_tokens, "scratch_mask": args.scratch_mask,
            "kv_layout": args.kv_layout, "scale_dtype": case.scale_dtype,
            "num_splits": r["S"],
            "splits_chosen_by": "library" if args.splits == 0 else "caller",
            "kv_bytes_per_call": kv_bytes, "input_copies_rotated": r["reps"],
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(r["achieved"], 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(r["achieved"] / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "kernel": "paged_decode_split_kernel",
            "avg_kernel_us": round(r["avg_decode_ms"] * 1e3, 2),
            "kernel_us_p10_p50_p90": r["kernel_pct"],
            "bytes_per_launch": kv_bytes,
        },
        "wall_s_timed_region": round(r["wall"], 4),
    }
    if "read_ceiling" in r:
        line["read_ceiling"] = r["read_ceiling"]
        line["roofline"]["frac_of_read_ceiling"] = round(
            r["achieved"] / r["read_ceiling"]["GBps"], 4)
    if "copy_calibration_bytes" in r:
        line["copy_calibration_bytes"] = r["copy_calibration_bytes"]
    if cpu is not None:
        line["cpu_baseline"] = cpu
    del case, r
    torch.cuda.empty_cache()

    # The fp8-KV workload beside the headline (the metric names both), timed
    # the same way: its own line in the same JSON object.
    sec = [] if args.secondary == "none" or args.secondary == cfg.name else [args.secondary]
    line["secondary"] = []
    for name in sec:
        scfg = CONFIGS[name] if name in CONFIGS else VARIANT_CONFIGS[name]
        scase = make_config_case(scfg)
        sr = time_decode(scase, args, 0, "none", "token", not args.no_read_ceiling, 0)
        sb = scase.kv_bytes()
        block = {
            "workload": scfg.name, "description": scfg.description,
            "dtype": "fp8e4m3+bf16" if scase.kv_dtype == "fp8" else scase.q_dtype,
            "num_splits": sr["S"], "splits_chosen_by": "library",
            "kv_bytes_per_call": sb, "input_copies_rotated": sr["reps"],
            "us_per_call": round(sr["ms_per_step"] * 1e3, 2),
            "GBps": round(sr["value"], 2),
            "pct_of_peak": round(100.0 * sr["value"] / PEAK_HBM_GBS, 2),
            "timing": sr["timing"],
            "call_us_p10_p50_p90": sr["call_pct"],
            "eager_us_per_call": round(sr["eager_ms"] * 1e3, 2),
            "avg_kernel_us": round(sr["avg_decode_ms"] * 1e3, 2),
            "kernel_us_p10_p50_p90": sr["kernel_pct"],
            "kernel_GBps": round(sr["achieved"], 2),
            "kernel_frac": round(sr["achieved"] / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(scfg.name, 0),
        }
        if "read_ceiling" in sr:
            block["read_ceiling_GBps"] = sr["read_ceiling"]["GBps"]
            block["kernel_frac_of_read_ceiling"] = round(
                sr["achieved"] / sr["read_ceiling"]["GBps"], 4)
        line["secondary"].append(block)
        del scase, sr
        torch.cuda.empty_cache()
    print(json.dumps(line), flush=True)
    return 0


def time_decode(case, args, splits: int, scratch_mask: str, kv_layout: str,
                with_ceiling: bool, copy_calibration_mib: int) -> dict:
    """Time run + reduce on one workload: eager launches with HIP events around
    each decode kernel, then graph replays; input copies rotate until at
    least 1 GiB of inputs is in use, so no call reads another's data from a
    cache."""
    import torch
    from paged_kv_attention_14_amd import DecodeConfig, PagedDecoder, _lib

    kv_bytes = case.kv_bytes()
    reps = max(1, -(-(1 << 30) // kv_bytes))  # rotate copies until >= 1 GiB
    dev = []
    for r in range(reps):
        dev.append({k: (None if getattr(case, k) is None else getattr(case, k).cuda())
                    for k in ("q", "k_pages", "v_pages", "block_table", "context_lens",
                              "k_scale", "v_scale", "scratch_k", "scratch_v")})
    dec = PagedDecoder(DecodeConfig(
        num_q_heads=case.num_q_heads, num_kv_heads=case.num_kv_heads,
        head_dim=case.head_dim, block_size=case.block_size, q_tokens=case.q_tokens,
        scratch_tokens=case.scratch_tokens, q_dtype=case.q_dtype, kv_dtype=case.kv_dtype,
        max_batch=case.batch, max_blocks_per_seq=case.table_width,
        max_num_splits=max(64, splits), scratch_mask=scratch_mask,
        kv_layout=kv_layout, scale_dtype=case.scale_dtype))
    S = dec.num_splits(case.batch, splits)
    ws = dec.alloc_workspace(case.batch, splits)
    outs = [torch.empty_like(d["q"]) for d in dev]
    lses = [torch.empty(d["q"].shape[:3], dtype=torch.float32, device="cuda") for d in dev]
    cargs = [dec.make_args(d["q"], d["k_pages"], d["v_pages"], d["block_table"],
                           d["context_lens"], outs[i], softmax_scale=case.scale,
                           lse=lses[i], num_splits=splits, k_scale=d["k_scale"],
                           v_scale=d["v_scale"], scratch_k=d["scratch_k"],
                           scratch_v=d["scratch_v"]) for i, d in enumerate(dev)]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream  # eager launches go to torch's current stream
    wsp = 0 if ws is None else ws.data_ptr()
    wsn = 0 if ws is None else ws.numel()

    def step(i, sp, ev_mid=None):
        a = cargs[i % reps]
        _lib.check(_lib.paged_decode_run(dec.handle, a, wsp, wsn, sp))
        if ev_mid is not None:
            ev_mid.record(torch.cuda.current_stream())
        _lib.check(_lib.paged_decode_reduce(dec.handle, a, wsp, wsn, sp))

    for i in range(args.warmup):
        step(i, sp)
    torch.cuda.synchronize()
    K = args.steps

    # Eager pass: per-launch events around the decode kernel (roofline) and
    # the eager per-call time.
    ev_before = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev_mid = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        ev_before[i].record(stream)
        step(i, sp, ev_mid[i])
    end.record(stream)
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - wall0
    eager_ms = start.elapsed_time(end) / K
    decode_ms = [ev_before[i].elapsed_time(ev_mid[i]) for i in range(K)]
    avg_decode_ms = sum(decode_ms) / K
    srt = sorted(decode_ms)
    pct = [srt[min(K - 1, int(q * (K - 1) + 0.5))] * 1e3 for q in (0.1, 0.5, 0.9)]

    # Graph pass: one captured graph per input copy, replayed K times.
    graph_ms = None
    wall_graph = None
    call_pct = None
    if args.timing == "graph":
        graphs = []
        for r in range(reps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(r, torch.cuda.current_stream().cuda_stream)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % reps].replay()
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        start.record(stream)
        for i in range(K):
            graphs[i % reps].replay()
        end.record(stream)
        torch.cuda.synchronize()
        wall_graph = time.perf_counter() - wall0
        graph_ms = start.elapsed_time(end) / K
        # Spread of single calls, from a separate pass with an event between
        # replays (which adds a few µs per call, so the mean above comes from
        # the undisturbed pass).
        ev_rep = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        ev_rep[0].record(stream)
        for i in range(K):
            graphs[i % reps].replay()
            ev_rep[i + 1].record(stream)
        torch.cuda.synchronize()
        rep_ms = sorted(ev_rep[i].elapsed_time(ev_rep[i + 1]) for i in range(K))
        call_pct = [rep_ms[min(K - 1, int(q * (K - 1) + 0.5))] * 1e3 for q in (0.1, 0.5, 0.9)]
        del graphs

    ms_per_step = graph_ms if graph_ms is not None else eager_ms
    out = {
        "S": S, "reps": reps, "ms_per_step": ms_per_step, "eager_ms": eager_ms,
        "avg_decode_ms": avg_decode_ms,
        "kernel_pct": [round(x, 2) for x in pct],
        "call_pct": None if call_pct is None else [round(x, 2) for x in call_pct],
        "timing": "hip graph replay of run + reduce" if graph_ms is not None else "eager launches",
        "wall": wall_graph if wall_graph is not None else wall_eager,
        "value": kv_bytes / (ms_per_step * 1e-3) / 1e9,
        "achieved": kv_bytes / (avg_decode_ms * 1e-3) / 1e9,
    }
    if with_ceiling:
        out["read_ceiling"] = read_ceiling(dev, K, args.warmup)
    if copy_calibration_mib:
        n = copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = n
        del src, dst
    dec.close()
    return out


if __name__ == "__main__":
    sys.exit(main())
