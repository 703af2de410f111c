"""Benchmark of the fused KV-cache write epilog on one MI355X.

A step is one kvepi_run over the whole workload: 262144 bf16 token rows of
d = 576, RMSNorm over the 512 nope columns, interleaved RoPE over the last 64,
group-64 FP8 E4M3 quantisation with bf16 scales, scattered as 672-byte rows
into a paged cache [2048, 128, 1, 672] whose block stride is 1.25x the dense
one, 3% of the tokens skipped.  Inputs are seeded synthetic data resident in
HBM before timing starts.

Prints one JSON line: tokens/s (T / kernel time); the roofline of the
epilog kernel (algorithmic bytes per launch / mean launch time, against the
8 TB/s HBM peak, with the measured HBM bytes when they were taken on the
current kernel code); a plain device copy timed in the same run; single
launches after a cache scrub ("cold"); and the CPU oracle timed on one host
core as a reported baseline.  --config N selects the other epilog workloads
and --drq NAME the dequant -> RoPE -> int8 operator's.
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

import numpy as np  # noqa: E402

import kvgen  # noqa: E402

HBM_PEAK_GBPS = 8000.0
METRIC = "tokens/s and effective HBM GB/s (% of peak), d=576 fused epilog"
KERNEL_SRC = os.path.join(ROOT, "kv_cache_epilog_amd", "csrc", "kvepi_kernels.hip")
DRQ_SRC = os.path.join(ROOT, "kv_cache_epilog_amd", "csrc", "kvepi_drq.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def algorithmic_bytes(w: kvgen.Workload, dense: bool = False) -> int:
    """Bytes the method must move: 4 B slot per token; for every hit row the
    x row (plus its cos and sin rows with RoPE) and the bytes written; gamma
    once.  dense: the x (and cos / sin) rows of skipped tokens counted as
    read too."""
    from kv_cache_epilog_amd import kvepi_row_bytes
    hits = w.hits
    x_row = 2 * w.d
    rope = 2 * 2 * 64 if w.cos is not None else 0
    if w.mode == kvgen.MODE_BF16_SPLIT:
        written = 2 * (w.d - 64) + 2 * 64
    elif w.mode in (kvgen.MODE_MXFP4, kvgen.MODE_MXFP8, kvgen.MODE_FP8_ROW):
        _, kc, sc = kvepi_row_bytes(w.mode, w.d, w.group_size)
        written = kc + sc * w.aux.elem_bytes  # codes + the cache_scale row
    else:
        _, kc, _ = kvepi_row_bytes(w.mode, w.d, w.group_size)
        written = kc
    gamma = 2 * (w.d - 64) if w.gamma is not None else 0
    read_rows = w.T if dense else hits
    return 4 * w.T + read_rows * (x_row + rope) + hits * written + gamma


def code_text(text: str) -> str:
    """C++ source with its comments removed and every run of blank space
    made one space: what the compiler sees of it (no string literal of the
    kernel sources holds a comment marker)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_hash(src: str = KERNEL_SRC) -> str:
    """sha256[:16] of a kernel source's code: measured traffic belongs to
    the code, so a change to it invalidates the figure and an edit of a
    comment does not."""
    with open(src, encoding="utf-8") as f:
        return hashlib.sha256(code_text(f.read()).encode()).hexdigest()[:16]


def measured_traffic(workload: str, src: str = KERNEL_SRC):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on another kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload)
    if not e or e.get("kernel_sha256_16") != kernel_hash(src):
        return None
    return e.get("bytes_per_launch")


def _counter_rows(csv_path: str, counter: str):
    """(kernel name, value) of every dispatch in a rocprofv3 --pmc CSV."""
    import csv
    out = []
    with open(csv_path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def _mean_of(rows, pick):
    vals = [v for k, v in rows if pick(k)]
    if not vals:
        raise SystemExit("no matching dispatches in the counter file")
    big = max(vals)
    vals = [v for v in vals if v >= 0.5 * big]  # the timed-size launches
    return sum(vals) / len(vals)


def write_traffic(workload: str, fetch_csv: str, write_csv: str, copy_fetch_csv: str,
                  copy_write_csv: str, copy_bytes: int, kernel: str = "epilog_kernel",
                  src: str = KERNEL_SRC):
    """Turn FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the epilog kernel
    into HBM bytes per launch.  Each counter is scaled by the factor that
    makes it read true on a plain device copy of copy_bytes (which reads and
    writes exactly copy_bytes)."""
    is_epi = lambda k: kernel in k  # noqa: E731
    is_copy = lambda k: "copy" in k.lower()  # noqa: E731
    kf = _mean_of(_counter_rows(fetch_csv, "FETCH_SIZE"), is_epi)
    kw = _mean_of(_counter_rows(write_csv, "WRITE_SIZE"), is_epi)
    cf = _mean_of(_counter_rows(copy_fetch_csv, "FETCH_SIZE"), is_copy)
    cw = _mean_of(_counter_rows(copy_write_csv, "WRITE_SIZE"), is_copy)
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    read_b = kf * 1024.0 * f_scale
    write_b = kw * 1024.0 * w_scale
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    table[workload] = {
        "kernel_sha256_16": kernel_hash(src), "bytes_per_launch": read_b + write_b,
        "read_bytes": read_b, "write_bytes": write_b,
        "fetch_kib_raw": kf, "write_kib_raw": kw,
        "copy_bytes": copy_bytes, "copy_fetch_kib_raw": cf, "copy_write_kib_raw": cw,
        "fetch_scale": f_scale, "write_scale": w_scale,
    }
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(table[workload]))


def copy_probe(mib: int, steps: int):
    """A plain device-to-device copy of mib MiB, launched steps times: the
    calibration run for the HBM byte counters."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": steps}), flush=True)


def cold_launches(step, dev, stream, launches: int = 20, scrub_mib: int = 512,
                  scrub: bool = True):
    """Mean kernel time with the device caches cold: before each launch a
    read-only reduction over scrub_mib MiB (twice the 256 MB Infinity Cache
    and far beyond L2) evicts the inputs and leaves clean lines, so no
    write-back of the scrub lands inside the timed launch; HIP events on the
    launch stream time each launch alone (its dispatch included)."""
    import torch
    n = scrub_mib << 20
    a = torch.zeros(n // 4, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    evs = []
    with torch.cuda.stream(stream):
        for _ in range(launches):
            if scrub:
                torch.amax(a, out=sink)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            evs.append((e0, e1))
    torch.cuda.synchronize()
    del a, sink
    return sum(e0.elapsed_time(e1) for e0, e1 in evs) / launches


def copy_ceiling(dev, stream, mib: int = 512, warmup: int = 20, steps: int = 50):
    """Achieved bandwidth of a plain device-to-device copy (torch's copy_,
    the runtime's copy kernel) of mib MiB, timed in the same run with HIP
    events on the launch stream: the practical ceiling that the kernel's
    effective bandwidth is also compared with.  Bytes = read + written."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            dst.copy_(src)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            dst.copy_(src)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del src, dst
    return 2 * n / (ms * 1e-3) / 1e9


def upload(w: kvgen.Workload, dev):
    import torch

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def cache(spec, init):
        flat = torch.from_numpy(init).to(dev)
        if spec.elem_bytes == 2:
            flat = flat.view(torch.bfloat16)
        elif spec.elem_bytes == 4:
            flat = flat.view(torch.float32)
        view = flat.as_strided((spec.block_num, spec.block_size, 1, spec.head_dim),
                               (spec.block_stride, spec.head_dim, spec.head_dim, 1))
        return view, flat

    t = dict(x=bf(w.x), slots=torch.from_numpy(w.slots).to(dev),
             gamma=None if w.gamma is None else bf(w.gamma),
             cos=None if w.cos is None else bf(w.cos), sin=None if w.sin is None else bf(w.sin))
    t["cache"], t["cache_flat"] = cache(w.cache, w.cache_init)
    t["aux"] = t["aux_flat"] = None
    if w.aux is not None:
        t["aux"], t["aux_flat"] = cache(w.aux, w.aux_init)
    return t


def host_info():
    """Host core count and CPU model (for the CPU baseline's record)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return os.cpu_count(), model


class _pinned:
    """Runs the enclosed block on one host core (restores the mask after)."""

    def __enter__(self):
        self.prev = os.sched_getaffinity(0)
        self.core = min(self.prev)
        os.sched_setaffinity(0, {self.core})
        return self

    def __exit__(self, *exc):
        os.sched_setaffinity(0, self.prev)
        return False


def cpu_baseline(w: kvgen.Workload, max_seconds: float):
    """The oracle as it stands (single-threaded C) on the same workload, on
    leading tokens until about max_seconds of CPU time, pinned to one host
    core."""
    with _pinned():
        return _cpu_baseline(w, max_seconds)


def _cpu_baseline(w: kvgen.Workload, max_seconds: float):
    import oracle
    cache = w.cache_init.copy()
    aux = None if w.aux_init is None else w.aux_init.copy()
    # calibrate on a small prefix, then size the sample
    probe = min(w.T, 2048)
    t0 = time.perf_counter()
    _run_oracle_prefix(oracle, w, probe, cache, aux)
    dt = time.perf_counter() - t0
    n = int(min(w.T, max(probe, probe * max_seconds / max(dt, 1e-6))))
    cache = w.cache_init.copy()
    aux = None if w.aux_init is None else w.aux_init.copy()
    t0 = time.perf_counter()
    _run_oracle_prefix(oracle, w, n, cache, aux)
    dt = time.perf_counter() - t0
    return n, dt, cache, aux


def _run_oracle_prefix(oracle, w, n, cache, aux):
    oracle.epilog(w.mode, w.x[:n], w.slots[:n], cache, w.cache.geom, group_size=w.group_size,
                  gamma=w.gamma, cos=None if w.cos is None else w.cos[:n],
                  sin=None if w.sin is None else w.sin[:n], eps=w.eps, aux_bytes=aux,
                  aux_geom=None if w.aux is None else w.aux.geom)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", type=int, default=4,
                    choices=range(len(kvgen.CONFIG_NAMES)),
                    help="workload index (default 4: the d=576 fused epilog; 5 and 6: "
                         "the MX-FP8 and per-row FP8 indexer modes)")
    ap.add_argument("--drq", choices=kvgen.DRQ_NAMES,
                    help="time the dequant -> RoPE -> int8 KV cache operator on this "
                         "workload instead of the epilog")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe", type=int, metavar="MIB",
                    help="only run a plain device copy of MIB MiB --steps times "
                         "(counter calibration)")
    ap.add_argument("--write-traffic", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="record HBM bytes per launch of --config's kernel from "
                         "rocprofv3 --pmc counter files; needs --copy-probe's size")
    args = ap.parse_args()
    if args.write_traffic:
        if not args.copy_probe:
            raise SystemExit("--write-traffic needs --copy-probe MIB (the calibration size)")
        if args.drq:
            write_traffic(args.drq, *args.write_traffic, copy_bytes=args.copy_probe << 20,
                          kernel="drq_kernel", src=DRQ_SRC)
        else:
            write_traffic(kvgen.CONFIG_NAMES[args.config], *args.write_traffic,
                          copy_bytes=args.copy_probe << 20)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe(args.copy_probe, args.steps)
        return
    if args.drq:
        main_drq(args)
        return

    import torch
    from kv_cache_epilog_amd import kvepi_run

    w = kvgen.config(args.config)
    dev = torch.device("cuda:0")
    t = upload(w, dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        kvepi_run(t["x"], t["slots"], t["cache"], w.mode, w.group_size, gamma=t["gamma"],
                  cos=t["cos"], sin=t["sin"], cache_aux=t["aux"], eps=w.eps, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # HIP events on the launch stream around the K back-to-back launches:
    # the host enqueues faster than the kernel runs, so the region is the
    # kernels plus their dispatch gaps (an event between launches would
    # add its own gap to every launch)
    total0 = torch.cuda.Event(enable_timing=True)
    total1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    total0.record(stream)
    for _ in range(args.steps):
        step()
    total1.record(stream)
    torch.cuda.synchronize()
    ms_total = total0.elapsed_time(total1)
    ms_per_step = ms_total / args.steps
    ms_kernel = ms_per_step

    abytes = algorithmic_bytes(w)
    achieved = abytes / (ms_kernel * 1e-3) / 1e9
    tokens_per_s = w.T / (ms_per_step * 1e-3)

    result = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded)",
        "config": {"workload": w.name, "tokens": w.T, "d": w.d, "quant_mode": w.mode,
                   "group_size": w.group_size, "rmsnorm": w.gamma is not None,
                   "rope": w.cos is not None, "hit_rows": w.hits,
                   "cache": [w.cache.block_num, w.cache.block_size, 1, w.cache.head_dim],
                   "block_stride_bytes": w.cache.block_stride * w.cache.elem_bytes,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(w.name),
                     "algorithmic_bytes_per_launch": abytes,
                     "dense_bytes_per_launch": algorithmic_bytes(w, dense=True),
                     "kernel_ms_mean": ms_kernel},
    }
    cc = copy_ceiling(dev, stream)
    result["copy_ceiling"] = {"achieved": cc, "unit": "GB/s", "kernel": "device copy, 512 MiB",
                              "frac": achieved / cc}
    ms_cold = cold_launches(step, dev, stream)
    ms_single = cold_launches(step, dev, stream, scrub=False)
    result["cold"] = {"ms_per_launch": ms_cold, "tokens_per_s": w.T / (ms_cold * 1e-3),
                      "achieved": abytes / (ms_cold * 1e-3) / 1e9, "unit": "GB/s",
                      "frac": abytes / (ms_cold * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                      "launches": 20, "scrub": "512 MiB read-only reduction before each launch",
                      "ms_per_launch_unscrubbed": ms_single}
    if not args.no_cpu:
        n, dt, ocache, oaux = cpu_baseline(w, args.cpu_seconds)
        ncpu, model = host_info()
        result["cpu_baseline"] = {
            "value": n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            # the same algorithmic bytes, prorated to the tokens of the sample
            "gbps": abytes * n / w.T / dt / 1e9,
            "sample": f"first {n} of {w.T} tokens of {w.name}, single-threaded C oracle "
                      f"pinned to one of {ncpu} host cores ({model}), {dt:.1f} s"}
        # the timed GPU path wrote the same rows: compare the tokens the
        # oracle covered
        got = t["cache_flat"].view(torch.uint8).cpu().numpy()
        rows = [w.cache.row_offset(s) for s in w.slots[:n] if 0 <= s < w.cache.num_slots]
        kc = w.cache.head_dim * w.cache.elem_bytes
        idx = (np.asarray(rows)[:, None] + np.arange(kc)[None, :]).reshape(-1)
        result["parity_sample_bytes_equal"] = bool(np.array_equal(got[idx], ocache[idx]))
    print(json.dumps(result), flush=True)


# ---- the dequant -> RoPE -> int8 KV cache operator -------------------------------

def drq_algorithmic_bytes(w) -> int:
    """Bytes the operator must move: per token the x row, cos and sin, the
    index (and activation scale), q_out (and k_out, v_out); per token with a
    cache row the int8 k and v rows; once the weight scales, bias and the
    per-channel scales and offsets."""
    H = (w.nq + 2 * w.nkv) * w.D
    xb = 4 if w.x_dtype == kvgen.DT_INT32 else 2
    if w.cache_mode == 0:
        hits = int(np.count_nonzero((w.index >= 0) & (w.index < w.geom[0] * w.geom[1])))
    else:
        hits = int(sum(max(0, min(w.seq_len, w.geom[1] - v)) for v in w.index if v >= 0))
    per_token = H * xb + 2 * 2 * w.D + 4 + (4 if w.act_scale is not None else 0)
    per_token += 2 * w.nq * w.D + (2 * 2 * w.nkv * w.D if w.kv_output else 0)
    once = sum(a.nbytes for a in (w.weight_scale, w.bias, w.scale_k, w.scale_v, w.offset_k,
                                  w.offset_v) if a is not None)
    return w.T * per_token + hits * 2 * w.nkv * w.D + once


def main_drq(args):
    import torch
    from kv_cache_epilog_amd import binding as B

    w = kvgen.drq_config(args.drq)
    dev = torch.device("cuda:0")
    t16 = torch.bfloat16 if w.out_dtype == kvgen.DT_BF16 else torch.float16

    def up(a, dtype=None):
        if a is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        return t.view(dtype) if dtype is not None else t

    x = up(w.x) if w.x_dtype == kvgen.DT_INT32 else up(w.x.view(np.int16), t16)
    bias = None
    if w.bias is not None:
        bias = up(w.bias) if w.bias_dtype in (kvgen.DT_FP32, kvgen.DT_INT32) else up(
            w.bias.view(np.int16), torch.bfloat16 if w.bias_dtype == kvgen.DT_BF16 else
            torch.float16)
    bn, bs, head, stride = w.geom
    kflat = torch.full((bn * stride,), 0xAB, dtype=torch.uint8, device=dev)
    vflat = torch.full((bn * stride,), 0xAB, dtype=torch.uint8, device=dev)
    kview = kflat.as_strided((bn, bs, 1, head), (stride, head, head, 1))
    vview = vflat.as_strided((bn, bs, 1, head), (stride, head, head, 1))
    q = torch.empty((w.T, w.nq * w.D), dtype=t16, device=dev)
    ko = torch.empty((w.T, w.nkv * w.D), dtype=t16, device=dev) if w.kv_output else None
    vo = torch.empty((w.T, w.nkv * w.D), dtype=t16, device=dev) if w.kv_output else None
    p = B.drq_params(x, up(w.cos.view(np.int16), t16), up(w.sin.view(np.int16), t16), kview,
                     vview, up(w.index), nq=w.nq, nkv=w.nkv, head_dim=w.D,
                     scale_k=up(w.scale_k), scale_v=up(w.scale_v), q_out=q, k_out=ko, v_out=vo,
                     weight_scale=up(w.weight_scale), act_scale=up(w.act_scale), bias=bias,
                     offset_k=up(w.offset_k), offset_v=up(w.offset_v), cache_mode=w.cache_mode,
                     seq_len=w.seq_len)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        B.kvepi_drq_run(p, stream=stream)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        B.kvepi_drq_run(p, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    abytes = drq_algorithmic_bytes(w)
    achieved = abytes / (ms * 1e-3) / 1e9
    H = (w.nq + 2 * w.nkv) * w.D
    result = {
        "metric": "tokens/s and effective HBM GB/s (% of peak), dequant-RoPE-int8 KV cache",
        "value": w.T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded)",
        "config": {"workload": args.drq, "tokens": w.T, "hidden": H, "nq": w.nq, "nkv": w.nkv,
                   "head_dim": w.D, "x_dtype": ["bf16", "fp16", "int32"][w.x_dtype],
                   "cache_mode": ["page", "contiguous"][w.cache_mode],
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(args.drq, DRQ_SRC),
                     "algorithmic_bytes_per_launch": abytes, "kernel_ms_mean": ms},
    }
    cc = copy_ceiling(dev, stream)
    result["copy_ceiling"] = {"achieved": cc, "unit": "GB/s", "kernel": "device copy, 512 MiB",
                              "frac": achieved / cc}
    ms_cold = cold_launches(lambda: B.kvepi_drq_run(p, stream=stream), dev, stream)
    ms_single = cold_launches(lambda: B.kvepi_drq_run(p, stream=stream), dev, stream,
                              scrub=False)
    result["cold"] = {"ms_per_launch": ms_cold, "tokens_per_s": w.T / (ms_cold * 1e-3),
                      "achieved": abytes / (ms_cold * 1e-3) / 1e9, "unit": "GB/s",
                      "frac": abytes / (ms_cold * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                      "launches": 20, "scrub": "512 MiB read-only reduction before each launch",
                      "ms_per_launch_unscrubbed": ms_single}
    if not args.no_cpu:
        import oracle
        kc = np.full(bn * stride, 0xAB, np.uint8)
        vc = np.full(bn * stride, 0xAB, np.uint8)

        def run_prefix(n):
            t0 = time.perf_counter()
            oracle.drq(w.x[:n], w.x_dtype, w.nq, w.nkv, w.D, w.cos[:n], w.sin[:n], w.out_dtype,
                       scale_k=w.scale_k, scale_v=w.scale_v, k_cache_bytes=kc,
                       v_cache_bytes=vc, cache_geom=w.geom, index=w.index[:n],
                       weight_scale=w.weight_scale,
                       act_scale=None if w.act_scale is None else w.act_scale[:n], bias=w.bias,
                       bias_dtype=w.bias_dtype, offset_k=w.offset_k, offset_v=w.offset_v,
                       kv_output=w.kv_output)
            return time.perf_counter() - t0

        # calibrate on a small prefix, then time about cpu_seconds of tokens
        with _pinned():
            probe = min(w.T, 1024)
            dt = run_prefix(probe)
            n = int(min(w.T, max(probe, probe * args.cpu_seconds / max(dt, 1e-6))))
            dt = run_prefix(n)
        ncpu, model = host_info()
        result["cpu_baseline"] = {"value": n / dt, "unit": "tokens/s", "cores": 1,
                                  "kind": "oracle",
                                  "gbps": abytes * n / w.T / dt / 1e9,
                                  "sample": f"first {n} of {w.T} tokens, single-threaded C "
                                            f"oracle pinned to one of {ncpu} host cores "
                                            f"({model}), {dt:.1f} s"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
