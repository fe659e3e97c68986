#!/usr/bin/env python3
"""Paged decode attention on one MI355X: achieved KV GB/s, fraction of the
HBM roofline and decode tokens/s, with the fp64 oracle timed on the host
cores as a CPU baseline.

A step is one call of the whole operation (paged_attn_decode through the
library's C ABI: a single kernel launch) over one synthetic decode batch
whose inputs are already resident in HBM.  Before every step, outside the timed
events, a 1 GiB device buffer is READ (a reduction) so that no K/V byte of
the previous step is still in L2 or the 256 MB MALL.  The flush only
reads: a flush that writes leaves dirty lines whose write-back then lands
inside the next timed kernel (measured: ~25% lower read bandwidth).

    python bench.py [--steps K] [--warmup W] [--workload N]

prints one JSON line.  Default workload: large-batch serving decode, batch
256, 32 query / 8 KV heads, head_dim 128, bf16, 16-token blocks, lognormal
lengths (median 1000), groups of 8 sequences sharing a 512-token prefix
(workload 5 of workload.py), through paged_attn_decode_shared; the GQA
batch (workload 3) and the long-context batch (workload 4) follow as
sub-entries with their own roofline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 matrix, published
METRIC = "paged decode attention: achieved KV GB/s (% of HBM peak) and tokens/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
CSRC = os.path.join(ROOT, "paged_kv_cache_196_amd", "csrc")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".h", ".hip")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, unique_kv: int) -> dict:
    """Bytes the operation must move at least once per call: every attended
    K/V element (shared blocks once), q, the fp32 output, the table entries
    of the attended blocks and the lengths."""
    S, Hq, D = w.q.shape
    nb = int(w.blocks_per_seq().sum())
    parts = {
        "kv": unique_kv,
        "q": S * Hq * D * w.esize,
        "out": S * Hq * D * 4,
        "tables": 4 * nb,
        "lens": 4 * S,
    }
    parts["total"] = sum(parts.values())
    return parts


def _traffic_entries() -> list:
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return []
    return t.get("entries", []) if isinstance(t, dict) else []


def read_traffic(src_hash: str, kernel_name: str, workload_name: str):
    """HBM bytes per decode launch from the committed rocprofv3 counter runs,
    or None when none were taken on these kernel sources for this kernel
    and workload."""
    for t in _traffic_entries():
        if t.get("source_hash") == src_hash and t.get("kernel") == kernel_name and \
                t.get("workload") == workload_name:
            return t.get("hbm_bytes_per_launch")
    return None


COPY_BYTES = 512 << 20  # calibration copy: reads and writes this many bytes per launch


def copy_calibration(launches: int = 5) -> int:
    """A plain elementwise copy (out = src * 1) of COPY_BYTES, `launches`
    times: the reference that FETCH_SIZE / WRITE_SIZE are scaled by."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(launches):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "launches": launches}), flush=True)
    return 0


def _counter_rows(path: str):
    """(kernel name, counter name, value) rows of rocprofv3 counter CSVs
    found under `path`."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                rows.append((r.get("Kernel_Name", ""), r.get("Counter_Name", ""),
                             float(r.get("Counter_Value", "nan"))))
    return rows


def _mean_counter(rows, counter: str, name_part: str) -> float:
    vals = [v for k, c, v in rows if c == counter and name_part in k]
    if not vals:
        raise SystemExit(f"no {counter} rows for kernels matching {name_part!r}")
    return sum(vals) / len(vals)


def make_workload(wid: str, seed=None):
    """A workload by its bench name: a config number ("1".."5") or the
    multi-query batch ("mqa32", "mqa64")."""
    import workload as wl
    if wid.startswith("mqa"):
        return wl.make_mqa(int(wid[3:]), seed)
    return wl.make(int(wid), seed)


def summarize_counters(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, workload_id, kernel,
                       shared: bool):
    """Turns four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE, each on
    this benchmark and on the calibration copy) into HBM bytes per decode
    launch, scaled by the copy's known bytes, and stores the entry for this
    (kernel, workload) in TRAFFIC_FILE."""
    import workload as wl
    w = make_workload(workload_id)
    kname = decode_kernel_name(w, kernel, shared)
    part = "decode_shared_kernel" if kname.startswith("decode_shared") else "decode_kernel"
    kib = 1024.0
    dec_fetch = _mean_counter(_counter_rows(fetch_dir), "FETCH_SIZE", part) * kib
    dec_write = _mean_counter(_counter_rows(write_dir), "WRITE_SIZE", part) * kib
    cp_fetch = _mean_counter(_counter_rows(copy_fetch_dir), "FETCH_SIZE", "Mul") * kib
    cp_write = _mean_counter(_counter_rows(copy_write_dir), "WRITE_SIZE", "Mul") * kib
    f_fetch = COPY_BYTES / cp_fetch
    f_write = COPY_BYTES / cp_write
    alg = algorithmic_bytes(w, wl.kv_bytes(w, unique=True))
    hbm = dec_fetch * f_fetch + dec_write * f_write
    out = {
        "kernel": kname,
        "workload": w.name,
        "source_hash": kernel_source_hash(),
        "hbm_bytes_per_launch": round(hbm),
        "read_bytes_per_launch": round(dec_fetch * f_fetch),
        "write_bytes_per_launch": round(dec_write * f_write),
        "raw_fetch_size_bytes": round(dec_fetch),
        "raw_write_size_bytes": round(dec_write),
        "copy_calibration": {"bytes": COPY_BYTES, "fetch_counter_bytes": round(cp_fetch),
                             "write_counter_bytes": round(cp_write),
                             "fetch_scale": round(f_fetch, 4), "write_scale": round(f_write, 4)},
        "algorithmic_bytes_per_launch": alg["total"],
        "traffic_over_algorithmic": round(hbm / alg["total"], 4),
    }
    entries = [e for e in _traffic_entries()
               if not (e.get("kernel") == kname and e.get("workload") == w.name)]
    entries.append(out)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump({"entries": entries}, f, indent=1)
        f.write("\n")
    print(json.dumps(out), flush=True)
    return 0


def decode_kernel_name(w, kernel: str, shared: bool) -> str:
    """Name of the decode kernel a call on workload w runs (as reported in
    the bench line and matched against counter runs)."""
    use_mfma = kernel == "mfma" or (kernel == "auto" and w.dtype != "f32")
    if shared and use_mfma and w.num_groups > 0 and w.group in (1, 2, 4, 8):
        return f"decode_shared_kernel<{w.dtype},B{w.block_size},G{w.group}>"
    return f"decode_kernel<{w.dtype},B{w.block_size},G{w.group},{'mfma' if use_mfma else 'valu'}>"


PROBE_SRC = os.path.join(ROOT, "bench_read_probe.hip")
PROBE_LIB = os.path.join(ROOT, "bench_read_probe.so")


def build_read_probe(verbose: bool = False) -> str:
    """hipcc bench_read_probe.hip -> bench_read_probe.so (gfx950)."""
    import subprocess
    from paged_kv_cache_196_amd import build as hipbuild
    tmp = PROBE_LIB + f".tmp{os.getpid()}"
    cmd = [hipbuild.hipcc(), f"--offload-arch={hipbuild.ARCH}", "-O3", "-std=c++17", "-fPIC",
           "-shared", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           PROBE_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stderr)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def read_probe(flush, dev, reps: int = 10) -> dict:
    """Best streaming-read rate on this device: bench_read_probe.hip over a
    separate 1 GiB buffer for a few grid sizes and both load policies, the
    flush run before each rep so that no part of the probe buffer is still
    cached.  Reported: the best median."""
    import ctypes
    import torch
    if not os.path.exists(PROBE_LIB):
        build_read_probe()
    lib = ctypes.CDLL(PROBE_LIB)
    lib.pa_bench_read_probe.restype = ctypes.c_int
    lib.pa_bench_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    nbytes = 1 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    grids = (1024, 2048, 4096, 8192)
    sink = torch.zeros(max(grids), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    best = None
    for variant in (0, 1):
        for grid in grids:
            ms = []
            for i in range(reps + 2):
                flush()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                rc = lib.pa_bench_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(), grid, variant,
                                             stream.cuda_stream)
                e1.record(stream)
                if rc != 0:
                    raise RuntimeError(f"read probe launch failed: {rc}")
                e1.synchronize()
                if i >= 2:
                    ms.append(e0.elapsed_time(e1))
            med = statistics.median(ms)
            if best is None or med < best[0]:
                best = (med, grid, variant)
    del buf, sink
    med, grid, variant = best
    return {"kernel": "bench_read_probe.hip: 16-byte loads, 8 in flight per lane",
            "bytes": nbytes, "grid": grid, "loads": "nontemporal" if variant else "default",
            "ms_median": round(med, 5), "gbps": round(nbytes / (med * 1e-3) / 1e9, 1)}


def cpu_baseline(w, kv_bytes: int, budget_s: float) -> dict:
    import oracle
    O = oracle.load()
    threads = len(os.sched_getaffinity(0))
    times = []
    t_all = time.perf_counter()
    while len(times) < 3 or (time.perf_counter() - t_all < budget_s and len(times) < 500):
        t0 = time.perf_counter()
        O.run_workload(w, num_threads=threads)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_all > 3 * budget_s:
            break
    med = statistics.median(times)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(kv_bytes / med / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"whole workload (all {w.num_seqs} sequences), fp64 C oracle with OpenMP, "
                  f"median of {len(times)} runs",
        "seconds_per_call": round(med, 4),
        "tokens_per_s": round(w.num_seqs / med, 2),
        "cpu_model": model,
    }


def _time_events(fn, flush, stream, reps: int, warmup: int = 3):
    """Mean / median ms of `fn` between HIP events on `stream`, the cache
    flush before every call outside the events."""
    import torch
    ms = []
    for i in range(warmup + reps):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        if i >= warmup:
            ms.append(e0.elapsed_time(e1))
    return statistics.mean(ms), statistics.median(ms)


def _cpu_time(fn, budget_s: float = 2.0) -> float:
    times = []
    t_all = time.perf_counter()
    while len(times) < 3 or (time.perf_counter() - t_all < budget_s and len(times) < 200):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return statistics.median(times)


def cache_writes(w, kp, vp, dev, flush, stream, with_cpu: bool) -> dict:
    """The two cache writes on the same pools: appending the next token of
    every sequence (the step before the next decode call) and copying
    random live blocks into every free block of the pool (copy-on-write at
    scale).  Neither touches a slot the decode call reads (the appended
    slot is at position L, the copies land in unreferenced blocks).  Each
    is timed with HIP events like the decode call; the oracle's byte-level
    routine is timed on the host copies, one thread."""
    import numpy as np
    import torch

    import paged_kv_cache_196_amd as pa
    import workload as wl

    rng = np.random.default_rng(w.seed + 1000)
    B, S, H, D, es = w.block_size, w.num_seqs, w.num_kv_heads, w.head_dim, w.esize
    tables = w.block_tables.copy()
    used = np.zeros(w.num_blocks, bool)
    used[tables[tables >= 0]] = True
    free = list(rng.permutation(np.nonzero(~used)[0]))
    pos = w.seq_lens.astype(np.int32).copy()
    for b in range(S):
        if pos[b] // B >= tables.shape[1]:
            pos[b] = -1  # the table row is full: no next slot
        elif pos[b] % B == 0:
            tables[b, pos[b] // B] = free.pop()
    dtype_code = {"f32": pa.PA_F32, "f16": pa.PA_F16, "bf16": pa.PA_BF16}[w.dtype]
    desc = pa.PaDesc(S, H, H, D, B, w.num_blocks, tables.shape[1], dtype_code, pa.PA_F32, 0, 0)
    if pa.pa_validate_append_host(desc, np.ascontiguousarray(tables), pos) != 0:
        raise RuntimeError("append preconditions do not hold")
    shape = (S, H, D)
    kn = wl.round_to(rng.standard_normal(shape, dtype=np.float32), w.dtype).reshape(shape)
    vn = wl.round_to(rng.standard_normal(shape, dtype=np.float32), w.dtype).reshape(shape)

    def up(x):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    kn_d, vn_d = up(kn), up(vn)
    tb_d = torch.from_numpy(tables).to(dev)
    pos_d = torch.from_numpy(pos).to(dev)
    sh = stream.cuda_stream
    live = int((pos >= 0).sum())
    app_bytes = 2 * 2 * live * H * D * es + 4 * S + 4 * live
    a_mean, a_med = _time_events(
        lambda: pa.paged_kv_append(kn_d, vn_d, kp, vp, tb_d, pos_d, desc, sh), flush, stream, 50)

    n = len(free)
    src = rng.choice(np.nonzero(used)[0], size=n).astype(np.int32)
    dst = np.asarray(free, np.int32)
    if pa.pa_validate_copy_host(desc, src, dst, n) != 0:
        raise RuntimeError("copy preconditions do not hold")
    src_d, dst_d = torch.from_numpy(src).to(dev), torch.from_numpy(dst).to(dev)
    block_bytes = H * B * D * es
    copy_bytes = 2 * 2 * n * block_bytes + 8 * n
    c_mean, c_med = _time_events(
        lambda: pa.paged_kv_copy_blocks(kp, vp, src_d, dst_d, n, desc, sh), flush, stream, 20)

    res = {
        "workload": w.name,
        "append": {
            "kernel": f"append_kernel<{es}>", "tokens": live,
            "us_per_call": round(a_mean * 1e3, 2), "us_median": round(a_med * 1e3, 2),
            "algorithmic_bytes": app_bytes,
            "gbps": round(app_bytes / (a_mean * 1e-3) / 1e9, 2),
            "frac_of_hbm_peak": round(app_bytes / (a_mean * 1e-3) / 1e9 / HBM_PEAK_GBPS, 5),
            "bound": "launch latency: one call moves well under 1 MB",
        },
        "copy_blocks": {
            "kernel": "copy_blocks_kernel", "pairs": n, "block_bytes_per_pool": block_bytes,
            "us_per_call": round(c_mean * 1e3, 2), "us_median": round(c_med * 1e3, 2),
            "algorithmic_bytes": copy_bytes,
            "gbps": round(copy_bytes / (c_mean * 1e-3) / 1e9, 2),
            "roofline": {"bound": "hbm", "achieved": round(copy_bytes / (c_mean * 1e-3) / 1e9, 2),
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(copy_bytes / (c_mean * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        },
    }
    if with_cpu:
        import oracle
        O = oracle.load()
        hk, hv = np.ascontiguousarray(w.k_pool).copy(), np.ascontiguousarray(w.v_pool).copy()
        t_app = _cpu_time(lambda: O.append(kn, vn, hk, hv, tables, pos, inplace=True))
        t_cp = _cpu_time(lambda: O.copy_blocks(hk, hv, src, dst, inplace=True))
        res["append"]["cpu_oracle"] = {"us_per_call": round(t_app * 1e6, 1), "cores": 1,
                                       "kind": "oracle", "sample": "same call, host pools"}
        res["copy_blocks"]["cpu_oracle"] = {"us_per_call": round(t_cp * 1e6, 1), "cores": 1,
                                            "gbps": round(copy_bytes / t_cp / 1e9, 2),
                                            "kind": "oracle", "sample": "same call, host pools"}
    return res


def eviction_scores(w, kp, vp, dev, flush, stream, with_cpu: bool) -> dict:
    """Block-wise eviction scoring (paged_kv_block_scores) over the same
    pools, every length cut to a whole number of blocks so that every
    sequence chooses a block: the scan reads every full block's K and V of
    every KV head once.  Timed with HIP events (two launches per call); the
    oracle is timed on a bounded sample of the sequences."""
    import numpy as np
    import torch

    import paged_kv_cache_196_amd as pa

    B, S, H, D, es = w.block_size, w.num_seqs, w.num_kv_heads, w.head_dim, w.esize
    lens = (w.seq_lens // B * B).astype(np.int32)
    full = lens // B
    dtype_code = {"f32": pa.PA_F32, "f16": pa.PA_F16, "bf16": pa.PA_BF16}[w.dtype]
    M = w.max_blocks_per_seq
    desc = pa.PaDesc(S, H, H, D, B, w.num_blocks, M, dtype_code, pa.PA_F32, 0, 0)
    if pa.pa_validate_host(desc, np.ascontiguousarray(w.block_tables), lens) != 0:
        raise RuntimeError("score preconditions do not hold")
    bt_d = torch.from_numpy(w.block_tables).to(dev)
    lens_d = torch.from_numpy(lens).to(dev)
    scores = torch.empty((S, M), dtype=torch.float32, device=dev)
    evict = torch.empty(S, dtype=torch.int32, device=dev)
    sh = stream.cuda_stream
    kv = int(full.sum()) * H * B * D * es * 2
    alg = kv + S * M * 4 + 4 * S + 4 * S + 4 * int(full.sum())
    mean, med = _time_events(
        lambda: pa.paged_kv_block_scores(kp, vp, bt_d, lens_d, scores, evict, desc, sh), flush,
        stream, 20)
    gbps = alg / (mean * 1e-3) / 1e9
    res = {
        "workload": w.name + " (lengths cut to whole blocks)",
        "kernels": ["block_score_kernel", "evict_choice_kernel"],
        "us_per_call": round(mean * 1e3, 2), "us_median": round(med * 1e3, 2),
        "kv_bytes": kv, "algorithmic_bytes": alg, "gbps": round(gbps, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4)},
    }
    if with_cpu:
        import oracle
        O = oracle.load()
        n = min(S, 4)
        t = _cpu_time(lambda: O.block_scores(w.k_pool, w.v_pool, w.block_tables[:n], lens[:n],
                                             dtype=w.dtype), budget_s=5.0)
        kv_n = int(full[:n].sum()) * H * B * D * es * 2
        res["cpu_oracle"] = {"gbps": round(kv_n / t / 1e9, 3), "seconds": round(t, 3), "cores": 1,
                             "kind": "oracle", "sample": f"first {n} of {S} sequences, fp64 C"}
    return res


def prefill_timing(dev, flush, stream, with_cpu: bool, dtype: str = "bf16") -> dict:
    """Causal paged prefill (paged_attn_prefill) of 8 whole prompts of 2048
    tokens with the GQA batch's head shapes (32 query / 8 KV heads, D 128,
    B 16, shuffled blocks), inputs and output in `dtype` (bf16: the
    benchmarked prefill; f16: the same prompts in fp16, whose weighted values
    take P in fp16 alone).  Algorithmic flops: 4 * D per (query row, query
    head, attended key): 2 D for q.k and 2 D for the weighted value sum; row
    i of a whole prompt attends i + 1 keys.  Timed with HIP events; the
    oracle is timed on a bounded sample (the last 32 rows of the first
    prompt).  The matrix peak is the same for both types."""
    import numpy as np
    import torch

    import paged_kv_cache_196_amd as pa
    import workload
    from workload import to_device as device_tensor

    w, q, qs = workload.prefill_workload(dtype=dtype)
    out_type = torch.bfloat16 if dtype == "bf16" else torch.float16
    n = np.diff(qs).astype(np.int64)
    L = w.seq_lens.astype(np.int64)
    keys = int(sum(((Lb - nb + 1) + Lb) * nb // 2 for Lb, nb in zip(L, n)))  # sum of (p + 1)
    flops = 4 * w.head_dim * w.num_q_heads * keys
    args = [device_tensor(q, w.dtype), device_tensor(w.k_pool, w.dtype),
            device_tensor(w.v_pool, w.dtype), torch.from_numpy(w.block_tables).to(dev),
            torch.from_numpy(w.seq_lens).to(dev), torch.from_numpy(qs).to(dev)]
    out = torch.empty(q.shape, dtype=out_type, device=dev)
    max_q = int(n.max())
    mean, med = _time_events(
        lambda: pa.prefill(*args, float(w.scale), max_q_len=max_q, out=out,
                           out_dtype=out_type, stream=stream, check_rows=False),
        flush, stream, 10)
    tflops = flops / (mean * 1e-3) / 1e12
    res = {
        "workload": w.name, "kernel": "prefill_kernel", "query_rows": int(qs[-1]),
        "us_per_call": round(mean * 1e3, 2), "us_median": round(med * 1e3, 2),
        "algorithmic_flops": flops, "tflops": round(tflops, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)},
    }
    if with_cpu:
        import oracle
        O = oracle.load()
        rows = 32
        Lb = int(L[0])
        qs_s = np.array([0, rows], np.int32)
        q_s = np.ascontiguousarray(q[qs[1] - rows: qs[1]])
        t = _cpu_time(lambda: O.paged_prefill(q_s, w.k_pool, w.v_pool, w.block_tables[:1],
                                              w.seq_lens[:1], qs_s, np.float64(np.float32(w.scale)),
                                              num_kv_heads=w.num_kv_heads, block_size=w.block_size,
                                              dtype=w.dtype, num_threads=1), budget_s=5.0)
        f_s = 4 * w.head_dim * w.num_q_heads * sum(Lb - rows + 1 + i for i in range(rows))
        res["cpu_oracle"] = {"tflops": round(f_s / t / 1e12, 5), "seconds": round(t, 3), "cores": 1,
                             "kind": "oracle",
                             "sample": f"last {rows} rows of the first prompt, fp64 C, one thread"}
    return res


def block_manager_timing(w, with_cpu: bool, steps: int = 50) -> dict:
    """Host block manager (pa_bm_*) latencies: allocating and releasing a
    large batch of single blocks (per block, one call each way), and the
    append preparation of one decode step for the workload's batch (tables
    built by the manager without sharing, `steps` consecutive steps, mean
    per step, the C entry point called directly with preallocated arrays).
    The plain model in oracle/ is timed on the same steps."""
    import ctypes

    import numpy as np

    import paged_kv_cache_196_amd as pa

    B, S = w.block_size, w.num_seqs
    NB = max(w.num_blocks, int((-(-w.seq_lens.astype(np.int64) // B)).sum()) + S * (steps // B + 2))
    bm = pa.BlockManager(NB, B)
    n = min(NB, 1 << 16)
    ta, tr = [], []
    for _ in range(20):
        t0 = time.perf_counter()
        st, ids = bm.alloc(n)
        t1 = time.perf_counter()
        st2 = bm.release(ids)
        t2 = time.perf_counter()
        if st or st2:
            raise RuntimeError("block manager alloc / release failed")
        ta.append(t1 - t0)
        tr.append(t2 - t1)
    lens0 = w.seq_lens.astype(np.int32)
    M = int(-(-(int(lens0.max()) + steps) // B)) + 1

    def fresh(model=None):
        tables = np.full((S, M), -1, np.int32)
        for b, L in enumerate(lens0):
            k = -(-int(L) // B)
            st, ids = (model.alloc(k) if model is not None else bm.alloc(k))
            tables[b, :k] = ids
        return tables

    tables = fresh()
    lens = lens0.copy()
    pos, src, dst = (np.zeros(S, np.int32) for _ in range(3))
    ncow = ctypes.c_int32(0)
    fn = pa.load().pa_bm_prepare_append
    args = (bm.h, tables.ctypes.data, M, lens.ctypes.data, S, pos.ctypes.data, src.ctypes.data,
            dst.ctypes.data, ctypes.byref(ncow))
    t0 = time.perf_counter()
    for _ in range(steps):
        if fn(*args):
            raise RuntimeError("prepare_append failed")
        lens += 1
    t_step = (time.perf_counter() - t0) / steps
    bm.close()
    contended = contended_alloc_timing(NB, B)
    res = {
        "bound": "host (no device work)",
        "alloc_ns_per_block": round(statistics.median(ta) / n * 1e9, 2),
        "release_ns_per_block": round(statistics.median(tr) / n * 1e9, 2),
        "blocks_per_call": n,
        "prepare_append_us_per_step": round(t_step * 1e6, 2),
        "sequences": S,
        "contended": contended,
    }
    if with_cpu:
        from oracle.block_manager import BlockManagerModel
        m = BlockManagerModel(NB, B)
        mt = [list(r) for r in fresh(m)]
        ml = [int(x) for x in lens0]
        t0 = time.perf_counter()
        for _ in range(steps):
            st, pos, cows = m.prepare_append(mt, ml)
            ml = [x + 1 for x in ml]
        res["model_prepare_append_us_per_step"] = round((time.perf_counter() - t0) / steps * 1e6, 1)
    return res


def contended_alloc_timing(NB: int, B: int, threads: int = 8) -> dict:
    """The lock-free manager under contention, timed natively (Python
    threads would measure the interpreter lock): the library's timing
    driver runs `threads` host threads that each allocate a batch of blocks
    with one pa_bm_alloc call and release them with one pa_bm_release
    call, over and over, on one shared manager; reported per block
    allocated and released, summed over all threads, beside one thread
    alone, for 64 blocks per call (a scheduler step) and 1 block per call
    (the worst case: every block an exchange on the shared words)."""
    import json as _json
    import subprocess

    import paged_kv_cache_196_amd as pa
    from paged_kv_cache_196_amd import build as pab

    exe = pab.BM_CONTEND
    if not os.path.exists(exe):
        raise RuntimeError(f"{exe} is not built (python -m paged_kv_cache_196_amd.build)")
    pa.load()
    res = {}
    for batch in (64, 1):
        nb = max(NB, threads * batch)
        r = subprocess.run([exe, str(threads), str(batch), "300", str(nb)], capture_output=True,
                           text=True, timeout=60)
        if r.returncode != 0:
            raise RuntimeError("bm_contend failed: " + r.stdout + r.stderr)
        res[f"batch_{batch}"] = _json.loads(r.stdout)
    return res


def decode_leg(w, args, dev, flush, stream, O, shared: bool, steps: int, warmup: int) -> dict:
    """Upload workload w, check every output against the oracle, then time
    `steps` decode calls (after `warmup`) between HIP events on the launch
    stream, the read-only flush before every call outside the events.  With
    shared=True a workload with prefix groups goes through
    paged_attn_decode_shared (every shared block read once per group)."""
    import numpy as np
    import torch

    import paged_kv_cache_196_amd as pa
    import workload

    kv_logical = workload.kv_bytes(w)
    kv_unique = workload.kv_bytes(w, unique=True)
    alg = algorithmic_bytes(w, kv_unique)
    q, kp, vp = (workload.to_device(x, w.dtype, dev) for x in (w.q, w.k_pool, w.v_pool))
    bt = torch.from_numpy(w.block_tables).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    kern = {"auto": pa.PA_KERNEL_AUTO, "valu": pa.PA_KERNEL_VALU, "mfma": pa.PA_KERNEL_MFMA}[args.kernel]
    use_groups = shared and w.num_groups > 0
    hint = 0 if (use_groups or args.no_prefix_hint) else w.shared_prefix_blocks
    desc = pa.make_desc(q, kp, bt, out_dtype=torch.float32, kernel=kern, cached_prefix_blocks=hint)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    sh = stream.cuda_stream
    scale = float(w.scale)
    kname = decode_kernel_name(w, args.kernel, use_groups)
    if use_groups:
        gs = torch.from_numpy(w.group_start).to(dev)
        gsh = torch.from_numpy(w.group_shared).to(dev)
        ws = pa.new_shared_workspace(desc, dev)
        grid = pa.pa_decode_shared_grid(desc, w.num_groups)

        def call():
            pa.paged_attn_decode_shared(q, kp, vp, bt, lens, gs, gsh, w.num_groups, scale, out,
                                        desc, ws, ws.numel(), sh)
    else:
        ws = pa.new_workspace(desc, dev)
        grid = pa.pa_decode_grid(desc)

        def call():
            pa.paged_attn_decode(q, kp, vp, bt, lens, scale, out, desc, ws, ws.numel(), sh)

    max_err = None
    if O is not None:
        call()
        torch.cuda.synchronize()
        max_err = float(np.max(np.abs(out.double().cpu().numpy() - O.run_workload(w))))
    for _ in range(warmup):
        if not args.no_flush:
            flush()
        call()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if not args.no_flush:
            flush()
        evs[i][0].record(stream)
        call()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tot_ms = [e[0].elapsed_time(e[1]) for e in evs]
    t_step = statistics.mean(tot_ms)
    kv_gbps = kv_unique / (t_step * 1e-3) / 1e9
    achieved = alg["total"] / (t_step * 1e-3) / 1e9  # one kernel per call
    src_hash = kernel_source_hash()
    traffic = read_traffic(src_hash, kname, w.name)
    return {
        "workload": w.name,
        "config": {
            "workload": w.name, "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads,
            "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
            "seq_len_mean": round(float(w.seq_lens.mean()), 1),
            "seq_len_min": int(w.seq_lens.min()), "seq_len_max": int(w.seq_lens.max()),
            "num_blocks": w.num_blocks, "shared_prefix_blocks": w.shared_prefix_blocks,
            "prefix_groups": w.num_groups if use_groups else 0,
            "cached_prefix_blocks": hint, "seed": w.seed, "kernel": args.kernel,
            "entry_point": "paged_attn_decode_shared" if use_groups else "paged_attn_decode",
            "decode_grid": grid, "parallelism": "single GPU",
        },
        "dtype": w.dtype,
        "ms_per_step": round(t_step, 5),
        "kv_gbps": round(kv_gbps, 2),
        "hbm_frac": round(kv_gbps / HBM_PEAK_GBPS, 4),
        "tokens_per_s": round(w.num_seqs / (t_step * 1e-3), 1),
        "kv_bytes": kv_unique,
        "kv_bytes_logical": kv_logical,
        "kv_gbps_logical": round(kv_logical / (t_step * 1e-3) / 1e9, 2),
        "ms": {
            "step_mean": round(t_step, 5), "step_median": round(statistics.median(tot_ms), 5),
            "step_p10": round(sorted(tot_ms)[len(tot_ms) // 10], 5),
            "step_p90": round(sorted(tot_ms)[(9 * len(tot_ms)) // 10], 5),
        },
        "roofline": {
            "bound": "hbm", "kernel": kname, "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic, "algorithmic_bytes": alg["total"],
        },
        "wall_s_timed_loop": round(wall, 4),
        "max_abs_err_vs_oracle": max_err,
        "kernel_source_hash": src_hash,
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="5", choices=["1", "2", "3", "4", "5", "mqa32", "mqa64"],
                    help="the timed workload: a config number, or mqa32 / mqa64 (the multi-query "
                         "batch; used for its counter runs)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--kernel", choices=["auto", "valu", "mfma"], default="auto")
    ap.add_argument("--no-flush", action="store_true", help="skip the cache flush between steps")
    ap.add_argument("--no-prefix-groups", action="store_true",
                    help="run a workload with prefix groups through paged_attn_decode (every "
                         "shared block read once per sequence) instead of paged_attn_decode_shared")
    ap.add_argument("--no-prefix-hint", action="store_true",
                    help="with --no-prefix-groups: no shared-prefix cache hint either")
    ap.add_argument("--other-workloads", default="3,4,mqa64",
                    help="comma-separated workloads timed after the headline one as sub-entries: "
                         "config numbers, or mqa32 / mqa64 for the multi-query decode ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true", help="skip the oracle check")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-read-probe", action="store_true")
    ap.add_argument("--no-cache-writes", action="store_true",
                    help="skip timing the append / block-copy calls")
    ap.add_argument("--no-eviction-scores", action="store_true",
                    help="skip timing the block-wise eviction scoring")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip timing the causal paged prefill")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only the calibration copy (for rocprofv3 counter scaling)")
    ap.add_argument("--summarize-counters", nargs=4, metavar="DIR",
                    help="FETCH_SIZE run, WRITE_SIZE run, copy FETCH_SIZE run, copy WRITE_SIZE run")
    args = ap.parse_args()

    if args.summarize_counters:
        return summarize_counters(*args.summarize_counters, args.workload, args.kernel,
                                  shared=not args.no_prefix_groups)
    if args.copy_calibration:
        return copy_calibration()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(see the sharding notes); run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    import paged_kv_cache_196_amd as pa
    import workload

    pa.ensure_built()
    pa.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    flush_src = torch.zeros((1 << 30) // 4, dtype=torch.float32, device=dev)

    def flush():
        # read-only pass over 1 GiB: evicts L2 and MALL without dirtying them
        return flush_src.sum()

    O = None
    if not args.no_check:
        import oracle
        O = oracle.load()
    shared = not args.no_prefix_groups
    w = make_workload(args.workload, args.seed)
    head = decode_leg(w, args, dev, flush, stream, O, shared, args.steps, args.warmup)
    probe = None if args.no_read_probe else read_probe(flush, dev)

    result = {
        "metric": METRIC,
        "value": head["kv_gbps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": head["config"],
        "hbm_frac": head["hbm_frac"],
        "tokens_per_s": head["tokens_per_s"],
        "kv_bytes": head["kv_bytes"],
        "kv_bytes_logical": head["kv_bytes_logical"],
        "kv_gbps_logical": head["kv_gbps_logical"],
        "read_probe": probe,
        "frac_of_read_probe": round(head["kv_gbps"] / probe["gbps"], 4) if probe else None,
        "ms": head["ms"],
        "roofline": head["roofline"],
        "timing": "HIP events on the launch stream around each kernel of each step; "
                  + ("read-only 1 GiB cache flush before every step, outside the events" if not args.no_flush
                     else "no cache flush"),
        "wall_s_timed_loop": head["wall_s_timed_loop"],
        "max_abs_err_vs_oracle": head["max_abs_err_vs_oracle"],
        "kernel_source_hash": head["kernel_source_hash"],
        "context": {
            "pages_paged_vs_contiguous": "paged kernel ~20-26% slower than a contiguous one "
                                         "(original vLLM paper, hardware not stated)",
            "pages_serving_throughput": "2-4x serving throughput at the same latency (vLLM, end to end)",
        },
    }
    if w.num_groups > 0 and shared:
        # the same batch through the ordinary call (each shared block read
        # once per sequence, with the cache hint), for comparison
        plain = decode_leg(w, args, dev, flush, stream, None, False, max(10, args.steps // 2),
                           max(3, args.warmup // 2))
        result["without_prefix_groups"] = {k: plain[k] for k in (
            "ms_per_step", "kv_gbps", "hbm_frac", "tokens_per_s", "roofline")}
        result["without_prefix_groups"]["entry_point"] = plain["config"]["entry_point"]
        result["without_prefix_groups"]["cached_prefix_blocks"] = plain["config"]["cached_prefix_blocks"]
    others = [x.strip() for x in args.other_workloads.split(",") if x.strip()]
    subs = {}
    for wid in others:
        if wid == str(args.workload):
            continue
        wo = make_workload(wid)
        leg = decode_leg(wo, args, dev, flush, stream, O, shared, args.steps, args.warmup)
        subs[wid] = {k: leg[k] for k in (
            "workload", "dtype", "ms_per_step", "kv_gbps", "hbm_frac", "tokens_per_s", "kv_bytes",
            "roofline", "max_abs_err_vs_oracle", "ms")}
        subs[wid]["decode_grid"] = leg["config"]["decode_grid"]
        del wo
    if subs:
        result["workloads"] = subs
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, head["kv_bytes"], args.cpu_seconds)
    # the adjacent rows are measured on the GQA batch (workload 3)
    wa = workload.make(3)
    result["block_manager"] = block_manager_timing(wa, with_cpu=not args.no_cpu_baseline)
    if not (args.no_eviction_scores and args.no_cache_writes):
        kp = workload.to_device(wa.k_pool, wa.dtype, dev)
        vp = workload.to_device(wa.v_pool, wa.dtype, dev)
        if not args.no_eviction_scores:
            result["eviction_scores"] = eviction_scores(wa, kp, vp, dev, flush, stream,
                                                        with_cpu=not args.no_cpu_baseline)
        if not args.no_cache_writes:
            # these write (unread) pool slots of their own upload
            result["cache_writes"] = cache_writes(wa, kp, vp, dev, flush, stream,
                                                  with_cpu=not args.no_cpu_baseline)
        del kp, vp
    if not args.no_prefill:
        result["prefill"] = prefill_timing(dev, flush, stream, with_cpu=not args.no_cpu_baseline)
        result["prefill_f16"] = prefill_timing(dev, flush, stream, with_cpu=False, dtype="f16")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
