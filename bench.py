"""Benchmark of the fused rotate + INT4 quantise path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--group G]

One step is one hq_rotate_quant call over one whole batch of the workload
(default: 16384 tokens x 4096 bf16, full 4096-point randomized Hadamard,
per-token INT4, fp32 scales; --group G times hq_rotate_quant_grouped with one
scale per G rotated elements instead).  The inputs are resident in HBM before timing
starts; steps cycle through several independent buffer sets whose total
size is well above the 256 MB last-level cache, so every step streams from
HBM.  Before the W warm-up steps the same call runs untimed for at least
SETTLE_S seconds: on this GPU the first tens of milliseconds of a burst of
calls run up to 60 % slower while clocks and translation caches settle, and
the timed steps are meant to measure the steady state.  Rank 0 prints one
JSON line.

`value` is GB/s of algorithmic traffic (input + codes + scales) per second of
kernel time; `roofline` relates it to the 8 TB/s HBM peak; `cpu_baseline` is
the CPU oracle timed on a bounded sample of the same workload.  The inverse
path (dequantise + inverse rotation) and a same-size device copy are timed
alongside for context.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
LLC_BYTES = 256 * 2 ** 20
METRIC = "fused rotate+INT4-quant GB/s and % of HBM peak at 16384x4096 bf16"
SETTLE_S = 0.05  # untimed calls before the warm-up steps (see the docstring)


def copy_bytes_for(bytes_call: int) -> int:
    """Size of the plain device copy timed beside the kernel (it moves the
    same number of bytes: half read, half written)."""
    return bytes_call // 2


# The sources each workload's timed launch is built from: the dispatch and
# shared primitives, plus the kernel that the workload's shape selects.
_COMMON_SOURCES = ("hq_api.hip", "hq_internal.h", "hq_device.h", "hq_fast_impl.h",
                   "hq_mfma_impl.h", "hq_mfma.hip")
TRAFFIC_SOURCES = {
    "hidden_4096": _COMMON_SOURCES + ("hq_mfma_rq.hip",),
    "qk_heads": _COMMON_SOURCES + ("hq_mfma_rq.hip",),
    "kv_cache": _COMMON_SOURCES + ("hq_mfma_rq.hip",),
    "ffn_11008": _COMMON_SOURCES + ("hq_mfma_long.hip",),
    "tiny_int8": _COMMON_SOURCES + ("hq_fast.hip", "hq_fast_rq.hip"),
    "ffn_11008_full": _COMMON_SOURCES + ("hq_paley.hip", "hq_paley_mfma.hip"),
}


def source_hash(workload: str) -> str:
    """Hash of the kernel sources a stored traffic measurement of `workload`
    belongs to."""
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES[workload]:
        p = os.path.join(ROOT, "hadamard_rotation_amd", "csrc", name)
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def _counter_means(path: str, counter: str) -> dict:
    """Mean per dispatch of `counter` for every (kernel name, grid size) in a
    rocprofv3 --pmc result (its SQLite database, *_results.db, or a
    counter_collection CSV), with the dispatch count and the first dispatch
    id."""
    rows = []
    if path.endswith(".db"):
        import sqlite3
        db = sqlite3.connect(path)
        rows = db.execute("select kernel_name, grid_size, value, dispatch_id from "
                          "counters_collection where counter_name = ?", (counter,)).fetchall()
        db.close()
    else:
        import csv
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    rows.append((r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"]),
                                 int(r["Dispatch_Id"])))
    acc: dict = {}
    first: dict = {}
    for name, grid, value, disp in rows:
        key = (name, int(grid))
        acc.setdefault(key, []).append(float(value))
        first[key] = min(first.get(key, 1 << 62), int(disp))
    return {k: (sum(v) / len(v), len(v), first[k]) for k, v in acc.items()}


def write_traffic(workload: str, fetch_csv: str, write_csv: str, copy_bytes: int,
                  tcc_db: str | None = None) -> dict:
    """HBM bytes per launch of the dominant hq kernel from two rocprofv3
    --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE; both in KiB per
    dispatch), each scaled by what the same counter reads for the plain
    device copy of `copy_bytes` bytes that the script also times (the
    copy launch repeated most often; other copies, e.g. buffer clones,
    have other grid sizes)."""
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    copy_key = max((k for k in fetch if "copyBuffer" in k[0]), key=lambda k: fetch[k][1])
    # the timed launch: the first library kernel the script dispatches more
    # than once (the extras, inverse, append and attention, come after it;
    # a once-per-GPU set-up launch, such as the Paley operand table, before)
    kern_key = min((k for k in fetch if "hq::" in k[0] and fetch[k][1] > 1), key=lambda k: fetch[k][2])
    f_scale = copy_bytes / (fetch[copy_key][0] * 1024.0)
    w_scale = copy_bytes / (write[copy_key][0] * 1024.0)
    fb = fetch[kern_key][0] * 1024.0 * f_scale
    wb = write[kern_key][0] * 1024.0 * w_scale
    if tcc_db:
        # Reads counted from the L2's memory read requests themselves: on this
        # GPU a request is 32 or 128 bytes, and TCC_BUBBLE, through which
        # FETCH_SIZE's formula counts 128-byte requests, reads 0 (so
        # FETCH_SIZE counts them as 64 bytes: half).  Writes: WRITE_SIZE
        # as read (its formula matches the 32/64-byte write requests).
        rd = _counter_means(tcc_db, "TCC_EA0_RDREQ_sum")
        r32 = _counter_means(tcc_db, "TCC_EA0_RDREQ_32B_sum")
        bub = _counter_means(tcc_db, "TCC_BUBBLE_sum")
        kk = min((k for k in rd if "hq::" in k[0] and rd[k][1] > 1), key=lambda k: rd[k][2])
        n_rd, n32 = rd[kk][0], r32[kk][0]
        req_read = (n_rd - n32) * 128.0 + n32 * 32.0
        req = {"read_requests": n_rd, "read_requests_32B": n32, "bubble": bub[kk][0],
               "read_bytes": req_read, "write_bytes": write[kern_key][0] * 1024.0,
               "bytes_per_launch": req_read + write[kern_key][0] * 1024.0}
    out = {"workload": workload, "kernel": kern_key[0], "source_hash": source_hash(workload),
           "fetch_kib_raw": fetch[kern_key][0], "write_kib_raw": write[kern_key][0],
           "copy_bytes": copy_bytes, "copy_grid": copy_key[1],
           "copy_fetch_kib_raw": fetch[copy_key][0], "copy_write_kib_raw": write[copy_key][0],
           "fetch_scale": f_scale, "write_scale": w_scale, "fetch_bytes": fb,
           "write_bytes": wb, "bytes_per_launch": fb + wb}
    if tcc_db:
        out["from_requests"] = req
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    return out


def load_traffic(workload: str):
    """HBM bytes per launch measured with rocprofv3 counters for the current
    kernel sources, scaled by the copy (None if no measurement matches the
    sources), and the same from the read requests themselves (None if not
    measured)."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None, None
    with open(p) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash(workload):
        return None, None
    return t.get("bytes_per_launch"), t.get("from_requests", {}).get("bytes_per_launch")


def cpu_baseline(workload, target_s: float = 24.0) -> dict:
    """Time the CPU oracle (as it stands, all host cores) on a bounded sample
    of the same workload: a probe of about 3e9 multiply-adds sizes the
    sample to roughly target_s seconds, capped at the whole workload."""
    from hadamard_rotation_amd import workloads as W
    from oracle import oracle as O

    w = W.WORKLOADS[workload]
    threads = O.default_threads()
    per_row_mac = w.n * w.b
    probe_rows = max(threads, min(w.rows, int(3e9 // per_row_mac)))
    data = W.generate(workload, seed=42, tokens=(probe_rows + w.unit - 1) // w.unit)
    raw, s = data[w.tensors[0]][:probe_rows], data["s"]
    t0 = time.perf_counter()
    O.rotate_quant(raw, w.x_dtype, w.b, s, w.bits, w.scale_dtype, threads=threads,
                   want_preround=False)
    dt = max(time.perf_counter() - t0, 1e-3)
    rows = int(min(w.rows, probe_rows * target_s / dt))
    rows = max(probe_rows, rows - rows % w.unit)
    data = W.generate(workload, seed=42, tokens=(rows + w.unit - 1) // w.unit)
    raw = data[w.tensors[0]][:rows]
    t0 = time.perf_counter()
    O.rotate_quant(raw, w.x_dtype, w.b, data["s"], w.bits, w.scale_dtype,
                   threads=threads, want_preround=False)
    dt = time.perf_counter() - t0
    gbs = w.bytes_per_call(rows) / dt / 1e9
    return {"value": round(gbs, 6), "unit": "GB/s", "cores": threads, "cpu": cpu_model(),
            "kind": "oracle",
            "sample": f"{rows} of {w.rows} rows of the same workload (seed 42, same "
                      f"generator), {dt:.2f} s wall on {threads} threads; explicit fp64 "
                      f"H_{w.b} product per block, scalar quantisation"}


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_workload(name: str, dev, stream, ev0, ev1, calls: int = 200) -> dict:
    """One workload at its full size: the seeded tensors (every tensor of the
    workload, e.g. Q and K) resident in HBM, enough copies to exceed the
    last-level cache, a settle phase, then `calls` timed calls of
    hq_rotate_quant cycling through them (HIP events on the launch stream).
    For workloads with an inverse in their definition (the K/V cache round
    trip), the inverse of the same codes is timed too (fp32 output)."""
    import numpy as np
    import torch

    import hadamard_rotation_amd as hq
    from hadamard_rotation_amd import workloads as W

    w = W.WORKLOADS[name]
    data = W.generate(name, seed=42)
    s = torch.from_numpy(data["s"]).to(dev)
    tdt = {W.F32: torch.float32, W.BF16: torch.bfloat16, W.F16: torch.float16}[w.x_dtype]
    base = []
    for t in w.tensors:
        raw = data[t]
        if w.x_dtype == W.F32:
            base.append(torch.from_numpy(raw).to(dev))
        else:
            base.append(torch.from_numpy(raw.view(np.int16)).to(dev).view(tdt))
    del data
    rows, n = base[0].shape
    bytes_call = w.bytes_per_call(rows)
    copies = max(1, int(np.ceil(3 * LLC_BYTES / (bytes_call * len(base)))))
    xs = [x if c == 0 else x.clone() for c in range(copies) for x in base]
    sd = torch.float32 if w.scale_dtype == W.F32 else torch.float16
    cw = n // 2 if w.bits == 4 else n
    cdt = torch.uint8 if w.bits == 4 else torch.int8
    codes = [torch.empty((rows, cw), dtype=cdt, device=dev) for _ in xs]
    scales = [torch.empty((rows,), dtype=sd, device=dev) for _ in xs]

    def call(i):
        k = i % len(xs)
        hq.hq_rotate_quant(xs[k], s, w.b, w.bits, sd, codes=codes[k], scales=scales[k],
                           stream=stream)

    def timed(fn, k):
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < SETTLE_S:
            for _ in range(10):
                fn(i)
                i += 1
            torch.cuda.synchronize()
        ev0.record(stream)
        for j in range(k):
            fn(j)
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) * 1e3 / k

    us = timed(call, calls)
    print(f"[bench] {name}: {us:.2f} us per call", file=sys.stderr, flush=True)
    traffic, traffic_req = load_traffic(name)
    rec = {"workload": f"{name}: {w.description}", "tensors": len(w.tensors), "rows": rows,
           "n": n, "b": w.b, "bits": w.bits, "bytes_per_call": bytes_call,
           "us_per_call": round(us, 3), "GB/s": round(bytes_call / us / 1e3, 3),
           "frac_of_8TBs": round(bytes_call / us / 1e3 / HBM_PEAK_GBS, 4),
           "traffic": traffic, "traffic_from_requests": traffic_req}
    if name == "kv_cache":
        ys = [torch.empty((rows, n), dtype=torch.float32, device=dev) for _ in range(2)]

        def inv(i):
            k = i % len(xs)
            hq.hq_dequant_rotate_inv(codes[k], scales[k], s, w.b, w.bits, y=ys[i % 2],
                                     stream=stream)

        for i in range(len(xs)):
            call(i)
        ius = timed(inv, max(20, calls // 2))
        ib = rows * (cw + (4 if w.scale_dtype == W.F32 else 2) + 4 * n)
        rec["inverse"] = {"us_per_call": round(ius, 3), "GB/s": round(ib / ius / 1e3, 3),
                          "bytes_per_call": ib, "out_dtype": "f32"}
    del xs, codes, scales
    torch.cuda.empty_cache()
    return rec


def time_append(dev, stream, ev0, ev1, seqs: int = 32, heads: int = 8, n: int = 128,
                cache_tokens: int = 131072, calls: int = 200) -> dict:
    """One decode step of a K cache: `seqs` sequences append one token of
    `heads` 128-wide heads (bf16) each, rotated and quantised to INT4 with
    fp16 scales, into a [cache_tokens * heads, 64] code cache at their own
    positions.  Launch-latency bound: a few kB move per call."""
    import numpy as np
    import torch

    import hadamard_rotation_amd as hq
    from hadamard_rotation_amd import workloads as W

    rows = seqs * heads
    raw, s_np = W.random_rows(7, rows, n, W.BF16, outliers=1)
    x = torch.from_numpy(raw.view(np.int16)).to(dev).view(torch.bfloat16)
    s = torch.from_numpy(s_np).to(dev)
    rng = np.random.default_rng(8)
    pos = rng.choice(cache_tokens, size=seqs, replace=False)
    dst = torch.from_numpy((pos[:, None] * heads + np.arange(heads)[None, :])
                           .reshape(-1).astype(np.int64)).to(dev)
    codes = torch.zeros((cache_tokens * heads, n // 2), dtype=torch.uint8, device=dev)
    scales = torch.zeros((cache_tokens * heads,), dtype=torch.float16, device=dev)
    for _ in range(10):
        hq.hq_rotate_quant_append(x, s, n, dst, codes, scales, 4, stream=stream)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(calls):
        hq.hq_rotate_quant_append(x, s, n, dst, codes, scales, 4, stream=stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / calls
    nbytes = rows * (2 * n + n // 2 + 2) + rows * 8
    return {"rows": rows, "n": n, "cache_rows": cache_tokens * heads,
            "us_per_call": round(us, 3), "GB/s": round(nbytes / us / 1e3, 3),
            "bytes_per_call": nbytes}


def time_attention(dev, stream, ev0, ev1, tokens: int = 131072, kv_heads: int = 8,
                   q_heads: int = 32, calls: int = 200) -> dict:
    """Decode attention of 32 query heads over the 131072-token x 8-head INT4
    K/V cache (fp16 scales): the consumer of the codes.  Two cache copies
    alternate so that the 138 MB read per call exceeds the last-level cache
    over two calls.  Algorithmic bytes: the K and V codes and scales, q and
    the output; the workspace traffic (4 MB) is not counted."""
    import numpy as np
    import torch

    import hadamard_rotation_amd as hq

    n = 128
    g = torch.Generator(device="cpu").manual_seed(5)
    caches = []
    for _ in range(2):
        kc = torch.randint(0, 256, (tokens, kv_heads, n // 2), dtype=torch.uint8, generator=g)
        vc = torch.randint(0, 256, (tokens, kv_heads, n // 2), dtype=torch.uint8, generator=g)
        ks = (torch.rand((tokens, kv_heads), generator=g) * 0.5 + 0.1).to(torch.float16)
        vs = (torch.rand((tokens, kv_heads), generator=g) * 0.5 + 0.1).to(torch.float16)
        caches.append([t.to(dev) for t in (kc, ks, vc, vs)])
    q = torch.randn((q_heads, n), generator=g).to(torch.bfloat16).to(dev)
    s = torch.from_numpy(np.where(np.arange(n) % 3 == 0, -1, 1).astype(np.int8)).to(dev)
    out = torch.empty((q_heads, n), dtype=torch.float32, device=dev)
    ws = torch.empty(hq.hq_decode_attention_workspace(q_heads, kv_heads, tokens),
                     dtype=torch.uint8, device=dev)

    def call(i):
        kc, ks, vc, vs = caches[i % 2]
        hq.hq_decode_attention(q, s, n, kc, ks, vc, vs, 4, out=out, workspace=ws, stream=stream)

    # the same untimed settle phase as the headline, then the timed calls
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(10):
            call(i)
            i += 1
        torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(calls):
        call(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / calls
    nbytes = 2 * tokens * kv_heads * (n // 2 + 2) + q_heads * n * (2 + 4)
    return {"tokens": tokens, "kv_heads": kv_heads, "q_heads": q_heads, "head_dim": n,
            "us_per_call": round(us, 3), "GB/s": round(nbytes / us / 1e3, 3),
            "frac_of_8TBs": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
            "bytes_per_call": nbytes}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="hidden_4096")
    ap.add_argument("--group", type=int, default=None,
                    help="group-wise scales: one per GROUP rotated elements")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the inverse-path, copy, append, attention and other-workload "
                         "timings")
    ap.add_argument("--copy", action="store_true",
                    help="with --no-extras: still time the same-size device copy (the "
                         "reference the traffic counters are scaled by)")
    ap.add_argument("--attention-only", action="store_true",
                    help="time only the decode attention call (the record that the default "
                         "run reports as decode_attention) and print it as one JSON line")
    ap.add_argument("--traffic", nargs="+", metavar="PMC_RESULT",
                    help="turn rocprofv3 --pmc runs of this script (FETCH_SIZE, then "
                         "WRITE_SIZE, optionally TCC_EA0_RDREQ_sum TCC_BUBBLE_sum "
                         "TCC_EA0_RDREQ_32B_sum; their *_results.db or CSV) into "
                         "profiles/traffic_<workload>.json and exit")
    args = ap.parse_args(argv)

    if args.traffic:
        from hadamard_rotation_amd import workloads as W
        w = W.WORKLOADS[args.workload]
        if len(args.traffic) not in (2, 3):
            ap.error("--traffic takes the FETCH_SIZE and WRITE_SIZE results and "
                     "optionally the read-request counters")
        out = write_traffic(args.workload, args.traffic[0], args.traffic[1],
                            copy_bytes_for(w.bytes_per_call()),
                            args.traffic[2] if len(args.traffic) == 3 else None)
        print(json.dumps(out))
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not "
              "supported (rows are independent, so a multi-GPU run is the one-GPU "
              "throughput per shard)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import hadamard_rotation_amd as hq
    from hadamard_rotation_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    hq.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.attention_only:
        stream = torch.cuda.current_stream()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        print(json.dumps({"decode_attention": time_attention(dev, stream, ev0, ev1,
                                                             calls=args.steps)}))
        return 0
    w = W.WORKLOADS[args.workload]
    data = W.generate(args.workload, seed=42)
    raw, s_np = data[w.tensors[0]], data["s"]
    rows, n = raw.shape
    g = args.group
    bytes_call = w.bytes_per_call(rows, g)
    sets = min(64, max(4, int(np.ceil(3 * LLC_BYTES / bytes_call))))

    x_dtype = {W.F32: torch.float32, W.BF16: torch.bfloat16, W.F16: torch.float16}[w.x_dtype]
    if w.x_dtype == W.F32:
        x0 = torch.from_numpy(raw).to(dev)
    else:
        x0 = torch.from_numpy(raw.view(np.int16)).to(dev).view(x_dtype)
    s = torch.from_numpy(s_np).to(dev)
    sd = torch.float32 if w.scale_dtype == W.F32 else torch.float16
    xs = [x0.clone() for _ in range(sets)]
    cw = n // 2 if w.bits == 4 else n
    cdt = torch.uint8 if w.bits == 4 else torch.int8
    codes = [torch.empty((rows, cw), dtype=cdt, device=dev) for _ in range(sets)]
    sshape = (rows,) if g is None else (rows, n // g)
    scales = [torch.empty(sshape, dtype=sd, device=dev) for _ in range(sets)]
    del x0
    stream = torch.cuda.current_stream()

    def step(i):
        k = i % sets
        if g is None:
            hq.hq_rotate_quant(xs[k], s, w.b, w.bits, sd, codes=codes[k], scales=scales[k],
                               stream=stream)
        else:
            hq.hq_rotate_quant_grouped(xs[k], s, w.b, g, w.bits, sd, codes=codes[k],
                                       scales=scales[k], stream=stream)

    def inverse(k, y):
        if g is None:
            hq.hq_dequant_rotate_inv(codes[k], scales[k], s, w.b, w.bits, y=y, stream=stream)
        else:
            hq.hq_dequant_rotate_inv_grouped(codes[k], scales[k], s, w.b, g, w.bits, y=y,
                                             stream=stream)

    # untimed settle phase (at least SETTLE_S seconds of the same calls)
    t_settle = time.perf_counter()
    i = 0
    while time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(20):
            step(i)
            i += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    sec = ms / 1e3
    value = bytes_call * args.steps / sec / 1e9
    ms_step = ms / args.steps
    launch_us = ms_step * 1e3  # one kernel launch per step

    traffic, traffic_req = load_traffic(args.workload) if g is None else (None, None)
    if g is not None:
        metric = f"fused rotate+quant GB/s, workload {args.workload}, group {g}"
    elif args.workload == "hidden_4096":
        metric = METRIC
    else:
        metric = f"fused rotate+quant GB/s, workload {args.workload}"
    out = {
        "metric": metric,
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: {w.description}",
            "rows": rows, "n": n, "b": w.b, "bits": w.bits, "group": g or n,
            "x_dtype": W.DTYPE_NAMES[w.x_dtype], "scale_dtype": W.DTYPE_NAMES[w.scale_dtype],
            "bytes_per_call": bytes_call, "buffer_sets": sets,
            "rows_per_s": round(rows * args.steps / sec, 1),
            "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(bytes_call / (launch_us * 1e-6) / 1e9, 3),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(bytes_call / (launch_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_from_requests": traffic_req,
            "kernel_us": round(launch_us, 3),
        },
    }

    if not args.no_extras:
        # inverse path on the same workload: codes + scales -> fp32 rows
        ys = [torch.empty((rows, n), dtype=torch.float32, device=dev) for _ in range(2)]
        t0 = time.perf_counter()  # the same untimed settle phase as the headline
        i = 0
        while time.perf_counter() - t0 < SETTLE_S:
            for _ in range(10):
                inverse(i % sets, ys[i % 2])
                i += 1
            torch.cuda.synchronize()
        ev0.record(stream)
        k_inv = max(10, args.steps // 4)
        for i in range(k_inv):
            inverse(i % sets, ys[i % 2])
        ev1.record(stream)
        torch.cuda.synchronize()
        inv_s = ev0.elapsed_time(ev1) / 1e3 / k_inv
        n_sc = 1 if g is None else n // g
        inv_bytes = rows * (cw + (4 if w.scale_dtype == W.F32 else 2) * n_sc + 4 * n)
        out["inverse"] = {"us_per_call": round(inv_s * 1e6, 3),
                          "GB/s": round(inv_bytes / inv_s / 1e9, 3),
                          "bytes_per_call": inv_bytes, "out_dtype": "f32"}
        del ys
    if not args.no_extras or args.copy:
        # same-byte-count device copy as the achievable-bandwidth reference
        nb = copy_bytes_for(bytes_call)
        src = [torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(sets)]
        dst = [torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(sets)]
        for i in range(5):
            dst[i % sets].copy_(src[i % sets])
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(50):
            dst[i % sets].copy_(src[i % sets])
        ev1.record(stream)
        torch.cuda.synchronize()
        cs = ev0.elapsed_time(ev1) / 1e3 / 50
        out["copy_reference"] = {"bytes_moved": 2 * nb, "GB/s": round(2 * nb / cs / 1e9, 3)}
        del src, dst
    if not args.no_extras:
        out["append"] = time_append(dev, stream, ev0, ev1)
        out["decode_attention"] = time_attention(dev, stream, ev0, ev1)
        # every workload of the path at its full size (the headline's own
        # line is the one above), and the full 11008-point Paley rotation
        del xs, codes, scales
        torch.cuda.empty_cache()
        out["workloads"] = [time_workload(name, dev, stream, ev0, ev1)
                            for name in W.ORDER + ("ffn_11008_full",) if name != args.workload]

    if not args.no_cpu_baseline and g is None:
        out["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
