"""Benchmark of the grouped-query attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle S] [--no-cpu-baseline] [--no-sweep]

Headline step: one causal bf16 prefill of the workload B=1, h_q=32, h_kv=8,
d_h=128, T=4096 (fp32 output), whose throughput is reported as TFLOP/s of
algorithmic work (4 h_q d_h FLOPs per visible query/key pair).  The decode
half of the path is timed in the same run on B=64, h_q=32, h_kv=8, d_h=128,
T=8192 (HBM GB/s of algorithmic bytes: the visible K/V plus Q and O), and,
unless --no-sweep, on the MHA / GQA / MQA sweep at T=32000 and the ragged
append + decode workload, over a contiguous cache and over 64-row pages.  Inputs are synthetic (seeded N(0,1), bf16) and
already resident in device memory when each timed region starts.

Prints ONE JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak
FLUSH_BYTES = 512 << 20        # larger than the 256 MB Infinity Cache
METRIC = "GQA decode HBM GB/s (% peak) + causal prefill TFLOP/s (% MFMA peak), 1 GPU"
# Untimed back-to-back launches before each timed region.  Coming out of idle (even
# 0.2 s of it) the GPU needs ~40 ms of sustained load before its clocks settle: the
# prefill kernel takes 0.16-0.17 ms per launch for the first ~200 launches and
# 0.138 ms after.  Every leg starts after seconds of host-side input generation, so
# each one settles first and the timed steps measure the sustained rate.
SETTLE_S = 0.3

# decode workloads timed besides the headline ones: (workload, page size or 0 for a contiguous cache)
SWEEP = [("decode_mha_B8_T32000", 0), ("decode_gqa_B8_T32000", 0), ("decode_mqa_B8_T32000", 0),
         ("ragged_append_decode_B32", 0), ("ragged_append_decode_B32", 64)]

# HBM traffic of each timed row's kernel(s), from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
# (profiles/traffic.json, written by --write-traffic): row -> (bench.py arguments that run
# it alone, the kernels counted and how, the sources those kernels are built from).  A
# row's entry counts only while the hash of its sources matches.
_COMMON = ["internal.h", "mfma_common.h"]
TRAFFIC_ROWS = {
    "prefill_causal_bf16_T4096": (["--only", "prefill"], ("prefill_bf16_kernel<128, false, false>", "mean"),
                                  ["prefill_bf16.hip", "rope_common.h", *_COMMON]),
    "decode_bf16_B64_T8192": (["--only", "decode"], ("decode_main", "mean"),
                              ["decode_bf16.hip", "rope_common.h", *_COMMON]),
    **{(n + (f"_paged{ps}" if ps else "")): (["--only", "sweep", "--workload", n + (f":{ps}" if ps else "")],
                                             ("decode_main", "mean"), ["decode_bf16.hip", "rope_common.h", *_COMMON])
       for n, ps in SWEEP},
    "prefill_causal_bf16_T4096_qk_rope": (["--only", "rope"], ("rope_heads_kernel", "largest_grid"),
                                          ["rope.hip", "rope_common.h", "internal.h"]),
    "prefill_causal_bf16_T4096_backward": (["--only", "backward"],
                                           (("bwd_dkdv", "bwd_dq_kernel"), "sum_of_means"),
                                           ["backward_bf16.hip", *_COMMON]),
}
COPY_ROW = (["--only", "copy"], ("copyBuffer", "mean"))
TRAFFIC_COUNTERS = ("FETCH_SIZE", "WRITE_SIZE")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "grouped_query_attention_prefill_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(row: str):
    """HBM bytes per launch of the row's kernel(s) from profiles/traffic.json, if the
    entry was taken from the current sources; else None."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            e = json.load(f).get("rows", {}).get(row)
    except (OSError, ValueError):
        return None
    if not e or e.get("source_hash") != source_hash(TRAFFIC_ROWS[row][2]):
        return None
    return e.get("hbm_bytes_per_launch")


def traffic_commands(out_dir: str):
    """The rocprofv3 runs behind profiles/traffic.json: one counter per run (FETCH_SIZE
    alone fills three of the four TCC counters), each bench.py row alone."""
    runs = [("copy", COPY_ROW[0])] + [(row, spec[0]) for row, spec in TRAFFIC_ROWS.items()]
    cmds = []
    for counter in TRAFFIC_COUNTERS:
        for row, args in runs:
            d = os.path.join(out_dir, f"{counter.lower()}_{row}")
            cmds.append((counter, row, d, ["rocprofv3", "--pmc", counter, "--output-format", "csv", "-d", d,
                                           "-o", "p", "--", "python3", os.path.join(ROOT, "bench.py"), *args,
                                           "--steps", "3", "--warmup", "1", "--settle", "0"]))
    return cmds


def _per_dispatch(csv_dir: str, counter: str):
    """{kernel name: [(grid size, value per dispatch), ...]} from one rocprofv3 --pmc run."""
    import csv
    import glob

    files = glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {csv_dir}")
    per = {}
    for path in files:
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    per.setdefault(r["Kernel_Name"], []).append((int(r["Grid_Size"]), float(r["Counter_Value"])))
    return per


def _select(per, how):
    """KiB per launch of the selected kernel(s) and the names counted."""
    what, mode = how

    def match(name, key):
        if key == "decode_main":
            return "gqa::" in name and "decode" in name and "_kernel" in name and "combine" not in name
        return key in name

    if mode == "sum_of_means":
        total, names = 0.0, []
        for key in what:
            hits = [n for n in per if match(n, key)]
            if len(hits) != 1:
                raise SystemExit(f"expected one kernel matching {key!r}, found {hits}")
            vals = [v for _, v in per[hits[0]]]
            total += sum(vals) / len(vals)
            names.append(hits[0])
        return total, names
    hits = [n for n in per if match(n, what)]
    if len(hits) != 1:
        raise SystemExit(f"expected one kernel matching {what!r}, found {hits}")
    rows = per[hits[0]]
    if mode == "largest_grid":
        g = max(gs for gs, _ in rows)
        rows = [(gs, v) for gs, v in rows if gs == g]
    vals = [v for _, v in rows]
    return sum(vals) / len(vals), hits


def write_traffic(out_dir: str):
    """profiles/traffic.json and profiles/hbm_traffic_counters.md from the runs of traffic_commands()."""
    import subprocess

    dirs = {(c, row): d for c, row, d, _ in traffic_commands(out_dir)}
    fetch_copy, _ = _select(_per_dispatch(dirs[("FETCH_SIZE", "copy")], "FETCH_SIZE"), COPY_ROW[1])
    write_copy, _ = _select(_per_dispatch(dirs[("WRITE_SIZE", "copy")], "WRITE_SIZE"), COPY_ROW[1])
    n = 1 << 30   # the copy reads and writes 1 GiB
    fs, ws = n / (fetch_copy * 1024), n / (write_copy * 1024)
    try:
        rev = subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT, capture_output=True,
                             text=True).stdout.strip()
    except OSError:
        rev = ""
    out = {"_calibration": {"copy_bytes_read": n, "copy_bytes_written": n, "copy_FETCH_SIZE_KiB": fetch_copy,
                            "copy_WRITE_SIZE_KiB": write_copy, "fetch_scale": fs, "write_scale": ws},
           "source_revision": rev, "rows": {}}
    table = []
    for row, (args, how, files) in TRAFFIC_ROWS.items():
        fk, names = _select(_per_dispatch(dirs[("FETCH_SIZE", row)], "FETCH_SIZE"), how)
        wk, _ = _select(_per_dispatch(dirs[("WRITE_SIZE", row)], "WRITE_SIZE"), how)
        rd, wr = round(fk * 1024 * fs), round(wk * 1024 * ws)
        out["rows"][row] = {"kernels": names, "counted": how[1], "FETCH_SIZE_KiB": fk, "WRITE_SIZE_KiB": wk,
                            "read": rd, "written": wr, "hbm_bytes_per_launch": rd + wr,
                            "source_hash": source_hash(files)}
        table.append((row, names, fk, wk, rd, wr))
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    cmds = traffic_commands("<out>")
    lines = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             f"Source revision: `{rev}`.  Written by `python bench.py --write-traffic <out>` from the runs below "
             "(one counter per run, each bench.py row alone; `<repo>` is the repository root).", "",
             "```"]
    for _, _, _, c in cmds:
        lines.append("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 " +
                     " ".join(c).replace(ROOT, "<repo>"))
    lines += ["```", "",
              f"Calibration: a plain 1 GiB device copy (`bench.py --only copy`) reports FETCH_SIZE = "
              f"{fetch_copy:.1f} KiB and WRITE_SIZE = {write_copy:.1f} KiB per dispatch, so FETCH_SIZE is scaled "
              f"by {fs:.4f} and WRITE_SIZE by {ws:.4f}.", "",
              "| bench row | kernel(s) counted | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes read (scaled) | "
              "HBM bytes written (scaled) | total per launch |", "|---|---|---|---|---|---|---|"]
    for row, names, fk, wk, rd, wr in table:
        short = " + ".join("`" + nm.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0] + "`"
                           for nm in names)
        lines.append(f"| {row} | {short} | {fk:.1f} | {wk:.1f} | {rd:,} | {wr:,} | {rd + wr:,} |")
    with open(os.path.join(ROOT, "profiles", "hbm_traffic_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(out["rows"], indent=1))


def settle(fn, seconds: float):
    """Call fn back to back, untimed, for at least `seconds` of wall time."""
    import torch

    t0 = time.perf_counter()
    n = 0
    while seconds > 0:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
        n += 8
        if time.perf_counter() - t0 >= seconds:
            break
    return n


def time_calls(fn, steps: int, warmup: int, flush=None):
    """Run fn warmup+steps times; HIP events around every timed call on the current stream.

    Returns (wall seconds of the timed region, list of per-call milliseconds).
    """
    import torch

    for _ in range(warmup):
        fn()
    settle((lambda: (flush(), fn())) if flush is not None else fn, SETTLE_S)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        if flush is not None:
            flush()
        evs[i][0].record()
        fn()
        evs[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [a.elapsed_time(b) for a, b in evs]


def spread(per):
    """Median and minimum of per-call milliseconds (the mean is the reported value)."""
    t = sorted(per)
    return {"ms_median": round(t[len(t) // 2], 5), "ms_min": round(t[0], 5)}


def time_region(fn, steps: int, warmup: int):
    """Run fn warmup+steps times back to back; one HIP event pair on the current stream
    around the timed launches.  Returns (wall seconds of the timed region, average ms per
    launch).  For compute-bound kernels whose inputs need no cache eviction: the average
    is the sustained per-launch duration, which is what the kernel trace reports."""
    import torch

    for _ in range(warmup):
        fn()
    settle(fn, SETTLE_S)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1) / steps


def to_dev(x, dtype):
    import numpy as np
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def ints(x):
    import numpy as np
    import torch

    return torch.as_tensor(np.asarray(x, dtype=np.int32)).cuda()


# ---------------------------------------------------------------------------------------- prefill
def bench_prefill(steps, warmup):
    import torch

    from grouped_query_attention_prefill_amd import inputs, ops

    w = inputs.WORKLOADS["prefill_causal_bf16_T4096"]
    log(f"[bench] generating {w.name}")
    x = inputs.make_workload(w)
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    out = torch.empty((w.B, w.h_q, w.T, w.d_h), dtype=torch.float32, device="cuda")
    # algorithmic work: 4 d_h FLOPs (QK and PV) per visible (query, key) pair per query head
    flops = 4 * w.B * w.h_q * w.d_h * (w.T * (w.T + 1) // 2)
    fn = lambda: ops.gqa_prefill(q, k, v, causal=True, out=out)
    log(f"[bench] timing {w.name}: {warmup} warmup + {steps} steps")
    wall, kern_ms = time_region(fn, steps, warmup)
    ms_step = wall * 1e3 / steps
    achieved = flops / (kern_ms * 1e-3) / 1e12
    value = flops / (ms_step * 1e-3) / 1e12
    res = {
        "workload": w, "x": x, "flops": flops, "ms_per_step": ms_step, "kernel_ms": kern_ms,
        "value": value, "achieved": achieved,
    }
    del q, k, v, out
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------------------- decode
def decode_bytes(w, seq_lens, appended: bool):
    # visible K and V rows (bf16), plus Q (bf16) and O (fp32); the append adds its two rows written
    kv = sum(2 * w.h_kv * int(L) * w.d_h * 2 for L in seq_lens)
    qo = w.B * w.h_q * w.d_h * (2 + 4)
    app = 2 * w.B * w.h_kv * w.d_h * 2 * 2 if appended else 0   # read new rows + write them
    return kv + qo + app


def paginate_on_device(cache, page_size, seed):
    """Scatter a contiguous cache (B, h_kv, T_cap, d) into a page pool in shuffled order.

    Returns (pool (B * T_cap / page_size, h_kv, page_size, d), block_table (B, T_cap / page_size) int32).
    """
    import numpy as np
    import torch

    B, h, T, d = cache.shape
    mp = T // page_size
    perm = torch.as_tensor(np.random.default_rng(seed).permutation(B * mp), device=cache.device)
    pages = cache.view(B, h, mp, page_size, d).permute(0, 2, 1, 3, 4).reshape(B * mp, h, page_size, d)
    pool = torch.empty_like(pages)
    pool[perm] = pages
    return pool, perm.view(B, mp).to(torch.int32).contiguous()


def bench_decode(name, steps, warmup, flush_buf, page_size=0):
    import numpy as np
    import torch

    from grouped_query_attention_prefill_amd import inputs, ops

    w = inputs.WORKLOADS[name]
    log(f"[bench] generating {w.name}")
    x = inputs.make_workload(w)
    qd = to_dev(x["q"], "bf16")
    kd, vd = to_dev(x["k_cache"], "bf16"), to_dev(x["v_cache"], "bf16")
    del x["k_cache"], x["v_cache"]
    bt = None
    if page_size:
        kd, bt = paginate_on_device(kd, page_size, w.seed)
        vd, _ = paginate_on_device(vd, page_size, w.seed)
        torch.cuda.empty_cache()
    sl, qp = ints(x["seq_lens"]), ints(x["q_pos"])
    msl = int(x["seq_lens"].max())
    out = torch.empty((w.B, w.h_q, 1, w.d_h), dtype=torch.float32, device="cuda")
    ws_bytes = ops.gqa_decode_workspace_bytes(w.B, w.h_q, w.h_kv, w.T, w.d_h, torch.bfloat16)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    appended = w.path == "append_decode"
    if page_size:
        dec = lambda: ops.gqa_decode_paged(qd, kd, vd, bt, sl, q_pos=qp, max_seq_len=msl, out=out, workspace=ws)
    else:
        dec = lambda: ops.gqa_decode(qd, kd, vd, sl, q_pos=qp, max_seq_len=msl, out=out, workspace=ws)
    if appended:
        # one call per step: the decode kernel writes the new rows and reads them in place
        kn, vn, wp = to_dev(x["k_new"], "bf16"), to_dev(x["v_new"], "bf16"), ints(x["write_pos"])
        if page_size:
            fn = lambda: ops.gqa_append_decode_paged(qd, kd, vd, kn, vn, bt, wp, sl, q_pos=qp, max_seq_len=msl,
                                                     out=out, workspace=ws)
        else:
            fn = lambda: ops.gqa_append_decode(qd, kd, vd, kn, vn, wp, sl, q_pos=qp, max_seq_len=msl, out=out,
                                               workspace=ws)
    else:
        fn = dec
    # read (not write) a buffer larger than the Infinity Cache: evicts the inputs
    # without leaving dirty lines to be written back inside the next timed call
    flush = lambda: flush_buf.sum()
    log(f"[bench] timing {w.name}: {warmup} warmup + {steps} steps (Infinity Cache flushed before each)")
    wall, per = time_calls(fn, steps, warmup, flush=flush)
    kern_ms = sum(per) / len(per)
    nbytes = decode_bytes(w, x["seq_lens"], appended)
    gbs = nbytes / (kern_ms * 1e-3) / 1e9
    wname = w.name + (f"_paged{page_size}" if page_size else "")
    res = {
        "workload": wname, "B": w.B, "h_q": w.h_q, "h_kv": w.h_kv, "d_h": w.d_h, "T_cap": w.T,
        "max_seq_len": msl, "algorithmic_bytes": nbytes, "ms_per_call": round(kern_ms, 5), **spread(per),
        "value": round(gbs, 1), "unit": "GB/s",
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(wname)},
        "kernels": "decode split (append fused) + combine" if appended else "decode split + combine",
    }
    if page_size:
        res["page_size"] = page_size
    del qd, kd, vd, out, ws, bt
    torch.cuda.empty_cache()
    res["read_floor"] = read_floor(nbytes, steps, warmup, flush, kern_ms)
    return res, x


_FLOOR_LIB = None


def read_floor(nbytes, steps, warmup, flush, row_ms):
    """Time one streaming read of nbytes (libgqa_readfloor.so) the way a decode row is
    timed: inputs evicted from the Infinity Cache, HIP events around each call.  The
    row's time over this floor says how far the row is from what reading its bytes
    once costs on this GPU."""
    import ctypes
    import os

    import torch

    global _FLOOR_LIB
    if _FLOOR_LIB is None:
        path = os.path.join(ROOT, "grouped_query_attention_prefill_amd", "libgqa_readfloor.so")
        lib = ctypes.CDLL(path)
        lib.gqa_read_floor.restype = ctypes.c_int
        lib.gqa_read_floor.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
        lib.gqa_read_floor_grid.restype = ctypes.c_int
        _FLOOR_LIB = lib
    lib = _FLOOR_LIB
    n = (nbytes + 15) // 16 * 16
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    out = torch.empty(max(lib.gqa_read_floor_grid(), 1), dtype=torch.int32, device="cuda")

    def fn():
        st = lib.gqa_read_floor(buf.data_ptr(), n, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == 0, "gqa_read_floor failed"

    _, per = time_calls(fn, steps, warmup, flush=flush)
    ms = sum(per) / len(per)
    del buf, out
    torch.cuda.empty_cache()
    return {"kernel": "streaming read of the row's algorithmic bytes", "ms_per_call": round(ms, 5),
            "GB/s": round(n / (ms * 1e-3) / 1e9, 1), "row_over_floor": round(row_ms / ms, 3)}


# ---------------------------------------------------------------------------------------- backward
def bench_backward(steps, warmup):
    """Gradients of the prefill workload: delta, dK/dV and dQ kernels per call.

    Algorithmic work: five products over the visible (query, key) pairs -- S, dP,
    dV, dK, dQ -- 2 d_h FLOPs each per pair and query head, i.e. 2.5 times the
    forward's 4 d_h; the second recomputation of S and dP is overhead, not counted.
    """
    import torch

    from grouped_query_attention_prefill_amd import inputs, ops

    w = inputs.WORKLOADS["prefill_causal_bf16_T4096"]
    shape_q, shape_kv = (w.B, w.h_q, w.T, w.d_h), (w.B, w.h_kv, w.T, w.d_h)
    q = torch.randn(shape_q, device="cuda").to(torch.bfloat16)
    k = torch.randn(shape_kv, device="cuda").to(torch.bfloat16)
    v = torch.randn(shape_kv, device="cuda").to(torch.bfloat16)
    do = torch.randn(shape_q, device="cuda").to(torch.bfloat16)
    o, lse = ops.gqa_prefill_lse(q, k, v)
    dq = torch.empty(shape_q, dtype=torch.float32, device="cuda")
    dk = torch.empty(shape_kv, dtype=torch.float32, device="cuda")
    dv = torch.empty(shape_kv, dtype=torch.float32, device="cuda")
    ws = torch.empty(ops.gqa_prefill_backward_workspace_bytes(w.B, w.h_q, w.T), dtype=torch.uint8, device="cuda")
    fn = lambda: ops.gqa_prefill_backward(q, k, v, o, do, lse, dq=dq, dk=dk, dv=dv, workspace=ws)
    log(f"[bench] timing the backward of {w.name}")
    wall, ms = time_region(fn, steps, warmup)
    flops = 10 * w.B * w.h_q * w.d_h * (w.T * (w.T + 1) // 2)
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": w.name + "_backward", "algorithmic_flops": flops, "ms_per_call": round(ms, 5),
            "value": round(tf, 2), "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": measured_traffic(w.name + "_backward")},
            "kernels": "dQ (with delta) + dK/dV (traffic: the two kernels' bytes summed)", "grad_dtype": "fp32"}


# ---------------------------------------------------------------------------------------- rotary encoding
def bench_rope(steps, warmup, flush_buf):
    """Rotary encoding of the prefill workload's Q and K (out of place, bf16): HBM bytes
    are the rows read plus the rows written."""
    import torch

    from grouped_query_attention_prefill_amd import inputs, ops

    w = inputs.WORKLOADS["prefill_causal_bf16_T4096"]
    q = torch.randn((w.B, w.h_q, w.T, w.d_h), device="cuda").to(torch.bfloat16)
    k = torch.randn((w.B, w.h_kv, w.T, w.d_h), device="cuda").to(torch.bfloat16)
    qo, ko = torch.empty_like(q), torch.empty_like(k)

    def fn():
        ops.gqa_rope_qk(q, k, q_out=qo, k_out=ko)

    log(f"[bench] timing rotary encoding of {w.name} Q and K")
    wall, per = time_calls(fn, steps, warmup, flush=lambda: flush_buf.sum())
    ms = sum(per) / len(per)
    nbytes = 2 * (q.numel() + k.numel()) * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    # the prefill with Q rotated inside the kernel, against gqa_rope on Q then the prefill
    v = torch.randn((w.B, w.h_kv, w.T, w.d_h), device="cuda").to(torch.bfloat16)
    out = torch.empty((w.B, w.h_q, w.T, w.d_h), dtype=torch.float32, device="cuda")
    flops = 4 * w.B * w.h_q * w.d_h * (w.T * (w.T + 1) // 2)
    log(f"[bench] timing {w.name} with Q rotated inside the prefill kernel, and rotated beforehand")
    _, fused_ms = time_region(lambda: ops.gqa_prefill_rope(q, ko, v, out=out), steps, warmup)
    _, sep_ms = time_region(lambda: (ops.gqa_rope(q, out=qo), ops.gqa_prefill(qo, ko, v, out=out)), steps, warmup)
    del v, out
    return {"workload": w.name + "_qk_rope", "rows": w.B * (w.h_q + w.h_kv) * w.T, "d_h": w.d_h,
            "algorithmic_bytes": nbytes, "ms_per_call": round(ms, 5), **spread(per), "value": round(gbs, 1),
            "unit": "GB/s",
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic(w.name + "_qk_rope")},
            "kernels": "rope (Q and K, one launch)",
            "prefill_rope_fused": {"ms_per_call": round(fused_ms, 5),
                                   "tflops": round(flops / (fused_ms * 1e-3) / 1e12, 2),
                                   "rope_then_prefill_ms": round(sep_ms, 5)}}


# ---------------------------------------------------------------------------------------- CPU oracle
def cpu_baseline_prefill(res, min_s=10.0, max_s=30.0):
    """The float64 oracle on the prefill workload: whole query heads at full T, repeated
    over passes until at least min_s seconds of CPU work (stopping at max_s)."""
    import numpy as np

    import oracle
    from grouped_query_attention_prefill_amd import inputs

    w, x = res["workload"], res["x"]
    r = w.h_q // w.h_kv
    cores = len(os.sched_getaffinity(0))
    log(f"[bench] timing the CPU oracle on {w.name} (>= {min_s:.0f} s, {cores} cores)")
    heads, flops, t0 = 0, 0, time.perf_counter()
    while True:
        for a in range(w.h_q):
            g = a // r
            qa = inputs.to_f32(x["q"][:, a:a + 1], "bf16").astype(np.float64)
            kg = inputs.to_f32(x["k"][:, g:g + 1], "bf16").astype(np.float64)
            vg = inputs.to_f32(x["v"][:, g:g + 1], "bf16").astype(np.float64)
            oracle.attention(qa, kg, vg, causal=True)
            heads += 1
            flops += 4 * w.d_h * w.T * (w.T + 1) // 2
            if time.perf_counter() - t0 > max_s:
                break
        if time.perf_counter() - t0 >= min_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{heads} query-head passes over {w.name} (all {w.h_q} heads per pass, full T={w.T}, "
                      f"float64, materialized S and P) in {dt:.1f} s", "seconds": round(dt, 2)}


def cpu_baseline_decode(x, name, n_seq=2):
    import numpy as np

    import oracle
    from grouped_query_attention_prefill_amd import inputs

    w = inputs.WORKLOADS[name]
    dt, nbytes = 0.0, 0
    for b in range(n_seq):
        L = int(x["seq_lens"][b])
        kb = inputs.normal_row(w.seed, "k", b, (w.h_kv, w.T, w.d_h), "bf16")[None, :, :L]
        vb = inputs.normal_row(w.seed, "v", b, (w.h_kv, w.T, w.d_h), "bf16")[None, :, :L]
        qb, kb, vb = (inputs.to_f32(a, "bf16").astype(np.float64) for a in (x["q"][b:b + 1], kb, vb))
        t1 = time.perf_counter()
        oracle.attention(qb, kb, vb, causal=True, q_pos=np.array([[x["q_pos"][b]]]), kv_len=np.array([L]))
        dt += time.perf_counter() - t1
        nbytes += 2 * w.h_kv * L * w.d_h * 2
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle", "sample": f"{n_seq} of {w.B} sequences of {name}, {dt:.2f} s of oracle time"}


def bench_copy(steps, warmup):
    """Plain 1 GiB device copy: the reference kernel that calibrates HBM byte counters."""
    import torch

    n = 1 << 30
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    wall, per = time_calls(lambda: b.copy_(a), steps, warmup)
    ms = sum(per) / len(per)
    return {"workload": "device_copy_1GiB", "bytes_read": n, "bytes_written": n, "ms_per_call": round(ms, 5),
            "value": round(2 * n / (ms * 1e-3) / 1e9, 1), "unit": "GB/s"}


def main():
    global SETTLE_S
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed back-to-back launches before each timed region (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "sweep", "copy", "rope", "backward"],
                    help="run one part alone (for profiler runs); prints that part's JSON")
    ap.add_argument("--traffic-commands", metavar="OUT",
                    help="print the rocprofv3 counter runs behind profiles/traffic.json (output under OUT), one a line")
    ap.add_argument("--write-traffic", metavar="OUT",
                    help="write profiles/traffic.json and hbm_traffic_counters.md from those runs' output under OUT")
    ap.add_argument("--workload", action="append", default=None,
                    help="with --only sweep: run only this sweep entry (NAME, or NAME:PAGE for a paged cache); "
                         "may be repeated")
    args = ap.parse_args()
    if args.traffic_commands:
        for _, _, _, c in traffic_commands(args.traffic_commands):
            print(" ".join(c))
        return
    if args.write_traffic:
        write_traffic(args.write_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from grouped_query_attention_prefill_amd import ops

    ops.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    steps, warmup = max(1, args.steps), max(0, args.warmup)
    SETTLE_S = max(0.0, args.settle)

    if args.only == "copy":
        print(json.dumps(bench_copy(steps, warmup)), flush=True)
        return
    if args.only == "backward":
        print(json.dumps(bench_backward(steps, warmup)), flush=True)
        return
    if args.only == "rope":
        flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        print(json.dumps(bench_rope(steps, warmup, flush_buf)), flush=True)
        return
    if args.only == "prefill":
        r = bench_prefill(steps, warmup)
        print(json.dumps({k: v for k, v in r.items() if k not in ("workload", "x")}), flush=True)
        return
    if args.only in ("decode", "sweep"):
        flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        runs = [("decode_bf16_B64_T8192", 0)] if args.only == "decode" else SWEEP
        if args.only == "sweep" and args.workload:
            want = [(w.split(":")[0], int(w.split(":")[1]) if ":" in w else 0) for w in args.workload]
            unknown = [w for w in want if w not in SWEEP]
            if unknown:
                raise SystemExit(f"unknown sweep entries {unknown}; choose from {SWEEP}")
            runs = want
        print(json.dumps([bench_decode(n, steps, warmup, flush_buf, ps)[0] for n, ps in runs]), flush=True)
        return

    pre = bench_prefill(steps, warmup)
    flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    dec, dec_x = bench_decode("decode_bf16_B64_T8192", steps, warmup, flush_buf)
    sweep = []
    if not args.no_sweep:
        for name, ps in SWEEP:
            r, _ = bench_decode(name, steps, warmup, flush_buf, ps)
            sweep.append(r)
    rope = bench_rope(steps, warmup, flush_buf)
    bwd = bench_backward(steps, warmup)
    del flush_buf
    torch.cuda.empty_cache()

    w = pre["workload"]
    line = {
        "metric": METRIC,
        "value": round(pre["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": round(pre["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q/K/V rounded to bf16, resident in HBM",
        "config": {"workload": w.name, "B": w.B, "h_q": w.h_q, "h_kv": w.h_kv, "d_h": w.d_h, "T": w.T,
                   "causal": True, "out_dtype": "fp32", "algorithmic_flops": pre["flops"]},
        "roofline": {"bound": "mfma", "achieved": round(pre["achieved"], 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(pre["achieved"] / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(w.name),
                     "kernel_ms": round(pre["kernel_ms"], 5)},
        "decode": dec,
        "decode_sweep": sweep,
        "rope": rope,
        "backward": bwd,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_prefill(pre)
        dec["cpu_baseline"] = cpu_baseline_decode(dec_x, "decode_bf16_B64_T8192")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
