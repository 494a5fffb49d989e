"""Benchmark of the paged split-KV decode step on one MI355X.

A step is one pass of the whole path over one batch: the append of the new
tokens (workloads with an append), the split partials and the fixed-order
merge, all through the C ABI on one stream.  Inputs are seeded synthetic
tensors resident in HBM before timing starts.  Before every timed step a
1 GiB buffer is read so the K/V bytes come from HBM, not from the L2s or the
256 MB last-level cache; the step itself is timed with HIP events on the
stream the kernels run on.

Prints one JSON line: value = algorithmic K/V bytes / step time (GB/s),
plus the roofline of the dominant kernel (the split partial), the practical
read ceiling (the same bytes read as a plain stream and as random 4 KB blocks
by the probes of libnbx_read_ceiling.so, after the same flush) and the oracle
timed on the host cores over a bounded sample of the same workload.
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

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}
METRIC = "paged split-KV decode: K/V GB/s (% of HBM peak) + us/step, B=32 ctx 4k"
WORKLOAD_TEXT = {
    1: "tiny paged decode: B=1, 1/1 heads, D=64, fp32 pool 16 pages x 16, L=100, one 256 split",
    2: "batched GQA decode: B=32, L~U[1,4096], 32/8 heads, D=128, bf16 pool T=16 shuffled, "
       "1 query row, splits 256 capped at 64, append 1 token per sequence first",
    3: "verify window: 4 sequences x 16 causal rows, 24/4 heads, D=256, 32768 keys, bf16 T=16",
    4: "prompt chunk: 1 sequence, 128 causal rows, 24/4 heads, D=256, 32768 keys, fp8 e4m3 "
       "pool, bf16 Q",
    5: "long mixed decode: B=8, L log-uniform [1024,131072], 64/8 heads, D=128, bf16 T=32, "
       "K x4, append 1 then read",
    6: "ragged verify windows: 4 sequences with 16, 12, 8 and 4 causal rows, 24/4 heads, D=256, "
       "32768 keys, bf16 T=16",
    7: "latent-attention decode: B=32, L~U[1,4096], 16/16 heads, q/k head dim 192, v head dim "
       "128, bf16 pool T=16 shuffled, 1 query row, append 1 token per sequence first",
}


class HipEvent:
    """A HIP event recorded with a device-scope release, so recording it costs no
    system-scope cache write-back between the kernels it brackets."""
    _hip = None
    RELEASE_TO_DEVICE = 0x40000000

    def __init__(self):
        import ctypes
        if HipEvent._hip is None:
            import torch  # noqa: F401  (loads the HIP runtime)
            HipEvent._hip = ctypes.CDLL("libamdhip64.so")
            HipEvent._hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            HipEvent._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                          ctypes.c_void_p, ctypes.c_void_p]
        self._ct = ctypes
        self.ev = ctypes.c_void_p()
        st = HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.ev),
                                                   ctypes.c_uint(self.RELEASE_TO_DEVICE))
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {st}")

    def record(self, stream_ptr: int):
        st = HipEvent._hip.hipEventRecord(self.ev, self._ct.c_void_p(stream_ptr))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed: {st}")

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = self._ct.c_float()
        st = HipEvent._hip.hipEventElapsedTime(self._ct.byref(ms), self.ev, end.ev)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {st}")
        return float(ms.value)

    def __del__(self):
        if HipEvent._hip is not None and self.ev:
            HipEvent._hip.hipEventDestroy(self.ev)


# Kernel sources whose text decides the split partial's memory traffic: the
# headers every matrix-core partial includes, and the file of the kernel that
# serves the shape (multi-row for more than 16 rows per KV head).
_CSRC = "paged_split_kv_append_amd/csrc/"
_COMMON_SOURCES = (_CSRC + "partial_common.h", _CSRC + "mfma_common.h", _CSRC + "device_common.h")


def partial_sources(workload: int):
    from paged_split_kv_append_amd import synth
    cfg = synth.WORKLOADS[workload]
    if cfg["kv_dtype"] == synth.F32:
        return (_CSRC + "partial_valu.hip", _CSRC + "device_common.h")
    rows = cfg["q_heads"] // cfg["kv_heads"] * cfg["q_rows"]
    kernel = "partial_multirow.hip" if rows > 16 else "partial_mfma.hip"
    return (_CSRC + kernel,) + _COMMON_SOURCES


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace collapsed, so that a
    comment edit does not count as a kernel change."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def partial_source_hash(workload: int) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in partial_sources(workload):
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_file(workload: int, fused: bool) -> str:
    tag = "step" if fused else "split_partial"
    return os.path.join(ROOT, "profiles", f"traffic_{tag}_workload{workload}.txt")


def load_traffic(workload: int, fused: bool):
    """HBM bytes per launch of the split partial from the committed counter summary,
    or None when there is none or the kernel sources changed since it was taken."""
    path = traffic_file(workload, fused)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("partial_source_sha256_16") != partial_source_hash(workload):
        return None
    return int(kv["traffic_bytes_per_launch"])


def _counter_means(d: str, name_part: str):
    """{kernel name: (dispatches, mean counter value)} from a rocprofv3 --pmc csv."""
    import csv
    import glob
    out = {}
    for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(fn) as f:
            for r in csv.DictReader(f):
                if name_part in r["Kernel_Name"]:
                    key = (r["Kernel_Name"], r["Grid_Size"])
                    n, t = out.get(key, (0, 0.0))
                    out[key] = (n + 1, t + float(r["Counter_Value"]))
    return {k: (n, t / n) for k, (n, t) in out.items()}


def summarize_counters(fetch_dir: str, write_dir: str, copy_mib: int, workload: int):
    """Per-launch HBM traffic of the split partial from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the same
    counter reads for a plain device copy of copy_mib MiB (reads and writes
    copy_mib MiB)."""
    copy_kib = copy_mib * 1024.0

    def one(d, counter):
        copies = [v for (name, grid), v in _counter_means(d, "copyBuffer").items()
                  if v[1] > copy_kib / 8]
        if not copies:
            raise SystemExit(f"no copy kernel of {copy_mib} MiB in {d}")
        factor = copy_kib / copies[0][1]
        parts = [(name, v) for (name, grid), v in _counter_means(d, "nbx::").items()
                 if "persistent" in name or "mfma" in name or "valu" in name]
        return factor, copies[0][1], parts

    ff, fcopy, fparts = one(fetch_dir, "FETCH_SIZE")
    wf, wcopy, wparts = one(write_dir, "WRITE_SIZE")
    fk = max(fparts, key=lambda t: t[1][1])
    wk = [v for n, v in wparts if n == fk[0]][0]
    fetch_b = fk[1][1] * ff * 1024
    write_b = wk[1] * wf * 1024
    lines = [
        f"# split partial HBM traffic, workload {workload}",
        f"kernel: {fk[0]}",
        f"dispatches_counted: {fk[1][0]}",
        f"copy_reference_mib: {copy_mib}",
        f"fetch_size_copy_kib: {fcopy:.2f}",
        f"fetch_factor: {ff:.5f}",
        f"write_size_copy_kib: {wcopy:.2f}",
        f"write_factor: {wf:.5f}",
        f"fetch_size_kib_per_dispatch: {fk[1][1]:.2f}",
        f"write_size_kib_per_dispatch: {wk[1]:.2f}",
        f"fetch_bytes_per_launch: {int(fetch_b)}",
        f"write_bytes_per_launch: {int(write_b)}",
        f"traffic_bytes_per_launch: {int(fetch_b + write_b)}",
        f"partial_source_sha256_16: {partial_source_hash(workload)}",
    ]
    return "\n".join(lines)


def summarize_trace(trace_dir: str):
    """The kernel-stats table of a rocprofv3 --kernel-trace --stats run, in us."""
    import csv
    import glob
    fn = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)[0]
    rows = list(csv.DictReader(open(fn)))
    out = [f"{'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'pct':>6}  kernel"]
    for r in rows:
        name = r["Name"]
        if len(name) > 90:
            name = name[:87] + "..."
        out.append(f"{int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>9.2f} "
                   f"{float(r['MinNs']) / 1e3:>9.2f} {float(r['MaxNs']) / 1e3:>9.2f} "
                   f"{float(r['Percentage']):>6.2f}  {name}")
    return "\n".join(out)


def summarize_ceiling(trace_dir: str, workload: int):
    """Kernel-trace times of the read-ceiling probe in a rocprofv3 --kernel-trace
    run of bench.py: its dispatches in launch order, in runs of one grid size
    (address order at 1024, 2048, 4096 workgroups, then random order at the same
    grids), each run's first dispatch left out as its warm-up."""
    import csv
    import glob
    from paged_split_kv_append_amd import synth
    nbytes = -(-synth.make_case(workload, poison=False).kv_bytes() // 4096) * 4096
    fn = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)[0]
    rows = [r for r in csv.DictReader(open(fn)) if "block_read_kernel" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    runs = []
    for r in rows:
        grid = int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"])
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if not runs or runs[-1][0] != grid:
            runs.append((grid, []))
        runs[-1][1].append(us)
    out = [f"{'order':>10} {'workgroups':>10} {'dispatches':>10} {'median_us':>10} {'GB/s':>8}"]
    for i, (grid, us) in enumerate(runs):
        order = "address" if i < len(runs) // 2 else "random"
        med = float(np.median(us[1:] if len(us) > 1 else us))
        out.append(f"{order:>10} {grid:>10} {len(us) - 1:>10} {med:>10.2f} "
                   f"{nbytes / (med * 1e-6) / 1e9:>8.1f}")
    return "\n".join(out)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def flops_of(case) -> float:
    """QK^T and PV multiply-adds over the keys each row sees (2 flops each)."""
    D = case.head_dim + case.v_head_dim
    tot = 0.0
    for b, L in enumerate(case.seq_lens.astype(np.int64)):
        W = int(case.rows_per_seq[b]) if case.rows_per_seq is not None else case.q_rows
        if case.causal:
            keys = sum(max(0, int(L) - W + r + 1) for r in range(W))
        else:
            keys = int(L) * W
        tot += keys
    return tot * case.q_heads * 2 * D


def cpu_baseline(case, budget_s: float = 10.0):
    """The float64 oracle (append + attention) over the whole batch, pass after pass,
    until about budget_s seconds of work; a pass cut short by the budget counts the
    sequences it finished and its share of the append."""
    import oracle
    esz = {"f32": 4, "bf16": 2, "fp8": 1}[case.kv_dtype]
    done_bytes, n_seq, passes, secs = 0, 0, 0, 0.0
    while secs < budget_s:
        t0 = time.perf_counter()
        kp, vp = case.k_pool, case.v_pool
        if case.new_k is not None:
            kp, vp, _ = oracle.case_append(case)
        t_app = time.perf_counter() - t0
        t_attn, done = 0.0, 0
        for b in range(case.batch):
            t1 = time.perf_counter()
            wb = int(case.rows_per_seq[b]) if case.rows_per_seq is not None else case.q_rows
            if wb > 0:                          # the sequence alone, with its own window
                oracle.attention(case.q[b:b + 1, :, :wb].contiguous(), case.q_dtype, kp, vp,
                                 case.kv_dtype, case.block_table[b:b + 1],
                                 case.seq_lens[b:b + 1], case.softmax_scale, case.causal,
                                 case.k_scale, case.v_scale)
            t_attn += time.perf_counter() - t1
            done_bytes += (int(case.seq_lens[b]) * case.kv_heads *
                           (case.head_dim + case.v_head_dim) * esz)
            done += 1
            if secs + t_app + t_attn >= budget_s:
                break
        secs += t_attn + t_app * (done / case.batch)
        n_seq += done
        passes += 1
        if done < case.batch:                  # the budget ended inside this pass
            break
    return {
        "value": done_bytes / secs / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{n_seq} sequence reads over {passes} pass(es) of the batch of "
                  f"{case.batch} (all query rows of each; the append's share pro rata); "
                  f"{secs:.2f} s of float64 work",
    }


def read_ceiling(kv_bytes: int, flush_caches, stream_ptr: int, reps: int = 15):
    """The practical ceiling of a read of kv_bytes on this GPU: the same bytes
    (rounded up to 4 KB) read by one probe kernel as 4 KB blocks, one wave per
    block, in address order (a plain stream) and in a seeded random order (the
    decode reads 16-position pages of one KV head, 4 KB at D = 128 bf16), after
    the same cache flush as the step and timed with HIP events; for each order
    the best median GB/s over grids of 1024, 2048 and 4096 workgroups."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "paged_split_kv_append_amd", "libnbx_read_ceiling.so")
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is missing: build it with "
                                "`python -m paged_split_kv_append_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32 = ctypes.c_void_p, ctypes.c_int32
    lib.nbx_ceiling_block_read.argtypes = [P, P, I32, I32, P, P]
    dev = torch.device("cuda:0")
    nblocks = -(-kv_bytes // 4096)
    raw = torch.ones(nblocks * 4096 + 4096, dtype=torch.uint8, device=dev)
    base = (raw.data_ptr() + 4095) // 4096 * 4096          # 4 KB aligned, nblocks * 4096 bytes
    gen = torch.Generator().manual_seed(4096)
    orders = {"stream": torch.arange(nblocks, dtype=torch.int32, device=dev),
              "random_4k": torch.randperm(nblocks, generator=gen).to(torch.int32).to(dev)}
    grids = (1024, 2048, 4096)
    sink = torch.zeros(max(grids) * 256, dtype=torch.int32, device=dev)

    def run(order, wgs):
        st = lib.nbx_ceiling_block_read(P(base), P(order.data_ptr()), nblocks, wgs,
                                        P(sink.data_ptr()), P(stream_ptr))
        if st != 0:
            raise RuntimeError(f"read-ceiling launch: status {st}")

    res = {"bytes": nblocks * 4096, "reps": reps, "timing": "HIP events around the probe "
           "launch after the flush, median of reps, best grid"}
    for kind, order in orders.items():
        best = None
        for wgs in grids:
            run(order, wgs)
            evs = [(HipEvent(), HipEvent()) for _ in range(reps)]
            for a, b in evs:
                flush_caches()
                a.record(stream_ptr)
                run(order, wgs)
                b.record(stream_ptr)
            torch.cuda.synchronize()
            med = float(np.median([a.elapsed_ms(b) for a, b in evs]))
            if best is None or med < best[0]:
                best = (med, wgs)
        res[kind + "_read_gbs"] = round(nblocks * 4096 / (best[0] * 1e-3) / 1e9, 1)
        res[kind + "_read_us_median"] = round(best[0] * 1e3, 2)
        res[kind + "_workgroups"] = best[1]
    del raw, orders, sink
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush-mib", type=int, default=1024)
    ap.add_argument("--unfused", action="store_true",
                    help="time the append, partial and merge as three calls instead of the "
                         "single-launch step")
    ap.add_argument("--bounds", action="store_true",
                    help="attach per-page K/V bounds to the pools (fixed-shift softmax), "
                         "computed by nbx_paged_kv_bounds before timing")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (a known-size "
                         "reference for the profiler's byte counters)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the read-ceiling probes (plain stream and random 4 KB blocks)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print the kernel table of a rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--summarize-ceiling", metavar="DIR",
                    help="print the read-ceiling probe's kernel times from a rocprofv3 "
                         "--kernel-trace run of bench.py (of --workload)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the split partial's traffic from FETCH_SIZE / WRITE_SIZE runs "
                         "made with --copy-mib")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.summarize_ceiling:
        print(summarize_ceiling(args.summarize_ceiling, args.workload))
        return
    if args.summarize_counters:
        print(summarize_counters(*args.summarize_counters, args.copy_mib or 256, args.workload))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    from paged_split_kv_append_amd import binding as nb
    from paged_split_kv_append_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.perf_counter()
    case = synth.make_case(args.workload, seed=args.seed, poison=False)
    log(f"generated {case.name} in {time.perf_counter() - t0:.1f}s; kv bytes {case.kv_bytes()}")

    q = case.q.to(dev)
    k = case.k_pool.to(dev)
    v = case.v_pool.to(dev)
    bt = torch.from_numpy(case.block_table).to(dev)
    lens = torch.from_numpy(case.seq_lens).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    kp, vp = nb.KVPool(k, case.k_scale), nb.KVPool(v, case.v_scale)
    has_append = case.new_k is not None
    if args.bounds:
        kp.bounds = torch.zeros(k.shape[0], k.shape[1], device=dev)
        vp.bounds = torch.zeros(k.shape[0], k.shape[1], device=dev)
        held = case.seq_lens - 1 if has_append else case.seq_lens   # the step appends the rest
        nb.nbx_paged_kv_bounds(kp, vp, bt, torch.from_numpy(held.astype(np.int32)).to(dev),
                               dev_err=err)
    if has_append:
        new_k, new_v = case.new_k.to(dev), case.new_v.to(dev)
        slots = torch.from_numpy(case.slot_mapping).to(dev)
    n_split, split = nb.case_plan(case)
    rows, D = case.rows, case.v_head_dim          # partial and output columns
    o_part = torch.empty(rows, n_split, D, device=dev)
    m_part = torch.empty(rows, n_split, device=dev)
    l_part = torch.empty(rows, n_split, device=dev)
    out = torch.empty(case.batch, case.q_heads, case.q_rows, D, device=dev)
    flush = torch.ones(args.flush_mib * (1 << 18), device=dev) if args.flush_mib else None
    stream_ptr = torch.cuda.current_stream().cuda_stream

    windows = case.rows_per_seq is not None
    if windows:
        rows_b = torch.from_numpy(case.rows_per_seq).to(dev)
    fused = not args.unfused and not windows
    if fused:
        ws = torch.empty(nb.nbx_paged_decode_workspace_bytes(rows, n_split, D), dtype=torch.uint8,
                         device=dev)
        o_ws, m_ws, l_ws = nb.workspace_partials(ws, rows, n_split, D)
        nk4 = new_k.unsqueeze(1) if has_append else None
        nv4 = new_v.unsqueeze(1) if has_append else None

    def step(part_ev=None):
        if fused:
            # the append runs inside the split-partial launch (one kernel), then the merge
            if part_ev is None:
                nb.nbx_paged_decode_step(q, kp, vp, bt, lens, case.softmax_scale, split, n_split,
                                         ws, out, new_k=nk4, new_v=nv4, causal=case.causal,
                                         dev_err=err)
            else:
                part_ev[0].record(stream_ptr)
                nb.nbx_paged_decode_step(q, kp, vp, bt, lens, case.softmax_scale, split, n_split,
                                         ws, None, new_k=nk4, new_v=nv4, causal=case.causal,
                                         dev_err=err)
                part_ev[1].record(stream_ptr)
                nb.nbx_paged_decode_merge(o_ws, m_ws, l_ws, out)
            return
        if has_append and case.head_dim == case.v_head_dim:
            nb.nbx_paged_kv_append(new_k, new_v, kp, vp, slots, dev_err=err)
        elif has_append:                         # pools of different head dims: one call each
            nb.nbx_paged_kv_append(new_k, None, kp, None, slots, dev_err=err)
            nb.nbx_paged_kv_append(new_v, None, vp, None, slots, dev_err=err)
        if part_ev is not None:
            part_ev[0].record(stream_ptr)
        if windows:
            nb.nbx_paged_decode_partial_windows(q, kp, vp, bt, lens, rows_b, case.softmax_scale,
                                                split, n_split, o_part, m_part, l_part,
                                                causal=case.causal, dev_err=err)
        else:
            nb.nbx_paged_decode_partial(q, kp, vp, bt, lens, case.softmax_scale, split, n_split,
                                        o_part, m_part, l_part, causal=case.causal, dev_err=err)
        if part_ev is not None:
            part_ev[1].record(stream_ptr)
        nb.nbx_paged_decode_merge(o_part, m_part, l_part, out)

    def flush_caches():
        if flush is not None:
            flush.sum()                      # read 1 GiB: evicts K/V from L2 and MALL

    if args.copy_mib:
        src = torch.ones(args.copy_mib * (1 << 18), device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        flush_caches()
        step()
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        raise RuntimeError(f"device error flags {int(err.item())}")

    K = args.steps
    # Pass 1: whole steps, events only at the step boundaries.
    ev_step = [(HipEvent(), HipEvent()) for _ in range(K)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(K):
        flush_caches()
        ev_step[i][0].record(stream_ptr)
        step()
        ev_step[i][1].record(stream_ptr)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    step_ms = np.array([a.elapsed_ms(b) for a, b in ev_step])
    # Pass 2: the same steps with events bracketing the split partial alone.
    ev_part = [(HipEvent(), HipEvent()) for _ in range(K)]
    for i in range(K):
        flush_caches()
        step(ev_part[i])
    torch.cuda.synchronize()
    part_ms = np.array([a.elapsed_ms(b) for a, b in ev_part])
    if int(err.item()) != 0:
        raise RuntimeError(f"device error flags {int(err.item())}")

    kv = case.kv_bytes()
    t_step = float(step_ms.mean()) * 1e-3
    t_part = float(part_ms.mean()) * 1e-3
    value = kv / t_step / 1e9
    achieved = kv / t_part / 1e9
    # The dominant kernel's bound: HBM unless its matrix-core time at peak
    # exceeds its K/V read time at peak (the 128-row prompt chunk).  fp8 codes
    # are widened to bf16 before the products, so the bf16 MFMA peak applies.
    traffic = None if args.bounds else load_traffic(args.workload, fused)
    kernel_name = ("split partial with the append fused in" if fused and has_append
                   else "split partial")
    mfma_info = None
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": kernel_name, "us_per_launch": round(t_part * 1e6, 2),
                "us_per_launch_median": round(float(np.median(part_ms)) * 1e3, 2)}
    if case.kv_dtype in MFMA_PEAK_TFLOPS and case.q_rows > 1:
        fl = flops_of(case)
        tflops = fl / t_part / 1e12
        mfma_info = {"flops_per_launch": fl, "achieved_tflops": round(tflops, 2),
                     "peak_bf16_tflops": MFMA_PEAK_TFLOPS["bf16"],
                     "frac_of_bf16_peak": round(tflops / MFMA_PEAK_TFLOPS["bf16"], 4)}
        if fl / (MFMA_PEAK_TFLOPS["bf16"] * 1e12) > kv / (HBM_PEAK_GBS * 1e9):
            roofline = {"bound": "mfma", "achieved": round(tflops, 2),
                        "peak": MFMA_PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                        "frac": round(tflops / MFMA_PEAK_TFLOPS["bf16"], 4), "traffic": traffic,
                        "kernel": kernel_name, "us_per_launch": round(t_part * 1e6, 2),
                        "hbm_gbs": round(achieved, 2)}
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(float(step_ms.mean()), 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8_e4m3"}[case.kv_dtype],
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "kv_bytes": kv,
                   "path": (("nbx_paged_decode_step: append fused into the split-partial "
                             "launch, then the merge" if has_append else
                             "nbx_paged_decode_step: split partials, then the merge")
                            if fused else
                            "nbx_paged_decode_partial_windows, nbx_paged_decode_merge"
                            if windows else
                            "nbx_paged_kv_append, nbx_paged_decode_partial, "
                            "nbx_paged_decode_merge"),
                   "n_split": n_split, "split_size": split, "rows": rows,
                   "softmax": ("fixed shift from per-page K/V bounds" if args.bounds
                               else "running maximum"),
                   "seed": args.seed if args.seed is not None else args.workload},
        "ms_per_step_median": round(float(np.median(step_ms)), 5),
        "us_per_step": round(float(step_ms.mean()) * 1e3, 2),
        "us_per_step_median": round(float(np.median(step_ms)) * 1e3, 2),
        "us_per_step_p10_p90": [round(float(np.percentile(step_ms, 10)) * 1e3, 2),
                                round(float(np.percentile(step_ms, 90)) * 1e3, 2)],
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "wall_s_timed_loop": round(wall, 4),
        "roofline": roofline,
    }
    if mfma_info is not None:
        res["mfma"] = mfma_info
    if not args.no_ceiling:
        ceil = read_ceiling(kv, flush_caches, stream_ptr)
        ceil["partial_frac_of_random_4k"] = round(achieved / ceil["random_4k_read_gbs"], 4)
        ceil["step_frac_of_random_4k"] = round(value / ceil["random_4k_read_gbs"], 4)
        res["practical_ceiling"] = ceil
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
