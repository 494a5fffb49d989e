"""Benchmark of the paged split-KV decode step on one MI355X.

A step is one pass of the whole path over one batch: the append of the new
tokens (workloads with an append), the split partials and the fixed-order
merge, all through the C ABI on one stream.  Inputs are seeded synthetic
tensors resident in HBM before timing starts.  Before every timed step a
1 GiB buffer is read so the K/V bytes come from HBM, not from the L2s or the
256 MB last-level cache; the step itself is timed with HIP events on the
stream the kernels run on.

Prints one JSON line: value = algorithmic K/V bytes / step time (GB/s),
plus the roofline of the dominant kernel (the split partial) and the oracle
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
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def flops_of(case) -> float:
    """QK^T and PV multiply-adds over the keys each row sees (2 flops each)."""
    W, D = case.q_rows, case.head_dim
    tot = 0.0
    for L in case.seq_lens.astype(np.int64):
        if case.causal:
            keys = sum(max(0, int(L) - W + r + 1) for r in range(W))
        else:
            keys = int(L) * W
        tot += keys
    return tot * case.q_heads * 2 * 2 * D


def cpu_baseline(case, budget_s: float = 12.0):
    """The float64 oracle (append + attention) over whole sequences until the budget."""
    import oracle
    t0 = time.perf_counter()
    kp, vp = case.k_pool, case.v_pool
    if case.new_k is not None:
        kp, vp, _ = oracle.case_append(case)
    t_app = time.perf_counter() - t0
    rows_per_seq = case.q_heads * case.q_rows
    done_bytes = 0
    n_seq = 0
    esz = {"f32": 4, "bf16": 2, "fp8": 1}[case.kv_dtype]
    t_attn = 0.0
    for b in range(case.batch):
        t1 = time.perf_counter()
        oracle.attention(case.q, case.q_dtype, kp, vp, case.kv_dtype, case.block_table,
                         case.seq_lens, case.softmax_scale, case.causal, case.k_scale,
                         case.v_scale, rows=(b * rows_per_seq, (b + 1) * rows_per_seq))
        t_attn += time.perf_counter() - t1
        done_bytes += int(case.seq_lens[b]) * case.kv_heads * case.head_dim * esz * 2
        n_seq += 1
        if t_attn + t_app >= budget_s:
            break
    secs = t_attn + t_app * (n_seq / case.batch)
    return {
        "value": done_bytes / secs / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"sequences 0..{n_seq - 1} of {case.batch} (all their query rows), "
                  f"append share pro rata; {secs:.2f} s of float64 work",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush-mib", type=int, default=1024)
    args = ap.parse_args()

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
    if has_append:
        new_k, new_v = case.new_k.to(dev), case.new_v.to(dev)
        slots = torch.from_numpy(case.slot_mapping).to(dev)
    if case.split_policy[0] == "fixed":
        n_split, split = case.split_policy[2], case.split_policy[1]
    else:
        n_split, split = nb.nbx_paged_decode_plan(int(case.seq_lens.max()), case.split_policy[1],
                                                  case.split_policy[2])
    rows, D = case.rows, case.head_dim
    o_part = torch.empty(rows, n_split, D, device=dev)
    m_part = torch.empty(rows, n_split, device=dev)
    l_part = torch.empty(rows, n_split, device=dev)
    out = torch.empty(case.batch, case.q_heads, case.q_rows, D, device=dev)
    flush = torch.ones(args.flush_mib * (1 << 18), device=dev) if args.flush_mib else None
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if has_append:
            nb.nbx_paged_kv_append(new_k, new_v, kp, vp, slots, dev_err=err)
        if ev is not None:
            ev[0].record(stream)
        nb.nbx_paged_decode_partial(q, kp, vp, bt, lens, case.softmax_scale, split, n_split,
                                    o_part, m_part, l_part, causal=case.causal, dev_err=err)
        if ev is not None:
            ev[1].record(stream)
        nb.nbx_paged_decode_merge(o_part, m_part, l_part, out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        raise RuntimeError(f"device error flags {int(err.item())}")

    K = args.steps
    ev_step = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(K)]
    ev_part = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(K)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(K):
        if flush is not None:
            flush.sum()                      # read 1 GiB: evicts K/V from L2 and MALL
        ev_step[i][0].record(stream)
        step(ev_part[i])
        ev_step[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    step_ms = np.array([a.elapsed_time(b) for a, b in ev_step])
    part_ms = np.array([a.elapsed_time(b) for a, b in ev_part])

    # warm steps (no flush) for context
    for i in range(K):
        ev_step[i][0].record(stream)
        step()
        ev_step[i][1].record(stream)
    torch.cuda.synchronize()
    warm_ms = np.array([a.elapsed_time(b) for a, b in ev_step])

    kv = case.kv_bytes()
    t_step = float(step_ms.mean()) * 1e-3
    t_part = float(part_ms.mean()) * 1e-3
    value = kv / t_step / 1e9
    achieved = kv / t_part / 1e9
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
                   "n_split": n_split, "split_size": split, "rows": rows,
                   "seed": args.seed if args.seed is not None else args.workload},
        "us_per_step": round(float(step_ms.mean()) * 1e3, 2),
        "us_per_step_p10_p90": [round(float(np.percentile(step_ms, 10)) * 1e3, 2),
                                round(float(np.percentile(step_ms, 90)) * 1e3, 2)],
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "warm_us_per_step": round(float(warm_ms.mean()) * 1e3, 2),
        "wall_s_timed_loop": round(wall, 4),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "split partial", "us_per_launch": round(t_part * 1e6, 2),
        },
    }
    if case.kv_dtype in MFMA_PEAK_TFLOPS and case.q_rows > 1:
        fl = flops_of(case)
        res["mfma"] = {"flops_per_launch": fl, "achieved_tflops": round(fl / t_part / 1e12, 2),
                       "peak_bf16_tflops": MFMA_PEAK_TFLOPS["bf16"],
                       "frac_of_bf16_peak": round(fl / t_part / 1e12 / MFMA_PEAK_TFLOPS["bf16"], 4)}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
