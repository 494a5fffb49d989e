"""Seeded synthetic inputs for the paged split-KV attention path.

This module only draws and lays out inputs: sequence lengths, a scattered page
assignment, Q, the K/V pools in their storage dtype, and the new tokens of an
append step with their slot mapping. It holds none of the attention arithmetic,
so that the GPU library and the float64 oracle can both be fed from it.

Workloads follow the five shapes this library is measured on:

1. ``tiny``      1 sequence of 100 positions, 1 head, D=64, fp32 pool of 16
                 pages x 16 positions, one 256-position split.
2. ``gqa``       batch 32, lengths uniform in [1, 4096], 32 query / 8 KV heads,
                 D=128, bf16 pool (16-position pages, shuffled), one new token
                 appended per sequence before the read.
3. ``verify``    4 sequences x 16 causal query rows over 32768 keys, 24 / 4
                 heads, D=256, bf16 pool (16-position pages).
4. ``chunk``     1 sequence, 128 causal query rows over 32768 keys, 24 / 4
                 heads, D=256, fp8 e4m3 pool with per-tensor fp32 scales, bf16 Q.
5. ``long``      batch 8, lengths log-uniform in [1024, 131072], 64 / 8 heads,
                 D=128, bf16 pool with 32-position fragmented pages, K stored x4
                 (peaked logits), one new token appended per sequence first.
6. ``windows``   the verify shape with windows of 16, 12, 8 and 4 rows for its
                 four sequences (Q padded to 16 rows).
7. ``mla``       the batched decode shape with latent-attention head sizes: q and
                 k rows of 192, v rows of 128 (value head dim independent of the
                 query/key one), 16 query heads each with its own KV head,
                 lengths uniform in [1, 4096], bf16, one new token appended.

Random streams: ``numpy.random.SeedSequence(seed).spawn(8)`` in the fixed roles
[lengths, page order, q, k, v, new k, new v, spare]; the default seed of a
workload is its number.  Storage-dtype rounding uses torch's CPU casts
(round-to-nearest-even), so both consumers read the very same stored bits.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

# storage dtype names used throughout the Python side
F32, BF16, FP8 = "f32", "bf16", "fp8"

WORKLOADS = {
    1: dict(name="tiny", batch=1, q_heads=1, kv_heads=1, head_dim=64, kv_dtype=F32,
            q_dtype=F32, page_tokens=16, q_rows=1, causal=False,
            lens=("fixed", 100), num_pages=16, max_pages=16,
            split=("fixed", 256, 1), append=False, k_mult=1.0),
    2: dict(name="gqa", batch=32, q_heads=32, kv_heads=8, head_dim=128, kv_dtype=BF16,
            q_dtype=BF16, page_tokens=16, q_rows=1, causal=False,
            lens=("uniform", 1, 4096), split=("rule", 256, 64), append=True, k_mult=1.0),
    3: dict(name="verify", batch=4, q_heads=24, kv_heads=4, head_dim=256, kv_dtype=BF16,
            q_dtype=BF16, page_tokens=16, q_rows=16, causal=True,
            lens=("fixed", 32768), split=("rows",), append=False, k_mult=1.0),
    4: dict(name="chunk", batch=1, q_heads=24, kv_heads=4, head_dim=256, kv_dtype=FP8,
            q_dtype=BF16, page_tokens=16, q_rows=128, causal=True,
            lens=("fixed", 32768), split=("rows",), append=False, k_mult=1.0),
    5: dict(name="long", batch=8, q_heads=64, kv_heads=8, head_dim=128, kv_dtype=BF16,
            q_dtype=BF16, page_tokens=32, q_rows=1, causal=False,
            lens=("loguniform", 1024, 131072), split=("rule", 256, 64), append=True,
            k_mult=4.0),
    6: dict(name="windows", batch=4, q_heads=24, kv_heads=4, head_dim=256, kv_dtype=BF16,
            q_dtype=BF16, page_tokens=16, q_rows=16, causal=True,
            lens=("fixed", 32768), split=("rows",), append=False, k_mult=1.0,
            windows=(16, 12, 8, 4)),
    7: dict(name="mla", batch=32, q_heads=16, kv_heads=16, head_dim=192, v_head_dim=128,
            kv_dtype=BF16, q_dtype=BF16, page_tokens=16, q_rows=1, causal=False,
            lens=("uniform", 1, 4096), split=("rule", 256, 64), append=True, k_mult=1.0),
}

_TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}
FP8_MAX = 448.0


@dataclasses.dataclass
class PagedCase:
    """One batch of synthetic inputs (all tensors on the CPU)."""
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    q_rows: int
    causal: bool
    kv_dtype: str
    q_dtype: str
    page_tokens: int
    num_pages: int
    max_pages: int
    seq_lens: np.ndarray            # [B] int32, window rows and appended token included
    block_table: np.ndarray         # [B, max_pages] int32, -1 padded
    q: torch.Tensor                 # [B, H_q, W, D] fp32 or bf16
    k_pool: torch.Tensor            # [P, H_kv, T, D] fp32 / bf16 / uint8 (e4m3 codes)
    v_pool: torch.Tensor            # [P, H_kv, T, Dv]
    k_scale: float                  # fp32 dequant factor (1.0 unless fp8)
    v_scale: float
    softmax_scale: float            # an fp32 value: 1/sqrt(D) rounded to fp32
    split_policy: tuple             # ("fixed", S, n), ("rule", positions, cap) or ("rows",)
    new_k: Optional[torch.Tensor] = None     # [N_tok, H_kv, D] fp32
    new_v: Optional[torch.Tensor] = None     # [N_tok, H_kv, Dv] fp32
    slot_mapping: Optional[np.ndarray] = None  # [N_tok] int32
    rows_per_seq: Optional[np.ndarray] = None  # [B] int32 window rows (ragged windows)
    v_head_dim: int = 0                     # Dv, the V pool's head dim (0: = head_dim)

    def __post_init__(self):
        if not self.v_head_dim:
            self.v_head_dim = self.head_dim

    @property
    def rows(self) -> int:
        return self.batch * self.q_heads * self.q_rows

    def kv_bytes(self) -> int:
        """Algorithmic K/V bytes one read pass touches (each element once)."""
        esz = {F32: 4, BF16: 2, FP8: 1}[self.kv_dtype]
        return (int(self.seq_lens.astype(np.int64).sum()) * self.kv_heads *
                (self.head_dim + self.v_head_dim) * esz)


def _draw_lens(spec, batch, rng):
    kind = spec[0]
    if kind == "fixed":
        return np.full(batch, spec[1], dtype=np.int64)
    if kind == "uniform":                      # ("uniform", lo, hi[, step]): multiples of step
        lo, hi = spec[1], spec[2]
        step = spec[3] if len(spec) > 3 else 1
        return rng.integers(-(-lo // step), hi // step + 1, size=batch, dtype=np.int64) * step
    if kind == "loguniform":
        lo, hi = spec[1], spec[2]
        x = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=batch)))
        return np.clip(x, lo, hi).astype(np.int64)
    raise ValueError(kind)


def _normals(rng, n, mult=1.0):
    x = rng.standard_normal(n, dtype=np.float32)
    if mult != 1.0:
        x *= np.float32(mult)
    return torch.from_numpy(x)


def _store(x: torch.Tensor, dtype: str):
    """Round fp32 values to the storage dtype; returns (stored tensor, fp32 scale)."""
    if dtype in _TORCH_DTYPE:
        return x.to(_TORCH_DTYPE[dtype]), 1.0
    amax = float(x.abs().max()) if x.numel() else 1.0
    scale = float(np.float32(max(amax, 1e-30) / FP8_MAX))
    codes = (x / torch.tensor(scale, dtype=torch.float32)).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8), scale


def nan_bits(dtype: str, like: torch.Tensor):
    if dtype == F32:
        return torch.tensor(float("nan"), dtype=torch.float32)
    if dtype == BF16:
        return torch.tensor(float("nan"), dtype=torch.bfloat16)
    return torch.tensor(0x7F, dtype=torch.uint8)


def make_case(workload: int, seed: Optional[int] = None, poison: bool = True,
              **override) -> PagedCase:
    """Draw one batch of the given workload.

    ``override`` may replace any field of the workload table (e.g. ``batch``,
    ``lens=("uniform", 1, 700)``) to get oracle-sized versions of a shape.
    ``poison`` fills every slot that no sequence position uses (unused pages,
    tails of last pages, and the slots an append is about to fill) with NaN,
    so a read of the wrong slot shows up in the output.
    """
    cfg = dict(WORKLOADS[workload])
    cfg.update(override)
    if seed is None:
        seed = workload
    ss = np.random.SeedSequence(seed).spawn(8)
    r_len, r_page, r_q, r_k, r_v, r_nk, r_nv, _ = [np.random.default_rng(s) for s in ss]

    B, Hq, Hkv, D = cfg["batch"], cfg["q_heads"], cfg["kv_heads"], cfg["head_dim"]
    Dv = int(cfg.get("v_head_dim") or D)
    T, W = cfg["page_tokens"], cfg["q_rows"]
    lens = _draw_lens(cfg["lens"], B, r_len)
    lens = np.maximum(lens, W if cfg["causal"] else 1)
    pages_per_seq = -(-lens // T)
    used = int(pages_per_seq.sum())
    P = int(cfg.get("num_pages") or math.ceil(1.25 * used))
    P = max(P, used)
    max_pages = int(cfg.get("max_pages") or max(1, int(pages_per_seq.max())))
    order = r_page.permutation(P).astype(np.int64)
    bt = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(pages_per_seq[b])
        bt[b, :n] = order[off:off + n]
        off += n

    kf = _normals(r_k, P * Hkv * T * D, cfg["k_mult"]).view(P, Hkv, T, D)
    vf = _normals(r_v, P * Hkv * T * Dv).view(P, Hkv, T, Dv)
    q = _normals(r_q, B * Hq * W * D).view(B, Hq, W, D).to(_TORCH_DTYPE[cfg["q_dtype"]])

    new_k = new_v = slots = None
    if cfg["append"]:
        new_k = _normals(r_nk, B * Hkv * D, cfg["k_mult"]).view(B, Hkv, D)
        new_v = _normals(r_nv, B * Hkv * Dv).view(B, Hkv, Dv)
        pos = lens - 1
        slots = (bt[np.arange(B), pos // T].astype(np.int64) * T + pos % T).astype(np.int32)

    k_pool, k_scale = _store(kf, cfg["kv_dtype"])
    v_pool, v_scale = _store(vf, cfg["kv_dtype"])
    del kf, vf

    if poison:
        live = np.zeros((P, T), dtype=bool)
        for b in range(B):
            for j in range(int(pages_per_seq[b])):
                n_in = min(T, int(lens[b]) - j * T)
                live[bt[b, j], :n_in] = True
        if slots is not None:
            for s in slots:
                live[s // T, s % T] = False
        dp, dt = np.nonzero(~live)
        if dp.size:
            nb = nan_bits(cfg["kv_dtype"], k_pool)
            ip, it = torch.from_numpy(dp), torch.from_numpy(dt)
            k_pool[ip, :, it, :] = nb
            v_pool[ip, :, it, :] = nb

    split_policy = tuple(cfg["split"])

    return PagedCase(
        name=cfg["name"], batch=B, q_heads=Hq, kv_heads=Hkv, head_dim=D, q_rows=W,
        causal=bool(cfg["causal"]), kv_dtype=cfg["kv_dtype"], q_dtype=cfg["q_dtype"],
        page_tokens=T, num_pages=P, max_pages=max_pages,
        seq_lens=lens.astype(np.int32), block_table=bt, q=q,
        k_pool=k_pool, v_pool=v_pool, k_scale=k_scale, v_scale=v_scale,
        softmax_scale=float(np.float32(1.0 / math.sqrt(D))),
        split_policy=split_policy, new_k=new_k, new_v=new_v, slot_mapping=slots,
        rows_per_seq=(np.array(cfg["windows"], dtype=np.int32) if cfg.get("windows") else None),
        v_head_dim=Dv)


def describe(workload: int) -> str:
    c = WORKLOADS[workload]
    dv = f"/{c['v_head_dim']}" if c.get("v_head_dim") else ""
    return (f"{c['name']}: B={c['batch']} Hq={c['q_heads']} Hkv={c['kv_heads']} D={c['head_dim']}{dv} "
            f"W={c['q_rows']} causal={c['causal']} kv={c['kv_dtype']} T={c['page_tokens']} "
            f"lens={c['lens']}")
