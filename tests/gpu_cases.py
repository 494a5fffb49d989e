"""Helpers for the GPU tests: move a synthetic case to the device and run the
library on it through the C ABI (via the ctypes binding)."""
from __future__ import annotations

import numpy as np
import torch

from paged_split_kv_append_amd import binding as nb
from paged_split_kv_append_amd import synth

TOL = {"f32": 1e-5, "bf16": 2e-3, "fp8": 2e-2}


class DevCase:
    def __init__(self, case: synth.PagedCase, device="cuda"):
        self.case = case
        self.q = case.q.to(device)
        self.k = case.k_pool.to(device)
        self.v = case.v_pool.to(device)
        self.bt = torch.from_numpy(case.block_table).to(device)
        self.lens = torch.from_numpy(case.seq_lens).to(device)
        self.new_k = case.new_k.to(device) if case.new_k is not None else None
        self.new_v = case.new_v.to(device) if case.new_v is not None else None
        self.slots = (torch.from_numpy(case.slot_mapping).to(device)
                      if case.slot_mapping is not None else None)
        self.err = torch.zeros(1, dtype=torch.int32, device=device)
        self.kb = self.vb = None               # per-page bounds (fixed-shift softmax)

    def pools(self):
        return (nb.KVPool(self.k, self.case.k_scale, self.kb),
                nb.KVPool(self.v, self.case.v_scale, self.vb))

    def attach_bounds(self, lens=None):
        """Allocate per-page bounds for both pools and compute them with
        nbx_paged_kv_bounds over the rows of `lens` (default: the case's lengths)."""
        P, H = self.k.shape[0], self.k.shape[1]
        self.kb = torch.full((P, H), -1.0, device=self.k.device)   # overwritten by the call
        self.vb = torch.full((P, H), -1.0, device=self.k.device)
        lens_d = self.lens if lens is None else torch.as_tensor(
            np.asarray(lens, dtype=np.int32)).to(self.k.device)
        kp, vp = self.pools()
        nb.nbx_paged_kv_bounds(kp, vp, self.bt, lens_d, dev_err=self.err)

    def detach_bounds(self):
        self.kb = self.vb = None

    def plan(self):
        return nb.case_plan(self.case)

    def append(self):
        kp, vp = self.pools()
        if self.k.shape[3] == self.v.shape[3]:
            nb.nbx_paged_kv_append(self.new_k, self.new_v, kp, vp, self.slots, dev_err=self.err)
        else:                                  # pools of different head dims: one call each
            nb.nbx_paged_kv_append(self.new_k, None, kp, None, self.slots, dev_err=self.err)
            nb.nbx_paged_kv_append(self.new_v, None, vp, None, self.slots, dev_err=self.err)

    def decode(self, n_split=None, split_size=None, out_dtype=torch.float32):
        if n_split is None:
            n_split, split_size = self.plan()
        c = self.case
        kp, vp = self.pools()
        rows = c.rows
        ws = torch.empty(nb.nbx_paged_decode_workspace_bytes(rows, n_split, c.v_head_dim),
                         dtype=torch.uint8, device=self.q.device)
        out = torch.empty(c.batch, c.q_heads, c.q_rows, c.v_head_dim, dtype=out_dtype,
                          device=self.q.device)
        nb.nbx_paged_decode(self.q, kp, vp, self.bt, self.lens, c.softmax_scale, split_size,
                            n_split, ws, out, causal=c.causal, dev_err=self.err)
        return out.reshape(rows, c.v_head_dim)

    def step(self, new_k=None, new_v=None, n_split=None, split_size=None,
             out_dtype=torch.float32):
        """nbx_paged_decode_step; new_k / new_v [batch, n_new, kv_heads, D / Dv] (default:
        the case's own new tokens, one per sequence)."""
        if n_split is None:
            n_split, split_size = self.plan()
        c = self.case
        if new_k is None and self.new_k is not None:
            new_k, new_v = self.new_k.unsqueeze(1), self.new_v.unsqueeze(1)
        kp, vp = self.pools()
        dev = self.q.device
        ws = torch.empty(nb.nbx_paged_decode_workspace_bytes(c.rows, n_split, c.v_head_dim),
                         dtype=torch.uint8, device=dev)
        out = torch.empty(c.batch, c.q_heads, c.q_rows, c.v_head_dim, dtype=out_dtype,
                          device=dev)
        nb.nbx_paged_decode_step(self.q, kp, vp, self.bt, self.lens, c.softmax_scale, split_size,
                                 n_split, ws, out, new_k=new_k, new_v=new_v, causal=c.causal,
                                 dev_err=self.err)
        return out.reshape(c.rows, c.v_head_dim)

    def partial(self, n_split=None, split_size=None):
        if n_split is None:
            n_split, split_size = self.plan()
        c = self.case
        kp, vp = self.pools()
        dev = self.q.device
        o = torch.empty(c.rows, n_split, c.v_head_dim, dtype=torch.float32, device=dev)
        m = torch.empty(c.rows, n_split, dtype=torch.float32, device=dev)
        l = torch.empty(c.rows, n_split, dtype=torch.float32, device=dev)
        nb.nbx_paged_decode_partial(self.q, kp, vp, self.bt, self.lens, c.softmax_scale,
                                    split_size, n_split, o, m, l, causal=c.causal,
                                    dev_err=self.err)
        return o, m, l

    def err_bits(self) -> int:
        return int(self.err.item())


def max_abs(gpu: torch.Tensor, ref: np.ndarray) -> float:
    g = gpu.detach().double().cpu().numpy().reshape(ref.shape)
    return float(np.max(np.abs(g - ref))) if ref.size else 0.0
