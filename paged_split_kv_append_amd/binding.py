"""ctypes binding of libnbx_paged.so (argument marshalling only).

Every function here has the name of the C entry point it calls and does no
arithmetic of its own: torch tensors are turned into device pointers, sizes
and strides, the current HIP stream is passed along, and a non-zero status is
raised as :class:`NbxError`.  The library is loaded on first use; if it has not
been built the call raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading
from dataclasses import dataclass
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnbx_paged.so")
HEADER_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "include", "nbx_paged.h")

NBX_F32, NBX_BF16, NBX_FP8_E4M3 = 0, 1, 2
NBX_ERR_SCRATCH_LIMIT = -8
STEP_SCRATCH_BYTES = 32 << 20              # NBX_STEP_SCRATCH_BYTES
DEVERR_SLOT_RANGE, DEVERR_PAGE_RANGE, DEVERR_SEQ_RANGE = 0x1, 0x2, 0x4


class NbxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_str(status)})")


class nbx_kv_pool(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("kv_heads", ctypes.c_int32),
        ("page_tokens", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("stride_page", ctypes.c_int64),
        ("stride_head", ctypes.c_int64),
        ("stride_token", ctypes.c_int64),
        ("scale", ctypes.c_float),
        ("bounds", ctypes.c_void_p),
    ]


_lock = threading.Lock()
_lib = None


def load_library():
    """Load libnbx_paged.so (raises FileNotFoundError if it was never built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise FileNotFoundError(
                    f"{LIB_PATH} is missing: build it with `python -m paged_split_kv_append_amd.build`")
            lib = ctypes.CDLL(LIB_PATH)
            P, I32, I64, F, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                  ctypes.c_size_t)
            PP = ctypes.POINTER(nbx_kv_pool)
            lib.nbx_paged_kv_append.argtypes = [P, P, I32, I64, I64, I64, PP, PP, P, P, P]
            lib.nbx_paged_kv_append.restype = ctypes.c_int
            lib.nbx_paged_decode_plan.argtypes = [I32, I32, I32, ctypes.POINTER(I32),
                                                  ctypes.POINTER(I32)]
            lib.nbx_paged_decode_plan.restype = ctypes.c_int
            lib.nbx_paged_decode_plan_rows.argtypes = [I32, I32, I32, I32, I32, I32,
                                                       ctypes.POINTER(I32), ctypes.POINTER(I32)]
            lib.nbx_paged_decode_plan_rows.restype = ctypes.c_int
            lib.nbx_paged_decode_workspace_bytes.argtypes = [I64, I32, I32]
            lib.nbx_paged_decode_workspace_bytes.restype = SZ
            lib.nbx_paged_decode_partial.argtypes = [P, I32, I32, I32, I32, I32, PP, PP, P, I32, P,
                                                     F, I32, I32, P, P, P, P, P]
            lib.nbx_paged_decode_partial.restype = ctypes.c_int
            lib.nbx_paged_decode_merge.argtypes = [P, P, P, I64, I32, I32, P, I32, P]
            lib.nbx_paged_decode_merge.restype = ctypes.c_int
            lib.nbx_paged_decode.argtypes = [P, I32, I32, I32, I32, I32, PP, PP, P, I32, P, F, I32,
                                             I32, P, SZ, P, I32, P, P]
            lib.nbx_paged_decode.restype = ctypes.c_int
            lib.nbx_paged_decode_step.argtypes = [P, I32, I32, I32, I32, I32, P, P, I32, I32, PP,
                                                  PP, P, I32, P, F, I32, I32, P, ctypes.c_size_t,
                                                  P, I32, P, P]
            lib.nbx_paged_decode_step.restype = ctypes.c_int
            lib.nbx_paged_decode_step_noalloc.argtypes = [P, I32, I32, I32, I32, I32, P, P, I32,
                                                          I32, PP, PP, P, I32, P, F, I32, I32, P,
                                                          I32, P, P]
            lib.nbx_paged_decode_step_noalloc.restype = ctypes.c_int
            lib.nbx_paged_lens_advance.argtypes = [P, I32, I32, P]
            lib.nbx_paged_lens_advance.restype = ctypes.c_int
            lib.nbx_paged_decode_partial_windows.argtypes = [P, I32, I32, I32, I32, P, I32, PP, PP,
                                                             P, I32, P, F, I32, I32, P, P, P, P,
                                                             P]
            lib.nbx_paged_decode_partial_windows.restype = ctypes.c_int
            lib.nbx_paged_kv_bounds.argtypes = [PP, PP, P, I32, P, I32, P, P]
            lib.nbx_paged_kv_bounds.restype = ctypes.c_int
            lib.nbx_status_str.argtypes = [ctypes.c_int]
            lib.nbx_status_str.restype = ctypes.c_char_p
            lib.nbx_version.restype = ctypes.c_int
            _lib = lib
    return _lib


def declared_symbols() -> list[str]:
    """Function names declared in include/nbx_paged.h."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^\S[^;(]*?\b(nbx_\w+)\s*\(", text, flags=re.M)))


def status_str(status: int) -> str:
    return load_library().nbx_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise NbxError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    """Device pointer of a GPU tensor (every array argument of the C ABI is a
    device pointer: a host tensor would hand a kernel a host address)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("every array argument must be a GPU tensor")
    return ctypes.c_void_p(t.data_ptr())


def _int32_vector(t: torch.Tensor, n: int, name: str):
    if t.dtype != torch.int32 or t.numel() != n or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor of {n} elements")


def _dev_err(t: Optional[torch.Tensor]):
    if t is not None and (t.dtype != torch.int32 or t.numel() < 1):
        raise ValueError("dev_err must be an int32 tensor of at least one element")
    return _ptr(t)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return NBX_F32
    if t.dtype == torch.bfloat16:
        return NBX_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return NBX_FP8_E4M3
    raise TypeError(f"unsupported element type {t.dtype}")


@dataclass
class KVPool:
    """A paged pool view [num_pages, kv_heads, page_tokens, head_dim] on the GPU.

    ``data`` may be any strided view whose last dim is contiguous; fp8 pools are
    uint8 (or float8_e4m3fn) tensors of E4M3FN codes with a per-tensor ``scale``.
    ``bounds``: optional contiguous fp32 [num_pages, kv_heads] tensor of per-page
    bounds (K row norms / V magnitudes) that turns on the fixed-shift softmax."""
    data: torch.Tensor
    scale: float = 1.0
    bounds: Optional[torch.Tensor] = None

    def desc(self) -> nbx_kv_pool:
        t = self.data
        if t.dim() != 4 or t.stride(3) != 1 or not t.is_cuda:
            raise ValueError("a pool is a GPU [num_pages, kv_heads, page_tokens, head_dim] view "
                             "with a contiguous last dim")
        P, H, T, D = t.shape
        bp = None
        if self.bounds is not None:
            b = self.bounds
            if b.dtype != torch.float32 or tuple(b.shape) != (P, H) or not b.is_contiguous() \
                    or not b.is_cuda:
                raise ValueError("bounds must be a contiguous fp32 [num_pages, kv_heads] GPU tensor")
            bp = b.data_ptr()
        return nbx_kv_pool(t.data_ptr(), _dtype_code(t), P, H, T, D, t.stride(0), t.stride(1),
                           t.stride(2), float(self.scale), bp)


def nbx_version() -> int:
    return load_library().nbx_version()


def nbx_paged_decode_plan(max_seq_len: int, split_positions: int = 256, max_splits: int = 64):
    """Returns (n_split, split_size) by the paged decode split rule."""
    n = ctypes.c_int32()
    s = ctypes.c_int32()
    _check(load_library().nbx_paged_decode_plan(int(max_seq_len), int(split_positions),
                                                int(max_splits), ctypes.byref(n), ctypes.byref(s)),
           "nbx_paged_decode_plan")
    return n.value, s.value


def nbx_paged_decode_plan_rows(batch: int, q_heads: int, kv_heads: int, q_rows: int,
                               head_dim: int, max_seq_len: int):
    """Returns (n_split, split_size): the pages' rule for decode rows, one round of
    multi-row workgroups over the device's compute units for more rows per KV head."""
    n = ctypes.c_int32()
    s = ctypes.c_int32()
    _check(load_library().nbx_paged_decode_plan_rows(int(batch), int(q_heads), int(kv_heads),
                                                     int(q_rows), int(head_dim),
                                                     int(max_seq_len), ctypes.byref(n),
                                                     ctypes.byref(s)),
           "nbx_paged_decode_plan_rows")
    return n.value, s.value


def case_plan(case):
    """(n_split, split_size) of a synthetic case's split policy: ("fixed", S, n),
    ("rule", positions, cap) -> nbx_paged_decode_plan, ("rows",) ->
    nbx_paged_decode_plan_rows."""
    pol = case.split_policy
    longest = int(case.seq_lens.max()) if len(case.seq_lens) else 1
    if pol[0] == "fixed":
        return pol[2], pol[1]
    if pol[0] == "rows":
        return nbx_paged_decode_plan_rows(case.batch, case.q_heads, case.kv_heads, case.q_rows,
                                          case.head_dim, longest)
    return nbx_paged_decode_plan(longest, pol[1], pol[2])


def nbx_paged_decode_workspace_bytes(rows: int, n_split: int, head_dim: int) -> int:
    return int(load_library().nbx_paged_decode_workspace_bytes(int(rows), int(n_split),
                                                               int(head_dim)))


def nbx_paged_kv_append(new_k: torch.Tensor, new_v: Optional[torch.Tensor], k_pool: KVPool,
                        v_pool: Optional[KVPool], slot_mapping: torch.Tensor,
                        dev_err: Optional[torch.Tensor] = None, stream=None):
    """new_k / new_v [n_tok, kv_heads, head_dim] (fp32 or bf16, last dim contiguous)."""
    if new_k.dim() != 3 or new_k.stride(2) != 1:
        raise ValueError("new positions are [n_tok, kv_heads, head_dim] with a contiguous last dim")
    if new_v is not None and (new_v.shape != new_k.shape or new_v.stride() != new_k.stride()
                              or new_v.dtype != new_k.dtype):
        raise ValueError("new_v must match new_k in shape, strides and dtype")
    if new_k.shape[1] != k_pool.data.shape[1] or new_k.shape[2] != k_pool.data.shape[3]:
        raise ValueError("new positions do not fit the pool")
    _int32_vector(slot_mapping, new_k.shape[0], "slot_mapping")
    kd = k_pool.desc()
    vd = v_pool.desc() if v_pool is not None else None
    st = load_library().nbx_paged_kv_append(
        _ptr(new_k), _ptr(new_v), _dtype_code(new_k), new_k.shape[0], new_k.stride(0),
        new_k.stride(1), ctypes.byref(kd), ctypes.byref(vd) if vd is not None else None,
        _ptr(slot_mapping), _dev_err(dev_err), _stream(stream))
    _check(st, "nbx_paged_kv_append")


def _workspace_bytes(workspace) -> int:
    if not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return workspace.numel() * workspace.element_size()


def _partials_shape(o_part, m_part, l_part, rows: int, n_split: int, dv: int):
    for name, t, shape in (("o_part", o_part, (rows, n_split, dv)), ("m_part", m_part, (rows, n_split)),
                           ("l_part", l_part, (rows, n_split))):
        if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous fp32 {shape}")


def _decode_common(q, k_pool, v_pool, block_table, seq_lens):
    if q.dim() != 4 or not q.is_contiguous():
        raise ValueError("q is a contiguous [batch, q_heads, q_rows, head_dim] tensor")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous int32 [batch, max_pages] tensor")
    _int32_vector(seq_lens, q.shape[0], "seq_lens")
    if block_table.shape[0] != q.shape[0]:
        raise ValueError("block_table rows must equal the batch")
    return k_pool.desc(), v_pool.desc()


def nbx_paged_decode_partial(q, k_pool: KVPool, v_pool: KVPool, block_table, seq_lens,
                             scale: float, split_size: int, n_split: int, o_part, m_part, l_part,
                             causal: bool = False, dev_err=None, stream=None):
    kd, vd = _decode_common(q, k_pool, v_pool, block_table, seq_lens)
    B, Hq, W, _ = q.shape
    _partials_shape(o_part, m_part, l_part, B * Hq * W, n_split, v_pool.data.shape[3])
    st = load_library().nbx_paged_decode_partial(
        _ptr(q), _dtype_code(q), B, Hq, W, int(bool(causal)), ctypes.byref(kd), ctypes.byref(vd),
        _ptr(block_table), block_table.shape[1], _ptr(seq_lens), float(scale), int(split_size),
        int(n_split), _ptr(o_part), _ptr(m_part), _ptr(l_part), _dev_err(dev_err), _stream(stream))
    _check(st, "nbx_paged_decode_partial")


def nbx_paged_decode_merge(o_part, m_part, l_part, out, stream=None):
    if o_part.dim() != 3:
        raise ValueError("o_part must be [rows, n_split, head_dim]")
    rows, n_split, D = o_part.shape
    _partials_shape(o_part, m_part, l_part, rows, n_split, D)
    if out.shape[-1] != D or out.numel() != rows * D or not out.is_contiguous():
        raise ValueError("out must be contiguous with rows * head_dim elements")
    st = load_library().nbx_paged_decode_merge(_ptr(o_part), _ptr(m_part), _ptr(l_part), rows,
                                               n_split, D, _ptr(out), _dtype_code(out),
                                               _stream(stream))
    _check(st, "nbx_paged_decode_merge")


def nbx_paged_decode(q, k_pool: KVPool, v_pool: KVPool, block_table, seq_lens, scale: float,
                     split_size: int, n_split: int, workspace, out, causal: bool = False,
                     dev_err=None, stream=None):
    """One call: partial then merge; ``workspace`` a uint8 device tensor of at least
    nbx_paged_decode_workspace_bytes(rows, n_split, v_head_dim) bytes; ``out`` is
    [batch, q_heads, q_rows, v_head_dim]."""
    kd, vd = _decode_common(q, k_pool, v_pool, block_table, seq_lens)
    B, Hq, W, _ = q.shape
    Dv = v_pool.data.shape[3]
    if out.numel() != B * Hq * W * Dv or not out.is_contiguous():
        raise ValueError("out must be contiguous [batch, q_heads, q_rows, v_head_dim]")
    st = load_library().nbx_paged_decode(
        _ptr(q), _dtype_code(q), B, Hq, W, int(bool(causal)), ctypes.byref(kd), ctypes.byref(vd),
        _ptr(block_table), block_table.shape[1], _ptr(seq_lens), float(scale), int(split_size),
        int(n_split), _ptr(workspace), _workspace_bytes(workspace), _ptr(out),
        _dtype_code(out), _dev_err(dev_err), _stream(stream))
    _check(st, "nbx_paged_decode")


def _new_rows(new_k, new_v, B, k_pool, D, Dv):
    """(n_new, dtype code) of a step's new rows (0, 0 without them), shapes checked."""
    if new_k is None:
        return 0, 0
    if new_v is None or new_k.shape[:3] != new_v.shape[:3] or new_k.dtype != new_v.dtype:
        raise ValueError("new_k and new_v must match")
    if new_k.dim() != 4 or new_k.shape[0] != B or new_k.shape[2] != k_pool.data.shape[1] \
            or new_k.shape[3] != D or new_v.shape[3] != Dv \
            or not (new_k.is_contiguous() and new_v.is_contiguous()):
        raise ValueError("new_k / new_v must be contiguous [batch, n_new, kv_heads, "
                         "head_dim / v_head_dim]")
    return new_k.shape[1], _dtype_code(new_k)


def nbx_paged_decode_step(q, k_pool: KVPool, v_pool: KVPool, block_table, seq_lens, scale: float,
                          split_size: int, n_split: int, workspace, out, new_k=None, new_v=None,
                          causal: bool = False, dev_err=None, stream=None):
    """One decode step: new_k [batch, n_new, kv_heads, head_dim] and new_v [batch, n_new,
    kv_heads, v_head_dim] (fp32 or bf16, contiguous) written at each sequence's last n_new
    positions, then partial and merge.  ``seq_lens`` count the new positions; ``workspace``
    as for nbx_paged_decode.  With ``out=None`` the step stops after the partials, which
    stay in the workspace."""
    kd, vd = _decode_common(q, k_pool, v_pool, block_table, seq_lens)
    B, Hq, W, D = q.shape
    Dv = v_pool.data.shape[3]
    if out is not None and (out.numel() != B * Hq * W * Dv or not out.is_contiguous()):
        raise ValueError("out must be contiguous [batch, q_heads, q_rows, v_head_dim]")
    n_new, new_dt = _new_rows(new_k, new_v, B, k_pool, D, Dv)
    st = load_library().nbx_paged_decode_step(
        _ptr(q), _dtype_code(q), B, Hq, W, int(bool(causal)), _ptr(new_k), _ptr(new_v), new_dt,
        n_new, ctypes.byref(kd), ctypes.byref(vd), _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), float(scale), int(split_size), int(n_split), _ptr(workspace),
        _workspace_bytes(workspace), _ptr(out),
        _dtype_code(out) if out is not None else 0, _dev_err(dev_err), _stream(stream))
    _check(st, "nbx_paged_decode_step")


def nbx_paged_decode_step_noalloc(q, k_pool: KVPool, v_pool: KVPool, block_table, seq_lens,
                                  scale: float, split_size: int, n_split: int, out, new_k=None,
                                  new_v=None, causal: bool = False, dev_err=None, stream=None):
    """nbx_paged_decode_step with the partials in the library's static device scratch
    (no workspace argument; the call allocates nothing).  ``out`` is required."""
    kd, vd = _decode_common(q, k_pool, v_pool, block_table, seq_lens)
    B, Hq, W, D = q.shape
    Dv = v_pool.data.shape[3]
    if out is None or out.numel() != B * Hq * W * Dv or not out.is_contiguous():
        raise ValueError("out must be contiguous [batch, q_heads, q_rows, v_head_dim]")
    n_new, new_dt = _new_rows(new_k, new_v, B, k_pool, D, Dv)
    st = load_library().nbx_paged_decode_step_noalloc(
        _ptr(q), _dtype_code(q), B, Hq, W, int(bool(causal)), _ptr(new_k), _ptr(new_v), new_dt,
        n_new, ctypes.byref(kd), ctypes.byref(vd), _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), float(scale), int(split_size), int(n_split), _ptr(out), _dtype_code(out),
        _dev_err(dev_err), _stream(stream))
    _check(st, "nbx_paged_decode_step_noalloc")


def workspace_partials(workspace, rows: int, n_split: int, head_dim: int):
    """Views (o [rows, n_split, D], m, l [rows, n_split]) of the partials a step or a
    one-call decode leaves in ``workspace`` (fp32, each part 256-byte aligned)."""
    r256 = lambda x: (x + 255) // 256 * 256
    o_b = rows * n_split * head_dim * 4
    ml_b = rows * n_split * 4
    need = r256(o_b) + 2 * r256(ml_b)
    if workspace.dtype != torch.uint8 or workspace.numel() < need:
        raise ValueError("workspace too small for the partials")
    o = workspace[:o_b].view(torch.float32).view(rows, n_split, head_dim)
    m = workspace[r256(o_b):r256(o_b) + ml_b].view(torch.float32).view(rows, n_split)
    off = r256(o_b) + r256(ml_b)
    l = workspace[off:off + ml_b].view(torch.float32).view(rows, n_split)
    return o, m, l


def nbx_paged_kv_bounds(k_pool: KVPool, v_pool: KVPool, block_table, seq_lens, dev_err=None,
                        stream=None):
    """Recompute k_pool.bounds and v_pool.bounds from the rows the sequences hold."""
    if k_pool.bounds is None or v_pool.bounds is None:
        raise ValueError("both pools need a bounds tensor")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous int32 [batch, max_pages] tensor")
    _int32_vector(seq_lens, block_table.shape[0], "seq_lens")
    kd, vd = k_pool.desc(), v_pool.desc()
    st = load_library().nbx_paged_kv_bounds(ctypes.byref(kd), ctypes.byref(vd), _ptr(block_table),
                                            block_table.shape[1], _ptr(seq_lens),
                                            block_table.shape[0], _dev_err(dev_err), _stream(stream))
    _check(st, "nbx_paged_kv_bounds")


def nbx_paged_lens_advance(seq_lens, n: int, stream=None):
    """seq_lens[b] += n on the device (int32 device tensor)."""
    if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 tensor")
    st = load_library().nbx_paged_lens_advance(_ptr(seq_lens), int(seq_lens.numel()), int(n),
                                               _stream(stream))
    _check(st, "nbx_paged_lens_advance")


def nbx_paged_decode_partial_windows(q, k_pool: KVPool, v_pool: KVPool, block_table, seq_lens,
                                     rows_per_seq, scale: float, split_size: int, n_split: int,
                                     o_part, m_part, l_part, causal: bool = True, dev_err=None,
                                     stream=None):
    """Split partials with a window of rows_per_seq[b] rows for sequence b (q padded
    to [batch, q_heads, longest window, head_dim])."""
    kd, vd = _decode_common(q, k_pool, v_pool, block_table, seq_lens)
    _int32_vector(rows_per_seq, q.shape[0], "rows_per_seq")
    B, Hq, W, D = q.shape
    _partials_shape(o_part, m_part, l_part, B * Hq * W, n_split, v_pool.data.shape[3])
    st = load_library().nbx_paged_decode_partial_windows(
        _ptr(q), _dtype_code(q), B, Hq, W, _ptr(rows_per_seq), int(bool(causal)),
        ctypes.byref(kd), ctypes.byref(vd), _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), float(scale), int(split_size), int(n_split), _ptr(o_part), _ptr(m_part),
        _ptr(l_part), _dev_err(dev_err), _stream(stream))
    _check(st, "nbx_paged_decode_partial_windows")
