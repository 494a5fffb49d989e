"""Float64 CPU oracle for paged split-KV attention (ctypes front end).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline call this; the GPU library never does, and this package never
imports the GPU library.  The arithmetic lives in ``nbx_oracle.c`` (plain C,
double precision, OpenMP over query rows); this file only marshals numpy /
torch CPU arrays into it.

Dtype names: "f32", "bf16", "fp8" (OCP E4M3FN codes stored as uint8).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nbx_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_CODES = {"f32": 0, "bf16": 1, "fp8": 2}
_lock = threading.Lock()
_lib = None

MUTATIONS = {
    "none": 0, "drop_last_split": 1, "head_mod": 2, "causal_off_by_one": 3,
    "swap_kv": 4, "shift_sign": 5, "page_offset": 6, "value_width": 7, "no_page_check": 8,
}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (C11, -O2, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            P, I, I64, D, S = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double,
                               ctypes.c_size_t)
            lib.oracle_decode_value.argtypes = [I, P, I64]
            lib.oracle_decode_value.restype = D
            lib.oracle_encode_value.argtypes = [I, D, D, P, I64]
            lib.oracle_append.argtypes = [P, I, I64, I, I, P, I, D, I64, I, P]
            lib.oracle_append.restype = I
            lib.oracle_split_plan.argtypes = [I64, I64, I64, I64, P, P]
            common = [P, I, I, I, I, I, I, I, P, P, I, D, D, I64, I, I, P, I, P, D]
            lib.oracle_attention_rows.argtypes = common + [I64, I64, P]
            lib.oracle_attention_rows.restype = I
            lib.oracle_attention.argtypes = common + [P]
            lib.oracle_attention.restype = I
            lib.oracle_partials.argtypes = common + [I64, I, P, P, P]
            lib.oracle_partials.restype = I
            lib.oracle_merge.argtypes = [P, P, P, I64, I, I, P]
            lib.oracle_fixed_shift_constants.argtypes = [I64, D, P, P, P]
            lib.oracle_fixed_shift_constants.restype = I
            lib.oracle_kv_bounds.argtypes = [P, I, I64, I, I, I, I, P, I, P, I, P]
            lib.oracle_kv_bounds.restype = I
            lib.oracle_set_mutation.argtypes = [I]
            lib.oracle_get_mutation.restype = I
            lib.oracle_num_threads.restype = I
            _lib = lib
    return _lib


def _np(x):
    """A contiguous numpy view of a numpy array or CPU torch tensor (raw bits)."""
    if isinstance(x, np.ndarray):
        return np.ascontiguousarray(x)
    import torch  # local: only for tensors handed in by callers
    t = x.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class mutation:
    """Context manager planting a known mistake in the oracle (checker-sanity tests)."""

    def __init__(self, name: str):
        self.code = MUTATIONS[name]

    def __enter__(self):
        _load().oracle_set_mutation(self.code)
        return self

    def __exit__(self, *exc):
        _load().oracle_set_mutation(0)


def num_threads() -> int:
    """Threads the oracle's parallel loops run on."""
    return int(_load().oracle_num_threads())


def decode_values(dtype: str, raw) -> np.ndarray:
    """Stored elements (raw bits) -> float64 values."""
    a = _np(raw).reshape(-1)
    lib = _load()
    return np.array([lib.oracle_decode_value(_CODES[dtype], _ptr(a), i) for i in range(a.size)])


def encode_values(dtype: str, values, scale: float = 1.0) -> np.ndarray:
    """fp32-representable float64 values -> stored bits (uint32 / uint16 / uint8)."""
    v = np.asarray(values, dtype=np.float64).reshape(-1)
    out = np.zeros(v.size, dtype={"f32": np.uint32, "bf16": np.uint16, "fp8": np.uint8}[dtype])
    lib = _load()
    for i, x in enumerate(v):
        lib.oracle_encode_value(_CODES[dtype], float(x), float(scale), _ptr(out), i)
    return out


def append(new_vals, src_dtype: str, pool, pool_dtype: str, scale: float, page_tokens: int,
           slot_mapping) -> tuple[np.ndarray, int]:
    """Scatter new [N_tok, H_kv, D] into a copy of pool [P, H_kv, T, D].

    Returns (updated pool bits, number of out-of-range slots)."""
    nv = _np(new_vals)
    pl = _np(pool).copy()
    sm = np.ascontiguousarray(np.asarray(slot_mapping, dtype=np.int32))
    n_tok, h_kv, d = nv.shape
    P = pl.shape[0]
    bad = _load().oracle_append(_ptr(nv), _CODES[src_dtype], n_tok, h_kv, d, _ptr(pl),
                                _CODES[pool_dtype], float(scale), P, page_tokens, _ptr(sm))
    return pl, bad


def split_plan(longest: int, positions: int = 256, max_splits: int = 64, align: int = 16):
    n = ctypes.c_int64()
    s = ctypes.c_int64()
    _load().oracle_split_plan(longest, positions, max_splits, align, ctypes.byref(n),
                              ctypes.byref(s))
    return int(n.value), int(s.value)


def _problem_args(q, q_dtype, k_pool, v_pool, kv_dtype, k_scale, v_scale, block_table,
                  seq_lens, scale, causal, q_rows):
    qn, kn, vn = _np(q), _np(k_pool), _np(v_pool)
    B, Hq, W, D = qn.shape
    assert W == q_rows
    P, Hkv, T, Dk = kn.shape
    Dv = vn.shape[3]
    assert Dk == D and vn.shape[:3] == kn.shape[:3]
    bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    keep = (qn, kn, vn, bt, sl)
    args = [_ptr(qn), _CODES[q_dtype], B, Hq, W, D, Dv, int(bool(causal)), _ptr(kn), _ptr(vn),
            _CODES[kv_dtype], float(k_scale), float(v_scale), P, Hkv, T, _ptr(bt),
            bt.shape[1], _ptr(sl), float(scale)]
    return args, keep, (B, Hq, W, Dv)


def attention(q, q_dtype, k_pool, v_pool, kv_dtype, block_table, seq_lens, scale,
              causal=False, k_scale=1.0, v_scale=1.0, rows=None) -> np.ndarray:
    """Plain-definition attention in float64: out [B*H_q*W, Dv] (rows (b, h, r)), Dv
    the value pool's head dim (which may differ from that of q and k).

    ``rows``: optional (begin, end) to compute only a sample of rows (others NaN)."""
    W = _np(q).shape[2]
    args, keep, (B, Hq, W, Dv) = _problem_args(q, q_dtype, k_pool, v_pool, kv_dtype, k_scale,
                                               v_scale, block_table, seq_lens, scale, causal, W)
    nrows = B * Hq * W
    out = np.full((nrows, Dv), np.nan)
    r0, r1 = (0, nrows) if rows is None else rows
    st = _load().oracle_attention_rows(*args, r0, r1, _ptr(out))
    if st != 0:
        raise ValueError(f"oracle: bad page or shape (status {st})")
    return out


def partials(q, q_dtype, k_pool, v_pool, kv_dtype, block_table, seq_lens, scale, split_len,
             n_split, causal=False, k_scale=1.0, v_scale=1.0):
    """Per-split (o, m, l) in float64: o [rows, n_split, Dv], m, l [rows, n_split]."""
    W = _np(q).shape[2]
    args, keep, (B, Hq, W, Dv) = _problem_args(q, q_dtype, k_pool, v_pool, kv_dtype, k_scale,
                                               v_scale, block_table, seq_lens, scale, causal, W)
    nrows = B * Hq * W
    o = np.zeros((nrows, n_split, Dv))
    m = np.zeros((nrows, n_split))
    l = np.zeros((nrows, n_split))
    st = _load().oracle_partials(*args, int(split_len), int(n_split), _ptr(o), _ptr(m), _ptr(l))
    if st != 0:
        raise ValueError(f"oracle: bad page or shape (status {st})")
    return o, m, l


def merge(o, m, l) -> np.ndarray:
    """Fixed-order combine of partials -> out [rows, D] float64."""
    o = np.ascontiguousarray(o, dtype=np.float64)
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    rows, n_split, D = o.shape
    out = np.zeros((rows, D))
    _load().oracle_merge(_ptr(o), _ptr(m), _ptr(l), rows, n_split, D, _ptr(out))
    return out


def fixed_shift_constants(n: int, v_max: float = 256.0):
    """(C, W, gate) of the fixed-shift softmax for N = n keys and values bounded by v_max."""
    c, w, g = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    st = _load().oracle_fixed_shift_constants(int(n), float(v_max), ctypes.byref(c),
                                              ctypes.byref(w), ctypes.byref(g))
    if st != 0:
        raise ValueError("oracle: n >= 1 and finite v_max >= 1 required")
    return int(c.value), int(w.value), int(g.value)


def kv_bounds(pool, dtype: str, block_table, seq_lens, is_value: bool) -> np.ndarray:
    """Per (page, KV head) bound over the rows the sequences hold: largest K row norm
    (is_value False) or largest |V element| (True), stored units -> [P, H_kv] float64."""
    pl = _np(pool)
    P, Hkv, T, D = pl.shape
    bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    out = np.zeros((P, Hkv))
    st = _load().oracle_kv_bounds(_ptr(pl), _CODES[dtype], P, Hkv, T, D, int(bool(is_value)),
                                  _ptr(bt), bt.shape[1], _ptr(sl), len(sl), _ptr(out))
    if st != 0:
        raise ValueError("oracle: a held position has no page in the pool")
    return out


def case_attention(case, rows=None):
    """Attention of a synthetic case (duck-typed: needs the generator's fields)."""
    return attention(case.q, case.q_dtype, case.k_pool, case.v_pool, case.kv_dtype,
                     case.block_table, case.seq_lens, case.softmax_scale, case.causal,
                     case.k_scale, case.v_scale, rows=rows)


def case_append(case):
    """The pools after appending the case's new tokens: (k_pool bits, v_pool bits, bad)."""
    kp, bk = append(case.new_k, "f32", case.k_pool, case.kv_dtype, case.k_scale,
                    case.page_tokens, case.slot_mapping)
    vp, bv = append(case.new_v, "f32", case.v_pool, case.kv_dtype, case.v_scale,
                    case.page_tokens, case.slot_mapping)
    return kp, vp, bk + bv
