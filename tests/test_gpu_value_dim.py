"""GPU parity with a value head dim of its own (Dv != D): the latent-attention
head sizes 192 (q, k) / 128 (v) on every kernel path, against the float64
oracle.  The value width is independent of the query/key width in the
nbxtensor attention_wrappers.py page (_math_attention's value head_dim) and in
the split kernel of the nbxtensor paged_decode_attn.py page (D_V)."""
import numpy as np
import pytest
import torch

import oracle
from paged_split_kv_append_amd import binding as nb
from paged_split_kv_append_amd import synth

from gpu_cases import TOL, DevCase, max_abs

pytestmark = pytest.mark.gpu

MLA = dict(head_dim=192, v_head_dim=128)


def _pool_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.uint8).numpy().reshape(-1)


def _bytes(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint8).reshape(-1)


def _oracle(case, kp=None, vp=None, rows=None):
    kp = case.k_pool if kp is None else kp
    vp = case.v_pool if vp is None else vp
    return oracle.attention(case.q, case.q_dtype, kp, vp, case.kv_dtype, case.block_table,
                            case.seq_lens, case.softmax_scale, case.causal, case.k_scale,
                            case.v_scale, rows=rows)


def _check(case, dc, out, ref):
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    assert out.shape == (case.rows, case.v_head_dim)
    assert torch.isfinite(out).all()
    err = max_abs(out, ref)
    assert err <= TOL[case.kv_dtype], f"max abs err {err}"


@pytest.mark.parametrize("seed", [None, 101])
def test_decode_after_append(seed):
    """Two append calls (one per pool width), then the persistent decode."""
    case = synth.make_case(7, seed=seed, batch=6, lens=("uniform", 1, 700))
    print(f"mla decode seed={seed} lens={case.seq_lens.tolist()}", flush=True)
    dc = DevCase(case)
    dc.append()
    out = dc.decode()
    kp, vp, bad = oracle.case_append(case)
    assert bad == 0
    _check(case, dc, out, _oracle(case, kp, vp))
    assert np.array_equal(_pool_bits(dc.k), _bytes(kp))
    assert np.array_equal(_pool_bits(dc.v), _bytes(vp))


@pytest.mark.parametrize("seed", [None, 102])
def test_step_single_launch(seed):
    """The fused step: each new K row (192) and V row (128) written by the wave
    that then reads it."""
    case = synth.make_case(7, seed=seed, batch=5, lens=("uniform", 1, 900))
    print(f"mla step seed={seed} lens={case.seq_lens.tolist()}", flush=True)
    dc = DevCase(case)
    out = dc.step()
    kp, vp, bad = oracle.case_append(case)
    assert bad == 0
    _check(case, dc, out, _oracle(case, kp, vp))
    assert np.array_equal(_pool_bits(dc.k), _bytes(kp))
    assert np.array_equal(_pool_bits(dc.v), _bytes(vp))


def test_partials_match_oracle():
    case = synth.make_case(7, seed=11, append=False, batch=4, lens=("uniform", 1, 500))
    dc = DevCase(case)
    S = 64
    n = -(-int(case.seq_lens.max()) // S) + 1          # one trailing empty split
    o, m, l = dc.partial(n_split=n, split_size=S)
    torch.cuda.synchronize()
    ro, rm, rl = oracle.partials(case.q, case.q_dtype, case.k_pool, case.v_pool, case.kv_dtype,
                                 case.block_table, case.seq_lens, case.softmax_scale, S, n)
    assert o.shape == (case.rows, n, 128) and ro.shape == (case.rows, n, 128)
    m_np, l_np, o_np = m.cpu().double().numpy(), l.cpu().double().numpy(), o.cpu().double().numpy()
    empty = rm == -np.inf                               # o of an empty split is not written
    assert np.all(m_np[empty] == -np.inf) and np.all(l_np[empty] == 0)
    ne = ~empty
    assert np.all(np.abs(m_np[ne] - rm[ne]) <= 1e-5 * np.maximum(1, np.abs(rm[ne])))
    tol = TOL[case.kv_dtype]
    assert np.max(np.abs(o_np[ne] / l_np[ne][:, None] - ro[ne] / rl[ne][:, None])) <= tol
    assert np.max(np.abs(l_np[ne] - rl[ne]) / rl[ne]) <= 10 * tol


MULTIROW = [
    ("verify_bf16_96rows", 3, dict(batch=2, lens=("uniform", 300, 900))),
    ("chunk_fp8_768rows", 4, dict(lens=("fixed", 1000))),
    ("gqa_bf16_32rows", 2, dict(batch=3, q_rows=8, causal=True, lens=("uniform", 8, 900),
                                append=False)),
]


@pytest.mark.parametrize("name,workload,over", MULTIROW, ids=[m[0] for m in MULTIROW])
def test_multirow_paths(name, workload, over):
    case = synth.make_case(workload, seed=62, **MLA, **over)
    print(f"mla multirow {name} lens={case.seq_lens.tolist()}", flush=True)
    dc = DevCase(case)
    out = dc.decode()
    _check(case, dc, out, _oracle(case))


def test_decode_batch_beyond_the_persistent_table():
    """batch > 256 runs the one-workgroup-per-split decode kernel."""
    case = synth.make_case(7, seed=63, append=False, batch=300, lens=("uniform", 1, 200))
    dc = DevCase(case)
    out = dc.decode()
    _check(case, dc, out, _oracle(case))


@pytest.mark.parametrize("kv_dtype,q_dtype", [("f32", "f32"), ("bf16", "f32")])
def test_vector_alu_path(kv_dtype, q_dtype):
    case = synth.make_case(7, seed=64, append=False, batch=3, lens=("uniform", 1, 300),
                           kv_dtype=kv_dtype, q_dtype=q_dtype)
    dc = DevCase(case)
    out = dc.decode()
    _check(case, dc, out, _oracle(case))


@pytest.mark.parametrize("over", [dict(kv_dtype="f32", q_dtype="f32", batch=3),
                                  dict(batch=300, lens=("uniform", 1, 120))],
                         ids=["f32_vector_alu", "batch300"])
def test_step_append_then_read_in_separate_launches(over):
    """Shapes the single-launch step does not take: the append kernel writes the
    192-wide K rows and the 128-wide V rows, then partial and merge run."""
    over = dict(dict(lens=("uniform", 1, 300)), **over)
    case = synth.make_case(7, seed=66, **over)
    dc = DevCase(case)
    out = dc.step()
    kp, vp, bad = oracle.case_append(case)
    assert bad == 0
    _check(case, dc, out, _oracle(case, kp, vp))
    assert np.array_equal(_pool_bits(dc.k), _bytes(kp))
    assert np.array_equal(_pool_bits(dc.v), _bytes(vp))


def test_unsupported_pair_is_refused():
    case = synth.make_case(7, seed=65, append=False, batch=1, lens=("fixed", 32),
                           v_head_dim=64)
    dc = DevCase(case)
    with pytest.raises(nb.NbxError) as e:
        dc.decode()
    assert e.value.status == -3


def test_full_size_sampled():
    """The full latent-attention decode shape (32 sequences, 16 heads, 192 / 128),
    step as bench.py times it; every row checked against the oracle."""
    case = synth.make_case(7)
    print(f"mla full size kv_bytes={case.kv_bytes()}", flush=True)
    dc = DevCase(case)
    out = dc.step()
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    kp, vp, _ = oracle.case_append(case)
    _check(case, dc, out, _oracle(case, kp, vp))
