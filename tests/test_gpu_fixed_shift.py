"""GPU parity of the fixed-shift softmax (maxdiffusion PR #477 page, fixed-m
splash attention with dynamic bounds): per-page K norm / V magnitude bounds
computed and maintained on the device, the shift m = ceil(U) - C(N) taken by
every group of rows that passes the gate, and the running maximum kept
otherwise.  Results are checked against the float64 oracle (the plain
definition); which path ran is read from the partials (a fixed shift is an
integer in log2 units) and from bitwise comparisons with the running-maximum
path."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from paged_split_kv_append_amd import binding as nb
from paged_split_kv_append_amd import synth

from gpu_cases import TOL, DevCase, max_abs

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ref(case, kp=None, vp=None):
    kp = case.k_pool if kp is None else kp
    vp = case.v_pool if vp is None else vp
    return oracle.attention(case.q, case.q_dtype, kp, vp, case.kv_dtype, case.block_table,
                            case.seq_lens, case.softmax_scale, case.causal, case.k_scale,
                            case.v_scale)


def _check_bounds(dc, case, kp=None, vp=None, lens=None):
    """Device bounds against the oracle's: K norms to fp32 rounding, V exactly."""
    kp = case.k_pool if kp is None else kp
    vp = case.v_pool if vp is None else vp
    lens = case.seq_lens if lens is None else lens
    rk = oracle.kv_bounds(kp, case.kv_dtype, case.block_table, lens, is_value=False)
    rv = oracle.kv_bounds(vp, case.kv_dtype, case.block_table, lens, is_value=True)
    gk = dc.kb.double().cpu().numpy()
    gv = dc.vb.double().cpu().numpy()
    assert np.all(np.isfinite(rk)) and np.all(np.isfinite(rv))
    assert np.all(np.abs(gk - rk) <= 1e-5 * rk), float(np.max(np.abs(gk - rk) / np.maximum(rk, 1)))
    assert np.array_equal(gv, rv)


def _fixed_fraction(m, l):
    """Share of non-empty splits whose m is an integer number of ln 2 (a fixed shift)."""
    m = m.double().cpu().numpy()
    l = l.double().cpu().numpy()
    ne = l > 0
    k = m[ne] / math.log(2.0)
    return float(np.mean(np.abs(k - np.round(k)) < 1e-4)) if ne.any() else 0.0


# ------------------------------------------------------------------ bounds

@pytest.mark.parametrize("workload,over", [
    (2, dict(batch=6, lens=("uniform", 1, 700), append=False)),
    (4, dict(lens=("fixed", 700))),
    (7, dict(batch=4, lens=("uniform", 1, 500), append=False)),
    (5, dict(batch=3, lens=("loguniform", 100, 3000), append=False)),
], ids=["gqa_bf16", "chunk_fp8", "mla_192_128", "long_t32"])
def test_bounds_match_oracle(workload, over):
    case = synth.make_case(workload, seed=71, **over)     # unheld slots hold NaN
    dc = DevCase(case)
    dc.attach_bounds()
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    _check_bounds(dc, case)


@pytest.mark.parametrize("how", ["slot_mapping", "step_single_launch", "step_separate_launches"])
def test_appends_raise_bounds(how):
    over = dict(batch=5, lens=("uniform", 2, 600))
    if how == "step_separate_launches":
        over.update(kv_dtype="f32", q_dtype="f32")           # the vector-ALU read: no fusion
    case = synth.make_case(2, seed=72, **over)
    dc = DevCase(case)
    dc.attach_bounds(lens=case.seq_lens - 1)                # before the new token
    if how == "slot_mapping":
        dc.append()
    else:
        dc.step()
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    kp, vp, _ = oracle.case_append(case)
    _check_bounds(dc, case, kp, vp)


# ------------------------------------------------------------------ parity

READS = [
    ("gqa_decode", 2, dict(batch=6, lens=("uniform", 1, 700))),
    ("long_decode_k4", 5, dict(batch=3, lens=("loguniform", 100, 3000))),
    ("verify_multirow", 3, dict(batch=2, lens=("uniform", 300, 900))),
    ("chunk_fp8_multirow", 4, dict(lens=("fixed", 1000))),
    ("mla_decode", 7, dict(batch=4, lens=("uniform", 1, 600))),
    ("decode_windows", 2, dict(batch=4, q_rows=4, causal=True, lens=("uniform", 8, 700),
                               append=False)),
]


@pytest.mark.parametrize("name,workload,over", READS, ids=[r[0] for r in READS])
def test_decode_with_bounds_matches_oracle(name, workload, over):
    case = synth.make_case(workload, seed=73, **over)
    print(f"fixed-shift read {name} lens={case.seq_lens.tolist()[:6]}", flush=True)
    dc = DevCase(case)
    if case.new_k is not None:
        dc.attach_bounds(lens=case.seq_lens - 1)
        out = dc.step()
        kp, vp, _ = oracle.case_append(case)
        ref = _ref(case, kp, vp)
    else:
        dc.attach_bounds()
        out = dc.decode()
        ref = _ref(case)
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    assert torch.isfinite(out).all()
    err = max_abs(out, ref)
    assert err <= TOL[case.kv_dtype], f"max abs err {err}"


def test_fixed_shift_runs_and_the_fallback_is_the_running_maximum():
    """With exact bounds every split of the decode takes the fixed shift (its m is an
    integer in log2 units); with NaN or huge bounds every group falls back and the
    output is bit-identical to the read without bounds."""
    case = synth.make_case(2, seed=74, batch=6, lens=("uniform", 1, 700), append=False)
    dc = DevCase(case)
    base = dc.decode().clone()
    _, m0, l0 = dc.partial()
    assert _fixed_fraction(m0, l0) < 0.05
    dc.attach_bounds()
    fixed = dc.decode().clone()
    _, m1, l1 = dc.partial()
    torch.cuda.synchronize()
    assert _fixed_fraction(m1, l1) == 1.0
    assert not torch.equal(fixed, base)
    assert max_abs(fixed, _ref(case)) <= TOL["bf16"]
    for fill in (float("nan"), 1e30):
        dc.kb.fill_(fill)
        out = dc.decode()
        _, m2, l2 = dc.partial()
        torch.cuda.synchronize()
        assert torch.equal(out, base), fill
        assert _fixed_fraction(m2, l2) < 0.05


def test_partials_with_a_fixed_shift_carry_the_same_mass():
    """o / l and l * exp(m) (the split's softmax mass) do not depend on the shift."""
    case = synth.make_case(3, seed=75, batch=2, lens=("uniform", 300, 900))
    dc = DevCase(case)
    dc.attach_bounds()
    S = 64
    n = -(-int(case.seq_lens.max()) // S) + 1
    o, m, l = dc.partial(n, S)
    torch.cuda.synchronize()
    assert _fixed_fraction(m, l) == 1.0
    ro, rm, rl = oracle.partials(case.q, case.q_dtype, case.k_pool, case.v_pool, case.kv_dtype,
                                 case.block_table, case.seq_lens, case.softmax_scale, S, n,
                                 case.causal)
    m_np, l_np, o_np = m.cpu().double().numpy(), l.cpu().double().numpy(), o.cpu().double().numpy()
    empty = rm == -np.inf
    assert np.all(m_np[empty] == -np.inf) and np.all(l_np[empty] == 0)
    ne = ~empty
    tol = TOL["bf16"]
    assert np.max(np.abs(o_np[ne] / l_np[ne][:, None] - ro[ne] / rl[ne][:, None])) <= tol
    mass = l_np[ne] * np.exp(m_np[ne] - rm[ne])
    assert np.max(np.abs(mass - rl[ne]) / rl[ne]) <= 10 * tol


# ------------------------------------------------------------------ the page's example

def _centered_keys_case(q0):
    """The adversarial example of the page: q = [q0, 2], half the keys [0, 1], half
    [0, -1], values +1 / -1, 4096 keys, softmax scale ln 2 (logits +-2 in base 2)."""
    g = json.load(open(os.path.join(GOLDEN, "softmax_mass_example.json")))
    n, D, T = 4096, 64, 16
    P = n // T
    k = torch.zeros(P, 1, T, D, dtype=torch.bfloat16)
    v = torch.zeros(P, 1, T, D, dtype=torch.bfloat16)
    sign = torch.ones(n)
    sign[n // 2:] = -1.0
    k.view(n, D)[:, 1] = (sign * g["k_pos"][1]).to(torch.bfloat16)
    v.view(n, D)[:] = (sign * g["v_pos"]).to(torch.bfloat16)[:, None]
    q = torch.zeros(1, 1, 1, D, dtype=torch.bfloat16)
    q[0, 0, 0, 0], q[0, 0, 0, 1] = q0, g["q"][1]
    bt = np.arange(P, dtype=np.int32)[None, :]
    lens = np.array([n], dtype=np.int32)
    return g, q, k, v, bt, lens, float(np.float32(g["softmax_scale"]))


@pytest.mark.parametrize("q0,takes_fixed", [(231.0, False), (100.0, True)])
def test_adversarial_centered_keys(q0, takes_fixed):
    """q0 = 231 is the page's input: U ~ 231 passes a W-sized gate (W = 232 at
    N = 4096) but not the shipped floor(W/2) = 116, so the read must fall back and
    give 15/17; q0 = 100 passes and the fixed shift gives 15/17 too."""
    g, q, k, v, bt, lens, scale = _centered_keys_case(q0)
    C, W, gate = oracle.fixed_shift_constants(4096, 1.0)
    assert math.ceil(math.hypot(q0, 2.0)) <= W
    assert (math.ceil(math.hypot(q0, 2.0)) <= gate) == takes_fixed
    dev = "cuda"
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    btd, ld = torch.from_numpy(bt).to(dev), torch.from_numpy(lens).to(dev)
    kb = torch.zeros(kd.shape[0], 1, device=dev)
    vb = torch.zeros(kd.shape[0], 1, device=dev)
    outs, parts = [], []
    for bounds in (False, True):
        kp = nb.KVPool(kd, 1.0, kb if bounds else None)
        vp = nb.KVPool(vd, 1.0, vb if bounds else None)
        if bounds:
            nb.nbx_paged_kv_bounds(kp, vp, btd, ld)
        o = torch.empty(1, 1, 64, device=dev)
        m = torch.empty(1, 1, device=dev)
        l = torch.empty(1, 1, device=dev)
        nb.nbx_paged_decode_partial(qd, kp, vp, btd, ld, scale, 4096, 1, o, m, l)
        out = torch.empty(1, 1, 1, 64, device=dev)
        ws = torch.empty(nb.nbx_paged_decode_workspace_bytes(1, 1, 64), dtype=torch.uint8,
                         device=dev)
        nb.nbx_paged_decode(qd, kp, vp, btd, ld, scale, 4096, 1, ws, out)
        torch.cuda.synchronize()
        outs.append(out.double().cpu().numpy().reshape(-1))
        parts.append((m.cpu().item(), l.cpu().item()))
    assert float(kb.max()) == 1.0 and float(vb.max()) == 1.0
    exact = g["expected_fraction"][0] / g["expected_fraction"][1]
    for o in outs:
        assert np.all(np.abs(o - exact) <= TOL["bf16"])
    k_fixed = parts[1][0] / math.log(2.0)
    assert (abs(k_fixed - round(k_fixed)) < 1e-4 and parts[1][0] != parts[0][0]) == takes_fixed
    if not takes_fixed:
        assert np.array_equal(outs[0], outs[1])


def test_full_size_decode_with_bounds():
    """The batched GQA decode step at full size with bounds attached: the append
    inside the single launch raises them, every split reads with a fixed shift."""
    case = synth.make_case(2)
    dc = DevCase(case)
    dc.attach_bounds(lens=case.seq_lens - 1)
    out = dc.step()
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    kp, vp, _ = oracle.case_append(case)
    err = max_abs(out, _ref(case, kp, vp))
    assert err <= TOL["bf16"], err
