"""Pins of the float64 oracle against facts fixed outside it (CPU only).

Each test checks the oracle against something other than its own formula:
library routines on special cases (torch's fp8 / bf16 casts, torch's float64
scaled-dot-product attention), closed forms of softmax attention, a worked
example printed on the maxdiffusion PR #477 page, hand-written append and split
examples, and invariants (page placement, GQA = replicated MHA, zero-padded
head dim, the merge identity, causal rows = shorter decodes, value columns
computed independently of the value head dim).  The last tests
plant known mistakes in the oracle and require that some pin goes red.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from paged_split_kv_append_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers

def contiguous_problem(seed, B=2, Hq=4, Hkv=2, W=1, D=16, T=16, lens=(37, 50), causal=False,
                       kv_dtype="f32", Dv=None):
    """Random contiguous K [B, Hkv, L, D] and V [B, Hkv, L, Dv] laid into pages through an
    identity table (Dv defaults to D)."""
    Dv = D if Dv is None else Dv
    g = torch.Generator().manual_seed(seed)
    L = max(lens)
    pages = -(-L // T)
    Kc = torch.randn(B, Hkv, pages * T, D, generator=g, dtype=torch.float64)
    Vc = torch.randn(B, Hkv, pages * T, Dv, generator=g, dtype=torch.float64)
    Q = torch.randn(B, Hq, W, D, generator=g, dtype=torch.float64)
    if kv_dtype == "f32":
        Kc, Vc, Q = Kc.float().double(), Vc.float().double(), Q.float().double()
    pool_k = Kc.view(B, Hkv, pages, T, D).permute(0, 2, 1, 3, 4).reshape(B * pages, Hkv, T, D)
    pool_v = Vc.view(B, Hkv, pages, T, Dv).permute(0, 2, 1, 3, 4).reshape(B * pages, Hkv, T, Dv)
    bt = np.arange(B * pages, dtype=np.int32).reshape(B, pages)
    return dict(Q=Q, K=Kc, V=Vc, pool_k=pool_k.float(), pool_v=pool_v.float(), bt=bt,
                lens=np.array(lens, dtype=np.int32), causal=causal, W=W)


def oracle_on(p, scale, **kw):
    return oracle.attention(p["Q"].float(), "f32", p["pool_k"], p["pool_v"], "f32", p["bt"],
                            p["lens"], scale, causal=p["causal"], **kw)


def sdpa_reference(p, scale):
    """torch's float64 scaled_dot_product_attention per sequence (library routine)."""
    Q, K, V, lens = p["Q"], p["K"], p["V"], p["lens"]
    B, Hq, W, _ = Q.shape
    Dv = V.shape[-1]
    G = Hq // K.shape[1]
    outs = []
    for b in range(B):
        L = int(lens[b])
        k = K[b, :, :L].repeat_interleave(G, dim=0)
        v = V[b, :, :L].repeat_interleave(G, dim=0)
        mask = None
        if p["causal"]:
            r = torch.arange(W)[:, None]
            j = torch.arange(L)[None, :]
            mask = j <= (L - W + r)
        o = torch.nn.functional.scaled_dot_product_attention(Q[b], k, v, attn_mask=mask,
                                                             scale=scale)
        outs.append(o.reshape(Hq * W, Dv))
    return torch.cat(outs).numpy()


# ----------------------------------------------------------------- storage formats

def test_fp8_decode_table_matches_ocp_definition_and_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_values("fp8", codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    assert np.array_equal(ours[~np.isnan(ours)], lib[~np.isnan(lib)])
    # OCP E4M3FN spot values
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9 and ours[0x07] == 7 * 2.0 ** -9
    assert ours[0x38] == 1.0 and ours[0x40] == 2.0
    assert math.isnan(ours[0x7F]) and math.isnan(ours[0xFF])
    assert ours[0x80] == 0.0 and math.copysign(1, ours[0x80]) == -1
    assert np.isnan(ours).sum() == 2


def test_bf16_decode_table_matches_definition_and_torch():
    """Every one of the 65,536 bf16 codes: the oracle's value equals torch's
    bfloat16 -> float64 cast bit for bit (NaN codes both NaN), and spot codes
    equal the format's definition (the upper 16 bits of a binary32)."""
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_values("bf16", codes)
    lib = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint64), lib[~nan].view(np.uint64))
    # exponent all ones with a non-zero fraction: 2 * 127 codes
    assert nan.sum() == 2 * 127
    assert ours[0x3F80] == 1.0 and ours[0x4000] == 2.0 and ours[0xC040] == -3.0
    assert ours[0x3F81] == 1.0 + 2.0 ** -7
    assert ours[0x7F80] == math.inf and ours[0xFF80] == -math.inf
    assert ours[0x7F7F] == (2.0 - 2.0 ** -7) * 2.0 ** 127
    assert ours[0x0080] == 2.0 ** -126 and ours[0x0001] == 2.0 ** -133
    assert ours[0x8000] == 0.0 and math.copysign(1, ours[0x8000]) == -1


def _fp32_samples(seed, n=4000):
    rng = np.random.default_rng(seed)
    x = np.concatenate([
        rng.standard_normal(n).astype(np.float32),
        (rng.standard_normal(n) * 1e-38).astype(np.float32),         # bf16 subnormal range
        (rng.standard_normal(n) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, 3.4e38, 1e-45, -1e-45], np.float32),
    ])
    # exact ties: values halfway between two bf16 neighbours
    base = rng.integers(0x3F80, 0x4F80, size=200).astype(np.uint32) << 16
    ties = (base | 0x8000).view(np.float32)
    return np.concatenate([x, ties])


def test_bf16_encode_matches_torch_rne():
    x = _fp32_samples(1)
    ours = oracle.encode_values("bf16", x.astype(np.float64))
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, lib)
    nan = oracle.encode_values("bf16", [float("nan"), float("-nan")])
    assert list(nan) == [0x7FC0, 0xFFC0]


def test_fp8_encode_matches_torch_rne_in_range_and_saturates():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.uniform(-464, 464, 3000), rng.standard_normal(3000) * 0.01,
                        rng.standard_normal(3000)]).astype(np.float32)
    # exact ties between neighbouring e4m3 values
    codes = np.arange(0, 0x7E, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, np.float32([464.0, -464.0])])
    ours = oracle.encode_values("fp8", x.astype(np.float64), 1.0)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, lib)
    sat = oracle.encode_values("fp8", [465.0, 1e30, -500.0, float("inf"), float("nan")], 1.0)
    assert list(sat) == [0x7E, 0x7E, 0xFE, 0x7E, 0x7F]


def test_fp8_encode_with_scale_uses_fp32_quotient():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(5000).astype(np.float32) * 3
    scale = np.float32(np.abs(x).max() / 448.0)
    ours = oracle.encode_values("fp8", x.astype(np.float64), float(scale))
    lib = (torch.from_numpy(x) / torch.tensor(scale)).to(torch.float8_e4m3fn)
    assert np.array_equal(ours, lib.view(torch.uint8).numpy())


# ----------------------------------------------------------------- append

def test_append_worked_example():
    # T=4 positions per page, 3 pages, 2 KV heads, D=3
    T, P, H, D = 4, 3, 2, 3
    pool = np.zeros((P, H, T, D), np.float32)
    new = np.arange(4 * H * D, dtype=np.float32).reshape(4, H, D) + 1
    slots = np.array([5, -1, 11, 12], np.int32)   # page 1 pos 1; skipped; page 2 pos 3; out of range
    out, bad = oracle.append(new, "f32", pool, "f32", 1.0, T, slots)
    out = out.view(np.float32)
    expect = np.zeros_like(pool)
    expect[1, 0, 1] = [1, 2, 3]
    expect[1, 1, 1] = [4, 5, 6]
    expect[2, 0, 3] = [13, 14, 15]
    expect[2, 1, 3] = [16, 17, 18]
    assert bad == 1
    assert np.array_equal(out, expect)


def test_append_same_dtype_copies_bits_including_nan_payloads():
    new = np.array([[[0x7FFF, 0xFFC1, 0x3F80, 0x0001]]], np.uint16)   # two NaN payloads
    pool = np.zeros((1, 1, 16, 4), np.uint16)
    out, _ = oracle.append(new, "bf16", pool, "bf16", 1.0, 16, np.array([3], np.int32))
    assert np.array_equal(out.reshape(16, 4)[3], new[0, 0])
    assert np.all(out.reshape(16, 4)[[0, 1, 2, 4]] == 0)


def test_append_casts_like_the_library_casts():
    rng = np.random.default_rng(4)
    new = rng.standard_normal((3, 2, 8)).astype(np.float32)
    slots = np.array([0, 9, 6], np.int32)
    pool = np.zeros((4, 2, 4, 8), np.uint16)
    out, _ = oracle.append(new, "f32", pool, "bf16", 1.0, 4, slots)
    got = out.reshape(4, 2, 4, 8)
    lib = torch.from_numpy(new).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for t, s in enumerate(slots):
        assert np.array_equal(got[s // 4, :, s % 4], lib[t])


# ----------------------------------------------------------------- split plan

@pytest.mark.parametrize("longest,expect", [
    (1, (1, 16)), (100, (1, 112)), (256, (1, 256)), (257, (2, 144)), (300, (2, 160)),
    (4096, (16, 256)), (16384, (64, 256)), (16385, (64, 272)), (32768, (64, 512)),
    (131072, (64, 2048)),
])
def test_split_plan_rule(longest, expect):
    assert oracle.split_plan(longest) == expect


def test_split_plan_covers_with_the_smallest_aligned_split():
    # the split count is fixed first; the aligned split length may leave the
    # last splits of the longest sequence empty (e.g. 16392 -> 64 x 272)
    for L in range(1, 140000, 37):
        n, S = oracle.split_plan(L)
        per = -(-L // n)
        assert S % 16 == 0 and n * S >= L and S - 16 < per <= S and 1 <= n <= 64
        assert n == min(64, -(-L // 256))


# ----------------------------------------------------------------- closed forms

def test_uniform_logits_give_mean_of_visible_values():
    p = contiguous_problem(5, W=4, lens=(30, 45), causal=True)
    p["Q"] = torch.zeros_like(p["Q"])
    out = oracle_on(p, 0.25)
    B, Hq, W, D = p["Q"].shape
    G = Hq // p["K"].shape[1]
    for b in range(B):
        L = int(p["lens"][b])
        for h in range(Hq):
            for r in range(W):
                n = L - W + r + 1
                ref = p["V"][b, h // G, :n].mean(0).numpy()
                assert np.allclose(out[(b * Hq + h) * W + r], ref, atol=1e-12)


def test_dominant_logit_gives_that_value_row():
    p = contiguous_problem(6, B=1, Hq=2, Hkv=1, lens=(40,))
    q = p["Q"][0, 0, 0]
    j_star = 17
    k = p["K"].clone()
    k[0, 0, j_star] = q * 80.0 / float(q @ q)      # logit 80 * scale vs |others| << 40
    p["K"] = k
    T = 16
    p["pool_k"] = k.view(1, 1, 3, T, -1).permute(0, 2, 1, 3, 4).reshape(3, 1, T, -1).float()
    p["Q"][0, 1, 0] = q                              # both heads share the query
    out = oracle_on(p, 1.0)
    others = float((p["K"][0, 0, :40].float().double() @ q.float().double()).sort().values[-2])
    assert 80.0 - others > 40
    assert np.allclose(out[0], p["V"][0, 0, j_star].float().numpy(), atol=1e-12)
    assert np.allclose(out[1], p["V"][0, 0, j_star].float().numpy(), atol=1e-12)


def test_golden_softmax_mass_example():
    g = json.load(open(os.path.join(GOLDEN, "softmax_mass_example.json")))
    n = g["keys_each_sign"]
    D = 2
    K = np.array([g["k_pos"]] * n + [g["k_neg"]] * n, np.float32)
    V = np.array([[g["v_pos"]] * D] * n + [[g["v_neg"]] * D] * n, np.float32)
    T = 16
    pool_k = np.zeros((1, 1, T, D), np.float32)
    pool_v = np.zeros((1, 1, T, D), np.float32)
    pool_k[0, 0, :2 * n] = K
    pool_v[0, 0, :2 * n] = V
    q = np.array(g["q"], np.float32).reshape(1, 1, 1, D)
    scale = float(np.float32(g["softmax_scale"]))
    out = oracle.attention(q, "f32", pool_k, pool_v, "f32", np.zeros((1, 1), np.int32),
                           np.array([2 * n], np.int32), scale)
    num, den = g["expected_fraction"]
    assert abs(out[0, 0] - num / den) < 1e-6 and abs(out[0, 1] - g["expected_output"]) < 1e-6
    assert abs(out[0, 0] - g["flushed_output"]) > 0.1


def test_zero_visible_keys_give_zero():
    p = contiguous_problem(7, lens=(0, 20))
    out = oracle_on(p, 0.25)
    Hq = p["Q"].shape[1]
    assert np.all(out[:Hq] == 0.0) and np.all(np.isfinite(out))


# ----------------------------------------------------------------- library routine

@pytest.mark.parametrize("seed,W,causal,Hq,Hkv,D,T,lens", [
    (10, 1, False, 4, 2, 16, 16, (37, 50)),
    (11, 1, False, 8, 1, 64, 32, (1, 95)),
    (12, 5, True, 6, 2, 32, 16, (33, 64)),
    (13, 16, True, 3, 3, 16, 16, (16, 40)),
])
def test_matches_torch_sdpa_float64(seed, W, causal, Hq, Hkv, D, T, lens):
    p = contiguous_problem(seed, B=len(lens), Hq=Hq, Hkv=Hkv, W=W, D=D, T=T, lens=lens,
                           causal=causal)
    scale = float(np.float32(1 / math.sqrt(D)))
    assert np.allclose(oracle_on(p, scale), sdpa_reference(p, scale), atol=1e-12, rtol=0)


# value head dim independent of the query/key one (nbxtensor attention_wrappers.py,
# _math_attention; the split kernel's D_V): torch's attention takes a value width of
# its own too
@pytest.mark.parametrize("seed,W,causal,Hq,Hkv,D,Dv,lens", [
    (14, 1, False, 4, 4, 24, 16, (37, 50)),
    (15, 3, True, 6, 2, 16, 40, (20, 61)),
    (16, 1, False, 8, 2, 48, 32, (1, 95)),
])
def test_value_head_dim_matches_torch_sdpa_float64(seed, W, causal, Hq, Hkv, D, Dv, lens):
    p = contiguous_problem(seed, B=len(lens), Hq=Hq, Hkv=Hkv, W=W, D=D, Dv=Dv, lens=lens,
                           causal=causal)
    scale = float(np.float32(1 / math.sqrt(D)))
    out = oracle_on(p, scale)
    assert out.shape == (len(lens) * Hq * W, Dv)
    assert np.allclose(out, sdpa_reference(p, scale), atol=1e-12, rtol=0)


# the storage formats inside attention: a bf16 pool with bf16 Q, and an fp8 pool with
# per-tensor scales, against torch's float64 attention on torch's own decoding of the
# same bits (bfloat16 / float8_e4m3fn -> float64, times the scale)
@pytest.mark.parametrize("seed,kv_dtype,W,causal,Hq,Hkv,D,T,lens,k_scale,v_scale", [
    (17, "bf16", 1, False, 8, 2, 64, 16, (45, 100), 1.0, 1.0),
    (18, "bf16", 4, True, 6, 2, 32, 32, (20, 77), 1.0, 1.0),
    (19, "fp8", 1, False, 4, 1, 32, 16, (31, 64), 0.5, 2.0),
    (20, "fp8", 3, True, 4, 2, 16, 16, (17, 50), 0.125, 0.25),
])
def test_storage_formats_match_torch_sdpa_float64(seed, kv_dtype, W, causal, Hq, Hkv, D, T,
                                                   lens, k_scale, v_scale):
    p = contiguous_problem(seed, B=len(lens), Hq=Hq, Hkv=Hkv, W=W, D=D, T=T, lens=lens,
                           causal=causal)
    tdt = torch.bfloat16 if kv_dtype == "bf16" else torch.float8_e4m3fn
    pk = (p["pool_k"] / k_scale).to(tdt)       # the pool's stored codes
    pv = (p["pool_v"] / v_scale).to(tdt)
    qb = p["Q"].to(torch.bfloat16)
    scale = float(np.float32(1 / math.sqrt(D)))
    out = oracle.attention(qb, "bf16", pk, pv, kv_dtype, p["bt"], p["lens"], scale,
                           causal=causal, k_scale=k_scale, v_scale=v_scale)
    # the reference sees torch's decoding of the same codes, laid back out per sequence
    B, pages = len(lens), p["bt"].shape[1]
    kd = pk.double().reshape(B, pages, Hkv, T, D).permute(0, 2, 1, 3, 4).reshape(B, Hkv, -1, D)
    vd = pv.double().reshape(B, pages, Hkv, T, D).permute(0, 2, 1, 3, 4).reshape(B, Hkv, -1, D)
    ref = sdpa_reference(dict(p, Q=qb.double(), K=kd * k_scale, V=vd * v_scale), scale)
    assert np.allclose(out, ref, atol=1e-12, rtol=0)


# ----------------------------------------------------------------- fixed-shift bounds

def test_fixed_shift_constants_match_the_page_examples():
    g = json.load(open(os.path.join(GOLDEN, "fixed_shift_constants.json")))
    for ex in g["examples"]:
        assert oracle.fixed_shift_constants(ex["N"], g["v_max_bound"]) == \
            (ex["C"], ex["W"], ex["gate"]), ex["where"]
    adv = g["adversarial"]
    C, W, gate = oracle.fixed_shift_constants(adv["N"], g["v_max_bound"])
    U = math.hypot(*adv["q"]) * adv["max_key_norm"]
    assert (math.ceil(U) <= W) == adv["passes_a_W_sized_gate"]
    assert (math.ceil(U) <= gate) == adv["passes_the_shipped_gate"]


@pytest.mark.parametrize("n,vmax,c", [(1, 1.0, 127), (2, 1.0, 126), (4096, 256.0, 107),
                                      (4097, 256.0, 106), (4096, 257.0, 106),
                                      (4096, 255.5, 107), (131072, 448.0, 101)])
def test_fixed_shift_constants_at_power_of_two_edges(n, vmax, c):
    C, W, gate = oracle.fixed_shift_constants(n, vmax)
    assert C == c and W == c + 125 and gate == (c + 125) // 2


def test_fixed_shift_gate_keeps_every_term_normal_and_every_sum_finite():
    # the page's argument: for |z| <= U and m = ceil(U) - C, every z - m lies in
    # [-125, C] once ceil(U) <= gate, so 2^(z - m) is a normal fp32 number and N
    # terms of size <= Vmax sum below 2^127
    for n, vmax in ((4096, 256.0), (75600, 256.0), (131072, 448.0), (1, 1.0)):
        C, W, gate = oracle.fixed_shift_constants(n, vmax)
        for cu in range(0, gate + 1):
            U = float(cu)                      # worst case U = ceil(U)
            m = cu - C
            assert -U - m >= -125 and U - m <= C
            assert n * 2.0 ** (U - m) * vmax <= 2.0 ** 127
        # one step past the gate the lowest term can leave the normal range
        U = float(gate + 1)
        assert -U - (gate + 1 - C) < -125


def test_kv_bounds_closed_forms():
    # rows c * e_i have norm |c|; the V bound is the largest |element| held
    T, D, P, H = 16, 32, 4, 2
    k = np.zeros((P, H, T, D), np.float32)
    v = np.zeros((P, H, T, D), np.float32)
    for p_ in range(P):
        for h in range(H):
            for r in range(T):
                k[p_, h, r, (r + h) % D] = (p_ + 1) * (r + 1) * (-1) ** r
                v[p_, h, r, (3 * r) % D] = -(p_ * 10 + h + r * 0.5)
    bt = np.array([[2, 0, -1], [3, -1, -1]], np.int32)     # page 1 belongs to nobody
    lens = np.array([20, 7], np.int32)                     # page 0 holds rows 0-3 only
    kb = oracle.kv_bounds(k, "f32", bt, lens, is_value=False)
    vb = oracle.kv_bounds(v, "f32", bt, lens, is_value=True)
    # held rows: page 2 rows 0-15, page 0 rows 0-3, page 3 rows 0-6
    for h in range(H):
        assert kb[2, h] == 3 * 16 and kb[0, h] == 1 * 4 and kb[3, h] == 4 * 7 and kb[1, h] == 0
        assert vb[2, h] == 20 + h + 7.5 and vb[0, h] == h + 1.5 and vb[3, h] == 30 + h + 3.0
        assert vb[1, h] == 0
    v[0, 1, 2, 5] = np.nan                               # held row: NaN sticks
    v[0, 0, 9, 5] = np.nan                               # unheld row of a held page: ignored
    vb = oracle.kv_bounds(v, "f32", bt, lens, is_value=True)
    assert np.isnan(vb[0, 1]) and vb[0, 0] == 1.5


def test_kv_bounds_bound_every_logit():
    # Cauchy-Schwarz: |scale q . k_j| <= scale |q| max_j |k_j| over the held rows
    c = synth.make_case(2, seed=29, batch=3, lens=("uniform", 1, 300), append=False)
    kb = oracle.kv_bounds(c.k_pool, c.kv_dtype, c.block_table, c.seq_lens, is_value=False)
    vb = oracle.kv_bounds(c.v_pool, c.kv_dtype, c.block_table, c.seq_lens, is_value=True)
    assert np.all(np.isfinite(kb)) and np.all(np.isfinite(vb))
    k = c.k_pool.float().numpy().astype(np.float64)
    v = c.v_pool.float().numpy().astype(np.float64)
    T = c.page_tokens
    for b in range(c.batch):
        for j in range(int(c.seq_lens[b])):
            p_ = c.block_table[b, j // T]
            for h in range(c.kv_heads):
                assert np.linalg.norm(k[p_, h, j % T]) <= kb[p_, h] * (1 + 1e-15)
                assert np.max(np.abs(v[p_, h, j % T])) <= vb[p_, h]


# ----------------------------------------------------------------- invariants

def test_page_placement_invariance_is_exact():
    c = synth.make_case(2, seed=21, batch=3, lens=("uniform", 1, 300), append=False)
    a = oracle.case_attention(c)
    # move every page to a new physical slot
    P = c.num_pages
    perm = np.random.default_rng(0).permutation(P)
    k2 = torch.empty_like(c.k_pool)
    v2 = torch.empty_like(c.v_pool)
    k2[perm] = c.k_pool
    v2[perm] = c.v_pool
    bt2 = np.where(c.block_table >= 0, perm[np.maximum(c.block_table, 0)], -1).astype(np.int32)
    b = oracle.attention(c.q, c.q_dtype, k2, v2, c.kv_dtype, bt2, c.seq_lens, c.softmax_scale)
    assert np.all(np.isfinite(a)) and np.array_equal(a, b)


def test_gqa_equals_mha_with_replicated_kv_heads():
    p = contiguous_problem(22, Hq=6, Hkv=2, lens=(29, 41))
    out_gqa = oracle_on(p, 0.3)
    G = 3
    p2 = dict(p)
    p2["pool_k"] = p["pool_k"].repeat_interleave(G, dim=1)
    p2["pool_v"] = p["pool_v"].repeat_interleave(G, dim=1)
    assert np.array_equal(out_gqa, oracle_on(p2, 0.3))


def test_zero_padding_the_head_dim_is_exact():
    p = contiguous_problem(23, D=16, lens=(20, 33))
    base = oracle_on(p, 0.25)
    pad = lambda t: torch.cat([t, torch.zeros(*t.shape[:-1], 8, dtype=t.dtype)], dim=-1)
    p2 = dict(p, Q=pad(p["Q"]), pool_k=pad(p["pool_k"]), pool_v=pad(p["pool_v"]))
    padded = oracle_on(p2, 0.25)          # scale stays at the true D
    assert np.allclose(padded[:, :16], base, atol=1e-14) and np.all(padded[:, 16:] == 0)


def test_value_columns_do_not_depend_on_the_value_width():
    # each output column is the same weighted sum whatever other columns V has:
    # V of 48 columns, then its first 16 and its last 32 as pools of their own
    p = contiguous_problem(25, Hq=6, Hkv=3, W=2, D=32, Dv=48, lens=(29, 47), causal=True)
    wide = oracle_on(p, 0.2)
    lo = oracle_on(dict(p, pool_v=p["pool_v"][..., :16].contiguous()), 0.2)
    hi = oracle_on(dict(p, pool_v=p["pool_v"][..., 16:].contiguous()), 0.2)
    assert np.all(np.isfinite(wide))
    assert np.array_equal(wide[:, :16], lo) and np.array_equal(wide[:, 16:], hi)


def test_uniform_logits_with_a_narrower_value_head():
    p = contiguous_problem(26, Hq=4, Hkv=2, D=40, Dv=8, lens=(13, 30))
    p["Q"] = torch.zeros_like(p["Q"])
    out = oracle_on(p, 0.5)
    for b in range(2):
        for h in range(4):
            ref = p["V"][b, h // 2, :int(p["lens"][b])].mean(0).numpy()
            assert np.allclose(out[b * 4 + h], ref, atol=1e-12)


def test_merge_identity_with_a_value_head_of_its_own():
    c = synth.make_case(7, seed=27, batch=3, lens=("uniform", 1, 200), append=False)
    assert c.head_dim == 192 and c.v_head_dim == 128
    ref = oracle.case_attention(c)
    n, S = oracle.split_plan(int(c.seq_lens.max()), positions=48)
    o, m, l = oracle.partials(c.q, c.q_dtype, c.k_pool, c.v_pool, c.kv_dtype, c.block_table,
                              c.seq_lens, c.softmax_scale, S, n)
    assert o.shape == (c.rows, n, 128) and ref.shape == (c.rows, 128)
    assert np.allclose(oracle.merge(o, m, l), ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("split_len", [16, 48, 112, 4096])
def test_merge_identity_over_split_covers(split_len):
    c = synth.make_case(3, seed=24, batch=2, lens=("uniform", 20, 300), q_rows=4,
                        q_heads=4, kv_heads=2, head_dim=32)
    ref = oracle.case_attention(c)
    n_split = -(-int(c.seq_lens.max()) // split_len)
    o, m, l = oracle.partials(c.q, c.q_dtype, c.k_pool, c.v_pool, c.kv_dtype, c.block_table,
                              c.seq_lens, c.softmax_scale, split_len, n_split, causal=True)
    assert np.allclose(oracle.merge(o, m, l), ref, atol=1e-12, rtol=0)
    # one split: o / l is the answer
    if n_split == 1:
        assert np.allclose(o[:, 0] / l[:, :1], ref, atol=1e-12)


def test_empty_splits_are_exact_identity():
    c = synth.make_case(2, seed=25, batch=2, lens=("fixed", 40), append=False)
    o, m, l = oracle.partials(c.q, c.q_dtype, c.k_pool, c.v_pool, c.kv_dtype, c.block_table,
                              c.seq_lens, c.softmax_scale, 16, 5)
    assert np.all(m[:, 3:] == -np.inf) and np.all(l[:, 3:] == 0) and np.all(o[:, 3:] == 0)
    assert np.all(np.isfinite(m[:, :3]))


def test_causal_rows_equal_shorter_single_row_decodes():
    c = synth.make_case(3, seed=26, batch=2, lens=("uniform", 30, 90), q_rows=6,
                        q_heads=4, kv_heads=2, head_dim=16)
    multi = oracle.case_attention(c).reshape(c.batch, c.q_heads, c.q_rows, -1)
    for r in range(c.q_rows):
        lens_r = (c.seq_lens - c.q_rows + r + 1).astype(np.int32)
        single = oracle.attention(c.q[:, :, r:r + 1], c.q_dtype, c.k_pool, c.v_pool, c.kv_dtype,
                                  c.block_table, lens_r, c.softmax_scale)
        assert np.array_equal(single.reshape(c.batch, c.q_heads, -1), multi[:, :, r])


def test_split_invariance_of_merged_partials():
    c = synth.make_case(5, seed=27, batch=2, lens=("loguniform", 40, 600), append=False)
    outs = []
    for S in (16, 64, 256):
        n = -(-int(c.seq_lens.max()) // S)
        outs.append(oracle.merge(*oracle.partials(
            c.q, c.q_dtype, c.k_pool, c.v_pool, c.kv_dtype, c.block_table, c.seq_lens,
            c.softmax_scale, S, n)))
    assert np.allclose(outs[0], outs[1], atol=1e-12) and np.allclose(outs[0], outs[2], atol=1e-12)


def test_poisoned_unused_slots_stay_unread():
    c = synth.make_case(2, seed=28, batch=3, lens=("uniform", 1, 200))
    kp, vp, bad = oracle.case_append(c)
    assert bad == 0
    out = oracle.attention(c.q, c.q_dtype, kp, vp, c.kv_dtype, c.block_table, c.seq_lens,
                           c.softmax_scale)
    assert np.all(np.isfinite(out))
    # without the append the newest positions are still NaN and must poison the rows
    out_pre = oracle.case_attention(c)
    assert np.all(np.isnan(out_pre))


# ----------------------------------------------------------------- planted controls

def _pins_pass():
    """A bundle of the pins above, as booleans; a planted mistake must fail one."""
    ok = []
    p = contiguous_problem(40, B=2, Hq=4, Hkv=2, W=3, D=16, lens=(35, 50), causal=True)
    ok.append(np.allclose(oracle_on(p, 0.25), sdpa_reference(p, 0.25), atol=1e-10))
    p = contiguous_problem(41, B=2, Hq=4, Hkv=2, W=1, D=16, lens=(35, 50))
    ok.append(np.allclose(oracle_on(p, 0.25), sdpa_reference(p, 0.25), atol=1e-10))
    c = synth.make_case(3, seed=42, batch=2, lens=("uniform", 40, 200), q_rows=2,
                        q_heads=2, kv_heads=1, head_dim=16)
    ref = oracle.case_attention(c)
    o, m, l = oracle.partials(c.q, c.q_dtype, c.k_pool, c.v_pool, c.kv_dtype, c.block_table,
                              c.seq_lens, c.softmax_scale, 32, 7, causal=True)
    ok.append(np.allclose(oracle.merge(o, m, l), ref, atol=1e-10))
    p = contiguous_problem(43, B=2, Hq=4, Hkv=2, W=1, D=16, Dv=24, lens=(35, 50))
    try:
        ok.append(np.allclose(oracle_on(p, 0.25), sdpa_reference(p, 0.25), atol=1e-10))
    except ValueError:                    # a planted mistake the oracle refuses to run
        ok.append(False)
    # a -1 entry inside a sequence's range maps no page: the oracle must refuse it
    p = contiguous_problem(44, B=2, Hq=2, Hkv=1, W=1, D=16, lens=(35, 50))
    p["bt"] = p["bt"].copy()
    p["bt"][1, 1] = -1
    try:
        oracle_on(p, 0.25)
        ok.append(False)
    except ValueError:
        ok.append(True)
    return all(ok), ok


def test_pins_pass_without_mutation():
    assert _pins_pass()[0]


@pytest.mark.parametrize("name", ["drop_last_split", "head_mod", "causal_off_by_one",
                                  "swap_kv", "shift_sign", "page_offset", "value_width",
                                  "no_page_check"])
def test_planted_mistake_goes_red(name):
    with oracle.mutation(name):
        passed, detail = _pins_pass()
    assert not passed, f"planted mistake {name} was not caught: {detail}"
