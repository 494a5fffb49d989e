"""GPU parity: the library (through its C ABI) against the float64 oracle.

Every case is seeded synthetic input with NaN in every pool slot no sequence
position uses, so a read of the wrong slot poisons the output.  Tolerances
are max-abs against the oracle: 1e-5 for fp32 pools, 2e-3 for bf16 and 2e-2
for fp8 e4m3; the append and all indexing are compared bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from paged_split_kv_append_amd import binding as nb
from paged_split_kv_append_amd import synth

from gpu_cases import TOL, DevCase, max_abs

pytestmark = pytest.mark.gpu

# oracle-sized versions of the five workloads: several splits and tiles, ragged tails
REDUCED = {
    1: dict(),
    2: dict(batch=6, lens=("uniform", 1, 700)),
    3: dict(batch=2, lens=("uniform", 300, 900)),
    4: dict(lens=("fixed", 1000)),
    5: dict(batch=3, lens=("loguniform", 100, 3000)),
}


def _reference(case, dc):
    """Oracle output for the case after its append (if any)."""
    if case.new_k is not None:
        kp, vp, bad = oracle.case_append(case)
        assert bad == 0
    else:
        kp, vp = case.k_pool, case.v_pool
    return oracle.attention(case.q, case.q_dtype, kp, vp, case.kv_dtype, case.block_table,
                            case.seq_lens, case.softmax_scale, case.causal, case.k_scale,
                            case.v_scale), kp, vp


def _pool_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bytes of a pool (NaN-safe bit comparison)."""
    return t.detach().cpu().contiguous().view(torch.uint8).numpy().reshape(-1)


def _bytes(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint8).reshape(-1)


@pytest.mark.parametrize("workload", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("seed", [None, 101])
def test_decode_matches_oracle(workload, seed):
    case = synth.make_case(workload, seed=seed, **REDUCED[workload])
    print(f"case workload={workload} seed={seed} {case.name} lens={case.seq_lens.tolist()[:8]}",
          flush=True)
    dc = DevCase(case)
    if case.new_k is not None:
        dc.append()
    out = dc.decode()
    torch.cuda.synchronize()
    ref, _, _ = _reference(case, dc)
    assert dc.err_bits() == 0
    assert torch.isfinite(out).all()
    err = max_abs(out, ref)
    assert err <= TOL[case.kv_dtype], f"max abs err {err}"


@pytest.mark.parametrize("workload", [2, 5])
def test_append_is_bit_exact(workload):
    case = synth.make_case(workload, seed=7, **REDUCED[workload])
    dc = DevCase(case)
    dc.append()
    torch.cuda.synchronize()
    kp, vp, bad = oracle.case_append(case)
    assert bad == 0 and dc.err_bits() == 0
    assert np.array_equal(_pool_bits(dc.k), _bytes(kp))
    assert np.array_equal(_pool_bits(dc.v), _bytes(vp))


@pytest.mark.parametrize("pool_dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("src", [torch.float32, torch.bfloat16])
def test_append_casts_bit_exact(pool_dtype, src):
    g = torch.Generator().manual_seed(3)
    P, H, T, D, n = 5, 2, 16, 64, 9
    pool = {"f32": torch.zeros(P, H, T, D), "bf16": torch.zeros(P, H, T, D, dtype=torch.bfloat16),
            "fp8": torch.zeros(P, H, T, D, dtype=torch.uint8)}[pool_dtype]
    new = (torch.randn(n, H, D, generator=g) * 3).to(src)
    new[0, 0, :4] = torch.tensor([float("nan"), 1e-40, 500.0, -2.0 ** -10])
    slots = torch.tensor([0, 17, -1, 33, 79, 50, 2, 64, 31], dtype=torch.int32)
    scale = 0.037 if pool_dtype == "fp8" else 1.0
    from paged_split_kv_append_amd import binding as nb
    pk = pool.clone().cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    nb.nbx_paged_kv_append(new.cuda(), None, nb.KVPool(pk, scale), None, slots.cuda(),
                           dev_err=err)
    torch.cuda.synchronize()
    ref, bad = oracle.append(new, "f32" if src == torch.float32 else "bf16", pool, pool_dtype,
                             scale, T, slots.numpy())
    assert bad == 0 and int(err.item()) == 0
    assert np.array_equal(_pool_bits(pk), _bytes(ref))


def test_append_flags_out_of_range_and_skips_negative():
    from paged_split_kv_append_amd import binding as nb
    P, H, T, D = 2, 1, 16, 64
    pool = torch.full((P, H, T, D), 7.0, device="cuda")
    new = torch.ones(3, H, D, device="cuda")
    slots = torch.tensor([-5, 32, 40], dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    nb.nbx_paged_kv_append(new, None, nb.KVPool(pool), None, slots, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == nb.DEVERR_SLOT_RANGE
    assert torch.all(pool == 7.0)


@pytest.mark.parametrize("workload", [2, 3, 4, 5])
def test_partials_match_oracle(workload):
    case = synth.make_case(workload, seed=11, append=False, **REDUCED[workload])
    dc = DevCase(case)
    S = 64
    n = -(-int(case.seq_lens.max()) // S) + 1          # one trailing empty split
    o, m, l = dc.partial(n, S)
    torch.cuda.synchronize()
    ro, rm, rl = oracle.partials(case.q, case.q_dtype, case.k_pool, case.v_pool, case.kv_dtype,
                                 case.block_table, case.seq_lens, case.softmax_scale, S, n,
                                 case.causal, case.k_scale, case.v_scale)
    m_np, l_np, o_np = m.cpu().double().numpy(), l.cpu().double().numpy(), o.cpu().double().numpy()
    empty = rm == -np.inf                               # o of an empty split is not written
    assert np.all(m_np[empty] == -np.inf) and np.all(l_np[empty] == 0)
    ne = ~empty
    assert np.all(np.abs(m_np[ne] - rm[ne]) <= 1e-5 * np.maximum(1, np.abs(rm[ne])))
    # compare o / l (the normalised split output), robust to the split's own max
    tol = TOL[case.kv_dtype]
    assert np.max(np.abs(o_np[ne] / l_np[ne][:, None] - ro[ne] / rl[ne][:, None])) <= tol
    assert np.max(np.abs(l_np[ne] - rl[ne]) / rl[ne]) <= 10 * tol


@pytest.mark.parametrize("rows,ns,D", [(37, 9, 128), (11, 150, 64), (5, 70, 256), (3, 4096, 128),
                                       (9, 64, 256), (4, 65, 128)])
def test_merge_matches_oracle_on_oracle_partials(rows, ns, D):
    """Up to 64 splits take the one-round-trip form, more the looping one."""
    rng = np.random.default_rng(5 + ns)
    m = rng.normal(size=(rows, ns)) * 5
    m[:, 3] = -np.inf
    empty_row = min(4, rows - 1)
    m[empty_row] = -np.inf                             # a row with no visible key
    l = np.where(m == -np.inf, 0.0, rng.uniform(1, 50, size=(rows, ns)))
    o = rng.normal(size=(rows, ns, D)) * l[:, :, None]
    o64, m64, l64 = (np.float32(x).astype(np.float64) for x in (o, m, l))
    ref = oracle.merge(o64, m64, l64)
    # fp32 sums of ns weighted terms: error within ns * 2^-24 of the absolute sum (x 4)
    top = np.max(m64, axis=1, keepdims=True)
    top = np.where(top == -np.inf, 0.0, top)          # the empty row: every weight is 0
    w = np.where(m64 == -np.inf, 0.0, np.exp(m64 - top))
    den = np.maximum((w * l64).sum(1), 1e-300)
    bound = 4 * (ns + 8) * 2.0 ** -24 * ((w[:, :, None] * np.abs(o64)).sum(1) / den[:, None]
                                         + np.abs(ref))
    o[m == -np.inf] = np.nan                           # an empty split's o is never read
    m32, l32, o32 = (np.float32(x) for x in (m, l, o))
    from paged_split_kv_append_amd import binding as nb
    out = torch.empty(rows, D, device="cuda")
    nb.nbx_paged_decode_merge(torch.from_numpy(o32).cuda(), torch.from_numpy(m32).cuda(),
                              torch.from_numpy(l32).cuda(), out)
    torch.cuda.synchronize()
    err = np.abs(out.double().cpu().numpy() - ref)
    assert np.all(err <= bound + 1e-7), float(np.max(err - bound))
    assert torch.all(out[empty_row] == 0)


@pytest.mark.parametrize("workload", [2, 5])
def test_split_count_invariance(workload):
    case = synth.make_case(workload, seed=12, append=False, **REDUCED[workload])
    dc = DevCase(case)
    ref, _, _ = _reference(case, dc)
    L = int(case.seq_lens.max())
    for S in (16, 256, 2048):
        out = dc.decode(-(-L // S), S)
        torch.cuda.synchronize()
        assert max_abs(out, ref) <= TOL[case.kv_dtype], S


@pytest.mark.parametrize("workload", [2, 3])
def test_page_placement_is_bitwise_invariant(workload):
    case = synth.make_case(workload, seed=13, append=False, **REDUCED[workload])
    a = DevCase(case).decode()
    P = case.num_pages
    perm = np.random.default_rng(1).permutation(P)
    k2 = torch.empty_like(case.k_pool)
    v2 = torch.empty_like(case.v_pool)
    k2[perm] = case.k_pool
    v2[perm] = case.v_pool
    case.k_pool, case.v_pool = k2, v2
    case.block_table = np.where(case.block_table >= 0,
                                perm[np.maximum(case.block_table, 0)], -1).astype(np.int32)
    b = DevCase(case).decode()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("workload", [2, 4])
def test_repeated_runs_are_bitwise_identical(workload):
    case = synth.make_case(workload, seed=14, append=False, **REDUCED[workload])
    dc = DevCase(case)
    outs = [dc.decode().clone() for _ in range(5)]
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])


def test_bf16_output_within_tolerance_plus_half_ulp():
    case = synth.make_case(2, seed=15, append=False, **REDUCED[2])
    dc = DevCase(case)
    out = dc.decode(out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref, _, _ = _reference(case, dc)
    half_ulp = np.abs(ref) * 2.0 ** -9 + 1e-30
    err = np.abs(out.double().cpu().numpy() - ref)
    assert np.all(err <= TOL["bf16"] + half_ulp)


def test_interleaved_kv_allocation_gives_identical_bits():
    """K and V as strided views of one [P, 2, H, T, D] allocation."""
    case = synth.make_case(2, seed=16, append=False, **REDUCED[2])
    a = DevCase(case).decode()
    both = torch.stack([case.k_pool, case.v_pool], dim=1).cuda()
    dc = DevCase(case)
    dc.k, dc.v = both[:, 0], both[:, 1]
    b = dc.decode()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_bad_page_sets_flag_and_stays_finite():
    case = synth.make_case(2, seed=17, append=False, batch=2, lens=("fixed", 100))
    case.block_table[1, 2] = -1
    dc = DevCase(case)
    out = dc.decode()
    torch.cuda.synchronize()
    from paged_split_kv_append_amd import binding as nb
    assert dc.err_bits() & nb.DEVERR_PAGE_RANGE
    assert torch.isfinite(out).all()
    # the sequence without a bad page is unaffected
    ref, _, _ = _reference(synth.make_case(2, seed=17, append=False, batch=2, lens=("fixed", 100)),
                           dc)
    G = case.q_heads
    assert max_abs(out[:G], ref[:G]) <= TOL["bf16"]


def test_zero_length_sequence_gives_zero_rows():
    case = synth.make_case(2, seed=18, append=False, batch=3, lens=("fixed", 50))
    case.seq_lens[1] = 0
    dc = DevCase(case)
    out = dc.decode()
    torch.cuda.synchronize()
    H = case.q_heads
    assert torch.all(out[H:2 * H] == 0)
    ref = oracle.attention(case.q, case.q_dtype, case.k_pool, case.v_pool, case.kv_dtype,
                           case.block_table, case.seq_lens, case.softmax_scale)
    assert max_abs(out, ref) <= TOL["bf16"]


# ------------------------------------------------------------------ large batches

@pytest.mark.parametrize("kv_dtype,split", [("bf16", 64), ("bf16", 256), ("bf16", 1024),
                                            ("fp8", 256)])
def test_batch_beyond_the_persistent_table(kv_dtype, split):
    """More than 256 sequences: one workgroup per (split, sequence x KV head) with
    1, 2 or 4 waves taking interleaved chunks of the split (by split length)."""
    case = synth.make_case(2, seed=68, append=False, batch=300, lens=("uniform", 1, 1000),
                           kv_dtype=kv_dtype)
    print(f"batch 300 {kv_dtype} split {split}", flush=True)
    dc = DevCase(case)
    n_split = -(-int(case.seq_lens.max()) // split)
    out = dc.decode(n_split=n_split, split_size=split)
    torch.cuda.synchronize()
    ref, _, _ = _reference(case, dc)
    assert dc.err_bits() == 0
    assert torch.isfinite(out).all()
    assert max_abs(out, ref) <= TOL[kv_dtype]


# ------------------------------------------------------------------ full sizes

def _full_rows(case):
    """Row ranges compared with the oracle at full size: every row of the decode
    shapes; for the 16-row verify window, the rows of every query head of KV
    head g in sequence g (all four KV heads, all four sequences); for the
    128-row prompt chunk, the first and last 16-row tile of every query head
    (every 128-row block of every KV head)."""
    if case.q_rows == 1:
        return [(0, case.rows)]
    G = case.q_heads // case.kv_heads
    W = case.q_rows
    if W == 16:
        return [(((g % case.batch) * case.q_heads + g * G) * W,
                 ((g % case.batch) * case.q_heads + (g + 1) * G) * W)
                for g in range(case.kv_heads)]
    out = []
    for b in range(case.batch):
        for h in range(case.q_heads):
            r = (b * case.q_heads + h) * W
            out += [(r, r + 16), (r + W - 16, r + W)]
    return out


@pytest.mark.parametrize("workload", [2, 3, 4, 5])
def test_full_size_against_oracle(workload):
    case = synth.make_case(workload)
    print(f"full-size workload={workload} kv_bytes={case.kv_bytes()}", flush=True)
    dc = DevCase(case)
    if case.new_k is not None:
        dc.append()
    out = dc.decode()
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    assert torch.isfinite(out).all()
    if case.new_k is not None:
        kp, vp, _ = oracle.case_append(case)
    else:
        kp, vp = case.k_pool, case.v_pool
    ranges = _full_rows(case)
    if workload in (3, 4):                     # every KV head is sampled
        G, W = case.q_heads // case.kv_heads, case.q_rows
        assert {(r0 // W % case.q_heads) // G for r0, _ in ranges} == set(range(case.kv_heads))
    for r0, r1 in ranges:
        ref = oracle.attention(case.q, case.q_dtype, kp, vp, case.kv_dtype, case.block_table,
                               case.seq_lens, case.softmax_scale, case.causal, case.k_scale,
                               case.v_scale, rows=(r0, r1))
        err = max_abs(out[r0:r1], ref[r0:r1])
        assert err <= TOL[case.kv_dtype], (r0, r1, err)


# ------------------------------------------------------------------ multi-row shapes

MULTIROW = [
    # (name, overrides): rows per KV head = GQA group x window rows
    ("d128_bf16_32rows", dict(batch=3, q_rows=8, causal=True, lens=("uniform", 8, 900),
                              append=False)),
    ("d128_bf16_192rows", dict(batch=2, q_rows=48, causal=True, lens=("uniform", 48, 700),
                               append=False)),
    ("d64_fp8_24rows", dict(batch=3, head_dim=64, kv_dtype="fp8", q_rows=6, causal=True,
                            lens=("uniform", 6, 800), append=False)),
    ("d128_fp8_noncausal_80rows", dict(batch=2, kv_dtype="fp8", q_rows=20, causal=False,
                                       lens=("uniform", 1, 600), append=False)),
    # two row tiles per wave (more than 128 rows, D <= 128): fp8, and a second
    # 256-row block holding 32 rows, so that most of its waves have none
    ("d128_fp8_160rows", dict(batch=2, kv_dtype="fp8", q_rows=40, causal=True,
                              lens=("uniform", 40, 700), append=False)),
    ("d64_bf16_288rows", dict(batch=2, head_dim=64, q_rows=72, causal=True,
                              lens=("uniform", 72, 600), append=False)),
    # at most 96 rows: two loader waves; 96 rows exactly at D = 256, a ragged
    # last row tile (76 rows), the 192 / 128 pair (K and V pieces per tile
    # differ), and 100 rows just past the loader form
    ("d256_bf16_96rows", dict(batch=2, head_dim=256, q_rows=24, causal=True,
                              lens=("uniform", 24, 700), append=False)),
    ("d128_fp8_76rows", dict(batch=3, kv_dtype="fp8", q_rows=19, causal=True,
                             lens=("uniform", 19, 800), append=False)),
    ("d192_v128_bf16_64rows", dict(batch=2, head_dim=192, v_head_dim=128, q_rows=16,
                                   causal=True, lens=("uniform", 16, 600), append=False)),
    ("d128_bf16_100rows", dict(batch=2, q_rows=25, causal=True, lens=("uniform", 25, 600),
                               append=False)),
]


@pytest.mark.parametrize("name,over", MULTIROW, ids=[m[0] for m in MULTIROW])
def test_multirow_shapes_match_oracle(name, over):
    case = synth.make_case(2, seed=61, **over)
    print(f"multirow {name} rows/kv={case.q_heads // case.kv_heads * case.q_rows} "
          f"lens={case.seq_lens.tolist()}", flush=True)
    dc = DevCase(case)
    for n_split, split in (dc.plan(), (3, 256)):
        if n_split * split < int(case.seq_lens.max()):
            continue
        out = dc.decode(n_split=n_split, split_size=split)
        torch.cuda.synchronize()
        ref, _, _ = _reference(case, dc)
        assert dc.err_bits() == 0
        assert torch.isfinite(out).all()
        err = max_abs(out, ref)
        assert err <= TOL[case.kv_dtype], (n_split, split, err)


@pytest.mark.parametrize("workload", [3, 4], ids=["bf16", "fp8"])
@pytest.mark.parametrize("keys", [2100, 9000])
def test_verify_window_edge_lengths_match_oracle(workload, keys):
    """16-row causal windows (6 query heads per KV head, D = 256) over 2,100 and
    9,000 keys: lengths that are not a multiple of the 64-position chunk, read
    with the planned splits and with one split of the whole sequence (a split
    whose page ids take more than one batch of tiles)."""
    case = synth.make_case(workload, seed=70 + keys % 97, batch=2, q_rows=16,
                           lens=("fixed", keys))
    print(f"window edge: workload {workload} {case.kv_dtype} keys {keys}", flush=True)
    dc = DevCase(case)
    ref, _, _ = _reference(case, dc)
    for n_split, split in (dc.plan(), (1, -(-keys // 16) * 16)):
        out = dc.decode(n_split=n_split, split_size=split)
        torch.cuda.synchronize()
        assert dc.err_bits() == 0
        assert torch.isfinite(out).all()
        err = max_abs(out, ref)
        assert err <= TOL[case.kv_dtype], (n_split, split, err)


# ------------------------------------------------------------------ other page sizes

@pytest.mark.parametrize("workload,page_tokens", [(2, 48), (2, 128), (3, 48), (4, 80), (5, 64)])
def test_page_sizes_match_oracle(workload, page_tokens):
    """Pages of 48, 64, 80 and 128 positions: tiles start at non-zero rows of a
    page, and a split may start mid-page."""
    over = {2: dict(batch=5, lens=("uniform", 1, 900)), 3: dict(batch=2, lens=("uniform", 300, 900)),
            4: dict(lens=("fixed", 700)), 5: dict(batch=3, lens=("loguniform", 100, 3000))}[workload]
    case = synth.make_case(workload, seed=81, page_tokens=page_tokens, **over)
    print(f"pages of {page_tokens}: workload {workload} lens={case.seq_lens.tolist()}", flush=True)
    dc = DevCase(case)
    if case.new_k is not None:
        out = dc.step()
    else:
        out = dc.decode()
    torch.cuda.synchronize()
    ref, _, _ = _reference(case, dc)
    assert dc.err_bits() == 0
    assert torch.isfinite(out).all()
    assert max_abs(out, ref) <= TOL[case.kv_dtype]


# ------------------------------------------------------------------ ragged windows

WINDOWS = [
    # (name, workload, overrides, window rows per sequence)
    ("verify_d256_bf16", 3, dict(batch=4, lens=("uniform", 300, 900)), [16, 5, 1, 11]),
    ("decode_gqa_d128", 2, dict(batch=4, q_rows=4, causal=True, lens=("uniform", 8, 700)),
     [4, 1, 3, 0]),
    ("chunk_fp8_d256", 4, dict(batch=3, q_rows=32, lens=("uniform", 64, 600)), [32, 7, 20]),
    ("tiny_f32", 1, dict(batch=3, q_rows=5, causal=True, lens=("uniform", 10, 200),
                         num_pages=None, max_pages=None), [5, 2, 0]),
]


@pytest.mark.parametrize("name,workload,over,windows", WINDOWS, ids=[w[0] for w in WINDOWS])
def test_ragged_windows_match_per_sequence_oracle(name, workload, over, windows):
    """Sequences with windows of different lengths in one launch: each sequence's
    rows equal the oracle run on that sequence alone with its own window, and
    padding rows merge to exactly 0."""
    case = synth.make_case(workload, seed=85, append=False, **over)
    rows_b = np.array(windows, dtype=np.int32)
    print(f"windows {name}: {rows_b.tolist()} lens={case.seq_lens.tolist()}", flush=True)
    dc = DevCase(case)
    n_split, split = dc.plan()
    B, Hq, W, D = case.q.shape
    dev = "cuda"
    o = torch.empty(case.rows, n_split, D, device=dev)
    m = torch.empty(case.rows, n_split, device=dev)
    l = torch.empty(case.rows, n_split, device=dev)
    kp, vp = dc.pools()
    nb.nbx_paged_decode_partial_windows(dc.q, kp, vp, dc.bt, dc.lens,
                                        torch.from_numpy(rows_b).to(dev), case.softmax_scale,
                                        split, n_split, o, m, l, causal=case.causal,
                                        dev_err=dc.err)
    out = torch.empty(case.rows, D, device=dev)
    nb.nbx_paged_decode_merge(o, m, l, out)
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    got = out.double().cpu().numpy().reshape(B, Hq, W, D)
    for b, wb in enumerate(rows_b.tolist()):
        assert np.all(got[b, :, wb:, :] == 0.0)
        if wb == 0:
            continue
        qb = case.q[b:b + 1, :, :wb, :].contiguous()
        ref = oracle.attention(qb, case.q_dtype, case.k_pool, case.v_pool, case.kv_dtype,
                               case.block_table[b:b + 1], case.seq_lens[b:b + 1],
                               case.softmax_scale, case.causal, case.k_scale, case.v_scale)
        err = float(np.max(np.abs(got[b, :, :wb, :].reshape(-1, D) - ref)))
        assert err <= TOL[case.kv_dtype], (b, wb, err)


def test_ragged_window_entry_out_of_range_is_flagged():
    case = synth.make_case(2, seed=86, append=False, batch=2, q_rows=4, causal=True,
                           lens=("uniform", 8, 300))
    dc = DevCase(case)
    n_split, split = dc.plan()
    o = torch.empty(case.rows, n_split, case.head_dim, device="cuda")
    m = torch.empty(case.rows, n_split, device="cuda")
    l = torch.empty_like(m)
    kp, vp = dc.pools()
    rows_b = torch.tensor([9, 2], dtype=torch.int32, device="cuda")   # 9 > 4 window rows
    nb.nbx_paged_decode_partial_windows(dc.q, kp, vp, dc.bt, dc.lens, rows_b, case.softmax_scale,
                                        split, n_split, o, m, l, causal=True, dev_err=dc.err)
    torch.cuda.synchronize()
    assert dc.err_bits() & 0x4


def test_ragged_windows_full_size_sampled():
    """The four-stream ragged-window shape at full size (32768 keys): the
    4-row stream in full and the first 48 rows of the 16-row stream."""
    case = synth.make_case(6)
    print(f"full-size windows {case.rows_per_seq.tolist()} kv_bytes={case.kv_bytes()}", flush=True)
    dc = DevCase(case)
    n_split, split = dc.plan()
    B, Hq, W, D = case.q.shape
    o = torch.empty(case.rows, n_split, D, device="cuda")
    m = torch.empty(case.rows, n_split, device="cuda")
    l = torch.empty_like(m)
    kp, vp = dc.pools()
    nb.nbx_paged_decode_partial_windows(dc.q, kp, vp, dc.bt, dc.lens,
                                        torch.from_numpy(case.rows_per_seq).cuda(),
                                        case.softmax_scale, split, n_split, o, m, l, causal=True,
                                        dev_err=dc.err)
    out = torch.empty(case.rows, D, device="cuda")
    nb.nbx_paged_decode_merge(o, m, l, out)
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    got = out.double().cpu().numpy().reshape(B, Hq, W, D)
    for b, rows in ((3, None), (0, (0, 48))):
        wb = int(case.rows_per_seq[b])
        assert np.all(got[b, :, wb:, :] == 0.0)
        ref = oracle.attention(case.q[b:b + 1, :, :wb].contiguous(), case.q_dtype, case.k_pool,
                               case.v_pool, case.kv_dtype, case.block_table[b:b + 1],
                               case.seq_lens[b:b + 1], case.softmax_scale, True, rows=rows)
        g = got[b, :, :wb, :].reshape(-1, D)
        r0, r1 = rows if rows else (0, g.shape[0])
        err = float(np.max(np.abs(g[r0:r1] - ref[r0:r1])))
        assert err <= TOL["bf16"], (b, err)


DTYPE_MATRIX = [(kv, q, D, W) for kv in ("f32", "bf16", "fp8") for q in ("f32", "bf16")
                for D in (64, 128) for W in (1, 5)]


@pytest.mark.parametrize("kv,q,D,W", DTYPE_MATRIX,
                         ids=[f"{kv}-q{q}-d{D}-w{W}" for kv, q, D, W in DTYPE_MATRIX])
def test_dtype_matrix(kv, q, D, W):
    """Every (pool dtype, Q dtype) pair the header supports, at two head dims, for
    decode rows (W = 1: 4 rows per KV head) and a causal window (W = 5: 20 rows,
    the multi-row kernel for 16/8-bit pools with bf16 Q; fp32 on either side
    takes the vector-ALU kernel)."""
    case = synth.make_case(2, batch=3, lens=("uniform", W, 400), kv_dtype=kv, q_dtype=q,
                           head_dim=D, q_rows=W, causal=W > 1, append=False)
    print(f"case kv={kv} q={q} D={D} W={W} lens={case.seq_lens.tolist()}", flush=True)
    dc = DevCase(case)
    out = dc.decode()
    torch.cuda.synchronize()
    ref, _, _ = _reference(case, dc)
    assert dc.err_bits() == 0
    err = max_abs(out, ref)
    assert err <= TOL[kv], err
