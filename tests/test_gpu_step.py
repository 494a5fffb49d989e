"""GPU parity of nbx_paged_decode_step (append at each sequence's last
positions, then partial and merge, in one launch where the shape allows)
against the float64 oracle's append followed by its attention.

The slots the step fills hold NaN beforehand, so an output computed from the
old contents of a slot is not finite; the pools after the step are compared
bit for bit with the oracle's append."""
import numpy as np
import pytest
import torch

import oracle
from paged_split_kv_append_amd import binding as nb
from paged_split_kv_append_amd import synth

from gpu_cases import TOL, DevCase, max_abs

pytestmark = pytest.mark.gpu

REDUCED = {
    2: dict(batch=6, lens=("uniform", 1, 700)),
    5: dict(batch=3, lens=("loguniform", 100, 3000)),
}


def _pool_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.uint8).numpy().reshape(-1)


def _bytes(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint8).reshape(-1)


def _tail_slots(case, n_new):
    """Slots of positions L_b - n_new .. L_b - 1 of every sequence, [batch * n_new]."""
    T = case.page_tokens
    out = []
    for b in range(case.batch):
        for i in range(n_new):
            pos = int(case.seq_lens[b]) - n_new + i
            out.append(int(case.block_table[b, pos // T]) * T + pos % T)
    return np.array(out, dtype=np.int32)


def _poison_slots(case, slots):
    for pool, dt in ((case.k_pool, case.kv_dtype), (case.v_pool, case.kv_dtype)):
        nan = synth.nan_bits(dt, pool)
        for s in slots:
            pool[s // case.page_tokens, :, s % case.page_tokens, :] = nan


def _check_step(case, dc, out, new_k, new_v, slots):
    """Output against the oracle after its append of new_k/new_v at `slots`; pools bitwise."""
    n_tok = new_k.shape[0] * new_k.shape[1]
    H, D, Dv = case.kv_heads, case.head_dim, case.v_head_dim
    nk = new_k.float().cpu().reshape(n_tok, H, D)
    nv = new_v.float().cpu().reshape(n_tok, H, Dv)
    kp, bk = oracle.append(nk, "f32", case.k_pool, case.kv_dtype, case.k_scale, case.page_tokens,
                           slots)
    vp, bv = oracle.append(nv, "f32", case.v_pool, case.kv_dtype, case.v_scale, case.page_tokens,
                           slots)
    assert bk == 0 and bv == 0
    assert np.array_equal(_pool_bits(dc.k), _bytes(kp))
    assert np.array_equal(_pool_bits(dc.v), _bytes(vp))
    ref = oracle.attention(case.q, case.q_dtype, kp, vp, case.kv_dtype, case.block_table,
                           case.seq_lens, case.softmax_scale, case.causal, case.k_scale,
                           case.v_scale)
    assert torch.isfinite(out).all()
    err = max_abs(out, ref)
    assert err <= TOL[case.kv_dtype], f"max abs err {err}"


@pytest.mark.parametrize("workload", [2, 5])
@pytest.mark.parametrize("seed", [None, 103])
def test_step_single_launch_matches_oracle(workload, seed):
    case = synth.make_case(workload, seed=seed, **REDUCED[workload])
    print(f"step workload={workload} seed={seed} lens={case.seq_lens.tolist()}", flush=True)
    dc = DevCase(case)
    out = dc.step()
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    _check_step(case, dc, out, case.new_k.unsqueeze(1), case.new_v.unsqueeze(1),
                case.slot_mapping)


@pytest.mark.parametrize("batch,kv_dtype", [(65, "bf16"), (200, "fp8"), (256, "bf16")])
def test_step_batches_past_one_lane_block(batch, kv_dtype):
    """65 to 256 sequences: the single-launch step's sequence table (one lane
    per sequence) spans several 64-lane blocks; batch 256 is the largest it
    takes.  Appended rows bit for bit, outputs against the oracle."""
    case = synth.make_case(2, seed=90 + batch, kv_dtype=kv_dtype, batch=batch,
                           lens=("uniform", 1, 300))
    print(f"step batch={batch} {kv_dtype}", flush=True)
    dc = DevCase(case)
    out = dc.step()
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    _check_step(case, dc, out, case.new_k.unsqueeze(1), case.new_v.unsqueeze(1),
                case.slot_mapping)


@pytest.mark.parametrize("batch,kv_dtype", [(129, "bf16"), (9, "fp8")])
def test_step_value_head_dim_single_launch(batch, kv_dtype):
    """The 192 / 128 K / V pair through the single-launch step: 129 sequences
    (past one 64-lane block of the sequence table) and an fp8 pool."""
    case = synth.make_case(7, seed=97, kv_dtype=kv_dtype, batch=batch, lens=("uniform", 1, 200))
    print(f"step 192/128 batch={case.batch} {kv_dtype}", flush=True)
    dc = DevCase(case)
    out = dc.step()
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    _check_step(case, dc, out, case.new_k.unsqueeze(1), case.new_v.unsqueeze(1),
                case.slot_mapping)


@pytest.mark.parametrize("workload,over", [
    (3, dict(q_rows=1, causal=False, batch=5, lens=("uniform", 1, 900))),
    (4, dict(q_rows=2, causal=True, batch=3, lens=("uniform", 2, 900))),
], ids=["d256_bf16_decode", "d256_fp8_window2"])
def test_step_head_dim_256_single_launch(workload, over):
    """D = 256 with at most 16 rows per KV head (6 GQA heads x 1 or 2 window
    rows) takes the single-launch step with the fused append: bf16 and fp8
    pools, appended rows bit for bit, outputs against the oracle."""
    case = synth.make_case(workload, seed=98 + workload, append=True, **over)
    print(f"step d256 workload={workload} rows/kv={case.q_heads // case.kv_heads * case.q_rows}",
          flush=True)
    dc = DevCase(case)
    out = dc.step()
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    _check_step(case, dc, out, case.new_k.unsqueeze(1), case.new_v.unsqueeze(1),
                case.slot_mapping)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_step_head_dim_64_single_launch(kv_dtype):
    """D = 64 through the single-launch step with the fused append."""
    case = synth.make_case(2, seed=96, kv_dtype=kv_dtype, head_dim=64, batch=7,
                           lens=("uniform", 1, 600))
    print(f"step d64 {kv_dtype}", flush=True)
    dc = DevCase(case)
    out = dc.step()
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    _check_step(case, dc, out, case.new_k.unsqueeze(1), case.new_v.unsqueeze(1),
                case.slot_mapping)


SWEEP = {
    1: {},
    2: REDUCED[2],
    3: dict(batch=2, lens=("uniform", 300, 900)),
    4: dict(lens=("fixed", 700)),
    5: REDUCED[5],
}


@pytest.mark.parametrize("seed", range(102, 111))
@pytest.mark.parametrize("workload", [1, 2, 3, 4, 5])
def test_seed_sweep_step_matches_oracle(workload, seed):
    """Seeds 102-110 of every shape (reduced in size, same structure: dtypes,
    heads, page size, window rows, length distribution) through the step the
    benchmark times: append and read where the shape appends, else partial and
    merge; outputs against the oracle, pools bit for bit."""
    case = synth.make_case(workload, seed=seed, **SWEEP[workload])
    print(f"sweep workload={workload} seed={seed} lens={case.seq_lens.tolist()[:8]}", flush=True)
    dc = DevCase(case)
    out = dc.step()
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    if case.new_k is not None:
        _check_step(case, dc, out, case.new_k.unsqueeze(1), case.new_v.unsqueeze(1),
                    case.slot_mapping)
        return
    ref = oracle.attention(case.q, case.q_dtype, case.k_pool, case.v_pool, case.kv_dtype,
                           case.block_table, case.seq_lens, case.softmax_scale, case.causal,
                           case.k_scale, case.v_scale)
    assert torch.isfinite(out).all()
    err = max_abs(out, ref)
    assert err <= TOL[case.kv_dtype], f"max abs err {err}"


@pytest.mark.parametrize("new_dtype", [torch.float32, torch.bfloat16])
def test_step_bf16_new_tokens_and_fp8_pool(new_dtype):
    """bf16 new tokens (bit copy into a bf16 pool) and fp32/bf16 tokens into an fp8 pool."""
    for pool_dtype in ("bf16", "fp8"):
        case = synth.make_case(2, seed=41, kv_dtype=pool_dtype, batch=5, lens=("uniform", 1, 500))
        print(f"step new={new_dtype} pool={pool_dtype}", flush=True)
        dc = DevCase(case)
        nk = case.new_k.to(new_dtype).unsqueeze(1).cuda()
        nv = case.new_v.to(new_dtype).unsqueeze(1).cuda()
        out = dc.step(nk, nv)
        torch.cuda.synchronize()
        assert dc.err_bits() == 0
        _check_step(case, dc, out, nk, nv, case.slot_mapping)


def test_step_window_append_multirow_path():
    """16 new positions per sequence with 16 causal rows (a verify window): the
    shape runs the append, multi-row partial and merge kernels in turn."""
    case = synth.make_case(3, seed=44, batch=2, lens=("uniform", 300, 900))
    n_new = case.q_rows
    slots = _tail_slots(case, n_new)
    _poison_slots(case, slots)
    g = torch.Generator().manual_seed(44)
    shape = (case.batch, n_new, case.kv_heads, case.head_dim)
    nk = torch.randn(shape, generator=g)
    nv = torch.randn(shape, generator=g)
    dc = DevCase(case)
    out = dc.step(nk.cuda(), nv.cuda())
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    _check_step(case, dc, out, nk, nv, slots)


def test_step_fp32_pool_vector_path():
    case = synth.make_case(1, append=True)
    dc = DevCase(case)
    out = dc.step()
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    _check_step(case, dc, out, case.new_k.unsqueeze(1), case.new_v.unsqueeze(1),
                case.slot_mapping)


def test_step_two_new_positions_across_a_split_boundary():
    """n_new = 2 with the two positions in different splits (and items)."""
    case = synth.make_case(2, seed=45, append=False, batch=4, lens=("fixed", 257))
    n_new = 2                                  # positions 255 and 256: splits 0 and 1 at S=256
    slots = _tail_slots(case, n_new)
    _poison_slots(case, slots)
    g = torch.Generator().manual_seed(45)
    shape = (case.batch, n_new, case.kv_heads, case.head_dim)
    nk = torch.randn(shape, generator=g)
    nv = torch.randn(shape, generator=g)
    dc = DevCase(case)
    out = dc.step(nk.cuda(), nv.cuda(), n_split=2, split_size=256)
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    _check_step(case, dc, out, nk, nv, slots)


def test_step_without_new_tokens_equals_decode_bitwise():
    case = synth.make_case(2, seed=46, append=False, batch=6, lens=("uniform", 1, 700))
    a = DevCase(case).decode()
    b = DevCase(case).step()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_step_is_bitwise_repeatable_and_equals_two_call_path():
    case = synth.make_case(2, seed=47, batch=6, lens=("uniform", 1, 700))
    d1, d2 = DevCase(case), DevCase(case)
    s1 = d1.step()
    s2 = d2.step()
    d3 = DevCase(case)
    d3.append()
    ref = d3.decode()
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    assert torch.equal(s1, ref)
    # pools hold NaN poison in unused slots: compare their bytes
    assert np.array_equal(_pool_bits(d1.k), _pool_bits(d3.k))
    assert np.array_equal(_pool_bits(d1.v), _pool_bits(d3.v))


def test_step_sequence_shorter_than_new_tokens_is_flagged():
    case = synth.make_case(2, seed=48, batch=3, lens=("fixed", 40))
    case.seq_lens[1] = 0
    dc = DevCase(case)
    out = dc.step()
    torch.cuda.synchronize()
    assert dc.err_bits() & 0x4
    H = case.q_heads
    assert torch.all(out[H:2 * H] == 0)
    keep = [0, 2]
    kp, _ = oracle.append(case.new_k[keep], "f32", case.k_pool, case.kv_dtype, 1.0,
                          case.page_tokens, case.slot_mapping[keep])
    vp, _ = oracle.append(case.new_v[keep], "f32", case.v_pool, case.kv_dtype, 1.0,
                          case.page_tokens, case.slot_mapping[keep])
    ref = oracle.attention(case.q, case.q_dtype, kp, vp, case.kv_dtype, case.block_table,
                           case.seq_lens, case.softmax_scale)
    assert max_abs(out, ref) <= TOL["bf16"]


def _two_call_reference(case, lens, slots, n_split, split):
    """The step's work as separate calls: nbx_paged_kv_append at `slots` (-1:
    skipped), then nbx_paged_decode with the device lengths `lens`."""
    dref = DevCase(case)
    dref.lens = torch.as_tensor(np.asarray(lens, dtype=np.int32)).to(dref.q.device)
    kp, vp = dref.pools()
    nb.nbx_paged_kv_append(dref.new_k, dref.new_v, kp, vp,
                           torch.as_tensor(np.asarray(slots, dtype=np.int32)).to(dref.q.device),
                           dev_err=dref.err)
    return dref, dref.decode(n_split, split)


def test_step_sequence_past_its_block_table_row_equals_two_call_path():
    """A length past max_pages * page_tokens: the single-launch step writes no
    new row for that sequence (the separate append skips it and flags it) and
    reads the sequence clamped to its block-table row, exactly as the two
    separate calls do."""
    case = synth.make_case(2, seed=61, batch=5, lens=("uniform", 40, 300))
    cap = case.max_pages * case.page_tokens
    lens = case.seq_lens.copy()
    lens[2] = cap + 1
    slots = case.slot_mapping.copy()
    slots[2] = -1                              # the two-call path's append skips it too
    n_split, split = 8, 48                     # covers the whole row (8 * 48 >= cap)
    assert n_split * split >= cap
    print(f"step with seq_len {cap + 1} past the row of {cap}", flush=True)
    dc = DevCase(case)
    dc.lens = torch.as_tensor(lens).to(dc.q.device)
    out = dc.step(n_split=n_split, split_size=split)
    dref, ref = _two_call_reference(case, lens, slots, n_split, split)
    torch.cuda.synchronize()
    assert dc.err_bits() & nb.DEVERR_SEQ_RANGE
    assert dc.err_bits() == dref.err_bits()
    assert np.array_equal(_pool_bits(dc.k), _pool_bits(dref.k))
    assert np.array_equal(_pool_bits(dc.v), _pool_bits(dref.v))
    assert torch.equal(out, ref)


def test_step_new_position_past_the_split_cover_equals_two_call_path():
    """Splits that cover fewer positions than some sequences hold (flagged): the
    new rows past n_split * split_size are still written, as the separate append
    writes them, and the read covers the same positions on both paths."""
    case = synth.make_case(2, seed=62, batch=6, lens=("uniform", 100, 300))
    n_split, split = 2, 64
    assert int(case.seq_lens.max()) > n_split * split
    print(f"step with cover {n_split * split} < longest {int(case.seq_lens.max())}", flush=True)
    dc = DevCase(case)
    out = dc.step(n_split=n_split, split_size=split)
    dref, ref = _two_call_reference(case, case.seq_lens, case.slot_mapping, n_split, split)
    torch.cuda.synchronize()
    assert dc.err_bits() & nb.DEVERR_SEQ_RANGE
    assert dc.err_bits() == dref.err_bits()
    assert np.array_equal(_pool_bits(dc.k), _pool_bits(dref.k))
    assert np.array_equal(_pool_bits(dc.v), _pool_bits(dref.v))
    assert torch.equal(out, ref)


@pytest.mark.parametrize("workload", [2, 5])
def test_step_full_size_against_oracle(workload):
    case = synth.make_case(workload)
    print(f"full-size step workload={workload} kv_bytes={case.kv_bytes()}", flush=True)
    dc = DevCase(case)
    out = dc.step()
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    _check_step(case, dc, out, case.new_k.unsqueeze(1), case.new_v.unsqueeze(1),
                case.slot_mapping)


def test_step_partials_only_then_merge_equals_full_step():
    case = synth.make_case(2, seed=49, batch=6, lens=("uniform", 1, 700))
    n_split, split = DevCase(case).plan()
    full = DevCase(case).step()
    dc = DevCase(case)
    kp, vp = dc.pools()
    ws = torch.empty(nb.nbx_paged_decode_workspace_bytes(case.rows, n_split, case.head_dim),
                     dtype=torch.uint8, device="cuda")
    nb.nbx_paged_decode_step(dc.q, kp, vp, dc.bt, dc.lens, case.softmax_scale, split, n_split,
                             ws, None, new_k=dc.new_k.unsqueeze(1), new_v=dc.new_v.unsqueeze(1),
                             dev_err=dc.err)
    o, m, l = nb.workspace_partials(ws, case.rows, n_split, case.head_dim)
    out = torch.empty(case.rows, case.head_dim, device="cuda")
    nb.nbx_paged_decode_merge(o, m, l, out)
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    assert torch.equal(out, full)


def test_step_bf16_output():
    case = synth.make_case(2, seed=53, batch=4, lens=("uniform", 1, 600))
    dc = DevCase(case)
    out = dc.step(out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    kp, vp, _ = oracle.case_append(case)
    ref = oracle.attention(case.q, case.q_dtype, kp, vp, case.kv_dtype, case.block_table,
                           case.seq_lens, case.softmax_scale)
    err = np.abs(out.double().cpu().numpy().reshape(ref.shape) - ref)
    half_ulp = np.abs(ref) * 2.0 ** -8
    assert np.all(err <= TOL["bf16"] + half_ulp)


# ------------------------------------------------------------------ device-side plan and graph replay

@pytest.mark.parametrize("workload", [1, 2, 3, 5])
def test_device_derived_split_equals_host_plan(workload):
    """split_size = 0 derives the split length from the device lengths by the
    plan's own rule, so the partials are bitwise those of the host plan."""
    over = {1: dict(), 2: dict(batch=6, lens=("uniform", 1, 700)),
            3: dict(batch=2, lens=("uniform", 300, 900)),
            5: dict(batch=3, lens=("loguniform", 100, 3000))}[workload]
    case = synth.make_case(workload, seed=72, append=False, **over)
    dc = DevCase(case)
    n_split, split = dc.plan()
    o1, m1, l1 = dc.partial(n_split, split)
    o2, m2, l2 = dc.partial(n_split, 0)
    torch.cuda.synchronize()
    assert dc.err_bits() == 0
    assert torch.equal(m1, m2) and torch.equal(l1, l2)
    keep = torch.isfinite(m1)                  # an empty split's o is left unwritten
    assert torch.equal(o1[keep], o2[keep])


def test_rows_plan_fills_one_round_of_compute_units():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for B, hq, hkv, W, D, L in ((4, 24, 4, 16, 256, 32768), (1, 24, 4, 128, 256, 32768),
                                (2, 8, 2, 48, 128, 700), (64, 24, 4, 16, 256, 5000)):
        n, S = nb.nbx_paged_decode_plan_rows(B, hq, hkv, W, D, L)
        rows = hq // hkv * W
        per_block = 256 if rows > 128 and D <= 128 else 128
        units = B * hkv * -(-rows // per_block)
        assert n == max(1, min(cus // units, 64, -(-L // 16))), (B, hq, hkv, W, D, L, n)
        assert S == (-(-L // n) + 15) // 16 * 16


def test_lens_advance():
    lens = torch.tensor([0, 5, 100, 7], dtype=torch.int32, device="cuda")
    nb.nbx_paged_lens_advance(lens, 3)
    torch.cuda.synchronize()
    assert lens.tolist() == [3, 8, 103, 10]


@pytest.mark.parametrize("bounds", [False, True], ids=["running_max", "fixed_shift"])
def test_step_graph_replays_as_lengths_grow(bounds):
    """One recorded graph of [lens advance, step with a device-derived split]
    replayed for four tokens: every replay appends at the new last position and
    attends to it, with the launch arguments unchanged.  With pool bounds the
    append inside the step raises them and the reads take the fixed shift."""
    steps = 4
    case = synth.make_case(2, seed=71, append=False, batch=5, lens=("uniform", 40, 600))
    final = case.seq_lens.copy()
    start = final - steps
    T = case.page_tokens
    slots = [np.array([int(case.block_table[b, p // T]) * T + p % T
                       for b, p in enumerate(start + k)], dtype=np.int32) for k in range(steps)]
    _poison_slots(case, np.concatenate(slots))
    n_split, _ = nb.nbx_paged_decode_plan(int(final.max()), 256, 64)
    H, D = case.kv_heads, case.head_dim

    # warm-up on a copy (fills the library's per-device launch cache)
    warm = DevCase(case)
    warm.lens.copy_(torch.from_numpy(start + 1))
    warm.step(torch.zeros(case.batch, 1, H, D, device="cuda"),
              torch.zeros(case.batch, 1, H, D, device="cuda"), n_split=n_split, split_size=0)
    torch.cuda.synchronize()

    dc = DevCase(case)
    dc.lens.copy_(torch.from_numpy(start))
    if bounds:
        dc.attach_bounds(lens=start)
    kp, vp = dc.pools()
    ws = torch.zeros(nb.nbx_paged_decode_workspace_bytes(case.rows, n_split, D),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty(case.batch, case.q_heads, 1, D, device="cuda")
    nk = torch.zeros(case.batch, 1, H, D, device="cuda")
    nv = torch.zeros_like(nk)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nb.nbx_paged_lens_advance(dc.lens, 1)
        nb.nbx_paged_decode_step(dc.q, kp, vp, dc.bt, dc.lens, case.softmax_scale, 0, n_split, ws,
                                 out, new_k=nk, new_v=nv, dev_err=dc.err)
    gen = torch.Generator().manual_seed(71)
    k_ref, v_ref = case.k_pool, case.v_pool
    for k in range(steps):
        tok_k = torch.randn(case.batch, 1, H, D, generator=gen)
        tok_v = torch.randn(case.batch, 1, H, D, generator=gen)
        nk.copy_(tok_k)
        nv.copy_(tok_v)
        g.replay()
        torch.cuda.synchronize()
        k_ref, _ = oracle.append(tok_k.reshape(-1, H, D), "f32", k_ref, case.kv_dtype, 1.0, T, slots[k])
        v_ref, _ = oracle.append(tok_v.reshape(-1, H, D), "f32", v_ref, case.kv_dtype, 1.0, T, slots[k])
        lens_k = (start + k + 1).astype(np.int32)
        assert dc.lens.cpu().numpy().tolist() == lens_k.tolist()
        ref = oracle.attention(case.q, case.q_dtype, k_ref, v_ref, case.kv_dtype,
                               case.block_table, lens_k, case.softmax_scale)
        print(f"replay {k}: lens {lens_k.tolist()}", flush=True)
        assert dc.err_bits() == 0
        assert torch.isfinite(out).all()
        assert max_abs(out.reshape(case.rows, D), ref) <= TOL["bf16"]
    if bounds:
        # every split of the last replay took a fixed shift (an integer in log2 units)
        _, m, l = nb.workspace_partials(ws, case.rows, n_split, D)
        m_np, l_np = m.double().cpu().numpy(), l.double().cpu().numpy()
        kq = m_np[l_np > 0] / np.log(2.0)
        assert kq.size and np.all(np.abs(kq - np.round(kq)) < 1e-4)
        # the bounds cover the appended rows: equal to the oracle's over the final lengths
        rk = oracle.kv_bounds(k_ref, case.kv_dtype, case.block_table, final, is_value=False)
        rv = oracle.kv_bounds(v_ref, case.kv_dtype, case.block_table, final, is_value=True)
        gk, gv = dc.kb.double().cpu().numpy(), dc.vb.double().cpu().numpy()
        assert np.all(np.abs(gk - rk) <= 1e-5 * rk) and np.array_equal(gv, rv)


def test_prompt_chunk_chain_over_a_growing_cache():
    """Three 128-row prompt chunks in turn (fp8 pool, the prompt-chunk shape):
    each step appends its 128 positions and attends causally over the cache so
    far, through the multi-row path."""
    chunk, n_chunks = 128, 3
    case = synth.make_case(4, seed=91, append=False, lens=("fixed", 200 + chunk * n_chunks))
    final = int(case.seq_lens[0])
    T, H, D = case.page_tokens, case.kv_heads, case.head_dim
    first = final - chunk * n_chunks
    slots = np.array([int(case.block_table[0, p // T]) * T + p % T
                      for p in range(first, final)], dtype=np.int32)
    _poison_slots(case, slots)
    gen = torch.Generator().manual_seed(91)
    dc = DevCase(case)
    k_ref, v_ref = case.k_pool, case.v_pool
    for i in range(n_chunks):
        L = first + chunk * (i + 1)
        dc.lens.fill_(L)
        nk = torch.randn(1, chunk, H, D, generator=gen)
        nv = torch.randn(1, chunk, H, D, generator=gen)
        q = torch.randn(1, case.q_heads, chunk, D, generator=gen).to(torch.bfloat16)
        dc.q.copy_(q)
        n_split, split = nb.nbx_paged_decode_plan(L, 2048, 16)
        out = dc.step(nk.cuda(), nv.cuda(), n_split=n_split, split_size=split)
        torch.cuda.synchronize()
        sl = slots[chunk * i:chunk * (i + 1)]
        k_ref, _ = oracle.append(nk.reshape(-1, H, D), "f32", k_ref, "fp8", case.k_scale, T, sl)
        v_ref, _ = oracle.append(nv.reshape(-1, H, D), "f32", v_ref, "fp8", case.v_scale, T, sl)
        ref = oracle.attention(q, "bf16", k_ref, v_ref, "fp8", case.block_table,
                               np.array([L], dtype=np.int32), case.softmax_scale, True,
                               case.k_scale, case.v_scale)
        print(f"chunk {i}: keys {L}", flush=True)
        assert dc.err_bits() == 0
        assert torch.isfinite(out).all()
        assert max_abs(out, ref) <= TOL["fp8"]
