"""nbx_paged_decode_step_noalloc (the step with its partials in the library's
static device scratch) against nbx_paged_decode_step with a caller workspace:
the same kernels on the same inputs, so outputs, pools and error bits agree
bit for bit.  Two calls in a row share the one scratch array, the second on a
smaller input, so partials left by the first must not leak into the second."""
import numpy as np
import pytest
import torch

from paged_split_kv_append_amd import binding as nb
from paged_split_kv_append_amd import synth

from gpu_cases import DevCase

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.uint8).numpy().reshape(-1)


def _noalloc(dc: DevCase, n_split, split_size, out_dtype=torch.float32):
    c = dc.case
    kp, vp = dc.pools()
    out = torch.empty(c.batch, c.q_heads, c.q_rows, c.v_head_dim, dtype=out_dtype,
                      device=dc.q.device)
    new_k = dc.new_k.unsqueeze(1) if dc.new_k is not None else None
    new_v = dc.new_v.unsqueeze(1) if dc.new_v is not None else None
    nb.nbx_paged_decode_step_noalloc(dc.q, kp, vp, dc.bt, dc.lens, c.softmax_scale, split_size,
                                     n_split, out, new_k=new_k, new_v=new_v, causal=c.causal,
                                     dev_err=dc.err)
    return out.reshape(c.rows, c.v_head_dim)


def _same_as_workspace_step(case, out_dtype=torch.float32):
    a, b = DevCase(case), DevCase(case)
    n_split, split = a.plan()
    got = _noalloc(a, n_split, split, out_dtype)
    ref = b.step(n_split=n_split, split_size=split, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert a.err_bits() == b.err_bits() == 0
    assert np.array_equal(_bits(a.k), _bits(b.k))
    assert np.array_equal(_bits(a.v), _bits(b.v))
    assert torch.isfinite(got).all()
    assert torch.equal(got, ref)


@pytest.mark.parametrize("first,second", [
    # the single-launch step (bf16 pool, 4 query rows per KV head), then a
    # smaller one with an fp8 pool
    (dict(workload=2, batch=32, lens=("uniform", 1, 4096)),
     dict(workload=2, batch=5, kv_dtype="fp8", lens=("uniform", 1, 700))),
    # 96 query rows per KV head (a 16-row verify window over 6 query heads:
    # append, multi-row partial and merge in turn), then a single-launch step
    # of fewer rows
    (dict(workload=3, batch=3, lens=("uniform", 16, 2000), append=True),
     dict(workload=2, batch=3, lens=("uniform", 1, 300))),
], ids=["decode_then_smaller_fp8", "window_then_smaller_decode"])
def test_noalloc_step_equals_workspace_step_twice(first, second):
    for i, kw in enumerate((first, second)):
        kw = dict(kw)
        case = synth.make_case(kw.pop("workload"), seed=300 + i, **kw)
        n_split, _ = DevCase(case).plan()
        need = nb.nbx_paged_decode_workspace_bytes(case.rows, n_split, case.v_head_dim)
        print(f"noalloc call {i}: batch {case.batch} rows {case.rows} {case.kv_dtype} "
              f"partials {need} B", flush=True)
        assert 0 < need <= nb.STEP_SCRATCH_BYTES
        _same_as_workspace_step(case, torch.bfloat16 if i else torch.float32)


def test_noalloc_step_refuses_partials_past_the_scratch():
    """Partials larger than the scratch: refused on the host, nothing launched,
    the pools untouched."""
    case = synth.make_case(2, seed=310, batch=4, lens=("uniform", 1, 100))
    dc = DevCase(case)
    n_split = 1024                             # rows * 1024 * Dv * 4 bytes > 32 MiB
    assert nb.nbx_paged_decode_workspace_bytes(case.rows, n_split, case.v_head_dim) > \
        nb.STEP_SCRATCH_BYTES
    k0, v0 = _bits(dc.k), _bits(dc.v)
    with pytest.raises(nb.NbxError) as e:
        _noalloc(dc, n_split, 16)
    assert e.value.status == nb.NBX_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert np.array_equal(_bits(dc.k), k0) and np.array_equal(_bits(dc.v), v0)
