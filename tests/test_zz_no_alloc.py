"""gattn_decode_noalloc (split partials in the library's per-GPU scratch array, no workspace
argument) against gattn_decode (caller workspace) on the same inputs: bit for bit, and within the
oracle's tolerances. Two calls in a row, the second with a smaller input (the scratch keeps the
first call's partials; the second must read only its own), then a third of the other family, and
an oversized call that must be rejected with nothing written."""
import numpy as np
import pytest

import __graft_entry__

__graft_entry__.ensure_built()

import oracle  # noqa: E402
import workloads  # noqa: E402

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 1e-2, 1e-3


def _noalloc(nat, d, b, split, max_ctx):
    import torch
    out = torch.full_like(d.out, 0x7FC0)   # bf16 NaN bits
    lse = torch.full_like(d.lse, float("nan"))
    nat.gattn_decode_noalloc(d.layer, d.q, d.k_pool, d.v_pool, d.num_pages, d.page_table, d.pt_stride, d.ctx_lens,
                             b.B, max_ctx, split, out, lse)
    torch.cuda.synchronize()
    from global_paged_gqa_amd import devio
    return devio.host_bf16(out).astype(np.float64), lse.cpu().numpy().astype(np.float64)


def test_noalloc_decode_matches_workspace_decode():
    import torch
    assert torch.cuda.is_available()
    from global_paged_gqa_amd import _native as nat
    from global_paged_gqa_amd import devio
    cases = [("global 32 rows (33.6 MB of partials)", workloads.cfg2_global_decode(), 512),
             ("global 8 rows, shorter", workloads.cfg2_global_decode(B=8, max_len=3000), 512),
             ("local 12 rows", workloads.cfg3_local_decode(B=12, lo=1, hi=6000), 512)]
    for tag, b, split in cases:
        max_ctx = int(b.ctx_lens.max())
        need = nat.gattn_decode_workspace_bytes(devio.layer_of(b.spec), b.B, max_ctx, split)
        assert 0 < need <= nat.NOALLOC_SCRATCH_BYTES
        d = devio.DeviceBatch(b)
        d.decode(split, max_ctx)
        ref_o, ref_l = d.result()
        o, l = _noalloc(nat, d, b, split, max_ctx)
        assert np.array_equal(o, ref_o) and np.array_equal(l, ref_l), tag
        want_o, want_l = oracle.attend_batch(b)
        eo, el = float(np.max(np.abs(o - want_o))), float(np.max(np.abs(l - want_l)))
        print(f"noalloc {tag}: bitwise equal to gattn_decode; max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
        assert eo <= TOL_O and el <= TOL_LSE


def test_noalloc_rejects_oversized_call_with_nothing_written():
    import torch
    from global_paged_gqa_amd import _native as nat
    from global_paged_gqa_amd import devio
    b = workloads.cfg2_global_decode(B=2, max_len=100, pt_stride=12500)
    d = devio.DeviceBatch(b)
    assert tuple(d.page_table.shape) == (2, 12500)
    out = torch.zeros_like(d.out)
    lse = torch.zeros_like(d.lse)
    # a grid bound of 2 rows x 200000 tokens at split 16: 2 * 32 * 12500 * 513 * 4 B > 64 MiB (the table
    # really has that stride, so even a launch would stay in bounds)
    with pytest.raises(nat.GattnError) as e:
        nat.gattn_decode_noalloc(d.layer, d.q, d.k_pool, d.v_pool, d.num_pages, d.page_table, 12500, d.ctx_lens,
                                 b.B, 200000, 16, out, lse)
    assert e.value.status == nat.ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(out)) == 0 and int(torch.count_nonzero(lse)) == 0
