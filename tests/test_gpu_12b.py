"""The 12B geometry on the GPU against the fp64 oracle (O max-abs 1e-2, LSE max-abs 1e-3).

Global family: 16 query heads over a single KV head (g = 16, head_dim 512), the degenerate
block-GQA case where a row's parallelism comes only from its splits. Local family: 16 query
heads over 8 KV heads, head_dim 256, window 1024. Decode at small and full batch (both run a
split's two page streams on two waves), chunked prefill on small
ragged rows and on the 12B mixed step's prefill rows (sampled queries).
"""
import numpy as np
import pytest

import __graft_entry__

__graft_entry__.ensure_built()

import oracle  # noqa: E402
import workloads  # noqa: E402

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 1e-2, 1e-3


@pytest.fixture(scope="module")
def devio():
    import torch
    assert torch.cuda.is_available()
    from global_paged_gqa_amd import devio as d
    return d


def check(ref, out, lse, tag):
    ref_o, ref_l = ref
    eo = float(np.max(np.abs(out - ref_o)))
    el = float(np.max(np.abs(lse - ref_l)))
    print(f"{tag}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    assert eo <= TOL_O and el <= TOL_LSE, (tag, eo, el)


@pytest.mark.parametrize("split", [512, 1024, 0])
def test_12b_global_decode_small(devio, split):
    b = workloads.cfg6_12b_global_decode(B=8, max_len=4000, poison=True)
    out, lse = devio.decode(b, split)
    check(oracle.attend_batch(b), out, lse, f"12B global decode B=8 split {split}")


def test_12b_global_decode_full(devio):
    b = workloads.cfg6_12b_global_decode()
    out, lse = devio.decode(b, 512)
    check(oracle.attend_batch(b), out, lse, "12B global decode B=32")


def test_12b_local_decode(devio):
    L = workloads.ragged((6, 2), 1, 9000, 12)
    L[0], L[1] = 1024, 1025
    b = workloads.make_batch(workloads.LOCAL_12B, L, np.ones(12, np.int32), (6, 2), back="visible", poison=True)
    out, lse = devio.decode(b, 512)
    check(oracle.attend_batch(b), out, lse, "12B local decode")


@pytest.mark.parametrize("spec", [workloads.GLOBAL_12B, workloads.LOCAL_12B], ids=["global", "local"])
def test_12b_prefill_small(devio, spec):
    b = workloads.make_batch(spec, [300, 1, 1100, 2049], [200, 1, 1100, 70], (6, 3, spec.num_kv_heads),
                             back="visible", poison=True)
    out, lse = devio.prefill(b)
    check(oracle.attend_batch(b), out, lse, f"12B {spec.family} prefill small")


@pytest.mark.parametrize("family", ["global", "local"])
def test_12b_mixed_prefill_sampled(devio, family):
    """The 12B mixed step's prefill rows at full size (4 x 2048 queries), sampled queries checked
    against the oracle; every output finite."""
    pre, _ = workloads.cfg6_12b_mixed(family)
    out, lse = devio.prefill(pre)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    rng = np.random.default_rng(6)
    picks = []
    for r in range(pre.B):
        C = int(pre.q_lens[r])
        fixed = [0, 1, 7, 8, 127, 128, 1023, 1024, C - 1]
        picks += [(r, i) for i in sorted(set(fixed + list(rng.integers(0, C, 6))))]
    s = pre.spec
    cq = pre.cu_q
    qs, ks, vs, lens, starts = [], [], [], [], []
    for r, i in picks:
        L, C, k0 = int(pre.ctx_lens[r]), int(pre.q_lens[r]), int(pre.k_starts[r])
        p = L - C + i
        kk, vv = pre.row_keys(r)
        qs.append(pre.q[cq[r] + i:cq[r] + i + 1])
        ks.append(kk[:p + 1 - k0])
        vs.append(vv[:p + 1 - k0])
        lens.append(p + 1)
        starts.append(k0)
    ref = oracle.attend(s.is_global, s.num_q_heads, s.num_kv_heads, s.head_dim, s.window, s.softmax_scale,
                        [1] * len(picks), lens, starts, np.concatenate(qs), np.concatenate(ks),
                        None if s.kv_shared else np.concatenate(vs))
    idx = [int(cq[r]) + i for r, i in picks]
    check(ref, out[idx], lse[idx], f"12B {family} mixed prefill (sampled)")
