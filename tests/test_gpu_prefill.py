"""Chunked causal prefill on the GPU against the fp64 oracle (O max-abs 1e-2, LSE 1e-3),
chunk parity, the mixed prefill + decode step, window counts and bitwise invariances."""
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


def oracle_queries(batch, picks):
    """Oracle outputs for chosen (row, query index) pairs: each query alone, attending the row's
    keys up to its own position (the oracle is a pure function of the position and those keys)."""
    s = batch.spec
    cq = batch.cu_q
    qs, ks, vs, lens, starts = [], [], [], [], []
    for r, i in picks:
        L, C, k0 = int(batch.ctx_lens[r]), int(batch.q_lens[r]), int(batch.k_starts[r])
        p = L - C + i
        kk, vv = batch.row_keys(r)
        qs.append(batch.q[cq[r] + i:cq[r] + i + 1])
        ks.append(kk[:p + 1 - k0])
        vs.append(vv[:p + 1 - k0])
        lens.append(p + 1)
        starts.append(k0)
    return oracle.attend(s.is_global, s.num_q_heads, s.num_kv_heads, s.head_dim, s.window, s.softmax_scale,
                         [1] * len(picks), lens, starts, np.concatenate(qs), np.concatenate(ks),
                         None if s.kv_shared else np.concatenate(vs))


def check(batch, out, lse, picks=None, tag="", bf16_slack=False):
    """O within 1e-2 and LSE within 1e-3 of the oracle. bf16_slack (only for geometries outside
    the 31B configs, where a query can see one or two keys at a sharp scale and |O| can pass 2.5)
    also admits the output format's own rounding: half a bf16 ulp of the reference, 2^-9 |O|."""
    if picks is None:
        ref_o, ref_l = oracle.attend_batch(batch)
    else:
        ref_o, ref_l = oracle_queries(batch, picks)
        idx = [int(batch.cu_q[r]) + i for r, i in picks]
        out, lse = out[idx], lse[idx]
    err = np.abs(out - ref_o)
    if bf16_slack:
        err = err - np.abs(ref_o) * 2.0 ** -9
    eo = float(np.max(err))
    el = float(np.max(np.abs(lse - ref_l)))
    print(f"{tag}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    assert eo <= TOL_O and el <= TOL_LSE, (eo, el)


SMALL = [  # (ctx_lens, q_lens)
    ([300], [200]),
    ([1], [1]),
    ([17, 16, 33], [17, 1, 5]),
    ([1100, 40, 2049], [1100, 40, 70]),
    ([5000, 1200], [130, 1200]),
]


@pytest.mark.parametrize("spec", [workloads.GLOBAL_31B, workloads.LOCAL_31B, workloads.GLOBAL_31B_KV_SHARED,
                                  workloads.LayerSpec("local", 12, 4, 512, window=100, scale=0.05),
                                  workloads.LayerSpec("global", 16, 1, 256)],
                         ids=["global", "local", "global-kv-shared", "local-hd512-g3", "global-hd256-g16"])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_prefill_small(devio, spec, case):
    L, C = SMALL[case]
    b = workloads.make_batch(spec, L, C, (30, case, spec.head_dim, spec.group), back="visible", poison=True)
    out, lse = devio.prefill(b)
    off_config = spec not in (workloads.GLOBAL_31B, workloads.LOCAL_31B, workloads.GLOBAL_31B_KV_SHARED)
    check(b, out, lse, tag=f"{spec.family} hd{spec.head_dim} g{spec.group} case{case}", bf16_slack=off_config)


def test_prefill_zero_length_rows(devio):
    spec = workloads.LOCAL_31B
    b = workloads.make_batch(spec, [50, 20, 70], [10, 0, 70], (31, 0), back="visible")
    out, lse = devio.prefill(b, max_q=70)
    check(b, out, lse, tag="zero-length row")


@pytest.fixture(scope="module", params=["global", "local"])
def cfg4_step(request, devio):
    """The mixed step at full size (4 prefill rows of 2048 queries after priors U{0..6144}, 60
    decode rows with contexts U{1..8192}): gattn_prefill then gattn_decode on one stream, the
    launch pair the benchmark times; results copied back once both have run."""
    import torch
    pre, dec = workloads.cfg4_mixed(request.param)
    dp, dd = devio.DeviceBatch(pre), devio.DeviceBatch(dec)
    stream = torch.cuda.current_stream()
    dp.prefill(stream=stream)
    dd.decode(512, stream=stream)
    torch.cuda.synchronize()
    return request.param, pre, dec, dp.result(), dd.result()


def test_cfg4_outputs_all_finite(cfg4_step):
    family, pre, dec, (out, lse), (dout, dlse) = cfg4_step
    assert out.shape[0] == int(pre.q_lens.sum()) and dout.shape[0] == dec.B
    for a in (out, lse, dout, dlse):
        assert np.all(np.isfinite(a)), family


def test_cfg4_prefill_full_rows(cfg4_step):
    """Every query of whole prefill rows against the oracle: all four local rows; for the global
    family the row with the shortest prior (about 3e11 fp64 flop), the others on sampled queries
    (chunk, tile and window edges, and random ones)."""
    family, pre, _, (out, lse), _ = cfg4_step
    full = list(range(pre.B)) if family == "local" else [int(np.argmin(pre.ctx_lens - pre.q_lens))]
    for r in full:
        ref_o, ref_l = oracle.attend_batch(pre, [r])
        cq = pre.cu_q
        o, l = out[cq[r]:cq[r + 1]], lse[cq[r]:cq[r + 1]]
        eo, el = float(np.max(np.abs(o - ref_o))), float(np.max(np.abs(l - ref_l)))
        print(f"cfg4 {family} prefill row {r} (all {cq[r + 1] - cq[r]} queries): max|dO|={eo:.3e} "
              f"max|dLSE|={el:.3e}", flush=True)
        assert eo <= TOL_O and el <= TOL_LSE, (r, eo, el)
    rng = np.random.default_rng(3)
    picks = []
    for r in range(pre.B):
        if r in full:
            continue
        C = int(pre.q_lens[r])
        fixed = [0, 1, 7, 8, 15, 16, 63, 64, 127, 128, 1023, 1024, C - 2, C - 1]
        picks += [(r, i) for i in sorted(set([i for i in fixed if 0 <= i < C] + list(rng.integers(0, C, 10))))]
    if picks:
        check(pre, out, lse, picks, tag=f"cfg4 {family} prefill (sampled on the other rows)")


def test_cfg4_decode_rows_after_prefill(cfg4_step):
    """All 60 decode rows of the step, issued after the prefill on the same stream, against the
    oracle element by element."""
    family, _, dec, _, (dout, dlse) = cfg4_step
    check(dec, dout, dlse, tag=f"cfg4 {family} decode rows after the prefill")


@pytest.mark.parametrize("family", ["global", "local"])
def test_chunk_parity(devio, family):
    """A prompt walked in 64-token chunks, in one chunk, and token by token (decode) each match
    the oracle; the oracle itself gives the same numbers for all three walks."""
    spec = workloads.GLOBAL_31B if family == "global" else workloads.LayerSpec("local", 32, 16, 256, window=100)
    N = 300
    whole = workloads.make_batch(spec, [N], [N], (32, 0), back="all")
    out_w, lse_w = devio.prefill(whole)
    check(whole, out_w, lse_w, tag="whole chunk")
    ref_o, ref_l = oracle.attend_batch(whole)
    for s in range(0, N, 64):
        e = min(N, s + 64)
        part = workloads.Batch(spec, np.array([e], np.int32), np.array([e - s], np.int32), np.zeros(1, np.int32),
                               whole.q[s:e], whole.k[:e], None if whole.v is None else whole.v[:e],
                               whole.page_table, whole.k_pool, whole.v_pool)
        o, l = devio.prefill(part)
        assert np.max(np.abs(o - ref_o[s:e])) <= TOL_O and np.max(np.abs(l - ref_l[s:e])) <= TOL_LSE
    for t in (0, 1, 63, 64, 150, 299):
        one = workloads.Batch(spec, np.array([t + 1], np.int32), np.array([1], np.int32), np.zeros(1, np.int32),
                              whole.q[t:t + 1], whole.k[:t + 1], None if whole.v is None else whole.v[:t + 1],
                              whole.page_table, whole.k_pool, whole.v_pool)
        o, l = devio.decode(one, 0)
        assert np.max(np.abs(o[0] - ref_o[t])) <= TOL_O and np.max(np.abs(l[0] - ref_l[t])) <= TOL_LSE


def test_mixed_step_on_one_stream(devio):
    """Prefill rows and decode rows of one layer issued back to back on one stream."""
    import torch
    for family in ("global", "local"):
        pre, dec = workloads.cfg4_mixed(family, n_prefill=2, chunk=512, max_prior=2000, n_decode=12,
                                        max_decode_len=3000)
        dp, dd = devio.DeviceBatch(pre), devio.DeviceBatch(dec)
        dp.prefill()
        dd.decode(512)
        torch.cuda.synchronize()
        check(pre, *dp.result(), tag=f"mixed {family}: prefill rows")
        check(dec, *dd.result(), tag=f"mixed {family}: decode rows")


def test_window_counts_multi_window_chunk(devio):
    """K = 0 over a 3*1024+5 chunk with prior 0: exp(LSE) = min(p + 1, 1024) for every query."""
    spec = workloads.LayerSpec("local", 4, 2, 256, window=1024)
    C = 3 * 1024 + 5
    b = workloads.make_batch(spec, [C], [C], (33, 0), back="all")
    b.k_pool[:] = 0
    _, lse = devio.prefill(b)
    n = np.minimum(np.arange(C) + 1, 1024)
    assert np.array_equal(np.round(np.exp(lse)).astype(np.int64), np.repeat(n[:, None], 4, 1))


@pytest.mark.parametrize("spec", [workloads.LayerSpec("local", 4, 2, 256, window=1024, scale=1.0),
                                  workloads.LayerSpec("global", 16, 2, 512, scale=1.0)], ids=["local", "global"])
def test_prefill_position_probe(devio, spec):
    """One key dominates: every query is e_0 and K[t*] = 200 e_0 (all other keys 0), so for a query
    that sees t* every other weight underflows to exactly 0 and O must equal V[t*] bit for bit; a
    query that cannot see t* (before it, or past the window) gets the uniform mean of the others.
    t* sweeps page, 32-key block, query-tile and window edges of a 1300-query chunk after 200
    cached tokens."""
    prior, C = 200, 1300
    L = prior + C
    for t_star in (0, 15, 16, 31, 32, 199, 200, 201, 263, 264, 700, 1023, 1024, L - 1):
        b = workloads.make_batch(spec, [L], [C], (35, t_star), back="all")
        P = spec.page_size
        b.q[:] = 0
        b.q[:, :, 0] = workloads.f32_to_bf16_bits(np.float32([1.0]))[0]
        kk = np.zeros_like(b.k)
        kk[t_star, :, 0] = workloads.f32_to_bf16_bits(np.float32([200.0]))[0]
        code = workloads.f32_to_bf16_bits(np.float32(np.arange(spec.head_dim) + 0.5 + (t_star % 97)))
        vv = b.v.copy()
        vv[t_star] = code
        for t in range(L):
            b.k_pool[b.page_table[0, t // P], :, t % P, :] = kk[t]
            b.v_pool[b.page_table[0, t // P], :, t % P, :] = vv[t]
        b.k[:] = kk
        b.v[:] = vv
        out, lse = devio.prefill(b)
        want = workloads.bf16_bits_to_f32(code).astype(np.float64)
        pos = prior + np.arange(C)
        sees = (pos >= t_star) & ((pos - t_star < spec.window) if not spec.is_global else True)
        assert sees.any(), t_star
        for i in np.nonzero(sees)[0]:
            for h in range(spec.num_q_heads):
                assert np.array_equal(out[i, h], want), (t_star, i, h)
        check(b, out, lse, tag=f"{spec.family} position probe t*={t_star}", bf16_slack=True)


def test_prefill_bitwise_invariances(devio):
    spec = workloads.GLOBAL_31B
    b = workloads.make_batch(spec, [700, 300, 1500], [200, 300, 90], (34, 0), back="all")
    o1, l1 = devio.prefill(b)
    o2, l2 = devio.prefill(b)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    bp = workloads.permute_pages(b, (34, 1), extra_pages=3, fill=int(workloads.BF16_NAN))
    o3, l3 = devio.prefill(bp)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)
    bn = workloads.make_batch(spec, [700, 300, 1500], [200, 300, 90], (34, 0), back="all", poison=True)
    o4, l4 = devio.prefill(bn)
    assert np.array_equal(o1, o4) and np.array_equal(l1, l4)
    # one row alone gives the same bits as inside the batch
    cq = b.cu_q
    sub = workloads.Batch(spec, b.ctx_lens[[2]], b.q_lens[[2]], b.k_starts[[2]], b.q[cq[2]:cq[3]], b.k, b.v,
                          b.page_table[[2]], b.k_pool, b.v_pool)
    o5, l5 = devio.prefill(sub)
    assert np.array_equal(o5, o1[cq[2]:cq[3]]) and np.array_equal(l5, l1[cq[2]:cq[3]])


@pytest.mark.parametrize("family", ["global", "local"])
def test_mixed_step_single_launch(devio, family):
    """A mixed step's prefill rows and q_len-1 decode rows as one batch in one gattn_prefill call:
    every output against the oracle (decode rows at their full visible range)."""
    pre, dec = workloads.cfg4_mixed(family, n_prefill=2, chunk=300, max_prior=1500, n_decode=10,
                                    max_decode_len=3000)
    mix = workloads.concat_batches(pre, dec)
    out, lse = devio.prefill(mix)
    check(mix, out, lse, tag=f"single-launch mixed {family}")


@pytest.mark.parametrize("spec", [workloads.GLOBAL_31B, workloads.LOCAL_31B], ids=["global", "local"])
def test_prefill_fails_closed(devio, spec):
    """Device-side data the call cannot serve gives NaN O and LSE for the affected rows only, with
    no read outside the table or the pool: page 0 (seen by every query, contexts < window) out of
    range (row 1) or -1 (row 3); more queries than cached tokens (row 4); a context past the page
    table (row 5); more queries than max_q (row 6: 700 queries against max_q 300, so its queries
    past the grid's last tile are written NaN as well). Rows 0 and 2 match the oracle and are
    bitwise what a clean call gives them."""
    import torch
    L = np.array([700, 400, 650, 300, 500, 450, 900], np.int32)
    C = np.array([200, 150, 100, 120, 50, 60, 700], np.int32)
    b = workloads.make_batch(spec, L, C, (36, spec.head_dim), back="visible")
    d = devio.DeviceBatch(b)
    d.prefill(max_q=700)
    clean_o, clean_l = d.result()
    pt = b.page_table.copy()
    pt[1, 0] = b.num_pages + 3
    pt[3, 0] = -1
    d.page_table.copy_(torch.from_numpy(pt).cuda())
    cl = b.ctx_lens.copy()
    cl[4] = C[4] - 1
    cl[5] = b.pt_stride * 16 + 1
    d.ctx_lens.copy_(torch.from_numpy(cl).cuda())
    d.out.fill_(0)
    d.lse.fill_(0)
    d.prefill(max_q=300)
    out, lse = d.result()
    cq = b.cu_q
    for r in range(b.B):
        o, l = out[cq[r]:cq[r + 1]], lse[cq[r]:cq[r + 1]]
        if r in (0, 2):
            assert np.array_equal(o, clean_o[cq[r]:cq[r + 1]]) and np.array_equal(l, clean_l[cq[r]:cq[r + 1]]), r
        else:
            assert np.all(np.isnan(o)) and np.all(np.isnan(l)), r
    ref_o, ref_l = oracle.attend_batch(b, [0, 2])
    idx = np.concatenate([np.arange(cq[0], cq[1]), np.arange(cq[2], cq[3])])
    eo, el = float(np.max(np.abs(out[idx] - ref_o))), float(np.max(np.abs(lse[idx] - ref_l)))
    print(f"{spec.family} fail-closed good rows: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O and el <= TOL_LSE
