"""Pins for the fp64 oracle: checks against things the pages and the mathematics fix.

Each test names what it pins. None of them compares the oracle with itself through
a retyped formula: brute force uses its own mask/mapping/softmax formulation at 50
digits, closed forms are exact, boundary counts follow from the window definition,
and the bytes-per-token figure is printed on the Core AI card.
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from brute import as_floats, brute_attend
from conftest import read_golden


def _draw(key, shape):
    return workloads.normal_bf16(workloads.generator(*key), shape)


def _tiny_case(key, L, Hq, Hkv, hd):
    q = _draw((900, *key, 0), (L, Hq, hd))
    k = _draw((900, *key, 1), (L, Hkv, hd))
    v = _draw((900, *key, 2), (L, Hkv, hd))
    return q, k, v


# ---------------------------------------------------------------- P1: brute force on tiny inputs
TINY = []
_rng = np.random.default_rng(7)
for L in (1, 2, 3, 5, 9, 17, 40):
    for W in sorted({1, 2, 3, 7, max(1, L - 1), L, L + 1}):
        for fam in ("local", "global"):
            if fam == "global" and W != 1:
                continue
            for shared in (False, True):
                heads = [(2, 1), (4, 2), (3, 3), (6, 2)][int(_rng.integers(0, 4))]
                hd = (1, 2, 4)[int(_rng.integers(0, 3))]
                TINY.append((L, W, fam, shared, heads, hd))


@pytest.mark.parametrize("L,W,fam,shared,heads,hd", TINY)
def test_p1_brute_force_prefill_all_positions(L, W, fam, shared, heads, hd):
    """One prefill over the whole row covers every decode prefix length 1..L."""
    Hq, Hkv = heads
    q, k, v = _tiny_case((L, W, hd, Hq, Hkv, int(shared)), L, Hq, Hkv, hd)
    if shared:
        v = k
    scale = 0.37
    is_g = fam == "global"
    out, lse = oracle.attend(is_g, Hq, Hkv, hd, W, scale, [L], [L], [0], q, k, None if shared else v)
    bo, bl = brute_attend(is_g, Hq, Hkv, hd, W, scale, L, list(range(L)), as_floats(q), as_floats(k),
                          as_floats(v))
    assert np.max(np.abs(out - np.array(bo, dtype=float))) < 1e-12
    assert np.max(np.abs(lse - np.array(bl, dtype=float))) < 1e-12


def test_p1_brute_force_ragged_decode_batch():
    """Several rows of different lengths in one call, decode queries, 2 KV heads, g = 3."""
    Hq, Hkv, hd, W = 6, 2, 4, 5
    lens = [1, 4, 6, 11]
    qs, ks, vs, refs = [], [], [], []
    for i, L in enumerate(lens):
        q, k, v = _tiny_case((77, i), L, Hq, Hkv, hd)
        qs.append(q[-1:])
        ks.append(k)
        vs.append(v)
        refs.append(brute_attend(False, Hq, Hkv, hd, W, 0.5, L, [L - 1], as_floats(q[-1:]),
                                 as_floats(k), as_floats(v)))
    out, lse = oracle.attend(False, Hq, Hkv, hd, W, 0.5, [1] * 4, lens, [0] * 4,
                             np.concatenate(qs), np.concatenate(ks), np.concatenate(vs))
    for i in range(4):
        assert np.max(np.abs(out[i] - np.array(refs[i][0][0], float))) < 1e-12
        assert np.max(np.abs(lse[i] - np.array(refs[i][1][0], float))) < 1e-12


# ---------------------------------------------------------------- P2: closed forms
def test_p2_zero_keys_give_uniform_weights():
    """K = 0: every visible key weighs 1/n, so LSE = ln n and O = mean of visible V rows."""
    Hq, Hkv, hd, W, L = 4, 2, 8, 5, 13
    q, _, v = _tiny_case((11,), L, Hq, Hkv, hd)
    k = np.zeros((L, Hkv, hd), np.uint16)
    out, lse = oracle.attend(False, Hq, Hkv, hd, W, 0.9, [L], [L], [0], q, k, v)
    vf = workloads.bf16_bits_to_f32(v).astype(float)
    for p in range(L):
        lo = max(0, p - W + 1)
        n = p - lo + 1
        assert np.allclose(lse[p], math.log(n), atol=1e-15, rtol=0)
        for h in range(Hq):
            assert np.max(np.abs(out[p, h] - vf[lo:p + 1, h // 2].mean(axis=0))) < 1e-14


def test_p2_scale_zero_is_uniform():
    Hq, Hkv, hd, L = 2, 1, 4, 9
    q, k, v = _tiny_case((12,), L, Hq, Hkv, hd)
    out, lse = oracle.attend(True, Hq, Hkv, hd, 0, 0.0, [1], [L], [0], q[-1:], k, v)
    assert np.allclose(lse[0], math.log(L), atol=1e-15, rtol=0)
    vf = workloads.bf16_bits_to_f32(v).astype(float)
    assert np.max(np.abs(out[0, 0] - vf[:, 0].mean(axis=0))) < 1e-14


def test_p2_single_key():
    """One key: O = V_0 and LSE = scale * q . k exactly (no other term)."""
    Hq, Hkv, hd = 2, 1, 16
    q, k, v = _tiny_case((13,), 1, Hq, Hkv, hd)
    out, lse = oracle.attend(True, Hq, Hkv, hd, 0, 0.25, [1], [1], [0], q, k, v)
    qf = workloads.bf16_bits_to_f32(q).astype(float)
    kf = workloads.bf16_bits_to_f32(k).astype(float)
    vf = workloads.bf16_bits_to_f32(v).astype(float)
    for h in range(Hq):
        assert np.array_equal(out[0, h], vf[0, 0])
        assert abs(lse[0, h] - 0.25 * float(np.dot(qf[0, h], kf[0, 0]))) < 1e-13


def test_p2_window_one_reads_only_current_token():
    Hq, Hkv, hd, L = 4, 4, 8, 7
    q, k, v = _tiny_case((14,), L, Hq, Hkv, hd)
    out, _ = oracle.attend(False, Hq, Hkv, hd, 1, 0.3, [L], [L], [0], q, k, v)
    vf = workloads.bf16_bits_to_f32(v).astype(float)
    for p in range(L):
        for h in range(Hq):
            assert np.array_equal(out[p, h], vf[p, h])


def test_p2_equal_value_rows():
    Hq, Hkv, hd, L = 2, 1, 8, 20
    q, k, v = _tiny_case((15,), L, Hq, Hkv, hd)
    v[:] = v[3]
    out, _ = oracle.attend(True, Hq, Hkv, hd, 0, 1.0, [1], [L], [0], q[-1:], k, v)
    vf = workloads.bf16_bits_to_f32(v[3, 0]).astype(float)
    assert np.max(np.abs(out[0] - vf)) < 1e-14


def test_p2_wide_window_equals_global():
    """W >= L: the local family reads every key, exactly like the global family."""
    Hq, Hkv, hd, L = 4, 2, 8, 30
    q, k, v = _tiny_case((16,), L, Hq, Hkv, hd)
    og, lg = oracle.attend(True, Hq, Hkv, hd, 0, 0.2, [L], [L], [0], q, k, v)
    for W in (L, L + 1, 10 * L):
        ol, ll = oracle.attend(False, Hq, Hkv, hd, W, 0.2, [L], [L], [0], q, k, v)
        assert np.array_equal(og, ol) and np.array_equal(lg, ll)


def test_p2_block_gqa_mapping():
    """Query heads 0..g-1 read KV head 0, g..2g-1 read KV head 1 (block, not interleaved)."""
    Hq, Hkv, hd, L = 6, 2, 4, 9
    q, k, v = _tiny_case((17,), L, Hq, Hkv, hd)
    k[:, 1, :] = 0  # KV head 1: uniform weights
    _, lse = oracle.attend(True, Hq, Hkv, hd, 0, 1.0, [1], [L], [0], q[-1:], k, v)
    for h in range(Hq):
        uniform = abs(lse[0, h] - math.log(L)) < 1e-15
        assert uniform == (h >= 3)


# ---------------------------------------------------------------- P3: window boundaries (G1)
def _uniform_probe(L, W, positions_q, j_probe):
    """K = 0 and V = indicator of key j_probe: out[.,.,0] = 1/n if j_probe visible else 0."""
    Hq, Hkv, hd = 2, 1, 2
    C = len(positions_q)
    k = np.zeros((L, Hkv, hd), np.uint16)
    v = np.zeros((L, Hkv, hd), np.uint16)
    if j_probe is not None:
        v[j_probe, 0, 0] = workloads.f32_to_bf16_bits(np.float32([1.0]))[0]
    q = _draw((18, L), (C, Hq, hd))
    out, lse = oracle.attend(False, Hq, Hkv, hd, W, 1.0, [C], [L], [0], q, k, v)
    return out, lse


@pytest.mark.parametrize("L,n,first", [(1023, 1023, 0), (1024, 1024, 0), (1025, 1024, 1)])
def test_p3_window_edge_decode(L, n, first):
    """Decode at L = 1023, 1024, 1025 with W = 1024: n visible and the first visible key."""
    _, lse = _uniform_probe(L, 1024, [L - 1], None)
    assert round(math.exp(lse[0, 0])) == n and abs(lse[0, 0] - math.log(n)) < 1e-12
    if first > 0:
        out, _ = _uniform_probe(L, 1024, [L - 1], first - 1)
        assert out[0, 0, 0] == 0.0
    out, _ = _uniform_probe(L, 1024, [L - 1], first)
    assert abs(out[0, 0, 0] - 1.0 / n) < 1e-15


@pytest.mark.parametrize("L", [2048, 2049, 3073, 4097])
def test_p3_multi_window_continuation_decode(L):
    _, lse = _uniform_probe(L, 1024, [L - 1], None)
    assert abs(lse[0, 0] - math.log(1024)) < 1e-12
    out, _ = _uniform_probe(L, 1024, [L - 1], L - 1024)
    assert abs(out[0, 0, 0] - 1.0 / 1024) < 1e-15
    out, _ = _uniform_probe(L, 1024, [L - 1], L - 1025)
    assert out[0, 0, 0] == 0.0


def test_p3_multi_window_prefill_chunk():
    """Prior 0, chunk of 3*1024+5 queries: query p sees exactly its last min(p+1, 1024) keys."""
    C = 3 * 1024 + 5
    _, lse = _uniform_probe(C, 1024, list(range(C)), None)
    n = np.minimum(np.arange(C) + 1, 1024)
    assert np.max(np.abs(lse[:, 0] - np.log(n))) < 1e-12


# ---------------------------------------------------------------- P4: alternation (G2)
def test_p4_layer_schedule_ends_on_global():
    fam = [oracle.layer_is_global(l, 60) for l in range(60)]
    assert sum(fam) == 10 and fam.count(0) == 50
    assert fam[59] == 1
    assert fam[:6] == [0, 0, 0, 0, 0, 1]
    assert oracle.layer_is_global(0, 61) == -1 and oracle.layer_is_global(60, 60) == -1


# ---------------------------------------------------------------- P5: batch invariance (G3, G4)
def test_p5_rows_are_independent_and_reorderable():
    Hq, Hkv, hd, W = 4, 2, 8, 6
    lens = [3, 9, 1, 14, 7]
    cases = [_tiny_case((19, i), L, Hq, Hkv, hd) for i, L in enumerate(lens)]
    q = np.concatenate([c[0][-1:] for c in cases])
    k = np.concatenate([c[1] for c in cases])
    v = np.concatenate([c[2] for c in cases])
    ob, lb = oracle.attend(False, Hq, Hkv, hd, W, 0.4, [1] * 5, lens, None, q, k, v)
    for i, (cq, ck, cv) in enumerate(cases):
        o1, l1 = oracle.attend(False, Hq, Hkv, hd, W, 0.4, [1], [lens[i]], None, cq[-1:], ck, cv)
        assert np.array_equal(o1[0], ob[i]) and np.array_equal(l1[0], lb[i])
    perm = [3, 0, 4, 2, 1]
    o2, l2 = oracle.attend(False, Hq, Hkv, hd, W, 0.4, [1] * 5, [lens[i] for i in perm], None,
                           np.concatenate([cases[i][0][-1:] for i in perm]),
                           np.concatenate([cases[i][1] for i in perm]),
                           np.concatenate([cases[i][2] for i in perm]))
    assert np.array_equal(o2, ob[perm]) and np.array_equal(l2, lb[perm])


# ---------------------------------------------------------------- P6: stored range
def test_p6_partial_storage_matches_full_storage():
    """A local row stored only from its first visible key equals the same row stored whole."""
    Hq, Hkv, hd, W, L = 4, 2, 8, 16, 50
    q, k, v = _tiny_case((20,), L, Hq, Hkv, hd)
    of, lf = oracle.attend(False, Hq, Hkv, hd, W, 0.3, [1], [L], [0], q[-1:], k, v)
    s = L - W
    op, lp = oracle.attend(False, Hq, Hkv, hd, W, 0.3, [1], [L], [s], q[-1:], k[s:], v[s:])
    assert np.array_equal(of, op) and np.array_equal(lf, lp)
    with pytest.raises(oracle.OracleError):
        oracle.attend(False, Hq, Hkv, hd, W, 0.3, [1], [L], [s + 1], q[-1:], k[s + 1:], v[s + 1:])


# ---------------------------------------------------------------- P7: split equals unsplit
@pytest.mark.parametrize("fam,W", [("global", 0), ("local", 37)])
@pytest.mark.parametrize("S", [1, 3, 16, 64, 1000])
def test_p7_split_merge_equals_unsplit(fam, W, S):
    Hq, Hkv, hd = 4, 2, 8
    lens = [1, 2, 15, 16, 17, 100, 129]
    cases = [_tiny_case((21, i), L, Hq, Hkv, hd) for i, L in enumerate(lens)]
    q = np.concatenate([c[0][-1:] for c in cases])
    k = np.concatenate([c[1] for c in cases])
    v = np.concatenate([c[2] for c in cases])
    is_g = fam == "global"
    o, l = oracle.attend(is_g, Hq, Hkv, hd, W, 0.35, [1] * len(lens), lens, None, q, k, v)
    os_, ls = oracle.decode_split(is_g, Hq, Hkv, hd, W, 0.35, lens, None, q, k, v, S)
    assert np.max(np.abs(o - os_)) < 1e-12 and np.max(np.abs(l - ls)) < 1e-12


def test_p7_standalone_merge_of_disjoint_pieces():
    """Pieces attended separately (each normalised, with its own LSE) merge to the whole row, and
    empty pieces (lse = -inf) are ignored, whatever their o holds."""
    Hq, Hkv, hd, L = 2, 1, 8, 40
    q, k, v = _tiny_case((24,), L, Hq, Hkv, hd)
    whole_o, whole_l = oracle.attend(True, Hq, Hkv, hd, 0, 0.5, [1], [L], None, q[-1:], k, v)
    cuts = [0, 7, 8, 23, 40]
    lps, ops = [], []
    for a, e in zip(cuts[:-1], cuts[1:]):
        # attend keys [a, e) from the final query: a local window ending at e - 1 starting at a
        qq = q[-1:]
        o, l = oracle.attend(False, Hq, Hkv, hd, e - a, 0.5, [1], [e], [a], qq, k[a:e], v[a:e])
        lps.append(l[0])
        ops.append(o[0])
    lps.append(np.full(Hq, -np.inf))
    ops.append(np.full((Hq, hd), np.nan))
    lp = np.stack(lps, axis=1)            # [Hq][n]
    op = np.stack(ops, axis=1)            # [Hq][n][hd]
    mo, ml = oracle.merge(lp, np.nan_to_num(op, nan=1e300))
    assert np.max(np.abs(mo - whole_o[0])) < 1e-12 and np.max(np.abs(ml - whole_l[0])) < 1e-12
    eo, el = oracle.merge(np.full((1, 3), -np.inf), np.zeros((1, 3, 4)))
    assert el[0] == -np.inf and np.all(eo == 0)


# ---------------------------------------------------------------- P8: chunk parity (G5)
@pytest.mark.parametrize("fam,W", [("global", 0), ("local", 64)])
def test_p8_chunks_equal_token_by_token(fam, W):
    """A prompt walked in 64-token chunks gives the same numbers as walking it token by token."""
    Hq, Hkv, hd, N = 4, 2, 8, 300
    q, k, v = _tiny_case((22,), N, Hq, Hkv, hd)
    is_g = fam == "global"
    whole_o, whole_l = oracle.attend(is_g, Hq, Hkv, hd, W, 0.3, [N], [N], None, q, k, v)
    ch_o, ch_l = [], []
    for s in range(0, N, 64):
        e = min(N, s + 64)
        o, l = oracle.attend(is_g, Hq, Hkv, hd, W, 0.3, [e - s], [e], None, q[s:e], k[:e], v[:e])
        ch_o.append(o)
        ch_l.append(l)
    tk_o, tk_l = [], []
    for t in range(N):
        o, l = oracle.attend(is_g, Hq, Hkv, hd, W, 0.3, [1], [t + 1], None, q[t:t + 1], k[:t + 1], v[:t + 1])
        tk_o.append(o)
        tk_l.append(l)
    assert np.array_equal(np.concatenate(ch_o), whole_o) and np.array_equal(np.concatenate(ch_l), whole_l)
    assert np.array_equal(np.concatenate(tk_o), whole_o) and np.array_equal(np.concatenate(tk_l), whole_l)


# ---------------------------------------------------------------- P11: bytes per token (worked number)
def test_p11_bytes_per_token_matches_card():
    from global_paged_gqa_amd import traffic
    g = read_golden("kv_bytes_per_token.txt")
    head = {k: v for row in g for k, v in row.items() if k not in ("ctx", "gb")}
    n = int(head["layers"])
    per_tok = traffic.kv_bytes_per_token([(int(head["kv_heads"]), int(head["head_dim"]), False)] * n,
                                         int(head["bytes_per_elem"]))
    assert per_tok == int(head["bytes_per_token"])
    for row in g:
        if "ctx" in row:
            assert round(per_tok * int(row["ctx"]) / 1e9, 2 if float(row["gb"]) < 10 else 1) == float(row["gb"])
    # the hybrid 31B cache under the same formula: 50 local (16 x 256) + 10 global (4 x 512) layers
    hybrid = [(16, 256, False)] * 50 + [(4, 512, False)] * 10
    assert traffic.kv_bytes_per_token(hybrid) == 50 * 16 * 256 * 4 + 10 * 4 * 512 * 4 == 901120
    hybrid_shared = [(16, 256, False)] * 50 + [(4, 512, True)] * 10
    assert traffic.kv_bytes_per_token(hybrid_shared) == 860160


# ---------------------------------------------------------------- the pins have power
def test_brute_force_distinguishes_interleaved_mapping():
    """An interleaved head mapping (kv = h mod Hkv) would disagree with the oracle by far more than
    the 1e-12 bar, so the brute-force pin above does pin the block mapping."""
    Hq, Hkv, hd, L = 4, 2, 4, 6
    q, k, v = _tiny_case((23,), L, Hq, Hkv, hd)
    out, _ = oracle.attend(True, Hq, Hkv, hd, 0, 0.5, [L], [L], [0], q, k, v)
    bo, _ = brute_attend(True, Hq, Hkv, hd, 0, 0.5, L, list(range(L)), as_floats(q), as_floats(k),
                         as_floats(v), kv_of=lambda h, Hq, Hkv: h % Hkv)
    assert np.max(np.abs(out - np.array(bo, float))) > 1e-3


# ------------------------------------------------------------------------ KV append
def _append_case(spec, ctx_lens, n_new, key):
    """A batch whose pool holds every token, the pool with the last n_new tokens of each row
    cleared, and those tokens' K/V rows gathered from the contiguous side."""
    b = workloads.make_batch(spec, ctx_lens, np.ones(len(ctx_lens), np.int32), key, back="all")
    n_new = np.asarray(n_new, np.int32)
    cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
    k_new, v_new = [], []
    for r in range(b.B):
        kk, vv = b.row_keys(r)
        n = int(n_new[r])
        k_new.append(kk[len(kk) - n:])
        v_new.append(vv[len(vv) - n:])
    k_new = np.concatenate(k_new)
    v_new = None if spec.kv_shared else np.concatenate(v_new)
    return b, cu, k_new, v_new


@pytest.mark.parametrize("spec", [workloads.GLOBAL_31B, workloads.LOCAL_31B, workloads.GLOBAL_31B_KV_SHARED],
                         ids=["global", "local", "kv-shared"])
def test_kv_append_rebuilds_the_scattered_pool(spec):
    """Appending each row's last n tokens into a pool where their slots were zeroed gives back the
    pool that workloads' own scatter built (n crossing page edges, 0-token rows included), and no
    other byte changes; every written slot is where the library's checked helper places it."""
    L = [1, 17, 40, 300, 513, 1024]
    n_new = [1, 2, 0, 45, 16, 300]
    b, cu, k_new, v_new = _append_case(spec, L, n_new, (40, spec.num_kv_heads, int(spec.kv_shared)))
    P = spec.page_size
    kp0, vp0 = b.k_pool.copy(), None if b.v_pool is None else b.v_pool.copy()
    # clear the appended tokens' slots by walking the table directly (independent of the oracle)
    for r in range(b.B):
        for t in range(L[r] - n_new[r], L[r]):
            kp0[b.page_table[r, t // P], :, t % P, :] = 0
            if vp0 is not None:
                vp0[b.page_table[r, t // P], :, t % P, :] = 0
    kp, vp, skipped = oracle.kv_append(spec.num_kv_heads, spec.head_dim, P, cu, L, b.page_table, b.num_pages,
                                       k_new, v_new, kp0, vp0)
    assert skipped == 0
    assert np.array_equal(kp, b.k_pool)
    if vp is not None:
        assert np.array_equal(vp, b.v_pool)
    import global_paged_gqa_amd as g
    lay = g.make_layer(spec.family, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.window,
                       spec.kv_shared)
    flat = kp.reshape(-1)
    for r, t, kvh in ((3, L[3] - 45, 0), (3, L[3] - 1, spec.num_kv_heads - 1), (5, 724, 1), (1, 16, 0)):
        off = g.gattn_kv_offset(lay, b.page_table, b.B, b.pt_stride, r, t, kvh, b.num_pages)
        i = int(cu[r]) + t - (L[r] - n_new[r])
        assert np.array_equal(flat[off:off + spec.head_dim], k_new[i, kvh]), (r, t)


def test_kv_append_fails_closed():
    """A token whose page id is out of range or -1, or whose position is beyond the table, is
    skipped and counted; a row with fewer cached tokens than new ones writes none of them; the
    rest are written."""
    Hkv, hd, P = 2, 8, 16
    pt = np.array([[2, -1, 9], [0, 1, 2]], np.int32)       # row 0: page 1 unbacked, page 2 = id 9 >= 4
    kp = np.zeros((4, Hkv, P, hd), np.uint16)
    L = np.array([40, 3], np.int32)
    n_new = np.array([30, 5], np.int32)                    # row 0: tokens 10..39; row 1: 5 > L
    cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
    k_new = (np.arange(int(cu[-1]) * Hkv * hd, dtype=np.int64) % 60000 + 1).astype(np.uint16).reshape(-1, Hkv, hd)
    kp2, _, skipped = oracle.kv_append(Hkv, hd, P, cu, L, pt, 4, k_new, None, kp, None)
    # row 0: tokens 10..15 in page 2 (written); 16..31 page -1 (skipped); 32..39 page 9 (skipped)
    # row 1: 5 new tokens but 3 cached: none written
    assert skipped == 16 + 8 + 5
    assert np.array_equal(kp2[2, :, 10:16], np.transpose(k_new[0:6], (1, 0, 2)))
    untouched = np.ones(kp.shape, bool)
    untouched[2, :, 10:16] = False
    assert np.all(kp2[untouched] == 0)
    # a declared bound max_new below row 0's 30 new tokens: that row writes nothing either
    kp3, _, skipped3 = oracle.kv_append(Hkv, hd, P, cu, L, pt, 4, k_new, None, kp, None, max_new=29)
    assert skipped3 == 30 + 5 and np.all(kp3 == 0)
    kp4, _, skipped4 = oracle.kv_append(Hkv, hd, P, cu, L, pt, 4, k_new, None, kp, None, max_new=30)
    assert skipped4 == skipped and np.array_equal(kp4, kp2)

