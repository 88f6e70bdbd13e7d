"""Pins of the oracle's FP8 KV pieces against what the format and the mathematics fix.

E4M3 (OCP 8-bit floating point, the variant without infinities) has a closed definition: sign,
4 exponent bits with bias 7, 3 mantissa bits, subnormals at exponent field 0, S.1111.111 = NaN.
The decode table is checked value by value against that definition's landmarks and against
torch's float8_e4m3fn (a library routine); the encoder against the round trip, the midpoints
(ties to the even code), saturation and torch's rounding inside the finite range. Attention over
an FP8 pool is checked against mpmath brute force on tiny inputs and against the bf16 oracle on
values both can hold exactly; the FP8 append against the bf16 append composed with the encoder.
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from brute import brute_attend


def _codes():
    return np.arange(256, dtype=np.uint8)


def test_e4m3_landmark_values():
    v = oracle.e4m3_value(_codes())
    expect = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
              0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x77: 240.0, 0x78: 256.0, 0x7E: 448.0,
              0x80: -0.0, 0x81: -(2.0 ** -9), 0xB8: -1.0, 0xFE: -448.0}
    for c, x in expect.items():
        assert v[c] == x and math.copysign(1, v[c]) == math.copysign(1, x), hex(c)
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert int(np.isnan(v).sum()) == 2
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                      # finite magnitudes increase with the code
    assert np.array_equal(v[0x80:0xFF], -v[:0x7F])       # the sign bit only negates
    # each binade holds 8 evenly spaced values; subnormals continue the first binade's spacing
    assert np.allclose(np.diff(pos[:16]), 2.0 ** -9)


def test_e4m3_table_matches_torch():
    import torch
    t = torch.from_numpy(_codes()).view(torch.float8_e4m3fn).double().numpy()
    v = oracle.e4m3_value(_codes())
    both = ~np.isnan(v)
    assert np.array_equal(np.isnan(t), ~both)
    assert np.array_equal(v[both], t[both])


def test_e4m3_encode_round_trip_and_ties():
    codes = _codes()
    v = oracle.e4m3_value(codes)
    finite = ~np.isnan(v)
    assert np.array_equal(oracle.e4m3_encode(v[finite].astype(np.float32)), codes[finite])
    # midpoints of neighbouring codes (exact in fp32) go to the even code; a hair off goes to the nearer
    lo, hi = np.arange(0, 0x7E), np.arange(1, 0x7F)
    mid = ((v[lo] + v[hi]) / 2).astype(np.float32)
    assert np.all(mid.astype(np.float64) == (v[lo] + v[hi]) / 2)
    even = np.where(lo % 2 == 0, lo, hi)
    assert np.array_equal(oracle.e4m3_encode(mid), even)
    assert np.array_equal(oracle.e4m3_encode(-mid), even | 0x80)
    assert np.array_equal(oracle.e4m3_encode(np.nextafter(mid, np.float32(-1))), lo)
    assert np.array_equal(oracle.e4m3_encode(np.nextafter(mid, np.float32(1e9))), hi)


def test_e4m3_encode_saturates_and_keeps_nan_and_sign():
    f = np.float32
    enc = oracle.e4m3_encode(np.array([448.0, 449.0, 464.0, 480.0, 1e30, np.inf, -500.0, -np.inf, np.nan, -np.nan,
                                       -0.0, 0.0, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -10 * 1.0001, 1e-30],
                                      dtype=f))
    assert list(enc) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0xFF, 0x80, 0x00, 0x00, 0x80, 0x01,
                         0x00]


def test_e4m3_encode_matches_torch_in_range():
    import torch
    g = np.random.default_rng(3)
    x = np.concatenate([g.standard_normal(200000) * s for s in (0.003, 0.1, 1.0, 30.0)]).astype(np.float32)
    x = x[np.abs(x) < 448]
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x), t)


def _fp8_case(L, Hkv, hd, key):
    g = np.random.default_rng(key)
    k8 = g.integers(0, 256, size=(L, Hkv, hd), dtype=np.uint8)
    v8 = g.integers(0, 256, size=(L, Hkv, hd), dtype=np.uint8)
    for a in (k8, v8):   # keep the codes finite and moderate (|value| <= 15)
        a[:] = np.where((a & 0x7F) > 0x57, a & 0xD7, a)
    return k8, v8


@pytest.mark.parametrize("fam,W", [("local", 3), ("global", 0)])
def test_attend_fp8kv_brute_force(fam, W):
    """A tiny ragged prefill over random E4M3 codes, with two different non-dyadic scales, against
    the 50-digit brute force on the dequantized values."""
    Hq, Hkv, hd, L = 4, 2, 3, 7
    k8, v8 = _fp8_case(L, Hkv, hd, 5)
    ks, vs = 0.0371, 0.53
    q = workloads.normal_bf16(workloads.generator(99, 1), (L, Hq, hd))
    out, lse = oracle.attend_fp8kv(fam == "global", Hq, Hkv, hd, W, 0.41, [L], [L], [0], q, k8, v8, ks, vs)
    kf = (oracle.e4m3_value(k8) * ks).tolist()
    vf = (oracle.e4m3_value(v8) * vs).tolist()
    bo, bl = brute_attend(fam == "global", Hq, Hkv, hd, W, 0.41, L, list(range(L)),
                          workloads.bf16_bits_to_f32(q).astype(float).tolist(), kf, vf)
    assert np.max(np.abs(out - np.array(bo, dtype=float))) < 1e-12
    assert np.max(np.abs(lse - np.array(bl, dtype=float))) < 1e-12


def test_attend_fp8kv_equals_bf16_attend_on_shared_values():
    """With power-of-two scales every dequantized value is a bf16 value, and the FP8 oracle must
    give the bf16 oracle's result on those values bit for bit; non-dyadic scales move the scores
    and the output exactly as the scales say."""
    spec = workloads.LOCAL_31B
    b = workloads.make_batch(spec, [40, 300, 1100], [1, 1, 3], (61, 1), back="visible")
    k8, v8 = workloads.e4m3_codes(b.k, 1.0), workloads.e4m3_codes(b.v, 1.0)
    ks, vs = 2.0 ** -3, 2.0 ** 2
    kb = workloads.f32_to_bf16_bits((oracle.e4m3_value(k8) * ks).astype(np.float32))
    vb = workloads.f32_to_bf16_bits((oracle.e4m3_value(v8) * vs).astype(np.float32))
    args = (False, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.window, spec.softmax_scale, b.q_lens,
            b.ctx_lens, b.k_starts, b.q)
    o8, l8 = oracle.attend_fp8kv(*args, k8, v8, ks, vs)
    ob, lb = oracle.attend(*args, kb, vb)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)
    # k_scale multiplies every score, v_scale the output
    ks2, vs2 = 0.0371, 0.0213
    o2, l2 = oracle.attend_fp8kv(*args, k8, v8, ks2, vs2)
    o1, l1 = oracle.attend_fp8kv(False, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.window,
                                 spec.softmax_scale * ks2, b.q_lens, b.ctx_lens, b.k_starts, b.q, k8, v8, 1.0, 1.0)
    assert np.max(np.abs(l2 - l1)) < 1e-12
    assert np.max(np.abs(o2 - o1 * vs2)) < 1e-12


def test_kv_append_fp8_is_the_bf16_append_then_the_encoder():
    """Each written slot holds the E4M3 code of the fp32 quotient value / scale, every other byte
    keeps its value, and the same tokens are skipped as by the bf16 append."""
    spec = workloads.LOCAL_31B
    Hkv, hd, P = spec.num_kv_heads, spec.head_dim, spec.page_size
    L = np.array([1, 17, 40, 300, 513], np.int32)
    n_new = np.array([1, 2, 0, 45, 300], np.int32)
    b = workloads.make_batch(spec, L, np.ones(5, np.int32), (62, 1), back="all", extra_pages=2)
    pt = b.page_table.copy()
    pt[4, (L[4] - 1) // P] = b.num_pages + 3     # one page out of range: its tokens are skipped
    cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
    T = int(cu[-1])
    k_new = workloads.normal_bf16(workloads.generator(62, 2), (T, Hkv, hd))
    v_new = workloads.normal_bf16(workloads.generator(62, 3), (T, Hkv, hd))
    ks, vs = 0.0371, 0.0213
    g = np.random.default_rng(8)
    k8 = g.integers(0, 256, size=b.k_pool.shape, dtype=np.uint8)
    v8 = g.integers(0, 256, size=b.k_pool.shape, dtype=np.uint8)
    kp8, vp8, skipped8 = oracle.kv_append_fp8(Hkv, hd, P, cu, L, pt, b.num_pages, k_new, v_new, ks, vs, k8, v8)
    # the bf16 append on a marker pool tells which slots are written and with what
    mark = np.zeros(b.k_pool.shape, np.uint16)
    kpb, vpb, skipped = oracle.kv_append(Hkv, hd, P, cu, L, pt, b.num_pages, k_new, v_new, mark, mark)
    ones = np.ones((T, Hkv, hd), np.uint16)
    w, _, _ = oracle.kv_append(Hkv, hd, P, cu, L, pt, b.num_pages, ones, None, mark, None)
    written = w == 1
    assert skipped8 == skipped > 0
    qk = workloads.bf16_bits_to_f32(kpb) / np.float32(ks)
    qv = workloads.bf16_bits_to_f32(vpb) / np.float32(vs)
    assert np.array_equal(kp8, np.where(written, oracle.e4m3_encode(qk), k8))
    assert np.array_equal(vp8, np.where(written, oracle.e4m3_encode(qv), v8))


def test_kv_append_fp8_special_values():
    """NaN keeps its sign, infinities saturate to +-448, -0 stays -0, whatever the scale."""
    Hkv, hd, P = 1, 8, 16
    vals = np.array([0x7FC0, 0xFFC0, 0x7F81, 0x7F80, 0xFF80, 0x8000, 0x0000, 0x3F80], np.uint16)  # bf16 bits
    k_new = vals.reshape(1, Hkv, hd)
    pool = np.zeros((1, Hkv, P, hd), np.uint8)
    for ks in (1.0, 0.0371, 1e-30):
        kp, _, skipped = oracle.kv_append_fp8(Hkv, hd, P, [0, 1], [1], np.zeros((1, 1), np.int32), 1, k_new, None,
                                              ks, 1.0, pool, None)
        one = oracle.e4m3_encode(np.array([1.0 / np.float32(ks)], np.float32))[0]
        assert skipped == 0
        assert list(kp[0, 0, 0]) == [0x7F, 0xFF, 0x7F, 0x7E, 0xFE, 0x80, 0x00, one], ks
