"""Brute-force attention at 50 decimal digits (mpmath), for tiny inputs only.

Written independently of the oracle: the visible set is built by enumerating
keys and testing the two conditions the pages name (causal: key not after the
query; sliding window: fewer than W positions back), the KV head is found by
scaling the query head index, and the softmax is exp / sum with no max shift.
"""
import mpmath as mp

import workloads


def block_kv(h, Hq, Hkv):
    """KV head read by query head h: consecutive query heads share one KV head."""
    return (h * Hkv) // Hq


def brute_attend(is_global, Hq, Hkv, hd, W, scale, L, positions, q, k, v, kv_of=block_kv):
    """q: [len(positions)][Hq][hd] floats; k, v: [L][Hkv][hd] floats (all tokens 0..L-1).

    Returns (out [n][Hq][hd], lse [n][Hq]) as mpf."""
    mp.mp.dps = 50
    outs, lses = [], []
    for qi, p in enumerate(positions):
        o_row, l_row = [], []
        for h in range(Hq):
            kv = kv_of(h, Hq, Hkv)
            visible = {j for j in range(L) if j <= p and (is_global or p - j < W)}
            e = {}
            for j in sorted(visible):
                dot = mp.fsum(mp.mpf(q[qi][h][d]) * mp.mpf(k[j][kv][d]) for d in range(hd))
                e[j] = mp.exp(mp.mpf(scale) * dot)
            Z = mp.fsum(e.values())
            l_row.append(mp.log(Z))
            o_row.append([mp.fsum(e[j] * mp.mpf(v[j][kv][d]) for j in e) / Z for d in range(hd)])
        outs.append(o_row)
        lses.append(l_row)
    return outs, lses


def as_floats(bits):
    return workloads.bf16_bits_to_f32(bits).astype(float).tolist()
