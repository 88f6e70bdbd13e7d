"""The seeded input generators: the bf16 recipe and the full-size paged layouts (CPU)."""
import numpy as np
import torch

import workloads


def test_bf16_rounding_matches_torch_rne():
    """f32_to_bf16_bits is round-to-nearest-even: torch's float32 -> bfloat16 cast is an
    independent implementation of the same rounding."""
    g = np.random.default_rng(7)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32) * 10.0 ** g.integers(-20, 20, 100000),
                        np.float32([0.0, -0.0, 1.0, -1.0, 3.0e38, 1.0e-40, np.inf, -np.inf])])
    # ties: float32 values exactly halfway between two bf16 values
    ties = (np.arange(1, 2001, dtype=np.uint32) << np.uint32(16)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32)])
    ours = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_normal_bf16_is_the_plain_recipe():
    """The chunked generator equals the recipe written out: float64 N(0,1) draws, float32 by
    RNE, bf16 by RNE (sizes around the chunk boundary included)."""
    for n in (1, 7, (1 << 22) - 1, (1 << 22) + 5):
        got = workloads.normal_bf16(workloads.generator(11, n % 5, 1), (n,))
        x = workloads.generator(11, n % 5, 1).standard_normal(n).astype(np.float32)
        ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, ref), n


def test_paged_layout_local_backs_window_pages_only():
    lay = workloads.paged_layout(workloads.LOCAL_31B, [32768, 1500, 20, 1024], (77, 0), rows=(1, 3))
    P, W = 16, 1024
    ids = lay.page_table[lay.page_table >= 0]
    assert len(np.unique(ids)) == len(ids) == lay.num_pages
    assert ids.min() == 0 and ids.max() == lay.num_pages - 1
    for r, L in enumerate(lay.ctx_lens):
        lo = max(0, int(L) - W)
        backed = np.nonzero(lay.page_table[r] >= 0)[0]
        assert backed[0] == lo // P and backed[-1] == (int(L) - 1) // P and len(backed) == backed[-1] - backed[0] + 1
        assert lay.k_starts[r] == (lo // P) * P
    # the oracle side of a sampled row: its stored range is exactly the visible keys
    assert np.array_equal(lay.host.k_starts, [max(0, 1500 - W), 0])
    assert lay.host.k.shape[0] == (1500 - 476) + 1024


def test_paged_layout_global_and_sampled_rows_round_trip():
    """Scatter the sampled rows' token-major draws into a pool by their page ids and read them
    back through the page table: the contiguous oracle side is what the pool holds."""
    spec = workloads.GLOBAL_31B
    lay = workloads.paged_layout(spec, [300, 33, 64], (78, 0), rows=(0, 2))
    P = spec.page_size
    pool = np.zeros((lay.num_pages, spec.num_kv_heads, P, spec.head_dim), np.uint16)
    for r in lay.rows:
        n = len(lay.row_pages[r])
        pool[lay.row_pages[r]] = lay.k_tok[r].reshape(n, P, spec.num_kv_heads, spec.head_dim).transpose(0, 2, 1, 3)
    off = 0
    for i, r in enumerate(lay.rows):
        L = int(lay.ctx_lens[r])
        t = np.arange(L)
        got = pool[lay.page_table[r, t // P], :, t % P, :]
        assert np.array_equal(got, lay.host.k[off:off + L])
        assert np.array_equal(lay.host.q[i], lay.q[r])
        off += L
    assert lay.host.v.shape == lay.host.k.shape


def test_sweep_layer_shapes():
    g = workloads.sweep_layer(5, "global")
    assert g.spec.kv_shared and g.spec.head_dim == 512 and g.spec.num_kv_heads == 4
    assert g.num_pages == 16 * 2048 and g.host is None and not g.k_tok
    l = workloads.sweep_layer(0, "local")
    assert l.num_pages == 16 * 64 and l.spec.window == 1024


def test_concat_batches_keeps_every_row_and_page():
    """The concatenated batch's pool gives back each row's contiguous K/V, its queries follow in
    order, and b's page ids point past a's pool."""
    pre, dec = workloads.cfg4_mixed("local", n_prefill=2, chunk=64, max_prior=300, n_decode=5, max_decode_len=900)
    mix = workloads.concat_batches(pre, dec)
    assert mix.B == pre.B + dec.B and mix.num_pages == pre.num_pages + dec.num_pages
    assert np.array_equal(mix.q, np.concatenate([pre.q, dec.q]))
    for r in range(mix.B):
        kk, vv = mix.row_keys(r)
        assert np.array_equal(workloads.gather_row_from_pool(mix, r, mix.k_pool), kk)
        assert np.array_equal(workloads.gather_row_from_pool(mix, r, mix.v_pool), vv)
    src = [(pre, r) for r in range(pre.B)] + [(dec, r) for r in range(dec.B)]
    for r, (b, rr) in enumerate(src):
        assert np.array_equal(mix.row_keys(r)[0], b.row_keys(rr)[0])
    assert np.all(mix.page_table[pre.B:][mix.page_table[pre.B:] >= 0] >= pre.num_pages)
