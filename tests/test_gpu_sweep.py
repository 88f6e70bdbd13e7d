"""The 60-layer decode sweep and the 65536-token global decode, at full size, on the GPU.

Sweep: layers 0..59, 16 rows at 32768 tokens each. The family of each layer comes from the
library's schedule (gattn_layer_family), checked against the oracle's own schedule: five local
layers then one global, ten times, the last layer global. Local layers are head_dim 256 with 16
KV heads, a 1024-token window and 512-token splits, and back only their window pages; global
layers are head_dim 512 with 4 KV heads, V reading the K cache, and 1024-token splits. All 60
layers' pools are resident together (about 34 GB), and the sweep is the same 60 back-to-back
gattn_decode calls on one stream that the benchmark times. Sampled rows of every layer (their
K/V drawn on the host) are compared with the fp64 oracle; every output of every layer must be
finite.

Long run: one 65536-token global row with K=V, every output compared with the oracle at the
sweep's split size, unsplit and at 512.

Tolerances: O max-abs 1e-2, LSE max-abs 1e-3.
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


def compare(lay, out, lse, tag):
    ref_o, ref_l = oracle.attend_batch(lay.host)
    eo = float(np.max(np.abs(out - ref_o)))
    el = float(np.max(np.abs(lse - ref_l)))
    print(f"{tag}: rows {lay.rows} max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O and el <= TOL_LSE, (tag, eo, el)


def sampled_rows(layer, family):
    g = workloads.generator(5, layer, 99)
    return tuple(sorted(g.choice(workloads.SWEEP_B, size=1 if family == "global" else 2, replace=False)))


def test_sweep_60_layers(devio):
    import torch
    nat = devio.nat
    n = workloads.SWEEP_LAYERS
    fams = [nat.gattn_layer_family(l, n) for l in range(n)]
    assert fams == [nat.GLOBAL if oracle.layer_is_global(l, n) else nat.LOCAL for l in range(n)]
    assert fams.count(nat.GLOBAL) == 10 and fams.count(nat.LOCAL) == 50 and fams[-1] == nat.GLOBAL

    layers = []
    for l in range(n):
        fam = "global" if fams[l] == nat.GLOBAL else "local"
        lay = workloads.sweep_layer(l, fam, sampled_rows(l, fam))
        layers.append((fam, devio.DeviceLayout(lay, workloads.fill_normal_bf16_device)))
        if l % 6 == 5:
            print(f"built layers 0..{l} ({torch.cuda.memory_allocated() / 2**30:.1f} GiB resident)", flush=True)
    ws_bytes = max(d.workspace_bytes(workloads.SWEEP_SPLIT[f]) for f, d in layers)
    ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device="cuda")
    calls = 0
    for fam, d in layers:
        d.workspace, d.ws_bytes = ws, ws_bytes
    # poison the shared workspace once: no layer may read another layer's partials
    ws.fill_(float("nan"))
    for fam, d in layers:
        d.decode(workloads.SWEEP_SPLIT[fam])
        calls += 1
    torch.cuda.synchronize()
    assert calls == n
    for l, (fam, d) in enumerate(layers):
        out, lse = d.result()
        assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse)), l
        compare(d.lay, out[list(d.lay.rows)], lse[list(d.lay.rows)], f"layer {l} {fam}")
        layers[l] = None
        del d


@pytest.fixture(scope="module")
def long_run(devio):
    lay = workloads.long_global_decode()
    return lay, devio.DeviceLayout(lay, workloads.fill_normal_bf16_device)


@pytest.mark.parametrize("split", [1024, 0, 512])
def test_long_global_kv_shared(devio, long_run, split):
    lay, d = long_run
    d.decode(split)
    out, lse = d.result()
    compare(lay, out, lse, f"65536 K=V S={split}")
