"""Seeded synthetic inputs for hybrid paged GQA attention (Gemma-4-31B shapes).

This module holds none of the attention arithmetic. It draws bf16 N(0,1) tensors,
ragged context lengths and page tables, and scatters contiguous per-row K/V into
the paged pool layout. Both sides of every parity check are fed from here: the
HIP library reads the paged pool, the oracle reads the contiguous copy.

Input recipe (stated once, used everywhere):
  * Seeds: numpy ``SeedSequence([20261202, config, layer, tensor])`` feeding PCG64.
    Tensor ids: 0 = Q, 1 = K, 2 = V, 3 = lengths, 4 = page permutation, 5 = priors.
  * Values: ``standard_normal`` in float64, rounded to float32 (RNE), then to
    bfloat16 (RNE on the float32 bits).
  * Pool layout: ``[num_pages][num_kv_heads][page_size][head_dim]`` bf16, so one
    (page, KV head) pair is a contiguous block. ``page_table[r][t // P]`` names
    the page holding token t of row r; ``-1`` marks pages that are not backed.
  * Page ids: every backed (row, logical page) pair gets a distinct physical page;
    the assignment is a seeded global shuffle across all rows.

Shapes follow the Gemma 4 31B description on the pegainfer issue pages (60 layers,
five local layers per global one, "twice the attention heads", a different global
KV head count) and the Core AI card's hybrid-pf64 section (32 query heads, 4 global
KV heads at head_dim 512); the local family is 16 KV heads at head_dim 256 with a
1024-token window.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

BASE_SEED = 20261202
PAGE_SIZE = 16

T_Q, T_K, T_V, T_LEN, T_PERM, T_PRIOR = range(6)

BF16_NAN = np.uint16(0x7FC0)


# --------------------------------------------------------------------------- rng / bf16
def generator(*key: int) -> np.random.Generator:
    """PCG64 stream for one (config, layer, tensor) key."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, *[int(k) for k in key]])))


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); returns uint16 bits."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(gen: np.random.Generator, shape) -> np.ndarray:
    """bf16 bits of N(0,1) draws: float64 -> float32 (RNE) -> bfloat16 (RNE).

    The draws go through fixed chunk buffers that are reused (fresh allocations per
    chunk are dominated by page faults); the values equal f32_to_bf16_bits applied to
    ``gen.standard_normal(n).astype(np.float32)``.
    """
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16)
    chunk = max(1, min(n, 1 << 22))
    f64 = np.empty(chunk, np.float64)
    f32 = np.empty(chunk, np.float32)
    u = f32.view(np.uint32)
    t = np.empty(chunk, np.uint32)
    for s in range(0, n, chunk):
        m = min(n, s + chunk) - s
        gen.standard_normal(out=f64[:m])
        f32[:m] = f64[:m]
        tm = t[:m]
        # round to nearest even on the float32 bits: add 0x7FFF + (bit 16), keep the high half
        np.right_shift(u[:m], np.uint32(16), out=tm)
        np.bitwise_and(tm, np.uint32(1), out=tm)
        np.add(tm, np.uint32(0x7FFF), out=tm)
        np.add(tm, u[:m], out=tm)
        np.right_shift(tm, np.uint32(16), out=tm)
        out[s:s + m] = tm
    return out.reshape(shape)


# --------------------------------------------------------------------------- layer shapes
@dataclass(frozen=True)
class LayerSpec:
    """One attention layer's geometry: family, head counts, window, page size, scale."""
    family: str                 # "local" (sliding window) or "global" (full causal)
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    window: int = 0             # keys visible to a query: the last `window` positions (local only)
    kv_shared: bool = False     # V reads the K cache
    scale: float = 0.0          # 0 -> 1/sqrt(head_dim)
    page_size: int = PAGE_SIZE

    @property
    def is_global(self) -> bool:
        return self.family == "global"

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale else 1.0 / math.sqrt(self.head_dim)


LOCAL_31B = LayerSpec("local", 32, 16, 256, window=1024)
GLOBAL_31B = LayerSpec("global", 32, 4, 512)
GLOBAL_31B_KV_SHARED = LayerSpec("global", 32, 4, 512, kv_shared=True)
# The 12B line: its global family keeps a single KV head (the Core AI card's 12B control, "1 global
# KV head"), here for 16 query heads (g = 16); its local family is read as 16 query heads over 8 KV
# heads. Both are readings: the pages give no full 12B head table.
LOCAL_12B = LayerSpec("local", 16, 8, 256, window=1024)
GLOBAL_12B = LayerSpec("global", 16, 1, 512)


# --------------------------------------------------------------------------- batches
@dataclass
class Batch:
    """A ragged batch of rows for one layer, in both contiguous and paged form."""
    spec: LayerSpec
    ctx_lens: np.ndarray        # int32 [B]: tokens present in the cache, including this step's
    q_lens: np.ndarray          # int32 [B]: queries per row (1 for decode)
    k_starts: np.ndarray        # int32 [B]: first token stored contiguously (and backed) per row
    q: np.ndarray               # uint16 [T][Hq][hd]
    k: np.ndarray               # uint16 [sum(L - k_start)][Hkv][hd] contiguous rows
    v: Optional[np.ndarray]     # same, or None when K=V
    page_table: np.ndarray      # int32 [B][pt_stride]
    k_pool: np.ndarray          # uint16 [num_pages][Hkv][P][hd]
    v_pool: Optional[np.ndarray]
    meta: dict = field(default_factory=dict)
    fp8: Optional["Fp8Kv"] = None  # an E4M3 copy of K/V (both sides), see with_fp8_kv

    @property
    def B(self) -> int:
        return int(self.ctx_lens.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def pt_stride(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def cu_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    def row_keys(self, r: int):
        """Contiguous K (and V) of row r, tokens [k_start, L)."""
        off = int(np.sum(self.ctx_lens[:r] - self.k_starts[:r]))
        n = int(self.ctx_lens[r] - self.k_starts[r])
        kk = self.k[off:off + n]
        vv = kk if self.v is None else self.v[off:off + n]
        return kk, vv

    def subset(self, rows) -> "Batch":
        """Contiguous-side view restricted to some rows (for sampled oracle checks)."""
        rows = list(rows)
        qs, ks, vs = [], [], []
        cq = self.cu_q
        for r in rows:
            qs.append(self.q[cq[r]:cq[r + 1]])
            kk, vv = self.row_keys(r)
            ks.append(kk)
            vs.append(vv)
        fp8 = None
        if self.fp8 is not None:
            offs = np.concatenate([[0], np.cumsum(self.ctx_lens - self.k_starts)])
            f = self.fp8
            fp8 = replace(f, k=np.concatenate([f.k[offs[r]:offs[r + 1]] for r in rows]),
                          v=np.concatenate([f.v[offs[r]:offs[r + 1]] for r in rows]))
        return Batch(self.spec, self.ctx_lens[rows].copy(), self.q_lens[rows].copy(),
                     self.k_starts[rows].copy(), np.concatenate(qs), np.concatenate(ks),
                     None if self.v is None else np.concatenate(vs),
                     self.page_table[rows].copy(), self.k_pool, self.v_pool, dict(self.meta), fp8)


@dataclass
class Fp8Kv:
    """An E4M3 (one byte per element) copy of a batch's K and V, on both sides: code c stands for
    value(c) * k_scale in K and value(c) * v_scale in V."""
    k: np.ndarray               # uint8, shaped like Batch.k
    v: np.ndarray               # uint8, shaped like Batch.v
    k_pool: np.ndarray          # uint8 [num_pages][Hkv][P][hd]
    v_pool: Optional[np.ndarray]  # None with K = V
    k_scale: float
    v_scale: float


# Scales of the FP8 copies: float32 values, not powers of two, different for K and V.
FP8_K_SCALE = float(np.float32(0.0371))
FP8_V_SCALE = float(np.float32(0.0213))


def e4m3_codes(bf16_bits: np.ndarray, scale: float) -> np.ndarray:
    """Input drawing only: E4M3 codes of bf16 values divided by ``scale`` (float32), by torch's
    float8_e4m3fn cast. NaN (poisoned slots) gives a NaN code."""
    import torch
    x = bf16_bits_to_f32(bf16_bits) / np.float32(scale)
    # torch's cast turns finite values beyond the format's range into NaN: the scale must avoid that
    assert not np.any(np.isfinite(x) & (np.abs(x) >= 464)), "scale too small for E4M3"
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def with_fp8_kv(b: Batch, k_scale: float = FP8_K_SCALE, v_scale: float = FP8_V_SCALE) -> Batch:
    """Attach an E4M3 copy of the batch's K/V (contiguous rows and pools, element by element, so
    the two sides hold the same codes). With K = V the V side is the K codes with the K scale and
    there is no V pool."""
    k8 = e4m3_codes(b.k, k_scale)
    kp8 = e4m3_codes(b.k_pool, k_scale)
    if b.v is None:
        b.fp8 = Fp8Kv(k8, k8, kp8, None, float(k_scale), float(k_scale))
    else:
        b.fp8 = Fp8Kv(k8, e4m3_codes(b.v, v_scale), kp8, e4m3_codes(b.v_pool, v_scale), float(k_scale),
                      float(v_scale))
    return b


def concat_batches(a: Batch, b: Batch) -> Batch:
    """One batch holding a's rows then b's (same layer): queries, contiguous K/V and pools
    concatenated, b's page ids shifted past a's pool. Data plumbing only (a mixed step's prefill
    and decode rows as one call)."""
    assert a.spec == b.spec and a.fp8 is None and b.fp8 is None
    stride = max(a.pt_stride, b.pt_stride)
    pt = np.full((a.B + b.B, stride), -1, dtype=np.int32)
    pt[:a.B, :a.pt_stride] = a.page_table
    pt[a.B:, :b.pt_stride] = np.where(b.page_table >= 0, b.page_table + a.num_pages, -1)
    cat = lambda x, y: None if x is None else np.concatenate([x, y])
    return Batch(a.spec, cat(a.ctx_lens, b.ctx_lens), cat(a.q_lens, b.q_lens), cat(a.k_starts, b.k_starts),
                 cat(a.q, b.q), cat(a.k, b.k), cat(a.v, b.v), pt, cat(a.k_pool, b.k_pool), cat(a.v_pool, b.v_pool),
                 {"concat": (a.meta, b.meta)})


def first_needed_token(spec: LayerSpec, ctx_len: int, q_len: int) -> int:
    """Earliest token any of the row's queries can see (0 for global rows)."""
    if spec.is_global:
        return 0
    first_pos = ctx_len - q_len
    return max(0, first_pos - spec.window + 1)


def make_batch(spec: LayerSpec, ctx_lens, q_lens, key, *, back: str = "visible",
               shuffle: bool = True, poison: bool = False, extra_pages: int = 0,
               pt_stride: Optional[int] = None) -> Batch:
    """Draw one layer's batch.

    back="visible": only pages holding a token some query can see are backed, other
    page-table entries are -1. back="all": every page up to the row length is backed.
    poison=True fills never-visible slots (before the first needed token, after the
    row's end) and ``extra_pages`` unused pages with bf16 NaN.
    """
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    B = ctx_lens.shape[0]
    P, Hkv, hd, Hq = spec.page_size, spec.num_kv_heads, spec.head_dim, spec.num_q_heads
    assert np.all(ctx_lens >= 1) and np.all(q_lens >= 0) and np.all(q_lens <= ctx_lens)
    need = np.array([first_needed_token(spec, int(L), int(C)) for L, C in zip(ctx_lens, q_lens)], np.int32)
    k_starts = need if back == "visible" else np.zeros(B, np.int32)
    first_pg = k_starts // P
    last_pg = (ctx_lens - 1) // P
    n_pg = last_pg - first_pg + 1
    total = int(n_pg.sum())
    if pt_stride is None:
        pt_stride = int(((ctx_lens.max() + P - 1) // P)) if B else 1
    ids = np.arange(total, dtype=np.int64)
    if shuffle:
        ids = generator(*key, T_PERM).permutation(total)
    page_table = np.full((B, pt_stride), -1, dtype=np.int32)
    pos = 0
    for r in range(B):
        page_table[r, first_pg[r]:last_pg[r] + 1] = ids[pos:pos + n_pg[r]]
        pos += n_pg[r]

    T = int(q_lens.sum())
    q = normal_bf16(generator(*key, T_Q), (T, Hq, hd))
    # Draw every slot of every backed page, row after row, then keep the row's stored range.
    full_tokens = total * P
    kfull = normal_bf16(generator(*key, T_K), (full_tokens, Hkv, hd))
    vfull = None if spec.kv_shared else normal_bf16(generator(*key, T_V), (full_tokens, Hkv, hd))

    num_pages = total + extra_pages
    k_pool = np.empty((num_pages, Hkv, P, hd), dtype=np.uint16)
    v_pool = None if spec.kv_shared else np.empty_like(k_pool)
    if extra_pages:
        k_pool[total:] = BF16_NAN if poison else 0
        if v_pool is not None:
            v_pool[total:] = BF16_NAN if poison else 0

    ks, vs = [], []
    pos_tok = 0
    for r in range(B):
        t0 = int(first_pg[r]) * P
        nt = int(n_pg[r]) * P
        kr = kfull[pos_tok:pos_tok + nt]
        vr = None if vfull is None else vfull[pos_tok:pos_tok + nt]
        pos_tok += nt
        lo_keep = int(k_starts[r]) - t0
        hi_keep = int(ctx_lens[r]) - t0
        ks.append(kr[lo_keep:hi_keep])
        if vr is not None:
            vs.append(vr[lo_keep:hi_keep])
        if poison:
            kr = kr.copy()
            kr[:lo_keep] = BF16_NAN
            kr[hi_keep:] = BF16_NAN
            if vr is not None:
                vr = vr.copy()
                vr[:lo_keep] = BF16_NAN
                vr[hi_keep:] = BF16_NAN
        pids = page_table[r, first_pg[r]:last_pg[r] + 1]
        # token-major rows [n_pg*P][Hkv][hd] -> page-major [n_pg][Hkv][P][hd]
        k_pool[pids] = kr.reshape(int(n_pg[r]), P, Hkv, hd).transpose(0, 2, 1, 3)
        if vr is not None:
            v_pool[pids] = vr.reshape(int(n_pg[r]), P, Hkv, hd).transpose(0, 2, 1, 3)
    k = np.concatenate(ks) if ks else np.zeros((0, Hkv, hd), np.uint16)
    v = None if spec.kv_shared else (np.concatenate(vs) if vs else np.zeros((0, Hkv, hd), np.uint16))
    return Batch(spec, ctx_lens, q_lens, k_starts, q, k, v, page_table, k_pool, v_pool,
                 {"key": tuple(key), "back": back, "shuffle": shuffle, "poison": poison})


def gather_row_from_pool(batch: Batch, r: int, pool: np.ndarray) -> np.ndarray:
    """Read row r's stored tokens back out of a paged pool (the inverse of the scatter)."""
    P = batch.spec.page_size
    t = np.arange(int(batch.k_starts[r]), int(batch.ctx_lens[r]))
    pids = batch.page_table[r, t // P]
    return pool[pids, :, t % P, :]


# --------------------------------------------------------------------------- configs
def ragged(key, lo: int, hi: int, n: int) -> np.ndarray:
    return generator(*key, T_LEN).integers(lo, hi + 1, size=n).astype(np.int32)


def cfg1_tiny_decode(**kw) -> Batch:
    """One row, one local layer (4 q heads, 2 KV heads, hd 256, W 1024), L = 1025, scale 1/16,
    65 pages taken from a seeded permutation of a 65-page pool."""
    spec = LayerSpec("local", 4, 2, 256, window=1024, scale=1.0 / 16.0)
    return make_batch(spec, [1025], [1], (1, 0), back="all", **kw)


def cfg2_global_decode(B: int = 32, max_len: int = 8192, **kw) -> Batch:
    """Global decode: B rows, 32 q heads, 4 KV heads, hd 512, L ~ U{1..max_len}; split 512."""
    L = ragged((2, 0), 1, max_len, B)
    return make_batch(GLOBAL_31B, L, np.ones(B, np.int32), (2, 0), back="all", **kw)


def cfg3_local_decode(B: int = 64, lo: int = 512, hi: int = 32768, **kw) -> Batch:
    """Local decode: B rows, 32 q heads, 16 KV heads, hd 256, W 1024, L ~ U{lo..hi}; only
    window pages are backed."""
    L = ragged((3, 0), lo, hi, B)
    return make_batch(LOCAL_31B, L, np.ones(B, np.int32), (3, 0), back="visible", **kw)


def _mixed(spec: LayerSpec, cfg: int, fam: int, n_prefill: int, chunk: int, max_prior: int, n_decode: int,
           max_decode_len: int, **kw):
    prior = generator(cfg, fam, T_PRIOR).integers(0, max_prior + 1, size=n_prefill).astype(np.int32)
    pre = make_batch(spec, prior + chunk, np.full(n_prefill, chunk, np.int32), (cfg, fam, 0),
                     back="visible", **kw)
    L = ragged((cfg, fam, 1), 1, max_decode_len, n_decode)
    dec = make_batch(spec, L, np.ones(n_decode, np.int32), (cfg, fam, 1), back="visible", **kw)
    return pre, dec


def cfg4_mixed(family: str, n_prefill: int = 4, chunk: int = 2048, max_prior: int = 6144,
               n_decode: int = 60, max_decode_len: int = 8192, **kw):
    """Mixed step: prefill rows (chunk queries after a prior ~ U{0..max_prior}) and decode rows
    (L ~ U{1..max_decode_len}) of one family. Returns (prefill_batch, decode_batch)."""
    spec = GLOBAL_31B if family == "global" else LOCAL_31B
    fam = 1 if family == "global" else 0
    return _mixed(spec, 4, fam, n_prefill, chunk, max_prior, n_decode, max_decode_len, **kw)


def cfg6_12b_global_decode(B: int = 32, max_len: int = 8192, **kw) -> Batch:
    """12B global decode: B rows, 16 q heads, one KV head, hd 512, L ~ U{1..max_len}; split 512."""
    L = ragged((6, 0), 1, max_len, B)
    return make_batch(GLOBAL_12B, L, np.ones(B, np.int32), (6, 0), back="all", **kw)


def cfg6_12b_mixed(family: str, n_prefill: int = 4, chunk: int = 2048, max_prior: int = 6144,
                   n_decode: int = 60, max_decode_len: int = 8192, **kw):
    """The mixed step at the 12B geometry (same row recipe as the 31B mixed step)."""
    spec = GLOBAL_12B if family == "global" else LOCAL_12B
    fam = 1 if family == "global" else 0
    return _mixed(spec, 6, fam, n_prefill, chunk, max_prior, n_decode, max_decode_len, **kw)


def cfg5_layer_spec(family: str) -> LayerSpec:
    """Sweep layer geometry: global layers share K and V; local layers are the 31B local family."""
    return GLOBAL_31B_KV_SHARED if family == "global" else LOCAL_31B


def permute_pages(batch: Batch, key, extra_pages: int = 0, fill=0) -> Batch:
    """Same rows and values, different physical pages: a seeded relabelling of every page
    id (plus ``extra_pages`` unused pages filled with ``fill`` bits)."""
    n = batch.num_pages
    perm = generator(*key, T_PERM).permutation(n + extra_pages)[:n]
    k_pool = np.full((n + extra_pages,) + batch.k_pool.shape[1:], fill, dtype=np.uint16)
    k_pool[perm] = batch.k_pool
    v_pool = None
    if batch.v_pool is not None:
        v_pool = np.full_like(k_pool, fill)
        v_pool[perm] = batch.v_pool
    pt = batch.page_table.copy()
    m = pt >= 0
    pt[m] = perm[pt[m]]
    out = replace(batch, page_table=pt, k_pool=k_pool, v_pool=v_pool)
    out.meta = dict(batch.meta, repaged=tuple(key))
    return out


# --------------------------------------------------------------------------- full-size layouts
SWEEP_LAYERS, SWEEP_B, SWEEP_L = 60, 16, 32768
SWEEP_SPLIT = {"local": 512, "global": 1024}
LONG_L = 65536


@dataclass
class PagedLayout:
    """One layer's paged batch at full size, with K/V values drawn on the host only for some rows.

    Every row gets its context length, its backed pages (a global seeded shuffle of page ids, as
    in ``make_batch``) and its queries. The K/V values of the rows in ``rows`` come from the host
    generator (one PCG64 stream per row and tensor), and ``host`` holds them contiguously for the
    oracle. The other rows' pages are meant to be filled on the device with
    ``fill_normal_bf16_device`` from ``fill_seed``: they load the call at its real size, and rows
    are independent, so the sampled rows' outputs do not depend on those values.
    """
    spec: LayerSpec
    ctx_lens: np.ndarray        # int32 [B]
    k_starts: np.ndarray        # int32 [B]: first backed token of each row (page-aligned down)
    page_table: np.ndarray      # int32 [B][pt_stride]
    num_pages: int
    q: np.ndarray               # uint16 [B][Hq][hd]
    rows: tuple                 # rows drawn on the host
    row_pages: dict             # r -> int64 physical page ids of row r's backed pages, in order
    k_tok: dict                 # r -> uint16 [n_pg * P][Hkv][hd]: every slot of row r's backed
                                #      pages, token-major from token k_starts[r]
    v_tok: dict                 # same for V (empty when K=V)
    host: Optional[Batch]       # contiguous side of the sampled rows (None when rows is empty)
    fill_seed: int

    @property
    def B(self) -> int:
        return int(self.ctx_lens.shape[0])

    @property
    def pt_stride(self) -> int:
        return int(self.page_table.shape[1])


def paged_layout(spec: LayerSpec, ctx_lens, key, rows=(), pt_stride: Optional[int] = None) -> PagedLayout:
    """Decode layout (one query per row) for ``spec``: global rows back every page up to L,
    local rows only the pages that hold a visible key (the rest of the table is -1)."""
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    B, P = int(ctx_lens.shape[0]), spec.page_size
    Hkv, hd, Hq = spec.num_kv_heads, spec.head_dim, spec.num_q_heads
    need = np.array([first_needed_token(spec, int(L), 1) for L in ctx_lens], np.int64)
    first_pg = need // P
    last_pg = (ctx_lens.astype(np.int64) - 1) // P
    n_pg = last_pg - first_pg + 1
    total = int(n_pg.sum())
    if pt_stride is None:
        pt_stride = int((ctx_lens.max() + P - 1) // P)
    ids = generator(*key, T_PERM).permutation(total)
    page_table = np.full((B, pt_stride), -1, dtype=np.int32)
    row_pages, pos = {}, 0
    for r in range(B):
        page_table[r, first_pg[r]:last_pg[r] + 1] = ids[pos:pos + n_pg[r]]
        row_pages[r] = ids[pos:pos + n_pg[r]].astype(np.int64)
        pos += int(n_pg[r])
    q = normal_bf16(generator(*key, T_Q), (B, Hq, hd))
    rows = tuple(int(r) for r in rows)
    k_tok, v_tok, ks, vs = {}, {}, [], []
    for r in rows:
        nt = int(n_pg[r]) * P
        lo_keep, hi_keep = int(need[r] - first_pg[r] * P), int(ctx_lens[r] - first_pg[r] * P)
        k_tok[r] = normal_bf16(generator(*key, r, T_K), (nt, Hkv, hd))
        ks.append(k_tok[r][lo_keep:hi_keep])
        if not spec.kv_shared:
            v_tok[r] = normal_bf16(generator(*key, r, T_V), (nt, Hkv, hd))
            vs.append(v_tok[r][lo_keep:hi_keep])
    host = None
    if rows:
        sel = list(rows)
        cat = (lambda xs: xs[0] if len(xs) == 1 else np.concatenate(xs))
        empty = np.zeros((0, Hkv, P, hd), np.uint16)
        host = Batch(spec, ctx_lens[sel].copy(), np.ones(len(sel), np.int32), need[sel].astype(np.int32),
                     q[sel].copy(), cat(ks), None if spec.kv_shared else cat(vs),
                     page_table[sel].copy(), empty, None, {"key": tuple(key), "rows": rows})
    fill_seed = int(generator(*key, T_PRIOR + 1).integers(1, 2 ** 62))
    return PagedLayout(spec, ctx_lens, (first_pg * P).astype(np.int32), page_table, total, q, rows,
                       row_pages, k_tok, v_tok, host, fill_seed)


def fill_normal_bf16_device(t, seed: int, chunk: int = 1 << 26) -> None:
    """Fill a device tensor (bf16, or int16 holding bf16 bits) with N(0,1) values rounded to
    bf16, drawn by torch's device generator from ``seed``."""
    import torch
    flat = t.view(torch.bfloat16).view(-1) if t.dtype == torch.int16 else t.view(-1)
    g = torch.Generator(device=t.device)
    g.manual_seed(int(seed))
    for s in range(0, flat.numel(), chunk):
        e = min(flat.numel(), s + chunk)
        flat[s:e] = torch.randn(e - s, generator=g, device=t.device, dtype=torch.float32).to(torch.bfloat16)


def fill_e4m3_device(t, seed: int, scale: float, chunk: int = 1 << 26) -> None:
    """Fill a device uint8 tensor with E4M3 codes of N(0,1) / scale (torch's device generator and
    float8_e4m3fn cast; values beyond the format's range are clamped first so no code is NaN)."""
    import torch
    flat = t.view(-1)
    g = torch.Generator(device=t.device)
    g.manual_seed(int(seed))
    for s in range(0, flat.numel(), chunk):
        e = min(flat.numel(), s + chunk)
        x = torch.randn(e - s, generator=g, device=t.device, dtype=torch.float32) / scale
        flat[s:e] = x.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def sweep_layer(layer: int, family: str, rows=()) -> PagedLayout:
    """Layer ``layer`` of the 60-layer decode sweep: 16 rows at 32768 tokens; global layers share
    K and V (head_dim 512, 4 KV heads), local layers are the 31B local family (window pages only)."""
    return paged_layout(cfg5_layer_spec(family), np.full(SWEEP_B, SWEEP_L, np.int32), (5, layer), rows)


def long_global_decode(rows=(0,)) -> PagedLayout:
    """One 65536-token global decode row with K=V (split 1024 in the sweep's global setting)."""
    return paged_layout(GLOBAL_31B_KV_SHARED, np.array([LONG_L], np.int32), (5, SWEEP_LAYERS), rows)
