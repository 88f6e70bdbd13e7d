"""Device-side convenience around the C ABI for tests and the benchmark.

Moves a workloads.Batch (numpy, bf16 bit patterns) into torch device tensors and
calls gattn_decode / gattn_prefill through the binding. Argument marshalling
only: no attention arithmetic happens here.
"""
import numpy as np
import torch

from . import _native as nat


def dev(a, dtype=None):
    """numpy -> cuda tensor; uint16 (bf16 bits) travels as int16 with the same bits."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def host_bf16(t):
    """cuda int16 tensor of bf16 bits -> numpy float32."""
    u = t.detach().cpu().numpy().view(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def layer_of(spec):
    return nat.make_layer(spec.family, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.window,
                          spec.kv_shared, spec.softmax_scale)


class DeviceBatch:
    """A Batch's paged side resident on the GPU."""

    def __init__(self, batch):
        self.batch = batch
        s = batch.spec
        self.layer = layer_of(s)
        self.q = dev(batch.q)
        self.k_pool = dev(batch.k_pool)
        self.v_pool = None if batch.v_pool is None else dev(batch.v_pool)
        self.page_table = dev(batch.page_table.astype(np.int32))
        self.ctx_lens = dev(batch.ctx_lens.astype(np.int32))
        self.cu_q = dev(batch.cu_q.astype(np.int32))
        self.num_pages = batch.num_pages
        self.pt_stride = batch.pt_stride
        T = int(batch.q_lens.sum())
        self.out = torch.empty((T, s.num_q_heads, s.head_dim), dtype=torch.int16, device="cuda")
        self.lse = torch.empty((T, s.num_q_heads), dtype=torch.float32, device="cuda")
        self.workspace = None
        self.ws_bytes = 0
        f = getattr(batch, "fp8", None)
        self.k_pool8 = None if f is None else dev(f.k_pool)
        self.v_pool8 = None if f is None or f.v_pool is None else dev(f.v_pool)

    def _workspace(self, split_tokens, max_ctx, poison_workspace):
        need = nat.gattn_decode_workspace_bytes(self.layer, self.batch.B, max_ctx, split_tokens)
        if need > self.ws_bytes:
            self.workspace = torch.empty(need // 4, dtype=torch.float32, device="cuda")
            self.ws_bytes = need
            if poison_workspace:
                self.workspace.fill_(float("nan"))

    def decode(self, split_tokens, max_ctx=None, stream=None, poison_workspace=True):
        b = self.batch
        B = b.B
        max_ctx = int(b.ctx_lens.max()) if max_ctx is None else int(max_ctx)
        self._workspace(split_tokens, max_ctx, poison_workspace)
        nat.gattn_decode(self.layer, self.q, self.k_pool, self.v_pool, self.num_pages, self.page_table,
                         self.pt_stride, self.ctx_lens, B, max_ctx, split_tokens, self.workspace, self.ws_bytes,
                         self.out, self.lse, stream)

    def decode_fp8(self, split_tokens, max_ctx=None, stream=None, poison_workspace=True):
        """gattn_decode_fp8kv over the batch's E4M3 pools (Batch.fp8)."""
        b = self.batch
        max_ctx = int(b.ctx_lens.max()) if max_ctx is None else int(max_ctx)
        self._workspace(split_tokens, max_ctx, poison_workspace)
        nat.gattn_decode_fp8kv(self.layer, self.q, self.k_pool8, self.v_pool8, b.fp8.k_scale, b.fp8.v_scale,
                               self.num_pages, self.page_table, self.pt_stride, self.ctx_lens, b.B, max_ctx,
                               split_tokens, self.workspace, self.ws_bytes, self.out, self.lse, stream)

    def prefill(self, max_q=None, stream=None):
        b = self.batch
        max_q = int(b.q_lens.max()) if max_q is None else int(max_q)
        nat.gattn_prefill(self.layer, self.q, self.k_pool, self.v_pool, self.num_pages, self.page_table,
                          self.pt_stride, self.cu_q, self.ctx_lens, b.B, max_q, self.out, self.lse, stream)

    def result(self):
        torch.cuda.synchronize()
        return host_bf16(self.out).astype(np.float64), self.lse.cpu().numpy().astype(np.float64)


def decode(batch, split_tokens, max_ctx=None):
    d = DeviceBatch(batch)
    d.decode(split_tokens, max_ctx)
    return d.result()


def decode_fp8(batch, split_tokens, max_ctx=None):
    d = DeviceBatch(batch)
    d.decode_fp8(split_tokens, max_ctx)
    return d.result()


def prefill(batch, max_q=None):
    d = DeviceBatch(batch)
    d.prefill(max_q)
    return d.result()


class DeviceLayout:
    """A full-size paged decode layout (workloads.PagedLayout) resident on the GPU.

    Pools are filled on the device by ``fill(tensor, seed)``; the host-drawn rows' pages are then
    scattered in with torch indexing (page-major blocks from the token-major host rows). The
    workspace may be shared between layouts that run one after another on one stream.
    """

    def __init__(self, lay, fill, workspace=None, fp8=None):
        """fp8 = (k_scale, v_scale): E4M3 pools (one byte per element) filled by
        ``fill(tensor, seed, scale)``, read by gattn_decode_fp8kv; no host rows."""
        s = lay.spec
        self.lay = lay
        self.layer = layer_of(s)
        self.fp8 = fp8
        shape = (lay.num_pages, s.num_kv_heads, s.page_size, s.head_dim)
        if fp8 is not None:
            assert not lay.rows
            self.k_pool = torch.empty(shape, dtype=torch.uint8, device="cuda")
            fill(self.k_pool, lay.fill_seed, fp8[0])
            self.v_pool = None
            if not s.kv_shared:
                self.v_pool = torch.empty(shape, dtype=torch.uint8, device="cuda")
                fill(self.v_pool, lay.fill_seed + 1, fp8[1])
        else:
            self.k_pool = torch.empty(shape, dtype=torch.int16, device="cuda")
            fill(self.k_pool, lay.fill_seed)
            self.v_pool = None
            if not s.kv_shared:
                self.v_pool = torch.empty(shape, dtype=torch.int16, device="cuda")
                fill(self.v_pool, lay.fill_seed + 1)
        for r in lay.rows:
            pids = torch.from_numpy(lay.row_pages[r]).to("cuda")
            for pool, tok in ((self.k_pool, lay.k_tok.get(r)), (self.v_pool, lay.v_tok.get(r))):
                if pool is None or tok is None:
                    continue
                t = dev(tok).view(len(lay.row_pages[r]), s.page_size, s.num_kv_heads, s.head_dim)
                pool[pids] = t.permute(0, 2, 1, 3).contiguous()
        self.q = dev(lay.q)
        self.page_table = dev(lay.page_table.astype(np.int32))
        self.ctx_lens = dev(lay.ctx_lens.astype(np.int32))
        self.out = torch.empty((lay.B, s.num_q_heads, s.head_dim), dtype=torch.int16, device="cuda")
        self.lse = torch.empty((lay.B, s.num_q_heads), dtype=torch.float32, device="cuda")
        self.workspace = workspace
        self.ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()

    def workspace_bytes(self, split_tokens, max_ctx=None):
        max_ctx = int(self.lay.ctx_lens.max()) if max_ctx is None else int(max_ctx)
        return nat.gattn_decode_workspace_bytes(self.layer, self.lay.B, max_ctx, split_tokens)

    def decode(self, split_tokens, max_ctx=None, stream=None):
        lay = self.lay
        max_ctx = int(lay.ctx_lens.max()) if max_ctx is None else int(max_ctx)
        need = self.workspace_bytes(split_tokens, max_ctx)
        if need > self.ws_bytes:
            self.workspace = torch.empty(need // 4, dtype=torch.float32, device="cuda")
            self.ws_bytes = need
        if self.fp8 is not None:
            nat.gattn_decode_fp8kv(self.layer, self.q, self.k_pool, self.v_pool, self.fp8[0], self.fp8[1],
                                   lay.num_pages, self.page_table, lay.pt_stride, self.ctx_lens, lay.B, max_ctx,
                                   split_tokens, self.workspace, self.ws_bytes, self.out, self.lse, stream)
            return
        nat.gattn_decode(self.layer, self.q, self.k_pool, self.v_pool, lay.num_pages, self.page_table,
                         lay.pt_stride, self.ctx_lens, lay.B, max_ctx, split_tokens, self.workspace, self.ws_bytes,
                         self.out, self.lse, stream)

    def result(self, rows=None):
        torch.cuda.synchronize()
        o = host_bf16(self.out).astype(np.float64)
        l = self.lse.cpu().numpy().astype(np.float64)
        if rows is not None:
            o, l = o[list(rows)], l[list(rows)]
        return o, l
