"""Buffer ownership around the C-ABI calls: pools, tables and workspaces as torch tensors.

``SegPagedLayer`` holds one layout (one layer's per-head page tables over one pool): it is
built once from dense K/V and then serves any number of attention calls (page "RedKnot
SegPagedAttention runtime design", section 5: layout work belongs at KV-write time and is
reused). ``DenseMaskLayer`` is the dense-plus-mask comparison path over the same shapes.
torch supplies device memory and the stream; the arithmetic is in libsegpaged's kernels.
"""

from __future__ import annotations

import numpy as np
import torch

from . import binding as B

_TORCH = {"bf16": torch.bfloat16, "f32": torch.float32}


def _device_f32(x, device) -> torch.Tensor:
    """A contiguous float32 device tensor holding x (a tensor or a host array)."""
    if isinstance(x, torch.Tensor):
        return x.to(device=device, dtype=torch.float32).contiguous()
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32))).to(device)


def _check_importance(importance, Hkv: int, ctx_len) -> None:
    """RETRIEVAL importance must be head-major, [Hkv, sum(ctx_len)]."""
    shape = tuple(importance.shape)
    want = (int(Hkv), int(np.asarray(ctx_len, dtype=np.int64).sum()))
    if shape != want:
        raise ValueError("importance must be [Hkv, sum(ctx_len)] = %s (head-major), got %s"
                         % (want, shape))


def _dt(dtype) -> str:
    return "bf16" if B._dtype_code(dtype) == B.SP_BF16 else "f32"


class SegPagedLayer:
    def __init__(self, dtype, Hq: int, Hkv: int, D: int, page_size: int, ctx_len, q_len, policy,
                 device: str = "cuda"):
        self.dtype = _dt(dtype)
        self.Hq, self.Hkv, self.D, self.P = int(Hq), int(Hkv), int(D), int(page_size)
        self.ctx_len = np.asarray(ctx_len, dtype=np.int32)
        self.q_len = np.asarray(q_len, dtype=np.int32)
        self.policy = np.asarray(policy, dtype=np.int32).reshape(self.Hkv, 3)
        self.device = device
        self.n_virt = B.segpaged_plan_pages(self.ctx_len, self.q_len, self.policy, self.P)
        self.k_pool = self.v_pool = None
        self.seg_table = self.kv_len = self.v2p = None
        self.workspace = None
        self.n_phys = 0
        self.row_pos = None
        self.importance = None

    def build(self, k_dense: torch.Tensor, v_dense: torch.Tensor, free_pages,
              n_phys: int | None = None, stream=None, importance=None) -> None:
        """Allocate the pool and tables and fill them from dense [T, Hkv, D] K/V. Layouts with
        RETRIEVAL heads need ``importance`` (float32 [Hkv, T], head-major: each KV head's
        scores of all tokens contiguous; a device tensor or host array, kept on the device for
        rebuilds)."""
        if importance is not None:
            _check_importance(importance, self.Hkv, self.ctx_len)
        fl = np.asarray(free_pages, dtype=np.int32)
        self.n_phys = int(n_phys if n_phys is not None else max(self.n_virt, 1))
        t = _TORCH[self.dtype]
        self.k_pool = torch.empty((max(self.n_phys, 1), self.P, self.D), dtype=t,
                                  device=self.device)
        self.v_pool = torch.empty_like(self.k_pool)
        # one allocation, three adjacent tables: the build uploads them in a single copy
        Bn = max(len(self.ctx_len), 1)
        n_tab, n_kl = Bn * self.Hkv * 8, Bn * self.Hkv
        tables = torch.zeros((n_tab + n_kl + max(self.n_virt, 1),), dtype=torch.int32,
                             device=self.device)
        self.seg_table = tables[:n_tab].view(Bn, self.Hkv, 2, 4)
        self.kv_len = tables[n_tab:n_tab + n_kl].view(Bn, self.Hkv)
        self.v2p = tables[n_tab + n_kl:]
        if importance is not None:
            self.importance = _device_f32(importance, self.device)
            n_rows = B.segpaged_retrieval_rows(self.ctx_len, self.q_len, self.policy)
            self.row_pos = torch.zeros((max(n_rows, 1),), dtype=torch.int32, device=self.device)
        self.rebuild(k_dense, v_dense, fl, stream)

    def rebuild(self, k_dense: torch.Tensor, v_dense: torch.Tensor, free_pages,
                stream=None) -> None:
        """Refill the already allocated pool and tables (no allocation)."""
        fl = np.asarray(free_pages, dtype=np.int32)
        if self.importance is not None:
            B.segpaged_build_scored(self.dtype, self.D, self.P, self.ctx_len, self.q_len,
                                    self.policy, self.importance, k_dense, v_dense, fl,
                                    self.n_phys, self.k_pool, self.v_pool, self.seg_table,
                                    self.kv_len, self.v2p, self.row_pos, stream)
            return
        B.segpaged_build(self.dtype, self.D, self.P, self.ctx_len, self.q_len, self.policy,
                         k_dense, v_dense, fl, self.n_phys, self.k_pool, self.v_pool,
                         self.seg_table, self.kv_len, self.v2p, stream)

    def plan(self, stream=None) -> None:
        """Allocate the workspace and write the attention work list into it."""
        n = B.segpaged_attention_workspace_size(self.dtype, self.Hq, self.Hkv, self.D, self.P,
                                                self.ctx_len, self.q_len, self.policy)
        self.workspace = torch.zeros((n,), dtype=torch.uint8, device=self.device)
        B.segpaged_attention_plan(self.dtype, self.Hq, self.Hkv, self.D, self.P, self.ctx_len,
                                  self.q_len, self.policy, self.workspace, stream)

    def attention(self, q: torch.Tensor, scale: float, out: torch.Tensor | None = None,
                  stream=None, events=None) -> torch.Tensor:
        if self.workspace is None:
            self.plan(stream)
        if out is None:
            out = torch.empty_like(q)
        args = (self.dtype, self.Hq, self.Hkv, self.D, self.P, self.ctx_len, self.q_len,
                self.policy, q, self.k_pool, self.v_pool, self.n_phys, self.seg_table,
                self.kv_len, self.v2p, scale, out, self.workspace)
        if events is None:
            B.segpaged_attention(*args, stream=stream)
        else:
            B.segpaged_attention_profiled(*args, events[0], events[1], stream=stream)
        return out

    def check(self, stream=None) -> int:
        return B.segpaged_attention_check(self.workspace, stream)


class SegPagedLayers:
    """Several layers of one batch in ONE page pool, built by one call (page "RedKnot
    SegPagedAttention runtime design", section 3: the page table is keyed by (layer, head,
    segment)). Dense K/V come stacked as [n_layers, T, Hkv, D]; layer l is attended through its
    own slice of the tables, its own work list and the shared pools and v2p."""

    def __init__(self, dtype, n_layers: int, Hq: int, Hkv: int, D: int, page_size: int, ctx_len,
                 q_len, policies, device: str = "cuda"):
        self.dtype = _dt(dtype)
        self.n_layers = int(n_layers)
        self.Hq, self.Hkv, self.D, self.P = int(Hq), int(Hkv), int(D), int(page_size)
        self.ctx_len = np.asarray(ctx_len, dtype=np.int32)
        self.q_len = np.asarray(q_len, dtype=np.int32)
        self.policies = np.asarray(policies, dtype=np.int32).reshape(self.n_layers, self.Hkv, 3)
        self.device = device
        self.n_virt = B.segpaged_plan_pages_layers(self.ctx_len, self.q_len, self.policies,
                                                   self.P)
        self.k_pool = self.v_pool = None
        self.seg_table = self.kv_len = self.v2p = None
        self.workspaces = [None] * self.n_layers
        self.n_phys = 0

    def build(self, k_dense: torch.Tensor, v_dense: torch.Tensor, free_pages,
              n_phys: int | None = None, stream=None) -> None:
        """Allocate the shared pool and the tables and fill them from all layers' dense K/V."""
        self.n_phys = int(n_phys if n_phys is not None else max(self.n_virt, 1))
        t = _TORCH[self.dtype]
        self.k_pool = torch.empty((max(self.n_phys, 1), self.P, self.D), dtype=t,
                                  device=self.device)
        self.v_pool = torch.empty_like(self.k_pool)
        Bn = max(len(self.ctx_len), 1)
        n_tab, n_kl = self.n_layers * Bn * self.Hkv * 8, self.n_layers * Bn * self.Hkv
        tables = torch.zeros((n_tab + n_kl + max(self.n_virt, 1),), dtype=torch.int32,
                             device=self.device)
        self.seg_table = tables[:n_tab].view(self.n_layers, Bn, self.Hkv, 2, 4)
        self.kv_len = tables[n_tab:n_tab + n_kl].view(self.n_layers, Bn, self.Hkv)
        self.v2p = tables[n_tab + n_kl:]
        self.rebuild(k_dense, v_dense, free_pages, stream)

    def rebuild(self, k_dense: torch.Tensor, v_dense: torch.Tensor, free_pages,
                stream=None) -> None:
        """Refill the already allocated pool and tables (no allocation)."""
        B.segpaged_build_layers(self.dtype, self.D, self.P, self.ctx_len, self.q_len,
                                self.policies, k_dense, v_dense,
                                np.asarray(free_pages, dtype=np.int32), self.n_phys,
                                self.k_pool, self.v_pool, self.seg_table, self.kv_len, self.v2p,
                                stream)

    def attention(self, layer: int, q: torch.Tensor, scale: float,
                  out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        pol = self.policies[layer]
        if self.workspaces[layer] is None:
            n = B.segpaged_attention_workspace_size(self.dtype, self.Hq, self.Hkv, self.D,
                                                    self.P, self.ctx_len, self.q_len, pol)
            ws = torch.zeros((n,), dtype=torch.uint8, device=self.device)
            B.segpaged_attention_plan(self.dtype, self.Hq, self.Hkv, self.D, self.P,
                                      self.ctx_len, self.q_len, pol, ws, stream)
            self.workspaces[layer] = ws
        if out is None:
            out = torch.empty_like(q)
        B.segpaged_attention(self.dtype, self.Hq, self.Hkv, self.D, self.P, self.ctx_len,
                             self.q_len, pol, q, self.k_pool, self.v_pool, self.n_phys,
                             self.seg_table[layer], self.kv_len[layer], self.v2p, scale, out,
                             self.workspaces[layer], stream=stream)
        return out

    def check(self, layer: int, stream=None) -> int:
        return B.segpaged_attention_check(self.workspaces[layer], stream)


class SegPagedDecoder:
    """One layer's growable layout for decoding: built once (pages reserved for ``reserve``
    more tokens per request), then every step appends each request's new token and runs the
    table-driven decode, all on the device (page "RedKnot SegPagedAttention runtime design",
    section 3: LOCAL storage does not grow with the context; section 5: no layout work per
    call). ``ctx_now`` tracks the lengths on the host only to size the decode splits."""

    def __init__(self, dtype, Hq: int, Hkv: int, D: int, page_size: int, ctx_len, q_len, reserve,
                 policy, device: str = "cuda"):
        self.dtype = _dt(dtype)
        self.Hq, self.Hkv, self.D, self.P = int(Hq), int(Hkv), int(D), int(page_size)
        self.ctx_len = np.asarray(ctx_len, dtype=np.int32)
        self.q_len = np.asarray(q_len, dtype=np.int32)
        self.reserve = np.asarray(reserve, dtype=np.int32)
        self.policy = np.asarray(policy, dtype=np.int32).reshape(self.Hkv, 3)
        self.device = device
        self.n_virt = B.segpaged_plan_pages_growable(self.ctx_len, self.q_len, self.reserve,
                                                     self.policy, self.P)
        self.ctx_now = self.ctx_len.copy()
        self.k_pool = self.v_pool = None
        self.seg_table = self.kv_len = self.v2p = None
        self.error = None
        self.workspace = None
        self.row_pos = None
        self.n_phys = 0

    def build(self, k_dense: torch.Tensor, v_dense: torch.Tensor, free_pages,
              n_phys: int | None = None, stream=None, importance=None) -> None:
        """Layouts with RETRIEVAL heads need ``importance`` (float32 [Hkv, T], head-major; a
        device tensor or host array)."""
        if importance is not None:
            _check_importance(importance, self.Hkv, self.ctx_len)
        self.n_phys = int(n_phys if n_phys is not None else max(self.n_virt, 1))
        t = _TORCH[self.dtype]
        self.k_pool = torch.empty((max(self.n_phys, 1), self.P, self.D), dtype=t,
                                  device=self.device)
        self.v_pool = torch.empty_like(self.k_pool)
        Bn = max(len(self.ctx_len), 1)
        n_tab, n_kl = Bn * self.Hkv * 8, Bn * self.Hkv
        tables = torch.zeros((n_tab + n_kl + max(self.n_virt, 1) + 1,), dtype=torch.int32,
                             device=self.device)
        self.seg_table = tables[:n_tab].view(Bn, self.Hkv, 2, 4)
        self.kv_len = tables[n_tab:n_tab + n_kl].view(Bn, self.Hkv)
        self.v2p = tables[n_tab + n_kl:n_tab + n_kl + max(self.n_virt, 1)]
        self.error = tables[-1:]
        fl = np.asarray(free_pages, dtype=np.int32)
        if importance is not None:
            n_rows = B.segpaged_retrieval_rows(self.ctx_len, self.q_len, self.policy)
            self.row_pos = torch.zeros((max(n_rows, 1),), dtype=torch.int32, device=self.device)
            B.segpaged_build_scored(self.dtype, self.D, self.P, self.ctx_len, self.q_len,
                                    self.policy, _device_f32(importance, self.device), k_dense,
                                    v_dense, fl, self.n_phys,
                                    self.k_pool, self.v_pool, self.seg_table, self.kv_len,
                                    self.v2p, self.row_pos, stream, reserve=self.reserve)
        else:
            B.segpaged_build_growable(self.dtype, self.D, self.P, self.ctx_len, self.q_len,
                                      self.reserve, self.policy, k_dense, v_dense, fl,
                                      self.n_phys, self.k_pool, self.v_pool, self.seg_table,
                                      self.kv_len, self.v2p, stream)
        self.ctx_now = self.ctx_len.copy()

    def plan(self, stream=None) -> None:
        """(Re)plan the table-driven decode, with splits sized for the current lengths."""
        n = B.segpaged_decode_workspace_size(self.dtype, self.Hq, self.Hkv, self.D, self.P,
                                             self.ctx_now, self.policy)
        if self.workspace is None or self.workspace.numel() < n:
            self.workspace = torch.zeros((n,), dtype=torch.uint8, device=self.device)
        B.segpaged_decode_plan(self.dtype, self.Hq, self.Hkv, self.D, self.P, self.ctx_now,
                               self.policy, self.workspace, stream)

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor, n_new=None, stream=None) -> None:
        """k_new, v_new: [B, Hkv, D]; n_new: None (every request) or 0/1 per request (host
        array, copied to the device, or a device int32 tensor)."""
        dev_n = None
        if n_new is not None:
            if isinstance(n_new, torch.Tensor) and n_new.is_cuda:
                dev_n = n_new
                host_n = n_new.cpu().numpy()
            else:
                host_n = np.asarray(n_new, dtype=np.int32)
                dev_n = torch.from_numpy(host_n.copy()).to(self.device)
            self.ctx_now = self.ctx_now + host_n.astype(np.int32)
        else:
            self.ctx_now = self.ctx_now + 1
        B.segpaged_append(self.dtype, self.D, self.P, self.policy, dev_n, k_new, v_new,
                          self.k_pool, self.v_pool, self.n_phys, self.seg_table, self.kv_len,
                          self.v2p, self.error, stream)

    def decode(self, q: torch.Tensor, scale: float, out: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
        """q: [B, Hq, D], one query per request at its newest position."""
        if self.workspace is None:
            self.plan(stream)
        if out is None:
            out = torch.empty_like(q)
        B.segpaged_decode(self.dtype, self.Hq, self.Hkv, self.D, self.P, self.policy, q,
                          self.k_pool, self.v_pool, self.n_phys, self.seg_table, self.kv_len,
                          self.v2p, scale, out, self.workspace, stream)
        return out

    def capture_step(self, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                     out: torch.Tensor, scale: float) -> torch.cuda.CUDAGraph:
        """Captures one decode step (append every request's token from k_new / v_new, then
        decode q into out) as a HIP graph. The step launches only kernels: no host work, no
        copies, no memsets, no synchronisation. Replay it after writing the next token's rows
        and queries into the same buffers; each replay appends one token per request, so the
        reserve bounds the number of replays. ``ctx_now`` is not advanced by replays; call
        ``advance(n)`` to keep it for re-planning."""
        if self.workspace is None:
            self.plan()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            B.segpaged_append(self.dtype, self.D, self.P, self.policy, None, k_new, v_new,
                              self.k_pool, self.v_pool, self.n_phys, self.seg_table,
                              self.kv_len, self.v2p, self.error)
            B.segpaged_decode(self.dtype, self.Hq, self.Hkv, self.D, self.P, self.policy, q,
                              self.k_pool, self.v_pool, self.n_phys, self.seg_table, self.kv_len,
                              self.v2p, scale, out, self.workspace)
        return graph

    def advance(self, n: int = 1) -> None:
        """Records n appends of every request made outside ``append`` (graph replays)."""
        self.ctx_now = self.ctx_now + int(n)

    def check(self, stream=None) -> tuple[int, int]:
        """(append error word, decode workspace error word); reading clears both."""
        torch.cuda.synchronize()
        a = int(self.error.item())
        self.error.zero_()
        d = B.segpaged_attention_check(self.workspace, stream) if self.workspace is not None else 0
        return a, d


class DenseMaskLayer:
    def __init__(self, dtype, Hq: int, Hkv: int, D: int, ctx_len, q_len, policy,
                 device: str = "cuda"):
        self.dtype = _dt(dtype)
        self.Hq, self.Hkv, self.D = int(Hq), int(Hkv), int(D)
        self.ctx_len = np.asarray(ctx_len, dtype=np.int32)
        self.q_len = np.asarray(q_len, dtype=np.int32)
        self.policy = np.asarray(policy, dtype=np.int32).reshape(self.Hkv, 3)
        self.device = device
        self.workspace = None

    def plan(self, stream=None) -> None:
        n = B.segpaged_dense_mask_workspace_size(self.dtype, self.Hq, self.Hkv, self.D,
                                                 self.ctx_len, self.q_len, self.policy)
        self.workspace = torch.zeros((n,), dtype=torch.uint8, device=self.device)
        B.segpaged_dense_mask_plan(self.dtype, self.Hq, self.Hkv, self.D, self.ctx_len,
                                   self.q_len, self.policy, self.workspace, stream)

    def attention(self, q, k_dense, v_dense, scale: float, out=None, stream=None):
        if self.workspace is None:
            self.plan(stream)
        if out is None:
            out = torch.empty_like(q)
        B.segpaged_dense_mask_attention(self.dtype, self.Hq, self.Hkv, self.D, self.ctx_len,
                                        self.q_len, self.policy, q, k_dense, v_dense, scale,
                                        out, self.workspace, stream)
        return out
