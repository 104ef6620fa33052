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

    def build(self, k_dense: torch.Tensor, v_dense: torch.Tensor, free_pages,
              n_phys: int | None = None, stream=None) -> None:
        """Allocate the pool and tables and fill them from dense [T, Hkv, D] K/V."""
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
        self.rebuild(k_dense, v_dense, fl, stream)

    def rebuild(self, k_dense: torch.Tensor, v_dense: torch.Tensor, free_pages,
                stream=None) -> None:
        """Refill the already allocated pool and tables (no allocation)."""
        fl = np.asarray(free_pages, dtype=np.int32)
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
