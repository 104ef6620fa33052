"""segpaged_attention_static: the entry point for callers that cannot allocate device memory
(it runs on a library-owned static workspace). Its output must equal segpaged_attention's on
the same inputs, bit for bit, on two calls in a row with the second one smaller, and plans
beyond the static workspace are refused before anything is written."""

import numpy as np
import pytest
import torch

from head_aware_paged_segpaged_amd import binding as B
from tests.helpers import DEV, run_segpaged, to_device
from workloads import GLOBAL, LOCAL, custom_case

pytestmark = pytest.mark.gpu


def _static(layer, c, q, out, err):
    B.segpaged_attention_static(c.dtype, c.Hq, c.Hkv, c.D, c.P, c.ctx_len, c.q_len, c.policy, q,
                                layer.k_pool, layer.v_pool, layer.n_phys, layer.seg_table,
                                layer.kv_len, layer.v2p, c.scale, out, error=err)


def test_static_workspace_matches_workspace_call_twice():
    big = custom_case(901, dtype="bf16", Hq=32, Hkv=8, D=128, P=64, ctx_len=[8192, 3000, 1],
                      q_len=[512, 1, 1],
                      policy=[(GLOBAL, 0, 1), (LOCAL, 4, 512)] * 4)
    small = custom_case(902, dtype="f32", Hq=4, Hkv=2, D=64, P=16, ctx_len=[300, 40],
                        q_len=[17, 40], policy=[(LOCAL, 4, 32), (GLOBAL, 0, 1)])
    err = torch.full((1,), -99, dtype=torch.int32, device=DEV)
    for c in (big, small):  # the second call is smaller and reuses the same static array
        print("case static", c.name, c.dtype, list(c.ctx_len), list(c.q_len), flush=True)
        ref, layer = run_segpaged(c)  # the workspace entry point
        q = to_device(c.q, c.dtype)
        out = torch.full_like(ref, float("nan"))
        _static(layer, c, q, out, err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert torch.equal(out, ref), float((out.float() - ref.float()).abs().max())
        err.fill_(-99)


def test_static_workspace_refuses_plans_beyond_its_size():
    # 1100 requests of 2048-token chunks over 64 KV heads: 1.1 M work items, a plan of about
    # 70 MiB, more than the 64 MiB the library holds; refused before anything is launched
    n, L, Hkv = 1100, 2048, 64
    pol = np.array([(GLOBAL, 0, 1)] * Hkv, np.int32)
    ctx = np.full(n, L, np.int32)
    need = B.segpaged_attention_workspace_size("bf16", Hkv, Hkv, 128, 64, ctx, ctx, pol)
    assert need > (64 << 20)
    d = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    t = torch.zeros(16, dtype=torch.int32, device=DEV)
    with pytest.raises(B.SegPagedError) as e:
        B.segpaged_attention_static("bf16", Hkv, Hkv, 128, 64, ctx, ctx, pol, d, d, d, 1, t, t, t,
                                    0.1, d)
    assert e.value.status == B.SP_ERR_WORKSPACE_TOO_SMALL
