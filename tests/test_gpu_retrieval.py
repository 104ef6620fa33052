"""GPU parity of RETRIEVAL heads through the C ABI (needs gfx950): the scored build's tables,
kept-position list and pool rows against the oracle's plan and keep lists (bit-exact), and
attention against the dense oracle with the same importance input.
"""

import numpy as np
import pytest
import torch

import oracle
from head_aware_paged_segpaged_amd import SegPagedLayer
from head_aware_paged_segpaged_amd import binding as B
from tests.helpers import (COS_MIN, DEV, MAXABS, assert_parity, group_parity, head_major,
                           to_device, to_f64)
from workloads import (GLOBAL, LOCAL, RETRIEVAL, config_case, custom_case, free_list,
                       importance_scores)

pytestmark = pytest.mark.gpu


def _keep_lists(c, imp):
    """Oracle keep list of every RETRIEVAL (request, head), in (request, head) order."""
    out, row0 = {}, 0
    for b in range(c.B):
        L, q = int(c.ctx_len[b]), int(c.q_len[b])
        for h in range(c.Hkv):
            kind, sink, window = (int(x) for x in c.policy[h])
            if kind == RETRIEVAL and L - q > 0:
                out[(b, h)] = oracle.retrieval_keep(imp[row0:row0 + L, h], sink, window, L, q)
        row0 += L
    return out


def _run(c, imp, n_phys=None):
    layer = SegPagedLayer(c.dtype, c.Hq, c.Hkv, c.D, c.P, c.ctx_len, c.q_len, c.policy, DEV)
    fl = free_list(c.seed, layer.n_virt if n_phys is None else n_phys)
    layer.build(to_device(c.k, c.dtype), to_device(c.v, c.dtype), fl, n_phys=n_phys,
                importance=head_major(imp))
    out = layer.attention(to_device(c.q, c.dtype), c.scale)
    torch.cuda.synchronize()
    assert layer.check() == 0
    seg_o, kvl_o, n_virt = oracle.plan_tables(c.ctx_len, c.q_len, c.policy, c.P)
    np.testing.assert_array_equal(layer.seg_table.cpu().numpy(), seg_o)
    np.testing.assert_array_equal(layer.kv_len.cpu().numpy(), kvl_o)
    keeps = _keep_lists(c, imp)
    flat = [p for key in sorted(keeps) for p in keeps[key]]
    np.testing.assert_array_equal(layer.row_pos.cpu().numpy()[:len(flat)], flat)
    kp, vp = layer.k_pool.cpu(), layer.v_pool.cpu()
    kk, vv = to_device(c.k, c.dtype).cpu(), to_device(c.v, c.dtype).cpu()
    row0 = np.concatenate([[0], np.cumsum(c.ctx_len)[:-1]])
    for b in range(c.B):
        for h in range(c.Hkv):
            got = oracle.gather_positions(seg_o, fl, c.P, b, h, keeps.get((b, h)))
            if not got:
                continue
            pos = torch.tensor([g[0] for g in got], dtype=torch.long) + int(row0[b])
            ph = torch.tensor([g[1] for g in got], dtype=torch.long)
            sl = torch.tensor([g[2] for g in got], dtype=torch.long)
            assert torch.equal(kp[ph, sl], kk[pos, h]) and torch.equal(vp[ph, sl], vv[pos, h])
    ref = oracle.attention(c.q, c.k, c.v, c.ctx_len, c.q_len, c.policy, c.Hq, c.Hkv, c.scale,
                           c.dtype, importance=imp)
    assert_parity(to_f64(out), ref, c, "retrieval")
    return layer


def _cases(n=10, seed=880):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(rng.choice([2, 4]))
        G = int(rng.choice([1, 4, 8]))
        B = int(rng.integers(1, 4))
        P = int(rng.choice([16, 64, 128]))
        ctx = [int(rng.integers(1, 3000)) for _ in range(B)]
        q = [min(c, int(rng.choice([1, 1, 5, 77, 300]))) for c in ctx]
        pol = [(RETRIEVAL, int(rng.choice([0, 4])), int(rng.choice([1, 50, 300, 1000])))
               if h % 2 == 0 else
               ((GLOBAL, 0, 1) if rng.random() < 0.4 else (LOCAL, 4, int(rng.choice([64, 700]))))
               for h in range(Hkv)]
        dtype = "f32" if i % 4 == 3 else "bf16"
        out.append((900 + i, dtype, Hkv * G, Hkv, 128 if dtype == "bf16" else 64, P, ctx, q,
                    pol, 3 if i % 3 == 0 else 0))
    return out


@pytest.mark.parametrize("args", _cases(), ids=lambda a: "seed%d" % a[0])
def test_retrieval_heads_against_oracle(args):
    seed, dtype, Hq, Hkv, D, P, ctx, q, pol, levels = args
    print("case retrieval", args, flush=True)
    c = custom_case(seed, dtype=dtype, Hq=Hq, Hkv=Hkv, D=D, P=P, ctx_len=ctx, q_len=q,
                    policy=pol)
    _run(c, importance_scores(c, levels=levels))


def test_retrieval_table_decode_is_bitwise_the_planned_decode():
    pol = [(RETRIEVAL, 4, 100), (GLOBAL, 0, 1), (RETRIEVAL, 0, 30), (LOCAL, 4, 512)]
    ctx = [9000, 300, 20000, 5]
    c = custom_case(950, dtype="bf16", Hq=16, Hkv=4, D=128, P=64, ctx_len=ctx,
                    q_len=[1, 1, 1, 1], policy=pol)
    print("case retrieval table decode", flush=True)
    layer = _run(c, importance_scores(c))
    n = B.segpaged_decode_workspace_size("bf16", 16, 4, 128, 64, ctx, pol)
    ws = torch.zeros((n,), dtype=torch.uint8, device=DEV)
    B.segpaged_decode_plan("bf16", 16, 4, 128, 64, ctx, pol, ws)
    q = to_device(c.q, "bf16")
    a = layer.attention(q, c.scale)
    b = torch.empty_like(q)
    B.segpaged_decode("bf16", 16, 4, 128, 64, pol, q, layer.k_pool, layer.v_pool, layer.n_phys,
                      layer.seg_table, layer.kv_len, layer.v2p, c.scale, b, ws)
    torch.cuda.synchronize()
    assert B.segpaged_attention_check(ws) == 0
    assert torch.equal(a, b)


def test_full_size_retrieval_workload_all_rows():
    # The decode workload with two RETRIEVAL heads (10 % of each prefix kept): tables and
    # kept lists bit-exact, two retrieval heads' pool rows bit-exact, every output row
    # against the oracle.
    c = config_case(7)
    imp = importance_scores(c)
    print("case full-size", c.name, flush=True)
    layer = SegPagedLayer(c.dtype, c.Hq, c.Hkv, c.D, c.P, c.ctx_len, c.q_len, c.policy, DEV)
    fl = free_list(c.seed, layer.n_virt)
    layer.build(to_device(c.k, c.dtype), to_device(c.v, c.dtype), fl,
                importance=head_major(imp))
    out = to_f64(layer.attention(to_device(c.q, c.dtype), c.scale))
    torch.cuda.synchronize()
    assert layer.check() == 0
    seg_o, kvl_o, _ = oracle.plan_tables(c.ctx_len, c.q_len, c.policy, c.P)
    np.testing.assert_array_equal(layer.seg_table.cpu().numpy(), seg_o)
    np.testing.assert_array_equal(layer.kv_len.cpu().numpy(), kvl_o)
    keeps = _keep_lists(c, imp)
    flat = np.concatenate([keeps[key] for key in sorted(keeps)])
    np.testing.assert_array_equal(layer.row_pos.cpu().numpy(), flat)
    rng = np.random.default_rng(77)
    row0 = np.concatenate([[0], np.cumsum(c.ctx_len)[:-1]])
    retrieval_heads = [h for h in range(c.Hkv) if c.policy[h, 0] == RETRIEVAL]
    for _ in range(2):
        b, h = int(rng.integers(c.B)), int(rng.choice(retrieval_heads))
        got = oracle.gather_positions(seg_o, fl, c.P, b, h, keeps[(b, h)])
        pos = torch.tensor([g[0] for g in got], dtype=torch.long, device=DEV) + int(row0[b])
        ph = torch.tensor([g[1] for g in got], dtype=torch.long, device=DEV)
        sl = torch.tensor([g[2] for g in got], dtype=torch.long, device=DEV)
        k = to_device(c.k, c.dtype)
        assert torch.equal(layer.k_pool[ph, sl], k[pos, h])
    # every row: one decode query per (request, query head)
    groups = [(b, h, np.array([0])) for b in range(c.B) for h in range(c.Hkv)]
    worst_abs, worst_cos, rows = group_parity(c, out, groups, importance=imp, label="all rows")
    assert rows == c.B * c.Hq
    assert worst_abs <= MAXABS[c.dtype] and worst_cos > COS_MIN


@pytest.mark.parametrize("dtype,P", [("bf16", 256), ("f32", 16)])
def test_retrieval_edge_requests(dtype, P):
    # one request with no queries (its kept prefix is stored, nothing attends), one whose whole
    # context is the query chunk (no prefix: the chunk alone), one decode request, and sinks
    # longer than the prefix
    pol = [(RETRIEVAL, 4, 1), (RETRIEVAL, 700, 500), (GLOBAL, 0, 1), (RETRIEVAL, 0, 1000)]
    c = custom_case(960 + P, dtype=dtype, Hq=8, Hkv=4, D=128 if dtype == "bf16" else 64, P=P,
                    ctx_len=[500, 90, 1300, 7], q_len=[0, 90, 1, 3], policy=pol)
    print("case retrieval edges", dtype, P, flush=True)
    _run(c, importance_scores(c, levels=2))


def test_retrieval_many_requests_and_selection_tasks():
    # 200 requests with two retrieval heads each: more selection tasks than one launch holds
    # (two selection launches) and more (request) groups than one scatter launch holds with a
    # gather table per group (three scatter launches); heavily tied importance (4 levels) and
    # long prefixes (up to 40K tokens, so the radix select's histogram passes are deep);
    # kept lists, tables, pool rows and output against the oracle.
    rng = np.random.default_rng(4242)
    B = 200
    ctx = [int(x) for x in rng.integers(1, 4000, B)]
    ctx[0], ctx[1] = 40000, 25000
    q = [min(c, int(rng.choice([1, 1, 3, 40]))) for c in ctx]
    pol = [(RETRIEVAL, 4, 100), (GLOBAL, 0, 1), (RETRIEVAL, 0, 37), (LOCAL, 4, 256)]
    c = custom_case(977, dtype="bf16", Hq=8, Hkv=4, D=64, P=64, ctx_len=ctx, q_len=q,
                    policy=pol)
    print("case retrieval many requests", flush=True)
    _run(c, importance_scores(c, levels=4))
