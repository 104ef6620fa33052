"""A sweep of small seeded random layouts through the C ABI against the whole oracle (needs
gfx950): every head kind (GLOBAL, LOCAL, context-adaptive LOCAL, RETRIEVAL) mixed within a
layout, both dtypes and head dims, page sizes 16-256, 1-64 query heads per KV head, empty
contexts and empty query chunks, decode and prefill requests side by side. Bars as in
test_gpu_parity.py: tables bit-exact, O within max abs 2e-2 (bf16) / 1e-5 (fp32) and cosine >
0.99998 per (request, query head)."""

import numpy as np
import pytest
import torch

import oracle
from head_aware_paged_segpaged_amd import SegPagedLayer
from tests.helpers import DEV, assert_parity, head_major, to_device, to_f64
from workloads import (GLOBAL, LOCAL, LOCAL_ADAPTIVE, RETRIEVAL, custom_case, free_list,
                       importance_scores)

pytestmark = pytest.mark.gpu


def _policy(rng):
    r = rng.random()
    if r < 0.3:
        return (GLOBAL, 0, 1)
    if r < 0.6:
        return (LOCAL, int(rng.choice([0, 1, 4, 70])), int(rng.choice([1, 16, 63, 64, 65, 400])))
    if r < 0.8:
        return (LOCAL_ADAPTIVE, int(rng.choice([0, 4])), int(rng.choice([1, 2, 3, 7])))
    return (RETRIEVAL, int(rng.choice([0, 4, 100])), int(rng.choice([1, 100, 500, 999, 1000])))


def _shapes(n=160, seed=31337):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(rng.integers(1, 5))
        G = int(rng.choice([g for g in (1, 2, 3, 4, 8, 16, 32, 64) if g * Hkv <= 128]))
        B = int(rng.integers(1, 6))
        top = 5000 if i % 8 == 7 else 1200
        ctx = [int(rng.integers(0, top)) if rng.random() > 0.1 else 0 for _ in range(B)]
        q = [min(c, int(rng.choice([0, 1, 1, 2, 9, 64, 200]))) for c in ctx]
        out.append(dict(seed=5000 + i, dtype="f32" if i % 6 == 5 else "bf16", Hq=Hkv * G,
                        Hkv=Hkv, D=int(rng.choice([64, 128])),
                        P=int(rng.choice([16, 32, 64, 128, 256])), ctx_len=ctx, q_len=q,
                        policy=[_policy(rng) for _ in range(Hkv)]))
    return out


@pytest.mark.parametrize("args", _shapes(), ids=lambda a: "seed%d" % a["seed"])
def test_random_layout_sweep(args):
    a = dict(args)
    seed = a.pop("seed")
    c = custom_case(seed, **a)
    print("case sweep", seed, a, flush=True)
    retrieval = bool((c.policy[:, 0] == RETRIEVAL).any())
    imp = importance_scores(c, levels=3 if seed % 2 else 0) if retrieval else None
    layer = SegPagedLayer(c.dtype, c.Hq, c.Hkv, c.D, c.P, c.ctx_len, c.q_len, c.policy, DEV)
    layer.build(to_device(c.k, c.dtype), to_device(c.v, c.dtype), free_list(seed, layer.n_virt),
                importance=head_major(imp))
    out = layer.attention(to_device(c.q, c.dtype), c.scale)
    torch.cuda.synchronize()
    assert layer.check() == 0
    seg_o, kvl_o, n_virt = oracle.plan_tables(c.ctx_len, c.q_len, c.policy, c.P)
    assert layer.n_virt == n_virt
    np.testing.assert_array_equal(layer.seg_table.cpu().numpy()[:c.B], seg_o)
    np.testing.assert_array_equal(layer.kv_len.cpu().numpy()[:c.B], kvl_o)
    if c.tq_total:
        ref = oracle.attention(c.q, c.k, c.v, c.ctx_len, c.q_len, c.policy, c.Hq, c.Hkv,
                               c.scale, c.dtype, importance=imp)
        assert_parity(to_f64(out), ref, c, "sweep")


def _layer_shapes(n=24, seed=4141):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(rng.integers(1, 4))
        G = int(rng.choice([1, 4, 8, 32]))
        B = int(rng.integers(1, 4))
        ctx = [int(rng.integers(0, 1500)) for _ in range(B)]
        q = [min(c, int(rng.choice([0, 1, 7, 90]))) for c in ctx]
        layers = int(rng.integers(2, 6))
        # several layers take no importance, so their heads are GLOBAL, LOCAL or adaptive
        pols = [[_policy(rng) for _ in range(Hkv)] for _ in range(layers)]
        pols = [[p if p[0] != RETRIEVAL else (LOCAL, 4, 64) for p in pol] for pol in pols]
        out.append(dict(seed=6000 + i, dtype="f32" if i % 6 == 5 else "bf16", Hq=Hkv * G,
                        Hkv=Hkv, D=int(rng.choice([64, 128])),
                        P=int(rng.choice([16, 64, 256])), ctx_len=ctx, q_len=q, policies=pols))
    return out


@pytest.mark.parametrize("args", _layer_shapes(), ids=lambda a: "seed%d" % a["seed"])
def test_random_layers_sweep(args):
    # several layers of random policies built by one call into one pool: tables equal the
    # oracle's multi-layer tables and attention on every layer matches the oracle
    from head_aware_paged_segpaged_amd import SegPagedLayers
    a = dict(args)
    seed, pols = a.pop("seed"), a.pop("policies")
    cases = [custom_case(seed + 100 * l, policy=pol, **a) for l, pol in enumerate(pols)]
    c0 = cases[0]
    print("case layers sweep", seed, len(pols), a, flush=True)
    m = SegPagedLayers(c0.dtype, len(cases), c0.Hq, c0.Hkv, c0.D, c0.P, c0.ctx_len, c0.q_len,
                       pols, DEV)
    stack = lambda xs: torch.stack([to_device(x, c0.dtype) for x in xs])
    n_phys = m.n_virt + 3
    m.build(stack([c.k for c in cases]), stack([c.v for c in cases]),
            free_list(seed, n_phys), n_phys=n_phys)
    torch.cuda.synchronize()
    seg_o, kvl_o, n_virt = oracle.plan_tables_layers(c0.ctx_len, c0.q_len, pols, c0.P)
    assert m.n_virt == n_virt
    np.testing.assert_array_equal(m.seg_table.cpu().numpy(), seg_o)
    np.testing.assert_array_equal(m.kv_len.cpu().numpy(), kvl_o)
    for layer, c in enumerate(cases):
        out = m.attention(layer, to_device(c.q, c.dtype), c.scale)
        torch.cuda.synchronize()
        assert m.check(layer) == 0
        if c.tq_total:
            ref = oracle.attention(c.q, c.k, c.v, c.ctx_len, c.q_len, c.policy, c.Hq, c.Hkv,
                                   c.scale, c.dtype)
            assert_parity(to_f64(out), ref, c, "layer %d" % layer)
