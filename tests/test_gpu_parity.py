"""GPU parity of the HIP path against the CPU oracle, through the C ABI (needs gfx950).

Inputs are the seeded workloads of ``workloads``; expected values come only from ``oracle``.
Bars: page tables, lengths and the pool bit-exact; O within max-abs 2e-2 (bf16) / 1e-5 (fp32)
and cosine > 0.99998 per (request, query head).
"""

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import (COS_MIN, DEV, MAXABS, assert_parity, boundary_tokens, group_parity,
                           run_dense_mask, run_segpaged, to_device, to_f64)
from workloads import GLOBAL, LOCAL, LOCAL_ADAPTIVE, config_case, custom_case, free_list

pytestmark = pytest.mark.gpu

G_, L_, A_ = GLOBAL, LOCAL, LOCAL_ADAPTIVE


def _oracle(c, scale=None):
    return oracle.attention(c.q, c.k, c.v, c.ctx_len, c.q_len, c.policy, c.Hq, c.Hkv,
                            c.scale if scale is None else scale, c.dtype)


def test_tiny_workload_tables_pool_and_output():
    c = config_case(0)
    print("case", c.name, flush=True)
    out, layer = run_segpaged(c)
    seg_o, kvl_o, n_virt = oracle.plan_tables(c.ctx_len, c.q_len, c.policy, c.P)
    assert layer.n_virt == n_virt == 59
    np.testing.assert_array_equal(layer.seg_table.cpu().numpy(), seg_o)
    np.testing.assert_array_equal(layer.kv_len.cpu().numpy(), kvl_o)
    fl = free_list(c.seed, n_virt)
    np.testing.assert_array_equal(layer.v2p.cpu().numpy(), fl[:n_virt])
    kp = layer.k_pool.cpu().numpy()
    vp = layer.v_pool.cpu().numpy()
    for h in range(c.Hkv):
        for pos, page, slot in oracle.gather_positions(seg_o, fl, c.P, 0, h):
            np.testing.assert_array_equal(kp[page, slot], c.k[pos, h])
            np.testing.assert_array_equal(vp[page, slot], c.v[pos, h])
    assert_parity(to_f64(out), _oracle(c), c, "segpaged")


def test_llama8b_layer_full_oracle():
    c = config_case(1)
    print("case", c.name, flush=True)
    out, layer = run_segpaged(c)
    seg_o, kvl_o, n_virt = oracle.plan_tables(c.ctx_len, c.q_len, c.policy, c.P)
    np.testing.assert_array_equal(layer.seg_table.cpu().numpy(), seg_o)
    np.testing.assert_array_equal(layer.kv_len.cpu().numpy(), kvl_o)
    assert n_virt == 358
    assert_parity(to_f64(out), _oracle(c), c, "segpaged")


def _edge_cases():
    mk = custom_case
    return [
        ("multi_request", lambda: mk(21, dtype="bf16", Hq=12, Hkv=3, D=128, P=64,
                                     ctx_len=[300, 77, 1000], q_len=[300, 5, 129],
                                     policy=[(G_, 0, 1), (L_, 4, 50), (L_, 0, 20)])),
        ("decode_and_prefill_mix", lambda: mk(22, dtype="bf16", Hq=16, Hkv=2, D=128, P=64,
                                              ctx_len=[500, 64, 1000, 3, 700],
                                              q_len=[1, 2, 1, 3, 40],
                                              policy=[(L_, 4, 100), (G_, 0, 1)])),
        ("mha_d64_p32", lambda: mk(23, dtype="bf16", Hq=4, Hkv=4, D=64, P=32,
                                   ctx_len=[640], q_len=[200],
                                   policy=[(G_, 0, 1), (L_, 4, 33), (L_, 64, 64), (L_, 1, 1)])),
        ("gqa16", lambda: mk(24, dtype="bf16", Hq=32, Hkv=2, D=128, P=64, ctx_len=[900, 400],
                             q_len=[77, 400], policy=[(L_, 4, 128), (G_, 0, 1)])),
        ("gqa6_ragged", lambda: mk(25, dtype="bf16", Hq=12, Hkv=2, D=128, P=128,
                                   ctx_len=[1500], q_len=[97], policy=[(L_, 8, 300), (G_, 0, 1)])),
        ("page256_merged", lambda: mk(26, dtype="bf16", Hq=8, Hkv=2, D=128, P=256,
                                      ctx_len=[600, 50], q_len=[100, 50],
                                      policy=[(L_, 700, 3), (L_, 2, 4000)])),
        ("page16_bf16", lambda: mk(27, dtype="bf16", Hq=8, Hkv=4, D=64, P=16,
                                   ctx_len=[333, 129], q_len=[65, 1],
                                   policy=[(G_, 0, 1), (L_, 4, 64), (L_, 0, 17), (L_, 16, 5)])),
        ("empty_requests", lambda: mk(28, dtype="bf16", Hq=8, Hkv=2, D=128, P=64,
                                      ctx_len=[0, 200, 90, 0], q_len=[0, 0, 90, 0],
                                      policy=[(L_, 4, 20), (G_, 0, 1)])),
        ("fp32_multi", lambda: mk(29, dtype="f32", Hq=6, Hkv=3, D=64, P=16,
                                  ctx_len=[200, 130], q_len=[70, 1],
                                  policy=[(G_, 0, 1), (L_, 4, 40), (L_, 0, 9)])),
        ("fp32_d128", lambda: mk(30, dtype="f32", Hq=4, Hkv=2, D=128, P=64, ctx_len=[260],
                                 q_len=[130], policy=[(L_, 4, 70), (G_, 0, 1)])),
        ("decode_g16", lambda: mk(31, dtype="bf16", Hq=16, Hkv=1, D=128, P=64,
                                  ctx_len=[5000, 63, 64, 65], q_len=[1, 1, 1, 1],
                                  policy=[(L_, 4, 512)])),
        # more KV heads than one wave has lanes (the build enumerates heads 64 at a time)
        ("kv_heads_200", lambda: mk(33, dtype="bf16", Hq=200, Hkv=200, D=64, P=16,
                                    ctx_len=[150, 70, 300], q_len=[20, 1, 0],
                                    policy=[(G_, 0, 1) if h % 7 == 0 else (L_, h % 5, 1 + h % 40)
                                            for h in range(200)])),
        # 32 query heads per KV head: a 128-row tile holds 4 query positions
        ("gqa32", lambda: mk(34, dtype="bf16", Hq=64, Hkv=2, D=128, P=64, ctx_len=[700, 90],
                             q_len=[50, 9], policy=[(L_, 4, 100), (G_, 0, 1)])),
        # windows that follow each request's context length: 450, 150, 1000 and 180, 60, 400
        ("adaptive_windows", lambda: mk(32, dtype="bf16", Hq=12, Hkv=3, D=128, P=64,
                                        ctx_len=[900, 300, 2000], q_len=[100, 1, 257],
                                        policy=[(A_, 4, 2), (A_, 0, 5), (G_, 0, 1)])),
    ]


@pytest.mark.parametrize("name,make", _edge_cases(), ids=[n for n, _ in _edge_cases()])
def test_edge_cases(name, make):
    c = make()
    print("case", name, flush=True)
    out, layer = run_segpaged(c)
    seg_o, kvl_o, _ = oracle.plan_tables(c.ctx_len, c.q_len, c.policy, c.P)
    np.testing.assert_array_equal(layer.seg_table.cpu().numpy()[:c.B], seg_o)
    np.testing.assert_array_equal(layer.kv_len.cpu().numpy()[:c.B], kvl_o)
    if c.tq_total:
        assert_parity(to_f64(out), _oracle(c), c, name)


def test_sharp_softmax_scale_one():
    c = custom_case(40, dtype="bf16", Hq=8, Hkv=2, D=128, P=64, ctx_len=[700], q_len=[300],
                    policy=[(L_, 4, 64), (G_, 0, 1)], scale=1.0 / 128 ** 0.5, q_std=1.0)
    c.scale = 1.0
    print("case sharp", flush=True)
    out, _ = run_segpaged(c)
    # logits ~ N(0, 128): a few keys dominate; bf16 probabilities still hold the bar
    assert_parity(to_f64(out), _oracle(c), c, "sharp")


def test_page_permutation_and_repeat_are_bitwise_identical():
    c = config_case(1)
    print("case permutation", flush=True)
    out1, layer = run_segpaged(c)
    n = layer.n_virt
    perm2 = np.random.default_rng(99).permutation(n + 37).astype(np.int32)
    out2, _ = run_segpaged(c, free=perm2, n_phys=n + 37)
    assert torch.equal(out1, out2)
    out3 = layer.attention(to_device(c.q, c.dtype), c.scale)
    torch.cuda.synchronize()
    assert torch.equal(out1, out3)


def _bits(x):
    """Raw element bits of a device tensor or host array (bf16 has no numpy type)."""
    if isinstance(x, torch.Tensor):
        x = x.cpu()
        return (x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)).numpy()
    return x.view(np.int16) if x.dtype.itemsize == 2 else x.view(np.int32)


def _check_pool(c, seg, v2p, k_pool, v_pool):
    """Every stored (token, head) row of the pool equals its dense row, bit for bit."""
    kp, vp, kd, vd = _bits(k_pool), _bits(v_pool), _bits(c.k), _bits(c.v)
    row0 = np.concatenate([[0], np.cumsum(c.ctx_len)[:-1]])
    for b in range(c.B):
        for h in range(c.Hkv):
            g = oracle.gather_positions(seg, v2p, c.P, b, h)
            if not g:
                continue
            pos, page, slot = (np.array(t) for t in zip(*g))
            np.testing.assert_array_equal(kp[page, slot], kd[row0[b] + pos, h])
            np.testing.assert_array_equal(vp[page, slot], vd[row0[b] + pos, h])


@pytest.mark.parametrize("name", ["tiny", "page16_bf16", "multi_request", "decode_g16"])
def test_build_pool_bit_exact_with_adjacent_and_separate_tables(name):
    """The build uploads the three tables in one copy when they are adjacent (the layer's
    allocation) and in three otherwise; both give the oracle's tables and an exact pool,
    including segments that end inside a 64-token copy unit."""
    from head_aware_paged_segpaged_amd import binding
    c = config_case(0) if name == "tiny" else dict(_edge_cases())[name]()
    print("case build", name, flush=True)
    seg_o, kvl_o, n_virt = oracle.plan_tables(c.ctx_len, c.q_len, c.policy, c.P)
    _, layer = run_segpaged(c)
    np.testing.assert_array_equal(layer.seg_table.cpu().numpy(), seg_o)
    np.testing.assert_array_equal(layer.kv_len.cpu().numpy(), kvl_o)
    _check_pool(c, seg_o, layer.v2p.cpu().numpy(), layer.k_pool, layer.v_pool)
    # separate tables, another free list and a larger pool
    n_phys = n_virt + 11
    fl = np.random.default_rng(5).permutation(n_phys).astype(np.int32)
    k, v = to_device(c.k, c.dtype), to_device(c.v, c.dtype)
    kp = torch.empty((n_phys, c.P, c.D), dtype=k.dtype, device=DEV)
    vp = torch.empty_like(kp)
    seg = torch.full((c.B, c.Hkv, 2, 4), -7, dtype=torch.int32, device=DEV)
    gap = torch.empty(3, dtype=torch.int32, device=DEV)  # keeps the tables apart
    kvl = torch.full((c.B, c.Hkv), -7, dtype=torch.int32, device=DEV)
    v2p = torch.full((n_virt,), -7, dtype=torch.int32, device=DEV)
    binding.segpaged_build(c.dtype, c.D, c.P, c.ctx_len, c.q_len, c.policy, k, v, fl, n_phys,
                           kp, vp, seg, kvl, v2p)
    torch.cuda.synchronize()
    del gap
    np.testing.assert_array_equal(seg.cpu().numpy(), seg_o)
    np.testing.assert_array_equal(kvl.cpu().numpy(), kvl_o)
    np.testing.assert_array_equal(v2p.cpu().numpy(), fl[:n_virt])
    _check_pool(c, seg_o, fl, kp, vp)


@pytest.mark.parametrize("index", [0, 1])
def test_dense_mask_baseline_matches_oracle(index):
    c = config_case(index)
    print("case dense-mask", c.name, flush=True)
    out = run_dense_mask(c)
    assert_parity(to_f64(out), _oracle(c), c, "dense_mask")


def test_dense_mask_baseline_edge_cases():
    for name, make in _edge_cases()[:3]:
        c = make()
        print("case dense-mask", name, flush=True)
        out = run_dense_mask(c)
        assert_parity(to_f64(out), _oracle(c), c, "dense_mask " + name)


def test_plan_mismatch_is_reported_not_computed():
    c = config_case(0)
    out, layer = run_segpaged(c)
    other = custom_case(41, dtype="f32", Hq=8, Hkv=4, D=64, P=16, ctx_len=[500], q_len=[64],
                        policy=c.policy)
    q = to_device(other.q, other.dtype)
    o = torch.full_like(q, 7.0)
    from head_aware_paged_segpaged_amd import segpaged_attention
    segpaged_attention(other.dtype, other.Hq, other.Hkv, other.D, other.P, other.ctx_len,
                       other.q_len, other.policy, q, layer.k_pool, layer.v_pool, layer.n_phys,
                       layer.seg_table, layer.kv_len, layer.v2p, other.scale, o,
                       layer.workspace)
    torch.cuda.synchronize()
    assert layer.check() == -6  # SP_ERR_PLAN_MISMATCH
    assert bool((o == 7.0).all())


def test_decode_repeat_is_bitwise_identical():
    # Split-KV decode items merged by the combine kernel in a fixed order: every call of the
    # same inputs must give the same bits (a cross-wave LDS race would show up here).
    c = custom_case(42, dtype="bf16", Hq=64, Hkv=8, D=128, P=64,
                    ctx_len=[4100, 9000, 17000, 700, 64, 5000],
                    q_len=[1] * 6, policy=[(G_, 0, 1), (G_, 0, 1)] + [(L_, 4, 512)] * 6)
    print("case decode repeat", flush=True)
    out, layer = run_segpaged(c)
    assert_parity(to_f64(out), _oracle(c), c, "decode_repeat")
    q = to_device(c.q, c.dtype)
    for _ in range(30):
        o2 = layer.attention(q, c.scale)
        torch.cuda.synchronize()
        assert torch.equal(out, o2)
    assert layer.check() == 0


@pytest.mark.parametrize("B", [2, 24, 44])
def test_decode_launch_sizes(B):
    # The decode kernel's launch size follows the plan's item count: on a 256-CU MI355X these
    # batches plan 128, 1536 and 2112 decode items (bf16, D 128, 8 query heads per KV head), i.e.
    # one work group per SIMD with every item started at once, the full grid of two per SIMD,
    # and one per SIMD with the queues handing out the rest. Each must match the oracle, and
    # repeated calls must give the same bits.
    c = custom_case(4400 + B, dtype="bf16", Hq=64, Hkv=8, D=128, P=64, ctx_len=[4096] * B,
                    q_len=[1] * B, policy=[(G_, 0, 1)] * 8)
    print("case decode launch size", B, flush=True)
    out, layer = run_segpaged(c)
    assert_parity(to_f64(out), _oracle(c), c, "decode_launch_%d" % B)
    o2 = layer.attention(to_device(c.q, c.dtype), c.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, o2)
    assert layer.check() == 0


@pytest.mark.parametrize("index", [2, 3, 4, 5, 6])
def test_full_size_every_head(index):
    # The full workloads, planned for this device exactly as the benchmark runs them: page
    # tables bit-exact, two heads' pool pages bit-exact, and output rows of EVERY (request,
    # query head) against the oracle. Prefill workloads: 16 query tokens per (request, query
    # head), among them the chunk's first and last token and the tokens on both sides of
    # query-block boundaries, plus every row of two complete heads (a GLOBAL and a LOCAL one
    # of the longest request); decode workloads: all rows. The cosine is per (request, query
    # head) over its compared rows.
    c = config_case(index)
    print("case full-size", c.name, flush=True)
    out, layer = run_segpaged(c)
    seg_o, kvl_o, n_virt = oracle.plan_tables(c.ctx_len, c.q_len, c.policy, c.P)
    np.testing.assert_array_equal(layer.seg_table.cpu().numpy(), seg_o)
    np.testing.assert_array_equal(layer.kv_len.cpu().numpy(), kvl_o)
    assert layer.n_virt == n_virt
    fl = free_list(c.seed, n_virt)
    rng = np.random.default_rng(index)
    for _ in range(2):
        b, h = int(rng.integers(c.B)), int(rng.integers(c.Hkv))
        pos, page, slot = (np.array(x) for x in zip(*oracle.gather_positions(seg_o, fl, c.P, b, h)))
        base = int(np.sum(c.ctx_len[:b]))
        kp = layer.k_pool[torch.from_numpy(page).long().to(DEV), torch.from_numpy(slot).long().to(DEV)]
        vp = layer.v_pool[torch.from_numpy(page).long().to(DEV), torch.from_numpy(slot).long().to(DEV)]
        np.testing.assert_array_equal(kp.cpu().view(torch.int16).numpy(), c.k[base + pos, h].view(np.int16))
        np.testing.assert_array_equal(vp.cpu().view(torch.int16).numpy(), c.v[base + pos, h].view(np.int16))
    got = to_f64(out)
    G = c.Hq // c.Hkv
    bq = max(1, 128 // G)  # query tokens of one prefill work item
    groups = [(b, h, boundary_tokens(int(c.q_len[b]), bq, 16, rng))
              for b in range(c.B) for h in range(c.Hkv) if c.q_len[b] > 0]
    worst_abs, worst_cos, rows = group_parity(c, got, groups, label="every head")
    assert rows >= min(16, int(c.q_len.min())) * c.B * c.Hq
    assert worst_abs <= MAXABS[c.dtype]
    assert worst_cos > COS_MIN
    if int(c.q_len.max()) > 1:
        q_row0 = np.concatenate([[0], np.cumsum(c.q_len)[:-1]])
        b = int(np.argmax(c.ctx_len))
        for kind in (G_, L_):
            h = int(np.nonzero(c.policy[:, 0] == kind)[0][0])
            ref = oracle.attention_rows(c.q, c.k, c.v, c.ctx_len, c.q_len, c.policy, c.Hq,
                                        c.Hkv, c.scale, c.dtype, b, h * G)
            g = got[q_row0[b]:q_row0[b] + int(c.q_len[b]), h * G]
            err = float(np.abs(g - ref).max())
            cos = float(g.ravel() @ ref.ravel() / (np.linalg.norm(g) * np.linalg.norm(ref)))
            print("%s complete head (request %d, query head %d, %s): %d rows maxabs=%.3e cos=%.8f"
                  % (c.name, b, h * G, "GLOBAL" if kind == G_ else "LOCAL", len(g), err, cos),
                  flush=True)
            assert err <= MAXABS[c.dtype] and cos > COS_MIN


def _random_cases(n=16, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = "f32" if i % 5 == 4 else "bf16"
        D = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 3]))
        G = int(rng.choice([1, 2, 4, 6, 8, 16]))
        P = int(rng.choice([16, 32, 64, 128, 256]))
        B = int(rng.integers(1, 4))
        ctx = rng.integers(1, 1500, B)
        q = np.minimum(ctx, rng.choice([1, 1, 2, 5, 40, 200], B))
        pol = []
        for _ in range(Hkv):
            if rng.random() < 0.35:
                pol.append((G_, 0, 1))
            else:
                pol.append((L_, int(rng.choice([0, 1, 4, 100])), int(rng.choice([1, 17, 64, 300]))))
        out.append(dict(seed=500 + i, dtype=dtype, Hq=Hkv * G, Hkv=Hkv, D=D, P=P,
                        ctx_len=list(ctx), q_len=list(q), policy=pol))
    return out


def _adaptive_cases(n=6, seed=4048):
    """Random shapes whose LOCAL heads take windows from each request's context length."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(rng.choice([1, 2, 3]))
        G = int(rng.choice([1, 4, 8]))
        B = int(rng.integers(1, 4))
        ctx = rng.integers(1, 2500, B)
        q = np.minimum(ctx, rng.choice([1, 3, 64, 300], B))
        pol = [(A_, int(rng.choice([0, 4])), int(rng.choice([1, 2, 3, 8]))) for _ in range(Hkv)]
        if Hkv > 1:
            pol[0] = (G_, 0, 1)
        out.append(dict(seed=600 + i, dtype="f32" if i == 5 else "bf16", Hq=Hkv * G, Hkv=Hkv,
                        D=int(rng.choice([64, 128])), P=int(rng.choice([16, 64, 128])),
                        ctx_len=list(ctx), q_len=list(q), policy=pol))
    return out


def _large_group_cases(n=8, seed=8096):
    """Random shapes with 12-64 query heads per KV head (prefill tiles of 2-10 query tokens,
    decode queries as tiles), longer contexts and every page size."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([12, 24, 32, 64]))
        B = int(rng.integers(1, 4))
        ctx = rng.integers(1, 3000, B)
        q = np.minimum(ctx, rng.choice([1, 7, 60], B))
        pol = [(G_, 0, 1) if rng.random() < 0.4 else
               (L_, int(rng.choice([0, 4, 64])), int(rng.choice([1, 50, 700])))
               for _ in range(Hkv)]
        out.append(dict(seed=700 + i, dtype="f32" if i == 7 else "bf16", Hq=Hkv * G, Hkv=Hkv,
                        D=int(rng.choice([64, 128])), P=int(rng.choice([16, 32, 64, 256])),
                        ctx_len=list(ctx), q_len=list(q), policy=pol))
    return out


@pytest.mark.parametrize("args", _random_cases() + _adaptive_cases() + _large_group_cases(),
                         ids=lambda a: "seed%d" % a["seed"])
def test_random_shapes_against_oracle(args):
    # Seeded random shapes across dtypes, head dims, GQA groups, page sizes, request mixes
    # (decode and prefill together) and policies.
    a = dict(args)
    c = custom_case(a.pop("seed"), **a)
    print("case random", c.dtype, c.Hq, c.Hkv, c.D, c.P, list(c.ctx_len), list(c.q_len),
          c.policy.tolist(), flush=True)
    out, layer = run_segpaged(c)
    seg_o, kvl_o, _ = oracle.plan_tables(c.ctx_len, c.q_len, c.policy, c.P)
    np.testing.assert_array_equal(layer.seg_table.cpu().numpy()[:c.B], seg_o)
    np.testing.assert_array_equal(layer.kv_len.cpu().numpy()[:c.B], kvl_o)
    assert_parity(to_f64(out), _oracle(c), c, "random")


def test_layers_share_one_pool():
    # Three layers of one batch (different policies, one adaptive) built by one call into one
    # pool: each layer's tables equal the oracle's multi-layer tables, its stored rows equal
    # its dense rows bit for bit, and attention on each layer matches the oracle.
    from head_aware_paged_segpaged_amd import SegPagedLayers
    shapes = dict(dtype="bf16", Hq=8, Hkv=2, D=128, P=64, ctx_len=[700, 260], q_len=[90, 1])
    policies = [[(G_, 0, 1), (L_, 4, 100)], [(L_, 0, 33), (G_, 0, 1)], [(A_, 4, 3), (L_, 2, 500)]]
    cases = [custom_case(40 + i, policy=pol, **shapes) for i, pol in enumerate(policies)]
    print("case layers", len(cases), flush=True)
    c0 = cases[0]
    stack = lambda xs: torch.stack([to_device(x, c0.dtype) for x in xs])
    k_all, v_all = stack([c.k for c in cases]), stack([c.v for c in cases])
    m = SegPagedLayers(c0.dtype, len(cases), c0.Hq, c0.Hkv, c0.D, c0.P, c0.ctx_len, c0.q_len,
                       policies, DEV)
    n_phys = m.n_virt + 5
    fl = np.random.default_rng(8).permutation(n_phys).astype(np.int32)
    m.build(k_all, v_all, fl, n_phys=n_phys)
    torch.cuda.synchronize()
    seg_o, kvl_o, n_virt = oracle.plan_tables_layers(c0.ctx_len, c0.q_len, policies, c0.P)
    assert m.n_virt == n_virt
    np.testing.assert_array_equal(m.seg_table.cpu().numpy(), seg_o)
    np.testing.assert_array_equal(m.kv_len.cpu().numpy(), kvl_o)
    for layer, c in enumerate(cases):
        _check_pool(c, seg_o[layer], fl, m.k_pool, m.v_pool)
        out = m.attention(layer, to_device(c.q, c.dtype), c.scale)
        torch.cuda.synchronize()
        assert m.check(layer) == 0
        assert_parity(to_f64(out), _oracle(c), c, "layer %d" % layer)


@pytest.mark.parametrize("P", [16, 64, 256])
def test_build_many_segments_and_groups(P):
    # One build call over several layers with hundreds of segments (one scatter launch), and
    # one over 520 requests (more (layer, request) groups than one launch's arguments hold, so
    # the groups take two launches): tables equal the oracle's and every stored row of every
    # layer equals its dense row bit for bit.
    from head_aware_paged_segpaged_amd import SegPagedLayers
    rng = np.random.default_rng(900 + P)
    for n_layers, B, Hkv, lo, hi in ((5, 6, 8, 1, 3000), (1, 520, 2, 1, 200)):
        ctx = rng.integers(lo, hi, B)
        q = np.minimum(ctx, rng.choice([1, 7, 64, 300], B))
        policies = [[(G_, 0, 1) if rng.random() < 0.3 else
                     (L_, int(rng.choice([0, 4, 70])), int(rng.choice([1, 33, 200, 900])))
                     for _ in range(Hkv)] for _ in range(n_layers)]
        cases = [custom_case(1000 + 10 * P + i, dtype="bf16", Hq=Hkv, Hkv=Hkv, D=64, P=P,
                             ctx_len=list(ctx), q_len=list(q), policy=pol)
                 for i, pol in enumerate(policies)]
        c0 = cases[0]
        seg_o, kvl_o, n_virt = oracle.plan_tables_layers(c0.ctx_len, c0.q_len, policies, P)
        n_segs = int((seg_o[..., 1] > 0).sum())
        print("case build layers %d requests %d heads %d P %d: %d segments"
              % (n_layers, B, Hkv, P, n_segs), flush=True)
        assert n_segs > 128
        m = SegPagedLayers(c0.dtype, n_layers, c0.Hq, c0.Hkv, c0.D, P, c0.ctx_len, c0.q_len,
                           policies, DEV)
        stack = lambda xs: torch.stack([to_device(x, c0.dtype) for x in xs])
        n_phys = m.n_virt + 3
        fl = np.random.default_rng(P).permutation(n_phys).astype(np.int32)
        m.build(stack([c.k for c in cases]), stack([c.v for c in cases]), fl, n_phys=n_phys)
        torch.cuda.synchronize()
        assert m.n_virt == n_virt
        np.testing.assert_array_equal(m.seg_table.cpu().numpy(), seg_o)
        np.testing.assert_array_equal(m.kv_len.cpu().numpy(), kvl_o)
        for layer, c in enumerate(cases):
            _check_pool(c, seg_o[layer], fl, m.k_pool, m.v_pool)
