"""CPU tests of the C ABI: the library loads, exports every declared call, its host planner
matches the page-plan oracle bit-exactly, and invalid calls return their status codes before
anything touches a GPU."""

import os
import re

import numpy as np
import pytest

import head_aware_paged_segpaged_amd as sp
from head_aware_paged_segpaged_amd import binding
from oracle import plan_tables
from workloads import CONFIGS, config_case

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "segpaged.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(segpaged_\w+)\s*\(", text)))


def test_library_exports_every_declared_call():
    lib = sp.lib()
    declared = _declared()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(binding.EXPORTED) == declared


def test_status_strings():
    for code in range(-7, 1):
        assert sp.status_string(code)
    assert "unknown" in sp.status_string(42)


@pytest.mark.parametrize("index", range(len(CONFIGS)))
def test_layout_tables_match_oracle(index):
    c = config_case(index, with_tensors=False)
    seg, kvl = sp.segpaged_layout_tables(c.ctx_len, c.q_len, c.policy, c.P)
    seg_o, kvl_o, n_virt = plan_tables(c.ctx_len, c.q_len, c.policy, c.P)
    np.testing.assert_array_equal(seg, seg_o)
    np.testing.assert_array_equal(kvl, kvl_o)
    assert sp.segpaged_plan_pages(c.ctx_len, c.q_len, c.policy, c.P) == n_virt


def test_layout_tables_random_against_oracle():
    rng = np.random.default_rng(3)
    for _ in range(200):
        B = int(rng.integers(1, 4))
        Hkv = int(rng.integers(1, 4))
        P = int(rng.choice([16, 32, 64, 128, 256]))
        ctx = rng.integers(0, 700, size=B)
        q = np.array([rng.integers(0, c + 1) for c in ctx])
        pol = []
        for _ in range(Hkv):
            kind = int(rng.integers(0, 3))  # GLOBAL, LOCAL, LOCAL_ADAPTIVE (window = divisor)
            pol.append((kind, int(rng.integers(0, 70)),
                        int(rng.integers(1, 9 if kind == 2 else 600))))
        seg, kvl = sp.segpaged_layout_tables(ctx, q, pol, P)
        seg_o, kvl_o, n_virt = plan_tables(ctx, q, pol, P)
        np.testing.assert_array_equal(seg, seg_o)
        np.testing.assert_array_equal(kvl, kvl_o)
        assert sp.segpaged_plan_pages(ctx, q, pol, P) == n_virt


def _err(fn, *a):
    with pytest.raises(sp.SegPagedError) as e:
        fn(*a)
    return e.value.status


def test_invalid_arguments_are_rejected_on_the_host():
    pol = [(1, 4, 64)]
    E = binding
    assert _err(sp.segpaged_plan_pages, [10], [11], pol, 16) == E.SP_ERR_INVALID_ARG  # q > L
    assert _err(sp.segpaged_plan_pages, [10], [-1], pol, 16) == E.SP_ERR_INVALID_ARG
    assert _err(sp.segpaged_plan_pages, [10], [1], [(1, -1, 4)], 16) == E.SP_ERR_INVALID_ARG
    assert _err(sp.segpaged_plan_pages, [10], [1], [(1, 2, 0)], 16) == E.SP_ERR_INVALID_ARG
    assert _err(sp.segpaged_plan_pages, [10], [1], [(7, 2, 3)], 16) == E.SP_ERR_INVALID_ARG
    assert _err(sp.segpaged_plan_pages, [10], [1], [(2, 2, 0)], 16) == E.SP_ERR_INVALID_ARG
    assert _err(sp.segpaged_plan_pages, [10], [1], [(2, -1, 2)], 16) == E.SP_ERR_INVALID_ARG
    assert _err(sp.segpaged_plan_pages, [10], [1], [(4, 2, 2)], 16) == E.SP_ERR_INVALID_ARG
    assert _err(sp.segpaged_plan_pages, [10], [1], [(3, 2, 1001)], 16) == E.SP_ERR_INVALID_ARG
    assert _err(sp.segpaged_plan_pages, [10], [1], [(3, 2, 0)], 16) == E.SP_ERR_INVALID_ARG
    assert _err(sp.segpaged_plan_pages, [10], [1], pol, 48) == E.SP_ERR_UNSUPPORTED
    assert _err(sp.segpaged_plan_pages, [10], [1], pol, 8) == E.SP_ERR_UNSUPPORTED
    # attention shape checks run before any device query
    for bad in [dict(D=96), dict(Hq=6, Hkv=4), dict(dtype=7)]:
        args = dict(dtype="bf16", Hq=8, Hkv=4, D=128)
        args.update(bad)
        dtype = args["dtype"]
        code = binding.lib().segpaged_attention_workspace_size(
            dtype if isinstance(dtype, int) else 0, 1, args["Hq"], args["Hkv"], args["D"], 64,
            binding._ptr(np.array([10], np.int32)), binding._ptr(np.array([1], np.int32)),
            binding._ptr(np.array([(1, 4, 64)] * args["Hkv"], np.int32)),
            binding.ctypes.byref(binding._sz(0)))
        assert code in (E.SP_ERR_UNSUPPORTED, E.SP_ERR_INVALID_ARG), bad
    assert (binding.lib().segpaged_attention_workspace_size(0, 1, 8, 4, 128, 64, None, None,
                                                             None, None)
            == E.SP_ERR_INVALID_ARG)


def test_small_page_prefill_pool_limit_is_checked_on_the_host():
    # pages of 16 tokens, a prefill request, and a pool of 2^20 pages x 16 x 128 x 2 B = 4 GiB:
    # rejected before any device call (the pointers are never dereferenced)
    fake = binding.ctypes.c_void_p(0x10000)
    c, q = np.array([1000], np.int32), np.array([100], np.int32)
    pol = np.array([(0, 0, 1)], np.int32)
    code = binding.lib().segpaged_attention(
        0, 1, 8, 1, 128, 16, binding._ptr(c), binding._ptr(q), binding._ptr(pol), fake, fake,
        fake, 1 << 20, fake, fake, fake, binding.ctypes.c_float(0.1), fake, fake, 1 << 20, None)
    assert code == binding.SP_ERR_UNSUPPORTED


def test_build_validates_free_list_before_touching_memory():
    ctx, q, pol = np.array([100], np.int32), np.array([10], np.int32), [(0, 0, 1)]
    n_virt = sp.segpaged_plan_pages(ctx, q, pol, 16)
    assert n_virt == 7
    lib = binding.lib()
    c, ql, p = ctx, q, np.array(pol, np.int32)
    fake = binding._vp(0x1000)  # never dereferenced: validation fails first

    def build(free, n_free, n_phys):
        fl = np.asarray(free, np.int32)
        return lib.segpaged_build(0, 1, 1, 128, 16, binding._ptr(c), binding._ptr(ql),
                                  binding._ptr(p), fake, fake, binding._ptr(fl), n_free, n_phys,
                                  fake, fake, fake, fake, fake, None)

    assert build(np.arange(6), 6, 6) == binding.SP_ERR_POOL_TOO_SMALL
    assert build([0, 1, 2, 3, 4, 5, 5], 7, 8) == binding.SP_ERR_INVALID_ARG  # duplicate
    assert build([0, 1, 2, 3, 4, 5, 9], 7, 8) == binding.SP_ERR_INVALID_ARG  # out of range
    assert build([0, 1, 2, 3, 4, 5, -1], 7, 8) == binding.SP_ERR_INVALID_ARG
    assert lib.segpaged_build(0, 1, 1, 96, 16, binding._ptr(c), binding._ptr(ql),
                              binding._ptr(p), fake, fake, None, 0, 0, fake, fake, fake, fake,
                              fake, None) == binding.SP_ERR_UNSUPPORTED


def test_layers_layout_tables_match_oracle():
    # The multi-layer layout (one pool, pages numbered by request, layer, head, segment) from
    # the library's host code, against the oracle's tables.
    from oracle import plan_tables_layers
    rng = np.random.default_rng(21)
    for _ in range(60):
        n_layers, B, Hkv = int(rng.integers(1, 5)), int(rng.integers(1, 4)), int(rng.integers(1, 4))
        P = int(rng.choice([16, 64, 256]))
        ctx = rng.integers(0, 900, size=B)
        q = np.array([rng.integers(0, c + 1) for c in ctx])
        pol = np.array([[(int(rng.integers(0, 3)), int(rng.integers(0, 30)),
                          int(rng.integers(1, 5)) if rng.random() < 0.3 else int(rng.integers(1, 500)))
                         for _ in range(Hkv)] for _ in range(n_layers)], dtype=np.int32)
        pol[pol[:, :, 0] == 2, 2] = np.minimum(pol[pol[:, :, 0] == 2, 2], 8)  # adaptive: divisor
        seg, kvl = sp.segpaged_layout_tables_layers(ctx, q, pol, P)
        seg_o, kvl_o, n_virt = plan_tables_layers(ctx, q, pol, P)
        np.testing.assert_array_equal(seg, seg_o)
        np.testing.assert_array_equal(kvl, kvl_o)
        assert sp.segpaged_plan_pages_layers(ctx, q, pol, P) == n_virt


def test_layers_invalid_arguments():
    lib = binding.lib()
    c = np.array([10], np.int32)
    q = np.array([1], np.int32)
    pol = np.array([(1, 4, 64)], np.int32)
    out = binding._i64(0)
    assert lib.segpaged_plan_pages_layers(0, 1, binding._ptr(c), binding._ptr(q), 1,
                                          binding._ptr(pol), 16,
                                          binding.ctypes.byref(out)) == binding.SP_ERR_INVALID_ARG
    with pytest.raises(sp.SegPagedError):  # second layer's policy invalid
        sp.segpaged_plan_pages_layers([10], [1], [[(1, 4, 64)], [(1, 4, 0)]], 16)


def test_growable_layout_tables_match_oracle():
    # The growable layout (segments own pages for a reserve of decode tokens) from the library's
    # host code, against the oracle's tables; reserve 0 gives the build layout.
    from oracle import grow_tables
    rng = np.random.default_rng(31)
    for _ in range(300):
        B, Hkv = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        P = int(rng.choice([16, 32, 64, 128, 256]))
        ctx = rng.integers(1, 1500, size=B)
        q = np.array([rng.integers(1, c + 1) if rng.random() < 0.5 else 1 for c in ctx])
        reserve = rng.integers(0, 2000, size=B) * (rng.random(B) < 0.8)
        pol = [(0, 0, 1) if rng.random() < 0.3 else
               (3, int(rng.integers(0, 30)), int(rng.integers(1, 1001))) if rng.random() < 0.3
               else (1, int(rng.integers(0, 300)), int(rng.integers(1, 1200)))
               for _ in range(Hkv)]
        seg, kvl = sp.segpaged_layout_tables_growable(ctx, q, reserve, pol, P)
        seg_o, kvl_o, n_virt = grow_tables(ctx, q, reserve, pol, P)
        np.testing.assert_array_equal(seg, seg_o)
        np.testing.assert_array_equal(kvl, kvl_o)
        assert sp.segpaged_plan_pages_growable(ctx, q, reserve, pol, P) == n_virt
        seg0, _ = sp.segpaged_layout_tables_growable(ctx, q, np.zeros(B), pol, P)
        np.testing.assert_array_equal(seg0, sp.segpaged_layout_tables(ctx, q, pol, P)[0])


def test_growable_and_append_invalid_arguments():
    with pytest.raises(sp.SegPagedError) as e:  # context-adaptive heads do not grow
        sp.segpaged_plan_pages_growable([100], [1], [10], [(2, 4, 2)], 64)
    assert e.value.status == binding.SP_ERR_UNSUPPORTED
    for ctx, res in (([100], [-1]), ([0], [5])):
        with pytest.raises(sp.SegPagedError) as e:
            sp.segpaged_plan_pages_growable(ctx, [0] if ctx == [0] else [1], res,
                                            [(0, 0, 1)], 64)
        assert e.value.status == binding.SP_ERR_INVALID_ARG
    with pytest.raises(sp.SegPagedError) as e:
        sp.segpaged_plan_pages_growable([2 ** 31 - 10], [1], [100], [(0, 0, 1)], 64)
    assert e.value.status == binding.SP_ERR_UNSUPPORTED
    lib = binding.lib()
    fake = binding._vp(256)
    pol = np.array([(1, 4, 64)], np.int32)
    args = lambda p, hkv: (0, 2, hkv, 128, 64, binding._ptr(p), None, fake, fake, fake, fake,
                           10, fake, fake, fake, 10, fake, None)
    assert lib.segpaged_append(*args(np.array([(2, 4, 2)], np.int32), 1)) == \
        binding.SP_ERR_UNSUPPORTED
    assert lib.segpaged_append(*args(np.array([(1, 4, 0)], np.int32), 1)) == \
        binding.SP_ERR_INVALID_ARG
    assert lib.segpaged_append(*args(np.tile(pol, (129, 1)), 129)) == binding.SP_ERR_UNSUPPORTED
    bad = list(args(pol, 1))
    bad[7] = None  # k_new
    assert lib.segpaged_append(*bad) == binding.SP_ERR_INVALID_ARG
    bad = list(args(pol, 1))
    bad[15] = 0  # n_virt
    assert lib.segpaged_append(*bad) == binding.SP_ERR_INVALID_ARG


def test_retrieval_layout_tables_and_invalid_arguments():
    rng = np.random.default_rng(41)
    for _ in range(200):
        B, Hkv = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        P = int(rng.choice([16, 64, 256]))
        ctx = rng.integers(0, 900, size=B)
        q = np.array([rng.integers(0, c + 1) for c in ctx])
        pol = [(3, int(rng.integers(0, 9)), int(rng.integers(1, 1001))) if rng.random() < 0.6
               else (int(rng.integers(0, 2)), int(rng.integers(0, 9)), int(rng.integers(1, 300)))
               for _ in range(Hkv)]
        seg, kvl = sp.segpaged_layout_tables(ctx, q, pol, P)
        seg_o, kvl_o, n_virt = plan_tables(ctx, q, pol, P)
        np.testing.assert_array_equal(seg, seg_o)
        np.testing.assert_array_equal(kvl, kvl_o)
        rows = sum(seg_o[b, h, 0, 1] for b in range(B) for h in range(Hkv)
                   if pol[h][0] == 3 and ctx[b] - q[b] > 0)
        assert sp.segpaged_retrieval_rows(ctx, q, pol) == rows
    E = binding
    pol = [(3, 4, 100)]
    with pytest.raises(sp.SegPagedError) as e:  # the dense-plus-mask path cannot mask it
        sp.segpaged_dense_mask_workspace_size("bf16", 1, 1, 128, [100], [1], pol)
    assert e.value.status == E.SP_ERR_UNSUPPORTED
    with pytest.raises(sp.SegPagedError) as e:  # growing retrieval heads need a query chunk
        sp.segpaged_plan_pages_growable([100], [0], [4], pol, 64)
    assert e.value.status == E.SP_ERR_INVALID_ARG
    lib = binding.lib()
    fake = binding._vp(256)
    c, ql, p = (np.array(x, np.int32) for x in ([100], [1], pol))
    # the plain build has no importance for the kept rows; the scored build needs importance
    # (device) and row_pos when some head keeps rows, and checks that before queuing anything
    assert lib.segpaged_build(0, 1, 1, 128, 64, binding._ptr(c), binding._ptr(ql),
                              binding._ptr(p), fake, fake, binding._ptr(np.arange(4, dtype=np.int32)),
                              4, 4, fake, fake, fake, fake, fake, None) == E.SP_ERR_INVALID_ARG
    for imp, rp in ((None, fake), (fake, None)):
        assert lib.segpaged_build_scored(0, 1, 1, 128, 64, binding._ptr(c), binding._ptr(ql),
                                         None, binding._ptr(p), imp, fake, fake,
                                         binding._ptr(np.arange(4, dtype=np.int32)), 4, 4, fake,
                                         fake, fake, fake, fake, rp, None) == \
            E.SP_ERR_INVALID_ARG


def test_layers_build_rejects_retrieval_heads():
    # the several-layer build takes no importance, so layouts that keep RETRIEVAL rows are
    # rejected before anything is queued (the layout queries still describe them)
    lib = binding.lib()
    fake = binding._vp(256)
    c, ql = np.array([100], np.int32), np.array([1], np.int32)
    pol = np.array([[(3, 4, 100)], [(0, 0, 1)]], np.int32)
    n = sp.segpaged_plan_pages_layers([100], [1], pol, 64)
    fl = np.arange(n, dtype=np.int32)
    assert lib.segpaged_build_layers(0, 2, 1, 1, 128, 64, binding._ptr(c), binding._ptr(ql),
                                     binding._ptr(pol), fake, fake, binding._ptr(fl), n, n,
                                     fake, fake, fake, fake, fake, None) == \
        binding.SP_ERR_INVALID_ARG


def test_table_decode_groups_up_to_128_query_heads():
    """Groups of up to 16 query heads per KV head decode as one-wave items and larger ones (up to
    128, a prefill tile's rows) as prefill tiles; a larger group is refused on the host, before
    any GPU call."""
    pol = [(0, 0, 1)]
    for Hq in (16, 32, 64, 128):
        # accepted: the size needs the device's CU count, so without a GPU the call gets as far
        # as the HIP query
        try:
            assert sp.segpaged_decode_workspace_size("bf16", Hq, 1, 128, 64, [100, 200], pol) > 0
        except sp.SegPagedError as e:
            assert e.status == binding.SP_ERR_HIP
    with pytest.raises(sp.SegPagedError) as e:
        sp.segpaged_decode_workspace_size("bf16", 256, 1, 128, 64, [100, 200], pol)
    assert e.value.status == binding.SP_ERR_UNSUPPORTED
    lib = binding.lib()
    fake = binding._vp(256)
    p = np.array(pol, np.int32)
    st = lib.segpaged_decode(0, 2, 256, 1, 128, 64, binding._ptr(p), fake, fake, fake, 10, fake,
                             fake, fake, 0.1, fake, fake, 1 << 20, None)
    assert st == binding.SP_ERR_UNSUPPORTED
    st = lib.segpaged_decode_plan(0, 2, 256, 1, 128, 64, None, binding._ptr(p), fake, 1 << 20,
                                  None)
    assert st == binding.SP_ERR_UNSUPPORTED


def test_runtime_rejects_token_major_importance():
    """The library reads RETRIEVAL importance head-major, [Hkv][sum(ctx_len)]; the runtime
    refuses any other shape before it allocates or calls the library."""
    import torch

    from head_aware_paged_segpaged_amd import SegPagedDecoder, SegPagedLayer
    pol = [(3, 4, 100), (0, 0, 1), (1, 4, 32)]
    ctx, q = [300, 50], [20, 1]
    layer = SegPagedLayer("bf16", 6, 3, 64, 64, ctx, q, pol, "cpu")
    dec = SegPagedDecoder("bf16", 6, 3, 64, 64, ctx, q, [4, 4], pol, "cpu")
    k = torch.zeros((350, 3, 64), dtype=torch.bfloat16)
    for bad in (np.zeros((350, 3), np.float32), np.zeros((3, 349), np.float32)):
        with pytest.raises(ValueError):
            layer.build(k, k, np.arange(layer.n_virt), importance=bad)
        with pytest.raises(ValueError):
            dec.build(k, k, np.arange(dec.n_virt), importance=bad)
