"""The boundary as a C ABI (CPU only): tests/native/abi_c_client.c, plain C11 compiled by gcc
against include/segpaged.h and linked against libsegpaged.so, calls the host-only entry points
on seeded random layouts; its page counts and tables must equal the oracle's and its argument
checks must return the documented status codes."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from head_aware_paged_segpaged_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
LIBDIR = os.path.dirname(binding.LIB_PATH)


def _layouts(n=60, seed=777):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B, Hkv = int(rng.integers(1, 5)), int(rng.integers(1, 6))
        P = int(rng.choice([16, 32, 64, 128, 256]))
        ctx = [int(rng.integers(0, 3000)) for _ in range(B)]
        q = [int(rng.integers(0, c + 1)) if rng.random() < 0.5 else min(c, 1) for c in ctx]
        pol = []
        for _ in range(Hkv):
            k = int(rng.integers(0, 4))
            pol.append((k, int(rng.choice([0, 4, 64])),
                        int(rng.choice([1, 2, 5])) if k == 2 else
                        int(rng.choice([1, 100, 999, 1000])) if k == 3 else
                        int(rng.choice([1, 33, 64, 500]))))
        out.append((B, Hkv, P, ctx, q, pol))
    return out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_client_matches_oracle(tmp_path):
    binding.lib()  # the library must be built
    exe = str(tmp_path / "abi_c_client")
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-x", "c",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "native", "abi_c_client.c"),
           "-L", LIBDIR, "-l:libsegpaged.so", "-Wl,-rpath," + LIBDIR, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    layouts = _layouts()
    spec = []
    for B, Hkv, P, ctx, q, pol in layouts:
        spec.append("%d %d %d" % (B, Hkv, P))
        spec.append(" ".join(map(str, ctx)))
        spec.append(" ".join(map(str, q)))
        spec += ["%d %d %d" % p for p in pol]
    res = subprocess.run([exe], input="\n".join(spec) + "\n", capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-2000:]
    lines = res.stdout.splitlines()
    i = 0
    for B, Hkv, P, ctx, q, pol in layouts:
        st, n_pages, n_rows = (int(x) for x in lines[i].split())
        i += 1
        assert st == 0, (B, Hkv, P, ctx, q, pol, st)
        seg_o, kvl_o, n_virt = oracle.plan_tables(np.array(ctx), np.array(q), np.array(pol), P)
        assert n_pages == n_virt
        seg = np.array(lines[i].split(), dtype=np.int64).reshape(seg_o.shape)
        kvl = np.array(lines[i + 1].split(), dtype=np.int64).reshape(kvl_o.shape)
        i += 2
        np.testing.assert_array_equal(seg, seg_o)
        np.testing.assert_array_equal(kvl, kvl_o)
        rows = sum(int(seg_o[b, h, 0, 1]) for b in range(B) for h in range(Hkv)
                   if pol[h][0] == 3 and ctx[b] - q[b] > 0)
        assert n_rows == rows
    E = binding
    assert lines[i].split() == ["checks", str(E.SP_ERR_INVALID_ARG), str(E.SP_ERR_INVALID_ARG),
                                str(E.SP_ERR_UNSUPPORTED), str(E.SP_ERR_INVALID_ARG), "0",
                                "named"]
