"""The whole path from a plain C program (needs gfx950): tests/native/abi_c_gpu_client.c, C11
compiled by gcc against include/segpaged.h and linked against libsegpaged.so and the HIP
runtime, allocates its own device memory with hipMalloc (no Python, no torch in that process),
builds, plans and runs attention on seeded inputs written here; its O is compared with the
oracle at the parity bar."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from head_aware_paged_segpaged_amd import binding
from tests.helpers import assert_parity
from workloads import GLOBAL, LOCAL, LOCAL_ADAPTIVE, custom_case

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _compile(tmp_path):
    exe = str(tmp_path / "abi_c_gpu_client")
    libdir = os.path.dirname(binding.LIB_PATH)
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-x", "c",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "native", "abi_c_gpu_client.c"),
           "-L", libdir, "-l:libsegpaged.so", "-Wl,-rpath," + libdir,
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return exe


def _raw(x, dtype):
    x = np.ascontiguousarray(x)
    return x.view(np.uint16).tobytes() if dtype == "bf16" else x.astype(np.float32).tobytes()


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("dtype,D,P", [("bf16", 128, 64), ("bf16", 64, 16), ("f32", 64, 32)])
def test_c_program_runs_the_path(tmp_path, dtype, D, P):
    binding.lib()
    exe = _compile(tmp_path)
    pol = [(GLOBAL, 0, 1), (LOCAL, 4, 90), (LOCAL_ADAPTIVE, 0, 3)]
    c = custom_case(4242 + D + P, dtype=dtype, Hq=12, Hkv=3, D=D, P=P, ctx_len=[700, 33, 1500],
                    q_len=[120, 1, 64], policy=pol)
    print("case C client", dtype, D, P, flush=True)
    inp, outp = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    with open(inp, "wb") as f:
        f.write(np.array([0 if dtype == "bf16" else 1, c.B, c.Hq, c.Hkv, c.D, c.P],
                         dtype=np.int32).tobytes())
        f.write(c.ctx_len.astype(np.int32).tobytes())
        f.write(c.q_len.astype(np.int32).tobytes())
        f.write(c.policy.astype(np.int32).tobytes())
        f.write(np.array([c.scale], dtype=np.float32).tobytes())
        f.write(_raw(c.k, dtype) + _raw(c.v, dtype) + _raw(c.q, dtype))
    res = subprocess.run([exe, inp, outp], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, res.stderr
    raw = np.fromfile(outp, dtype=np.uint16 if dtype == "bf16" else np.float32)
    if dtype == "bf16":
        got = (raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        got = raw.astype(np.float64)
    got = got.reshape(int(c.q_len.sum()), c.Hq, c.D)
    ref = oracle.attention(c.q, c.k, c.v, c.ctx_len, c.q_len, c.policy, c.Hq, c.Hkv, c.scale,
                           c.dtype)
    assert_parity(got, ref, c, "C client")
