"""Seeded input generators (shapes, value distributions, head mixes).

Recipe, identical for every consumer:

* ``meta`` stream  = ``default_rng(SeedSequence(seed, spawn_key=(0,)))``. It draws, in this
  order, the per-request context lengths (when the workload draws them) and then the set of
  GLOBAL KV heads (``choice(Hkv, n, replace=False)``, sorted), when that set is drawn.
* Tensor ``t`` (1 = Q, 2 = K, 3 = V) is filled in chunks of ``CHUNK`` elements; chunk ``i``
  comes from ``default_rng(SeedSequence(seed, spawn_key=(t, i))).standard_normal`` in float32,
  times the workload's standard deviation, then rounded to nearest-even bfloat16 for bf16
  workloads (kept as float32 otherwise). Chunks are independent, so they are drawn on a
  thread pool and the result does not depend on the thread count.
* The free list of physical pages is ``default_rng(SeedSequence(seed, spawn_key=(4,)))
  .permutation(n_phys)``; the caller passes ``n_phys``.

Layouts (token-major, requests concatenated): Q ``[sum(q_len), Hq, D]``, dense K and V
``[sum(ctx_len), Hkv, D]``. bf16 tensors are returned as their uint16 bit patterns.

The workloads mirror the sizes, head counts and GLOBAL/LOCAL mixes that the RedKnot pages
describe for SegPagedAttention (page "RedKnot SegPagedAttention runtime design", sections 2-5;
page "RedKnot head classification", the published head configurations: about 15% GLOBAL heads
with a LOCAL window of 8192 and sink 4 for the 70B layer, GLOBAL heads 0, 8, ..., 56 with
window 128 for the 64-head layer, and the defaults window 512 / sink 4). The pages' own
datasets and weights are not available; Gaussian values of the stated shapes stand in.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

GLOBAL = 0
LOCAL = 1
LOCAL_ADAPTIVE = 2  # LOCAL with window = context length // divisor
RETRIEVAL = 3  # top fraction (window / 1000) of the prefix by importance, sink and chunk

CHUNK = 1 << 22


@dataclass
class Case:
    name: str
    dtype: str  # "bf16" or "f32"
    B: int
    Hq: int
    Hkv: int
    D: int
    P: int
    ctx_len: np.ndarray  # int32 [B]
    q_len: np.ndarray  # int32 [B]
    policy: np.ndarray  # int32 [Hkv, 3] = (kind, sink, window)
    scale: float
    seed: int
    q: np.ndarray = field(repr=False, default=None)  # [sum q_len, Hq, D] uint16 bits or float32
    k: np.ndarray = field(repr=False, default=None)  # [sum ctx_len, Hkv, D]
    v: np.ndarray = field(repr=False, default=None)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def t_total(self) -> int:
        return int(self.ctx_len.sum())

    @property
    def tq_total(self) -> int:
        return int(self.q_len.sum())


# The workloads. "draw_L" / "draw_global" say how the meta stream is used.
CONFIGS = [
    dict(name="tiny_fp32_L512", dtype="f32", Hq=8, Hkv=4, D=64, P=16, B=1,
         L=("fixed", [512]), q=("fixed", 64), globals=("fixed", [0]),
         sink=4, window=64, q_std=1.0, kv_std=1.0),
    dict(name="llama3_8b_layer_prefill512_of_8k", dtype="bf16", Hq=32, Hkv=8, D=128, P=64, B=1,
         L=("fixed", [8192]), q=("fixed", 512), globals=("draw", 2),
         sink=4, window=512, q_std=1.0 / math.sqrt(128), kv_std=1.0),
    dict(name="llama3.3_70b_layer_b4_prefill2048_of_16k_32k", dtype="bf16", Hq=64, Hkv=8, D=128,
         P=64, B=4, L=("uniform_int", 16384, 32768), q=("fixed", 2048), globals=("draw", 1),
         sink=4, window=8192, q_std=1.0 / math.sqrt(128), kv_std=1.0),
    dict(name="qwen3_32b_decode_b64_4k_128k", dtype="bf16", Hq=64, Hkv=8, D=128, P=64, B=64,
         L=("log_uniform", 4096, 131072), q=("fixed", 1), globals=("draw", 2),
         sink=4, window=512, q_std=1.0 / math.sqrt(128), kv_std=1.0),
    dict(name="mha64_128k_prefill4096", dtype="bf16", Hq=64, Hkv=64, D=128, P=64, B=1,
         L=("fixed", [131072]), q=("fixed", 4096), globals=("fixed", list(range(0, 64, 8))),
         sink=4, window=128, q_std=1.0 / math.sqrt(128), kv_std=1.0),
    # The long-context slice of the decode workload: every request at 32K-128K.
    dict(name="qwen3_32b_decode_b64_32k_128k", dtype="bf16", Hq=64, Hkv=8, D=128, P=64, B=64,
         L=("log_uniform", 32768, 131072), q=("fixed", 1), globals=("draw", 2),
         sink=4, window=512, q_std=1.0 / math.sqrt(128), kv_std=1.0),
    # The decode workload with LOCAL windows that follow each request's context, at half of
    # it (the head classification page's example): `window` is then the divisor.
    dict(name="qwen3_32b_decode_b64_4k_128k_half_window", dtype="bf16", Hq=64, Hkv=8, D=128,
         P=64, B=64, L=("log_uniform", 4096, 131072), q=("fixed", 1), globals=("draw", 2),
         sink=4, window=2, local_kind=LOCAL_ADAPTIVE, q_std=1.0 / math.sqrt(128), kv_std=1.0),
    # The decode workload (same seed: same lengths, GLOBAL heads and tensors) with its first
    # two LOCAL heads turned into RETRIEVAL heads that keep sink 4 and the top 10 % of their
    # prefix by importance (``importance_scores``).
    dict(name="qwen3_32b_decode_b64_4k_128k_retrieval", dtype="bf16", Hq=64, Hkv=8, D=128,
         P=64, B=64, L=("log_uniform", 4096, 131072), q=("fixed", 1), globals=("draw", 2),
         sink=4, window=512, retrieval=(2, 100), seed=4, q_std=1.0 / math.sqrt(128),
         kv_std=1.0),
]


def _meta_rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(0,)))


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill_normal(seed: int, tensor_id: int, n: int, std: float) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    n_chunks = (n + CHUNK - 1) // CHUNK

    def one(i: int) -> None:
        lo = i * CHUNK
        hi = min(n, lo + CHUNK)
        g = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tensor_id, i)))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if std != 1.0:
            out[lo:hi] *= np.float32(std)

    if n_chunks <= 1:
        for i in range(n_chunks):
            one(i)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(one, range(n_chunks)))
    return out


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to nearest-even bfloat16 and return the uint16 bit patterns."""
    import torch

    t = torch.from_numpy(x).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _draw_tensor(seed: int, tensor_id: int, shape, std: float, dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    x = _fill_normal(seed, tensor_id, n, std)
    if dtype == "bf16":
        x = _to_bf16_bits(x)
    return x.reshape(shape)


def _policy_table(Hkv: int, global_heads, sink: int, window: int,
                  local_kind: int = LOCAL) -> np.ndarray:
    pol = np.empty((Hkv, 3), dtype=np.int32)
    pol[:, 0] = local_kind
    pol[:, 1] = sink
    pol[:, 2] = window
    for h in global_heads:
        pol[h, 0] = GLOBAL
    return pol


def config_case(index: int, seed: int | None = None, with_tensors: bool = True) -> Case:
    """Workload ``index`` (0-based into ``CONFIGS``); the seed defaults to ``index + 1``."""
    cfg = CONFIGS[index]
    seed = cfg.get("seed", index + 1) if seed is None else seed
    rng = _meta_rng(seed)
    B = cfg["B"]
    kind = cfg["L"][0]
    if kind == "fixed":
        ctx = np.asarray(cfg["L"][1], dtype=np.int64)
    elif kind == "uniform_int":
        ctx = rng.integers(cfg["L"][1], cfg["L"][2] + 1, size=B)
    elif kind == "log_uniform":
        u = rng.uniform(math.log(cfg["L"][1]), math.log(cfg["L"][2]), size=B)
        ctx = np.floor(np.exp(u)).astype(np.int64)
    else:  # pragma: no cover
        raise ValueError(kind)
    ctx = ctx.astype(np.int32)
    q = np.full(B, cfg["q"][1], dtype=np.int32)
    gk, gv = cfg["globals"]
    if gk == "fixed":
        ghs = list(gv)
    else:
        ghs = sorted(int(h) for h in rng.choice(cfg["Hkv"], gv, replace=False))
    pol = _policy_table(cfg["Hkv"], ghs, cfg["sink"], cfg["window"], cfg.get("local_kind", LOCAL))
    if "retrieval" in cfg:
        n_r, permille = cfg["retrieval"]
        for h in [h for h in range(cfg["Hkv"]) if pol[h, 0] != GLOBAL][:n_r]:
            pol[h] = (RETRIEVAL, cfg["sink"], permille)
    case = Case(name=cfg["name"], dtype=cfg["dtype"], B=B, Hq=cfg["Hq"], Hkv=cfg["Hkv"],
                D=cfg["D"], P=cfg["P"], ctx_len=ctx, q_len=q, policy=pol,
                scale=1.0 / math.sqrt(cfg["D"]), seed=seed)
    if with_tensors:
        _attach_tensors(case, cfg["q_std"], cfg["kv_std"])
    return case


def custom_case(seed: int, *, dtype: str, Hq: int, Hkv: int, D: int, P: int, ctx_len, q_len,
                policy, scale: float | None = None, q_std: float = 1.0, kv_std: float = 1.0,
                name: str = "custom") -> Case:
    """A small case with explicit lengths and policy table (used by the tests)."""
    ctx = np.asarray(ctx_len, dtype=np.int32)
    q = np.asarray(q_len, dtype=np.int32)
    pol = np.asarray(policy, dtype=np.int32).reshape(Hkv, 3)
    case = Case(name=name, dtype=dtype, B=len(ctx), Hq=Hq, Hkv=Hkv, D=D, P=P, ctx_len=ctx,
                q_len=q, policy=pol, scale=(1.0 / math.sqrt(D)) if scale is None else scale,
                seed=seed)
    _attach_tensors(case, q_std, kv_std)
    return case


def _attach_tensors(case: Case, q_std: float, kv_std: float) -> None:
    case.q = _draw_tensor(case.seed, 1, (case.tq_total, case.Hq, case.D), q_std, case.dtype)
    case.k = _draw_tensor(case.seed, 2, (case.t_total, case.Hkv, case.D), kv_std, case.dtype)
    case.v = _draw_tensor(case.seed, 3, (case.t_total, case.Hkv, case.D), kv_std, case.dtype)


def decode_tokens(case: Case, n_steps: int, q_std: float | None = None,
                  kv_std: float = 1.0):
    """Seeded inputs of n_steps decode steps after ``case``'s context: the new token's K and V
    rows [n_steps, B, Hkv, D] and the step's queries [n_steps, B, Hq, D] (same dtype and
    distributions as the workload's own tensors; tensor ids 5-7 of the case's seed)."""
    if q_std is None:
        q_std = 1.0 / math.sqrt(128) if case.dtype == "bf16" else 1.0
    kv_shape = (n_steps, case.B, case.Hkv, case.D)
    k = _draw_tensor(case.seed, 5, kv_shape, kv_std, case.dtype)
    v = _draw_tensor(case.seed, 6, kv_shape, kv_std, case.dtype)
    q = _draw_tensor(case.seed, 7, (n_steps, case.B, case.Hq, case.D), q_std, case.dtype)
    return k, v, q


def importance_scores(case: Case, levels: int = 0) -> np.ndarray:
    """Seeded per-(token, KV head) importance, float32 [sum(ctx_len), Hkv], for RETRIEVAL
    heads: exp of a standard normal (a heavy right tail: a few tokens matter much more than the
    rest). levels > 0 rounds the draws to that many distinct values, so that ties occur."""
    x = _fill_normal(case.seed, 8, case.t_total * case.Hkv, 1.0)
    if levels > 0:
        x = np.floor((np.clip(x, -3.0, 3.0) + 3.0) / 6.0 * (levels - 1) + 0.5).astype(np.float32)
        return x.reshape(case.t_total, case.Hkv)
    return np.exp(x).astype(np.float32).reshape(case.t_total, case.Hkv)


def free_list(seed: int, n_phys: int) -> np.ndarray:
    """Seeded permutation of the physical page ids ``0 .. n_phys-1`` (int32)."""
    g = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(4,)))
    return g.permutation(n_phys).astype(np.int32)
