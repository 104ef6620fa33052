"""Shared helpers of the GPU tests: upload seeded inputs, run the library, compare."""

from __future__ import annotations

import numpy as np
import torch

from head_aware_paged_segpaged_amd import DenseMaskLayer, SegPagedLayer
from workloads import free_list

DEV = "cuda:0"

# Parity bar: cosine per (request, query head) > 0.99998 (page "RedKnot SegPagedAttention
# runtime design", section 4); max-abs 2e-2 for bf16 and 1e-5 for fp32.
COS_MIN = 0.99998
MAXABS = {"bf16": 2e-2, "f32": 1e-5}


def to_device(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def run_segpaged(case, free=None, n_phys=None, scale=None, q_dev=None, kv_dev=None):
    layer = SegPagedLayer(case.dtype, case.Hq, case.Hkv, case.D, case.P, case.ctx_len,
                          case.q_len, case.policy, DEV)
    if free is None:
        free = free_list(case.seed, layer.n_virt if n_phys is None else n_phys)
    k, v = kv_dev if kv_dev is not None else (to_device(case.k, case.dtype),
                                              to_device(case.v, case.dtype))
    layer.build(k, v, free, n_phys=n_phys)
    q = q_dev if q_dev is not None else to_device(case.q, case.dtype)
    out = layer.attention(q, case.scale if scale is None else scale)
    torch.cuda.synchronize()
    assert layer.check() == 0, "device-side error word set"
    return out, layer


def run_dense_mask(case, scale=None):
    layer = DenseMaskLayer(case.dtype, case.Hq, case.Hkv, case.D, case.ctx_len, case.q_len,
                           case.policy, DEV)
    k, v = to_device(case.k, case.dtype), to_device(case.v, case.dtype)
    q = to_device(case.q, case.dtype)
    out = layer.attention(q, k, v, case.scale if scale is None else scale)
    torch.cuda.synchronize()
    return out


def compare(got: np.ndarray, ref: np.ndarray, q_len, Hq: int):
    """(max abs error, min cosine over (request, query head))."""
    maxabs = float(np.abs(got - ref).max()) if got.size else 0.0
    cos_min = 1.0
    q0 = 0
    for nq in np.asarray(q_len):
        nq = int(nq)
        for hq in range(Hq):
            a = got[q0:q0 + nq, hq, :].ravel()
            b = ref[q0:q0 + nq, hq, :].ravel()
            na, nb = np.linalg.norm(a), np.linalg.norm(b)
            if na == 0 and nb == 0:
                continue
            cos_min = min(cos_min, float(a @ b / (na * nb)))
        q0 += nq
    return maxabs, cos_min


def assert_parity(got: np.ndarray, ref: np.ndarray, case, label=""):
    maxabs, cos = compare(got, ref, case.q_len, case.Hq)
    print("%s %s: maxabs=%.3e min_cos=%.8f" % (case.name, label, maxabs, cos), flush=True)
    assert maxabs <= MAXABS[case.dtype], (label, maxabs)
    assert cos > COS_MIN, (label, cos)


def sample_rows(case, budget_rows: int, seed: int = 4321):
    """Seeded sample of (request, query head, token indices) for full-size checks."""
    rng = np.random.default_rng(seed)
    picks = [(b, hq, int(case.q_len[b])) for b in range(case.B) if case.q_len[b] > 0
             for hq in range(case.Hq)]
    order = rng.permutation(len(picks))
    per = max(1, budget_rows // max(1, len(picks)))
    out, rows = [], 0
    for i in order:
        if rows >= budget_rows:
            break
        b, hq, nq = picks[i]
        toks = np.arange(nq) if nq <= per else np.sort(rng.choice(nq, per, replace=False))
        out.append((b, hq, toks))
        rows += len(toks)
    return out


def boundary_tokens(nq: int, bq: int, n: int, rng) -> np.ndarray:
    """Up to n query tokens of a chunk of nq: the first and last token, the two tokens on each
    side of the first, middle and last query-block boundaries (blocks of bq tokens), then
    seeded random ones."""
    pick = {0, nq - 1}
    nb = (nq + bq - 1) // bq
    for blk in sorted({1, nb // 2, nb - 1}):
        if 0 < blk < nb:
            pick.update((blk * bq - 1, blk * bq))
    pick = {t for t in pick if 0 <= t < nq}
    rest = np.setdiff1d(np.arange(nq), np.array(sorted(pick)))
    extra = max(0, min(n - len(pick), len(rest)))
    if extra:
        pick.update(int(t) for t in rng.choice(rest, extra, replace=False))
    return np.array(sorted(pick), dtype=np.int64)


def group_parity(case, got: np.ndarray, groups, importance=None, q=None, k=None, v=None,
                 ctx_len=None, q_len=None, q_row0=None, label=""):
    """Oracle rows for every (request, KV head, tokens) in `groups` (all query heads of the
    group), computed on host threads, against the GPU output `got` [rows, Hq, D].

    Returns (max abs error, min cosine over (request, query head), number of rows); the
    cosine of a (request, query head) is taken over all of its compared rows."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    q = case.q if q is None else q
    k = case.k if k is None else k
    v = case.v if v is None else v
    ctx_len = case.ctx_len if ctx_len is None else ctx_len
    q_len = case.q_len if q_len is None else q_len
    if q_row0 is None:
        q_row0 = np.concatenate([[0], np.cumsum(q_len)[:-1]])
    G = case.Hq // case.Hkv

    def one(g):
        b, h, toks = g
        ref = oracle.attention_group_rows(q, k, v, ctx_len, q_len, case.policy, case.Hq,
                                          case.Hkv, case.scale, case.dtype, b, h, toks,
                                          importance=importance)
        res = []
        for j in range(G):
            gg = got[q_row0[b] + toks, h * G + j, :]
            err = float(np.abs(gg - ref[j]).max()) if gg.size else 0.0
            na, nb = np.linalg.norm(gg), np.linalg.norm(ref[j])
            cos = 1.0 if na == 0 and nb == 0 else float(gg.ravel() @ ref[j].ravel() / (na * nb))
            res.append((err, cos, len(toks)))
        return b, h, res

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    worst_abs, worst_cos, rows, worst_at = 0.0, 1.0, 0, None
    with ThreadPoolExecutor(workers) as ex:
        for b, h, res in ex.map(one, groups):
            for j, (err, cos, n) in enumerate(res):
                worst_abs = max(worst_abs, err)
                if cos < worst_cos:
                    worst_cos, worst_at = cos, (b, h * G + j)
                rows += n
    print("%s %s: %d rows over %d (request, query head) pairs: maxabs=%.3e min_cos=%.8f at %s"
          % (case.name, label, rows, len(groups) * G, worst_abs, worst_cos, worst_at),
          flush=True)
    return worst_abs, worst_cos, rows


def head_major(imp):
    """The library's importance layout, [Hkv][T], from the workloads' token-major [T][Hkv]."""
    return None if imp is None else np.ascontiguousarray(np.asarray(imp).T)
