"""Comparison helpers for the GPU parity tests (test infrastructure).

Index sets: let s_(k) >= s_(k+1) be the k-th and (k+1)-th largest oracle
scores and tau their midpoint.  Indices with |s - tau| <= 1e-6 are ambiguous
(their order can flip under rounding); the GPU set must have k members and
agree with the oracle set outside the ambiguous ones.  Outputs are compared
against the oracle run with the GPU's own sets, so an ambiguous flip cannot
fail the float check.
"""

import concurrent.futures
import os

import numpy as np
import torch

BAND = 1e-6
BF16_MAXABS = 2e-2
BF16_RELL2 = 1e-2
F32_MAXABS = 1e-4


def device_tensor(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def check_set(gpu, scores, k, band=BAND):
    """Returns the number of ambiguous indices; asserts agreement elsewhere."""
    gpu = [int(x) for x in gpu]
    n = len(scores)
    assert len(gpu) == k, (len(gpu), k)
    assert gpu == sorted(gpu) and len(set(gpu)) == k
    if k == 0 or k == n:
        assert gpu == list(range(n)) if k == n else gpu == []
        return 0
    order = sorted(range(n), key=lambda j: (-float(scores[j]), j))
    ref = set(order[:k])
    s = np.sort(np.asarray(scores, dtype=np.float64))[::-1]
    tau = 0.5 * (s[k - 1] + s[k])
    amb = {j for j in range(n) if abs(float(scores[j]) - tau) <= band}
    assert set(gpu) - amb == ref - amb, (sorted(set(gpu) ^ ref), sorted(amb))
    return len(amb)


def out_errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    maxabs = float(np.max(np.abs(got - ref))) if got.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)) if got.size else 0.0
    return maxabs, rel


def assert_output(got, ref, dtype):
    maxabs, rel = out_errors(got, ref)
    if dtype == "bf16":
        assert maxabs <= BF16_MAXABS and rel <= BF16_RELL2, (maxabs, rel)
    else:
        assert maxabs <= F32_MAXABS and rel <= BF16_RELL2, (maxabs, rel)
    return maxabs, rel


def host_workers():
    """Worker threads for oracle work: the host cores visible to this
    process, at most 16 (the host share of one GPU)."""
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def run_parallel(fn, jobs, workers=None):
    """[fn(j) for j in jobs] on a thread pool with one BLAS thread per
    worker (NumPy releases the GIL inside its array kernels)."""
    from threadpoolctl import threadpool_limits
    workers = workers or host_workers()
    with threadpool_limits(limits=1):
        if workers == 1 or len(jobs) <= 1:
            return [fn(j) for j in jobs]
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(fn, jobs))
