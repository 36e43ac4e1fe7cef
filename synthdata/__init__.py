"""Seeded synthetic inputs for batched K-Means: points and initial centroids.

This module is shared by the tests, the benchmark and the oracle's callers. It
holds no step of the clustering method itself: it only draws Gaussian-mixture
points, picks initial centroids from them, and stores the points in the
requested element type (fp32, fp16 or bf16, each rounded to nearest-even from
fp32).

Workload shapes follow the pages:
  * the (32, 75600, 128) fp16 tensor clustered with 1000 clusters in the API
    example of "flash-kmeans and the return of exact K-Means on the GPU"
    (hysenlabs.com), section "Exact K-Means, with the assignment step written
    in Triton";
  * the B=32, N=65536, K=1024, d=128 shape whose IO breakdown is given on
    "Flash-KMeans：IO感知的精确K-Means…" (paixiangai.cn), section
    "它攻克的两大瓶颈" (the two bottlenecks);
  * the large-K (K=32768, d=128) out-of-core case of the same page, section
    "基准测试" (benchmarks), here at 1/64 of its point count so it fits one
    GPU; the pages give no distribution for it, so a Zipf-weighted mixture
    stands in to exercise hot clusters;
  * d > 512 for the split-D path (hysenlabs.com page, section "The point of
    the kernel is that the distance matrix never exists").
The pages benchmark on random tensors only, so no dataset is stood in for.

Element-type helpers:
  * ``to_storage`` rounds fp32 to the storage type (bf16 kept as uint16 bits);
  * ``to_f64`` widens stored values to float64 exactly;
  * ``to_torch`` wraps stored values as a torch tensor of the matching dtype.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

DTYPES = ("f32", "f16", "bf16")


# --------------------------------------------------------------------------
# element types
# --------------------------------------------------------------------------
def to_storage(a32: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float32 array to ``dtype`` (nearest-even); bf16 as uint16 bits."""
    a32 = np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "f32":
        return a32
    if dtype == "f16":
        return a32.astype(np.float16)
    if dtype == "bf16":
        bits = a32.view(np.uint32)
        # nearest-even on the 16 dropped bits (inputs are finite)
        bias = np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
        return ((bits + bias) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements."""
    if dtype in ("f32", "f16"):
        return np.asarray(a).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_torch(a: np.ndarray, dtype: str):
    """Host torch tensor holding the stored elements (bf16 reinterpreted)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        return t.view(torch.bfloat16)
    return t


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    name: str
    B: int
    N: int
    d: int
    K: int
    dtype: str
    max_iter: int
    tol: float
    seed: int
    x: np.ndarray          # (B, N, d) in storage type
    init: np.ndarray       # (B, K, d) in storage type (rows of x)
    labels: Optional[np.ndarray] = None   # generating mixture component (B, N)

    def x64(self) -> np.ndarray:
        return to_f64(self.x, self.dtype)

    def init64(self) -> np.ndarray:
        return to_f64(self.init, self.dtype)


# The five workload recipes: (B, N, d, K, dtype, max_iter, tol).
SHAPES = {
    "tiny_f32":      (1, 2048, 32, 16, "f32", 10, 0.0),
    "api_example":   (32, 75600, 128, 1000, "f16", 100, 1e-4),
    "io_breakdown":  (32, 65536, 128, 1024, "f16", 20, 0.0),
    "large_k_zipf":  (1, 1 << 24, 128, 32768, "f16", 10, 0.0),
    "split_d":       (8, 32768, 1024, 256, "bf16", 20, 0.0),
}
SEEDS = {"tiny_f32": 1001, "api_example": 1002, "io_breakdown": 1003,
         "large_k_zipf": 1004, "split_d": 1005}


def _workers() -> int:
    try:
        import os
        n = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        n = 4
    return max(1, min(16, n))


def make_mixture(B, N, d, K, dtype, *, n_comp, mean_std, weights=None,
                 seed, subspace_rank=None, iid=False, chunk_rows=1 << 16, out=None):
    """Gaussian-mixture points plus per-batch random-point initial centroids.

    One PCG64 stream seeded with ``seed`` draws, in order: the component means
    (all batches), the labels, then the init indices. The unit-variance noise
    of row chunk j (chunks of ``chunk_rows`` rows, batch-major) comes from its
    own stream, child j of ``SeedSequence(seed)``, so chunks can be drawn in
    parallel and the result does not depend on the thread count. ``out``, if
    given, is a (B, N, d) array of the storage type that receives the points
    (page-locked memory, say); the values do not depend on it.
    """
    import concurrent.futures as cf

    ss = np.random.SeedSequence(seed)
    rng = np.random.Generator(np.random.PCG64(ss))
    labels = None
    if iid:
        means = None
    elif subspace_rank is not None:
        r = subspace_rank
        bases = np.empty((B, d, r), dtype=np.float64)
        for b in range(B):
            q, _ = np.linalg.qr(rng.standard_normal((d, r)))
            bases[b] = q
        coeff = rng.standard_normal((B, n_comp, r)) * mean_std
        means = np.einsum("bdr,bkr->bkd", bases, coeff).astype(np.float32)
    else:
        means = (rng.standard_normal((B, n_comp, d)) * mean_std).astype(np.float32)
    if means is not None:
        if weights is None:
            labels = rng.integers(0, n_comp, size=(B, N), dtype=np.int64)
        else:
            p = np.asarray(weights, dtype=np.float64)
            p = p / p.sum()
            labels = rng.choice(n_comp, size=(B, N), p=p)
        labels = labels.astype(np.int32)
    init_idx = [rng.choice(N, size=K, replace=False) if K <= N else None for _ in range(B)]

    sdt = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]
    if out is None:
        x = np.empty((B, N, d), dtype=sdt)
    else:
        if out.shape != (B, N, d) or out.dtype != sdt:
            raise ValueError("out: wrong shape or dtype")
        x = out
    per_b = (N + chunk_rows - 1) // chunk_rows
    children = ss.spawn(B * per_b)

    def fill(j):
        b, c = divmod(j, per_b)
        n0 = c * chunk_rows
        n1 = min(N, n0 + chunk_rows)
        g = np.random.Generator(np.random.PCG64(children[j]))
        z = g.standard_normal((n1 - n0, d), dtype=np.float32)
        if means is not None:
            z += means[b][labels[b, n0:n1]]
        x[b, n0:n1] = to_storage(z, dtype)

    with cf.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(B * per_b)))
    if any(i is None for i in init_idx):
        raise ValueError("K > N: initial centroids are drawn without replacement")
    init = np.stack([x[b, init_idx[b]] for b in range(B)])
    return x, init, labels


def zipf_weights(K: int, s: float = 1.1) -> np.ndarray:
    m = np.arange(K, dtype=np.float64)
    w = (m + 1.0) ** (-s)
    return w / w.sum()


def make_workload(name: str, *, scale_n: Optional[int] = None, B: Optional[int] = None,
                  seed: Optional[int] = None) -> Workload:
    """One of the five named workloads.

    ``scale_n`` replaces N (same recipe, fewer points) and ``B`` replaces the
    batch count, for parity runs sized for the oracle.
    """
    B0, N0, d, K, dtype, max_iter, tol = SHAPES[name]
    B = B0 if B is None else B
    N = N0 if scale_n is None else scale_n
    seed = SEEDS[name] if seed is None else seed
    if name == "tiny_f32":
        rng = np.random.Generator(np.random.PCG64(seed))
        means = (rng.standard_normal((B, 16, d)) * 5.0).astype(np.float32)
        labels = rng.integers(0, 16, size=(B, N)).astype(np.int32)
        x32 = rng.standard_normal((B, N, d), dtype=np.float32)
        for b in range(B):
            x32[b] += means[b][labels[b]]
        x = to_storage(x32, dtype)
        init = x[:, :K].copy()          # the first K points
    elif name == "api_example":
        x, init, labels = make_mixture(B, N, d, K, dtype, n_comp=0, mean_std=0.0,
                                       seed=seed, iid=True)
    elif name == "io_breakdown":
        x, init, labels = make_mixture(B, N, d, K, dtype, n_comp=1024, mean_std=2.0,
                                       seed=seed)
    elif name == "large_k_zipf":
        x, init, labels = make_mixture(B, N, d, K, dtype, n_comp=32768, mean_std=3.0,
                                       weights=zipf_weights(32768), seed=seed)
    elif name == "split_d":
        x, init, labels = make_mixture(B, N, d, K, dtype, n_comp=256, mean_std=2.0,
                                       seed=seed, subspace_rank=16)
    else:
        raise KeyError(name)
    return Workload(name, B, N, d, K, dtype, max_iter, tol, seed, x, init, labels)


def random_problem(B, N, d, K, dtype, seed, *, spread=1.0, n_comp=None):
    """Small free-form problem: mixture (or i.i.d. if n_comp is None) + random-point init."""
    if n_comp is None:
        x, init, _ = make_mixture(B, N, d, K, dtype, n_comp=0, mean_std=0.0,
                                  seed=seed, iid=True)
    else:
        x, init, _ = make_mixture(B, N, d, K, dtype, n_comp=n_comp, mean_std=spread,
                                  seed=seed)
    return x, init


def zipf_ids(B: int, N: int, K: int, seed: int, s: float = 1.1) -> np.ndarray:
    """Cluster ids drawn i.i.d. from Zipf(s) over K clusters (hot-cluster update input)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.choice(K, size=(B, N), p=zipf_weights(K, s)).astype(np.int32)


def uniform_ids(B: int, N: int, K: int, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, K, size=(B, N)).astype(np.int32)
