"""The user-facing calls the pages show, over the C ABI of libfkmeans.

* ``batch_kmeans_Euclid(x, n_clusters, tol, verbose)`` returns
  ``(cluster_ids, centers, n_iter)`` for a device tensor of shape (B, N, d)
  or (N, d) ("flash-kmeans and the return of exact K-Means on the GPU",
  section on the API: the functional entry point and its README example).
* ``FlashKMeans(d, k, niter, dtype, device)`` with ``train``,
  ``fit_predict`` and ``predict`` (same page, the class interface described
  as similar to faiss/sklearn, and the multi-GPU section's example).

Everything on the path runs in the library's kernels: ``fk_lloyd`` for
training, ``fk_norms`` + ``fk_assign`` for prediction. This module only
checks arguments, picks the initial centroids (an index choice, seeded on
the host) and moves data to the device. A host tensor is copied to the
device whole; the pages' chunked host-to-device stream for data larger than
device memory is not part of this package.
"""
from __future__ import annotations

from typing import Optional, Tuple

from . import _binding as fk

_DTYPES = ("float16", "bfloat16", "float32")


def _torch():
    import torch
    return torch


def _as_batched(x, dtype=None, device=None):
    """(N,d) or (B,N,d) tensor -> contiguous (B,N,d) on the device, and whether it was 2-D."""
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        raise TypeError("x must be a torch.Tensor")
    if x.dim() not in (2, 3):
        raise ValueError(f"x must have shape (N, d) or (B, N, d), got {tuple(x.shape)}")
    flat = x.dim() == 2
    if flat:
        x = x.unsqueeze(0)
    if dtype is not None:
        x = x.to(dtype)
    if str(x.dtype).replace("torch.", "") not in _DTYPES:
        raise TypeError(f"x must be float16, bfloat16 or float32, got {x.dtype}")
    if device is not None:
        x = x.to(device)
    if x.device.type != "cuda":
        raise ValueError("x must be on a GPU device (or pass device=...)")
    return x.contiguous(), flat


def random_init(x, n_clusters: int, seed: int = 0):
    """K distinct points of each problem, chosen by a seeded host generator.

    x is (B,N,d) on the device; the result is (B,K,d) in x's dtype. With
    K > N the choice repeats points (a problem with fewer points than
    clusters keeps some clusters empty)."""
    torch = _torch()
    B, N, _ = x.shape
    g = torch.Generator().manual_seed(int(seed))
    if n_clusters <= N:
        idx = torch.stack([torch.randperm(N, generator=g)[:n_clusters] for _ in range(B)])
    else:
        idx = torch.randint(0, N, (B, n_clusters), generator=g)
    idx = idx.to(x.device)
    return torch.gather(x, 1, idx.unsqueeze(-1).expand(-1, -1, x.shape[2])).contiguous()


def batch_kmeans_Euclid(x, n_clusters: int, tol: float = 1e-4, verbose: bool = False,
                        max_iter: int = 100, init=None, seed: int = 0
                        ) -> Tuple[object, object, int]:
    """Exact Lloyd's K-Means on every problem of a batch.

    x: (B,N,d) or (N,d), float16/bfloat16/float32, on the GPU.
    Returns (cluster_ids int32 (B,N), centers float32 (B,K,d), n_iter); for a
    2-D x the batch axis is dropped. Stops after max_iter iterations or when
    every problem's centre shift sum_k ||c_new - c_old||^2 is below tol.
    init: (B,K,d) or (K,d) starting centroids in x's dtype; by default K
    distinct points per problem (seeded)."""
    if int(n_clusters) < 1:
        raise ValueError("n_clusters must be at least 1")
    if not (tol >= 0):
        raise ValueError("tol must be >= 0")
    if int(max_iter) < 0:
        raise ValueError("max_iter must be >= 0")
    xb, flat = _as_batched(x)
    K = int(n_clusters)
    if init is None:
        c0 = random_init(xb, K, seed)
    else:
        c0 = init.unsqueeze(0) if init.dim() == 2 else init
        if tuple(c0.shape) != (xb.shape[0], K, xb.shape[2]):
            raise ValueError(f"init must have shape {(xb.shape[0], K, xb.shape[2])}")
        c0 = c0.to(device=xb.device, dtype=xb.dtype).contiguous()
    if verbose:
        torch = _torch()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
    ids, centers, n_iter = fk.fk_lloyd(xb, c0, int(max_iter), float(tol))
    if verbose:
        t1.record()
        t1.synchronize()
        B, N, d = xb.shape
        print(f"flash k-means: B={B} N={N} d={d} K={K} {xb.dtype}: {n_iter} iterations "
              f"in {t0.elapsed_time(t1):.2f} ms")
    if flat:
        ids, centers = ids[0], centers[0]
    return ids, centers, n_iter


class FlashKMeans:
    """K-Means with the faiss/sklearn-like surface the pages show.

    d, k: dimension and number of clusters; niter: iteration cap; tol: stop
    when every problem's centre shift is below it (0: run niter iterations);
    dtype: the type points are clustered in (float16, bfloat16, float32;
    None keeps the input's); device: the GPU to use."""

    def __init__(self, d: int, k: int, niter: int = 100, tol: float = 1e-4, dtype=None,
                 device="cuda:0", seed: int = 0, verbose: bool = False):
        if int(d) < 1 or int(k) < 1 or int(niter) < 0:
            raise ValueError("d and k must be at least 1 and niter non-negative")
        self.d, self.k, self.niter, self.tol = int(d), int(k), int(niter), float(tol)
        self.dtype, self.device, self.seed, self.verbose = dtype, device, int(seed), verbose
        self.centroids = None   # (K,d) or (B,K,d) float32 after train
        self.n_iter = 0

    def _prepare(self, data):
        xb, flat = _as_batched(data, self.dtype, self.device)
        if xb.shape[2] != self.d:
            raise ValueError(f"data has dimension {xb.shape[2]}, the model {self.d}")
        return xb, flat

    def train(self, data, init=None):
        """Fit the centroids to data ((N,d) or (B,N,d)); returns self."""
        self.fit_predict(data, init)
        return self

    def fit_predict(self, data, init=None):
        """Fit, then return the ids of the last assignment step of the loop:
        those computed against the centroids before the last update, not a
        fresh assignment against the returned centroids (call predict() for
        that; the two agree once the loop has reached a fixed point)."""
        xb, flat = self._prepare(data)
        ids, centers, n_iter = batch_kmeans_Euclid(xb, self.k, self.tol, self.verbose,
                                                   self.niter, init, self.seed)
        self.centroids = centers[0] if flat else centers
        self.n_iter = n_iter
        return ids[0] if flat else ids

    def predict(self, data):
        """Nearest trained centroid of every point (one FlashAssign pass)."""
        if self.centroids is None:
            raise RuntimeError("predict before train")
        xb, flat = self._prepare(data)
        c = self.centroids.unsqueeze(0) if self.centroids.dim() == 2 else self.centroids
        if c.shape[0] != xb.shape[0]:
            raise ValueError("data must have as many problems as the trained model")
        c_lp, cnorm = fk.fk_norms(c.contiguous(), xb.dtype)
        ids = fk.fk_assign(xb, c_lp, cnorm)
        return ids[0] if flat else ids
