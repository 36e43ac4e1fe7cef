"""Oracle: exact batched Lloyd's K-Means, written from the definition in fp64.

TEST INFRASTRUCTURE ONLY -- imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library. Independent of the HIP
path: no shared code, helpers, constants or generated tables.

What it computes (the pages' definition)
----------------------------------------
* The method is standard Lloyd's K-Means with unchanged mathematics; its
  speed comes only from how data moves on the GPU, and its output is the
  same as plain Lloyd's ("Flash-KMeans：IO感知的精确K-Means…", paixiangai.cn,
  section "什么是 Flash-KMeans"; itinai.com summary, first paragraph;
  "Flash-KMeans: Fast and Memory-Efficient Exact K-Means", Abstract).
* One iteration = an assignment step (distance from every point to every
  centroid, keep the nearest) followed by an update step (each centroid
  becomes the average of its points) (paixiangai.cn page, sections
  "什么是 Flash-KMeans" and "交互式讲解", live-clustering panel).
* The input is a batch of B independent problems of N points in d
  dimensions, clustered into K clusters, with a centre-shift tolerance
  ``tol`` ("flash-kmeans and the return of exact K-Means on the GPU",
  section "Exact K-Means, with the assignment step written in Triton").

Readings where the pages are silent (each also listed in the design notes)
------------------------------------------------------------------------
R1 Centroid precision used by the assignment: the master centroids are
   real numbers (fp64 here); before each assignment they are rounded to
   nearest-even in the input element type, and that rounded copy c_hat is
   what distances are measured to.  ``round_centroids=False`` turns this off
   (plain real-valued Lloyd, used by the pins).
R2 Ties: the lowest centroid index wins.
R3 Empty cluster: keeps its previous (master) centroid.
R4 Centre shift: shift[b] = sum_k ||c_new[b,k] - c_old[b,k]||^2, evaluated
   after the update; the loop stops once max_b shift[b] < tol (strict), so
   tol = 0 runs exactly max_iter iterations.
R5 One loop for all B problems; finished problems keep iterating.
R6 Returned ids come from the last assignment, returned centres from the
   last update, and the iteration count is the number of completed
   assignment+update pairs.
R7 Near-tie band: a point whose best-vs-second distance gap is below
   1e-3 * (||x||^2 + ||c_hat_best||^2) may legitimately be assigned to any
   centroid within that band of the best; ``assign`` reports those sets.

Two evaluation forms of the distance
------------------------------------
``form="direct"`` evaluates sum_j (x_j - c_j)^2 literally.  ``form="expanded"``
uses the identity ||x - c||^2 = ||x||^2 - 2 x.c + ||c||^2 with a matrix
product for speed at large sizes, and then re-scores with the direct form
every row whose expanded gap is below 1e-9 of its scale, so both forms pick
the same ids (pinned in the tests). The near-tie sets of the expanded form
come from its own distances: their error, about 1e-15 of the scale, is twelve
orders of magnitude below the band.

Parity pins (tests/test_oracle_pins.py)
---------------------------------------
round_to_dtype   exact rational rounding (fractions) incl. halfway cases;
                 numpy/torch library casts where they round from the same value.
assign           exact rational brute force with duplicate centroids; library
                 routine (scikit-learn pairwise_distances_argmin); closed forms
                 (K=1, d=1 midpoints, K=N with c_hat = x).
update           exact integer sums for fp16 data; exact rational means;
                 K=1 global mean; point-permutation invariance.
lloyd            objective never increases (real centroids) and its rounding
                 slack bound (rounded centroids); scikit-learn KMeans(lloyd)
                 centres; batch independence; a hand-worked example.
Every function has at least one pin that does not re-use its own code.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

BAND_REL = 1e-3          # R7
RESCORE_REL = 1e-9       # expanded-form safety margin


# --------------------------------------------------------------------------
# R1: rounding to the element type
# --------------------------------------------------------------------------
_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_to_dtype(a, dtype: str) -> np.ndarray:
    """Nearest-even rounding of real values to ``dtype``; returned as fp64.

    fp32 and fp16 use NumPy's casts, which round a float64 directly to the
    target format.  bf16 (8 significant bits, fp32's exponent range) is
    written out: scale by the unit in the last place, round half to even,
    scale back; results above the largest finite bf16 become infinities.
    """
    a = np.asarray(a, dtype=np.float64)
    if dtype == "f32":
        with np.errstate(over="ignore"):
            return a.astype(np.float32).astype(np.float64)
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return a.astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        _, e = np.frexp(a)                      # |a| in [2^(e-1), 2^e)
        e = np.maximum(e, -125)                 # below 2^-126: subnormal spacing
        ulp = np.ldexp(1.0, e - 8)              # 8 significant bits
        r = np.rint(a / ulp) * ulp              # rint: half to even
        return np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, a), r)
    raise ValueError(f"unknown dtype {dtype!r}")


def centroid_sqnorms(c: np.ndarray) -> np.ndarray:
    """||c[b,k]||^2 for (B,K,d) centroids, fp64."""
    c = np.asarray(c, dtype=np.float64)
    return np.einsum("bkd,bkd->bk", c, c)


# --------------------------------------------------------------------------
# assignment step
# --------------------------------------------------------------------------
def sq_distances(x: np.ndarray, c: np.ndarray) -> np.ndarray:
    """D[n,k] = sum_j (x[n,j] - c[k,j])^2 for one problem (direct form)."""
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    diff = x[:, None, :] - c[None, :, :]
    return np.einsum("nkj,nkj->nk", diff, diff)


@dataclasses.dataclass
class AssignResult:
    ids: np.ndarray            # (B,N) int64, lowest index among minima (R2)
    dmin: np.ndarray           # (B,N) best squared distance
    gap: np.ndarray            # (B,N) second-best minus best (inf when K == 1)
    band: np.ndarray           # (B,N) 1e-3*(||x||^2 + ||c_hat_best||^2)  (R7)
    near: Dict[Tuple[int, int], np.ndarray]  # (b,n) -> all k with D-dmin < band, for gap < band

    def n_band(self) -> int:
        return int((self.gap < self.band).sum())


def _row_chunk(K: int, d: int, budget: int) -> int:
    return max(1, budget // max(1, K * d))


def _best_two(D: np.ndarray):
    """Per row: index of the first minimum, the minimum, the second-best value."""
    r = np.arange(D.shape[0])
    i = np.argmin(D, axis=1)                     # first occurrence = lowest index (R2)
    best = D[r, i]
    if D.shape[1] > 1:
        D2 = D.copy()
        D2[r, i] = np.inf
        second = D2.min(axis=1)
    else:
        second = np.full(D.shape[0], np.inf)
    return i, best, second


def assign(x: np.ndarray, c_hat: np.ndarray, *, form: str = "direct",
           budget: int = 1 << 24, want_near: bool = True) -> AssignResult:
    """Nearest centroid of every point, per problem.

    x: (B,N,d) real values of the points; c_hat: (B,K,d) centroids exactly as
    the assignment uses them (already rounded, R1).  ids[b,n] is the smallest
    k minimising D = sum_j (x - c_hat_k)^2.
    """
    if form not in ("direct", "expanded"):
        raise ValueError(form)
    x = np.asarray(x, dtype=np.float64)
    c_hat = np.asarray(c_hat, dtype=np.float64)
    B, N, d = x.shape
    K = c_hat.shape[1]
    ids = np.empty((B, N), dtype=np.int64)
    dmin = np.empty((B, N))
    gap = np.empty((B, N))
    band = np.empty((B, N))
    near: Dict[Tuple[int, int], np.ndarray] = {}
    step = _row_chunk(K, d if form == "direct" else 1, budget)
    for b in range(B):
        xb, cb = x[b], c_hat[b]
        xx = np.einsum("nj,nj->n", xb, xb)
        cc = np.einsum("kj,kj->k", cb, cb)
        for n0 in range(0, N, step):
            n1 = min(N, n0 + step)
            xs = xb[n0:n1]
            if form == "direct":
                D = sq_distances(xs, cb)
                i, dd, s2 = _best_two(D)
                Ddirect, rows = D, np.arange(n1 - n0)
            else:
                D = xx[n0:n1, None] + cc[None, :] - 2.0 * (xs @ cb.T)
                i, dd, s2 = _best_two(D)
                # rows whose two best are within 1e-9 of the scale: decide the id
                # with the direct form (row blocks sized to the memory budget)
                scale = xx[n0:n1] + cc[i]
                rows = np.nonzero(s2 - dd < RESCORE_REL * scale)[0]
                sub = max(1, budget // max(1, K * d))
                for r0 in range(0, rows.size, sub):
                    rr = rows[r0:r0 + sub]
                    Dd = sq_distances(xs[rr], cb)
                    ri, rd, rs = _best_two(Dd)
                    i[rr], dd[rr], s2[rr] = ri, rd, rs
                    D[rr] = Dd
                Ddirect, rows = D, np.arange(n1 - n0)
            bd = BAND_REL * (xx[n0:n1] + cc[i])
            if want_near:
                for j, r in enumerate(rows):
                    if s2[r] - dd[r] < bd[r]:
                        near[(b, n0 + int(r))] = np.nonzero(Ddirect[j] - dd[r] < bd[r])[0]
            ids[b, n0:n1], dmin[b, n0:n1], band[b, n0:n1] = i, dd, bd
            gap[b, n0:n1] = s2 - dd
    return AssignResult(ids, dmin, gap, band, near)


# --------------------------------------------------------------------------
# update step
# --------------------------------------------------------------------------
@dataclasses.dataclass
class UpdateResult:
    counts: np.ndarray         # (B,K) int64
    sums: np.ndarray           # (B,K,d) fp64
    centers: np.ndarray        # (B,K,d) fp64
    shift: np.ndarray          # (B,)   fp64  (R4)


def update(x: np.ndarray, ids: np.ndarray, c_old: np.ndarray) -> UpdateResult:
    """Each centroid becomes the mean of the points assigned to it.

    counts[b,k] = #{n : ids[b,n] = k}; sums[b,k] = sum of those points;
    a cluster with no point keeps c_old (R3); shift per R4.
    """
    x = np.asarray(x, dtype=np.float64)
    c_old = np.asarray(c_old, dtype=np.float64)
    ids = np.asarray(ids)
    B, N, d = x.shape
    K = c_old.shape[1]
    if N and (ids.min() < 0 or ids.max() >= K):
        raise ValueError("ids out of range")
    counts = np.zeros((B, K), dtype=np.int64)
    sums = np.zeros((B, K, d))
    for b in range(B):
        counts[b] = np.bincount(ids[b], minlength=K)
        for j in range(d):
            sums[b, :, j] = np.bincount(ids[b], weights=x[b, :, j], minlength=K)
    nonempty = counts > 0
    centers = c_old.copy()
    centers[nonempty] = sums[nonempty] / counts[nonempty][:, None]
    delta = centers - c_old
    shift = np.einsum("bkd,bkd->b", delta, delta)
    return UpdateResult(counts, sums, centers, shift)


def objective(x: np.ndarray, c: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """J[b] = sum_n ||x[b,n] - c[b, ids[b,n]]||^2 (fp64, direct)."""
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    B = x.shape[0]
    J = np.empty(B)
    for b in range(B):
        diff = x[b] - c[b][ids[b]]
        J[b] = np.einsum("nj,nj->", diff, diff)
    return J


# --------------------------------------------------------------------------
# the Lloyd loop
# --------------------------------------------------------------------------
@dataclasses.dataclass
class LloydResult:
    ids: np.ndarray            # (B,N) from the last assignment (R6)
    centers: np.ndarray        # (B,K,d) fp64 after the last update
    n_iter: int
    trace: Optional[List[dict]] = None


def lloyd(x: np.ndarray, c0: np.ndarray, max_iter: int, tol: float, dtype: str, *,
          round_centroids: bool = True, form: str = "expanded",
          record: bool = False, want_near: bool = True) -> LloydResult:
    """Lloyd iterations from initial centroids c0 (values of the element type).

    Per iteration t: c_hat = round(c) (R1); assign; update; stop when
    max_b shift_b < tol (R4, R5).  With ``record`` each iteration's c (before),
    c_hat, assignment, counts, new centres, shift and objective are kept.
    """
    if max_iter < 0 or not (tol >= 0):
        raise ValueError("max_iter >= 0 and tol >= 0 required")
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(c0, dtype=np.float64).copy()
    B, N, _ = x.shape
    ids = np.zeros((B, N), dtype=np.int64)
    trace: List[dict] = []
    it = 0
    for t in range(max_iter):
        c_hat = round_to_dtype(c, dtype) if round_centroids else c
        a = assign(x, c_hat, form=form, want_near=want_near)
        u = update(x, a.ids, c)
        if record:
            trace.append(dict(c=c, c_hat=c_hat, assign=a, counts=u.counts,
                              centers=u.centers, shift=u.shift,
                              J=a.dmin.sum(axis=1)))
        ids, c, it = a.ids, u.centers, t + 1
        if u.shift.max() < tol:
            break
    return LloydResult(ids, c, it, trace if record else None)
