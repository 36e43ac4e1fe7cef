"""GPU parity along whole Lloyd runs, at the recipes' full sizes.

The library is deterministic (for K <= 65536), so fk_lloyd(x, init, t, 0)
reproduces, for every t, the state the loop reaches after t iterations; the
tests read the run one iteration at a time that way and check each step
against the oracle in lockstep:

  * assign: the oracle assigns a sample of rows against the centroids the
    GPU used in that iteration (its previous centres rounded to the element
    type); every GPU id must be the oracle's or inside the near-tie band;
  * update: for a sample of clusters the oracle averages the points the GPU
    assigned to them; centres within 2e-3 (per-centroid max norm), empty
    clusters keep their previous centre bit for bit.

The headline recipe's tol-stopped run is also checked against the oracle's
own (free-running) trajectory, stored as per-iteration digests in
tests/golden/api_example_b2_trajectory.json (written by the script beside
it, which calls only the oracle): the two must agree iteration for iteration
until the first in-band flip, and with no flip they must stop at the same
iteration.
"""
import hashlib
import json
import os

import numpy as np
import pytest

import oracle
import synthdata
from gpu_helpers import CENTROID_RTOL, centroid_rel_err, check_ids, f64_to_storage, to_dev

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "api_example_b2_trajectory.json")


def digest(a) -> str:
    return hashlib.sha256(np.ascontiguousarray(a, dtype="<i4").tobytes()).hexdigest()[:16]


def lockstep_step(x, dtype, ids_t, c_prev, c_t, rng, rows, clusters, where, all_rows=False):
    """One GPU iteration (ids_t from centres c_prev, centres c_t) against the
    oracle on sampled rows and clusters; returns the band statistics."""
    B, N, _ = x.shape
    K = c_prev.shape[1]
    c_hat = oracle.round_to_dtype(c_prev.astype(np.float64), dtype)
    tot = {"n": 0, "n_band": 0, "n_flip_in_band": 0}
    worst = 0.0
    for b in range(B):
        r = np.arange(N) if all_rows else np.sort(rng.choice(N, size=min(N, rows), replace=False))
        xs = synthdata.to_f64(x[b, r], dtype)[None]
        a = oracle.assign(xs, c_hat[b:b + 1], form="expanded")
        st = check_ids(ids_t[b:b + 1, r], a, f"{where} problem {b}")
        for k in tot:
            tot[k] += st[k]
        ks = np.sort(rng.choice(K, size=min(K, clusters), replace=False))
        sel = np.isin(ids_t[b], ks)
        remap = np.full(K, -1)
        remap[ks] = np.arange(ks.size)
        u = oracle.update(synthdata.to_f64(x[b, sel], dtype)[None], remap[ids_t[b, sel]][None],
                          c_prev[b:b + 1, ks].astype(np.float64))
        got = c_t[b:b + 1, ks]
        empty = u.counts[0] == 0
        assert np.array_equal(got[0, empty].view(np.uint32), c_prev[b, ks[empty]].view(np.uint32)), \
            f"{where} problem {b}: an empty cluster moved"
        if (~empty).any():
            worst = max(worst, centroid_rel_err(got[:, ~empty], u.centers[:, ~empty]))
    assert worst <= CENTROID_RTOL, (where, worst)
    return tot, worst


def gpu_run(fk, x_dev, init_dev, T):
    """The GPU loop's state after t = 1 .. T iterations (ids, centres)."""
    for t in range(1, T + 1):
        ids, c, n = fk.fk_lloyd(x_dev, init_dev, t, 0.0)
        assert n == t
        yield t, ids.cpu().numpy(), c.cpu().numpy()


def test_headline_tol_stop_against_the_oracle(fk):
    """api_example at full N (75600 points, K = 1000, fp16) on two problems,
    tol = 1e-4, up to 100 iterations: the tol-stopped run equals the t-step
    run of its iteration count bit for bit (the iteration it enqueued past
    the stop is rolled back), every iteration matches the oracle in lockstep,
    the stop rule holds on the GPU's own shifts, and the run follows the
    oracle's own trajectory until the first in-band flip (same stop
    iteration when there is none)."""
    with open(GOLDEN) as f:
        gold = json.load(f)
    w = synthdata.make_workload("api_example", B=2)
    x_dev, init_dev = to_dev(w.x, w.dtype), to_dev(w.init, w.dtype)
    ids_tol, c_tol, n_gpu = fk.fk_lloyd(x_dev, init_dev, 100, w.tol)
    ids_tol, c_tol = ids_tol.cpu().numpy(), c_tol.cpu().numpy()
    assert 1 <= n_gpu < 100, n_gpu          # stopped by the tol test, rollback exercised
    rng = np.random.default_rng(17)
    c_prev = synthdata.to_f64(w.init, w.dtype).astype(np.float32)
    first_div, flips = None, 0
    for t, ids_t, c_t in gpu_run(fk, x_dev, init_dev, n_gpu):
        diverged = first_div is None and (t > len(gold["iterations"]) or
                                          digest(ids_t) != gold["iterations"][t - 1]["ids"])
        if diverged:
            first_div = t
        # the iteration where the run leaves the oracle's path: every row
        st, err = lockstep_step(w.x, w.dtype, ids_t, c_prev, c_t, rng, 4096, 96,
                                f"api_example tol run it {t}", all_rows=diverged)
        flips += st["n_flip_in_band"]
        s = ((c_t.astype(np.float64) - c_prev) ** 2).sum(axis=(1, 2)).max()
        if t < n_gpu:
            assert s >= w.tol * (1 + 1e-3), (t, s)      # the loop had to go on
        else:
            assert s < w.tol * (1 - 1e-3), (t, s)       # and stopped here
        c_prev = c_t
    assert np.array_equal(ids_tol, ids_t)
    assert np.array_equal(c_tol.view(np.uint32), c_t.view(np.uint32))
    print(f"tol run: GPU n_iter {n_gpu}, oracle n_iter {gold['n_iter']}; first departure from "
          f"the oracle's trajectory: {first_div}; in-band flips on sampled rows {flips}; "
          f"n_flip_outside_band = 0")
    if first_div is None:
        assert n_gpu == gold["n_iter"]


@pytest.mark.parametrize("tol", [0.0, 1e-30])
def test_long_clusters_free_running_f16(fk, tol):
    """fp16, clusters of thousands of points (summed in pieces): the loop's
    long-cluster division runs in the next norms pass (tol = 0) or in the
    finalize kernel (tol > 0). Free-running against the oracle from the same
    init: identical ids (band rule) and centres within 2e-3 until the first
    in-band flip."""
    x, init, _ = synthdata.make_mixture(2, 40000, 128, 16, "f16", n_comp=12, mean_std=2.0,
                                        seed=41)
    T = 6
    res = oracle.lloyd(synthdata.to_f64(x, "f16"), synthdata.to_f64(init, "f16"), T, 0.0, "f16",
                       record=True)
    assert max(tr["counts"].max() for tr in res.trace) > 8 * 256
    x_dev, init_dev = to_dev(x, "f16"), to_dev(init, "f16")
    first_flip = None
    for t in range(1, T + 1):
        ids, c, n = fk.fk_lloyd(x_dev, init_dev, t, tol)
        assert n == t
        tr = res.trace[t - 1]
        st = check_ids(ids.cpu().numpy(), tr["assign"], f"long clusters it {t}")
        if first_flip is None and st["n_flip_in_band"]:
            first_flip = t
        if first_flip is None:
            err = centroid_rel_err(c.cpu().numpy(), tr["centers"])
            assert err <= CENTROID_RTOL, (t, err)
    print(f"tol {tol}: first in-band flip at iteration {first_flip}; n_flip_outside_band = 0")


@pytest.mark.parametrize("name,rows,clusters", [("io_breakdown", 512, 32),
                                                ("split_d", 1024, 64),
                                                ("large_k_zipf", 4096, 64)])
def test_full_size_recipe_lockstep(fk, name, rows, clusters):
    """The recipe at its full size over its own iteration count (20, 20, 10):
    every iteration of fk_lloyd checked in lockstep on sampled rows and
    clusters."""
    w = synthdata.make_workload(name)
    x_dev, init_dev = to_dev(w.x, w.dtype), to_dev(w.init, w.dtype)
    rng = np.random.default_rng(23)
    c_prev = synthdata.to_f64(w.init, w.dtype).astype(np.float32)
    flips = 0
    for t, ids_t, c_t in gpu_run(fk, x_dev, init_dev, w.max_iter):
        st, err = lockstep_step(w.x, w.dtype, ids_t, c_prev, c_t, rng, rows, clusters,
                                f"{name} it {t}")
        flips += st["n_flip_in_band"]
        c_prev = c_t
    print(f"{name}: {w.max_iter} iterations in lockstep; in-band flips on sampled rows "
          f"{flips}; n_flip_outside_band = 0")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_resume_from_centres(fk, dtype):
    """Lloyd's whole state is its fp32 centres: T iterations, then the rest
    resumed from the returned centres (init=None), equal one run bit for bit,
    for a fixed iteration count (10 = 4 + 6) and for a tol-stopped run (the
    resumed call stops at the same iteration). Clusters of thousands of points
    make the first call end on the long clusters' deferred division and the
    resumed call start right after it; a centroid far from every point keeps
    its cluster empty throughout."""
    x, init, _ = synthdata.make_mixture(2, 30000, 128, 24, dtype, n_comp=12, mean_std=2.0,
                                        seed=43)
    init = synthdata.to_f64(init, dtype)
    init[:, 1] = 64.0                        # cluster 1 never wins a point
    init = f64_to_storage(init, dtype)
    x_dev, init_dev = to_dev(x, dtype), to_dev(init, dtype)
    ids10, c10, n = fk.fk_lloyd(x_dev, init_dev, 10, 0.0)
    assert n == 10
    _, c4, _ = fk.fk_lloyd(x_dev, init_dev, 4, 0.0)
    ids_r, c_r, n_r = fk.fk_lloyd(x_dev, None, 6, 0.0, centers=c4.clone())
    assert n_r == 6
    assert np.array_equal(ids_r.cpu().numpy(), ids10.cpu().numpy())
    assert np.array_equal(c_r.cpu().numpy().view(np.uint32), c10.cpu().numpy().view(np.uint32))
    tol = 1e-3
    ids_t, c_t, n_t = fk.fk_lloyd(x_dev, init_dev, 100, tol)
    assert 6 <= n_t < 100, n_t
    ids_r, c_r, n_r = fk.fk_lloyd(x_dev, None, 100, tol, centers=c4.clone())
    assert n_r == n_t - 4, (n_t, n_r)
    assert np.array_equal(ids_r.cpu().numpy(), ids_t.cpu().numpy())
    assert np.array_equal(c_r.cpu().numpy().view(np.uint32), c_t.cpu().numpy().view(np.uint32))
    print(f"{dtype}: resume after 4 of 10 iterations and of a tol run of {n_t} iterations: "
          f"bit-identical")
