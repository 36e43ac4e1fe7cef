"""The Python API (batch_kmeans_Euclid, FlashKMeans) over the C ABI.

Host tests check argument handling without a GPU; GPU tests check that the
API returns what the C entry points return for the same inputs, and that
those agree with the oracle under the usual comparison rules.
"""
import numpy as np
import pytest

import oracle
import synthdata
from gpu_helpers import CENTROID_RTOL, centroid_rel_err, check_ids, host_f64, to_dev


def _torch():
    import torch
    return torch


# ---------------------------------------------------------------------------
# host: argument checks (nothing reaches the library)
# ---------------------------------------------------------------------------
def test_api_rejects_bad_arguments_on_host():
    torch = _torch()
    from exact_means_clustering_flashassign_amd import FlashKMeans, batch_kmeans_Euclid

    x = torch.zeros(10, 4)
    with pytest.raises(ValueError):
        batch_kmeans_Euclid(x, 0)                      # no clusters
    with pytest.raises(ValueError):
        batch_kmeans_Euclid(x, 3, tol=-1.0)
    with pytest.raises(ValueError):
        batch_kmeans_Euclid(x, 3, max_iter=-1)
    with pytest.raises(ValueError):
        batch_kmeans_Euclid(torch.zeros(4), 3)         # neither (N,d) nor (B,N,d)
    with pytest.raises(TypeError):
        batch_kmeans_Euclid(torch.zeros(10, 4, dtype=torch.int32), 3)
    with pytest.raises(TypeError):
        batch_kmeans_Euclid(np.zeros((10, 4)), 3)
    with pytest.raises(ValueError):
        batch_kmeans_Euclid(x, 3)                      # a host tensor without a device
    with pytest.raises(ValueError):
        FlashKMeans(d=0, k=3)
    km = FlashKMeans(d=4, k=3)
    with pytest.raises(RuntimeError):
        km.predict(x)                                  # not trained


# ---------------------------------------------------------------------------
# GPU
# ---------------------------------------------------------------------------
def _mixture(B, N, d, K, dtype, seed):
    x, _, _ = synthdata.make_mixture(B, N, d, 1, dtype, n_comp=K, mean_std=2.0, seed=seed)
    return x, synthdata.to_f64(x, dtype)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_batch_kmeans_matches_fk_lloyd_and_oracle(fk, dtype):
    torch = _torch()
    B, N, d, K, T = 2, 3000, 64, 20, 4
    x, x64 = _mixture(B, N, d, K, dtype, seed=11)
    xd = to_dev(x, dtype)
    init = fk.random_init(xd, K, seed=5)
    ids, centers, n_iter = fk.batch_kmeans_Euclid(xd, K, tol=0.0, max_iter=T, seed=5)
    ids_c, centers_c, n_c = fk.fk_lloyd(xd, init, T, 0.0)
    torch.cuda.synchronize()
    assert n_iter == n_c == T
    # long clusters are summed with atomics in no fixed order, so two runs may
    # differ by fp32 reassociation in the centres, and a later assign may flip
    # a point whose two best centroids are that close
    assert int((ids != ids_c).sum()) <= ids.numel() // 10000
    assert centroid_rel_err(centers.cpu().numpy(), centers_c.double().cpu().numpy()) <= 1e-5
    # the first iteration against the oracle from the same starting points
    init64 = host_f64(init, dtype)
    ids1, centers1, _ = fk.batch_kmeans_Euclid(xd, K, tol=0.0, max_iter=1, seed=5)
    res = oracle.lloyd(x64, init64, 1, 0.0, dtype, record=True)
    st = check_ids(ids1.cpu().numpy(), res.trace[0]["assign"], f"api {dtype}")
    if st["n_flip_in_band"] == 0:
        assert centroid_rel_err(centers1.cpu().numpy(), res.centers) <= CENTROID_RTOL


@pytest.mark.gpu
def test_batch_kmeans_two_dimensional_input_and_init(fk):
    torch = _torch()
    x, _ = _mixture(1, 2500, 32, 12, "f16", seed=3)
    xd = to_dev(x, "f16")
    ids3, c3, n3 = fk.batch_kmeans_Euclid(xd, 12, tol=0.0, max_iter=1, seed=9)
    ids2, c2, n2 = fk.batch_kmeans_Euclid(xd[0], 12, tol=0.0, max_iter=1, seed=9)
    assert ids2.shape == (2500,) and c2.shape == (12, 32) and n2 == n3 == 1
    assert torch.equal(ids2, ids3[0])
    assert centroid_rel_err(c2.cpu().numpy(), c3[0].double().cpu().numpy()) <= 1e-5
    init = fk.random_init(xd, 12, seed=9)[0]           # an explicit (K,d) init
    ids_i, c_i, _ = fk.batch_kmeans_Euclid(xd[0], 12, tol=0.0, max_iter=1, init=init)
    assert torch.equal(ids_i, ids2)
    assert centroid_rel_err(c_i.cpu().numpy(), c2.double().cpu().numpy()) <= 1e-5


@pytest.mark.gpu
def test_batch_kmeans_tol_stops_early(fk):
    x, _ = _mixture(2, 4000, 16, 8, "f16", seed=21)
    xd = to_dev(x, "f16")
    _, _, n_loose = fk.batch_kmeans_Euclid(xd, 8, tol=1e30, max_iter=50)
    _, _, n_none = fk.batch_kmeans_Euclid(xd, 8, tol=0.0, max_iter=50)
    assert n_loose == 1 and n_none == 50


@pytest.mark.gpu
def test_flashkmeans_train_predict(fk):
    torch = _torch()
    x, x64 = _mixture(1, 5000, 128, 30, "f16", seed=7)
    xd = to_dev(x, "f16")[0]
    km = fk.FlashKMeans(d=128, k=30, niter=6, tol=0.0, seed=2)
    ids_fit = km.fit_predict(xd)
    assert km.centroids.shape == (30, 128) and km.n_iter == 6
    ids_pred = km.predict(xd)
    torch.cuda.synchronize()
    # predict is one assign against the trained centroids: compare with the
    # oracle's assign on the same centroids rounded to the input type
    c_hat = oracle.round_to_dtype(km.centroids.double().cpu().numpy(), "f16")
    a = oracle.assign(x64, c_hat[None], form="expanded")
    check_ids(ids_pred.cpu().numpy()[None], a, "FlashKMeans.predict")
    # fit_predict returns the ids of the last assign (before the last update)
    assert ids_fit.shape == (5000,) and ids_fit.dtype == torch.int32
    assert km.train(xd) is km
    # a float32 model clusters float32 data the same way through the fp32 path
    km32 = fk.FlashKMeans(d=128, k=30, niter=2, tol=0.0, dtype=torch.float32, seed=2)
    ids32 = km32.fit_predict(xd)
    assert ids32.dtype == torch.int32 and km32.centroids.dtype == torch.float32


@pytest.mark.gpu
@pytest.mark.parametrize("tol", [1e30, 1e-2])
def test_tol_stop_returns_the_stopping_iteration(fk, tol):
    """fk_lloyd with tol > 0 enqueues the next iteration before the stop test
    of the current one is read; on a stop, the results must be those of the
    stopping iteration (the rolled-back one leaves no trace)."""
    torch = _torch()
    x, _ = _mixture(2, 6000, 64, 30, "f16", seed=13)
    xd = to_dev(x, "f16")
    init = fk.random_init(xd, 30, seed=4)
    ids_t, c_t, n = fk.fk_lloyd(xd, init, 60, tol)
    ids_0, c_0, n0 = fk.fk_lloyd(xd, init, n, 0.0)
    torch.cuda.synchronize()
    assert n0 == n and 1 <= n < 60
    if n == 1:   # the first assign sees the initial centroids: ids bit-exact
        assert torch.equal(ids_t, ids_0)
    else:        # later assigns see centres summed in no fixed order
        assert int((ids_t != ids_0).sum()) <= ids_t.numel() // 10000
    assert centroid_rel_err(c_t.cpu().numpy(), c_0.double().cpu().numpy()) <= 1e-5
