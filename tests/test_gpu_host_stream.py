"""fk_lloyd_host: the Lloyd loop over points kept in host memory, streamed to
the device in chunks every iteration, against the oracle's trajectory and
against fk_lloyd on the same inputs."""
import numpy as np
import pytest

import oracle
import synthdata
from gpu_helpers import CENTROID_RTOL, centroid_rel_err, check_ids, host_f64, to_dev

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _host(x, dtype, pinned=True):
    t = synthdata.to_torch(x, dtype).contiguous()
    return t.pin_memory() if pinned else t


CASES = [
    # dtype, B, N, d, K, chunk, iterations
    ("f16", 2, 5000, 128, 100, 1300, 3),      # ragged last chunk, both buffers reused
    ("f16", 1, 20000, 128, 64, 4096, 3),      # several rounds of the two buffers
    ("bf16", 1, 3000, 64, 37, 3000, 2),       # one chunk
    ("bf16", 2, 2500, 1024, 40, 1000, 2),     # split-D assign on the chunks
    ("f32", 1, 2048, 32, 16, 500, 3),
    ("f16", 1, 700, 16, 300, 10000, 2),       # chunk above N
]


@pytest.mark.parametrize("dtype,B,N,d,K,chunk,T", CASES)
def test_host_stream_follows_the_oracle(fk, dtype, B, N, d, K, chunk, T):
    torch = _torch()
    x, _, _ = synthdata.make_mixture(B, N, d, 1, dtype, n_comp=max(2, K // 2), mean_std=1.5,
                                     seed=B * 7 + N + d + K)
    x64 = synthdata.to_f64(x, dtype)
    xh = _host(x, dtype)
    init = fk.random_init(to_dev(x, dtype), K, seed=3)
    init64 = host_f64(init, dtype)
    res = oracle.lloyd(x64, init64, T, 0.0, dtype, record=True)
    first_flip = None
    for t in range(1, T + 1):
        ids, centers, n_iter = fk.fk_lloyd_host(xh, init, t, 0.0, chunk)
        torch.cuda.synchronize()
        assert n_iter == t
        st = check_ids(ids.cpu().numpy(), res.trace[t - 1]["assign"], f"host stream it {t}")
        if first_flip is None and st["n_flip_in_band"]:
            first_flip = t
        if first_flip is None:
            err = centroid_rel_err(centers.cpu().numpy(), res.trace[t - 1]["centers"])
            assert err <= CENTROID_RTOL, (t, err)


def test_host_stream_matches_device_loop(fk):
    torch = _torch()
    x, _, _ = synthdata.make_mixture(3, 6000, 128, 1, "f16", n_comp=40, mean_std=1.5, seed=5)
    xd = to_dev(x, "f16")
    init = fk.random_init(xd, 120, seed=8)
    ids_h, c_h, n_h = fk.fk_lloyd_host(_host(x, "f16"), init, 1, 0.0, 1500)
    ids_d, c_d, n_d = fk.fk_lloyd(xd, init, 1, 0.0)
    torch.cuda.synchronize()
    assert n_h == n_d == 1
    assert torch.equal(ids_h, ids_d)                 # the first assign sees the same centroids
    assert centroid_rel_err(c_h.cpu().numpy(), c_d.double().cpu().numpy()) <= 1e-5


def test_host_stream_pageable_memory_and_tol(fk):
    torch = _torch()
    x, _, _ = synthdata.make_mixture(1, 4000, 64, 1, "f16", n_comp=10, mean_std=2.0, seed=9)
    xd = to_dev(x, "f16")
    init = fk.random_init(xd, 10, seed=1)
    ids_p, c_p, _ = fk.fk_lloyd_host(_host(x, "f16", pinned=False), init, 2, 0.0, 1000)
    ids_q, c_q, _ = fk.fk_lloyd_host(_host(x, "f16"), init, 2, 0.0, 1000)
    torch.cuda.synchronize()
    assert int((ids_p != ids_q).sum()) <= 1
    assert centroid_rel_err(c_p.cpu().numpy(), c_q.double().cpu().numpy()) <= 1e-5
    _, _, n_loose = fk.fk_lloyd_host(_host(x, "f16"), init, 30, 1e30, 1000)
    assert n_loose == 1
    ids0, c0, n0 = fk.fk_lloyd_host(_host(x, "f16"), init, 0, 0.0, 1000)
    torch.cuda.synchronize()
    assert n0 == 0 and int(ids0.abs().sum()) == 0
    np.testing.assert_array_equal(c0.cpu().numpy(), host_f64(init, "f16").astype(np.float32))
