"""GPU parity of the contrast baselines (libfkbaseline) against the oracle.

The materialised-distance assign and the scatter-atomic update compute the
same Lloyd steps as the library's own path; they are held to the same rules
(ids bit-exact outside the near-tie band, counts bit-exact, centroids within
the relative tolerance).
"""
import zlib

import numpy as np
import pytest

import oracle
import synthdata
from gpu_helpers import CENTROID_RTOL, centroid_rel_err, check_ids, to_dev, torch_dtype

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _seed(*key) -> int:
    return zlib.crc32(repr(key).encode()) % 100000


@pytest.mark.parametrize("dtype,B,N,d,K", [
    ("f16", 2, 3000, 128, 1000),
    ("bf16", 1, 2000, 64, 300),
    ("f32", 1, 2048, 32, 16),
    ("f16", 1, 777, 3, 5),
])
def test_materialized_assign_parity(fk, dtype, B, N, d, K):
    torch = _torch()
    seed = _seed("mat", dtype, B, N, d, K)
    x, _, _ = synthdata.make_mixture(B, N, d, 1, dtype, n_comp=max(2, K // 3), mean_std=1.5,
                                     seed=seed)
    x64 = synthdata.to_f64(x, dtype)
    rng = np.random.default_rng(seed + 1)
    idx = np.stack([rng.choice(N, size=K, replace=K > N) for _ in range(B)])
    c_hat = oracle.round_to_dtype(np.take_along_axis(x64, idx[..., None], axis=1)
                                  + 0.25 * rng.standard_normal((B, K, d)), dtype)
    xd = to_dev(x, dtype)
    c_lp, cn = fk.fk_norms(torch.from_numpy(c_hat.astype(np.float32)).cuda(), torch_dtype(dtype))
    ids_b = fk.fkb_assign_materialized(xd, c_lp, cn)
    ids_f = fk.fk_assign(xd, c_lp, cn)
    torch.cuda.synchronize()
    a = oracle.assign(x64, c_hat, form="expanded")
    check_ids(ids_b.cpu().numpy(), a, f"materialised {dtype}")
    check_ids(ids_f.cpu().numpy(), a, f"flash {dtype}")


@pytest.mark.parametrize("dtype,B,N,d,K,kind", [
    ("f16", 2, 5000, 128, 1000, "uniform"),
    ("f16", 1, 20000, 128, 64, "zipf"),
    ("bf16", 1, 3000, 1024, 256, "uniform"),
    ("f32", 1, 777, 3, 5, "zipf"),
])
def test_atomic_update_parity(fk, dtype, B, N, d, K, kind):
    torch = _torch()
    seed = _seed("atomic", dtype, B, N, d, K, kind)
    x, _, _ = synthdata.make_mixture(B, N, d, 1, dtype, n_comp=8, mean_std=1.0, seed=seed)
    x64 = synthdata.to_f64(x, dtype)
    ids = (synthdata.uniform_ids(B, N, K, seed + 1) if kind == "uniform"
           else synthdata.zipf_ids(B, N, K, seed + 1))
    c_old = np.random.default_rng(seed + 2).standard_normal((B, K, d)).astype(np.float32)
    c_dev = torch.from_numpy(c_old).cuda()
    _, counts = fk.fkb_update_atomic(to_dev(x, dtype), torch.from_numpy(ids).cuda(), c_dev)
    torch.cuda.synchronize()
    u = oracle.update(x64, ids, c_old.astype(np.float64))
    np.testing.assert_array_equal(counts.cpu().numpy(), u.counts)
    c_new = c_dev.cpu().numpy()
    empty = u.counts == 0
    np.testing.assert_array_equal(c_new[empty], c_old[empty])
    assert centroid_rel_err(c_new, u.centers) <= CENTROID_RTOL
