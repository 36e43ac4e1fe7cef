"""GPU parity: every HIP entry point against the fp64 oracle, through the C ABI.

Inputs come from the seeded generators or from the oracle's own Lloyd
trajectory; expected values come from the oracle only. Comparison rules are in
gpu_helpers. Sizes: reduced versions of the five workload recipes (several
tiles plus ragged tails in N, K and d) compared element by element, and the
full workload sizes, in the launch configuration the benchmark times,
compared on sampled rows / clusters.
"""
import os
import zlib

import numpy as np
import pytest

import oracle
import synthdata
from gpu_helpers import (CENTROID_RTOL, centroid_rel_err, check_ids, check_shift,
                         f64_to_storage, host_f64, to_dev, torch_dtype)

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def stable_seed(*key) -> int:
    return zlib.crc32(repr(key).encode()) % 100000


def gpu_norms_assign(fk, x_dev, c_hat64, dtype):
    """fk_norms on the fp32 copy of c_hat (exactly representable), then fk_assign."""
    torch = _torch()
    c32 = torch.from_numpy(c_hat64.astype(np.float32)).cuda()
    c_lp, cn = fk.fk_norms(c32, torch_dtype(dtype))
    ids = fk.fk_assign(x_dev, c_lp, cn)
    torch.cuda.synchronize()
    return c_lp, cn, ids.cpu().numpy()


def make_centroids(x64, K, dtype, seed, jitter=0.25, dup=True):
    """Centroids near data points, rounded to dtype; centroid 1 duplicates 0."""
    rng = np.random.default_rng(seed)
    B, N, d = x64.shape
    idx = np.stack([rng.choice(N, size=K, replace=K > N) for _ in range(B)])
    c = np.take_along_axis(x64, idx[..., None], axis=1)
    c = c + jitter * rng.standard_normal(c.shape)
    c = oracle.round_to_dtype(c, dtype)
    if dup and K >= 2:
        c[:, 1] = c[:, 0]
    return c


# ---------------------------------------------------------------------------
# fk_norms
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,d", [("f16", 100), ("bf16", 100), ("f32", 100), ("f16", 99),
                                     ("bf16", 1024), ("f16", 4), ("bf16", 30)])
def test_norms_rounding_and_sqnorms(fk, dtype, d):
    torch = _torch()
    rng = np.random.default_rng(100 + d)
    B, K = 3, 77
    c = (rng.standard_normal((B, K, d)) * 10.0 ** rng.integers(-3, 3, (B, K, 1))).astype(np.float32)
    if dtype != "f32":
        # exact halfway points between neighbours, and values next to them
        p = 11 if dtype == "f16" else 8
        r = oracle.round_to_dtype(c[0].astype(np.float64), dtype)
        ulp = np.ldexp(1.0, np.frexp(np.abs(r))[1] - p)
        mid = (r + np.sign(r) * ulp / 2).astype(np.float32)
        c[1] = mid
        c[2, :, ::2] = np.nextafter(mid[:, ::2], np.float32(np.inf))
    c_lp, cn = fk.fk_norms(torch.from_numpy(c).cuda(), torch_dtype(dtype))
    want = oracle.round_to_dtype(c.astype(np.float64), dtype)
    np.testing.assert_array_equal(host_f64(c_lp, dtype), want)
    ref = oracle.centroid_sqnorms(want)
    got = cn.cpu().numpy().astype(np.float64)
    assert (np.abs(got - ref) <= d * 2.0 ** -23 * ref + 1e-30).all()


# ---------------------------------------------------------------------------
# fk_assign: shapes across both MFMA paths and the fp32 path
# ---------------------------------------------------------------------------
ASSIGN_CASES = [
    # dtype, B, N, d, K, force split-D
    ("f16", 2, 3000, 128, 1000, False),     # reduced headline shape, ragged N and K
    ("f16", 4, 40000, 128, 150, False),     # more point blocks than resident blocks:
    ("bf16", 3, 50000, 128, 100, False),    # blocks move on to a second point block
    ("f16", 1, 777, 1, 5, False),
    ("f16", 1, 500, 3, 40, False),
    ("f16", 1, 600, 8, 70, False),
    ("bf16", 2, 700, 31, 65, False),
    ("f16", 1, 700, 33, 129, False),
    ("bf16", 1, 900, 100, 200, False),
    ("f16", 1, 640, 127, 64, False),
    ("f16", 1, 520, 129, 100, False),
    ("bf16", 1, 400, 255, 90, False),
    ("f16", 1, 300, 500, 70, False),
    ("bf16", 1, 300, 512, 33, False),
    ("f16", 2, 1500, 32, 90, False),        # whole 32-unit rows: 64 rows per staging load
    ("bf16", 1, 3000, 64, 300, False),      # whole 64-unit rows, three tiles
    ("bf16", 1, 300, 513, 40, False),       # split-D from here on
    ("bf16", 2, 1000, 1024, 256, False),
    ("f16", 1, 200, 1000, 150, False),
    ("bf16", 1, 150, 2048, 60, False),
    ("f16", 1, 400, 640, 300, False),       # two 256-row K tiles over five d-chunks
    # direct-to-LDS staging (whole rows, an even number of 128-wide d-chunks):
    ("bf16", 2, 5000, 768, 700, False),     # three K tiles, the last ragged (188 rows)
    ("f16", 1, 3000, 512, 257, True),       # forced at d = 512: a one-row last K tile
    ("bf16", 3, 2100, 1280, 100, False),    # 128-row tiles, ten d-chunks, ragged N
    ("f16", 2, 70000, 1024, 40, False),     # more point blocks than resident blocks
    ("f16", 2, 1000, 128, 300, True),       # split-D forced at small d
    ("bf16", 1, 500, 60, 130, True),
    ("f32", 1, 2048, 32, 16, False),
    ("f32", 2, 999, 3, 50, False),
    ("f32", 1, 500, 100, 70, False),
    ("f32", 2, 3000, 128, 300, False),      # fp32 MFMA, several tiles and point blocks
    ("f32", 1, 2000, 64, 200, False),       # fp32 MFMA, 8-wave blocks with prefetch
    ("f32", 1, 1000, 256, 100, False),      # fp32 MFMA at its widest rows
    ("f32", 1, 500, 100, 70, True),         # fp32 split-D (forced at small d)
    ("f32", 1, 400, 300, 50, False),        # fp32 split-D (d > 256)
    ("f32", 2, 1000, 600, 300, False),      # fp32 split-D, two 256-row K tiles
    ("f32", 1, 1500, 384, 200, False),      # fp32 split-D with direct-to-LDS staging
    ("f16", 1, 5, 16, 1, False),            # K = 1
    ("f16", 1, 10, 16, 40, False),          # K > N
    ("bf16", 3, 33, 64, 7, False),          # N below one tile
]


@pytest.mark.parametrize("dtype,B,N,d,K,force", ASSIGN_CASES)
def test_assign_parity(fk, monkeypatch, dtype, B, N, d, K, force):
    if force:
        monkeypatch.setenv("FK_FORCE_SPLITD", "1")
    else:
        monkeypatch.delenv("FK_FORCE_SPLITD", raising=False)
    seed = stable_seed(dtype, B, N, d, K)
    x, _, _ = synthdata.make_mixture(B, N, d, 1, dtype, n_comp=max(2, K // 3), mean_std=1.5,
                                  seed=seed)
    x64 = synthdata.to_f64(x, dtype)
    c_hat = make_centroids(x64, K, dtype, seed + 1)
    c_lp, _, ids = gpu_norms_assign(fk, to_dev(x, dtype), c_hat, dtype)
    np.testing.assert_array_equal(host_f64(c_lp, dtype), c_hat)
    a = oracle.assign(x64, c_hat, form="direct" if N * K * d < 2e7 else "expanded")
    stats = check_ids(ids, a, f"assign {dtype} B{B} N{N} d{d} K{K}")
    if K >= 2:   # centroid 1 duplicates 0: it wins only where 0 would (an exact tie)
        assert (a.ids[ids == 1] == 0).all()
    print(stats)


@pytest.mark.parametrize("dtype,B,N,d,K", [("bf16", 2, 6000, 1024, 256),
                                             ("f16", 1, 5000, 768, 600),
                                             ("f32", 1, 3000, 256, 100)])
def test_splitd_staging_paths_agree(fk, monkeypatch, dtype, B, N, d, K):
    """Whole-row split-D problems staged straight into LDS and staged through
    registers (FK_SPLITD_REGISTER_STAGING=1): both against the oracle under
    the band rule. The two add -||c||^2/2 at different points of the fp32
    sum, so they may differ only on near-tie rows (in-band for both)."""
    monkeypatch.setenv("FK_FORCE_SPLITD", "1")
    seed = stable_seed(dtype, B, N, d, K, "staging")
    x, _, _ = synthdata.make_mixture(B, N, d, 1, dtype, n_comp=max(2, K // 3), mean_std=1.5,
                                  seed=seed)
    x64 = synthdata.to_f64(x, dtype)
    c_hat = make_centroids(x64, K, dtype, seed + 1)
    x_dev = to_dev(x, dtype)
    monkeypatch.delenv("FK_SPLITD_REGISTER_STAGING", raising=False)
    _, _, ids_lds = gpu_norms_assign(fk, x_dev, c_hat, dtype)
    monkeypatch.setenv("FK_SPLITD_REGISTER_STAGING", "1")
    _, _, ids_reg = gpu_norms_assign(fk, x_dev, c_hat, dtype)
    a = oracle.assign(x64, c_hat, form="expanded")
    st_lds = check_ids(ids_lds, a, f"split-D LDS staging {dtype} B{B} N{N} d{d} K{K}")
    st_reg = check_ids(ids_reg, a, f"split-D register staging {dtype} B{B} N{N} d{d} K{K}")
    differ = int((ids_lds != ids_reg).sum())
    assert differ <= st_lds["n_band"] + st_reg["n_band"], (differ, st_lds, st_reg)
    print(st_lds, st_reg, f"rows that differ: {differ}")


# ---------------------------------------------------------------------------
# fk_update
# ---------------------------------------------------------------------------
UPDATE_CASES = [
    # dtype, B, N, d, K, ids kind
    ("f16", 2, 5000, 128, 1000, "uniform"),
    ("f16", 1, 20000, 128, 64, "zipf"),
    ("bf16", 2, 3000, 1024, 256, "uniform"),
    ("f32", 1, 2048, 32, 16, "uniform"),
    ("f16", 1, 4000, 100, 37, "one"),          # every point in one cluster
    ("bf16", 1, 300, 33, 1000, "uniform"),     # K > N: many empty clusters
    ("f16", 2, 10000, 130, 40000, "uniform"),  # K above one LDS bin range
    ("f32", 1, 777, 3, 5, "zipf"),
    ("f16", 1, 9000, 2000, 20, "uniform"),     # d above one segreduce pass
    ("f16", 2, 300000, 32, 8, "zipf"),         # clusters over 32 runs: Q1 block sums
    ("bf16", 1, 300000, 64, 5, "one"),         # one cluster over 1024 runs: a Q2 block sum
    ("f16", 1, 262144, 48, 4, "one"),          # 1024 runs, no block sums: 1023 pieces added one by one
    ("f32", 1, 70000, 36, 3, "zipf"),          # long pieces with d % 4 == 0, fp32 slices
    ("f16", 1, 70000, 33, 3, "zipf"),          # long pieces with ragged d (scalar stores)
    ("f16", 2, 20000, 64, 5000, "zipf"),       # ids over 11 bits: the two-pass LDS sort
    ("bf16", 1, 50000, 64, 2047, "uniform"),   # the widest ids of the direct scatter
    ("f16", 1, 200000, 64, 4096, "zipf"),      # chunks x clusters above one offsets block
    ("bf16", 3, 120000, 32, 3000, "uniform"),  # the same, three problems
]


def _ids(kind, B, N, K, seed):
    if kind == "uniform":
        return synthdata.uniform_ids(B, N, K, seed)
    if kind == "zipf":
        return synthdata.zipf_ids(B, N, K, seed)
    return np.full((B, N), K // 2, dtype=np.int32)


@pytest.mark.parametrize("dtype,B,N,d,K,kind", UPDATE_CASES)
def test_update_parity(fk, dtype, B, N, d, K, kind):
    torch = _torch()
    seed = stable_seed(dtype, B, N, d, K, kind)
    x, _, _ = synthdata.make_mixture(B, N, d, 1, dtype, n_comp=8, mean_std=1.0, seed=seed)
    x64 = synthdata.to_f64(x, dtype)
    ids = _ids(kind, B, N, K, seed + 1)
    c_old = np.random.default_rng(seed + 2).standard_normal((B, K, d)).astype(np.float32)
    c_dev = torch.from_numpy(c_old).cuda()
    _, counts, shift = fk.fk_update(to_dev(x, dtype), torch.from_numpy(ids).cuda(), c_dev)
    torch.cuda.synchronize()
    u = oracle.update(x64, ids, c_old.astype(np.float64))
    np.testing.assert_array_equal(counts.cpu().numpy(), u.counts)
    c_new = c_dev.cpu().numpy()
    empty = u.counts == 0
    np.testing.assert_array_equal(c_new[empty], c_old[empty])     # kept bit for bit
    err = centroid_rel_err(c_new, u.centers)
    assert err <= CENTROID_RTOL, err
    check_shift(shift.cpu().numpy().astype(np.float64), u.shift, u.centers)


RADIX_CASES = [c for c in UPDATE_CASES if c[4] <= 65536 and c[2] * c[1] <= 700000]


@pytest.mark.parametrize("dtype,B,N,d,K,kind", RADIX_CASES)
def test_update_parity_radix(fk, monkeypatch, dtype, B, N, d, K, kind):
    """The same cases with perm built by the whole-problem radix passes."""
    monkeypatch.setenv("FK_FORCE_RADIX", "1")
    test_update_parity(fk, dtype, B, N, d, K, kind)


@pytest.mark.parametrize("radix", [False, True])
def test_update_is_deterministic(fk, monkeypatch, radix):
    """Hot clusters (pieces over many runs): ten fk_update calls on the same
    ids give bit-identical centroids, counts and shift; the perm is the
    stable order (each cluster's points by increasing index)."""
    torch = _torch()
    if radix:
        monkeypatch.setenv("FK_FORCE_RADIX", "1")
    else:
        monkeypatch.delenv("FK_FORCE_RADIX", raising=False)
    x, _, _ = synthdata.make_mixture(2, 120000, 128, 1, "f16", n_comp=8, mean_std=1.0, seed=31)
    ids = synthdata.zipf_ids(2, 120000, 300, 32)
    c0 = np.random.default_rng(33).standard_normal((2, 300, 128)).astype(np.float32)
    x_dev, ids_dev = to_dev(x, "f16"), torch.from_numpy(ids).cuda()
    outs = []
    for _ in range(10):
        c = torch.from_numpy(c0).cuda()
        _, counts, shift = fk.fk_update(x_dev, ids_dev, c)
        torch.cuda.synchronize()
        outs.append((c.cpu().numpy(), counts.cpu().numpy(), shift.cpu().numpy()))
    for c, counts, shift in outs[1:]:
        assert np.array_equal(c.view(np.uint32), outs[0][0].view(np.uint32))
        assert np.array_equal(counts, outs[0][1])
        assert np.array_equal(shift.view(np.uint32), outs[0][2].view(np.uint32))
    u = oracle.update(synthdata.to_f64(x, "f16"), ids, c0.astype(np.float64))
    assert u.counts.max() > 20 * 256                # long clusters over many runs
    assert centroid_rel_err(outs[0][0], u.centers) <= CENTROID_RTOL


# ---------------------------------------------------------------------------
# lockstep: the GPU steps follow the oracle's own trajectory
# ---------------------------------------------------------------------------
RECIPES = [
    # name, reduced N, reduced B, iterations
    ("tiny_f32", None, None, 10),
    ("api_example", 6000, 2, 4),
    ("io_breakdown", 8192, 2, 4),
    ("large_k_zipf", 36000, 1, 2),
    ("split_d", 4096, 2, 3),
]


@pytest.fixture(scope="module")
def trajectories():
    cache = {}

    def get(name, n, b, T):
        key = (name, n, b, T)
        if key not in cache:
            w = synthdata.make_workload(name, scale_n=n, B=b)
            res = oracle.lloyd(w.x64(), w.init64(), T, 0.0, w.dtype, record=True)
            cache[key] = (w, res)
        return cache[key]
    return get


@pytest.mark.parametrize("name,n,b,T", RECIPES)
def test_lockstep(fk, trajectories, name, n, b, T):
    torch = _torch()
    w, res = trajectories(name, n, b, T)
    x_dev = to_dev(w.x, w.dtype)
    for t, tr in enumerate(res.trace):
        c_lp, _, ids = gpu_norms_assign(fk, x_dev, tr["c_hat"], w.dtype)
        np.testing.assert_array_equal(host_f64(c_lp, w.dtype), tr["c_hat"])
        stats = check_ids(ids, tr["assign"], f"{name} iteration {t}")
        c_dev = torch.from_numpy(tr["c"].astype(np.float32)).cuda()
        ids_o = torch.from_numpy(tr["assign"].ids.astype(np.int32)).cuda()
        _, counts, shift = fk.fk_update(x_dev, ids_o, c_dev)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(counts.cpu().numpy(), tr["counts"])
        err = centroid_rel_err(c_dev.cpu().numpy(), tr["centers"])
        assert err <= CENTROID_RTOL, (name, t, err)
        check_shift(shift.cpu().numpy().astype(np.float64), tr["shift"], tr["centers"],
                    f"{name} it {t}")
        print(name, t, stats, "centroid rel err %.2e" % err)


# ---------------------------------------------------------------------------
# free-running: fk_lloyd alone from the same init
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,n,b,T", RECIPES)
def test_free_running(fk, trajectories, name, n, b, T):
    w, res = trajectories(name, n, b, T)
    x_dev, init_dev = to_dev(w.x, w.dtype), to_dev(w.init, w.dtype)
    first_flip = None
    for t in range(1, T + 1):
        ids, centers, n_iter = fk.fk_lloyd(x_dev, init_dev, t, 0.0)
        assert n_iter == t
        tr = res.trace[t - 1]
        stats = check_ids(ids.cpu().numpy(), tr["assign"], f"{name} free-running it {t}")
        if first_flip is None and stats["n_flip_in_band"]:
            first_flip = t
        if first_flip is None:
            err = centroid_rel_err(centers.cpu().numpy(), tr["centers"])
            assert err <= CENTROID_RTOL, (name, t, err)
    print(name, "first in-band flip at iteration", first_flip)


# ---------------------------------------------------------------------------
# full workload sizes, sampled
# ---------------------------------------------------------------------------
def _sampled_assign_check(x64, c_hat, ids, rng, per_batch):
    B, N, _ = x64.shape
    total = {"n": 0, "n_band": 0, "n_flip_in_band": 0}
    for b in range(B):
        rows = np.sort(rng.choice(N, size=min(N, per_batch), replace=False))
        a = oracle.assign(x64[b:b + 1, rows], c_hat[b:b + 1], form="expanded")
        st = check_ids(ids[b:b + 1, rows], a, f"batch {b} sampled rows")
        for k in total:
            total[k] += st[k]
    return total


@pytest.mark.parametrize("name,per_batch", [("api_example", 256), ("io_breakdown", 256),
                                            ("split_d", 512), ("large_k_zipf", 2048)])
def test_full_size_assign_sampled(fk, name, per_batch):
    w = synthdata.make_workload(name)
    x_dev = to_dev(w.x, w.dtype)
    c_hat = w.init64()
    _, _, ids = gpu_norms_assign(fk, x_dev, c_hat, w.dtype)
    rng = np.random.default_rng(7)
    x64 = w.x64() if w.B * w.N * w.d <= 4e8 else None
    if x64 is None:    # very large: widen only the sampled rows
        rows = np.sort(rng.choice(w.N, size=per_batch, replace=False))
        xs = synthdata.to_f64(w.x[:, rows], w.dtype)
        a = oracle.assign(xs, c_hat, form="expanded")
        st = check_ids(ids[:, rows], a, f"{name} sampled rows")
    else:
        st = _sampled_assign_check(x64, c_hat, ids, rng, per_batch)
    print(name, st)


def test_full_size_assign_f32_sweep_shape(fk):
    """One size of the fp32 large-tensor sweep (N = 2^20, K = 1024, d = 128,
    i.i.d. normal points), assigned on the GPU whole, checked on sampled rows."""
    N, K, d = 1 << 20, 1024, 128
    x, init, _ = synthdata.make_mixture(1, N, d, K, "f32", n_comp=0, mean_std=0.0, seed=3020,
                                        iid=True)
    _, _, ids = gpu_norms_assign(fk, to_dev(x, "f32"), init.astype(np.float64), "f32")
    st = _sampled_assign_check(x.astype(np.float64), init.astype(np.float64), ids,
                               np.random.default_rng(9), 1024)
    print(st)


@pytest.mark.parametrize("name,kind", [("api_example", "uniform"), ("split_d", "uniform")])
def test_full_size_update(fk, name, kind):
    torch = _torch()
    w = synthdata.make_workload(name)
    ids = _ids(kind, w.B, w.N, w.K, 11)
    c_old = w.init64().astype(np.float32)
    c_dev = torch.from_numpy(c_old).cuda()
    _, counts, shift = fk.fk_update(to_dev(w.x, w.dtype), torch.from_numpy(ids).cuda(), c_dev)
    torch.cuda.synchronize()
    u = oracle.update(w.x64(), ids, c_old.astype(np.float64))
    np.testing.assert_array_equal(counts.cpu().numpy(), u.counts)
    assert centroid_rel_err(c_dev.cpu().numpy(), u.centers) <= CENTROID_RTOL
    check_shift(shift.cpu().numpy().astype(np.float64), u.shift, u.centers)


def test_full_size_update_hot_clusters(fk):
    """Large-K shape with ids drawn from Zipf(1.1): hottest segment ~14% of N."""
    torch = _torch()
    w = synthdata.make_workload("large_k_zipf")
    ids = synthdata.zipf_ids(1, w.N, w.K, 12)
    c_old = w.init64().astype(np.float32)
    c_dev = torch.from_numpy(c_old).cuda()
    _, counts, _ = fk.fk_update(to_dev(w.x, w.dtype), torch.from_numpy(ids).cuda(), c_dev)
    torch.cuda.synchronize()
    want = np.bincount(ids[0], minlength=w.K)
    np.testing.assert_array_equal(counts.cpu().numpy()[0], want)
    assert want.max() > 0.1 * w.N
    # oracle on a subset of clusters: the hottest 4 and 60 random others
    rng = np.random.default_rng(3)
    pick = np.unique(np.concatenate([np.argsort(want)[-4:], rng.choice(w.K, 60, replace=False)]))
    sel = np.isin(ids[0], pick)
    remap = np.full(w.K, -1)
    remap[pick] = np.arange(pick.size)
    sub = oracle.update(synthdata.to_f64(w.x[0, sel], w.dtype)[None], remap[ids[0, sel]][None],
                        c_old[:, pick].astype(np.float64))
    err = centroid_rel_err(c_dev.cpu().numpy()[:, pick], sub.centers)
    assert err <= CENTROID_RTOL, err


def test_full_size_lloyd_headline(fk):
    """fk_lloyd at the headline size, one iteration: ids against the oracle on
    sampled rows; every non-empty centre is the mean of the points the GPU
    assigned to it (validity of the GPU's own labelling)."""
    w = synthdata.make_workload("api_example")
    ids, centers, n_iter = fk.fk_lloyd(to_dev(w.x, w.dtype), to_dev(w.init, w.dtype), 1, 0.0)
    assert n_iter == 1
    ids = ids.cpu().numpy()
    x64 = w.x64()
    _sampled_assign_check(x64, w.init64(), ids, np.random.default_rng(5), 256)
    cg = centers.cpu().numpy()
    for b in range(0, w.B, 7):
        cnt = np.bincount(ids[b], minlength=w.K)
        sums = np.stack([np.bincount(ids[b], weights=x64[b, :, j], minlength=w.K)
                         for j in range(w.d)], axis=1)
        ne = cnt > 0
        mean = sums[ne] / cnt[ne][:, None]
        assert centroid_rel_err(cg[b][ne], mean) <= CENTROID_RTOL
        np.testing.assert_array_equal(cg[b][~ne], w.init64()[b][~ne])


# ---------------------------------------------------------------------------
# edge cases and error handling
# ---------------------------------------------------------------------------
def test_empty_problems(fk):
    torch = _torch()
    x = torch.empty((2, 0, 16), dtype=torch.float16, device="cuda")
    init = torch.randn((2, 5, 16), device="cuda").half()
    ids, centers, n_iter = fk.fk_lloyd(x, init, 3, 0.0)
    assert n_iter == 3 and ids.numel() == 0
    assert torch.equal(centers, init.float())
    ids, centers, n_iter = fk.fk_lloyd(x, init, 3, 1e-4)
    assert n_iter == 1                         # shift 0 < tol after the first iteration
    c = torch.randn((2, 5, 16), device="cuda")
    c0 = c.clone()
    _, counts, shift = fk.fk_update(x, torch.empty((2, 0), dtype=torch.int32, device="cuda"), c)
    torch.cuda.synchronize()
    assert (counts == 0).all() and (shift == 0).all() and torch.equal(c, c0)
    xb = torch.empty((0, 10, 16), dtype=torch.float16, device="cuda")
    ib = torch.empty((0, 5, 16), dtype=torch.float16, device="cuda")
    assert fk.fk_lloyd(xb, ib, 3, 0.0)[2] == 0


def test_zero_iterations_returns_init(fk):
    torch = _torch()
    w = synthdata.make_workload("tiny_f32")
    ids, centers, n_iter = fk.fk_lloyd(to_dev(w.x, "f32"), to_dev(w.init, "f32"), 0, 0.0)
    assert n_iter == 0 and (ids == 0).all()
    np.testing.assert_array_equal(centers.cpu().numpy(), w.init)


@pytest.mark.parametrize("tol", [0.0, 1e-30])
def test_lloyd_is_deterministic(fk, tol):
    """Long clusters (a 12-component mixture clustered into K = 16, so every
    cluster holds thousands of points and is summed in pieces): ten fk_lloyd
    runs give bit-identical ids, centres and iteration counts, with and
    without the tol test (the deferred division in the norms pass and the
    finalize kernel)."""
    torch = _torch()
    x, init, _ = synthdata.make_mixture(2, 40000, 128, 16, "f16", n_comp=12, mean_std=2.0,
                                        seed=41)
    x_dev, init_dev = to_dev(x, "f16"), to_dev(init, "f16")
    runs = [fk.fk_lloyd(x_dev, init_dev, 6, tol) for _ in range(10)]
    ids0, c0, n0 = runs[0]
    counts = np.bincount(ids0.cpu().numpy()[0], minlength=16)
    assert counts.max() > 4 * 256
    for ids, c, n in runs[1:]:
        assert n == n0
        assert torch.equal(ids, ids0)
        assert torch.equal(c.view(torch.int32), c0.view(torch.int32))


def test_status_codes_through_binding(fk):
    torch = _torch()
    x = torch.randn((1, 100, 16), device="cuda").half()
    init = x[:, :4].contiguous()
    ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(fk.FKError) as e:
        fk.fk_lloyd(x, init, 2, 0.0, ws=ws)
    assert e.value.status == 3
    with pytest.raises(fk.FKError) as e:
        fk.fk_lloyd(x, init, -1, 0.0)
    assert e.value.status == 1


@pytest.mark.parametrize("wl,kw", [("io_breakdown", {}),
                                   ("split_d", {"scale_n": 4096, "B": 2}),
                                   ("tiny_f32", {})])
def test_trace_records_phases(fk, wl, kw):
    """The trace's phases (kernel-stamped norms and assign, update between
    them) are positive and add up to at most the call's own time on the
    stream, and, where the device and not the host's launches sets the pace
    (the whole io_breakdown batch, about 0.6 ms an iteration), to most of
    it."""
    torch = _torch()
    w = synthdata.make_workload(wl, **kw)
    x, init = to_dev(w.x, w.dtype), to_dev(w.init, w.dtype)
    fk.fk_lloyd(x, init, 1, 0.0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fk.fk_trace_begin(8)
    e0.record()
    fk.fk_lloyd(x, init, 5, 0.0)
    e1.record()
    torch.cuda.synchronize()
    tr = fk.fk_trace_end()
    assert tr["iterations"] == 5
    assert tr["assign_ms"] > 0 and tr["update_ms"] > 0 and tr["norms_ms"] > 0
    total = tr["norms_ms"] + tr["assign_ms"] + tr["update_ms"]
    wall = e0.elapsed_time(e1)
    print(wl, f"phases {total:.4f} ms of {wall:.4f} ms")
    assert total <= 1.02 * wall + 0.02
    # the small cases are launch-bound: their kernels take microseconds to
    # tens of microseconds and the stream idles between launches, so only
    # the upper bound holds there
    if wl == "io_breakdown":
        assert 0.5 * wall <= total


def test_trace_over_calls_and_capacity(fk):
    """One trace over two calls, its capacity ending inside the second, and a
    traced run with a tol stop: every traced iteration is counted."""
    w = synthdata.make_workload("io_breakdown", scale_n=20000, B=2)
    x, init = to_dev(w.x, w.dtype), to_dev(w.init, w.dtype)
    fk.fk_trace_begin(3)
    fk.fk_lloyd(x, init, 2, 0.0)
    fk.fk_lloyd(x, init, 2, 0.0)
    tr = fk.fk_trace_end()
    assert tr["iterations"] == 3
    assert min(tr["norms_ms"], tr["assign_ms"], tr["update_ms"]) > 0
    fk.fk_trace_begin(100)
    _, _, n = fk.fk_lloyd(x, init, 100, 1e-3)
    tr = fk.fk_trace_end()
    print(f"tol run: {n} iterations, {tr['iterations']} traced")
    # a tol stop runs one iteration past the stop, then undoes it
    assert 1 <= n <= 100 and tr["iterations"] in (n, n + 1)
    assert min(tr["norms_ms"], tr["assign_ms"], tr["update_ms"]) > 0


# ---------------------------------------------------------------------------
# tile candidates (FK_TILE) and the shard-local partial update
# ---------------------------------------------------------------------------
TILE_CASES = [
    # tile, dtype, B, N, d, K
    ("8w128", "f16", 2, 3000, 128, 1000),     # the ring: eight tiles per point block
    ("8w128", "bf16", 1, 5000, 64, 300),      # 64-unit rows, three tiles, ragged K
    ("8w128", "f16", 1, 2100, 32, 100),       # one tile (no ring), ragged N
    ("4w128", "f16", 2, 3000, 128, 1000),
    ("4w128", "bf16", 3, 2500, 40, 257),      # column-padded rows, a one-row last tile
    ("4w128", "f32", 1, 2000, 64, 200),       # fp32: 128-unit rows
    ("4w64", "f16", 2, 3000, 128, 1000),
    ("4w64", "bf16", 1, 5000, 64, 65),
    ("4w64", "f16", 1, 700, 17, 130),
    ("lds8", "bf16", 2, 3000, 1024, 300),     # split-D candidates
    ("lds4", "bf16", 2, 3000, 1024, 300),     # 128-row tiles: three K tiles
    ("reg8", "f16", 1, 2000, 768, 600),
    ("reg4", "f16", 1, 2000, 640, 200),
    ("lds4", "f32", 1, 1500, 384, 100),
]


@pytest.mark.parametrize("tile,dtype,B,N,d,K", TILE_CASES)
def test_assign_tile_candidates(fk, monkeypatch, tile, dtype, B, N, d, K):
    """Each tile candidate the dispatch table can pick, forced with FK_TILE,
    against the oracle (band rule)."""
    monkeypatch.setenv("FK_TILE", tile)
    monkeypatch.delenv("FK_FORCE_SPLITD", raising=False)
    seed = stable_seed(tile, dtype, B, N, d, K)
    x, _, _ = synthdata.make_mixture(B, N, d, 1, dtype, n_comp=max(2, K // 3), mean_std=1.5,
                                  seed=seed)
    x64 = synthdata.to_f64(x, dtype)
    c_hat = make_centroids(x64, K, dtype, seed + 1)
    _, _, ids = gpu_norms_assign(fk, to_dev(x, dtype), c_hat, dtype)
    a = oracle.assign(x64, c_hat, form="direct" if N * K * d < 2e7 else "expanded")
    print(tile, check_ids(ids, a, f"tile {tile} {dtype} B{B} N{N} d{d} K{K}"))


@pytest.mark.parametrize("dtype,B,N,d,K,shards", [("f16", 2, 30000, 128, 300, 3),
                                                   ("bf16", 1, 50000, 1024, 64, 4),
                                                   ("f32", 1, 9000, 33, 5, 2)])
def test_update_partial_over_shards(fk, dtype, B, N, d, K, shards):
    """fk_update_partial on contiguous row blocks (ragged), accumulated into
    zeroed sums and counts: counts equal the oracle's bit for bit, the means
    sums/counts are within 2e-3 of the oracle's centroids."""
    torch = _torch()
    seed = stable_seed(dtype, B, N, d, K, shards)
    x, _, _ = synthdata.make_mixture(B, N, d, 1, dtype, n_comp=8, mean_std=1.0, seed=seed)
    x64 = synthdata.to_f64(x, dtype)
    ids = _ids("zipf", B, N, K, seed + 1)
    bounds = np.linspace(0, N, shards + 1).astype(int)
    bounds[1:-1] += 7                             # ragged blocks
    sums = torch.zeros((B, K, d), dtype=torch.float32, device="cuda")
    counts = torch.zeros((B, K), dtype=torch.int32, device="cuda")
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        xs = to_dev(np.ascontiguousarray(x[:, lo:hi]), dtype)
        fk.fk_update_partial(xs, torch.from_numpy(np.ascontiguousarray(ids[:, lo:hi])).cuda(),
                             sums, counts)
    torch.cuda.synchronize()
    u = oracle.update(x64, ids, np.zeros((B, K, d)))
    np.testing.assert_array_equal(counts.cpu().numpy(), u.counts)
    ne = u.counts > 0
    means = sums.cpu().numpy()[ne] / u.counts[ne][:, None]
    err = centroid_rel_err(means[None], u.centers[ne][None])
    assert err <= CENTROID_RTOL, err
