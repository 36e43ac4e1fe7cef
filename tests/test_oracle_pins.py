"""Pins for the CPU oracle: each function checked against something other than itself.

Sources of truth used here (none re-uses the oracle's own code):
  * exact rational arithmetic (``fractions``) on tiny inputs: rounding,
    distances, ties, means;
  * library routines: scikit-learn ``pairwise_distances_argmin`` and
    ``KMeans(algorithm="lloyd")``, torch's fp32->bf16 cast;
  * closed forms (K=1, d=1 midpoints, K=N with centroids at the points);
  * invariants (objective monotone, its rounding slack, permutation and batch
    independence, integer-exact fp16 sums);
  * a hand-worked example under tests/golden/.
The last block plants plausible mistakes in copies of oracle functions and
checks that the pins catch every one of them.
"""
import json
import math
import os
import warnings
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import kmeans as L
import synthdata

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

FORMATS = {  # significant bits, min normal exponent, max exponent
    "f16": (11, -14, 15),
    "bf16": (8, -126, 127),
    "f32": (24, -126, 127),
}


# --------------------------------------------------------------------------
# exact rational helpers (independent of the oracle)
# --------------------------------------------------------------------------
def rne_fraction(v: Fraction, fmt: str):
    """Round a rational to the nearest representable value (ties to even)."""
    p, emin, emax = FORMATS[fmt]
    if v == 0:
        return Fraction(0)
    s = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - p + 1)
    q = a / ulp
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    if r > (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax:
        return math.inf * s
    return s * r


def frac_assign(x, c):
    """Exact nearest-centroid ids (lowest index on ties) for one problem."""
    xs = [[Fraction(float(v)) for v in row] for row in x]
    cs = [[Fraction(float(v)) for v in row] for row in c]
    ids = []
    for row in xs:
        best, bi = None, -1
        for k, cr in enumerate(cs):
            dist = sum((a - b) ** 2 for a, b in zip(row, cr))
            if best is None or dist < best:
                best, bi = dist, k
        ids.append(bi)
    return np.array(ids)


def frac_means(x, ids, K):
    out = {}
    for k in range(K):
        rows = [x[n] for n in range(len(ids)) if ids[n] == k]
        if rows:
            out[k] = [sum(Fraction(float(r[j])) for r in rows) / len(rows)
                      for j in range(len(rows[0]))]
    return out


def representable_grid(rng, fmt, n, lo_exp=-3, hi_exp=4):
    """Random values exactly representable in fmt (moderate exponents)."""
    p = FORMATS[fmt][0]
    e = rng.integers(lo_exp, hi_exp, size=n)
    m = rng.integers(2 ** (p - 1), 2 ** p, size=n)
    s = rng.choice([-1.0, 1.0], size=n)
    return s * np.ldexp(m.astype(np.float64), e - (p - 1))


# --------------------------------------------------------------------------
# pin helpers: each takes the function under test, so mutants can be fed in
# --------------------------------------------------------------------------
def pin_rounding(round_fn, fmt, seed=0):
    rng = np.random.default_rng(seed)
    p, emin, emax = FORMATS[fmt]
    vals = list(rng.standard_normal(300) * 10.0 ** rng.integers(-6, 6, 300))
    # exact midpoints between neighbours (ties) and just beside them
    grid = representable_grid(rng, fmt, 200, -2, 6)
    for g in grid:
        ulp = 2.0 ** (math.frexp(abs(g))[1] - p)
        mid = g + math.copysign(ulp / 2, g)
        vals += [mid, np.nextafter(mid, 0.0), np.nextafter(mid, np.inf)]
    # subnormals and the overflow edge
    tiny = 2.0 ** (emin - p + 1)
    vals += [tiny * k for k in (0.25, 0.5, 0.75, 1, 1.5, 2.5, 3.5, 7.25)]
    big = (2 - 2.0 ** (1 - p)) * 2.0 ** emax
    half_ulp_top = 2.0 ** (emax - p)
    vals += [big, big + half_ulp_top * 0.999, big + half_ulp_top, -big - half_ulp_top]
    vals += [0.0, -0.0]
    a = np.array(vals, dtype=np.float64)
    got = round_fn(a, fmt)
    for v, g in zip(a, got):
        want = rne_fraction(Fraction(float(v)), fmt)
        if isinstance(want, float):
            assert math.isinf(g) and math.copysign(1, g) == math.copysign(1, want), (v, g)
        else:
            assert Fraction(float(g)) == want, (fmt, v, g, float(want))


def pin_assign_fractions(assign_fn, seed=1, form="direct"):
    rng = np.random.default_rng(seed)
    for trial in range(6):
        N, K, d = int(rng.integers(8, 48)), int(rng.integers(1, 8)), int(rng.integers(1, 7))
        x = representable_grid(rng, "f16", N * d, -2, 2).reshape(1, N, d)
        c = x[0, rng.choice(N, size=K, replace=K > N)].copy()
        if K >= 3:
            c[2] = c[0]                      # duplicate centroid: exact ties
        # a point exactly halfway between centroid 0 and another one
        if K >= 2:
            x[0, 0] = (c[0] + c[1]) / 2
        ids = assign_fn(x, c[None], form=form).ids[0]
        np.testing.assert_array_equal(ids, frac_assign(x[0], c), err_msg=f"trial {trial}")


def pin_update_fractions(update_fn, seed=2):
    rng = np.random.default_rng(seed)
    for trial in range(5):
        N, K, d = int(rng.integers(5, 40)), int(rng.integers(1, 9)), int(rng.integers(1, 6))
        x = representable_grid(rng, "f16", N * d).reshape(1, N, d)
        ids = rng.integers(0, K, size=(1, N))
        c_old = representable_grid(rng, "f16", K * d).reshape(1, K, d)
        u = update_fn(x, ids, c_old)
        means = frac_means(x[0], ids[0], K)
        shift = Fraction(0)
        for k in range(K):
            cnt = int((ids[0] == k).sum())
            assert u.counts[0, k] == cnt
            if cnt:
                want = means[k]
                # exact sum, one correctly rounded division
                assert all(float(w) == float(g) for w, g in zip(want, u.centers[0, k]))
                shift += sum((w - Fraction(float(o))) ** 2 for w, o in zip(want, c_old[0, k]))
            else:
                np.testing.assert_array_equal(u.centers[0, k], c_old[0, k])
        assert abs(Fraction(float(u.shift[0])) - shift) <= shift * Fraction(1, 10 ** 12) + \
            Fraction(1, 10 ** 300)


def pin_golden(lloyd_fn):
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        x = np.array(case["x"], dtype=np.float64)
        c0 = np.array(case["init"], dtype=np.float64)
        res = lloyd_fn(x, c0, case["max_iter"], case["tol"], case["dtype"], record=True)
        assert res.n_iter == case["n_iter"], case["name"]
        for t, want in enumerate(case["iterations"]):
            tr = res.trace[t]
            np.testing.assert_array_equal(tr["assign"].ids[0], want["ids"])
            np.testing.assert_array_equal(tr["counts"][0], want["counts"])
            wc = np.array([[float(Fraction(v)) for v in row] for row in want["centers"]])
            np.testing.assert_array_equal(tr["centers"][0], wc)
            assert tr["shift"][0] == pytest.approx(float(Fraction(want["shift"])), rel=1e-14,
                                                   abs=0)


# --------------------------------------------------------------------------
# round_to_dtype
# --------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", ["f16", "bf16", "f32"])
def test_rounding_exact_rational(fmt):
    pin_rounding(oracle.round_to_dtype, fmt)


def test_bf16_rounding_matches_torch_cast_of_fp32():
    import torch

    rng = np.random.default_rng(3)
    a32 = (rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000)).astype(np.float32)
    want = torch.from_numpy(a32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_to_dtype(a32.astype(np.float64), "bf16"), want)


def test_generator_bf16_storage_matches_torch():
    import torch

    rng = np.random.default_rng(4)
    a32 = (rng.standard_normal(5000) * 100).astype(np.float32)
    bits = synthdata.to_storage(a32, "bf16")
    want = torch.from_numpy(a32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, want)


# --------------------------------------------------------------------------
# assign
# --------------------------------------------------------------------------
@pytest.mark.parametrize("form", ["direct", "expanded"])
def test_assign_exact_rational(form):
    pin_assign_fractions(oracle.assign, form=form)


def test_assign_matches_sklearn():
    from sklearn.metrics import pairwise_distances_argmin

    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 3000, 24))
    c = rng.standard_normal((2, 97, 24))
    for form in ("direct", "expanded"):
        a = oracle.assign(x, c, form=form)
        for b in range(2):
            ref = pairwise_distances_argmin(x[b], c[b])
            clear = a.gap[b] > 1e-9 * (a.band[b] / 1e-3)
            assert clear.mean() > 0.99
            np.testing.assert_array_equal(a.ids[b][clear], ref[clear])


def test_assign_closed_forms():
    rng = np.random.default_rng(6)
    # K = 1: everyone in cluster 0, gap infinite
    x = rng.standard_normal((2, 50, 5))
    a = oracle.assign(x, rng.standard_normal((2, 1, 5)))
    assert (a.ids == 0).all() and np.isinf(a.gap).all()
    # K = N with centroids at the (distinct) points: id[n] = n, distance 0
    a = oracle.assign(x, x.copy())
    np.testing.assert_array_equal(a.ids, np.tile(np.arange(50), (2, 1)))
    assert (a.dmin == 0).all()
    # d = 1: nearest centroid from the sorted midpoints
    c = np.sort(rng.choice(np.arange(-500, 500), 40, replace=False)).astype(np.float64) / 8
    perm = rng.permutation(40)
    cp = c[perm]
    xs = rng.uniform(-70, 70, 4000)
    mids = (c[1:] + c[:-1]) / 2
    xs = xs[~np.isin(xs, mids)]
    pos = np.searchsorted(mids, xs)          # sorted rank of the nearest centroid
    inv = np.argsort(perm)
    want = inv[pos]
    for form in ("direct", "expanded"):
        a = oracle.assign(xs[None, :, None], cp[None, :, None], form=form)
        np.testing.assert_array_equal(a.ids[0], want)


def test_assign_near_sets_are_the_band():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, 400, 8)).astype(np.float16).astype(np.float64)
    c = x[:, :60].copy()
    c[0, 5] = c[0, 3]
    a = oracle.assign(x, c, form="direct")
    e = oracle.assign(x, c, form="expanded")
    assert set(a.near) == set(e.near) and len(a.near) > 0
    for (b, n), ks in a.near.items():
        D = [float(sum((Fraction(float(p)) - Fraction(float(q))) ** 2
                       for p, q in zip(x[b, n], c[b, k]))) for k in range(60)]
        dm = min(D)
        xx = float(sum(Fraction(float(p)) ** 2 for p in x[b, n]))
        cb = float(sum(Fraction(float(q)) ** 2 for q in c[b, int(np.argmin(D))]))
        band = 1e-3 * (xx + cb)
        np.testing.assert_array_equal(ks, [k for k in range(60) if D[k] - dm < band])
        np.testing.assert_array_equal(e.near[(b, n)], ks)


# --------------------------------------------------------------------------
# update
# --------------------------------------------------------------------------
def test_update_exact_rational():
    pin_update_fractions(oracle.update)


def test_update_integer_exact_fp16_sums():
    rng = np.random.default_rng(8)
    B, N, d, K = 2, 20000, 16, 37
    x = rng.standard_normal((B, N, d)).astype(np.float16).astype(np.float64)
    ids = rng.integers(0, K, size=(B, N))
    u = oracle.update(x, ids, np.zeros((B, K, d)))
    xi = np.rint(x * 2.0 ** 24).astype(np.int64)      # fp16 values are k * 2^-24
    assert (xi.astype(np.float64) == x * 2.0 ** 24).all()
    for b in range(B):
        s = np.zeros((K, d), dtype=np.int64)
        np.add.at(s, ids[b], xi[b])
        np.testing.assert_array_equal(u.sums[b] * 2.0 ** 24, s.astype(np.float64))


def test_update_single_cluster_is_global_mean():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((3, 500, 7)).astype(np.float16).astype(np.float64)
    u = oracle.update(x, np.zeros((3, 500), dtype=np.int64), np.zeros((3, 1, 7)))
    assert (u.counts == 500).all()
    for b in range(3):
        want = [float(sum(Fraction(float(v)) for v in x[b, :, j]) / 500) for j in range(7)]
        np.testing.assert_array_equal(u.centers[b, 0], want)


def test_update_permutation_invariance():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((1, 3000, 9)).astype(np.float16).astype(np.float64)
    ids = rng.integers(0, 12, size=(1, 3000))
    c = rng.standard_normal((1, 12, 9))
    p = rng.permutation(3000)
    u1 = oracle.update(x, ids, c)
    u2 = oracle.update(x[:, p], ids[:, p], c)
    np.testing.assert_array_equal(u1.sums, u2.sums)
    np.testing.assert_array_equal(u1.counts, u2.counts)


# --------------------------------------------------------------------------
# the loop
# --------------------------------------------------------------------------
def test_golden_hand_worked():
    pin_golden(oracle.lloyd)


def test_objective_monotone_real_centroids():
    x, init = synthdata.random_problem(1, 3000, 6, 25, "f16", seed=11, n_comp=12, spread=3.0)
    x64, c0 = synthdata.to_f64(x, "f16"), synthdata.to_f64(init, "f16")
    res = oracle.lloyd(x64, c0, 15, 0.0, "f16", round_centroids=False, record=True)
    J = [tr["J"][0] for tr in res.trace]
    assert all(J[t + 1] <= J[t] * (1 + 1e-12) for t in range(len(J) - 1))
    assert J[-1] < J[0]


def test_objective_slack_rounded_centroids():
    """J_{t+1} <= J_t + sum_k n_k ||c_k - c_hat_k||^2 (mean minimises the in-cluster sum)."""
    for dtype in ("f16", "bf16"):
        x, init = synthdata.random_problem(2, 2000, 8, 30, dtype, seed=12, n_comp=10, spread=2.0)
        x64, c0 = synthdata.to_f64(x, dtype), synthdata.to_f64(init, dtype)
        res = oracle.lloyd(x64, c0, 12, 0.0, dtype, record=True)
        for t in range(len(res.trace) - 1):
            tr, nx = res.trace[t], res.trace[t + 1]
            c_new, c_hat_new = nx["c"], nx["c_hat"]
            slack = np.einsum("bk,bkd->b", tr["counts"], (c_new - c_hat_new) ** 2)
            assert (nx["J"] <= tr["J"] + slack + 1e-9 * tr["J"]).all()
            # the objective of the un-rounded new centres never exceeds J_t
            Jm = oracle.objective(x64, c_new, tr["assign"].ids)
            assert (Jm <= tr["J"] * (1 + 1e-12)).all()


def test_lloyd_matches_sklearn_kmeans():
    from sklearn.cluster import KMeans

    rng = np.random.default_rng(13)
    for trial in range(3):
        K, m = 8, 6
        means = rng.standard_normal((K, 5)) * 4
        x = means[rng.integers(0, K, 1500)] + rng.standard_normal((1500, 5))
        c0 = x[rng.choice(1500, K, replace=False)]
        res = oracle.lloyd(x[None], c0[None], m, 0.0, "f32", round_centroids=False,
                           record=True)
        assert all((tr["counts"] > 0).all() for tr in res.trace)
        with warnings.catch_warnings():
            warnings.simplefilter("ignore")
            km = KMeans(n_clusters=K, init=c0, n_init=1, algorithm="lloyd", tol=0.0,
                        max_iter=m).fit(x)
        np.testing.assert_allclose(res.centers[0], km.cluster_centers_, rtol=1e-9, atol=1e-9)


def test_lloyd_batch_independence_and_tol():
    x, init = synthdata.random_problem(3, 1200, 6, 20, "f16", seed=14, n_comp=8)
    x64, c0 = synthdata.to_f64(x, "f16"), synthdata.to_f64(init, "f16")
    full = oracle.lloyd(x64, c0, 7, 0.0, "f16")
    assert full.n_iter == 7
    for b in range(3):
        one = oracle.lloyd(x64[b:b + 1], c0[b:b + 1], 7, 0.0, "f16")
        np.testing.assert_array_equal(one.ids[0], full.ids[b])
        np.testing.assert_array_equal(one.centers[0], full.centers[b])
    # a generous tol stops after the first iteration; max_iter = 0 returns init
    assert oracle.lloyd(x64, c0, 7, 1e30, "f16").n_iter == 1
    z = oracle.lloyd(x64, c0, 0, 0.0, "f16")
    assert z.n_iter == 0 and np.array_equal(z.centers, c0)


def test_generator_recipes_small():
    w = synthdata.make_workload("io_breakdown", scale_n=4096, B=2)
    assert w.x.shape == (2, 4096, 128) and w.x.dtype == np.float16
    assert w.init.shape == (2, 1024, 128)
    x64 = w.x64()
    for b in range(2):     # init rows are distinct points of the same problem
        rows = {r.tobytes() for r in w.x[b]}
        assert all(r.tobytes() in rows for r in w.init[b])
    w2 = synthdata.make_workload("io_breakdown", scale_n=4096, B=2)
    np.testing.assert_array_equal(w.x, w2.x)
    assert abs(x64.std() - math.sqrt(1 + 4)) < 0.1
    s = synthdata.make_workload("split_d", scale_n=512, B=2)
    assert s.x.dtype == np.uint16 and s.x.shape == (2, 512, 1024)
    t = synthdata.make_workload("tiny_f32")
    np.testing.assert_array_equal(t.init[0], t.x[0, :16])


# --------------------------------------------------------------------------
# planted mistakes: every mutant must fail at least one pin
# --------------------------------------------------------------------------
def _fails(fn, *args, **kw):
    try:
        fn(*args, **kw)
    except AssertionError:
        return True
    return False


def test_pins_catch_planted_rounding_mistakes():
    def truncating(a, fmt):
        a = np.asarray(a, np.float64)
        if fmt != "bf16":
            return oracle.round_to_dtype(a, fmt)
        _, e = np.frexp(a)
        ulp = np.ldexp(1.0, np.maximum(e, -125) - 8)
        return np.trunc(a / ulp) * ulp

    def half_away(a, fmt):
        a = np.asarray(a, np.float64)
        _, e = np.frexp(a)
        p, emin, _ = FORMATS[fmt]
        ulp = np.ldexp(1.0, np.maximum(e, emin + 1) - p)
        return np.sign(a) * np.floor(np.abs(a) / ulp + 0.5) * ulp

    assert _fails(pin_rounding, truncating, "bf16")
    assert _fails(pin_rounding, half_away, "f16")


def test_pins_catch_planted_assign_mistakes():
    real = L.sq_distances

    def highest_index_tie(x, c, **kw):
        r = oracle.assign(x[:, :, :], c[:, ::-1], **kw)
        r.ids = c.shape[1] - 1 - r.ids
        return r

    def no_square(xa, ca):
        return np.abs(np.asarray(xa)[:, None, :] - np.asarray(ca)[None]).sum(-1)

    def sign_flip(xa, ca):
        xa, ca = np.asarray(xa), np.asarray(ca)
        return ((xa[:, None, :] + ca[None]) ** 2).sum(-1)

    assert _fails(pin_assign_fractions, highest_index_tie)
    for bad in (no_square, sign_flip):
        L.sq_distances = bad
        try:
            assert _fails(pin_assign_fractions, oracle.assign)
        finally:
            L.sq_distances = real


def test_pins_catch_planted_update_mistakes():
    def off_by_one(x, ids, c):
        u = oracle.update(x, ids, c)
        nz = u.counts > 0
        u.centers[nz] = u.sums[nz] / (u.counts[nz][:, None] + 1)
        return u

    def empty_to_zero(x, ids, c):
        u = oracle.update(x, ids, c)
        u.centers[u.counts == 0] = 0.0
        return u

    def shift_not_squared(x, ids, c):
        u = oracle.update(x, ids, c)
        u.shift = np.sqrt(u.shift)
        return u

    for bad in (off_by_one, empty_to_zero, shift_not_squared):
        assert _fails(pin_update_fractions, bad), bad.__name__


def test_pins_catch_planted_loop_mistakes():
    def stop_le(x, c0, m, tol, dtype, record=False):
        """The loop with '<=' in place of the strict '<' stop test."""
        c, trace, it = np.asarray(c0, np.float64).copy(), [], 0
        ids = None
        for t in range(m):
            c_hat = oracle.round_to_dtype(c, dtype)
            a = oracle.assign(x, c_hat)
            u = oracle.update(x, a.ids, c)
            trace.append(dict(c=c, c_hat=c_hat, assign=a, counts=u.counts,
                              centers=u.centers, shift=u.shift))
            ids, c, it = a.ids, u.centers, t + 1
            if u.shift.max() <= tol:
                break
        return L.LloydResult(ids, c, it, trace)

    def no_rounding(x, c0, m, tol, dtype, **kw):
        return oracle.lloyd(x, c0, m, tol, dtype, round_centroids=False, **kw)

    assert _fails(pin_golden, stop_le)
    x, init = synthdata.random_problem(1, 500, 8, 12, "f16", seed=15, n_comp=6)
    assert _fails(pin_rounded_centroids, no_rounding, synthdata.to_f64(x, "f16"),
                  synthdata.to_f64(init, "f16"))


def pin_rounded_centroids(lloyd_fn, x64, c0):
    """Every assignment uses centroids representable in the element type (fp16)."""
    res = lloyd_fn(x64, c0, 4, 0.0, "f16", record=True)
    for tr in res.trace:
        np.testing.assert_array_equal(tr["c_hat"], tr["c_hat"].astype(np.float16).astype(np.float64))
        ref = oracle.assign(x64, tr["c_hat"]).ids
        np.testing.assert_array_equal(tr["assign"].ids, ref)
    assert any((tr["c"] != tr["c_hat"]).any() for tr in res.trace[1:])


def test_lloyd_uses_rounded_centroids():
    x, init = synthdata.random_problem(1, 500, 8, 12, "f16", seed=15, n_comp=6)
    pin_rounded_centroids(oracle.lloyd, synthdata.to_f64(x, "f16"), synthdata.to_f64(init, "f16"))


def test_sqnorms_and_objective_exact_rational():
    rng = np.random.default_rng(16)
    c = representable_grid(rng, "bf16", 2 * 5 * 6).reshape(2, 5, 6)
    nrm = oracle.centroid_sqnorms(c)
    for b in range(2):
        for k in range(5):
            assert Fraction(float(nrm[b, k])) == sum(Fraction(float(v)) ** 2 for v in c[b, k])
    x = representable_grid(rng, "f16", 2 * 30 * 6, -2, 2).reshape(2, 30, 6)
    cc = representable_grid(rng, "f16", 2 * 5 * 6, -2, 2).reshape(2, 5, 6)
    ids = rng.integers(0, 5, size=(2, 30))
    J = oracle.objective(x, cc, ids)
    for b in range(2):
        want = sum(sum((Fraction(float(p)) - Fraction(float(q))) ** 2
                       for p, q in zip(x[b, n], cc[b, ids[b, n]])) for n in range(30))
        assert Fraction(float(J[b])) == want
