"""Results must not depend on what the workspace held before a call: every
kernel that reads workspace memory first writes it (or a kernel before it
clears it). Each update and loop runs twice, on a workspace filled with
0xFF bytes (NaN floats, -1 ints) and on a zeroed one; ids, counts, centres
and shift must agree bit for bit. The shapes reach every perm builder: the
direct LDS scatter, the per-chunk LDS sort, the radix passes after a large
count matrix (forced), the histogram above one LDS bin range, and
long-cluster pieces with block sums."""
import numpy as np
import pytest

import synthdata
from gpu_helpers import to_dev

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


UPDATE_SHAPES = [
    # dtype, B, N, d, K, ids kind, forced radix
    ("f16", 2, 20000, 128, 1000, "uniform", False),    # direct scatter
    ("f16", 1, 40000, 64, 5000, "zipf", False),        # per-chunk LDS sort
    ("bf16", 3, 120000, 32, 3000, "uniform", True),    # radix after a large count matrix
    ("f16", 1, 30000, 48, 40000, "uniform", False),    # K above one LDS bin range
    ("f32", 1, 300000, 36, 3, "zipf", False),          # long pieces with Q1/Q2 block sums
]


def _ids(kind, B, N, K, seed):
    return synthdata.uniform_ids(B, N, K, seed) if kind == "uniform" else synthdata.zipf_ids(B, N, K, seed)


@pytest.mark.parametrize("dtype,B,N,d,K,kind,radix", UPDATE_SHAPES)
def test_update_ignores_workspace_contents(fk, monkeypatch, dtype, B, N, d, K, kind, radix):
    torch = _torch()
    if radix:
        monkeypatch.setenv("FK_FORCE_RADIX", "1")
    else:
        monkeypatch.delenv("FK_FORCE_RADIX", raising=False)
    x, _, _ = synthdata.make_mixture(B, N, d, 1, dtype, n_comp=8, mean_std=1.0, seed=K + N)
    ids = torch.from_numpy(_ids(kind, B, N, K, K + 1)).cuda()
    c0 = np.random.default_rng(K).standard_normal((B, K, d)).astype(np.float32)
    xd = to_dev(x, dtype)
    outs = []
    for fill in (0xFF, 0x00):
        ws = fk.workspace(xd.dtype, B, N, d, K, xd.device)
        ws.fill_(fill)
        c = torch.from_numpy(c0).cuda()
        _, counts, shift = fk.fk_update(xd, ids, c, ws=ws)
        torch.cuda.synchronize()
        outs.append((c.cpu().numpy(), counts.cpu().numpy(), shift.cpu().numpy()))
    for a, b in zip(outs[0], outs[1]):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("wl,kw", [("io_breakdown", {"scale_n": 20000, "B": 2}),
                                   ("split_d", {"scale_n": 4096, "B": 2})])
def test_lloyd_ignores_workspace_contents(fk, wl, kw):
    torch = _torch()
    w = synthdata.make_workload(wl, **kw)
    x, init = to_dev(w.x, w.dtype), to_dev(w.init, w.dtype)
    outs = []
    for fill in (0xFF, 0x00):
        ws = fk.workspace(x.dtype, w.B, w.N, w.d, w.K, x.device)
        ws.fill_(fill)
        ids, centers, n = fk.fk_lloyd(x, init, 4, 0.0, ws=ws)
        torch.cuda.synchronize()
        outs.append((ids.cpu().numpy(), centers.cpu().numpy(), n))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])
    assert outs[0][2] == outs[1][2] == 4
