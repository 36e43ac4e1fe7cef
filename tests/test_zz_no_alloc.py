"""fk_update_noalloc (the update with the library's own device scratch, no
workspace argument) against fk_update, through the C ABI: two calls in a
row, the second on a smaller problem, each bit-identical to fk_update on the
same inputs (the update is deterministic); sizes beyond the scratch are
rejected before anything runs."""
import numpy as np
import pytest

import synthdata
from gpu_helpers import to_dev

pytestmark = pytest.mark.gpu


def _case(B, N, d, K, dtype, seed):
    x, _, _ = synthdata.make_mixture(B, N, d, 1, dtype, n_comp=6, mean_std=1.0, seed=seed)
    ids = synthdata.zipf_ids(B, N, K, seed + 1)
    c0 = np.random.default_rng(seed + 2).standard_normal((B, K, d)).astype(np.float32)
    return x, ids, c0


def _both(fk, x, ids, c0, dtype):
    import torch
    x_dev, ids_dev = to_dev(x, dtype), torch.from_numpy(ids).cuda()
    B, K = c0.shape[0], c0.shape[1]
    c_ref = torch.from_numpy(c0).cuda()
    _, cnt_ref, sh_ref = fk.fk_update(x_dev, ids_dev, c_ref)
    c_na = torch.from_numpy(c0).cuda()
    cnt_na = torch.empty((B, K), dtype=torch.int32, device="cuda")
    sh_na = torch.empty((B,), dtype=torch.float32, device="cuda")
    fk.fk_update_noalloc(x_dev, ids_dev, c_na, cnt_na, sh_na)
    torch.cuda.synchronize()
    return (c_ref, cnt_ref, sh_ref), (c_na, cnt_na, sh_na)


def test_noalloc_matches_fk_update_twice(fk):
    import torch
    for (B, N, d, K, dtype, seed) in [(4, 60000, 128, 500, "f16", 71),
                                      (2, 9000, 96, 70, "bf16", 72)]:
        tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
        assert fk.fk_workspace_size(tdt, B, N, d, K) <= fk.FK_NOALLOC_SCRATCH_BYTES
        x, ids, c0 = _case(B, N, d, K, dtype, seed)
        ref, na = _both(fk, x, ids, c0, dtype)
        assert torch.equal(na[1], ref[1])
        assert torch.equal(na[0].view(torch.int32), ref[0].view(torch.int32))
        assert torch.equal(na[2].view(torch.int32), ref[2].view(torch.int32))
        print(f"noalloc B{B} N{N} d{d} K{K} {dtype}: bit-identical to fk_update")


def test_noalloc_rejects_sizes_beyond_scratch(fk):
    import torch
    # the long-segment slots alone are B*N*d/32 bytes: 64 MiB here (x is 4 GiB,
    # allocated but never read: the call is refused first)
    B, N, d, K = 1, 1 << 21, 1024, 8
    assert fk.fk_workspace_size(torch.float16, B, N, d, K) > fk.FK_NOALLOC_SCRATCH_BYTES
    x = torch.empty((B, N, d), dtype=torch.float16, device="cuda")
    ids = torch.zeros((B, N), dtype=torch.int32, device="cuda")
    c = torch.zeros((B, K, d), dtype=torch.float32, device="cuda")
    counts = torch.full((B, K), -7, dtype=torch.int32, device="cuda")
    shift = torch.zeros((B,), dtype=torch.float32, device="cuda")
    with pytest.raises(fk.FKError) as e:
        fk.fk_update_noalloc(x, ids, c, counts, shift)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert (counts == -7).all()           # nothing ran
