"""Shared helpers for the GPU parity tests (comparison rules, tensor moves).

Comparison rules (from the stated tolerances):
  * ids: equal to the oracle's except at points inside the near-tie band, where
    the GPU id must be one of the oracle's acceptable ids (all centroids whose
    distance is within 1e-3*(||x||^2 + ||c_best||^2) of the best);
  * counts: bit-exact;
  * centroids: per-centroid max-norm relative error
      max_k ||c_gpu[k] - c_ref[k]||_inf / max(||c_ref[k]||_inf, 1e-6)  <= 2e-3;
  * the loop's shift: |sqrt(s_gpu) - sqrt(s_ref)| <= 4e-3*||c_new||_F + 1e-30,
    which follows from the centroid tolerance by the triangle inequality
    (the difference matrices differ by at most the two centroid errors).
"""
import numpy as np

import synthdata

CENTROID_RTOL = 2e-3


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def to_dev(arr: np.ndarray, dtype: str):
    return synthdata.to_torch(arr, dtype).cuda()


def f64_to_storage(a64: np.ndarray, dtype: str) -> np.ndarray:
    """Values already representable in dtype -> storage array (exact)."""
    if dtype == "f32":
        out = a64.astype(np.float32)
    elif dtype == "f16":
        out = a64.astype(np.float16)
    else:
        out = (a64.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    assert np.array_equal(synthdata.to_f64(out, dtype), a64), "not representable"
    return out


def host_f64(t, dtype: str) -> np.ndarray:
    """Device tensor in dtype -> exact float64 array."""
    import torch
    if dtype == "bf16":
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return synthdata.to_f64(bits, "bf16")
    return t.cpu().numpy().astype(np.float64)


def check_ids(gpu_ids: np.ndarray, a, where: str = "", rows=None) -> dict:
    """Band rule for ids; ``rows`` maps local row j -> (b, n) key for a.near."""
    gpu = np.asarray(gpu_ids, dtype=np.int64)
    mism = np.argwhere(gpu != a.ids)
    bad = []
    for b, n in mism:
        key = (int(b), int(n))
        ok = a.near.get(key)
        if ok is None or int(gpu[b, n]) not in set(int(v) for v in ok):
            bad.append((key, int(gpu[b, n]), int(a.ids[b, n]), float(a.gap[b, n]),
                        float(a.band[b, n])))
    assert not bad, f"{where}: {len(bad)} ids outside the near-tie band; first {bad[:4]}"
    return {"n": int(gpu.size), "n_band": int(a.n_band()), "n_flip_in_band": int(len(mism))}


def centroid_rel_err(c_gpu: np.ndarray, c_ref: np.ndarray) -> float:
    if c_ref.size == 0:
        return 0.0
    num = np.abs(np.asarray(c_gpu, np.float64) - c_ref).max(axis=-1)
    den = np.maximum(np.abs(c_ref).max(axis=-1), 1e-6)
    return float((num / den).max())


def check_shift(s_gpu: np.ndarray, s_ref: np.ndarray, c_new_ref: np.ndarray, where=""):
    fro = np.sqrt(np.einsum("bkd,bkd->b", c_new_ref, c_new_ref))
    err = np.abs(np.sqrt(np.maximum(s_gpu, 0)) - np.sqrt(s_ref))
    assert (err <= 2 * CENTROID_RTOL * fro + 1e-30).all(), (where, s_gpu, s_ref)
