"""Shared helpers of the GPU tests: move seeded cases to the device, run the
library through its binding, compare with the oracle."""

from __future__ import annotations

import numpy as np
import torch

from oracle.dtypes import half_ulp

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# Tolerances (max-abs) on fp32 outputs: 1e-5 for fp32 inputs, 2e-3 for 16-bit.
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def to_dev(a: np.ndarray, dtype: str | None = None) -> torch.Tensor:
    """A storage-format numpy array as a GPU tensor of the matching dtype."""
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(TORCH_DT[dtype])
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.cuda()


def pool_to_dev(a: np.ndarray, dtype: str, head_major: bool = False) -> torch.Tensor:
    """A [NB, B, Hkv, d] pool on the GPU; with head_major its memory is a
    contiguous [NB, Hkv, B, d] buffer viewed as [NB, B, Hkv, d]."""
    if not head_major:
        return to_dev(a, dtype)
    return to_dev(np.ascontiguousarray(a.transpose(0, 2, 1, 3)), dtype).permute(0, 2, 1, 3)


def case_to_dev(c, head_major: bool = False):
    return dict(q=to_dev(c.q, c.dtype), k_pool=pool_to_dev(c.k_pool, c.dtype, head_major),
                v_pool=pool_to_dev(c.v_pool, c.dtype, head_major), block_table=to_dev(c.block_table),
                context_lens=to_dev(c.context_lens),
                query_start_loc=None if c.query_start_loc is None else to_dev(c.query_start_loc))


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def assert_close_f32_out(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "",
                         factor: float = 1.0):
    """Max-abs check against TOL[dtype] * factor (factor > 1 only for scores
    larger than the standard scale gives; see score_factor)."""
    tol = TOL[dtype] * factor
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"{what}: max-abs error {worst:.3e} > {tol:.1e}"
    return worst


def score_factor(c) -> float:
    """How far a decode case's scaled scores exceed the standard range.

    The kernels compute the scores s * scale in fp32, so their rounding error
    grows with |s * scale|; the tolerances above hold for the standard
    1/sqrt(d) scale on unit-normal data, where |s * scale| stays below about
    4.  This returns max(1, X / 4), X = the largest |s * scale| over the
    case's attended keys (computed in fp64 from the stored inputs)."""
    from oracle.dtypes import to_f64
    q = to_f64(c.q, c.dtype)
    k = to_f64(c.k_pool, c.dtype)
    S, H, _ = q.shape
    Hkv, B = k.shape[2], k.shape[1]
    G = H // Hkv
    x_max = 0.0
    for s in range(S):
        n = int(c.context_lens[s])
        if n == 0:
            continue
        t = np.arange(n)
        rows = k[c.block_table[s, t // B].astype(np.int64), t % B]  # [n, Hkv, d]
        for h in range(H):
            x_max = max(x_max, float(np.abs(rows[:, h // G] @ q[s, h]).max()) * abs(c.scale))
    return max(1.0, x_max / 4.0)


def assert_close_native_out(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    """Outputs stored in the input's 16-bit format: tolerance plus half an ulp
    of that format at the oracle's value."""
    bound = TOL[dtype] + half_ulp(ref, dtype)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs beyond tol+ulp/2, worst excess " \
                          f"{float((err - bound).max()):.3e}"
