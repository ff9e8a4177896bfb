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


def case_to_dev(c):
    return dict(q=to_dev(c.q, c.dtype), k_pool=to_dev(c.k_pool, c.dtype),
                v_pool=to_dev(c.v_pool, c.dtype), block_table=to_dev(c.block_table),
                context_lens=to_dev(c.context_lens),
                query_start_loc=None if c.query_start_loc is None else to_dev(c.query_start_loc))


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def assert_close_f32_out(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    worst = float(err.max()) if err.size else 0.0
    assert worst <= TOL[dtype], f"{what}: max-abs error {worst:.3e} > {TOL[dtype]:.1e}"
    return worst


def assert_close_native_out(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    """Outputs stored in the input's 16-bit format: tolerance plus half an ulp
    of that format at the oracle's value."""
    bound = TOL[dtype] + half_ulp(ref, dtype)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs beyond tol+ulp/2, worst excess " \
                          f"{float((err - bound).max()):.3e}"
