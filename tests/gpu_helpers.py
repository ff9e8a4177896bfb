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


# Worst max-abs error seen per named workload in this session (written to
# the file named by PA_PARITY_REPORT at the end of the session).
MAX_ABS = {}


def record_max_abs(name: str, worst: float):
    MAX_ABS[name] = max(MAX_ABS.get(name, 0.0), float(worst))


def assert_close_f32_out(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "",
                         extra: np.ndarray | float = 0.0, record: str | None = None):
    """Max-abs check against TOL[dtype], plus an optional additive,
    per-element term ``extra`` (see f32_score_rounding_bound).  Returns the
    largest error; with ``record`` it is also kept under that name."""
    bound = TOL[dtype] + np.asarray(extra, dtype=np.float64)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    worst = float(err.max()) if err.size else 0.0
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} outputs beyond the bound, max-abs error "
                           f"{worst:.3e}, worst excess {float((err - bound).max()):.3e} "
                           f"(TOL {TOL[dtype]:.1e})")
    if record:
        record_max_abs(record, worst)
    return worst


U32 = 2.0 ** -24  # unit roundoff of fp32


def f32_score_rounding_bound(c) -> np.ndarray:
    """Additive first-order bound on what forming the scores in fp32 adds to
    a decode output, for a case with fp32 inputs, per element [S, H, d].

    The kernel forms y_t = scale * (q . k_t) by an fp32 dot product of d
    terms and exponentiates y_t - max in fp32.  With u = 2^-24:
      |error of q . k_t| <= gamma_d * A_t,   gamma_d = d u / (1 - d u),
                                           A_t = sum_i |q_i k_ti|;
      multiplying by the rounded scale * log2(e) adds <= 2u |y_t|;
      the subtraction of the maximum adds <= u |y_t - y_max|;
      the exponential adds <= 2^-22 (relative).
    So each weight p_t carries a relative error
      eps_t <= |scale| gamma_d A_t + 2u |y_t| + u |y_t - y_max| + 2^-22,
    and, because the output normalises by the sum of the same weights,
      |delta o_j| <= sum_t p_t eps_t |v_tj - o_j|   (to first order).
    A common shift of every y_t (the maximum's own error) cancels in that
    normalisation.  The term is a worst-case bound (every rounding error
    taken with the same sign) and grows with the scores' size: about 2e-5
    at the standard scale 1/sqrt(d) on unit-normal data (where the
    workloads' fixed 1e-5 applies instead) and up to about 1e-3 at a scale
    of 0.5 or 2 with d = 128."""
    import oracle
    from oracle.dtypes import to_f64
    q = to_f64(c.q, c.dtype)
    kp = to_f64(c.k_pool, c.dtype)
    vp = to_f64(c.v_pool, c.dtype)
    S, H, d = q.shape
    B, Hkv = kp.shape[1], kp.shape[2]
    G = H // Hkv
    gamma = d * U32 / (1.0 - d * U32)
    out = np.zeros((S, H, d))
    for s in range(S):
        n = int(c.context_lens[s])
        if n == 0:
            continue
        t = np.arange(n)
        blk = c.block_table[s, t // B].astype(np.int64)
        for h in range(H):
            k = kp[blk, t % B, h // G]
            v = vp[blk, t % B, h // G]
            o, _, p = oracle.decode_row(c.q, c.k_pool, c.v_pool, c.block_table,
                                        c.context_lens, c.scale, c.dtype, s, h)
            y = c.scale * (k @ q[s, h])
            a = np.abs(k) @ np.abs(q[s, h])
            eps = abs(c.scale) * gamma * a + 2 * U32 * np.abs(y) + U32 * np.abs(y - y.max()) \
                + 2.0 ** -22
            out[s, h] = (p * eps) @ np.abs(v - o)
    return out


def assert_close_native_out(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    """Outputs stored in the input's 16-bit format: tolerance plus half an ulp
    of that format at the oracle's value."""
    bound = TOL[dtype] + half_ulp(ref, dtype)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs beyond tol+ulp/2, worst excess " \
                          f"{float((err - bound).max()):.3e}"
