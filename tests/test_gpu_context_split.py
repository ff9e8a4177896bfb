"""Decode over a context split into key ranges, joined by pa_merge_states.

A very long context can be spread over several GPUs by contiguous ranges of
its logical blocks.  Each GPU runs pa_decode_lse on its range and the
partial states are joined with pa_merge_states.  These tests run every
range on the one GPU here: the log-sum-exps must match the oracle's, and the
joined result must match the oracle on the whole context."""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_decode_amd import workloads as W
from tests.gpu_helpers import assert_close_f32_out, case_to_dev, out_to_f64, to_dev

pytestmark = pytest.mark.gpu

LSE_TOL = 1e-4  # natural log; fp32 scores over at most ~10^5 keys


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_decode_amd import binding
    binding.lib()
    return binding


def assert_lse_close(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    inf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf_ref), f"{what}: -inf pattern differs"
    err = np.abs(got[~inf_ref] - ref[~inf_ref])
    assert (err.max() if err.size else 0.0) <= LSE_TOL, f"{what}: lse error {err.max():.2e}"


@pytest.mark.parametrize("workers", ["", "7", "300"])
@pytest.mark.parametrize("dtype,G", [("bf16", 4), ("f16", 8), ("f32", 2)])
def test_decode_lse_matches_oracle(pa, monkeypatch, workers, dtype, G):
    if workers:
        monkeypatch.setenv("PA_DECODE_WORKERS", workers)
    else:
        monkeypatch.delenv("PA_DECODE_WORKERS", raising=False)
    d = 64 if dtype == "f32" else 128
    c = W.make_decode_case(1400 + G, 9, 2 * G, 2, d, 16, dtype,
                           lens=[0, 1, 16, 17, 333, 1000, 2500, 0, 64])
    dev = case_to_dev(c)
    out, lse = pa.decode_lse(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                             dev["context_lens"], c.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens,
                                 c.scale, c.dtype)
    what = f"{dtype} G={G} workers={workers or 'default'}"
    assert_close_f32_out(out_to_f64(out), ref, dtype, what)
    assert_lse_close(lse.cpu().numpy(), ref_lse, what)
    # The output is pa_decode's, bit for bit.
    plain = pa.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                      dev["context_lens"], c.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(plain, out)


def split_by_blocks(c, cuts):
    """Tables and lengths of the key ranges [cuts[p] * B, cuts[p+1] * B) of
    every sequence (cuts in blocks; ranges past a sequence's end are empty)."""
    B = c.block_size
    parts = []
    for b0, b1 in zip(cuts[:-1], cuts[1:]):
        tab = np.zeros((c.block_table.shape[0], max(1, b1 - b0)), np.int32)
        w = min(b1, c.block_table.shape[1]) - b0
        if w > 0:
            tab[:, :w] = c.block_table[:, b0:b0 + w]
        lens = np.clip(c.context_lens.astype(np.int64) - b0 * B, 0, (b1 - b0) * B)
        parts.append((tab, lens.astype(np.int32)))
    return parts


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_context_split_and_merge(pa, out_dtype):
    c = W.make_decode_case(1410, 6, 32, 8, 128, 16, "bf16",
                           lens=[3000, 17, 1200, 0, 2049, 640])
    dev = case_to_dev(c)
    cuts = [0, 20, 21, 90, 200]  # block ranges of unequal size; some empty
    outs, lses = [], []
    for tab, lens in split_by_blocks(c, cuts):
        o, l = pa.decode_lse(dev["q"], dev["k_pool"], dev["v_pool"], to_dev(tab),
                             to_dev(lens), c.scale, out_dtype=torch.float32)
        outs.append(o)
        lses.append(l)
    part_out, part_lse = torch.stack(outs), torch.stack(lses)
    out, lse = pa.merge_states(part_out, part_lse, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens,
                                 c.scale, c.dtype)
    if out_dtype == torch.float32:
        assert_close_f32_out(out_to_f64(out), ref, "bf16", "merged")
    else:
        from tests.gpu_helpers import assert_close_native_out
        assert_close_native_out(out_to_f64(out), ref, "bf16", "merged, bf16 out")
    assert_lse_close(lse.cpu().numpy(), ref_lse, "merged")
    # One part is the identity; a part order change moves only rounding.
    one, one_lse = pa.merge_states(part_out[:1].contiguous(), part_lse[:1].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(one, part_out[0])
    assert torch.equal(torch.nan_to_num(one_lse, neginf=-1e30),
                       torch.nan_to_num(part_lse[0], neginf=-1e30))


def test_long_context_eight_way_share(pa):
    """The long-context workload (4 x 100,000 keys) as eight block ranges,
    each one GPU's share, joined: sampled rows against the oracle."""
    c = W.long_bf16_decode()
    dev = case_to_dev(c)
    nblk = -(-100_000 // 16)
    cuts = [round(i * nblk / 8) for i in range(9)]
    outs, lses = [], []
    for tab, lens in split_by_blocks(c, cuts):
        o, l = pa.decode_lse(dev["q"], dev["k_pool"], dev["v_pool"], to_dev(tab),
                             to_dev(lens), c.scale, out_dtype=torch.float32)
        outs.append(o)
        lses.append(l)
    out, lse = pa.merge_states(torch.stack(outs), torch.stack(lses))
    torch.cuda.synchronize()
    got, got_lse = out_to_f64(out), lse.cpu().numpy()
    rng = np.random.default_rng(3)
    for s, h in [(0, 0), (3, 31), *[(int(rng.integers(4)), int(rng.integers(32)))
                                    for _ in range(4)]]:
        ref, ref_lse, _ = oracle.decode_row(c.q, c.k_pool, c.v_pool, c.block_table,
                                            c.context_lens, c.scale, c.dtype, s, h)
        assert_close_f32_out(got[s, h], ref, "bf16", f"8-way s={s} h={h}")
        assert abs(got_lse[s, h] - ref_lse) <= LSE_TOL, (s, h, got_lse[s, h], ref_lse)
