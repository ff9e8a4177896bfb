"""pa_decode_noalloc (the decode entry point that allocates nothing: its
workspace is a fixed per-GPU array in the library) against pa_decode.

Both run the same kernels with the same worker count, so their outputs must
be identical bit for bit; the first is also checked against the oracle.  Two
calls in a row, the second on a smaller input (fewer units, a smaller
partial region, counters left at zero by the first), and a third larger one
again."""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_decode_amd import workloads as W
from tests.gpu_helpers import assert_close_f32_out, case_to_dev, out_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_decode_amd import binding
    binding.lib()
    return binding


def run_both(pa, c):
    d = case_to_dev(c)
    args = (d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"], c.scale)
    got = pa.decode_noalloc(*args, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = pa.decode(*args, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return got, ref


def test_noalloc_matches_decode_on_consecutive_calls(pa):
    big = W.make_decode_case(901, 48, 32, 8, 128, 16, "bf16", len_range=(1, 4000))
    small = W.make_decode_case(902, 5, 32, 8, 128, 16, "bf16", lens=[0, 17, 3000, 700, 9000])
    got, ref = run_both(pa, big)
    assert torch.equal(got, ref), "first call differs from pa_decode"
    want = oracle.decode(big.q, big.k_pool, big.v_pool, big.block_table, big.context_lens,
                         big.scale, big.dtype)[0]
    assert_close_f32_out(out_to_f64(got), want, "bf16", "noalloc vs oracle")
    got, ref = run_both(pa, small)
    assert torch.equal(got, ref), "second (smaller) call differs from pa_decode"
    want = oracle.decode(small.q, small.k_pool, small.v_pool, small.block_table,
                         small.context_lens, small.scale, small.dtype)[0]
    assert_close_f32_out(out_to_f64(got), want, "bf16", "noalloc (smaller) vs oracle")
    assert np.all(out_to_f64(got)[0] == 0)  # the empty context
    got, ref = run_both(pa, big)
    assert torch.equal(got, ref), "third call differs from pa_decode"


def test_noalloc_native_out_and_f32(pa):
    for c in (W.make_decode_case(903, 7, 8, 2, 64, 32, "f32", len_range=(1, 2000)),
              W.make_decode_case(904, 9, 16, 2, 128, 64, "f16", len_range=(1, 3000))):
        d = case_to_dev(c)
        args = (d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"], c.scale)
        got = pa.decode_noalloc(*args)
        ref = pa.decode(*args)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), c.dtype


def test_noalloc_rejects_oversize_without_launching(pa, monkeypatch):
    c = W.make_decode_case(905, 4, 8, 2, 128, 16, "bf16", len_range=(1, 500))
    d = case_to_dev(c)
    monkeypatch.setenv("PA_DECODE_WORKERS", "100000")
    out = torch.full(c.q.shape, 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(pa.PAError) as e:
        pa.decode_noalloc(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"],
                          c.scale, out=out)
    assert e.value.status == -6
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
