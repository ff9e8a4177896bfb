"""Every output of the three largest workloads against the CPU oracle.

* long-bf16-decode: 4 sequences x 100,000 keys, 32/8 heads, d = 128, bf16;
* causal-bf16-prefill: 8 prompts of 512..4096 tokens, 32/8 heads, bf16;
* prefix-shared-bf16-decode: 256 sequences sharing a 2048-token prefix, at
  block sizes 16, 32, 64 and 128, through plain pa_decode and through
  pa_decode_shared_prefix.

All compare the fp32 output element by element with the fp64 oracle at
max-abs 2e-3 (16-bit inputs, fp32 accumulation), and record the largest
error under the workload's name (reported at the end of the session when
PA_PARITY_REPORT names a file).  The prefix-shared workload holds the same
logical q, K, V and lengths at every block size; the oracle iterates
logical tokens, so its result does not depend on the block size (pinned
bit for bit by tests/test_oracle_pins.py) and is computed once.
"""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_decode_amd import workloads as W
from tests.gpu_helpers import assert_close_f32_out, assert_close_native_out, case_to_dev, out_to_f64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_decode_amd import binding
    binding.lib()
    return binding


def oracle_decode(c):
    return oracle.decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale,
                         c.dtype)[0]


def test_long_bf16_decode_full(pa):
    """4 x 100,000 keys, bf16: all 4 x 32 outputs, fp32 and bf16 out."""
    c = W.long_bf16_decode()
    dev = case_to_dev(c)
    got = out_to_f64(pa.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                               dev["context_lens"], c.scale, out_dtype=torch.float32))
    nat = out_to_f64(pa.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                               dev["context_lens"], c.scale))
    torch.cuda.synchronize()
    del dev
    ref = oracle_decode(c)
    assert_close_f32_out(got, ref, "bf16", "long-bf16-decode", record="long-bf16-decode")
    assert_close_native_out(nat, ref, "bf16", "long-bf16-decode bf16 out")


def test_causal_bf16_prefill_full(pa):
    """8 prompts of 512..4096 tokens, causal, bf16: every (row, head) output."""
    c = W.causal_bf16_prefill()
    dev = case_to_dev(c)
    args = (dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"], dev["context_lens"],
            dev["query_start_loc"], c.max_query_len, c.scale)
    got = out_to_f64(pa.prefill(*args, causal=True, out_dtype=torch.float32))
    nat = out_to_f64(pa.prefill(*args, causal=True))
    torch.cuda.synchronize()
    del dev
    ref, _ = oracle.prefill(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens,
                            c.query_start_loc, c.scale, True, c.dtype)
    assert_close_f32_out(got, ref, "bf16", "causal-bf16-prefill", record="causal-bf16-prefill")
    assert_close_native_out(nat, ref, "bf16", "causal-bf16-prefill bf16 out")


@pytest.fixture(scope="module")
def prefix_ref():
    c = W.prefix_shared_bf16_decode(16)
    return c, oracle_decode(c)


@pytest.mark.parametrize("B", [16, 32, 64, 128])
def test_prefix_shared_full(pa, prefix_ref, B):
    """256 sequences over a shared 2048-token prefix: every output of plain
    decode and of the shared-prefix call, at block size B."""
    c16, ref = prefix_ref
    c = c16 if B == 16 else W.prefix_shared_bf16_decode(B)
    # Only the paging differs between block sizes.
    assert np.array_equal(c.q, c16.q) and np.array_equal(c.context_lens, c16.context_lens)
    dev = case_to_dev(c)
    args = (dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"], dev["context_lens"])
    plain = out_to_f64(pa.decode(*args, c.scale, out_dtype=torch.float32))
    shared = out_to_f64(pa.decode_shared_prefix(*args, c.meta["prefix_len"], c.scale,
                                                out_dtype=torch.float32))
    shared_nat = out_to_f64(pa.decode_shared_prefix(*args, c.meta["prefix_len"], c.scale))
    torch.cuda.synchronize()
    name = f"prefix-shared-bf16-decode-B{B}"
    assert_close_f32_out(plain, ref, "bf16", name + " pa_decode", record=name + " pa_decode")
    assert_close_f32_out(shared, ref, "bf16", name + " shared-prefix call",
                         record=name + " pa_decode_shared_prefix")
    assert_close_native_out(shared_nat, ref, "bf16", name + " shared-prefix call, bf16 out")
