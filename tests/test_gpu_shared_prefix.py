"""GPU parity of pa_decode_shared_prefix (prefix attended once per KV head on
the matrix cores, suffixes by the decode kernel, log-sum-exp merge) against
the CPU oracle, which knows nothing of the split: it attends every
sequence's full context through its table."""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_decode_amd import workloads as W
from tests.gpu_helpers import (assert_close_f32_out, assert_close_native_out, case_to_dev,
                               out_to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_decode_amd import binding
    binding.lib()
    return binding


def run(pa, c, dev, prefix_len, out_dtype=torch.float32):
    out = pa.decode_shared_prefix(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                                  dev["context_lens"], prefix_len, c.scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


def oracle_all(c):
    return oracle.decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale,
                         c.dtype)[0]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("B", [16, 32, 64, 128])
def test_shared_prefix_small(pa, dtype, B):
    """20 sequences, a 256-token prefix, suffixes of 0 .. 300 tokens (some
    sequences are only the prefix)."""
    c = W.make_prefix_shared_case(700 + B, B, num_seqs=20, prefix_len=256,
                                  suffix_range=(0, 300), dtype=dtype)
    dev = case_to_dev(c)
    ref = oracle_all(c)
    got = out_to_f64(run(pa, c, dev, 256))
    assert_close_f32_out(got, ref, dtype, f"{dtype} B={B}")
    nat = out_to_f64(run(pa, c, dev, 256, out_dtype=dev["q"].dtype))
    assert_close_native_out(nat, ref, dtype, f"{dtype} B={B} native out")


def test_shared_prefix_only_and_empty_suffixes(pa):
    """Every sequence is exactly the prefix (no suffix keys at all)."""
    c = W.make_prefix_shared_case(710, 16, num_seqs=9, prefix_len=512, suffix_range=(0, 0),
                                  dtype="bf16")
    assert (c.context_lens == 512).all()
    dev = case_to_dev(c)
    got = out_to_f64(run(pa, c, dev, 512))
    assert_close_f32_out(got, oracle_all(c), "bf16", "prefix only")


@pytest.mark.parametrize("G,Hkv", [(1, 4), (2, 4), (4, 2), (8, 2)])
def test_shared_prefix_group_sizes(pa, G, Hkv):
    c = W.make_prefix_shared_case(720 + G, 16, num_seqs=70, prefix_len=192,
                                  suffix_range=(1, 130), num_heads=G * Hkv, num_kv_heads=Hkv,
                                  dtype="bf16")
    dev = case_to_dev(c)
    assert_close_f32_out(out_to_f64(run(pa, c, dev, 192)), oracle_all(c), "bf16", f"G={G}")


def test_shared_prefix_zero_is_plain_decode(pa):
    c = W.make_prefix_shared_case(730, 16, num_seqs=12, prefix_len=128, suffix_range=(1, 200),
                                  dtype="bf16")
    dev = case_to_dev(c)
    plain = pa.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                      dev["context_lens"], c.scale, out_dtype=torch.float32)
    assert torch.equal(run(pa, c, dev, 0), plain)
    # A shorter declared prefix (a prefix of the shared part) is also valid.
    assert_close_f32_out(out_to_f64(run(pa, c, dev, 64)), oracle_all(c), "bf16", "prefix 64")


@pytest.mark.parametrize("B", [16, 128])
def test_shared_prefix_full_workload_sampled(pa, B):
    """256 sequences sharing a 2048-token prefix: sampled outputs against
    the oracle, and the whole output against plain pa_decode."""
    c = W.prefix_shared_bf16_decode(B)
    dev = case_to_dev(c)
    got = out_to_f64(run(pa, c, dev, 2048))
    rng = np.random.default_rng(B + 1)
    for s in rng.choice(c.num_seqs, size=6, replace=False):
        for h in rng.choice(32, size=2, replace=False):
            ref, _, _ = oracle.decode_row(c.q, c.k_pool, c.v_pool, c.block_table,
                                          c.context_lens, c.scale, c.dtype, int(s), int(h))
            assert_close_f32_out(got[s, h], ref, "bf16", f"B={B} s={s} h={h}")
    plain = out_to_f64(pa.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                                 dev["context_lens"], c.scale, out_dtype=torch.float32))
    assert np.abs(got - plain).max() <= 2e-3


def test_shared_prefix_errors(pa):
    c = W.make_prefix_shared_case(740, 32, num_seqs=4, prefix_len=64, suffix_range=(1, 50),
                                  dtype="bf16")
    dev = case_to_dev(c)
    for bad in (16, -32, 32 * 1000):  # not a block multiple / negative / past the table
        with pytest.raises(pa.PAError) as e:
            run(pa, c, dev, bad)
        assert e.value.status == -8
    c32 = W.make_prefix_shared_case(741, 16, num_seqs=4, prefix_len=64, suffix_range=(1, 50),
                                    dtype="f32")
    d32 = case_to_dev(c32)
    with pytest.raises(pa.PAError) as e:
        run(pa, c32, d32, 64)
    assert e.value.status == -5
