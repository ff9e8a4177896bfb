"""Pools in the head-major block layout.

The library reads [NB, B, Hkv, d] pools either fully contiguous
(token-major: a token's Hkv rows adjacent) or head-major within each block
(a contiguous [NB, Hkv, B, d] buffer viewed as [NB, B, Hkv, d]).  The
arithmetic does not depend on where a row lives, so every call must give
the same bits in both layouts, and the oracle's result."""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_decode_amd import workloads as W
from tests.gpu_helpers import (assert_close_f32_out, case_to_dev, out_to_f64, pool_to_dev,
                               to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_decode_amd import binding
    binding.lib()
    return binding


def bits(t):
    return t.contiguous().view(torch.int32 if t.element_size() == 4 else torch.int16).cpu()


@pytest.mark.parametrize("dtype,d,G,B", [("f16", 128, 4, 16), ("bf16", 128, 8, 32),
                                         ("f32", 64, 2, 64), ("f16", 64, 1, 128),
                                         ("bf16", 128, 4, 16)])
def test_decode_head_major(pa, dtype, d, G, B):
    c = W.make_decode_case(1100 + d + G + B, 12, 2 * G, 2, d, B, dtype,
                           lens=[0, 1, 15, 16, 17, 100, 333, 1000, 2049, 64, 5, 3000])
    outs = []
    for hm in (False, True):
        dev = case_to_dev(c, head_major=hm)
        assert dev["k_pool"].is_contiguous() != hm
        outs.append(pa.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                              dev["context_lens"], c.scale, out_dtype=torch.float32))
        torch.cuda.synchronize()
    assert torch.equal(bits(outs[0]), bits(outs[1]))
    ref, _ = oracle.decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale,
                           c.dtype)
    assert_close_f32_out(out_to_f64(outs[1]), ref, dtype, f"head-major {dtype} d={d} G={G}")


@pytest.mark.parametrize("dtype,G", [("bf16", 4), ("f16", 8), ("bf16", 2)])
def test_prefill_head_major(pa, dtype, G):
    c = W.make_prefill_case(1200 + G, 3, 2 * G, 2, 128, 16, dtype, lens=[300, 65, 700],
                            query_lens=[300, 10, 200], causal=True)
    outs = []
    for hm in (False, True):
        dev = case_to_dev(c, head_major=hm)
        outs.append(pa.prefill(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                               dev["context_lens"], dev["query_start_loc"], c.max_query_len,
                               c.scale, causal=True, out_dtype=torch.float32))
        torch.cuda.synchronize()
    assert torch.equal(bits(outs[0]), bits(outs[1]))
    ref, _ = oracle.prefill(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens,
                            c.query_start_loc, c.scale, True, c.dtype)
    assert_close_f32_out(out_to_f64(outs[1]), ref, dtype, f"head-major prefill G={G}")


@pytest.mark.parametrize("dtype,G,B", [("bf16", 4, 16), ("f16", 8, 64), ("f16", 1, 32)])
def test_shared_prefix_head_major(pa, dtype, G, B):
    c = W.make_prefix_shared_case(1300 + G + B, B, num_seqs=20, prefix_len=4 * B,
                                  suffix_range=(0, 300), num_heads=2 * G, num_kv_heads=2,
                                  dtype=dtype)
    outs = []
    for hm in (False, True):
        dev = case_to_dev(c, head_major=hm)
        outs.append(pa.decode_shared_prefix(dev["q"], dev["k_pool"], dev["v_pool"],
                                            dev["block_table"], dev["context_lens"],
                                            4 * B, c.scale, out_dtype=torch.float32))
        torch.cuda.synchronize()
    assert torch.equal(bits(outs[0]), bits(outs[1]))
    ref, _ = oracle.decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale,
                           c.dtype)
    assert_close_f32_out(out_to_f64(outs[1]), ref, dtype, f"head-major shared prefix G={G}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_write_kv_and_copy_blocks_head_major(pa, dtype):
    rng = np.random.default_rng(14)
    NB, B, Hkv, d, N = 30, 32, 4, 128, 200
    kp = W.f32_to_storage(rng.standard_normal((NB, B, Hkv, d), dtype=np.float32), dtype)
    vp = W.f32_to_storage(rng.standard_normal((NB, B, Hkv, d), dtype=np.float32), dtype)
    kn = W.f32_to_storage(rng.standard_normal((N, Hkv, d), dtype=np.float32), dtype)
    vn = W.f32_to_storage(rng.standard_normal((N, Hkv, d), dtype=np.float32), dtype)
    slots = rng.permutation(NB * B)[:N].astype(np.int32)
    slots[::9] = -1
    k_ref, v_ref = oracle.write_kv(kn, vn, slots, kp, vp)
    kd, vd = pool_to_dev(kp, dtype, True), pool_to_dev(vp, dtype, True)
    pa.write_kv(to_dev(kn, dtype), to_dev(vn, dtype), to_dev(slots), kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(bits(kd), bits(to_dev(k_ref, dtype)))
    assert torch.equal(bits(vd), bits(to_dev(v_ref, dtype)))
    # Whole-block copies: the same blocks in either layout.
    src = np.array([3, 7, 0, 29], np.int32)
    dst = np.array([10, 11, 12, 1], np.int32)
    k_ref[dst], v_ref[dst] = k_ref[src], v_ref[src]
    pa.copy_blocks(kd, vd, to_dev(src), to_dev(dst))
    torch.cuda.synchronize()
    assert torch.equal(bits(kd), bits(to_dev(k_ref, dtype)))
    assert torch.equal(bits(vd), bits(to_dev(v_ref, dtype)))
