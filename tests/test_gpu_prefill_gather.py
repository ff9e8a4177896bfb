"""Bit-exact pins of the prefill kernel's paged gather, and its V-range contract.

The paged gather must be exact: every (logical block -> physical block,
slot) translation the kernel makes is pinned by a needle.  With q = e0,
scale 1 and K = 0 except k_j = 200 e0 for one key j per (sequence, KV head),
a query row that sees key j has scores 200 for j and 0 for every other key;
exp(-200) underflows to zero in fp32, so the softmax row is exactly one-hot
and the output must be v_j bit for bit ("FlashAttention and PagedAttention:
two fixes for two different bottlenecks", "FlashAttention - How it works":
the tiled result is the exact one; "How PagedAttention and RadixAttention
optimise KV-cache handling", "How PagedAttention works": K and V are
gathered through the block table).  The needles sit in whole-visible tiles,
on diagonal tiles and in the partly filled last block, for every block
size, with whole prompts and with the last L_q positions of a longer
context.  The P.V product of the prefill kernel runs on fp16 matrix cores,
so a bf16 V value reaches the output as its fp16 rounding -- the value
itself for every bf16 value of magnitude 2^-17 and up within fp16's range
(fp16's subnormal quantum is 2^-24, a bf16 value carries 8 significant
bits), which the assertions make explicit.

Physical placement and block size must not change a single bit either: the
kernel reduces over logical key positions in 64-key tiles whatever the
block size or the placement.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.dtypes import round_to, to_f64
from paged_kv_cache_decode_amd import workloads as W
from tests.gpu_helpers import (assert_close_f32_out, case_to_dev, out_to_f64, record_max_abs,
                               to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_decode_amd import binding
    binding.lib()
    return binding


def storage(x, dtype):
    return W.f32_to_storage(np.asarray(x, dtype=np.float32), dtype)


def needle_inputs(c, picks):
    """q = e0 for every row and head; K = 0 in every used slot except
    k[j] = 200 e0 at key j of each pick (sequence s, KV head g, key j)."""
    dt = c.dtype
    q = np.zeros_like(c.q)
    q[..., 0] = storage([1.0], dt)[0]
    k = c.k_pool.copy()
    used = ~np.isnan(to_f64(k, dt))
    k[used] = storage([0.0], dt)[0]
    B = c.block_size
    for s, g, j in picks:
        blk = c.block_table[s, j // B]
        k[blk, j % B, g, 0] = storage([200.0], dt)[0]
    return q, k


def as_pv_precision(v64, dtype):
    """What the fp16 P.V product makes of stored V values: fp16 rounding for
    bf16 (the identity for every bf16 value fp16 represents), none for f16."""
    return round_to(v64, "f16") if dtype == "bf16" else v64


def run_prefill(pa, c, q, k, dev):
    out = pa.prefill(to_dev(q, c.dtype), to_dev(k, c.dtype), dev["v_pool"], dev["block_table"],
                     dev["context_lens"], dev["query_start_loc"], c.max_query_len, 1.0,
                     causal=c.causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("B", [16, 32, 64, 128])
def test_prefill_needle_bit_exact(pa, dtype, B):
    lens = [210, 130, 64, 77]
    qlens = [210, 130, 64, 20]  # the last prompt continues a 57-key context
    c = W.make_prefill_case(2100 + B, 4, 8, 2, 128, B, dtype, lens=lens, query_lens=qlens,
                            causal=True)
    dev = case_to_dev(c)
    v64 = to_f64(c.v_pool, dtype)
    qsl = c.query_start_loc
    # Needle positions per (sequence, KV head): first key, inside whole
    # tiles, on a diagonal tile, the partly filled last block, the last key.
    rounds = [[(0, 0, 0), (0, 1, 63), (1, 0, 64), (1, 1, 129), (2, 0, 17), (2, 1, 63),
               (3, 0, 56), (3, 1, 76)],
              [(0, 0, 200), (0, 1, 209), (1, 0, 5), (1, 1, 100), (2, 0, 0), (2, 1, 40),
               (3, 0, 60), (3, 1, 0)]]
    checked = 0
    for picks in rounds:
        q, k = needle_inputs(c, picks)
        out = run_prefill(pa, c, q, k, dev)
        for s, g, j in picks:
            n, L = int(c.context_lens[s]), int(qsl[s + 1] - qsl[s])
            blk = c.block_table[s, j // B]
            want = as_pv_precision(v64[blk, j % B, g], dtype)
            for i in range(L):
                if n - L + i < j:
                    continue  # the row does not see the needle
                for h in range(4 * g, 4 * g + 4):
                    assert np.array_equal(out[qsl[s] + i, h], want), (s, g, j, i, h)
                    checked += 1
    assert checked > 1000


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_placement_and_block_size_invariance(pa, dtype):
    """The same logical prompts paged at block sizes 16..128, each with two
    different random placements: every output identical, bit for bit."""
    lens = [300, 1, 64, 129, 700]
    base = W.make_prefill_case(2200, 5, 8, 2, 128, 16, dtype, lens=lens, contiguous=True)
    outs = []
    for B in (16, 32, 64, 128):
        for i in range(2):
            rng = np.random.default_rng([2200, B, i])
            nblk = [math.ceil(n / B) for n in lens]
            NB, cols, spare = W._place_blocks(rng, nblk, 1.5)
            kp, vp = W._fill_pools(dtype, NB, B, 2, 128, cols, base.meta["k_contig"],
                                   base.meta["v_contig"])
            c = W.PagedCase(dtype, base.q, kp, vp, W._table(cols, max(nblk), spare),
                            base.context_lens, base.scale, query_start_loc=base.query_start_loc,
                            causal=True)
            d = case_to_dev(c)
            outs.append(pa.prefill(d["q"], d["k_pool"], d["v_pool"], d["block_table"],
                                   d["context_lens"], d["query_start_loc"], c.max_query_len,
                                   c.scale, causal=True, out_dtype=torch.float32))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    ref = oracle.prefill(base.q, kp, vp, c.block_table, c.context_lens, c.query_start_loc,
                         c.scale, True, dtype)[0]
    assert_close_f32_out(out_to_f64(outs[0]), ref, dtype, "placement/block size")


@pytest.mark.parametrize("B", [16, 64])
def test_shared_prefix_needle_bit_exact(pa, B):
    """pa_decode_shared_prefix: a needle in the shared prefix (attended by
    the prefix step, the prefill kernel in key chunks) or in a sequence's own
    suffix (the decode kernel) gives v_j exactly for every query head of the
    KV head."""
    c = W.make_prefix_shared_case(2300 + B, B, num_seqs=12, prefix_len=512,
                                  suffix_range=(1, 200), num_heads=8, num_kv_heads=2)
    dev = case_to_dev(c)
    v64 = to_f64(c.v_pool, "bf16")
    P = c.meta["prefix_len"]
    rng = np.random.default_rng(B)
    S = c.num_seqs
    # The prefix blocks are shared, so a needle in the prefix is seen by every
    # sequence: round 0 puts one prefix needle per KV head, round 1 one suffix
    # needle per (sequence, KV head), round 2 a prefix needle for KV head 0
    # and suffix needles for KV head 1.
    for rnd in range(3):
        pre = [int(rng.integers(0, P)) for _ in range(2)]
        picks = []
        for s in range(S):
            n = int(c.context_lens[s])
            for g in range(2):
                in_prefix = rnd == 0 or (rnd == 2 and g == 0)
                picks.append((s, g, pre[g] if in_prefix else int(rng.integers(P, n))))
        q, k = needle_inputs(c, picks)
        out = pa.decode_shared_prefix(to_dev(q, "bf16"), to_dev(k, "bf16"), dev["v_pool"],
                                      dev["block_table"], dev["context_lens"], P, 1.0,
                                      out_dtype=torch.float32)
        out = out.cpu().numpy().astype(np.float64)
        for s, g, j in picks:
            blk = c.block_table[s, j // B]
            # Prefix keys pass through the fp16 P.V product; suffix keys
            # through the decode kernel's fp32 one.
            want = v64[blk, j % B, g]
            if j < P:
                want = as_pv_precision(want, "bf16")
            for h in range(4 * g, 4 * g + 4):
                assert np.array_equal(out[s, h], want), (rnd, s, g, j, h)


def test_prefill_bf16_v_range(pa):
    """The bf16 -> fp16 narrowing of V in the P.V product, at the edges of
    the contract: V values up to 65,280 in magnitude (the largest bf16 values
    below fp16's overflow threshold) and V values below fp16's normal range
    (2^-14), where the product keeps fp16's subnormal quantum 2^-24.
    Measured against the oracle at 2e-3 x max|v|, plus half that quantum
    (2^-25) for the subnormal-range case."""
    lens = [200, 64, 513]
    for kind in ("large", "subnormal"):
        c = W.make_prefill_case(2400, 3, 8, 2, 128, 16, "bf16", lens=lens, causal=True)
        v = to_f64(c.v_pool, "bf16")
        used = ~np.isnan(v)
        rng = np.random.default_rng(2401)
        if kind == "large":
            x = np.clip(rng.standard_normal(v.shape) * 30000.0, -65280.0, 65280.0)
            x.flat[::97] = 65280.0
            x.flat[1::97] = -65280.0
        else:
            x = rng.standard_normal(v.shape) * 2.0 ** -17  # mostly below 2^-14
        vp = c.v_pool.copy()
        vp[used] = storage(x[used], "bf16")
        c = W.PagedCase("bf16", c.q, c.k_pool, vp, c.block_table, c.context_lens, c.scale,
                        query_start_loc=c.query_start_loc, causal=True)
        vmax = float(np.abs(to_f64(vp, "bf16")[used]).max())
        d = case_to_dev(c)
        got = out_to_f64(pa.prefill(d["q"], d["k_pool"], d["v_pool"], d["block_table"],
                                    d["context_lens"], d["query_start_loc"], c.max_query_len,
                                    c.scale, causal=True, out_dtype=torch.float32))
        ref = oracle.prefill(c.q, c.k_pool, vp, c.block_table, c.context_lens,
                             c.query_start_loc, c.scale, True, "bf16")[0]
        bound = 2e-3 * vmax + (2.0 ** -25 if kind == "subnormal" else 0.0)
        err = float(np.abs(got - ref).max())
        print(f"V range {kind}: max|v| {vmax:.4g}, max-abs error {err:.3e}, bound {bound:.3e}")
        record_max_abs(f"prefill bf16 V range {kind} (max|v| {vmax:.4g})", err)
        assert np.all(np.isfinite(got)), kind
        assert err <= bound, (kind, err, bound)
