"""GPU parity of pa_decode against the CPU oracle (run through the C ABI)."""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_decode_amd import workloads as W
from tests.gpu_helpers import (TOL, assert_close_f32_out, assert_close_native_out, case_to_dev,
                               out_to_f64, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_decode_amd import binding
    binding.lib()
    return binding


def run_decode(pa, c, out_dtype=torch.float32, dev=None):
    dev = dev or case_to_dev(c)
    out = pa.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                    dev["context_lens"], c.scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


def oracle_decode(c):
    return oracle.decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale,
                         c.dtype)[0]


def test_tiny_f32_decode(pa):
    c = W.tiny_f32_decode()
    got = out_to_f64(run_decode(pa, c))
    assert_close_f32_out(got, oracle_decode(c), "f32", "tiny-f32-decode", record="tiny-f32-decode")


EDGE_LENS = [0, 1, 15, 16, 17, 63, 64, 65, 100, 257, 1000, 1537]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_shapes(pa, dtype, d, G):
    Hkv = 2
    c = W.make_decode_case(100 + d + G, len(EDGE_LENS), G * Hkv, Hkv, d, 16, dtype,
                           lens=EDGE_LENS)
    ref = oracle_decode(c)
    dev = case_to_dev(c)
    got = out_to_f64(run_decode(pa, c, dev=dev))
    assert_close_f32_out(got, ref, dtype, f"{dtype} d={d} G={G}")
    assert np.all(got[0] == 0)  # empty context
    if dtype != "f32":
        nat = out_to_f64(run_decode(pa, c, out_dtype=dev["q"].dtype, dev=dev))
        assert_close_native_out(nat, ref, dtype, f"{dtype} native out")


@pytest.mark.parametrize("B", [16, 32, 64, 128])
def test_decode_block_sizes(pa, B):
    c = W.make_decode_case(200 + B, 6, 8, 2, 128, B, "bf16", lens=[1, 31, 129, 700, 2048, 3000])
    got = out_to_f64(run_decode(pa, c))
    assert_close_f32_out(got, oracle_decode(c), "bf16", f"B={B}")


@pytest.mark.parametrize("workers", ["1", "3", "7", "64", "1000", "100000", ""])
def test_decode_worker_count_invariance(pa, monkeypatch, workers):
    """Any number of workers (so any split of the contexts into partitions,
    including many empty workers and one worker for everything) gives the
    oracle's result; splits differ from each other only by rounding."""
    c = W.make_decode_case(300, 6, 8, 2, 128, 16, "f16", lens=[5, 700, 0, 2049, 4096, 3333],
                           max_blocks=256)
    ref = oracle_decode(c)
    dev = case_to_dev(c)
    monkeypatch.setenv("PA_DECODE_WORKERS", "1")
    one = out_to_f64(run_decode(pa, c, dev=dev))
    monkeypatch.setenv("PA_DECODE_WORKERS", workers)
    got = out_to_f64(run_decode(pa, c, dev=dev))
    assert_close_f32_out(got, ref, "f16", f"workers={workers or 'default'}")
    assert np.all(got[2] == 0)
    assert np.abs(got - one).max() <= 1e-5


def test_decode_many_sequences(pa):
    """1,500 short sequences (lengths 0 .. 200): thousands of units, most
    workers crossing many unit boundaries, the lengths read from memory
    rather than from one register of 64."""
    rng = np.random.default_rng(77)
    lens = [int(x) for x in rng.integers(0, 201, size=1500)]
    c = W.make_decode_case(770, 1500, 8, 2, 128, 16, "bf16", lens=lens)
    got = out_to_f64(run_decode(pa, c))
    assert_close_f32_out(got, oracle_decode(c), "bf16", "1500 sequences")


def test_decode_is_deterministic(pa):
    c = W.make_decode_case(301, 8, 32, 8, 128, 16, "bf16", len_range=(1, 3000))
    dev = case_to_dev(c)
    a = run_decode(pa, c, dev=dev)
    b = run_decode(pa, c, dev=dev)
    assert torch.equal(a, b)


def test_decode_workspace_reuse_across_calls_and_streams(pa, monkeypatch):
    """The per-unit counters of the kept workspace return to zero after every
    call: alternating shapes (more units, then fewer, then a split of every
    unit over many workers) on one stream and on a second stream reproduce
    each shape's first result bit for bit, and match the oracle."""
    monkeypatch.setenv("PA_DECODE_WORKERS", "512")
    small = W.make_decode_case(303, 3, 8, 2, 128, 16, "f16", lens=[900, 4000, 17],
                               max_blocks=256)
    big = W.make_decode_case(304, 24, 32, 8, 128, 16, "f16", len_range=(1, 4096),
                             max_blocks=256)
    cases = [(small, case_to_dev(small)), (big, case_to_dev(big))]
    refs = [oracle_decode(c) for c, _ in cases]
    first = [run_decode(pa, c, dev=d) for c, d in cases]
    for (c, _), got, ref in zip(cases, first, refs):
        assert_close_f32_out(out_to_f64(got), ref, "f16", "workspace reuse")
    side = torch.cuda.Stream()
    for rep in range(3):
        for i in (1, 0):
            c, d = cases[i]
            assert torch.equal(run_decode(pa, c, dev=d), first[i]), (rep, i)
            with torch.cuda.stream(side):
                out = pa.decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"],
                                d["context_lens"], c.scale, out_dtype=torch.float32,
                                stream=side.cuda_stream)
            side.synchronize()
            assert torch.equal(out, first[i]), ("side stream", rep, i)
    pa.workspace_release(side.cuda_stream)
    side.synchronize()


def test_decode_placement_invariance_bit_exact(pa):
    """Same logical K/V, two different physical placements: identical bits."""
    base = W.make_decode_case(302, 4, 8, 2, 128, 16, "bf16", lens=[33, 300, 1000, 2500],
                              contiguous=True)
    outs = []
    for i in range(2):
        rng = np.random.default_rng([302, i])
        nblk = [math.ceil(n / 16) for n in base.meta["lens"]]
        NB, cols, spare = W._place_blocks(rng, nblk, 1.5)
        kp, vp = W._fill_pools("bf16", NB, 16, 2, 128, cols, base.meta["k_contig"],
                               base.meta["v_contig"])
        c = W.PagedCase("bf16", base.q, kp, vp, W._table(cols, max(nblk), spare),
                        base.context_lens, base.scale)
        outs.append(run_decode(pa, c))
    assert torch.equal(outs[0], outs[1])


def test_needle_bit_exact_every_position(pa):
    """q = e0, K = 0 except k_j = 200 e0, scale 1: out must equal v_j exactly."""
    c = W.tiny_f32_decode()
    n = int(c.context_lens[0])
    q = np.zeros_like(c.q)
    q[0, 0, 0] = 1.0
    dev = case_to_dev(c)
    qd = to_dev(q)
    kz = np.where(np.isnan(c.k_pool), c.k_pool, 0.0).astype(np.float32)
    for j in range(n):
        kp = kz.copy()
        blk, slot = c.block_table[0, j // 16], j % 16
        kp[blk, slot, 0, 0] = 200.0
        out = pa.decode(qd, to_dev(kp), dev["v_pool"], dev["block_table"], dev["context_lens"],
                        1.0)
        want = torch.from_numpy(c.v_pool[blk, slot, 0].copy()).cuda()
        assert torch.equal(out[0, 0], want), j


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_needle_bit_exact_16bit(pa, dtype):
    c = W.make_decode_case(303, 3, 8, 2, 128, 16, dtype, lens=[40, 1000, 2100])
    rng = np.random.default_rng(7)
    k = c.k_pool.copy()
    one = W.f32_to_storage(np.array([1.0], np.float32), dtype)[0]
    needle = W.f32_to_storage(np.array([200.0], np.float32), dtype)[0]
    zero = np.uint16(0)
    valid = ~np.isnan(oracle.dtypes.to_f64(k, dtype))
    k[valid] = zero
    q = np.zeros_like(c.q)
    q[:, :, 0] = one
    picks = []
    for s in range(3):
        j = int(rng.integers(0, c.context_lens[s]))
        blk, slot = c.block_table[s, j // 16], j % 16
        k[blk, slot, :, 0] = needle
        picks.append((blk, slot))
    dev = case_to_dev(c)
    out = pa.decode(to_dev(q, dtype), to_dev(k, dtype), dev["v_pool"], dev["block_table"],
                    dev["context_lens"], 1.0)
    for s, (blk, slot) in enumerate(picks):
        for h in range(8):
            want = to_dev(c.v_pool[blk, slot, h // 4].copy(), dtype)
            assert torch.equal(out[s, h], want), (s, h)


def test_scale_zero_is_mean_of_exactly_n(pa):
    c = W.make_decode_case(304, 5, 4, 4, 64, 16, "f32", lens=[1, 15, 16, 17, 47], scale=0.0)
    got = out_to_f64(run_decode(pa, c))
    assert_close_f32_out(got, oracle_decode(c), "f32", "scale 0")


def test_gqa_f16_decode_full(pa):
    """64 sequences, 32/8 heads, d=128, lengths in [128, 4096], f16: every output."""
    c = W.gqa_f16_decode()
    ref = oracle_decode(c)
    dev = case_to_dev(c)
    got = out_to_f64(run_decode(pa, c, dev=dev))
    worst = assert_close_f32_out(got, ref, "f16", "gqa-f16-decode", record="gqa-f16-decode")
    print(f"gqa-f16-decode max-abs {worst:.2e}")
    nat = out_to_f64(run_decode(pa, c, out_dtype=torch.float16, dev=dev))
    assert_close_native_out(nat, ref, "f16", "gqa-f16-decode native")


@pytest.mark.parametrize("B", [16, 32, 64, 128])
def test_prefix_shared_tables_match_private_copies(pa, B):
    """256 sequences sharing a 2048-token prefix: for the first 16, tables
    that point at the shared blocks give the same bits as tables that point
    at private copies of the prefix (every output of the workload is checked
    against the oracle in test_gpu_full_configs.py)."""
    c = W.prefix_shared_bf16_decode(B)
    dev = case_to_dev(c)
    # Private copies of the prefix for the first 16 sequences.
    S = 16
    nsh = c.meta["shared_blocks"]
    tab = c.block_table[:S].copy()
    NB = c.k_pool.shape[0]
    kp = np.concatenate([c.k_pool] + [c.k_pool[tab[0, :nsh]]] * S)
    vp = np.concatenate([c.v_pool] + [c.v_pool[tab[0, :nsh]]] * S)
    for s in range(S):
        tab[s, :nsh] = NB + s * nsh + np.arange(nsh)
    out_priv = pa.decode(dev["q"][:S].contiguous(), to_dev(kp, "bf16"), to_dev(vp, "bf16"),
                         to_dev(tab), dev["context_lens"][:S].contiguous(), c.scale,
                         out_dtype=torch.float32)
    out_shared = pa.decode(dev["q"][:S].contiguous(), dev["k_pool"], dev["v_pool"],
                           dev["block_table"][:S].contiguous(),
                           dev["context_lens"][:S].contiguous(), c.scale,
                           out_dtype=torch.float32)
    assert torch.equal(out_priv, out_shared)


def test_decode_plan_and_errors(pa):
    c = W.gqa_f16_decode()
    dev = case_to_dev(c)
    out = torch.empty(c.q.shape, dtype=torch.float32, device="cuda")
    plan = pa.decode_plan(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                          dev["context_lens"], out)
    assert plan["workers"] >= 256 and plan["grid"][0] == -(-plan["workers"] // 4)
    with pytest.raises(pa.PAError) as ei:
        pa.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"].float(),
                  dev["context_lens"], c.scale)
    assert ei.value.status == -2
