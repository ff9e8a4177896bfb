"""GPU parity of pa_prefill (and pa_write_kv) against the CPU oracle."""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_decode_amd import workloads as W
from tests.gpu_helpers import (assert_close_f32_out, assert_close_native_out, case_to_dev,
                               out_to_f64, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_decode_amd import binding
    binding.lib()
    return binding


def run_prefill(pa, c, out_dtype=torch.float32, dev=None):
    dev = dev or case_to_dev(c)
    out = pa.prefill(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                     dev["context_lens"], dev["query_start_loc"], c.max_query_len, c.scale,
                     causal=c.causal, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


def oracle_prefill(c):
    return oracle.prefill(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens,
                          c.query_start_loc, c.scale, c.causal, c.dtype)[0]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_small(pa, dtype, G, causal):
    lens = [1, 63, 64, 65, 200, 130]
    c = W.make_prefill_case(400 + G, len(lens), 2 * G, 2, 128, 16, dtype, lens=lens,
                            causal=causal)
    ref = oracle_prefill(c)
    dev = case_to_dev(c)
    got = out_to_f64(run_prefill(pa, c, dev=dev))
    assert_close_f32_out(got, ref, dtype, f"prefill {dtype} G={G} causal={causal}")
    nat = out_to_f64(run_prefill(pa, c, out_dtype=dev["q"].dtype, dev=dev))
    assert_close_native_out(nat, ref, dtype, "native out")


@pytest.mark.parametrize("B", [16, 32, 64, 128])
def test_prefill_chunked_block_sizes(pa, B):
    """Queries are the last L_q of n_s positions (bottom-right causal)."""
    lens = [300, 129, 1000, 64]
    qlens = [37, 129, 200, 1]
    c = W.make_prefill_case(410 + B, 4, 8, 2, 128, B, "bf16", lens=lens, query_lens=qlens,
                            causal=True)
    got = out_to_f64(run_prefill(pa, c))
    assert_close_f32_out(got, oracle_prefill(c), "bf16", f"chunked B={B}")


def test_prefill_deterministic(pa):
    c = W.make_prefill_case(420, 3, 32, 8, 128, 16, "bf16", lens=[700, 1300, 99])
    dev = case_to_dev(c)
    assert torch.equal(run_prefill(pa, c, dev=dev), run_prefill(pa, c, dev=dev))


def test_prefill_last_row_matches_decode(pa):
    from tests.test_gpu_decode import run_decode  # noqa: F401  (same binding)
    c = W.make_prefill_case(421, 3, 32, 8, 128, 16, "f16", lens=[500, 77, 1025])
    dev = case_to_dev(c)
    pre = run_prefill(pa, c, dev=dev)
    last = torch.from_numpy(c.query_start_loc[1:] - 1).long().cuda()
    dec = pa.decode(dev["q"][last].contiguous(), dev["k_pool"], dev["v_pool"],
                    dev["block_table"], dev["context_lens"], c.scale, out_dtype=torch.float32)
    assert (pre[last] - dec).abs().max().item() <= 2e-3


def test_prefill_many_prompts(pa):
    """90 prompts, mostly short (the padded grid then holds far more empty
    query-tile slots than real ones), some continuing a longer context:
    sampled rows, including every prompt's first and last row."""
    rng = np.random.default_rng(430)
    S = 90
    lens = [int(x) for x in rng.integers(1, 300, size=S)]
    lens[7], lens[50] = 1500, 900
    qlens = [n if rng.random() < 0.7 else int(rng.integers(1, n + 1)) for n in lens]
    c = W.make_prefill_case(431, S, 8, 2, 128, 16, "bf16", lens=lens, query_lens=qlens,
                            causal=True)
    got = out_to_f64(run_prefill(pa, c))
    qsl = c.query_start_loc
    rows = []
    for s in range(S):
        for t in {int(qsl[s]), int(qsl[s + 1] - 1), int(rng.integers(qsl[s], qsl[s + 1]))}:
            rows.append((t, int(rng.integers(0, 8))))
    ref, _ = oracle.prefill_rows(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, qsl,
                                 c.scale, True, c.dtype, rows)
    sel = np.stack([got[t, h] for t, h in rows])
    assert_close_f32_out(sel, ref, "bf16", "90 prompts")


@pytest.mark.parametrize("G,S", [(4, 64), (4, 65), (2, 24), (1, 8), (8, 40)])
def test_prefill_work_order(pa, G, S):
    """32 query heads in head groups that split evenly over the 8 XCDs: the
    kernel orders each XCD's query tiles itself (sequences by decreasing
    context length, ties by position, tiles from the last).  64 (group,
    sequence) pairs per XCD is the largest such case (G = 4, S = 64); S = 65
    takes the plain order.  Prompts of 0 and 1 query rows, prompts that
    continue a longer context and equal context lengths; every 7th row and
    each prompt's first and last rows, at a random head each, so every query
    tile is checked."""
    rng = np.random.default_rng(440 + 10 * G + S)
    lens = [int(x) for x in rng.integers(1, 300, size=S)]
    for i in range(0, S, 9):
        lens[i] = lens[(i + 4) % S]                  # ties in context length
    qlens = []
    for i, n in enumerate(lens):
        r = rng.random()
        qlens.append(0 if i % 11 == 3 else 1 if i % 13 == 5 else
                     n if r < 0.7 else int(rng.integers(1, n + 1)))
    c = W.make_prefill_case(450 + G, S, 32, 32 // G, 128, 16, "bf16", lens=lens,
                            query_lens=qlens, causal=True)
    got = out_to_f64(run_prefill(pa, c))
    qsl = c.query_start_loc
    rows = set()
    for s in range(S):
        if qsl[s + 1] > qsl[s]:
            rows.update({int(qsl[s]), int(qsl[s + 1] - 1)})
    rows.update(range(0, int(qsl[-1]), 7))
    rows = [(t, int(rng.integers(0, 32))) for t in sorted(rows)]
    ref, _ = oracle.prefill_rows(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, qsl,
                                 c.scale, True, c.dtype, rows)
    sel = np.stack([got[t, h] for t, h in rows])
    assert_close_f32_out(sel, ref, "bf16", f"work order G={G} S={S}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_write_kv_bit_exact(pa, dtype):
    rng = np.random.default_rng(5)
    NB, B, Hkv, d, N = 40, 16, 8, 128, 300
    kp = W.f32_to_storage(rng.standard_normal((NB, B, Hkv, d), dtype=np.float32), dtype)
    vp = W.f32_to_storage(rng.standard_normal((NB, B, Hkv, d), dtype=np.float32), dtype)
    kn = W.f32_to_storage(rng.standard_normal((N, Hkv, d), dtype=np.float32), dtype)
    vn = W.f32_to_storage(rng.standard_normal((N, Hkv, d), dtype=np.float32), dtype)
    slots = rng.permutation(NB * B)[:N].astype(np.int32)
    slots[::7] = -1
    k_ref, v_ref = oracle.write_kv(kn, vn, slots, kp, vp)
    kd, vd = to_dev(kp, dtype), to_dev(vp, dtype)
    pa.write_kv(to_dev(kn, dtype), to_dev(vn, dtype), to_dev(slots), kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(kd.cpu(), to_dev(k_ref, dtype).cpu())
    assert torch.equal(vd.cpu(), to_dev(v_ref, dtype).cpu())
