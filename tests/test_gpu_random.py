"""Randomised parity sweeps: many small seeded configurations of every
compute call, each checked against the CPU oracle.

The fixed tests pin chosen edge cases; these draw the shape (dtype, head
size, group size, KV heads, block size, batch), the length mix (empty,
single-key, short, long contexts), the scale (including negative and
large), the decode worker count and the pool layout, so that combinations
nobody listed are exercised too.  Every draw is seeded: a failure names its seed."""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_decode_amd import workloads as W
from tests.gpu_helpers import (assert_close_f32_out, assert_close_native_out, case_to_dev,
                               f32_score_rounding_bound, out_to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_decode_amd import binding
    binding.lib()
    return binding


def draw_lens(rng, S, hi=3000):
    """A length mix: some empty, some of a few keys, most medium, some long."""
    kind = rng.choice(4, size=S, p=[0.1, 0.15, 0.55, 0.2])
    lo_hi = [(0, 0), (1, 16), (17, 1200), (1201, hi)]
    return [int(rng.integers(lo_hi[k][0], lo_hi[k][1] + 1)) for k in kind]


@pytest.mark.parametrize("seed", range(16))
def test_decode_random_configs(pa, monkeypatch, seed):
    rng = np.random.default_rng(5000 + seed)
    dtype = str(rng.choice(["f32", "f16", "bf16"]))
    d = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.choice([16, 32, 64, 128]))
    S = int(rng.integers(1, 100))
    scale = float(rng.choice([1.0 / np.sqrt(d), 0.5, -0.3, 2.0]))
    workers = str(rng.choice(["", "", "37", "300", "4000"]))
    if workers:
        monkeypatch.setenv("PA_DECODE_WORKERS", workers)
    else:
        monkeypatch.delenv("PA_DECODE_WORKERS", raising=False)
    lens = draw_lens(rng, S)
    hm = bool(rng.integers(0, 2))  # pool layout: head-major within blocks
    what = (f"seed={seed} {dtype} d={d} G={G} Hkv={Hkv} B={B} S={S} scale={scale} "
            f"workers={workers or 'default'} head_major={hm}")
    print(what, flush=True)
    c = W.make_decode_case(6000 + seed, S, G * Hkv, Hkv, d, B, dtype, lens=lens, scale=scale)
    dev = case_to_dev(c, head_major=hm)
    ref, _ = oracle.decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale,
                           c.dtype)
    got = pa.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                    dev["context_lens"], c.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    # 16-bit inputs: 2e-3 at every drawn scale.  fp32 inputs: 1e-5 plus the
    # derived effect of forming large scores in fp32.
    extra = f32_score_rounding_bound(c) if dtype == "f32" else 0.0
    assert_close_f32_out(out_to_f64(got), ref, dtype, what, extra=extra)
    if dtype != "f32":
        nat = pa.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                        dev["context_lens"], c.scale)
        torch.cuda.synchronize()
        assert_close_native_out(out_to_f64(nat), ref, dtype, what + " native out")


@pytest.mark.parametrize("seed", range(16))
def test_prefill_random_configs(pa, seed):
    rng = np.random.default_rng(7000 + seed)
    dtype = str(rng.choice(["f16", "bf16"]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.choice([16, 32, 64, 128]))
    S = int(rng.integers(1, 7))
    causal = bool(rng.integers(0, 2))
    scale = float(rng.choice([1.0 / np.sqrt(128), 0.2, -0.1]))
    lens = [int(x) for x in rng.integers(1, 700, size=S)]
    # Whole prompts or the last L_q positions of a longer context.
    qlens = [n if rng.random() < 0.5 else int(rng.integers(1, n + 1)) for n in lens]
    hm = bool(rng.integers(0, 2))
    what = (f"seed={seed} {dtype} G={G} Hkv={Hkv} B={B} S={S} causal={causal} "
            f"scale={scale} lens={lens} qlens={qlens} head_major={hm}")
    print(what, flush=True)
    c = W.make_prefill_case(8000 + seed, S, G * Hkv, Hkv, 128, B, dtype, lens=lens,
                            query_lens=qlens, causal=causal, scale=scale)
    dev = case_to_dev(c, head_major=hm)
    got = out_to_f64(pa.prefill(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                                dev["context_lens"], dev["query_start_loc"], c.max_query_len,
                                c.scale, causal=c.causal, out_dtype=torch.float32))
    torch.cuda.synchronize()
    T, H = c.q.shape[0], c.q.shape[1]
    pick = rng.choice(T * H, size=min(T * H, 400), replace=False)
    rows = [(int(i // H), int(i % H)) for i in pick]
    ref, _ = oracle.prefill_rows(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens,
                                 c.query_start_loc, c.scale, c.causal, c.dtype, rows)
    sel = np.stack([got[t, h] for t, h in rows])
    assert_close_f32_out(sel, ref, dtype, what)


@pytest.mark.parametrize("seed", range(6))
def test_shared_prefix_random_configs(pa, seed):
    rng = np.random.default_rng(9000 + seed)
    B = int(rng.choice([16, 32, 64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4]))
    S = int(rng.integers(1, 90))
    prefix_len = B * int(rng.integers(1, 40))
    hi = int(rng.choice([0, 50, 700]))
    dtype = str(rng.choice(["f16", "bf16"]))
    hm = bool(rng.integers(0, 2))
    what = (f"seed={seed} {dtype} G={G} Hkv={Hkv} B={B} S={S} prefix={prefix_len} "
            f"suffix<={hi} head_major={hm}")
    print(what, flush=True)
    c = W.make_prefix_shared_case(9100 + seed, B, num_seqs=S, prefix_len=prefix_len,
                                  suffix_range=(0, hi), num_heads=G * Hkv,
                                  num_kv_heads=Hkv, dtype=dtype)
    dev = case_to_dev(c, head_major=hm)
    got = out_to_f64(pa.decode_shared_prefix(dev["q"], dev["k_pool"], dev["v_pool"],
                                             dev["block_table"], dev["context_lens"],
                                             prefix_len, c.scale, out_dtype=torch.float32))
    torch.cuda.synchronize()
    ref, _ = oracle.decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale,
                           c.dtype)
    assert_close_f32_out(got, ref, dtype, what)
