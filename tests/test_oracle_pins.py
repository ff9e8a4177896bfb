"""Pins of the CPU oracle to facts fixed by the pages and by mathematics.

Each ``pin_*`` function raises ``AssertionError`` when the oracle disagrees
with the fact it checks.  The ``test_*`` functions run them, and the mutation
tests at the bottom plant plausible mistakes in the oracle (on the CPU) and
show that some pin fails for each.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A
from oracle import dtypes as D
from oracle.dtypes import half_ulp, round_to, to_f64
from paged_kv_cache_decode_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# Storage-format conversions
# ---------------------------------------------------------------------------

def pin_bf16_decode_known_bits():
    bits = np.array([0x3F80, 0xC000, 0x7F7F, 0x0001, 0x8000, 0x7F80, 0x3EAB],
                    dtype=np.uint16)
    got = D.to_f64(bits, "bf16")
    want = [1.0, -2.0, float.fromhex("0x1.fep+127"), 2.0 ** -133, -0.0, math.inf,
            float.fromhex("0x1.56p-2")]
    assert np.array_equal(got, np.array(want)), got
    assert math.copysign(1.0, got[4]) == -1.0
    assert np.isnan(D.to_f64(np.array([0x7FC0], dtype=np.uint16), "bf16"))[0]


def pin_f16_decode_known_bits():
    bits = np.array([0x3C00, 0x7BFF, 0x0001, 0xFC00, 0x3555], dtype=np.uint16)
    got = to_f64(bits, "f16")
    want = [1.0, 65504.0, 2.0 ** -24, -math.inf, float.fromhex("0x1.554p-2")]
    assert np.array_equal(got, np.array(want)), got


def pin_round_to_even():
    # bf16 keeps 8 significant bits: spacing 2^-7 just above 1.
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -(1 + 2 ** -8),
                  2.0 ** -134, 3 * 2.0 ** -134, 2.0 ** 128])
    want = np.array([1.0, 1 + 2 ** -6, 1 + 2 ** -7, -1.0, 0.0, 2.0 ** -132, math.inf])
    assert np.array_equal(round_to(x, "bf16"), want), round_to(x, "bf16")
    # f16 keeps 11 significant bits, max finite 65504, subnormal quantum 2^-24.
    x = np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 65519.0, 65520.0, 2.0 ** -25,
                  3 * 2.0 ** -25])
    want = np.array([1.0, 1 + 2 ** -9, 65504.0, math.inf, 0.0, 2.0 ** -23])
    assert np.array_equal(round_to(x, "f16"), want), round_to(x, "f16")
    # Cross-check against numpy's own float64 -> float16 rounding.
    r = np.random.default_rng(0).standard_normal(10000) * 30
    assert np.array_equal(round_to(r, "f16"), r.astype(np.float16).astype(np.float64))
    assert np.array_equal(round_to(r, "f32"), r.astype(np.float32).astype(np.float64))
    assert np.all(half_ulp(np.array([1.0, 1.5, 2.0]), "bf16") == [2 ** -8, 2 ** -8, 2 ** -7])


def test_dtype_pins():
    pin_bf16_decode_known_bits()
    pin_f16_decode_known_bits()
    pin_round_to_even()


def test_generator_rounding_matches_torch():
    """The input generator's bf16/f16 rounding equals torch's conversion."""
    x = np.random.default_rng(1).standard_normal(100000).astype(np.float32) * 7
    x[:4] = [1 + 2 ** -8, 1 + 3 * 2 ** -8, -0.0, 3.0e38]
    bf = W.f32_to_storage(x, "bf16")
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf, tb)
    hf = W.f32_to_storage(x[4:], "f16")
    th = torch.from_numpy(x[4:]).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(hf, th)


# ---------------------------------------------------------------------------
# Closed forms and special cases of the definition
# ---------------------------------------------------------------------------

def _small_case(seed=5, dtype="f32", B=16, lens=(1, 7, 16, 33, 100), H=4, Hkv=2, d=32,
                **kw):
    return W.make_decode_case(seed, len(lens), H, Hkv, d, B, dtype, lens=list(lens), **kw)


def _run_decode(c):
    return oracle.decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale,
                         c.dtype)


def pin_rows_sum_to_one():
    c = _small_case(dtype="bf16")
    for s in range(c.num_seqs):
        for h in range(c.q.shape[1]):
            _, _, p = oracle.decode_row(c.q, c.k_pool, c.v_pool, c.block_table,
                                        c.context_lens, c.scale, c.dtype, s, h)
            assert p.shape[0] == c.context_lens[s]
            assert abs(p.sum() - 1.0) <= 1e-14
            assert np.all(p >= 0)


def pin_single_key_returns_v():
    c = _small_case(lens=(1, 1, 1), dtype="f16")
    out, lse = _run_decode(c)
    G = c.q.shape[1] // c.k_pool.shape[2]
    for s in range(c.num_seqs):
        blk = c.block_table[s, 0]
        for h in range(c.q.shape[1]):
            v0 = to_f64(c.v_pool[blk, 0, h // G], "f16")
            assert np.array_equal(out[s, h], v0)  # p = 1 exactly
            k0 = to_f64(c.k_pool[blk, 0, h // G], "f16")
            assert lse[s, h] == pytest.approx(c.scale * float(k0 @ to_f64(c.q[s, h], "f16")),
                                              abs=1e-12)


def pin_identical_keys_give_mean():
    c = _small_case(dtype="f32")
    c.k_pool[:] = c.k_pool[c.block_table[0, 0], 0]  # every slot gets the same key rows
    out, _ = _run_decode(c)
    G = c.q.shape[1] // c.k_pool.shape[2]
    for s in range(c.num_seqs):
        n = int(c.context_lens[s])
        for h in range(c.q.shape[1]):
            v = to_f64(A._gather_tokens(c.v_pool, c.block_table[s], n, h // G, c.block_size),
                       "f32")
            np.testing.assert_allclose(out[s, h], v.mean(axis=0), rtol=0, atol=1e-13)


def pin_scale_zero_mean_over_exactly_n():
    """scale = 0 makes every weight 1/n_s: the output is the mean of exactly the
    first n_s values.  Unused slots are NaN, so a leaked slot would show."""
    c = _small_case(dtype="bf16", lens=(1, 15, 16, 17, 47), scale=0.0)
    out, _ = _run_decode(c)
    assert np.all(np.isfinite(out))
    G = c.q.shape[1] // c.k_pool.shape[2]
    for s in range(c.num_seqs):
        n = int(c.context_lens[s])
        rows = []
        for t in range(n):  # token-by-token, written out independently
            rows.append(c.v_pool[c.block_table[s, t // c.block_size], t % c.block_size])
        rows = to_f64(np.stack(rows), "bf16")
        for h in range(c.q.shape[1]):
            np.testing.assert_allclose(out[s, h], rows[:, h // G].mean(axis=0), rtol=0,
                                       atol=1e-13)


def pin_needle_is_one_hot():
    """q = e0, K = 0 except k_j = 200 e0, scale 1: the weight of key j is 1 to
    within 1e-80, so out = v_j.  Run for every logical position j."""
    c = W.tiny_f32_decode()
    n = int(c.context_lens[0])
    q = np.zeros_like(c.q)
    q[0, 0, 0] = 1.0
    for j in range(n):
        k_pool = np.where(np.isnan(c.k_pool), c.k_pool, 0.0).astype(np.float32)
        blk, slot = c.block_table[0, j // 16], j % 16
        k_pool[blk, slot, 0, 0] = 200.0
        out, _ = oracle.decode(q, k_pool, c.v_pool, c.block_table, c.context_lens, 1.0, "f32")
        np.testing.assert_allclose(out[0, 0], c.v_pool[blk, slot, 0].astype(np.float64),
                                   rtol=0, atol=1e-80)


def pin_empty_context():
    c = _small_case(lens=(0, 5))
    out, lse = _run_decode(c)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(out[1]))


def test_closed_forms():
    pin_rows_sum_to_one()
    pin_single_key_returns_v()
    pin_identical_keys_give_mean()
    pin_scale_zero_mean_over_exactly_n()
    pin_needle_is_one_hot()
    pin_empty_context()


# ---------------------------------------------------------------------------
# Invariances of the paging
# ---------------------------------------------------------------------------

def _same_logical_cases(B_list, seed=11, lens=(5, 64, 129, 300), dtype="bf16", H=8, Hkv=2,
                        d=64):
    """Identical logical K/V/q placed in pools of different block sizes and
    placements (generated once, laid out per block size)."""
    base = W.make_decode_case(seed, len(lens), H, Hkv, d, 16, dtype, lens=list(lens),
                              contiguous=True)
    cases = []
    for i, B in enumerate(B_list):
        rng = np.random.default_rng([seed, B, i])
        nblk = [int(math.ceil(n / B)) for n in lens]
        NB, cols, spare = W._place_blocks(rng, nblk, 1.5)
        kp, vp = W._fill_pools(dtype, NB, B, Hkv, d, cols, base.meta["k_contig"],
                               base.meta["v_contig"])
        cases.append(W.PagedCase(dtype, base.q, kp, vp, W._table(cols, max(nblk), spare),
                                 base.context_lens, base.scale))
    return base, cases


def pin_placement_invariance():
    _, (c1, c2) = _same_logical_cases([16, 16])
    assert not np.array_equal(c1.block_table, c2.block_table)
    o1, l1 = _run_decode(c1)
    o2, l2 = _run_decode(c2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_block_size_invariance():
    _, cases = _same_logical_cases([16, 32, 64, 128])
    ref = _run_decode(cases[0])
    for c in cases[1:]:
        o, l = _run_decode(c)
        assert np.array_equal(o, ref[0]) and np.array_equal(l, ref[1])


def pin_prefix_sharing_equals_private_copies():
    shared = W.make_prefix_shared_case(77, 32, num_seqs=5, prefix_len=128,
                                       suffix_range=(1, 70), num_heads=4, num_kv_heads=2,
                                       head_dim=32)
    tab = shared.block_table
    nsh = shared.meta["shared_blocks"]
    assert np.all(tab[:, :nsh] == tab[0, :nsh])
    # Private copies: give every sequence its own copy of the prefix blocks.
    NB = shared.k_pool.shape[0]
    S = shared.num_seqs
    kp = np.concatenate([shared.k_pool] + [shared.k_pool[tab[0, :nsh]]] * S)
    vp = np.concatenate([shared.v_pool] + [shared.v_pool[tab[0, :nsh]]] * S)
    priv = tab.copy()
    for s in range(S):
        priv[s, :nsh] = NB + s * nsh + np.arange(nsh)
    o1, l1 = _run_decode(shared)
    o2, l2 = oracle.decode(shared.q, kp, vp, priv, shared.context_lens, shared.scale,
                           shared.dtype)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_golden_block_table_example():
    """The pages' two-request table: with a context inside the shared blocks the
    two requests see the same keys; past them they do not."""
    g = json.load(open(os.path.join(GOLDEN, "block_table_example.json")))
    B = g["block_size"]
    t1, t2 = g["tables"]["request_1"], g["tables"]["request_2"]
    assert sorted(set(t1) & set(t2)) == g["shared_physical_blocks"]
    rng = np.random.default_rng(3)
    NB, Hkv, d = 16, 1, 8
    kp = W.f32_to_storage(rng.standard_normal((NB, B, Hkv, d), dtype=np.float32), "f16")
    vp = W.f32_to_storage(rng.standard_normal((NB, B, Hkv, d), dtype=np.float32), "f16")
    q1 = W.f32_to_storage(rng.standard_normal((1, 1, d), dtype=np.float32), "f16")
    q = np.concatenate([q1, q1])
    table = np.array([t1, t2], dtype=np.int32)
    inside = np.array([2 * B, 2 * B], dtype=np.int32)
    o, _ = oracle.decode(q, kp, vp, table, inside, 0.5, "f16")
    assert np.array_equal(o[0], o[1])
    past = np.array([2 * B + 5, 2 * B + 5], dtype=np.int32)
    o, _ = oracle.decode(q, kp, vp, table, past, 0.5, "f16")
    assert not np.array_equal(o[0], o[1])


def test_paging_invariances():
    pin_placement_invariance()
    pin_block_size_invariance()
    pin_prefix_sharing_equals_private_copies()
    pin_golden_block_table_example()


# ---------------------------------------------------------------------------
# Brute force against a library routine (torch CPU SDPA in float64)
# ---------------------------------------------------------------------------

def _sdpa_dense(q, k, v, scale, mask=None):
    """torch's scaled_dot_product_attention in float64 on [heads, L, d]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask,
        scale=scale).numpy()


def pin_decode_vs_dense_sdpa():
    c = W.make_decode_case(21, 3, 8, 2, 64, 16, "f16", lens=[1, 77, 300], contiguous=True)
    out, _ = _run_decode(c)
    G = 4
    for s in range(c.num_seqs):
        k = to_f64(c.meta["k_contig"][s], "f16").transpose(1, 0, 2).repeat(G, axis=0)
        v = to_f64(c.meta["v_contig"][s], "f16").transpose(1, 0, 2).repeat(G, axis=0)
        qq = to_f64(c.q[s], "f16")[:, None, :]
        ref = _sdpa_dense(qq, k, v, c.scale)[:, 0]
        np.testing.assert_allclose(out[s], ref, rtol=0, atol=1e-12)


def pin_prefill_vs_dense_sdpa():
    # whole prompts (L_q = n) and chunked (L_q < n, bottom-right causal)
    for qlens, causal in (((None), True), ((3, 40, 64), True), ((None), False)):
        c = W.make_prefill_case(31, 3, 4, 2, 32, 16, "bf16", lens=[9, 70, 64],
                                query_lens=qlens, causal=causal, contiguous=True)
        out, _ = oracle.prefill(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens,
                                c.query_start_loc, c.scale, c.causal, c.dtype)
        qsl = c.query_start_loc
        for s in range(c.num_seqs):
            n = int(c.context_lens[s])
            L = int(qsl[s + 1] - qsl[s])
            k = to_f64(c.meta["k_contig"][s], "bf16").transpose(1, 0, 2).repeat(2, axis=0)
            v = to_f64(c.meta["v_contig"][s], "bf16").transpose(1, 0, 2).repeat(2, axis=0)
            qq = to_f64(c.q[qsl[s]:qsl[s + 1]], "bf16").transpose(1, 0, 2)
            mask = None
            if causal:
                i = np.arange(L)[:, None]
                t = np.arange(n)[None, :]
                mask = torch.from_numpy(t <= (n - L + i))
            ref = _sdpa_dense(qq, k, v, c.scale, mask).transpose(1, 0, 2)
            np.testing.assert_allclose(out[qsl[s]:qsl[s + 1]], ref, rtol=0, atol=1e-12)


def pin_prefill_pages_shape_example():
    """The pages' causal example shape (2, 8, 1024, 64), fp16 inputs: same
    output shape, and equal to torch's causal SDPA on it (float64)."""
    g = json.load(open(os.path.join(GOLDEN, "sdpa_shape.json")))
    Bt, H, L, d = g["batch"], g["heads"], g["seq_len"], g["head_dim"]
    c = W.make_prefill_case(41, Bt, H, H, d, 16, "f16", lens=[L] * Bt, causal=True,
                            contiguous=True)
    out, _ = oracle.prefill(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens,
                            c.query_start_loc, c.scale, True, "f16")
    out = out.reshape(Bt, L, H, d).transpose(0, 2, 1, 3)
    assert list(out.shape) == g["out_shape"]
    for b in range(Bt):
        qq = to_f64(c.q[b * L:(b + 1) * L], "f16").transpose(1, 0, 2)
        k = to_f64(c.meta["k_contig"][b], "f16").transpose(1, 0, 2)
        v = to_f64(c.meta["v_contig"][b], "f16").transpose(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qq), torch.from_numpy(k), torch.from_numpy(v),
            is_causal=True).numpy()
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def pin_gqa_equals_mha_with_repeated_heads():
    c = _small_case(dtype="f16", H=8, Hkv=2)
    out, lse = _run_decode(c)
    G = 4
    kp = np.repeat(c.k_pool, G, axis=2)
    vp = np.repeat(c.v_pool, G, axis=2)
    o2, l2 = oracle.decode(c.q, kp, vp, c.block_table, c.context_lens, c.scale, "f16")
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)


def test_brute_force_and_library():
    pin_decode_vs_dense_sdpa()
    pin_prefill_vs_dense_sdpa()
    pin_gqa_equals_mha_with_repeated_heads()


def test_pages_shape_example():
    pin_prefill_pages_shape_example()


# ---------------------------------------------------------------------------
# Algebra used by the split-context GPU path, checked against the oracle
# ---------------------------------------------------------------------------

def _partitioned_model(q, k, v, scale, P):
    """Online softmax over partitions of P keys, then a log-sum-exp merge
    (float64, written independently of the oracle)."""
    parts = []
    for a in range(0, k.shape[0], P):
        x = scale * (k[a:a + P] @ q)
        m = x.max()
        w = np.exp(x - m)
        parts.append((m, w.sum(), w @ v[a:a + P]))
    M = max(p[0] for p in parts)
    num = sum(np.exp(m - M) * o for m, _, o in parts)
    den = sum(np.exp(m - M) * l for m, l, _ in parts)
    return num / den


def pin_split_merge_algebra():
    c = W.make_decode_case(51, 2, 2, 1, 32, 16, "bf16", lens=[1000, 37], contiguous=True)
    out, _ = _run_decode(c)
    for s in range(2):
        k = to_f64(c.meta["k_contig"][s][:, 0], "bf16")
        v = to_f64(c.meta["v_contig"][s][:, 0], "bf16")
        for h in range(2):
            qv = to_f64(c.q[s, h], "bf16")
            for P in (16, 512, k.shape[0]):
                np.testing.assert_allclose(_partitioned_model(qv, k, v, c.scale, P), out[s, h],
                                           rtol=0, atol=1e-12)


def pin_prefill_decode_cross_consistency():
    c = W.make_prefill_case(61, 2, 4, 2, 32, 16, "f16", lens=[50, 17], causal=True)
    out, _ = oracle.prefill(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens,
                            c.query_start_loc, c.scale, True, "f16")
    last = c.query_start_loc[1:] - 1
    qd = c.q[last]
    od, _ = oracle.decode(qd, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale,
                          "f16")
    # The two forms sum in different orders (matrix vs vector products).
    np.testing.assert_allclose(out[last], od, rtol=0, atol=1e-14)
    # non-causal prefill with one query per sequence is decode
    qsl = np.arange(3, dtype=np.int32)
    on, _ = oracle.prefill(qd, c.k_pool, c.v_pool, c.block_table, c.context_lens, qsl,
                           c.scale, False, "f16")
    np.testing.assert_allclose(on, od, rtol=0, atol=1e-15)
    # prefill_rows (row-at-a-time) equals the matrix form
    rows = [(0, 0), (10, 3), (49, 1), (50, 2), (66, 0)]
    orow, _ = oracle.prefill_rows(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens,
                                  c.query_start_loc, c.scale, True, "f16", rows)
    for r, (t, h) in enumerate(rows):
        np.testing.assert_allclose(orow[r], out[t, h], rtol=0, atol=1e-14)


def test_algebra_and_cross_consistency():
    pin_split_merge_algebra()
    pin_prefill_decode_cross_consistency()


# ---------------------------------------------------------------------------
# Workload sizing against the pages' numbers
# ---------------------------------------------------------------------------

def test_kv_sizing_golden():
    g = json.load(open(os.path.join(GOLDEN, "kv_sizing.json")))
    per_token = g["layers"] * g["kv_heads"] * g["head_dim"] * 2 * g["bytes_per_value"]
    assert per_token == g["stated_kib_per_token"] * 1024
    assert per_token // g["layers"] == 4096  # one layer: the decode workloads' 4 KiB/token
    total_gib = per_token * g["context_tokens"] / 2 ** 30
    assert total_gib == pytest.approx(12.207, abs=1e-3)


def test_write_kv_oracle():
    rng = np.random.default_rng(0)
    kp = np.zeros((4, 16, 2, 8), np.float32)
    vp = np.zeros_like(kp)
    kn = rng.standard_normal((3, 2, 8)).astype(np.float32)
    vn = rng.standard_normal((3, 2, 8)).astype(np.float32)
    k2, v2 = oracle.write_kv(kn, vn, np.array([17, -1, 63]), kp, vp)
    assert np.array_equal(k2[1, 1], kn[0]) and np.array_equal(v2[3, 15], vn[2])
    assert np.count_nonzero(k2) == 2 * 16 and np.count_nonzero(kp) == 0


# ---------------------------------------------------------------------------
# Planted mistakes: each must make at least one pin fail
# ---------------------------------------------------------------------------

def _expect_some_pin_fails(pins):
    failed = []
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "no pin caught the planted mistake"


def test_planted_swapped_block_and_slot(monkeypatch):
    def bad(pool, row, n, g, B):
        t = np.arange(n, dtype=np.int64)
        return pool[row[t % B % len(row)].astype(np.int64), t // B % B, g, :]
    monkeypatch.setattr(A, "_gather_tokens", bad)
    _expect_some_pin_fails([pin_placement_invariance, pin_decode_vs_dense_sdpa])


def test_planted_off_by_one_causal(monkeypatch):
    monkeypatch.setattr(A, "_visible",
                        lambda n, L, i, causal: n if not causal else max(0, min(n, n - L + i)))
    _expect_some_pin_fails([pin_prefill_vs_dense_sdpa])


def test_planted_wrong_gqa_mapping(monkeypatch):
    monkeypatch.setattr(A, "_kv_head_of", lambda h, H, Hkv: h % Hkv)
    _expect_some_pin_fails([pin_decode_vs_dense_sdpa, pin_gqa_equals_mha_with_repeated_heads])


def test_planted_unnormalised_softmax(monkeypatch):
    def bad(x, v):
        if x.shape[0] == 0:
            return np.zeros(v.shape[1]), -np.inf, np.zeros(0)
        w = np.exp(x - x.max())
        return w @ v, x.max(), w
    monkeypatch.setattr(A, "_softmax_weighted_sum", bad)
    _expect_some_pin_fails([pin_rows_sum_to_one, pin_identical_keys_give_mean])


def test_planted_transposed_bf16_halves(monkeypatch):
    real = D.to_f64

    def bad(a, dtype):
        if dtype == "bf16":
            return (a.astype(np.uint32)).view(np.float32).astype(np.float64)
        return real(a, dtype)
    monkeypatch.setattr(D, "to_f64", bad)
    monkeypatch.setattr(A, "to_f64", bad)
    _expect_some_pin_fails([pin_bf16_decode_known_bits])
