"""Seeded synthetic inputs for paged-KV attention (shared by tests, bench, smoke).

This module draws random numbers and lays them out in a paged pool; it holds
none of the attention arithmetic.  Both the GPU path and the CPU oracle are
fed from it, and neither is imported here.

Storage conventions: ``"f32"`` arrays are ``numpy.float32``; ``"f16"`` and
``"bf16"`` arrays are ``numpy.uint16`` bit patterns.  Values are drawn as
float32 standard normals and rounded to the storage format with
round-to-nearest-even.

Layout of a case (names follow the pages' domain):

* ``k_pool``, ``v_pool``: ``[NB, B, Hkv, d]`` -- ``NB`` physical blocks of
  ``B`` token slots, each slot holding one row of ``d`` values per KV head.
* ``block_table``: int32 ``[S, MB]``; row ``s`` lists the physical blocks of
  sequence ``s`` in logical order.
* ``context_lens``: int32 ``[S]`` -- keys per sequence.
* ``q``: ``[S, H, d]`` for decode, packed ``[T, H, d]`` for prefill with
  ``query_start_loc`` int32 ``[S+1]``.

Poison: every pool slot that no sequence uses (spare blocks and the tail of a
partially filled last block) is NaN, and table entries past a sequence's last
block point at a NaN spare block, so any stray read shows up as NaN.

Draw order per case: lengths, then block placement, then q, then K, then V,
all from ``numpy.random.default_rng(seed)``; the five named workloads use
``seed = 1000 + workload_number``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0}


def f32_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage format (round to nearest even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32)
        # Add 0x7FFF plus the lowest kept bit, then truncate: ties go to even.
        bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        r = ((u + bias) >> np.uint32(16)).astype(np.uint16)
        nan = np.isnan(x)
        if nan.any():
            r[nan] = NAN_BITS["bf16"]
        return r
    raise ValueError(dtype)


def _randn(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return f32_to_storage(rng.standard_normal(shape, dtype=np.float32), dtype)


def _nan_array(shape, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.full(shape, np.nan, dtype=np.float32)
    return np.full(shape, NAN_BITS[dtype], dtype=np.uint16)


@dataclass
class PagedCase:
    dtype: str
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    block_table: np.ndarray
    context_lens: np.ndarray
    scale: float
    query_start_loc: np.ndarray | None = None
    causal: bool = False
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.block_table.shape[0])

    @property
    def block_size(self) -> int:
        return int(self.k_pool.shape[1])

    @property
    def max_query_len(self) -> int:
        if self.query_start_loc is None:
            return 1
        return int(np.max(np.diff(self.query_start_loc))) if self.num_seqs else 0


def _place_blocks(rng, blocks_per_seq, pool_factor, min_spare=1, shared=0):
    """Assign physical blocks to logical blocks through a random permutation.

    ``shared`` leading logical blocks are common to every sequence (a shared
    prefix); the rest are private.  Returns ``(NB, table_cols, spare_block)``
    where ``table_cols[s]`` lists sequence ``s``'s physical blocks.
    """
    used = shared + int(sum(blocks_per_seq))
    NB = max(int(math.ceil(pool_factor * used)), used + min_spare)
    perm = rng.permutation(NB)
    prefix = perm[:shared]
    cols, pos = [], shared
    for nb in blocks_per_seq:
        cols.append(np.concatenate([prefix, perm[pos:pos + nb]]))
        pos += nb
    spare = int(perm[used]) if used < NB else -1
    return NB, cols, spare


def _fill_pools(dtype, NB, B, Hkv, d, cols, seq_tokens_k, seq_tokens_v):
    """Scatter each sequence's contiguous K/V rows into its blocks."""
    k_pool = _nan_array((NB, B, Hkv, d), dtype)
    v_pool = _nan_array((NB, B, Hkv, d), dtype)
    kf = k_pool.reshape(NB * B, Hkv, d)
    vf = v_pool.reshape(NB * B, Hkv, d)
    for c, kt, vt in zip(cols, seq_tokens_k, seq_tokens_v):
        n = kt.shape[0]
        t = np.arange(n)
        rows = c[t // B].astype(np.int64) * B + t % B
        kf[rows] = kt
        vf[rows] = vt
    return k_pool, v_pool


def _table(cols, MB, spare):
    S = len(cols)
    table = np.full((S, MB), spare if spare >= 0 else 0, dtype=np.int32)
    for s, c in enumerate(cols):
        table[s, :len(c)] = c
    return table


def make_decode_case(seed, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                     dtype, lens=None, len_range=None, max_blocks=None, pool_factor=1.25,
                     scale=None, contiguous=False):
    """A decode case: one query token per sequence over a paged KV cache.

    Either ``lens`` (explicit context lengths) or ``len_range=(lo, hi)``
    (uniform integers, inclusive) is given.  ``max_blocks`` defaults to the
    longest sequence's block count.  ``contiguous=True`` also returns the
    pre-scatter K/V per sequence in ``meta`` (for brute-force checks).
    """
    rng = np.random.default_rng(seed)
    S, H, Hkv, d, B = num_seqs, num_heads, num_kv_heads, head_dim, block_size
    if lens is None:
        lo, hi = len_range
        lens = rng.integers(lo, hi + 1, size=S)
    lens = np.asarray(lens, dtype=np.int64)
    nblk = [int(math.ceil(n / B)) for n in lens]
    MB = max_blocks if max_blocks is not None else max(1, max(nblk) if nblk else 1)
    NB, cols, spare = _place_blocks(rng, nblk, pool_factor)
    q = _randn(rng, (S, H, d), dtype)
    ks = [_randn(rng, (int(n), Hkv, d), dtype) for n in lens]
    vs = [_randn(rng, (int(n), Hkv, d), dtype) for n in lens]
    k_pool, v_pool = _fill_pools(dtype, NB, B, Hkv, d, cols, ks, vs)
    meta = dict(seed=seed, NB=NB, MB=MB, lens=lens.tolist(), spare_block=spare)
    if contiguous:
        meta["k_contig"], meta["v_contig"] = ks, vs
    return PagedCase(dtype, q, k_pool, v_pool, _table(cols, MB, spare),
                     lens.astype(np.int32),
                     float(scale if scale is not None else 1.0 / math.sqrt(d)), meta=meta)


def make_prefill_case(seed, num_seqs, num_heads, num_kv_heads, head_dim, block_size, dtype,
                      lens=None, len_range=None, query_lens=None, causal=True,
                      pool_factor=1.25, scale=None, contiguous=False):
    """A prefill case: packed queries over a paged KV cache.

    ``lens`` are the context lengths ``n_s`` (keys, including the prompt's
    own tokens); ``query_lens`` default to ``lens`` (a whole prompt).  With
    ``query_lens < lens`` the queries are the last ``L_q`` positions.
    """
    rng = np.random.default_rng(seed)
    S, H, Hkv, d, B = num_seqs, num_heads, num_kv_heads, head_dim, block_size
    if lens is None:
        lo, hi = len_range
        lens = rng.integers(lo, hi + 1, size=S)
    lens = np.asarray(lens, dtype=np.int64)
    qlens = lens.copy() if query_lens is None else np.asarray(query_lens, dtype=np.int64)
    nblk = [int(math.ceil(n / B)) for n in lens]
    MB = max(1, max(nblk) if nblk else 1)
    NB, cols, spare = _place_blocks(rng, nblk, pool_factor)
    T = int(qlens.sum())
    q = _randn(rng, (T, H, d), dtype)
    ks = [_randn(rng, (int(n), Hkv, d), dtype) for n in lens]
    vs = [_randn(rng, (int(n), Hkv, d), dtype) for n in lens]
    k_pool, v_pool = _fill_pools(dtype, NB, B, Hkv, d, cols, ks, vs)
    qsl = np.zeros(S + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(qlens)
    meta = dict(seed=seed, NB=NB, MB=MB, lens=lens.tolist(), query_lens=qlens.tolist(),
                spare_block=spare)
    if contiguous:
        meta["k_contig"], meta["v_contig"] = ks, vs
    return PagedCase(dtype, q, k_pool, v_pool, _table(cols, MB, spare),
                     lens.astype(np.int32),
                     float(scale if scale is not None else 1.0 / math.sqrt(d)),
                     query_start_loc=qsl, causal=causal, meta=meta)


def make_prefix_shared_case(seed, block_size, num_seqs=256, prefix_len=2048,
                            suffix_range=(64, 1024), num_heads=32, num_kv_heads=8,
                            head_dim=128, dtype="bf16", pool_factor=1.25):
    """Decode over a common prefix stored once in shared physical blocks.

    Every table's first ``prefix_len / B`` entries are the same physical
    blocks; each sequence then has a private suffix.  The token values and
    suffix lengths depend only on ``seed`` (not on ``block_size``); the
    placement uses a second generator seeded with ``(seed, block_size)``, so
    sweeping ``block_size`` changes only the paging.
    """
    rng = np.random.default_rng(seed)
    S, H, Hkv, d, B = num_seqs, num_heads, num_kv_heads, head_dim, block_size
    if prefix_len % B:
        raise ValueError("prefix must be a whole number of blocks")
    u = rng.integers(suffix_range[0], suffix_range[1] + 1, size=S)
    q = _randn(rng, (S, H, d), dtype)
    k_pre = _randn(rng, (prefix_len, Hkv, d), dtype)
    k_suf = [_randn(rng, (int(n), Hkv, d), dtype) for n in u]
    v_pre = _randn(rng, (prefix_len, Hkv, d), dtype)
    v_suf = [_randn(rng, (int(n), Hkv, d), dtype) for n in u]
    prng = np.random.default_rng([seed, B])
    shared = prefix_len // B
    nblk = [int(math.ceil(n / B)) for n in u]
    NB, cols, spare = _place_blocks(prng, nblk, pool_factor, shared=shared)
    lens = (prefix_len + u).astype(np.int64)
    MB = shared + max(nblk)
    k_pool = _nan_array((NB, B, Hkv, d), dtype)
    v_pool = _nan_array((NB, B, Hkv, d), dtype)
    kf = k_pool.reshape(NB * B, Hkv, d)
    vf = v_pool.reshape(NB * B, Hkv, d)
    t = np.arange(prefix_len)
    pre_rows = cols[0][t // B].astype(np.int64) * B + t % B
    kf[pre_rows] = k_pre
    vf[pre_rows] = v_pre
    for c, kt, vt in zip(cols, k_suf, v_suf):
        t = np.arange(kt.shape[0])
        rows = c[shared + t // B].astype(np.int64) * B + t % B
        kf[rows] = kt
        vf[rows] = vt
    meta = dict(seed=seed, NB=NB, MB=MB, lens=lens.tolist(), spare_block=spare,
                prefix_len=prefix_len, shared_blocks=shared,
                unique_tokens=int(prefix_len + u.sum()))
    return PagedCase(dtype, q, k_pool, v_pool, _table(cols, MB, spare), lens.astype(np.int32),
                     1.0 / math.sqrt(d), meta=meta)


# ---------------------------------------------------------------------------
# The five named workloads.
# ---------------------------------------------------------------------------

WORKLOADS = {
    1: "tiny-f32-decode",
    2: "gqa-f16-decode",
    3: "long-bf16-decode",
    4: "causal-bf16-prefill",
    5: "prefix-shared-bf16-decode",
}


def tiny_f32_decode():
    """1 sequence, 1 head, d=64, 256 keys, B=16, a 32-block pool with the 16
    used blocks placed by a seeded permutation, scale 1/8, float32."""
    return make_decode_case(1001, 1, 1, 1, 64, 16, "f32", lens=[256], pool_factor=2.0,
                            scale=0.125)


def gqa_f16_decode():
    """64 sequences, 32 query / 8 KV heads, d=128, lengths uniform in
    [128, 4096], B=16, pool = 1.25 x used blocks, float16."""
    return make_decode_case(1002, 64, 32, 8, 128, 16, "f16", len_range=(128, 4096),
                            max_blocks=256)


def long_bf16_decode(num_seqs=4, context=100_000):
    """4 sequences of 100,000 keys, 32/8 heads, d=128, B=16, bfloat16."""
    return make_decode_case(1003, num_seqs, 32, 8, 128, 16, "bf16",
                            lens=[context] * num_seqs)


def causal_bf16_prefill(num_kv_heads=8):
    """8 prompts, lengths uniform in [512, 4096], 32/8 heads, d=128, B=16,
    causal, bfloat16; the prompts' own K/V are in the pool.  Other KV head
    counts give the same prompts with other group sizes."""
    return make_prefill_case(1004, 8, 32, num_kv_heads, 128, 16, "bf16",
                             len_range=(512, 4096), causal=True)


def prefix_shared_bf16_decode(block_size):
    """256 sequences sharing a 2048-token prefix plus private suffixes of
    uniform length in [64, 1024]; 32/8 heads, d=128, bfloat16."""
    return make_prefix_shared_case(1005, block_size)


def decode_bytes(case: PagedCase, out_bytes_per_elem: int) -> int:
    """Algorithmic HBM bytes of one decode call.

    K and V rows of every attended token, once per (sequence, KV head);
    q and out once; the table entries actually used and the lengths.
    """
    e = case.q.dtype.itemsize
    S, H, d = case.q.shape
    Hkv = case.k_pool.shape[2]
    B = case.block_size
    n = case.context_lens.astype(np.int64)
    kv = int(n.sum()) * Hkv * d * 2 * e
    qo = S * H * d * (e + out_bytes_per_elem)
    tab = int(np.sum((n + B - 1) // B)) * 4 + 4 * S
    return kv + qo + tab


def prefill_bytes(case: PagedCase, out_bytes_per_elem: int = 2) -> int:
    """Compulsory HBM bytes of one prefill call: Q and O once, each context
    token's K and V rows once per KV head, the context lengths, the query
    start offsets and the table entries that cover the contexts."""
    T, H, d = case.q.shape
    Hkv = case.k_pool.shape[2]
    B = case.k_pool.shape[1]
    esz = case.q.dtype.itemsize
    keys = int(case.context_lens.astype(np.int64).sum())
    blocks = int(sum(-(-int(n) // B) for n in case.context_lens))
    return (T * H * d * (esz + out_bytes_per_elem) + keys * Hkv * d * esz * 2 +
            4 * (blocks + 2 * case.num_seqs + 1))


def prefill_flops(case: PagedCase) -> int:
    """Algorithmic FLOPs of one prefill call: 4*d per visible (query, key)
    pair per head (2*d for Q.K, 2*d for P.V); exponentials not counted."""
    H, d = case.q.shape[1], case.q.shape[2]
    qsl = case.query_start_loc.astype(np.int64)
    total = 0
    for s in range(case.num_seqs):
        L = int(qsl[s + 1] - qsl[s])
        n = int(case.context_lens[s])
        if case.causal:
            # rows i see n - L + i + 1 keys
            pairs = L * (n - L) + L * (L + 1) // 2
        else:
            pairs = L * n
        total += 4 * d * H * pairs
    return total
