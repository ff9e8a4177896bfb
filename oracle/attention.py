"""Paged-KV attention, written out from its definition in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed (and where the pages define it):

* Attention for one query row is ``softmax(q K^T * scale) V`` --
  "FlashAttention and PagedAttention: two fixes for two different
  bottlenecks", section "Why attention is expensive"; the scale there is
  1/sqrt(d) and is taken here as a caller-supplied number.
* The keys and values of a sequence live in fixed-size blocks of ``B``
  token slots; a per-sequence block table maps logical block ``j`` to a
  physical block, and the attention kernel reads the scattered blocks
  through that table -- same page, section "PagedAttention - How it works";
  "How PagedAttention and RadixAttention optimise KV-cache handling",
  section "How PagedAttention works".
* Block-wise attention, eq. (4) of "Flash Attention vs Paged Attention",
  section "Paged Attention: memory blocking": query ``i`` attends to the
  keys of blocks ``1 .. ceil(i/B)``; the sum over blocks of ``V_j A_ij`` is
  the ordinary weighted sum over the individual keys.  Blocks fill left to
  right and the unfilled tail of the last block is reserved (same section),
  so only the first ``n_s`` logical tokens of a sequence take part.
* The fused, tiled method returns exactly this result ("FlashAttention -
  How it works": it is not an approximation), which is why a plain,
  materialised softmax is the reference.

Readings where the pages are silent or garbled (each is listed, with its
reason, in the design notes of the repository):

* ``g = h // G`` maps query head ``h`` to KV head ``g`` (contiguous groups).
* Token ``t`` of sequence ``s`` sits in physical block
  ``block_table[s, t // B]`` at slot ``t % B``.
* ``context_lens[s] = n_s`` counts the keys attended, including the token
  being decoded; table entries past ``ceil(n_s/B)`` are never read.
* The softmax subtracts the row maximum before exponentiating (identical in
  exact arithmetic to eq. (4), which has no max term).
* Causal prefill aligns bottom-right: query row ``i`` of a sequence with
  ``L_q`` queries and ``n_s`` keys sits at absolute position
  ``n_s - L_q + i`` and sees keys ``t <= n_s - L_q + i``.
* An empty context (``n_s = 0``) gives an all-zero output and
  ``lse = -inf``.

Inputs are storage-format arrays (see ``oracle.dtypes``); every value is
widened exactly to float64 before any arithmetic.  Matrix products use
numpy's ``@`` (a library primitive) on the gathered rows; there is no
tiling, no online softmax and no reordering beyond the definition.
"""

from __future__ import annotations

import numpy as np

from .dtypes import to_f64


def _gather_tokens(pool: np.ndarray, block_table_row: np.ndarray, n: int, g: int,
                   block_size: int) -> np.ndarray:
    """Rows of KV head ``g`` for logical tokens ``0..n-1`` of one sequence.

    Logical token ``t`` is in physical block ``block_table_row[t // B]`` at
    slot ``t % B`` (block-table address translation).  Returns the raw
    storage rows, shape ``[n, d]``.
    """
    t = np.arange(n, dtype=np.int64)
    phys = block_table_row[t // block_size].astype(np.int64)
    slot = t % block_size
    return pool[phys, slot, g, :]


def _kv_head_of(h: int, num_heads: int, num_kv_heads: int) -> int:
    """KV head shared by query head ``h``: contiguous groups of ``H / Hkv``."""
    return h // (num_heads // num_kv_heads)


def _softmax_weighted_sum(x: np.ndarray, v: np.ndarray):
    """Materialised softmax of score vector ``x`` and the weighted sum of ``v``.

    Returns ``(out, lse, p)``: ``p = exp(x - max x) / sum(exp(x - max x))``,
    ``out = p @ v`` and ``lse = max x + log(sum exp(x - max x))``.
    """
    if x.shape[0] == 0:
        return np.zeros(v.shape[1], dtype=np.float64), -np.inf, np.zeros(0)
    m = np.max(x)
    w = np.exp(x - m)
    z = np.sum(w)
    p = w / z
    return p @ v, m + np.log(z), p


def decode_row(q, k_pool, v_pool, block_table, context_lens, scale, dtype, s, h):
    """Decode attention for one (sequence ``s``, query head ``h``).

    Shapes: ``q [S, H, d]``; pools ``[NB, B, Hkv, d]``; ``block_table
    [S, MB]`` int32; ``context_lens [S]`` int32.  Returns ``(out[d], lse, p)``
    in float64, with ``p`` the full softmax row over the ``n_s`` keys.
    """
    H = q.shape[1]
    Hkv = k_pool.shape[2]
    B = k_pool.shape[1]
    g = _kv_head_of(h, H, Hkv)
    n = int(context_lens[s])
    k = to_f64(_gather_tokens(k_pool, block_table[s], n, g, B), dtype)
    v = to_f64(_gather_tokens(v_pool, block_table[s], n, g, B), dtype)
    qv = to_f64(q[s, h], dtype)
    x = float(scale) * (k @ qv)
    return _softmax_weighted_sum(x, v)


def decode(q, k_pool, v_pool, block_table, context_lens, scale, dtype):
    """Decode attention for every sequence and query head.

    One query token per sequence attends to its ``n_s`` cached keys.
    Returns ``(out [S, H, d], lse [S, H])`` in float64.
    """
    S, H, d = q.shape
    out = np.zeros((S, H, d), dtype=np.float64)
    lse = np.full((S, H), -np.inf, dtype=np.float64)
    for s in range(S):
        for h in range(H):
            o, l, _ = decode_row(q, k_pool, v_pool, block_table, context_lens, scale,
                                 dtype, s, h)
            out[s, h] = o
            lse[s, h] = l
    return out, lse


def _visible(n: int, L: int, i: int, causal: bool) -> int:
    """Number of leading keys visible to query row ``i`` (bottom-right causal)."""
    if not causal:
        return n
    return max(0, min(n, n - L + i + 1))


def prefill_rows(q, k_pool, v_pool, block_table, context_lens, query_start_loc, scale,
                 causal, dtype, rows):
    """Prefill attention for selected packed query rows.

    ``rows`` is an iterable of ``(token_index, head)`` pairs into the packed
    query tensor ``q [T, H, d]``.  Sequence ``s`` owns packed rows
    ``query_start_loc[s] .. query_start_loc[s+1]-1``.  Returns a float64
    array ``[len(rows), d]`` and the matching ``lse``.
    """
    H = q.shape[1]
    Hkv = k_pool.shape[2]
    B = k_pool.shape[1]
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    rows = list(rows)
    out = np.zeros((len(rows), q.shape[2]), dtype=np.float64)
    lse = np.full(len(rows), -np.inf, dtype=np.float64)
    for r, (tok, h) in enumerate(rows):
        s = int(np.searchsorted(qsl, tok, side="right") - 1)
        L = int(qsl[s + 1] - qsl[s])
        i = int(tok - qsl[s])
        n = int(context_lens[s])
        vis = _visible(n, L, i, causal)
        g = _kv_head_of(h, H, Hkv)
        k = to_f64(_gather_tokens(k_pool, block_table[s], vis, g, B), dtype)
        v = to_f64(_gather_tokens(v_pool, block_table[s], vis, g, B), dtype)
        x = float(scale) * (k @ to_f64(q[tok, h], dtype))
        o, l, _ = _softmax_weighted_sum(x, v)
        out[r] = o
        lse[r] = l
    return out, lse


def prefill(q, k_pool, v_pool, block_table, context_lens, query_start_loc, scale, causal,
            dtype):
    """Prefill attention for every packed query row and head.

    For each sequence and head the full ``L_q x n_s`` score matrix is built,
    masked (bottom-right causal when ``causal``), soft-maxed row by row and
    multiplied with V.  Returns ``(out [T, H, d], lse [T, H])`` in float64.
    """
    T, H, d = q.shape
    Hkv = k_pool.shape[2]
    B = k_pool.shape[1]
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    S = qsl.shape[0] - 1
    out = np.zeros((T, H, d), dtype=np.float64)
    lse = np.full((T, H), -np.inf, dtype=np.float64)
    for s in range(S):
        t0, t1 = int(qsl[s]), int(qsl[s + 1])
        L = t1 - t0
        n = int(context_lens[s])
        if L == 0 or n == 0:
            continue
        vis = np.array([_visible(n, L, i, causal) for i in range(L)], dtype=np.int64)
        mask = np.arange(n)[None, :] < vis[:, None]  # [L, n]
        for h in range(H):
            g = _kv_head_of(h, H, Hkv)
            k = to_f64(_gather_tokens(k_pool, block_table[s], n, g, B), dtype)
            v = to_f64(_gather_tokens(v_pool, block_table[s], n, g, B), dtype)
            qs = to_f64(q[t0:t1, h], dtype)
            x = float(scale) * (qs @ k.T)
            x = np.where(mask, x, -np.inf)
            m = np.max(x, axis=1, keepdims=True)
            has = np.isfinite(m[:, 0])
            m = np.where(np.isfinite(m), m, 0.0)
            w = np.where(mask, np.exp(x - m), 0.0)
            z = np.sum(w, axis=1, keepdims=True)
            p = np.divide(w, z, out=np.zeros_like(w), where=z > 0)
            out[t0:t1, h] = p @ v
            lse[t0:t1, h] = np.where(has, m[:, 0] + np.log(np.where(has, z[:, 0], 1.0)),
                                     -np.inf)
    return out, lse


def write_kv(k_new, v_new, slot_mapping, k_pool, v_pool):
    """Append new tokens' K/V rows into their pool slots.

    A slot number ``x`` names physical block ``x // B`` and in-block position
    ``x % B`` (blocks fill left to right; "Flash Attention vs Paged
    Attention", memory-management paragraph).  Negative slots mean "skip".
    Returns new pool arrays; the inputs are not modified.
    """
    B = k_pool.shape[1]
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    for i, x in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if x < 0:
            continue
        k_out[x // B, x % B] = k_new[i]
        v_out[x // B, x % B] = v_new[i]
    return k_out, v_out
