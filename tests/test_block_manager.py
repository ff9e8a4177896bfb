"""The host block manager (pa_bm_*) on the CPU: allocation on demand, forks
that share blocks, copy-on-write, release, tables -- and, end to end, that
the tables it hands out make the paged oracle reproduce attention over each
sequence's logical tokens.

Which free block the manager picks is its own choice, so the tests check
what is fixed (token order, sharing, refcounts, where copies are needed)
and that everything else is valid (no block held twice unless shared, every
block either free or held)."""

import numpy as np
import pytest

import oracle
from paged_kv_cache_decode_amd import binding as B


def test_append_allocates_on_demand():
    bm = B.BlockManager(10, 4)
    bm.add(7)
    s = bm.append(7, 6)
    assert bm.num_free == 8  # ceil(6 / 4) blocks taken
    blocks = s // 4
    assert len(set(blocks[:4])) == 1 and len(set(blocks[4:])) == 1 and blocks[0] != blocks[4]
    assert list(s % 4) == [0, 1, 2, 3, 0, 1]
    s2 = bm.append(7, 3)  # fills the second block, then takes a third
    assert list(s2 % 4) == [2, 3, 0] and s2[0] // 4 == blocks[4] and bm.num_free == 7
    table, lens = bm.block_table([7], 5)
    assert lens[0] == 9 and list(table[0, 3:]) == [-1, -1]
    assert list(table[0, :3]) == [blocks[0], blocks[4], s2[2] // 4]
    assert len(bm.append(7, 0)) == 0 and bm.num_free == 7


def test_fork_shares_and_free_returns_blocks():
    bm = B.BlockManager(6, 4)
    bm.add(0)
    bm.append(0, 8)  # two full blocks
    bm.fork(0, 1)
    t, lens = bm.block_table([0, 1], 4)
    assert (t[0] == t[1]).all() and list(lens) == [8, 8]
    assert all(bm.refcount(int(b)) == 2 for b in t[0, :2])
    bm.append(1, 1)  # full last block: a new block, no copy
    assert bm.take_copies()[0].size == 0
    bm.free(0)
    assert bm.num_free == 6 - 3 and all(bm.refcount(int(b)) == 1 for b in t[0, :2])
    bm.free(1)
    assert bm.num_free == 6


def test_copy_on_write_of_a_shared_partial_block():
    bm = B.BlockManager(8, 4)
    bm.add(0)
    bm.append(0, 6)  # block a full, block b holds 2 tokens
    bm.fork(0, 1)
    t0, _ = bm.block_table([0], 4)
    a, b = int(t0[0, 0]), int(t0[0, 1])
    s = bm.append(1, 1)  # child writes into shared b: copied first
    src, dst = bm.take_copies()
    assert list(src) == [b] and dst.size == 1 and int(dst[0]) not in (a, b)
    assert s[0] == int(dst[0]) * 4 + 2
    assert bm.refcount(b) == 1 and bm.refcount(int(dst[0])) == 1 and bm.refcount(a) == 2
    s = bm.append(0, 1)  # the parent now owns b alone: writes in place
    assert s[0] == b * 4 + 2 and bm.take_copies()[0].size == 0


def test_out_of_blocks_leaves_state_unchanged():
    bm = B.BlockManager(3, 4)
    bm.add(0)
    bm.append(0, 10)
    before = bm.block_table([0], 4)
    with pytest.raises(B.PAError) as e:
        bm.append(0, 5)  # needs 2 more blocks, 0 free... 3 used
    assert e.value.status == -6
    after = bm.block_table([0], 4)
    assert (before[0] == after[0]).all() and before[1][0] == after[1][0] == 10
    bm.fork(0, 1)
    with pytest.raises(B.PAError):
        bm.append(1, 1)  # copy-on-write needs a block too
    assert bm.take_copies()[0].size == 0


def test_errors():
    with pytest.raises(B.PAError):
        B.BlockManager(0, 16)
    bm = B.BlockManager(4, 16)
    bm.add(1)
    for f in (lambda: bm.add(1), lambda: bm.add(-2), lambda: bm.append(9, 1),
              lambda: bm.fork(9, 3), lambda: bm.fork(1, 1), lambda: bm.free(9),
              lambda: bm.append(1, -1), lambda: bm.block_table([9], 4)):
        with pytest.raises(B.PAError):
            f()
    bm.append(1, 40)  # 3 blocks
    with pytest.raises(B.PAError) as e:
        bm.block_table([1], 2)
    assert e.value.status == -3


def run_scenario(seed, NB=48, Bs=4, Hkv=2, d=16, steps=120):
    """Random adds / appends / forks / frees against a Python model of each
    sequence's logical K/V rows; the pools are written through the slots
    the manager returns (after applying its copy-on-write pairs)."""
    rng = np.random.default_rng(seed)
    bm = B.BlockManager(NB, Bs)
    kp = np.full((NB, Bs, Hkv, d), np.nan, np.float32)
    vp = np.full((NB, Bs, Hkv, d), np.nan, np.float32)
    logical = {}  # seq -> (K rows list, V rows list)
    next_id = 0
    for _ in range(steps):
        op = rng.integers(0, 4)
        if op == 0 or not logical:
            bm.add(next_id)
            logical[next_id] = ([], [])
            next_id += 1
        elif op == 1:
            sid = int(rng.choice(list(logical)))
            n = int(rng.integers(1, 9))
            try:
                slots = bm.append(sid, n)
            except B.PAError as e:
                assert e.status == -6
                continue
            src, dst = bm.take_copies()
            for a_, b_ in zip(src, dst):  # copy-on-write before writing
                kp[b_] = kp[a_]
                vp[b_] = vp[a_]
            kn = rng.standard_normal((n, Hkv, d)).astype(np.float32)
            vn = rng.standard_normal((n, Hkv, d)).astype(np.float32)
            for i, x in enumerate(slots):
                assert bm.refcount(int(x) // Bs) == 1  # written blocks are exclusive
                kp[x // Bs, x % Bs] = kn[i]
                vp[x // Bs, x % Bs] = vn[i]
            logical[sid][0].extend(kn)
            logical[sid][1].extend(vn)
        elif op == 2:
            sid = int(rng.choice(list(logical)))
            bm.fork(sid, next_id)
            logical[next_id] = (list(logical[sid][0]), list(logical[sid][1]))
            next_id += 1
        else:
            sid = int(rng.choice(list(logical)))
            bm.free(sid)
            del logical[sid]
    return bm, kp, vp, logical


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_random_scenario_tables_gather_the_logical_tokens(seed):
    NB, Bs = 48, 4
    bm, kp, vp, logical = run_scenario(seed, NB, Bs)
    ids = sorted(logical)
    MB = NB
    table, lens = bm.block_table(ids, MB)
    held = {}
    for row, sid in zip(table, ids):
        n = len(logical[sid][0])
        nblk = -(-n // Bs)
        assert (row[nblk:] == -1).all() and (row[:nblk] >= 0).all()
        for b in row[:nblk]:
            held[int(b)] = held.get(int(b), 0) + 1
        if n:
            t = np.arange(n)
            got_k = kp[row[t // Bs], t % Bs]
            got_v = vp[row[t // Bs], t % Bs]
            assert np.array_equal(got_k, np.stack(logical[sid][0]))
            assert np.array_equal(got_v, np.stack(logical[sid][1]))
    # Every block is either free or held, with the refcount the tables imply.
    assert bm.num_free + len(held) == NB
    assert all(bm.refcount(b) == c for b, c in held.items())


def test_random_scenario_attention_matches_dense():
    """Decode through the manager's tables (paged oracle) equals attention
    over each sequence's contiguous logical rows."""
    Bs, Hkv, d, G = 4, 2, 16, 2
    bm, kp, vp, logical = run_scenario(11, 48, Bs, Hkv, d)
    ids = [s for s in sorted(logical) if logical[s][0]]
    assert len(ids) >= 2
    table, lens = bm.block_table(ids, 48)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((len(ids), Hkv * G, d)).astype(np.float32)
    paged, _ = oracle.decode(q, kp, vp, table, lens, 0.25, "f32")
    for i, sid in enumerate(ids):
        K = np.stack(logical[sid][0]).astype(np.float64)  # [n, Hkv, d]
        V = np.stack(logical[sid][1]).astype(np.float64)
        for h in range(Hkv * G):
            x = K[:, h // G] @ q[i, h].astype(np.float64) * 0.25
            p = np.exp(x - x.max())
            ref = (p / p.sum()) @ V[:, h // G]
            assert np.allclose(paged[i, h], ref, rtol=0, atol=1e-12)


def test_queued_copy_keeps_its_source_out_of_the_free_list():
    """A shared partial block X is copied for sequence 1 (pair X -> Y
    queued); its other holder is freed before the pair is taken.  X must not
    return to the free list while the pair waits, so a second copy-on-write
    in the same batch cannot be handed X as its fresh destination (which
    would make one batch copy into X and out of X at once)."""
    bm = B.BlockManager(8, 4)
    bm.add(0)
    bm.append(0, 2)                 # X, 2 of 4 slots used
    x = int(bm.block_table([0], 1)[0][0, 0])
    bm.fork(0, 1)
    bm.append(1, 1)                 # X shared and partial: X -> Y queued
    free_before = bm.num_free
    bm.free(0)                      # X's last holder leaves; the pair still names X
    assert bm.num_free == free_before and bm.refcount(x) == 0
    bm.add(3)
    bm.append(3, 2)
    bm.fork(3, 4)
    bm.append(4, 1)                 # a second copy-on-write in the same batch
    src, dst = bm.take_copies()
    assert len(src) == 2
    assert not set(src.tolist()) & set(dst.tolist()) and len(set(dst.tolist())) == 2
    assert x not in dst.tolist()
    # Sequence 3's block and the second copy's destination were taken; X was
    # freed when its pair was taken.
    assert bm.num_free == free_before - 2 + 1
    bm.free(1)
    bm.free(3)
    bm.free(4)
    assert bm.num_free == 8


def test_copy_of_a_queued_destination_is_refused():
    """A block that is the destination of a queued pair holds no copied data
    yet; copying it again in the same batch is refused, state unchanged, and
    allowed once the queue has been taken."""
    bm = B.BlockManager(8, 4)
    bm.add(0)
    bm.append(0, 2)
    bm.fork(0, 1)
    bm.append(1, 1)                 # X -> Y queued; sequence 1 now holds Y
    bm.fork(1, 2)                   # Y shared by 1 and 2 while still a queued destination
    before = (bm.num_free, bm.block_table([1, 2], 2))
    with pytest.raises(B.PAError) as e:
        bm.append(2, 1)
    assert e.value.status == -8
    after = (bm.num_free, bm.block_table([1, 2], 2))
    assert before[0] == after[0] and (before[1][0] == after[1][0]).all()
    assert (before[1][1] == after[1][1]).all()
    src, dst = bm.take_copies()
    assert len(src) == 1
    y = int(dst[0])
    bm.append(2, 1)                 # now Y -> Z is queued
    src2, dst2 = bm.take_copies()
    assert list(src2) == [y] and int(dst2[0]) != y


@pytest.mark.parametrize("seed", [4, 5, 6, 7])
def test_batched_copies_are_independent(seed):
    """Random adds / appends / forks / frees with the copy queue taken only
    every few operations, following the documented order of work (run a
    batch's copies, then write the tokens of the appends before it; write
    pending tokens before a fork).  Every batch is a set of independent
    pairs, and the final tables gather every sequence's logical tokens."""
    rng = np.random.default_rng(seed)
    NB, Bs, Hkv, d = 40, 4, 1, 4
    bm = B.BlockManager(NB, Bs)
    kp = np.full((NB, Bs, Hkv, d), np.nan, np.float32)
    logical = {}
    writes = []  # (seq, slots, rows) appended since the last flush
    next_id = 0

    def flush():
        src, dst = bm.take_copies()
        assert not set(src.tolist()) & set(dst.tolist()), (src, dst)
        assert len(set(dst.tolist())) == len(dst)
        for a_, b_ in zip(src, dst):
            kp[b_] = kp[a_]
        for sid, slots, rows in writes:
            if sid in logical:  # a freed sequence's tokens are dropped
                for x, r in zip(slots, rows):
                    kp[x // Bs, x % Bs] = r
        writes.clear()

    for step in range(300):
        op = rng.integers(0, 5)
        if op == 0 or not logical:
            bm.add(next_id)
            logical[next_id] = []
            next_id += 1
        elif op in (1, 2):
            sid = int(rng.choice(list(logical)))
            n = int(rng.integers(1, 6))
            try:
                slots = bm.append(sid, n)
            except B.PAError as e:
                if e.status == -8:      # copy of a queued destination: flush, retry
                    flush()
                    try:
                        slots = bm.append(sid, n)
                    except B.PAError as e2:
                        assert e2.status == -6
                        continue
                else:
                    assert e.status == -6
                    continue
            rows = rng.standard_normal((n, Hkv, d)).astype(np.float32)
            writes.append((sid, slots, rows))
            logical[sid].extend(rows)
        elif op == 3:
            sid = int(rng.choice(list(logical)))
            flush()  # the child shares the parent's slots: write them first
            bm.fork(sid, next_id)
            logical[next_id] = list(logical[sid])
            next_id += 1
        else:
            sid = int(rng.choice(list(logical)))
            bm.free(sid)
            del logical[sid]
        if rng.random() < 0.2:
            flush()
    flush()
    ids = sorted(logical)
    table, lens = bm.block_table(ids, NB)
    held = {}
    for row, sid in zip(table, ids):
        n = len(logical[sid])
        assert lens[ids.index(sid)] == n
        for b in row[:-(-n // Bs)]:
            held[int(b)] = held.get(int(b), 0) + 1
        if n:
            t = np.arange(n)
            assert np.array_equal(kp[row[t // Bs], t % Bs], np.stack(logical[sid]))
    assert bm.num_free + len(held) == NB
    assert all(bm.refcount(b) == c for b, c in held.items())
