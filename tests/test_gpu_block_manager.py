"""GPU side of block management: pa_copy_blocks (copy-on-write) bit-exact,
and a random serving scenario -- sequences added, appended through the
host block manager's slots (pa_write_kv), forked (shared blocks), copied on
write (pa_copy_blocks), freed -- whose tables then drive pa_decode, checked
against the oracle on each sequence's logical tokens."""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_decode_amd import workloads as W
from tests.gpu_helpers import assert_close_f32_out, out_to_f64, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_decode_amd import binding
    binding.lib()
    return binding


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_copy_blocks_bit_exact(pa, dtype):
    rng = np.random.default_rng(21)
    NB, B, Hkv, d = 64, 16, 8, 128
    kp = W.f32_to_storage(rng.standard_normal((NB, B, Hkv, d), dtype=np.float32), dtype)
    vp = W.f32_to_storage(rng.standard_normal((NB, B, Hkv, d), dtype=np.float32), dtype)
    perm = rng.permutation(NB).astype(np.int32)
    src, dst = perm[:20], perm[20:40]  # disjoint
    k_ref, v_ref = kp.copy(), vp.copy()
    k_ref[dst] = kp[src]
    v_ref[dst] = vp[src]
    kd, vd = to_dev(kp, dtype), to_dev(vp, dtype)
    pa.copy_blocks(kd, vd, to_dev(src), to_dev(dst))
    pa.copy_blocks(kd, vd, to_dev(src[:0]), to_dev(dst[:0]))  # nothing to copy
    torch.cuda.synchronize()
    assert torch.equal(kd.cpu(), to_dev(k_ref, dtype).cpu())
    assert torch.equal(vd.cpu(), to_dev(v_ref, dtype).cpu())


def test_manager_driven_decode(pa):
    """Random serving scenario on the device pools; decode through the
    manager's tables equals attention over the logical tokens."""
    dtype, NB, Bs, Hkv, G, d = "bf16", 96, 16, 2, 4, 128
    rng = np.random.default_rng(33)
    bm = pa.BlockManager(NB, Bs)
    # Unwritten slots hold NaN: a read of one would poison the result.
    kd = to_dev(np.full((NB, Bs, Hkv, d), W.NAN_BITS[dtype], np.uint16), dtype)
    vd = kd.clone()
    logical = {}
    next_id = 0
    for _ in range(80):
        op = int(rng.integers(0, 4))
        if op == 0 or not logical:
            bm.add(next_id)
            logical[next_id] = ([], [])
            next_id += 1
        elif op == 1:
            sid = int(rng.choice(list(logical)))
            n = int(rng.integers(1, 40))
            try:
                slots = bm.append(sid, n)
            except pa.PAError as e:
                assert e.status == -6
                continue
            src, dst = bm.take_copies()
            if src.size:
                pa.copy_blocks(kd, vd, to_dev(src), to_dev(dst))
            kn = W.f32_to_storage(rng.standard_normal((n, Hkv, d), dtype=np.float32), dtype)
            vn = W.f32_to_storage(rng.standard_normal((n, Hkv, d), dtype=np.float32), dtype)
            pa.write_kv(to_dev(kn, dtype), to_dev(vn, dtype), to_dev(slots), kd, vd)
            logical[sid][0].extend(kn)
            logical[sid][1].extend(vn)
        elif op == 2:
            sid = int(rng.choice(list(logical)))
            bm.fork(sid, next_id)
            logical[next_id] = (list(logical[sid][0]), list(logical[sid][1]))
            next_id += 1
        elif len(logical) > 2:
            sid = int(rng.choice(list(logical)))
            bm.free(sid)
            del logical[sid]
    ids = [s for s in sorted(logical) if logical[s][0]]
    assert len(ids) >= 3
    MB = NB
    table, lens = bm.block_table(ids, MB)
    table[table < 0] = 0  # padding entries are never read; any id will do
    q = W.f32_to_storage(rng.standard_normal((len(ids), Hkv * G, d), dtype=np.float32), dtype)
    scale = 1.0 / np.sqrt(d)
    torch.cuda.synchronize()
    out = pa.decode(to_dev(q, dtype), kd, vd, to_dev(table), to_dev(lens), scale,
                    out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = out_to_f64(out)
    # Oracle on contiguous per-sequence layouts (one block per sequence).
    for i, sid in enumerate(ids):
        K = np.stack(logical[sid][0])[None]  # [1, n, Hkv, d] as one block
        V = np.stack(logical[sid][1])[None]
        n = K.shape[1]
        ref, _ = oracle.decode(q[i:i + 1], K, V, np.zeros((1, 1), np.int32),
                               np.array([n], np.int32), scale, dtype)
        assert_close_f32_out(got[i:i + 1], ref, dtype, f"sequence {sid} ({n} tokens)")
