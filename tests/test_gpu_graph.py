"""HIP graph capture of the library's calls.

A decode/prefill step captured once and replayed must give, at every
replay, exactly what the same call gives eagerly on the buffers' contents at
that time (the kernels are deterministic: same inputs, same bits -- every
merge of split work reads its parts in a fixed order, whichever workgroup
happens to run it).  Between
replays the test changes the inputs with eager work on another stream and
synchronises, as a serving loop would.  A decode call whose stream workspace
would have to grow during a capture must fail cleanly instead of recording
an allocation."""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_decode_amd import workloads as W
from tests.gpu_helpers import assert_close_f32_out, case_to_dev, out_to_f64, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_decode_amd import binding
    binding.lib()
    return binding


def new_q(c, seed):
    rng = np.random.default_rng(seed)
    return W.f32_to_storage(rng.standard_normal(c.q.shape, dtype=np.float32), c.dtype)


def test_decode_graph_replays(pa):
    c = W.make_decode_case(801, 24, 32, 8, 128, 16, "bf16", len_range=(1, 900))
    dev = case_to_dev(c)
    args = lambda: (dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                    dev["context_lens"], c.scale)
    s = torch.cuda.Stream()
    out_g = torch.empty(dev["q"].shape, dtype=torch.float32, device="cuda")
    with torch.cuda.stream(s):
        pa.decode(*args(), out=out_g)  # sizes this stream's workspace
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pa.decode(*args(), out=out_g)
    for i in range(3):
        qi = new_q(c, 900 + i)
        dev["q"].copy_(to_dev(qi, c.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = pa.decode(*args(), out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(out_g, eager), f"replay {i}"
    ref, _ = oracle.decode(qi, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale,
                           c.dtype)
    assert_close_f32_out(out_to_f64(out_g), ref, c.dtype, "last replay vs oracle")
    pa.workspace_release(s)


def test_decode_graph_survives_workspace_growth(pa, monkeypatch):
    """A graph captured on a stream keeps working after a later, larger
    eager call on that stream grows the stream's workspace: the captured
    buffer is kept, not freed (the library frees it only at
    pa_workspace_release).  Every replay equals the eager call bit for bit,
    and the last one the oracle."""
    monkeypatch.setenv("PA_DECODE_WORKERS", "256")
    small = W.make_decode_case(811, 6, 32, 8, 128, 16, "bf16", len_range=(300, 2000))
    big = W.make_decode_case(812, 96, 32, 8, 128, 16, "bf16", len_range=(1, 3000))
    ds, db = case_to_dev(small), case_to_dev(big)
    args_s = lambda: (ds["q"], ds["k_pool"], ds["v_pool"], ds["block_table"],  # noqa: E731
                      ds["context_lens"], small.scale)
    s = torch.cuda.Stream()
    out_g = torch.empty(ds["q"].shape, dtype=torch.float32, device="cuda")
    with torch.cuda.stream(s):
        pa.decode(*args_s(), out=out_g)  # sizes the stream's workspace for `small`
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pa.decode(*args_s(), out=out_g)
    plan_s = pa.decode_plan(ds["q"], ds["k_pool"], ds["v_pool"], ds["block_table"],
                            ds["context_lens"], out_g)
    out_b = torch.empty(db["q"].shape, dtype=torch.float32, device="cuda")
    plan_b = pa.decode_plan(db["q"], db["k_pool"], db["v_pool"], db["block_table"],
                            db["context_lens"], out_b)
    assert plan_b["workspace_bytes"] > 2 * plan_s["workspace_bytes"]  # the call below grows it
    for i in range(3):
        with torch.cuda.stream(s):
            pa.decode(db["q"], db["k_pool"], db["v_pool"], db["block_table"],
                      db["context_lens"], big.scale, out=out_b, stream=s.cuda_stream)
        s.synchronize()
        qi = new_q(small, 1100 + i)
        ds["q"].copy_(to_dev(qi, small.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = pa.decode(*args_s(), out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(out_g, eager), f"replay {i}"
    ref, _ = oracle.decode(qi, small.k_pool, small.v_pool, small.block_table,
                           small.context_lens, small.scale, small.dtype)
    assert_close_f32_out(out_to_f64(out_g), ref, small.dtype, "last replay vs oracle")
    ref_b, _ = oracle.decode(big.q, big.k_pool, big.v_pool, big.block_table, big.context_lens,
                             big.scale, big.dtype)
    assert_close_f32_out(out_to_f64(out_b), ref_b, big.dtype, "the growing call vs oracle")
    del g
    pa.workspace_release(s)
    s.synchronize()


def test_decode_capture_without_workspace_fails_cleanly(pa):
    c = W.make_decode_case(802, 8, 32, 8, 128, 16, "f16", len_range=(200, 700))
    dev = case_to_dev(c)
    out = torch.empty(dev["q"].shape, dtype=torch.float32, device="cuda")
    pa.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"], dev["context_lens"],
              c.scale, out=out)  # first use of this instance happens outside any capture
    torch.cuda.synchronize()
    s = torch.cuda.Stream()  # no call on it yet: no workspace
    g = torch.cuda.CUDAGraph()
    with pytest.raises(pa.PAError) as e:
        with torch.cuda.graph(g, stream=s):
            pa.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                      dev["context_lens"], c.scale, out=out)
    assert e.value.status == -6
    # The stream is usable afterwards, eagerly and in a new capture.
    with torch.cuda.stream(s):
        pa.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                  dev["context_lens"], c.scale, out=out)
    s.synchronize()
    eager = out.clone()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2, stream=s):
        pa.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                  dev["context_lens"], c.scale, out=out)
    out.zero_()
    torch.cuda.synchronize()
    g2.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, eager)
    pa.workspace_release(s)


def test_prefill_graph_replays(pa):
    c = W.make_prefill_case(803, 3, 32, 8, 128, 16, "bf16", lens=[300, 129, 530],
                            query_lens=[300, 64, 200], causal=True)
    dev = case_to_dev(c)
    args = lambda: (dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                    dev["context_lens"], dev["query_start_loc"], c.max_query_len, c.scale)
    out_g = torch.empty(dev["q"].shape, dtype=torch.float32, device="cuda")
    pa.prefill(*args(), causal=True, out=out_g)  # first use outside any capture
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pa.prefill(*args(), causal=True, out=out_g)
    for i in range(3):
        dev["q"].copy_(to_dev(new_q(c, 910 + i), c.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = pa.prefill(*args(), causal=True, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(out_g, eager), f"replay {i}"


def test_decode_step_graph_with_write_kv(pa):
    """One serving step -- store the new token's K/V, then attend -- captured
    once; each replay appends one more token per sequence (slots and lengths
    are device buffers the host updates between replays)."""
    dtype, S, Hkv, G, d, B = "bf16", 6, 8, 4, 128, 16
    steps = 3
    base = [40, 17, 130, 1, 64, 95]
    c = W.make_decode_case(804, S, Hkv * G, Hkv, d, B, dtype,
                           lens=[n + steps for n in base])
    dev = case_to_dev(c)
    k_eager, v_eager = dev["k_pool"].clone(), dev["v_pool"].clone()
    lens_dev = to_dev(np.array(base, np.int32))
    slots_dev = to_dev(np.zeros(S, np.int32))
    k_new = torch.empty((S, Hkv, d), dtype=dev["q"].dtype, device="cuda")
    v_new = torch.empty_like(k_new)
    out_g = torch.empty(dev["q"].shape, dtype=torch.float32, device="cuda")

    def step(kp, vp, slots, lens, out):
        pa.write_kv(k_new, v_new, slots, kp, vp)
        pa.decode(dev["q"], kp, vp, dev["block_table"], lens, c.scale, out=out)

    # First use of write_kv outside any capture, on a scratch pool of one block.
    scratch = torch.zeros((1, B, Hkv, d), dtype=dev["q"].dtype, device="cuda")
    pa.write_kv(k_new[:1].zero_(), v_new[:1].zero_(), slots_dev[:1], scratch, scratch.clone())
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):  # sizes the workspace; writes are redone below
        pa.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                  to_dev(np.array([n + steps for n in base], np.int32)), c.scale, out=out_g)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(dev["k_pool"], dev["v_pool"], slots_dev, lens_dev, out_g)
    rng = np.random.default_rng(5)
    for i in range(steps):
        pos = np.array(base) + i  # the new token's position
        slots = np.array([c.block_table[j, p // B] * B + p % B for j, p in enumerate(pos)],
                         np.int32)
        slots_dev.copy_(to_dev(slots))
        lens_dev.copy_(to_dev((pos + 1).astype(np.int32)))
        k_new.copy_(to_dev(W.f32_to_storage(
            rng.standard_normal((S, Hkv, d), dtype=np.float32), dtype), dtype))
        v_new.copy_(to_dev(W.f32_to_storage(
            rng.standard_normal((S, Hkv, d), dtype=np.float32), dtype), dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = torch.empty_like(out_g)
        step(k_eager, v_eager, slots_dev, lens_dev, eager)
        torch.cuda.synchronize()
        assert torch.equal(out_g, eager), f"step {i}"
        # Unwritten slots hold NaN: compare the pools' bits.
        assert torch.equal(dev["k_pool"].view(torch.int16), k_eager.view(torch.int16))
        assert torch.equal(dev["v_pool"].view(torch.int16), v_eager.view(torch.int16))
    pa.workspace_release(s)


def test_shared_prefix_graph_replays(pa):
    c = W.make_prefix_shared_case(805, 16, num_seqs=20, prefix_len=256, suffix_range=(0, 200),
                                  dtype="bf16")
    dev = case_to_dev(c)
    args = lambda: (dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                    dev["context_lens"], 256, c.scale)
    out_g = torch.empty(dev["q"].shape, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        pa.decode_shared_prefix(*args(), out=out_g)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pa.decode_shared_prefix(*args(), out=out_g)
    for i in range(3):
        qi = new_q(c, 920 + i)
        dev["q"].copy_(to_dev(qi, c.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = pa.decode_shared_prefix(*args(), out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(out_g, eager), f"replay {i}"
    ref, _ = oracle.decode(qi, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale,
                           c.dtype)
    assert_close_f32_out(out_to_f64(out_g), ref, c.dtype, "last replay vs oracle")
    pa.workspace_release(s)


def test_context_split_graph_replays(pa):
    """Two key ranges decoded with pa_decode_lse into slices of one buffer and
    joined with pa_merge_states, captured once and replayed."""
    from tests.test_gpu_context_split import split_by_blocks
    c = W.make_decode_case(805, 10, 32, 8, 128, 16, "bf16", len_range=(1, 1500))
    dev = case_to_dev(c)
    parts = [(to_dev(t), to_dev(n)) for t, n in split_by_blocks(c, [0, 40, 200])]
    S, H, d = c.q.shape
    part_out = torch.empty((2, S, H, d), dtype=torch.float32, device="cuda")
    part_lse = torch.empty((2, S, H), dtype=torch.float32, device="cuda")

    def step(out, lse):
        for p, (tab, lens) in enumerate(parts):
            pa.decode_lse(dev["q"], dev["k_pool"], dev["v_pool"], tab, lens, c.scale,
                          out=part_out[p], lse=part_lse[p])
        pa.merge_states(part_out, part_lse, out=out, lse=lse)

    out_g = torch.empty((S, H, d), dtype=torch.float32, device="cuda")
    lse_g = torch.empty((S, H), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step(out_g, lse_g)  # sizes this stream's workspace
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(out_g, lse_g)
    for i in range(3):
        qi = new_q(c, 910 + i)
        dev["q"].copy_(to_dev(qi, c.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        out_e, lse_e = torch.empty_like(out_g), torch.empty_like(lse_g)
        step(out_e, lse_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {i}"
        assert torch.equal(lse_g, lse_e), f"replay {i} lse"
    ref, ref_lse = oracle.decode(qi, c.k_pool, c.v_pool, c.block_table, c.context_lens,
                                 c.scale, c.dtype)
    assert_close_f32_out(out_to_f64(out_g), ref, c.dtype, "last replay vs oracle")
    assert np.abs(lse_g.cpu().numpy() - ref_lse).max() <= 1e-4
    pa.workspace_release(s)
