"""The library's measurement aids on the GPU: per-launch kernel times and the
shader-clock probe the benchmark uses."""

import pytest
import torch

from paged_kv_cache_decode_amd import workloads as W
from tests.gpu_helpers import case_to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_decode_amd import binding
    binding.lib()
    return binding


def test_profiler_samples_match_totals(pa):
    c = W.tiny_f32_decode()
    dev = case_to_dev(c)
    pa.profiler_reset()
    pa.profiler_enable(True)
    try:
        for _ in range(5):
            pa.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_table"],
                      dev["context_lens"], c.scale)
        torch.cuda.synchronize()
    finally:
        pa.profiler_enable(False)
    total, n = pa.profiler_read("decode_partitions")
    samples = pa.profiler_samples("decode_partitions")
    assert n == 5 and len(samples) == 5
    assert all(s > 0 for s in samples)
    assert abs(sum(samples) - total) <= 1e-6 * max(1.0, total)
    assert pa.profiler_samples("write_kv") == []
    pa.profiler_reset()
    assert pa.profiler_samples("decode_partitions") == []


def test_clock_probe_counts_the_reference_ticks_it_waits(pa):
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    pa.clock_probe(out, 20000, stream=side)  # 0.2 ms of the 100 MHz counter
    torch.cuda.synchronize()
    shader, ref = (int(x) for x in out.tolist())
    assert 20000 <= ref < 20000 + 5000
    mhz = 100.0 * shader / ref
    assert 300.0 < mhz < 4000.0, mhz
