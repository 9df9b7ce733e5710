"""The achievable-peak probes the bench reports its kernels against: each runs on the GPU and
gives a rate within what an MI355X can deliver (published peaks: 2.5 PFLOP/s bf16 and
157.3 TFLOP/s fp32 on the matrix cores, 8 TB/s HBM, 2.4 GHz peak engine clock)."""
import pytest
import torch

import block_sparse_attention_scores_amd as sa

pytestmark = pytest.mark.gpu


def _rate(kind, buf, iters):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = 0.0
    for rep in range(3):
        e0.record()
        work = sa.peak_probe(kind, buf, iters)
        e1.record()
        torch.cuda.synchronize()
        if rep:
            best = max(best, work / (e0.elapsed_time(e1) * 1e-3))
    return best


def test_probe_rates_are_within_the_chip():
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")   # halves beyond the 256 MB cache
    bf16 = _rate(0, buf, 200) / 1e12
    fp32 = _rate(1, buf, 20) / 1e12
    copy = _rate(2, buf, 1) / 1e9
    print(f"\n[probe] bf16 {bf16:.0f} TFLOP/s, fp32 {fp32:.1f} TFLOP/s, copy {copy:.0f} GB/s", flush=True)
    assert 500 < bf16 <= 2516 * 1.01
    assert 20 < fp32 <= 157.3 * 1.01
    assert 1000 < copy <= 8000 * 1.05


def test_clock_probe_reads_a_plausible_shader_clock():
    buf = torch.zeros(16 << 20, dtype=torch.uint8, device="cuda")
    rate = sa.peak_probe(3, buf, 200)
    torch.cuda.synchronize()
    ticks = buf[:16].view(torch.int64).cpu().tolist()
    assert rate > 0 and ticks[0] > 0 and ticks[1] > 0
    ghz = ticks[0] / (ticks[1] / rate) / 1e9
    print(f"\n[probe] wall clock {rate / 1e6:.1f} MHz, shader clock under matrix load {ghz:.3f} GHz",
          flush=True)
    assert 0.5 < ghz <= 2.4 * 1.05
