"""The matrix-instruction probe used to state the clock-limited peak beside
the datasheet one: its rate cannot exceed the datasheet peak, its clock is in
the chip's range, and all-zero operands (no toggling data) sustain at least
the rate of random ones."""
import pytest
import torch

import workloads
from gpu_util import note

pytestmark = pytest.mark.gpu

DATASHEET_BF16_TFLOPS = 2516.6  # 256 CUs x 2.4 GHz x 4096 flop/clk


@pytest.fixture(scope="module")
def mf():
    import packed_varlen_attention_amd as m
    return m


def _operands(bits):
    return torch.from_numpy(bits.view("int16")).view(torch.bfloat16).to("cuda")


def test_probe_rate_and_clock(mf):
    rnd = _operands(workloads.normal(11, 0, (mf.PROBE_VECTORS * 8,), "bf16"))
    zero = torch.zeros(mf.PROBE_VECTORS * 8, dtype=torch.bfloat16, device="cuda")
    blocks = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    mf.mfma_probe(rnd, blocks, 2000)  # warm-up
    r = mf.mfma_probe(rnd, blocks, 20000)
    z = mf.mfma_probe(zero, blocks, 20000)
    note(f"probe random: {r['tflops']:.0f} TFLOP/s at {r['sclk_mhz']:.0f} MHz; "
         f"zeros: {z['tflops']:.0f} TFLOP/s at {z['sclk_mhz']:.0f} MHz")
    for x in (r, z):
        assert 100.0 < x["tflops"] <= DATASHEET_BF16_TFLOPS * 1.02
        assert 300.0 < x["sclk_mhz"] < 3000.0
    assert z["tflops"] >= 0.95 * r["tflops"]
