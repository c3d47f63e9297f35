"""The MFMA rate measurement that the bench reports beside the roofline:
each mode runs, and what it reports is physically consistent (a positive
rate no higher than the matrix pipe's rate at the measured clock, a clock
within the part's range)."""

import pytest
import torch

pytestmark = pytest.mark.gpu

PEAK_AT_2400 = 2516.6  # dense bf16 TFLOP/s at the 2.4 GHz top clock (256 CUs x 4 SIMDs x 1024 flop/cycle)


@pytest.fixture(scope="module")
def vsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_flashattention_amd as m

    m.load_library()
    return m


@pytest.mark.parametrize("mode", ["random", "zero", "pingpong_softmax"])
def test_measure_mfma_reports_a_consistent_rate(vsa, mode):
    print(f"[gpu-measure] mode {mode}", flush=True)
    r = vsa.vsa_measure_mfma(mode, iters=20000)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    pipe = PEAK_AT_2400 * cus / 256 * r["clock_mhz"] / 2400.0  # MFMA rate at the measured clock
    print(f"[gpu-measure] {mode}: {r['tflops']:.1f} TFLOP/s at {r['clock_mhz']:.0f} MHz", flush=True)
    assert 300.0 < r["clock_mhz"] < 2600.0
    assert 0.0 < r["tflops"] <= 1.05 * pipe
