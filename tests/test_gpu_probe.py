"""The register-only FP4 MFMA probe (moe_mxfp4_mfma_probe), a measurement aid
for the MFMA-bound kernels' roofline: its figures must be physically possible
and its argument checks must hold."""
import pytest

from tests.moe_cases import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def binding(gpu_device):
    from mixture_experts_mxfp4_amd import binding
    return binding


@pytest.mark.parametrize("small_tile", [False, True])
@pytest.mark.parametrize("random_operands", [True, False])
def test_mfma_probe_rate_is_physical(binding, random_operands, small_tile):
    r = binding.moe_mxfp4_mfma_probe(random_operands, 20000, small_tile=small_tile)
    log(f"mfma probe random={random_operands} 16x16x128={small_tile}: {r}")
    assert 300.0 < r["shader_mhz"] < 3000.0
    # at most the FP4 peak per clock, one 32x32x64 MFMA per 32 cycles per SIMD
    # (a little slack for the two clocks' read points), and at most the
    # published peak times the clock ratio
    assert 0.05 < r["per_clock_frac"] <= 1.02
    assert 0.0 < r["tflops"] <= 10100.0 * r["shader_mhz"] / 2400.0 * 1.02


def test_mfma_probe_rejects_bad_arguments(binding):
    for iters in (0, -1, (1 << 24) + 1):
        with pytest.raises(binding.MoeMxfp4Error):
            binding.moe_mxfp4_mfma_probe(True, iters)
    for flags in (4, 8, -1):
        with pytest.raises(binding.MoeMxfp4Error):
            binding.moe_mxfp4_mfma_probe(True, 100, flags=flags)
