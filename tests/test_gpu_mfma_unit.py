"""One block-scaled FP4 MFMA instruction (moe_mxfp4_debug_mfma) against the
oracle's MX dot product, for both instruction shapes the kernels use and every
scale byte select: the operand, scale and result layouts that every GEMM
kernel here relies on.

With one scale for all operands every product is a multiple of the same power
of two and the 32-bit accumulation is exact, so the result must equal the
oracle's fp64 dot bit for bit. With scales that differ per 32-element block,
the instruction's fp32 accumulation may round: the bound is 2^-22 of the sum of
the products' magnitudes."""
import numpy as np
import pytest
import torch

import oracle
from tests.moe_cases import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def binding(gpu_device):
    from mixture_experts_mxfp4_amd import binding as b
    return b


def _operands(rng, R, K, scale_lo, scale_hi):
    codes = rng.integers(0, 256, (R, K // 2), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi + 1, (R, K // 32)).astype(np.uint8)
    return codes, scales


def _oracle_product(a, as_, b, bs):
    R = a.shape[0]
    out = np.empty((R, R), dtype=np.float64)
    mag = np.empty((R, R), dtype=np.float64)
    da = oracle.dequantize_rows(a, as_)
    db = oracle.dequantize_rows(b, bs)
    for i in range(R):
        for j in range(R):
            out[i, j] = oracle.mx_dot(a[i], as_[i], b[j], bs[j])
            mag[i, j] = np.abs(da[i] * db[j]).sum()
    return out, mag


@pytest.mark.parametrize("sel", [0, 1, 2, 3])
@pytest.mark.parametrize("rows", [16, 32])
def test_mfma_matches_oracle_dot(binding, rows, sel):
    K = 128 if rows == 16 else 64
    rng = np.random.default_rng(100 * rows + sel)
    for label, lo, hi in (("one scale", 127, 127), ("mixed scales", 118, 136)):
        a, as_ = _operands(rng, rows, K, lo, hi)
        b, bs = _operands(rng, rows, K, lo, hi)
        if lo == hi:
            as_[:] = lo
            bs[:] = lo
        got = binding.moe_mxfp4_debug_mfma(*(torch.from_numpy(x).cuda() for x in (a, as_, b, bs)),
                                          sel=sel)
        torch.cuda.synchronize()
        got = got.cpu().numpy().astype(np.float64)
        want, mag = _oracle_product(a, as_, b, bs)
        err = np.abs(got - want)
        log(f"mfma {rows}x{rows} sel {sel} {label}: max |err| {err.max():.3g}, "
            f"max |want| {np.abs(want).max():.3g}")
        assert np.all(np.isfinite(got)), "a scale byte outside `sel` reached the instruction"
        if lo == hi:
            np.testing.assert_array_equal(got, want)
        else:
            assert np.all(err <= mag * 2.0 ** -22)


def test_mfma_transposition_and_layout(binding):
    """A single nonzero element in A row i and B row j lands at out[i][j]
    only: rows of the first operand run down the result, the second's across."""
    for rows in (16, 32):
        K = 128 if rows == 16 else 64
        for i, j, k in ((0, 0, 0), (rows - 1, 2, K - 1), (5, rows - 3, 37)):
            a = np.zeros((rows, K // 2), np.uint8)
            b = np.zeros((rows, K // 2), np.uint8)
            code = 0x2                                  # E2M1 1.0
            a[i, k // 2] = code << (4 * (k % 2))
            b[j, k // 2] = code << (4 * (k % 2))
            s = np.full((rows, K // 32), 127, np.uint8)
            got = binding.moe_mxfp4_debug_mfma(*(torch.from_numpy(x).cuda() for x in (a, s, b, s)))
            torch.cuda.synchronize()
            want = np.zeros((rows, rows), np.float32)
            want[i, j] = 1.0
            np.testing.assert_array_equal(got.cpu().numpy(), want)


def test_mfma_rejects_bad_arguments(binding):
    a = torch.zeros((16, 64), dtype=torch.uint8, device="cuda")
    s = torch.zeros((16, 4), dtype=torch.uint8, device="cuda")
    for sel in (-1, 4):
        with pytest.raises(binding.MoeMxfp4Error):
            binding.moe_mxfp4_debug_mfma(a, s, a, s, sel=sel)
    with pytest.raises(ValueError):
        binding.moe_mxfp4_debug_mfma(a[:8], s[:8], a[:8], s[:8])
