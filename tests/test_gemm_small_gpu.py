"""GPU tolerance tests of the small-product GEMM path (one wave per 32 x 32
output tile, operands straight into registers): E2M1 with E8M0 scales on
the scaled FP4 instruction (block 32, and block 16 as two runs per K-half
with the other block of A zeroed; gonzo_ML/3986 "Форматы FP4": groups of 16
with power-of-two scales), E2M1 with the f16-exact scale formats
(E4M3, E3M4, E2M5, E1M6; gonzo_ML/3986 "Форматы FP4") converted to f16, and
with UE5M3 and the other wide-exponent formats (ue5m3-fp4-pretraining "Что
сделали") converted to bf16 in registers.

As for the tiled kernels: the operands are quantized on the GPU and by the
oracle and checked byte-identical, and every bf16 output must be the bf16
rounding of some value within 1e-5 * sum_k |a_k||b_k| of the binary64
product of the exactly dequantized operands.  The bound on the path
(fp4_set_gemm_small_outputs) is raised so that mid-sized shapes take it too,
and set to 0 to check that the same shapes still run on the tiled kernels.
"""
import numpy as np
import pytest
import torch

import fp4_inputs as inputs
import oracle
from tests.gpu_util import assert_bytes_equal, host, to_device

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp4_block_scaled_quantize_amd")


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture
def small_path():
    """Every product below takes the small path, whatever its size."""
    prev = fq.set_gemm_small_outputs(1 << 40)
    try:
        yield
    finally:
        fq.set_gemm_small_outputs(prev)


def _quant_both(x_np, block, fmt):
    pol = "none" if fmt == "e8m0" else "current"
    qt = fq.fp4_quantize(to_device(x_np), block, fmt, amax=pol)
    q, s, g, _ = oracle.quantize_tensor(x_np, block, fmt, pol, nthreads=8)
    torch.cuda.synchronize()
    assert_bytes_equal(host(qt.q), q, f"{fmt}/{block} operand codes")
    assert_bytes_equal(host(qt.scales), s, f"{fmt}/{block} operand scales")
    return qt, oracle.dequantize_f64(q, s, g, block, fmt)


def _check(c_gpu, a_hat, w_hat, tag):
    cref, tol = oracle.gemm_ref(a_hat, w_hat)
    c = c_gpu.float().cpu().numpy().astype(np.float64)
    ok = oracle.gemm_check(c, cref, tol)
    if not ok.all():
        i, j = np.argwhere(~ok)[0]
        raise AssertionError(f"{tag}: {int((~ok).sum())} of {ok.size} outputs out of tolerance; first ({i},{j}) "
                             f"got {c[i, j]!r} ref {cref[i, j]!r} tol {tol[i, j]!r}")


def _normal(rows, cols, seed, std=1.0):
    return (np.random.default_rng(seed).standard_normal((rows, cols)) * std).astype(np.float32)


def test_small_configuration_default_bound():
    """The 64x256 @ (256x256)^T NVFP4 product of the 1%-outlier matrices at
    the default bound (16384 outputs: the small path)."""
    qa, a = _quant_both(inputs.small_a(), 16, "e4m3")
    qb, b = _quant_both(inputs.small_b(), 16, "e4m3")
    c = fq.fp4_gemm(qa, qb)
    torch.cuda.synchronize()
    _check(c, a, b, "small configuration")


# M, N ragged against the 32 x 32 wave tiles and the four-wave workgroups;
# K = 128 (two chunks, fewer than the eight in flight), 8 + 2 chunks, and
# 64 chunks (eight rounds of eight)
SHAPES = [(64, 256, 256), (1, 33, 128), (70, 300, 384), (257, 513, 640), (33, 1000, 4096), (5, 130, 1152)]


@pytest.mark.parametrize("fmt,block", [("e4m3", 16), ("e4m3", 32), ("e3m4", 16), ("e2m5", 32), ("e1m6", 16),
                                       ("e8m0", 32), ("e8m0", 16), ("ue5m3", 16), ("e5m2", 32), ("e6m1", 16),
                                       ("e7m0", 16)])
@pytest.mark.parametrize("m,n,k", SHAPES)
def test_small_path_formats(small_path, fmt, block, m, n, k):
    qa, a = _quant_both(_normal(m, k, 11 + m), block, fmt)
    qb, b = _quant_both(_normal(n, k, 12 + n, 0.02), block, fmt)
    c = fq.fp4_gemm(qa, qb)
    torch.cuda.synchronize()
    _check(c, a, b, f"small {fmt}/{block} {m}x{n}x{k}")


@pytest.mark.parametrize("fa,fb", [("e4m3", "e3m4"), ("e1m6", "e4m3"), ("e2m5", "e3m4"), ("e4m3", "ue5m3"),
                                   ("ue5m3", "e7m0")])
def test_small_path_mixed_formats(small_path, fa, fb):
    """Different scale formats on the two operands (each decoded by its own
    format; f16 pairs, and pairs that need bf16)."""
    qa, a = _quant_both(_normal(45, 768, 21), 16, fa)
    qb, b = _quant_both(_normal(90, 768, 22, 0.02), 16, fb)
    c = fq.fp4_gemm(qa, qb)
    torch.cuda.synchronize()
    _check(c, a, b, f"small {fa} x {fb}")


def test_small_path_wide_range_and_outliers(small_path):
    """Rows spanning many binades (x 2^-20 .. 2^20 per row) with 1% outliers
    x50: block scales over the whole E4M3 range, and E8M0 scales far apart."""
    rng = np.random.default_rng(5)
    for fmt, block in (("e4m3", 16), ("e8m0", 32), ("e8m0", 16), ("ue5m3", 16), ("e7m0", 32)):
        a = _normal(40, 512, 31) * np.exp2(rng.integers(-20, 21, (40, 1))).astype(np.float32)
        w = _normal(72, 512, 32, 0.02)
        w[rng.random(w.shape) < 0.01] *= 50
        qa, ah = _quant_both(a, block, fmt)
        qb, bh = _quant_both(w, block, fmt)
        c = fq.fp4_gemm(qa, qb)
        torch.cuda.synchronize()
        _check(c, ah, bh, f"wide range {fmt}/{block}")


def test_small_path_strided_output(small_path):
    """An output with an odd row stride (element stores) and one with a
    padded even stride: the columns past N are left as they were."""
    qa, a = _quant_both(_normal(37, 256, 41), 16, "e4m3")
    qb, b = _quant_both(_normal(70, 256, 42, 0.02), 16, "e4m3")
    for ld in (71, 76):
        buf = torch.full((37, ld), 3.0, dtype=torch.bfloat16, device="cuda")
        fq.fp4_gemm(qa, qb, out=buf[:, :70])
        torch.cuda.synchronize()
        _check(buf[:, :70], a, b, f"ldc {ld}")
        assert bool((buf[:, 70:] == 3.0).all())


@pytest.mark.parametrize("fmt,block", [("e4m3", 16), ("e8m0", 32)])
def test_bound_selects_the_path(fmt, block):
    """The same mid-sized product (300 x 4000 outputs) with the bound at 0
    (tiled kernels) and above it (small path): both within the error bound."""
    qa, a = _quant_both(_normal(300, 1024, 51), block, fmt)
    qb, b = _quant_both(_normal(4000, 1024, 52, 0.02), block, fmt)
    prev = fq.set_gemm_small_outputs(0)
    try:
        c0 = fq.fp4_gemm(qa, qb)
        fq.set_gemm_small_outputs(8 * 300 * 4000)
        c1 = fq.fp4_gemm(qa, qb)
    finally:
        fq.set_gemm_small_outputs(prev)
    torch.cuda.synchronize()
    _check(c0, a, b, f"tiled {fmt}/{block}")
    _check(c1, a, b, f"small {fmt}/{block}")


def _quant_elem(x_np, block, fmt, elem):
    pol = "none" if fmt == "e8m0" else "current"
    qt = fq.fp4_quantize(to_device(x_np), block, fmt, amax=pol, element=elem)
    q, s, g, _ = oracle.quantize_tensor(x_np, block, fmt, pol, nthreads=8, elem=elem)
    torch.cuda.synchronize()
    assert_bytes_equal(host(qt.q), q, f"{elem} {fmt}/{block} operand codes")
    assert_bytes_equal(host(qt.scales), s, f"{elem} {fmt}/{block} operand scales")
    return qt, oracle.dequantize_f64(q, s, g, block, fmt, elem=elem)


@pytest.mark.parametrize("elem,fmt,block", [("fp8_e4m3", "e8m0", 32), ("fp8_e4m3", "e8m0", 16),
                                            ("int8", "e4m3", 16), ("int8", "e4m3", 32)])
@pytest.mark.parametrize("m,n,k", SHAPES)
def test_small_path_8bit(small_path, elem, fmt, block, m, n, k):
    """The 8-bit pairings of the register-conversion kernel on the small
    path (quant_prune_distill/486 "Метод": MXFP8; quant_prune_distill/574
    "Метод": INT8 beside FP8): MXFP8 to bf16 with the E8M0 scale applied,
    INT8 with E4M3 scales to f16; 32 bytes per lane per chunk."""
    qa, a = _quant_elem(_normal(m, k, 61 + m), block, fmt, elem)
    qb, b = _quant_elem(_normal(n, k, 62 + n, 0.02), block, fmt, elem)
    c = fq.fp4_gemm(qa, qb)
    torch.cuda.synchronize()
    _check(c, a, b, f"small {elem} {fmt}/{block} {m}x{n}x{k}")


@pytest.mark.parametrize("elem,fmt,block", [("fp8_e4m3", "e8m0", 32), ("int8", "e4m3", 16)])
def test_small_path_8bit_wide_range(small_path, elem, fmt, block):
    """Rows spanning many binades with outliers on the 8-bit grids."""
    rng = np.random.default_rng(8)
    a = _normal(40, 512, 33) * np.exp2(rng.integers(-20, 21, (40, 1))).astype(np.float32)
    w = _normal(72, 512, 34, 0.02)
    w[rng.random(w.shape) < 0.01] *= 50
    qa, ah = _quant_elem(a, block, fmt, elem)
    qb, bh = _quant_elem(w, block, fmt, elem)
    c = fq.fp4_gemm(qa, qb)
    torch.cuda.synchronize()
    _check(c, ah, bh, f"wide range {elem} {fmt}/{block}")


@pytest.mark.parametrize("elem,fmt", [("fp8_e4m3", "e8m0"), ("int8", "e4m3")])
def test_small_path_8bit_every_code(small_path, elem, fmt):
    """Every 8-bit element code through the small path's decode (the tiled
    kernels' every-code case, run here with the small path forced)."""
    from tests import test_8bit_gpu
    test_8bit_gpu.test_8bit_gemm_every_code(elem, fmt)


def test_small_path_mxfp8_subnormal_products(small_path):
    """MXFP8 products below bf16's normal range through the small path (the
    tiled kernels' subnormal case, run here with the small path forced)."""
    from tests import test_8bit_gpu
    test_8bit_gpu.test_mxfp8_gemm_subnormal_products()
