"""GPU tolerance tests of the block-scaled GEMM and the weight-only GEMM.

Reference: the oracle quantizes the same seeded inputs, dequantizes them
exactly in binary64 and takes the product; a bf16 output passes iff it is the
bf16 rounding of some value within 1e-5 * sum_k |a_k||b_k| of the exact
product.  The GPU operands are first checked to be byte-identical to the
oracle's, so the reference never depends on the HIP path.
"""
import numpy as np
import pytest
import torch

import fp4_inputs as inputs
import oracle
from tests.gpu_util import assert_bytes_equal, check_gemm_every_output, host, to_device

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp4_block_scaled_quantize_amd")


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(autouse=True)
def _tiled_kernels():
    """These tests cover the tiled kernels, small shapes included (the
    small-product path has its own tests)."""
    prev = fq.set_gemm_small_outputs(0)
    try:
        yield
    finally:
        fq.set_gemm_small_outputs(prev)


def _policy(fmt):
    return "none" if fmt == "e8m0" else "current"


def _quant_both(x_np, block, fmt):
    """GPU quantization and the oracle's; asserts they are identical and
    returns (gpu QTensor, oracle exact binary64 dequantization)."""
    pol = _policy(fmt)
    qt = fq.fp4_quantize(to_device(x_np), block, fmt, amax=pol)
    q, s, g, _ = oracle.quantize_tensor(x_np, block, fmt, pol, nthreads=8)
    torch.cuda.synchronize()
    assert_bytes_equal(host(qt.q), q, "operand codes")
    assert_bytes_equal(host(qt.scales), s, "operand scales")
    return qt, oracle.dequantize_f64(q, s, g, block, fmt)


def _check_gemm(c_gpu, a_hat, w_hat, rows=None, tag=""):
    if rows is not None:
        a_hat = a_hat[rows]
    cref, tol = oracle.gemm_ref(a_hat, w_hat)
    c = c_gpu.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        c = c[rows]
    ok = oracle.gemm_check(c, cref, tol)
    if not ok.all():
        i, j = np.argwhere(~ok)[0]
        raise AssertionError(f"{tag}: {int((~ok).sum())} of {ok.size} outputs out of tolerance; first ({i},{j}) "
                             f"got {c[i, j]!r} ref {cref[i, j]!r} tol {tol[i, j]!r}")


def _normal(rows, cols, seed, std=1.0, dtype="f32"):
    x = (np.random.default_rng(seed).standard_normal((rows, cols)) * std).astype(np.float32)
    return inputs.f32_to_bf16_bits(x) if dtype == "bf16" else x


# ---------------------------------------------------------------------------
def test_small_nvfp4_gemm():
    """64x256 @ (256x256)^T, NVFP4 E4M3 block 16 from the 1%-outlier matrix."""
    qa, a = _quant_both(inputs.small_a(), 16, "e4m3")
    qb, b = _quant_both(inputs.small_b(), 16, "e4m3")
    c = fq.fp4_gemm(qa, qb)
    torch.cuda.synchronize()
    _check_gemm(c, a, b, tag="small nvfp4")


@pytest.mark.parametrize("m,n,k", [(64, 256, 256), (70, 300, 256), (300, 70, 512), (1, 33, 128), (257, 513, 384),
                                   (512, 256, 1024), (96, 200, 768), (130, 260, 1280), (40, 520, 1536)])
def test_mxfp4_native_shapes(m, n, k):
    """K in 256-element stages with scales in groups of four stages: K/256 =
    2, 3, 4, 5, 6 cover a partial last group, odd and even; K = 256 and
    multiples of 128 take the 128-element stages."""
    qa, a = _quant_both(_normal(m, k, 1), 32, "e8m0")
    qb, b = _quant_both(_normal(n, k, 2, 0.02), 32, "e8m0")
    c = fq.fp4_gemm(qa, qb)
    torch.cuda.synchronize()
    _check_gemm(c, a, b, tag=f"mxfp4 {m}x{n}x{k}")


@pytest.mark.parametrize("fmt", ["e4m3", "ue5m3", "e3m4", "e1m6", "e2m5", "e5m2", "e6m1", "e7m0"])
@pytest.mark.parametrize("block", [16, 32])
def test_dequant_path_formats(fmt, block):
    m, n, k = 96, 160, 256
    qa, a = _quant_both(_normal(m, k, 3, dtype="bf16"), block, fmt)
    qb, b = _quant_both(_normal(n, k, 4, 0.02, dtype="bf16"), block, fmt)
    c = fq.fp4_gemm(qa, qb)
    torch.cuda.synchronize()
    _check_gemm(c, a, b, tag=f"{fmt}/{block}")


def test_e8m0_at_block16_and_mixed_formats():
    m, n, k = 40, 72, 256
    x = _normal(m, k, 5)
    w = _normal(n, k, 6, 0.05)
    qa, a = _quant_both(x, 16, "e8m0")
    qb, b = _quant_both(w, 16, "e8m0")
    c = fq.fp4_gemm(qa, qb)
    torch.cuda.synchronize()
    _check_gemm(c, a, b, tag="e8m0/16")
    qa, a = _quant_both(x, 16, "e4m3")
    qb, b = _quant_both(w, 16, "ue5m3")
    c = fq.fp4_gemm(qa, qb)
    torch.cuda.synchronize()
    _check_gemm(c, a, b, tag="e4m3 x ue5m3")
    qa, a = _quant_both(x, 32, "e8m0")
    qb, b = _quant_both(w, 32, "e4m3")
    c = fq.fp4_gemm(qa, qb)
    torch.cuda.synchronize()
    _check_gemm(c, a, b, tag="e8m0 x e4m3")


@pytest.mark.parametrize("fmt,block", [("ue5m3", 16), ("e5m2", 32), ("e7m0", 16)])
@pytest.mark.parametrize("m,n,k", [(257, 513, 384), (300, 70, 1280), (64, 256, 128), (1, 33, 640)])
def test_bf16_register_path_shapes(fmt, block, m, n, k):
    """Scale formats whose products need bf16 (5 or more exponent bits),
    converted in registers: ragged tiles, one and many stages."""
    qa, a = _quant_both(_normal(m, k, 21, dtype="bf16"), block, fmt)
    qb, b = _quant_both(_normal(n, k, 22, 0.02, dtype="bf16"), block, fmt)
    c = fq.fp4_gemm(qa, qb)
    torch.cuda.synchronize()
    _check_gemm(c, a, b, tag=f"{fmt}/{block} {m}x{n}x{k}")


def test_ue5m3_wide_block_range():
    """Blocks whose magnitudes span 2^-40 .. 1 (current amax): the small
    blocks take UE5M3's smallest scale codes, the products stay exact."""
    m, n, k = 128, 256, 512
    rng = np.random.default_rng(23)
    def ranged(rows, seed):
        x = np.random.default_rng(seed).standard_normal((rows, k)).astype(np.float32)
        e = rng.integers(-40, 1, size=(rows, k // 16)).astype(np.float32)
        return (x * np.repeat(np.exp2(e), 16, axis=1)).astype(np.float32)
    xa, xw = ranged(m, 24), ranged(n, 25)
    for fa, fw in (("ue5m3", "ue5m3"), ("e4m3", "ue5m3"), ("ue5m3", "e4m3")):
        qa, a = _quant_both(xa, 16, fa)
        qb, b = _quant_both(xw, 16, fw)
        c = fq.fp4_gemm(qa, qb)
        torch.cuda.synchronize()
        _check_gemm(c, a, b, tag=f"{fa} x {fw} wide range")


def test_unsupported_pair_is_rejected():
    x = torch.randn(32, 128, device="cuda")
    qa = fq.fp4_quantize(x, 16, "e1m6")
    qb = fq.fp4_quantize(x, 16, "ue5m3")
    with pytest.raises(fq.Fp4Error) as e:
        fq.fp4_gemm(qa, qb)
    assert e.value.status == -2


def test_zero_operand():
    qa, a = _quant_both(np.zeros((33, 256), dtype=np.float32), 16, "e4m3")
    qb, b = _quant_both(_normal(40, 256, 7), 16, "e4m3")
    c = fq.fp4_gemm(qa, qb)
    torch.cuda.synchronize()
    assert not bool(c.float().abs().sum() > 0)


@pytest.mark.parametrize("fmt,block", [("e8m0", 32), ("e4m3", 16)])
def test_empty_k_gives_zero(fmt, block):
    """K = 0: C and Y are empty sums, all zero, whatever the output held; no
    operand is read."""
    pol = _policy(fmt)
    qa = fq.fp4_quantize(torch.zeros((33, 0), dtype=torch.float32, device="cuda"), block, fmt, amax=pol)
    qw = fq.fp4_quantize(torch.zeros((40, 0), dtype=torch.float32, device="cuda"), block, fmt, amax=pol)
    c = torch.full((33, 48), 7.0, dtype=torch.bfloat16, device="cuda")
    fq.fp4_gemm(qa, qw, out=c[:, :40])
    y = torch.full((3, 48), 7.0, dtype=torch.bfloat16, device="cuda")
    fq.fp4_wo_gemm(torch.zeros((3, 0), dtype=torch.bfloat16, device="cuda"), qw, out=y[:, :40])
    torch.cuda.synchronize()
    assert bool((c[:, :40] == 0).all()) and bool((c[:, 40:] == 7.0).all())
    assert bool((y[:, :40] == 0).all()) and bool((y[:, 40:] == 7.0).all())


@pytest.mark.parametrize("fmt,block", [("e8m0", 32), ("e4m3", 16), ("ue5m3", 16)])
@pytest.mark.parametrize("wname", ["up", "down", "sq"])
def test_llama_shapes_every_output(fmt, block, wname):
    """Llama-2 7B linears at M = 8192 (batch 4 x seq 2048): every output
    checked against the binary64 reference, in blocks of 1024 rows."""
    shapes = {"a": (8192, 4096), "up": (11008, 4096), "down": (4096, 11008), "sq": (4096, 4096)}
    k = shapes[wname][1]
    a_shape = (8192, k)
    xa = inputs.llama("a", {**shapes, "a": a_shape})
    xw = inputs.llama(wname, shapes)
    qa, a = _quant_both(xa, block, fmt)
    qw, w = _quant_both(xw, block, fmt)
    c = fq.fp4_gemm(qa, qw)
    torch.cuda.synchronize()
    check_gemm_every_output(c, a, w, f"llama {wname} {fmt}")


# ---------------------------------------------------------------------------
# weight-only GEMM
# ---------------------------------------------------------------------------
def _check_wo(y_gpu, x_bits, w_hat, tag=""):
    xf = inputs.bf16_bits_to_f32(x_bits).astype(np.float64)
    _check_gemm(y_gpu, xf, w_hat, tag=tag)


@pytest.mark.parametrize("m", [1, 3, 8, 16])
@pytest.mark.parametrize("n,k", [(100, 256), (16, 512), (33, 1024)])
def test_wo_gemm_small(m, n, k):
    qw, w = _quant_both(_normal(n, k, 11, 0.02, dtype="bf16"), 16, "e4m3")
    x = _normal(m, k, 12, dtype="bf16")
    y = fq.fp4_wo_gemm(to_device(x), qw)
    torch.cuda.synchronize()
    _check_wo(y, x, w, tag=f"wo {m}x{n}x{k}")


@pytest.mark.parametrize("fmt,block", [("e8m0", 32), ("ue5m3", 16), ("e7m0", 16), ("e1m6", 32)])
def test_wo_gemm_formats(fmt, block):
    qw, w = _quant_both(_normal(48, 512, 13, 0.02, dtype="bf16"), block, fmt)
    x = _normal(5, 512, 14, dtype="bf16")
    y = fq.fp4_wo_gemm(to_device(x), qw)
    torch.cuda.synchronize()
    _check_wo(y, x, w, tag=f"wo {fmt}/{block}")


@pytest.mark.parametrize("fmt,block", [("e4m3", 16), ("e4m3", 32), ("e8m0", 32), ("e8m0", 16), ("ue5m3", 16),
                                       ("e7m0", 16), ("e1m6", 32), ("e3m4", 16)])
@pytest.mark.parametrize("n,k", [(37, 256), (300, 2048), (8200, 4096), (129, 8448)])
def test_wo_gemm_single_row(fmt, block, n, k):
    """M = 1 (one X row, loaded in 4-byte pieces): scale formats decoded by
    table, E8M0 as a power of two, E1M6 split into two exact bf16 terms; K
    from one 128-element chunk per wave to many with a ragged last round
    (K = 8448), ragged row groups."""
    qw, w = _quant_both(_normal(n, k, 31, 0.02, dtype="bf16"), block, fmt)
    x = _normal(1, k, 32, dtype="bf16")
    y = fq.fp4_wo_gemm(to_device(x), qw)
    torch.cuda.synchronize()
    _check_wo(y, x, w, tag=f"wo m=1 {fmt}/{block} {n}x{k}")


@pytest.mark.parametrize("fmt,block", [("e4m3", 16), ("e8m0", 32), ("e1m6", 32)])
def test_wo_gemm_many_row_groups(fmt, block):
    """N = 8200: 513 groups of 16 rows (the launch that pairs row groups),
    the last pair ragged; M in each X-load class."""
    qw, w = _quant_both(_normal(8200, 256, 15, 0.02, dtype="bf16"), block, fmt)
    for m in (1, 2, 5, 12):
        x = _normal(m, 256, 16 + m, dtype="bf16")
        y = fq.fp4_wo_gemm(to_device(x), qw)
        torch.cuda.synchronize()
        _check_wo(y, x, w, tag=f"wo many {fmt}/{block} m={m}")


@pytest.mark.parametrize("wname", ["up", "down"])
def test_wo_gemm_qwen_decode_shapes(wname):
    """Qwen-2.5 decode shapes: W [18944, 3584] / [3584, 18944] NVFP4 E4M3
    block 16, X [M, K] for M in {1, 8, 16}; every output checked."""
    xw = inputs.decode_weight(wname)
    qw, w = _quant_both(xw, 16, "e4m3")
    k = w.shape[1]
    for m in (1, 8, 16):
        x = inputs.decode_x(m, k)
        y = fq.fp4_wo_gemm(to_device(x), qw)
        torch.cuda.synchronize()
        _check_wo(y, x, w, tag=f"qwen {wname} m={m}")
