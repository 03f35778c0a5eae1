"""GPU tests of the weight-only GEMM on the 8- and 6-bit element grids
(MXFP8 / MXINT8 / MXFP6 / MXINT6-style weights, bf16 activations) against
the oracle.

The weights are quantized on the GPU and by the oracle and first checked
byte-identical; the output passes iff it is the bf16 rounding of some value
within 1e-5 * sum_k |x_k||w_k| of the binary64 product of the exact
dequantized weights (quant_prune_distill/486 "Метод": the MX family's 8- and
6-bit members with E8M0 scales, and the same grids with the other scale
encodings).  A second test sends every element code through the kernel's
decode with a one-hot X, where the result is exact.  Every call goes through
the C ABI.
"""
import numpy as np
import pytest
import torch

import fp4_inputs as inputs
import oracle
from tests.gpu_util import assert_bytes_equal, host, to_device

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp4_block_scaled_quantize_amd")

WIDE = ["fp8_e4m3", "int8", "fp6_e2m3", "fp6_e3m2", "int6"]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _normal(rows, cols, seed, std=1.0):
    x = (np.random.default_rng(seed).standard_normal((rows, cols)) * std).astype(np.float32)
    return inputs.f32_to_bf16_bits(x)


def _quant_pair(x_np, block, fmt, elem):
    pol = "none" if fmt == "e8m0" else "current"
    qt = fq.fp4_quantize(to_device(x_np), block, fmt, amax=pol, element=elem)
    q, s, g, _ = oracle.quantize_tensor(x_np, block, fmt, pol, nthreads=8, elem=elem)
    torch.cuda.synchronize()
    assert_bytes_equal(host(qt.q), q, f"{elem} {fmt} weight codes")
    assert_bytes_equal(host(qt.scales), s, f"{elem} {fmt} weight scales")
    return qt, oracle.dequantize_f64(q, s, g, block, fmt, elem=elem)


def _check_wo(y_gpu, x_bits, w_hat, tag):
    xf = inputs.bf16_bits_to_f32(x_bits).astype(np.float64)
    cref, tol = oracle.gemm_ref(xf, w_hat)
    c = y_gpu.float().cpu().numpy().astype(np.float64)
    ok = oracle.gemm_check(c, cref, tol)
    if not ok.all():
        i, j = np.argwhere(~ok)[0]
        raise AssertionError(f"{tag}: {int((~ok).sum())} of {ok.size} outputs out of tolerance; first ({i},{j}) "
                             f"got {c[i, j]!r} ref {cref[i, j]!r} tol {tol[i, j]!r}")


# M in each X-load class; N from one ragged 16-row group to 513 groups (the
# launch that pairs row groups, the last pair ragged); K from one 128-element
# chunk per wave to many with a ragged last round (K = 8448)
SHAPES = [(1, 37, 256), (3, 300, 2048), (8, 129, 1024), (16, 64, 8448), (1, 8200, 512), (12, 8200, 256)]


@pytest.mark.parametrize("elem", WIDE)
@pytest.mark.parametrize("fmt,block", [("e8m0", 32), ("e8m0", 16), ("e4m3", 16), ("ue5m3", 32), ("e3m4", 16),
                                       ("e1m6", 32)])
def test_wo_wide_grids(elem, fmt, block):
    """Scales exact with the grid's elements in bf16 (E8M0 always; E4M3 /
    UE5M3 for FP8 and FP6 E2M3) and the products that take the two-term
    split (INT8 with any non-power-of-two scale, E3M4 / E1M6 scales)."""
    for i, (m, n, k) in enumerate(SHAPES):
        qw, w = _quant_pair(_normal(n, k, 40 + i, 0.02), block, fmt, elem)
        x = _normal(m, k, 60 + i)
        y = fq.fp4_wo_gemm(to_device(x), qw)
        torch.cuda.synchronize()
        _check_wo(y, x, w, f"wo {elem} {fmt}/{block} {m}x{n}x{k}")


@pytest.mark.parametrize("elem,fmt,block", [("fp8_e4m3", "e8m0", 32), ("int6", "e4m3", 16)])
def test_wo_wide_qwen_up(elem, fmt, block):
    """The Qwen-2.5 7B up projection W [18944, 3584] on a wide grid, M = 1
    and 16; every output checked."""
    qw, w = _quant_pair(inputs.decode_weight("up"), block, fmt, elem)
    k = w.shape[1]
    for m in (1, 16):
        x = inputs.decode_x(m, k)
        y = fq.fp4_wo_gemm(to_device(x), qw)
        torch.cuda.synchronize()
        _check_wo(y, x, w, f"qwen up {elem} {fmt}/{block} m={m}")


def _pack6(codes):
    """Six-bit codes [rows, cols] to the little-endian row stream."""
    out = np.zeros((codes.shape[0], codes.shape[1] * 3 // 4), dtype=np.uint8)
    for r in range(codes.shape[0]):
        big = 0
        for j, v in enumerate(codes[r]):
            big |= int(v) << (6 * j)
        out[r] = np.frombuffer(big.to_bytes(out.shape[1], "little"), dtype=np.uint8)
    return out


@pytest.mark.parametrize("elem", WIDE)
@pytest.mark.parametrize("fmt", ["e8m0", "e4m3", "e1m6"])
def test_wo_wide_every_code(elem, fmt):
    """W[n, k] = code (n + k) mod C (C the number of codes: 256 bytes with
    the two FP8 NaN codes replaced, or 64 six-bit codes) with mixed block
    scales; X holds 16 one-hot rows (x[m, 16 m + 3] = 1), so Y[m, n] is the
    bf16 rounding of one exact weight value: every code of every row's
    selected column goes through the decode (the two-term split for E1M6)."""
    n = k = 256
    ncodes = 64 if elem.startswith(("fp6", "int6")) else 256
    codes = (np.arange(n)[:, None] + np.arange(k)[None, :]) % ncodes
    if elem == "fp8_e4m3":
        codes[(codes & 0x7F) == 0x7F] = 0
    q_w = _pack6(codes) if ncodes == 64 else codes.astype(np.uint8)
    block = 32 if fmt == "e8m0" else 16
    rng = np.random.default_rng(29)
    if fmt == "e8m0":
        s_w = rng.integers(110, 145, (n, k // block), dtype=np.uint8)
        g, pol = 1.0, "none"
    else:
        s_w = rng.integers(0, 0x7F, (n, k // block), dtype=np.uint8)
        g, pol = 0.0625, "current"          # a power of two: g * acc stays exact
    qw = fq.QTensor(torch.from_numpy(q_w).cuda(), torch.from_numpy(s_w).cuda(),
                    torch.tensor([g, 0.0], dtype=torch.float32).cuda(), n, k, block, fmt, amax=pol, element=elem)
    x = np.zeros((16, k), dtype=np.float32)
    x[np.arange(16), 16 * np.arange(16) + 3] = 1.0
    y = fq.fp4_wo_gemm(to_device(inputs.f32_to_bf16_bits(x)), qw)
    torch.cuda.synchronize()
    w_hat = oracle.dequantize_f64(q_w, s_w, np.float32(g), block, fmt, elem=elem)
    want = oracle.round_to_bf16(w_hat[:, 16 * np.arange(16) + 3].T)
    got = y.float().cpu().numpy().astype(np.float64)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (f"{elem} {fmt}: {len(bad)} outputs differ; first {tuple(bad[0])}: got "
                           f"{got[tuple(bad[0])]!r} want {want[tuple(bad[0])]!r}")
