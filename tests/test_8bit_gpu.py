"""GPU parity of the 8-bit MX element grids (MXFP8-style FP8 E4M3 elements,
MXINT8-style symmetric INT8; one byte per element) against the CPU oracle:
codes, scales and tensor scale bit for bit for every scale encoding, both
rounding modes, the single-pass and two-pass refreshes and the Hadamard
transform; dequantization bit for bit; the paths that do not take 8-bit
grids reject them.  Every call goes through the C ABI.
"""
import numpy as np
import pytest
import torch

import fp4_inputs as inputs
import oracle
from tests.gpu_util import assert_bytes_equal, bf16_bits, f32_bits, host, to_device

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp4_block_scaled_quantize_amd")

ELEMS = ["fp8_e4m3", "int8"]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _policy(fmt, default="current"):
    return "none" if fmt == "e8m0" else default


def _like(rows, cols, seed, dtype="bf16"):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)) * 0.02
    m = rng.random((rows, cols)) < 0.001
    x[m] *= 100
    x = x.astype(np.float32)
    return inputs.f32_to_bf16_bits(x) if dtype == "bf16" else x


def _check(x_np, block, fmt, policy, elem, *, rounding="nearest", seed=0, offset=0, rht=None, rows=None, tag=""):
    st = fq.AmaxState(1) if policy == "current" else None
    qt = fq.fp4_quantize(to_device(x_np), block, fmt, rounding=rounding, amax=policy, state=st, seed=seed,
                         offset=offset, rht_signs=rht, element=elem)
    torch.cuda.synchronize()
    sr = rounding == "stochastic"
    if rows is None:
        q, s, g, a = oracle.quantize_tensor(x_np, block, fmt, policy, stochastic=sr, seed=seed, offset=offset,
                                            nthreads=8, rht_signs=rht, elem=elem)
        assert_bytes_equal(host(qt.scales), s, f"{tag} scales")
        assert_bytes_equal(host(qt.q), q, f"{tag} codes")
    else:
        g, a = oracle.resolve_tensor_scale(x_np, fmt, policy, elem=elem)
        for r in rows:
            q, s = oracle.quantize(x_np, block, fmt, g, stochastic=sr, seed=seed, offset=offset, rows=(r, r + 1),
                                   elem=elem)
            assert_bytes_equal(host(qt.q[r:r + 1]), q, f"{tag} row {r} codes")
            assert_bytes_equal(host(qt.scales[r:r + 1]), s, f"{tag} row {r} scales")
    assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([g, a]), f"{tag} tensor_scale")
    return qt


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("fmt,block", [("e8m0", 32), ("e8m0", 16), ("e4m3", 16), ("ue5m3", 32), ("e1m6", 16)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rounding", ["nearest", "stochastic"])
def test_8bit_quantize_parity(elem, fmt, block, dtype, rounding):
    x = _like(67, 320, 700 + block, dtype)
    _check(x, block, fmt, _policy(fmt), elem, rounding=rounding, seed=0x5EED, offset=5,
           tag=f"{elem} {fmt}/{block}/{dtype}/{rounding}")


@pytest.mark.parametrize("elem", ELEMS)
def test_8bit_full_size_two_pass_and_transform(elem):
    x = inputs.sweep()
    _check(x, 32, "e8m0", "none", elem, tag=f"{elem} sweep mx")
    _check(x, 16, "e4m3", "current", elem, tag=f"{elem} sweep nv")
    big = _like(4104, 4096, 71)
    _check(big, 16, "e4m3", "current", elem, rows=[0, 7, 2052, 4103], tag=f"{elem} two-pass")
    small = _like(40, 512, 72)
    _check(small, 32, "e8m0", "none", elem, rht=0x9E3779B9, tag=f"{elem} rht")
    _check(small, 16, "e4m3", "current", elem, rht=0x12345678, rounding="stochastic", seed=3, offset=1,
           tag=f"{elem} rht sr")


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("fmt,block", [("e8m0", 32), ("e4m3", 16)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_8bit_dequantize_parity(elem, fmt, block, out):
    rng = np.random.default_rng(19)
    rows, cols = 19, 256
    q = rng.integers(0, 256, (rows, cols), dtype=np.uint8)
    if elem == "fp8_e4m3":
        q[(q & 0x7F) == 0x7F] = 0x33                        # no NaN element codes
    lo, hi = (100, 140) if fmt == "e8m0" else (0, 0x7E)
    s = rng.integers(lo, hi, (rows, cols // block), dtype=np.uint8)
    g = np.float32(0.0213) if fmt != "e8m0" else np.float32(1.0)
    qt = fq.QTensor(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(),
                    torch.tensor([g, 0.0], dtype=torch.float32).cuda(), rows, cols, block, fmt,
                    amax="none" if fmt == "e8m0" else "current", element=elem)
    y = fq.fp4_dequantize(qt, torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    want = oracle.dequantize(q, s, float(g), block, fmt, out=out, elem=elem)
    if out == "f32":
        assert_bytes_equal(f32_bits(host(y)), f32_bits(want), f"{elem} dequant f32")
    else:
        assert_bytes_equal(bf16_bits(y), want, f"{elem} dequant bf16")


def test_8bit_quantize_dequantize_roundtrip_bound():
    """MXFP8 reconstruction error bound, a property that holds at any size:
    half an E4M3 step (relative 2^-4), half the subnormal step 2^-9 s at the
    bottom, and the saturation of x / s in [448, 512) to 448 at the top."""
    x = inputs.bf16_bits_to_f32(_like(256, 1024, 73))
    qt = fq.fp4_quantize(torch.from_numpy(x).cuda(), 32, "e8m0", amax="none", element="fp8_e4m3")
    y = host(fq.fp4_dequantize(qt, torch.float32))
    s = 2.0 ** (host(qt.scales).astype(np.float64) - 127)
    sb = np.repeat(s, 32, axis=1)
    err = np.abs(y.astype(np.float64) - x)
    bound = np.maximum(np.maximum(np.abs(x) * 2.0 ** -4, sb * 2.0 ** -9), np.abs(x) - 448.0 * sb)
    assert np.all(err <= bound + 1e-30)


def test_8bit_rejected_elsewhere():
    xd = to_device(_like(64, 256, 74, "f32"))
    q8 = fq.fp4_quantize(xd, 32, "e8m0", amax="none", element="int8")
    for call in (lambda: fq.fp4_gemm(q8, q8),
                 lambda: fq.fp4_wo_gemm(torch.zeros((1, 256), dtype=torch.bfloat16, device="cuda"), q8),
                 lambda: fq.fp4_quantize_transposed(xd, 32, "e8m0", amax="none", element="int8"),
                 lambda: fq.fp4_quantize_both(xd, 32, "e8m0", amax="none", element="int8")):
        with pytest.raises(fq.Fp4Error) as e:
            call()
        assert e.value.status == -2
