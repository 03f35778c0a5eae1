"""GPU parity of the INT4 element grid (NVINT4: block 16 with E4M3 scales,
MXINT4: block 32 with E8M0 scales, and the other scale encodings) against the
CPU oracle: codes, scales and tensor scale bit for bit (row-wise,
column-wise, with and without the Hadamard transform), dequantization bit
for bit, and the GEMM within 1e-5 * sum|a||b| of the exact product of the
oracle's dequantized operands.  Every call goes through the C ABI.
"""
import numpy as np
import pytest
import torch

import fp4_inputs as inputs
import oracle
from tests.gpu_util import assert_bytes_equal, bf16_bits, f32_bits, host, to_device

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp4_block_scaled_quantize_amd")


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


def _check(x_np, block, fmt, policy, *, rounding="nearest", seed=0, offset=0, rht=None, tag="", rows=None):
    st = fq.AmaxState(1) if policy == "current" else None
    qt = fq.fp4_quantize(to_device(x_np), block, fmt, rounding=rounding, amax=policy, state=st, seed=seed,
                         offset=offset, rht_signs=rht, element="int4")
    torch.cuda.synchronize()
    sr = rounding == "stochastic"
    if rows is None:
        q, s, g, a = oracle.quantize_tensor(x_np, block, fmt, policy, stochastic=sr, seed=seed, offset=offset,
                                            nthreads=8, rht_signs=rht, elem="int4")
        assert_bytes_equal(host(qt.scales), s, f"{tag} scales")
        assert_bytes_equal(host(qt.q), q, f"{tag} codes")
    else:
        g, a = oracle.resolve_tensor_scale(x_np, fmt, policy, elem="int4")
        for r in rows:
            q, s = oracle.quantize(x_np, block, fmt, g, stochastic=sr, seed=seed, offset=offset, rows=(r, r + 1),
                                   elem="int4")
            assert_bytes_equal(host(qt.q[r:r + 1]), q, f"{tag} row {r} codes")
            assert_bytes_equal(host(qt.scales[r:r + 1]), s, f"{tag} row {r} scales")
    assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([g, a]), f"{tag} tensor_scale")
    return qt


@pytest.mark.parametrize("fmt", ["e4m3", "ue5m3", "e3m4", "e1m6", "e8m0"])
@pytest.mark.parametrize("block", [16, 32])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rounding", ["nearest", "stochastic"])
def test_int4_quantize_parity(fmt, block, dtype, rounding):
    x = _like(67, 320, 400 + block, dtype)
    _check(x, block, fmt, _policy(fmt), rounding=rounding, seed=0x5EED, offset=9, tag=f"int4 {fmt}/{block}/{dtype}")
    if fmt != "e8m0":
        _check(x, block, fmt, "none", rounding=rounding, seed=1, offset=2, tag=f"int4 {fmt}/{block}/{dtype}/none")


def test_int4_with_hadamard_transform():
    x = _like(40, 512, 41)
    for fmt, block in (("e4m3", 16), ("e8m0", 32)):
        _check(x, block, fmt, _policy(fmt), rht=0x9E3779B9, tag=f"int4 rht {fmt}")
        _check(x, block, fmt, _policy(fmt), rht=0x12345678, rounding="stochastic", seed=3, offset=4,
               tag=f"int4 rht sr {fmt}")


def test_int4_sweep_full_size_and_two_pass():
    x = inputs.sweep()
    _check(x, 16, "e4m3", "current", tag="NVINT4 sweep")
    _check(x, 32, "e8m0", "none", tag="MXINT4 sweep")
    big = _like(4104, 4096, 43)
    _check(big, 16, "e4m3", "current", tag="NVINT4 two-pass", rows=[0, 5, 2050, 4103])


@pytest.mark.parametrize("fmt,block", [("e4m3", 16), ("e8m0", 32), ("ue5m3", 16)])
@pytest.mark.parametrize("rounding", ["nearest", "stochastic"])
def test_int4_transposed_parity(fmt, block, rounding):
    x = _like(352, 136, 44)
    pol = _policy(fmt)
    st = fq.AmaxState(1) if pol == "current" else None
    qt = fq.fp4_quantize_transposed(to_device(x), block, fmt, rounding=rounding, amax=pol, state=st, seed=7,
                                    offset=1, element="int4")
    torch.cuda.synchronize()
    xt = np.ascontiguousarray(x.T)
    q, s, g, a = oracle.quantize_tensor(xt, block, fmt, pol, stochastic=(rounding == "stochastic"), seed=7, offset=1,
                                        elem="int4")
    assert_bytes_equal(host(qt.scales), s, "int4 T scales")
    assert_bytes_equal(host(qt.q), q, "int4 T codes")
    assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([g, a]), "int4 T tensor_scale")


@pytest.mark.parametrize("fmt,block", [("e4m3", 16), ("e8m0", 32), ("e1m6", 16)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("rht", [None, 0x5A5A0F0F])
def test_int4_dequantize_parity(fmt, block, out, rht):
    rng = np.random.default_rng(17)
    rows, cols = 19, 256
    q = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    lo, hi = (110, 140) if fmt == "e8m0" else (0, 0x7E)
    s = rng.integers(lo, hi, (rows, cols // block), dtype=np.uint8)
    g = np.float32(0.0213) if fmt != "e8m0" else np.float32(1.0)
    qt = fq.QTensor(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(),
                    torch.tensor([g, 0.0], dtype=torch.float32).cuda(), rows, cols, block, fmt,
                    amax="none" if fmt == "e8m0" else "current", transform="none" if rht is None else "rht",
                    rht_signs=rht or 0, element="int4")
    y = fq.fp4_dequantize(qt, torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    if rht is None:
        want = oracle.dequantize(q, s, float(g), block, fmt, out=out, elem="int4")
    else:
        x = oracle.rht_inverse(oracle.dequantize(q, s, float(g), block, fmt, elem="int4"), block, rht)
        want = oracle.f32_to_bf16_bits_array(x) if out == "bf16" else x
    got = host(y) if out == "f32" else bf16_bits(y)
    if out == "f32":
        assert_bytes_equal(f32_bits(got), f32_bits(want), f"int4 dequant {fmt}")
    else:
        assert_bytes_equal(got, want, f"int4 dequant {fmt} bf16")


@pytest.mark.parametrize("fmt,block,m,n,k", [("e4m3", 16, 200, 330, 1024), ("e8m0", 32, 130, 260, 768),
                                             ("e1m6", 16, 64, 96, 512), ("ue5m3", 32, 96, 200, 512)])
def test_int4_gemm(fmt, block, m, n, k):
    a = _like(m, k, 51, "f32")
    w = _like(n, k, 52, "f32")
    pol = _policy(fmt)
    qa = fq.fp4_quantize(to_device(a), block, fmt, amax=pol, element="int4")
    qw = fq.fp4_quantize(to_device(w), block, fmt, amax=pol, element="int4")
    c = fq.fp4_gemm(qa, qw)
    torch.cuda.synchronize()
    oa = oracle.quantize_tensor(a, block, fmt, pol, elem="int4")
    ow = oracle.quantize_tensor(w, block, fmt, pol, elem="int4")
    assert_bytes_equal(host(qa.q), oa[0], "A codes")
    assert_bytes_equal(host(qw.q), ow[0], "W codes")
    a_hat = oracle.dequantize_f64(oa[0], oa[1], oa[2], block, fmt, elem="int4")
    w_hat = oracle.dequantize_f64(ow[0], ow[1], ow[2], block, fmt, elem="int4")
    cref, tol = oracle.gemm_ref(a_hat, w_hat)
    ok = oracle.gemm_check(c.float().cpu().numpy().astype(np.float64), cref, tol)
    assert ok.all(), f"int4 gemm {fmt}: {int((~ok).sum())} of {ok.size} outputs out of tolerance"


def test_int4_mixed_grids_rejected():
    x = to_device(_like(64, 256, 53, "f32"))
    q4 = fq.fp4_quantize(x, 16, "e4m3", element="int4")
    qf = fq.fp4_quantize(x, 16, "e4m3")
    with pytest.raises(fq.Fp4Error) as e:
        fq.fp4_gemm(q4, qf)
    assert e.value.status == -2


@pytest.mark.parametrize("fmt,block", [("e4m3", 16), ("e8m0", 32), ("e1m6", 16), ("e2m5", 32), ("ue5m3", 16)])
@pytest.mark.parametrize("n", [48, 8200])
def test_int4_weight_only_gemm(fmt, block, n):
    """Weight-only GEMM with INT4 weights: bf16 dequant in registers (split
    into two exact bf16 terms where int * s needs more than 8 bits), every M
    class, few and many row groups."""
    k = 512
    w = _like(n, k, 54, "bf16")
    pol = _policy(fmt)
    qw = fq.fp4_quantize(to_device(w), block, fmt, amax=pol, element="int4")
    ow = oracle.quantize_tensor(w, block, fmt, pol, elem="int4")
    torch.cuda.synchronize()
    assert_bytes_equal(host(qw.q), ow[0], "W codes")
    w_hat = oracle.dequantize_f64(ow[0], ow[1], ow[2], block, fmt, elem="int4")
    for m in (1, 3, 8, 16):
        xb = inputs.f32_to_bf16_bits((np.random.default_rng(55 + m).standard_normal((m, k))).astype(np.float32))
        y = fq.fp4_wo_gemm(to_device(xb), qw)
        torch.cuda.synchronize()
        cref, tol = oracle.gemm_ref(inputs.bf16_bits_to_f32(xb).astype(np.float64), w_hat)
        ok = oracle.gemm_check(y.float().cpu().numpy().astype(np.float64), cref, tol)
        assert ok.all(), f"int4 wo {fmt} n={n} m={m}: {int((~ok).sum())} outputs out of tolerance"
