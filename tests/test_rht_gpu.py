"""GPU parity of quantization with the blockwise randomized Hadamard
transform (applied before quantization) against the CPU oracle.

Codes, scales and the tensor scale must match the oracle bit for bit (the
transform is binary32 in the same butterfly order on both sides); the
dequantization with the inverse transform too; the GEMM of two operands
transformed with the same signs must pass the 1e-5 * sum|a||b| bracket
against the exact product of the oracle's dequantized (transformed) operands.
Every call goes through the C ABI.
"""
import numpy as np
import pytest
import torch

import fp4_inputs as inputs
import oracle
from tests.gpu_util import assert_bytes_equal, bf16_bits, f32_bits, host, to_device

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp4_block_scaled_quantize_amd")

SIGNS = [0x0, 0xFFFFFFFF, 0x9E3779B9, 0x5A5A0F0F]


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


def _check_rht(x_np, block, fmt, policy, signs, *, rounding="nearest", seed=0, offset=0, state=None, ostate=None,
               tag="", rows=None):
    xd = to_device(x_np)
    if state is None and policy == "current":
        state = fq.AmaxState(1)
    qt = fq.fp4_quantize(xd, block, fmt, rounding=rounding, amax=policy, state=state, seed=seed, offset=offset,
                         rht_signs=signs)
    torch.cuda.synchronize()
    if rows is None:
        q, s, g, a = oracle.quantize_tensor(x_np, block, fmt, policy, state=ostate,
                                            stochastic=(rounding == "stochastic"), seed=seed, offset=offset,
                                            nthreads=8, rht_signs=signs)
        assert_bytes_equal(host(qt.scales), s, f"{tag} scales")
        assert_bytes_equal(host(qt.q), q, f"{tag} codes")
    else:
        y = oracle.rht_forward(x_np, block, signs)
        g, a = oracle.resolve_tensor_scale(y, fmt, policy, ostate)
        for r in rows:
            q, s = oracle.quantize(y, block, fmt, g, stochastic=(rounding == "stochastic"), seed=seed,
                                   offset=offset, rows=(r, r + 1))
            assert_bytes_equal(host(qt.q[r:r + 1]), q, f"{tag} row {r} codes")
            assert_bytes_equal(host(qt.scales[r:r + 1]), s, f"{tag} row {r} scales")
    assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([g, a]), f"{tag} tensor_scale")
    return qt


@pytest.mark.parametrize("fmt", ["e4m3", "ue5m3", "e1m6", "e8m0"])
@pytest.mark.parametrize("block", [16, 32])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rounding", ["nearest", "stochastic"])
def test_rht_quantize_parity(fmt, block, dtype, rounding):
    x = _like(67, 320, 300 + block, dtype)
    for signs in SIGNS[:2] if rounding == "stochastic" else SIGNS:
        _check_rht(x, block, fmt, _policy(fmt), signs, rounding=rounding, seed=0x5EED, offset=3,
                   tag=f"rht {fmt}/{block}/{dtype}/{rounding}/{signs:#x}")
    if fmt != "e8m0":
        _check_rht(x, block, fmt, "none", SIGNS[2], tag=f"rht {fmt}/{block}/{dtype} none")


@pytest.mark.parametrize("block", [16, 32])
def test_rht_two_pass_refresh_sampled_rows(block):
    """4104 x 4096 bf16 does not fit the single-pass grid: the amax kernel
    takes the maximum of the transformed tensor, then the quantize pass."""
    x = _like(4104, 4096, 71)
    x[4103, 4095] = inputs.f32_to_bf16_bits(np.array([-9216.0], dtype=np.float32))[0]
    rows = [0, 1, 17, 2048, 4095, 4096, 4103]
    _check_rht(x, block, "e4m3", "current", SIGNS[2], tag=f"rht 2-pass B{block}", rows=rows)


def test_rht_sweep_full_size():
    """The 4096x4096 bf16 sweep tensor (single-pass current amax), every byte."""
    x = inputs.sweep()
    _check_rht(x, 16, "e4m3", "current", SIGNS[2], tag="rht sweep e4m3")
    _check_rht(x, 32, "e8m0", "none", SIGNS[3], tag="rht sweep e8m0")


def test_rht_delayed_sequence():
    st = fq.AmaxState(4)
    ost = oracle.AmaxState(interval=4)
    for t in range(9):
        x = _like(32, 256, 900 + t)
        if t == 2:
            x = inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(x) * np.float32(8.0))
        _check_rht(x, 16, "e4m3", "delayed", SIGNS[2], rounding="stochastic", seed=11, offset=t, state=st,
                   ostate=ost, tag=f"rht delayed {t}")


@pytest.mark.parametrize("fmt,block", [("e4m3", 16), ("ue5m3", 32), ("e8m0", 32), ("e8m0", 16)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_rht_dequantize_parity(fmt, block, out):
    rng = np.random.default_rng(13)
    rows, cols = 21, 512
    q = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    lo, hi = (120, 135) if fmt == "e8m0" else (0, 0x7E)
    s = rng.integers(lo, hi, (rows, cols // block), dtype=np.uint8)
    g = np.float32(0.0173) if fmt != "e8m0" else np.float32(1.0)
    signs = SIGNS[2]
    qt = fq.QTensor(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(),
                    torch.tensor([g, 0.0], dtype=torch.float32).cuda(), rows, cols, block, fmt,
                    amax="none" if fmt == "e8m0" else "current", transform="rht", rht_signs=signs)
    y = fq.fp4_dequantize(qt, torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    want = oracle.dequantize_rht(q, s, float(g), block, fmt, signs, out=out)
    got = host(y) if out == "f32" else bf16_bits(y)
    assert_bytes_equal(f32_bits(got) if out == "f32" else got, f32_bits(want) if out == "f32" else want,
                       f"rht dequant {fmt}/{block}/{out}")


def test_rht_roundtrip_through_binding():
    x = _like(64, 512, 5, "f32")
    qt = fq.fp4_quantize(to_device(x), 16, "e4m3", rht_signs=SIGNS[3])
    y = fq.fp4_dequantize(qt, torch.float32)
    torch.cuda.synchronize()
    q, s, g, _ = oracle.quantize_tensor(x, 16, "e4m3", "current", rht_signs=SIGNS[3])
    assert_bytes_equal(f32_bits(host(y)), f32_bits(oracle.dequantize_rht(q, s, g, 16, "e4m3", SIGNS[3])),
                       "rht roundtrip")


def _gemm_check(c_gpu, a_hat, w_hat, tag):
    cref, tol = oracle.gemm_ref(a_hat, w_hat)
    c = c_gpu.float().cpu().numpy().astype(np.float64)
    ok = oracle.gemm_check(c, cref, tol)
    assert ok.all(), f"{tag}: {int((~ok).sum())} of {ok.size} outputs out of tolerance"


@pytest.mark.parametrize("fmt,block", [("e8m0", 32), ("e4m3", 16)])
def test_rht_gemm_same_signs(fmt, block):
    """Both operands transformed with the same signs along K: within the
    bracket of the exact product of the oracle's dequantized operands, and
    close to the product of the untransformed inputs."""
    m, n, k = 192, 320, 1024
    a = _like(m, k, 61, "f32")
    w = _like(n, k, 62, "f32")
    signs = SIGNS[2]
    pol = _policy(fmt)
    qa = fq.fp4_quantize(to_device(a), block, fmt, amax=pol, rht_signs=signs)
    qw = fq.fp4_quantize(to_device(w), block, fmt, amax=pol, rht_signs=signs)
    c = fq.fp4_gemm(qa, qw)
    torch.cuda.synchronize()
    oa = oracle.quantize_tensor(a, block, fmt, pol, rht_signs=signs)
    ow = oracle.quantize_tensor(w, block, fmt, pol, rht_signs=signs)
    assert_bytes_equal(host(qa.q), oa[0], "A codes")
    assert_bytes_equal(host(qw.q), ow[0], "W codes")
    a_hat = oracle.dequantize_f64(oa[0], oa[1], oa[2], block, fmt)
    w_hat = oracle.dequantize_f64(ow[0], ow[1], ow[2], block, fmt)
    _gemm_check(c, a_hat, w_hat, f"rht gemm {fmt}")
    # the transform is orthogonal along K: the product approximates A W^T
    exact = a.astype(np.float64) @ w.astype(np.float64).T
    err = np.abs(c.float().cpu().numpy() - exact)
    assert np.median(err) < 0.2 * np.median(np.abs(exact)) + 1e-6
    # operands transformed differently are rejected
    qw2 = fq.fp4_quantize(to_device(w), block, fmt, amax=pol, rht_signs=signs ^ 1)
    with pytest.raises(fq.Fp4Error) as e:
        fq.fp4_gemm(qa, qw2)
    assert e.value.status == -2


@pytest.mark.parametrize("fmt,block", [("e4m3", 16), ("e8m0", 32), ("ue5m3", 32)])
@pytest.mark.parametrize("rounding", ["nearest", "stochastic"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rht_transposed_parity(fmt, block, rounding, dtype):
    """Column-wise quantization with the transform down the columns of x;
    a current-amax refresh takes the maximum of the transformed tensor
    (tiled amax kernel, ragged tiles in both directions)."""
    x = _like(352, 136, 77, dtype)
    pol = _policy(fmt)
    st = fq.AmaxState(1) if pol == "current" else None
    signs = SIGNS[2]
    qt = fq.fp4_quantize_transposed(to_device(x), block, fmt, rounding=rounding, amax=pol, state=st, seed=5,
                                    offset=6, rht_signs=signs)
    torch.cuda.synchronize()
    q, s, g, a = oracle.quantize_transposed_tensor(x, block, fmt, pol, stochastic=(rounding == "stochastic"),
                                                   seed=5, offset=6, rht_signs=signs, nthreads=8)
    assert_bytes_equal(host(qt.scales), s, "rht T scales")
    assert_bytes_equal(host(qt.q), q, "rht T codes")
    assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([g, a]), "rht T tensor_scale")
    # dequantizing the transposed operand inverts the transform along its rows
    y = fq.fp4_dequantize(qt, torch.float32)
    torch.cuda.synchronize()
    assert_bytes_equal(f32_bits(host(y)), f32_bits(oracle.dequantize_rht(q, s, g, block, fmt, signs)), "rht T dequant")


def test_rht_transposed_grads_sampled():
    """8192x8192 gradients, column-wise, transform + SR + delayed amax (a
    refresh on the first call): tensor scale over the whole transformed
    tensor, sampled output rows."""
    x = inputs.grads(1)
    signs = SIGNS[3]
    st = fq.AmaxState(50)
    qt = fq.fp4_quantize_transposed(to_device(x), 16, "e4m3", rounding="stochastic", amax="delayed", state=st,
                                    seed=0x5EED, offset=1, rht_signs=signs)
    torch.cuda.synchronize()
    xt = np.ascontiguousarray(x.T)
    y = oracle.rht_forward(xt, 16, signs)
    a = oracle.amax(y)
    g = oracle.tensor_scale(a, "e4m3")
    assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([g, a]), "rht T grads tensor_scale")
    for c in (0, 63, 64, 4097, 8191):
        q, s = oracle.quantize(y, 16, "e4m3", g, stochastic=True, seed=0x5EED, offset=1, rows=(c, c + 1))
        assert_bytes_equal(host(qt.q[c:c + 1]), q, f"rht T grads col {c} codes")
        assert_bytes_equal(host(qt.scales[c:c + 1]), s, f"rht T grads col {c} scales")
