"""GPU parity of the 8-bit MX element grids (MXFP8-style FP8 E4M3 elements,
MXINT8-style symmetric INT8; one byte per element) against the CPU oracle:
codes, scales and tensor scale bit for bit for every scale encoding, both
rounding modes, the single-pass and two-pass refreshes and the Hadamard
transform; column-wise quantization bit for bit; dequantization bit for
bit; the GEMM within the binary64
reference's tolerance on every scale pairing it takes; a GEMM of operands on
different grids is rejected.  Every call goes through the C ABI.
"""
import numpy as np
import pytest
import torch

import fp4_inputs as inputs
import oracle
from tests.gpu_util import assert_bytes_equal, bf16_bits, check_gemm_every_output, f32_bits, host, to_device

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp4_block_scaled_quantize_amd")

ELEMS = ["fp8_e4m3", "int8"]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(autouse=True)
def _tiled_kernels():
    """These GEMM tests cover the tiled kernels, small shapes included (the
    small-product path runs the every-code and subnormal cases below in its
    own tests)."""
    prev = fq.set_gemm_small_outputs(0)
    try:
        yield
    finally:
        fq.set_gemm_small_outputs(prev)


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


def _e4m3_values():
    """The 127 non-negative finite E4M3 values (codes 0x00..0x7E), from the
    format's definition: bias 7, 3 mantissa bits, subnormals below 2^-6."""
    out = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        out.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(out)


def test_fp8_rtn_every_midpoint():
    """Nearest-even FP8 encoding at every decision point: each E4M3 value,
    each midpoint between neighbours (ties to even) and the binary32 values
    on either side of it, the saturation range (448, 512) and both signs.
    Every block holds 256, so its E8M0 scale is exactly 1 and the encoder
    sees the values unchanged."""
    q = _e4m3_values()
    mid = (q[:-1] + q[1:]) / 2
    f32 = lambda a: np.asarray(a, dtype=np.float32)
    vals = np.concatenate([f32(q), f32(mid), np.nextafter(f32(mid), f32(np.inf)),
                           np.nextafter(f32(mid), f32(-np.inf)),
                           f32([448.5, 449, 463.99, 464, 464.01, 479, 480, 500, 511.99])])
    vals = np.concatenate([vals, -vals])
    per = 31
    nblk = -(-vals.size // per)
    vals = np.concatenate([vals, np.zeros(nblk * per - vals.size, dtype=np.float32)])
    blocks = np.concatenate([np.full((nblk, 1), 256.0, dtype=np.float32), vals.reshape(nblk, per)], axis=1)
    cols = 512
    nblk_pad = -(-nblk // (cols // 32)) * (cols // 32)
    blocks = np.concatenate([blocks, np.tile(blocks[:1], (nblk_pad - nblk, 1))])
    x = np.ascontiguousarray(blocks.reshape(-1, cols))
    qt = _check(x, 32, "e8m0", "none", "fp8_e4m3", tag="fp8 midpoints")
    assert np.all(host(qt.scales) == 127)


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


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("fmt,block,pol", [("e8m0", 32, "none"), ("e8m0", 16, "none"), ("e4m3", 16, "current"),
                                           ("ue5m3", 32, "current")])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rounding", ["nearest", "stochastic"])
def test_8bit_transposed_parity(elem, fmt, block, pol, dtype, rounding):
    """Column-wise quantization on the 8-bit grids: 320 rows (a partial
    256-row tile) by 200 columns (a partial 64-column tile), against the
    oracle's quantization of the transpose."""
    x = _like(320, 200, 720 + block, dtype)
    st = fq.AmaxState(1) if pol == "current" else None
    qt = fq.fp4_quantize_transposed(to_device(x), block, fmt, rounding=rounding, amax=pol, state=st, seed=0x5EED,
                                    offset=5, element=elem)
    torch.cuda.synchronize()
    q, s, g, a = oracle.quantize_transposed_tensor(x, block, fmt, pol, stochastic=rounding == "stochastic",
                                                   seed=0x5EED, offset=5, nthreads=8, elem=elem)
    tag = f"{elem} {fmt}/{block}/{dtype}/{rounding} transposed"
    assert_bytes_equal(host(qt.scales), s, f"{tag} scales")
    assert_bytes_equal(host(qt.q), q, f"{tag} codes")
    assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([g, a]), f"{tag} tensor_scale")


@pytest.mark.parametrize("elem", ELEMS)
def test_8bit_transposed_transform_and_larger(elem):
    """The column-wise Hadamard transform (its own amax kernel) and a
    2048 x 1000 tensor (8 x 16 tiles, ragged in columns)."""
    x = _like(512, 136, 730)
    st = fq.AmaxState(1)
    qt = fq.fp4_quantize_transposed(to_device(x), 16, "e4m3", amax="current", state=st, rht_signs=0x13579BDF,
                                    element=elem)
    torch.cuda.synchronize()
    q, s, g, a = oracle.quantize_transposed_tensor(x, 16, "e4m3", "current", nthreads=8, rht_signs=0x13579BDF,
                                                   elem=elem)
    assert_bytes_equal(host(qt.q), q, f"{elem} rht transposed codes")
    assert_bytes_equal(host(qt.scales), s, f"{elem} rht transposed scales")
    assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([g, a]), f"{elem} rht transposed ts")
    big = _like(2048, 1000, 731)
    qt = fq.fp4_quantize_transposed(to_device(big), 32, "e8m0", amax="none", rounding="stochastic", seed=4,
                                    element=elem)
    torch.cuda.synchronize()
    q, s, _, _ = oracle.quantize_transposed_tensor(big, 32, "e8m0", "none", stochastic=True, seed=4, nthreads=8,
                                                   elem=elem)
    assert_bytes_equal(host(qt.q), q, f"{elem} large transposed codes")
    assert_bytes_equal(host(qt.scales), s, f"{elem} large transposed scales")


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


def _gemm_check(c, a_hat, w_hat, rows=None, tag=""):
    if rows is not None:
        a_hat = a_hat[rows]
    cref, tol = oracle.gemm_ref(a_hat, w_hat)
    got = c.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        got = got[rows]
    ok = oracle.gemm_check(got, cref, tol)
    assert ok.all(), f"{tag}: {int((~ok).sum())} of {ok.size} outputs out of tolerance"


def _quant_pair(x, block, fmt, elem, *, rounding="nearest", seed=0, rht=None):
    """GPU and oracle quantization of one operand; codes, scales and tensor
    scale must agree bit for bit.  Returns (QTensor, oracle binary64 values)."""
    pol = _policy(fmt)
    qt = fq.fp4_quantize(to_device(x), block, fmt, amax=pol, rounding=rounding, seed=seed, rht_signs=rht,
                         element=elem)
    q, s, g, _ = oracle.quantize_tensor(x, block, fmt, pol, stochastic=rounding == "stochastic", seed=seed,
                                        nthreads=8, rht_signs=rht, elem=elem)
    torch.cuda.synchronize()
    assert_bytes_equal(host(qt.q), q, f"{elem} {fmt} operand codes")
    assert_bytes_equal(host(qt.scales), s, f"{elem} {fmt} operand scales")
    return qt, oracle.dequantize_f64(q, s, g, block, fmt, elem=elem)


# Every scale pairing the exact dequantize GEMM takes for the 8-bit grids:
# FP8 elements in bf16 for scales with at most 3 mantissa bits, INT8 in bf16
# for power-of-two scales and in f16 for E4M3 scales.
GEMM_8BIT = [("fp8_e4m3", "e8m0", 32), ("fp8_e4m3", "e8m0", 16), ("fp8_e4m3", "e4m3", 16),
             ("fp8_e4m3", "ue5m3", 32), ("fp8_e4m3", "e5m2", 16), ("fp8_e4m3", "e6m1", 32),
             ("fp8_e4m3", "e7m0", 16), ("int8", "e8m0", 32), ("int8", "e7m0", 16), ("int8", "e4m3", 16),
             ("int8", "e4m3", 32)]


@pytest.mark.parametrize("elem,fmt,block", GEMM_8BIT)
def test_8bit_gemm(elem, fmt, block):
    """Ragged M and N (partial 256-row tiles on both sides), K over several
    64-element stages."""
    m, n, k = 200, 330, 768
    qa, a = _quant_pair(_like(m, k, 81, "f32"), block, fmt, elem)
    qw, w = _quant_pair(_like(n, k, 82, "f32"), block, fmt, elem)
    c = fq.fp4_gemm(qa, qw)
    torch.cuda.synchronize()
    assert c.shape == (m, n)
    _gemm_check(c, a, w, tag=f"{elem} {fmt}/{block} gemm")


@pytest.mark.parametrize("elem,fmt,block", [("fp8_e4m3", "e8m0", 32), ("fp8_e4m3", "e8m0", 16), ("int8", "e4m3", 16),
                                            ("int8", "e4m3", 32)])
@pytest.mark.parametrize("m,n,k", [(1, 33, 128), (257, 513, 384), (64, 256, 1152)])
def test_8bit_gemm_register_path_shapes(elem, fmt, block, m, n, k):
    """The pairings converted in registers (MXFP8; INT8 with E4M3 scales):
    one 128-element stage, odd stage counts past the two-stage ring, ragged
    M and N, a single output row."""
    qa, a = _quant_pair(_like(m, k, 91 + k, "f32"), block, fmt, elem)
    qw, w = _quant_pair(_like(n, k, 92 + k, "f32"), block, fmt, elem)
    c = fq.fp4_gemm(qa, qw)
    torch.cuda.synchronize()
    _gemm_check(c, a, w, tag=f"{elem} {fmt}/{block} {m}x{n}x{k}")


@pytest.mark.parametrize("elem", ELEMS)
def test_8bit_gemm_transform_and_sr(elem):
    """Both operands Hadamard-rotated with the same signs (the product is
    that of the rotated operands) and stochastically rounded operands."""
    fmt, block = ("e8m0", 32)
    xa, xw = _like(96, 512, 83, "f32"), _like(72, 512, 84, "f32")
    qa, a = _quant_pair(xa, block, fmt, elem, rht=0x2468ACE1)
    qw, w = _quant_pair(xw, block, fmt, elem, rht=0x2468ACE1)
    c = fq.fp4_gemm(qa, qw)
    torch.cuda.synchronize()
    _gemm_check(c, a, w, tag=f"{elem} rht gemm")
    qa, a = _quant_pair(xa, block, fmt, elem, rounding="stochastic", seed=11)
    qw, w = _quant_pair(xw, block, fmt, elem, rounding="stochastic", seed=12)
    c = fq.fp4_gemm(qa, qw)
    torch.cuda.synchronize()
    _gemm_check(c, a, w, tag=f"{elem} sr gemm")


@pytest.mark.parametrize("elem,fmt,block", [("fp8_e4m3", "e8m0", 32), ("int8", "e4m3", 16)])
def test_8bit_gemm_llama_every_output(elem, fmt, block):
    """Llama-2 7B square projection at M = 8192 (batch 4 x seq 2048), the
    launch the GEMM timing uses: every output against the binary64
    reference."""
    shapes = {"a": (8192, 4096), "sq": (4096, 4096)}
    qa, a = _quant_pair(inputs.llama("a", shapes), block, fmt, elem)
    qw, w = _quant_pair(inputs.llama("sq", shapes), block, fmt, elem)
    c = fq.fp4_gemm(qa, qw)
    torch.cuda.synchronize()
    check_gemm_every_output(c, a, w, f"{elem} {fmt} llama sq")


@pytest.mark.parametrize("elem,fmt", [("fp8_e4m3", "e8m0"), ("int8", "e8m0"), ("int8", "e4m3")])
def test_8bit_gemm_every_code(elem, fmt):
    """Every element code through the GEMM's decode, subnormals and signed
    zeros included: A holds all 256 codes (the two FP8 NaN codes replaced)
    with mixed block scales, W selects one column per output
    (W[n, k] = 1 if k == n, one scale of 1), so C[m, n] is the bf16 rounding
    of A's value at (m, n) times the tensor scales."""
    k = 256
    codes = np.arange(256, dtype=np.uint8)
    if elem == "fp8_e4m3":
        codes[(codes & 0x7F) == 0x7F] = 0x00
    q_a = np.stack([codes, codes[::-1], np.roll(codes, 77)])
    rng = np.random.default_rng(23)
    block = 32 if fmt == "e8m0" else 16
    if fmt == "e8m0":
        s_a = rng.integers(110, 145, (3, k // block), dtype=np.uint8)
        one, g_a, pol = 127, 1.0, "none"
    else:
        s_a = rng.integers(0, 0x7F, (3, k // block), dtype=np.uint8)
        one, g_a, pol = 0x38, 0.0625, "current"   # a power of two: g * acc stays exact
    q_w = np.zeros((k, k), dtype=np.uint8)
    q_w[np.arange(k), np.arange(k)] = 0x38 if elem == "fp8_e4m3" else 1
    s_w = np.full((k, k // block), one, dtype=np.uint8)

    def qt(q, s, g):
        return fq.QTensor(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(),
                          torch.tensor([g, 0.0], dtype=torch.float32).cuda(), q.shape[0], k, block, fmt, amax=pol,
                          element=elem)
    c = fq.fp4_gemm(qt(q_a, s_a, g_a), qt(q_w, s_w, 1.0))
    torch.cuda.synchronize()
    a_hat = oracle.dequantize_f64(q_a, s_a, np.float32(g_a), block, fmt, elem=elem)
    w_hat = oracle.dequantize_f64(q_w, s_w, np.float32(1.0), block, fmt, elem=elem)
    assert np.array_equal(w_hat, np.eye(k))
    want = oracle.round_to_bf16(a_hat)
    got = c.float().cpu().numpy().astype(np.float64)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (f"{elem} {fmt}: {len(bad)} outputs differ; first {tuple(bad[0])}: got "
                           f"{got[tuple(bad[0])]!r} want {want[tuple(bad[0])]!r}")


def test_mxfp8_gemm_subnormal_products():
    """MXFP8 with E8M0 scales 2^-127 .. 2^-116: every FP8 code times a scale
    near the bottom of the range, so many products lie below bf16's normal
    range.  W selects one column per output (as in the every-code test).
    Products that bf16 holds exactly (its subnormals included) must come out
    exactly; the others within one bf16 subnormal step (2^-133)."""
    k = 256
    codes = np.arange(256, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00
    q_a = np.stack([codes, codes[::-1], np.roll(codes, 77), np.roll(codes, 150)])
    rng = np.random.default_rng(31)
    s_a = rng.integers(0, 12, (4, k // 32), dtype=np.uint8)
    q_w = np.zeros((k, k), dtype=np.uint8)
    q_w[np.arange(k), np.arange(k)] = 0x38
    s_w = np.full((k, k // 32), 127, dtype=np.uint8)

    def qt(q, s):
        return fq.QTensor(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(),
                          torch.tensor([1.0, 0.0], dtype=torch.float32).cuda(), q.shape[0], k, 32, "e8m0",
                          amax="none", element="fp8_e4m3")
    c = fq.fp4_gemm(qt(q_a, s_a), qt(q_w, s_w))
    torch.cuda.synchronize()
    a_hat = oracle.dequantize_f64(q_a, s_a, np.float32(1.0), 32, "e8m0", elem="fp8_e4m3")
    got = c.float().cpu().numpy().astype(np.float64)
    exact = oracle.round_to_bf16(a_hat) == a_hat
    bad = np.argwhere(exact & (got != a_hat))
    assert bad.size == 0, (f"{len(bad)} bf16-exact products differ; first {tuple(bad[0])}: got "
                           f"{got[tuple(bad[0])]!r} want {a_hat[tuple(bad[0])]!r}")
    far = np.argwhere(~exact & (np.abs(got - a_hat) > 2.0 ** -133))
    assert far.size == 0, f"{len(far)} outputs beyond one bf16 subnormal step; first {tuple(far[0])}"


@pytest.mark.parametrize("elem,fmt", [("fp8_e4m3", "e3m4"), ("fp8_e4m3", "e1m6"), ("int8", "ue5m3"),
                                      ("int8", "e3m4"), ("int8", "e5m2")])
def test_8bit_gemm_inexact_pairing_rejected(elem, fmt):
    """Scale formats whose products with the grid's elements no 16-bit type
    holds exactly are refused, not rounded."""
    xd = to_device(_like(64, 256, 85, "f32"))
    q = fq.fp4_quantize(xd, 16, fmt, element=elem)
    with pytest.raises(fq.Fp4Error) as e:
        fq.fp4_gemm(q, q)
    assert e.value.status == -2


def test_8bit_gemm_mixed_grids_rejected():
    xd = to_device(_like(64, 256, 74, "f32"))
    q8 = fq.fp4_quantize(xd, 32, "e8m0", amax="none", element="int8")
    f8 = fq.fp4_quantize(xd, 32, "e8m0", amax="none", element="fp8_e4m3")
    f4 = fq.fp4_quantize(xd, 32, "e8m0", amax="none")
    for call in (lambda: fq.fp4_gemm(q8, f8),
                 lambda: fq.fp4_gemm(f8, f4)):
        with pytest.raises(fq.Fp4Error) as e:
            call()
        assert e.value.status == -2
