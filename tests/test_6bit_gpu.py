"""GPU parity of the 6-bit MX element grids (MXFP6-style FP6 E2M3 and E3M2
elements, MXINT6-style symmetric INT6; six bits per element, packed as a
little-endian bit stream) against the CPU oracle: codes, scales and tensor
scale bit for bit for every scale encoding, both rounding modes, the
single-pass and two-pass refreshes, the Hadamard transform and ragged row
counts; every FP6 rounding midpoint; dequantization of every code bit for
bit; the GEMM within the binary64 reference's tolerance on every scale
pairing it takes and bit for bit on every code; a GEMM of operands on
different grids is rejected.  Every call goes
through the C ABI.
"""
import numpy as np
import pytest
import torch

import fp4_inputs as inputs
import oracle
from tests.gpu_util import assert_bytes_equal, bf16_bits, f32_bits, host, to_device

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp4_block_scaled_quantize_amd")

ELEMS = ["fp6_e2m3", "fp6_e3m2", "int6"]


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
def test_6bit_quantize_parity(elem, fmt, block, dtype, rounding):
    """67 rows: a ragged last wave of units; 320 columns: 10 or 20 blocks."""
    x = _like(67, 320, 900 + block, dtype)
    _check(x, block, fmt, _policy(fmt), elem, rounding=rounding, seed=0x5EED, offset=5,
           tag=f"{elem} {fmt}/{block}/{dtype}/{rounding}")


@pytest.mark.parametrize("elem", ELEMS)
def test_6bit_full_size_two_pass_and_transform(elem):
    x = inputs.sweep()
    _check(x, 32, "e8m0", "none", elem, tag=f"{elem} sweep mx")
    _check(x, 16, "e4m3", "current", elem, tag=f"{elem} sweep nv")
    big = _like(4104, 4096, 91)
    _check(big, 16, "e4m3", "current", elem, rows=[0, 7, 2052, 4103], tag=f"{elem} two-pass")
    small = _like(40, 512, 92)
    _check(small, 32, "e8m0", "none", elem, rht=0x9E3779B9, tag=f"{elem} rht")
    _check(small, 16, "e4m3", "current", elem, rht=0x12345678, rounding="stochastic", seed=3, offset=1,
           tag=f"{elem} rht sr")


def _fp6_positive(elem):
    eb, mb, bias = (2, 3, 1) if elem == "fp6_e2m3" else (3, 2, 3)
    out = []
    for c in range(32):
        e, m = c >> mb, c & ((1 << mb) - 1)
        out.append(m * 2.0 ** (1 - bias - mb) if e == 0 else (1 + m / 2 ** mb) * 2.0 ** (e - bias))
    return np.array(out)


@pytest.mark.parametrize("elem,emax", [("fp6_e2m3", 2), ("fp6_e3m2", 4)])
def test_fp6_rtn_every_midpoint(elem, emax):
    """Every FP6 value, every midpoint between neighbours, the binary32
    values on either side of each midpoint, and the saturation range below
    2^(emax+1), both signs; every block holds 2^emax, so its E8M0 scale is
    exactly 1 and the encoder sees the values unchanged."""
    q = _fp6_positive(elem)
    mid = (q[:-1] + q[1:]) / 2
    f32 = lambda a: np.asarray(a, dtype=np.float32)
    top = 2.0 ** (emax + 1)
    vals = np.concatenate([f32(q), f32(mid), np.nextafter(f32(mid), f32(np.inf)),
                           np.nextafter(f32(mid), f32(-np.inf)),
                           f32([q[-1] * 1.01, (q[-1] + top) / 2, top * 0.999])])
    vals = np.concatenate([vals, -vals])
    per = 31
    nblk = -(-vals.size // per)
    vals = np.concatenate([vals, np.zeros(nblk * per - vals.size, dtype=np.float32)])
    blocks = np.concatenate([np.full((nblk, 1), 2.0 ** emax, dtype=np.float32), vals.reshape(nblk, per)], axis=1)
    cols = 256
    nblk_pad = -(-nblk // (cols // 32)) * (cols // 32)
    blocks = np.concatenate([blocks, np.tile(blocks[:1], (nblk_pad - nblk, 1))])
    x = np.ascontiguousarray(blocks.reshape(-1, cols))
    qt = _check(x, 32, "e8m0", "none", elem, tag=f"{elem} midpoints")
    assert np.all(host(qt.scales) == 127)


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("fmt,block", [("e8m0", 32), ("e4m3", 16)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_6bit_dequantize_parity(elem, fmt, block, out):
    """Random codes (every 6-bit pattern is a valid code) over 19 rows."""
    rng = np.random.default_rng(29)
    rows, cols = 19, 256
    q = rng.integers(0, 256, (rows, cols * 3 // 4), dtype=np.uint8)
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
def test_6bit_dequantize_rht_roundtrip_parity(elem):
    x = _like(40, 512, 93, "f32")
    qt = _check(x, 32, "e8m0", "none", elem, rht=0x2468ACE1, tag=f"{elem} rht")
    y = host(fq.fp4_dequantize(qt, torch.float32))
    q, s, g, _ = oracle.quantize_tensor(x, 32, "e8m0", "none", rht_signs=0x2468ACE1, elem=elem)
    want = oracle.rht_inverse(oracle.dequantize(q, s, float(g), 32, "e8m0", elem=elem), 32, 0x2468ACE1)
    assert_bytes_equal(f32_bits(y), f32_bits(want), f"{elem} rht dequant")


@pytest.mark.parametrize("elem", ELEMS + ["fp8_e4m3", "int8"])
def test_wide_grid_edge_shapes(elem):
    """Empty tensors (no rows, no columns), the smallest row (one 16-element
    block), strided input rows and strided dequantized output, for the 6- and
    8-bit grids."""
    for shape in [(0, 64), (64, 0), (0, 0)]:
        x = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
        qt = fq.fp4_quantize(x, 16, "e4m3", element=elem)
        y = fq.fp4_dequantize(qt, torch.bfloat16)
        torch.cuda.synchronize()
        assert tuple(y.shape) == shape
    x1 = _like(1, 16, 101, "f32")
    _check(x1, 16, "e4m3", "current", elem, tag=f"{elem} 1x16")
    _check(x1, 16, "e8m0", "none", elem, rounding="stochastic", seed=2, tag=f"{elem} 1x16 sr")
    big = _like(37, 512, 102, "f32")
    xs = to_device(big)[:, 64:448]                      # rows strided by 512, 384 columns
    sub = np.ascontiguousarray(big[:, 64:448])
    qt = fq.fp4_quantize(xs, 32, "e8m0", amax="none", element=elem)
    q, s, g, _ = oracle.quantize_tensor(sub, 32, "e8m0", "none", elem=elem)
    torch.cuda.synchronize()
    assert_bytes_equal(host(qt.q), q, f"{elem} strided codes")
    assert_bytes_equal(host(qt.scales), s, f"{elem} strided scales")
    wide = torch.full((37, 400), -1.0, dtype=torch.float32, device="cuda")
    fq.fp4_dequantize(qt, torch.float32, out=wide[:, :384])
    torch.cuda.synchronize()
    want = oracle.dequantize(q, s, float(g), 32, "e8m0", out="f32", elem=elem)
    assert_bytes_equal(f32_bits(host(wide[:, :384])), f32_bits(want), f"{elem} strided dequant")
    assert bool((wide[:, 384:] == -1.0).all())            # padding columns untouched


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("fmt,block,pol", [("e8m0", 32, "none"), ("e8m0", 16, "none"), ("e4m3", 16, "current")])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rounding", ["nearest", "stochastic"])
def test_6bit_transposed_parity(elem, fmt, block, pol, dtype, rounding):
    """Column-wise quantization on the 6-bit grids: 320 rows (a partial
    256-row tile of 64 rows) by 200 columns (a partial 64-column tile)."""
    x = _like(320, 200, 740 + block, dtype)
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
def test_6bit_transposed_ue5m3_delayed_and_strided(elem):
    """Column-wise 6-bit quantization with UE5M3 scales at block 32, a delayed
    maximum across a refresh (interval 3, five calls, the later tensors
    growing so the stored maximum saturates them), and a row-strided view."""
    x = _like(320, 200, 760)
    qt = fq.fp4_quantize_transposed(to_device(x), 32, "ue5m3", amax="current", element=elem)
    torch.cuda.synchronize()
    q, s, g, a = oracle.quantize_transposed_tensor(x, 32, "ue5m3", "current", nthreads=8, elem=elem)
    assert_bytes_equal(host(qt.q), q, f"{elem} ue5m3 transposed codes")
    assert_bytes_equal(host(qt.scales), s, f"{elem} ue5m3 transposed scales")
    assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([g, a]), f"{elem} ue5m3 transposed ts")
    st = fq.AmaxState(3)
    ost = oracle.AmaxState(interval=3)
    for t in range(5):
        xt = _like(192, 136, 761 + t, "f32") * np.float32(1.0 + 0.5 * t)
        qt = fq.fp4_quantize_transposed(to_device(xt), 16, "e4m3", amax="delayed", state=st, element=elem,
                                        rounding="stochastic" if t % 2 else "nearest", seed=9, offset=t)
        torch.cuda.synchronize()
        q, s, g, a = oracle.quantize_transposed_tensor(xt, 16, "e4m3", "delayed", state=ost, nthreads=8, elem=elem,
                                                       stochastic=bool(t % 2), seed=9, offset=t)
        assert_bytes_equal(host(qt.q), q, f"{elem} delayed call {t} codes")
        assert_bytes_equal(host(qt.scales), s, f"{elem} delayed call {t} scales")
        assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([g, a]), f"{elem} delayed call {t} ts")
    xs = _like(256, 200, 770, "f32")
    wide = torch.zeros((256, 264), dtype=torch.float32, device="cuda")
    wide[:, :200] = torch.from_numpy(xs).cuda()
    qt = fq.fp4_quantize_transposed(wide[:, :200], 32, "e8m0", amax="none", element=elem)
    torch.cuda.synchronize()
    q, s, _, _ = oracle.quantize_transposed_tensor(xs, 32, "e8m0", "none", nthreads=8, elem=elem)
    assert_bytes_equal(host(qt.q), q, f"{elem} strided transposed codes")
    assert_bytes_equal(host(qt.scales), s, f"{elem} strided transposed scales")


@pytest.mark.parametrize("elem", ELEMS)
def test_6bit_transposed_transform_larger_and_shape_rule(elem):
    x = _like(512, 136, 750)
    qt = fq.fp4_quantize_transposed(to_device(x), 16, "e4m3", amax="current", rht_signs=0x13579BDF, element=elem)
    torch.cuda.synchronize()
    q, s, g, a = oracle.quantize_transposed_tensor(x, 16, "e4m3", "current", nthreads=8, rht_signs=0x13579BDF,
                                                   elem=elem)
    assert_bytes_equal(host(qt.q), q, f"{elem} rht transposed codes")
    assert_bytes_equal(host(qt.scales), s, f"{elem} rht transposed scales")
    assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([g, a]), f"{elem} rht transposed ts")
    big = _like(2048, 1000, 751)
    qt = fq.fp4_quantize_transposed(to_device(big), 32, "e8m0", amax="none", rounding="stochastic", seed=4,
                                    element=elem)
    torch.cuda.synchronize()
    q, s, _, _ = oracle.quantize_transposed_tensor(big, 32, "e8m0", "none", stochastic=True, seed=4, nthreads=8,
                                                   elem=elem)
    assert_bytes_equal(host(qt.q), q, f"{elem} large transposed codes")
    assert_bytes_equal(host(qt.scales), s, f"{elem} large transposed scales")
    with pytest.raises(fq.Fp4Error) as e:                 # R = 96: not a multiple of 64
        fq.fp4_quantize_transposed(to_device(_like(96, 64, 752)), 32, "e8m0", amax="none", element=elem)
    assert e.value.status == -3


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
    pol = _policy(fmt)
    qt = fq.fp4_quantize(to_device(x), block, fmt, amax=pol, rounding=rounding, seed=seed, rht_signs=rht,
                         element=elem)
    q, s, g, _ = oracle.quantize_tensor(x, block, fmt, pol, stochastic=rounding == "stochastic", seed=seed,
                                        nthreads=8, rht_signs=rht, elem=elem)
    torch.cuda.synchronize()
    assert_bytes_equal(host(qt.q), q, f"{elem} {fmt} operand codes")
    assert_bytes_equal(host(qt.scales), s, f"{elem} {fmt} operand scales")
    return qt, oracle.dequantize_f64(q, s, g, block, fmt, elem=elem)


# Scale pairings the exact dequantize GEMM takes for the 6-bit grids: FP6
# E2M3 (4 significant bits) in bf16 for scales with at most 3 mantissa bits,
# E3M2 (3 bits) for at most 4, INT6 (5 bits) in bf16 for at most 2 and in
# f16 for E4M3 / E3M4 / E2M5.
GEMM_6BIT = [("fp6_e2m3", "e8m0", 32), ("fp6_e2m3", "e4m3", 16), ("fp6_e2m3", "ue5m3", 32),
             ("fp6_e3m2", "e8m0", 32), ("fp6_e3m2", "e3m4", 16), ("fp6_e3m2", "e4m3", 16),
             ("int6", "e8m0", 32), ("int6", "e5m2", 16), ("int6", "e4m3", 16), ("int6", "e3m4", 32),
             ("int6", "e2m5", 16)]


@pytest.mark.parametrize("elem,fmt,block", GEMM_6BIT)
def test_6bit_gemm(elem, fmt, block):
    """Ragged M and N (partial 256-row tiles), K over several 64-element
    stages."""
    m, n, k = 200, 330, 768
    qa, a = _quant_pair(_like(m, k, 95, "f32"), block, fmt, elem)
    qw, w = _quant_pair(_like(n, k, 96, "f32"), block, fmt, elem)
    c = fq.fp4_gemm(qa, qw)
    torch.cuda.synchronize()
    assert c.shape == (m, n)
    _gemm_check(c, a, w, tag=f"{elem} {fmt}/{block} gemm")


@pytest.mark.parametrize("elem", ELEMS)
def test_6bit_gemm_transform_sr_and_llama(elem):
    """Hadamard-rotated and stochastically rounded operands, then the Llama-2
    7B square projection at M = 8192 on sampled output rows."""
    fmt, block = "e8m0", 32
    xa, xw = _like(96, 512, 97, "f32"), _like(72, 512, 98, "f32")
    qa, a = _quant_pair(xa, block, fmt, elem, rht=0x2468ACE1)
    qw, w = _quant_pair(xw, block, fmt, elem, rht=0x2468ACE1)
    _gemm_check(fq.fp4_gemm(qa, qw), a, w, tag=f"{elem} rht gemm")
    qa, a = _quant_pair(xa, block, fmt, elem, rounding="stochastic", seed=11)
    qw, w = _quant_pair(xw, block, fmt, elem, rounding="stochastic", seed=12)
    _gemm_check(fq.fp4_gemm(qa, qw), a, w, tag=f"{elem} sr gemm")
    shapes = {"a": (8192, 4096), "sq": (4096, 4096)}
    qa, a = _quant_pair(inputs.llama("a", shapes), block, fmt, elem)
    qw, w = _quant_pair(inputs.llama("sq", shapes), block, fmt, elem)
    c = fq.fp4_gemm(qa, qw)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([rng.integers(0, 8192, 16), [0, 255, 256, 8191]]))
    _gemm_check(c, a, w, rows=rows, tag=f"{elem} llama sq")


@pytest.mark.parametrize("elem,fmt", [("fp6_e2m3", "e8m0"), ("fp6_e3m2", "e8m0"), ("int6", "e8m0"),
                                      ("int6", "e4m3")])
def test_6bit_gemm_every_code(elem, fmt):
    """All 64 codes through the GEMM's decode: A holds every code (four
    times per row, shifted) with mixed block scales, W selects one column per
    output (one code of value 1, one scale of 1), so C[m, n] is the bf16
    rounding of A's value at (m, n)."""
    k = 256
    codes = np.tile(np.arange(64, dtype=np.int64), 4)
    rows_codes = np.stack([codes, codes[::-1], np.roll(codes, 21)])

    def pack(c):
        out = np.zeros((c.shape[0], c.shape[1] * 3 // 4), dtype=np.uint8)
        for r in range(c.shape[0]):
            big = 0
            for j, v in enumerate(c[r]):
                big |= int(v) << (6 * j)
            out[r] = np.frombuffer(big.to_bytes(out.shape[1], "little"), dtype=np.uint8)
        return out
    one = {"fp6_e2m3": 0x08, "fp6_e3m2": 0x0C, "int6": 0x01}[elem]      # the code of 1.0
    block = 32 if fmt == "e8m0" else 16
    rng = np.random.default_rng(27)
    if fmt == "e8m0":
        s_a = rng.integers(110, 145, (3, k // block), dtype=np.uint8)
        s_one, g_a, pol = 127, 1.0, "none"
    else:
        s_a = rng.integers(0, 0x7F, (3, k // block), dtype=np.uint8)
        s_one, g_a, pol = 0x38, 0.0625, "current"
    q_a = pack(rows_codes)
    w_codes = np.zeros((k, k), dtype=np.int64)
    w_codes[np.arange(k), np.arange(k)] = one
    q_w = pack(w_codes)
    s_w = np.full((k, k // block), s_one, dtype=np.uint8)

    def qt(q, s, g, rows):
        return fq.QTensor(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(),
                          torch.tensor([g, 0.0], dtype=torch.float32).cuda(), rows, k, block, fmt, amax=pol,
                          element=elem)
    c = fq.fp4_gemm(qt(q_a, s_a, g_a, 3), qt(q_w, s_w, 1.0, k))
    torch.cuda.synchronize()
    a_hat = oracle.dequantize_f64(q_a, s_a, np.float32(g_a), block, fmt, elem=elem)
    w_hat = oracle.dequantize_f64(q_w, s_w, np.float32(1.0), block, fmt, elem=elem)
    assert np.array_equal(w_hat, np.eye(k))
    want = oracle.round_to_bf16(a_hat)
    got = c.float().cpu().numpy().astype(np.float64)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (f"{elem} {fmt}: {len(bad)} outputs differ; first {tuple(bad[0])}: got "
                           f"{got[tuple(bad[0])]!r} want {want[tuple(bad[0])]!r}")


@pytest.mark.parametrize("elem,fmt", [("fp6_e2m3", "e3m4"), ("fp6_e3m2", "e1m6"), ("int6", "ue5m3"),
                                      ("int6", "e1m6")])
def test_6bit_gemm_inexact_pairing_rejected(elem, fmt):
    xd = to_device(_like(64, 256, 99, "f32"))
    q = fq.fp4_quantize(xd, 16, fmt, element=elem)
    with pytest.raises(fq.Fp4Error) as e:
        fq.fp4_gemm(q, q)
    assert e.value.status == -2


def test_6bit_gemm_mixed_grids_rejected():
    xd = to_device(_like(64, 256, 94, "f32"))
    for elem in ELEMS:
        q6 = fq.fp4_quantize(xd, 32, "e8m0", amax="none", element=elem)
        f6 = fq.fp4_quantize(xd, 32, "e8m0", amax="none", element="fp6_e3m2" if elem != "fp6_e3m2" else "int6")
        for call in (lambda: fq.fp4_gemm(q6, f6),):
            with pytest.raises(fq.Fp4Error) as e:
                call()
            assert e.value.status == -2
