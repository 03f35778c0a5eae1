"""GPU parity of the 6-bit MX element grids (MXFP6-style FP6 E2M3 and E3M2
elements, MXINT6-style symmetric INT6; six bits per element, packed as a
little-endian bit stream) against the CPU oracle: codes, scales and tensor
scale bit for bit for every scale encoding, both rounding modes, the
single-pass and two-pass refreshes, the Hadamard transform and ragged row
counts; every FP6 rounding midpoint; dequantization of every code bit for
bit; the paths that do not take 6-bit grids reject them.  Every call goes
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


def test_6bit_rejected_elsewhere():
    xd = to_device(_like(64, 256, 94, "f32"))
    for elem in ELEMS:
        q6 = fq.fp4_quantize(xd, 32, "e8m0", amax="none", element=elem)
        for call in (lambda: fq.fp4_gemm(q6, q6),
                     lambda: fq.fp4_wo_gemm(torch.zeros((1, 256), dtype=torch.bfloat16, device="cuda"), q6),
                     lambda: fq.fp4_quantize_transposed(xd, 32, "e8m0", amax="none", element=elem),
                     lambda: fq.fp4_quantize_both(xd, 32, "e8m0", amax="none", element=elem)):
            with pytest.raises(fq.Fp4Error) as e:
                call()
            assert e.value.status == -2
