"""GPU parity of the two-orientation quantize call (one read of x, the
row-wise and the column-wise outputs) against the CPU oracle: each output
bit-identical to the oracle's single-orientation quantization (row-wise: x;
column-wise: x^T), with the shared tensor scale.  Every call goes through the
C ABI.
"""
import numpy as np
import pytest
import torch

import fp4_inputs as inputs
import oracle
from tests.gpu_util import assert_bytes_equal, f32_bits, host, to_device

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


def _check_both(x, block, fmt, pol, *, rounding="nearest", seed=0, offset=0, element="e2m1", tag=""):
    st = fq.AmaxState(1) if pol == "current" else None
    qr, qc = fq.fp4_quantize_both(to_device(x), block, fmt, rounding=rounding, amax=pol, state=st, seed=seed,
                                  offset=offset, element=element)
    torch.cuda.synchronize()
    sr = rounding == "stochastic"
    q, s, g, a = oracle.quantize_tensor(x, block, fmt, pol, stochastic=sr, seed=seed, offset=offset, nthreads=8,
                                        elem=element)
    assert_bytes_equal(host(qr.scales), s, f"{tag} row scales")
    assert_bytes_equal(host(qr.q), q, f"{tag} row codes")
    assert_bytes_equal(f32_bits(host(qr.tensor_scale)), f32_bits([g, a]), f"{tag} row tensor_scale")
    q, s, g, a = oracle.quantize_transposed_tensor(x, block, fmt, pol, stochastic=sr, seed=seed, offset=offset,
                                                   nthreads=8, elem=element)
    assert_bytes_equal(host(qc.scales), s, f"{tag} col scales")
    assert_bytes_equal(host(qc.q), q, f"{tag} col codes")
    assert_bytes_equal(f32_bits(host(qc.tensor_scale)), f32_bits([g, a]), f"{tag} col tensor_scale")


@pytest.mark.parametrize("fmt", ["e4m3", "ue5m3", "e1m6", "e8m0"])
@pytest.mark.parametrize("block", [16, 32])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rounding", ["nearest", "stochastic"])
def test_both_parity(fmt, block, dtype, rounding):
    # 352 rows (one whole and one partial 256-row tile), 160 columns (two
    # whole 64-column tiles and a partial one)
    x = _like(352, 160, 600 + block, dtype)
    _check_both(x, block, fmt, _policy(fmt), rounding=rounding, seed=0x5EED, offset=3, tag=f"both {fmt}/{block}/{dtype}")


@pytest.mark.parametrize("fmt,block", [("e4m3", 16), ("e8m0", 32)])
@pytest.mark.parametrize("rounding", ["nearest", "stochastic"])
def test_both_int4(fmt, block, rounding):
    x = _like(256, 192, 61)
    _check_both(x, block, fmt, _policy(fmt), rounding=rounding, seed=9, offset=1, element="int4", tag="both int4")


WIDE = ["fp8_e4m3", "int8", "fp6_e2m3", "fp6_e3m2", "int6"]


@pytest.mark.parametrize("element", WIDE)
@pytest.mark.parametrize("fmt,block", [("e8m0", 32), ("e8m0", 16), ("e4m3", 16), ("ue5m3", 32)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rounding", ["nearest", "stochastic"])
def test_both_wide_grids(element, fmt, block, dtype, rounding):
    """The 8- and 6-bit grids: row-wise codes one byte (or six bits in the
    row-major stream) per element, column-wise as the transposed call.  320
    rows (a whole and a partial 256-row tile, a multiple of 64 for the 6-bit
    column-wise chunks) by 160 columns (two whole 64-column tiles and a
    partial one)."""
    x = _like(320, 160, 800 + block, dtype)
    _check_both(x, block, fmt, _policy(fmt), rounding=rounding, seed=0x5EED, offset=3, element=element,
                tag=f"both {element} {fmt}/{block}/{dtype}/{rounding}")


@pytest.mark.parametrize("element", WIDE)
def test_both_wide_grids_larger_and_delayed(element):
    """2048 x 1536 bf16 with E4M3 scales at block 16, three delayed-amax
    calls on new tensors (a refresh at the first, the stored maximum after
    it; nearest rounding first, then stochastic), each against the oracle's
    sequence."""
    st = fq.AmaxState(50)
    ost = oracle.AmaxState(50)
    for t in range(3):
        x = _like(2048, 1536, 900 + t)
        qr, qc = fq.fp4_quantize_both(to_device(x), 16, "e4m3", rounding="stochastic" if t else "nearest",
                                      amax="delayed", state=st, seed=77, offset=t, element=element)
        torch.cuda.synchronize()
        sr = t > 0
        o_before = ost.calls
        q, s, g, a = oracle.quantize_tensor(x, 16, "e4m3", "delayed", stochastic=sr, seed=77, offset=t, nthreads=8,
                                            state=ost, elem=element)
        tag = f"both {element} call {t}"
        assert_bytes_equal(host(qr.scales), s, f"{tag} row scales")
        assert_bytes_equal(host(qr.q), q, f"{tag} row codes")
        assert_bytes_equal(f32_bits(host(qr.tensor_scale)), f32_bits([g, a]), f"{tag} row tensor_scale")
        ost.calls = o_before
        q, s, g, a = oracle.quantize_transposed_tensor(x, 16, "e4m3", "delayed", stochastic=sr, seed=77, offset=t,
                                                       nthreads=8, state=ost, elem=element)
        assert_bytes_equal(host(qc.scales), s, f"{tag} col scales")
        assert_bytes_equal(host(qc.q), q, f"{tag} col codes")
        assert_bytes_equal(f32_bits(host(qc.tensor_scale)), f32_bits([g, a]), f"{tag} col tensor_scale")


@pytest.mark.parametrize("element", ["fp6_e2m3", "fp6_e3m2", "int6"])
def test_both_6bit_shape_rule(element):
    """The 6-bit column-wise output needs R % 64 == 0: 96 rows are refused
    with SHAPE before any launch."""
    xd = to_device(_like(96, 64, 95))
    with pytest.raises(fq.Fp4Error) as e:
        fq.fp4_quantize_both(xd, 32, "e8m0", amax="none", element=element)
    assert e.value.status == -3


def test_both_sweep_full_size():
    _check_both(inputs.sweep(), 16, "e4m3", "current", tag="both sweep")


def test_both_grads_sampled_and_matches_single_calls():
    """8192x8192 gradients, SR, delayed amax: both outputs equal the two
    single-orientation GPU calls byte for byte, and sampled rows of each
    equal the oracle."""
    x = inputs.grads(2)
    xd = to_device(x)
    st, s1, s2 = fq.AmaxState(50), fq.AmaxState(50), fq.AmaxState(50)
    qr, qc = fq.fp4_quantize_both(xd, 16, "e4m3", rounding="stochastic", amax="delayed", state=st, seed=0x5EED,
                                  offset=2)
    r1 = fq.fp4_quantize(xd, 16, "e4m3", rounding="stochastic", amax="delayed", state=s1, seed=0x5EED, offset=2)
    c1 = fq.fp4_quantize_transposed(xd, 16, "e4m3", rounding="stochastic", amax="delayed", state=s2, seed=0x5EED,
                                    offset=2)
    torch.cuda.synchronize()
    for got, want, what in ((qr.q, r1.q, "row codes"), (qr.scales, r1.scales, "row scales"),
                            (qc.q, c1.q, "col codes"), (qc.scales, c1.scales, "col scales"),
                            (qr.tensor_scale, r1.tensor_scale, "row ts"), (qc.tensor_scale, c1.tensor_scale, "col ts")):
        assert torch.equal(got, want), what
    a = oracle.amax(x)
    g = oracle.tensor_scale(a, "e4m3")
    assert_bytes_equal(f32_bits(host(qr.tensor_scale)), f32_bits([g, a]), "grads ts")
    xt = np.ascontiguousarray(x.T)
    for i in (0, 1, 4095, 8191):
        q, s = oracle.quantize(x, 16, "e4m3", g, stochastic=True, seed=0x5EED, offset=2, rows=(i, i + 1))
        assert_bytes_equal(host(qr.q[i:i + 1]), q, f"grads row {i}")
        assert_bytes_equal(host(qr.scales[i:i + 1]), s, f"grads row {i} scales")
        q, s = oracle.quantize(xt, 16, "e4m3", g, stochastic=True, seed=0x5EED, offset=2, rows=(i, i + 1))
        assert_bytes_equal(host(qc.q[i:i + 1]), q, f"grads col {i}")
        assert_bytes_equal(host(qc.scales[i:i + 1]), s, f"grads col {i} scales")
    assert st.get()[0] == 1


def test_both_reused_transformed_output_and_mismatch():
    """A reused output that carried the Hadamard transform is quantized
    without it (the two-orientation call takes no transform; the library's
    own UNSUPPORTED for a transformed operand is checked through the ABI on
    the CPU)."""
    x = _like(64, 64, 62)
    xd = to_device(x)
    qr, qc = fq.fp4_quantize_both(xd, 16, "e4m3", out=(fq.QTensor.empty(64, 64, 16, "e4m3"),
                                                       fq.QTensor.empty(64, 64, 16, "e4m3", transform="rht",
                                                                        rht_signs=3)))
    torch.cuda.synchronize()
    assert qc.transform == "none" and qc.rht_signs == 0
    q, s, g, a = oracle.quantize_transposed_tensor(x, 16, "e4m3", "current", nthreads=8)
    assert_bytes_equal(host(qc.q), q, "reused colwise codes")
    assert_bytes_equal(host(qc.scales), s, "reused colwise scales")
    # a column-wise output of the wrong shape: the binding refuses it before
    # the call (the library's own SHAPE status is checked through the ABI
    # on the CPU)
    with pytest.raises(ValueError):
        fq.fp4_quantize_both(xd, 16, "e4m3", out=(fq.QTensor.empty(64, 64, 16, "e4m3"),
                                                  fq.QTensor.empty(32, 64, 16, "e4m3")))


def test_both_empty_and_tiny():
    for shape in [(0, 64), (64, 0), (32, 32)]:
        x = np.zeros(shape, dtype=np.float32)
        if shape == (32, 32):
            x = _like(32, 32, 63, "f32")
        _check_both(x, 16, "e4m3", "current", tag=f"both {shape}")


def test_both_strided_rows():
    """A row stride larger than the row (a column slice of a wider tensor):
    both outputs as for the contiguous tensor."""
    x = _like(96, 128, 64)
    big = np.zeros((96, 200), dtype=np.uint16)
    big[:, :128] = x
    xd = to_device(big)[:, :128]
    assert xd.stride(0) == 200
    st = fq.AmaxState(1)
    qr, qc = fq.fp4_quantize_both(xd, 16, "e4m3", rounding="stochastic", state=st, seed=4, offset=8)
    torch.cuda.synchronize()
    q, s, g, a = oracle.quantize_tensor(x, 16, "e4m3", "current", stochastic=True, seed=4, offset=8)
    assert_bytes_equal(host(qr.q), q, "strided both row codes")
    assert_bytes_equal(host(qr.scales), s, "strided both row scales")
    q, s, g, a = oracle.quantize_transposed_tensor(x, 16, "e4m3", "current", stochastic=True, seed=4, offset=8)
    assert_bytes_equal(host(qc.q), q, "strided both col codes")
    assert_bytes_equal(host(qc.scales), s, "strided both col scales")
