"""GPU parity of column-wise (transposed) quantization against the CPU oracle.

fp4_quantize_transposed(x) must equal, bit for bit, the oracle's quantization
of x^T: codes, scales and tensor scale, round-to-nearest and stochastic
rounding (counter index of x^T), every scale format, ragged tiles, strided
rows, the delayed amax policy, and the 8192^2 gradient workload on sampled
output rows.  Every call goes through the C ABI.
"""
import numpy as np
import pytest
import torch

import fp4_inputs as inputs
import oracle
from tests.gpu_util import assert_bytes_equal, f32_bits, host, to_device

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp4_block_scaled_quantize_amd")

ALL_FMTS = ["e4m3", "ue5m3", "e3m4", "e1m6", "e2m5", "e5m2", "e6m1", "e7m0", "e8m0"]


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


def _check_t(x_np, block, fmt, policy, *, rounding="nearest", seed=0, offset=0, x_dev=None, state=None,
             ostate=None, tag=""):
    xd = to_device(x_np) if x_dev is None else x_dev
    if state is None and policy == "current":
        state = fq.AmaxState(1)
    qt = fq.fp4_quantize_transposed(xd, block=block, scale=fmt, rounding=rounding, amax=policy, state=state,
                                    seed=seed, offset=offset)
    torch.cuda.synchronize()
    q, s, g, a = oracle.quantize_transposed_tensor(x_np, block, fmt, policy, state=ostate,
                                                   stochastic=(rounding == "stochastic"), seed=seed,
                                                   offset=offset, nthreads=8)
    assert (qt.rows, qt.cols) == (x_np.shape[1], x_np.shape[0])
    assert_bytes_equal(host(qt.scales), s, f"{tag} scales")
    assert_bytes_equal(host(qt.q), q, f"{tag} codes")
    assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([g, a]), f"{tag} tensor_scale")
    return qt


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("block", [16, 32])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_transposed_formats_ragged(fmt, block, dtype):
    # 352 rows = one whole and one partial 256-row tile; 136 columns = two
    # whole and one partial 64-column tile
    x = _like(352, 136, 200 + block, dtype)
    _check_t(x, block, fmt, _policy(fmt), tag=f"T {fmt}/{block}/{dtype}")
    if fmt != "e8m0":
        _check_t(x, block, fmt, "none", tag=f"T {fmt}/{block}/{dtype}/none")


@pytest.mark.parametrize("seed,offset", [(0, 0), (0x5EED, 7), (0xFFFFFFFF12345678, 2**40 + 3)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("block,fmt", [(16, "e4m3"), (32, "e8m0")])
def test_transposed_stochastic_parity(seed, offset, dtype, block, fmt):
    x = _like(544, 200, 31, dtype)
    _check_t(x, block, fmt, _policy(fmt), rounding="stochastic", seed=seed, offset=offset, tag="T sr")


def test_transposed_small_fp32_outliers():
    """The 256x256 fp32 N(0,1) matrix with 1% x50 outliers, E4M3 block 16."""
    _check_t(inputs.small_b(), 16, "e4m3", "current", tag="T small_b")


def test_transposed_strided_rows():
    x = _like(96, 128, 9)
    big = np.zeros((96, 200), dtype=np.uint16)
    big[:, :128] = x
    xd = to_device(big)[:, :128]
    assert xd.stride(0) == 200
    _check_t(x, 16, "e4m3", "current", x_dev=xd, tag="T strided")
    _check_t(x, 16, "e4m3", "current", rounding="stochastic", seed=5, offset=2, x_dev=xd, tag="T strided sr")


def test_transposed_sweep_full_size():
    """The 4096x4096 bf16 sweep tensor, E4M3 block 16 with current amax and
    E8M0 block 32, every byte."""
    x = inputs.sweep()
    _check_t(x, 16, "e4m3", "current", tag="T sweep e4m3")
    _check_t(x, 32, "e8m0", "none", tag="T sweep e8m0")


def test_transposed_delayed_sequence():
    """Delayed amax (interval 3) through the transposed path: refreshes on
    calls 0, 3, 6; a tensor that outgrew the stored maximum saturates."""
    st = fq.AmaxState(3)
    ost = oracle.AmaxState(interval=3)
    for t in range(8):
        x = _like(64, 48, 500 + t)
        if t == 1:
            x = inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(x) * np.float32(10.0))
        _check_t(x, 16, "e4m3", "delayed", rounding="stochastic", seed=0x5EED, offset=t, state=st, ostate=ost,
                 tag=f"T delayed call {t}")
    calls, amax = st.get()
    assert calls == 8 and amax == ost.amax


def test_transposed_grads_full_size_sampled_rows():
    """8192x8192 bf16 Laplace(1e-4) gradients, column-wise with SR (Philox
    seed/offset) and delayed amax: tensor scale over the whole tensor, codes
    and scales on sampled output rows (columns of the gradient)."""
    x = inputs.grads(0)
    st = fq.AmaxState(50)
    qt = fq.fp4_quantize_transposed(to_device(x), 16, "e4m3", rounding="stochastic", amax="delayed", state=st,
                                    seed=0x5EED, offset=0)
    torch.cuda.synchronize()
    a = oracle.amax(x)
    g = oracle.tensor_scale(a, "e4m3")
    assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([g, a]), "T grads tensor_scale")
    rng = np.random.default_rng(1)
    cols = sorted(set(rng.integers(0, 8192, 24).tolist()) | {0, 63, 64, 8191})
    xt = np.ascontiguousarray(x.T)
    for c in cols:
        q, s = oracle.quantize(xt, 16, "e4m3", g, stochastic=True, seed=0x5EED, offset=0, rows=(c, c + 1))
        assert_bytes_equal(host(qt.q[c:c + 1]), q, f"T grads col {c} codes")
        assert_bytes_equal(host(qt.scales[c:c + 1]), s, f"T grads col {c} scales")


def test_transposed_matches_rowwise_of_materialized_transpose():
    """Property at any size: the column-wise call equals the row-wise call on
    the contiguous transpose, SR included (same counters)."""
    x = torch.randn(1024, 520, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    a = fq.fp4_quantize_transposed(x, 16, "e4m3", rounding="stochastic", seed=77, offset=4)
    b = fq.fp4_quantize(x.t().contiguous(), 16, "e4m3", rounding="stochastic", seed=77, offset=4)
    torch.cuda.synchronize()
    assert torch.equal(a.q, b.q) and torch.equal(a.scales, b.scales)
    assert torch.equal(a.tensor_scale, b.tensor_scale)


def test_transposed_edge_values():
    """Zeros, signed zeros, midpoints, saturation and subnormals, laid out
    down the columns."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 7.99]
    col = [4.0] + mids + [-m for m in mids] + [0.0, -0.0, 1e-30, -1e-30, 0.5, 3.0, -6.0, 2.0, 1.0, 0.1, 0.9]
    cols = [col[:32], [0.0] * 32, [-0.0] * 32, [1e-40, -3e-42, 1e-45] + [0.0] * 29, [1e30] + [1e-30] * 31,
            [3e38, -3e38] + [1.0] * 30, [0.37] * 32, [-2.5] * 32]
    x = np.array(cols, dtype=np.float32).T.copy()          # [32, 8]
    x = np.concatenate([x, x * np.float32(1e-20), x * np.float32(0.37)], axis=0)   # [96, 8]
    for fmt, block in [("e8m0", 32), ("e4m3", 16), ("e1m6", 16), ("ue5m3", 32), ("e7m0", 16)]:
        for pol in (["none"] if fmt == "e8m0" else ["none", "current"]):
            _check_t(x, block, fmt, pol, tag=f"T edge {fmt} {pol}")
            _check_t(x, block, fmt, pol, rounding="stochastic", seed=3, offset=1, tag=f"T edge sr {fmt} {pol}")


def test_transposed_empty():
    for shape in [(0, 64), (64, 0)]:
        xd = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
        qt = fq.fp4_quantize_transposed(xd, 16, "e4m3", amax="current")
        torch.cuda.synchronize()
        assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([1.0, 0.0]), f"T empty {shape}")
