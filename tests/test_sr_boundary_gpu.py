"""Stochastic rounding at its decision boundaries, on every E2M1 path.

The reading (gonzo_ML/3986 "Стохастическая квантизация": up or down with a
probability set by the distance) rounds |v| up from its lower grid
neighbour iff r16 / 2^16 < frac.  Here every element's value is placed next
to its own decision boundary: with the element's Philox bits r16 (the
oracle's generator), x = lo + (r16 + d) / 2^16 * (hi - lo) rounded to
binary32, for offsets d just below, at and just above 0, in every binade of
the grid, plus values next to multiples of 2^-17 and subnormals.  Every
block of 32 holds an anchor 4.0, so its E8M0 scale is 1 and the quantizer
rounds x itself.  Row-wise, column-wise (the index of x^T) and the
two-orientation kernel's row-wise output must equal the oracle bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_bytes_equal, host

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp4_block_scaled_quantize_amd")

SEED, OFFSET = 0x5EED, 7
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
OFFS = np.array([0.0, 2.0 ** -7, -2.0 ** -7, 2.0 ** -17, -2.0 ** -17, 0.5, 2.0 ** -12, -0.25])


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _boundary_tensor(rows, cols, seed, offset):
    """rows x cols fp32 (row-major SR index i = r * cols + c), every value at
    its element's decision boundary."""
    n = rows * cols
    r16 = oracle.sr_bits_array(seed, offset, 0, n).astype(np.float64)
    i = np.arange(n)
    b = i % 7                                      # binade: lo = GRID[b], hi = GRID[b + 1]
    lo, hi = GRID[b], GRID[b + 1]
    d = OFFS[(i // 7) % len(OFFS)]
    t = np.clip((r16 + d) / 65536.0, 0.0, 1.0 - 2.0 ** -30)
    x = lo + t * (hi - lo)
    sign = np.where((i // 56) % 2 == 1, -1.0, 1.0)
    x = (sign * x).astype(np.float32)
    tiny = (i % 97) == 5                           # values next to multiples of 2^-17, and subnormals
    k = (i % 127) + 1
    xt = (k * 2.0 ** -17 + np.where(i % 3 == 0, 2.0 ** -40, np.where(i % 3 == 1, -2.0 ** -40, 0.0)))
    x[tiny] = xt[tiny].astype(np.float32)
    sub = (i % 211) == 3
    x[sub] = (np.float32(2.0 ** -149) * (i[sub] % 50 + 1)).astype(np.float32)
    x = x.reshape(rows, cols)
    x[:, ::32] = np.float32(4.0)                    # anchors: E8M0 scale 1 for every block
    return x


def test_rowwise_sr_boundaries():
    x = _boundary_tensor(256, 1024, SEED, OFFSET)
    qt = fq.fp4_quantize(torch.from_numpy(x).cuda(), 32, "e8m0", rounding="stochastic", amax="none", seed=SEED,
                         offset=OFFSET)
    torch.cuda.synchronize()
    q, s = oracle.quantize(x, 32, "e8m0", 1.0, stochastic=True, seed=SEED, offset=OFFSET, nthreads=8)
    assert np.all(s == 127)
    assert_bytes_equal(host(qt.scales), s, "row-wise scales")
    assert_bytes_equal(host(qt.q), q, "row-wise SR codes at the boundaries")


def test_colwise_sr_boundaries():
    # y is the tensor the column-wise call quantizes (x^T): build y with the
    # boundaries of its own indices, hand the call x = y^T
    y = _boundary_tensor(256, 1024, SEED, OFFSET + 1)
    x = np.ascontiguousarray(y.T)
    qt = fq.fp4_quantize_transposed(torch.from_numpy(x).cuda(), 32, "e8m0", rounding="stochastic", amax="none",
                                    seed=SEED, offset=OFFSET + 1)
    torch.cuda.synchronize()
    q, s = oracle.quantize(y, 32, "e8m0", 1.0, stochastic=True, seed=SEED, offset=OFFSET + 1, nthreads=8)
    assert_bytes_equal(host(qt.scales), s, "column-wise scales")
    assert_bytes_equal(host(qt.q), q, "column-wise SR codes at the boundaries")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_both_orientations_rowwise_sr_boundaries(dtype):
    x = _boundary_tensor(256, 512, SEED, OFFSET + 2)
    if dtype == "bf16":
        from fp4_inputs import f32_to_bf16_bits
        xb = f32_to_bf16_bits(x)
        xd = torch.from_numpy(xb.view(np.int16).copy()).view(torch.bfloat16).cuda()
        xo = xb
    else:
        xd = torch.from_numpy(x).cuda()
        xo = x
    qr, qc = fq.fp4_quantize_both(xd, 32, "e8m0", rounding="stochastic", amax="none", seed=SEED, offset=OFFSET + 2)
    torch.cuda.synchronize()
    q, s, _, _ = oracle.quantize_tensor(xo, 32, "e8m0", "none", stochastic=True, seed=SEED, offset=OFFSET + 2,
                                        nthreads=8)
    assert_bytes_equal(host(qr.q), q, f"{dtype} both-call row-wise SR codes")
    q2, s2, _, _ = oracle.quantize_transposed_tensor(xo, 32, "e8m0", "none", stochastic=True, seed=SEED,
                                                     offset=OFFSET + 2, nthreads=8)
    assert_bytes_equal(host(qc.q), q2, f"{dtype} both-call column-wise SR codes")
