"""The hardware E2M1 pack (round to nearest even, saturating, sign kept)
against the oracle's brute-force nearest search, through the quantizer.

Every block of 32 fp32 elements carries an anchor in [4, 8), so its E8M0
scale is exactly 1 and the quantizer encodes the inputs themselves.  The
probes: every binary32 value within 4096 ulps of each E2M1 grid point and
each midpoint between neighbours (both signs), the values just below 8, and
a strided sweep of all binary32 patterns in [0, 8) (subnormals included),
both signs.  (gonzo_ML/3986 "Стохастическая квантизация": round to the
nearest grid value; the tie and saturation rules are the readings stated in
the oracle.)
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_bytes_equal, host

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp4_block_scaled_quantize_amd")


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _probes():
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    pts = []
    for c in grid + mids + [8.0]:
        b = np.float32(c).view(np.uint32).astype(np.int64)
        k = np.arange(-4096, 4097, dtype=np.int64)
        bits = b + k
        bits = bits[(bits >= 0)]
        pts.append(bits.astype(np.uint32).view(np.float32))
    strided = np.arange(0, np.float32(8.0).view(np.uint32), 997, dtype=np.uint32).view(np.float32)
    v = np.concatenate(pts + [strided])
    v = v[np.abs(v) < 8.0]
    return np.concatenate([v, -v]).astype(np.float32)


def test_e2m1_pack_every_probe():
    v = _probes()
    n = v.size
    nblk = -(-n // 31)
    blocks = np.zeros((nblk, 32), dtype=np.float32)
    blocks[:, 0] = np.float32(4.0)                        # E8M0 code 127: scale 1
    flat = np.zeros(nblk * 31, dtype=np.float32)
    flat[:n] = v
    blocks[:, 1:] = flat.reshape(nblk, 31)
    cols = 4096
    rows = -(-nblk * 32 // cols)
    x = np.zeros(rows * cols, dtype=np.float32)
    x[:nblk * 32] = blocks.reshape(-1)
    x[nblk * 32:] = np.float32(4.0)
    x = x.reshape(rows, cols)
    print(f"E2M1 sweep: {n} probes in a {rows}x{cols} fp32 tensor", flush=True)
    qt = fq.fp4_quantize(torch.from_numpy(x).cuda(), 32, "e8m0", amax="none")
    torch.cuda.synchronize()
    q, s = oracle.quantize(x, 32, "e8m0", 1.0, nthreads=8)
    assert np.all(s == 127)
    assert_bytes_equal(host(qt.scales), s, "scales")
    assert_bytes_equal(host(qt.q), q, "codes")
    # and the oracle's codes are the nearest-even rule written out here
    mag = oracle.e2m1_rtn_array(np.abs(v))
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    a = np.abs(v.astype(np.float64))
    d = np.abs(a[:, None] - grid[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    want = np.where(cand.sum(axis=1) == 1, cand.argmax(axis=1), even.argmax(axis=1))
    want = np.where(a >= 6.0, 7, want)
    assert np.array_equal(mag, want)
