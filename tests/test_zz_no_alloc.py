"""fp4_quantize_noalloc through the C ABI against fp4_quantize (with its own
amax state) on the same inputs: codes, scales and tensor scale byte for
byte, on calls in a row with shrinking inputs (the static workspace keeps
the previous call's contents), covering the two-pass refresh, the
single-pass refresh, stochastic rounding, the transform and no tensor
scale.  The noalloc calls get preallocated outputs; the library allocates
nothing for them."""
import ctypes

import numpy as np
import pytest
import torch

import fp4_inputs as inputs
from tests.gpu_util import assert_bytes_equal, host, to_device

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp4_block_scaled_quantize_amd")


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _x(rows, cols, seed, dtype):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    x[rng.random((rows, cols)) < 0.001] *= 100
    return inputs.f32_to_bf16_bits(x) if dtype == "bf16" else x


CASES = [  # rows, cols, dtype, block, scale, policy, rounding, rht
    (4104, 4096, "bf16", 16, "e4m3", "current", "nearest", None),        # two-pass refresh
    (4096, 4096, "bf16", 16, "e4m3", "current", "nearest", None),        # single pass, every CU
    (1000, 512, "f32", 32, "ue5m3", "current", "stochastic", None),      # single pass, fewer workgroups
    (640, 256, "bf16", 16, "e4m3", "current", "nearest", 0x2468ACE1),    # transform
    (96, 128, "bf16", 32, "e8m0", "none", "stochastic", None),           # no tensor scale
]


def _noalloc_c(x, out, seed, offset):
    tc = out.c()
    L = fq.lib()
    return L.fp4_quantize_noalloc(x.data_ptr(), fq.DTYPE[x.dtype], x.stride(0), ctypes.byref(tc), seed, offset,
                                  torch.cuda.current_stream().cuda_stream)


def test_noalloc_matches_quantize_on_shrinking_calls():
    for i, (rows, cols, dtype, block, scale, pol, rnd, rht) in enumerate(CASES):
        print(f"noalloc call {i}: {rows}x{cols} {dtype} {scale}/{block} {pol} {rnd} rht={rht}", flush=True)
        xd = to_device(_x(rows, cols, 50 + i, dtype))
        ref = fq.fp4_quantize(xd, block, scale, rounding=rnd, amax=pol,
                              state=fq.AmaxState(1) if pol == "current" else None, seed=77, offset=i,
                              rht_signs=rht)
        out = fq.QTensor.empty(rows, cols, block, scale, rnd, pol, device="cuda",
                               transform="none" if rht is None else "rht", rht_signs=rht or 0)
        out.q.fill_(0xAB)
        out.scales.fill_(0xCD)
        out.tensor_scale.fill_(-1.0)
        torch.cuda.synchronize()
        assert _noalloc_c(xd, out, 77, i) == 0
        torch.cuda.synchronize()
        tag = f"call {i}"
        assert_bytes_equal(host(out.q), host(ref.q), f"{tag} codes")
        assert_bytes_equal(host(out.scales), host(ref.scales), f"{tag} scales")
        assert_bytes_equal(host(out.tensor_scale).view(np.uint32), host(ref.tensor_scale).view(np.uint32),
                           f"{tag} tensor scale")


def test_noalloc_rejects_delayed_and_binding():
    xd = to_device(_x(64, 64, 3, "bf16"))
    out = fq.QTensor.empty(64, 64, 16, "e4m3", "nearest", "delayed", device="cuda")
    assert _noalloc_c(xd, out, 0, 0) == -2
    # the binding form, twice in a row with a smaller second input
    for rows in (256, 128):
        x = to_device(_x(rows, 256, 4 + rows, "bf16"))
        o = fq.QTensor.empty(rows, 256, 16, "e4m3", device="cuda")
        fq.fp4_quantize_noalloc(x, o, 16, "e4m3")
        ref = fq.fp4_quantize(x, 16, "e4m3", state=fq.AmaxState(1))
        torch.cuda.synchronize()
        assert_bytes_equal(host(o.q), host(ref.q), f"binding {rows} codes")
        assert_bytes_equal(host(o.scales), host(ref.scales), f"binding {rows} scales")
