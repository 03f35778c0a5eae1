"""The single-pass refresh without co-residency: workgroups that give up
waiting for the others read the whole tensor themselves.

The wait bound is forced to zero from the host (fp4_set_exchange_wait), so
almost every workgroup takes that path; every kernel still exits normally.
Codes, scales and the tensor scale must still equal the oracle's bit for
bit, and later calls on the same state (with the bound restored) must not
see any word the forced calls left behind (the epoch protocol).
ue5m3-fp4-pretraining "Что сделали": the tensor maximum of the call, or the
one stored at the last refresh, sets the tensor scale.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_bytes_equal, f32_bits, host, to_device

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp4_block_scaled_quantize_amd")


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture
def zero_wait():
    prev = fq.set_exchange_wait(0)
    try:
        yield
    finally:
        fq.set_exchange_wait(prev)


def _tensor(rows, cols, seed, where, dtype="bf16"):
    """Sweep-like values with the maximum placed in the first, middle or last
    workgroup's share of the tensor."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    r = {"first": 3, "mid": rows // 2 + 1, "last": rows - 2}[where]
    x[r, cols // 3] = np.float32(-7.5 if seed % 2 else 9.25)
    if dtype == "bf16":
        from fp4_inputs import f32_to_bf16_bits
        return f32_to_bf16_bits(x)
    return x


def _check(qt, x_np, block, fmt, policy, state_o=None, rht=None, tag=""):
    q, s, g, a = oracle.quantize_tensor(x_np, block, fmt, policy, state=state_o, nthreads=8, rht_signs=rht)
    assert_bytes_equal(host(qt.scales), s, f"{tag} scales")
    assert_bytes_equal(host(qt.q), q, f"{tag} codes")
    assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([g, a]), f"{tag} tensor_scale")


def test_forced_fallback_is_exact(zero_wait):
    st = fq.AmaxState(1)
    for i, (where, block, fmt) in enumerate([("last", 16, "e4m3"), ("first", 32, "ue5m3"), ("mid", 16, "e3m4")]):
        x_np = _tensor(4096, 4096, 10 + i, where)
        print(f"forced fallback: 4096x4096 bf16 {fmt} block {block}, max in the {where} share", flush=True)
        qt = fq.fp4_quantize(to_device(x_np), block, fmt, amax="current", state=st)
        torch.cuda.synchronize()
        _check(qt, x_np, block, fmt, "current", tag=f"{fmt}/{where}")
    assert st.fallbacks() > 0


def test_forced_fallback_transform_and_strided(zero_wait):
    st = fq.AmaxState(1)
    x_np = _tensor(2048, 4096, 21, "last", dtype="f32")
    xd = torch.zeros((2048, 4160), dtype=torch.float32, device="cuda")
    xd[:, :4096] = torch.from_numpy(x_np).cuda()
    print("forced fallback: 2048x4096 fp32 strided rows, E4M3 block 16", flush=True)
    qt = fq.fp4_quantize(xd[:, :4096], 16, "e4m3", amax="current", state=st)
    torch.cuda.synchronize()
    _check(qt, x_np, 16, "e4m3", "current", tag="strided")
    x2 = _tensor(1024, 4096, 22, "mid")
    print("forced fallback: 1024x4096 bf16 with the Hadamard transform, block 32", flush=True)
    qt = fq.fp4_quantize(to_device(x2), 32, "e4m3", amax="current", state=st, rht_signs=0x9E3779B9)
    torch.cuda.synchronize()
    _check(qt, x2, 32, "e4m3", "current", rht=0x9E3779B9, tag="rht")
    assert st.fallbacks() > 0


def test_epochs_survive_forced_fallbacks():
    """Alternate forced-fallback calls and normal calls on one state, with the
    maximum in a different share each time and decreasing, so a stale word
    from an earlier call would raise the tensor maximum of a later one."""
    st = fq.AmaxState(1)
    for i in range(8):
        x_np = _tensor(4096, 4096, 30 + i, ("last", "first", "mid")[i % 3])
        x_np = (x_np.astype(np.uint32) << 16).view(np.float32)          # bf16 bits -> f32 values
        x_np = x_np * np.float32(1.0 / (1 + i))
        forced = i % 2 == 0
        prev = fq.set_exchange_wait(0) if forced else None
        try:
            print(f"epoch sequence call {i}: forced={forced}", flush=True)
            qt = fq.fp4_quantize(to_device(x_np), 16, "e4m3", amax="current", state=st)
            torch.cuda.synchronize()
        finally:
            if forced:
                fq.set_exchange_wait(prev)
        _check(qt, x_np, 16, "e4m3", "current", tag=f"call {i}")
    n = st.fallbacks()
    print(f"fallbacks: {n}", flush=True)
    assert n > 0
