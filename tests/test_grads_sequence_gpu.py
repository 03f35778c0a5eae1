"""The backward-pass gradient workload at full size, as a sequence: 8192 x
8192 bf16 Laplace(0, 1e-4) gradients drawn on the host (tensor t from its own
seed), NVFP4 block 16 with E4M3 scales, stochastic rounding from Philox with
offset t, and the tensor maximum refreshed every 50 calls from the current
tensor and stored in between (ue5m3-fp4-pretraining "Что сделали";
gonzo_ML/3986 "Стохастическая квантизация").  Calls 0 .. 51 cross the
refresh at call 50.  Every call's tensor scale is checked bit for bit, and
the codes and scales of sampled rows (first, last and six drawn rows per
call) against the oracle, which quantizes those rows of the same tensor with
the same counters.
"""
import numpy as np
import pytest
import torch

import fp4_inputs as inputs
import oracle
from tests.gpu_util import assert_bytes_equal, f32_bits, host, to_device

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp4_block_scaled_quantize_amd")

SEED = 0x5EED
CALLS = 52


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("orientation", ["rowwise"])
def test_grads_sequence_refresh_at_50(orientation):
    st = fq.AmaxState(50)
    ost = oracle.AmaxState(interval=50)
    rng = np.random.default_rng(7)
    xd = torch.empty((8192, 8192), dtype=torch.bfloat16, device="cuda")
    out = fq.QTensor.empty(8192, 8192, 16, "e4m3", "stochastic", "delayed", device="cuda")
    saturated_calls = 0
    for t in range(CALLS):
        x = inputs.grads(t)
        xd.copy_(to_device(x))
        fq.fp4_quantize(xd, 16, "e4m3", rounding="stochastic", amax="delayed", state=st, seed=SEED, offset=t,
                        out=out)
        torch.cuda.synchronize()
        g, a = oracle.resolve_tensor_scale(x, "e4m3", "delayed", ost)
        assert_bytes_equal(f32_bits(host(out.tensor_scale)), f32_bits([g, a]), f"call {t} tensor_scale")
        rows = sorted({0, 8191} | set(rng.integers(0, 8192, 6).tolist()))
        for r in rows:
            q, s = oracle.quantize(x, 16, "e4m3", g, stochastic=True, seed=SEED, offset=t, rows=(r, r + 1))
            assert_bytes_equal(host(out.q[r:r + 1]), q, f"call {t} row {r} codes")
            assert_bytes_equal(host(out.scales[r:r + 1]), s, f"call {t} row {r} scales")
        if oracle.amax(x) > a:
            saturated_calls += 1
        print(f"grads sequence call {t}: amax used {a:.6g}, rows {rows} exact", flush=True)
    calls, stored = st.get()
    assert calls == CALLS and np.float32(stored) == np.float32(ost.amax)
    print(f"calls whose tensor outgrew the stored maximum: {saturated_calls}", flush=True)
