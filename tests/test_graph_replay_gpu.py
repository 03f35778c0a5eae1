"""Column-wise, two-orientation and Hadamard-transformed quantize calls
captured once in a HIP graph and replayed with new input values (eager
copies and synchronizations between replays): every replay agrees with the
oracle, the current-amax refreshes included (the captured amax kernel and
its partials run again on every replay)."""
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


def _like(rows, cols, seed, scale):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * 0.02 * scale).astype(np.float32)
    return inputs.f32_to_bf16_bits(x)


def test_graph_replay_transposed_both_and_transform():
    R, C = 320, 192
    x = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    x.zero_()
    st_t, st_b, st_r = fq.AmaxState(1), fq.AmaxState(1), fq.AmaxState(1)
    out_t = fq.QTensor.empty(C, R, 16, "e4m3", rounding="stochastic")
    out_b = (fq.QTensor.empty(R, C, 16, "e4m3"), fq.QTensor.empty(C, R, 16, "e4m3"))
    out_r = fq.QTensor.empty(R, C, 32, "e8m0", amax="none")
    signs = 0x2468ACE1

    def record():
        fq.fp4_quantize_transposed(x, 16, "e4m3", rounding="stochastic", state=st_t, seed=7, offset=3, out=out_t)
        fq.fp4_quantize_both(x, 16, "e4m3", state=st_b, out=out_b)
        fq.fp4_quantize(x, 32, "e8m0", amax="none", rht_signs=signs, out=out_r)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        record()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        record()
    torch.cuda.synchronize()
    for rep in range(4):
        h = _like(R, C, 5000 + rep, 10.0 ** (rep - 1))
        x.copy_(to_device(h))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        q, s, g, a = oracle.quantize_transposed_tensor(h, 16, "e4m3", "current", stochastic=True, seed=7, offset=3)
        assert_bytes_equal(host(out_t.q), q, f"replay {rep} transposed codes")
        assert_bytes_equal(host(out_t.scales), s, f"replay {rep} transposed scales")
        assert_bytes_equal(f32_bits(host(out_t.tensor_scale)), f32_bits([g, a]), f"replay {rep} transposed ts")
        q, s, g, a = oracle.quantize_tensor(h, 16, "e4m3", "current")
        assert_bytes_equal(host(out_b[0].q), q, f"replay {rep} both row codes")
        assert_bytes_equal(host(out_b[0].scales), s, f"replay {rep} both row scales")
        q, s, g, a = oracle.quantize_transposed_tensor(h, 16, "e4m3", "current")
        assert_bytes_equal(host(out_b[1].q), q, f"replay {rep} both col codes")
        assert_bytes_equal(f32_bits(host(out_b[1].tensor_scale)), f32_bits([g, a]), f"replay {rep} both ts")
        q, s, _, _ = oracle.quantize_tensor(h, 32, "e8m0", "none", rht_signs=signs)
        assert_bytes_equal(host(out_r.q), q, f"replay {rep} transform codes")
        assert_bytes_equal(host(out_r.scales), s, f"replay {rep} transform scales")
