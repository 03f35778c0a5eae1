"""Column-wise, two-orientation, Hadamard-transformed and 8- / 6-bit grid
quantize calls, the small NVFP4 / MXFP4 configuration, GEMMs and dequantize
calls
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


WIDE = ["fp8_e4m3", "int8", "fp6_e2m3", "fp6_e3m2", "int6"]


def test_graph_replay_wide_grids_gemm_and_dequantize():
    """The 8- and 6-bit grids in one captured graph: single-pass current-amax
    quantize calls (the grid exchange's epoch advances on every replay),
    GEMMs of two MXFP8 operands and of two INT8 operands with E4M3 block-16
    scales quantized in the same graph, and a dequantize of an MXFP6 tensor;
    each replay with new input values agrees with the oracle."""
    R, C, N = 96, 256, 72
    x = torch.zeros((R, C), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((N, C), dtype=torch.bfloat16, device="cuda")
    states = {e: fq.AmaxState(1) for e in WIDE}
    outs = {e: fq.QTensor.empty(R, C, 16, "e4m3", element=e) for e in WIDE}
    qa = fq.QTensor.empty(R, C, 32, "e8m0", amax="none", element="fp8_e4m3")
    qw = fq.QTensor.empty(N, C, 32, "e8m0", amax="none", element="fp8_e4m3")
    q6 = fq.QTensor.empty(R, C, 32, "e8m0", amax="none", element="fp6_e3m2")
    st_a8, st_w8 = fq.AmaxState(1), fq.AmaxState(1)
    qa8 = fq.QTensor.empty(R, C, 16, "e4m3", element="int8")
    qw8 = fq.QTensor.empty(N, C, 16, "e4m3", element="int8")
    c = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
    c8 = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((R, C), dtype=torch.float32, device="cuda")

    def record():
        for e in WIDE:
            fq.fp4_quantize(x, 16, "e4m3", state=states[e], out=outs[e], element=e)
        fq.fp4_quantize(x, 32, "e8m0", amax="none", out=qa, element="fp8_e4m3")
        fq.fp4_quantize(w, 32, "e8m0", amax="none", out=qw, element="fp8_e4m3")
        fq.fp4_gemm(qa, qw, out=c)
        fq.fp4_quantize(x, 16, "e4m3", state=st_a8, out=qa8, element="int8")
        fq.fp4_quantize(w, 16, "e4m3", state=st_w8, out=qw8, element="int8")
        fq.fp4_gemm(qa8, qw8, out=c8)
        fq.fp4_quantize(x, 32, "e8m0", amax="none", out=q6, element="fp6_e3m2")
        fq.fp4_dequantize(q6, torch.float32, out=y)
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
        hx = _like(R, C, 6000 + rep, 10.0 ** (rep - 1))
        hw = _like(N, C, 7000 + rep, 1.0)
        x.copy_(to_device(hx))
        w.copy_(to_device(hw))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for e in WIDE:
            q, s, g, a = oracle.quantize_tensor(hx, 16, "e4m3", "current", elem=e)
            assert_bytes_equal(host(outs[e].q), q, f"replay {rep} {e} codes")
            assert_bytes_equal(host(outs[e].scales), s, f"replay {rep} {e} scales")
            assert_bytes_equal(f32_bits(host(outs[e].tensor_scale)), f32_bits([g, a]), f"replay {rep} {e} ts")
        oa = oracle.quantize_tensor(hx, 32, "e8m0", "none", elem="fp8_e4m3")
        ow = oracle.quantize_tensor(hw, 32, "e8m0", "none", elem="fp8_e4m3")
        a_hat = oracle.dequantize_f64(oa[0], oa[1], oa[2], 32, "e8m0", elem="fp8_e4m3")
        w_hat = oracle.dequantize_f64(ow[0], ow[1], ow[2], 32, "e8m0", elem="fp8_e4m3")
        cref, tol = oracle.gemm_ref(a_hat, w_hat)
        ok = oracle.gemm_check(c.float().cpu().numpy().astype(np.float64), cref, tol)
        assert ok.all(), f"replay {rep} gemm: {int((~ok).sum())} outputs out of tolerance"
        oa = oracle.quantize_tensor(hx, 16, "e4m3", "current", elem="int8")
        ow = oracle.quantize_tensor(hw, 16, "e4m3", "current", elem="int8")
        assert_bytes_equal(host(qa8.q), oa[0], f"replay {rep} int8 a codes")
        assert_bytes_equal(host(qw8.q), ow[0], f"replay {rep} int8 w codes")
        a_hat = oracle.dequantize_f64(oa[0], oa[1], oa[2], 16, "e4m3", elem="int8")
        w_hat = oracle.dequantize_f64(ow[0], ow[1], ow[2], 16, "e4m3", elem="int8")
        cref, tol = oracle.gemm_ref(a_hat, w_hat)
        ok = oracle.gemm_check(c8.float().cpu().numpy().astype(np.float64), cref, tol)
        assert ok.all(), f"replay {rep} int8 gemm: {int((~ok).sum())} outputs out of tolerance"
        q, s, g, _ = oracle.quantize_tensor(hx, 32, "e8m0", "none", elem="fp6_e3m2")
        want = oracle.dequantize(q, s, float(g), 32, "e8m0", out="f32", elem="fp6_e3m2")
        assert_bytes_equal(f32_bits(host(y)), f32_bits(want), f"replay {rep} fp6 dequant")


def test_graph_replay_small_configuration():
    """The small NVFP4 configuration captured once: the 256x256 and 64x256
    fp32 current-amax quantize calls (each fits one workgroup: no grid
    exchange), a 1024x512 call between them that exchanges on the same state,
    the small-product GEMM C = A B^T, and the same product of MXFP4 operands;
    every replay with new values (the maximum moving between the tensors)
    agrees with the oracle."""
    b = torch.zeros((256, 256), dtype=torch.float32, device="cuda")
    a = torch.zeros((64, 256), dtype=torch.float32, device="cuda")
    z = torch.zeros((1024, 512), dtype=torch.float32, device="cuda")
    st = fq.AmaxState(1)
    qb = fq.QTensor.empty(256, 256, 16, "e4m3")
    qa = fq.QTensor.empty(64, 256, 16, "e4m3")
    qz = fq.QTensor.empty(1024, 512, 16, "e4m3")
    mb = fq.QTensor.empty(256, 256, 32, "e8m0", amax="none")
    ma = fq.QTensor.empty(64, 256, 32, "e8m0", amax="none")
    c = torch.empty((64, 256), dtype=torch.bfloat16, device="cuda")
    cm = torch.empty((64, 256), dtype=torch.bfloat16, device="cuda")

    def record():
        fq.fp4_quantize(b, 16, "e4m3", state=st, out=qb)
        fq.fp4_quantize(z, 16, "e4m3", state=st, out=qz)
        fq.fp4_quantize(a, 16, "e4m3", state=st, out=qa)
        fq.fp4_gemm(qa, qb, out=c)
        fq.fp4_quantize(b, 32, "e8m0", amax="none", out=mb)
        fq.fp4_quantize(a, 32, "e8m0", amax="none", out=ma)
        fq.fp4_gemm(ma, mb, out=cm)
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
    rng = np.random.default_rng(77)
    for rep in range(4):
        hb = inputs.small_b() * np.float32(2.0 ** (rep - 2))
        ha = inputs.small_a() * np.float32(3.0 ** (1 - rep))
        hz = (rng.standard_normal((1024, 512)) * 10.0 ** (rep - 1)).astype(np.float32)
        b.copy_(torch.from_numpy(hb).cuda())
        a.copy_(torch.from_numpy(ha).cuda())
        z.copy_(torch.from_numpy(hz).cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        hats = {}
        for name, h, qt in (("b", hb, qb), ("z", hz, qz), ("a", ha, qa)):
            q, s, g, am = oracle.quantize_tensor(h, 16, "e4m3", "current", nthreads=8)
            assert_bytes_equal(host(qt.q), q, f"replay {rep} {name} codes")
            assert_bytes_equal(host(qt.scales), s, f"replay {rep} {name} scales")
            assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([g, am]), f"replay {rep} {name} ts")
            hats[name] = oracle.dequantize_f64(q, s, g, 16, "e4m3")
        cref, tol = oracle.gemm_ref(hats["a"], hats["b"])
        ok = oracle.gemm_check(c.float().cpu().numpy().astype(np.float64), cref, tol)
        assert ok.all(), f"replay {rep} nvfp4 gemm: {int((~ok).sum())} outputs out of tolerance"
        for h, qt, key in ((hb, mb, "mb"), (ha, ma, "ma")):
            q, s, g, _ = oracle.quantize_tensor(h, 32, "e8m0", "none", nthreads=8)
            assert_bytes_equal(host(qt.q), q, f"replay {rep} {key} codes")
            hats[key] = oracle.dequantize_f64(q, s, g, 32, "e8m0")
        cref, tol = oracle.gemm_ref(hats["ma"], hats["mb"])
        ok = oracle.gemm_check(cm.float().cpu().numpy().astype(np.float64), cref, tol)
        assert ok.all(), f"replay {rep} mxfp4 gemm: {int((~ok).sum())} outputs out of tolerance"
