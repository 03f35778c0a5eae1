"""GPU parity of quantize / dequantize / amax against the CPU oracle.

Codes, scales and the tensor scale must match bit for bit (round-to-nearest
and stochastic rounding), on small ragged shapes, on the 4096^2 scale-format
sweep at full size, and on sampled rows of the 8192^2 gradient workload.
Every call goes through the C ABI (fp4_block_scaled_quantize_amd binding).
"""
import numpy as np
import pytest
import torch

import fp4_inputs as inputs
import oracle
from tests.gpu_util import assert_bytes_equal, bf16_bits, f32_bits, host, to_device

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp4_block_scaled_quantize_amd")

ALL_FMTS = ["e4m3", "ue5m3", "e3m4", "e1m6", "e2m5", "e5m2", "e6m1", "e7m0", "e8m0"]


def _skip_no_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(autouse=True)
def _gpu():
    _skip_no_gpu()


def _policy(fmt, default="current"):
    return "none" if fmt == "e8m0" else default


def _check_quant(x_np, block, fmt, policy, *, rounding="nearest", seed=0, offset=0, x_dev=None, tag=""):
    """Quantize on the GPU and with the oracle; compare every byte."""
    xd = to_device(x_np) if x_dev is None else x_dev
    state = fq.AmaxState(1) if policy == "current" else None
    qt = fq.fp4_quantize(xd, block=block, scale=fmt, rounding=rounding, amax=policy, state=state,
                         seed=seed, offset=offset)
    torch.cuda.synchronize()
    q, s, g, a = oracle.quantize_tensor(x_np, block, fmt, policy, stochastic=(rounding == "stochastic"),
                                        seed=seed, offset=offset, nthreads=8)
    assert_bytes_equal(host(qt.scales), s, f"{tag} scales")
    assert_bytes_equal(host(qt.q), q, f"{tag} codes")
    ts = host(qt.tensor_scale)
    assert_bytes_equal(f32_bits(ts), f32_bits([g, a]), f"{tag} tensor_scale")
    return qt


def _sweep_like(rows, cols, seed, dtype="bf16"):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)) * 0.02
    m = rng.random((rows, cols)) < 0.001
    x[m] *= 100
    x = x.astype(np.float32)
    return inputs.f32_to_bf16_bits(x) if dtype == "bf16" else x


# ---------------------------------------------------------------------------
def test_small_nvfp4_fp32_outliers():
    """256x256 fp32 N(0,1) with 1% x50 outliers, E4M3 block 16, current amax."""
    b = inputs.small_b()
    _check_quant(b, 16, "e4m3", "current", tag="small_b")
    a = inputs.small_a()
    _check_quant(a, 16, "e4m3", "current", tag="small_a")


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("block", [16, 32])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_formats_ragged(fmt, block, dtype):
    x = _sweep_like(67, 320, 100 + block, dtype)
    _check_quant(x, block, fmt, _policy(fmt), tag=f"{fmt}/{block}/{dtype}")
    if fmt != "e8m0":
        _check_quant(x, block, fmt, "none", tag=f"{fmt}/{block}/{dtype}/none")


@pytest.mark.parametrize("fmt,block", [("e4m3", 16), ("ue5m3", 16), ("e3m4", 16), ("e1m6", 16), ("e8m0", 32)])
def test_sweep_full_size(fmt, block):
    """The 4096x4096 bf16 scale-format sweep at full size, every byte."""
    x = inputs.sweep()
    _check_quant(x, block, fmt, _policy(fmt), tag=f"sweep {fmt}")


def test_strided_rows_match_contiguous():
    x = _sweep_like(40, 256, 7)
    big = np.zeros((40, 384), dtype=np.uint16)
    big[:, :256] = x
    xd = to_device(big)[:, :256]
    assert xd.stride(0) == 384
    _check_quant(x, 16, "e4m3", "current", x_dev=xd, tag="strided")
    _check_quant(x, 16, "e4m3", "current", rounding="stochastic", seed=99, offset=3, x_dev=xd, tag="strided sr")


@pytest.mark.parametrize("seed,offset", [(0, 0), (0x5EED, 7), (0xFFFFFFFF12345678, 2**40 + 3)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_stochastic_parity(seed, offset, dtype):
    x = _sweep_like(33, 512, 11, dtype)
    _check_quant(x, 16, "e4m3", "current", rounding="stochastic", seed=seed, offset=offset, tag="sr")


@pytest.mark.parametrize("fmt,block", [("ue5m3", 16), ("e8m0", 32), ("e1m6", 32)])
def test_stochastic_other_formats(fmt, block):
    x = _sweep_like(24, 256, 12)
    _check_quant(x, block, fmt, _policy(fmt), rounding="stochastic", seed=1234, offset=5, tag=f"sr {fmt}")


def test_grads_full_size_sampled_rows():
    """8192x8192 bf16 Laplace(1e-4) gradients, SR with Philox (seed, offset):
    the tensor amax over the whole tensor, codes/scales on sampled rows."""
    x = inputs.grads(0)
    xd = to_device(x)
    st = fq.AmaxState(50)
    qt = fq.fp4_quantize(xd, 16, "e4m3", rounding="stochastic", amax="delayed", state=st, seed=0x5EED, offset=0)
    torch.cuda.synchronize()
    a = oracle.amax(x)
    g = oracle.tensor_scale(a, "e4m3")
    assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([g, a]), "grads tensor_scale")
    rng = np.random.default_rng(0)
    rows = sorted(set(rng.integers(0, 8192, 48).tolist()) | {0, 8191})
    for r in rows:
        q, s = oracle.quantize(x, 16, "e4m3", g, stochastic=True, seed=0x5EED, offset=0, rows=(r, r + 1))
        assert_bytes_equal(host(qt.q[r:r + 1]), q, f"grads row {r} codes")
        assert_bytes_equal(host(qt.scales[r:r + 1]), s, f"grads row {r} scales")


def test_delayed_sequence_and_saturation():
    """Delayed amax refreshed every 50 calls across a sequence; a tensor that
    outgrew the stored maximum saturates exactly as the oracle says."""
    st = fq.AmaxState(50)
    ost = oracle.AmaxState(interval=50)
    for t in range(120):
        x = _sweep_like(16, 256, 1000 + t)
        if t == 1:
            x = inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(x) * np.float32(10.0))
        xd = to_device(x)
        qt = fq.fp4_quantize(xd, 16, "e4m3", rounding="stochastic", amax="delayed", state=st,
                             seed=0x5EED, offset=t)
        torch.cuda.synchronize()
        q, s, g, a = oracle.quantize_tensor(x, 16, "e4m3", "delayed", state=ost, stochastic=True,
                                            seed=0x5EED, offset=t)
        assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([g, a]), f"call {t} ts")
        assert_bytes_equal(host(qt.scales), s, f"call {t} scales")
        assert_bytes_equal(host(qt.q), q, f"call {t} codes")
        if t == 1:
            mags = np.stack([q & 7, q >> 4 & 7], -1)
            assert (mags == 7).sum() > 0
    calls, amax = st.get()
    assert calls == 120 and amax == ost.amax


def test_amax_state_checkpoint_resume():
    xs = [_sweep_like(8, 128, 2000 + t) for t in range(80)]
    st = fq.AmaxState(50)
    outs = []
    for t, x in enumerate(xs):
        qt = fq.fp4_quantize(to_device(x), 16, "e4m3", amax="delayed", state=st)
        outs.append(host(qt.q).copy())
        if t == 72:
            ck = st.get()
    st2 = fq.AmaxState(50)
    st2.set(*ck)
    for t in range(73, 80):
        qt = fq.fp4_quantize(to_device(xs[t]), 16, "e4m3", amax="delayed", state=st2)
        assert_bytes_equal(host(qt.q), outs[t], f"resume call {t}")


def test_refresh_paths_see_the_whole_tensor():
    """The tensor maximum of a refresh must cover every element whichever
    path computes it: the single-pass kernel (tensor held in registers,
    maximum agreed across the grid) up to 4096x4096 bf16 on a 256-CU device,
    the amax kernel plus a second read beyond.  The maximum sits in the
    first, a middle or the last unit; codes and scales are compared on
    sampled rows."""
    rng = np.random.default_rng(7)
    for rows, where in [(4096, "last"), (4096, "first"), (4104, "last"), (4104, "mid"), (24, "last")]:
        x = _sweep_like(rows, 4096, 77 + rows)
        r, c = {"first": (0, 0), "mid": (rows // 2, 2049), "last": (rows - 1, 4095)}[where]
        x[r, c] = inputs.f32_to_bf16_bits(np.array([-9216.0], dtype=np.float32))[0]
        st = fq.AmaxState(1)
        qt = fq.fp4_quantize(to_device(x), 16, "e4m3", amax="current", state=st)
        torch.cuda.synchronize()
        a = oracle.amax(x)
        g = oracle.tensor_scale(a, "e4m3")
        assert a == np.float32(9216.0)
        assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([g, a]), f"{rows} {where} tensor_scale")
        sample = sorted(set(rng.integers(0, rows, 12).tolist()) | {0, r, rows - 1})
        for i in sample:
            q, s_ = oracle.quantize(x, 16, "e4m3", g, rows=(i, i + 1))
            assert_bytes_equal(host(qt.q[i:i + 1]), q, f"{rows} {where} row {i} codes")
            assert_bytes_equal(host(qt.scales[i:i + 1]), s_, f"{rows} {where} row {i} scales")
        st.get()                       # raises if a grid exchange timed out


def test_current_repeated_calls_one_state():
    """Many current-amax calls through one state, single-workgroup launches
    (16 x 256, 8 x 64: no exchange, no slot written) in turn with exchanging
    ones (512 x 384, 2048 x 2048): every call's tensor scale comes from its
    own tensor, never from a slot left by an earlier call."""
    st = fq.AmaxState(1)
    shapes = [(16, 256), (512, 384), (2048, 2048), (8, 64)]
    for t in range(40):
        rows, cols = shapes[t % len(shapes)]
        x = _sweep_like(rows, cols, 3000 + t)
        # the maximum alternates between large and small so stale values show
        scale = np.float32(1000.0 if t % 2 else 0.001)
        x = inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(x) * scale)
        qt = fq.fp4_quantize(to_device(x), 16, "ue5m3", amax="current", state=st)
        torch.cuda.synchronize()
        q, s_, g, a = oracle.quantize_tensor(x, 16, "ue5m3", "current", nthreads=8)
        assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([g, a]), f"call {t} ts")
        assert_bytes_equal(host(qt.scales), s_, f"call {t} scales")
        assert_bytes_equal(host(qt.q), q, f"call {t} codes")
    calls, amax = st.get()
    assert calls == 40


def test_current_amax_under_graph_replay():
    """Current-amax quantize calls captured once in a HIP graph and replayed
    with new input values each time (eager copies and synchronizations in
    between): every replay agrees with the oracle."""
    st = fq.AmaxState(1)
    shapes = [(64, 512), (1024, 1024)]
    xs = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    outs = [fq.QTensor.empty(r, c, 16, "e4m3") for r, c in shapes]
    for x in xs:
        x.zero_()

    def record():
        for x, o in zip(xs, outs):
            fq.fp4_quantize(x, 16, "e4m3", amax="current", state=st, out=o)
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
    for rep in range(5):
        hosts = []
        for i, (r, c) in enumerate(shapes):
            h = _sweep_like(r, c, 4000 + 10 * rep + i)
            h = inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(h) * np.float32(10.0 ** (rep - 2)))
            xs[i].copy_(to_device(h))
            hosts.append(h)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, h in enumerate(hosts):
            q, s_, g, a = oracle.quantize_tensor(h, 16, "e4m3", "current", nthreads=8)
            assert_bytes_equal(f32_bits(host(outs[i].tensor_scale)), f32_bits([g, a]), f"replay {rep}.{i} ts")
            assert_bytes_equal(host(outs[i].scales), s_, f"replay {rep}.{i} scales")
            assert_bytes_equal(host(outs[i].q), q, f"replay {rep}.{i} codes")
    st.get()


def test_edge_values():
    """Zeros, signed zeros, exact E2M1 midpoints, saturation, subnormals,
    single-outlier blocks and scales that underflow/saturate (E1M6)."""
    vals = []
    # E8M0 blocks whose maximum is 4 so the scale is exactly 1: midpoints
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 7.99]
    row = [4.0] + mids + [-m for m in mids] + [0.0, -0.0, 1e-30, -1e-30, 0.5, 3.0, -6.0, 2.0, 1.0, 0.1, 0.9]
    row = row[:32]
    vals.append(row)
    vals.append([0.0] * 32)
    vals.append([-0.0] * 32)
    vals.append([1e-40, -3e-42, 1e-45] + [0.0] * 29)       # fp32 subnormals
    vals.append([1e30] + [1e-30] * 31)                       # single outlier
    vals.append([3e38, -3e38] + [1.0] * 30)
    x = np.array(vals, dtype=np.float32)
    x = np.concatenate([x, x * np.float32(1e-20), x * np.float32(0.37)], axis=0)
    for fmt, block in [("e8m0", 32), ("e4m3", 16), ("e1m6", 16), ("ue5m3", 32), ("e7m0", 16), ("e5m2", 16)]:
        for pol in (["none"] if fmt == "e8m0" else ["none", "current"]):
            _check_quant(x, block, fmt, pol, tag=f"edge {fmt} {pol}")
            _check_quant(x, block, fmt, pol, rounding="stochastic", seed=3, offset=1, tag=f"edge sr {fmt} {pol}")


@pytest.mark.parametrize("shape", [(0, 64), (64, 0), (0, 0)])
@pytest.mark.parametrize("element", ["e2m1", "int4"])
def test_empty_tensor(shape, element):
    """No rows or no columns: nothing is read (a [64, 0] tensor carries row
    stride 1, which is not an aligned leading dimension) and the tensor
    scale is that of an all-zero tensor."""
    x = np.zeros(shape, dtype=np.float32)
    xd = torch.zeros(shape, dtype=torch.float32, device="cuda")
    qt = fq.fp4_quantize(xd, 16, "e4m3", amax="current", element=element)
    y = fq.fp4_dequantize(qt, torch.bfloat16)
    torch.cuda.synchronize()
    assert tuple(y.shape) == shape
    g, a = oracle.resolve_tensor_scale(x, "e4m3", "current", elem=element)
    assert_bytes_equal(f32_bits(host(qt.tensor_scale)), f32_bits([g, a]), "empty ts")


@pytest.mark.parametrize("fmt,block", [("e4m3", 16), ("ue5m3", 16), ("e1m6", 32), ("e8m0", 32), ("e7m0", 16)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequantize_parity(fmt, block, out):
    rng = np.random.default_rng(5)
    rows, cols = 19, 256
    q = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    s = rng.integers(0, 256, (rows, cols // block), dtype=np.uint8)
    g = np.float32(0.0173) if fmt != "e8m0" else np.float32(1.0)
    qt = fq.QTensor(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(),
                    torch.tensor([g, 0.0], dtype=torch.float32).cuda(), rows, cols, block, fmt,
                    amax="none" if fmt == "e8m0" else "current")
    y = fq.fp4_dequantize(qt, torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    want = oracle.dequantize(q, s, float(g), block, fmt, out=out)
    if out == "f32":
        got = host(y)
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan)
        assert_bytes_equal(f32_bits(got)[~nan], f32_bits(want)[~nan], "dequant f32")
    else:
        got = bf16_bits(y)
        wf = inputs.bf16_bits_to_f32(want)
        nan = np.isnan(wf)
        assert np.array_equal(np.isnan(inputs.bf16_bits_to_f32(got)), nan)
        assert_bytes_equal(got[~nan], want[~nan], "dequant bf16")


def test_quantize_dequantize_roundtrip_small():
    b = inputs.small_b()
    qt = fq.fp4_quantize(to_device(b), 16, "e4m3", amax="current")
    y = fq.fp4_dequantize(qt, torch.float32)
    torch.cuda.synchronize()
    q, s, g, _ = oracle.quantize_tensor(b, 16, "e4m3", "current")
    want = oracle.dequantize(q, s, g, 16, "e4m3")
    assert_bytes_equal(f32_bits(host(y)), f32_bits(want), "roundtrip")


def test_error_leaves_outputs_untouched():
    x = torch.zeros((4, 72), dtype=torch.bfloat16, device="cuda")
    qt = fq.QTensor.empty(4, 72, 16, "e4m3")
    qt.q.fill_(0xA5)
    qt.scales.fill_(0x5A)
    qt.tensor_scale.fill_(7.0)
    with pytest.raises(fq.Fp4Error) as e:
        fq.fp4_quantize(x, 16, "e4m3", out=qt)          # 72 % 16 != 0
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert bool((qt.q == 0xA5).all()) and bool((qt.scales == 0x5A).all())
    assert bool((qt.tensor_scale == 7.0).all())
    with pytest.raises(fq.Fp4Error) as e:
        fq.fp4_quantize(torch.zeros((4, 64), device="cuda"), 32, "e8m0", amax="current")
    assert e.value.status == -2
