"""GEMM of E2M1 operands with E8M0 scales per 16 elements (gonzo_ML/3986
"Форматы FP4": groups of 16 with power-of-two scales) on the gfx950 scaled
FP4 matrix instruction, where each 32-element K-half runs as two
instructions with one 16-element block zeroed; and FP8 operands at K where
the GEMM takes the exact dequantize path.  Tolerance as every GEMM
test: the bf16 rounding of some value within 1e-5 * sum|a||b| of the exact
binary64 product of the oracle's operands (checked byte-identical first).
Shapes cover partial 256-row tiles, several stages, scale groups cut short
at the end of K, and the Llama-2 7B up and down projections (K = 4096 and
11008) on sampled rows."""
import numpy as np
import pytest
import torch

import fp4_inputs as inputs
import oracle
from tests.gpu_util import assert_bytes_equal, check_gemm_every_output, host, to_device

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp4_block_scaled_quantize_amd")


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _quant(x, block, elem, *, rounding="nearest", seed=0, rht=None):
    qt = fq.fp4_quantize(to_device(x), block, "e8m0", rounding=rounding, amax="none", seed=seed, rht_signs=rht,
                         element=elem)
    q, s, g, _ = oracle.quantize_tensor(x, block, "e8m0", "none", stochastic=rounding == "stochastic", seed=seed,
                                        nthreads=8, rht_signs=rht, elem=elem)
    torch.cuda.synchronize()
    assert_bytes_equal(host(qt.q), q, f"{elem}/{block} operand codes")
    assert_bytes_equal(host(qt.scales), s, f"{elem}/{block} operand scales")
    return qt, oracle.dequantize_f64(q, s, g, block, "e8m0", elem=elem)


def _check(c, a_hat, w_hat, rows=None, tag=""):
    if rows is not None:
        a_hat = a_hat[rows]
    cref, tol = oracle.gemm_ref(a_hat, w_hat)
    got = c.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        got = got[rows]
    ok = oracle.gemm_check(got, cref, tol)
    if not ok.all():
        i, j = np.argwhere(~ok)[0]
        raise AssertionError(f"{tag}: {int((~ok).sum())} of {ok.size} outside; first ({i},{j}) got {got[i, j]!r} "
                             f"ref {cref[i, j]!r} tol {tol[i, j]!r}")


def _x(rows, cols, seed, std=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)) * std
    x *= np.exp(rng.uniform(-3, 3, (rows, cols // 16))).repeat(16, axis=1)      # spread block scales
    return x.astype(np.float32)


CASES = [("e2m1", 16)]


@pytest.mark.parametrize("elem,block", CASES)
@pytest.mark.parametrize("m,n,k", [(64, 256, 256), (300, 520, 1280), (257, 513, 512), (1, 33, 1024),
                                   (96, 80, 2304)])
def test_scaled_shapes(elem, block, m, n, k):
    if elem == "e2m1" and k % 256:
        pytest.skip("E2M1 block 16 needs whole 256-element stages")
    qa, a = _quant(_x(m, k, 31 + m), block, elem)
    qw, w = _quant(_x(n, k, 32 + n, 0.1), block, elem)
    c = fq.fp4_gemm(qa, qw)
    torch.cuda.synchronize()
    _check(c, a, w, tag=f"{elem}/{block} {m}x{n}x{k}")


@pytest.mark.parametrize("elem,block", CASES)
def test_scaled_transform_and_sr(elem, block):
    xa, xw = _x(96, 512, 41), _x(72, 512, 42)
    qa, a = _quant(xa, block, elem, rht=0x2468ACE1)
    qw, w = _quant(xw, block, elem, rht=0x2468ACE1)
    c = fq.fp4_gemm(qa, qw)
    torch.cuda.synchronize()
    _check(c, a, w, tag=f"{elem}/{block} rht")
    qa, a = _quant(xa, block, elem, rounding="stochastic", seed=5)
    qw, w = _quant(xw, block, elem, rounding="stochastic", seed=6)
    c = fq.fp4_gemm(qa, qw)
    torch.cuda.synchronize()
    _check(c, a, w, tag=f"{elem}/{block} sr")


@pytest.mark.parametrize("elem,block", CASES)
@pytest.mark.parametrize("wname", ["up", "down"])
def test_scaled_llama_every_output(elem, block, wname):
    """The Llama-2 7B launch the bench times (M = 8192): every output
    against the binary64 reference."""
    shapes = {"a": (8192, 4096 if wname == "up" else 11008), "up": (11008, 4096), "down": (4096, 11008)}
    qa, a = _quant_rows(inputs.llama("a", shapes), block, elem)
    qw, w = _quant_rows(inputs.llama(wname, shapes), block, elem)
    c = fq.fp4_gemm(qa, qw)
    torch.cuda.synchronize()
    check_gemm_every_output(c, a, w, f"{elem}/{block} llama {wname}")


def _quant_rows(x, block, elem):
    """As _quant for large operands: codes compared whole, dequantized fully."""
    return _quant(x, block, elem)


def test_fp8_every_code_k512():
    """All 256 FP8 codes (NaN codes replaced) times mixed E8M0 block-16 and
    block-32 scales at K = 512: W selects one column per output, so C[m, n]
    is the bf16 rounding of A's value at (m, n)."""
    k = 512
    codes = np.arange(256, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00
    row = np.concatenate([codes, np.roll(codes, 91)])
    q_a = np.stack([row, row[::-1], np.roll(row, 77)])
    rng = np.random.default_rng(24)
    for block in (16, 32):
        s_a = rng.integers(110, 145, (3, k // block), dtype=np.uint8)
        q_w = np.zeros((k, k), dtype=np.uint8)
        q_w[np.arange(k), np.arange(k)] = 0x38                      # 1.0
        s_w = np.full((k, k // block), 127, dtype=np.uint8)

        def qt(q, s):
            return fq.QTensor(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(),
                              torch.tensor([1.0, 0.0], dtype=torch.float32).cuda(), q.shape[0], k, block, "e8m0",
                              amax="none", element="fp8_e4m3")
        c = fq.fp4_gemm(qt(q_a, s_a), qt(q_w, s_w))
        torch.cuda.synchronize()
        a_hat = oracle.dequantize_f64(q_a, s_a, np.float32(1.0), block, "e8m0", elem="fp8_e4m3")
        want = oracle.round_to_bf16(a_hat)
        got = c.float().cpu().numpy().astype(np.float64)
        bad = np.argwhere(got != want)
        assert bad.size == 0, (f"block {block}: {len(bad)} outputs differ; first {tuple(bad[0])}: "
                               f"got {got[tuple(bad[0])]!r} want {want[tuple(bad[0])]!r}")


def test_e2m1_block16_every_code():
    """Every E2M1 code in both halves of every 32-element K-half, with
    different E8M0 scales on the two 16-element blocks, against W = I."""
    k = 256
    nib = np.arange(16, dtype=np.uint8)
    row = np.tile(nib[0::2] | (nib[1::2] << 4), 16)[: k // 2]                      # 128 bytes
    q_a = np.stack([row, np.roll(row, 5), row[::-1]])
    rng = np.random.default_rng(25)
    s_a = rng.integers(100, 150, (3, k // 16), dtype=np.uint8)
    q_w = np.zeros((k, k // 2), dtype=np.uint8)
    for i in range(k):
        q_w[i, i // 2] = 0x02 if i % 2 == 0 else 0x20                          # 1.0 at column i
    s_w = np.full((k, k // 16), 127, dtype=np.uint8)

    def qt(q, s):
        return fq.QTensor(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(),
                          torch.tensor([1.0, 0.0], dtype=torch.float32).cuda(), q.shape[0], k, 16, "e8m0",
                          amax="none")
    c = fq.fp4_gemm(qt(q_a, s_a), qt(q_w, s_w))
    torch.cuda.synchronize()
    a_hat = oracle.dequantize_f64(q_a, s_a, np.float32(1.0), 16, "e8m0")
    w_hat = oracle.dequantize_f64(q_w, s_w, np.float32(1.0), 16, "e8m0")
    assert np.array_equal(w_hat, np.eye(k))
    want = oracle.round_to_bf16(a_hat)
    got = c.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got, want)
