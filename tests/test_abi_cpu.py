"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/fp4.h declares, and rejects invalid arguments before
touching the device (the pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

import fp4_block_scaled_quantize_amd as fq


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "fp4.h"), encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = fq.lib()
    names = _declared_functions()
    assert {"fp4_quantize", "fp4_dequantize", "fp4_gemm", "fp4_wo_gemm"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    assert fq.lib().fp4_version() >= 100
    assert fq.status_string(0) == "ok"
    for st in (-1, -2, -3, -4, -5):
        assert fq.status_string(st) not in ("ok", "unknown status")


FAKE = 0x10000      # 16-byte aligned, never dereferenced: validation fails first


def _tensor(block=16, scale=0, rounding=0, amax=1, rows=4, cols=64, q=FAKE, s=FAKE, ts=FAKE):
    return fq.Fp4TensorC(q, s, ts, rows, cols, fq.Fp4Format(block, scale, rounding, amax))


@pytest.mark.parametrize("kw,want", [
    (dict(block=8), -1),                 # block size not 16/32
    (dict(scale=42), -1),                # unknown scale format
    (dict(rounding=7), -1),
    (dict(amax=9), -1),
    (dict(q=0), -1),                     # null codes
    (dict(cols=72), -3),                 # cols % block
    (dict(q=FAKE + 2), -4),              # codes misaligned
    (dict(scale=4, block=32), -2),       # E8M0 with a tensor-scale policy
])
def test_quantize_rejects_before_launch(kw, want):
    t = _tensor(**kw)
    st = fq.lib().fp4_quantize(FAKE, 1, t.cols, ctypes.byref(t), FAKE, 0, 0, None)
    assert st == want


def test_quantize_requires_state_for_tensor_scale():
    t = _tensor(amax=2)
    assert fq.lib().fp4_quantize(FAKE, 1, 64, ctypes.byref(t), None, 0, 0, None) == -1


def test_quantize_input_checks():
    t = _tensor()
    L = fq.lib()
    assert L.fp4_quantize(None, 1, 64, ctypes.byref(t), FAKE, 0, 0, None) == -1
    assert L.fp4_quantize(FAKE, 5, 64, ctypes.byref(t), FAKE, 0, 0, None) == -1
    assert L.fp4_quantize(FAKE, 1, 32, ctypes.byref(t), FAKE, 0, 0, None) == -3      # ld < cols
    assert L.fp4_quantize(FAKE + 8, 1, 64, ctypes.byref(t), FAKE, 0, 0, None) == -4  # x misaligned
    assert L.fp4_quantize(FAKE, 1, 68, ctypes.byref(t), FAKE, 0, 0, None) == -4      # ld*2 % 16


def test_gemm_and_wo_gemm_shape_checks():
    L = fq.lib()
    a = _tensor(rows=8, cols=256)
    b = _tensor(rows=8, cols=512)
    assert L.fp4_gemm(ctypes.byref(a), ctypes.byref(b), FAKE, 8, None) == -3        # K mismatch
    b32 = _tensor(rows=8, cols=256, block=32)
    assert L.fp4_gemm(ctypes.byref(a), ctypes.byref(b32), FAKE, 8, None) == -2      # block mismatch
    a96 = _tensor(rows=8, cols=96)
    assert L.fp4_gemm(ctypes.byref(a96), ctypes.byref(a96), FAKE, 8, None) == -3    # K % 128
    assert L.fp4_gemm(ctypes.byref(a), ctypes.byref(a), FAKE, 4, None) == -3        # ldc < N
    assert L.fp4_gemm(ctypes.byref(a), ctypes.byref(a), FAKE + 1, 8, None) == -4    # c misaligned
    w = _tensor(rows=8, cols=256)
    assert L.fp4_wo_gemm(FAKE, 256, 0, ctypes.byref(w), FAKE, 8, None) == -2        # M = 0
    assert L.fp4_wo_gemm(FAKE, 256, 17, ctypes.byref(w), FAKE, 8, None) == -2       # M > 16
    w2 = _tensor(rows=8, cols=128)
    assert L.fp4_wo_gemm(FAKE, 128, 1, ctypes.byref(w2), FAKE, 8, None) == -3       # K % 256


def test_amax_state_argument_checks():
    L = fq.lib()
    h = ctypes.c_void_p()
    assert L.fp4_amax_state_create(0, ctypes.byref(h)) == -1
    assert L.fp4_amax_state_create(50, None) == -1
    assert L.fp4_amax_state_destroy(None) == -1


def test_quantize_transposed_checks():
    L = fq.lib()
    t = _tensor(rows=64, cols=32)                 # x is [32, 64]
    assert L.fp4_quantize_transposed(FAKE, 1, 63, ctypes.byref(t), FAKE, 0, 0, None) == -3   # ld < 64
    assert L.fp4_quantize_transposed(FAKE, 1, 68, ctypes.byref(t), FAKE, 0, 0, None) == -4   # ld*2 % 16
    assert L.fp4_quantize_transposed(FAKE + 8, 1, 64, ctypes.byref(t), FAKE, 0, 0, None) == -4
    t6 = _tensor(rows=60, cols=32)                 # x columns not a multiple of 8
    assert L.fp4_quantize_transposed(FAKE, 1, 64, ctypes.byref(t6), FAKE, 0, 0, None) == -3
    tq = _tensor(rows=64, cols=32, q=FAKE + 4)     # codes not 16-byte aligned
    assert L.fp4_quantize_transposed(FAKE, 1, 64, ctypes.byref(tq), FAKE, 0, 0, None) == -4
    tb = _tensor(rows=64, cols=40)                 # x rows not a multiple of the block
    assert L.fp4_quantize_transposed(FAKE, 1, 64, ctypes.byref(tb), FAKE, 0, 0, None) == -3
    te = _tensor(rows=64, cols=32, scale=4, block=32)
    assert L.fp4_quantize_transposed(FAKE, 1, 64, ctypes.byref(te), FAKE, 0, 0, None) == -2
    assert L.fp4_quantize_transposed(FAKE, 1, 64, ctypes.byref(t), None, 0, 0, None) == -1   # no state


def test_transform_checks():
    L = fq.lib()
    assert L.fp4_version() >= 101
    t = _tensor()
    t.fmt.transform = 7                                            # unknown transform
    assert L.fp4_quantize(FAKE, 1, t.cols, ctypes.byref(t), FAKE, 0, 0, None) == -1
    a = _tensor(rows=8, cols=256)
    b = _tensor(rows=8, cols=256)
    a.fmt.transform, a.fmt.transform_signs = 1, 5
    assert L.fp4_gemm(ctypes.byref(a), ctypes.byref(b), FAKE, 8, None) == -2   # only one operand transformed
    b.fmt.transform, b.fmt.transform_signs = 1, 6
    assert L.fp4_gemm(ctypes.byref(a), ctypes.byref(b), FAKE, 8, None) == -2   # different signs
    w = _tensor(rows=8, cols=256)
    w.fmt.transform = 1
    assert L.fp4_wo_gemm(FAKE, 256, 1, ctypes.byref(w), FAKE, 8, None) == -2
    tt = _tensor(rows=60, cols=32)                 # supported, so the shape check decides
    tt.fmt.transform = 1
    assert L.fp4_quantize_transposed(FAKE, 1, 64, ctypes.byref(tt), FAKE, 0, 0, None) == -3


def test_element_checks():
    L = fq.lib()
    assert L.fp4_version() >= 102
    t = _tensor()
    t.fmt.element = 7
    assert L.fp4_quantize(FAKE, 1, t.cols, ctypes.byref(t), FAKE, 0, 0, None) == -1
    a = _tensor(rows=8, cols=256)
    b = _tensor(rows=8, cols=256)
    a.fmt.element = 1
    assert L.fp4_gemm(ctypes.byref(a), ctypes.byref(b), FAKE, 8, None) == -2     # mixed grids
    w = _tensor(rows=8, cols=256)
    w.fmt.element = 1
    assert L.fp4_wo_gemm(FAKE, 256, 0, ctypes.byref(w), FAKE, 8, None) == -2      # INT4 weights accepted: M = 0 decides


def test_quantize_both_checks():
    L = fq.lib()
    r = _tensor(rows=32, cols=64)
    c = _tensor(rows=64, cols=32)
    bad = _tensor(rows=64, cols=64)
    assert L.fp4_quantize_both(FAKE, 1, 64, ctypes.byref(r), ctypes.byref(bad), FAKE, 0, 0, None) == -3
    c2 = _tensor(rows=64, cols=32, scale=1)                       # different scale encoding
    assert L.fp4_quantize_both(FAKE, 1, 64, ctypes.byref(r), ctypes.byref(c2), FAKE, 0, 0, None) == -2
    c3 = _tensor(rows=64, cols=32)
    c3.fmt.transform = 1
    assert L.fp4_quantize_both(FAKE, 1, 64, ctypes.byref(r), ctypes.byref(c3), FAKE, 0, 0, None) == -2
    assert L.fp4_quantize_both(FAKE, 1, 60, ctypes.byref(r), ctypes.byref(c), FAKE, 0, 0, None) == -3   # ld < C
    assert L.fp4_quantize_both(FAKE + 8, 1, 64, ctypes.byref(r), ctypes.byref(c), FAKE, 0, 0, None) == -4
    assert L.fp4_quantize_both(FAKE, 1, 64, ctypes.byref(r), ctypes.byref(c), None, 0, 0, None) == -1   # no state


def test_8bit_element_checks():
    L = fq.lib()
    assert L.fp4_version() >= 103
    t = _tensor(q=FAKE + 4)
    t.fmt.element = 2                                  # 8-bit codes need 8-byte alignment
    assert L.fp4_quantize(FAKE, 1, t.cols, ctypes.byref(t), FAKE, 0, 0, None) == -4
    t.fmt.element = 7
    assert L.fp4_quantize(FAKE, 1, t.cols, ctypes.byref(t), FAKE, 0, 0, None) == -1


def test_6bit_element_checks():
    L = fq.lib()
    assert L.fp4_version() >= 104
    for elem in (4, 5, 6):
        t = _tensor(q=FAKE + 4)                        # 6-bit codes need 8-byte alignment
        t.fmt.element = elem
        assert L.fp4_quantize(FAKE, 1, t.cols, ctypes.byref(t), FAKE, 0, 0, None) == -4
        tt = _tensor(rows=64, cols=32)                 # column-wise 6-bit codes need R % 64 == 0
        tt.fmt.element = elem
        assert L.fp4_quantize_transposed(FAKE, 1, 64, ctypes.byref(tt), FAKE, 0, 0, None) == -3
        a = _tensor(rows=8, cols=256, scale=3)         # E1M6 scales: no 16-bit type is exact
        b = _tensor(rows=8, cols=256, scale=3)
        a.fmt.element = b.fmt.element = elem
        assert L.fp4_gemm(ctypes.byref(a), ctypes.byref(b), FAKE, 8, None) == -2
        w = _tensor(rows=8, cols=256, q=FAKE)
        w.fmt.element = elem
        assert L.fp4_wo_gemm(FAKE, 256, 0, ctypes.byref(w), FAKE, 8, None) == -2   # 6-bit weights accepted: M = 0 decides
        w.q = FAKE + 4                                 # ... after the 8-byte alignment of their codes
        assert L.fp4_wo_gemm(FAKE, 256, 1, ctypes.byref(w), FAKE, 8, None) == -4


def test_binding_refuses_buffers_too_small_for_the_grid():
    """The binding checks buffer sizes before any call: codes allocated for
    4-bit elements cannot describe an 8- or 6-bit tensor."""
    q4 = fq.QTensor.empty(4, 64, 16, "e4m3", device="cpu")
    for elem in ("fp8_e4m3", "int8", "fp6_e2m3", "int6"):
        q4.element = elem
        with pytest.raises(ValueError):
            q4.c()
    q4.element = "e2m1"
    q4.c()
    with pytest.raises(ValueError):
        fq._check_out(q4, 4, 64, 16, "int8")
    fq._check_out(q4, 4, 64, 16, "int4")


class _NoCalls:
    """Stands in for the library: any call is a test failure."""
    def __getattr__(self, name):
        raise AssertionError(f"library function {name} reached")


def test_binding_checks_every_buffer_before_any_call(monkeypatch):
    import torch
    monkeypatch.setattr(fq, "lib", lambda: _NoCalls())
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    q = fq.QTensor.empty(4, 64, 16, "e4m3", device="cpu")
    # host tensors never reach the kernels
    for call in (lambda: fq.fp4_quantize(x), lambda: fq.fp4_quantize_transposed(x.t().contiguous().t()[:, :]),
                 lambda: fq.fp4_quantize_both(x), lambda: fq.fp4_dequantize(q), lambda: fq.fp4_gemm(q, q),
                 lambda: fq.fp4_wo_gemm(x, q)):
        with pytest.raises(ValueError):
            call()
    # a weight with a different K than x
    w = fq.QTensor.empty(8, 128, 16, "e4m3", device="cpu")
    with pytest.raises(ValueError, match="columns"):
        fq.fp4_wo_gemm(x, w)
    # outputs: exact shape, dtype and unit column stride
    fq._check_dense_out(torch.empty(4, 8, dtype=torch.bfloat16), (4, 8), (torch.bfloat16,), "t")
    for bad in (torch.empty(3, 8, dtype=torch.bfloat16), torch.empty(4, 8, dtype=torch.float32),
                torch.empty(8, 4, dtype=torch.bfloat16).t()):
        with pytest.raises(ValueError):
            fq._check_dense_out(bad, (4, 8), (torch.bfloat16,), "t")
    # quantized buffers must be dense
    q.q = torch.empty(4, 64, dtype=torch.uint8)[:, ::2]
    with pytest.raises(ValueError, match="contiguous"):
        q.c()


def test_transposed_call_resets_a_reused_outputs_transform(monkeypatch):
    """A reused output that carried the Hadamard transform must not keep it
    on a later call without one (the format the library receives is
    checked through a recording stand-in for the library)."""
    import torch
    seen = []

    class _Rec:
        def fp4_quantize_transposed(self, xp, dt, ld, tc, st, seed, off, s):
            t = tc._obj
            seen.append((t.fmt.transform, t.fmt.transform_signs))
            return 0

    monkeypatch.setattr(fq, "lib", lambda: _Rec())
    monkeypatch.setattr(fq, "_on_device", lambda what, *t: torch.device("cpu"))
    monkeypatch.setattr(fq, "_stream", lambda stream, device=None: 0)
    x = torch.zeros(32, 16, dtype=torch.bfloat16)
    out = fq.QTensor.empty(16, 32, 16, "e8m0", amax="none", device="cpu")
    fq.fp4_quantize_transposed(x, 16, "e8m0", amax="none", out=out, rht_signs=0x1234)
    fq.fp4_quantize_transposed(x, 16, "e8m0", amax="none", out=out)
    assert seen == [(1, 0x1234), (0, 0)]
    assert out.transform == "none" and out.rht_signs == 0


def test_quantize_noalloc_rejects_before_launch():
    """The no-allocation quantize validates like fp4_quantize and refuses the
    delayed policy before touching the device."""
    L = fq.lib()
    t = _tensor(rows=4, cols=64)
    assert L.fp4_quantize_noalloc(FAKE, 1, 64, None, 0, 0, None) == -1
    t.fmt.amax = 2
    assert L.fp4_quantize_noalloc(FAKE, 1, 64, ctypes.byref(t), 0, 0, None) == -2
    t.fmt.amax = 1
    t.fmt.scale = 4                                     # E8M0 with a tensor scale
    assert L.fp4_quantize_noalloc(FAKE, 1, 64, ctypes.byref(t), 0, 0, None) == -2
    t.fmt.scale = 0
    assert L.fp4_quantize_noalloc(FAKE, 1, 32, ctypes.byref(t), 0, 0, None) == -3   # ld < cols


def test_gemm_small_outputs_bound():
    """fp4_set_gemm_small_outputs swaps the process-wide bound, returns the
    previous one (2^21 by default) and rejects a negative bound."""
    L = fq.lib()
    assert L.fp4_version() >= 107
    prev = ctypes.c_int64(-1)
    assert L.fp4_set_gemm_small_outputs(5, ctypes.byref(prev)) == 0
    first = prev.value
    assert first == 1 << 21
    assert L.fp4_set_gemm_small_outputs(first, ctypes.byref(prev)) == 0
    assert prev.value == 5
    assert L.fp4_set_gemm_small_outputs(-1, None) == -1
    assert fq.set_gemm_small_outputs(first) == first
