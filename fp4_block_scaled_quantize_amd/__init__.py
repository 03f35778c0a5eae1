"""Python binding of the gfx950 block-scaled FP4 library (libfp4.so).

Argument marshalling only: every step of quantize, dequantize and the GEMMs
runs in the HIP kernels behind the C ABI of include/fp4.h.  torch provides
device memory and the current stream.  There is no fallback: if libfp4.so is
missing or fails to load, every call raises.

Names follow the C ABI: fp4_quantize, fp4_quantize_transposed, fp4_quantize_both, fp4_dequantize, fp4_gemm, fp4_wo_gemm,
plus the amax state (per-tensor maximum refreshed every N calls,
ue5m3-fp4-pretraining "Что сделали").
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4.so")

SCALE_FORMATS = {"e4m3": 0, "ue5m3": 1, "e3m4": 2, "e1m6": 3, "e8m0": 4, "e2m5": 5, "e5m2": 6, "e6m1": 7,
                 "e7m0": 8}
ROUNDING = {"nearest": 0, "stochastic": 1}
AMAX = {"none": 0, "current": 1, "delayed": 2}
TRANSFORM = {"none": 0, "rht": 1}
ELEMENT = {"e2m1": 0, "int4": 1, "fp8_e4m3": 2, "int8": 3, "fp6_e2m3": 4, "fp6_e3m2": 5, "int6": 6}
ELEMENT_BITS = {"e2m1": 4, "int4": 4, "fp8_e4m3": 8, "int8": 8, "fp6_e2m3": 6, "fp6_e3m2": 6, "int6": 6}
DTYPE = {torch.float32: 0, torch.bfloat16: 1}

FP4_OK = 0


class Fp4Format(ctypes.Structure):
    _fields_ = [("block", ctypes.c_int32), ("scale", ctypes.c_int32), ("rounding", ctypes.c_int32),
                ("amax", ctypes.c_int32), ("transform", ctypes.c_int32), ("transform_signs", ctypes.c_uint32),
                ("element", ctypes.c_int32)]


class Fp4TensorC(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("tensor_scale", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("fmt", Fp4Format)]


class Fp4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


_lib = None


def lib():
    """The loaded libfp4.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u64, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32
    T = ctypes.POINTER(Fp4TensorC)
    sig = {
        "fp4_version": (i32, []),
        "fp4_status_string": (ctypes.c_char_p, [i32]),
        "fp4_amax_state_create": (i32, [u32, ctypes.POINTER(vp)]),
        "fp4_amax_state_destroy": (i32, [vp]),
        "fp4_amax_state_get": (i32, [vp, ctypes.POINTER(u64), ctypes.POINTER(ctypes.c_float)]),
        "fp4_amax_state_set": (i32, [vp, u64, ctypes.c_float]),
        "fp4_amax_state_fallbacks": (i32, [vp, ctypes.POINTER(u32)]),
        "fp4_set_exchange_wait": (i32, [u64, ctypes.POINTER(u64)]),
        "fp4_set_gemm_small_outputs": (i32, [i64, ctypes.POINTER(i64)]),
        "fp4_quantize": (i32, [vp, i32, i64, T, vp, u64, u64, vp]),
        "fp4_quantize_noalloc": (i32, [vp, i32, i64, T, u64, u64, vp]),
        "fp4_quantize_transposed": (i32, [vp, i32, i64, T, vp, u64, u64, vp]),
        "fp4_quantize_both": (i32, [vp, i32, i64, T, T, vp, u64, u64, vp]),
        "fp4_dequantize": (i32, [T, vp, i32, i64, vp]),
        "fp4_gemm": (i32, [T, T, vp, i64, vp]),
        "fp4_wo_gemm": (i32, [vp, i64, i64, T, vp, i64, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().fp4_status_string(status).decode()


def _check(status: int, what: str):
    if status != FP4_OK:
        raise Fp4Error(status, what)


def _stream(stream, device: torch.device | None = None) -> int:
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _on_device(what: str, *tensors: torch.Tensor) -> torch.device:
    """Every tensor a call hands to the library must be a CUDA tensor, all on
    one device (the kernels dereference these pointers on that device)."""
    dev = None
    for t in tensors:
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{what}: every tensor must be a CUDA tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{what}: tensors on different devices ({dev} and {t.device})")
    return dev


def _check_dense_out(out: torch.Tensor, shape: tuple, dtypes: tuple, what: str):
    """An output the kernels write row by row through (pointer, row stride):
    exactly the shape, one of the dtypes and unit column stride."""
    if tuple(out.shape) != tuple(shape) or out.dtype not in dtypes or (out.dim() == 2 and out.numel() != 0
                                                                         and out.stride(1) != 1):
        raise ValueError(f"{what}: out must be {list(shape)} with unit column stride and dtype in {dtypes}")


# ---------------------------------------------------------------------------
@dataclass
class QTensor:
    """A quantized tensor: codes [rows, cols/2] (low nibble = even element),
    scales [rows, cols/block], tensor_scale [2] = {g, amax used}; transform
    "rht" with rht_signs marks a blockwise randomized Hadamard transform
    applied before quantization."""
    q: torch.Tensor
    scales: torch.Tensor
    tensor_scale: torch.Tensor
    rows: int
    cols: int
    block: int
    scale: str
    rounding: str = "nearest"
    amax: str = "current"
    transform: str = "none"
    rht_signs: int = 0
    element: str = "e2m1"

    @classmethod
    def empty(cls, rows: int, cols: int, block: int, scale: str, rounding: str = "nearest",
              amax: str = "current", device="cuda", transform: str = "none", rht_signs: int = 0,
              element: str = "e2m1"):
        q = torch.empty((rows, cols * ELEMENT_BITS[element] // 8), dtype=torch.uint8, device=device)
        s = torch.empty((rows, cols // block), dtype=torch.uint8, device=device)
        ts = torch.empty(2, dtype=torch.float32, device=device)
        return cls(q, s, ts, rows, cols, block, scale, rounding, amax, transform, rht_signs, element)

    def c(self) -> Fp4TensorC:
        # the library reads or writes rows * cols * bits / 8 code bytes and
        # rows * cols / block scale bytes through these pointers, densely
        qb = self.rows * (self.cols * ELEMENT_BITS[self.element] // 8)
        if not (self.q.is_contiguous() and self.scales.is_contiguous() and self.tensor_scale.is_contiguous()):
            raise ValueError("QTensor buffers must be contiguous")
        if self.q.numel() * self.q.element_size() < qb or \
                self.scales.numel() * self.scales.element_size() < self.rows * (self.cols // self.block) or \
                self.tensor_scale.numel() < 2:
            raise ValueError(f"QTensor buffers are smaller than a [{self.rows}, {self.cols}] tensor on the "
                             f"{self.element} grid needs")
        fmt = Fp4Format(self.block, SCALE_FORMATS[self.scale], ROUNDING[self.rounding], AMAX[self.amax],
                        TRANSFORM[self.transform], self.rht_signs & 0xFFFFFFFF, ELEMENT[self.element])
        return Fp4TensorC(self.q.data_ptr(), self.scales.data_ptr(), self.tensor_scale.data_ptr(),
                          self.rows, self.cols, fmt)


class AmaxState:
    """Per-tensor amax state: refreshed every `interval` calls (CURRENT uses
    it too, refreshing on every call).  Owns 17664 bytes of device memory."""

    def __init__(self, interval: int = 50):
        h = ctypes.c_void_p()
        _check(lib().fp4_amax_state_create(interval, ctypes.byref(h)), "fp4_amax_state_create")
        self._h = h
        self.interval = interval

    @property
    def handle(self):
        return self._h

    def get(self):
        calls, amax = ctypes.c_uint64(), ctypes.c_float()
        _check(lib().fp4_amax_state_get(self._h, ctypes.byref(calls), ctypes.byref(amax)), "fp4_amax_state_get")
        return calls.value, amax.value

    def set(self, calls: int, amax: float):
        _check(lib().fp4_amax_state_set(self._h, calls, amax), "fp4_amax_state_set")

    def fallbacks(self) -> int:
        """Workgroups of single-pass refreshes on this state that gave up
        waiting for the others and read the whole tensor themselves."""
        n = ctypes.c_uint32()
        _check(lib().fp4_amax_state_fallbacks(self._h, ctypes.byref(n)), "fp4_amax_state_fallbacks")
        return n.value

    def close(self):
        if self._h is not None and self._h.value:
            lib().fp4_amax_state_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def set_exchange_wait(ticks: int) -> int:
    """Set the process-wide bound on a single-pass refresh's wait for the
    other workgroups (ticks of the 100 MHz device clock); returns the
    previous bound."""
    prev = ctypes.c_uint64()
    _check(lib().fp4_set_exchange_wait(ticks, ctypes.byref(prev)), "fp4_set_exchange_wait")
    return prev.value


def set_gemm_small_outputs(outputs: int) -> int:
    """Set the process-wide bound on M * N up to which fp4_gemm takes the
    one-wave-per-32x32-tile path for the pairings it covers (E8M0 operands:
    an eighth of it; 0 turns the path off); returns the previous bound."""
    prev = ctypes.c_int64()
    _check(lib().fp4_set_gemm_small_outputs(outputs, ctypes.byref(prev)), "fp4_set_gemm_small_outputs")
    return prev.value


# One amax workspace per (device, stream) for calls with the current policy
# that bring no state: calls on one stream run in order, so they can share
# it, and no call allocates.
_default_states: dict = {}


def _default_state(device: torch.device, stream_handle: int) -> AmaxState:
    key = (device.index, stream_handle)
    st = _default_states.get(key)
    if st is None:
        with torch.cuda.device(device):
            st = AmaxState(1)
        _default_states[key] = st
    return st


def _resolve_state(amax: str, state: AmaxState | None, device: torch.device, stream_handle: int):
    if amax == "none" or state is not None:
        return state
    if amax == "delayed":
        raise ValueError("the delayed amax policy needs an AmaxState")
    return _default_state(device, stream_handle)


def _check_out(t: QTensor, rows: int, cols: int, block: int, element: str):
    """A caller-provided output must hold the codes and scales of a [rows,
    cols] tensor on `element` (the kernels write exactly that many bytes)."""
    qb = cols * ELEMENT_BITS[element] // 8
    if (t.rows, t.cols) != (rows, cols) or t.q.numel() < rows * qb or t.scales.numel() < rows * (cols // block) \
            or t.tensor_scale.numel() < 2 or not (t.q.is_contiguous() and t.scales.is_contiguous()):
        raise ValueError(f"out does not hold a [{rows}, {cols}] tensor on the {element} grid with block {block}")


def fp4_quantize(x: torch.Tensor, block: int = 16, scale: str = "e4m3", rounding: str = "nearest",
                 amax: str = "current", state: AmaxState | None = None, seed: int = 0, offset: int = 0,
                 out: QTensor | None = None, stream=None, rht_signs: int | None = None,
                 element: str = "e2m1") -> QTensor:
    """Quantize a 2-D fp32/bf16 CUDA tensor (rows may be strided: x.stride(1)
    must be 1).  DELAYED needs an AmaxState; CURRENT without one uses a
    workspace shared by the calls on the same device and stream.  rht_signs (32-bit sign mask) applies the
    blockwise randomized Hadamard transform before quantization; element
    selects the grid: "e2m1" (default), "int4" (-7..7), the one-byte
    "fp8_e4m3" and "int8" (-127..127), or the six-bit "fp6_e2m3",
    "fp6_e3m2" and "int6" (-31..31)."""
    if x.dim() != 2 or (x.stride(1) != 1 and x.numel() != 0):
        raise ValueError("x must be 2-D with unit column stride")
    if x.dtype not in DTYPE:
        raise ValueError("x must be float32 or bfloat16")
    _on_device("fp4_quantize", x, *(() if out is None else (out.q, out.scales, out.tensor_scale)))
    rows, cols = x.shape
    if out is None:
        out = QTensor.empty(rows, cols, block, scale, rounding, amax, device=x.device, element=element)
    else:
        _check_out(out, rows, cols, block, element)
        out.block, out.scale, out.rounding, out.amax = block, scale, rounding, amax
    out.transform, out.rht_signs = ("none", 0) if rht_signs is None else ("rht", rht_signs & 0xFFFFFFFF)
    out.element = element
    sh = _stream(stream, x.device)
    state = _resolve_state(amax, state, x.device, sh)
    out._state = state        # keep the state alive while work is queued
    tc = out.c()
    st = lib().fp4_quantize(x.data_ptr(), DTYPE[x.dtype], x.stride(0), ctypes.byref(tc),
                            state.handle if state is not None else None, seed, offset, sh)
    _check(st, "fp4_quantize")
    return out


def fp4_quantize_noalloc(x: torch.Tensor, out: QTensor, block: int = 16, scale: str = "e4m3",
                         rounding: str = "nearest", amax: str = "current", seed: int = 0, offset: int = 0,
                         stream=None, rht_signs: int | None = None, element: str = "e2m1") -> QTensor:
    """fp4_quantize into a caller-provided output with no allocation: the
    current-amax workspace is the library's static per-device array (calls
    that overlap on one device must be ordered by the caller).  Policies
    "none" and "current"."""
    if x.dim() != 2 or (x.stride(1) != 1 and x.numel() != 0):
        raise ValueError("x must be 2-D with unit column stride")
    if x.dtype not in DTYPE:
        raise ValueError("x must be float32 or bfloat16")
    _on_device("fp4_quantize_noalloc", x, out.q, out.scales, out.tensor_scale)
    rows, cols = x.shape
    _check_out(out, rows, cols, block, element)
    out.block, out.scale, out.rounding, out.amax, out.element = block, scale, rounding, amax, element
    out.transform, out.rht_signs = ("none", 0) if rht_signs is None else ("rht", rht_signs & 0xFFFFFFFF)
    tc = out.c()
    _check(lib().fp4_quantize_noalloc(x.data_ptr(), DTYPE[x.dtype], x.stride(0), ctypes.byref(tc), seed, offset,
                                      _stream(stream, x.device)), "fp4_quantize_noalloc")
    return out


def fp4_quantize_transposed(x: torch.Tensor, block: int = 16, scale: str = "e4m3", rounding: str = "nearest",
                            amax: str = "current", state: AmaxState | None = None, seed: int = 0, offset: int = 0,
                            out: QTensor | None = None, stream=None, element: str = "e2m1",
                            rht_signs: int | None = None) -> QTensor:
    """Column-wise quantization of a 2-D fp32/bf16 CUDA tensor x [R, C]: the
    result is the quantized x^T [C, R] (blocks run down the columns of x)."""
    if x.dim() != 2 or (x.stride(1) != 1 and x.numel() != 0):
        raise ValueError("x must be 2-D with unit column stride")
    if x.dtype not in DTYPE:
        raise ValueError("x must be float32 or bfloat16")
    _on_device("fp4_quantize_transposed", x, *(() if out is None else (out.q, out.scales, out.tensor_scale)))
    r, c = x.shape
    if out is None:
        out = QTensor.empty(c, r, block, scale, rounding, amax, device=x.device, element=element)
    else:
        _check_out(out, c, r, block, element)
        out.block, out.scale, out.rounding, out.amax = block, scale, rounding, amax
    out.element = element
    out.transform, out.rht_signs = ("none", 0) if rht_signs is None else ("rht", rht_signs & 0xFFFFFFFF)
    sh = _stream(stream, x.device)
    state = _resolve_state(amax, state, x.device, sh)
    out._state = state
    tc = out.c()
    st = lib().fp4_quantize_transposed(x.data_ptr(), DTYPE[x.dtype], x.stride(0), ctypes.byref(tc),
                                       state.handle if state is not None else None, seed, offset, sh)
    _check(st, "fp4_quantize_transposed")
    return out


def fp4_quantize_both(x: torch.Tensor, block: int = 16, scale: str = "e4m3", rounding: str = "nearest",
                      amax: str = "current", state: AmaxState | None = None, seed: int = 0, offset: int = 0,
                      out: tuple | None = None, stream=None, element: str = "e2m1"):
    """Row-wise and column-wise quantization of x [R, C] from one read:
    returns (rowwise [R, C], colwise [C, R]) QTensors, each identical to the
    corresponding single-orientation call."""
    if x.dim() != 2 or (x.stride(1) != 1 and x.numel() != 0):
        raise ValueError("x must be 2-D with unit column stride")
    if x.dtype not in DTYPE:
        raise ValueError("x must be float32 or bfloat16")
    r, c = x.shape
    if out is None:
        out = (QTensor.empty(r, c, block, scale, rounding, amax, device=x.device, element=element),
               QTensor.empty(c, r, block, scale, rounding, amax, device=x.device, element=element))
    qr, qc = out
    _on_device("fp4_quantize_both", x, qr.q, qr.scales, qr.tensor_scale, qc.q, qc.scales, qc.tensor_scale)
    _check_out(qr, r, c, block, element)
    _check_out(qc, c, r, block, element)
    for t in (qr, qc):
        t.block, t.scale, t.rounding, t.amax, t.element = block, scale, rounding, amax, element
        t.transform, t.rht_signs = "none", 0
    sh = _stream(stream, x.device)
    state = _resolve_state(amax, state, x.device, sh)
    qr._state = qc._state = state
    tr, tcw = qr.c(), qc.c()
    st = lib().fp4_quantize_both(x.data_ptr(), DTYPE[x.dtype], x.stride(0), ctypes.byref(tr), ctypes.byref(tcw),
                                 state.handle if state is not None else None, seed, offset, sh)
    _check(st, "fp4_quantize_both")
    return qr, qc


def fp4_dequantize(t: QTensor, dtype=torch.float32, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    dev = _on_device("fp4_dequantize", t.q, t.scales, t.tensor_scale, *(() if out is None else (out,)))
    if out is None:
        out = torch.empty((t.rows, t.cols), dtype=dtype, device=dev)
    _check_dense_out(out, (t.rows, t.cols), (torch.float32, torch.bfloat16), "fp4_dequantize")
    tc = t.c()
    _check(lib().fp4_dequantize(ctypes.byref(tc), out.data_ptr(), DTYPE[out.dtype], out.stride(0),
                                _stream(stream, dev)), "fp4_dequantize")
    return out


def fp4_gemm(a: QTensor, b: QTensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """C[M, N] = A[M, K] @ W[N, K]^T in bf16 (fp32 accumulation)."""
    dev = _on_device("fp4_gemm", a.q, a.scales, a.tensor_scale, b.q, b.scales, b.tensor_scale,
                     *(() if out is None else (out,)))
    if out is None:
        out = torch.empty((a.rows, b.rows), dtype=torch.bfloat16, device=dev)
    _check_dense_out(out, (a.rows, b.rows), (torch.bfloat16,), "fp4_gemm")
    ta, tb = a.c(), b.c()
    _check(lib().fp4_gemm(ctypes.byref(ta), ctypes.byref(tb), out.data_ptr(), out.stride(0), _stream(stream, dev)),
           "fp4_gemm")
    return out


def fp4_wo_gemm(x: torch.Tensor, w: QTensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y[M, N] = X[M, K] (bf16) @ W[N, K]^T with W quantized (bf16 out)."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or (x.stride(1) != 1 and x.numel() != 0):
        raise ValueError("x must be a 2-D bf16 tensor with unit column stride")
    if x.shape[1] != w.cols:
        raise ValueError(f"x has {x.shape[1]} columns, the weight {w.cols}")
    dev = _on_device("fp4_wo_gemm", x, w.q, w.scales, w.tensor_scale, *(() if out is None else (out,)))
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, w.rows), dtype=torch.bfloat16, device=dev)
    _check_dense_out(out, (m, w.rows), (torch.bfloat16,), "fp4_wo_gemm")
    tw = w.c()
    _check(lib().fp4_wo_gemm(x.data_ptr(), x.stride(0), m, ctypes.byref(tw), out.data_ptr(), out.stride(0),
                             _stream(stream, dev)), "fp4_wo_gemm")
    return out


__all__ = ["fp4_quantize", "fp4_quantize_transposed", "fp4_quantize_both", "fp4_dequantize", "fp4_gemm",
           "fp4_wo_gemm", "AmaxState", "QTensor", "Fp4Error", "SCALE_FORMATS", "lib", "status_string", "LIB_PATH",
           "set_exchange_wait", "set_gemm_small_outputs", "fp4_quantize_noalloc"]
