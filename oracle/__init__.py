"""CPU oracle for block-scaled FP4 quantization and the GEMMs that consume it.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark, never by the product package.  It shares no
code with the HIP library.

The arithmetic lives in fp4_oracle.c (plain C, binary32 step sequence with no
contraction); this module marshals numpy arrays into it and adds the GEMM
reference, which is the binary64 product of the exactly dequantized operands
(numpy matmul as the library primitive) with the per-element tolerance
T = 1e-5 * sum_k |a_k||b_k|.

Page citations (see fp4_oracle.c for the full list):
  quant_prune_distill/486 "Метод": NVFP4 = E2M1 / group 16 / E4M3 scale,
  MXFP = group 32 / E8M0 scale.
  gonzo_ML/3986 "Форматы FP4" and "Стохастическая квантизация".
  ue5m3-fp4-pretraining "Что сделали": UE5M3, tensor max refreshed every 50.

Parity status: every function here is pinned by tests/test_oracle_pins.py
except the UE5M3 exponent bias, which the pages do not give (parity unpinned
beyond the format's own round-trip and the unsigned property).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_fp4.so")

# scale format name -> (exponent bits, mantissa bits, has sign bit)
FORMATS = {
    "e4m3": (4, 3, 1),
    "ue5m3": (5, 3, 0),
    "e3m4": (3, 4, 1),
    "e1m6": (1, 6, 1),
    "e2m5": (2, 5, 1),
    "e5m2": (5, 2, 1),
    "e6m1": (6, 1, 1),
    "e7m0": (7, 0, 1),
    "e8m0": (8, 0, 0),
}

ELEMS = {"e2m1": 0, "int4": 1, "fp8_e4m3": 2, "int8": 3, "fp6_e2m3": 4, "fp6_e3m2": 5, "int6": 6}
ELEM_BITS = {"e2m1": 4, "int4": 4, "fp8_e4m3": 8, "int8": 8, "fp6_e2m3": 6, "fp6_e3m2": 6, "int6": 6}

_lib = None


def _elem(elem: str) -> int:
    try:
        return ELEMS[elem]
    except KeyError:
        raise ValueError(f"unknown element grid {elem!r}") from None


def lib():
    """Load (building first if needed) the oracle shared library."""
    global _lib
    if _lib is not None:
        return _lib
    src = os.path.join(_HERE, "fp4_oracle.c")
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        from . import build as _b
        _b.build()
    L = ctypes.CDLL(_LIB_PATH)
    c_i64, c_u64, c_f, c_d, c_int, c_p = (ctypes.c_int64, ctypes.c_uint64, ctypes.c_float,
                                         ctypes.c_double, ctypes.c_int, ctypes.c_void_p)
    sig = {
        "or_e2m1_decode": (c_d, [c_int]),
        "or_e2m1_rtn": (c_int, [c_f]),
        "or_e2m1_sr": (c_int, [c_f, ctypes.c_uint32]),
        "or_scale_is_nan": (c_int, [c_int, c_int, c_int, c_int]),
        "or_scale_decode": (c_d, [c_int, c_int, c_int, c_int]),
        "or_scale_max": (c_d, [c_int, c_int, c_int]),
        "or_scale_encode": (c_int, [c_int, c_int, c_int, c_f]),
        "or_e8m0_block_code": (c_int, [c_f]),
        "or_tensor_scale": (c_f, [c_f, c_int, c_int, c_int]),
        "or_philox4x32_10": (None, [c_p, c_p, c_p]),
        "or_sr_bits": (ctypes.c_uint32, [c_u64, c_u64, c_u64]),
        "or_amax": (c_f, [c_p, c_int, c_i64, c_i64, c_i64]),
        "or_quantize": (c_int, [c_p, c_int, c_i64, c_i64, c_i64, c_int, c_int, c_int, c_int, c_f,
                                c_int, c_u64, c_u64, c_i64, c_i64, c_p, c_p, c_int]),
        "or_f32_to_bf16": (ctypes.c_uint16, [c_f]),
        "or_dequantize": (c_int, [c_p, c_p, c_f, c_i64, c_i64, c_int, c_int, c_int, c_int, c_int,
                                  c_p, c_i64]),
        "or_dequantize_f64": (c_int, [c_p, c_p, c_f, c_i64, c_i64, c_int, c_int, c_int, c_int, c_p]),
        "or_round_to_bf16": (c_d, [c_d]),
        "or_round_to_bf16_array": (None, [c_p, c_p, c_i64]),
        "or_e2m1_rtn_array": (None, [c_p, c_p, c_i64]),
        "or_e2m1_sr_array": (None, [c_p, c_p, c_p, c_i64]),
        "or_sr_bits_array": (None, [c_u64, c_u64, c_u64, c_i64, c_p]),
        "or_rht_norm": (c_f, [c_int]),
        "or_int4_decode": (c_d, [c_int]),
        "or_int8_decode": (c_d, [c_int]),
        "or_int8_rtn": (c_int, [c_f]),
        "or_int8_sr": (c_int, [c_f, ctypes.c_uint32]),
        "or_e8m0_block_code_emax": (c_int, [c_f, c_int]),
        "or_int4_rtn": (c_int, [c_f]),
        "or_int4_sr": (c_int, [c_f, ctypes.c_uint32]),
        "or_tensor_scale_elem": (c_f, [c_f, c_int, c_int, c_int, c_int]),
        "or_quantize_elem": (c_int, [c_p, c_int, c_i64, c_i64, c_i64, c_int, c_int, c_int, c_int, c_f,
                                     c_int, c_u64, c_u64, c_i64, c_i64, c_p, c_p, c_int, c_int]),
        "or_dequantize_elem": (c_int, [c_p, c_p, c_f, c_i64, c_i64, c_int, c_int, c_int, c_int, c_int,
                                       c_p, c_i64, c_int]),
        "or_dequantize_f64_elem": (c_int, [c_p, c_p, c_f, c_i64, c_i64, c_int, c_int, c_int, c_int, c_p, c_int]),
        "or_rht_forward": (c_int, [c_p, c_int, c_i64, c_i64, c_int, ctypes.c_uint32, c_p]),
        "or_rht_inverse": (c_int, [c_p, c_i64, c_i64, c_int, ctypes.c_uint32, c_p]),
        "or_f32_to_bf16_array": (None, [c_p, c_p, c_i64]),
        "or_elem_mag_array": (None, [c_p, c_p, c_p, c_i64, c_int, c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _fmt(fmt: str):
    try:
        return FORMATS[fmt]
    except KeyError:
        raise ValueError(f"unknown scale format {fmt!r}") from None


def _as_input(x: np.ndarray):
    """x is float32, or uint16 holding bf16 bit patterns."""
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), 0
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), 1
    raise TypeError("oracle input must be float32 or uint16 (bf16 bits)")


# --------------------------------------------------------------------------
# element / scale codecs
# --------------------------------------------------------------------------
def e2m1_decode(code: int) -> float:
    return lib().or_e2m1_decode(int(code))


def e2m1_rtn(v: float) -> int:
    return lib().or_e2m1_rtn(float(v))


def e2m1_sr(v: float, r16: int) -> int:
    return lib().or_e2m1_sr(float(v), int(r16))


def e2m1_rtn_array(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    out = np.empty(v.size, dtype=np.uint8)
    lib().or_e2m1_rtn_array(_ptr(v), _ptr(out), v.size)
    return out


def e2m1_sr_array(v: np.ndarray, r16: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    r = np.ascontiguousarray(r16, dtype=np.uint32).ravel()
    assert r.size == v.size
    out = np.empty(v.size, dtype=np.uint8)
    lib().or_e2m1_sr_array(_ptr(v), _ptr(r), _ptr(out), v.size)
    return out


def elem_mag_array(v: np.ndarray, elem: str, r16: np.ndarray | None = None) -> np.ndarray:
    """Magnitude codes of the scaled values v on an element grid: nearest
    rounding, or stochastic with the given 16-bit variates."""
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    out = np.empty(v.size, dtype=np.uint8)
    if r16 is None:
        lib().or_elem_mag_array(_ptr(v), None, _ptr(out), v.size, _elem(elem), 0)
    else:
        r = np.ascontiguousarray(r16, dtype=np.uint32).ravel()
        assert r.size == v.size
        lib().or_elem_mag_array(_ptr(v), _ptr(r), _ptr(out), v.size, _elem(elem), 1)
    return out


def sr_bits_array(seed: int, offset: int, i0: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    lib().or_sr_bits_array(seed, offset, i0, n, _ptr(out))
    return out


def scale_decode(fmt: str, code: int) -> float:
    return lib().or_scale_decode(*_fmt(fmt), int(code))


def scale_is_nan(fmt: str, code: int) -> bool:
    return bool(lib().or_scale_is_nan(*_fmt(fmt), int(code)))


def scale_max(fmt: str) -> float:
    return lib().or_scale_max(*_fmt(fmt))


def scale_encode(fmt: str, u: float) -> int:
    if fmt == "e8m0":
        raise ValueError("E8M0 block scales use the exponent rule (e8m0_block_code)")
    return lib().or_scale_encode(*_fmt(fmt), float(u))


def e8m0_block_code(amax_b: float) -> int:
    return lib().or_e8m0_block_code(float(amax_b))


def tensor_scale(amax_t: float, fmt: str, elem: str = "e2m1") -> float:
    return lib().or_tensor_scale_elem(float(amax_t), *_fmt(fmt), _elem(elem))


def int8_decode(code: int) -> float:
    return lib().or_int8_decode(int(code))


def int8_rtn(v: float) -> int:
    return lib().or_int8_rtn(float(v))


def int8_sr(v: float, r16: int) -> int:
    return lib().or_int8_sr(float(v), int(r16))


def e8m0_block_code_emax(amax_b: float, emax: int) -> int:
    return lib().or_e8m0_block_code_emax(float(amax_b), int(emax))


def int4_decode(code: int) -> float:
    return lib().or_int4_decode(int(code))


def int4_rtn(v: float) -> int:
    return lib().or_int4_rtn(float(v))


def int4_sr(v: float, r16: int) -> int:
    return lib().or_int4_sr(float(v), int(r16))


def philox4x32_10(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib().or_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_bits(seed: int, offset: int, i: int) -> int:
    return lib().or_sr_bits(seed, offset, i)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    f = lib().or_f32_to_bf16
    return np.array([f(float(v)) for v in x], dtype=np.uint16)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Correct (RNE) rounding of binary64 values to bf16, returned as binary64."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    lib().or_round_to_bf16_array(_ptr(x), _ptr(y), x.size)
    return y


# --------------------------------------------------------------------------
# tensor operations
# --------------------------------------------------------------------------
def amax(x: np.ndarray) -> float:
    x, is_bf16 = _as_input(x)
    rows, cols = x.shape
    return lib().or_amax(_ptr(x), is_bf16, rows, cols, cols)


def quantize(x: np.ndarray, block: int, fmt: str, g: float, *, stochastic: bool = False,
             seed: int = 0, offset: int = 0, rows: tuple | None = None, nthreads: int = 1, elem: str = "e2m1"):
    """Quantize rows [r0, r1) of x (all rows by default) with tensor scale g.

    Returns (q, scales): q is uint8 [r1-r0, cols/2] (low nibble = even
    element), scales is uint8 [r1-r0, cols/block].
    """
    x, is_bf16 = _as_input(x)
    nrows, cols = x.shape
    r0, r1 = (0, nrows) if rows is None else rows
    q = np.zeros((r1 - r0, cols * ELEM_BITS[elem] // 8), dtype=np.uint8)
    s = np.zeros((r1 - r0, cols // block), dtype=np.uint8)
    rc = lib().or_quantize_elem(_ptr(x), is_bf16, nrows, cols, cols, block, *_fmt(fmt), float(g),
                                int(stochastic), seed, offset, r0, r1, _ptr(q), _ptr(s), nthreads, _elem(elem))
    if rc != 0:
        raise ValueError("oracle quantize: argument outside the contract")
    return q, s


def dequantize(q: np.ndarray, scales: np.ndarray, g: float, block: int, fmt: str,
               out: str = "f32", elem: str = "e2m1") -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, cols = q.shape[0], q.shape[1] * 8 // ELEM_BITS[elem]
    if out == "f32":
        y = np.empty((rows, cols), dtype=np.float32)
    elif out == "bf16":
        y = np.empty((rows, cols), dtype=np.uint16)
    else:
        raise ValueError(out)
    rc = lib().or_dequantize_elem(_ptr(q), _ptr(scales), float(g), rows, cols, block, *_fmt(fmt),
                                  int(out == "bf16"), _ptr(y), cols, _elem(elem))
    if rc != 0:
        raise ValueError("oracle dequantize: argument outside the contract")
    return y


def dequantize_f64(q: np.ndarray, scales: np.ndarray, g: float, block: int, fmt: str,
                   elem: str = "e2m1") -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, cols = q.shape[0], q.shape[1] * 8 // ELEM_BITS[elem]
    y = np.empty((rows, cols), dtype=np.float64)
    rc = lib().or_dequantize_f64_elem(_ptr(q), _ptr(scales), float(g), rows, cols, block, *_fmt(fmt), _ptr(y),
                                      _elem(elem))
    if rc != 0:
        raise ValueError("oracle dequantize_f64: argument outside the contract")
    return y


# --------------------------------------------------------------------------
# blockwise randomized Hadamard transform (ue5m3-fp4-pretraining "Что
# сделали": a randomized Hadamard transform spreads outliers before
# quantization; quant_prune_distill/574 "Метод": Hadamard rotations make
# distributions closer to Gaussian).  See fp4_oracle.c for the reading.
# --------------------------------------------------------------------------
def rht_norm(block: int) -> float:
    return lib().or_rht_norm(block)


def rht_forward(x: np.ndarray, block: int, signs: int) -> np.ndarray:
    """y = c_B * H_B * D * v for every block of `block` elements of a row
    (binary32 butterfly); returns float32 [rows, cols]."""
    x, is_bf16 = _as_input(x)
    rows, cols = x.shape
    y = np.empty((rows, cols), dtype=np.float32)
    if lib().or_rht_forward(_ptr(x), is_bf16, rows, cols, block, signs & 0xFFFFFFFF, _ptr(y)) != 0:
        raise ValueError("oracle rht_forward: argument outside the contract")
    return y


def rht_inverse(y: np.ndarray, block: int, signs: int) -> np.ndarray:
    """v = D * (c_B * H_B * y) per block (binary32 butterfly)."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    rows, cols = y.shape
    x = np.empty((rows, cols), dtype=np.float32)
    if lib().or_rht_inverse(_ptr(y), rows, cols, block, signs & 0xFFFFFFFF, _ptr(x)) != 0:
        raise ValueError("oracle rht_inverse: argument outside the contract")
    return x


def f32_to_bf16_bits_array(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, dtype=np.uint16)
    lib().or_f32_to_bf16_array(_ptr(x), _ptr(y), x.size)
    return y


def dequantize_rht(q: np.ndarray, scales: np.ndarray, g: float, block: int, fmt: str, signs: int,
                   out: str = "f32") -> np.ndarray:
    """Dequantize a tensor quantized after the blockwise RHT: the binary32
    dequantized values, then the inverse transform, then (bf16 output) one
    more nearest-even rounding."""
    x = rht_inverse(dequantize(q, scales, g, block, fmt, out="f32"), block, signs)
    return f32_to_bf16_bits_array(x) if out == "bf16" else x


# --------------------------------------------------------------------------
# amax policies (ue5m3-fp4-pretraining "Что сделали": the tensor maximum is
# refreshed once every 50 steps and the stored value is used in between)
# --------------------------------------------------------------------------
@dataclass
class AmaxState:
    interval: int = 50
    calls: int = 0
    amax: float = 0.0


def resolve_tensor_scale(x: np.ndarray, fmt: str, policy: str, state: AmaxState | None = None,
                         elem: str = "e2m1"):
    """Return (g, amax_used) for one quantize call and advance a delayed state.

    policy: "none" (g = 1), "current" (amax of this tensor), or "delayed"
    (refresh from this tensor when calls % interval == 0, else reuse).
    """
    if policy == "none":
        return 1.0, 0.0
    if policy == "current":
        a = amax(x)
        return tensor_scale(a, fmt, elem), a
    if policy == "delayed":
        if state is None:
            raise ValueError("delayed policy needs a state")
        if state.calls % state.interval == 0:
            state.amax = amax(x)
        state.calls += 1
        return tensor_scale(state.amax, fmt, elem), state.amax
    raise ValueError(policy)


def quantize_tensor(x: np.ndarray, block: int, fmt: str, policy: str, *, state: AmaxState | None = None,
                    stochastic: bool = False, seed: int = 0, offset: int = 0, nthreads: int = 1,
                    rht_signs: int | None = None, elem: str = "e2m1"):
    """Whole quantize call: tensor scale per policy, then every block.
    With rht_signs the blockwise randomized Hadamard transform is applied
    first (rht_forward) and everything after it, the tensor maximum
    included, sees the transformed binary32 tensor.
    elem: "e2m1" (FP4), "int4" (the integer grid -7..7, two's-complement
    nibbles; quant_prune_distill/574 "Метод": NVINT4 / MXINT4), or the 8-bit
    grids "fp8_e4m3" and "int8" (-127..127), one byte per element (MXFP8 /
    MXINT8), or the 6-bit grids "fp6_e2m3", "fp6_e3m2" and "int6" (-31..31),
    packed as a little-endian bit stream of 6 bits per element (MXFP6 /
    MXINT6).
    Returns (q, scales, g, amax_used)."""
    if rht_signs is not None:
        x = rht_forward(x, block, rht_signs)
    g, a = resolve_tensor_scale(x, fmt, policy, state, elem)
    q, s = quantize(x, block, fmt, g, stochastic=stochastic, seed=seed, offset=offset, nthreads=nthreads,
                    elem=elem)
    return q, s, g, a


# --------------------------------------------------------------------------
# GEMM references
# --------------------------------------------------------------------------
def gemm_ref(a_hat: np.ndarray, b_hat: np.ndarray):
    """C = A_hat @ B_hat^T in binary64 and T = 1e-5 * |A_hat| @ |B_hat|^T.

    a_hat: [M, K], b_hat: [N, K] exact binary64 dequantized operands (both
    blocked along K; the weight is stored [N, K])."""
    c = a_hat @ b_hat.T
    t = 1e-5 * (np.abs(a_hat) @ np.abs(b_hat).T)
    return c, t


def gemm_check(c_out: np.ndarray, c_ref: np.ndarray, tol: np.ndarray) -> np.ndarray:
    """Boolean mask of bf16 outputs (given as float values) that are the bf16
    rounding of some value within [c_ref - tol, c_ref + tol]."""
    lo = round_to_bf16(c_ref - tol)
    hi = round_to_bf16(c_ref + tol)
    c = np.asarray(c_out, dtype=np.float64)
    return (lo <= c) & (c <= hi)


# --------------------------------------------------------------------------
# column-wise (transposed) quantization: the operands of the backward pass
# (gonzo_ML/3986 "Стохастическая квантизация": stochastic rounding for the
# backward gradients; ue5m3-fp4-pretraining "Что сделали": every linear layer
# in FP4, so the weight-gradient product needs its operands blocked along the
# token dimension, i.e. along the columns of x)
# --------------------------------------------------------------------------
def quantize_transposed_tensor(x: np.ndarray, block: int, fmt: str, policy: str, *,
                               state: AmaxState | None = None, stochastic: bool = False, seed: int = 0,
                               offset: int = 0, nthreads: int = 1, rht_signs: int | None = None,
                               elem: str = "e2m1"):
    """The whole quantize call applied to the transpose of x.

    x: [R, C]; the result describes x^T: codes [C, R/2], scales [C, R/block],
    blocks of `block` consecutive rows of one column of x.  The logical
    element index of the stochastic-rounding counter is that of x^T
    (i = c * R + r).  Reading: the pages give no layout for the transposed
    operand; taking it as the plain quantization of x^T makes it the [N, K]
    operand the GEMM consumes.  Returns (q, scales, g, amax_used)."""
    xt = np.ascontiguousarray(np.asarray(x).T)
    return quantize_tensor(xt, block, fmt, policy, state=state, stochastic=stochastic, seed=seed,
                           offset=offset, nthreads=nthreads, rht_signs=rht_signs, elem=elem)
