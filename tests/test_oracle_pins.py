"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every test here checks the oracle against something other than itself: values
the pages print (tests/golden), closed forms of the formats, an independent
library implementation (torch's float8 conversions, rocRAND's Philox engine),
exact rational arithmetic, and invariants of the method.  None needs a GPU.
"""
import math
import os
import shutil
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests.conftest import ROOT, read_golden

ALL_FMTS = ["e1m6", "e2m5", "e3m4", "e4m3", "e5m2", "e6m1", "e7m0", "ue5m3", "e8m0"]
GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def f32(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


# ---------------------------------------------------------------------------
# E2M1 element codec
# ---------------------------------------------------------------------------
def test_e2m1_decode_matches_grid_fixture():
    rows = read_golden("e2m1_grid.txt")
    assert len(rows) == 16
    for code, val in rows:
        v = oracle.e2m1_decode(int(code))
        assert v == float(val)
        assert math.copysign(1.0, v) == math.copysign(1.0, float(val))


def _rtn_threshold_form(a: np.ndarray) -> np.ndarray:
    """Nearest-even E2M1 magnitude by counting crossed midpoints: a midpoint
    between an even code and the next odd code rounds down (strict >), a
    midpoint between an odd code and the next even code rounds up (>=);
    everything at or beyond 6 is code 7."""
    a = np.abs(a.astype(np.float64))
    return ((a > 0.25).astype(np.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
            + (a > 2.5) + (a >= 3.5) + (a > 5.0)).astype(np.uint8)


def test_e2m1_rtn_against_midpoint_closed_form():
    # every fp32 within +-4096 ulps of each midpoint and grid point, both signs
    centres = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] + GRID[1:] + [8.0]
    pieces = []
    for c in centres:
        b = np.float32(c).view(np.uint32).astype(np.int64)
        pieces.append(np.arange(b - 4096, b + 4097, dtype=np.int64))
    # plus a strided sweep of all fp32 in [0, 16) and the subnormals
    pieces.append(np.arange(0, 0x41800000, 997, dtype=np.int64))
    pieces.append(np.arange(0, 1 << 23, 4099, dtype=np.int64))
    bits = np.concatenate(pieces).astype(np.uint32)
    for sign in (0, 0x80000000):
        v = f32(bits | np.uint32(sign))
        got = oracle.e2m1_rtn_array(v)
        want = _rtn_threshold_form(v)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (v[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_e2m1_rtn_is_nearest_with_even_ties_exact():
    # exact rational check on random values: chosen magnitude is at minimum
    # distance and on ties its code is even; beyond 6 it saturates.
    rng = np.random.default_rng(11)
    v = rng.uniform(0, 7, 20000).astype(np.float32)
    got = oracle.e2m1_rtn_array(v)
    for x, c in zip(v, got):
        fx = Fraction(float(x))
        if fx >= 6:
            assert c == 7
            continue
        d = [abs(fx - Fraction(g)) for g in GRID]
        m = min(d)
        best = [i for i in range(8) if d[i] == m]
        want = best[0] if len(best) == 1 else [i for i in best if i % 2 == 0][0]
        assert c == want


# ---------------------------------------------------------------------------
# stochastic rounding: unbiased in expectation (gonzo_ML/3986,
# "Стохастическая квантизация": its role is to remove rounding bias)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("v", [0.1, 0.25, 0.3333, 0.6, 0.75, 1.01, 1.7, 2.2, 2.5, 3.9, 4.5, 5.99,
                               0.0, 0.5, 1.5, 4.0, 6.0])
def test_sr_exact_expectation_over_all_random_values(v):
    v = np.float32(v)
    r = np.arange(1 << 16, dtype=np.uint32)
    mags = oracle.e2m1_sr_array(np.full(r.size, v, dtype=np.float32), r)
    vals = np.array(GRID)[mags]
    # result is always one of the two neighbours
    lo = max(g for g in GRID if g <= v)
    hi = min([g for g in GRID if g > v] or [6.0])
    assert set(np.unique(vals)) <= {lo, hi}
    total = sum(Fraction(float(x)) for x in vals)
    mean = total / (1 << 16)
    fv = Fraction(float(v))
    if fv >= 6:
        assert mean == 6
        return
    # unbiased up to the 2^-16 resolution of the uniform variate
    assert abs(mean - fv) <= Fraction(hi - lo) / (1 << 16)
    # exact when the position between neighbours is a multiple of 2^-16
    pos = (fv - Fraction(lo)) / Fraction(hi - lo)
    if (pos * (1 << 16)).denominator == 1:
        assert mean == fv
    # a grid value never moves
    if fv in [Fraction(g) for g in GRID]:
        assert np.all(vals == float(v))


def test_sr_statistical_unbiasedness_over_philox_stream():
    # mean of SR over consecutive Philox-indexed elements of one value
    n = 1 << 18
    r = oracle.sr_bits_array(0x5EED, 3, 0, n)
    for v in (0.3, 1.2, 2.7, 4.9):
        mags = oracle.e2m1_sr_array(np.full(n, v, dtype=np.float32), r)
        vals = np.array(GRID)[mags]
        lo = max(g for g in GRID if g <= v)
        hi = min(g for g in GRID if g > v)
        p = (np.float32(v) - lo) / (hi - lo)
        sd = (hi - lo) * math.sqrt(p * (1 - p) / n)
        assert abs(vals.mean() - float(np.float32(v))) < 6 * sd


def test_sr_bits_uniformity():
    r = oracle.sr_bits_array(1, 0, 0, 1 << 18)
    assert r.max() < (1 << 16)
    hist = np.bincount(r >> 12, minlength=16)
    expected = r.size / 16
    chi2 = float(((hist - expected) ** 2 / expected).sum())
    assert chi2 < 60  # 15 dof; p ~ 1e-7 threshold


# ---------------------------------------------------------------------------
# Philox4x32-10 against rocRAND's independent engine (host build)
# ---------------------------------------------------------------------------
def _rocrand_ref_binary():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    hdr = "/opt/rocm/include/rocrand/rocrand_kernel.h"
    if not (os.path.exists(hipcc) and os.path.exists(hdr)):
        pytest.skip("rocRAND headers / hipcc not available")
    out = os.path.join(tempfile.gettempdir(), f"rocrand_philox_ref_{os.getpid()}")
    src = os.path.join(ROOT, "tests", "helpers", "rocrand_philox_ref.cpp")
    subprocess.run([hipcc, "-O1", "-o", out, src], check=True, capture_output=True)
    return out


@pytest.mark.parametrize("seed,subseq,first", [
    (0, 0, 0), (0x5EED, 3, 0), (0x0123456789ABCDEF, 7, 0xFFFFFFFE), (2**64 - 1, 2**40 + 5, 123456789)])
def test_philox_matches_rocrand(seed, subseq, first):
    exe = _rocrand_ref_binary()
    n = 64
    res = subprocess.run([exe, str(seed), str(subseq), str(first), str(n)], check=True,
                         capture_output=True, text=True)
    lines = res.stdout.strip().splitlines()
    assert len(lines) == n
    key = [seed & 0xFFFFFFFF, seed >> 32]
    for j, line in enumerate(lines):
        c = first + j
        ctr = [c & 0xFFFFFFFF, (c >> 32) & 0xFFFFFFFF, subseq & 0xFFFFFFFF, subseq >> 32]
        want = [int(w, 16) for w in line.split()]
        assert list(oracle.philox4x32_10(ctr, key)) == want


def test_sr_bits_word_and_half_selection():
    # element i uses Philox call i/8 (counter = (i>>3, offset)), word (i>>1)&3,
    # half i&1 -- checked against the generator output directly
    seed, off = 0xDEADBEEF12345678, 9
    for i in [0, 1, 2, 3, 6, 7, 8, 15, 16, 12345, 2**33 + 5]:
        blk = i >> 3
        w = oracle.philox4x32_10([blk & 0xFFFFFFFF, blk >> 32, off, 0], [seed & 0xFFFFFFFF, seed >> 32])
        want = (int(w[(i >> 1) & 3]) >> (16 * (i & 1))) & 0xFFFF
        assert oracle.sr_bits(seed, off, i) == want


# ---------------------------------------------------------------------------
# scale formats
# ---------------------------------------------------------------------------
def test_scale_ranges_match_fixture():
    for fmt, mx, mn in read_golden("scale_format_ranges.txt"):
        vals = [oracle.scale_decode(fmt, c) for c in range(256)]
        fin = [v for v in vals if v == v]
        assert oracle.scale_max(fmt) == float(mx), fmt
        assert min(v for v in fin if v > 0) == float(mn), fmt


def test_e1m6_has_narrowest_range():
    # gonzo_ML/3986 "Форматы FP4": of E1M6..E8M0 only E1M6 (narrowest range) diverges
    def dyn(fmt):
        fin = [oracle.scale_decode(fmt, c) for c in range(256)]
        fin = [v for v in fin if v == v and v > 0]
        return max(fin) / min(fin)
    ranges = {f: dyn(f) for f in ALL_FMTS}
    assert min(ranges, key=ranges.get) == "e1m6"


def test_e4m3_decode_matches_torch_float8_e4m3fn():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for c in range(256):
        v = oracle.scale_decode("e4m3", c)
        if math.isnan(t[c]):
            assert math.isnan(v)
        else:
            assert v == t[c] and math.copysign(1, v) == math.copysign(1, t[c])


def test_e5m2_decode_matches_torch_below_top_binade():
    # torch's float8_e5m2 is IEEE-style (top exponent = Inf/NaN); below it the
    # two agree bit for bit.
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).double().numpy()
    for c in range(256):
        if ((c >> 2) & 0x1F) == 0x1F:
            continue
        assert oracle.scale_decode("e5m2", c) == t[c]


def test_e8m0_decode_matches_torch_float8_e8m0fnu():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    for c in range(256):
        v = oracle.scale_decode("e8m0", c)
        if c == 255:
            assert math.isnan(v) and math.isnan(t[c])
        else:
            assert v == t[c] == 2.0 ** (c - 127)


def test_ue5m3_unsigned_and_monotone():
    # ue5m3-fp4-pretraining "Что сделали": no sign bit, the scale is never negative
    vals = [oracle.scale_decode("ue5m3", c) for c in range(256)]
    assert all(v >= 0 for v in vals if v == v)
    assert sum(1 for v in vals if v != v) == 1
    fin = [v for v in vals if v == v]
    assert all(a < b for a, b in zip(fin, fin[1:]))


@pytest.mark.parametrize("fmt", [f for f in ALL_FMTS if f != "e8m0"])
def test_signed_formats_monotone_one_nan(fmt):
    n = 256 if fmt == "ue5m3" else 128
    vals = [oracle.scale_decode(fmt, c) for c in range(n)]
    fin = [v for v in vals if v == v]
    assert len(fin) == n - 1 and vals[-1] != vals[-1]
    assert all(a < b for a, b in zip(fin, fin[1:]))


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(5)
    u = np.concatenate([
        rng.uniform(0, 464, 50000),
        np.exp(rng.uniform(np.log(1e-4), np.log(464), 50000)),
        # every midpoint between adjacent codes (ties) and their neighbours
        *[np.array([(a + b) / 2]) for a, b in zip(
            [oracle.scale_decode("e4m3", c) for c in range(126)],
            [oracle.scale_decode("e4m3", c) for c in range(1, 127)])],
    ]).astype(np.float32)
    u = np.concatenate([u, np.nextafter(u, np.float32(0)), np.nextafter(u, np.float32(1e9))])
    u = u[(u > 0) & (u <= 464)]
    want = torch.from_numpy(u).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.scale_encode("e4m3", float(x)) for x in u], dtype=np.uint8)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt", [f for f in ALL_FMTS if f != "e8m0"])
def test_scale_encode_nearest_even_exact(fmt):
    # exact rational nearest over the decoded code set, ties to the even code,
    # saturation at the maximum
    n = 256 if fmt == "ue5m3" else 128
    table = [(c, Fraction(oracle.scale_decode(fmt, c))) for c in range(n)
             if not oracle.scale_is_nan(fmt, c)]
    mx = oracle.scale_max(fmt)
    mn = min(float(v) for _, v in table if v > 0)
    rng = np.random.default_rng(hash(fmt) & 0xFFFF)
    u = np.exp(rng.uniform(np.log(mn / 4), np.log(mx * 2), 3000)).astype(np.float32)
    mids = [float((a[1] + b[1]) / 2) for a, b in zip(table, table[1:])][::3]
    u = np.concatenate([u, np.array(mids, dtype=np.float32)])
    for x in u:
        fx = Fraction(float(x))
        d = [(abs(fx - v), c) for c, v in table]
        m = min(dd for dd, _ in d)
        cands = [c for dd, c in d if dd == m]
        want = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        assert oracle.scale_encode(fmt, float(x)) == want, (fmt, float(x))


def test_e8m0_block_code_closed_form():
    # the block maximum lands in [4, 8) after scaling by 2^-(code-127)
    rng = np.random.default_rng(8)
    a = np.exp(rng.uniform(np.log(1e-30), np.log(1e30), 5000)).astype(np.float32)
    for x in a:
        c = oracle.e8m0_block_code(float(x))
        s = 2.0 ** (c - 127)
        assert 4 * s <= float(x) < 8 * s
    for k in range(-120, 120, 7):
        assert oracle.e8m0_block_code(4.0 * 2.0 ** k) == 127 + k
        assert oracle.e8m0_block_code(np.nextafter(np.float32(8.0 * 2.0 ** k), np.float32(0))) == 127 + k
    assert oracle.e8m0_block_code(0.0) == 0
    assert oracle.e8m0_block_code(3.4e38) == 252     # floor(log2) = 127, minus 2, plus bias
    assert oracle.e8m0_block_code(1e-44) == 0      # clamped: the exponent would be below -127


def test_tensor_scale_nvfp4_recipe():
    # NVFP4 tensor scale amax / (6 * 448): the block holding the tensor maximum
    # then gets the largest E4M3 scale
    for a in [1.0, 3.7, 2688.0, 1e-20, 5e30]:
        assert oracle.tensor_scale(a, "e4m3") == np.float32(np.float32(a) / np.float32(2688.0))
    assert oracle.tensor_scale(0.0, "e4m3") == 1.0
    assert oracle.tensor_scale(5.0, "e8m0") == 1.0


# ---------------------------------------------------------------------------
# bf16 (quant_prune_distill/574, "Точность имеет значение": 1 + 1e-3 == 1)
# ---------------------------------------------------------------------------
def test_bf16_absorbs_small_update():
    rows = {r[0]: r[1:] for r in read_golden("page_facts.txt")}
    base, upd = float(rows["bf16_absorbs"][0]), float(rows["bf16_absorbs"][1])
    x = np.float32(base) + np.float32(upd)
    assert oracle.f32_to_bf16_bits(np.array([x]))[0] == oracle.f32_to_bf16_bits(np.array([base]))[0]
    assert oracle.round_to_bf16(np.array([base + upd]))[0] == base


def test_f32_to_bf16_matches_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)
    bits = np.concatenate([bits, (bits & 0xFFFF0000) | 0x8000])     # exact ties
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f32_to_bf16_bits(x)
    assert np.array_equal(got, want)


def test_round_to_bf16_matches_torch_on_f32_values():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(100000).astype(np.float32) * np.float32(1e3)
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    got = oracle.round_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)
    # double inputs between bf16 neighbours, including exact ties
    assert oracle.round_to_bf16(np.array([1.0 + 2**-8]))[0] == 1.0            # tie -> even
    assert oracle.round_to_bf16(np.array([1.0 + 3 * 2**-8]))[0] == 1.0 + 2**-6  # tie -> even
    assert oracle.round_to_bf16(np.array([1.0 + 2**-8 + 2**-40]))[0] == 1.0 + 2**-7


# ---------------------------------------------------------------------------
# whole-tensor quantization invariants
# ---------------------------------------------------------------------------
def _sweep_like(rows, cols, seed, bf16=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)) * 0.02
    m = rng.random((rows, cols)) < 0.01
    x[m] *= 100
    x = x.astype(np.float32)
    if bf16:
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return x


def _to_f32(x):
    return (x.astype(np.uint32) << 16).view(np.float32) if x.dtype == np.uint16 else x


def test_bits_per_param_from_pages():
    facts = [r for r in read_golden("page_facts.txt") if r[0] == "bits_per_param"]
    assert len(facts) == 2
    for _, name, block, fmt, bits in (f[:5] for f in facts):
        block = int(block)
        x = _sweep_like(32, 256, 1)
        q, s, g, _ = oracle.quantize_tensor(x, block, fmt, "none" if fmt == "e8m0" else "current")
        total_bits = 8 * (q.nbytes + s.nbytes)
        assert total_bits / x.size == float(bits)


@pytest.mark.parametrize("fmt", [f for f in ALL_FMTS if f != "e8m0"])
def test_tensor_max_maps_to_six_and_max_scale(fmt):
    # with a current tensor scale amax/(6*Smax) the block holding the tensor
    # maximum takes the largest scale code and its maximum encodes to +-6
    x = _sweep_like(64, 256, 2)
    q, s, g, a = oracle.quantize_tensor(x, 16, fmt, "current")
    xf = _to_f32(x)
    r, c = np.unravel_index(np.argmax(np.abs(xf)), xf.shape)
    n = 256 if fmt == "ue5m3" else 128
    maxcode = max(cc for cc in range(n) if not oracle.scale_is_nan(fmt, cc))
    assert s[r, c // 16] == maxcode
    nib = (q[r, c // 2] >> (4 * (c & 1))) & 0xF
    assert nib & 7 == 7 and (nib >> 3) == (xf[r, c] < 0)
    assert a == float(np.abs(xf).max())


@pytest.mark.parametrize("fmt,block", [("e4m3", 16), ("ue5m3", 16), ("e3m4", 16), ("e1m6", 16),
                                       ("e8m0", 32), ("e4m3", 32)])
def test_sign_symmetry_and_power_of_two_equivariance(fmt, block):
    x = _sweep_like(16, 128, 3, bf16=False)
    pol = "none" if fmt == "e8m0" else "current"
    q, s, g, _ = oracle.quantize_tensor(x, block, fmt, pol)
    qn, sn, gn, _ = oracle.quantize_tensor(-x, block, fmt, pol)
    assert np.array_equal(s, sn) and g == gn
    assert np.array_equal(qn, q ^ 0x88)
    if fmt != "e8m0":
        q2, s2, g2, _ = oracle.quantize_tensor(x * np.float32(8.0), block, fmt, pol)
        assert np.array_equal(q2, q) and np.array_equal(s2, s) and g2 == g * 8
    else:
        q2, s2, _, _ = oracle.quantize_tensor(x * np.float32(8.0), block, fmt, pol)
        assert np.array_equal(q2, q) and np.array_equal(s2.astype(int), s.astype(int) + 3)


def test_permutation_within_block():
    x = _sweep_like(8, 64, 4, bf16=False)
    rng = np.random.default_rng(0)
    perm = np.concatenate([rng.permutation(16) + 16 * b for b in range(4)])
    q, s, g, _ = oracle.quantize_tensor(x, 16, "e4m3", "current")
    qp, sp, gp, _ = oracle.quantize_tensor(np.ascontiguousarray(x[:, perm]), 16, "e4m3", "current")

    def unpack(qq):
        return np.stack([qq & 0xF, qq >> 4], axis=-1).reshape(qq.shape[0], -1)
    assert np.array_equal(s, sp)
    assert np.array_equal(unpack(q)[:, perm], unpack(qp))


def test_e8m0_blocks_are_exact_nearest_of_x_over_scale():
    # with a power-of-two scale x * 2^-e is exact, so each code must be the
    # exact nearest-even E2M1 value of x / s, saturated at 6 (brute force)
    x = _sweep_like(8, 128, 5, bf16=False)
    q, s, _, _ = oracle.quantize_tensor(x, 32, "e8m0", "none")
    for r in range(x.shape[0]):
        for c in range(x.shape[1]):
            sc = Fraction(2) ** (int(s[r, c // 32]) - 127)
            amax_b = max(abs(Fraction(float(v))) for v in x[r, (c // 32) * 32:(c // 32 + 1) * 32])
            assert 4 * sc <= amax_b < 8 * sc
            v = abs(Fraction(float(x[r, c]))) / sc
            if v >= 6:
                want = 7
            else:
                d = [abs(v - Fraction(gv)) for gv in GRID]
                m = min(d)
                cands = [i for i in range(8) if d[i] == m]
                want = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
            nib = (q[r, c // 2] >> (4 * (c & 1))) & 0xF
            assert nib & 7 == want
            assert (nib >> 3) == (np.signbit(x[r, c]))


@pytest.mark.parametrize("fmt", ["e4m3", "ue5m3", "e3m4", "e1m6"])
def test_reconstruction_within_half_spacing(fmt):
    # every non-saturated element is within half a grid step of x / S (up to
    # the binary32 rounding of the reciprocal and product), and elements that
    # differ from the exact nearest are rare and sit next to a midpoint
    x = _sweep_like(64, 256, 6)
    q, s, g, _ = oracle.quantize_tensor(x, 16, fmt, "current")
    xf = _to_f32(x).astype(np.float64)
    mags = np.stack([q & 7, (q >> 4) & 7], axis=-1).reshape(x.shape)
    sc = np.array([oracle.scale_decode(fmt, c) for c in range(256)])[s]
    S = (sc.astype(np.float32) * np.float32(g)).astype(np.float64)
    S = np.repeat(S, 16, axis=1)
    v = np.abs(xf) / np.where(S > 0, S, 1)
    grid = np.array(GRID)
    got = grid[mags]
    nearest = grid[_rtn_threshold_form(v.astype(np.float32))]
    ok = (S > 0) & (v < 6)
    step = np.diff(np.concatenate([grid, [8.0]]))
    lo_idx = np.clip(np.searchsorted(grid, v, side="right") - 1, 0, 7)
    half = step[lo_idx] / 2
    assert np.all(np.abs(got - v)[ok] <= half[ok] * (1 + 2**-20))
    # the reciprocal-then-multiply sequence can only differ from the exact
    # nearest of x / S where x / S sits within a few ulps of a midpoint
    differ = ok & (got != nearest)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    dist = np.min(np.abs(v[differ][:, None] - mids[None, :]), axis=1)
    assert np.all(dist <= v[differ] * 2.0**-21)
    assert differ.sum() <= 1e-2 * ok.sum()


def test_zero_tensor():
    x = np.zeros((4, 64), dtype=np.float32)
    q, s, g, a = oracle.quantize_tensor(x, 16, "e4m3", "current")
    assert g == 1.0 and a == 0.0 and not q.any() and not s.any()
    xn = -x
    q, s, g, a = oracle.quantize_tensor(xn, 16, "e4m3", "current")
    assert np.all(q == 0x88)


def test_delayed_refresh_schedule():
    # ue5m3-fp4-pretraining "Что сделали": the maximum is refreshed once per
    # 50 steps, the stored value used in between
    facts = {r[0]: r[1:] for r in read_golden("page_facts.txt")}
    n = int(facts["amax_refresh_interval"][0])
    st = oracle.AmaxState(interval=n)
    refreshed = []
    prev = None
    for t in range(200):
        x = np.full((2, 32), np.float32(1.0 + t), dtype=np.float32)
        g, a = oracle.resolve_tensor_scale(x, "e4m3", "delayed", st)
        if a != prev:
            refreshed.append(t)
        prev = a
        assert a == float(1 + (t // n) * n)
    assert refreshed == [0, 50, 100, 150]
    assert st.calls == 200


def test_stale_amax_saturates():
    # a tensor whose maximum grew 10x since the last refresh saturates at +-6
    st = oracle.AmaxState(interval=50)
    x0 = _sweep_like(8, 64, 7, bf16=False)
    oracle.resolve_tensor_scale(x0, "e4m3", "delayed", st)
    x1 = x0 * np.float32(10.0)
    g, a = oracle.resolve_tensor_scale(x1, "e4m3", "delayed", st)
    q, s = oracle.quantize(x1, 16, "e4m3", g)
    assert a == oracle.amax(x0)
    mags = np.stack([q & 7, (q >> 4) & 7], axis=-1).reshape(x1.shape)
    big = np.abs(x1) > a * (1 + 1e-6)     # beyond the stale maximum: the block scale saturated
    assert np.all(mags[big] == 7)


def test_stochastic_quantize_uses_global_index_and_offset():
    x = _sweep_like(8, 64, 8, bf16=False)
    g = oracle.tensor_scale(oracle.amax(x), "e4m3")
    q_all, s_all = oracle.quantize(x, 16, "e4m3", g, stochastic=True, seed=42, offset=5)
    q_part, s_part = oracle.quantize(x, 16, "e4m3", g, stochastic=True, seed=42, offset=5, rows=(3, 6))
    assert np.array_equal(q_all[3:6], q_part) and np.array_equal(s_all[3:6], s_part)
    q_o, _ = oracle.quantize(x, 16, "e4m3", g, stochastic=True, seed=42, offset=6)
    assert not np.array_equal(q_all, q_o)
    q_r, s_r = oracle.quantize(x, 16, "e4m3", g)
    assert np.array_equal(s_all, s_r)          # SR changes elements only


# ---------------------------------------------------------------------------
# dequantization and the GEMM reference
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fmt,block", [("e4m3", 16), ("ue5m3", 16), ("e1m6", 16), ("e8m0", 32)])
def test_dequantize_is_rounded_exact_product(fmt, block):
    rng = np.random.default_rng(9)
    q = rng.integers(0, 256, (4, block * 2), dtype=np.uint8)
    n = 256 if fmt in ("ue5m3", "e8m0") else 128
    s = rng.integers(0, n - 1, (4, 4), dtype=np.uint8)
    s = np.where([[oracle.scale_is_nan(fmt, int(c)) for c in row] for row in s], 1, s).astype(np.uint8)
    g = np.float32(0.0123) if fmt != "e8m0" else np.float32(1.0)
    y = oracle.dequantize(q, s, float(g), block, fmt)
    yb = oracle.dequantize(q, s, float(g), block, fmt, out="bf16")
    for r in range(4):
        for c in range(block * 2 * 2):
            code = (q[r, c // 2] >> (4 * (c & 1))) & 0xF
            exact = (Fraction(oracle.e2m1_decode(code)) * Fraction(oracle.scale_decode(fmt, int(s[r, c // block])))
                     * Fraction(float(g)))
            want = np.float32(float(exact)) if abs(exact) < 2**128 else np.float32(np.inf) * np.sign(float(exact))
            assert y[r, c] == want or (np.isinf(want) and np.isinf(y[r, c]))
            if np.isfinite(y[r, c]):
                wb = torch.tensor(float(y[r, c]), dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item() & 0xFFFF
                assert yb[r, c] == wb


def test_gemm_reference_exact_integer_case_and_orientation():
    # E8M0 scales at 2^0 and g = 1: 2*value is an integer, so C is an exact
    # rational computed with Python integers; M != N catches a transpose
    rng = np.random.default_rng(10)
    M, N, K = 5, 7, 64
    qa = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    qb = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sa = np.full((M, K // 32), 127, dtype=np.uint8)
    sb = np.full((N, K // 32), 128, dtype=np.uint8)        # x2
    a = oracle.dequantize_f64(qa, sa, 1.0, 32, "e8m0")
    b = oracle.dequantize_f64(qb, sb, 1.0, 32, "e8m0")
    c, t = oracle.gemm_ref(a, b)

    def val(qq, r, k):
        code = (qq[r, k // 2] >> (4 * (k & 1))) & 0xF
        mag = [0, 1, 2, 3, 4, 6, 8, 12][code & 7]       # 2 * E2M1 magnitude
        return -mag if code & 8 else mag
    for i in range(M):
        for j in range(N):
            # a = val_a / 2 and b = 2 * (val_b / 2), so 2 * C = sum val_a * val_b
            exact = sum(val(qa, i, k) * val(qb, j, k) for k in range(K))
            assert c[i, j] * 2 == exact
            absum = sum(abs(val(qa, i, k) * val(qb, j, k)) for k in range(K))
            assert t[i, j] == pytest.approx(1e-5 * absum / 2, rel=1e-12)


def test_gemm_check_bracket():
    c_ref = np.array([1.0, 100.0, -3.3, 0.0])
    tol = np.array([1e-5, 1e-3, 1e-5, 0.0])
    exact = oracle.round_to_bf16(c_ref)
    assert oracle.gemm_check(exact, c_ref, tol).all()
    off = exact + np.array([2**-6, 1.0, 2**-5, 2**-130])      # two bf16 ulps away or more
    assert not oracle.gemm_check(off, c_ref, tol).any()


# ---------------------------------------------------------------------------
# column-wise (transposed) quantization: the backward-pass operands
# ---------------------------------------------------------------------------
def _nib(q, r, c):
    return (int(q[r, c // 2]) >> (4 * (c & 1))) & 0xF


@pytest.mark.parametrize("block", [16, 32])
def test_transposed_blocks_run_down_columns_closed_form(block):
    # column c of x holds +-6 * 2^(c-8) with the sign alternating down the
    # rows: blocked down the columns every block maximum is 6 * 2^(c-8), so
    # the E8M0 code of output row c is 127 + (c - 8) (floor(log2(6 * 2^k)) -
    # 2 = k) and every element encodes to +-6.  Blocking along the rows of x
    # instead would mix columns of different magnitude in one block.
    R, C = 2 * block, 24
    mag = 6.0 * 2.0 ** (np.arange(C) - 8.0)
    sign = np.where(np.arange(R) % 2 == 0, 1.0, -1.0)
    x = (sign[:, None] * mag[None, :]).astype(np.float32)
    q, s, g, a = oracle.quantize_transposed_tensor(x, block, "e8m0", "none")
    assert q.shape == (C, R // 2) and s.shape == (C, R // block)
    assert (g, a) == (1.0, 0.0)
    for c in range(C):
        assert np.all(s[c] == 127 + c - 8)
        for r in range(R):
            assert _nib(q, c, r) == (7 | (8 if r % 2 else 0))


def test_transposed_tensor_max_invariant():
    # current E4M3 tensor scale: the output block holding the maximum takes
    # code 0x7E (448) and the maximum itself encodes to +-6, at the transposed
    # position (row = column of x, element = row of x)
    x = _sweep_like(96, 48, 21, bf16=False)
    q, s, g, a = oracle.quantize_transposed_tensor(x, 16, "e4m3", "current")
    r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert a == float(np.abs(x).max()) and g == np.float32(a) / np.float32(2688.0)
    assert s[c, r // 16] == 0x7E
    nib = _nib(q, c, r)
    assert nib & 7 == 7 and (nib >> 3) == (x[r, c] < 0)


def test_transposed_stochastic_counter_uses_transposed_index():
    # every block of x^T holds one 4 (E8M0 code 127, scale 1) and otherwise
    # 0.75, the midpoint of 0.5 and 1: that element rounds up iff its 16
    # random bits are below 2^15, the bits of logical index i = c * R + r
    R, C, seed, offset = 32, 8, 0xC0FFEE, 9
    x = np.full((R, C), 0.75, dtype=np.float32)
    x[0::16, :] = 4.0
    q, s, _, _ = oracle.quantize_transposed_tensor(x, 16, "e8m0", "none", stochastic=True, seed=seed,
                                                   offset=offset)
    assert np.all(s == 127)
    ups = 0
    for c in range(C):
        for r in range(R):
            if r % 16 == 0:
                assert _nib(q, c, r) == 6                 # 4 is on the grid
                continue
            want = 2 if oracle.sr_bits(seed, offset, c * R + r) < 0x8000 else 1
            assert _nib(q, c, r) == want, (r, c)
            ups += want == 2
    assert 0 < ups < C * (R - 2)


# ---------------------------------------------------------------------------
# blockwise randomized Hadamard transform (applied before quantization)
# ---------------------------------------------------------------------------
def _sylvester(n):
    i = np.arange(n)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def test_rht_norm_correctly_rounded():
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    assert oracle.rht_norm(16) == 0.25
    c = np.float32(oracle.rht_norm(32))
    t = Decimal(1) / Decimal(32).sqrt()
    for nb in (np.nextafter(c, np.float32(0)), np.nextafter(c, np.float32(1))):
        assert abs(Decimal(float(c)) - t) < abs(Decimal(float(nb)) - t)


@pytest.mark.parametrize("block", [16, 32])
def test_rht_matches_sylvester_closed_form(block):
    # integer inputs keep every butterfly sum exact, so the binary32 result
    # is the closed-form matrix product times c_B, rounded once
    rng = np.random.default_rng(40 + block)
    rows, cols = 6, 4 * block
    x = rng.integers(-50, 51, (rows, cols)).astype(np.float32)
    signs = int(rng.integers(0, 2**32))
    d = np.array([-1.0 if (signs >> j) & 1 else 1.0 for j in range(block)])
    H = _sylvester(block)
    want = np.empty((rows, cols), dtype=np.float32)
    c = float(np.float32(oracle.rht_norm(block)))
    for r in range(rows):
        for b0 in range(0, cols, block):
            want[r, b0:b0 + block] = ((H @ (d * x[r, b0:b0 + block].astype(np.float64))) * c).astype(np.float32)
    got = oracle.rht_forward(x, block, signs)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("block", [16, 32])
def test_rht_signs_apply_before_the_transform(block):
    # a unit vector at position j with bit j set maps to -c * column j of H
    # (D after H would flip entries by row instead)
    c = np.float32(oracle.rht_norm(block))
    H = _sylvester(block)
    for j in (0, 3, block - 1):
        x = np.zeros((1, block), dtype=np.float32)
        x[0, j] = 1.0
        signs = (1 << j) | (1 << ((j + 5) % block))
        y = oracle.rht_forward(x, block, signs)
        assert np.array_equal(y[0], (-H[:, j] * c).astype(np.float32))


@pytest.mark.parametrize("block", [16, 32])
def test_rht_inverse_is_orthogonal_inverse(block):
    rng = np.random.default_rng(7 + block)
    x = (rng.standard_normal((20, 8 * block)) * 0.02).astype(np.float32)
    signs = 0xA5C3_1E77
    y = oracle.rht_forward(x, block, signs)
    back = oracle.rht_inverse(y, block, signs)
    # orthogonal up to binary32 rounding: relative error a few ulps of the block norm
    err = np.abs(back.astype(np.float64) - x)
    nrm = np.sqrt((x.astype(np.float64).reshape(20, -1, block) ** 2).sum(-1, keepdims=True))
    assert (err.reshape(20, -1, block) <= 8 * 2.0 ** -24 * nrm).all()
    # Parseval: block norms are preserved
    ny = np.sqrt((y.astype(np.float64).reshape(20, -1, block) ** 2).sum(-1))
    assert np.allclose(ny, nrm[..., 0], rtol=1e-6)
    if block == 16:
        xi = rng.integers(-1000, 1001, (4, 64)).astype(np.float32)
        assert np.array_equal(oracle.rht_inverse(oracle.rht_forward(xi, 16, signs), 16, signs), xi)


def test_rht_quantize_uses_transformed_tensor_max():
    # with the transform, the tensor maximum is that of the transformed
    # values: the block holding it takes the largest E4M3 code and encodes
    # to +-6 there
    x = _sweep_like(32, 256, 23, bf16=False)
    signs = 0x0F0F_3C3C
    q, s, g, a = oracle.quantize_tensor(x, 16, "e4m3", "current", rht_signs=signs)
    y = oracle.rht_forward(x, 16, signs)
    assert a == float(np.abs(y).max()) and a != float(np.abs(x).max())
    r, c = np.unravel_index(np.argmax(np.abs(y)), y.shape)
    assert s[r, c // 16] == 0x7E
    nib = (int(q[r, c // 2]) >> (4 * (c & 1))) & 0xF
    assert nib & 7 == 7 and (nib >> 3) == (y[r, c] < 0)


@pytest.mark.parametrize("block,fmt", [(16, "e4m3"), (32, "e8m0")])
def test_rht_dequantize_error_equals_transformed_error(block, fmt):
    # the inverse transform is orthogonal, so the reconstruction error of x
    # per block equals the quantization error of the transformed block
    x = _sweep_like(16, 512, 29, bf16=False)
    signs = 0x1234_5678
    pol = "none" if fmt == "e8m0" else "current"
    q, s, g, _ = oracle.quantize_tensor(x, block, fmt, pol, rht_signs=signs)
    y = oracle.rht_forward(x, block, signs).astype(np.float64)
    yh = oracle.dequantize(q, s, g, block, fmt).astype(np.float64)
    xh = oracle.dequantize_rht(q, s, g, block, fmt, signs).astype(np.float64)
    e_y = np.sqrt(((yh - y).reshape(16, -1, block) ** 2).sum(-1))
    e_x = np.sqrt(((xh - x).reshape(16, -1, block) ** 2).sum(-1))
    scale = np.sqrt((x.astype(np.float64).reshape(16, -1, block) ** 2).sum(-1))
    assert np.all(np.abs(e_x - e_y) <= 1e-6 * scale + 1e-30)
    bf = oracle.dequantize_rht(q, s, g, block, fmt, signs, out="bf16")
    assert np.array_equal(bf, oracle.f32_to_bf16_bits(xh.astype(np.float32)).reshape(bf.shape))


# ---------------------------------------------------------------------------
# INT4 element grid (NVINT4 / MXINT4)
# ---------------------------------------------------------------------------
def test_int4_decode_is_twos_complement():
    for code in range(16):
        assert oracle.int4_decode(code) == float(np.array([code << 4], dtype=np.uint8).view(np.int8)[0] >> 4)


def test_int4_rtn_matches_numpy_rint():
    # numpy's rint rounds half to even; the grid saturates at 7
    centres = [k + 0.5 for k in range(8)] + list(range(9))
    pieces = []
    for c in centres:
        b = np.float32(c).view(np.uint32).astype(np.int64)
        pieces.append(np.arange(max(b - 2048, 0), b + 2049, dtype=np.int64))
    pieces.append(np.arange(0, 0x41400000, 1013, dtype=np.int64))
    bits = np.unique(np.concatenate(pieces)).astype(np.uint32)
    v = bits.view(np.float32)
    want = np.minimum(np.rint(v.astype(np.float64)), 7).astype(int)
    got = np.array([oracle.int4_rtn(float(x)) for x in v[::7]])
    assert np.array_equal(got, want[::7])
    for x in (-3.5, -2.5, 0.5, 1.5, 6.5, 7.49, 100.0):
        assert oracle.int4_rtn(x) == min(int(np.rint(abs(x))), 7)


@pytest.mark.parametrize("v", [0.3, 1.0, 2.75, 4.5, 6.999, -5.25, 7.0, 9.0])
def test_int4_sr_exact_expectation(v):
    # over all 2^16 random values the mean code is lo + ceil(frac 2^16) / 2^16
    a = abs(v)
    mags = np.array([oracle.int4_sr(v, r) for r in range(0, 65536, 1)])
    if a >= 7:
        assert np.all(mags == 7)
        return
    lo = np.floor(a)
    frac = a - lo
    assert set(np.unique(mags)) <= {int(lo), int(lo) + 1}
    assert (mags == lo + 1).sum() == int(np.ceil(np.float64(np.float32(frac)) * 65536))


def test_int4_tensor_max_maps_to_seven():
    x = _sweep_like(48, 256, 31, bf16=False)
    for fmt in ("e4m3", "ue5m3"):
        q, s, g, a = oracle.quantize_tensor(x, 16, fmt, "current", elem="int4")
        assert g == np.float32(a) / (np.float32(7.0) * np.float32(oracle.scale_max(fmt)))
        r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
        n = 256 if fmt == "ue5m3" else 128
        assert s[r, c // 16] == max(cc for cc in range(n) if not oracle.scale_is_nan(fmt, cc))
        nib = (int(q[r, c // 2]) >> (4 * (c & 1))) & 0xF
        assert oracle.int4_decode(nib) == (7.0 if x[r, c] > 0 else -7.0)


def test_int4_e8m0_blocks_are_exact_nearest():
    # MX rule: code = floor(log2 amax_b) - 2 + 127, so x / s is exact and the
    # element is the nearest-even integer of it, clamped to +-7
    x = _sweep_like(8, 256, 33, bf16=False)
    q, s, g, _ = oracle.quantize_tensor(x, 32, "e8m0", "none", elem="int4")
    assert g == 1.0
    for r in range(8):
        for b in range(8):
            blk = x[r, 32 * b:32 * b + 32].astype(np.float64)
            am = np.abs(blk).max()
            assert s[r, b] == int(np.floor(np.log2(am))) - 2 + 127
            scaled = blk * 2.0 ** (127 - int(s[r, b]))
            want = np.clip(np.rint(scaled), -7, 7)
            for k in range(32):
                col = 32 * b + k
                nib = (int(q[r, col // 2]) >> (4 * (col & 1))) & 0xF
                assert oracle.int4_decode(nib) == want[k]


def test_int4_dequantize_exact_product_and_gemm_orientation():
    rng = np.random.default_rng(3)
    q = rng.integers(0, 256, (6, 32), dtype=np.uint8)
    s = rng.integers(0x30, 0x60, (6, 4), dtype=np.uint8)
    g = np.float32(0.0371)
    y = oracle.dequantize(q, s, float(g), 16, "e4m3", elem="int4")
    yd = oracle.dequantize_f64(q, s, float(g), 16, "e4m3", elem="int4")
    for r in range(6):
        for c in range(64):
            code = (int(q[r, c // 2]) >> (4 * (c & 1))) & 0xF
            sv = oracle.scale_decode("e4m3", int(s[r, c // 16]))
            exact = Fraction(oracle.int4_decode(code)) * Fraction(sv) * Fraction(float(g))
            assert Fraction(float(yd[r, c])) == exact           # exact in binary64
            t = np.float32(np.float32(oracle.int4_decode(code)) * np.float32(sv))
            assert y[r, c] == np.float32(t * g)


# ---------------------------------------------------------------------------
# 8-bit MX element grids (MXFP8 with E4M3 elements, MXINT8)
# ---------------------------------------------------------------------------
def test_e8m0_emax_rule_closed_form():
    rng = np.random.default_rng(81)
    for emax in (2, 6, 8):
        for a in np.exp(rng.uniform(np.log(1e-20), np.log(1e20), 400)).astype(np.float32):
            c = oracle.e8m0_block_code_emax(float(a), emax)
            s = 2.0 ** (c - 127)
            assert 2.0 ** emax * s <= float(a) < 2.0 ** (emax + 1) * s
    assert oracle.e8m0_block_code_emax(0.0, 8) == 0


def _unit_scale_blocks(rng, rows, lim, top):
    # 32-element blocks whose maximum |x| is `top` in [2^emax, 2^(emax+1)), so
    # the E8M0 code is 127 (scale exactly 1) and the elements are encoded as is
    x = rng.uniform(-lim, lim, (rows, 32 * 8)).astype(np.float32)
    x[:, ::32] = np.float32(top)
    return x


def test_fp8_elements_match_torch_float8_e4m3fn():
    rng = np.random.default_rng(82)
    x = _unit_scale_blocks(rng, 16, 448.0, 300.0)
    x[:, 5] = 0.0
    x[:, 6] = -0.0
    x[:, 7] = np.float32(1e-5)                          # below half the smallest subnormal
    q, s, g, _ = oracle.quantize_tensor(x, 32, "e8m0", "none", elem="fp8_e4m3")
    assert np.all(s == 127) and g == 1.0
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, want)


def test_int8_elements_match_numpy_rint():
    rng = np.random.default_rng(83)
    x = _unit_scale_blocks(rng, 16, 127.0, 100.0)
    x[:, 9] = np.float32(2.5)
    x[:, 10] = np.float32(-3.5)
    q, s, g, _ = oracle.quantize_tensor(x, 32, "e8m0", "none", elem="int8")
    assert np.all(s == 127)
    want = np.clip(np.rint(x.astype(np.float64)), -127, 127).astype(np.int8).view(np.uint8)
    assert np.array_equal(q, want)
    for code in range(256):
        assert oracle.int8_decode(code) == float(np.array([code], dtype=np.uint8).view(np.int8)[0])


@pytest.mark.parametrize("v", [0.3, 17.75, 126.9, -44.1, 200.0])
def test_int8_sr_exact_expectation(v):
    mags = np.array([oracle.int8_sr(v, r) for r in range(65536)])
    a = abs(v)
    if a >= 127:
        assert np.all(mags == 127)
        return
    lo = np.floor(np.float32(a))
    frac = np.float64(np.float32(a)) - lo
    assert set(np.unique(mags)) <= {int(lo), int(lo) + 1}
    assert (mags == lo + 1).sum() == int(np.ceil(frac * 65536))


def test_fp8_sr_rounds_between_grid_neighbours():
    # E8M0 block 32 with scale 1 (block maximum 300): 100.5 lies between the
    # E4M3 neighbours 96 and 104 (spacing 8), frac = 4.5 / 8; every block is
    # seeded differently, so the up fraction approaches 0.5625
    x = np.full((64, 256), 100.5, dtype=np.float32)
    x[:, ::32] = 300.0
    q, s, _, _ = oracle.quantize_tensor(x, 32, "e8m0", "none", elem="fp8_e4m3", stochastic=True, seed=9,
                                        offset=0)
    vals = torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).float().numpy()
    mid = vals[:, [c for c in range(256) if c % 32]]
    assert set(np.unique(mid)) <= {96.0, 104.0}
    frac_up = float((mid == 104.0).mean())
    assert abs(frac_up - 4.5 / 8) < 0.02


@pytest.mark.parametrize("elem,qmax", [("fp8_e4m3", 448.0), ("int8", 127.0)])
def test_8bit_tensor_max_maps_to_grid_max(elem, qmax):
    x = _sweep_like(32, 256, 84, bf16=False)
    q, s, g, a = oracle.quantize_tensor(x, 16, "e4m3", "current", elem=elem)
    assert g == np.float32(a) / (np.float32(qmax) * np.float32(448.0))
    r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert s[r, c // 16] == 0x7E
    if elem == "fp8_e4m3":
        v = float(torch.tensor([int(q[r, c])], dtype=torch.uint8).view(torch.float8_e4m3fn).float()[0])
    else:
        v = oracle.int8_decode(int(q[r, c]))
    assert v == (qmax if x[r, c] > 0 else -qmax)


@pytest.mark.parametrize("elem", ["fp8_e4m3", "int8"])
def test_8bit_dequantize_exact_product(elem):
    rng = np.random.default_rng(85)
    q = rng.integers(0, 256, (4, 64), dtype=np.uint8)
    if elem == "fp8_e4m3":
        q[(q & 0x7F) == 0x7F] = 0x11                      # no NaN codes
    s = rng.integers(0x30, 0x60, (4, 4), dtype=np.uint8)
    g = np.float32(0.0173)
    y = oracle.dequantize(q, s, float(g), 16, "e4m3", elem=elem)
    for r in range(4):
        for c in range(64):
            if elem == "fp8_e4m3":
                e = float(torch.tensor([int(q[r, c])], dtype=torch.uint8).view(torch.float8_e4m3fn).float()[0])
            else:
                e = float(np.array([q[r, c]], dtype=np.uint8).view(np.int8)[0])
            sv = oracle.scale_decode("e4m3", int(s[r, c // 16]))
            assert y[r, c] == np.float32(np.float32(np.float32(e) * np.float32(sv)) * g)


# ---------------------------------------------------------------------------
# 6-bit MX element grids (MXFP6 with FP6 E2M3 / E3M2 elements, MXINT6)
# ---------------------------------------------------------------------------
def _fp6_values(elem):
    """Signed values of the 64 FP6 codes, written out from the format
    definitions: E2M3 = 1 sign, 2 exponent (bias 1), 3 mantissa bits; E3M2 =
    1 sign, 3 exponent (bias 3), 2 mantissa bits; exponent 0 is subnormal and
    every code is finite."""
    eb, mb, bias = (2, 3, 1) if elem == "fp6_e2m3" else (3, 2, 3)
    out = []
    for code in range(64):
        mag = code & 31
        e, m = mag >> mb, mag & ((1 << mb) - 1)
        v = Fraction(m, 1 << mb) * Fraction(2) ** (1 - bias) if e == 0 else \
            (1 + Fraction(m, 1 << mb)) * Fraction(2) ** (e - bias)
        out.append(-v if code & 32 else v)
    return out


def _unpack6(q, cols):
    """Independent bit-stream unpack: element c of a row at bits 6c..6c+5
    (little-endian over the row's bytes)."""
    out = np.zeros((q.shape[0], cols), dtype=np.int64)
    for r in range(q.shape[0]):
        big = int.from_bytes(bytes(q[r]), "little")
        for c in range(cols):
            out[r, c] = (big >> (6 * c)) & 63
    return out


def test_fp6_format_facts():
    for elem, top, sub, norm in [("fp6_e2m3", 7.5, 0.125, 1.0), ("fp6_e3m2", 28.0, 0.0625, 0.25)]:
        vals = _fp6_values(elem)
        pos = sorted(set(v for v in vals[:32]))
        assert len(pos) == 32 and pos[0] == 0 and max(pos) == top
        assert pos[1] == sub                     # smallest subnormal
        assert min(v for v in pos if v >= norm) == norm


@pytest.mark.parametrize("elem", ["fp6_e2m3", "fp6_e3m2"])
def test_fp6_dequantize_decodes_every_code(elem):
    # every code in a row with E8M0 scale 1: the oracle's values are the
    # definition's
    q_codes = np.arange(64, dtype=np.int64).reshape(1, 64)
    big = 0
    for c in range(64):
        big |= int(q_codes[0, c]) << (6 * c)
    q = np.frombuffer(big.to_bytes(48, "little"), dtype=np.uint8).reshape(1, 48).copy()
    s = np.full((1, 2), 127, dtype=np.uint8)
    y = oracle.dequantize_f64(q, s, 1.0, 32, "e8m0", elem=elem)
    want = [float(v) for v in _fp6_values(elem)]
    assert np.array_equal(y[0], np.array(want))


@pytest.mark.parametrize("elem,top,emax", [("fp6_e2m3", 6.0, 2), ("fp6_e3m2", 20.0, 4)])
def test_fp6_rtn_is_brute_force_nearest(elem, top, emax):
    # blocks whose maximum is in [2^emax, 2^(emax+1)) get the E8M0 scale 1;
    # each element must be the nearest FP6 value (ties to the even code,
    # saturating at the top), found by brute force over the 32 magnitudes
    rng = np.random.default_rng(91)
    vals = _fp6_values(elem)
    pos = [float(v) for v in vals[:32]]
    mids = [(pos[i] + pos[i + 1]) / 2 for i in range(31)]
    extra = np.array(mids + pos + [pos[-1] * 1.01, 0.999 * 2.0 ** (emax + 1)], dtype=np.float32)
    x = rng.uniform(-2 ** (emax + 1), 2 ** (emax + 1), (8, 256)).astype(np.float32)
    flat = x.reshape(-1)
    flat[1:1 + extra.size] = extra
    flat[300:300 + extra.size] = -extra
    x[:, ::32] = np.float32(top)
    q, s, g, _ = oracle.quantize_tensor(x, 32, "e8m0", "none", elem=elem)
    assert np.all(s == 127) and g == 1.0
    codes = _unpack6(q, 256)
    for r in range(8):
        for c in range(256):
            a = abs(float(x[r, c]))
            d = [abs(a - p) for p in pos]
            best = min(d)
            cands = [i for i in range(32) if d[i] == best]
            mag = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
            want = mag | (32 if np.signbit(x[r, c]) else 0)
            assert codes[r, c] == want, (r, c, x[r, c])


def test_int6_rtn_and_layout():
    rng = np.random.default_rng(92)
    x = rng.uniform(-32, 32, (8, 256)).astype(np.float32)
    x[:, ::32] = np.float32(20.0)                        # E8M0 offset 4: scale 1
    x[0, 1:5] = [2.5, -3.5, 31.6, -31.9]
    q, s, g, _ = oracle.quantize_tensor(x, 32, "e8m0", "none", elem="int6")
    assert np.all(s == 127) and q.shape == (8, 192)
    codes = _unpack6(q, 256)
    want = np.clip(np.rint(x.astype(np.float64)), -31, 31).astype(np.int64) & 63
    assert np.array_equal(codes, want)
    y = oracle.dequantize_f64(q, s, 1.0, 32, "e8m0", elem="int6")
    assert np.array_equal(y, np.clip(np.rint(x.astype(np.float64)), -31, 31))


@pytest.mark.parametrize("elem,emax", [("fp6_e2m3", 2), ("fp6_e3m2", 4), ("int6", 4)])
def test_6bit_e8m0_offset_closed_form(elem, emax):
    rng = np.random.default_rng(93)
    x = (rng.standard_normal((16, 256)) * np.exp(rng.uniform(-6, 6, (16, 1)))).astype(np.float32)
    _, s, _, _ = oracle.quantize_tensor(x, 32, "e8m0", "none", elem=elem)
    amax = np.abs(x).reshape(16, 8, 32).max(axis=2).astype(np.float64)
    sc = 2.0 ** (s.astype(np.float64) - 127)
    assert np.all((2.0 ** emax * sc <= amax) & (amax < 2.0 ** (emax + 1) * sc))


@pytest.mark.parametrize("elem,v,lo,hi", [("fp6_e2m3", 2.6, 2.5, 2.75), ("fp6_e3m2", 11.0, 10.0, 12.0),
                                          ("int6", 7.3, 7.0, 8.0)])
def test_6bit_sr_between_neighbours(elem, v, lo, hi):
    x = np.full((64, 256), v, dtype=np.float32)
    x[:, ::32] = np.float32(6.0 if elem == "fp6_e2m3" else 20.0)
    q, s, _, _ = oracle.quantize_tensor(x, 32, "e8m0", "none", elem=elem, stochastic=True, seed=5)
    assert np.all(s == 127)
    y = oracle.dequantize_f64(q, s, 1.0, 32, "e8m0", elem=elem)
    mid = y[:, [c for c in range(256) if c % 32]]
    assert set(np.unique(mid)) <= {lo, hi}
    frac_up = float((mid == hi).mean())
    assert abs(frac_up - (np.float64(np.float32(v)) - lo) / (hi - lo)) < 0.02


@pytest.mark.parametrize("elem,qmax", [("fp6_e2m3", 7.5), ("fp6_e3m2", 28.0), ("int6", 31.0)])
def test_6bit_tensor_max_maps_to_grid_max(elem, qmax):
    x = _sweep_like(32, 256, 94, bf16=False)
    q, s, g, a = oracle.quantize_tensor(x, 16, "e4m3", "current", elem=elem)
    assert g == np.float32(a) / (np.float32(qmax) * np.float32(448.0))
    y = oracle.dequantize_f64(q, s, 1.0, 16, "e4m3", elem=elem)
    r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert s[r, c // 16] == 0x7E
    assert y[r, c] == (qmax if x[r, c] > 0 else -qmax) * 448.0


@pytest.mark.parametrize("elem,f8,shift", [("fp6_e2m3", torch.float8_e4m3fn, -6), ("fp6_e3m2", torch.float8_e5m2, -12)])
def test_fp6_is_scaled_fp8(elem, f8, shift):
    """The identity behind encoding and decoding FP6 with FP8 conversions:
    FP6 E2M3 (E3M2) times 2^-6 (2^-12) is FP8 E4M3 (E5M2) with the same low
    five code bits, and nearest-even FP8 rounding of a scaled value, after
    the clamp to the FP6 maximum, lands on the scaled FP6 nearest-even
    result.  torch's float8 types stand in for the FP8 side; the FP6 side
    is the oracle (itself pinned by brute force above)."""
    vals = [float(v) for v in _fp6_values(elem)[:32]]
    top = vals[-1]
    for code, v in enumerate(vals):
        b = torch.tensor([v * 2.0 ** shift], dtype=torch.float32).to(f8).view(torch.uint8).item()
        assert b == code, (elem, code, v, b)
    mids = [(vals[i] + vals[i + 1]) / 2 for i in range(31)]
    probe = np.array(mids + vals, dtype=np.float32)
    probe = np.concatenate([probe, np.nextafter(probe, np.float32(np.inf)), np.nextafter(probe, np.float32(-np.inf)),
                            np.float32([top * 1.01, top * 1.3])])
    probe = probe[(probe >= 0) & (probe < 2.0 ** (2 if elem == "fp6_e2m3" else 4) * 2)]
    x = np.zeros((1, 32 * (probe.size // 31 + 1)), dtype=np.float32)
    blocks = x.reshape(-1, 32)
    blocks[:, 0] = 2.0 ** (2 if elem == "fp6_e2m3" else 4)            # E8M0 scale 1
    flat = blocks[:, 1:].reshape(-1)
    flat[:probe.size] = probe
    blocks[:, 1:] = flat.reshape(blocks.shape[0], 31)
    x = blocks.reshape(1, -1)
    q, s, _, _ = oracle.quantize_tensor(x, 32, "e8m0", "none", elem=elem)
    assert np.all(s == 127)
    big = int.from_bytes(bytes(q[0]), "little")
    codes = [(big >> (6 * c)) & 63 for c in range(x.shape[1])]
    hw = torch.from_numpy(np.clip(x[0], -top, top) * np.float32(2.0 ** shift)).to(f8).view(torch.uint8).numpy()
    for c in range(x.shape[1]):
        assert codes[c] == (int(hw[c]) & 0x1F) | ((int(hw[c]) >> 2) & 0x20), (elem, c, x[0, c])


# ---------------------------------------------------------------------------
# Exact stochastic-rounding expectation on the FP8 E4M3 and FP6 grids
# (gonzo_ML/3986 "Стохастическая квантизация": up or down with a probability
# set by the distance to the neighbours).  Every one of the 2^16 variates is
# fed in; the set that rounds up must be exactly {r16 < ceil(frac * 2^16)}
# with frac computed here in exact rationals from the format definitions, and
# every result must be one of the two neighbours.  Values whose frac * 2^16 is
# an integer separate "u < frac" from "u <= frac"; values at and beyond the
# largest finite magnitude check the saturation; subnormal values and values
# next to a power of two check the binade and subnormal neighbours.
# ---------------------------------------------------------------------------
def _e4m3_magnitudes():
    """Non-negative FP8 E4M3 values written out from the definition: 4
    exponent bits (bias 7), 3 mantissa bits, exponent 0 subnormal, the
    all-ones code 0x7F NaN (so 0x7E = 448 is the largest finite)."""
    out = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        out.append(Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    return out


def test_e4m3_magnitudes_agree_with_torch():
    mags = _e4m3_magnitudes()
    assert mags[-1] == 448 and mags[1] == Fraction(1, 512)
    dec = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert [Fraction(float(v)) for v in dec] == mags


_SR_PROBES = {
    "fp8_e4m3": [100.5, -100.5, 0.3, 2.0 ** -10, 3 * 2.0 ** -9 + 2.0 ** -11, 2.0 ** -30, 1.0 + 1.0 / 24,
                 float(np.nextafter(np.float32(2.0), np.float32(0))), 2.0, 0.0, 440.0, 447.9, 448.0, 449.0, 500.0,
                 1e6, 0.015625 + 2.0 ** -12],
    "fp6_e2m3": [2.6, -2.6, 0.0625, 0.01, float(np.nextafter(np.float32(1.0), np.float32(0))), 1.0, 7.25, 7.4, 7.5,
                 8.0, 100.0, 0.0, 3.3, 2.0 ** -20],
    "fp6_e3m2": [11.0, -11.0, 0.03125, 0.2, float(np.nextafter(np.float32(4.0), np.float32(0))), 4.0, 26.0, 27.9,
                 28.0, 29.0, 1e5, 0.0, 0.3, 2.0 ** -20],
}


def _grid(elem):
    if elem == "fp8_e4m3":
        return _e4m3_magnitudes()
    return [v for v in _fp6_values(elem)[:32]]


@pytest.mark.parametrize("elem", ["fp8_e4m3", "fp6_e2m3", "fp6_e3m2"])
def test_fp8_fp6_sr_exact_enumeration(elem):
    grid = _grid(elem)
    top = len(grid) - 1
    r16 = np.arange(65536, dtype=np.uint32)
    for v in _SR_PROBES[elem]:
        v32 = np.float32(v)
        mags = oracle.elem_mag_array(np.full(65536, v32, dtype=np.float32), elem, r16)
        a = abs(Fraction(float(v32)))
        if a >= grid[top]:
            assert np.all(mags == top), (elem, v)
            continue
        lo = max(i for i in range(top + 1) if grid[i] <= a)
        frac = (a - grid[lo]) / (grid[lo + 1] - grid[lo])
        n_up = math.ceil(frac * 65536)
        assert set(np.unique(mags).tolist()) <= {lo, lo + 1}, (elem, v)
        up = mags == lo + 1
        assert np.array_equal(np.nonzero(up)[0], np.arange(n_up)), (elem, v, n_up, int(up.sum()))


@pytest.mark.parametrize("elem", ["fp8_e4m3", "fp6_e2m3", "fp6_e3m2"])
def test_fp8_fp6_rtn_saturates_explicitly(elem):
    # nearest rounding at and beyond the largest finite magnitude gives its
    # code (never the NaN code 0x7F of E4M3)
    grid = _grid(elem)
    top = len(grid) - 1
    v = np.array([float(grid[top]), float(grid[top]) * 1.01, 1e9, 3e38], dtype=np.float32)
    assert np.all(oracle.elem_mag_array(v, elem) == top)
    assert np.all(oracle.elem_mag_array(-v, elem) == top)


@pytest.mark.parametrize("fmt", ["e4m3", "ue5m3", "e3m4", "e1m6", "e2m5", "e5m2", "e6m1", "e7m0"])
def test_scale_encode_saturates_far_above_the_top(fmt):
    # the largest finite code, also where binary64 can no longer tell the
    # distances to the two largest values apart
    top = max(c for c in range(256 if fmt == "ue5m3" else 128) if not oracle.scale_is_nan(fmt, c))
    for u in (oracle.scale_max(fmt), oracle.scale_max(fmt) * 1.5, 1e30, 3e38):
        assert oracle.scale_encode(fmt, u) == top, (fmt, u)


def test_sr_boundary_tensor_hits_both_outcomes():
    """The GPU boundary test's tensor (every element next to its own SR
    decision boundary) does exercise both outcomes in the oracle."""
    from tests.test_sr_boundary_gpu import SEED, OFFSET, _boundary_tensor
    x = _boundary_tensor(64, 256, SEED, OFFSET)
    q, _ = oracle.quantize(x, 32, "e8m0", 1.0, stochastic=True, seed=SEED, offset=OFFSET)
    qn, _ = oracle.quantize(x, 32, "e8m0", 1.0)
    assert ((q & 15) != (qn & 15)).any() and ((q & 15) == (qn & 15)).any()
