"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

Holds no quantization arithmetic: only random draws and the RNE casts
fp64 -> fp32 -> bf16 that turn them into input tensors.  Both the oracle side
and the HIP side receive the same arrays from here.

Workloads (shapes follow the pages' models: Llama-2 7B from the "FP4 all the
way" review, Qwen-2.5 from the NVFP4 weight-only RL post; the pages publish no
tensors, so the values are synthetic):

  small    A 64x256 N(0,1) (seed 2); B 256x256 fp32 N(0,1) with 1% of entries
           x50 (seed 1).
  sweep    4096x4096 bf16 N(0, 0.02) with 0.1% of entries x100 (seed 3).
  grads    8192x8192 bf16 Laplace(0, b=1e-4), tensor t drawn from seed 1000+t.
  llama    A 8192x4096, W_up [11008, 4096], W_down [4096, 11008],
           W_sq [4096, 4096], all bf16 N(0, 0.02) (seeds 4, 5, 6, 7).
  decode   W_up [18944, 3584] (seed 8), W_down [3584, 18944] (seed 9) bf16
           N(0, 0.02); X [M, K] bf16 N(0, 1) (seed 10 + M), M in {1, 8, 16}.

Host generation uses numpy's PCG64 (exact, used for parity).  Device
generation for the large benchmark rotations uses torch's seeded CUDA
generator with the same distributions (used only for timing).
"""
from __future__ import annotations

import numpy as np

SEEDS = {"small_b": 1, "small_a": 2, "sweep": 3, "llama_a": 4, "llama_up": 5, "llama_down": 6,
         "llama_sq": 7, "decode_up": 8, "decode_down": 9}
GRADS_SEED0 = 1000


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """RNE cast fp32 -> bf16, returned as uint16 bit patterns (via torch)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal(shape, std: float, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape, dtype=np.float64) * std


def with_outliers(x64: np.ndarray, p: float, factor: float, seed: int) -> np.ndarray:
    """Scale a Bernoulli(p) subset of the entries by `factor`."""
    rng = np.random.default_rng(seed + 0x5F5F)
    mask = rng.random(x64.shape) < p
    y = x64.copy()
    y[mask] *= factor
    return y


def small_b() -> np.ndarray:
    """256x256 fp32 N(0,1), 1% of entries x50."""
    return with_outliers(normal((256, 256), 1.0, SEEDS["small_b"]), 0.01, 50.0,
                         SEEDS["small_b"]).astype(np.float32)


def small_a() -> np.ndarray:
    """64x256 fp32 N(0,1)."""
    return normal((64, 256), 1.0, SEEDS["small_a"]).astype(np.float32)


def sweep(rows: int = 4096, cols: int = 4096) -> np.ndarray:
    """bf16 bits, N(0, 0.02) with 0.1% of entries x100."""
    x = with_outliers(normal((rows, cols), 0.02, SEEDS["sweep"]), 0.001, 100.0, SEEDS["sweep"])
    return f32_to_bf16_bits(x.astype(np.float32))


def grads(t: int, rows: int = 8192, cols: int = 8192) -> np.ndarray:
    """bf16 bits, Laplace(0, 1e-4), tensor t of the successive sequence."""
    rng = np.random.default_rng(GRADS_SEED0 + t)
    x = rng.laplace(0.0, 1e-4, size=(rows, cols))
    return f32_to_bf16_bits(x.astype(np.float32))


def llama(name: str, shapes: dict | None = None) -> np.ndarray:
    """bf16 bits for one Llama-2 7B linear operand: 'a', 'up', 'down', 'sq'."""
    shapes = shapes or {"a": (8192, 4096), "up": (11008, 4096), "down": (4096, 11008), "sq": (4096, 4096)}
    seed = SEEDS["llama_" + name]
    return f32_to_bf16_bits(normal(shapes[name], 0.02, seed).astype(np.float32))


def decode_weight(name: str) -> np.ndarray:
    """bf16 bits: 'up' [18944, 3584] or 'down' [3584, 18944], N(0, 0.02)."""
    shape = {"up": (18944, 3584), "down": (3584, 18944)}[name]
    return f32_to_bf16_bits(normal(shape, 0.02, SEEDS["decode_" + name]).astype(np.float32))


def decode_x(m: int, k: int) -> np.ndarray:
    """bf16 bits, activations [m, k] N(0, 1), seed 10 + m."""
    return f32_to_bf16_bits(normal((m, k), 1.0, 10 + m).astype(np.float32))


def device_normal(shape, std: float, seed: int, dtype, device="cuda"):
    """Seeded device-side draw (torch CUDA generator) for large timing runs."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std).to(dtype)


def device_laplace(shape, scale: float, seed: int, dtype, device="cuda"):
    """Seeded device-side Laplace(0, scale) by inverse CDF of a uniform draw."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    u = torch.rand(shape, generator=g, device=device, dtype=torch.float32) - 0.5
    x = -scale * torch.sign(u) * torch.log1p(-2.0 * u.abs())
    return x.to(dtype)


def device_outliers(x, p: float, factor: float, seed: int):
    import torch
    g = torch.Generator(device=x.device)
    g.manual_seed(seed + 0x5F5F)
    m = torch.rand(x.shape, generator=g, device=x.device) < p
    return torch.where(m, x.float() * factor, x.float()).to(x.dtype)
