"""Helpers shared by the GPU tests: numpy <-> torch device transfers and the
mapping of test parameters onto the oracle and onto the C ABI binding."""
import numpy as np
import torch


def to_device(x: np.ndarray) -> torch.Tensor:
    """float32 arrays stay fp32; uint16 arrays are bf16 bit patterns."""
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()
    if x.dtype == np.float32:
        return torch.from_numpy(x.copy()).cuda()
    raise TypeError(x.dtype)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_bytes_equal(got: np.ndarray, want: np.ndarray, what: str):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    if bad.size:
        idx = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches; first at {idx}: got {got[idx]!r} want {want[idx]!r}")


def f32_bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).view(np.uint32)
