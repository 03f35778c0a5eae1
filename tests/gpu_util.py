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


def check_gemm_every_output(c_gpu: torch.Tensor, a_hat: np.ndarray, w_hat: np.ndarray, tag: str, block_rows=1024):
    """Every bf16 output of C = A W^T within the oracle's bound (the bf16
    rounding of some value within 1e-5 * sum_k |a||w| of the binary64
    product), the reference taken 1024 rows at a time to bound its memory."""
    import oracle
    c = c_gpu.float().cpu().numpy().astype(np.float64)
    wt, wabs = np.ascontiguousarray(w_hat.T), np.ascontiguousarray(np.abs(w_hat).T)
    for r0 in range(0, c.shape[0], block_rows):
        ab = a_hat[r0:r0 + block_rows]
        cref = ab @ wt
        tol = 1e-5 * (np.abs(ab) @ wabs)
        ok = oracle.gemm_check(c[r0:r0 + block_rows], cref, tol)
        if not ok.all():
            i, j = np.argwhere(~ok)[0]
            raise AssertionError(f"{tag}: {int((~ok).sum())} outputs in rows {r0}.. out of tolerance; first "
                                 f"({r0 + i},{j}) got {c[r0 + i, j]!r} ref {cref[i, j]!r} tol {tol[i, j]!r}")
