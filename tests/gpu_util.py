"""Shared helpers of the GPU parity tests (host <-> device copies, byte compares)."""
import numpy as np
import torch


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> int16 device tensor holding the same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def assert_same(got, want, what: str):
    got = to_host(got) if isinstance(got, torch.Tensor) else got
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if np.array_equal(got, want):
        return
    bad = np.argwhere(got != want)
    first = [(tuple(int(i) for i in ix), int(got[tuple(ix)]), int(want[tuple(ix)]))
             for ix in bad[:8]]
    raise AssertionError(f"{what}: {len(bad)} of {want.size} differ; first (index, gpu, oracle): {first}")


def assert_dbias_close(got, want, y_abs_colsum, what: str = "dbias"):
    """|g - r| <= 1e-3 |r| + 1e-6 sum_m |y[m][k]| (fp32 summation order differs
    from the oracle's double sum; the second term only matters where the
    column sum cancels to near zero)."""
    got = to_host(got).astype(np.float64) if isinstance(got, torch.Tensor) else got
    want = want.astype(np.float64)
    tol = 1e-3 * np.abs(want) + 1e-6 * y_abs_colsum
    bad = np.abs(got - want) > tol
    assert not bad.any(), (what, int(bad.sum()), np.argwhere(bad)[:5].ravel(), got[bad][:5], want[bad][:5])


def mx_outputs_equal(g: dict, o: dict, what: str, keys=("q_row", "s_row", "q_col", "s_col")):
    for k in keys:
        if o.get(k) is None:
            continue
        assert_same(g[k], o[k], f"{what} {k}")
