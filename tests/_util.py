"""Shared helpers of the parity tests (no method arithmetic here)."""
import numpy as np
import torch


def dev_bf16(a: np.ndarray, device="cuda:0") -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 device tensor (bit-exact)."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)


def dev(a: np.ndarray, device="cuda:0") -> torch.Tensor:
    if a.dtype == np.uint16:
        return dev_bf16(a, device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_near_tie_sets(gpu_idx: np.ndarray, ora_idx: np.ndarray, pi: np.ndarray, rel: float = 1e-6):
    """Per selection group: GPU and oracle position sets may differ only at
    positions whose oracle score is within `rel` (relative) of the k-th oracle
    score.  Returns the number of differing positions."""
    ndiff = 0
    for g in range(gpu_idx.shape[0]):
        a, b = gpu_idx[g], ora_idx[g]
        assert len(a) == len(b)
        assert np.all(np.diff(a) > 0), "GPU position list not strictly ascending"
        assert a.min() >= 0 and a.max() < pi.shape[1]
        kth = pi[g][b].min()
        diff = np.setxor1d(a, b)
        ndiff += len(diff)
        if len(diff):
            bad = diff[np.abs(pi[g][diff] - kth) > rel * kth]
            assert len(bad) == 0, (f"group {g}: positions {bad[:8]} differ with oracle scores "
                                   f"{pi[g][bad[:8]]} vs k-th {kth}")
    return ndiff


def dev_padded(a: np.ndarray, device="cuda:0") -> torch.Tensor:
    """2-D host array -> device view whose row pitch is rounded up to 16 bytes
    (the library's layout rule); the padding holds NaN, which must never be read."""
    T, K = a.shape
    mult = 8 if a.dtype == np.uint16 else 4
    ld = -(-K // mult) * mult
    if ld == K:
        return dev(a, device)
    fill = 0x7fc0 if a.dtype == np.uint16 else np.nan
    buf = np.full((T, ld), fill, dtype=a.dtype)
    buf[:, :K] = a
    return dev(buf, device)[:, :K]
