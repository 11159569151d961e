"""Helpers shared by the GPU tests (no method arithmetic here)."""
import sys

import numpy as np
import torch

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_MAX_ABS = 1e-4
LSE_MAX_ABS = 1e-3


def announce(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a crash report says which."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def dev(x: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dtype).cuda()


def dev_u8(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, np.uint8)).cuda()


def dev_i32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, np.int32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.float().cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


def assert_close_bf16(got: np.ndarray, ref: np.ndarray, what: str, max_abs=BF16_MAX_ABS, mean_abs=BF16_MEAN_ABS):
    d = np.abs(got - ref)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert d.max() <= max_abs, f"{what}: max-abs {d.max():.3e} > {max_abs}"
    assert d.mean() <= mean_abs, f"{what}: mean-abs {d.mean():.3e} > {mean_abs}"


def assert_lse_close(got: np.ndarray, ref: np.ndarray, what: str, tol=LSE_MAX_ABS):
    fin = np.isfinite(ref)
    assert (np.isfinite(got) == fin).all(), f"{what}: -inf pattern differs"
    if fin.any():
        d = np.abs(got[fin] - ref[fin]).max()
        assert d <= tol, f"{what}: lse max-abs {d:.3e} > {tol}"
