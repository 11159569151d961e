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


# Gradients: the kernels round P and dS to bf16 before their products and each
# output once to bf16, and take Delta from the forward's bf16 O. Emulating those
# roundings on random unit-scale inputs against the fp64 definition gives a
# largest error of at most 5e-3 of the tensor's largest magnitude and a mean error
# of about 2.3e-3 of its mean magnitude (8e-3 with 4x larger logits, where the
# softmax is peaked); the bounds below leave about 3x room.
GRAD_MAX_REL = 1.5e-2
GRAD_MEAN_REL = 7e-3


def assert_grad_close(got: np.ndarray, ref: np.ndarray, what: str, max_rel=GRAD_MAX_REL, mean_rel=GRAD_MEAN_REL):
    d = np.abs(got - ref)
    assert np.isfinite(got).all(), f"{what}: non-finite gradient"
    big, avg = np.abs(ref).max(), np.abs(ref).mean()
    assert d.max() <= max_rel * big, f"{what}: max-abs {d.max():.3e} > {max_rel} x {big:.3e}"
    assert d.mean() <= mean_rel * avg, f"{what}: mean-abs {d.mean():.3e} > {mean_rel} x {avg:.3e}"
