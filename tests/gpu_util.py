"""Helpers shared by the GPU parity tests (no arithmetic of the method here)."""
import numpy as np
import torch

TOL_F32 = 1e-5   # max|delta| / max|ref| on fp32 inputs
TOL_BF16 = 5e-3  # max|delta| / max|ref| on bf16 inputs with fp32 state


def dev(x: np.ndarray, dtype=torch.float32) -> torch.Tensor:
    """Host array -> contiguous device tensor (bf16 inputs are bf16-valued already)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(dtype).contiguous()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite output"
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref)) / (scale if scale > 0 else 1.0)) if ref.size else 0.0
    print(f"    max|d|/max|ref| = {err:.3e}", flush=True)
    return err


def announce(msg: str):
    print(f"[case] {msg}", flush=True)
