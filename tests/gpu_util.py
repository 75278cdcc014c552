"""Helpers shared by the GPU tests: tensor transfer and the parity criterion."""
import numpy as np
import torch


def dev_bf16(x32: np.ndarray) -> torch.Tensor:
    """float32 values that are exactly bf16 -> device bf16 tensor (bit-exact)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    assert not np.any(u & 0xFFFF)
    bits = (u >> 16).astype(np.uint16).view(np.int16)
    return torch.from_numpy(bits.copy()).cuda().view(torch.bfloat16)


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def dev_u8(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).cuda()


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def rms(x: np.ndarray) -> float:
    return float(np.sqrt(np.mean(np.square(x, dtype=np.float64))))


def assert_parity(gpu: np.ndarray, ref: np.ndarray, tol: float = 2e-2, name: str = "") -> float:
    """The parity bar: max |gpu - ref| <= tol * RMS(ref), per tensor.  Returns the ratio."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite values"
    r = rms(ref)
    err = float(np.max(np.abs(gpu - ref))) if gpu.size else 0.0
    ratio = err / r if r > 0 else err
    assert err <= tol * r or (r == 0 and err == 0), f"{name}: max|diff|={err:.3e} > {tol}*RMS={tol * r:.3e}"
    return ratio
