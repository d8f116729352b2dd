"""Test-side helpers to move seeded numpy inputs to and from the GPU."""
import numpy as np
import pytest
import torch


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def to_dev(a: np.ndarray, dt: str) -> torch.Tensor:
    """numpy (float32 / float16 / bf16 bits as uint16) -> device tensor of dt."""
    a = np.ascontiguousarray(a)
    if dt == "f32":
        t = torch.from_numpy(a.astype(np.float32, copy=False))
    elif dt == "f16":
        t = torch.from_numpy(a.view(np.float16))
    else:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy: float32 stays float32; fp16 / bf16 -> uint16 bits."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def empty(shape, dt: str) -> torch.Tensor:
    return torch.empty(shape, dtype={"f32": torch.float32, "f16": torch.float16,
                                     "bf16": torch.bfloat16}[dt], device="cuda")


def misaligned(t: torch.Tensor) -> torch.Tensor:
    """Same values, data pointer moved off 16-byte alignment (a 1-element offset view)."""
    buf = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    v = buf[1:1 + t.numel()].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 != 0
    return v


ORACLE_DT = {"f32": 0, "f16": 1, "bf16": 2}


def gpu_normal(shape, dt: str, seed: int, mean: float = 0.0, std: float = 1.0) -> torch.Tensor:
    """N(mean, std^2) draws made on the device by a seeded torch generator (fp32,
    rounded once to dt), in 2^26-element chunks: for inputs of billions of
    elements, where a host draw and copy would dominate the test. The oracle
    gets the values back from the device (sampled)."""
    n = 1
    for s in shape:
        n *= int(s)
    out = empty((n,), dt)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    chunk = 1 << 26
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        v = torch.randn(m, generator=g, device="cuda", dtype=torch.float32)
        if std != 1.0:
            v.mul_(std)
        if mean != 0.0:
            v.add_(mean)
        out[i:i + m].copy_(v)
    return out.view(shape)
