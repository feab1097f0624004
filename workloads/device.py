"""Upload / download of bf16 bit patterns as torch tensors (no arithmetic)."""
import numpy as np


def dev_bits(a: np.ndarray, device: str = "cuda"):
    """uint16 bf16 bits -> contiguous torch.bfloat16 tensor on `device`."""
    import torch
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)


def host_bits(t) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns on the host."""
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
