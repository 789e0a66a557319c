"""Small helpers shared by the tests: moving torch tensors into the oracle's numpy storage."""
import numpy as np
import torch


def to_storage(t: torch.Tensor) -> np.ndarray:
    """Raw element storage on the host: float32 as np.float32, 16-bit types as
    np.uint16, bytes (q8_0 tiles) as np.uint8."""
    t = t.detach().contiguous().cpu()
    if t.dtype in (torch.float32, torch.uint8):
        return t.numpy().copy()
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def from_storage(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    if dtype == torch.float32:
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(dtype)


def layer_storage(w, layer: int = 0):
    k, v = w.layer_views(layer)
    return to_storage(k), to_storage(v)


def decoded(a: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Storage -> float64 through torch's own conversion (a library routine)."""
    return from_storage(a, dtype).to(torch.float64).numpy()
