"""Move stored synthetic maps (numpy) onto a torch device without changing a bit."""
import numpy as np
import torch

from . import BF16, F16, F32


def to_device(a: np.ndarray, dtype: int, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if dtype == F32:
        t = torch.from_numpy(a.astype(np.float32, copy=False))
    elif dtype == F16:
        t = torch.from_numpy(a.astype(np.float16, copy=False))
    elif dtype == BF16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        raise ValueError(dtype)
    return t.to(device)
