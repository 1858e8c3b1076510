"""Upload of generated inputs to device memory (torch tensors).

x is moved as its raw 16-bit patterns (bf16 or fp16 bits in an int16 tensor),
y as fp32: no value is converted on the way.
"""
from __future__ import annotations

import numpy as np


def to_device_x(x_bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(device)


def to_device_y(y, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).to(device)
