"""Move seeded host arrays to the GPU (torch tensors on cuda:0).

Shared by the tests and the benchmark.  Holds no arithmetic of the method:
it only copies bytes (bf16 arrays, stored as uint16 bit patterns on the host,
become torch.bfloat16 tensors with the same bits)."""
import numpy as np
import torch

DEV = "cuda:0"


def to_dev(a, bf16=False):
    """Copy a NumPy array to the device; bf16=True reinterprets uint16 bit
    patterns as bfloat16."""
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
