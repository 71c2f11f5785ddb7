"""Host storage arrays <-> torch device tensors (plumbing only)."""

import numpy as np


def to_dev(arr, dtype, device="cuda"):
    """Upload a storage array ("bf16" bits, "f32", "fp8" codes, "i32")."""
    import torch
    arr = np.ascontiguousarray(arr)
    if dtype == "bf16":
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    elif dtype == "f32":
        t = torch.from_numpy(arr.astype(np.float32, copy=False))
    elif dtype == "fp8":
        t = torch.from_numpy(arr.astype(np.uint8, copy=False))
    elif dtype == "int8":
        t = torch.from_numpy(arr.astype(np.int8, copy=False))
    elif dtype == "i32":
        t = torch.from_numpy(arr.astype(np.int32, copy=False))
    else:
        raise ValueError(dtype)
    return t.to(device)


def to_host(t, dtype):
    """Download a device tensor as the storage array of ``dtype``."""
    import torch
    t = t.detach().cpu()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    if dtype == "f32":
        return t.numpy()
    if dtype == "fp8":
        return t.view(torch.uint8).numpy()
    if dtype == "int8":
        return t.view(torch.int8).numpy()
    raise ValueError(dtype)
