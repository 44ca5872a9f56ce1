"""Helpers for the GPU parity tests: device transfer of the canonical inputs and
the comparison metrics. No arithmetic of the layer lives here."""

import numpy as np
import torch

DEV = "cuda"


def dev(arr, dtype):
    """numpy canonical input (bf16 bits uint16 / fp32 / int) -> device tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(DEV)
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(DEV)
    if dtype == "i32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.int32)).to(DEV)
    raise ValueError(dtype)


def host(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def log(*a):
    print(*a, flush=True)
