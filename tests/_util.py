"""Helpers for the GPU parity tests: host arrays <-> device tensors, ulp distance."""
import sys

import numpy as np


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_f16(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).cuda()


def dev_x(X: np.ndarray):
    """uint16 bf16 bits -> torch.bfloat16 on device; float16 -> torch.float16."""
    import torch
    if X.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(X).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(X, dtype=np.float16)).cuda()


def dev_f32(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.int32:
        return t.cpu().numpy().view(np.uint32)
    if t.dtype == torch.float16:
        return t.cpu().numpy()
    return t.cpu().numpy()


def ulp_dist(a: np.ndarray, b: np.ndarray) -> int:
    """max distance in units of last place between two fp32 arrays (same sign assumed)."""
    ia = np.asarray(a, dtype=np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, dtype=np.float32).view(np.int32).astype(np.int64)
    return int(np.abs(ia - ib).max()) if ia.size else 0


def argmin_ok(gpu_k: int, oracle_errs: np.ndarray, oracle_k: int, rel: float = 1e-4) -> bool:
    """gpu's choice equals the oracle's, or the oracle's errors tie within `rel`."""
    if gpu_k == oracle_k:
        return True
    return oracle_errs[gpu_k] <= oracle_errs[oracle_k] * (1.0 + rel)
