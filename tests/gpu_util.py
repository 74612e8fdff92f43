"""Helpers shared by the GPU parity tests (host <-> device marshalling and
the acceptance metric).  No arithmetic of the method lives here."""

import sys

import numpy as np


def dev():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a HIP device")
    return torch.device("cuda:0")


def to_dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def to_dev(arr):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr)).to(dev())


def bf16_bits(t):
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def u8(t):
    return t.detach().cpu().numpy().view(np.uint8)


def empty_u8(shape, guard=4096):
    """uint8 device buffer with a guard tail filled with 0xA5; returns
    (view, full) so the guard can be checked after the kernel ran."""
    import torch
    n = int(np.prod(shape))
    full = torch.full((n + guard,), 0xA5, dtype=torch.uint8, device=dev())
    return full[:n].view(*shape), full


def guard_intact(full, n):
    tail = full[n:].cpu().numpy()
    return bool(np.all(tail == 0xA5))


def rel_fro(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()
