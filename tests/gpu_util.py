"""Helpers shared by the GPU parity tests (device upload, error metrics)."""
import numpy as np
import torch


def dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def host(t):
    return t.detach().cpu().numpy()


def rel_max_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def bf16_bits(a):
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even (torch's conversion)."""
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def sync():
    torch.cuda.synchronize()
