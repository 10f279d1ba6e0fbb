"""Helpers shared by the GPU tests: moving seeded host arrays to the GPU and back."""
import numpy as np
import torch


def dev():
    return torch.device("cuda:0")


def to_gpu_bf16(bits):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 tensor on cuda:0."""
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).to(dev()).view(torch.bfloat16)


def to_np_u8(t):
    return t.detach().cpu().numpy().astype(np.uint8)


def to_np_f32(t):
    return t.detach().float().cpu().numpy()


def scalar_gpu(v):
    return torch.tensor([np.float32(v)], dtype=torch.float32, device=dev())


def out_to_np(c):
    if c.dtype == torch.bfloat16:
        return c.float().cpu().numpy().astype(np.float64)
    return c.cpu().numpy().astype(np.float64)


def first_mismatch(a, b):
    idx = np.argwhere(np.asarray(a) != np.asarray(b))
    if len(idx) == 0:
        return None
    i = tuple(idx[0])
    return f"{len(idx)} mismatches; first at {i}: got {np.asarray(a)[i]!r} want {np.asarray(b)[i]!r}"
