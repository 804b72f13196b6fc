"""Helpers for GPU tests: move numpy arrays to and from cuda:0 as raw bytes."""
import numpy as np


def to_dev(x: np.ndarray):
    import torch

    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to("cuda:0")
    if x.dtype == np.uint8:
        return torch.from_numpy(x).to("cuda:0")
    raise TypeError(x.dtype)


def bf16_from_dev(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def bytes_from_dev(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint8).reshape(-1)


def empty_bf16(shape, fill=-1):
    import torch

    t = torch.empty(shape, dtype=torch.int16, device="cuda:0")
    t.fill_(fill)
    return t


def empty_bytes(n, fill=0xA5):
    import torch

    t = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    t.fill_(fill)
    return t
