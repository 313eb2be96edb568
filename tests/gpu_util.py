"""Host <-> device marshalling for the GPU tests (numpy bit patterns in,
numpy bit patterns out)."""

import numpy as np
import torch

DEV = "cuda:0"


def to_dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def to_dev_i8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int8)).to(DEV)


def to_dev_bf16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).to(DEV)
    return t.view(torch.bfloat16)


def to_dev(a, dtype=None):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bf16_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f32(t):
    return t.float().cpu().numpy() if t.dtype != torch.float32 else t.cpu().numpy()


def show(*parts):
    """Name the case before each GPU step so a crash log says what ran."""
    print("[case]", *parts, flush=True)
