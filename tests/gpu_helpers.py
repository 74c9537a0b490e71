"""Shared helpers of the GPU parity tests (host <-> device marshalling only)."""

import numpy as np
import torch

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def f32_bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def bf16_bits(t):
    """uint16 bit patterns of a torch bf16 tensor."""
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def weights(n, k, seed, dtype):
    """(torch tensor on the GPU, fp32 numpy copy the oracle sees) of N(0, 0.02^2) weights."""
    from ternary_weight_linear_bit_amd import inputs as I
    w32 = I.master_weights(n, k, seed)
    if dtype == "bf16":
        wt = I.to_bf16(w32)
        return wt.to(DEV), wt.float().numpy()
    return dev(w32), w32


def acts(m, k, seed, dtype):
    from ternary_weight_linear_bit_amd import inputs as I
    x32 = I.activations(m, k, seed)
    if dtype == "bf16":
        xt = I.to_bf16(x32)
        return xt.to(DEV), xt.float().numpy()
    return dev(x32), x32
