"""Test-side glue: torch tensors -> the raw storage arrays the oracle reads."""
import numpy as np
import torch

from oracle import cache as OC


def storage(t):
    """Raw storage words of a tensor, on the host: uint32 (f32), uint16 (bf16), uint8."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.float32:
        return t.numpy().view(np.uint32)
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.uint8:
        return t.numpy()
    raise TypeError(t.dtype)


def f64(t, dtype_code=None, scale=None):
    """fp64 values of a tensor as the oracle decodes them."""
    if dtype_code is None:
        dtype_code = {torch.float32: OC.F32, torch.bfloat16: OC.BF16, torch.uint8: OC.FP8_E4M3}[t.dtype]
    return OC.to_f64(storage(t), dtype_code, scale)


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))
