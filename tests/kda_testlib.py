"""Helpers shared by the GPU tests: move seeded numpy inputs to the device in
the operator's dtypes and run the oracle on the same (rounded) values."""

import numpy as np
import torch

TOL = {"bf16": 2e-3, "f32": 1e-5}   # max relative error (normwise), per output tensor


def dev(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(dtype).contiguous()


def tdtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def random_state(rng, shape, scale=0.5):
    return (scale * rng.standard_normal(shape)).astype(np.float32)


def flush(msg):
    print(msg, flush=True)
