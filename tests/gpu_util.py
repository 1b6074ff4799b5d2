"""Helpers shared by the GPU tests: device transfer, error measures, tolerances.

Tolerances (relative L2 over the compared tensor), derived from the arithmetic:
* a step whose output is stored in bf16 carries the bf16 rounding of every
  element, relative error <= 2^-9 each and about 2^-9/sqrt(3) ~ 1.1e-3 in L2;
  fp32 accumulation adds ~sqrt(K)*2^-24 ~ 1e-5.  Bound: 4e-3.
* attention rounds the probabilities to bf16 before the PV product and its
  output to bf16: two such roundings, bound 6e-3.
* fp32 residual updates fed the same bf16 operands differ only by summation
  order: bound 1e-4 on the update itself.
* one whole block (all intermediates bf16, fp32 residual): the contract is
  rel-L2 <= 1e-2 on x_out; after the full depth <= 3e-2.
"""
import sys

import numpy as np

TOL_BF16_OUT = 4e-3
TOL_ATTN = 6e-3
TOL_RESID_DELTA = 1e-4
TOL_BLOCK = 1e-2
TOL_DEPTH = 3e-2


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def dev(a, device="cuda"):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device)
    return torch.from_numpy(a).to(device)


def host_bf16(t) -> np.ndarray:
    """Device bf16/int16 tensor -> float64 values."""
    import torch
    u = t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32)
    return (u << 16).view(np.float32).astype(np.float64)
