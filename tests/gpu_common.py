"""Shared setup of the GPU parity tests: the same seeded weights feed the HIP
path (on the device) and the oracle (float64 copies on the host)."""
import numpy as np
import torch

from oracle.model import OracleModel

TOL_F32 = 1e-4     # rel-Linf on logits, float32 path
TOL_BF16 = 2e-2    # rel-Linf on logits, bf16 path (spec bound)
MARGIN = 1e-3      # decisions closer than this to a tie or threshold are excluded


def to_dev(w):
    return {k: (None if v is None else v.to("cuda").contiguous()) for k, v in w.items()}


def oracle_model(shape, w):
    return OracleModel.from_torch(shape, w)


def rel_linf(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def i32(x):
    return torch.tensor(np.asarray(x, dtype=np.int32), device="cuda")


def ws(nbytes):
    return torch.empty(int(nbytes), dtype=torch.uint8, device="cuda")


def say(*a):
    print(*a, flush=True)
