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


def exclusion(zg, zo, inv_temp):
    """Margin below which a sampled / arg-max decision may legitimately differ.

    Both sides maximise score = z * s + G with identical Gumbel noise G (the
    same Philox words; s = 1/T, or 1 for greedy), so if every score differs by
    less than half the oracle's top-2 gap, the arg-max must agree.  The bound
    is twice the measured score discrepancy (plus float32 log rounding), and
    never below MARGIN."""
    s = 1.0 if inv_temp == 0.0 else inv_temp
    dz = float(np.max(np.abs(np.asarray(zg, np.float64) - np.asarray(zo, np.float64))))
    return max(MARGIN, 2.0 * (s * dz + 1e-5))
