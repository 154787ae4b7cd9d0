"""Host <-> device plumbing for the GPU tests (no layer arithmetic here)."""
import numpy as np
import torch

DEV = "cuda"


def dev(a):
    """Host array -> device tensor (uint16 = bf16 bits, float32, integer -> int32)."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to(DEV)
    if np.issubdtype(a.dtype, np.integer):
        return torch.from_numpy(a.astype(np.int32)).to(DEV)
    raise TypeError(a.dtype)


def host(t):
    """Device tensor -> numpy (bf16 as uint16 bit patterns)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f64(a):
    """Exact fp64 value of a host array or device tensor (bf16 bits decoded)."""
    if isinstance(a, torch.Tensor):
        a = host(a)
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def rel_err(got, ref) -> float:
    got = f64(got)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def by_expert(idx, gate):
    """Each token's chosen experts in ascending order, with their gates alongside."""
    o = np.argsort(idx, axis=1, kind="stable")
    return np.take_along_axis(idx, o, axis=1), np.take_along_axis(gate, o, axis=1)


def empty_like_poisoned(shape, dtype):
    """A device buffer filled with a NaN pattern, to show which elements a kernel wrote."""
    t = torch.empty(shape, dtype=dtype, device=DEV)
    t.fill_(float("nan"))
    return t


# tolerances: bf16 inputs with fp32 accumulation vs the fp64 oracle
TOL_BF16 = 2e-2
TOL_F32 = 1e-4
GATE_ATOL = 1e-5
