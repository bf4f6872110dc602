"""Helpers shared by the GPU tests: move seeded synthetic inputs to the device
and compare results.  Holds none of the estimator's arithmetic."""
import numpy as np
import torch


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def logits_to_device(case):
    """Cached logits of a head case as a device tensor (fp32, or bf16 from its bits)."""
    if "logits_bf16" in case:
        return dev(case["logits_bf16"].view(np.int16)).view(torch.bfloat16)
    return dev(case["logits"])


def logits_values(case):
    """The same logits as exact fp64 host values (for the oracle)."""
    if "logits_bf16" in case:
        return (case["logits_bf16"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return case["logits"].astype(np.float64)


def gpu_matmul(X, W):
    """Clean forward z = X W^T on the GPU (input generation only)."""
    with torch.no_grad():
        return (dev(X) @ dev(W).T).cpu().numpy()
