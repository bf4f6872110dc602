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


def ulp32(x):
    """Spacing of fp32 numbers at |x|."""
    x = np.maximum(np.abs(np.asarray(x, np.float64)), 1e-30)
    return np.exp2(np.floor(np.log2(x)) - 23)


def check_quantized_rewards(r_gpu, r_orc, ce0_orc, *, tol_l2=5e-3, min_rows_for_l2=1000, bulk_frac=0.85):
    """Parity of rewards whose downstream rounds GEMM operands to bf16.

    Both sides round the GELU and LayerNorm outputs to bf16 from fp32 values;
    the kernel's fp32 values carry the MFMA accumulation order, so on rare rows
    a value sitting within an ulp of a bf16 tie rounds the other way and the
    loss of that row moves by one bf16 step of one operand.  Therefore:
      * the bulk of the rewards agrees within the fp32 resolution of the losses
        (8 ulp of the clean loss), which catches any systematic error;
      * the rare rounding-flip outliers are bounded by a quarter of the rms reward;
      * over enough rewards the relative L2 difference, an estimate of the
        relative L2 error of G_W, is within ``tol_l2``.
    Returns a dict of the measured statistics."""
    r_gpu = np.asarray(r_gpu, np.float64)
    r_orc = np.asarray(r_orc, np.float64)
    tol = 8 * ulp32(np.asarray(ce0_orc))[None, :] + 1e-4 * np.abs(r_orc)
    d = np.abs(r_gpu - r_orc)
    bulk = float((d <= tol).mean())
    rms = float(np.sqrt((r_orc ** 2).mean()))
    stats = {"bulk": bulk, "max_abs": float(d.max()), "rms_reward": rms, "rel_l2": rel_l2(r_gpu, r_orc), "n": d.size}
    assert bulk >= bulk_frac, stats
    assert d.max() <= 0.25 * rms, stats
    if d.size >= min_rows_for_l2:
        assert stats["rel_l2"] <= tol_l2, stats
    return stats
