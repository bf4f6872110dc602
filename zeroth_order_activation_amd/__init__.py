"""Dust per-token activation-perturbation gradient estimator for MI355X (gfx950).

Thin Python binding of ``libdust.so`` (C ABI declared in ``include/dust.h``):
argument marshalling only.  Every step of the estimator runs in the library's
HIP kernels; torch provides device memory and the current stream.  There is no
CPU fallback: if the library is missing, every call raises.

Method (the Dust pages, Q Labs 2026; TL;DR page "Dust: zeroth-order
Transformer pretraining without backprop", section 1): each token's layer
output y_t = W x_t gets K Gaussian perturbations sigma a_t^(i); the loss is
recomputed per draw; r_t^(i) = CE_clean - CE_perturbed;
g_hat_t = -(1/(K sigma)) sum_i r_t^(i) a_t^(i); G_W = sum_t g_hat_t x_t^T.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdust.so")
F32, BF16 = 0, 1
_lib = None

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_u32 = ctypes.c_uint32
_u64 = ctypes.c_uint64
_f32 = ctypes.c_float


class DustError(RuntimeError):
    """A non-OK dust_status; ``status`` holds the code."""

    def __init__(self, status: int, msg: str):
        super().__init__(f"dust status {status}: {msg}")
        self.status = status


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m zeroth_order_activation_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        L.dust_abi_version.restype = ctypes.c_int
        L.dust_last_error.restype = ctypes.c_char_p
        L.dust_set_stage_event.restype = ctypes.c_int
        L.dust_set_stage_event.argtypes = [ctypes.c_int, _vp]
        L.dust_noise.restype = ctypes.c_int
        L.dust_noise.argtypes = [_u64, _u32, _u32, _i64, _u64, _i64, _i64, _vp, _vp, _vp]
        L.dust_debug_noise.restype = ctypes.c_int
        L.dust_debug_noise.argtypes = [_u64, _u32, _u32, _u64, _i64, _vp, _vp, _vp]
        L.dust_outer_workspace_bytes.restype = ctypes.c_size_t
        L.dust_outer_workspace_bytes.argtypes = [_i64, _i64, _i64]
        L.dust_outer_product.restype = ctypes.c_int
        L.dust_outer_product.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp, _vp, ctypes.c_size_t, _vp]
        L.dust_head_workspace_bytes.restype = ctypes.c_size_t
        L.dust_head_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64]
        L.dust_estimate_head.restype = ctypes.c_int
        L.dust_estimate_head.argtypes = [_vp, ctypes.c_int, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _u64, _u32,
                                         _u64, _u32, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.dust_estimate_head_noalloc.restype = ctypes.c_int
        L.dust_estimate_head_noalloc.argtypes = [_vp, ctypes.c_int, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _u64,
                                                 _u32, _u64, _u32, _vp, _vp, _vp, _vp]
        L.dust_head_noalloc_max_bytes.restype = ctypes.c_size_t
        L.dust_head_noalloc_max_bytes.argtypes = []
        L.dust_head_subset_workspace_bytes.restype = ctypes.c_size_t
        L.dust_head_subset_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64]
        L.dust_estimate_head_subset.restype = ctypes.c_int
        L.dust_estimate_head_subset.argtypes = [_vp, ctypes.c_int, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _f32,
                                                _u64, _u32, _u64, _u32, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.dust_attn_workspace_bytes.restype = ctypes.c_size_t
        L.dust_attn_workspace_bytes.argtypes = [ctypes.c_int, _i64, _i64, _i64, _i64, _i64]
        L.dust_estimate_attn.restype = ctypes.c_int
        L.dust_estimate_attn.argtypes = [ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _f32,
                                         ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint32,
                                         _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.dust_attn_v_workspace_bytes.restype = ctypes.c_size_t
        L.dust_attn_v_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, _i64]
        L.dust_estimate_attn_v.restype = ctypes.c_int
        L.dust_estimate_attn_v.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _f32,
                                           ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint32,
                                           _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.dust_linear_workspace_bytes.restype = ctypes.c_size_t
        L.dust_linear_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, _i64]
        L.dust_estimate_linear.restype = ctypes.c_int
        L.dust_estimate_linear.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _f32,
                                           _f32, _u64, _u32, _u64, _u32, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.dust_set_kernel_events.restype = ctypes.c_int
        L.dust_set_kernel_events.argtypes = [ctypes.c_int, _vp, _vp, ctypes.c_int]
        L.dust_kernel_event_count.restype = ctypes.c_int
        L.dust_kernel_event_count.argtypes = [ctypes.c_int]
        for nm in ("dust_lm_param_count", "dust_lm_rewards_count", "dust_lm_workspace_bytes"):
            getattr(L, nm).restype = ctypes.c_size_t
        L.dust_lm_param_count.argtypes = [_vp]
        L.dust_lm_rewards_count.argtypes = [_vp, _vp]
        L.dust_lm_workspace_bytes.argtypes = [_vp, _vp]
        L.dust_lm_forward.restype = ctypes.c_int
        L.dust_lm_forward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.dust_lm_estimate.restype = ctypes.c_int
        L.dust_lm_estimate.argtypes = [_vp, _vp, _vp, _vp, _vp, _u64, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.dust_lm_sgd.restype = ctypes.c_int
        L.dust_lm_sgd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp]
        L.dust_lm_step.restype = ctypes.c_int
        L.dust_lm_step.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _u64, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise DustError(status, lib().dust_last_error().decode())


def _p(t):
    return None if t is None else _vp(t.data_ptr())


def _dev_tensor(t, name, dtypes):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(t):
    return _vp(torch.cuda.current_stream(t.device).cuda_stream)


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def set_stage_event(stage: int, event) -> None:
    """Record ``event`` (a torch.cuda.Event) after ``stage`` of each estimator call
    from this thread (0: estimator kernel, 1: outer product); None clears it.
    The event must already exist (torch creates it at its first ``record``)."""
    if event is None:
        ptr = None
    else:
        if not event.cuda_event:
            raise ValueError("record the event once before handing it to the library")
        ptr = _vp(event.cuda_event)
    _check(lib().dust_set_stage_event(stage, ptr))


_hip = None


TIMED_KERNELS = {"lm_gemm": 0, "lm_head": 1, "attn_main": 2, "mlp_gemm1": 3, "mlp_gemm2": 4, "head": 5,
                 "outer": 6}


def set_kernel_events(kernel: str, starts, ends) -> None:
    """Record starts[i] / ends[i] (torch.cuda.Events that already exist) around the i-th
    launch of ``kernel`` (a key of TIMED_KERNELS) from this thread; None clears."""
    kid = TIMED_KERNELS[kernel]
    if starts is None:
        _check(lib().dust_set_kernel_events(kid, None, None, 0))
        return
    n = min(len(starts), len(ends))
    arr_s = (_vp * n)(*[e.cuda_event for e in starts[:n]])
    arr_e = (_vp * n)(*[e.cuda_event for e in ends[:n]])
    _check(lib().dust_set_kernel_events(kid, arr_s, arr_e, n))


def kernel_event_count(kernel: str) -> int:
    return int(lib().dust_kernel_event_count(TIMED_KERNELS[kernel]))


def event_elapsed_ms(start, end) -> float:
    """Milliseconds between two recorded torch.cuda.Events, read with
    hipEventElapsedTime (the library records stage events itself, which torch's
    own bookkeeping does not see)."""
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _vp, _vp]
        _hip.hipEventElapsedTime.restype = ctypes.c_int
    ms = ctypes.c_float(0.0)
    st = _hip.hipEventElapsedTime(ctypes.byref(ms), _vp(start.cuda_event), _vp(end.cuda_event))
    if st != 0:
        raise RuntimeError(f"hipEventElapsedTime failed with status {st}")
    return float(ms.value)


def noise(seed: int, layer: int, draw_offset: int, K: int, token_offset: int, T: int, n: int,
          device="cuda", raw: bool = False):
    """The Gaussian noise a[K,T,n] the estimators use (and the raw Philox words if ``raw``)."""
    g = torch.empty((K, T, n), dtype=torch.float32, device=device)
    w = torch.empty((K, T, 4 * ((n + 3) // 4)), dtype=torch.int32, device=device) if raw else None
    _check(lib().dust_noise(seed, layer, draw_offset, K, token_offset, T, n, _p(w), _p(g), _stream(g)))
    return (g, w.view(torch.uint32) if hasattr(torch, "uint32") else w) if raw else g


def debug_noise(seed: int, layer: int, draw: int, token: int, n: int, device="cuda", raw: bool = False):
    """The noise a[n] of one (draw, token) (and the raw Philox words if ``raw``)."""
    g = torch.empty((n,), dtype=torch.float32, device=device)
    w = torch.empty((4 * ((n + 3) // 4),), dtype=torch.int32, device=device) if raw else None
    _check(lib().dust_debug_noise(seed, layer, draw, token, n, _p(w), _p(g), _stream(g)))
    return (g, w.view(torch.uint32) if hasattr(torch, "uint32") else w) if raw else g


def outer_product(ghat, x, grad_w=None, workspace=None):
    """grad_w = ghat^T x for ghat [T,n], x [T,d] (fp32)."""
    _dev_tensor(ghat, "ghat", (torch.float32,))
    _dev_tensor(x, "x", (torch.float32,))
    T, n = ghat.shape
    d = x.shape[1]
    if x.shape[0] != T:
        raise ValueError("ghat and x must have the same number of rows")
    if grad_w is None:
        grad_w = torch.empty((n, d), dtype=torch.float32, device=ghat.device)
    ws, nb = _workspace(lib().dust_outer_workspace_bytes(T, n, d), ghat.device, workspace)
    _check(lib().dust_outer_product(_p(ghat), _p(x), T, n, d, _p(grad_w), _p(ws), nb, _stream(ghat)))
    return grad_w


def head_workspace_bytes(T: int, V: int, d: int, K: int) -> int:
    return int(lib().dust_head_workspace_bytes(T, V, d, K))


def estimate_head(logits, x, labels, K: int, sigma: float, seed: int, layer: int,
                  token_offset: int = 0, draw_offset: int = 0, *, grad_w=None, ghat=None,
                  rewards=None, workspace=None):
    """LM-head estimator on cached logits [T,V] (fp32 or bf16).  Returns grad_w [V,d].

    Pass preallocated ``ghat`` [T,V] / ``rewards`` [K,T] fp32 tensors to receive
    g_hat and the rewards as well.
    """
    _dev_tensor(logits, "logits", (torch.float32, torch.bfloat16))
    _dev_tensor(x, "x", (torch.float32,))
    _dev_tensor(labels, "labels", (torch.int32,))
    T, V = logits.shape
    d = x.shape[1]
    if x.shape[0] != T or labels.numel() != T:
        raise ValueError("logits, x and labels disagree on T")
    dt = F32 if logits.dtype == torch.float32 else BF16
    if grad_w is None:
        grad_w = torch.empty((V, d), dtype=torch.float32, device=logits.device)
    # with ghat given, only the outer product's split partial sums need scratch space
    need = (lib().dust_outer_workspace_bytes(T, V, d) if ghat is not None
            else lib().dust_head_workspace_bytes(T, V, d, K))
    ws, nb = _workspace(need, logits.device, workspace)
    _check(lib().dust_estimate_head(_p(logits), dt, _p(x), _p(labels), T, V, d, K, sigma, seed, layer,
                                    token_offset, draw_offset, _p(grad_w), _p(ghat), _p(rewards), _p(ws), nb,
                                    _stream(logits)))
    return grad_w


def estimate_head_noalloc(logits, x, labels, K: int, sigma: float, seed: int, layer: int,
                          token_offset: int = 0, draw_offset: int = 0, *, grad_w, ghat=None, rewards=None):
    """dust_estimate_head_noalloc: the LM-head estimator with the library's static
    scratch instead of a workspace.  The caller passes every output (``grad_w`` [V,d]
    and optionally ``ghat`` [T,V], ``rewards`` [K,T]); nothing is allocated here."""
    _dev_tensor(logits, "logits", (torch.float32, torch.bfloat16))
    _dev_tensor(x, "x", (torch.float32,))
    _dev_tensor(labels, "labels", (torch.int32,))
    _dev_tensor(grad_w, "grad_w", (torch.float32,))
    T, V = logits.shape
    d = x.shape[1]
    if x.shape[0] != T or labels.numel() != T or tuple(grad_w.shape) != (V, d):
        raise ValueError("logits, x, labels and grad_w disagree on T, V or d")
    dt = F32 if logits.dtype == torch.float32 else BF16
    _check(lib().dust_estimate_head_noalloc(_p(logits), dt, _p(x), _p(labels), T, V, d, K, sigma, seed, layer,
                                            token_offset, draw_offset, _p(grad_w), _p(ghat), _p(rewards),
                                            _stream(logits)))
    return grad_w


def head_noalloc_max_bytes() -> int:
    return int(lib().dust_head_noalloc_max_bytes())


def head_subset_workspace_bytes(T: int, V: int, d: int, K: int) -> int:
    return int(lib().dust_head_subset_workspace_bytes(T, V, d, K))


def estimate_head_subset(logits, x, labels, K: int, m: int, sigma: float, seed: int, layer: int,
                         token_offset: int = 0, draw_offset: int = 0, *, grad_w=None, ghat=None,
                         rewards=None, workspace=None):
    """Vocabulary-subset LM-head estimator: per draw a window of m channels (a
    multiple of 4) plus the label is perturbed (see dust_estimate_head_subset in
    include/dust.h).  Returns grad_w [V,d]."""
    _dev_tensor(logits, "logits", (torch.float32, torch.bfloat16))
    _dev_tensor(x, "x", (torch.float32,))
    _dev_tensor(labels, "labels", (torch.int32,))
    T, V = logits.shape
    d = x.shape[1]
    if x.shape[0] != T or labels.numel() != T:
        raise ValueError("logits, x and labels disagree on T")
    dt = F32 if logits.dtype == torch.float32 else BF16
    if grad_w is None:
        grad_w = torch.empty((V, d), dtype=torch.float32, device=logits.device)
    ws, nb = _workspace(lib().dust_head_subset_workspace_bytes(T, V, d, K), logits.device, workspace)
    _check(lib().dust_estimate_head_subset(_p(logits), dt, _p(x), _p(labels), T, V, d, K, m, sigma, seed, layer,
                                           token_offset, draw_offset, _p(grad_w), _p(ghat), _p(rewards), _p(ws),
                                           nb, _stream(logits)))
    return grad_w


def linear_workspace_bytes(T: int, d: int, n: int, V: int, K: int) -> int:
    return int(lib().dust_linear_workspace_bytes(T, d, n, V, K))


def _bf16_bits(t, name):
    if t.dtype == torch.bfloat16:
        return t
    if t.dtype in (torch.int16,) or str(t.dtype) == "torch.uint16":
        return t
    raise TypeError(f"{name} must hold bf16 values (torch.bfloat16 or 16-bit integer bits)")


def estimate_linear(u, h, x_res, w2, w_head, labels, K: int, sigma: float, seed: int, layer: int,
                    token_offset: int = 0, draw_offset: int = 0, *, ln_eps: float = 1e-5, grad_w=None,
                    ghat=None, rewards=None, workspace=None):
    """Interior MLP-linear estimator (W1 of a pre-LN block).  Returns grad_w [n,d].

    u [T,d], h [T,n], x_res [T,d] fp32; w2 [d,n], w_head [V,d] bf16; labels [T] int32.
    """
    for t, nm in ((u, "u"), (h, "h"), (x_res, "x_res")):
        _dev_tensor(t, nm, (torch.float32,))
    _dev_tensor(labels, "labels", (torch.int32,))
    for t, nm in ((w2, "w2"), (w_head, "w_head")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{nm} must be a contiguous CUDA (HIP) tensor")
        _bf16_bits(t, nm)
    T, d = u.shape
    n = h.shape[1]
    V = w_head.shape[0]
    if h.shape[0] != T or x_res.shape != (T, d) or w2.shape != (d, n) or w_head.shape != (V, d) or labels.numel() != T:
        raise ValueError("inconsistent shapes for the MLP-linear estimator")
    if grad_w is None:
        grad_w = torch.empty((n, d), dtype=torch.float32, device=u.device)
    ws, nb = _workspace(lib().dust_linear_workspace_bytes(T, d, n, V, K), u.device, workspace)
    _check(lib().dust_estimate_linear(_p(u), _p(h), _p(x_res), _p(w2), _p(w_head), _p(labels), T, d, n, V, K,
                                      sigma, ln_eps, seed, layer, token_offset, draw_offset, _p(grad_w), _p(ghat),
                                      _p(rewards), _p(ws), nb, _stream(u)))
    return grad_w


def attn_v_workspace_bytes(T: int, S: int, d: int, H: int, K: int) -> int:
    return int(lib().dust_attn_v_workspace_bytes(T, S, d, H, K))


def estimate_attn_v(q, k, e, u, S: int, H: int, K: int, sigma: float, seed: int, layer: int,
                    token_offset: int = 0, draw_offset: int = 0, *, grad_w=None, ghat=None, rewards=None,
                    workspace=None):
    """Attention value-projection estimator (see dust_estimate_attn_v in dust.h).  Returns
    grad_w [d,d].  q, k, e, u [T,d] fp32; sequences of S tokens; H heads of 64 channels."""
    for t, nm in ((q, "q"), (k, "k"), (e, "e"), (u, "u")):
        _dev_tensor(t, nm, (torch.float32,))
    T, d = q.shape
    if k.shape != (T, d) or e.shape != (T, d) or u.shape != (T, d):
        raise ValueError("q, k, e and u must share the shape [T, d]")
    if grad_w is None:
        grad_w = torch.empty((d, d), dtype=torch.float32, device=q.device)
    ws, nb = _workspace(lib().dust_attn_v_workspace_bytes(T, S, d, H, K), q.device, workspace)
    _check(lib().dust_estimate_attn_v(_p(q), _p(k), _p(e), _p(u), T, S, d, H, K, sigma, seed, layer, token_offset,
                                      draw_offset, _p(grad_w), _p(ghat), _p(rewards), _p(ws), nb, _stream(q)))
    return grad_w


ATTN_PROJ = {"q": 0, "k": 1, "v": 2}


def attn_workspace_bytes(proj: str, T: int, S: int, d: int, H: int, K: int) -> int:
    return int(lib().dust_attn_workspace_bytes(ATTN_PROJ[proj], T, S, d, H, K))


def estimate_attn(proj: str, q, k, v, e, u, S: int, H: int, K: int, sigma: float, seed: int, layer: int,
                  token_offset: int = 0, draw_offset: int = 0, *, grad_w=None, ghat=None, rewards=None,
                  workspace=None):
    """Attention projection estimator ('q', 'k' or 'v'; see dust_estimate_attn in dust.h).
    Returns grad_w [d,d].  q, k, v, e, u [T,d] fp32 (v may be None for 'v')."""
    if proj not in ATTN_PROJ:
        raise ValueError("proj must be 'q', 'k' or 'v'")
    for t, nm in ((q, "q"), (k, "k"), (e, "e"), (u, "u")) + (((v, "v"),) if v is not None else ()):
        _dev_tensor(t, nm, (torch.float32,))
    T, d = q.shape
    if any(x is not None and x.shape != (T, d) for x in (k, v, e, u)):
        raise ValueError("q, k, v, e and u must share the shape [T, d]")
    if grad_w is None:
        grad_w = torch.empty((d, d), dtype=torch.float32, device=q.device)
    ws, nb = _workspace(attn_workspace_bytes(proj, T, S, d, H, K), q.device, workspace)
    _check(lib().dust_estimate_attn(ATTN_PROJ[proj], _p(q), _p(k), _p(v), _p(e), _p(u), T, S, d, H, K, sigma, seed,
                                    layer, token_offset, draw_offset, _p(grad_w), _p(ghat), _p(rewards), _p(ws), nb,
                                    _stream(q)))
    return grad_w


# ---- one full Dust step on a small causal LM (see dust_lm_* in dust.h) ----------------
class LMConfig(ctypes.Structure):
    """dust_lm_config: V, d = 64 H, H, L blocks, MLP width n, sequence length S, batch B."""
    _fields_ = [("V", ctypes.c_int32), ("d", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32),
                ("n", ctypes.c_int32), ("S", ctypes.c_int32), ("B", ctypes.c_int32), ("ln_eps", ctypes.c_float)]


class LMHparams(ctypes.Structure):
    """dust_lm_hparams: draws per pass K, ES pairs M, the noise scale of every pass,
    the SGD-momentum settings."""
    _fields_ = [("K", ctypes.c_int32), ("M", ctypes.c_int32)] + [
        (nm, ctypes.c_float) for nm in ("sigma_emb", "sigma_q", "sigma_k", "sigma_v", "sigma_o", "sigma_up",
                                        "sigma_down", "sigma_head", "sigma_es", "lr", "lr_scalar", "momentum")] + [
        ("chunk", ctypes.c_int32)]


LM_TYPES = ("emb", "q", "k", "v", "o", "up", "down", "head")


def lm_config(V: int, d: int, H: int, L: int, n: int, S: int, B: int, ln_eps: float = 1e-5) -> LMConfig:
    return LMConfig(V, d, H, L, n, S, B, ln_eps)


def lm_hparams(K: int, M: int, sigma, sigma_es: float, lr: float = 0.0, lr_scalar: float = 0.0,
               momentum: float = 0.0, chunk: int = 0) -> LMHparams:
    """``sigma``: one noise scale for every pass, or a dict over LM_TYPES; ``chunk``: most
    draws per chunk of change tensors (0: as many as fit in 1 GiB)."""
    sg = sigma if isinstance(sigma, dict) else dict.fromkeys(LM_TYPES, float(sigma))
    return LMHparams(K, M, *(sg[t] for t in LM_TYPES), sigma_es, lr, lr_scalar, momentum, chunk)


def lm_param_count(cfg: LMConfig) -> int:
    return int(lib().dust_lm_param_count(ctypes.byref(cfg)))


def lm_rewards_count(cfg: LMConfig, hp: LMHparams) -> int:
    return int(lib().dust_lm_rewards_count(ctypes.byref(cfg), ctypes.byref(hp)))


def lm_workspace_bytes(cfg: LMConfig, hp: LMHparams | None = None) -> int:
    return int(lib().dust_lm_workspace_bytes(ctypes.byref(cfg), None if hp is None else ctypes.byref(hp)))


def _lm_inputs(cfg, params, tokens, labels):
    _dev_tensor(params, "params", (torch.float32,))
    _dev_tensor(tokens, "tokens", (torch.int32,))
    _dev_tensor(labels, "labels", (torch.int32,))
    T = cfg.B * cfg.S
    if params.numel() != lm_param_count(cfg) or tokens.numel() != T or labels.numel() != T:
        raise ValueError("params must hold dust_lm_param_count floats, tokens and labels B*S ids")


def lm_forward(cfg: LMConfig, params, tokens, labels, *, ce=None, workspace=None):
    """Clean per-token cross-entropy [B*S] of the model."""
    _lm_inputs(cfg, params, tokens, labels)
    if ce is None:
        ce = torch.empty(cfg.B * cfg.S, dtype=torch.float32, device=params.device)
    ws, nb = _workspace(lm_workspace_bytes(cfg), params.device, workspace)
    _check(lib().dust_lm_forward(ctypes.byref(cfg), _p(params), _p(tokens), _p(labels), _p(ce), _p(ws), nb,
                                 _stream(params)))
    return ce


def lm_estimate(cfg: LMConfig, hp: LMHparams, params, tokens, labels, seed: int, *, grads=None, rewards=None,
                workspace=None):
    """Every gradient estimate of one Dust step, packed like the parameters."""
    _lm_inputs(cfg, params, tokens, labels)
    if grads is None:
        grads = torch.empty_like(params)
    ws, nb = _workspace(lm_workspace_bytes(cfg, hp), params.device, workspace)
    _check(lib().dust_lm_estimate(ctypes.byref(cfg), ctypes.byref(hp), _p(params), _p(tokens), _p(labels), seed,
                                  _p(grads), _p(rewards), _p(ws), nb, _stream(params)))
    return grads


def lm_sgd(cfg: LMConfig, hp: LMHparams, params, momentum, grads) -> None:
    """m <- momentum m + grads; params <- params - lr m (lr_scalar on the 2L scalars)."""
    for t, nm in ((params, "params"), (momentum, "momentum"), (grads, "grads")):
        _dev_tensor(t, nm, (torch.float32,))
    _check(lib().dust_lm_sgd(ctypes.byref(cfg), ctypes.byref(hp), _p(params), _p(momentum), _p(grads),
                             _stream(params)))


def lm_step(cfg: LMConfig, hp: LMHparams, params, momentum, tokens, labels, seed: int, *, grads=None, rewards=None,
            workspace=None):
    """One Dust update in place on params and momentum; returns the estimates."""
    _lm_inputs(cfg, params, tokens, labels)
    _dev_tensor(momentum, "momentum", (torch.float32,))
    if grads is None:
        grads = torch.empty_like(params)
    ws, nb = _workspace(lm_workspace_bytes(cfg, hp), params.device, workspace)
    _check(lib().dust_lm_step(ctypes.byref(cfg), ctypes.byref(hp), _p(params), _p(momentum), _p(tokens), _p(labels),
                              seed, _p(grads), _p(rewards), _p(ws), nb, _stream(params)))
    return grads
