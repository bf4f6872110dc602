"""Seeded synthetic inputs for the Dust estimator workloads.

This module only draws random inputs and runs the *upstream* clean forward
that produces the cached tensors the estimator consumes (the logits z = W x of
the LM head; the LayerNorm input and W1 output of an MLP block).  It holds none
of the estimator's own arithmetic: no noise, no perturbation, no loss, no
reward.  Both the HIP path and the oracle are fed the very same arrays.

The pages measure on FineWeb; no dataset is available here, so these seeded
distributions stand in for it: activations N(0,1), weights N(0, 1/fan_in),
labels uniform or Zipf(s=1.1) over the vocabulary (token-frequency skew).
"""
from __future__ import annotations

import numpy as np

NOISE_SEED_BASE = 0x4455535400000000  # noise seed of workload i is this + i
HEAD_LAYER = 1
W1_LAYER = 0
WV_LAYER = 2


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round to nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def zipf_labels(rng: np.random.Generator, T: int, V: int, s: float = 1.1) -> np.ndarray:
    p = (np.arange(1, V + 1, dtype=np.float64)) ** (-s)
    p /= p.sum()
    return rng.choice(V, size=T, p=p).astype(np.int32)


def uniform_labels(rng: np.random.Generator, T: int, V: int) -> np.ndarray:
    return rng.integers(0, V, size=T, dtype=np.int64).astype(np.int32)


def _layernorm_noaffine(x: np.ndarray, eps: float) -> np.ndarray:
    """Pre-LN of the upstream block (gamma=1, beta=0), used only to build the
    cached W1 input u = LN(x)."""
    x64 = x.astype(np.float64)
    mu = x64.mean(axis=1, keepdims=True)
    var = ((x64 - mu) ** 2).mean(axis=1, keepdims=True)
    return ((x64 - mu) / np.sqrt(var + eps)).astype(np.float32)


def head_case(T: int, V: int, d: int, *, seed: int, labels: str = "zipf",
              logits_dtype: str = "f32", matmul=None) -> dict:
    """LM-head workload: X ~ N(0,1) [T,d], W ~ N(0,1/d) [V,d], z = X W^T.

    ``logits_dtype`` "bf16" stores the cached logits as bfloat16 bits (RNE).
    ``matmul(a, b)`` may be passed to run the clean forward elsewhere (e.g. on
    a GPU through torch); default is numpy fp32.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    X = rng.standard_normal((T, d), dtype=np.float32)
    W = (rng.standard_normal((V, d), dtype=np.float32) * np.float32(1.0 / np.sqrt(d))).astype(np.float32)
    lab = zipf_labels(rng, T, V) if labels == "zipf" else uniform_labels(rng, T, V)
    Z = (matmul(X, W) if matmul is not None else X @ W.T).astype(np.float32)
    out = {"x": X, "labels": lab, "T": T, "V": V, "d": d}
    if logits_dtype == "bf16":
        out["logits_bf16"] = bf16_bits(Z)
    else:
        out["logits"] = np.ascontiguousarray(Z)
    return out


def linear_case(T: int, d: int, n: int, V: int, *, seed: int, ln_eps: float = 1e-5) -> dict:
    """Interior MLP-linear workload (pre-LN block, no biases, no LN affine):
    x ~ N(0,1) [T,d]; u = LN(x); W1 ~ N(0,1/d) [n,d]; h = u W1^T (cached W1
    output); W2 ~ N(0,1/n) [d,n] and W_head ~ N(0,1/d) [V,d] stored bf16;
    labels Zipf(1.1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    X = rng.standard_normal((T, d), dtype=np.float32)
    U = _layernorm_noaffine(X, ln_eps)
    W1 = (rng.standard_normal((n, d), dtype=np.float32) * np.float32(1.0 / np.sqrt(d))).astype(np.float32)
    H = (U @ W1.T).astype(np.float32)
    W2 = rng.standard_normal((d, n), dtype=np.float32) * np.float32(1.0 / np.sqrt(n))
    WH = rng.standard_normal((V, d), dtype=np.float32) * np.float32(1.0 / np.sqrt(d))
    lab = zipf_labels(rng, T, V)
    return {"u": U, "h": H, "x_res": X, "w1": W1, "w2_bf16": bf16_bits(W2),
            "w_head_bf16": bf16_bits(WH), "labels": lab, "T": T, "d": d, "n": n, "V": V,
            "ln_eps": ln_eps}


def attn_case(B: int, S: int, H: int, seed: int, dh: int = 64, matmul=None) -> dict:
    """Inputs of the attention value-projection estimator: the attention input
    u ~ N(0,1) [T,d] (T = B S, d = H dh), projections W_Q, W_K, W_V ~ N(0, 1/d)
    and their clean outputs q, k, v = u W^T, and the error at the attention
    output e ~ N(0,1) [T,d] (it stands in for the back-projected output error
    of W_O).  ``matmul(X, W)`` computes X W^T (numpy by default)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T, d = B * S, H * dh
    U = rng.standard_normal((T, d), dtype=np.float32)
    Ws = [(rng.standard_normal((d, d), dtype=np.float32) / np.float32(np.sqrt(d))) for _ in range(3)]
    E = rng.standard_normal((T, d), dtype=np.float32)
    mm = matmul or (lambda X, W: (X.astype(np.float64) @ W.astype(np.float64).T).astype(np.float32))
    q, k, v = (np.ascontiguousarray(mm(U, W), dtype=np.float32) for W in Ws)
    return {"u": U, "q": q, "k": k, "v": v, "e": E, "T": T, "S": S, "H": H, "d": d}


LM_NOISE_SEED = NOISE_SEED_BASE + 7


def lm_param_layout(V: int, d: int, L: int, n: int, S: int):
    """Named tensors of a small LM's packed fp32 parameter vector, in storage
    order (weights [out, in]; scal = alpha_0, beta_0, alpha_1, beta_1, ...)."""
    out = [("emb", (V, d)), ("pos", (S, d))]
    for l in range(L):
        out += [(f"wq{l}", (d, d)), (f"wk{l}", (d, d)), (f"wv{l}", (d, d)), (f"wo{l}", (d, d)),
                (f"w1{l}", (n, d)), (f"w2{l}", (d, n))]
    return out + [("head", (V, d)), ("scal", (2 * L,))]


def lm_case(V: int, d: int, H: int, L: int, n: int, S: int, B: int, *, seed: int, scal: float = 1.0) -> dict:
    """A small causal LM at random initialisation and a batch of B sequences:
    embeddings N(0,1), weights N(0, 1/fan_in), residual scalars ``scal``; token
    sequences of S + 1 Zipf(1.1) ids over [0, V), inputs the first S, labels the
    next token.  Parameters are packed fp32 (see lm_param_layout)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    parts = []
    for name, shp in lm_param_layout(V, d, L, n, S):
        if name == "scal":
            parts.append(np.full(shp, scal, np.float32))
        elif name in ("emb", "pos"):
            parts.append(rng.standard_normal(shp, dtype=np.float32))
        else:
            parts.append(rng.standard_normal(shp, dtype=np.float32) / np.float32(np.sqrt(shp[1])))
    seq = zipf_labels(rng, B * (S + 1), V).reshape(B, S + 1)
    return {"params": np.concatenate([p_.reshape(-1) for p_ in parts]).astype(np.float32),
            "tokens": np.ascontiguousarray(seq[:, :S].reshape(-1), dtype=np.int32),
            "labels": np.ascontiguousarray(seq[:, 1:].reshape(-1), dtype=np.int32),
            "V": V, "d": d, "H": H, "L": L, "n": n, "S": S, "B": B, "T": B * S}


# The named workloads (token counts are batch x sequence, flattened t = b*S + s).
WORKLOADS = {
    1: dict(kind="head", T=256, V=512, d=64, K=64, sigma=1e-2, labels="uniform", logits_dtype="f32"),
    2: dict(kind="head", T=4096, V=8192, d=512, K=256, sigma=1e-2, labels="zipf", logits_dtype="f32"),
    3: dict(kind="linear", T=4096, d=512, n=2048, V=8192, K=64, sigma=1e-2),
    4: dict(kind="head", T=8192, V=50304, d=1024, K=16, sigma=5e-3, labels="zipf", logits_dtype="bf16"),
    5: dict(kind="linear", T=2048, d=512, n=2048, V=8192, K=(64, 256, 1024, 4096, 16384), sigma=1e-2),
    6: dict(kind="attn_v", B=2, S=2048, H=8, K=64, sigma=1e-2),
    # one full Dust step of a 2M-class causal LM (2.5M parameters): every pass K draws
    7: dict(kind="lm", V=8192, d=128, H=2, L=2, n=512, S=256, B=4, K=64, M=32, sigma=1e-2, sigma_es=1e-2),
}


def workload(i: int, matmul=None) -> dict:
    """Inputs of named workload i, with its estimator settings."""
    w = dict(WORKLOADS[i])
    if w["kind"] == "head":
        case = head_case(w["T"], w["V"], w["d"], seed=1000 + i, labels=w["labels"],
                         logits_dtype=w["logits_dtype"], matmul=matmul)
        case["layer"] = HEAD_LAYER
    elif w["kind"] == "lm":
        case = lm_case(w["V"], w["d"], w["H"], w["L"], w["n"], w["S"], w["B"], seed=1000 + i)
        case.update(K=w["K"], M=w["M"], sigma=w["sigma"], sigma_es=w["sigma_es"], seed_noise=LM_NOISE_SEED,
                    kind="lm")
        return case
    elif w["kind"] == "attn_v":
        case = attn_case(w["B"], w["S"], w["H"], seed=1000 + i, matmul=matmul)
        case["layer"] = WV_LAYER
    else:
        case = linear_case(w["T"], w["d"], w["n"], w["V"], seed=1000 + i)
        case["layer"] = W1_LAYER
    case.update(K=w["K"], sigma=w["sigma"], seed_noise=NOISE_SEED_BASE + i, kind=w["kind"])
    return case
