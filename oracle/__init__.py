"""Oracle for the Dust per-token activation-perturbation gradient estimator.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
CPU reference the HIP library is checked against.  Only the tests, the smoke
check and the CPU-baseline leg of the benchmark may import it.  It shares no
code with the HIP library, and the library never calls it.

Pieces:
  * ``dust_oracle.c`` (plain C, fp64): Philox4x32-10, Box-Muller, and the
    LM-head estimator on cached logits.
  * this module (numpy, fp64): the interior MLP-linear estimator with its
    downstream recomputed per draw, the weight-gradient outer product, and the
    analytic (backprop) gradients used as pins.

The method (the Dust pages, Q Labs 2026):
  * "Dust: zeroth-order Transformer pretraining without backprop" (TL;DR page,
    agentlenshq.com), section 1: per-token Gaussian noise on each linear
    output ("activation-space perturbation"); reward = loss reduction at the
    token; g_hat_t = -(1/(K sigma)) sum_i r_t^(i) a_t^(i); G_W = sum_t g_hat_t
    x_t^T ("credit assignment without backprop"); the head is jittered on
    cached logits ("reducing interference").  Section 2, "gradient
    alignment": cos(K) = c_max / sqrt(1 + c/K).
  * "Training Transformers without backprop" (news article, tahou.com),
    mechanism paragraph: cache unperturbed intermediates, head on cached
    logits with only the loss recomputed.
  * "Dust: pretraining transformers without backpropagation" (iitog.ru),
    mechanics paragraph: noise on every linear output independently per token;
    the reward-weighted mean noise is the output-error estimate, its outer
    product with the layer input the weight gradient.

Readings where the pages are silent (each also listed in the design notes):
  reward r = CE_clean - CE_perturbed in nats; divide by K (not K-1); no
  baseline other than the clean loss; the tokens' losses are summed; noise
  a ~ N(0, I) scaled by sigma; interior block is pre-LN with no biases and no
  LN affine, exact-erf GELU, LN eps given; the interior downstream runs with
  bf16 GEMM operands: the perturbed activation h + sigma a is an fp32 tensor
  (rounded to fp32, like the cached h it perturbs); the GELU output and the LN
  output are each rounded to fp32 and then to bf16 (round to nearest even) --
  the bf16 decision is taken from an fp32 value, as in the kernels.  With
  ``quantize=False`` the downstream is exact fp64 (used for the linearisation
  pins).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dust_oracle.c")
_SO = os.path.join(_HERE, "_liboracle.so")
_lib_handle = None

_u32p = np.ctypeslib.ndpointer(dtype=np.uint32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")


def build(force: bool = True) -> str:
    """Compile the C part of the oracle with gcc (plain C99 + OpenMP)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-D_DEFAULT_SOURCE", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_SO):
            build(force=True)
        L = ctypes.CDLL(_SO)
        L.orc_philox4x32_10.argtypes = [_u32p, _u32p, _u32p]
        L.orc_noise_raw.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                    ctypes.c_uint32, ctypes.c_int64, _u32p]
        L.orc_noise.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                ctypes.c_uint32, ctypes.c_int64, _f64p]
        L.orc_noise_block.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                      ctypes.c_int64, ctypes.c_uint32, ctypes.c_int64,
                                      ctypes.c_int64, _f64p]
        L.orc_head_estimate.argtypes = [_f64p, _i32p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_double, ctypes.c_uint64,
                                        ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                        _f64p, ctypes.c_void_p, ctypes.c_void_p]
        L.orc_window_offset.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                        ctypes.c_uint32]
        L.orc_window_offset.restype = ctypes.c_uint32
        L.orc_head_estimate_subset.argtypes = [_f64p, _i32p, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.c_uint64,
                                               ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                               _f64p, ctypes.c_void_p, ctypes.c_void_p]
        L.orc_num_threads.restype = ctypes.c_int
        _lib_handle = L
    return _lib_handle


def num_threads() -> int:
    """Host threads the oracle's OpenMP loops use."""
    return int(_lib().orc_num_threads())


# --------------------------------------------------------------------------
# Noise stream
# --------------------------------------------------------------------------
def philox4x32_10(ctr, key) -> np.ndarray:
    """Philox4x32-10 (SC'11) of a 4-word counter under a 2-word key."""
    out = np.zeros(4, np.uint32)
    _lib().orc_philox4x32_10(np.asarray(ctr, np.uint32), np.asarray(key, np.uint32), out)
    return out


def noise_raw(seed: int, layer: int, draw: int, token: int, n: int) -> np.ndarray:
    """Raw Philox words behind channels [0, n) of one (draw, token)."""
    out = np.zeros(4 * ((n + 3) // 4), np.uint32)
    _lib().orc_noise_raw(seed, layer, draw, token, n, out)
    return out


def noise(seed: int, layer: int, draw: int, token: int, n: int) -> np.ndarray:
    """Standard-normal noise a_t^(i)[0..n) (fp64)."""
    out = np.zeros(n, np.float64)
    _lib().orc_noise(seed, layer, draw, token, n, out)
    return out


def noise_block(seed: int, layer: int, draw_offset: int, K: int, token_offset: int,
                T: int, n: int) -> np.ndarray:
    """Noise for draws [draw_offset, +K) x tokens [token_offset, +T): shape [K,T,n]."""
    out = np.zeros((K, T, n), np.float64)
    _lib().orc_noise_block(seed, layer, draw_offset, K, token_offset, T, n, out)
    return out


# --------------------------------------------------------------------------
# LM head on cached logits
# --------------------------------------------------------------------------
def head_estimate(logits, labels, K: int, sigma: float, seed: int, layer: int,
                  token_offset: int = 0, draw_offset: int = 0):
    """Head estimator on cached logits [T,V] (fp32 or bf16-valued; upcast exactly).

    Returns (ghat [T,V], rewards [K,T], ce0 [T]), all fp64.
    """
    z = np.ascontiguousarray(logits, dtype=np.float64)
    y = np.ascontiguousarray(labels, dtype=np.int32)
    T, V = z.shape
    ghat = np.zeros((T, V), np.float64)
    rew = np.zeros((K, T), np.float64)
    ce0 = np.zeros(T, np.float64)
    _lib().orc_head_estimate(z, y, T, V, K, float(sigma), seed, layer, token_offset,
                             draw_offset, ghat, rew.ctypes.data, ce0.ctypes.data)
    return ghat, rew, ce0


def window_offset(seed: int, layer: int, draw: int, token: int, nq: int) -> int:
    """Offset of the perturbed window of channel quads for (token, draw) in the
    vocabulary-subset head estimator (see head_estimate_subset)."""
    return int(_lib().orc_window_offset(seed, layer, draw, token, nq))


def head_estimate_subset(logits, labels, K: int, m: int, sigma: float, seed: int, layer: int,
                         token_offset: int = 0, draw_offset: int = 0):
    """Head estimator with a vocabulary subset per draw (TL;DR page, section 1,
    "reducing interference"; the pages give no subset rule, this is a reading): a cyclic
    window of m/4 channel quads at a per-(token, draw) Philox offset, plus the
    label, perturbed with the full estimator's noise; the plain cross-entropy of
    the perturbed row; each channel weighted by the inverse of its inclusion
    probability.  Returns (ghat [T,V], rewards [K,T], ce0 [T]), fp64."""
    if m < 4 or m % 4:
        raise ValueError("m must be a positive multiple of 4")
    z = np.ascontiguousarray(logits, dtype=np.float64)
    y = np.ascontiguousarray(labels, dtype=np.int32)
    T, V = z.shape
    ghat = np.zeros((T, V), np.float64)
    rew = np.zeros((K, T), np.float64)
    ce0 = np.zeros(T, np.float64)
    _lib().orc_head_estimate_subset(z, y, T, V, K, m, float(sigma), seed, layer, token_offset,
                                    draw_offset, ghat, rew.ctypes.data, ce0.ctypes.data)
    return ghat, rew, ce0


def grad_w(ghat, x) -> np.ndarray:
    """Weight-gradient estimate G_W = sum_t g_hat_t x_t^T = G^T X (TL;DR page,
    section 1, eq. for G_W), in fp64."""
    return np.asarray(ghat, np.float64).T @ np.asarray(x, np.float64)


def head_analytic(logits, labels) -> np.ndarray:
    """Backprop gradient of sum_t CE_t w.r.t. the logits: softmax(z_t) - onehot(y_t)."""
    z = np.asarray(logits, np.float64)
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    p /= p.sum(axis=1, keepdims=True)
    p[np.arange(z.shape[0]), np.asarray(labels)] -= 1.0
    return p


# --------------------------------------------------------------------------
# Interior MLP linear (W1 of a pre-LN block), downstream recomputed per draw
# --------------------------------------------------------------------------
def bf16_round(x) -> np.ndarray:
    """fp32 -> bf16, round to nearest even, returned as the (exact) fp64 values."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def bf16_bits_value(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _erf(x):
    from scipy.special import erf
    return erf(x)


def gelu(x) -> np.ndarray:
    """Exact-erf GELU: x * Phi(x)."""
    return 0.5 * x * (1.0 + _erf(x / np.sqrt(2.0)))


def layernorm(y, eps: float) -> np.ndarray:
    """LayerNorm with no affine: (y - mean) / sqrt(var + eps), population variance."""
    mu = y.mean(axis=1, keepdims=True)
    var = ((y - mu) ** 2).mean(axis=1, keepdims=True)
    return (y - mu) / np.sqrt(var + eps)


def _ce_rows(z, y) -> np.ndarray:
    m = z.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(z - m).sum(axis=1))
    return lse - z[np.arange(z.shape[0]), y]


def mlp_downstream_ce(htilde, xres, labels, w2, w_head, eps: float, quantize: bool = True):
    """Per-row loss of the cached downstream of W1:
    m = GELU(h~) -> o = W2 m -> y = x + o -> f = LN(y) -> z = W_head f -> CE(z, label).
    With ``quantize`` the GEMM operands m and f are bf16 (fp32 then RNE)."""
    m = gelu(htilde)
    if quantize:
        m = bf16_round(m)
    o = m @ w2.T
    f = layernorm(xres + o, eps)
    if quantize:
        f = bf16_round(f)
    return _ce_rows(f @ w_head.T, labels)


def linear_estimate(h, x_res, w2_bits, w_head_bits, labels, K: int, sigma: float, eps: float,
                    seed: int, layer: int, token_offset: int = 0, draw_offset: int = 0,
                    tokens=None, quantize: bool = True, token_chunk: int = 64):
    """Interior-linear estimator on the rows ``tokens`` (default: all).

    For each token t: CE0 = D_t(h_t); for each draw i: r = CE0 - D_t(h_t + sigma a),
    g_hat_t = -(1/(K sigma)) sum_i r a.  Returns (ghat [nt,n], rewards [K,nt], ce0 [nt]).
    """
    h = np.asarray(h, np.float64)
    xr = np.asarray(x_res, np.float64)
    w2 = bf16_bits_value(w2_bits) if np.asarray(w2_bits).dtype == np.uint16 else np.asarray(w2_bits, np.float64)
    wh = bf16_bits_value(w_head_bits) if np.asarray(w_head_bits).dtype == np.uint16 else np.asarray(w_head_bits, np.float64)
    lab = np.asarray(labels, np.int64)
    T, n = h.shape
    toks = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    nt = len(toks)
    ghat = np.zeros((nt, n))
    rew = np.zeros((K, nt))
    ce0 = np.zeros(nt)
    for c0 in range(0, nt, token_chunk):
        sel = toks[c0:c0 + token_chunk]
        b = len(sel)
        a = np.empty((K, b, n))
        for j, t in enumerate(sel):
            for i in range(K):
                a[i, j] = noise(seed, layer, draw_offset + i, token_offset + int(t), n)
        hrows = np.concatenate([h[sel][None], h[sel][None] + sigma * a], axis=0).reshape(-1, n)
        if quantize:
            # the perturbed activation is an fp32 tensor, like the cached h it perturbs
            hrows = hrows.astype(np.float32).astype(np.float64)
        xrows = np.broadcast_to(xr[sel][None], (K + 1, b, xr.shape[1])).reshape(-1, xr.shape[1])
        lrows = np.broadcast_to(lab[sel][None], (K + 1, b)).reshape(-1)
        ce = mlp_downstream_ce(hrows, xrows, lrows, w2, wh, eps, quantize).reshape(K + 1, b)
        r = ce[0][None, :] - ce[1:]
        ce0[c0:c0 + b] = ce[0]
        rew[:, c0:c0 + b] = r
        ghat[c0:c0 + b] = -np.einsum("kb,kbn->bn", r, a) / (K * sigma)
    return ghat, rew, ce0


def mlp_analytic(h, x_res, w2_bits, w_head_bits, labels, eps: float) -> np.ndarray:
    """Backprop gradient of sum_t CE_t w.r.t. the W1 output h (fp64, no rounding),
    by the chain rule through head, LayerNorm, residual, W2 and GELU."""
    from scipy.special import erf
    h = np.asarray(h, np.float64)
    xr = np.asarray(x_res, np.float64)
    w2 = bf16_bits_value(w2_bits) if np.asarray(w2_bits).dtype == np.uint16 else np.asarray(w2_bits, np.float64)
    wh = bf16_bits_value(w_head_bits) if np.asarray(w_head_bits).dtype == np.uint16 else np.asarray(w_head_bits, np.float64)
    m = gelu(h)
    y = xr + m @ w2.T
    mu = y.mean(axis=1, keepdims=True)
    s = np.sqrt(((y - mu) ** 2).mean(axis=1, keepdims=True) + eps)
    fh = (y - mu) / s
    gz = head_analytic(fh @ wh.T, labels)
    gf = gz @ wh
    gy = (gf - gf.mean(axis=1, keepdims=True) - fh * (gf * fh).mean(axis=1, keepdims=True)) / s
    gm = gy @ w2
    dgelu = 0.5 * (1.0 + erf(h / np.sqrt(2.0))) + h * np.exp(-0.5 * h * h) / np.sqrt(2.0 * np.pi)
    return gm * dgelu


def cosine(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def cosine_law_c(g, x) -> float:
    """Constant c of the alignment law cos(K) = 1/sqrt(1 + c/K) in the linear regime.

    With r = -sigma a.g the estimate g_hat = (1/K) sum_i a_i (a_i.g) has covariance
    (|g|^2 I + g g^T)/K for a ~ N(0, I_n), so E|G_hat - G|_F^2 = (n+1) sum_t
    |x_t|^2 |g_t|^2 / K and c = (n+1) sum_t |x_t|^2 |g_t|^2 / |G|_F^2 (TL;DR page,
    section 2 "gradient alignment": the c_max/sqrt(1+c/K) form, with c_max = 1)."""
    g = np.asarray(g, np.float64)
    x = np.asarray(x, np.float64)
    G = g.T @ x
    n = g.shape[1]
    num = (n + 1) * np.sum((x * x).sum(1) * (g * g).sum(1))
    return float(num / np.sum(G * G))


# --------------------------------------------------------------------------
# Attention internals: the value projection
# --------------------------------------------------------------------------
# TL;DR page, section 1, "credit assignment without backprop": attention
# internals are handled like the other linear layers, but their reward is the
# change of the attention output rather than the token's loss; the news
# article's mechanism paragraph judges that change against the error signal;
# the iitog.ru mechanics paragraph takes the error at the attention output over
# the current and future tokens.  Reading: with e_s the error (gradient of the
# loss) at the attention output of token s, the reward of token t's noise is
# the first-order loss reduction over the outputs it can move,
#     r_t = -sum_{s >= t, same sequence} <e_s, o'_s - o_s>,
# every token of the sequence being perturbed in the same draw.  For the value
# projection (y_t = v_t = W_V u_t) only the values move, so the probabilities
# stay those of the clean pass.

def causal_attention(q, k, v, S: int, H: int) -> np.ndarray:
    """Causal multi-head self-attention within sequences of S tokens (tokens
    t = b S + s): o_s = concat_h sum_{t <= s} softmax_t(q_s . k_t / sqrt(dh)) v_t,
    dh = d / H, in fp64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, d = q.shape
    dh = d // H
    o = np.zeros((T, d))
    future = np.triu(np.ones((S, S), bool), 1)
    for b in range(T // S):
        rows = slice(b * S, (b + 1) * S)
        for h in range(H):
            ch = slice(h * dh, (h + 1) * dh)
            L = q[rows, ch] @ k[rows, ch].T / np.sqrt(dh)
            L[future] = -np.inf
            L -= L.max(axis=1, keepdims=True)
            P = np.exp(L)
            P /= P.sum(axis=1, keepdims=True)
            o[rows, ch] = P @ v[rows, ch]
    return o


def _perturbed(proj: str, q, k, v, pert):
    return (q + pert, k, v) if proj == "q" else (q, k + pert, v) if proj == "k" else (q, k, v + pert)


def _check_proj(proj: str):
    if proj not in ("q", "k", "v"):
        raise ValueError("proj must be 'q', 'k' or 'v'")


def attn_estimate(proj: str, q, k, v, e, S: int, H: int, K: int, sigma: float, seed: int, layer: int,
                  token_offset: int = 0, draw_offset: int = 0):
    """Estimator of the attention projection ``proj`` ('q', 'k' or 'v'): per draw i
    its output y' = y + sigma a^(i) on every token, o' the recomputed attention
    output, c_s = <e_s, o'_s - o_s>, and the reward of token t the change over the
    outputs its perturbation can move: r_t = -sum_{s >= t in t's sequence} c_s for
    keys and values, r_t = -c_t for queries (o_s depends on q_t only for s = t).
    g_hat_t = -(1/(K sigma)) sum_i r_t^(i) a_t^(i).  Returns (g_hat [T,d], rewards [K,T])."""
    _check_proj(proj)
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    e = np.asarray(e, np.float64)
    T, d = q.shape
    o = causal_attention(q, k, v, S, H)
    ghat = np.zeros((T, d))
    rew = np.zeros((K, T))
    for i in range(K):
        a = noise_block(seed, layer, draw_offset + i, 1, token_offset, T, d)[0]
        c = np.sum(e * (causal_attention(*_perturbed(proj, q, k, v, sigma * a), S, H) - o), axis=1)
        if proj == "q":
            rew[i] = -c
        else:
            for b in range(T // S):
                cs = c[b * S:(b + 1) * S]
                rew[i, b * S:(b + 1) * S] = -np.cumsum(cs[::-1])[::-1]
        ghat -= rew[i][:, None] * a
    return ghat / (K * sigma), rew


def attn_v_estimate(q, k, v, e, S: int, H: int, K: int, sigma: float, seed: int, layer: int,
                    token_offset: int = 0, draw_offset: int = 0):
    """The value-projection estimator (attn_estimate with proj = 'v')."""
    return attn_estimate("v", q, k, v, e, S, H, K, sigma, seed, layer, token_offset, draw_offset)


def attn_estimate_tokens(proj: str, q, k, v, e, S: int, H: int, K: int, sigma: float, seed: int, layer: int,
                         tokens, token_offset: int = 0, draw_offset: int = 0):
    """attn_estimate on the tokens ``tokens`` only: the attention outputs the rewards
    of those tokens need (query s = t for queries, s >= t in the sequence otherwise)
    are recomputed row by row (for sampled checks of large inputs).  Returns
    (g_hat [len(tokens), d], rewards [K, len(tokens)])."""
    _check_proj(proj)
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    e = np.asarray(e, np.float64)
    T, d = q.shape
    dh = d // H
    tokens = [int(t) for t in tokens]
    span = (lambda t: [t]) if proj == "q" else (lambda t: list(range(t, (t // S + 1) * S)))
    need = sorted({s for t in tokens for s in span(t)})

    def row(s, qq, kk, vv):  # attention output of query s
        b0 = (s // S) * S
        out = np.zeros(d)
        for h in range(H):
            ch = slice(h * dh, (h + 1) * dh)
            L = kk[b0:s + 1, ch] @ qq[s, ch] / np.sqrt(dh)
            P = np.exp(L - L.max())
            out[ch] = (P / P.sum()) @ vv[b0:s + 1, ch]
        return out

    o = {s: row(s, q, k, v) for s in need}
    ghat = np.zeros((len(tokens), d))
    rew = np.zeros((K, len(tokens)))
    for i in range(K):
        a = noise_block(seed, layer, draw_offset + i, 1, token_offset, T, d)[0]
        qq, kk, vv = _perturbed(proj, q, k, v, sigma * a)
        c = {s: float(e[s] @ (row(s, qq, kk, vv) - o[s])) for s in need}
        for j, t in enumerate(tokens):
            rew[i, j] = -sum(c[s] for s in span(t))
            ghat[j] -= rew[i, j] * a[t]
    return ghat / (K * sigma), rew


def attn_v_estimate_tokens(q, k, v, e, S: int, H: int, K: int, sigma: float, seed: int, layer: int,
                           tokens, token_offset: int = 0, draw_offset: int = 0):
    """The value-projection estimator on a token subset (attn_estimate_tokens, 'v')."""
    return attn_estimate_tokens("v", q, k, v, e, S, H, K, sigma, seed, layer, tokens, token_offset, draw_offset)


def attn_v_analytic(q, k, e, S: int, H: int) -> np.ndarray:
    """Gradient of sum_s <e_s, o_s> w.r.t. the values: per head, P^T e (fp64)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    e = np.asarray(e, np.float64)
    T, d = q.shape
    dh = d // H
    g = np.zeros((T, d))
    future = np.triu(np.ones((S, S), bool), 1)
    for b in range(T // S):
        rows = slice(b * S, (b + 1) * S)
        for h in range(H):
            ch = slice(h * dh, (h + 1) * dh)
            L = q[rows, ch] @ k[rows, ch].T / np.sqrt(dh)
            L[future] = -np.inf
            L -= L.max(axis=1, keepdims=True)
            P = np.exp(L)
            P /= P.sum(axis=1, keepdims=True)
            g[rows, ch] = P.T @ e[rows, ch]
    return g
