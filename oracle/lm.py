"""Oracle of one full Dust update step on a small causal language model.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and the CPU-baseline leg of the benchmark may use it; the HIP
library never calls it and shares no code with it.

What the pages fix:
  * TL;DR page (agentlenshq.com), section 1, "reducing interference": each layer
    type is jittered in a forward pass of its own with a noise scale of its own;
    attention internals are jittered with only the attention output recomputed;
    the head is jittered on cached logits.  Section 1, "credit assignment without
    backprop": reward = loss reduction at the token, g_hat_t = -(1/(K sigma))
    sum_i r_t^(i) a_t^(i), G_W = sum_t g_hat_t x_t^T.  Section 2, "pretraining
    results": the optimiser is SGD with momentum.
  * iitog.ru, mechanics paragraph: every weight is trained by the per-token
    estimator except the 2L residual mixing scalars (L layers), which ordinary
    weight-space evolution strategies train; attention internals are judged by
    the error at the attention output over current and future tokens.

Readings where the pages are silent (each also listed in the design notes):
  * Model: tokens t = b S + s; x_0 = E[token] + P[s]; L pre-LN blocks
        x <- x + alpha_l * W_O attn(LN(x) W_Q^T, LN(x) W_K^T, LN(x) W_V^T)
        x <- x + beta_l  * W_2 GELU(W_1 LN(x))
    then LN, head W_head, cross-entropy against the next token.  Causal
    multi-head attention within each sequence, scale 1/sqrt(d_h); exact-erf
    GELU; LN without affine (eps given); no biases; W stored [out, in].  The
    2L residual mixing scalars are (alpha_l, beta_l), one per residual branch.
  * Passes (all at the same parameters, then one SGD-momentum update):
      - head: the head estimator on the cached logits;
      - one pass per linear type "emb" (the embedding sum x_0), "o" (W_O
        output), "up" (W_1 output), "down" (W_2 output): every point of that
        type (one per layer) is perturbed in the same draw with its own noise,
        the rest of the network is recomputed, and the reward of token t is its
        own loss reduction CE_t - CE'_t (no future-token discount);
      - attention internals "q", "k", "v" per layer: the attention estimator
        with the error at the attention output e_l = g_hat_O,l W_O,l, i.e. the
        W_O pass's output-error estimate taken back through W_O;
      - residual scalars: antithetic ES on the summed loss with M pairs,
        g = (1/(2 M sigma)) sum_j (L(s + sigma eps_j) - L(s - sigma eps_j)) eps_j.
    The tokens' losses are summed throughout (as in the estimator).
  * Weight gradients: G = g_hat^T (layer input); for the embeddings, the
    input is one-hot: G_E[v] = sum over tokens equal to v of g_hat, G_P[s] =
    sum over sequences of g_hat at position s.
  * SGD with momentum (no dampening, no weight decay): m <- mu m + G,
    theta <- theta - lr m; the scalars take their own learning rate.
  * Noise counters: layer word 1 (embedding), 2 (head), 3 (ES, draw j = pair,
    token 0, channel = scalar index), 16 (l + 1) + {q 0, k 1, v 2, o 3, up 4,
    down 5} for layer l.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import attn_estimate, causal_attention, gelu, head_estimate, noise, noise_block

LID_EMB, LID_HEAD, LID_ES = 1, 2, 3
KINDS = ("q", "k", "v", "o", "up", "down")
ACT_TYPES = ("emb", "o", "up", "down")
ALL_TYPES = ("emb", "q", "k", "v", "o", "up", "down", "head")


def lid(layer: int, kind: str) -> int:
    """Noise-counter layer word of the linear ``kind`` in block ``layer``."""
    return 16 * (layer + 1) + KINDS.index(kind)


@dataclass(frozen=True)
class LMConfig:
    V: int
    d: int
    H: int
    L: int
    n: int
    S: int
    eps: float = 1e-5


def param_shapes(cfg: LMConfig):
    """Named tensors of the packed parameter vector, in storage order."""
    V, d, n = cfg.V, cfg.d, cfg.n
    out = [("emb", (V, d)), ("pos", (cfg.S, d))]
    for l in range(cfg.L):
        out += [(f"wq{l}", (d, d)), (f"wk{l}", (d, d)), (f"wv{l}", (d, d)), (f"wo{l}", (d, d)),
                (f"w1{l}", (n, d)), (f"w2{l}", (d, n))]
    out += [("head", (V, d)), ("scal", (2 * cfg.L,))]
    return out


def param_count(cfg: LMConfig) -> int:
    return int(sum(np.prod(s) for _, s in param_shapes(cfg)))


def unpack(cfg: LMConfig, flat) -> dict:
    """Views of the packed vector by name (scal = alpha_0, beta_0, alpha_1, ...)."""
    flat = np.asarray(flat)
    out, o = {}, 0
    for name, shp in param_shapes(cfg):
        m = int(np.prod(shp))
        out[name] = flat[o:o + m].reshape(shp)
        o += m
    return out


def _ln(x, eps):
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def _ce(z, y):
    m = z.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(z - m).sum(axis=1))
    return lse - z[np.arange(z.shape[0]), y]


def forward(cfg: LMConfig, flat, tokens, labels, inject=None, scal=None):
    """Forward pass in fp64.  ``inject`` maps a point ("emb",) or (layer, kind)
    with kind in o/up/down to an additive perturbation of that linear output;
    ``scal`` replaces the residual scalars.  Returns (ce [T], cache)."""
    p = {k: np.asarray(v, np.float64) for k, v in unpack(cfg, flat).items()}
    tokens = np.asarray(tokens, np.int64)
    labels = np.asarray(labels, np.int64)
    inject = inject or {}
    s = p["scal"] if scal is None else np.asarray(scal, np.float64)
    T = tokens.shape[0]
    c = {}
    x = p["emb"][tokens] + p["pos"][np.arange(T) % cfg.S]
    if ("emb",) in inject:
        x = x + inject[("emb",)]
    c["x0"] = x
    for l in range(cfg.L):
        u1 = _ln(x, cfg.eps)
        q, k, v = u1 @ p[f"wq{l}"].T, u1 @ p[f"wk{l}"].T, u1 @ p[f"wv{l}"].T
        o = causal_attention(q, k, v, cfg.S, cfg.H)
        ba = o @ p[f"wo{l}"].T
        if (l, "o") in inject:
            ba = ba + inject[(l, "o")]
        xm = x + s[2 * l] * ba
        u2 = _ln(xm, cfg.eps)
        h = u2 @ p[f"w1{l}"].T
        if (l, "up") in inject:
            h = h + inject[(l, "up")]
        m = gelu(h)
        bm = m @ p[f"w2{l}"].T
        if (l, "down") in inject:
            bm = bm + inject[(l, "down")]
        c.update({f"x{l}": x, f"u1_{l}": u1, f"q{l}": q, f"k{l}": k, f"v{l}": v, f"o{l}": o, f"ba{l}": ba,
                  f"xm{l}": xm, f"u2_{l}": u2, f"h{l}": h, f"m{l}": m, f"bm{l}": bm})
        x = xm + s[2 * l + 1] * bm
    uf = _ln(x, cfg.eps)
    z = uf @ p["head"].T
    c.update({"xL": x, "uf": uf, "z": z})
    return _ce(z, labels), c


def _points(cfg: LMConfig, kind: str):
    if kind == "emb":
        return [(("emb",), LID_EMB, cfg.d)]
    width = cfg.n if kind == "up" else cfg.d
    return [((l, kind), lid(l, kind), width) for l in range(cfg.L)]


def activation_pass(cfg: LMConfig, flat, tokens, labels, kind: str, K: int, sigma: float, seed: int,
                    draw_offset: int = 0):
    """One layer-type pass: every point of ``kind`` perturbed by sigma a in the same
    draw, the network recomputed, r_t = CE_t - CE'_t.  Returns (rewards [K,T],
    {point: g_hat [T, width]}, clean ce)."""
    if kind not in ACT_TYPES:
        raise ValueError("kind must be one of " + ", ".join(ACT_TYPES))
    ce0, _ = forward(cfg, flat, tokens, labels)
    T = len(tokens)
    pts = _points(cfg, kind)
    ghat = {pt: np.zeros((T, w)) for pt, _, w in pts}
    rew = np.zeros((K, T))
    for i in range(K):
        a = {pt: noise_block(seed, li, draw_offset + i, 1, 0, T, w)[0] for pt, li, w in pts}
        ce1, _ = forward(cfg, flat, tokens, labels, inject={pt: sigma * a[pt] for pt in a})
        rew[i] = ce0 - ce1
        for pt in a:
            ghat[pt] -= rew[i][:, None] * a[pt]
    return rew, {pt: g / (K * sigma) for pt, g in ghat.items()}, ce0


def es_scalars(cfg: LMConfig, flat, tokens, labels, M: int, sigma: float, seed: int):
    """Antithetic weight-space ES on the 2L residual scalars, summed loss.
    Returns (g [2L], dL_plus [M], dL_minus [M]) with dL = L(perturbed) - L(clean)."""
    base = unpack(cfg, flat)["scal"].astype(np.float64)
    L0 = forward(cfg, flat, tokens, labels)[0].sum()
    g = np.zeros(2 * cfg.L)
    dp, dm = np.zeros(M), np.zeros(M)
    for j in range(M):
        eps = noise(seed, LID_ES, j, 0, 2 * cfg.L)
        dp[j] = forward(cfg, flat, tokens, labels, scal=base + sigma * eps)[0].sum() - L0
        dm[j] = forward(cfg, flat, tokens, labels, scal=base - sigma * eps)[0].sum() - L0
        g += (dp[j] - dm[j]) * eps
    return g / (2 * M * sigma), dp, dm


def _pack_like(cfg: LMConfig, grads: dict) -> np.ndarray:
    return np.concatenate([np.asarray(grads[name], np.float64).reshape(-1) for name, _ in param_shapes(cfg)])


def estimate(cfg: LMConfig, flat, tokens, labels, K: int, M: int, sigma: dict, sigma_es: float, seed: int):
    """Every gradient estimate of one Dust step at the parameters ``flat``.

    sigma: noise scale per type (keys of ALL_TYPES).  Returns (G packed like the
    parameters, info) with info holding each pass's rewards and output errors."""
    p = {k: np.asarray(v, np.float64) for k, v in unpack(cfg, flat).items()}
    tokens = np.asarray(tokens, np.int64)
    labels = np.asarray(labels, np.int64)
    T, S = len(tokens), cfg.S
    ce0, c = forward(cfg, flat, tokens, labels)
    G, info = {}, {"ce": ce0}
    # head on the cached logits
    gz, rz, _ = head_estimate(c["z"], labels.astype(np.int32), K, sigma["head"], seed, LID_HEAD)
    G["head"] = gz.T @ c["uf"]
    info["rew_head"] = rz
    gh = {("head",): gz}
    # layer-type passes
    for kind in ACT_TYPES:
        rew, g, _ = activation_pass(cfg, flat, tokens, labels, kind, K, sigma[kind], seed)
        info["rew_" + kind] = rew
        gh.update(g)
    ge = gh[("emb",)]
    G["emb"] = np.zeros_like(p["emb"])
    np.add.at(G["emb"], tokens, ge)
    G["pos"] = ge.reshape(T // S, S, cfg.d).sum(axis=0)
    for l in range(cfg.L):
        G[f"wo{l}"] = gh[(l, "o")].T @ c[f"o{l}"]
        G[f"w1{l}"] = gh[(l, "up")].T @ c[f"u2_{l}"]
        G[f"w2{l}"] = gh[(l, "down")].T @ c[f"m{l}"]
        # attention internals: error at the attention output from the W_O estimate
        e = gh[(l, "o")] @ p[f"wo{l}"]
        info[f"e{l}"] = e
        for kind in ("q", "k", "v"):
            g, rew = attn_estimate(kind, c[f"q{l}"], c[f"k{l}"], c[f"v{l}"], e, S, cfg.H, K, sigma[kind], seed,
                                   lid(l, kind))
            G[f"w{kind}{l}"] = g.T @ c[f"u1_{l}"]
            info[f"rew_{kind}{l}"] = rew
            gh[(l, kind)] = g
    gs, dp, dm = es_scalars(cfg, flat, tokens, labels, M, sigma_es, seed)
    G["scal"] = gs
    info["es_plus"], info["es_minus"] = dp, dm
    info["ghat"] = gh
    return _pack_like(cfg, G), info


def sgd_momentum(cfg: LMConfig, flat, mom, G, lr: float, lr_scalar: float, mu: float):
    """m <- mu m + G; theta <- theta - lr m (lr_scalar for the residual scalars).
    Returns (theta', m')."""
    flat = np.asarray(flat, np.float64)
    m2 = mu * np.asarray(mom, np.float64) + np.asarray(G, np.float64)
    rate = np.full(flat.shape, lr)
    rate[-2 * cfg.L:] = lr_scalar
    return flat - rate * m2, m2


def step(cfg: LMConfig, flat, mom, tokens, labels, K: int, M: int, sigma: dict, sigma_es: float, seed: int,
         lr: float, lr_scalar: float, mu: float):
    """One Dust update: every estimate at ``flat``, then SGD with momentum."""
    G, info = estimate(cfg, flat, tokens, labels, K, M, sigma, sigma_es, seed)
    theta, m2 = sgd_momentum(cfg, flat, mom, G, lr, lr_scalar, mu)
    return theta, m2, G, info
