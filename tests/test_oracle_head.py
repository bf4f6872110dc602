"""Pins of the oracle's LM-head estimator against what the pages and mathematics fix.

- clean loss equals a library cross-entropy; uniform logits give ln V; V = 1 gives a zero estimate;
- each reward equals clean minus perturbed library cross-entropy on the same noise;
- same-noise linearisation: as sigma -> 0, g_hat_t -> (1/K) sum_i a_i (a_i . g_t) with the
  analytic g_t = softmax - onehot (fixes the sign and the 1/(K sigma) scale);
- statistical agreement with backprop: slope of G_hat on G near 1, cosine rising with K in the
  c_max/sqrt(1+c/K) form with the closed-form c;
- identity G_W = G_hat^T X; draw and token additivity through the offsets.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

SEED = 0x4455535400000001


def _logits(T, V, d, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    X = rng.standard_normal((T, d))
    W = rng.standard_normal((V, d)) / math.sqrt(d)
    y = rng.integers(0, V, size=T).astype(np.int32)
    return X, X @ W.T, y


def test_clean_loss_matches_library_and_uniform_case():
    X, Z, y = _logits(16, 40, 8, 1)
    _, _, ce0 = oracle.head_estimate(Z, y, 1, 1e-2, SEED, 1)
    ref = F.cross_entropy(torch.from_numpy(Z), torch.from_numpy(y).long(), reduction="none").numpy()
    np.testing.assert_allclose(ce0, ref, rtol=1e-13, atol=1e-13)
    Zu = np.full((5, 123), 0.37)
    _, _, ce0u = oracle.head_estimate(Zu, np.arange(5, dtype=np.int32), 1, 1e-2, SEED, 1)
    np.testing.assert_allclose(ce0u, math.log(123), rtol=1e-14)


def test_single_class_gives_zero_estimate():
    Z = np.random.default_rng(0).standard_normal((7, 1))
    ghat, rew, ce0 = oracle.head_estimate(Z, np.zeros(7, np.int32), 9, 0.3, SEED, 1)
    assert np.all(ce0 == 0.0) and np.all(rew == 0.0) and np.all(ghat == 0.0)


def test_rewards_are_clean_minus_perturbed_library_loss():
    X, Z, y = _logits(6, 50, 4, 2)
    K, sigma = 5, 0.05
    ghat, rew, _ = oracle.head_estimate(Z, y, K, sigma, SEED, 1, token_offset=3, draw_offset=7)
    a = oracle.noise_block(SEED, 1, 7, K, 3, 6, 50)
    zt = torch.from_numpy(Z)
    yt = torch.from_numpy(y).long()
    ce0 = F.cross_entropy(zt, yt, reduction="none").numpy()
    for i in range(K):
        cei = F.cross_entropy(zt + sigma * torch.from_numpy(a[i]), yt, reduction="none").numpy()
        np.testing.assert_allclose(rew[i], ce0 - cei, rtol=1e-10, atol=1e-14)
    # g_hat from its definition with the library rewards
    expect = -np.einsum("kt,ktv->tv", rew, a) / (K * sigma)
    np.testing.assert_allclose(ghat, expect, rtol=1e-12, atol=1e-14)


def test_same_noise_linearisation_fixes_sign_and_scale():
    T, V, d, K, sigma = 16, 48, 8, 2048, 1e-4
    X, Z, y = _logits(T, V, d, 3)
    ghat, _, _ = oracle.head_estimate(Z, y, K, sigma, SEED, 1)
    g = oracle.head_analytic(Z, y)
    a = oracle.noise_block(SEED, 1, 0, K, 0, T, V)
    lin = np.einsum("ktv,kt->tv", a, np.einsum("ktv,tv->kt", a, g)) / K
    rel = np.linalg.norm(ghat - lin) / np.linalg.norm(lin)
    assert rel < 1e-4
    # the deviation shrinks with sigma (second-order term)
    ghat2, _, _ = oracle.head_estimate(Z, y, K, 4 * sigma, SEED, 1)
    rel2 = np.linalg.norm(ghat2 - lin) / np.linalg.norm(lin)
    assert rel2 > 2 * rel


def test_backprop_agreement_slope_and_cosine_law():
    T, V, d = 24, 64, 12
    X, Z, y = _logits(T, V, d, 4)
    g = oracle.head_analytic(Z, y)
    G = g.T @ X
    c = oracle.cosine_law_c(g, X)
    cos_by_K = {}
    for K in (64, 256, 1024):
        cs, slopes = [], []
        for s in range(6):
            ghat, _, _ = oracle.head_estimate(Z, y, K, 1e-2, SEED + 100 * s, 1)
            Gh = oracle.grad_w(ghat, X)
            cs.append(oracle.cosine(Gh, G))
            slopes.append(float((Gh * G).sum() / (G * G).sum()))
        cos_by_K[K] = float(np.mean(cs))
        pred = 1.0 / math.sqrt(1.0 + c / K)
        assert abs(cos_by_K[K] - pred) < 0.04, (K, cos_by_K[K], pred)
        if K == 1024:
            assert abs(np.mean(slopes) - 1.0) < 0.05
    assert cos_by_K[64] < cos_by_K[256] < cos_by_K[1024]


def test_weight_gradient_identity_and_additivity():
    T, V, d, K, K1 = 10, 33, 5, 12, 5
    X, Z, y = _logits(T, V, d, 5)
    sigma = 2e-2
    gh, r, _ = oracle.head_estimate(Z, y, K, sigma, SEED, 1)
    gw = oracle.grad_w(gh, X)
    np.testing.assert_allclose(gw, sum(np.outer(gh[t], X[t]) for t in range(T)), rtol=1e-12, atol=1e-14)
    g1, r1, _ = oracle.head_estimate(Z, y, K1, sigma, SEED, 1)
    g2, r2, _ = oracle.head_estimate(Z, y, K - K1, sigma, SEED, 1, draw_offset=K1)
    np.testing.assert_allclose(K * gh, K1 * g1 + (K - K1) * g2, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(np.concatenate([r1, r2]), r)
    # token shards: rows t >= 4 computed alone with token_offset 4
    g3, _, _ = oracle.head_estimate(Z[4:], y[4:], K, sigma, SEED, 1, token_offset=4)
    np.testing.assert_array_equal(g3, gh[4:])
