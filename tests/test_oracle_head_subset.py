"""Pins of the oracle's vocabulary-subset head estimator (TL;DR page, section 1,
"reducing interference": only part of the vocabulary is perturbed per head draw; the
subset rule -- a cyclic window of m/4 channel quads at a per-(token, draw) offset, plus the
label -- and the inverse-inclusion-probability weights are a reading of that passage).

- a window covering the vocabulary reproduces the (separately pinned) full estimator exactly;
- the window offset is uniform over the quads (chi-square) and the label is always perturbed;
- each reward equals clean minus perturbed library cross-entropy, the perturbed row being
  the logits plus sigma a on the window and the label only;
- unbiased: as sigma -> 0 and K grows, the estimate regresses on the analytic softmax - onehot
  with slope 1 (the unweighted window estimate would give slope mq/nq).
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle

SEED = 0x4455535400000011


def _logits(T, V, d, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    X = rng.standard_normal((T, d))
    W = rng.standard_normal((V, d)) / math.sqrt(d)
    y = rng.integers(0, V, size=T).astype(np.int32)
    return X, X @ W.T, y


def test_window_covering_the_vocabulary_is_the_full_estimator():
    _, Z, y = _logits(7, 45, 6, 1)
    for m in (48, 64, 400):  # ceil(45/4) = 12 quads: any m >= 48 covers them
        full = oracle.head_estimate(Z, y, 9, 2e-2, SEED, 1, token_offset=5, draw_offset=3)
        sub = oracle.head_estimate_subset(Z, y, 9, m, 2e-2, SEED, 1, token_offset=5, draw_offset=3)
        for a, b in zip(full, sub):
            np.testing.assert_array_equal(a, b)


def test_window_offsets_are_uniform_and_label_always_perturbed():
    nq = 13
    offs = np.array([oracle.window_offset(SEED, 1, i, t, nq) for i in range(400) for t in range(50)])
    assert offs.min() >= 0 and offs.max() < nq
    counts = np.bincount(offs, minlength=nq)
    chi2 = ((counts - offs.size / nq) ** 2 / (offs.size / nq)).sum()
    assert chi2 < 40.0  # 12 degrees of freedom: the 99.99% point is about 38.1
    # with K = 1 every token's label column carries a contribution (reward * a_y != 0)
    _, Z, y = _logits(40, 52, 4, 2)
    g, r, _ = oracle.head_estimate_subset(Z, y, 1, 4, 5e-2, SEED, 1)
    assert np.all(g[np.arange(40), y] != 0.0)


def test_rewards_are_clean_minus_perturbed_library_loss_on_the_subset():
    _, Z, y = _logits(6, 50, 4, 3)
    K, m, sigma, t0, d0 = 5, 16, 0.05, 3, 7
    V = 50
    nq = (V + 3) // 4
    g, rew, _ = oracle.head_estimate_subset(Z, y, K, m, sigma, SEED, 1, token_offset=t0, draw_offset=d0)
    a = oracle.noise_block(SEED, 1, d0, K, t0, 6, V)
    zt = torch.from_numpy(Z)
    yt = torch.from_numpy(y).long()
    ce0 = F.cross_entropy(zt, yt, reduction="none").numpy()
    expect = np.zeros_like(g)
    for i in range(K):
        for t in range(6):
            o = oracle.window_offset(SEED, 1, d0 + i, t0 + t, nq)
            quads = (o + np.arange(m // 4)) % nq
            mask = np.zeros(V, bool)
            for q in quads:
                mask[4 * q:min(4 * q + 4, V)] = True
            mask[y[t]] = True
            cei = F.cross_entropy((zt[t] + sigma * torch.from_numpy(a[i, t] * mask))[None], yt[t:t + 1]).item()
            assert abs(rew[i, t] - (ce0[t] - cei)) <= 1e-10 * max(1.0, abs(ce0[t]))
            w = np.where(mask, 1.0 / ((m // 4) / nq), 0.0)
            w[y[t]] = 1.0
            expect[t] += rew[i, t] * a[i, t] * w
    np.testing.assert_allclose(g, -expect / (K * sigma), rtol=1e-12, atol=1e-14)


def test_estimate_is_unbiased_for_the_analytic_gradient():
    _, Z, y = _logits(4, 64, 8, 4)
    K, m, sigma = 24000, 16, 1e-4  # 4 of 16 quads per draw
    g, _, _ = oracle.head_estimate_subset(Z, y, K, m, sigma, SEED, 1)
    ga = oracle.head_analytic(Z, y)
    slope = float((g * ga).sum() / (ga * ga).sum())
    print(f"slope of the subset estimate on softmax - onehot: {slope:.3f}")
    assert abs(slope - 1.0) < 0.1  # the unweighted window estimate would sit near 0.25
