"""Pins of the oracle's attention projection estimators (TL;DR page, section 1,
"credit assignment without backprop": attention internals rewarded by the change of the
attention output; news article, mechanism paragraph: that change judged against the error
signal; iitog.ru, mechanics paragraph: the error at the attention output over the current
and future tokens).  Reading: r_t = -sum_{s >= t in t's sequence} <e_s, o'_s - o_s> for the
key and value projections, r_t = -<e_t, o'_t - o_t> for the query projection.

- the oracle's causal attention equals torch's scaled_dot_product_attention (fp64);
- every reward equals the definition evaluated with torch's attention on the perturbed
  q, k or v;
- the closed-form target P^T e equals torch autograd of sum_s <e_s, o_s> w.r.t. v;
- one-token sequences reduce to r = -sigma <e_t, a_t> for values and to r = 0 for queries
  and keys (a lone key's softmax weight is 1 whatever it is);
- unbiased: as K grows the estimate regresses on the analytic (autograd) gradient with
  slope 1, for each projection;
- draw additivity: two draw ranges combine to the estimate over their union.
"""
import numpy as np
import torch
import torch.nn.functional as F

import oracle

SEED = 0x4455535400000031


def _inputs(B, S, H, dh, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    T, d = B * S, H * dh
    return [rng.standard_normal((T, d)) for _ in range(4)]  # q, k, v, e


def _torch_attn(x_q, x_k, x_v, B, S, H):
    def heads(x):
        return torch.as_tensor(x, dtype=torch.float64).reshape(B, S, H, -1).permute(0, 2, 1, 3)
    o = F.scaled_dot_product_attention(heads(x_q), heads(x_k), heads(x_v), is_causal=True)
    return o.permute(0, 2, 1, 3).reshape(B * S, -1)


def test_causal_attention_is_torch_sdpa():
    B, S, H, dh = 2, 7, 3, 4
    q, k, v, _ = _inputs(B, S, H, dh, 1)
    np.testing.assert_allclose(oracle.causal_attention(q, k, v, S, H), _torch_attn(q, k, v, B, S, H).numpy(),
                               rtol=1e-12, atol=1e-12)


def test_rewards_are_the_output_change_against_the_error():
    B, S, H, dh = 2, 5, 2, 4
    q, k, v, e = _inputs(B, S, H, dh, 2)
    K, sigma, t0, d0 = 4, 3e-2, 11, 5
    g, rew = oracle.attn_v_estimate(q, k, v, e, S, H, K, sigma, SEED, 2, token_offset=t0, draw_offset=d0)
    a = oracle.noise_block(SEED, 2, d0, K, t0, B * S, H * dh)
    o = _torch_attn(q, k, v, B, S, H).numpy()
    expect = np.zeros_like(rew)
    for i in range(K):
        c = np.sum(e * (_torch_attn(q, k, v + sigma * a[i], B, S, H).numpy() - o), axis=1)
        for t in range(B * S):
            b = t // S
            expect[i, t] = -c[t:(b + 1) * S].sum()
    np.testing.assert_allclose(rew, expect, rtol=1e-9, atol=1e-13)
    np.testing.assert_allclose(g, -np.einsum("it,itd->td", rew, a) / (K * sigma), rtol=1e-12, atol=1e-14)


def test_analytic_target_is_autograd():
    B, S, H, dh = 2, 6, 2, 3
    q, k, v, e = _inputs(B, S, H, dh, 3)
    vt = torch.tensor(v, requires_grad=True)
    loss = (torch.as_tensor(e) * _torch_attn(q, k, vt, B, S, H)).sum()
    loss.backward()
    np.testing.assert_allclose(oracle.attn_v_analytic(q, k, e, S, H), vt.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_one_token_sequences_have_no_mixing():
    B, S, H, dh = 9, 1, 2, 4
    q, k, v, e = _inputs(B, S, H, dh, 4)
    K, sigma = 6, 0.1
    g, rew = oracle.attn_v_estimate(q, k, v, e, S, H, K, sigma, SEED, 2)
    a = oracle.noise_block(SEED, 2, 0, K, 0, B, H * dh)
    np.testing.assert_allclose(rew, -sigma * np.einsum("td,itd->it", e, a), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(g, np.einsum("itd,it->td", a, np.einsum("td,itd->it", e, a)) / K, rtol=1e-10)


def test_estimate_is_unbiased_for_the_analytic_gradient():
    B, S, H, dh = 2, 4, 2, 2
    q, k, v, e = _inputs(B, S, H, dh, 5)
    K, sigma = 20000, 1e-2
    g, _ = oracle.attn_v_estimate(q, k, v, e, S, H, K, sigma, SEED, 2)
    ga = oracle.attn_v_analytic(q, k, e, S, H)
    slope = float((g * ga).sum() / (ga * ga).sum())
    print(f"slope of the value-projection estimate on P^T e: {slope:.3f}, cosine {oracle.cosine(g, ga):.3f}")
    assert abs(slope - 1.0) < 0.06


def test_draw_ranges_combine():
    B, S, H, dh = 2, 5, 2, 4
    q, k, v, e = _inputs(B, S, H, dh, 6)
    sigma = 2e-2
    g_all, r_all = oracle.attn_v_estimate(q, k, v, e, S, H, 7, sigma, SEED, 2, draw_offset=3)
    g1, r1 = oracle.attn_v_estimate(q, k, v, e, S, H, 4, sigma, SEED, 2, draw_offset=3)
    g2, r2 = oracle.attn_v_estimate(q, k, v, e, S, H, 3, sigma, SEED, 2, draw_offset=7)
    np.testing.assert_allclose(r_all, np.concatenate([r1, r2]), rtol=0, atol=0)
    np.testing.assert_allclose(g_all, (4 * g1 + 3 * g2) / 7, rtol=1e-12, atol=1e-15)


def test_query_and_key_rewards_are_the_output_change_against_the_error():
    B, S, H, dh = 2, 5, 2, 4
    q, k, v, e = _inputs(B, S, H, dh, 7)
    K, sigma, t0, d0 = 3, 5e-2, 2, 9
    a = oracle.noise_block(SEED, 4, d0, K, t0, B * S, H * dh)
    o = _torch_attn(q, k, v, B, S, H).numpy()
    for proj in ("q", "k"):
        g, rew = oracle.attn_estimate(proj, q, k, v, e, S, H, K, sigma, SEED, 4, token_offset=t0, draw_offset=d0)
        expect = np.zeros_like(rew)
        for i in range(K):
            qq, kk = (q + sigma * a[i], k) if proj == "q" else (q, k + sigma * a[i])
            c = np.sum(e * (_torch_attn(qq, kk, v, B, S, H).numpy() - o), axis=1)
            for t in range(B * S):
                b = t // S
                expect[i, t] = -c[t] if proj == "q" else -c[t:(b + 1) * S].sum()
        np.testing.assert_allclose(rew, expect, rtol=1e-9, atol=1e-13)
        np.testing.assert_allclose(g, -np.einsum("it,itd->td", rew, a) / (K * sigma), rtol=1e-12, atol=1e-14)


def test_lone_queries_and_keys_move_nothing():
    B, S, H, dh = 5, 1, 2, 4
    q, k, v, e = _inputs(B, S, H, dh, 8)
    for proj in ("q", "k"):
        g, rew = oracle.attn_estimate(proj, q, k, v, e, S, H, 4, 0.1, SEED, 4)
        assert np.all(rew == 0.0) and np.all(g == 0.0)


def test_query_and_key_estimates_are_unbiased():
    B, S, H, dh = 2, 4, 2, 2
    q, k, v, e = _inputs(B, S, H, dh, 9)
    K, sigma = 20000, 1e-3
    for proj in ("q", "k"):
        x = torch.tensor(q if proj == "q" else k, requires_grad=True)
        loss = (torch.as_tensor(e) * (_torch_attn(x, k, v, B, S, H) if proj == "q"
                                      else _torch_attn(q, x, v, B, S, H))).sum()
        loss.backward()
        ga = x.grad.numpy()
        g, _ = oracle.attn_estimate(proj, q, k, v, e, S, H, K, sigma, SEED, 4)
        slope = float((g * ga).sum() / (ga * ga).sum())
        print(f"{proj}: slope on the autograd gradient {slope:.3f}, cosine {oracle.cosine(g, ga):.3f}")
        assert abs(slope - 1.0) < 0.08


def _token_subset(B, S, rng, extra):
    """First, a middle and the last token of every sequence, plus ``extra`` random ones."""
    toks = set()
    for b in range(B):
        toks.update({b * S, b * S + S // 2, b * S + S - 1})
    toks.update(int(t) for t in rng.choice(B * S, extra, replace=False))
    return sorted(toks)


def test_token_subset_checker_equals_the_full_estimator():
    # attn_estimate_tokens recomputes only the attention rows a token's reward needs;
    # row for row it must give attn_estimate's rewards and estimates, for each
    # projection, on tokens at both ends and inside each sequence (an off-by-one in
    # the span of later queries, or a wrong causal slice, breaks the first or last).
    B, S, H, dh = 3, 6, 2, 4
    q, k, v, e = _inputs(B, S, H, dh, 10)
    K, sigma, t0, d0 = 3, 4e-2, 5, 2
    toks = _token_subset(B, S, np.random.default_rng(0), 3)
    for proj in ("q", "k", "v"):
        g, rew = oracle.attn_estimate(proj, q, k, v, e, S, H, K, sigma, SEED, 6, token_offset=t0, draw_offset=d0)
        gs, rs = oracle.attn_estimate_tokens(proj, q, k, v, e, S, H, K, sigma, SEED, 6, toks,
                                             token_offset=t0, draw_offset=d0)
        np.testing.assert_allclose(rs, rew[:, toks], rtol=1e-10, atol=1e-14)
        np.testing.assert_allclose(gs, g[toks], rtol=1e-10, atol=1e-14)


def test_token_subset_checker_against_torch_attention():
    # The same subset checker against rewards formed directly from torch's causal
    # attention on the perturbed projection: keys and values sum the output change
    # over the token's own and every later query of its sequence, queries take their own.
    B, S, H, dh = 2, 7, 3, 4
    q, k, v, e = _inputs(B, S, H, dh, 11)
    K, sigma, t0, d0 = 2, 3e-2, 0, 4
    toks = _token_subset(B, S, np.random.default_rng(1), 2)
    a = oracle.noise_block(SEED, 7, d0, K, t0, B * S, H * dh)
    o = _torch_attn(q, k, v, B, S, H).numpy()
    for proj in ("q", "k", "v"):
        _, rs = oracle.attn_estimate_tokens(proj, q, k, v, e, S, H, K, sigma, SEED, 7, toks,
                                            token_offset=t0, draw_offset=d0)
        for i in range(K):
            pert = [q, k, v]
            pert["qkv".index(proj)] = pert["qkv".index(proj)] + sigma * a[i]
            c = np.sum(e * (_torch_attn(*pert, B, S, H).numpy() - o), axis=1)
            for j, t in enumerate(toks):
                end = (t // S + 1) * S
                ref = -c[t] if proj == "q" else -c[t:end].sum()
                assert abs(rs[i, j] - ref) <= 1e-9 * max(1.0, abs(ref)), (proj, i, t, rs[i, j], ref)
