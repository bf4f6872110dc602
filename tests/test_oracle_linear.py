"""Pins of the oracle's interior MLP-linear estimator.

- the unrounded downstream loss equals a torch forward (gelu, layer_norm, cross_entropy) in fp64;
- the hand-written chain-rule gradient equals torch.autograd in fp64;
- the bf16 rounding equals torch's fp32 -> bf16 conversion;
- same-noise linearisation of the unrounded estimator against the analytic gradient
  (sign, scale, every link of the chain);
- with bf16 operands the estimate still follows the alignment law (cosine to backprop);
- draw additivity through draw_offset, token sampling equals the full run.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle
import synth

SEED = 0x4455535400000003
EPS = 1e-5


def _case(T=8, d=16, n=64, V=40, seed=1):
    return synth.linear_case(T, d, n, V, seed=seed)


def _w(c):
    return (oracle.bf16_bits_value(c["w2_bf16"]), oracle.bf16_bits_value(c["w_head_bf16"]))


def test_downstream_loss_matches_torch_forward():
    c = _case()
    w2, wh = _w(c)
    h = c["h"].astype(np.float64)
    ce = oracle.mlp_downstream_ce(h, c["x_res"].astype(np.float64), c["labels"], w2, wh, EPS,
                                  quantize=False)
    th = torch.from_numpy(h)
    m = F.gelu(th)  # exact erf form
    yv = torch.from_numpy(c["x_res"].astype(np.float64)) + m @ torch.from_numpy(w2).T
    f = F.layer_norm(yv, (yv.shape[1],), eps=EPS)
    z = f @ torch.from_numpy(wh).T
    ref = F.cross_entropy(z, torch.from_numpy(c["labels"]).long(), reduction="none").numpy()
    np.testing.assert_allclose(ce, ref, rtol=1e-12, atol=1e-12)


def test_chain_rule_gradient_matches_autograd():
    c = _case(T=6, d=12, n=48, V=30, seed=2)
    w2, wh = _w(c)
    g = oracle.mlp_analytic(c["h"], c["x_res"], c["w2_bf16"], c["w_head_bf16"], c["labels"], EPS)
    th = torch.from_numpy(c["h"].astype(np.float64)).requires_grad_(True)
    yv = torch.from_numpy(c["x_res"].astype(np.float64)) + F.gelu(th) @ torch.from_numpy(w2).T
    z = F.layer_norm(yv, (yv.shape[1],), eps=EPS) @ torch.from_numpy(wh).T
    F.cross_entropy(z, torch.from_numpy(c["labels"]).long(), reduction="sum").backward()
    np.testing.assert_allclose(g, th.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(3).standard_normal(100000).astype(np.float32) * 10
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0]  # exact ties between bf16 neighbours
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.bf16_round(x), ref)


def test_linearisation_of_unrounded_estimator():
    c = _case(T=4, d=16, n=64, V=32, seed=4)
    K, sigma = 1024, 1e-4
    gh, _, _ = oracle.linear_estimate(c["h"], c["x_res"], c["w2_bf16"], c["w_head_bf16"],
                                      c["labels"], K, sigma, EPS, SEED, 0, quantize=False)
    g = oracle.mlp_analytic(c["h"], c["x_res"], c["w2_bf16"], c["w_head_bf16"], c["labels"], EPS)
    a = oracle.noise_block(SEED, 0, 0, K, 0, 4, 64)
    lin = np.einsum("ktn,kt->tn", a, np.einsum("ktn,tn->kt", a, g)) / K
    assert np.linalg.norm(gh - lin) / np.linalg.norm(lin) < 2e-3


def test_bf16_downstream_follows_alignment_law():
    c = _case(T=16, d=16, n=64, V=48, seed=5)
    g = oracle.mlp_analytic(c["h"], c["x_res"], c["w2_bf16"], c["w_head_bf16"], c["labels"], EPS)
    U = c["u"]
    G = g.T @ U.astype(np.float64)
    cc = oracle.cosine_law_c(g, U)
    K = 256
    cs = []
    for s in range(3):
        gh, _, _ = oracle.linear_estimate(c["h"], c["x_res"], c["w2_bf16"], c["w_head_bf16"],
                                          c["labels"], K, 1e-2, EPS, SEED + s, 0)
        cs.append(oracle.cosine(oracle.grad_w(gh, U), G))
    pred = 1.0 / math.sqrt(1.0 + cc / K)
    assert abs(np.mean(cs) - pred) < 0.08, (np.mean(cs), pred)


def test_additivity_and_token_sampling():
    c = _case(T=6, d=8, n=32, V=24, seed=6)
    args = (c["h"], c["x_res"], c["w2_bf16"], c["w_head_bf16"], c["labels"])
    K, K1 = 9, 4
    g, r, ce0 = oracle.linear_estimate(*args, K, 1e-2, EPS, SEED, 0)
    g1, r1, _ = oracle.linear_estimate(*args, K1, 1e-2, EPS, SEED, 0)
    g2, r2, _ = oracle.linear_estimate(*args, K - K1, 1e-2, EPS, SEED, 0, draw_offset=K1)
    np.testing.assert_allclose(K * g, K1 * g1 + (K - K1) * g2, rtol=1e-12, atol=1e-12)
    gs, rs, _ = oracle.linear_estimate(*args, K, 1e-2, EPS, SEED, 0, tokens=[5, 1])
    np.testing.assert_allclose(gs, g[[5, 1]], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(rs, r[:, [5, 1]], rtol=1e-13, atol=1e-15)


def _torch_quantized_ce(htilde64, x, labels, w2, wh, eps):
    """The bf16 downstream written with torch: GELU in fp64, its output cast to fp32 and
    then to bf16; W2 product and residual in fp64; LayerNorm in fp64, its output cast
    to fp32 and then to bf16; head product and cross-entropy in fp64."""
    bf = torch.bfloat16
    m = F.gelu(torch.from_numpy(htilde64)).to(torch.float32).to(bf).to(torch.float64)
    yv = torch.from_numpy(x.astype(np.float64)) + m @ torch.from_numpy(w2).T
    f = F.layer_norm(yv, (yv.shape[1],), eps=eps).to(torch.float32).to(bf).to(torch.float64)
    z = f @ torch.from_numpy(wh).T
    return F.cross_entropy(z, torch.from_numpy(labels).long(), reduction="none").numpy()


def test_bf16_rounding_points_match_explicit_torch_casts():
    # The rounding points of the quantised downstream: the GELU output and the
    # LayerNorm output, each taken to fp32 and then to bf16 (round to nearest even).
    # Rounding h~ instead of GELU(h~), or rounding before the LayerNorm, moves the
    # losses by about a bf16 step (1e-3 relative), far above this test's 1e-12.
    c = _case(T=24, d=32, n=128, V=64, seed=7)
    w2, wh = _w(c)
    rng = np.random.default_rng(8)
    h = c["h"].astype(np.float64) + 0.3 * rng.standard_normal(c["h"].shape)
    ce = oracle.mlp_downstream_ce(h, c["x_res"].astype(np.float64), c["labels"], w2, wh, EPS, quantize=True)
    ref = _torch_quantized_ce(h, c["x_res"], c["labels"], w2, wh, EPS)
    np.testing.assert_allclose(ce, ref, rtol=1e-12, atol=1e-12)
    # and the rounding matters at this size: the unrounded loss differs
    ce_exact = oracle.mlp_downstream_ce(h, c["x_res"].astype(np.float64), c["labels"], w2, wh, EPS, quantize=False)
    assert np.abs(ce_exact - ref).max() > 1e-6


def test_quantised_rewards_are_torch_loss_differences():
    # Every reward of the quantised estimator: the clean row through the bf16 downstream
    # minus the perturbed row, h~ = h + sigma a rounded to fp32 first (an fp32 tensor,
    # like the cached h), both written with torch's casts.
    c = _case(T=5, d=16, n=64, V=40, seed=9)
    w2, wh = _w(c)
    K, sigma, t0, d0 = 4, 2e-2, 3, 6
    g, rew, ce0 = oracle.linear_estimate(c["h"], c["x_res"], c["w2_bf16"], c["w_head_bf16"], c["labels"], K, sigma,
                                         EPS, SEED, 0, token_offset=t0, draw_offset=d0)
    a = oracle.noise_block(SEED, 0, d0, K, t0, 5, 64)
    h = c["h"].astype(np.float64)
    clean = _torch_quantized_ce(h, c["x_res"], c["labels"], w2, wh, EPS)
    np.testing.assert_allclose(ce0, clean, rtol=1e-12, atol=1e-12)
    for i in range(K):
        ht = (h + sigma * a[i]).astype(np.float32).astype(np.float64)
        r = clean - _torch_quantized_ce(ht, c["x_res"], c["labels"], w2, wh, EPS)
        np.testing.assert_allclose(rew[i], r, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(g, -np.einsum("kt,ktn->tn", rew, a) / (K * sigma), rtol=1e-12, atol=1e-14)
