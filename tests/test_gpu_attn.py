"""GPU parity of the attention projection estimators (values, keys, queries) against their oracle.

Small cases element by element (one and several query tiles per sequence, several
sequences and heads, more draws than one pass of the partial buffer holds, the longest
sequence accepted (4096) and sixteen heads), and the
full-size 2 x 2048-token, 8-head workload on tokens sampled near the ends of the
sequences (their rewards need the outputs of few later queries), the weight gradient
against the fp64 identity G = g_hat^T U, and determinism.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import zeroth_order_activation_amd as dust
from gpu_cases import dev, gpu_matmul, rel_l2

pytestmark = pytest.mark.gpu

TOL = 1e-4  # relative L2 on rewards and g_hat (bf16x3 products, fp32 accumulation)


def _run(c, K, sigma, seed, layer, tok0=0, draw0=0):
    T, d = c["T"], c["d"]
    ghat = torch.empty((T, d), dtype=torch.float32, device="cuda")
    rew = torch.empty((K, T), dtype=torch.float32, device="cuda")
    gw = dust.estimate_attn_v(dev(c["q"]), dev(c["k"]), dev(c["e"]), dev(c["u"]), c["S"], c["H"], K, sigma, seed,
                              layer, tok0, draw0, ghat=ghat, rewards=rew)
    torch.cuda.synchronize()
    return gw, ghat, rew


CASES = [
    # B, S, H, K, sigma
    (2, 64, 2, 5, 1e-2),    # one tile per sequence
    (1, 192, 1, 9, 3e-2),   # three query tiles: causal tiles below the diagonal
    (3, 128, 4, 3, 1e-2),   # several sequences and heads
    (1, 64, 1, 70, 1e-2),   # more draws than one pass of partials (64)
    (1, 4096, 1, 2, 1e-2),  # the longest sequence accepted: 64 query tiles
    (1, 64, 16, 3, 1e-2),   # sixteen heads
]


@pytest.mark.parametrize("B,S,H,K,sigma", CASES)
def test_attn_v_small_cases_elementwise(B, S, H, K, sigma):
    c = synth.attn_case(B, S, H, seed=41 + S + H)
    seed, layer, tok0, draw0 = 0x4455535400000040 + S, 2, 3, 5
    gw, ghat, rew = _run(c, K, sigma, seed, layer, tok0, draw0)
    og, orew = oracle.attn_v_estimate(c["q"], c["k"], c["v"], c["e"], S, H, K, sigma, seed, layer, tok0, draw0)
    e_g, e_r = rel_l2(ghat.cpu().numpy(), og), rel_l2(rew.cpu().numpy(), orew)
    e_w = rel_l2(gw.cpu().numpy(), oracle.grad_w(og, c["u"]))
    print(f"B={B} S={S} H={H} K={K} sigma={sigma}: rewards {e_r:.2e} ghat {e_g:.2e} grad_w {e_w:.2e}")
    assert e_r < TOL and e_g < TOL and e_w < 1e-3


def test_attn_v_full_workload_on_sampled_tokens():
    c = synth.workload(6, matmul=gpu_matmul)
    K, sigma, S = c["K"], c["sigma"], c["S"]
    gw, ghat, rew = _run(c, K, sigma, c["seed_noise"], c["layer"])
    gw2 = dust.estimate_attn_v(dev(c["q"]), dev(c["k"]), dev(c["e"]), dev(c["u"]), S, c["H"], K, sigma,
                               c["seed_noise"], c["layer"])
    torch.cuda.synchronize()
    assert torch.equal(gw, gw2)  # deterministic, with or without the g_hat and reward outputs
    toks = [S - 5, S - 2, 2 * S - 3, 2 * S - 1]
    og, orew = oracle.attn_v_estimate_tokens(c["q"], c["k"], c["v"], c["e"], S, c["H"], K, sigma, c["seed_noise"],
                                             c["layer"], toks)
    e_g = rel_l2(ghat[toks].cpu().numpy(), og)
    e_r = rel_l2(rew[:, toks].cpu().numpy(), orew)
    rows = np.random.default_rng(26).choice(c["d"], 64, replace=False)
    ref = ghat[:, rows].cpu().numpy().astype(np.float64).T @ c["u"].astype(np.float64)
    e_w = rel_l2(gw[rows].cpu().numpy(), ref)
    print(f"2x2048 tokens, 8 heads, K={K}: sampled rewards {e_r:.2e} ghat {e_g:.2e}; grad_w rows vs G^T U {e_w:.2e}")
    assert e_r < TOL and e_g < TOL and e_w < 6e-5


QK_CASES = [
    # proj, B, S, H, K, sigma
    ("k", 2, 64, 2, 5, 1e-2),
    ("k", 1, 192, 1, 9, 3e-2),   # causal tiles below the diagonal; larger logit changes
    ("k", 3, 128, 4, 3, 1e-2),
    ("q", 2, 64, 2, 5, 1e-2),
    ("q", 1, 192, 1, 9, 3e-2),
    ("q", 3, 128, 4, 70, 1e-2),  # more draws than one pass of partials
    ("k", 1, 64, 1, 70, 0.2),    # |delta| past the polynomial's range: exp - 1
    ("q", 2, 128, 2, 9, 0.2),    # the same for queries, over two key tiles
    ("k", 1, 4096, 1, 2, 1e-2),  # the longest sequence accepted
    ("q", 1, 4096, 1, 2, 1e-2),
    ("k", 1, 64, 16, 3, 1e-2),   # sixteen heads
    ("q", 1, 64, 16, 3, 1e-2),
]


@pytest.mark.parametrize("proj,B,S,H,K,sigma", QK_CASES)
def test_attn_query_key_small_cases_elementwise(proj, B, S, H, K, sigma):
    c = synth.attn_case(B, S, H, seed=43 + S + H)
    seed, layer, tok0, draw0 = 0x4455535400000050 + S, 3, 7, 2
    T, d = c["T"], c["d"]
    ghat = torch.empty((T, d), dtype=torch.float32, device="cuda")
    rew = torch.empty((K, T), dtype=torch.float32, device="cuda")
    gw = dust.estimate_attn(proj, dev(c["q"]), dev(c["k"]), dev(c["v"]), dev(c["e"]), dev(c["u"]), S, H, K, sigma,
                            seed, layer, tok0, draw0, ghat=ghat, rewards=rew)
    torch.cuda.synchronize()
    og, orew = oracle.attn_estimate(proj, c["q"], c["k"], c["v"], c["e"], S, H, K, sigma, seed, layer, tok0, draw0)
    e_g, e_r = rel_l2(ghat.cpu().numpy(), og), rel_l2(rew.cpu().numpy(), orew)
    e_w = rel_l2(gw.cpu().numpy(), oracle.grad_w(og, c["u"]))
    print(f"{proj}: B={B} S={S} H={H} K={K} sigma={sigma}: rewards {e_r:.2e} ghat {e_g:.2e} grad_w {e_w:.2e}")
    assert e_r < TOL and e_g < TOL and e_w < 1e-3


@pytest.mark.parametrize("proj", ["q", "k"])
def test_attn_query_key_full_workload_on_sampled_tokens(proj):
    c = synth.workload(6, matmul=gpu_matmul)
    K, sigma, S, H = c["K"], c["sigma"], c["S"], c["H"]
    T, d = c["T"], c["d"]
    ghat = torch.empty((T, d), dtype=torch.float32, device="cuda")
    rew = torch.empty((K, T), dtype=torch.float32, device="cuda")
    args = (dev(c["q"]), dev(c["k"]), dev(c["v"]), dev(c["e"]), dev(c["u"]), S, H, K, sigma, c["seed_noise"], 5)
    gw = dust.estimate_attn(proj, *args, ghat=ghat, rewards=rew)
    gw2 = dust.estimate_attn(proj, *args)
    torch.cuda.synchronize()
    assert torch.equal(gw, gw2)
    toks = [3, 1000, S - 2, 2 * S - 1] if proj == "q" else [S - 4, 2 * S - 2]
    og, orew = oracle.attn_estimate_tokens(proj, c["q"], c["k"], c["v"], c["e"], S, H, K, sigma, c["seed_noise"], 5,
                                           toks)
    e_g = rel_l2(ghat[toks].cpu().numpy(), og)
    e_r = rel_l2(rew[:, toks].cpu().numpy(), orew)
    rows = np.random.default_rng(27).choice(d, 64, replace=False)
    ref = ghat[:, rows].cpu().numpy().astype(np.float64).T @ c["u"].astype(np.float64)
    e_w = rel_l2(gw[rows].cpu().numpy(), ref)
    print(f"{proj}, 2x2048 tokens, 8 heads, K={K}: sampled rewards {e_r:.2e} ghat {e_g:.2e}; grad_w rows {e_w:.2e}")
    assert e_r < TOL and e_g < TOL and e_w < 6e-5
