"""GPU parity of the vocabulary-subset LM-head estimator against its oracle.

Small cases element by element (fp32 and bf16 logits, ragged V, a one-quad window,
windows spanning several quads per lane, the degree-6 polynomial, the widest row of
the one-pass kernel, more draws than one chunk), rows wider than LDS (the rewards +
accumulation passes, also over two chunks of draws), a
window covering the vocabulary (bitwise the full estimator), the full-size
4096 x 8192 shape with m = 1024 and the 243M-shape head with m = 4096 on sampled
tokens, and determinism.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import zeroth_order_activation_amd as dust
from gpu_cases import dev, gpu_matmul, logits_to_device, logits_values, rel_l2

pytestmark = pytest.mark.gpu

TOL = 1e-4  # relative L2 on g_hat rows and rewards (fp32 path)


def _run(case, K, m, sigma, seed, layer, tok0=0, draw0=0):
    T, V = case["T"], case["V"]
    ghat = torch.empty((T, V), dtype=torch.float32, device="cuda")
    rew = torch.empty((K, T), dtype=torch.float32, device="cuda")
    gw = dust.estimate_head_subset(logits_to_device(case), dev(case["x"]), dev(case["labels"]), K, m, sigma, seed,
                                   layer, tok0, draw0, ghat=ghat, rewards=rew)
    torch.cuda.synchronize()
    return gw, ghat, rew


SMALL = [
    # T, V, d, K, m, sigma, dtype
    (9, 1000, 16, 7, 64, 1e-2, "f32"),      # 16 of 250 quads, one per lane
    (7, 1003, 8, 5, 4, 1e-2, "bf16"),       # one-quad window, ragged V
    (13, 4097, 8, 5, 2048, 4e-2, "f32"),    # degree-6 polynomial, 2 quads per lane
    (5, 16384, 8, 3, 8192, 1e-2, "f32"),    # largest V, 8 quads per lane
    (6, 9000, 8, 4, 16000, 1e-2, "bf16"),   # 4000 >= 2250 quads: the window covers, full estimator path
    (8, 300, 8, 9, 120, 0.1, "f32"),        # library expm1 (large sigma)
    (2, 4097, 8, 600, 256, 1e-2, "bf16"),   # more draws than one chunk of per-draw terms (512)
    # rows wider than the one-pass kernel's LDS: rewards pass + accumulation pass
    (5, 20000, 8, 7, 2048, 1e-2, "f32"),
    (4, 50304, 8, 5, 4096, 5e-3, "bf16"),   # the 243M-shape vocabulary
    (3, 40001, 8, 3, 4, 1e-2, "bf16"),      # ragged, one-quad window
    (6, 30000, 8, 9, 1000, 0.1, "f32"),     # library expm1, window not a multiple of 64 quads
    (5, 65536, 8, 4, 60000, 5e-3, "bf16"),  # widest bf16 row, window almost everything
    (2, 20000, 8, 600, 1024, 1e-2, "bf16"), # two chunks of draws in both passes
]


@pytest.mark.parametrize("T,V,d,K,m,sigma,dt", SMALL)
def test_subset_small_cases_elementwise(T, V, d, K, m, sigma, dt):
    case = synth.head_case(T, V, d, seed=31 + V, labels="zipf", logits_dtype=dt)
    seed, layer, tok0, draw0 = 0x4455535400000020 + V, 1, 4, 2
    gw, ghat, rew = _run(case, K, m, sigma, seed, layer, tok0, draw0)
    og, orew, _ = oracle.head_estimate_subset(logits_values(case), case["labels"], K, m, sigma, seed, layer,
                                              tok0, draw0)
    e_g, e_r = rel_l2(ghat.cpu().numpy(), og), rel_l2(rew.cpu().numpy(), orew)
    e_w = rel_l2(gw.cpu().numpy(), oracle.grad_w(og, case["x"]))
    print(f"T={T} V={V} K={K} m={m} sigma={sigma} {dt}: ghat {e_g:.2e} rewards {e_r:.2e} grad_w {e_w:.2e}")
    assert e_r < TOL and e_g < TOL and e_w < 1e-3


def test_covering_window_is_the_full_estimator():
    case = synth.head_case(11, 2000, 8, seed=3, labels="zipf")
    z, x, y = logits_to_device(case), dev(case["x"]), dev(case["labels"])
    g_full = torch.empty((11, 2000), dtype=torch.float32, device="cuda")
    g_sub = torch.empty_like(g_full)
    w_full = dust.estimate_head(z, x, y, 6, 1e-2, 5, 1, ghat=g_full)
    w_sub = dust.estimate_head_subset(z, x, y, 6, 2000, 1e-2, 5, 1, ghat=g_sub)
    torch.cuda.synchronize()
    assert torch.equal(g_full, g_sub) and torch.equal(w_full, w_sub)


def test_workload2_shape_with_a_1024_channel_window():
    c = synth.workload(2, matmul=gpu_matmul)
    T, V, K, sigma, m = c["T"], c["V"], c["K"], c["sigma"], 1024
    ghat = torch.empty((T, V), dtype=torch.float32, device="cuda")
    rew = torch.empty((K, T), dtype=torch.float32, device="cuda")
    gw = dust.estimate_head_subset(logits_to_device(c), dev(c["x"]), dev(c["labels"]), K, m, sigma,
                                   c["seed_noise"], c["layer"], ghat=ghat, rewards=rew)
    gw2 = dust.estimate_head_subset(logits_to_device(c), dev(c["x"]), dev(c["labels"]), K, m, sigma,
                                    c["seed_noise"], c["layer"])
    torch.cuda.synchronize()
    assert torch.equal(gw, gw2)  # deterministic, with or without the g_hat output
    toks = np.random.default_rng(22).choice(T, 8, replace=False)
    zv = logits_values({k: (v[toks] if k == "logits" else v) for k, v in c.items()})
    rows_g, rows_r = [], []
    for j, t in enumerate(toks):
        g1, r1, _ = oracle.head_estimate_subset(zv[j][None], c["labels"][[t]], K, m, sigma, c["seed_noise"],
                                                c["layer"], token_offset=int(t))
        rows_g.append(g1[0])
        rows_r.append(r1[:, 0])
    e_g = rel_l2(ghat[toks].cpu().numpy(), np.stack(rows_g))
    e_r = rel_l2(rew[:, toks].cpu().numpy(), np.stack(rows_r, axis=1))
    rows = np.random.default_rng(23).choice(V, 64, replace=False)
    ref = ghat[:, rows].cpu().numpy().astype(np.float64).T @ c["x"].astype(np.float64)
    e_w = rel_l2(gw[rows].cpu().numpy(), ref)
    print(f"workload-2 shape, m={m}: sampled ghat {e_g:.2e} rewards {e_r:.2e}; grad_w rows vs G^T X {e_w:.2e}")
    assert e_g < TOL and e_r < TOL and e_w < 6e-5


def test_243m_shape_with_a_4096_channel_window():
    c = synth.workload(4, matmul=gpu_matmul)
    T, V, K, sigma, m = c["T"], c["V"], c["K"], c["sigma"], 4096
    ghat = torch.empty((T, V), dtype=torch.float32, device="cuda")
    rew = torch.empty((K, T), dtype=torch.float32, device="cuda")
    z, x, y = logits_to_device(c), dev(c["x"]), dev(c["labels"])
    gw = dust.estimate_head_subset(z, x, y, K, m, sigma, c["seed_noise"], c["layer"], ghat=ghat, rewards=rew)
    gw2 = dust.estimate_head_subset(z, x, y, K, m, sigma, c["seed_noise"], c["layer"])
    torch.cuda.synchronize()
    assert torch.equal(gw, gw2)  # deterministic, with or without the g_hat and reward outputs
    toks = np.random.default_rng(24).choice(T, 6, replace=False)
    zv = logits_values({k: (v[toks] if k == "logits_bf16" else v) for k, v in c.items()})
    rows_g, rows_r = [], []
    for j, t in enumerate(toks):
        g1, r1, _ = oracle.head_estimate_subset(zv[j][None], c["labels"][[t]], K, m, sigma, c["seed_noise"],
                                                c["layer"], token_offset=int(t))
        rows_g.append(g1[0])
        rows_r.append(r1[:, 0])
    e_g = rel_l2(ghat[toks].cpu().numpy(), np.stack(rows_g))
    e_r = rel_l2(rew[:, toks].cpu().numpy(), np.stack(rows_r, axis=1))
    rows = np.random.default_rng(25).choice(V, 64, replace=False)
    ref = ghat[:, rows].cpu().numpy().astype(np.float64).T @ c["x"].astype(np.float64)
    e_w = rel_l2(gw[rows].cpu().numpy(), ref)
    print(f"243M shape, m={m}: sampled ghat {e_g:.2e} rewards {e_r:.2e}; grad_w rows vs G^T X {e_w:.2e}")
    assert e_g < TOL and e_r < TOL and e_w < 6e-5
