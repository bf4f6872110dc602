"""GPU parity of the interior MLP-linear estimator against the oracle.

The downstream runs with bf16 GEMM operands on both sides (GELU output and
LayerNorm output rounded fp32 -> bf16).  The two sides agree up to fp32
accumulation order, and that order flips the bf16 rounding of a value lying
within an ulp of a tie on rare rows; see gpu_cases.check_quantized_rewards for
the resulting criterion (bulk within fp32 resolution, bounded outliers, and a
5e-3 relative L2 over >= 1000 rewards, the G_W tolerance).  The rest of the
chain is checked exactly: g_hat against the oracle's noise weighted by the
kernel's own rewards, and G_W against the fp64 identity G_W = G_hat^T U.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import zeroth_order_activation_amd as dust
from gpu_cases import check_quantized_rewards, dev, rel_l2

pytestmark = pytest.mark.gpu

TOL_GW = 5e-3   # relative L2 on G_W with a bf16 downstream


def _check_reduction(c, ghat_rows, rew_cols, toks, K, sigma, seed, layer, tok0=0, draw0=0):
    """g_hat_t = -(1/(K sigma)) sum_i r_i a_i with the kernel's rewards and the oracle's noise."""
    n = c["n"]
    for j, t in enumerate(toks):
        a = np.stack([oracle.noise(seed, layer, draw0 + i, tok0 + int(t), n) for i in range(K)])
        ref = -(rew_cols[:, j].astype(np.float64) @ a) / (K * sigma)
        assert rel_l2(ghat_rows[j], ref) < 2e-5


def _dev_case(c):
    w2 = dev(c["w2_bf16"].view(np.int16)).view(torch.bfloat16)
    wh = dev(c["w_head_bf16"].view(np.int16)).view(torch.bfloat16)
    return dev(c["u"]), dev(c["h"]), dev(c["x_res"]), w2, wh, dev(c["labels"])


def _run(c, K, sigma, seed, layer, tok0=0, draw0=0):
    u, h, x, w2, wh, y = _dev_case(c)
    T, n = c["T"], c["n"]
    ghat = torch.empty((T, n), dtype=torch.float32, device="cuda")
    rew = torch.empty((K, T), dtype=torch.float32, device="cuda")
    gw = dust.estimate_linear(u, h, x, w2, wh, y, K, sigma, seed, layer, tok0, draw0, ln_eps=c["ln_eps"],
                              ghat=ghat, rewards=rew)
    torch.cuda.synchronize()
    return gw, ghat, rew


def _oracle(c, K, sigma, seed, layer, tok0=0, draw0=0, tokens=None):
    return oracle.linear_estimate(c["h"], c["x_res"], c["w2_bf16"], c["w_head_bf16"], c["labels"], K, sigma,
                                  c["ln_eps"], seed, layer, tok0, draw0, tokens=tokens)


# K chosen so that every case has at least 1000 rewards: the relative L2 bars on
# rewards, g_hat and G_W then apply to every case.
SMALL = [
    # T, d, n, V, K, sigma
    (8, 256, 64, 40, 125, 1e-2),
    (37, 512, 128, 1000, 28, 1e-2),    # ragged vocabulary tile, ragged row tiles
    (70, 256, 96, 300, 15, 2e-2),
    (130, 512, 256, 2048, 8, 1e-2),
    (8, 256, 32, 777, 125, 1e-2),      # the narrowest layer accepted (n = 32), ragged vocabulary
    (4, 512, 64, 50304, 250, 1e-2),    # a 50304-entry vocabulary (197 tiles of 256)
]


@pytest.mark.parametrize("T,d,n,V,K,sigma", SMALL)
def test_linear_small_cases(T, d, n, V, K, sigma):
    c = synth.linear_case(T, d, n, V, seed=100 + T)
    seed, layer, tok0, draw0 = 0x4455535400000003 + T, 0, 11, 2
    gw, ghat, rew = _run(c, K, sigma, seed, layer, tok0, draw0)
    og, orew, oce0 = _oracle(c, K, sigma, seed, layer, tok0, draw0)
    st = check_quantized_rewards(rew.cpu().numpy(), orew, oce0)
    gh = ghat.cpu().numpy()
    _check_reduction(c, gh, rew.cpu().numpy(), range(T), K, sigma, seed, layer, tok0, draw0)
    u64 = c["u"].astype(np.float64)
    e_w = rel_l2(gw.cpu().numpy(), gh.astype(np.float64).T @ u64)
    e_go = rel_l2(gh, og)
    e_wo = rel_l2(gw.cpu().numpy(), oracle.grad_w(og, u64))
    print(f"T={T} d={d} n={n} V={V} K={K}: rewards {st}; g_hat vs oracle {e_go:.2e}; "
          f"grad_w vs oracle {e_wo:.2e}; grad_w vs G^T U {e_w:.2e}")
    assert e_w < 1e-5
    assert e_go < TOL_GW and e_wo < TOL_GW


def test_workload3_whole():
    """The MLP-linear workload at full size in the benchmark's configuration: every
    reward, every g_hat row and the whole G_W against the oracle run on all tokens."""
    c = synth.workload(3)
    K, sigma = c["K"], c["sigma"]
    print("workload 3: GPU estimate", flush=True)
    gw, ghat, rew = _run(c, K, sigma, c["seed_noise"], c["layer"])
    print("workload 3: oracle on every token", flush=True)
    og, orew, oce0 = _oracle(c, K, sigma, c["seed_noise"], c["layer"])
    st = check_quantized_rewards(rew.cpu().numpy(), orew, oce0)
    e_go = rel_l2(ghat.cpu().numpy(), og)
    e_wo = rel_l2(gw.cpu().numpy(), oracle.grad_w(og, c["u"]))
    print(f"workload 3 K={K}: rewards {st}; g_hat vs oracle {e_go:.2e}; grad_w vs oracle {e_wo:.2e}")
    assert e_go < TOL_GW and e_wo < TOL_GW


@pytest.mark.parametrize("wid,K,ntok", [(5, 256, 16), (5, 1024, 8), (5, 4096, 3), (5, 16384, 2)])
def test_named_workload_full_size(wid, K, ntok):
    """Full-size workload in the benchmark's configuration; sampled tokens against the
    oracle (every draw of each), all grad_w rows against the identity G_W = G^T U, and
    sampled rows of the oracle's G_W restricted to the sampled tokens."""
    c = synth.workload(wid)
    T, n, sigma = c["T"], c["n"], c["sigma"]
    print(f"workload {wid} K={K}: GPU estimate", flush=True)
    gw, ghat, rew = _run(c, K, sigma, c["seed_noise"], c["layer"])
    toks = np.random.default_rng(wid + K).choice(T, ntok, replace=False)
    og, orew, oce0 = _oracle(c, K, sigma, c["seed_noise"], c["layer"], tokens=toks)
    rw = rew[:, toks].cpu().numpy()
    st = check_quantized_rewards(rw, orew, oce0)
    gh_s = ghat[toks].cpu().numpy()
    _check_reduction(c, gh_s, rw, toks, K, sigma, c["seed_noise"], c["layer"])
    e_go = rel_l2(gh_s, og)
    u64 = c["u"].astype(np.float64)
    # the sampled tokens' share of G_W: their g_hat rows against the oracle's
    e_wo = rel_l2(gh_s.astype(np.float64).T @ u64[toks], og.T @ u64[toks])
    gw_h = gw.cpu().numpy()
    ref = ghat.cpu().numpy().astype(np.float64).T @ u64
    e_w = rel_l2(gw_h, ref)
    print(f"workload {wid} K={K}: sampled rewards {st}; g_hat vs oracle {e_go:.2e}; "
          f"sampled tokens' G_W vs oracle {e_wo:.2e}; grad_w vs G^T U {e_w:.2e}")
    assert e_w < 6e-5  # bf16-pair outer product
    assert e_go < TOL_GW and e_wo < TOL_GW


def test_linear_deterministic_additive_and_chunked():
    # T*(K+1)*d*2 bytes above 512 MiB forces several passes over the row chunks
    c = synth.linear_case(2048, 512, 64, 256, seed=9)
    K, K1, sigma, seed = 300, 120, 1e-2, 5
    gw, ghat, rew = _run(c, K, sigma, seed, 0)
    gw2, _, rew2 = _run(c, K, sigma, seed, 0)
    assert torch.equal(gw, gw2) and torch.equal(rew, rew2)
    g1, _, r1 = _run(c, K1, sigma, seed, 0)
    g2, _, r2 = _run(c, K - K1, sigma, seed, 0, draw0=K1)
    comb = (K1 * g1.double() + (K - K1) * g2.double()) / K
    assert rel_l2(comb.cpu().numpy(), gw.cpu().numpy()) < 1e-5
    assert torch.equal(torch.cat([r1, r2]), rew)
    toks = [0, 1500, 2047, 3, 777]
    og, orew, oce0 = _oracle(c, K, sigma, seed, 0, tokens=toks)
    check_quantized_rewards(rew[:, toks].cpu().numpy(), orew, oce0)
    _check_reduction(c, ghat[toks].cpu().numpy(), rew[:, toks].cpu().numpy(), toks, K, sigma, seed, 0)
