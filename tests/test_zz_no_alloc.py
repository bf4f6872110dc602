"""The no-allocation LM-head entry point (dust_estimate_head_noalloc) against
dust_estimate_head through the C ABI: the same kernels on the library's static
scratch instead of a caller workspace.  Two calls in a row, the second on a smaller
input, each equal bit for bit to the workspace entry point's result (and within the
head's 1e-3 relative L2 of the oracle); a shape too large for the scratch is
rejected on the host."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
import zeroth_order_activation_amd as dust
from gpu_cases import dev, logits_to_device, logits_values, rel_l2

pytestmark = pytest.mark.gpu


def _both(case, K, sigma, seed, layer, want_ghat):
    T, V, d = case["T"], case["V"], case["d"]
    z, x, y = logits_to_device(case), dev(case["x"]), dev(case["labels"])
    outs = []
    for fn in ("workspace", "noalloc"):
        gw = torch.full((V, d), float("nan"), dtype=torch.float32, device="cuda")
        gh = torch.full((T, V), float("nan"), dtype=torch.float32, device="cuda") if want_ghat else None
        rw = torch.full((K, T), float("nan"), dtype=torch.float32, device="cuda")
        if fn == "workspace":
            dust.estimate_head(z, x, y, K, sigma, seed, layer, 3, 1, grad_w=gw, ghat=gh, rewards=rw)
        else:
            dust.estimate_head_noalloc(z, x, y, K, sigma, seed, layer, 3, 1, grad_w=gw, ghat=gh, rewards=rw)
        torch.cuda.synchronize()
        outs.append((gw, gh, rw))
    return outs


@pytest.mark.parametrize("want_ghat", [False, True])
def test_noalloc_head_equals_workspace_entry_point(want_ghat):
    # first a case on the bf16-pair outer product (its scratch holds the g_hat and x
    # pairs), then a smaller one on the fp32 outer product, whose scratch layout differs
    # and which must not read what the first call left behind
    cases = [(synth.head_case(700, 8192, 384, seed=21, labels="zipf"), 6, 1e-2),
             (synth.head_case(37, 1001, 13, seed=22, labels="zipf", logits_dtype="bf16"), 5, 2e-2)]
    for c, K, sigma in cases:
        seed, layer = 0x4455535400000099, 1
        print(f"noalloc: T={c['T']} V={c['V']} d={c['d']} K={K} ghat={want_ghat}", flush=True)
        (gw_a, gh_a, rw_a), (gw_b, gh_b, rw_b) = _both(c, K, sigma, seed, layer, want_ghat)
        assert torch.equal(gw_a, gw_b) and torch.equal(rw_a, rw_b)
        if want_ghat:
            assert torch.equal(gh_a, gh_b)
        og, orew, _ = oracle.head_estimate(logits_values(c), c["labels"], K, sigma, seed, layer, 3, 1)
        e_w = rel_l2(gw_b.cpu().numpy(), oracle.grad_w(og, c["x"]))
        e_r = rel_l2(rw_b.cpu().numpy(), orew)
        print(f"noalloc: grad_w {e_w:.2e}, rewards {e_r:.2e} against the oracle")
        assert e_w < 1e-3 and e_r < 1e-4


def test_noalloc_rejects_shapes_beyond_the_scratch():
    cap = dust.head_noalloc_max_bytes()
    assert cap == 64 << 20
    T, V, d = 4096, 8192, 512  # the fp32 g_hat rows alone are 128 MiB
    assert dust.lib().dust_head_workspace_bytes(T, V, d, 4) > cap
    L = dust.lib()
    big = torch.empty(16, dtype=torch.float32, device="cuda")
    p = ctypes.c_void_p(big.data_ptr())
    st = L.dust_estimate_head_noalloc(p, 1, p, p, 1 << 20, 65536, 1024, 4, ctypes.c_float(0.01), 1, 1, 0, 0, p,
                                      None, None, None)
    assert st == 2 and "static scratch" in L.dust_last_error().decode()
