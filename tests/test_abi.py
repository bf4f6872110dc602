"""The C-ABI library loads on a host without a GPU, exports every entry point the
header declares, and rejects bad arguments on the host before touching a device."""
import ctypes
import os
import re

import pytest

import zeroth_order_activation_amd as dust

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # an aligned address; every call below must fail before using it
FAKE_MIS = 0x10004


def _declared():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(dust_\w+)\s*\(", src))
    return names


def test_library_exports_every_declared_symbol():
    L = dust.lib()
    names = _declared()
    assert {"dust_estimate_head", "dust_noise", "dust_outer_product", "dust_last_error"} <= names
    for n in sorted(names):
        assert hasattr(L, n), n
    assert L.dust_abi_version() == 2


def _head(**kw):
    a = dict(logits=FAKE, dt=0, x=FAKE, labels=FAKE, T=4, V=8, d=2, K=3, sigma=0.01, seed=1, layer=0,
             tok=0, draw=0, gw=FAKE, ghat=FAKE, rew=None, ws=None, wsb=0)
    a.update(kw)
    L = dust.lib()
    st = L.dust_estimate_head(a["logits"], a["dt"], a["x"], a["labels"], a["T"], a["V"], a["d"], a["K"],
                              ctypes.c_float(a["sigma"]), a["seed"], a["layer"], a["tok"], a["draw"], a["gw"],
                              a["ghat"], a["rew"], a["ws"], a["wsb"], None)
    return st, L.dust_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(logits=None), 1, "non-NULL"),
    (dict(gw=None), 1, "non-NULL"),
    (dict(dt=7), 2, "logits_dtype"),
    (dict(x=FAKE_MIS), 1, "aligned"),
    (dict(T=0), 1, "T must be"),
    (dict(K=0), 1, "K must be"),
    (dict(V=0), 1, "V must be"),
    (dict(d=-1), 1, "d must be"),
    (dict(sigma=0.0), 1, "sigma"),
    (dict(sigma=-1.0), 1, "sigma"),
    (dict(sigma=float("nan")), 1, "sigma"),
    (dict(sigma=float("inf")), 1, "sigma"),
    (dict(tok=2**32 - 2), 1, "token counter"),
    (dict(tok=2**40), 1, "token counter"),    # a 64-bit id past the 32-bit counter word
    (dict(draw=2**32 - 1), 1, "draw counter"),
    (dict(V=70000), 2, "65536"),
    (dict(V=40000, dt=0), 2, "LDS"),
    (dict(ghat=None), 3, "workspace"),
    (dict(ghat=None, ws=FAKE, wsb=16), 3, "workspace"),
])
def test_head_rejects_bad_arguments_on_host(kw, status, msg):
    st, err = _head(**kw)
    assert st == status, err
    assert msg in err


def test_head_subset_rejects_bad_arguments_on_host():
    L = dust.lib()

    def call(m, V=1000, T=4, dtype=0):
        st = L.dust_estimate_head_subset(FAKE, dtype, FAKE, FAKE, T, V, 8, 3, m, ctypes.c_float(0.01), 1, 0, 0, 0,
                                         FAKE, FAKE, None, None, 0, None)
        return st, L.dust_last_error().decode()

    for m in (0, -4, 6):
        st, err = call(m)
        assert st == 1 and "multiple of 4" in err
    st, err = call(1024, V=70000, dtype=1)  # beyond the widest row
    assert st == 2 and "65536" in err
    st, err = call(1024, V=40000, dtype=0)  # fp32 row wider than LDS holds
    assert st == 2 and "fp32" in err
    for shape in ((4096, 8192, 512, 256), (7, 1003, 8, 5)):  # rows in LDS: the full estimator's layout
        assert L.dust_head_subset_workspace_bytes(*shape) == L.dust_head_workspace_bytes(*shape)
    T, K = 8192, 16  # wider rows add K*T rewards and K*T window offsets
    assert (L.dust_head_subset_workspace_bytes(T, 50304, 1024, K)
            == L.dust_head_workspace_bytes(T, 50304, 1024, K) + 2 * 4 * K * T)


def test_attn_v_rejects_bad_arguments_on_host():
    L = dust.lib()

    def call(T=128, S=64, d=128, H=2, K=3, sigma=0.01):
        st = L.dust_estimate_attn_v(FAKE, FAKE, FAKE, FAKE, T, S, d, H, K, ctypes.c_float(sigma), 1, 2, 0, 0,
                                    FAKE, None, None, FAKE, 1 << 30, None)
        return st, L.dust_last_error().decode()

    assert call(d=96, H=2)[0] == 2       # heads of 64 channels only
    st, err = call(d=64 * 17, H=17)      # at most 16 heads
    assert st == 2 and "16 heads" in err
    assert call(S=96, T=192)[0] == 2     # sequences of whole 64-token tiles
    assert call(S=8192, T=8192)[0] == 2  # longest sequence 4096
    assert call(T=100)[0] == 1           # T a multiple of S
    assert call(sigma=0.0)[0] == 1
    assert call(K=0)[0] == 1
    assert L.dust_attn_v_workspace_bytes(4096, 2048, 512, 8, 64) > 4096 * 512 * 4
    assert L.dust_attn_v_workspace_bytes(4096, 2048, 512, 8, 64) == L.dust_attn_workspace_bytes(2, 4096, 2048, 512,
                                                                                                8, 64)

    def gen(proj, v=FAKE):
        st = L.dust_estimate_attn(proj, FAKE, FAKE, v, FAKE, FAKE, 128, 64, 128, 2, 3, ctypes.c_float(0.01), 1, 2, 0,
                                  0, FAKE, None, None, FAKE, 1 << 30, None)
        return st, L.dust_last_error().decode()

    assert gen(3)[0] == 1 and gen(-1)[0] == 1       # no such projection
    assert gen(0, None)[0] == 1 and gen(1, None)[0] == 1  # queries and keys need v
    assert L.dust_attn_workspace_bytes(3, 128, 64, 128, 2, 3) == 0
    assert L.dust_attn_workspace_bytes(1, 4096, 2048, 512, 8, 64) > L.dust_attn_workspace_bytes(2, 4096, 2048, 512,
                                                                                                 8, 64)


def test_outer_and_noise_reject_bad_arguments():
    L = dust.lib()
    assert L.dust_outer_product(None, FAKE, 4, 4, 4, FAKE, None, 0, None) == 1
    assert L.dust_outer_product(FAKE, FAKE, 0, 4, 4, FAKE, None, 0, None) == 1
    # a shape that needs split partial sums, without workspace
    assert L.dust_outer_workspace_bytes(4096, 2048, 512) > 0
    assert L.dust_outer_product(FAKE, FAKE, 4096, 2048, 512, FAKE, None, 0, None) == 3
    assert L.dust_noise(1, 0, 0, 1, 0, 1, 4, None, None, None) == 1
    assert L.dust_noise(1, 0, 2**32 - 1, 2, 0, 1, 4, None, FAKE, None) == 1
    assert L.dust_noise(1, 0, 0, 0, 0, 1, 4, None, FAKE, None) == 1
    assert L.dust_noise(1, 0, 0, 1, 2**33, 1, 4, None, FAKE, None) == 1
    # the single-(draw, token) export
    assert L.dust_debug_noise(1, 0, 0, 0, 4, None, None, None) == 1
    assert L.dust_debug_noise(1, 0, 0, 0, 0, None, FAKE, None) == 1
    assert L.dust_debug_noise(1, 0, 0, 2**32, 4, None, FAKE, None) == 1
    assert "2^32" in L.dust_last_error().decode()


def test_linear_rejects_oversized_weights_on_host():
    L = dust.lib()

    def call(V, d=512, n=2048):
        st = L.dust_estimate_linear(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, d, n, V, 2, ctypes.c_float(0.01),
                                    ctypes.c_float(1e-5), 1, 0, 0, 0, FAKE, None, None, None, 0, None)
        return st, L.dust_last_error().decode()

    st, err = call(V=(1 << 31) // 512)  # V*d = 2^31: the W_head offsets would wrap
    assert st == 2 and "2^31" in err, err
    st, err = call(V=8192, d=256, n=(1 << 31) // 256)
    assert st == 2, err
    st, err = call(V=(1 << 31) // 512 - 1)  # the largest accepted vocabulary: fails only on the workspace
    assert st == 3, err


def test_head_noalloc_rejects_on_host():
    L = dust.lib()
    assert L.dust_head_noalloc_max_bytes() == 64 << 20

    def call(T, V, d, ghat=None, logits=FAKE):
        st = L.dust_estimate_head_noalloc(logits, 1, FAKE, FAKE, T, V, d, 4, ctypes.c_float(0.01), 1, 1, 0, 0, FAKE,
                                          ghat, None, None)
        return st, L.dust_last_error().decode()

    st, err = call(4096, 8192, 512)  # 128 MiB of g_hat rows alone
    assert st == 2 and "static scratch" in err, err
    st, err = call(4, 8, 2, logits=None)
    assert st == 1 and "non-NULL" in err, err


def test_workspace_queries():
    L = dust.lib()
    # large product (bf16-pair outer product): the estimator writes the g_hat
    # pairs into the outer product's workspace, which then holds both operands
    T, V, d = 4096, 8192, 512
    need = L.dust_head_workspace_bytes(T, V, d, 256)
    assert need == L.dust_outer_workspace_bytes(T, V, d)
    assert need >= 2 * 2 * T * V + 2 * 2 * T * d
    # small product (fp32 outer product): g_hat needs a buffer of its own
    T, V, d = 256, 512, 64
    assert L.dust_head_workspace_bytes(T, V, d, 64) >= 4 * T * V + L.dust_outer_workspace_bytes(T, V, d)
    assert L.dust_head_workspace_bytes(0, V, d, 1) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(TypeError):
        dust.estimate_head(torch.zeros(2, 4), torch.zeros(2, 3), torch.zeros(2, dtype=torch.int32), 1, 0.1, 0, 0)


def _lm(cfg_kw=None, hp_kw=None, **kw):
    c = dict(V=100, d=64, H=1, L=2, n=128, S=128, B=2, ln_eps=1e-5)
    c.update(cfg_kw or {})
    h = dict(K=4, M=2, sigma=0.01, sigma_es=0.01)
    h.update(hp_kw or {})
    cfg = dust.LMConfig(**c)
    hp = dust.lm_hparams(h["K"], h["M"], h["sigma"], h["sigma_es"])
    a = dict(params=FAKE, tok=FAKE, lab=FAKE, grads=FAKE, rew=None, ws=None, wsb=0, hp=ctypes.byref(hp))
    a.update(kw)
    L = dust.lib()
    st = L.dust_lm_estimate(ctypes.byref(cfg), a["hp"], a["params"], a["tok"], a["lab"], 1, a["grads"], a["rew"],
                            a["ws"], a["wsb"], None)
    return st, L.dust_last_error().decode()


@pytest.mark.parametrize("cfg_kw,hp_kw,kw,status,msg", [
    (dict(d=96), None, {}, 2, "d = 64 H"),
    (dict(H=17, d=64 * 17), None, {}, 2, "d = 64 H"),
    (dict(S=100), None, {}, 2, "S must be"),
    (dict(S=8192), None, {}, 2, "S must be"),
    (dict(n=100), None, {}, 2, "n must be"),
    (dict(V=40000), None, {}, 2, "V must be"),
    (dict(L=0), None, {}, 2, "L must be"),
    (dict(L=33), None, {}, 2, "L must be"),
    (dict(B=0), None, {}, 1, "B must be"),
    (dict(ln_eps=0.0), None, {}, 1, "ln_eps"),
    (None, dict(K=0), {}, 1, "K and M"),
    (None, dict(M=0), {}, 1, "K and M"),
    (None, dict(sigma=0.0), {}, 1, "sigma"),
    (None, dict(sigma_es=float("nan")), {}, 1, "sigma"),
    (None, None, dict(hp=None), 1, "hp is NULL"),
    (None, None, dict(params=None), 1, "non-NULL"),
    (None, None, dict(params=FAKE_MIS), 1, "aligned"),
    (None, None, dict(ws=None), 3, "workspace"),
])
def test_lm_step_rejects_bad_arguments_on_host(cfg_kw, hp_kw, kw, status, msg):
    st, err = _lm(cfg_kw, hp_kw, **kw)
    assert st == status and msg in err, (st, err)


def test_lm_sizes():
    import synth

    for V, d, H, L, n, S in ((100, 64, 1, 2, 128, 128), (8192, 128, 2, 2, 512, 256), (7, 192, 3, 1, 64, 64)):
        cfg = dust.lm_config(V, d, H, L, n, S, 2)
        want = sum(int(ctypes.c_int64(1).value * __import__("math").prod(s)) for _, s in
                   synth.lm_param_layout(V, d, L, n, S))
        assert dust.lm_param_count(cfg) == want
        hp = dust.lm_hparams(5, 3, 0.01, 0.01)
        assert dust.lm_rewards_count(cfg, hp) == (5 + 3 * L) * 5 * 2 * S + 2 * 3
        assert dust.lm_workspace_bytes(cfg, hp) > 4 * want
    assert dust.lm_param_count(dust.lm_config(100, 96, 1, 2, 128, 128, 2)) == 0
    L = dust.lib()
    st = L.dust_lm_sgd(ctypes.byref(dust.lm_config(100, 64, 1, 2, 128, 128, 2)),
                       ctypes.byref(dust.lm_hparams(4, 2, 0.01, 0.01, lr=float("nan"))), FAKE, FAKE, FAKE, None)
    assert st == 1 and "finite" in L.dust_last_error().decode()
