"""Pins for the self-conditioning injection oracle: the GELU against torch's tanh
GELU (a library routine), closed forms on one-unit MLPs that fix which half of
w_gate_up is the gate, the embedding gather alone, and linearity in w_down.

Pages: [P1] "DiffusionGemma: vLLM에서 네이티브로 처음 지원되는 첫 번째 Diffusion LLM",
sections "안정성을 위한 셀프 컨디셔닝" and "ModelState 인터페이스".
"""
import numpy as np
import torch

from oracle.inject import gelu_tanh, selfcond_inject


def test_gelu_matches_torch_tanh_gelu():
    x = np.linspace(-8, 8, 4001)
    want = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    np.testing.assert_allclose(gelu_tanh(x), want, rtol=1e-12, atol=1e-15)


def test_gather_only_when_the_mlp_is_off():
    rng = np.random.default_rng(1)
    E = rng.standard_normal((50, 16))
    tokens = np.array([3, 49, 0, 3, 17])
    s = rng.standard_normal((5, 16))
    wgu = rng.standard_normal((16, 2 * 8))
    out = selfcond_inject(tokens, E, s, wgu, np.zeros((8, 16)))
    np.testing.assert_array_equal(out, E[tokens])
    # a zero gate (gelu(0) = 0) or a zero up projection also leaves only the gather
    for half in (slice(0, 8), slice(8, 16)):
        w = wgu.copy()
        w[:, half] = 0.0
        np.testing.assert_array_equal(selfcond_inject(tokens, E, s, w, rng.standard_normal((8, 16))), E[tokens])


def test_one_unit_closed_forms_fix_the_gate_half():
    """hidden = 1, s = e_0: gate = w_gate_up[0, 0], up = w_gate_up[0, 1];
    out = E[t] + gelu(gate) * up * w_down[0]."""
    d = 4
    E = np.arange(3 * d, dtype=np.float64).reshape(3, d)
    s = np.zeros((1, d))
    s[0, 0] = 1.0
    wd = np.array([[1.0, -2.0, 0.5, 3.0]])
    for gate, up in ((10.0, -3.0), (-3.0, 10.0), (0.5, 2.0)):
        wgu = np.zeros((d, 2))
        wgu[0] = [gate, up]
        g = 0.5 * gate * (1 + np.tanh(np.sqrt(2 / np.pi) * (gate + 0.044715 * gate ** 3)))
        out = selfcond_inject(np.array([2]), E, s, wgu, wd)
        np.testing.assert_allclose(out[0], E[2] + g * up * wd[0], rtol=1e-14, atol=1e-14)
    # gelu(10) = 10 to double precision and gelu(-3) is about -0.0036: the two orders differ by far
    a = selfcond_inject(np.array([0]), E, s, np.array([[10.0, -3.0]] + [[0, 0]] * 3), wd)
    b = selfcond_inject(np.array([0]), E, s, np.array([[-3.0, 10.0]] + [[0, 0]] * 3), wd)
    np.testing.assert_allclose(a[0] - E[0], -30.0 * wd[0], rtol=1e-12)
    assert np.abs(b[0] - E[0]).max() < 0.2


def test_linear_in_w_down():
    rng = np.random.default_rng(2)
    E = rng.standard_normal((20, 8))
    t = rng.integers(0, 20, 6)
    s = rng.standard_normal((6, 8))
    wgu = rng.standard_normal((8, 2 * 4))
    w1, w2 = rng.standard_normal((4, 8)), rng.standard_normal((4, 8))
    f = lambda w: selfcond_inject(t, E, s, wgu, w) - E[t]
    np.testing.assert_allclose(f(w1 + 2.0 * w2), f(w1) + 2.0 * f(w2), rtol=1e-12, atol=1e-12)
