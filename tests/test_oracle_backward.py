"""Pins of the backward oracle (oracle/backward.py) against things other than
itself: central finite differences of the FORWARD oracle (fkv_oracle.c, an
independent C statement of the forward definition), torch's float64
autograd of scaled_dot_product_attention on the materialised fused caches,
and identities of the method: softmax shift invariance, the selector weights
that reduce FusedKV to Lite, the one-token closed form, token permutation.

Pages cited (by title):
  [Deck]  "FusedKV: Reconstructing KV Caches with Cross-Layer Fusion", frames
          "FusedKV learns two-source, channel-wise fusion" (Eqs. (4)-(5),
          trained end to end), "Lite separates the key source from the value
          source" (Eq. (6)), "Post-RoPE fusion needs paired key weights".
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import backward as bw

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")

NAMES = ("q", "k1", "kn", "v1", "vn", "k_w1", "k_wn", "v_w1", "v_wn")


def _inputs(B, S, Hq, Hkv, D, seed, scale_w=1.0):
    r = np.random.default_rng(seed)
    x = dict(q=r.standard_normal((B, S, Hq, D)), k1=r.standard_normal((B, S, Hkv, D)),
             kn=r.standard_normal((B, S, Hkv, D)), v1=r.standard_normal((B, S, Hkv, D)),
             vn=r.standard_normal((B, S, Hkv, D)))
    for n in ("k_w1", "k_wn", "v_w1", "v_wn"):
        x[n] = scale_w * (0.5 + 0.25 * r.standard_normal((Hkv, D)))
    x["dout"] = r.standard_normal((B, S, Hq, D))
    return x


def _forward(x, causal):
    """Forward oracle (C, float64 inputs) as [B, S, Hq, D]."""
    B, S, Hq, D = x["q"].shape
    o, _ = oracle.attend(x["q"], x["k1"], x["v1"], x["kn"], x["vn"], k_w1=x["k_w1"].astype(np.float32),
                         k_wn=x["k_wn"].astype(np.float32), v_w1=x["v_w1"].astype(np.float32),
                         v_wn=x["v_wn"].astype(np.float32), causal=causal)
    return o.reshape(B, Hq, S, D).transpose(0, 2, 1, 3)


def _grads(x, causal, scale=None):
    return bw.backward(x["q"], x["k1"], x["v1"], x["dout"], x["kn"], x["vn"], k_w1=x["k_w1"], k_wn=x["k_wn"],
                       v_w1=x["v_w1"], v_wn=x["v_wn"], causal=causal, scale=scale)


@pytest.mark.parametrize("causal", [True, False])
def test_matches_finite_differences_of_the_forward_oracle(causal):
    """Every gradient entry against a central difference of L = <dO, O(x)>,
    with O from the C forward oracle.  The forward oracle takes its fusion
    weights as float32, so the weights here are float32-representable and
    are perturbed by a float32-exact step."""
    x = _inputs(1, 5, 4, 2, 4, 11)
    for n in ("k_w1", "k_wn", "v_w1", "v_wn"):
        x[n] = x[n].astype(np.float32).astype(np.float64)
    g = _grads(x, causal)
    key = {"q": "dq", "k1": "dk1", "kn": "dkn", "v1": "dv1", "vn": "dvn",
           "k_w1": "dk_w1", "k_wn": "dk_wn", "v_w1": "dv_w1", "v_wn": "dv_wn"}

    def loss(y):
        return float((_forward(y, causal) * y["dout"]).sum())

    for n in NAMES:
        h = 2.0 ** -12 if n.endswith(("w1", "wn")) else 1e-6
        num = np.zeros_like(x[n])
        for idx in np.ndindex(*x[n].shape):
            y = {k: v.copy() for k, v in x.items()}
            y[n][idx] += h
            lp = loss(y)
            y[n][idx] -= 2 * h
            lm = loss(y)
            num[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(num - g[key[n]])) / max(1.0, np.max(np.abs(num)))
        assert err < 2e-6, (n, err)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("G", [1, 2, 4])
def test_matches_torch_autograd_float64(causal, G):
    """Library routine: torch float64 autograd through the fusion and
    scaled_dot_product_attention (KV heads repeated G times)."""
    Hkv = 2
    x = _inputs(2, 33, Hkv * G, Hkv, 16, 20 + G)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=(k != "dout")) for k, v in x.items()}
    kf = t["k_w1"] * t["k1"] + t["k_wn"] * t["kn"]
    vf = t["v_w1"] * t["v1"] + t["v_wn"] * t["vn"]

    def bhsd(z, rep):
        z = z.permute(0, 2, 1, 3)
        return z.repeat_interleave(rep, dim=1) if rep > 1 else z

    o = F.scaled_dot_product_attention(bhsd(t["q"], 1), bhsd(kf, G), bhsd(vf, G), is_causal=causal)
    (o.permute(0, 2, 1, 3) * t["dout"]).sum().backward()
    g = _grads(x, causal)
    for n, k in (("q", "dq"), ("k1", "dk1"), ("kn", "dkn"), ("v1", "dv1"), ("vn", "dvn"),
                 ("k_w1", "dk_w1"), ("k_wn", "dk_wn"), ("v_w1", "dv_w1"), ("v_wn", "dv_wn")):
        ref = t[n].grad.numpy()
        assert np.max(np.abs(ref - g[k])) <= 1e-10 * max(1.0, np.max(np.abs(ref))), n


def test_softmax_shift_invariance_zeroes_the_key_gradient_sum():
    """Adding one vector to every visible key leaves each softmax row
    unchanged, so the fused-key gradient sums to zero over the tokens of
    every (batch, KV head) -- also under the causal mask, where every query
    row still sees token 0."""
    x = _inputs(2, 40, 8, 2, 8, 31)
    for causal in (True, False):
        g = _grads(x, causal)
        s = np.abs(g["dkf"].sum(axis=1))
        assert np.max(s) < 1e-12 * max(1.0, np.max(np.abs(g["dkf"]))) * 40


def test_selector_weights_reduce_to_lite():
    """(a, a', b, b') = (0, 1, 1, 0) reads exactly K^n and V^1, the Lite
    layer: dK^1 = dV^n = 0 and the other gradients equal Lite's bit for bit."""
    x = _inputs(1, 17, 4, 2, 8, 41)
    z, o = np.zeros((2, 8)), np.ones((2, 8))
    x.update(k_w1=z, k_wn=o, v_w1=o, v_wn=z)
    g = _grads(x, True)
    lite = bw.backward(x["q"], x["kn"], x["v1"], x["dout"], causal=True)
    assert np.all(g["dk1"] == 0) and np.all(g["dvn"] == 0)
    assert np.array_equal(g["dkn"], lite["dk"]) and np.array_equal(g["dv1"], lite["dv"])
    assert np.array_equal(g["dq"], lite["dq"])


def test_one_token_closed_form():
    """S = 1: the softmax of one score is 1 whatever the score, so dQ = 0
    and dK~ = 0, and dV~ is the sum of dO over the KV head's query heads."""
    x = _inputs(2, 1, 6, 2, 8, 51)
    g = _grads(x, True)
    assert np.all(g["dq"] == 0) and np.all(g["dkf"] == 0)
    ref = x["dout"].reshape(2, 1, 2, 3, 8).sum(axis=3)
    assert np.allclose(g["dvf"], ref, rtol=0, atol=1e-14)
    w = x["v_w1"]
    assert np.allclose(g["dv_w1"], (ref * x["v1"]).sum(axis=(0, 1)), rtol=0, atol=1e-13)
    assert np.allclose(g["dv1"], w[None, None] * ref, rtol=0, atol=1e-14)


def test_token_permutation_without_mask():
    """Without the mask, permuting the cached tokens permutes dK and dV and
    leaves dQ and the weight gradients unchanged."""
    x = _inputs(1, 12, 4, 2, 8, 61)
    perm = np.random.default_rng(3).permutation(12)
    y = dict(x)
    for n in ("k1", "kn", "v1", "vn"):
        y[n] = x[n][:, perm]
    gx, gy = _grads(x, False), _grads(y, False)
    assert np.allclose(gy["dq"], gx["dq"], rtol=0, atol=1e-13)
    for n in ("dk1", "dkn", "dv1", "dvn"):
        assert np.allclose(gy[n], gx[n][:, perm], rtol=0, atol=1e-13)
    for n in ("dk_w1", "dk_wn", "dv_w1", "dv_wn"):
        assert np.allclose(gy[n], gx[n], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("pairing", ["interleaved", "half"])
def test_tied_key_weight_gradient(pairing):
    """A tied key weight (one parameter per RoPE pair) receives the sum of
    its two channels' gradients: torch autograd through the tied
    parameterisation against tie_pairs of the per-channel oracle gradient."""
    x = _inputs(1, 9, 4, 2, 8, 71)
    D = 8
    idx = np.arange(D) // 2 if pairing == "interleaved" else np.arange(D) % (D // 2)
    c = torch.tensor(np.random.default_rng(5).standard_normal((2, D // 2)), dtype=torch.float64, requires_grad=True)
    a = c[:, torch.as_tensor(idx)]
    x["k_w1"] = a.detach().numpy().copy()
    t = {k: torch.tensor(v, dtype=torch.float64) for k, v in x.items()}
    kf = a * t["k1"] + t["k_wn"] * t["kn"]
    vf = t["v_w1"] * t["v1"] + t["v_wn"] * t["vn"]
    o = F.scaled_dot_product_attention(t["q"].permute(0, 2, 1, 3), kf.permute(0, 2, 1, 3).repeat_interleave(2, 1),
                                       vf.permute(0, 2, 1, 3).repeat_interleave(2, 1), is_causal=True)
    (o.permute(0, 2, 1, 3) * t["dout"]).sum().backward()
    g = _grads(x, True)
    assert np.allclose(bw.tie_pairs(g["dk_w1"], pairing), c.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_scale_argument():
    """The scale enters the scores only: dQ and dK~ at scale c equal the
    gradients at the default scale with the query multiplied by c sqrt(D)
    (dQ also multiplied by that factor)."""
    x = _inputs(1, 10, 2, 1, 16, 81)
    c = 0.37
    f = c * np.sqrt(16)
    g1 = _grads(x, True, scale=c)
    y = dict(x)
    y["q"] = x["q"] * f
    g2 = _grads(y, True)
    assert np.allclose(g1["dq"], g2["dq"] * f, rtol=1e-12, atol=1e-13)
    assert np.allclose(g1["dkf"], g2["dkf"], rtol=1e-12, atol=1e-13)
    assert np.allclose(g1["dvf"], g2["dvf"], rtol=1e-12, atol=1e-13)


def test_flops_closed_form():
    # S = 2, causal: 3 visible pairs; 5 products of 2 D flops each
    assert bw.flops(1, 2, 1, 1) == 30
    assert bw.flops(4, 8192, 16, 128) == 5 * 2 * 128 * (8192 * 8193 // 2) * 4 * 16
    assert bw.flops(1, 4, 1, 2, causal=False) == 5 * 2 * 2 * 16
