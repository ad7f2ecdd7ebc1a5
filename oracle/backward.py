"""Backward pass of FusedKV reconstruction-layer attention, fp64 on the CPU.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the tests, the smoke
check and the benchmark's CPU-baseline leg use it; the product path never
does, and this file imports nothing from the HIP package.

Pages cited (by title):
  [Deck]  "FusedKV: Reconstructing KV Caches with Cross-Layer Fusion",
          frame "FusedKV learns two-source, channel-wise fusion"
          (Eqs. (4)-(5)): the fusion vectors are learned with the language
          model, trained end to end (no separate reconstruction loss), so a
          training step needs gradients through the fused attention with
          respect to the queries, the four source caches and the four
          per-channel vectors.  Frame "Lite separates the key source from the
          value source" (Eq. (6)) for the single-source form.
  [Notes] "FusedKV:通过跨层融合重构 KV 缓存", sections 2.1-2.3.

The pages print no backward formulas; what follows is the chain rule through
the definitions the forward oracle implements (fkv_oracle.c), for a loss whose
gradient with respect to the output O is dO (the LSE output is not
differentiated):

  Kf = a * K1 + a' * Kn,  Vf = bv * V1 + bv' * Vn           (fusion, per channel)
  s_pt = scale * <Q_p, Kf_t>,  P = softmax over visible t,  O_p = sum_t P_pt Vf_t
  dVf_t  = sum_{h in group} sum_p P_pt dO_p                   (O is linear in Vf)
  dP_pt  = <dO_p, Vf_t>
  dS_pt  = P_pt (dP_pt - sum_u P_pu dP_pu)                   (softmax Jacobian)
  dQ_p   = scale * sum_t dS_pt Kf_t
  dKf_t  = scale * sum_{h in group} sum_p dS_pt Q_p
  dK1 = a * dKf, dKn = a' * dKf, dV1 = bv * dVf, dVn = bv' * dVf
  da[g,d]  = sum_{b,t} dKf[b,t,g,d] K1[b,t,g,d]   (likewise a', bv, bv')

Masked (invisible) pairs have P = 0 and so contribute nothing.  Weight
gradients are per channel; a RoPE-tied key weight (one parameter for both
channels of a pair) has the sum of its two channels' gradients
(``tie_pairs``).  Matrix products are numpy matmuls in float64; nothing is
blocked or reordered beyond that.
"""
from __future__ import annotations

import math

import numpy as np


def _f64(x):
    """float32, float64 or bfloat16 bit patterns (uint16) -> float64, exactly."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError("inputs are float32, float64 or bfloat16 bits, got %s" % x.dtype)


def backward(q, k1, v1, dout, kn=None, vn=None, *, k_w1=None, k_wn=None, v_w1=None, v_wn=None,
             causal=True, scale=None, heads=None):
    """Gradients of one layer's attention.

    q, dout: [B, S, Hq, D]; caches [B, S, Hkv, D] (any strides); weights
    [Hkv, D].  FusedKV when kn/vn and the four weights are given, otherwise
    single-source (Lite with (K^n, V^1), or the plain control).

    ``heads``: optional list of KV heads g to compute (the others are left
    zero); the full-size tests use it to bound the work.

    Returns a dict of float64 arrays: dq [B,S,Hq,D]; fused: dk1, dkn, dv1,
    dvn [B,S,Hkv,D] and dk_w1, dk_wn, dv_w1, dv_wn [Hkv,D]; single: dk, dv.
    Also the intermediate dkf, dvf (gradients of the fused key and value).
    """
    Q = _f64(q)
    dO = _f64(dout)
    K1 = _f64(k1)
    V1 = _f64(v1)
    fused = kn is not None
    B, S, Hq, D = Q.shape
    Sk, Hkv = K1.shape[1], K1.shape[2]
    if Sk != S:
        raise ValueError("the backward pass takes Sq == Sk")
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if fused:
        Kn, Vn = _f64(kn), _f64(vn)
        wa, wan, wb, wbn = (np.asarray(w, dtype=np.float64).reshape(Hkv, D) for w in (k_w1, k_wn, v_w1, v_wn))
        Kf = wa[None, None] * K1 + wan[None, None] * Kn
        Vf = wb[None, None] * V1 + wbn[None, None] * Vn
    else:
        Kf, Vf = K1, V1
    dq = np.zeros_like(Q)
    dkf = np.zeros_like(Kf)
    dvf = np.zeros_like(Vf)
    vis = np.tril(np.ones((S, S), dtype=bool)) if causal else np.ones((S, S), dtype=bool)
    for b in range(B):
        for g in (range(Hkv) if heads is None else heads):
            K = Kf[b, :, g, :]
            V = Vf[b, :, g, :]
            for h in range(g * G, (g + 1) * G):
                q_ = Q[b, :, h, :]
                do = dO[b, :, h, :]
                s = sc * (q_ @ K.T)
                s = np.where(vis, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                e = np.where(vis, np.exp(s - m), 0.0)
                P = e / e.sum(axis=1, keepdims=True)
                dP = do @ V.T
                rowdot = (P * dP).sum(axis=1, keepdims=True)
                dS = P * (dP - rowdot)
                dq[b, :, h, :] = sc * (dS @ K)
                dkf[b, :, g, :] += sc * (dS.T @ q_)
                dvf[b, :, g, :] += P.T @ do
    out = {"dq": dq, "dkf": dkf, "dvf": dvf}
    if fused:
        out["dk1"] = wa[None, None] * dkf
        out["dkn"] = wan[None, None] * dkf
        out["dv1"] = wb[None, None] * dvf
        out["dvn"] = wbn[None, None] * dvf
        out["dk_w1"] = (dkf * K1).sum(axis=(0, 1))
        out["dk_wn"] = (dkf * Kn).sum(axis=(0, 1))
        out["dv_w1"] = (dvf * V1).sum(axis=(0, 1))
        out["dv_wn"] = (dvf * Vn).sum(axis=(0, 1))
    else:
        out["dk"] = dkf
        out["dv"] = dvf
    return out


def tie_pairs(grad, pairing="interleaved"):
    """Gradient of RoPE-tied key weights: one parameter per (head, pair),
    shared by the pair's two channels, receives the sum of their per-channel
    gradients ([Deck] frame "Post-RoPE fusion needs paired key weights",
    Eqs. (7)-(8)).
    Returns [Hkv, D/2]."""
    g = np.asarray(grad, dtype=np.float64)
    D = g.shape[-1]
    if pairing == "interleaved":
        return g[..., 0::2] + g[..., 1::2]
    if pairing == "half":
        return g[..., : D // 2] + g[..., D // 2:]
    raise ValueError("pairing is 'interleaved' or 'half'")


def flops(B, S, Hq, D, causal=True):
    """Algorithmic matrix-product flops of one backward call: the five
    products (recomputed scores, dP, dV, dQ, dK) over the visible pairs,
    an FMA counted as 2."""
    pairs = S * (S + 1) // 2 if causal else S * S
    return 5 * 2 * D * pairs * B * Hq
