"""Rounding budget of the backward kernels (helper of the tests, not a test
module, and not an implementation the kernels are compared with).

The fp64 backward oracle (oracle/backward.py) is evaluated a second time
with bfloat16 rounding applied at the points where the kernels round:
  * the fused key and value tiles (matrix-core operands),
  * the probabilities P and dS = P (dP - Delta) (matrix-core operands;
    the key-tile kernel forms its dS from P rounded once to binary16,
    2^-11, which is left out here as an eighth of a bfloat16 rounding),
  * Delta = rowsum(dO * O) taken from the bfloat16 forward output O,
  * the bfloat16 gradient outputs.
Its error against the exact oracle is the error this arithmetic has by
itself; the GPU parity tests allow twice that (and never less than 1e-2).
Softmax gradients cancel (every dS row sums to zero), which is why single
2^-9 roundings grow to a few percent on the early causal rows.

Metrics (per output tensor x against the exact r):
  elementwise  max_i |x_i - r_i| / max(|r_i|, rms(r))
  normwise     ||x - r||_2 / ||r||_2
"""
import math

import numpy as np
import torch

from oracle import backward as bw


def bf16(x):
    """float64 -> nearest bfloat16 (ties to even) -> float64."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def elementwise(x, r):
    x = np.asarray(x, np.float64).ravel()
    r = np.asarray(r, np.float64).ravel()
    if r.size == 0:
        return 0.0
    rms = math.sqrt(float(np.mean(r * r)))
    floor = np.maximum(np.abs(r), rms if rms > 0 else 1.0)
    return float(np.max(np.abs(x - r) / floor))


def normwise(x, r):
    x = np.asarray(x, np.float64).ravel()
    r = np.asarray(r, np.float64).ravel()
    n = float(np.linalg.norm(r))
    return float(np.linalg.norm(x - r)) / (n if n > 0 else 1.0)


def model(q, k1, v1, dout, kn=None, vn=None, *, k_w1=None, k_wn=None, v_w1=None, v_wn=None, causal=True,
          heads=None):
    """Gradients with the kernels' rounding points (same arguments and
    result keys as oracle.backward.backward)."""
    Q, dO = bw._f64(q), bw._f64(dout)
    K1, V1 = bw._f64(k1), bw._f64(v1)
    fused = kn is not None
    B, S, Hq, D = Q.shape
    Hkv = K1.shape[2]
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(D)
    if fused:
        Kn, Vn = bw._f64(kn), bw._f64(vn)
        w = [np.asarray(x, np.float64).reshape(Hkv, D) for x in (k_w1, k_wn, v_w1, v_wn)]
        Kx = w[0][None, None] * K1 + w[1][None, None] * Kn
        Vx = w[2][None, None] * V1 + w[3][None, None] * Vn
    else:
        Kx, Vx = K1, V1
    Kb, Vb = bf16(Kx), bf16(Vx)
    vis = np.tril(np.ones((S, S), dtype=bool)) if causal else np.ones((S, S), dtype=bool)
    dq = np.zeros_like(Q)
    dkf = np.zeros_like(Kx)
    dvf = np.zeros_like(Vx)
    for b in range(B):
        for g in (range(Hkv) if heads is None else heads):
            for h in range(g * G, (g + 1) * G):
                s = np.where(vis, sc * (Q[b, :, h] @ Kx[b, :, g].T), -np.inf)
                m = s.max(axis=1, keepdims=True)
                e = np.where(vis, np.exp(s - m), 0.0)
                P = e / e.sum(axis=1, keepdims=True)
                O = bf16(P @ Vx[b, :, g])
                do = dO[b, :, h]
                delta = (do * O).sum(axis=1, keepdims=True)
                sb = np.where(vis, sc * (Q[b, :, h] @ Kb[b, :, g].T), -np.inf)
                Pb = np.where(vis, np.exp(sb - (m + np.log(e.sum(axis=1, keepdims=True)))), 0.0)
                dS = bf16(Pb * (do @ Vb[b, :, g].T - delta))
                dq[b, :, h] = sc * (dS @ Kb[b, :, g])
                dkf[b, :, g] += sc * (dS.T @ Q[b, :, h])
                dvf[b, :, g] += bf16(Pb).T @ do
    out = {"dq": bf16(dq)}
    if fused:
        out.update(dk1=bf16(w[0][None, None] * dkf), dkn=bf16(w[1][None, None] * dkf),
                   dv1=bf16(w[2][None, None] * dvf), dvn=bf16(w[3][None, None] * dvf),
                   dk_w1=(dkf * K1).sum(axis=(0, 1)), dk_wn=(dkf * Kn).sum(axis=(0, 1)),
                   dv_w1=(dvf * V1).sum(axis=(0, 1)), dv_wn=(dvf * Vn).sum(axis=(0, 1)))
    else:
        out.update(dk=bf16(dkf), dv=bf16(dvf))
    return out
