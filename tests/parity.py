"""Helpers shared by the GPU parity tests (not a test module).

Parity metric: err = max_i |x_i - r_i| / max(|r_i|, rms(r_row)) against the
fp64 oracle r, where r_row is the output row (the D channels of one
(b, h, p)) holding element i; LSE: |x - r| <= tol * max(1, |r|).  The floor is
per row because causal rows differ in scale (a row averaging p+1 values has
magnitude ~ 1/sqrt(p+1)) while bf16 output rounding is relative to each row.
Tolerances: 1e-5 for float32 data, 1e-2 for bfloat16 data (float32
accumulation).
"""
import sys

import numpy as np
import torch

import oracle
from cross_layer_kv_amd import inputs

TOL = {torch.float32: 1e-5, torch.bfloat16: 1e-2}


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def rel_err(x, r):
    """x, r: [rows, D]."""
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    floor = np.maximum(np.abs(r), np.where(rms > 0, rms, 1.0))
    return float(np.max(np.abs(x - r) / floor))


def lse_err(x, r):
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    both_inf = np.isneginf(x) & np.isneginf(r)
    xs, rs = np.where(both_inf, 0.0, x), np.where(both_inf, 0.0, r)
    d = np.abs(xs - rs) / np.maximum(1.0, np.abs(rs))
    return float(np.max(d)) if d.size else 0.0


def oracle_layer(L, *, fused=True, causal=False, rows=None, batch=None, single=("kn", "v1")):
    """Oracle output for LayerInputs L (optionally only batch rows `batch`
    [list of b], then rows index that sub-batch)."""
    def h(t):
        if batch is not None:
            t = t[batch]
        return inputs.host_array(t)
    sl = None
    if L.seqlens_k is not None:
        sl = L.seqlens_k.cpu().numpy()
        if batch is not None:
            sl = sl[batch]
    if fused:
        w = [x.cpu().numpy() for x in L.weights]
        return oracle.attend(h(L.q), h(L.k1), h(L.v1), h(L.kn), h(L.vn), k_w1=w[0], k_wn=w[1], v_w1=w[2],
                             v_wn=w[3], causal=causal, seqlens_k=sl, rows=rows)
    k = getattr(L, single[0])
    v = getattr(L, single[1])
    return oracle.attend(h(L.q), h(k), h(v), causal=causal, seqlens_k=sl, rows=rows)


def gpu_rows(out, B, Hq, Sq, D):
    """[B, Sq, Hq, D] GPU output as oracle row order [(b, h, p), D]."""
    return out.float().cpu().numpy().transpose(0, 2, 1, 3).reshape(B * Hq * Sq, D)
