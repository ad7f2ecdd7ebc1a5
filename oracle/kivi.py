"""KIVI-style 4-bit source caches for the FusedKV oracle.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the tests, the smoke
check and the benchmark's CPU-baseline leg use it; the product path never
does, and this file imports nothing from the HIP package.

Pages cited (by title):
  [Deck]  "FusedKV: Reconstructing KV Caches with Cross-Layer Fusion",
          frame "Four-bit KV quantization is the stronger combination"
          (Tables 14-15): FusedKV composed with 4-bit KIVI caches, a 4-fold
          payload cut on top of FusedKV's halving, 1/8 of an FP16 vanilla
          cache excluding quantisation metadata.
  [Notes] "FusedKV:通过跨层融合重构 KV 缓存", section A.6.5.

The pages name KIVI but print no format.  Reading taken (the published KIVI
scheme, 4-bit, without its full-precision window of recent tokens):
  * asymmetric integer codes: x ~ mn + sc * q, q in 0..15;
  * keys are grouped per channel over 32 consecutive tokens, values per token
    over 32 consecutive channels (the last group of an axis may be shorter);
  * mn is the group minimum and sc = (max - min) / 15, both stored as IEEE
    binary16; the code of x is rint((x - mn16) * (1 / sc16)) clamped to
    0..15, every step in float32 (so that a kernel taking the same decision
    in float32 reproduces it), and 0 when sc16 == 0.
Dequantisation mn16 + sc16 * q is exact in float64, and the attention of a
layer over quantised sources is the plain oracle attention over the
dequantised caches (fusion after dequantisation, as the pages compose them).

Arrays here are the plain form of that definition, one code per element
(how a library packs codes into bytes is its own storage choice):
  key codes    uint8   [B, H, S, D]           0..15
  key meta     float16 [B, H, ceil(S/32), D]  (scale, minimum) per token group and channel
  value codes  uint8   [B, H, S, D]           0..15
  value meta   float16 [B, H, S, ceil(D/32)]  (scale, minimum) per token and channel group
"""
from __future__ import annotations

import numpy as np

from . import oracle

GROUP = 32
LEVELS = 15


def _as_f32(x):
    """bfloat16 bit patterns (uint16) or float32 -> float32, exactly."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    if x.dtype == np.float32:
        return x
    raise TypeError("quantise bfloat16 bits or float32, got %s" % x.dtype)


def _quantise_group(xs, axis):
    """Codes, scale (fp16) and minimum (fp16) of groups laid along ``axis``."""
    f32 = np.float32
    mn = xs.min(axis=axis, keepdims=True)
    mx = xs.max(axis=axis, keepdims=True)
    sc = (mx - mn) / f32(LEVELS)
    mn16 = mn.astype(np.float16)
    sc16 = sc.astype(np.float16)
    m = mn16.astype(f32)
    s = sc16.astype(f32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s > 0, f32(1) / s, f32(0)).astype(f32)
        t = ((xs - m).astype(f32) * r).astype(f32)
    q = np.clip(np.rint(t), 0, LEVELS)
    q = np.where(s > 0, q, 0).astype(np.uint8)
    return q, np.squeeze(sc16, axis), np.squeeze(mn16, axis)


def quantise_keys(k):
    """k: [B, S, H, D] (bf16 bits or float32, any strides) -> (codes
    [B, H, S, D], scale, minimum [B, H, ceil(S/32), D]): per-channel groups of
    32 tokens."""
    x = np.ascontiguousarray(np.transpose(_as_f32(k), (0, 2, 1, 3)))  # [B, H, S, D]
    B, H, S, D = x.shape
    ng = (S + GROUP - 1) // GROUP
    q = np.zeros((B, H, S, D), dtype=np.uint8)
    sc = np.zeros((B, H, ng, D), dtype=np.float16)
    mn = np.zeros((B, H, ng, D), dtype=np.float16)
    for j in range(ng):
        t0, t1 = j * GROUP, min(S, (j + 1) * GROUP)
        q[:, :, t0:t1], sc[:, :, j], mn[:, :, j] = _quantise_group(x[:, :, t0:t1], axis=2)
    return q, sc, mn


def quantise_values(v):
    """v: [B, S, H, D] -> (codes [B, H, S, D], scale, minimum
    [B, H, S, ceil(D/32)]): per-token groups of 32 channels."""
    x = np.ascontiguousarray(np.transpose(_as_f32(v), (0, 2, 1, 3)))  # [B, H, S, D]
    B, H, S, D = x.shape
    ng = (D + GROUP - 1) // GROUP
    q = np.zeros((B, H, S, D), dtype=np.uint8)
    sc = np.zeros((B, H, S, ng), dtype=np.float16)
    mn = np.zeros((B, H, S, ng), dtype=np.float16)
    for c in range(ng):
        d0, d1 = c * GROUP, min(D, (c + 1) * GROUP)
        q[..., d0:d1], sc[..., c], mn[..., c] = _quantise_group(x[..., d0:d1], axis=3)
    return q, sc, mn


def dequantise_keys(q, sc, mn):
    """-> float64 [B, S, H, D]: mn16 + sc16 * q of each token's group, exact."""
    S = q.shape[2]
    tok_group = np.arange(S) // GROUP
    x = mn.astype(np.float64)[:, :, tok_group, :] + sc.astype(np.float64)[:, :, tok_group, :] * q
    return np.transpose(x, (0, 2, 1, 3))


def dequantise_values(q, sc, mn):
    """-> float64 [B, S, H, D]: mn16 + sc16 * q of each channel's group, exact."""
    D = q.shape[3]
    ch_group = np.arange(D) // GROUP
    x = mn.astype(np.float64)[..., ch_group] + sc.astype(np.float64)[..., ch_group] * q
    return np.transpose(x, (0, 2, 1, 3))


def _q_f64(q):
    return _as_f32(q).astype(np.float64)


def attend(q, k1, v1, kn=None, vn=None, **kw):
    """Oracle attention over quantised sources.  k1/kn are (codes, scale,
    minimum) key triples, v1/vn value triples, in the plain form above;
    keyword arguments as ``oracle.attend`` (weights, causal, scale,
    seqlens_k, rows)."""
    qd = _q_f64(q)
    K1 = dequantise_keys(*k1)
    V1 = dequantise_values(*v1)
    if kn is None:
        return oracle.attend(qd, K1, V1, **kw)
    return oracle.attend(qd, K1, V1, dequantise_keys(*kn), dequantise_values(*vn), **kw)


def payload_bytes(L, S, Hkv, D, method, bits):
    """Resident cache payload of an L-layer model in bytes, metadata
    excluded: capacity elements ([Deck] Table 1) times bits / 8."""
    return oracle.cache_capacity(method, L, S, Hkv, D) * bits // 8


def metadata_bytes(S, Hkv, D, B=1):
    """fp16 scale and minimum of one quantised source, for a store that keeps
    value metadata per whole 32-token block (so a partial last block counts
    whole): keys and values have the same count when S and D are multiples
    of 32."""
    keys = B * Hkv * ((S + GROUP - 1) // GROUP) * D * 2 * 2
    values = B * Hkv * ((S + GROUP - 1) // GROUP) * GROUP * ((D + GROUP - 1) // GROUP) * 2 * 2
    return keys, values
