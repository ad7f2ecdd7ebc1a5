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
    in float32 reproduces it), and 0 when sc16 == 0;
  * two codes per byte, channel 2i in the low nibble and 2i+1 in the high one.
Dequantisation mn16 + sc16 * q is exact in float64, and the attention of a
layer over quantised sources is the plain oracle attention over the
dequantised caches (fusion after dequantisation, as the pages compose them).

Array layouts (those of the library's quantised caches; a storage choice,
the pages fix none):
  key codes    uint8   [B, H, S, D/2]            channel 2i low nibble, 2i+1 high
  key meta     float16 [B, H, ceil(S/32), D]     (scale and minimum, one each)
  value codes  uint8   [B, H, NB, D, 16]         NB = ceil(S/32) blocks of 32 tokens
  value meta   float16 [B, H, NB, ceil(D/32), 32]
Value codes are channel-major inside each 32-token block: the 16 bytes of
(block, channel) are four 4-byte words w = 0..3, and word w holds the eight
tokens  4w + (e % 4) + 16 (e // 4),  e = 0..7,  element e in nibble e // 2
(bits 4 (e//2)) when e is even and in nibble 4 + e // 2 when e is odd.  The
value scale and minimum of (block, channel group) list the block's 32 tokens
in that same order, position 8w + e.  Tokens past S in the last block have
code 0, scale 0 and minimum 0.
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


def _pack(q):
    """[..., D] codes 0..15 -> [..., D/2] bytes (even channel in the low nibble)."""
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def _unpack(codes):
    lo = codes & 0x0F
    hi = codes >> 4
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def quantise_keys(k):
    """k: [B, S, H, D] (bf16 bits or float32, any strides) -> (codes, scale,
    minimum) with per-channel groups of 32 tokens."""
    x = np.ascontiguousarray(np.transpose(_as_f32(k), (0, 2, 1, 3)))  # [B, H, S, D]
    B, H, S, D = x.shape
    ng = (S + GROUP - 1) // GROUP
    q = np.zeros((B, H, S, D), dtype=np.uint8)
    sc = np.zeros((B, H, ng, D), dtype=np.float16)
    mn = np.zeros((B, H, ng, D), dtype=np.float16)
    for j in range(ng):
        t0, t1 = j * GROUP, min(S, (j + 1) * GROUP)
        q[:, :, t0:t1], sc[:, :, j], mn[:, :, j] = _quantise_group(x[:, :, t0:t1], axis=2)
    return _pack(q), sc, mn


def block_token(w, e):
    """Token (within its 32-token block) of element e of word w."""
    return 4 * w + (e % 4) + 16 * (e // 4)


def _nibble(e):
    """Nibble position of element e inside its 4-byte word."""
    return e // 2 if e % 2 == 0 else 4 + e // 2


def quantise_values(v):
    """v: [B, S, H, D] -> (codes, scale, minimum) with per-token groups of 32
    channels, in the block layout described above."""
    x = np.ascontiguousarray(np.transpose(_as_f32(v), (0, 2, 1, 3)))  # [B, H, S, D]
    B, H, S, D = x.shape
    ng = (D + GROUP - 1) // GROUP
    q = np.zeros((B, H, S, D), dtype=np.uint8)
    sc = np.zeros((B, H, S, ng), dtype=np.float16)
    mn = np.zeros((B, H, S, ng), dtype=np.float16)
    for c in range(ng):
        d0, d1 = c * GROUP, min(D, (c + 1) * GROUP)
        q[..., d0:d1], sc[..., c], mn[..., c] = _quantise_group(x[..., d0:d1], axis=3)
    return _to_blocks(q, sc, mn)


def _to_blocks(q, sc, mn):
    """Token-major codes [B, H, S, D] (0..15) and per-token metadata
    [B, H, S, ng] -> the block layout."""
    B, H, S, D = q.shape
    ng = sc.shape[-1]
    nb = (S + GROUP - 1) // GROUP
    codes = np.zeros((B, H, nb, D, 16), dtype=np.uint8)
    bsc = np.zeros((B, H, nb, ng, GROUP), dtype=np.float16)
    bmn = np.zeros((B, H, nb, ng, GROUP), dtype=np.float16)
    for j in range(nb):
        for w in range(4):
            for e in range(8):
                t = j * GROUP + block_token(w, e)
                if t >= S:
                    continue
                p = _nibble(e)
                byte = 4 * w + p // 2
                shift = 4 * (p % 2)
                codes[:, :, j, :, byte] |= (q[:, :, t, :] << shift).astype(np.uint8)
                bsc[:, :, j, :, 8 * w + e] = sc[:, :, t, :]
                bmn[:, :, j, :, 8 * w + e] = mn[:, :, t, :]
    return codes, bsc, bmn


def value_tokens(codes, sc, mn, S):
    """Block layout -> token-major codes [B, H, S, D] (0..15) and per-token
    scale and minimum [B, H, S, ng]."""
    B, H, nb, D, _ = codes.shape
    ng = sc.shape[3]
    q = np.zeros((B, H, nb * GROUP, D), dtype=np.uint8)
    s = np.zeros((B, H, nb * GROUP, ng), dtype=np.float16)
    m = np.zeros((B, H, nb * GROUP, ng), dtype=np.float16)
    for j in range(nb):
        for w in range(4):
            for e in range(8):
                t = j * GROUP + block_token(w, e)
                p = _nibble(e)
                q[:, :, t, :] = (codes[:, :, j, :, 4 * w + p // 2] >> (4 * (p % 2))) & 0x0F
                s[:, :, t, :] = sc[:, :, j, :, 8 * w + e]
                m[:, :, t, :] = mn[:, :, j, :, 8 * w + e]
    return q[:, :, :S], s[:, :, :S], m[:, :, :S]


def dequantise_keys(codes, sc, mn):
    """-> float64 [B, S, H, D]: mn16 + sc16 * q, exact."""
    q = _unpack(codes).astype(np.float64)  # [B, H, S, D]
    S = q.shape[2]
    tok_group = np.arange(S) // GROUP
    x = mn.astype(np.float64)[:, :, tok_group, :] + sc.astype(np.float64)[:, :, tok_group, :] * q
    return np.transpose(x, (0, 2, 1, 3))


def dequantise_values(codes, sc, mn, S):
    """Block layout of an S-token value cache -> float64 [B, S, H, D]."""
    q, s, m = value_tokens(codes, sc, mn, S)
    q = q.astype(np.float64)
    D = q.shape[3]
    ch_group = np.arange(D) // GROUP
    x = m.astype(np.float64)[..., ch_group] + s.astype(np.float64)[..., ch_group] * q
    return np.transpose(x, (0, 2, 1, 3))


def _q_f64(q):
    return _as_f32(q).astype(np.float64)


def attend(q, k1, v1, kn=None, vn=None, **kw):
    """Oracle attention over quantised sources.  k1/kn are (codes, scale,
    minimum) key triples, v1/vn value triples; keyword arguments as
    ``oracle.attend`` (weights, causal, scale, seqlens_k, rows)."""
    qd = _q_f64(q)
    K1 = dequantise_keys(*k1)
    S = K1.shape[1]
    V1 = dequantise_values(*v1, S)
    if kn is None:
        return oracle.attend(qd, K1, V1, **kw)
    return oracle.attend(qd, K1, V1, dequantise_keys(*kn), dequantise_values(*vn, S), **kw)


def payload_bytes(L, S, Hkv, D, method, bits):
    """Resident cache payload of an L-layer model in bytes, metadata
    excluded: capacity elements ([Deck] Table 1) times bits / 8."""
    return oracle.cache_capacity(method, L, S, Hkv, D) * bits // 8


def metadata_bytes(S, Hkv, D, B=1):
    """fp16 scale and minimum of one quantised source: keys and values have
    the same count when S and D are multiples of 32 (value metadata is
    stored per 32-token block, so a partial last block counts whole)."""
    keys = B * Hkv * ((S + GROUP - 1) // GROUP) * D * 2 * 2
    values = B * Hkv * ((S + GROUP - 1) // GROUP) * GROUP * ((D + GROUP - 1) // GROUP) * 2 * 2
    return keys, values
