"""Test-side converter between the oracle's plain 4-bit arrays
(``oracle/kivi.py``: one code per element, token-major metadata) and the
library's packed storage of a 4-bit cache (``include/fusedkv.h``).  It only
moves bits and indexes (no quantisation arithmetic), so the tests can hand
oracle-quantised caches to the GPU and compare GPU-quantised caches with the
oracle's, bit for bit.

Library storage, as ``include/fusedkv.h`` states it (NB = ceil(S/32)):
  key codes    uint8   [B, H, S, D/2]      channel 2i low nibble, 2i+1 high
  key meta     float16 [B, H, NB, D]       same as the plain form
  value codes  uint8   [B, H, NB, D, 16]   channel-major per 32-token block:
               the 16 bytes of (block, channel) are four 4-byte words; word w
               holds tokens 4w + e%4 + 16(e//4), e = 0..7, element e in
               nibble e//2 (even e) or 4 + e//2 (odd e)
  value meta   float16 [B, H, NB, ceil(D/32), 32]  the block's tokens in the
               same order (position 8w + e); padding tokens hold 0
"""
from __future__ import annotations

import numpy as np

GROUP = 32


def block_token(w, e):
    """Token (within its 32-token block) of element e of word w."""
    return 4 * w + (e % 4) + 16 * (e // 4)


def nibble(e):
    """Nibble position of element e inside its 4-byte word."""
    return e // 2 if e % 2 == 0 else 4 + e // 2


def pack_pairs(q):
    """[..., D] codes 0..15 -> [..., D/2] bytes (even channel in the low nibble)."""
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def unpack_pairs(codes):
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = codes & 0x0F
    out[..., 1::2] = codes >> 4
    return out


def keys_to_lib(q, sc, mn):
    return pack_pairs(q), sc, mn


def keys_from_lib(codes, sc, mn):
    return unpack_pairs(codes), sc, mn


def values_to_lib(q, sc, mn):
    """Plain value codes [B, H, S, D] and metadata [B, H, S, ng] -> the block
    layout."""
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
                p = nibble(e)
                codes[:, :, j, :, 4 * w + p // 2] |= (q[:, :, t, :] << (4 * (p % 2))).astype(np.uint8)
                bsc[:, :, j, :, 8 * w + e] = sc[:, :, t, :]
                bmn[:, :, j, :, 8 * w + e] = mn[:, :, t, :]
    return codes, bsc, bmn


def values_from_lib(codes, bsc, bmn, S):
    """Block layout of an S-token value cache -> plain codes [B, H, S, D] and
    metadata [B, H, S, ng]."""
    B, H, nb, D, _ = codes.shape
    ng = bsc.shape[3]
    q = np.zeros((B, H, nb * GROUP, D), dtype=np.uint8)
    s = np.zeros((B, H, nb * GROUP, ng), dtype=np.float16)
    m = np.zeros((B, H, nb * GROUP, ng), dtype=np.float16)
    for j in range(nb):
        for w in range(4):
            for e in range(8):
                t = j * GROUP + block_token(w, e)
                p = nibble(e)
                q[:, :, t, :] = (codes[:, :, j, :, 4 * w + p // 2] >> (4 * (p % 2))) & 0x0F
                s[:, :, t, :] = bsc[:, :, j, :, 8 * w + e]
                m[:, :, t, :] = bmn[:, :, j, :, 8 * w + e]
    return q[:, :, :S], s[:, :, :S], m[:, :, :S]


def padding_is_zero(codes, bsc, bmn, S):
    """True when every token of the last block at or past S has code,
    scale and minimum 0 (the header's padding rule)."""
    nb = codes.shape[2]
    ok = True
    for w in range(4):
        for e in range(8):
            t = (nb - 1) * GROUP + block_token(w, e)
            if t < S:
                continue
            p = nibble(e)
            ok &= bool(np.all(((codes[:, :, nb - 1, :, 4 * w + p // 2] >> (4 * (p % 2))) & 0x0F) == 0))
            ok &= bool(np.all(bsc[:, :, nb - 1, :, 8 * w + e] == 0)) and bool(np.all(bmn[:, :, nb - 1, :, 8 * w + e] == 0))
    return ok
