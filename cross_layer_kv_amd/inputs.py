"""Seeded synthetic inputs for FusedKV reconstruction-layer attention.

This module is the one place both the HIP path and the fp64 oracle take their
inputs from.  It holds no part of the method's arithmetic (no fusion, no
attention): only random draws, the rotary position embedding that turns raw
draws into post-RoPE keys and queries, and rounding to the storage dtype.

Pages cited (by title):
  [Deck]  "FusedKV: Reconstructing KV Caches with Cross-Layer Fusion"
  [Notes] "FusedKV:通过跨层融合重构 KV 缓存"

Recipe (the workloads are shaped like the pages' models; values are synthetic):
  * activations Q, K^1, K^n, V^1, V^n ~ N(0, 1), drawn in float32;
  * keys and queries are stored post-RoPE ([Deck] frame "Post-RoPE fusion needs
    paired key weights"; [Notes] section 2.4): keys rotated at their cache
    positions 0..S-1, a decode query at S-1, prefill queries at 0..S-1, with
    base 10000 ([Notes] section 3 gives the pre-training RoPE base).  The
    rotation angle pos * base^(-2j/D) and its cos/sin are formed in float64,
    then the rotated value is rounded once to the storage dtype;
  * RoPE pairs are either interleaved (2j, 2j+1) -- the papers' notation -- or
    half-split (j, j + D/2), the layout of Qwen3-style checkpoints;
  * fusion weights ~ N(0.5, 0.25) (std 0.25), float32.  Key weights are tied
    across both coordinates of each RoPE pair (one draw per (kv head, pair)),
    as the post-RoPE frame requires; value weights are drawn per channel;
  * bfloat16 values are the round-to-nearest-even image of the float32 draws.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

ROPE_BASE = 10000.0


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def rope_pairs(D: int, pairing: str):
    """Index arrays (first, second) of the RoPE rotation pairs of a head."""
    if D % 2:
        raise ValueError("head_dim must be even for RoPE")
    j = np.arange(D // 2)
    if pairing == "interleaved":
        return 2 * j, 2 * j + 1
    if pairing == "half":
        return j, j + D // 2
    raise ValueError("pairing is 'interleaved' or 'half'")


def rope_rotate(x: torch.Tensor, positions: torch.Tensor, base: float = ROPE_BASE,
                pairing: str = "interleaved") -> torch.Tensor:
    """Rotate x [..., S, H, D] (float64) at positions [S] (int64).

    Pair j of channels (u, w) at position p is turned by the angle
    p * base^(-2j/D): (u, w) -> (u cos - w sin, u sin + w cos).
    """
    D = x.shape[-1]
    i1, i2 = rope_pairs(D, pairing)
    j = torch.arange(D // 2, dtype=torch.float64, device=x.device)
    inv_freq = torch.pow(torch.tensor(base, dtype=torch.float64, device=x.device), -2.0 * j / D)
    ang = positions.to(torch.float64)[:, None] * inv_freq[None, :]          # [S, D/2]
    cos = torch.cos(ang)[:, None, :]                                          # [S, 1, D/2]
    sin = torch.sin(ang)[:, None, :]
    i1 = torch.as_tensor(i1, device=x.device)
    i2 = torch.as_tensor(i2, device=x.device)
    u = x[..., i1]
    w = x[..., i2]
    out = torch.empty_like(x)
    out[..., i1] = u * cos - w * sin
    out[..., i2] = u * sin + w * cos
    return out


def _store(x64: torch.Tensor, dtype: torch.dtype) -> torch.Tensor:
    return x64.to(torch.float32).to(dtype)


def _normal(shape, gen, device) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)


def make_cache(B: int, S: int, H: int, D: int, dtype: torch.dtype, seed: int, device="cpu",
               layout: str = "bhsd", rotate: bool = True, pairing: str = "interleaved",
               base: float = ROPE_BASE, chunk_elems: int = 1 << 27, pos0: int = 0) -> torch.Tensor:
    """One cache as a logical [B, S, H, D] tensor.

    layout 'bhsd' stores it head-major ([B, H, S, D] buffer, a permuted view is
    returned); 'bshd' stores it token-major.  Keys are rotated at positions
    pos0..pos0+S-1 when ``rotate`` (the raw draws do not depend on pos0).
    Generation runs in slices of the batch/head axes so the float64 temporary
    stays small.
    """
    gen = _gen(seed, device)
    if layout == "bhsd":
        buf = torch.empty(B, H, S, D, dtype=dtype, device=device)
    elif layout == "bshd":
        buf = torch.empty(B, S, H, D, dtype=dtype, device=device)
    else:
        raise ValueError("layout is 'bhsd' or 'bshd'")
    pos = torch.arange(S, dtype=torch.int64, device=device) + int(pos0)
    per_slice = max(1, chunk_elems // max(1, S * D))
    for b in range(B):
        for h0 in range(0, H, per_slice):
            h1 = min(H, h0 + per_slice)
            x = _normal((S, h1 - h0, D), gen, device).to(torch.float64)
            if rotate:
                x = rope_rotate(x, pos, base, pairing)
            x = _store(x, dtype)
            if layout == "bhsd":
                buf[b, h0:h1] = x.permute(1, 0, 2)
            else:
                buf[b, :, h0:h1] = x
    return buf.permute(0, 2, 1, 3) if layout == "bhsd" else buf


def make_queries(B: int, Sq: int, Hq: int, D: int, dtype: torch.dtype, seed: int, device="cpu",
                 positions=None, pairing: str = "interleaved", base: float = ROPE_BASE) -> torch.Tensor:
    """Contiguous [B, Sq, Hq, D] queries rotated at ``positions`` ([Sq] ints,
    default 0..Sq-1)."""
    gen = _gen(seed, device)
    if positions is None:
        positions = torch.arange(Sq, dtype=torch.int64)
    positions = torch.as_tensor(positions, dtype=torch.int64, device=device)
    out = torch.empty(B, Sq, Hq, D, dtype=dtype, device=device)
    for b in range(B):
        x = _normal((Sq, Hq, D), gen, device).to(torch.float64)
        out[b] = _store(rope_rotate(x, positions, base, pairing), dtype)
    return out


def make_grad_output(B: int, S: int, Hq: int, D: int, dtype: torch.dtype, seed: int, device="cpu",
                     std: float = 1.0) -> torch.Tensor:
    """Output gradient dO [B, S, Hq, D] for a backward call: N(0, std^2)
    draws (on the CPU generator, so that every device gets the same values),
    rounded to ``dtype``."""
    gen = _gen(seed, "cpu")
    x = std * _normal((B, S, Hq, D), gen, "cpu")
    return x.to(dtype).to(device)


def make_weights(Hkv: int, D: int, seed: int, pairing: str = "interleaved", tied: bool = True,
                 mean: float = 0.5, std: float = 0.25, device="cpu"):
    """Per-layer fusion vectors (a, a', b, b') as float32 [Hkv, D] tensors.

    Key weights get one draw per RoPE pair (both coordinates equal) unless
    ``tied`` is False; value weights are drawn per channel.
    """
    gen = _gen(seed, "cpu")
    i1, i2 = rope_pairs(D, pairing)

    def key_w():
        if not tied:
            return mean + std * torch.randn(Hkv, D, generator=gen, dtype=torch.float32)
        c = mean + std * torch.randn(Hkv, D // 2, generator=gen, dtype=torch.float32)
        w = torch.empty(Hkv, D, dtype=torch.float32)
        w[:, torch.as_tensor(i1)] = c
        w[:, torch.as_tensor(i2)] = c
        return w

    k_w1 = key_w()
    k_wn = key_w()
    v_w1 = mean + std * torch.randn(Hkv, D, generator=gen, dtype=torch.float32)
    v_wn = mean + std * torch.randn(Hkv, D, generator=gen, dtype=torch.float32)
    return tuple(w.to(device) for w in (k_w1, k_wn, v_w1, v_wn))


@dataclasses.dataclass
class LayerInputs:
    """Inputs of one reconstruction-layer call."""
    q: torch.Tensor                   # [B, Sq, Hq, D]
    k1: torch.Tensor                  # [B, Sk, Hkv, D] views
    kn: torch.Tensor
    v1: torch.Tensor
    vn: torch.Tensor
    weights: tuple                    # (k_w1, k_wn, v_w1, v_wn) float32 [Hkv, D]
    seqlens_k: torch.Tensor | None    # int32 [B] or None


def make_layer(B, Sq, Sk, Hq, Hkv, D, dtype, seed, device="cpu", layout="bhsd",
               pairing="interleaved", decode=True, seqlens_k=None, pos0=0, tied=True) -> LayerInputs:
    """A full set of inputs.  Seeds of the parts are derived from ``seed`` so
    that each part can also be regenerated on its own.  ``pos0`` shifts every
    position (keys at pos0..pos0+Sk-1, the decode query at pos0+Sk-1) while
    keeping the raw draws; ``tied`` False draws untied key weights."""
    k1 = make_cache(B, Sk, Hkv, D, dtype, seed * 16 + 1, device, layout, True, pairing, pos0=pos0)
    kn = make_cache(B, Sk, Hkv, D, dtype, seed * 16 + 2, device, layout, True, pairing, pos0=pos0)
    v1 = make_cache(B, Sk, Hkv, D, dtype, seed * 16 + 3, device, layout, False, pairing)
    vn = make_cache(B, Sk, Hkv, D, dtype, seed * 16 + 4, device, layout, False, pairing)
    qpos = torch.full((Sq,), Sk - 1, dtype=torch.int64) if decode else torch.arange(Sq)
    q = make_queries(B, Sq, Hq, D, dtype, seed * 16 + 5, device, qpos + int(pos0), pairing)
    w = make_weights(Hkv, D, seed * 16 + 6, pairing, tied=tied, device=device)
    sl = None
    if seqlens_k is not None:
        sl = torch.as_tensor(seqlens_k, dtype=torch.int32).to(device)
    return LayerInputs(q, k1, kn, v1, vn, w, sl)


def host_array(t: torch.Tensor) -> np.ndarray:
    """The stored values of a tensor as a host numpy array, keeping its
    strides: float32 stays float32, bfloat16 becomes its uint16 bit pattern."""
    if t.dtype == torch.bfloat16:
        base = t.detach().cpu()
        return base.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.detach().cpu().numpy()
    raise TypeError("stored values are float32 or bfloat16")


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact float32 image of bfloat16 bit patterns (for tests that need the
    stored values as numbers)."""
    return (a.astype(np.uint32) << 16).view(np.float32)
