"""CPU tests of the test-side converter between the oracle's plain 4-bit
arrays and the library's packed storage (``tests/kivi_layout.py``,
``include/fusedkv.h``): round trips, the nibble order, and the value block
order checked on a hand-built cache."""
import numpy as np

import kivi_layout as kl
from oracle import kivi


def test_nibble_order():
    """Two codes per byte: channel 2i in the low nibble, 2i+1 in the high."""
    q = np.array([[1, 2, 15, 0, 7, 9]], np.uint8)
    assert list(kl.pack_pairs(q)[0]) == [0x21, 0x0F, 0x97]
    assert np.array_equal(kl.unpack_pairs(kl.pack_pairs(q)), q)


def test_round_trips():
    rng = np.random.default_rng(7)
    B, S, H, D = 2, 75, 3, 80
    x = rng.standard_normal((B, S, H, D)).astype(np.float32)
    kq = kivi.quantise_keys(x)
    back = kl.keys_from_lib(*kl.keys_to_lib(*kq))
    assert all(np.array_equal(a, b) for a, b in zip(kq, back))
    vq = kivi.quantise_values(x)
    lib = kl.values_to_lib(*vq)
    assert lib[0].shape == (B, H, 3, D, 16) and lib[1].shape == (B, H, 3, 3, 32)
    assert kl.padding_is_zero(*lib, S)
    back = kl.values_from_lib(*lib, S)
    assert all(np.array_equal(a, b) for a, b in zip(vq, back))


def test_value_block_layout():
    """Value codes are channel-major per 32-token block: word w of (block,
    channel) holds tokens 4w + e%4 + 16(e//4), element e in nibble e//2 (even
    e) or 4 + e//2 (odd e); metadata lists the tokens in the same order.
    Built by hand for single marked tokens, a 37-token cache (one full block
    and a 5-token tail whose padding is zero)."""
    B, S, H, D = 1, 37, 1, 32
    x = np.zeros((B, S, H, D), np.float32)
    x[0, 15, 0, :] = np.arange(D) * 0.5      # token 15: codes 0..15 ramp over 32 channels
    x[0, 33, 0, :] = -np.arange(D) * 0.25    # token 33: codes 15..0
    codes, sc, mn = kl.values_to_lib(*kivi.quantise_values(x))
    assert codes.shape == (1, 1, 2, D, 16) and sc.shape == (1, 1, 2, 1, 32)
    # token 15 = 4w + e%4 + 16(e//4) with w = 3, e = 3 -> nibble 4 + 1 = 5 of
    # word 3 -> byte 12 + 2, high half; its code at channel c is rint(c / 2 * 15 / 15.5)
    q15 = np.rint(np.arange(D) * 0.5 / np.float32(15.5 / 15)).clip(0, 15)
    got = (codes[0, 0, 0, :, 14] >> 4) & 0xF
    assert np.array_equal(got, q15.astype(np.uint8))
    assert sc[0, 0, 0, 0, 8 * 3 + 3] == np.float16(15.5 / 15) and sc[0, 0, 0, 0, 0] == 0
    # token 33 -> block 1, position 1 = (w 0, e 1): nibble 4 of word 0 -> byte 2, low half
    got33 = codes[0, 0, 1, :, 2] & 0xF
    assert got33[0] == 15 and got33[-1] == 0
    # padding tokens (37..63) have zero codes and metadata
    assert kl.padding_is_zero(codes, sc, mn, S)
    assert np.all(sc[0, 0, 1, 0, [8 * w + e for w in range(4) for e in range(8)
                                   if 32 + kl.block_token(w, e) >= S]] == 0)
