"""GPU tests of fkv_store_kv, the storage-layer cache write, through the C
ABI: the written positions hold the new rows bit for bit (the definition of
the write, checked on the host), every other position keeps its previous
bytes, and a storage-layer prefill over the written caches is bitwise the
prefill over the same rows read in place.  Every test prints its case
before touching the GPU."""
import numpy as np
import pytest
import torch

from cross_layer_kv_amd import binding, inputs
from parity import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bits(t):
    """Stored bytes of a tensor as an integer numpy array (bit-exact compare)."""
    t = t.detach().contiguous().cpu()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


def _case(B, Sn, S, H, D, pos0, dtype, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    kn = torch.randn(B, Sn, H, D, generator=g).to(dtype).to(DEV)          # token-major new rows
    vn = torch.randn(B, Sn, H, D, generator=g).to(dtype).to(DEV)
    # head-major caches filled with a sentinel pattern that the write must keep
    kc = torch.full((B, H, S, D), -7.5, dtype=dtype, device=DEV).transpose(1, 2)
    vc = torch.full((B, H, S, D), 3.25, dtype=dtype, device=DEV).transpose(1, 2)
    return kn, vn, kc, vc


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [64, 80, 96, 128])
def test_written_rows_and_untouched_rest(dtype, D):
    B, Sn, S, H, pos0 = 2, 173, 300, 3, 50
    say("store_kv dtype=%s D=%d B=%d S_new=%d S=%d H=%d pos0=%d" % (dtype, D, B, Sn, S, H, pos0))
    kn, vn, kc, vc = _case(B, Sn, S, H, D, pos0, dtype, 11 + D)
    before_k, before_v = _bits(kc), _bits(vc)
    binding.fkv_store_kv(kn, vn, kc, vc, pos0=pos0)
    torch.cuda.synchronize()
    for new, cache, before in ((kn, kc, before_k), (vn, vc, before_v)):
        want = before.copy()
        want[:, pos0:pos0 + Sn] = _bits(new)       # the definition: a slice assignment
        assert np.array_equal(_bits(cache), want)


def test_decode_append_and_empty_write():
    B, S, H, D = 3, 64, 2, 128
    say("store_kv append: one token at position S-1, then an empty write")
    kn, vn, kc, vc = _case(B, 1, S, H, D, S - 1, torch.bfloat16, 5)
    before = _bits(kc)
    binding.fkv_store_kv(kn, vn, kc, vc, pos0=S - 1)
    binding.fkv_store_kv(kn[:, :0], vn[:, :0], kc, vc, pos0=S)
    torch.cuda.synchronize()
    want = before.copy()
    want[:, S - 1:] = _bits(kn)
    assert np.array_equal(_bits(kc), want)
    assert np.array_equal(_bits(vc)[:, S - 1:], _bits(vn))


def test_storage_prefill_over_written_caches_is_bitwise_in_place():
    """1.5B-shape storage layer, 8192-token prompt: write the caches, then
    the plain (single-source) prefill over them equals the same prefill over
    the new rows read in place (same values, different strides)."""
    B, S, Hq, Hkv, D = 1, 8192, 16, 8, 128
    say("store_kv + storage-layer prefill B=%d S=%d %d/%d heads D=%d" % (B, S, Hq, Hkv, D))
    k = inputs.make_cache(B, S, Hkv, D, torch.bfloat16, 91, DEV, layout="bshd")
    v = inputs.make_cache(B, S, Hkv, D, torch.bfloat16, 92, DEV, layout="bshd", rotate=False)
    q = inputs.make_queries(B, S, Hq, D, torch.bfloat16, 93, DEV)
    kc = torch.empty(B, Hkv, S, D, dtype=torch.bfloat16, device=DEV).transpose(1, 2)
    vc = torch.empty_like(kc)
    binding.fkv_store_kv(k, v, kc, vc)
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    binding.fkv_lite_prefill(q, kc, vc, out=o1, causal=True)
    binding.fkv_lite_prefill(q, k, v, out=o2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(kc, k) and torch.equal(vc, v)
    assert torch.equal(o1, o2)
