"""GPU test of fkv_decode_noalloc, the decode entry point that takes no
workspace (split partials in the library's static per-GPU scratch), through
the C ABI: two calls in a row, the second with a smaller input, each equal to
fkv_decode with a caller workspace bit for bit (same plan, same kernels) and
within the bf16 tolerance of the fp64 oracle.  Prints its case before each
GPU step."""
import pytest
import torch

from cross_layer_kv_amd import binding, inputs
from parity import TOL, gpu_rows, lse_err, oracle_layer, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _both(L):
    B, _, Hq, D = L.q.shape
    need = binding.fkv_decode_workspace_size(binding.make_params(L.q, L.k1))
    assert 0 < need <= binding.NOALLOC_SCRATCH_BYTES
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    o_ws = torch.full_like(L.q, float("nan"))
    l_ws = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
    binding.fkv_decode(L.q, L.k1, L.kn, L.v1, L.vn, L.weights, out=o_ws, lse=l_ws, workspace=ws,
                       seqlens_k=L.seqlens_k)
    o_na = torch.full_like(L.q, float("nan"))
    l_na = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
    binding.fkv_decode_noalloc(L.q, L.k1, L.kn, L.v1, L.vn, L.weights, out=o_na, lse=l_na, seqlens_k=L.seqlens_k)
    torch.cuda.synchronize()
    return need, (o_ws, l_ws), (o_na, l_na)


def test_noalloc_decode_matches_workspace_decode_on_two_calls():
    cases = [
        # 16 (batch, KV head) units: the key axis is split into 16 parts
        dict(B=2, S=20000, Hq=16, Hkv=8, D=128, seed=0xA110C, seqlens=[20000, 13331]),
        # a smaller second call on the same scratch
        dict(B=1, S=3000, Hq=8, Hkv=4, D=96, seed=0xA110D, seqlens=None),
    ]
    for c in cases:
        say("noalloc decode B=%d S=%d Hq=%d Hkv=%d D=%d seqlens=%s" % (c["B"], c["S"], c["Hq"], c["Hkv"], c["D"],
                                                                      c["seqlens"]))
        L = inputs.make_layer(c["B"], 1, c["S"], c["Hq"], c["Hkv"], c["D"], torch.bfloat16, c["seed"], DEV,
                              seqlens_k=c["seqlens"])
        need, (o_ws, l_ws), (o_na, l_na) = _both(L)
        ro, rl = oracle_layer(L, fused=True)
        e = rel_err(gpu_rows(o_na, c["B"], c["Hq"], 1, c["D"]), ro)
        el = lse_err(l_na.cpu().numpy().reshape(-1), rl)
        say("  partials %d bytes; noalloc err=%.3e lse_err=%.3e; equal to workspace call: %s"
            % (need, e, el, torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws)))
        assert e <= TOL[torch.bfloat16] and el <= TOL[torch.bfloat16]
        assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws)


def test_noalloc_decode_refuses_plans_beyond_the_scratch():
    """64 query heads per KV head at batch 16, S = 32768: the partials need
    more than the static scratch, and the call is refused before launch."""
    say("noalloc decode: oversize plan refused (host check)")
    q = torch.zeros(16, 1, 128, 128, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(16, 32768, 2, 128, dtype=torch.bfloat16, device=DEV)
    w = [torch.zeros(2, 128, device=DEV) for _ in range(4)]
    assert binding.fkv_decode_workspace_size(binding.make_params(q, k)) > binding.NOALLOC_SCRATCH_BYTES
    with pytest.raises(binding.FkvError) as ei:
        binding.fkv_decode_noalloc(q, k, k, k, k, w, out=torch.empty_like(q))
    assert ei.value.status == binding.FKV_ERROR_WORKSPACE
