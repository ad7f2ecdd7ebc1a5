"""CPU tests of the C ABI: the library loads, exports every declared entry
point, and rejects invalid calls on the host before anything is enqueued.
No call here reaches a kernel launch (each one fails validation, or has an
empty batch)."""
import ctypes
import math
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fusedkv.h")


@pytest.fixture(scope="module")
def lib():
    from cross_layer_kv_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from cross_layer_kv_amd import build
        build.build()
    return binding.load_library()


@pytest.fixture(scope="module")
def B():
    from cross_layer_kv_amd import binding
    return binding


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fkv_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib, B):
    names = declared_functions()
    assert set(names) == set(B.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.fkv_abi_version() == B.ABI_VERSION == 7
    for s in range(5):
        assert lib.fkv_status_string(s)
    assert lib.fkv_status_string(99) == b"unknown status"


FAKE = 0x10000  # 16-byte aligned host value; never dereferenced


def _params(B, batch=2, sq=1, sk=64, hq=4, hkv=2, d=64, dtype=1, scale=0.0, causal=0):
    return B.fkv_params(batch, sq, sk, hq, hkv, d, dtype, scale, causal)


def _cache(B, d=64, hkv=2, sk=64, ptr=FAKE):
    return B.fkv_cache(ptr, hkv * sk * d, d, sk * d)


def _fusion(B, ptr=FAKE):
    return B.fkv_fusion(ptr, ptr + 256, ptr + 512, ptr + 768)


def _decode(lib, B, p, q=FAKE, caches=None, fusion="default", ws_bytes=None, ws=FAKE, seqlens=None, lse=None,
            out=FAKE):
    c = caches or [_cache(B, p.head_dim, p.num_kv_heads, p.seqlen_k)] * 4
    f = _fusion(B) if fusion == "default" else fusion
    if ws_bytes is None:
        ws_bytes = lib.fkv_decode_workspace_size(ctypes.byref(p)) if p else 0
    return lib.fkv_decode(ctypes.byref(p) if p else None, q, c[0], c[1], c[2], c[3],
                          ctypes.byref(f) if f is not None else None, seqlens, out, lse, ws, ws_bytes, None)


def _prefill(lib, B, p, q=FAKE, caches=None, fusion="default"):
    c = caches or [_cache(B, p.head_dim, p.num_kv_heads, p.seqlen_k)] * 4
    f = _fusion(B) if fusion == "default" else fusion
    return lib.fkv_prefill(ctypes.byref(p), q, c[0], c[1], c[2], c[3],
                           ctypes.byref(f) if f is not None else None, FAKE, None, None)


def test_decode_validation_codes(lib, B):
    INV, UNS, WS = B.FKV_ERROR_INVALID_VALUE, B.FKV_ERROR_UNSUPPORTED, B.FKV_ERROR_WORKSPACE
    assert lib.fkv_decode(None, FAKE, _cache(B), _cache(B), _cache(B), _cache(B), None, None, FAKE, None,
                          FAKE, 1 << 20, None) == INV
    assert lib.fkv_last_error()
    assert _decode(lib, B, _params(B, hq=5, hkv=2)) == INV
    assert _decode(lib, B, _params(B, d=72)) == UNS
    assert _decode(lib, B, _params(B, hq=6, hkv=2)) == UNS        # G = 3
    assert _decode(lib, B, _params(B, sq=2)) == INV
    assert _decode(lib, B, _params(B, dtype=7)) == INV
    assert _decode(lib, B, _params(B, scale=-1.0)) == INV
    assert _decode(lib, B, _params(B, scale=float("nan"))) == INV
    assert _decode(lib, B, _params(B, batch=-1)) == INV
    assert _decode(lib, B, _params(B), q=FAKE + 8) == INV           # misaligned q
    assert _decode(lib, B, _params(B), out=0) == INV
    assert _decode(lib, B, _params(B), fusion=None) == INV
    assert _decode(lib, B, _params(B), fusion=B.fkv_fusion(FAKE, 0, FAKE, FAKE)) == INV
    assert _decode(lib, B, _params(B), lse=FAKE + 2) == INV
    bad = B.fkv_cache(FAKE, 2 * 64 * 64, 60, 64 * 64)             # row stride breaks alignment
    assert _decode(lib, B, _params(B), caches=[bad] * 4) == INV
    overlap = B.fkv_cache(FAKE, 2 * 64 * 64, 32, 64 * 64)         # token stride < D
    assert _decode(lib, B, _params(B), caches=[overlap] * 4) == INV
    assert _decode(lib, B, _params(B), caches=[B.fkv_cache(0, 0, 64, 0)] * 4) == INV
    # a NULL cache is accepted only when it holds no tokens (it is never read)
    assert _decode(lib, B, _params(B, batch=0, sk=0), caches=[B.fkv_cache(0, 0, 64, 0)] * 4) == B.FKV_SUCCESS
    p = _params(B, sk=8192)   # 4 (batch, kv head) units: the key axis is split, a workspace is needed
    need = lib.fkv_decode_workspace_size(ctypes.byref(p))
    assert need > 0
    assert _decode(lib, B, p, ws_bytes=need - 1) == WS
    assert _decode(lib, B, p, ws=0) == WS
    assert _decode(lib, B, p, ws=FAKE + 16) == WS                  # not 256-byte aligned
    # an empty batch is a valid no-op: nothing is launched
    assert _decode(lib, B, _params(B, batch=0)) == B.FKV_SUCCESS
    assert lib.fkv_last_error() == b""
    # G = 64 runs on the matrix cores: bfloat16 only; G = 32 is not served
    assert _decode(lib, B, _params(B, hq=128, hkv=2, dtype=0)) == UNS
    assert _decode(lib, B, _params(B, hq=64, hkv=2)) == UNS


def _q4(B, ptr=FAKE):
    return B.fkv_q4_cache(ptr, ptr, ptr)


def _kivi_decode(lib, B, p, q=FAKE, caches=None, fusion="ok", out=FAKE, ws=FAKE, ws_bytes=1 << 24, lite=False):
    caches = caches or [_q4(B)] * 4
    if lite:
        return lib.fkv_kivi_lite_decode(ctypes.byref(p), q, caches[0], caches[1], None, out, None, ws, ws_bytes,
                                        None)
    f = _fusion(B) if fusion == "ok" else fusion
    return lib.fkv_kivi_decode(ctypes.byref(p), q, *caches, ctypes.byref(f) if f is not None else None, None, out,
                               None, ws, ws_bytes, None)


def test_kivi_validation_codes(lib, B):
    INV, UNS, WS = B.FKV_ERROR_INVALID_VALUE, B.FKV_ERROR_UNSUPPORTED, B.FKV_ERROR_WORKSPACE
    assert _kivi_decode(lib, B, _params(B, dtype=0)) == UNS                 # f32 queries
    assert _kivi_decode(lib, B, _params(B, hq=128, hkv=2)) == UNS           # G = 64
    assert _kivi_decode(lib, B, _params(B, hq=6, hkv=2)) == UNS             # G = 3
    assert _kivi_decode(lib, B, _params(B, d=72)) == UNS
    assert _kivi_decode(lib, B, _params(B, sq=2)) == INV
    assert _kivi_decode(lib, B, _params(B), fusion=None) == INV
    assert _kivi_decode(lib, B, _params(B), q=FAKE + 8) == INV
    assert _kivi_decode(lib, B, _params(B), caches=[B.fkv_q4_cache(FAKE, 0, FAKE)] * 4) == INV
    assert _kivi_decode(lib, B, _params(B), caches=[B.fkv_q4_cache(FAKE, FAKE + 2, FAKE)] * 4) == INV
    assert _kivi_decode(lib, B, _params(B, sq=2), lite=True) == INV
    assert _kivi_decode(lib, B, _params(B, batch=0)) == B.FKV_SUCCESS
    assert _kivi_decode(lib, B, _params(B, batch=0), lite=True) == B.FKV_SUCCESS
    # the workspace size is the largest of the decode plans; here the bf16
    # four-source plan (16-wave workgroups of 8-token wave steps, 128-token
    # workgroup steps: 64 splits of 128 tokens) needs more than the 4-bit
    # plans, which are checked exactly:
    # four-source 12 waves x 32-token blocks (22 splits of 384 tokens),
    # single-source 16 waves x 32-token blocks (16 splits of 512 tokens)
    p = _params(B, sk=8192)
    need = lib.fkv_decode_workspace_size(ctypes.byref(p))
    ws = lambda units, ns, G, D: math.ceil(units * ns * G * 2 * 4 / 256) * 256 + units * ns * G * D * 4
    assert need == ws(4, 64, 2, 64)
    assert _kivi_decode(lib, B, p, ws_bytes=ws(4, 22, 2, 64) - 1) == WS
    assert _kivi_decode(lib, B, p, ws_bytes=ws(4, 16, 2, 64) - 1, lite=True) == WS
    assert _kivi_decode(lib, B, p, ws=FAKE + 16) == WS
    # quantiser: bfloat16 source only, is_value 0 or 1, an empty cache is a no-op
    c = _cache(B)
    p = _params(B)
    assert lib.fkv_kivi_quantize(ctypes.byref(_params(B, dtype=0)), c, 0, _q4(B), None) == UNS
    assert lib.fkv_kivi_quantize(ctypes.byref(p), c, 2, _q4(B), None) == INV
    assert lib.fkv_kivi_quantize(ctypes.byref(p), c, 0, B.fkv_q4_cache(FAKE, None, FAKE), None) == INV
    assert lib.fkv_kivi_quantize(ctypes.byref(_params(B, sk=0)), c, 1, _q4(B, 0), None) == B.FKV_SUCCESS
    # array sizes: key codes D/2 bytes per token; key metadata per 32-token
    # group and channel (fp16)
    p = _params(B, batch=3, sk=100, hkv=2, hq=4, d=80)
    assert lib.fkv_kivi_codes_bytes(ctypes.byref(p), 0) == 3 * 2 * 100 * 40
    # values: 4 blocks of 32 tokens x 80 channels x 16 bytes; metadata per
    # (block, 32-channel group) lists 32 tokens
    assert lib.fkv_kivi_codes_bytes(ctypes.byref(p), 1) == 3 * 2 * 4 * 80 * 16
    assert lib.fkv_kivi_meta_bytes(ctypes.byref(p), 0) == 3 * 2 * 4 * 80 * 2
    assert lib.fkv_kivi_meta_bytes(ctypes.byref(p), 1) == 3 * 2 * 4 * 3 * 32 * 2


def test_lite_decode_validation_codes(lib, B):
    p = _params(B, sq=3)
    c = _cache(B)
    assert lib.fkv_lite_decode(ctypes.byref(p), FAKE, c, c, None, FAKE, None, FAKE, 1 << 20, None) == \
        B.FKV_ERROR_INVALID_VALUE
    p = _params(B, batch=0)
    assert lib.fkv_lite_decode(ctypes.byref(p), FAKE, c, c, None, FAKE, None, FAKE, 0, None) == B.FKV_SUCCESS


def test_prefill_validation_codes(lib, B):
    INV, UNS = B.FKV_ERROR_INVALID_VALUE, B.FKV_ERROR_UNSUPPORTED
    assert _prefill(lib, B, _params(B, sq=64, sk=64, dtype=0)) == UNS   # f32 prefill
    assert _prefill(lib, B, _params(B, sq=32, sk=64)) == UNS            # S_q != S_k
    assert _prefill(lib, B, _params(B, sq=64, sk=64, causal=2)) == INV
    assert _prefill(lib, B, _params(B, sq=64, sk=64, d=100)) == UNS
    assert _prefill(lib, B, _params(B, sq=64, sk=64), fusion=None) == INV
    assert _prefill(lib, B, _params(B, sq=64, sk=64), q=FAKE + 4) == INV
    assert _prefill(lib, B, _params(B, batch=0, sq=64, sk=64)) == B.FKV_SUCCESS
    assert _prefill(lib, B, _params(B, sq=0, sk=0)) == B.FKV_SUCCESS
    assert _prefill(lib, B, _params(B, sq=64, sk=64, hq=128, hkv=2)) == UNS  # G = 64: decode only
    p = _params(B, sq=64, sk=64)
    c = _cache(B)
    assert lib.fkv_lite_prefill(ctypes.byref(p), FAKE, c, B.fkv_cache(0, 0, 64, 0), FAKE, None, None) == INV
    assert lib.fkv_lite_prefill(ctypes.byref(p), FAKE + 8, c, c, FAKE, None, None) == INV
    # an empty prompt launches nothing
    assert lib.fkv_lite_prefill(ctypes.byref(_params(B, batch=0, sq=64, sk=64)), FAKE, c, c, FAKE, None,
                                None) == B.FKV_SUCCESS


def _grad(B, d=64, hkv=2, sk=64, ptr=FAKE):
    return B.fkv_grad(ptr, hkv * sk * d, d, sk * d)


def _bwd(lib, B, p, q=FAKE, fusion="ok", dfusion="ok", grads=None, ws=FAKE, ws_bytes=1 << 26, lse=FAKE, lite=False):
    c = _cache(B)
    g = grads or [_grad(B)] * 4
    if lite:
        return lib.fkv_lite_prefill_backward(ctypes.byref(p), q, c, c, FAKE, lse, FAKE, FAKE, g[0], g[1], ws,
                                             ws_bytes, None)
    f = _fusion(B) if fusion == "ok" else fusion
    df = B.fkv_fusion_grad(FAKE, FAKE, FAKE, FAKE) if dfusion == "ok" else dfusion
    return lib.fkv_prefill_backward(ctypes.byref(p), q, c, c, c, c, ctypes.byref(f) if f is not None else None,
                                    FAKE, lse, FAKE, FAKE, *g, ctypes.byref(df) if df is not None else None, ws,
                                    ws_bytes, None)


def test_backward_validation_codes(lib, B):
    INV, UNS, WS = B.FKV_ERROR_INVALID_VALUE, B.FKV_ERROR_UNSUPPORTED, B.FKV_ERROR_WORKSPACE
    ok = dict(sq=64, sk=64)
    assert _bwd(lib, B, _params(B, dtype=0, **ok)) == UNS                 # f32
    assert _bwd(lib, B, _params(B, sq=32, sk=64)) == UNS                  # S_q != S_k
    assert _bwd(lib, B, _params(B, hq=128, hkv=2, **ok)) == UNS           # G = 64
    assert _bwd(lib, B, _params(B, causal=2, **ok)) == INV
    assert _bwd(lib, B, _params(B, d=100, **ok)) == UNS
    assert _bwd(lib, B, _params(B, **ok), fusion=None) == INV
    assert _bwd(lib, B, _params(B, **ok), dfusion=None) == INV
    assert _bwd(lib, B, _params(B, **ok), dfusion=B.fkv_fusion_grad(FAKE, FAKE + 2, FAKE, FAKE)) == INV
    assert _bwd(lib, B, _params(B, **ok), q=FAKE + 4) == INV
    assert _bwd(lib, B, _params(B, **ok), lse=None) == INV
    assert _bwd(lib, B, _params(B, **ok), grads=[_grad(B, ptr=0)] * 4) == INV
    assert _bwd(lib, B, _params(B, **ok), grads=[B.fkv_grad(FAKE, 2 * 64 * 64, 60, 64 * 64)] * 4) == INV
    p = _params(B, **ok)
    need = lib.fkv_backward_workspace_size(ctypes.byref(p))
    # LSE*log2(e) and rowsum(dO*O) rows (B*Hq*S floats each, 256-byte
    # rounded) and the weight-gradient partials (B*Hkv key tiles x 4 x D);
    # no fused rows are stored
    rows = 2 * 4 * 64 * 4
    assert need == 2 * (-(-rows // 256) * 256) + 2 * 2 * 1 * 4 * 64 * 4
    assert _bwd(lib, B, p, ws_bytes=need - 1) == WS
    assert _bwd(lib, B, p, ws=FAKE + 64) == WS
    assert _bwd(lib, B, p, ws=None) == WS
    assert _bwd(lib, B, _params(B, sq=2, sk=64), lite=True) == UNS
    assert _bwd(lib, B, _params(B, batch=0, **ok)) == B.FKV_SUCCESS
    assert _bwd(lib, B, _params(B, sq=0, sk=0)) == B.FKV_SUCCESS
    assert _bwd(lib, B, _params(B, batch=0, **ok), lite=True) == B.FKV_SUCCESS
    assert lib.fkv_backward_workspace_size(ctypes.byref(_params(B, sq=1, sk=64))) == 0
    assert lib.fkv_backward_workspace_size(None) == 0


def test_workspace_size(lib, B):
    assert lib.fkv_decode_workspace_size(None) == 0
    p = _params(B, sq=2)
    assert lib.fkv_decode_workspace_size(ctypes.byref(p)) == 0
    # 650M-shape decode: 32 x 8 = 256 (batch, kv head) units fill the chip with
    # one workgroup each (the 4-bit single-source kernel too, with 16-wave
    # workgroups up to D = 96), so no plan splits the keys
    p = _params(B, batch=32, sk=8192, hq=16, hkv=8, d=96)
    assert lib.fkv_decode_workspace_size(ctypes.byref(p)) == 0
    # at D = 128 the 4-bit single-source kernel keeps 8-wave workgroups and
    # aims at two per CU: 2 splits of 4096 tokens
    p = _params(B, batch=32, sk=8192, hq=16, hkv=8, d=128)
    units, ns, G, D = 256, 2, 2, 128
    assert lib.fkv_decode_workspace_size(ctypes.byref(p)) == \
        math.ceil(units * ns * G * 2 * 4 / 256) * 256 + units * ns * G * D * 4
    # long context, batch 1: 8 units; the bf16 plans take 32 splits of 4096
    # tokens, the 4-bit single-source plan 64 splits of 2048 (the largest)
    p = _params(B, batch=1, sk=131072, hq=16, hkv=8, d=128)
    units, ns, G, D = 8, 64, 2, 128
    expect = math.ceil(units * ns * G * 2 * 4 / 256) * 256 + units * ns * G * D * 4
    assert lib.fkv_decode_workspace_size(ctypes.byref(p)) == expect
    # G = 64 (matrix-core decode) aims at 512 workgroups of 64-token tiles:
    # 32 units x 16 splits of 2048 tokens, D = 128
    p = _params(B, batch=16, sk=32768, hq=128, hkv=2, d=128)
    units, ns, G, D = 32, 16, 64, 128
    expect = math.ceil(units * ns * G * 2 * 4 / 256) * 256 + units * ns * G * D * 4
    assert lib.fkv_decode_workspace_size(ctypes.byref(p)) == expect
    # an empty cache needs no workspace
    p = _params(B, sk=0)
    assert lib.fkv_decode_workspace_size(ctypes.byref(p)) == 0


def test_check_tied(lib, B):
    from cross_layer_kv_amd import inputs
    for pairing in ("interleaved", "half"):
        kw1, kwn, vw1, _ = inputs.make_weights(3, 16, 1, pairing=pairing)
        assert B.fkv_check_tied(kw1, pairing)
        assert B.fkv_check_tied(kwn, pairing)
        assert not B.fkv_check_tied(vw1, pairing)
    kw1, _, _, _ = inputs.make_weights(2, 8, 2, pairing="half")
    assert not B.fkv_check_tied(kw1, "interleaved")
    w = torch.ones(2, 8)
    w[1, 3] += 1e-3
    assert not B.fkv_check_tied(w, "interleaved", 1e-4)
    assert B.fkv_check_tied(w, "interleaved", 1e-2)
    assert lib.fkv_check_tied(None, 2, 8, 0, 0.0) == B.FKV_ERROR_INVALID_VALUE
    assert lib.fkv_check_tied(ctypes.c_void_p(w.data_ptr()), 2, 7, 0, 0.0) == B.FKV_ERROR_INVALID_VALUE


def test_binding_refuses_host_tensors(B):
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    w = [torch.zeros(2, 64)] * 4
    with pytest.raises(TypeError):
        B.fkv_decode(q, k, k, k, k, w, out=q, workspace=torch.zeros(4096, dtype=torch.uint8))


# ---- the binding compares tensors with each other before any pointer is
# handed to the library (shape, dtype, contiguity, extent); these run on host
# tensors and must fail with ValueError / TypeError before the device check ----

def _host_decode_args(Hq=4, Hkv=2, D=64, Sk=16, Bt=2, dtype=torch.bfloat16):
    q = torch.zeros(Bt, 1, Hq, D, dtype=dtype)
    caches = [torch.zeros(Bt, Sk, Hkv, D, dtype=dtype) for _ in range(4)]
    w = [torch.zeros(Hkv, D) for _ in range(4)]
    return q, caches, w


def test_binding_refuses_mismatched_decode_tensors(B):
    q, c, w = _host_decode_args()
    ws = torch.zeros(4096, dtype=torch.uint8)

    def call(**kw):
        args = dict(q=q, k1=c[0], kn=c[1], v1=c[2], vn=c[3], weights=w, out=torch.zeros_like(q), workspace=ws)
        args.update(kw)
        B.fkv_decode(args.pop("q"), args.pop("k1"), args.pop("kn"), args.pop("v1"), args.pop("vn"),
                     args.pop("weights"), **args)

    bad = [
        dict(kn=torch.zeros(2, 8, 2, 64, dtype=torch.bfloat16)),            # kn shorter than k1
        dict(vn=torch.zeros(2, 16, 1, 64, dtype=torch.bfloat16)),           # other head count
        dict(v1=torch.zeros(3, 16, 2, 64, dtype=torch.bfloat16)),           # other batch
        dict(k1=torch.zeros(2, 16, 2, 64, dtype=torch.float32)),            # f32 cache, bf16 q
        dict(k1=torch.zeros(2, 16, 64, 2, dtype=torch.bfloat16).transpose(2, 3)),  # strided channels
        dict(weights=[torch.zeros(2, 32)] * 4),                             # weights not [Hkv, D]
        dict(weights=[torch.zeros(2, 64, dtype=torch.float64)] * 4),        # weights not float32
        dict(weights=[torch.zeros(2, 64)] * 3),                             # three weights
        dict(out=torch.zeros(2, 1, 2, 64, dtype=torch.bfloat16)),           # out smaller than q
        dict(out=torch.zeros(2, 1, 4, 64, dtype=torch.float32)),            # out dtype
        dict(q=torch.zeros(2, 1, 64, 4, dtype=torch.bfloat16).transpose(2, 3)),    # non-contiguous q
        dict(q=torch.zeros(2, 2, 4, 64, dtype=torch.bfloat16)),             # two query rows
        dict(q=torch.zeros(2, 1, 5, 64, dtype=torch.bfloat16), out=torch.zeros(2, 1, 5, 64, dtype=torch.bfloat16)),
        dict(lse=torch.zeros(2, 3)),                                        # lse smaller than B*Hq
        dict(lse=torch.zeros(2, 4, dtype=torch.float64)),                   # lse dtype
        dict(seqlens_k=torch.zeros(3, dtype=torch.int32)),                  # one length per batch row
        dict(seqlens_k=torch.zeros(2, dtype=torch.int64)),
        dict(workspace=torch.zeros(1024, dtype=torch.float32)),
    ]
    for kw in bad:
        with pytest.raises((ValueError, TypeError)) as ei:
            call(**kw)
        assert "GPU tensor" not in str(ei.value), kw
    # consistent host tensors pass every comparison and stop at the device check
    with pytest.raises(TypeError, match="GPU tensor"):
        call(lse=torch.zeros(2, 4), seqlens_k=torch.zeros(2, dtype=torch.int32))


def test_binding_refuses_mismatched_prefill_tensors(B):
    Bt, S, Hq, Hkv, D = 1, 32, 4, 2, 64
    q = torch.zeros(Bt, S, Hq, D, dtype=torch.bfloat16)
    c = [torch.zeros(Bt, S, Hkv, D, dtype=torch.bfloat16) for _ in range(4)]
    w = [torch.zeros(Hkv, D) for _ in range(4)]
    bad = [
        dict(k1=torch.zeros(Bt, S - 1, Hkv, D, dtype=torch.bfloat16)),      # S_k != S_q
        dict(lse=torch.zeros(Bt, Hq, S - 1)),                               # lse smaller than B*Hq*S
        dict(out=torch.zeros(Bt, S, Hq, D - 8, dtype=torch.bfloat16)),
    ]
    for kw in bad:
        args = dict(k1=c[0], kn=c[1], v1=c[2], vn=c[3], out=torch.zeros_like(q), lse=None)
        args.update(kw)
        with pytest.raises((ValueError, TypeError)) as ei:
            B.fkv_prefill(q, args["k1"], args["kn"], args["v1"], args["vn"], w, out=args["out"], lse=args["lse"])
        assert "GPU tensor" not in str(ei.value), kw
    with pytest.raises(ValueError):
        B.fkv_lite_prefill(q, c[0], torch.zeros(Bt, S, 1, D, dtype=torch.bfloat16), out=torch.zeros_like(q))
    with pytest.raises(TypeError, match="GPU tensor"):
        B.fkv_prefill(q, *c, w, out=torch.zeros_like(q), lse=torch.zeros(Bt, Hq, S))


def test_binding_refuses_mismatched_backward_tensors(B):
    Bt, S, Hq, Hkv, D = 1, 32, 4, 2, 64
    q = torch.zeros(Bt, S, Hq, D, dtype=torch.bfloat16)
    c = [torch.zeros(Bt, S, Hkv, D, dtype=torch.bfloat16) for _ in range(4)]
    w = [torch.zeros(Hkv, D) for _ in range(4)]
    lse = torch.zeros(Bt, Hq, S)
    ws = torch.zeros(4096, dtype=torch.uint8)

    def call(**kw):
        a = dict(dq=torch.zeros_like(q), dk1=torch.zeros_like(c[0]), dkn=torch.zeros_like(c[1]),
                 dv1=torch.zeros_like(c[2]), dvn=torch.zeros_like(c[3]), dweights=[torch.zeros(Hkv, D)] * 4,
                 lse=lse, dout=torch.zeros_like(q))
        a.update(kw)
        B.fkv_prefill_backward(q, *c, w, torch.zeros_like(q), a.pop("lse"), a.pop("dout"), workspace=ws, **a)

    bad = [dict(dq=torch.zeros(Bt, S, Hq, D, dtype=torch.float32)), dict(dout=torch.zeros(Bt, S - 1, Hq, D,
                                                                                          dtype=torch.bfloat16)),
           dict(dk1=torch.zeros(Bt, S, Hkv, D // 2, dtype=torch.bfloat16)), dict(lse=torch.zeros(Bt, Hq)),
           dict(dweights=[torch.zeros(Hkv, D - 1)] * 4), dict(lse=None)]
    for kw in bad:
        with pytest.raises((ValueError, TypeError)) as ei:
            call(**kw)
        assert "GPU tensor" not in str(ei.value), kw
    with pytest.raises(TypeError, match="GPU tensor"):
        call()


def test_binding_refuses_mismatched_kivi_tensors(B):
    Bt, S, Hq, Hkv, D = 2, 40, 4, 2, 64
    q = torch.zeros(Bt, 1, Hq, D, dtype=torch.bfloat16)
    keys = [B.kivi_empty(Bt, S, Hkv, D, False, "cpu") for _ in range(2)]
    vals = [B.kivi_empty(Bt, S, Hkv, D, True, "cpu") for _ in range(2)]
    w = [torch.zeros(Hkv, D) for _ in range(4)]
    ws = torch.zeros(4096, dtype=torch.uint8)
    cases = [
        (keys[0], keys[1], vals[0], B.kivi_empty(Bt, S + 64, Hkv, D, True, "cpu")),   # value blocks differ
        (keys[0], B.kivi_empty(Bt, S - 1, Hkv, D, False, "cpu"), vals[0], vals[1]),   # key tokens differ
        (keys[0], keys[1], keys[0], vals[1]),                                        # key cache as values
        (keys[0], keys[1], vals[0], B.kivi_empty(Bt, S, Hkv + 1, D, True, "cpu")),   # head count
    ]
    for k1, kn, v1, vn in cases:
        with pytest.raises((ValueError, TypeError)) as ei:
            B.fkv_kivi_decode(q, k1, kn, v1, vn, w, out=torch.zeros_like(q), workspace=ws)
        assert "GPU tensor" not in str(ei.value)
    with pytest.raises(TypeError, match="GPU tensor"):
        B.fkv_kivi_decode(q, keys[0], keys[1], vals[0], vals[1], w, out=torch.zeros_like(q), workspace=ws)


def test_store_kv_validation_codes(lib, B):
    INV = B.FKV_ERROR_INVALID_VALUE

    def store(p, pos0=0, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, new_stride_s=None):
        if p is None:
            c = B.fkv_cache(FAKE, 0, 64, 0)
            return lib.fkv_store_kv(None, 0, c, c, B.fkv_grad(FAKE, 0, 64, 0), B.fkv_grad(FAKE, 0, 64, 0), None)
        ss = new_stride_s if new_stride_s is not None else p.num_kv_heads * p.head_dim
        new = [B.fkv_cache(x, p.seqlen_q * ss, ss, p.head_dim) for x in (kn, vn)]   # token-major new rows
        cache = [B.fkv_grad(x, p.num_kv_heads * p.seqlen_k * p.head_dim, p.head_dim, p.seqlen_k * p.head_dim)
                 for x in (kc, vc)]                                                  # head-major caches
        return lib.fkv_store_kv(ctypes.byref(p), pos0, new[0], new[1], cache[0], cache[1], None)

    p = _params(B, sq=16, sk=64)
    assert store(None) == INV
    assert store(p, pos0=-1) == INV
    assert store(p, pos0=49) == INV                    # 49 + 16 > 64 tokens
    assert store(p, kn=0) == INV
    assert store(p, vc=0) == INV
    assert store(p, kc=FAKE + 8) == INV                # misaligned cache base
    assert store(p, new_stride_s=60) == INV            # rows overlap
    assert store(_params(B, sq=16, sk=64, d=72)) == B.FKV_ERROR_UNSUPPORTED
    # nothing to write launches nothing
    assert store(_params(B, batch=0, sq=16, sk=64)) == B.FKV_SUCCESS
    assert store(_params(B, sq=0, sk=64), pos0=64) == B.FKV_SUCCESS


def test_binding_refuses_mismatched_store_tensors(B):
    Bt, S, Hkv, D = 2, 32, 2, 64
    new = torch.zeros(Bt, 8, Hkv, D, dtype=torch.bfloat16)
    cache = torch.zeros(Bt, Hkv, S, D, dtype=torch.bfloat16).transpose(1, 2)
    cases = [
        dict(k_new=new, v_new=new, k_cache=cache, v_cache=cache, pos0=25),                    # past the end
        dict(k_new=new, v_new=new[:, :4], k_cache=cache, v_cache=cache, pos0=0),              # new rows differ
        dict(k_new=new, v_new=new, k_cache=cache, v_cache=cache.float(), pos0=0),             # dtype
        dict(k_new=new, v_new=new, k_cache=cache[:, :, :1], v_cache=cache[:, :, :1], pos0=0),  # heads
    ]
    for c in cases:
        with pytest.raises((ValueError, TypeError)) as ei:
            B.fkv_store_kv(c["k_new"], c["v_new"], c["k_cache"], c["v_cache"], pos0=c["pos0"])
        assert "GPU tensor" not in str(ei.value)
    with pytest.raises(TypeError, match="GPU tensor"):
        B.fkv_store_kv(new, new, cache, cache, pos0=24)
