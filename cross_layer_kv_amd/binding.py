"""Thin ctypes binding of libfusedkv (declared in include/fusedkv.h).

The Python functions carry the C entry points' names and only marshal
arguments: torch tensors become device pointers, shapes become an
``fkv_params`` block, cache tensors become ``fkv_cache`` views (their strides
are passed through, so head-major and token-major storage both work).  Every
step of the computation runs in the HIP kernels of the library; there is no
fallback.  Tensors must live on a GPU; the library must have been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfusedkv.so")

FKV_SUCCESS, FKV_ERROR_INVALID_VALUE, FKV_ERROR_UNSUPPORTED, FKV_ERROR_WORKSPACE, FKV_ERROR_LAUNCH = range(5)
FKV_F32, FKV_BF16 = 0, 1


class FkvError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s (status %d)" % (message, status))
        self.status = status


class fkv_cache(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_s", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


class fkv_params(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen_q", ctypes.c_int32),
                ("seqlen_k", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("causal", ctypes.c_int32)]


class fkv_q4_cache(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("minv", ctypes.c_void_p)]


class fkv_grad(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_s", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


class fkv_fusion_grad(ctypes.Structure):
    _fields_ = [("k_w1", ctypes.c_void_p), ("k_wn", ctypes.c_void_p),
                ("v_w1", ctypes.c_void_p), ("v_wn", ctypes.c_void_p)]


class fkv_fusion(ctypes.Structure):
    _fields_ = [("k_w1", ctypes.c_void_p), ("k_wn", ctypes.c_void_p),
                ("v_w1", ctypes.c_void_p), ("v_wn", ctypes.c_void_p)]


ABI_VERSION = 7

EXPORTS = ["fkv_abi_version", "fkv_status_string", "fkv_last_error", "fkv_decode_workspace_size",
           "fkv_decode", "fkv_lite_decode", "fkv_prefill", "fkv_lite_prefill",
           "fkv_check_tied",
           "fkv_kivi_codes_bytes", "fkv_kivi_meta_bytes", "fkv_kivi_quantize", "fkv_kivi_decode",
           "fkv_kivi_lite_decode", "fkv_backward_workspace_size", "fkv_prefill_backward",
           "fkv_lite_prefill_backward", "fkv_decode_noalloc", "fkv_store_kv"]

NOALLOC_SCRATCH_BYTES = 8 << 20

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libfusedkv.so and declare its signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libfusedkv.so is not built (expected at %s); run __graft_entry__.build()" % path)
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    lib.fkv_abi_version.restype = ctypes.c_int
    lib.fkv_abi_version.argtypes = []
    lib.fkv_status_string.restype = ctypes.c_char_p
    lib.fkv_status_string.argtypes = [ctypes.c_int]
    lib.fkv_last_error.restype = ctypes.c_char_p
    lib.fkv_last_error.argtypes = []
    lib.fkv_decode_workspace_size.restype = ctypes.c_size_t
    lib.fkv_decode_workspace_size.argtypes = [P(fkv_params)]
    lib.fkv_decode.restype = ctypes.c_int
    lib.fkv_decode.argtypes = [P(fkv_params), vp, fkv_cache, fkv_cache, fkv_cache, fkv_cache,
                               P(fkv_fusion), vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.fkv_decode_noalloc.restype = ctypes.c_int
    lib.fkv_decode_noalloc.argtypes = [P(fkv_params), vp, fkv_cache, fkv_cache, fkv_cache, fkv_cache,
                                       P(fkv_fusion), vp, vp, vp, vp]
    lib.fkv_lite_decode.restype = ctypes.c_int
    lib.fkv_lite_decode.argtypes = [P(fkv_params), vp, fkv_cache, fkv_cache, vp, vp, vp, vp,
                                    ctypes.c_size_t, vp]
    lib.fkv_prefill.restype = ctypes.c_int
    lib.fkv_prefill.argtypes = [P(fkv_params), vp, fkv_cache, fkv_cache, fkv_cache, fkv_cache,
                                P(fkv_fusion), vp, vp, vp]
    lib.fkv_lite_prefill.restype = ctypes.c_int
    lib.fkv_lite_prefill.argtypes = [P(fkv_params), vp, fkv_cache, fkv_cache, vp, vp, vp]
    lib.fkv_check_tied.restype = ctypes.c_int
    lib.fkv_check_tied.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float]
    lib.fkv_kivi_codes_bytes.restype = ctypes.c_size_t
    lib.fkv_kivi_codes_bytes.argtypes = [P(fkv_params), ctypes.c_int32]
    lib.fkv_kivi_meta_bytes.restype = ctypes.c_size_t
    lib.fkv_kivi_meta_bytes.argtypes = [P(fkv_params), ctypes.c_int32]
    lib.fkv_kivi_quantize.restype = ctypes.c_int
    lib.fkv_kivi_quantize.argtypes = [P(fkv_params), fkv_cache, ctypes.c_int32, fkv_q4_cache, vp]
    lib.fkv_kivi_decode.restype = ctypes.c_int
    lib.fkv_kivi_decode.argtypes = [P(fkv_params), vp, fkv_q4_cache, fkv_q4_cache, fkv_q4_cache, fkv_q4_cache,
                                    P(fkv_fusion), vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.fkv_kivi_lite_decode.restype = ctypes.c_int
    lib.fkv_kivi_lite_decode.argtypes = [P(fkv_params), vp, fkv_q4_cache, fkv_q4_cache, vp, vp, vp, vp,
                                         ctypes.c_size_t, vp]
    lib.fkv_backward_workspace_size.restype = ctypes.c_size_t
    lib.fkv_backward_workspace_size.argtypes = [P(fkv_params)]
    lib.fkv_prefill_backward.restype = ctypes.c_int
    lib.fkv_prefill_backward.argtypes = [P(fkv_params), vp, fkv_cache, fkv_cache, fkv_cache, fkv_cache,
                                         P(fkv_fusion), vp, vp, vp, vp, fkv_grad, fkv_grad, fkv_grad, fkv_grad,
                                         P(fkv_fusion_grad), vp, ctypes.c_size_t, vp]
    lib.fkv_store_kv.restype = ctypes.c_int
    lib.fkv_store_kv.argtypes = [P(fkv_params), ctypes.c_int32, fkv_cache, fkv_cache, fkv_grad, fkv_grad, vp]
    lib.fkv_lite_prefill_backward.restype = ctypes.c_int
    lib.fkv_lite_prefill_backward.argtypes = [P(fkv_params), vp, fkv_cache, fkv_cache, vp, vp, vp, vp, fkv_grad,
                                              fkv_grad, vp, ctypes.c_size_t, vp]
    if lib.fkv_abi_version() != ABI_VERSION:
        raise RuntimeError("libfusedkv ABI version mismatch")
    _lib = lib
    return lib


def _check(status):
    if status != FKV_SUCCESS:
        lib = load_library()
        raise FkvError(status, lib.fkv_last_error().decode() or lib.fkv_status_string(status).decode())


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FKV_F32
    if t.dtype == torch.bfloat16:
        return FKV_BF16
    raise TypeError("data must be float32 or bfloat16, got %s" % t.dtype)


def _dev(t, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    return t.data_ptr()


# ---- argument checks ----
# The C ABI sees only pointers, strides and the shape block, so a tensor whose
# shape, dtype or extent disagrees with the others would make the kernels read
# or write outside it.  These checks compare the tensors with each other
# before any pointer is handed over; they raise ValueError / TypeError.  They
# look at shapes, dtypes and strides only (the device check comes when the
# pointers are taken), so they run the same way on host tensors.

def _contig(t, name):
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _same_dtype(ref, t, name):
    if t.dtype != ref.dtype:
        raise TypeError("%s is %s, expected %s like q" % (name, t.dtype, ref.dtype))


def _check_qo(q, out, name_q="q", name_o="out"):
    """q, out: contiguous [B, S_q, H_q, D] tensors of one dtype and shape."""
    if q.dim() != 4:
        raise ValueError("%s must be [B, S_q, H_q, D]" % name_q)
    _contig(q, name_q)
    _contig(out, name_o)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("%s shape %s differs from %s shape %s" % (name_o, tuple(out.shape), name_q, tuple(q.shape)))
    _same_dtype(q, out, name_o)


def _check_caches(q, caches, names):
    """Every cache a [B, S_k, H_kv, D] view of q's dtype with B and D of q,
    H_q a multiple of H_kv, and all caches of one shape."""
    B, _, Hq, D = q.shape
    ref = None
    for c, n in zip(caches, names):
        if c.dim() != 4 or c.stride(3) != 1:
            raise ValueError("%s must be a [B, S, H_kv, D] view with a contiguous channel axis" % n)
        _same_dtype(q, c, n)
        if c.shape[0] != B or c.shape[3] != D:
            raise ValueError("%s shape %s does not match q (B=%d, D=%d)" % (n, tuple(c.shape), B, D))
        if c.shape[2] < 1 or Hq % c.shape[2]:
            raise ValueError("%s has %d KV heads; q has %d heads" % (n, c.shape[2], Hq))
        if ref is None:
            ref = (tuple(c.shape), n)
        elif tuple(c.shape) != ref[0]:
            raise ValueError("%s shape %s differs from %s shape %s" % (n, tuple(c.shape), ref[1], ref[0]))


def _check_weights(weights, Hkv, D, name="weights"):
    if weights is None or len(weights) != 4:
        raise ValueError("%s are the four [H_kv, D] float32 vectors (a, a', b, b')" % name)
    for w in weights:
        if w.dtype != torch.float32 or not w.is_contiguous():
            raise TypeError("%s must be contiguous float32" % name)
        if tuple(w.shape) != (Hkv, D):
            raise ValueError("%s must be [H_kv, D] = [%d, %d], got %s" % (name, Hkv, D, tuple(w.shape)))


def _check_lse(lse, q):
    """lse: contiguous float32 [B, H_q, S_q] (or [B, H_q] when S_q = 1)."""
    if lse is None:
        return
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TypeError("lse must be contiguous float32")
    B, Sq, Hq, _ = q.shape
    if lse.numel() != B * Hq * Sq:
        raise ValueError("lse holds %d elements, the call writes B*H_q*S_q = %d" % (lse.numel(), B * Hq * Sq))


def _check_seqlens(seqlens_k, B):
    if seqlens_k is None:
        return
    if seqlens_k.dtype != torch.int32 or not seqlens_k.is_contiguous() or seqlens_k.numel() != B:
        raise ValueError("seqlens_k must be a contiguous int32 tensor of B = %d elements" % B)


def _check_workspace(workspace):
    if workspace is None:
        return
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous uint8 tensor")


def cache_view(t: torch.Tensor) -> fkv_cache:
    """fkv_cache of a logical [B, S, H, D] tensor (any strides, channel axis
    contiguous)."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("a cache is a [B, S, H, D] view with a contiguous channel axis")
    _dev(t, "cache")
    return fkv_cache(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def make_params(q: torch.Tensor, k: torch.Tensor, *, softmax_scale: float = 0.0, causal: bool = False) -> fkv_params:
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    return fkv_params(B, Sq, Sk, Hq, Hkv, D, _dtype(q), float(softmax_scale), 1 if causal else 0)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _fusion(weights, Hkv, D) -> fkv_fusion:
    _check_weights(weights, Hkv, D)
    return fkv_fusion(*[_dev(w, "weight") for w in weights])


def _decode_checks(q, caches, names, out, lse, seqlens_k, workspace):
    _check_qo(q, out)
    if q.shape[1] != 1:
        raise ValueError("decode takes one query row per batch row (q is [B, 1, H_q, D])")
    _check_caches(q, caches, names)
    _check_lse(lse, q)
    _check_seqlens(seqlens_k, q.shape[0])
    _check_workspace(workspace)


def _prefill_checks(q, caches, names, out, lse):
    _check_qo(q, out)
    _check_caches(q, caches, names)
    if caches[0].shape[1] != q.shape[1]:
        raise ValueError("prefill needs S_q == S_k (q has %d rows, the caches %d tokens)"
                         % (q.shape[1], caches[0].shape[1]))
    _check_lse(lse, q)


def fkv_decode_workspace_size(params: fkv_params) -> int:
    return int(load_library().fkv_decode_workspace_size(ctypes.byref(params)))


def decode_workspace(q: torch.Tensor, k: torch.Tensor) -> torch.Tensor:
    """A zero-filled workspace for decode calls with these shapes."""
    n = fkv_decode_workspace_size(make_params(q, k))
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=q.device)


def fkv_decode(q, k1, kn, v1, vn, weights, *, out, workspace, lse=None, seqlens_k=None,
               softmax_scale=0.0, stream=None):
    """FusedKV decode step of one reconstruction layer (see fkv_decode in
    include/fusedkv.h).  q, out: [B, 1, Hq, D]; caches [B, Sk, Hkv, D]."""
    lib = load_library()
    _decode_checks(q, (k1, kn, v1, vn), ("k1", "kn", "v1", "vn"), out, lse, seqlens_k, workspace)
    p = make_params(q, k1, softmax_scale=softmax_scale)
    f = _fusion(weights, k1.shape[2], q.shape[3])
    _check(lib.fkv_decode(ctypes.byref(p), _dev(q, "q"), cache_view(k1), cache_view(kn), cache_view(v1),
                          cache_view(vn), ctypes.byref(f), _dev(seqlens_k, "seqlens_k"), _dev(out, "out"),
                          _dev(lse, "lse"), _dev(workspace, "workspace"), workspace.numel(), _stream(stream)))


def fkv_decode_noalloc(q, k1, kn, v1, vn, weights, *, out, lse=None, seqlens_k=None, softmax_scale=0.0,
                       stream=None):
    """fkv_decode without a workspace: split partials go to the library's
    static per-GPU scratch (fkv_decode_noalloc in include/fusedkv.h).  Calls
    that may overlap on one GPU race on that scratch."""
    lib = load_library()
    _decode_checks(q, (k1, kn, v1, vn), ("k1", "kn", "v1", "vn"), out, lse, seqlens_k, None)
    p = make_params(q, k1, softmax_scale=softmax_scale)
    f = _fusion(weights, k1.shape[2], q.shape[3])
    _check(lib.fkv_decode_noalloc(ctypes.byref(p), _dev(q, "q"), cache_view(k1), cache_view(kn), cache_view(v1),
                                  cache_view(vn), ctypes.byref(f), _dev(seqlens_k, "seqlens_k"), _dev(out, "out"),
                                  _dev(lse, "lse"), _stream(stream)))


def fkv_lite_decode(q, k_src, v_src, *, out, workspace, lse=None, seqlens_k=None, softmax_scale=0.0,
                    stream=None):
    """Single-source decode step: FusedKV-Lite with (K^n, V^1), or plain
    attention of a storage layer over its own caches."""
    lib = load_library()
    _decode_checks(q, (k_src, v_src), ("k_src", "v_src"), out, lse, seqlens_k, workspace)
    p = make_params(q, k_src, softmax_scale=softmax_scale)
    _check(lib.fkv_lite_decode(ctypes.byref(p), _dev(q, "q"), cache_view(k_src), cache_view(v_src),
                               _dev(seqlens_k, "seqlens_k"), _dev(out, "out"), _dev(lse, "lse"),
                               _dev(workspace, "workspace"), workspace.numel(), _stream(stream)))


def fkv_prefill(q, k1, kn, v1, vn, weights, *, out, lse=None, causal=True, softmax_scale=0.0, stream=None):
    """FusedKV prefill of one reconstruction layer (bf16), tiles fused inside
    the attention kernel.  q, out: [B, S, Hq, D]; caches [B, S, Hkv, D]."""
    lib = load_library()
    _prefill_checks(q, (k1, kn, v1, vn), ("k1", "kn", "v1", "vn"), out, lse)
    p = make_params(q, k1, softmax_scale=softmax_scale, causal=causal)
    f = _fusion(weights, k1.shape[2], q.shape[3])
    _check(lib.fkv_prefill(ctypes.byref(p), _dev(q, "q"), cache_view(k1), cache_view(kn), cache_view(v1),
                           cache_view(vn), ctypes.byref(f), _dev(out, "out"), _dev(lse, "lse"), _stream(stream)))


def fkv_lite_prefill(q, k_src, v_src, *, out, lse=None, causal=True, softmax_scale=0.0, stream=None):
    """Single-source prefill (FusedKV-Lite or the plain control)."""
    lib = load_library()
    _prefill_checks(q, (k_src, v_src), ("k_src", "v_src"), out, lse)
    p = make_params(q, k_src, softmax_scale=softmax_scale, causal=causal)
    _check(lib.fkv_lite_prefill(ctypes.byref(p), _dev(q, "q"), cache_view(k_src), cache_view(v_src),
                                _dev(out, "out"), _dev(lse, "lse"), _stream(stream)))


def fkv_check_tied(k_w: torch.Tensor, pairing: str = "interleaved", tol: float = 0.0) -> bool:
    """Host check that key weights [Hkv, D] are tied on RoPE pairs."""
    lib = load_library()
    w = k_w.detach().to("cpu", torch.float32).contiguous()
    code = {"interleaved": 0, "half": 1}[pairing]
    st = lib.fkv_check_tied(ctypes.c_void_p(w.data_ptr()), w.shape[0], w.shape[1], code, float(tol))
    if st == FKV_SUCCESS:
        return True
    if st == FKV_ERROR_INVALID_VALUE:
        return False
    _check(st)
    return False


# ---- KIVI-style 4-bit source caches ----

class Q4Cache:
    """Device arrays of one 4-bit source (layout in include/fusedkv.h).
    Keys: codes uint8 [B, Hkv, S, D/2], scale and minv float16
    [B, Hkv, NB, D]; values: codes uint8 [B, Hkv, NB, D, 16], scale and minv
    float16 [B, Hkv, NB, ceil(D/32), 32]; NB = ceil(S/32)."""

    def __init__(self, codes, scale, minv, is_value, seqlen=None):
        self.codes, self.scale, self.minv, self.is_value = codes, scale, minv, bool(is_value)
        self._seqlen = seqlen

    def view(self) -> fkv_q4_cache:
        return fkv_q4_cache(_dev(self.codes, "codes"), _dev(self.scale, "scale"), _dev(self.minv, "minv"))

    @property
    def seqlen(self):
        if not self.is_value:
            return self.codes.shape[2]
        return self._seqlen if self._seqlen is not None else self.codes.shape[2] * 32


def kivi_empty(B, S, Hkv, D, is_value, device="cuda"):
    """Uninitialised 4-bit cache arrays of the library's layout."""
    nb = (S + 31) // 32
    if is_value:
        codes = (B, Hkv, nb, D, 16)
        meta = (B, Hkv, nb, (D + 31) // 32, 32)
    else:
        codes = (B, Hkv, S, D // 2)
        meta = (B, Hkv, nb, D)
    return Q4Cache(torch.empty(codes, dtype=torch.uint8, device=device),
                   torch.empty(meta, dtype=torch.float16, device=device),
                   torch.empty(meta, dtype=torch.float16, device=device), is_value, S)


def _q4_shapes(B, S, Hkv, D, is_value):
    nb = (S + 31) // 32
    if is_value:
        return (B, Hkv, nb, D, 16), (B, Hkv, nb, (D + 31) // 32, 32)
    return (B, Hkv, S, D // 2), (B, Hkv, nb, D)


def _check_q4(c: Q4Cache, B, S, Hkv, D, is_value, name):
    """A 4-bit cache of the layout above for B batch rows, S tokens, Hkv heads
    and head dim D (values: S rounded up to whole 32-token blocks)."""
    if not isinstance(c, Q4Cache):
        raise TypeError("%s must be a Q4Cache" % name)
    if c.is_value != bool(is_value):
        raise ValueError("%s must be a %s cache" % (name, "value" if is_value else "key"))
    codes, meta = _q4_shapes(B, S, Hkv, D, is_value)
    if c.codes.dtype != torch.uint8 or tuple(c.codes.shape) != codes or not c.codes.is_contiguous():
        raise ValueError("%s codes must be contiguous uint8 %s, got %s %s"
                         % (name, codes, c.codes.dtype, tuple(c.codes.shape)))
    for t, n in ((c.scale, "scale"), (c.minv, "minv")):
        if t.dtype != torch.float16 or tuple(t.shape) != meta or not t.is_contiguous():
            raise ValueError("%s %s must be contiguous float16 %s, got %s %s"
                             % (name, n, meta, t.dtype, tuple(t.shape)))


def fkv_kivi_quantize(src: torch.Tensor, is_value: bool, *, dst: Q4Cache | None = None, num_q_heads=None,
                      stream=None) -> Q4Cache:
    """4-bit cache of a bf16 source [B, S, Hkv, D] (keys: is_value False)."""
    lib = load_library()
    if src.dim() != 4 or src.stride(3) != 1:
        raise ValueError("src must be a [B, S, H_kv, D] view with a contiguous channel axis")
    B, S, Hkv, D = src.shape
    if dst is None:
        dst = kivi_empty(B, S, Hkv, D, is_value, src.device)
    _check_q4(dst, B, S, Hkv, D, is_value, "dst")
    p = fkv_params(B, 1, S, num_q_heads or Hkv, Hkv, D, _dtype(src), 0.0, 0)
    _check(lib.fkv_kivi_quantize(ctypes.byref(p), cache_view(src), 1 if is_value else 0, dst.view(), _stream(stream)))
    return dst


def _kivi_params(q, c: Q4Cache, softmax_scale):
    """c: the KEY cache (its token count is exact; value codes are padded)."""
    B, Sq, Hq, D = q.shape
    return fkv_params(B, Sq, c.seqlen, Hq, c.codes.shape[1], D, _dtype(q), float(softmax_scale), 0)


def _kivi_checks(q, keys, values, out, lse, seqlens_k, workspace):
    """keys / values: (Q4Cache, name) pairs; all share the first key cache's
    batch, token count, KV heads and q's head dim."""
    _check_qo(q, out)
    if q.shape[1] != 1:
        raise ValueError("decode takes one query row per batch row (q is [B, 1, H_q, D])")
    B, _, Hq, D = q.shape
    k0 = keys[0][0]
    if not isinstance(k0, Q4Cache) or k0.codes.dim() != 4:
        raise TypeError("%s must be a key Q4Cache" % keys[0][1])
    S, Hkv = k0.seqlen, k0.codes.shape[1]
    if Hkv < 1 or Hq % Hkv:
        raise ValueError("%s has %d KV heads; q has %d heads" % (keys[0][1], Hkv, Hq))
    for c, n in keys:
        _check_q4(c, B, S, Hkv, D, False, n)
    for c, n in values:
        _check_q4(c, B, S, Hkv, D, True, n)
    _check_lse(lse, q)
    _check_seqlens(seqlens_k, B)
    _check_workspace(workspace)


def fkv_kivi_decode(q, k1: Q4Cache, kn: Q4Cache, v1: Q4Cache, vn: Q4Cache, weights, *, out, workspace, lse=None,
                    seqlens_k=None, softmax_scale=0.0, stream=None):
    """FusedKV decode over 4-bit sources (fkv_kivi_decode in fusedkv.h)."""
    lib = load_library()
    _kivi_checks(q, ((k1, "k1"), (kn, "kn")), ((v1, "v1"), (vn, "vn")), out, lse, seqlens_k, workspace)
    p = _kivi_params(q, k1, softmax_scale)
    f = _fusion(weights, k1.codes.shape[1], q.shape[3])
    _check(lib.fkv_kivi_decode(ctypes.byref(p), _dev(q, "q"), k1.view(), kn.view(), v1.view(), vn.view(),
                               ctypes.byref(f), _dev(seqlens_k, "seqlens_k"), _dev(out, "out"), _dev(lse, "lse"),
                               _dev(workspace, "workspace"), workspace.numel(), _stream(stream)))


def fkv_kivi_lite_decode(q, k_src: Q4Cache, v_src: Q4Cache, *, out, workspace, lse=None, seqlens_k=None,
                         softmax_scale=0.0, stream=None):
    """Single-source decode over 4-bit sources (FusedKV-Lite: K^n, V^1)."""
    lib = load_library()
    _kivi_checks(q, ((k_src, "k_src"),), ((v_src, "v_src"),), out, lse, seqlens_k, workspace)
    p = _kivi_params(q, k_src, softmax_scale)
    _check(lib.fkv_kivi_lite_decode(ctypes.byref(p), _dev(q, "q"), k_src.view(), v_src.view(),
                                    _dev(seqlens_k, "seqlens_k"), _dev(out, "out"), _dev(lse, "lse"),
                                    _dev(workspace, "workspace"), workspace.numel(), _stream(stream)))


# ---- backward pass ----

def grad_view(t: torch.Tensor) -> fkv_grad:
    """Writable fkv_grad of a logical [B, S, H, D] tensor (any strides, channel
    axis contiguous)."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("a gradient is a [B, S, H, D] view with a contiguous channel axis")
    _dev(t, "gradient")
    return fkv_grad(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _backward_checks(q, caches, names, out, lse, dout, dq, grads, gnames, workspace):
    """Forward tensors as fkv_prefill; out, dout, dq like q; each gradient
    view shaped and typed like its cache; lse the forward's [B, H_q, S]."""
    _prefill_checks(q, caches, names, out, None)
    _check_qo(q, dout, name_o="dout")
    _check_qo(q, dq, name_o="dq")
    if lse is None:
        raise ValueError("the backward pass needs the forward LSE")
    _check_lse(lse, q)
    for g, n, c in zip(grads, gnames, caches):
        if g.dim() != 4 or g.stride(3) != 1:
            raise ValueError("%s must be a [B, S, H_kv, D] view with a contiguous channel axis" % n)
        _same_dtype(q, g, n)
        if tuple(g.shape) != tuple(c.shape):
            raise ValueError("%s shape %s differs from its cache's %s" % (n, tuple(g.shape), tuple(c.shape)))
    _check_workspace(workspace)


def backward_workspace(q: torch.Tensor, k: torch.Tensor) -> torch.Tensor:
    """A workspace for backward calls with these shapes (contents ignored)."""
    n = load_library().fkv_backward_workspace_size(ctypes.byref(make_params(q, k, causal=True)))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)


def fkv_prefill_backward(q, k1, kn, v1, vn, weights, out, lse, dout, *, dq, dk1, dkn, dv1, dvn, dweights,
                         workspace, causal=True, softmax_scale=0.0, stream=None):
    """Gradients of one FusedKV prefill layer (fkv_prefill_backward in
    fusedkv.h).  dweights: four contiguous float32 [Hkv, D] tensors written
    with the gradients of (a, a', b, b')."""
    lib = load_library()
    _backward_checks(q, (k1, kn, v1, vn), ("k1", "kn", "v1", "vn"), out, lse, dout, dq, (dk1, dkn, dv1, dvn),
                     ("dk1", "dkn", "dv1", "dvn"), workspace)
    _check_weights(dweights, k1.shape[2], q.shape[3], "weight gradients")
    p = make_params(q, k1, softmax_scale=softmax_scale, causal=causal)
    f = _fusion(weights, k1.shape[2], q.shape[3])
    df = fkv_fusion_grad(*[_dev(w, "weight gradient") for w in dweights])
    _check(lib.fkv_prefill_backward(ctypes.byref(p), _dev(q, "q"), cache_view(k1), cache_view(kn), cache_view(v1),
                                    cache_view(vn), ctypes.byref(f), _dev(out, "out"), _dev(lse, "lse"),
                                    _dev(dout, "dout"), _dev(dq, "dq"), grad_view(dk1), grad_view(dkn),
                                    grad_view(dv1), grad_view(dvn), ctypes.byref(df), _dev(workspace, "workspace"),
                                    workspace.numel(), _stream(stream)))


def fkv_lite_prefill_backward(q, k_src, v_src, out, lse, dout, *, dq, dk, dv, workspace, causal=True,
                              softmax_scale=0.0, stream=None):
    """Gradients of a single-source prefill layer (FusedKV-Lite with (K^n,
    V^1), or the plain control): dk, dv are the gradients of k_src, v_src."""
    lib = load_library()
    _backward_checks(q, (k_src, v_src), ("k_src", "v_src"), out, lse, dout, dq, (dk, dv), ("dk", "dv"), workspace)
    p = make_params(q, k_src, softmax_scale=softmax_scale, causal=causal)
    _check(lib.fkv_lite_prefill_backward(ctypes.byref(p), _dev(q, "q"), cache_view(k_src), cache_view(v_src),
                                         _dev(out, "out"), _dev(lse, "lse"), _dev(dout, "dout"), _dev(dq, "dq"),
                                         grad_view(dk), grad_view(dv), _dev(workspace, "workspace"),
                                         workspace.numel(), _stream(stream)))


# ---- storage layers ----

def _store_checks(k_new, v_new, k_cache, v_cache, pos0):
    """k_new / v_new [B, S_new, H_kv, D] and k_cache / v_cache [B, S, H_kv, D]
    views of one dtype with contiguous channel axes; pos0 + S_new <= S."""
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        if not isinstance(t, torch.Tensor) or t.dim() != 4 or t.stride(3) != 1:
            raise ValueError("%s must be a [B, S, H_kv, D] view with a contiguous channel axis" % n)
        _same_dtype(k_new, t, n)
    if tuple(v_new.shape) != tuple(k_new.shape):
        raise ValueError("v_new shape %s differs from k_new's %s" % (tuple(v_new.shape), tuple(k_new.shape)))
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("v_cache shape %s differs from k_cache's %s" % (tuple(v_cache.shape), tuple(k_cache.shape)))
    B, Sn, H, D = k_new.shape
    if (k_cache.shape[0], k_cache.shape[2], k_cache.shape[3]) != (B, H, D):
        raise ValueError("caches %s do not match the new rows %s" % (tuple(k_cache.shape), tuple(k_new.shape)))
    if pos0 < 0 or pos0 + Sn > k_cache.shape[1]:
        raise ValueError("positions %d..%d are outside the caches' %d tokens" % (pos0, pos0 + Sn - 1,
                                                                                 k_cache.shape[1]))


def fkv_store_kv(k_new, v_new, k_cache, v_cache, *, pos0=0, stream=None):
    """Write a storage layer's new keys and values (token-major or any
    strides) into its caches at positions pos0.. (fkv_store_kv in
    fusedkv.h), bit for bit."""
    lib = load_library()
    _store_checks(k_new, v_new, k_cache, v_cache, int(pos0))
    B, Sn, H, D = k_new.shape
    p = fkv_params(B, Sn, k_cache.shape[1], H, H, D, _dtype(k_new), 0.0, 0)
    _check(lib.fkv_store_kv(ctypes.byref(p), int(pos0), cache_view(k_new), cache_view(v_new), grad_view(k_cache),
                            grad_view(v_cache), _stream(stream)))
