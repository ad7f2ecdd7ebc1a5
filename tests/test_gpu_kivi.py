"""GPU parity of the 4-bit (KIVI-style) source caches through the C ABI:
fkv_kivi_quantize bit for bit against the oracle's quantiser, and
fkv_kivi_decode / fkv_kivi_lite_decode against the fp64 oracle attention over
the dequantised caches.  Decode runs on caches quantised by the ORACLE and
uploaded, so its parity does not lean on the GPU quantiser; one test chains
the two GPU calls.  Every test prints its case before touching the GPU.

[Deck] "FusedKV: Reconstructing KV Caches with Cross-Layer Fusion", frame
"Four-bit KV quantization is the stronger combination" (Tables 14-15)."""
import numpy as np
import pytest
import torch

import kivi_layout as kl
from cross_layer_kv_amd import binding, inputs
from oracle import kivi
from parity import TOL, gpu_rows, lse_err, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
KEYS = ("k1", "kn")


def oracle_q4(L, name, batch=None):
    t = getattr(L, name)
    if batch is not None:
        t = t[batch]
    a = inputs.host_array(t)
    return kivi.quantise_keys(a) if name in KEYS else kivi.quantise_values(a)


def to_lib(trip, is_value):
    """The oracle's plain arrays in the library's packed storage."""
    return kl.values_to_lib(*trip) if is_value else kl.keys_to_lib(*trip)


def upload(trip, is_value):
    """Oracle plain triple -> device cache in the library's storage."""
    codes, sc, mn = to_lib(trip, is_value)
    S = trip[0].shape[2]
    return binding.Q4Cache(torch.from_numpy(codes).to(DEV), torch.from_numpy(sc).to(DEV),
                           torch.from_numpy(mn).to(DEV), is_value, S)


def quantised_layer(L):
    """Oracle-quantised 4-bit copies of the four sources: (host triples, device caches)."""
    host = {n: oracle_q4(L, n) for n in ("k1", "kn", "v1", "vn")}
    dev = {n: upload(host[n], n not in KEYS) for n in host}
    return host, dev


def run(L, dev, fused=True, single=("kn", "v1"), ws=None):
    B, _, Hq, D = L.q.shape
    out = torch.full_like(L.q, float("nan"))
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
    if ws is None:
        ws = binding.decode_workspace(L.q, L.k1)
    if fused:
        binding.fkv_kivi_decode(L.q, dev["k1"], dev["kn"], dev["v1"], dev["vn"], L.weights, out=out, lse=lse,
                                workspace=ws, seqlens_k=L.seqlens_k)
    else:
        binding.fkv_kivi_lite_decode(L.q, dev[single[0]], dev[single[1]], out=out, lse=lse, workspace=ws,
                                     seqlens_k=L.seqlens_k)
    torch.cuda.synchronize()
    return out, lse


def oracle_out(L, host, fused=True, single=("kn", "v1"), batch=None):
    q = L.q if batch is None else L.q[batch]
    sl = None
    if L.seqlens_k is not None:
        sl = L.seqlens_k.cpu().numpy()
        if batch is not None:
            sl = sl[batch]
    qh = inputs.host_array(q)
    if fused:
        w = [x.cpu().numpy() for x in L.weights]
        return kivi.attend(qh, host["k1"], host["v1"], host["kn"], host["vn"], k_w1=w[0], k_wn=w[1], v_w1=w[2],
                           v_wn=w[3], seqlens_k=sl)
    return kivi.attend(qh, host[single[0]], host[single[1]], seqlens_k=sl)


def check(L, host, dev, fused=True, single=("kn", "v1"), tol=None):
    B, _, Hq, D = L.q.shape
    out, lse = run(L, dev, fused, single)
    ro, rl = oracle_out(L, host, fused, single)
    tol = tol or TOL[torch.bfloat16]
    e = rel_err(gpu_rows(out, B, Hq, 1, D), ro)
    el = lse_err(lse.cpu().numpy().reshape(-1), rl)
    say("  fused=%s err=%.3e lse_err=%.3e tol=%.0e" % (fused, e, el, tol))
    assert e <= tol and el <= tol, (e, el)
    return out, lse


def same_q4(got: binding.Q4Cache, ref):
    """The GPU quantiser's packed cache equals the oracle's plain triple (ref)
    packed into the same storage, bit for bit."""
    codes, sc, mn = to_lib(ref, got.is_value)
    assert np.array_equal(got.codes.cpu().numpy(), codes)
    assert np.array_equal(got.scale.cpu().numpy().view(np.uint16), sc.view(np.uint16))
    assert np.array_equal(got.minv.cpu().numpy().view(np.uint16), mn.view(np.uint16))


# ---- quantiser ----

@pytest.mark.parametrize("layout", ["bhsd", "bshd"])
@pytest.mark.parametrize("D", [64, 80, 96, 128])
def test_quantiser_matches_oracle_bitwise(layout, D):
    """Keys (per-channel groups of 32 tokens, ragged last group of 13) and
    values (per-token groups of 32 channels, 16 in the last group of D = 80):
    codes, scales and minima equal the oracle's bit for bit."""
    say("kivi quantise layout=%s D=%d B=2 S=333 Hkv=2" % (layout, D))
    L = inputs.make_layer(2, 1, 333, 4, 2, D, torch.bfloat16, 1200 + D, DEV, layout=layout)
    for name in ("k1", "vn"):
        got = binding.fkv_kivi_quantize(getattr(L, name), name not in KEYS)
        torch.cuda.synchronize()
        same_q4(got, oracle_q4(L, name))


def test_quantiser_degenerate_groups():
    """Constant groups (zero scale: every code 0), a single-token key group,
    two-valued groups (codes 0 and 15 only) and a wide range."""
    say("kivi quantise degenerate groups B=1 S=65 Hkv=1 D=64")
    x = torch.randn(1, 65, 1, 64, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    x[:, :32] = 0.5                                   # constant key groups, constant value rows
    x[:, 32:48, :, 0::2] = -3.0
    x[:, 32:48, :, 1::2] = 7.0                        # two-valued value rows
    x[:, 48:64, 0, 5] = torch.linspace(-3e4, 3e4, 16).to(torch.bfloat16)
    x[:, 64] = 2.0                                    # token 64: a one-token key group
    xd = x.to(DEV)
    for is_value in (False, True):
        got = binding.fkv_kivi_quantize(xd, is_value)
        torch.cuda.synchronize()
        ref = (kivi.quantise_values if is_value else kivi.quantise_keys)(inputs.host_array(x))
        same_q4(got, ref)
    kc = binding.fkv_kivi_quantize(xd, False)
    assert torch.all(kc.codes[:, :, :32] == 0) and torch.all(kc.scale[:, :, 0] == 0)
    assert torch.all(kc.codes[:, :, 64] == 0)
    vc = binding.fkv_kivi_quantize(xd, True)
    torch.cuda.synchronize()
    q, _, _ = kl.values_from_lib(vc.codes.cpu().numpy(), vc.scale.cpu().numpy(), vc.minv.cpu().numpy(), 65)
    assert np.all(q[0, 0, 32:48, 0::2] == 0) and np.all(q[0, 0, 32:48, 1::2] == 15)


def test_quantiser_empty_cache_is_noop():
    say("kivi quantise S=0")
    x = torch.zeros(2, 0, 2, 64, dtype=torch.bfloat16, device=DEV)
    got = binding.fkv_kivi_quantize(x, False)
    torch.cuda.synchronize()
    assert got.codes.numel() == 0 and got.scale.numel() == 0


# ---- decode ----

@pytest.mark.parametrize("D", [64, 80, 96, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_head_dims_and_gqa_ratios(D, G):
    say("kivi decode D=%d G=%d B=2 S=333 Hkv=2" % (D, G))
    L = inputs.make_layer(2, 1, 333, 2 * G, 2, D, torch.bfloat16, 1300 + D + G, DEV)
    host, dev = quantised_layer(L)
    check(L, host, dev, fused=True)
    check(L, host, dev, fused=False)


@pytest.mark.parametrize("splits", [1, 2, 7, 64])
def test_decode_forced_splits_and_ragged(splits, monkeypatch):
    """Split counts (1: direct write, else partials + merge) over ragged
    lengths with an empty sequence, a single token and a partial key group."""
    monkeypatch.setenv("FKV_DECODE_SPLITS", str(splits))
    say("kivi decode splits=%d ragged seqlens B=4 S=4100 D=128 G=2" % splits)
    L = inputs.make_layer(4, 1, 4100, 8, 4, 128, torch.bfloat16, 1400 + splits, DEV,
                          seqlens_k=[4100, 0, 1, 1000])
    host, dev = quantised_layer(L)
    out, lse = check(L, host, dev, fused=True)
    assert torch.all(out[1] == 0) and torch.all(torch.isneginf(lse[1]))
    check(L, host, dev, fused=False)


def test_decode_poisoned_metadata_past_seqlens(monkeypatch):
    """Ragged rows whose 4-bit caches hold garbage past seqlens_k: NaN and
    +inf value scales and minima for every dead token, NaN key metadata for
    key groups wholly past the end, all-ones codes for dead tokens.  Dead
    tokens get probability 0 and their metadata must not reach the sums
    (0 * NaN): the result equals the clean run bit for bit."""
    monkeypatch.setenv("FKV_DECODE_SPLITS", "3")
    say("kivi decode poisoned metadata past seqlens B=4 S=700 D=96 G=2")
    L = inputs.make_layer(4, 1, 700, 8, 4, 96, torch.bfloat16, 1480, DEV, seqlens_k=[700, 0, 131, 77])
    host, dev = quantised_layer(L)
    clean = {f: run(L, dev, fused=f) for f in (True, False)}
    sl = L.seqlens_k.cpu().tolist()
    for value in (float("nan"), float("inf")):
        for n in ("k1", "kn", "v1", "vn"):
            c = dev[n]
            for b, ln in enumerate(sl):
                if n in KEYS:
                    c.codes[b, :, ln:] = 0xFF
                    g0 = (ln + 31) // 32           # first key group wholly past the end
                    c.scale[b, :, g0:] = value
                    c.minv[b, :, g0:] = value
                else:
                    # value metadata lists the 32 tokens of a block in the
                    # header's order: token 4w + e%4 + 16(e//4) at 8w + e
                    for j in range(ln // 32, c.codes.shape[2]):
                        for w in range(4):
                            for e in range(8):
                                if j * 32 + kl.block_token(w, e) >= ln:
                                    c.scale[b, :, j, :, 8 * w + e] = value
                                    c.minv[b, :, j, :, 8 * w + e] = value
        for fused in (True, False):
            out, lse = run(L, dev, fused=fused)
            assert torch.equal(out, clean[fused][0]) and torch.equal(lse, clean[fused][1]), (value, fused)
    check(L, host, dev, fused=True)


def test_decode_empty_cache():
    say("kivi decode seqlen_k=0")
    L = inputs.make_layer(2, 1, 0, 4, 2, 64, torch.bfloat16, 1450, DEV)
    host, dev = quantised_layer(L)
    out, lse = run(L, dev)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_decode_selector_weights_match_lite(monkeypatch):
    """(a, a', b, b') = (0, 1, 1, 0): the fused kernel reads K^n and V^1 only
    ([Deck] frame "Lite separates the key source from the value source"); it
    agrees with the single-source kernel up to float32 summation order."""
    monkeypatch.setenv("FKV_DECODE_SPLITS", "5")
    say("kivi decode selector weights vs lite")
    L = inputs.make_layer(3, 1, 1000, 8, 4, 80, torch.bfloat16, 1460, DEV)
    z = torch.zeros_like(L.weights[0])
    o = torch.ones_like(L.weights[0])
    L.weights = (z, o, o, z)
    host, dev = quantised_layer(L)
    of, lf = check(L, host, dev, fused=True)
    ol, ll = check(L, host, dev, fused=False)
    B, _, Hq, D = L.q.shape
    assert rel_err(gpu_rows(of, B, Hq, 1, D), gpu_rows(ol, B, Hq, 1, D)) <= 2 ** -8
    assert lse_err(lf.cpu().numpy(), ll.cpu().numpy()) <= 1e-5


def test_gpu_quantise_then_decode():
    """The two GPU calls chained (layout bshd), against the oracle's
    quantise-then-attend."""
    say("kivi quantise+decode bshd B=3 S=777 Hq=8 Hkv=4 D=96")
    L = inputs.make_layer(3, 1, 777, 8, 4, 96, torch.bfloat16, 1470, DEV, layout="bshd")
    host = {n: oracle_q4(L, n) for n in ("k1", "kn", "v1", "vn")}
    dev = {n: binding.fkv_kivi_quantize(getattr(L, n), n not in KEYS) for n in host}
    check(L, host, dev, fused=True)
    check(L, host, dev, fused=False)


def test_full_size_650m_kivi_decode():
    """650M shape (B=32, S=8192, 16/8 heads, D=96), the benchmarked launch:
    the GPU quantiser's caches for sampled batches equal the oracle's bit
    for bit, and decode over them matches the oracle on every head."""
    B, S, Hq, Hkv, D, seed = 32, 8192, 16, 8, 96, 0xF0007
    say("kivi full size B=%d S=%d Hq=%d Hkv=%d D=%d seed=%#x (sampled rows)" % (B, S, Hq, Hkv, D, seed))
    L = inputs.make_layer(B, 1, S, Hq, Hkv, D, torch.bfloat16, seed, DEV)
    dev = {n: binding.fkv_kivi_quantize(getattr(L, n), n not in KEYS) for n in ("k1", "kn", "v1", "vn")}
    torch.cuda.synchronize()
    bs = [0, 17, B - 1]
    host = {}
    for n in dev:
        host[n] = oracle_q4(L, n, batch=bs)
        same_q4(binding.Q4Cache(dev[n].codes[bs], dev[n].scale[bs], dev[n].minv[bs], n not in KEYS), host[n])
    for fused in (True, False):
        out, lse = run(L, dev, fused=fused)
        ro, rl = oracle_out(L, host, fused=fused, batch=bs)
        e = rel_err(gpu_rows(out[bs], len(bs), Hq, 1, D), ro)
        el = lse_err(lse[bs].cpu().numpy().reshape(-1), rl)
        say("  fused=%s batches=%s err=%.3e lse_err=%.3e" % (fused, bs, e, el))
        assert e <= 1e-2 and el <= 1e-2
        assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    del L, dev
    torch.cuda.empty_cache()
