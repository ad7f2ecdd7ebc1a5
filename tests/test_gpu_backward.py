"""GPU parity of fkv_prefill_backward / fkv_lite_prefill_backward against the
fp64 backward oracle (oracle/backward.py), through the C ABI.  The forward
output O and LSE the backward call consumes come from the forward oracle
(O rounded to bfloat16, LSE to float32); the training flow, with O and LSE
from the library's own fkv_prefill, has tests of its own.  Every test prints
its case before touching the GPU.

Tolerance, fixed and stated once (the pages and the configuration give none
for gradients).  Every product that involves a gradient keeps bfloat16
operands (unit roundoff u = 2^-8), and each gradient passes through four
bfloat16 roundings: a fused or source operand, a probability or dS operand,
the dO or Q operand, and the output.  Per output tensor:
  normwise      ||x - r||_2 / ||r||_2              <= 1e-2
  max-relative  max_i |x_i - r_i| / max_i |r_i|    <= 4u = 1.5625e-2
The per-element error against each element's own row scale is printed for
information only: softmax gradient rows sum to zero, so small elements of
early causal rows carry a few percent of relative error that no fixed
bfloat16 bound excludes.

[Deck] "FusedKV: Reconstructing KV Caches with Cross-Layer Fusion", frame
"FusedKV learns two-source, channel-wise fusion" (Eqs. (4)-(5), trained end
to end); frame "Lite separates the key source from the value source"."""
import numpy as np
import pytest
import torch

from cross_layer_kv_amd import binding, inputs
import oracle
from oracle import backward as bw
import bwd_rounding as rb
from parity import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-2                 # normwise
MAXREL = 4 * 2.0 ** -8     # max-relative: four bfloat16 roundings
WNAMES = ("dk_w1", "dk_wn", "dv_w1", "dv_wn")


class Case:
    """Inputs of one backward call, its forward (from the library) and its
    gradient buffers."""

    def __init__(self, B, S, Hq, Hkv, D, seed, causal=True, layout="bhsd", lite=False, dstd=1.0, fwd="oracle"):
        self.L = inputs.make_layer(B, S, S, Hq, Hkv, D, torch.bfloat16, seed, DEV, layout=layout, decode=False)
        self.dout = inputs.make_grad_output(B, S, Hq, D, torch.bfloat16, seed * 16 + 9, DEV, std=dstd)
        self.causal, self.lite, self.fwd = causal, lite, fwd
        self.shape = (B, S, Hq, Hkv, D)
        self.forward()

    def forward(self):
        L = self.L
        B, S, Hq, Hkv, D = self.shape
        if self.fwd == "oracle":
            h = inputs.host_array
            if self.lite:
                o, lse = oracle.attend(h(L.q), h(L.kn), h(L.v1), causal=self.causal)
            else:
                w = [x.cpu().numpy() for x in L.weights]
                o, lse = oracle.attend(h(L.q), h(L.k1), h(L.v1), h(L.kn), h(L.vn), k_w1=w[0], k_wn=w[1],
                                       v_w1=w[2], v_wn=w[3], causal=self.causal)
            o = np.ascontiguousarray(o.reshape(B, Hq, S, D).transpose(0, 2, 1, 3))
            self.out = torch.from_numpy(o.astype(np.float32)).to(torch.bfloat16).to(DEV)
            self.lse = torch.from_numpy(lse.reshape(B, Hq, S).astype(np.float32)).to(DEV)
            return
        self.out = torch.empty_like(L.q)
        self.lse = torch.empty(B, Hq, S, dtype=torch.float32, device=DEV)
        if self.lite:
            binding.fkv_lite_prefill(L.q, L.kn, L.v1, out=self.out, lse=self.lse, causal=self.causal)
        else:
            binding.fkv_prefill(L.q, L.k1, L.kn, L.v1, L.vn, L.weights, out=self.out, lse=self.lse,
                                causal=self.causal)

    def run(self):
        L = self.L
        B, S, Hq, Hkv, D = self.shape
        nan = float("nan")
        g = {"dq": torch.full_like(L.q, nan)}
        mk = lambda: torch.full((B, S, Hkv, D), nan, dtype=torch.bfloat16, device=DEV)
        ws = binding.backward_workspace(L.q, L.k1)
        if self.lite:
            g["dk"], g["dv"] = mk(), mk()
            binding.fkv_lite_prefill_backward(L.q, L.kn, L.v1, self.out, self.lse, self.dout, dq=g["dq"],
                                              dk=g["dk"], dv=g["dv"], workspace=ws, causal=self.causal)
        else:
            for n in ("dk1", "dkn", "dv1", "dvn"):
                g[n] = mk()
            for n in WNAMES:
                g[n] = torch.full((Hkv, D), nan, dtype=torch.float32, device=DEV)
            binding.fkv_prefill_backward(L.q, L.k1, L.kn, L.v1, L.vn, L.weights, self.out, self.lse, self.dout,
                                         dq=g["dq"], dk1=g["dk1"], dkn=g["dkn"], dv1=g["dv1"], dvn=g["dvn"],
                                         dweights=[g[n] for n in WNAMES], workspace=ws, causal=self.causal)
        torch.cuda.synchronize()
        return g

    def oracle(self, batch=None, heads=None, fn=bw.backward):
        L = self.L
        h = lambda t: inputs.host_array(t if batch is None else t[batch])
        if self.lite:
            return fn(h(L.q), h(L.kn), h(L.v1), h(self.dout), causal=self.causal, heads=heads)
        w = [x.cpu().numpy() for x in L.weights]
        return fn(h(L.q), h(L.k1), h(L.v1), h(self.dout), h(L.kn), h(L.vn), k_w1=w[0], k_wn=w[1],
                  v_w1=w[2], v_wn=w[3], causal=self.causal, heads=heads)

    def reference(self, batch=None, heads=None):
        """Exact fp64 oracle gradients."""
        return self.oracle(batch, heads)


def rows(x):
    """[..., D] -> [rows, D] float64 (GPU tensors or numpy)."""
    if isinstance(x, torch.Tensor):
        x = x.float().cpu().numpy()
    x = np.asarray(x, dtype=np.float64)
    return x.reshape(-1, x.shape[-1])


def maxrel(x, r):
    x = np.asarray(x, np.float64).ravel()
    r = np.asarray(r, np.float64).ravel()
    m = float(np.max(np.abs(r))) if r.size else 0.0
    return float(np.max(np.abs(x - r))) / (m if m > 0 else 1.0) if r.size else 0.0


def compare(got, ref, names):
    """The fixed bar above, per output tensor, against the exact oracle."""
    for n in names:
        x, r = rows(got[n]), rows(ref[n])
        en, em, ee = rb.normwise(x, r), maxrel(x, r), rb.elementwise(x, r)
        say("  %-6s normwise=%.3e max-relative=%.3e (per-row elementwise %.3e, not bounded)" % (n, en, em, ee))
        assert np.isfinite(x).all(), n
        assert en <= TOL and em <= MAXREL, (n, en, em)


FUSED_NAMES = ("dq", "dk1", "dkn", "dv1", "dvn") + WNAMES
LITE_NAMES = ("dq", "dk", "dv")


@pytest.mark.parametrize("D", [64, 80, 96, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_head_dims_and_gqa_ratios(D, G):
    """Causal, S = 200 (three full 64-row tiles and a ragged 8-row tail; one
    full 128-key tile and a partial one)."""
    say("backward D=%d G=%d B=2 S=200 Hkv=2 causal" % (D, G))
    c = Case(2, 200, 2 * G, 2, D, 2000 + D + G)
    compare(c.run(), c.reference(), FUSED_NAMES)
    c = Case(2, 200, 2 * G, 2, D, 2000 + D + G, lite=True)
    compare(c.run(), c.reference(), LITE_NAMES)


@pytest.mark.parametrize("S", [1, 31, 129, 300])
def test_lengths_and_full_attention(S):
    """Short and ragged lengths, causal and full (no mask)."""
    for causal in (True, False):
        say("backward S=%d causal=%s B=1 Hq=4 Hkv=2 D=128" % (S, causal))
        c = Case(1, S, 4, 2, 128, 2100 + S, causal=causal)
        compare(c.run(), c.reference(), FUSED_NAMES)


@pytest.mark.parametrize("D", [80, 128])
def test_whole_tiles(D):
    """S = 256: every 64-row query tile and 128-key block is whole.  Full
    attention has no masked tile at all (the key-tile kernel's unmasked loop
    alone); causal has masked diagonal tiles before unmasked ones."""
    for causal in (False, True):
        say("backward whole tiles D=%d causal=%s B=1 S=256 Hq=4 Hkv=2" % (D, causal))
        c = Case(1, 256, 4, 2, D, 2400 + D, causal=causal)
        compare(c.run(), c.reference(), FUSED_NAMES)
        c = Case(1, 256, 4, 2, D, 2400 + D, causal=causal, lite=True)
        compare(c.run(), c.reference(), LITE_NAMES)


@pytest.mark.parametrize("D", [96, 128])
def test_long_ragged_full_attention(D):
    """S = 1000 without a mask and G = 4: many query tiles through the
    key-tile kernel's P hand-off and its three tile buffers (at 128
    channels the copy-ahead loop with its buffer index unrolled), every key
    block live, a ragged 40-row tail."""
    say("backward long ragged full B=1 S=1000 Hq=8 Hkv=2 D=%d" % D)
    c = Case(1, 1000, 8, 2, D, 2501, causal=False)
    compare(c.run(), c.reference(), FUSED_NAMES)
    if D == 128:
        c = Case(1, 1000, 8, 2, D, 2502, causal=True, lite=True)
        compare(c.run(), c.reference(), LITE_NAMES)


@pytest.mark.parametrize("layout", ["bhsd", "bshd"])
def test_layouts(layout):
    say("backward layout=%s B=2 S=256 Hq=8 Hkv=4 D=96" % layout)
    c = Case(2, 256, 8, 4, 96, 2200, layout=layout)
    compare(c.run(), c.reference(), FUSED_NAMES)


def test_small_output_gradients():
    """Training-scale output gradients (std 1e-6): the bfloat16 operands
    keep their relative precision where fp16 would underflow."""
    say("backward dO std=1e-6 B=1 S=160 Hq=4 Hkv=2 D=64")
    c = Case(1, 160, 4, 2, 64, 2300, dstd=1e-6)
    compare(c.run(), c.reference(), FUSED_NAMES)


def test_selector_weights_match_lite_bitwise():
    """(a, a', b, b') = (0, 1, 1, 0): the fused kernels read K^n and V^1
    exactly, so dQ, dK^n and dV^1 equal the Lite call's bit for bit and
    dK^1, dV^n are zero."""
    say("backward selector weights vs lite B=2 S=190 Hq=4 Hkv=2 D=80")
    c = Case(2, 190, 4, 2, 80, 2400)
    z = torch.zeros_like(c.L.weights[0])
    o = torch.ones_like(c.L.weights[0])
    c.L.weights = (z, o, o, z)
    c.forward()
    g = c.run()
    lite = Case(2, 190, 4, 2, 80, 2400, lite=True)
    lite.out, lite.lse = c.out, c.lse  # the same forward results: only the backward kernels differ
    gl = lite.run()
    assert torch.equal(g["dq"], gl["dq"]) and torch.equal(g["dkn"], gl["dk"]) and torch.equal(g["dv1"], gl["dv"])
    assert torch.all(g["dk1"] == 0) and torch.all(g["dvn"] == 0)
    compare(g, c.reference(), FUSED_NAMES)


@pytest.mark.parametrize("lite", [False, True])
def test_training_flow_with_library_forward(lite):
    """O and LSE from the library's fkv_prefill, as a training step uses
    them; the same fixed bar."""
    say("backward after library forward lite=%s B=2 S=333 Hq=8 Hkv=4 D=128" % lite)
    c = Case(2, 333, 8, 4, 128, 2450, lite=lite, fwd="library")
    compare(c.run(), c.reference(), LITE_NAMES if lite else FUSED_NAMES)


def test_deterministic():
    say("backward run-to-run determinism B=2 S=300 Hq=16 Hkv=8 D=128")
    c = Case(2, 300, 16, 8, 128, 2500)
    a, b = c.run(), c.run()
    for n in FUSED_NAMES:
        assert torch.equal(a[n], b[n]), n


def _weight_partials(ws, B, Hq, Hkv, S, D):
    """The call's per-(batch, KV head, 128-key tile) weight-gradient partials,
    read from its workspace (fkv_backward_workspace_size's layout: per-row
    LSE and rowsum(dO * O) arrays, each 256-byte aligned, then the partials
    [B, Hkv, ceil(S/128), (a, a', b, b'), D] float32)."""
    r256 = lambda x: (x + 255) // 256 * 256
    rows_b = B * Hq * S * 4
    off = 2 * r256(rows_b)
    nkt = (S + 127) // 128
    n = B * Hkv * nkt * 4 * D
    return ws[off:off + 4 * n].view(torch.float32).view(B, Hkv, nkt, 4, D), nkt


def test_full_size_1p5b_backward():
    """1.5B shape (B=4, S=8192, 16/8 heads, D=128, causal), the benchmarked
    launch, after the library's own forward.  The oracle computes dQ, dK, dV
    of two (batch, KV head) units in full.  The weight gradients sum over
    all 32 units: the per-unit partials the call leaves in its workspace
    (one per 128-key tile) are checked against the oracle's sums over the
    same keys for both units, and the returned gradients against the fp64
    sum of all partials (the reduction)."""
    B, S, Hq, Hkv, D = 4, 8192, 16, 8, 128
    say("backward full size B=%d S=%d Hq=%d Hkv=%d D=%d (sampled units)" % (B, S, Hq, Hkv, D))
    c = Case(B, S, Hq, Hkv, D, 0xF0003, fwd="library")
    L = c.L
    g = {"dq": torch.empty_like(L.q)}
    for n in ("dk1", "dkn", "dv1", "dvn"):
        g[n] = torch.empty(B, S, Hkv, D, dtype=torch.bfloat16, device=DEV)
    for n in WNAMES:
        g[n] = torch.empty(Hkv, D, dtype=torch.float32, device=DEV)
    ws = binding.backward_workspace(L.q, L.k1)
    binding.fkv_prefill_backward(L.q, L.k1, L.kn, L.v1, L.vn, L.weights, c.out, c.lse, c.dout, dq=g["dq"],
                                 dk1=g["dk1"], dkn=g["dkn"], dv1=g["dv1"], dvn=g["dvn"],
                                 dweights=[g[n] for n in WNAMES], workspace=ws, causal=True)
    torch.cuda.synchronize()
    part, nkt = _weight_partials(ws, B, Hq, Hkv, S, D)
    part = part.double().cpu().numpy()
    G = Hq // Hkv
    h = inputs.host_array
    for b, kv in ((0, 0), (B - 1, Hkv - 1)):
        ref = c.reference(batch=[b], heads=[kv])
        got = {"dq": g["dq"][b:b + 1, :, kv * G:(kv + 1) * G], "dk1": g["dk1"][b:b + 1, :, kv:kv + 1],
               "dkn": g["dkn"][b:b + 1, :, kv:kv + 1], "dv1": g["dv1"][b:b + 1, :, kv:kv + 1],
               "dvn": g["dvn"][b:b + 1, :, kv:kv + 1]}
        r = {"dq": ref["dq"][:, :, kv * G:(kv + 1) * G]}
        for n in ("dk1", "dkn", "dv1", "dvn"):
            r[n] = ref[n][:, :, kv:kv + 1]
        say(" unit b=%d g=%d" % (b, kv))
        compare(got, r, ("dq", "dk1", "dkn", "dv1", "dvn"))
        # this unit's weight-gradient partials, tile by tile, from the oracle's
        # fused-key and fused-value gradients and the unit's own sources
        srcs = {"dk_w1": ("dkf", L.k1), "dk_wn": ("dkf", L.kn), "dv_w1": ("dvf", L.v1), "dv_wn": ("dvf", L.vn)}
        for w, n in enumerate(WNAMES):
            gf, src = srcs[n]
            x = bw._f64(h(src[b:b + 1, :, kv:kv + 1]))[0, :, 0, :]       # [S, D]
            d = ref[gf][0, :, kv, :]                                     # [S, D]
            want = np.stack([(d[t * 128:(t + 1) * 128] * x[t * 128:(t + 1) * 128]).sum(axis=0)
                             for t in range(nkt)])                       # [nkt, D]
            gotp = part[b, kv, :, w, :]
            en, em = rb.normwise(gotp, want), maxrel(gotp, want)
            say("  %s partials (%d tiles) normwise=%.3e max-relative=%.3e" % (n, nkt, en, em))
            assert en <= TOL and em <= MAXREL, (n, en, em)
    # the returned weight gradients are the sums of every unit's partials
    for w, n in enumerate(WNAMES):
        want = part[:, :, :, w, :].sum(axis=(0, 2))   # over batch rows and key tiles: [Hkv, D]
        e = rb.normwise(g[n].double().cpu().numpy(), want)
        say("  %s vs fp64 sum of the %d partials: normwise=%.3e" % (n, B * nkt, e))
        assert e <= 1e-5, (n, e)
    del c, g, ws
    torch.cuda.empty_cache()
