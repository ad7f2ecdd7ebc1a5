"""GPU parity of fkv_prefill / fkv_lite_prefill (bf16 data, binary16 matrix-core
operands, tiles fused inside the attention kernel) against the fp64 oracle,
through the C ABI.  Every test prints its case before touching the GPU."""
import numpy as np
import pytest
import torch

from cross_layer_kv_amd import binding, inputs
from parity import gpu_rows, lse_err, oracle_layer, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-2


def run_prefill(L, fused=True, causal=True, single=("kn", "v1")):
    B, S, Hq, D = L.q.shape
    out = torch.full_like(L.q, float("nan"))
    lse = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device=DEV)
    if fused:
        binding.fkv_prefill(L.q, L.k1, L.kn, L.v1, L.vn, L.weights, out=out, lse=lse, causal=causal)
    else:
        binding.fkv_lite_prefill(L.q, getattr(L, single[0]), getattr(L, single[1]), out=out, lse=lse,
                                 causal=causal)
    torch.cuda.synchronize()
    return out, lse


def errors(L, fused=True, causal=True, single=("kn", "v1")):
    B, S, Hq, D = L.q.shape
    ro, rl = oracle_layer(L, fused=fused, causal=causal, single=single)
    out, lse = run_prefill(L, fused, causal, single)
    return rel_err(gpu_rows(out, B, Hq, S, D), ro), lse_err(lse.cpu().numpy().reshape(-1), rl), out, lse


def check(L, fused=True, causal=True, single=("kn", "v1")):
    e, el, out, lse = errors(L, fused, causal, single)
    say("  fused=%s err=%.3e lse_err=%.3e" % (fused, e, el))
    assert e <= TOL and el <= TOL, (e, el)
    return out, lse


@pytest.mark.parametrize("D", [64, 80, 96, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_head_dims_and_gqa_ratios(D, G):
    say("prefill sweep D=%d G=%d B=1 S=200 causal" % (D, G))
    L = inputs.make_layer(1, 200, 200, 2 * G, 2, D, torch.bfloat16, 200 + D + G, DEV, decode=False)
    check(L, fused=True)
    check(L, fused=False)


@pytest.mark.parametrize("S", [1, 63, 64, 65, 130, 257, 600])
def test_ragged_lengths(S):
    say("prefill ragged S=%d D=128 G=2" % S)
    L = inputs.make_layer(2, S, S, 4, 2, 128, torch.bfloat16, 300 + S, DEV, decode=False)
    check(L, fused=True)
    check(L, fused=False)


@pytest.mark.parametrize("D", [80, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_reference_max_raised_mid_row(D, causal):
    """Keys of the first 64-key tile scaled by 0.05 and all later keys by 3:
    in about half of the rows the second tile's max exceeds the running max
    by more than 8 log2 units, so the accumulator rescale (and, at D <= 96,
    the re-base of the score chains on a non-zero reference) runs in the
    middle of a row.  Scores stay within ~30 log2 units."""
    say("prefill mid-row max raises D=%d causal=%s S=320" % (D, causal))
    S = 320
    L = inputs.make_layer(1, S, S, 4, 2, D, torch.bfloat16, 500 + D, DEV, decode=False)
    ramp = torch.where(torch.arange(S, device=DEV) < 64, 0.05, 3.0).to(torch.bfloat16).view(1, S, 1, 1)
    for t in (L.k1, L.kn):
        t.mul_(ramp)
    check(L, fused=True, causal=causal)
    check(L, fused=False, causal=causal)


def _wide_ramp_layer(D, seed):
    """Keys of 64-key tile j scaled by (1 + 3j) over five tiles: late keys
    reach ~13x their N(0,1) size, so causal rows see scores near 100 log2
    units and a near one-hot softmax."""
    S = 320
    L = inputs.make_layer(1, S, S, 4, 2, D, torch.bfloat16, seed, DEV, decode=False)
    ramp = (1.0 + 3.0 * (torch.arange(S, device=DEV) // 64).float()).to(torch.bfloat16).view(1, S, 1, 1)
    for t in (L.k1, L.kn):
        t.mul_(ramp)
    return L


@pytest.mark.xfail(reason="binary16 operand limit: scores near 100 log2 units carry ~2^-11 relative rounding "
                          "of the fused keys and the queries, which moves exponents by ~0.05 and the output by "
                          "2-3e-2 (measured 2.57e-2 at D = 80); documented with fkv_prefill", strict=False)
@pytest.mark.parametrize("D", [80, 128])
def test_wide_score_range_binary16_limit(D):
    """The binary16 operand limit stated with fkv_prefill: a row whose scores
    span ~100 log2 units.  Recorded as an expected failure with its measured
    error; the finite-output part is asserted before the tolerance."""
    say("prefill wide score range (keys x(1+3j) per tile) D=%d S=320" % D)
    L = _wide_ramp_layer(D, 520 + D)
    e, el, out, lse = errors(L, fused=True, causal=True)
    say("  err=%.3e lse_err=%.3e (tolerance %.0e)" % (e, el, TOL))
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    assert e <= TOL and el <= TOL, (e, el)


@pytest.mark.parametrize("D", [80, 128])
def test_non_causal(D):
    say("prefill non-causal D=%d S=190" % D)
    L = inputs.make_layer(1, 190, 190, 4, 2, D, torch.bfloat16, 400 + D, DEV, decode=False)
    check(L, fused=True, causal=False)
    check(L, fused=False, causal=False)


@pytest.mark.parametrize("layout", ["bhsd", "bshd"])
def test_layouts(layout):
    say("prefill layout=%s" % layout)
    L = inputs.make_layer(2, 300, 300, 16, 8, 96, torch.bfloat16, 500, DEV, layout=layout, decode=False)
    check(L, fused=True)


def test_selector_weights_equal_lite_bitwise():
    """(0, 1, 1, 0) weights give K~ = K^n and V~ = V^1 exactly (also after the
    binary16 rounding of the fused tiles), so the fused kernel must equal the
    Lite kernel bit for bit."""
    say("prefill selector weights vs lite")
    L = inputs.make_layer(1, 333, 333, 8, 4, 80, torch.bfloat16, 600, DEV, decode=False)
    z = torch.zeros_like(L.weights[0])
    o = torch.ones_like(L.weights[0])
    L.weights = (z, o, o, z)
    of, lf = run_prefill(L, fused=True)
    ol, ll = run_prefill(L, fused=False)
    assert torch.equal(of, ol) and torch.equal(lf, ll)


def test_vanilla_control_on_own_caches():
    say("prefill vanilla control (K1, V1)")
    L = inputs.make_layer(1, 257, 257, 16, 8, 128, torch.bfloat16, 700, DEV, decode=False)
    check(L, fused=False, single=("k1", "v1"))


def _sample_rows(B, Hq, S, bm, rng, per_bh=16):
    """Stratified rows: first/last rows, rows around every tile boundary and
    random rows for a few (b, h) pairs."""
    rows = []
    bhs = [(0, 0), (B - 1, Hq - 1), (int(rng.integers(B)), int(rng.integers(Hq)))]
    for b, h in bhs:
        ps = {0, 1, S - 1, S - 2}
        for t in range(bm, S, bm):
            ps.update({t - 1, t})
        ps.update(int(x) for x in rng.integers(0, S, size=per_bh))
        rows += [(b * Hq + h) * S + p for p in sorted(ps) if 0 <= p < S]
    return np.array(sorted(set(rows)), dtype=np.int64)


def _unit_rows(b, g, G, Hq, S):
    """Every row of one (batch, KV head) unit: its G query heads x S rows."""
    return np.array([(b * Hq + h) * S + p for h in range(g * G, (g + 1) * G) for p in range(S)], dtype=np.int64)


def _full_size(B, S, Hq, Hkv, D, seed):
    """The benchmarked launch.  FusedKV: every row of two whole (batch, KV
    head) units -- the first, and the last, which holds the last work item of
    the XCD-aware mapping -- plus rows around every tile boundary of three
    (b, h) pairs.  Lite: the stratified rows."""
    say("prefill full size B=%d S=%d Hq=%d Hkv=%d D=%d seed=%#x" % (B, S, Hq, Hkv, D, seed))
    G = Hq // Hkv
    L = inputs.make_layer(B, S, S, Hq, Hkv, D, torch.bfloat16, seed, DEV, decode=False)
    rng = np.random.default_rng(seed)
    sample = _sample_rows(B, Hq, S, 256 // G, rng)
    for fused in (True, False):
        out, lse = run_prefill(L, fused=fused)
        assert torch.isfinite(out).all() and torch.isfinite(lse).all()
        got_all = gpu_rows(out, B, Hq, S, D)
        lse_all = lse.cpu().numpy().reshape(-1)
        sets = [("sample", sample)]
        if fused:
            sets += [("unit(0,0)", _unit_rows(0, 0, G, Hq, S)), ("unit(%d,%d)" % (B - 1, Hkv - 1),
                                                                  _unit_rows(B - 1, Hkv - 1, G, Hq, S))]
        for name, rows in sets:
            ro, rl = oracle_layer(L, fused=fused, causal=True, rows=rows)
            e = rel_err(got_all[rows], ro)
            el = lse_err(lse_all[rows], rl)
            say("  fused=%s %s rows=%d (G*S=%d) err=%.3e lse_err=%.3e" % (fused, name, rows.size, G * S, e, el))
            assert e <= TOL and el <= TOL
    del L
    torch.cuda.empty_cache()


def test_full_size_1p5b_prefill():
    """1.5B shape: B=4, S=8192, 16/8 heads, D=128 (the benchmarked launch)."""
    _full_size(4, 8192, 16, 8, 128, 0xF0003)


def test_full_size_4b_prefill():
    """4B shape: B=1, S=16384, 32/16 heads, D=80."""
    _full_size(1, 16384, 32, 16, 80, 0xF0004)


@pytest.mark.parametrize("S", [200, 4100])
def test_first_token_row_equals_decode(S):
    """Time to first token needs only the final prompt position of a
    reconstruction layer.  Under the causal mask that row sees every cached
    token, so a decode with the same query (position S-1) over the S-token
    caches must reproduce the final prefill row and its LSE; both are checked
    against the oracle's causal row S-1 and against each other."""
    say("ttft: decode at S=%d vs causal prefill row S-1 (B=2 16/8 D=128)" % S)
    B, Hq, Hkv, D = 2, 16, 8, 128
    L = inputs.make_layer(B, S, S, Hq, Hkv, D, torch.bfloat16, 800 + S, DEV, decode=False)
    out_p, lse_p = run_prefill(L, fused=True)
    qlast = L.q[:, S - 1:S].contiguous()
    out_d = torch.full_like(qlast, float("nan"))
    lse_d = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
    binding.fkv_decode(qlast, L.k1, L.kn, L.v1, L.vn, L.weights, out=out_d, lse=lse_d,
                       workspace=binding.decode_workspace(qlast, L.k1))
    torch.cuda.synchronize()
    rows = np.array([(b * Hq + h) * S + S - 1 for b in range(B) for h in range(Hq)], dtype=np.int64)
    ro, rl = oracle_layer(L, fused=True, causal=True, rows=rows)
    got_d = gpu_rows(out_d, B, Hq, 1, D)
    got_p = gpu_rows(out_p[:, S - 1:S], B, Hq, 1, D)
    e_d, e_p = rel_err(got_d, ro), rel_err(got_p, ro)
    el_d = lse_err(lse_d.cpu().numpy().reshape(-1), rl)
    el_p = lse_err(lse_p[:, :, S - 1].cpu().numpy().reshape(-1), rl)
    e_pd = rel_err(got_p, got_d)
    say("  decode err=%.3e lse=%.3e  prefill err=%.3e lse=%.3e  prefill-vs-decode %.3e"
        % (e_d, el_d, e_p, el_p, e_pd))
    assert e_d <= TOL and el_d <= TOL and e_p <= TOL and el_p <= TOL and e_pd <= TOL
