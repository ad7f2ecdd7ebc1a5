// fkv_api.cpp -- host side of libfusedkv: argument validation, work planning
// and the exported C entry points.  No HIP headers: every check here reads
// only the host-side parameter structs and pointer values, so an invalid call
// returns before anything is enqueued.  The device work is in
// fkv_decode.hip / fkv_prefill.hip.
#include "fusedkv.h"
#include "fkv_internal.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>

namespace {

thread_local char g_last_error[256] = "";

fkv_status fail(fkv_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    if (std::getenv("FKV_LOG")) std::fprintf(stderr, "libfusedkv: %s\n", g_last_error);
    return s;
}

fkv_status ok()
{
    g_last_error[0] = '\0';
    return FKV_SUCCESS;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elt_size(int32_t dtype) { return dtype == FKV_F32 ? 4 : 2; }

bool supported_head_dim(int32_t d) { return d == 64 || d == 80 || d == 96 || d == 128; }

// GQA ratios: 1, 2, 4, 8 (all kernels) and 64 (decode on the matrix cores,
// bfloat16 only; prefill rejects it).
bool supported_group(int32_t g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == fkv::kHighGqa; }

// Shape checks common to decode and prefill.
fkv_status check_shape(const fkv_params* p)
{
    if (!p) return fail(FKV_ERROR_INVALID_VALUE, "params is NULL");
    if (p->batch < 0 || p->seqlen_q < 0 || p->seqlen_k < 0)
        return fail(FKV_ERROR_INVALID_VALUE, "negative batch or sequence length");
    if (p->num_kv_heads < 1 || p->num_q_heads < 1)
        return fail(FKV_ERROR_INVALID_VALUE, "head counts must be >= 1");
    if (p->num_q_heads % p->num_kv_heads != 0)
        return fail(FKV_ERROR_INVALID_VALUE, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                    p->num_q_heads, p->num_kv_heads);
    if (p->dtype != FKV_F32 && p->dtype != FKV_BF16)
        return fail(FKV_ERROR_INVALID_VALUE, "unknown dtype %d", p->dtype);
    if (!std::isfinite(p->softmax_scale) || p->softmax_scale < 0.0f)
        return fail(FKV_ERROR_INVALID_VALUE, "softmax_scale must be finite and >= 0 (0 = 1/sqrt(D))");
    if (!supported_head_dim(p->head_dim))
        return fail(FKV_ERROR_UNSUPPORTED, "head_dim %d not in {64, 80, 96, 128}", p->head_dim);
    if (!supported_group(p->num_q_heads / p->num_kv_heads))
        return fail(FKV_ERROR_UNSUPPORTED, "GQA ratio %d not in {1, 2, 4, 8, 64}",
                    p->num_q_heads / p->num_kv_heads);
    return FKV_SUCCESS;
}

// A cache view is usable when its base and every row start are 16-byte
// aligned and its strides are non-negative.
fkv_status check_cache(const fkv_params* p, const fkv_cache& c, const char* name)
{
    if (!c.data && p->seqlen_k == 0) return FKV_SUCCESS;  // an empty cache is never read
    if (!c.data) return fail(FKV_ERROR_INVALID_VALUE, "%s.data is NULL", name);
    if (!aligned16(c.data)) return fail(FKV_ERROR_INVALID_VALUE, "%s.data is not 16-byte aligned", name);
    if (c.stride_b < 0 || c.stride_s < 0 || c.stride_h < 0)
        return fail(FKV_ERROR_INVALID_VALUE, "%s has a negative stride", name);
    const int64_t e = (int64_t)elt_size(p->dtype);
    if ((c.stride_b * e) % 16 || (c.stride_s * e) % 16 || (c.stride_h * e) % 16)
        return fail(FKV_ERROR_INVALID_VALUE, "%s strides do not keep rows 16-byte aligned", name);
    if (p->seqlen_k > 1 && c.stride_s < p->head_dim)
        return fail(FKV_ERROR_INVALID_VALUE, "%s token stride overlaps a row", name);
    return FKV_SUCCESS;
}

fkv::View view_of(const fkv_cache& c)
{
    return fkv::View{c.data, c.stride_b, c.stride_s, c.stride_h};
}

float scale_log2_of(const fkv_params* p)
{
    const double s = p->softmax_scale != 0.0f ? (double)p->softmax_scale
                                              : 1.0 / std::sqrt((double)p->head_dim);
    return (float)(s * 1.4426950408889634); // log2(e)
}

// Split plan for decode.  A workgroup of `waves` waves (decode_waves) fills
// one compute unit, so the plan aims at one workgroup per CU of a 256-CU
// part: one split per (batch, KV head) when there are at least 256 of them,
// otherwise enough splits of the key axis to reach 256 workgroups, each split
// covering at least one workgroup iteration (waves * decode_wave_tokens).  Splits are
// multiples of 64 tokens and at most 256.  The plan depends on the
// parameters only (no device query), so the workspace size is a pure function
// of them.  FKV_DECODE_SPLITS overrides the split count (tuning and tests).
fkv::DecodePlan plan_decode(const fkv_params* p, bool fused, bool kivi = false)
{
    fkv::DecodePlan pl{};
    const int64_t G = p->num_q_heads / p->num_kv_heads;
    pl.waves = kivi ? fkv::kivi_waves(fused, (int)G, p->head_dim) : fkv::decode_waves(p->dtype == FKV_F32, fused, (int)G);
    const int64_t units = (int64_t)p->batch * p->num_kv_heads;
    const int64_t S = p->seqlen_k;
    // G = 64 runs the matrix-core kernel: 64-token tiles, and it aims at two
    // workgroups per CU
    const bool wide = G == fkv::kHighGqa;
    const int64_t iter = wide ? 64 : (int64_t)pl.waves * (kivi ? 32 : fkv::decode_wave_tokens(p->dtype == FKV_F32, fused, (int)G, p->head_dim));
    // (the 8-wave 4-bit single-source kernel fits two workgroups per CU)
    const int64_t target = (wide || (kivi && !fused && pl.waves == 8)) ? 512 : 256;
    const int64_t max_splits = S > 0 ? (S + iter - 1) / iter : 1;
    int64_t ns = units > 0 ? (target + units - 1) / units : 1;
    if (const char* env = std::getenv("FKV_DECODE_SPLITS")) {
        const long v = std::strtol(env, nullptr, 10);
        if (v > 0) ns = v;
    } else if (ns > max_splits) {
        ns = max_splits;
    }
    if (ns > 256) ns = 256;
    if (ns < 1) ns = 1;
    int64_t chunk = S > 0 ? (S + ns - 1) / ns : 64;
    chunk = (chunk + 63) / 64 * 64;
    ns = S > 0 ? (S + chunk - 1) / chunk : 1;
    pl.n_splits = (int32_t)ns;
    pl.chunk = (int32_t)chunk;
    if (ns > 1) {
        pl.ml_bytes = (size_t)((units * ns * G * 2 * 4 + 255) / 256 * 256);
        pl.part_bytes = (size_t)(units * ns * G * p->head_dim * 4);
    }
    pl.total_bytes = pl.ml_bytes + pl.part_bytes;
    return pl;
}

// noalloc: the split partials go to the library's static device scratch
// (fkv_decode_noalloc) instead of a caller workspace.
fkv_status decode_common(const fkv_params* p, const void* q, const fkv_cache* caches,
                         const char* const* names, int ncaches, const fkv_fusion* fusion,
                         const int32_t* seqlens_k, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream, bool noalloc = false)
{
    fkv_status s = check_shape(p);
    if (s) return s;
    if (p->seqlen_q != 1) return fail(FKV_ERROR_INVALID_VALUE, "decode needs seqlen_q == 1 (got %d)", p->seqlen_q);
    if (p->batch == 0) return ok();
    if (!q || !out) return fail(FKV_ERROR_INVALID_VALUE, "q or out is NULL");
    if (!aligned16(q) || !aligned16(out)) return fail(FKV_ERROR_INVALID_VALUE, "q or out is not 16-byte aligned");
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u))
        return fail(FKV_ERROR_INVALID_VALUE, "lse is not 4-byte aligned");
    if (seqlens_k && (reinterpret_cast<uintptr_t>(seqlens_k) & 3u))
        return fail(FKV_ERROR_INVALID_VALUE, "seqlens_k is not 4-byte aligned");
    for (int i = 0; i < ncaches; ++i)
        if ((s = check_cache(p, caches[i], names[i]))) return s;
    const bool fused = ncaches == 4;
    const bool wide = p->num_q_heads / p->num_kv_heads == fkv::kHighGqa;
    if (wide && p->dtype != FKV_BF16)
        return fail(FKV_ERROR_UNSUPPORTED, "GQA ratio %d decode runs on the matrix cores: bfloat16 only", fkv::kHighGqa);
    if (fused) {
        if (!fusion || !fusion->k_w1 || !fusion->k_wn || !fusion->v_w1 || !fusion->v_wn)
            return fail(FKV_ERROR_INVALID_VALUE, "fusion weights missing");
        if (!aligned16(fusion->k_w1) || !aligned16(fusion->k_wn) || !aligned16(fusion->v_w1) ||
            !aligned16(fusion->v_wn))
            return fail(FKV_ERROR_INVALID_VALUE, "fusion weights are not 16-byte aligned");
    }
    const fkv::DecodePlan pl = plan_decode(p, fused);
    if (noalloc && pl.total_bytes > 0) {
        if (pl.total_bytes > fkv::kNoallocScratchBytes)
            return fail(FKV_ERROR_WORKSPACE, "split partials need %zu bytes; the static scratch holds %zu "
                        "(use fkv_decode with a workspace)", pl.total_bytes, fkv::kNoallocScratchBytes);
        const int rc = fkv::scratch_pointer(&workspace);
        if (rc) return fail(FKV_ERROR_LAUNCH, "static scratch address lookup failed (HIP error %d)", rc);
        workspace_bytes = fkv::kNoallocScratchBytes;
    }
    if (pl.total_bytes > 0) {
        if (!workspace || workspace_bytes < pl.total_bytes)
            return fail(FKV_ERROR_WORKSPACE, "workspace needs %zu bytes (got %zu)", pl.total_bytes,
                        workspace ? workspace_bytes : (size_t)0);
        if (reinterpret_cast<uintptr_t>(workspace) & 255u)
            return fail(FKV_ERROR_WORKSPACE, "workspace is not 256-byte aligned");
    }

    fkv::DecodeArgs a{};
    a.q = q;
    a.k1 = view_of(caches[0]);
    a.v1 = view_of(caches[fused ? 2 : 1]);
    if (fused) {
        a.kn = view_of(caches[1]);
        a.vn = view_of(caches[3]);
        a.kw1 = fusion->k_w1;
        a.kwn = fusion->k_wn;
        a.vw1 = fusion->v_w1;
        a.vwn = fusion->v_wn;
    }
    a.seqlens = seqlens_k;
    a.out = out;
    a.lse = lse;
    char* ws = static_cast<char*>(workspace);
    a.ml = pl.total_bytes ? reinterpret_cast<float*>(ws) : nullptr;
    a.part = pl.total_bytes ? reinterpret_cast<float*>(ws + pl.ml_bytes) : nullptr;
    a.B = p->batch;
    a.Sk = p->seqlen_k;
    a.Hq = p->num_q_heads;
    a.Hkv = p->num_kv_heads;
    a.D = p->head_dim;
    a.G = p->num_q_heads / p->num_kv_heads;
    a.n_splits = pl.n_splits;
    a.chunk = pl.chunk;
    a.scale_log2 = scale_log2_of(p);
    if (std::getenv("FKV_TRACE"))
        std::fprintf(stderr, "libfusedkv: decode %s B=%d Sk=%d Hq=%d Hkv=%d D=%d waves=%d splits=%d chunk=%d\n",
                     fused ? "fused" : "single", a.B, a.Sk, a.Hq, a.Hkv, a.D, pl.waves, a.n_splits, a.chunk);
    const int rc = wide ? fkv::launch_decode_hgqa(a, fused, stream)
                        : fkv::launch_decode(a, fused, p->dtype, pl.waves, stream);
    if (rc) return fail(FKV_ERROR_LAUNCH, "decode launch failed (HIP error %d)", rc);
    return ok();
}

fkv_status prefill_common(const fkv_params* p, const void* q, const fkv_cache* caches,
                          const char* const* names, int ncaches, const fkv_fusion* fusion,
                          void* out, float* lse, void* stream)
{
    fkv_status s = check_shape(p);
    if (s) return s;
    if (p->dtype != FKV_BF16) return fail(FKV_ERROR_UNSUPPORTED, "prefill supports bfloat16 data only");
    if (p->seqlen_q != p->seqlen_k)
        return fail(FKV_ERROR_UNSUPPORTED, "prefill needs seqlen_q == seqlen_k (got %d, %d)", p->seqlen_q,
                    p->seqlen_k);
    if (p->causal != 0 && p->causal != 1) return fail(FKV_ERROR_INVALID_VALUE, "causal must be 0 or 1");
    if (p->batch == 0 || p->seqlen_q == 0) return ok();
    if (!q || !out) return fail(FKV_ERROR_INVALID_VALUE, "q or out is NULL");
    if (!aligned16(q) || !aligned16(out)) return fail(FKV_ERROR_INVALID_VALUE, "q or out is not 16-byte aligned");
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u))
        return fail(FKV_ERROR_INVALID_VALUE, "lse is not 4-byte aligned");
    for (int i = 0; i < ncaches; ++i)
        if ((s = check_cache(p, caches[i], names[i]))) return s;
    const bool fused = ncaches == 4;
    const bool wide = p->num_q_heads / p->num_kv_heads == fkv::kHighGqa;
    if (wide && p->dtype != FKV_BF16)
        return fail(FKV_ERROR_UNSUPPORTED, "GQA ratio %d decode runs on the matrix cores: bfloat16 only", fkv::kHighGqa);
    if (fused) {
        if (!fusion || !fusion->k_w1 || !fusion->k_wn || !fusion->v_w1 || !fusion->v_wn)
            return fail(FKV_ERROR_INVALID_VALUE, "fusion weights missing");
        if (!aligned16(fusion->k_w1) || !aligned16(fusion->k_wn) || !aligned16(fusion->v_w1) ||
            !aligned16(fusion->v_wn))
            return fail(FKV_ERROR_INVALID_VALUE, "fusion weights are not 16-byte aligned");
    }
    for (int i = 0; i < ncaches; ++i) {
        // each (batch, KV head) slab is read through a 32-bit buffer range
        const int64_t span = ((int64_t)(p->seqlen_k - 1) * caches[i].stride_s + p->head_dim) * 2;
        if (span >= ((int64_t)1 << 31))
            return fail(FKV_ERROR_UNSUPPORTED, "%s: one head's rows span %lld bytes (limit 2^31)", names[i],
                        (long long)span);
    }
    const int G = p->num_q_heads / p->num_kv_heads;
    const int bm = fkv::prefill_rows_per_tile(G);
    if (bm <= 0) return fail(FKV_ERROR_UNSUPPORTED, "GQA ratio %d not supported by prefill", G);

    fkv::PrefillArgs a{};
    a.q = q;
    a.k1 = view_of(caches[0]);
    a.v1 = view_of(caches[fused ? 2 : 1]);
    if (fused) {
        a.kn = view_of(caches[1]);
        a.vn = view_of(caches[3]);
        a.kw1 = fusion->k_w1;
        a.kwn = fusion->k_wn;
        a.vw1 = fusion->v_w1;
        a.vwn = fusion->v_wn;
    }
    a.out = out;
    a.lse = lse;
    a.B = p->batch;
    a.S = p->seqlen_q;
    a.Hq = p->num_q_heads;
    a.Hkv = p->num_kv_heads;
    a.D = p->head_dim;
    a.G = G;
    a.causal = p->causal;
    a.n_qtiles = (p->seqlen_q + bm - 1) / bm;
    a.scale_log2 = scale_log2_of(p);
    if (std::getenv("FKV_TRACE"))
        std::fprintf(stderr, "libfusedkv: prefill %s B=%d S=%d Hq=%d Hkv=%d D=%d qtiles=%d causal=%d\n",
                     fused ? "fused" : "single", a.B, a.S, a.Hq, a.Hkv, a.D, a.n_qtiles, a.causal);
    const int rc = fkv::launch_prefill(a, fused, stream);
    if (rc) return fail(FKV_ERROR_LAUNCH, "prefill launch failed (HIP error %d)", rc);
    return ok();
}

// ---- KIVI-style 4-bit caches ----

int64_t kivi_key_groups(int64_t S) { return (S + 31) / 32; }
int64_t kivi_value_groups(int64_t D) { return (D + 31) / 32; }

fkv_status check_q4(const fkv_params* p, const fkv_q4_cache& c, const char* name)
{
    if (p->seqlen_k == 0) return FKV_SUCCESS;  // an empty cache is never read
    if (!c.codes || !c.scale || !c.minv) return fail(FKV_ERROR_INVALID_VALUE, "%s has a NULL array", name);
    if (!aligned16(c.codes) || !aligned16(c.scale) || !aligned16(c.minv))
        return fail(FKV_ERROR_INVALID_VALUE, "%s arrays are not 16-byte aligned", name);
    return FKV_SUCCESS;
}

fkv::Q4View q4_of(const fkv_q4_cache& c) { return fkv::Q4View{c.codes, c.scale, c.minv}; }

fkv_status kivi_decode_common(const fkv_params* p, const void* q, const fkv_q4_cache* caches,
                              const char* const* names, int ncaches, const fkv_fusion* fusion,
                              const int32_t* seqlens_k, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream)
{
    fkv_status s = check_shape(p);
    if (s) return s;
    if (p->dtype != FKV_BF16) return fail(FKV_ERROR_UNSUPPORTED, "4-bit decode takes bfloat16 queries and outputs");
    if (p->num_q_heads / p->num_kv_heads == fkv::kHighGqa)
        return fail(FKV_ERROR_UNSUPPORTED, "4-bit decode supports GQA ratios 1, 2, 4, 8");
    if (p->seqlen_q != 1) return fail(FKV_ERROR_INVALID_VALUE, "decode needs seqlen_q == 1 (got %d)", p->seqlen_q);
    if (p->batch == 0) return ok();
    if (!q || !out) return fail(FKV_ERROR_INVALID_VALUE, "q or out is NULL");
    if (!aligned16(q) || !aligned16(out)) return fail(FKV_ERROR_INVALID_VALUE, "q or out is not 16-byte aligned");
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u))
        return fail(FKV_ERROR_INVALID_VALUE, "lse is not 4-byte aligned");
    if (seqlens_k && (reinterpret_cast<uintptr_t>(seqlens_k) & 3u))
        return fail(FKV_ERROR_INVALID_VALUE, "seqlens_k is not 4-byte aligned");
    for (int i = 0; i < ncaches; ++i)
        if ((s = check_q4(p, caches[i], names[i]))) return s;
    const bool fused = ncaches == 4;
    if (fused) {
        if (!fusion || !fusion->k_w1 || !fusion->k_wn || !fusion->v_w1 || !fusion->v_wn)
            return fail(FKV_ERROR_INVALID_VALUE, "fusion weights missing");
        if (!aligned16(fusion->k_w1) || !aligned16(fusion->k_wn) || !aligned16(fusion->v_w1) ||
            !aligned16(fusion->v_wn))
            return fail(FKV_ERROR_INVALID_VALUE, "fusion weights are not 16-byte aligned");
    }
    const fkv::DecodePlan pl = plan_decode(p, fused, true);
    if (pl.total_bytes > 0) {
        if (!workspace || workspace_bytes < pl.total_bytes)
            return fail(FKV_ERROR_WORKSPACE, "workspace needs %zu bytes (got %zu)", pl.total_bytes,
                        workspace ? workspace_bytes : (size_t)0);
        if (reinterpret_cast<uintptr_t>(workspace) & 255u)
            return fail(FKV_ERROR_WORKSPACE, "workspace is not 256-byte aligned");
    }
    fkv::KiviDecodeArgs a{};
    a.q = q;
    a.qk1 = q4_of(caches[0]);
    a.qv1 = q4_of(caches[fused ? 2 : 1]);
    if (fused) {
        a.qkn = q4_of(caches[1]);
        a.qvn = q4_of(caches[3]);
        a.kw1 = fusion->k_w1;
        a.kwn = fusion->k_wn;
        a.vw1 = fusion->v_w1;
        a.vwn = fusion->v_wn;
    }
    a.seqlens = seqlens_k;
    a.out = out;
    a.lse = lse;
    char* ws = static_cast<char*>(workspace);
    a.ml = pl.total_bytes ? reinterpret_cast<float*>(ws) : nullptr;
    a.part = pl.total_bytes ? reinterpret_cast<float*>(ws + pl.ml_bytes) : nullptr;
    a.B = p->batch;
    a.Sk = p->seqlen_k;
    a.Hq = p->num_q_heads;
    a.Hkv = p->num_kv_heads;
    a.D = p->head_dim;
    a.G = p->num_q_heads / p->num_kv_heads;
    a.n_splits = pl.n_splits;
    a.chunk = pl.chunk;
    a.scale_log2 = scale_log2_of(p);
    if (std::getenv("FKV_TRACE"))
        std::fprintf(stderr, "libfusedkv: 4-bit decode %s B=%d Sk=%d Hq=%d Hkv=%d D=%d waves=%d splits=%d chunk=%d\n",
                     fused ? "fused" : "single", a.B, a.Sk, a.Hq, a.Hkv, a.D, pl.waves, a.n_splits, a.chunk);
    const int rc = fkv::launch_kivi_decode(a, fused, pl.waves, stream);
    if (rc) return fail(FKV_ERROR_LAUNCH, "4-bit decode launch failed (HIP error %d)", rc);
    return ok();
}

// ---- backward ----

struct BwdLayout {
    size_t lse2, delta, wpart, total;
    int32_t nkt;
};

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

BwdLayout backward_layout(const fkv_params* p)
{
    BwdLayout l{};
    l.nkt = (p->seqlen_k + fkv::kBwdKeyTile - 1) / fkv::kBwdKeyTile;
    const size_t rows = (size_t)p->batch * p->num_q_heads * p->seqlen_q * 4;
    l.lse2 = 0;
    l.delta = round256(rows);
    l.wpart = l.delta + round256(rows);
    l.total = l.wpart + round256((size_t)p->batch * p->num_kv_heads * l.nkt * 4 * p->head_dim * 4);
    return l;
}

fkv_status check_grad(const fkv_params* p, const fkv_grad& c, const char* name)
{
    const fkv_cache v{c.data, c.stride_b, c.stride_s, c.stride_h};
    if (!c.data) return fail(FKV_ERROR_INVALID_VALUE, "%s.data is NULL", name);
    return check_cache(p, v, name);
}

fkv::OutView out_of(const fkv_grad& c) { return fkv::OutView{c.data, c.stride_b, c.stride_s, c.stride_h}; }

fkv_status backward_common(const fkv_params* p, const void* q, const fkv_cache* caches, const char* const* names,
                           int ncaches, const fkv_fusion* fusion, const void* out, const float* lse, const void* dout,
                           void* dq, const fkv_grad* grads, const char* const* gnames, const fkv_fusion_grad* dfusion,
                           void* workspace, size_t workspace_bytes, void* stream)
{
    fkv_status s = check_shape(p);
    if (s) return s;
    if (p->dtype != FKV_BF16) return fail(FKV_ERROR_UNSUPPORTED, "the backward pass supports bfloat16 data only");
    if (p->seqlen_q != p->seqlen_k)
        return fail(FKV_ERROR_UNSUPPORTED, "the backward pass needs seqlen_q == seqlen_k (got %d, %d)", p->seqlen_q,
                    p->seqlen_k);
    if (p->causal != 0 && p->causal != 1) return fail(FKV_ERROR_INVALID_VALUE, "causal must be 0 or 1");
    const int G = p->num_q_heads / p->num_kv_heads;
    if (G == fkv::kHighGqa) return fail(FKV_ERROR_UNSUPPORTED, "the backward pass supports GQA ratios 1, 2, 4, 8");
    if (p->batch == 0 || p->seqlen_q == 0) return ok();
    if (!q || !out || !dout || !dq || !lse) return fail(FKV_ERROR_INVALID_VALUE, "q, out, dout, dq or lse is NULL");
    if (!aligned16(q) || !aligned16(out) || !aligned16(dout) || !aligned16(dq))
        return fail(FKV_ERROR_INVALID_VALUE, "q, out, dout or dq is not 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(FKV_ERROR_INVALID_VALUE, "lse is not 4-byte aligned");
    for (int i = 0; i < ncaches; ++i)
        if ((s = check_cache(p, caches[i], names[i]))) return s;
    for (int i = 0; i < ncaches; ++i)
        if ((s = check_grad(p, grads[i], gnames[i]))) return s;
    const bool fused = ncaches == 4;
    if (fused) {
        if (!fusion || !fusion->k_w1 || !fusion->k_wn || !fusion->v_w1 || !fusion->v_wn)
            return fail(FKV_ERROR_INVALID_VALUE, "fusion weights missing");
        if (!aligned16(fusion->k_w1) || !aligned16(fusion->k_wn) || !aligned16(fusion->v_w1) ||
            !aligned16(fusion->v_wn))
            return fail(FKV_ERROR_INVALID_VALUE, "fusion weights are not 16-byte aligned");
        if (!dfusion || !dfusion->k_w1 || !dfusion->k_wn || !dfusion->v_w1 || !dfusion->v_wn)
            return fail(FKV_ERROR_INVALID_VALUE, "fusion weight gradients missing");
        const float* d4[4] = {dfusion->k_w1, dfusion->k_wn, dfusion->v_w1, dfusion->v_wn};
        for (const float* d : d4)
            if (reinterpret_cast<uintptr_t>(d) & 3u)
                return fail(FKV_ERROR_INVALID_VALUE, "fusion weight gradients are not 4-byte aligned");
    }
    const BwdLayout lay = backward_layout(p);
    if (!workspace || workspace_bytes < lay.total)
        return fail(FKV_ERROR_WORKSPACE, "workspace needs %zu bytes (got %zu)", lay.total,
                    workspace ? workspace_bytes : (size_t)0);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(FKV_ERROR_WORKSPACE, "workspace is not 256-byte aligned");

    fkv::BwdArgs a{};
    a.q = q;
    a.k1 = view_of(caches[0]);
    a.v1 = view_of(caches[fused ? 2 : 1]);
    a.dk1 = out_of(grads[0]);
    a.dv1 = out_of(grads[fused ? 2 : 1]);
    if (fused) {
        a.kn = view_of(caches[1]);
        a.vn = view_of(caches[3]);
        a.dkn = out_of(grads[1]);
        a.dvn = out_of(grads[3]);
        a.kw1 = fusion->k_w1;
        a.kwn = fusion->k_wn;
        a.vw1 = fusion->v_w1;
        a.vwn = fusion->v_wn;
        a.dkw1 = dfusion->k_w1;
        a.dkwn = dfusion->k_wn;
        a.dvw1 = dfusion->v_w1;
        a.dvwn = dfusion->v_wn;
    }
    a.out = out;
    a.lse = lse;
    a.dout = dout;
    a.dq = dq;
    char* ws = static_cast<char*>(workspace);
    a.lse2 = reinterpret_cast<float*>(ws + lay.lse2);
    a.delta = reinterpret_cast<float*>(ws + lay.delta);
    a.wpart = reinterpret_cast<float*>(ws + lay.wpart);
    a.B = p->batch;
    a.S = p->seqlen_q;
    a.Hq = p->num_q_heads;
    a.Hkv = p->num_kv_heads;
    a.D = p->head_dim;
    a.G = G;
    a.causal = p->causal;
    a.nkt = lay.nkt;
    a.scale_log2 = scale_log2_of(p);
    a.scale = (float)(p->softmax_scale != 0.0f ? (double)p->softmax_scale : 1.0 / std::sqrt((double)p->head_dim));
    if (std::getenv("FKV_TRACE"))
        std::fprintf(stderr, "libfusedkv: backward %s B=%d S=%d Hq=%d Hkv=%d D=%d causal=%d key tiles=%d\n",
                     fused ? "fused" : "single", a.B, a.S, a.Hq, a.Hkv, a.D, a.causal, a.nkt);
    const int rc = fkv::launch_backward(a, fused, stream);
    if (rc) return fail(FKV_ERROR_LAUNCH, "backward launch failed (HIP error %d)", rc);
    return ok();
}

}  // namespace

extern "C" {

int fkv_abi_version(void) { return FKV_ABI_VERSION; }

const char* fkv_status_string(fkv_status status)
{
    switch (status) {
    case FKV_SUCCESS: return "success";
    case FKV_ERROR_INVALID_VALUE: return "invalid value";
    case FKV_ERROR_UNSUPPORTED: return "unsupported";
    case FKV_ERROR_WORKSPACE: return "workspace missing or too small";
    case FKV_ERROR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

const char* fkv_last_error(void) { return g_last_error; }

size_t fkv_decode_workspace_size(const fkv_params* params)
{
    if (check_shape(params) != FKV_SUCCESS || params->seqlen_q != 1) return 0;
    size_t w = 0;
    for (int kivi = 0; kivi < 2; ++kivi)
        for (int fused = 0; fused < 2; ++fused) {
            const size_t b = plan_decode(params, fused != 0, kivi != 0).total_bytes;
            if (b > w) w = b;
        }
    return w;
}

fkv_status fkv_decode(const fkv_params* params, const void* q, fkv_cache k1, fkv_cache kn,
                      fkv_cache v1, fkv_cache vn, const fkv_fusion* fusion,
                      const int32_t* seqlens_k, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream)
{
    const fkv_cache c[4] = {k1, kn, v1, vn};
    static const char* const n[4] = {"k1", "kn", "v1", "vn"};
    return decode_common(params, q, c, n, 4, fusion, seqlens_k, out, lse, workspace,
                         workspace_bytes, stream);
}

fkv_status fkv_decode_noalloc(const fkv_params* params, const void* q, fkv_cache k1, fkv_cache kn,
                              fkv_cache v1, fkv_cache vn, const fkv_fusion* fusion,
                              const int32_t* seqlens_k, void* out, float* lse, void* stream)
{
    static_assert(fkv::kNoallocScratchBytes == FKV_NOALLOC_SCRATCH_BYTES, "scratch size in the header");
    const fkv_cache c[4] = {k1, kn, v1, vn};
    static const char* const n[4] = {"k1", "kn", "v1", "vn"};
    return decode_common(params, q, c, n, 4, fusion, seqlens_k, out, lse, nullptr, 0, stream, true);
}

fkv_status fkv_lite_decode(const fkv_params* params, const void* q, fkv_cache k_src,
                           fkv_cache v_src, const int32_t* seqlens_k, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream)
{
    const fkv_cache c[2] = {k_src, v_src};
    static const char* const n[2] = {"k_src", "v_src"};
    return decode_common(params, q, c, n, 2, nullptr, seqlens_k, out, lse, workspace,
                         workspace_bytes, stream);
}

fkv_status fkv_prefill(const fkv_params* params, const void* q, fkv_cache k1, fkv_cache kn,
                       fkv_cache v1, fkv_cache vn, const fkv_fusion* fusion, void* out,
                       float* lse, void* stream)
{
    const fkv_cache c[4] = {k1, kn, v1, vn};
    static const char* const n[4] = {"k1", "kn", "v1", "vn"};
    return prefill_common(params, q, c, n, 4, fusion, out, lse, stream);
}

fkv_status fkv_lite_prefill(const fkv_params* params, const void* q, fkv_cache k_src,
                            fkv_cache v_src, void* out, float* lse, void* stream)
{
    const fkv_cache c[2] = {k_src, v_src};
    static const char* const n[2] = {"k_src", "v_src"};
    return prefill_common(params, q, c, n, 2, nullptr, out, lse, stream);
}

fkv_status fkv_check_tied(const float* host_k_w, int32_t h_kv, int32_t d, int32_t pairing, float tol)
{
    if (!host_k_w || h_kv < 1 || d < 2 || (d & 1) || !(tol >= 0.0f))
        return fail(FKV_ERROR_INVALID_VALUE, "bad arguments to fkv_check_tied");
    if (pairing != 0 && pairing != 1) return fail(FKV_ERROR_INVALID_VALUE, "pairing must be 0 or 1");
    for (int32_t h = 0; h < h_kv; ++h) {
        const float* w = host_k_w + (int64_t)h * d;
        for (int32_t j = 0; j < d / 2; ++j) {
            const int32_t i1 = pairing == 0 ? 2 * j : j;
            const int32_t i2 = pairing == 0 ? 2 * j + 1 : j + d / 2;
            const float diff = std::fabs(w[i1] - w[i2]);
            if (!(diff <= tol))
                return fail(FKV_ERROR_INVALID_VALUE, "head %d channels %d and %d differ by %g", h, i1, i2,
                            (double)diff);
        }
    }
    return ok();
}

size_t fkv_kivi_codes_bytes(const fkv_params* params, int32_t is_value)
{
    if (!params || params->batch < 0 || params->seqlen_k < 0 || params->num_kv_heads < 1 ||
        !supported_head_dim(params->head_dim))
        return 0;
    const int64_t bh = (int64_t)params->batch * params->num_kv_heads;
    // values: whole 32-token blocks of D channels x 16 bytes
    return is_value ? (size_t)(bh * kivi_key_groups(params->seqlen_k) * params->head_dim * 16)
                    : (size_t)(bh * params->seqlen_k * (params->head_dim / 2));
}

size_t fkv_kivi_meta_bytes(const fkv_params* params, int32_t is_value)
{
    if (!params || params->batch < 0 || params->seqlen_k < 0 || params->num_kv_heads < 1 ||
        !supported_head_dim(params->head_dim))
        return 0;
    const int64_t bh = (int64_t)params->batch * params->num_kv_heads;
    const int64_t n = is_value ? bh * kivi_key_groups(params->seqlen_k) * kivi_value_groups(params->head_dim) * 32
                               : bh * kivi_key_groups(params->seqlen_k) * params->head_dim;
    return (size_t)n * 2;
}

fkv_status fkv_kivi_quantize(const fkv_params* params, fkv_cache src, int32_t is_value, fkv_q4_cache dst,
                             void* stream)
{
    fkv_status s = check_shape(params);
    if (s) return s;
    if (params->dtype != FKV_BF16) return fail(FKV_ERROR_UNSUPPORTED, "the 4-bit quantiser reads bfloat16 caches");
    if (is_value != 0 && is_value != 1) return fail(FKV_ERROR_INVALID_VALUE, "is_value must be 0 or 1");
    if (params->batch == 0 || params->seqlen_k == 0) return ok();
    if ((s = check_cache(params, src, "src"))) return s;
    if ((s = check_q4(params, dst, "dst"))) return s;
    fkv::KiviQuantArgs a{};
    a.src = view_of(src);
    a.codes = const_cast<void*>(dst.codes);
    a.scale = const_cast<void*>(dst.scale);
    a.minv = const_cast<void*>(dst.minv);
    a.B = params->batch;
    a.S = params->seqlen_k;
    a.H = params->num_kv_heads;
    a.D = params->head_dim;
    a.is_value = is_value;
    const int rc = fkv::launch_kivi_quantize(a, stream);
    if (rc) return fail(FKV_ERROR_LAUNCH, "4-bit quantiser launch failed (HIP error %d)", rc);
    return ok();
}

fkv_status fkv_kivi_decode(const fkv_params* params, const void* q, fkv_q4_cache k1, fkv_q4_cache kn,
                           fkv_q4_cache v1, fkv_q4_cache vn, const fkv_fusion* fusion,
                           const int32_t* seqlens_k, void* out, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream)
{
    const fkv_q4_cache c[4] = {k1, kn, v1, vn};
    static const char* const n[4] = {"k1", "kn", "v1", "vn"};
    return kivi_decode_common(params, q, c, n, 4, fusion, seqlens_k, out, lse, workspace, workspace_bytes, stream);
}

fkv_status fkv_kivi_lite_decode(const fkv_params* params, const void* q, fkv_q4_cache k_src, fkv_q4_cache v_src,
                                const int32_t* seqlens_k, void* out, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream)
{
    const fkv_q4_cache c[2] = {k_src, v_src};
    static const char* const n[2] = {"k_src", "v_src"};
    return kivi_decode_common(params, q, c, n, 2, nullptr, seqlens_k, out, lse, workspace, workspace_bytes, stream);
}

size_t fkv_backward_workspace_size(const fkv_params* params)
{
    if (check_shape(params) != FKV_SUCCESS || params->seqlen_q != params->seqlen_k) return 0;
    if (params->batch == 0 || params->seqlen_q == 0) return 0;
    return backward_layout(params).total;
}

fkv_status fkv_prefill_backward(const fkv_params* params, const void* q, fkv_cache k1, fkv_cache kn, fkv_cache v1,
                                fkv_cache vn, const fkv_fusion* fusion, const void* out, const float* lse,
                                const void* dout, void* dq, fkv_grad dk1, fkv_grad dkn, fkv_grad dv1, fkv_grad dvn,
                                const fkv_fusion_grad* dfusion, void* workspace, size_t workspace_bytes, void* stream)
{
    const fkv_cache c[4] = {k1, kn, v1, vn};
    const fkv_grad gr[4] = {dk1, dkn, dv1, dvn};
    static const char* const n[4] = {"k1", "kn", "v1", "vn"};
    static const char* const gn[4] = {"dk1", "dkn", "dv1", "dvn"};
    return backward_common(params, q, c, n, 4, fusion, out, lse, dout, dq, gr, gn, dfusion, workspace,
                           workspace_bytes, stream);
}

fkv_status fkv_lite_prefill_backward(const fkv_params* params, const void* q, fkv_cache k_src, fkv_cache v_src,
                                     const void* out, const float* lse, const void* dout, void* dq, fkv_grad dk,
                                     fkv_grad dv, void* workspace, size_t workspace_bytes, void* stream)
{
    const fkv_cache c[2] = {k_src, v_src};
    const fkv_grad gr[2] = {dk, dv};
    static const char* const n[2] = {"k_src", "v_src"};
    static const char* const gn[2] = {"dk", "dv"};
    return backward_common(params, q, c, n, 2, nullptr, out, lse, dout, dq, gr, gn, nullptr, workspace,
                           workspace_bytes, stream);
}

fkv_status fkv_store_kv(const fkv_params* params, int32_t pos0, fkv_cache k_new, fkv_cache v_new,
                        fkv_grad k_cache, fkv_grad v_cache, void* stream)
{
    fkv_status s = check_shape(params);
    if (s) return s;
    if (pos0 < 0) return fail(FKV_ERROR_INVALID_VALUE, "pos0 must be >= 0");
    if ((int64_t)pos0 + params->seqlen_q > params->seqlen_k)
        return fail(FKV_ERROR_INVALID_VALUE, "pos0 + seqlen_q (%lld) exceeds the cache's %d tokens",
                    (long long)pos0 + params->seqlen_q, params->seqlen_k);
    if (params->batch == 0 || params->seqlen_q == 0) return ok();
    // the new rows are checked as caches of seqlen_q tokens, the caches as
    // writable views of seqlen_k tokens
    fkv_params pn = *params;
    pn.seqlen_k = params->seqlen_q;
    if ((s = check_cache(&pn, k_new, "k_new")) || (s = check_cache(&pn, v_new, "v_new"))) return s;
    if (!k_new.data || !v_new.data) return fail(FKV_ERROR_INVALID_VALUE, "k_new / v_new data is NULL");
    if ((s = check_grad(params, k_cache, "k_cache")) || (s = check_grad(params, v_cache, "v_cache"))) return s;
    fkv::StoreArgs a{};
    a.k_new = view_of(k_new);
    a.v_new = view_of(v_new);
    a.k_cache = out_of(k_cache);
    a.v_cache = out_of(v_cache);
    a.B = params->batch;
    a.S_new = params->seqlen_q;
    a.H = params->num_kv_heads;
    a.D = params->head_dim;
    a.pos0 = pos0;
    a.elt = (int)elt_size(params->dtype);
    const int rc = fkv::launch_store_kv(a, stream);
    if (rc) return fail(FKV_ERROR_LAUNCH, "cache-write launch failed (HIP error %d)", rc);
    return ok();
}

}  // extern "C"
