/*
 * fkv_oracle.c -- plain fp64 CPU oracle for FusedKV reconstruction-layer
 * attention.
 *
 * TEST INFRASTRUCTURE ONLY.  The parity tests, the smoke check and the
 * benchmark's CPU-baseline leg load this file's shared object; nothing on the
 * product path may load, call or link it.  It shares no code, header, table or
 * helper with the HIP library: it is a second, independent statement of what
 * the method computes, written to be checked by eye against the pages.
 *
 * Pages cited (by title):
 *   [Deck]  "FusedKV: Reconstructing KV Caches with Cross-Layer Fusion"
 *           (reading slides of arXiv:2512.03870v3)
 *   [Notes] "FusedKV:通过跨层融合重构 KV 缓存" (reading notes of the same paper)
 *
 * What is computed, for one reconstruction layer i > n = L/2:
 *   1. Fusion, applied element-wise to the stored post-RoPE caches of layer 1
 *      and layer n with per-channel vectors broadcast over tokens
 *      ([Deck] frame "FusedKV learns two-source, channel-wise fusion",
 *      Eqs. (4)-(5); [Notes] section 2.3):
 *          Kf[b,t,g,d] = a [g,d] * K1[b,t,g,d] + a'[g,d] * Kn[b,t,g,d]
 *          Vf[b,t,g,d] = bv[g,d] * V1[b,t,g,d] + bv'[g,d] * Vn[b,t,g,d]
 *      FusedKV-Lite reads one key and one value source unchanged
 *      ([Deck] frame "Lite separates the key source from the value source",
 *      Eq. (6): K^i = K^n, V^i = V^1); plain storage-layer attention (the
 *      control) is the same single-source form applied to the layer's own
 *      caches.
 *   2. Scaled dot-product softmax attention of the layer's own queries over
 *      the reconstructed keys and values ([Deck] same frame: queries stay
 *      layer-specific), with grouped-query sharing: query head h reads KV head
 *      floor(h / G), G = Hq / Hkv (contiguous groups).
 *          s_t = scale * sum_d Q[b,p,h,d] * Kf[b,t,g,d]
 *          m   = max_t s_t,   l = sum_t exp(s_t - m)
 *          O[b,p,h,:] = sum_t exp(s_t - m) * Vf[b,t,g,:] / l
 *          LSE[b,h,p] = m + ln l
 *      over the visible set t in [0, len_b) and, when causal, t <= p +
 *      (len_b - Sq) (bottom-right alignment; with Sq == Sk this is t <= p).
 *      An empty visible set gives O = 0 and LSE = -inf.
 *
 * Arithmetic: every stored value (fp32 or bf16 bit pattern) is widened exactly
 * to double; all products and sums are plain sequential fp64 loops, with no
 * blocking, no reordering and no online-softmax rescaling.  Rows are
 * independent, so they are spread over OpenMP threads; the arithmetic inside
 * a row is the same whatever the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* A [B, S, H, D] view with element strides for b, s and h; d has stride 1. */
typedef struct {
    const void* data;
    int64_t sb, ss, sh;
} orc_view;

typedef struct {
    int32_t batch, seqlen_q, seqlen_k, num_q_heads, num_kv_heads, head_dim;
    int32_t dtype;  /* 0: float32, 1: bfloat16 bits, 2: float64 (dequantised
                       caches, which need more than float32 to hold exactly) */
    int32_t causal; /* 0: every cached token visible, 1: causal mask */
    double scale;   /* softmax scale applied to q.k */
} orc_shape;

/* Exact widening of one stored value to double.  A bfloat16 value is the
 * upper half of the float32 with the same bits; float64 is read as is. */
static double widen(const void* base, int32_t dtype, int64_t idx)
{
    if (dtype == 0) return (double)((const float*)base)[idx];
    if (dtype == 2) return ((const double*)base)[idx];
    uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int64_t at(const orc_view* v, int b, int t, int g, int d)
{
    return (int64_t)b * v->sb + (int64_t)t * v->ss + (int64_t)g * v->sh + d;
}

/* One element of the reconstructed cache of layer i (Eq. (4) for keys,
 * Eq. (5) for values).  single != 0 reads src1 alone (Lite, Eq. (6), or the
 * plain-attention control). */
static double reconstructed(const orc_view* src1, const orc_view* srcn,
                            const float* w1, const float* wn, int32_t dtype,
                            int D, int single, int b, int t, int g, int d)
{
    double x1 = widen(src1->data, dtype, at(src1, b, t, g, d));
    if (single) return x1;
    double xn = widen(srcn->data, dtype, at(srcn, b, t, g, d));
    return (double)w1[(int64_t)g * D + d] * x1 + (double)wn[(int64_t)g * D + d] * xn;
}

/*
 * orc_attend: attention output of one reconstruction layer for a list of
 * query rows.
 *
 *   single_source == 0 : FusedKV, keys from (k1, kn) with (kw1, kwn), values
 *                        from (v1, vn) with (vw1, vwn); weights are [Hkv, D]
 *                        float32 arrays.
 *   single_source != 0 : keys = k1, values = v1 (pass K^n / V^1 for Lite, or a
 *                        storage layer's own caches for the control); kn, vn
 *                        and the weights are ignored.
 *   q       : [B, Sq, Hq, D] contiguous, stored in shape->dtype.
 *   seqlens_k: NULL (every batch has seqlen_k keys) or [B] lengths; each is
 *              clamped to [0, seqlen_k].
 *   rows    : NULL for every row, else nrows indices r = (b*Hq + h)*Sq + p.
 *   out     : [nrows, D] doubles; lse: [nrows] doubles (natural log).
 *
 * Returns 0, or -1 on a malformed shape.
 */
int orc_attend(const orc_shape* shape, int single_source, const void* q,
               orc_view k1, orc_view kn, orc_view v1, orc_view vn,
               const float* kw1, const float* kwn, const float* vw1,
               const float* vwn, const int32_t* seqlens_k, const int64_t* rows,
               int64_t nrows, double* out, double* lse)
{
    const int B = shape->batch, Sq = shape->seqlen_q, Sk = shape->seqlen_k;
    const int Hq = shape->num_q_heads, Hkv = shape->num_kv_heads, D = shape->head_dim;
    if (B < 0 || Sq < 0 || Sk < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0) return -1;
    if (!single_source && (!kw1 || !kwn || !vw1 || !vwn)) return -1;
    const int G = Hq / Hkv;
    const int64_t total = (int64_t)B * Hq * Sq;
    const int64_t n = rows ? nrows : total;
    int bad = 0;

#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
        double* acc = (double*)malloc(sizeof(double) * (size_t)D);
        if (!s || !acc) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n; ++i) {
            if (!s || !acc) continue;
            const int64_t r = rows ? rows[i] : i;
            if (r < 0 || r >= total) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            const int p = (int)(r % Sq);
            const int h = (int)((r / Sq) % Hq);
            const int b = (int)(r / ((int64_t)Sq * Hq));
            const int g = h / G; /* grouped-query sharing: contiguous groups */

            int len = seqlens_k ? seqlens_k[b] : Sk;
            if (len < 0) len = 0;
            if (len > Sk) len = Sk;
            int last = len - 1; /* last visible key index */
            if (shape->causal && p + (len - Sq) < last) last = p + (len - Sq);

            double* o = out + i * D;
            if (last < 0) { /* nothing visible */
                for (int d = 0; d < D; ++d) o[d] = 0.0;
                lse[i] = -INFINITY;
                continue;
            }

            /* scores s_t = scale * q . Kf_t */
            const int64_t qoff = (((int64_t)b * Sq + p) * Hq + h) * D;
            double m = -INFINITY;
            for (int t = 0; t <= last; ++t) {
                double dot = 0.0;
                for (int d = 0; d < D; ++d)
                    dot += widen(q, shape->dtype, qoff + d) *
                           reconstructed(&k1, &kn, kw1, kwn, shape->dtype, D,
                                         single_source, b, t, g, d);
                s[t] = shape->scale * dot;
                if (s[t] > m) m = s[t];
            }

            /* softmax weights and the weighted sum of reconstructed values */
            double l = 0.0;
            for (int d = 0; d < D; ++d) acc[d] = 0.0;
            for (int t = 0; t <= last; ++t) {
                const double e = exp(s[t] - m);
                l += e;
                for (int d = 0; d < D; ++d)
                    acc[d] += e * reconstructed(&v1, &vn, vw1, vwn, shape->dtype, D,
                                                single_source, b, t, g, d);
            }
            for (int d = 0; d < D; ++d) o[d] = acc[d] / l;
            lse[i] = m + log(l);
        }
        free(s);
        free(acc);
    }
    return bad ? -1 : 0;
}

/*
 * Cache accounting, in elements, for an L-layer model with S cached tokens,
 * Hkv KV heads of dimension D ([Deck] frame "Capacity and bandwidth are
 * different bottlenecks": a plain model keeps 2*L*S*Hkv*D elements; [Deck]
 * frame "Half the storage can require 50% more cache I/O", Table 1; [Notes]
 * section 2.5).  method: 0 vanilla, 1 FusedKV-Lite (or YOCO), 2 FusedKV.
 *
 * capacity: elements that stay resident.  Vanilla stores K and V for all L
 *   layers; FusedKV and Lite store them only for the lower half.
 * reads: cache elements read by one decode step over all layers.  Every
 *   storage layer reads its own K and V; a Lite layer reads one K and one V
 *   source; a FusedKV layer reads two K and two V sources.
 */
int64_t orc_cache_capacity(int method, int64_t L, int64_t S, int64_t Hkv, int64_t D)
{
    const int64_t per_layer = 2 * S * Hkv * D; /* K and V of one layer */
    if (method == 0) return L * per_layer;
    return (L / 2) * per_layer;
}

int64_t orc_cache_reads(int method, int64_t L, int64_t S, int64_t Hkv, int64_t D)
{
    const int64_t per_layer = 2 * S * Hkv * D;
    const int64_t lower = L / 2, upper = L - L / 2;
    if (method == 0) return L * per_layer;
    if (method == 1) return lower * per_layer + upper * per_layer;
    return lower * per_layer + upper * 2 * per_layer;
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
