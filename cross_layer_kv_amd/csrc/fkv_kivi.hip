// fkv_kivi.hip -- FusedKV over KIVI-style 4-bit source caches on gfx950:
// the quantiser that writes such a cache, and split-K decode that
// dequantises each tile in registers before the fusion.
//
// Pages cited (by title):
//   [Deck]  "FusedKV: Reconstructing KV Caches with Cross-Layer Fusion",
//           frame "Four-bit KV quantization is the stronger combination"
//           (Tables 14-15): FusedKV composed with 4-bit KIVI caches, a 4-fold
//           payload cut on top of FusedKV's halving.
//   [Notes] "FusedKV:通过跨层融合重构 KV 缓存", section A.6.5.
//
// Format (the published KIVI scheme at 4 bits; the pages print none): keys
// are grouped per channel over 32 consecutive tokens, values per token over
// 32 consecutive channels; each group keeps an fp16 minimum and scale
// (max - min) / 15, and an element's code is rint((x - min) / scale)
// clamped to 0..15 (0 for a zero scale), decided in float32 with correctly
// rounded division so that any float32 implementation of the same steps
// gives the same codes.  Two codes per byte, channel 2i in the low nibble.
//
// Decode reads 4 code bytes (8 channels) per source per token and lane, in
// place of 16 bf16 bytes, and rebuilds the fused key of a 32-token group's
// channel as A1 q1 + An qn + C with A1 = a s1, An = a' sn, C = a m1 + a' mn
// (computed once per group), values as b (m1 + s1 q1) + b' (mn + sn qn).
// The work layout and the online softmax are those of the bf16 decode
// kernel (fkv_decode.hip): one workgroup per (batch, KV head, split), a lane
// owns 8 channels of a token, token groups sum scores with DPP.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fkv_internal.h"
#include "fkv_mfma_common.h"

namespace fkv {
namespace {

using namespace dev;

constexpr int kGroup = 32;       // elements per quantisation group
constexpr int kWaveTokens = 16;  // tokens per wave per iteration
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float h2f(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }
__device__ __forceinline__ uint16_t f2h(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }

// Group parameters and the code of x, float32 throughout: the minimum and
// scale are rounded once to fp16 and the code uses those rounded values.
struct QParams {
    uint16_t mn16, sc16;
    float m, r;  // fp16 minimum widened, 1 / fp16 scale (0 when the scale is 0)
};
__device__ __forceinline__ QParams qparams(float mn, float mx)
{
    QParams p;
    const float sc = __fdiv_rn(mx - mn, 15.0f);
    p.mn16 = f2h(mn);
    p.sc16 = f2h(sc);
    p.m = h2f(p.mn16);
    const float s = h2f(p.sc16);
    p.r = s > 0.0f ? __fdiv_rn(1.0f, s) : 0.0f;
    return p;
}
__device__ __forceinline__ uint32_t qcode(float x, const QParams& p)
{
    if (p.r == 0.0f) return 0u;
    const float t = __fmul_rn(__fsub_rn(x, p.m), p.r);
    return (uint32_t)fminf(fmaxf(rintf(t), 0.0f), 15.0f);
}

// Keys: one thread per (batch*head, 32-token group, channel pair).
__global__ __launch_bounds__(256) void kivi_quant_keys_kernel(const KiviQuantArgs a)
{
    const int np = a.D / 2, ng = (a.S + kGroup - 1) / kGroup;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)a.B * a.H * ng * np) return;
    const int cp = (int)(i % np);
    const int j = (int)((i / np) % ng);
    const int bh = (int)(i / ((int64_t)np * ng));
    const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
    const int t0 = j * kGroup, t1 = min(a.S, t0 + kGroup);
    const uint16_t* src = static_cast<const uint16_t*>(a.src.data) + (int64_t)b * a.src.sb + (int64_t)h * a.src.sh + 2 * cp;
    float lo_mn = INFINITY, lo_mx = -INFINITY, hi_mn = INFINITY, hi_mx = -INFINITY;
    for (int t = t0; t < t1; ++t) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(src + (int64_t)t * a.src.ss);
        const float x0 = bf16_lo(w), x1 = bf16_hi(w);
        lo_mn = fminf(lo_mn, x0);
        lo_mx = fmaxf(lo_mx, x0);
        hi_mn = fminf(hi_mn, x1);
        hi_mx = fmaxf(hi_mx, x1);
    }
    const QParams p0 = qparams(lo_mn, lo_mx), p1 = qparams(hi_mn, hi_mx);
    uint8_t* codes = static_cast<uint8_t*>(a.codes) + (int64_t)bh * a.S * np + cp;
    for (int t = t0; t < t1; ++t) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(src + (int64_t)t * a.src.ss);
        codes[(int64_t)t * np] = (uint8_t)(qcode(bf16_lo(w), p0) | (qcode(bf16_hi(w), p1) << 4));
    }
    const int64_t mo = ((int64_t)bh * ng + j) * a.D + 2 * cp;
    uint16_t* sc = static_cast<uint16_t*>(a.scale);
    uint16_t* mn = static_cast<uint16_t*>(a.minv);
    sc[mo] = p0.sc16;
    sc[mo + 1] = p1.sc16;
    mn[mo] = p0.mn16;
    mn[mo + 1] = p1.mn16;
}

// Values: one thread per (batch*head, token, 32-channel group).
__global__ __launch_bounds__(256) void kivi_quant_values_kernel(const KiviQuantArgs a)
{
    const int ng = (a.D + kGroup - 1) / kGroup, np = a.D / 2;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)a.B * a.H * a.S * ng) return;
    const int c = (int)(i % ng);
    const int t = (int)((i / ng) % a.S);
    const int bh = (int)(i / ((int64_t)ng * a.S));
    const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
    const int d0 = c * kGroup, n = min(kGroup, a.D - d0);  // 32, or 16 for the last group of D = 80
    const uint16_t* src = static_cast<const uint16_t*>(a.src.data) + (int64_t)b * a.src.sb + (int64_t)t * a.src.ss +
                          (int64_t)h * a.src.sh + d0;
    uint32_t w[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint4 u = make_uint4(0u, 0u, 0u, 0u);
        if (k * 8 < n) u = reinterpret_cast<const uint4*>(src)[k];
        w[4 * k] = u.x;
        w[4 * k + 1] = u.y;
        w[4 * k + 2] = u.z;
        w[4 * k + 3] = u.w;
    }
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        if (2 * k < n) {
            mn = fminf(mn, fminf(bf16_lo(w[k]), bf16_hi(w[k])));
            mx = fmaxf(mx, fmaxf(bf16_lo(w[k]), bf16_hi(w[k])));
        }
    }
    const QParams p = qparams(mn, mx);
    uint8_t* codes = static_cast<uint8_t*>(a.codes) + ((int64_t)bh * a.S + t) * np + d0 / 2;
#pragma unroll
    for (int k = 0; k < 16; ++k)
        if (2 * k < n) codes[k] = (uint8_t)(qcode(bf16_lo(w[k]), p) | (qcode(bf16_hi(w[k]), p) << 4));
    const int64_t mo = ((int64_t)bh * a.S + t) * ng + c;
    static_cast<uint16_t*>(a.scale)[mo] = p.sc16;
    static_cast<uint16_t*>(a.minv)[mo] = p.mn16;
}

// Codes of 8 channels (one 4-byte word) as floats 0..15, channel order.
__device__ __forceinline__ void unpack8(uint32_t w, float* f)
{
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = (float)((lo >> (8 * i)) & 0xFFu);
        f[2 * i + 1] = (float)((hi >> (8 * i)) & 0xFFu);
    }
}

template <int D, bool FUSED, int G, int NW>
__global__ __launch_bounds__(64 * NW) void q4_decode_kernel(const KiviDecodeArgs a)
{
    constexpr int NT = 64 * NW;
    constexpr int NP = D / 8;              // 8-channel pieces per row
    constexpr int LPT = NP <= 8 ? 8 : 16;  // lanes per token group
    constexpr int TPW = 64 / LPT;          // tokens per wave step
    constexpr int U = kWaveTokens / TPW;   // steps per iteration
    constexpr int NGV = (D + kGroup - 1) / kGroup;

    __shared__ float s_acc[NW][G][D];
    __shared__ float s_ml[NW][G][2];

    const int split = blockIdx.x;
    const int bg = blockIdx.y;  // b * Hkv + g
    const int b = bg / a.Hkv, g = bg - (bg / a.Hkv) * a.Hkv;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int grp = lane / LPT, pc = lane % LPT;
    const bool active = pc < NP;
    const int c0 = active ? pc * 8 : 0;
    const int vgrp = c0 / kGroup;  // this lane's value channel group

    int len = a.seqlens ? a.seqlens[b] : a.Sk;
    len = len < 0 ? 0 : (len > a.Sk ? a.Sk : len);
    const int t_begin = split * a.chunk;
    const int t_end = min(len, t_begin + a.chunk);
    const int ngk = (a.Sk + kGroup - 1) / kGroup;

    // Query of the G heads, pre-scaled into the log2 domain
    float qs[G][8];
    {
        const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.Hq + (int64_t)g * G) * D + c0;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            uint4 u = make_uint4(0u, 0u, 0u, 0u);
            if (active) u = *reinterpret_cast<const uint4*>(qp + (int64_t)hh * D);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qs[hh][2 * i] = bf16_lo(w[i]) * a.scale_log2;
                qs[hh][2 * i + 1] = bf16_hi(w[i]) * a.scale_log2;
            }
        }
    }
    float wk1[8], wkn[8], wv1[8], wvn[8];
    if constexpr (FUSED) {
        const int64_t wo = (int64_t)g * D + c0;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            wk1[c] = active ? a.kw1[wo + c] : 0.0f;
            wkn[c] = active ? a.kwn[wo + c] : 0.0f;
            wv1[c] = active ? a.vw1[wo + c] : 0.0f;
            wvn[c] = active ? a.vwn[wo + c] : 0.0f;
        }
    }

    // per-source pointers of this (batch, KV head): codes of channel c0 at
    // token 0, key group parameters of channel c0 at group 0, value group
    // parameters of group vgrp at token 0
    const int64_t bh = bg;
    auto codes_of = [&](const Q4View& v) { return static_cast<const uint8_t*>(v.codes) + bh * a.Sk * (D / 2) + c0 / 2; };
    auto kmeta = [&](const void* p) { return static_cast<const uint16_t*>(p) + bh * ngk * D + c0; };
    auto vmeta = [&](const void* p) { return static_cast<const uint16_t*>(p) + bh * a.Sk * NGV + vgrp; };
    const uint8_t* ck1 = codes_of(a.qk1);
    const uint8_t* cv1 = codes_of(a.qv1);
    const uint16_t* ks1 = kmeta(a.qk1.scale);
    const uint16_t* km1 = kmeta(a.qk1.minv);
    const uint16_t* vs1 = vmeta(a.qv1.scale);
    const uint16_t* vm1 = vmeta(a.qv1.minv);
    const uint8_t* ckn = ck1;
    const uint8_t* cvn = cv1;
    const uint16_t *ksn = ks1, *kmn = km1, *vsn = vs1, *vmn = vm1;
    if constexpr (FUSED) {
        ckn = codes_of(a.qkn);
        cvn = codes_of(a.qvn);
        ksn = kmeta(a.qkn.scale);
        kmn = kmeta(a.qkn.minv);
        vsn = vmeta(a.qvn.scale);
        vmn = vmeta(a.qvn.minv);
    }

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        m[hh] = -INFINITY;
        l[hh] = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[hh][c] = 0.0f;
    }

    for (int t0 = t_begin + wave * kWaveTokens; t0 < t_end; t0 += NW * kWaveTokens) {
        // key group parameters: the 16 tokens of a slice share one group
        // (splits start at multiples of 64 and slices at multiples of 16)
        float A1[8], An[8], C[8];
        {
            const int gi = t0 / kGroup;
            uint4 s1 = make_uint4(0u, 0u, 0u, 0u), m1 = s1, sn = s1, mn = s1;
            if (active) {
                s1 = *reinterpret_cast<const uint4*>(ks1 + (int64_t)gi * D);
                m1 = *reinterpret_cast<const uint4*>(km1 + (int64_t)gi * D);
                if constexpr (FUSED) {
                    sn = *reinterpret_cast<const uint4*>(ksn + (int64_t)gi * D);
                    mn = *reinterpret_cast<const uint4*>(kmn + (int64_t)gi * D);
                }
            }
            const uint32_t s1w[4] = {s1.x, s1.y, s1.z, s1.w}, m1w[4] = {m1.x, m1.y, m1.z, m1.w};
            const uint32_t snw[4] = {sn.x, sn.y, sn.z, sn.w}, mnw[4] = {mn.x, mn.y, mn.z, mn.w};
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float sc1 = h2f((uint16_t)(s1w[c / 2] >> (16 * (c & 1))));
                const float mi1 = h2f((uint16_t)(m1w[c / 2] >> (16 * (c & 1))));
                if constexpr (FUSED) {
                    const float scn = h2f((uint16_t)(snw[c / 2] >> (16 * (c & 1))));
                    const float min_ = h2f((uint16_t)(mnw[c / 2] >> (16 * (c & 1))));
                    A1[c] = wk1[c] * sc1;
                    An[c] = wkn[c] * scn;
                    C[c] = wk1[c] * mi1 + wkn[c] * min_;
                } else {
                    A1[c] = sc1;
                    An[c] = 0.0f;
                    C[c] = mi1;
                }
            }
        }

        uint32_t rk1[U], rkn[U], rv1[U], rvn[U];
        float vs1u[U], vm1u[U], vsnu[U], vmnu[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t0 + u * TPW + grp;
            ok[u] = t < t_end;
            const bool pr = active && ok[u];
            rk1[u] = pr ? *reinterpret_cast<const uint32_t*>(ck1 + (int64_t)t * (D / 2)) : 0u;
            rv1[u] = pr ? *reinterpret_cast<const uint32_t*>(cv1 + (int64_t)t * (D / 2)) : 0u;
            vs1u[u] = pr ? h2f(vs1[(int64_t)t * NGV]) : 0.0f;
            vm1u[u] = pr ? h2f(vm1[(int64_t)t * NGV]) : 0.0f;
            if constexpr (FUSED) {
                rkn[u] = pr ? *reinterpret_cast<const uint32_t*>(ckn + (int64_t)t * (D / 2)) : 0u;
                rvn[u] = pr ? *reinterpret_cast<const uint32_t*>(cvn + (int64_t)t * (D / 2)) : 0u;
                vsnu[u] = pr ? h2f(vsn[(int64_t)t * NGV]) : 0.0f;
                vmnu[u] = pr ? h2f(vmn[(int64_t)t * NGV]) : 0.0f;
            }
        }

        // scores of the U tokens of this lane's group, log2 domain
        float s[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float q1[8], kf[8];
            unpack8(rk1[u], q1);
            if constexpr (FUSED) {
                float qn[8];
                unpack8(rkn[u], qn);
#pragma unroll
                for (int c = 0; c < 8; ++c) kf[c] = A1[c] * q1[c] + (An[c] * qn[c] + C[c]);
            } else {
#pragma unroll
                for (int c = 0; c < 8; ++c) kf[c] = A1[c] * q1[c] + C[c];
            }
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                float d = 0.0f;
#pragma unroll
                for (int c = 0; c < 8; ++c) d += qs[hh][c] * kf[c];
                d = token_group_sum<LPT>(d);
                s[u][hh] = ok[u] ? d : -INFINITY;
            }
        }

        // online softmax: raise the running max if needed, then accumulate
        float msub[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            float mx = s[0][hh];
#pragma unroll
            for (int u = 1; u < U; ++u) mx = fmaxf(mx, s[u][hh]);
            if (mx > m[hh]) {
                const float corr = rel_weight(m[hh], mx);
                l[hh] *= corr;
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[hh][c] *= corr;
                m[hh] = mx;
            }
            msub[hh] = m[hh] == -INFINITY ? 0.0f : m[hh];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[8];
            unpack8(rv1[u], vf);
#pragma unroll
            for (int c = 0; c < 8; ++c) vf[c] = vm1u[u] + vs1u[u] * vf[c];
            if constexpr (FUSED) {
                float vn[8];
                unpack8(rvn[u], vn);
#pragma unroll
                for (int c = 0; c < 8; ++c) vf[c] = wv1[c] * vf[c] + wvn[c] * (vmnu[u] + vsnu[u] * vn[c]);
            }
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                const float p = exp2_fast(s[u][hh] - msub[hh]);
                l[hh] += p;
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[hh][c] += p * vf[c];
            }
        }
    }

    // merge the token groups of the wave (lanes with equal pc)
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const float mo = __shfl_xor(m[hh], off);
            const float lo = __shfl_xor(l[hh], off);
            const float M = fmaxf(m[hh], mo);
            const float fa = rel_weight(m[hh], M), fb = rel_weight(mo, M);
            l[hh] = l[hh] * fa + lo * fb;
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[hh][c] = acc[hh][c] * fa + __shfl_xor(acc[hh][c], off) * fb;
            m[hh] = M;
        }
    }
    if (grp == 0 && active) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
            for (int c = 0; c < 8; ++c) s_acc[wave][hh][c0 + c] = acc[hh][c];
    }
    if (lane == 0) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            s_ml[wave][hh][0] = m[hh];
            s_ml[wave][hh][1] = l[hh];
        }
    }
    __syncthreads();

    // merge the waves; write O/LSE (one split) or this split's partial row
    const bool final_out = a.n_splits == 1;
    const int64_t slot = (int64_t)bg * a.n_splits + split;
    for (int e = tid; e < G * D; e += NT) {
        const int hh = e / D, d = e - (e / D) * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, s_ml[w][hh][0]);
        float o = 0.0f, ls = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = rel_weight(s_ml[w][hh][0], M);
            o += s_acc[w][hh][d] * f;
            ls += s_ml[w][hh][1] * f;
        }
        if (final_out) {
            const int64_t row = (int64_t)b * a.Hq + (int64_t)g * G + hh;
            const uint32_t pk = pack2_bf16(ls > 0.0f ? o / ls : 0.0f, 0.0f);
            static_cast<uint16_t*>(a.out)[row * D + d] = (uint16_t)(pk & 0xffffu);
            if (d == 0 && a.lse) a.lse[row] = ls > 0.0f ? (M + log2f(ls)) * kLn2 : -INFINITY;
        } else {
            a.part[slot * G * D + e] = o;
            if (d == 0) {
                a.ml[(slot * G + hh) * 2 + 0] = M;
                a.ml[(slot * G + hh) * 2 + 1] = ls;
            }
        }
    }
}

template <int D, bool FUSED, int G>
int launch_q4(const KiviDecodeArgs& a, int waves, hipStream_t st)
{
    constexpr int NW = kivi_waves(FUSED, G);
    if (waves != NW) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL((q4_decode_kernel<D, FUSED, G, NW>), dim3(a.n_splits, a.B * a.Hkv), dim3(64 * NW), 0, st, a);
    const int rc = (int)hipGetLastError();
    if (rc || a.n_splits == 1) return rc;
    return launch_decode_combine_bf16(a, st);
}

template <int D, bool FUSED>
int launch_q4_g(const KiviDecodeArgs& a, int waves, hipStream_t st)
{
    switch (a.G) {
    case 1: return launch_q4<D, FUSED, 1>(a, waves, st);
    case 2: return launch_q4<D, FUSED, 2>(a, waves, st);
    case 4: return launch_q4<D, FUSED, 4>(a, waves, st);
    case 8: return launch_q4<D, FUSED, 8>(a, waves, st);
    default: return (int)hipErrorInvalidValue;
    }
}

template <bool FUSED>
int launch_q4_d(const KiviDecodeArgs& a, int waves, hipStream_t st)
{
    switch (a.D) {
    case 64: return launch_q4_g<64, FUSED>(a, waves, st);
    case 80: return launch_q4_g<80, FUSED>(a, waves, st);
    case 96: return launch_q4_g<96, FUSED>(a, waves, st);
    case 128: return launch_q4_g<128, FUSED>(a, waves, st);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace

int launch_kivi_quantize(const KiviQuantArgs& a, void* stream)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (a.B == 0 || a.S == 0) return 0;
    int64_t n;
    if (a.is_value) {
        n = (int64_t)a.B * a.H * a.S * ((a.D + kGroup - 1) / kGroup);
    } else {
        n = (int64_t)a.B * a.H * ((a.S + kGroup - 1) / kGroup) * (a.D / 2);
    }
    const int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
    if (a.is_value) hipLaunchKernelGGL(kivi_quant_values_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
    else hipLaunchKernelGGL(kivi_quant_keys_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
    return (int)hipGetLastError();
}

int launch_kivi_decode(const KiviDecodeArgs& a, bool fused, int waves, void* stream)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (a.B == 0) return 0;
    if (a.n_splits < 1 || a.n_splits > 256 || (int64_t)a.B * a.Hkv > 65535) return (int)hipErrorInvalidValue;
    return fused ? launch_q4_d<true>(a, waves, st) : launch_q4_d<false>(a, waves, st);
}

}  // namespace fkv
