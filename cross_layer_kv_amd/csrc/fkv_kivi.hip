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
// gives the same codes.  Key codes are token-major, two per byte (channel 2i
// in the low nibble).  Value codes are channel-major inside 32-token blocks:
// the 16 bytes of (block, channel) are four words, word w holding tokens
// 4w + (e%4) + 16(e/4) for e = 0..7 with element e in nibble e/2 (even e)
// or 4 + e/2 (odd e); value scales and minima list a block's tokens in the
// same order.  This is the order in which the matrix-core products below
// consume them, so every operand is one aligned 4- or 16-byte load.
//
// Decode runs both products of a 32-token block on the matrix cores
// (v_mfma_f32_16x16x32_f16), the query heads of the KV head padded to 16:
//   scores^T [16 tokens x 16 heads] = codes [16 x 32 ch] * U [32 ch x 16 heads]
// with U = scale*log2e * q * a * s (the key weight and the group's key
// scale folded into the query) and a per-(head, group) constant
// sum q * a * m added after; and
//   O [16 heads x 16 ch] += P' [16 heads x 32 tokens] * codes [32 tok x 16 ch]
// with P' = p * s (the token's value scale folded into the probability) and
// the value minima accumulated separately as sum p * m per channel group.
// The scores' accumulator layout (a lane holds one head and 4 tokens) is
// exactly the P' operand layout, so no data moves between the products.
// Codes enter the matrix cores as IEEE binary16 subnormals n * 2^-24 --
// exact, and one mask (and shift) per pair of codes -- and the 2^24 is put
// back in float32.  The fusion weights a, a' fold into U and b, b' are
// applied once per output channel.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "fkv_internal.h"
#include "fkv_mfma_common.h"

namespace fkv {
namespace {

using namespace dev;

constexpr int kGroup = 32;       // elements per quantisation group
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

// Keys: one workgroup per (batch*head, 32-token group).  The group's rows
// are staged in LDS with 16-byte loads; four threads per channel pair take
// the pair's minimum and maximum over 8 tokens each and combine them across
// their quad; then one thread per (token, 8-channel chunk) writes that
// chunk's 4 bytes of codes, so the codes leave as whole words.
__global__ __launch_bounds__(256) void kivi_quant_keys_kernel(const KiviQuantArgs a)
{
    constexpr int kMaxD = 128;
    __shared__ uint32_t xs[kGroup][kMaxD / 2 + 1];  // bf16 channel pairs of each token
    __shared__ float pm[kMaxD], pr[kMaxD];
    const int np = a.D / 2, cpr = a.D / 8, ng = (a.S + kGroup - 1) / kGroup;
    const int bh = blockIdx.x / ng, j = blockIdx.x - (blockIdx.x / ng) * ng;
    const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
    const int tid = threadIdx.x;
    const int t0 = j * kGroup, n = min(kGroup, a.S - t0);
    const uint16_t* src = static_cast<const uint16_t*>(a.src.data) + (int64_t)b * a.src.sb + (int64_t)h * a.src.sh;
    for (int e = tid; e < n * cpr; e += 256) {
        const int tt = e / cpr, c = e - (e / cpr) * cpr;
        const uint4 u = stream16(src + (int64_t)(t0 + tt) * a.src.ss + c * 8);
        xs[tt][c * 4 + 0] = u.x;
        xs[tt][c * 4 + 1] = u.y;
        xs[tt][c * 4 + 2] = u.z;
        xs[tt][c * 4 + 3] = u.w;
    }
    __syncthreads();
    {
        // (np <= 64: the 256 threads cover every pair; quads are lanes 4p..4p+3)
        const int cp = tid >> 2, q = tid & 3;
        float lo_mn = INFINITY, lo_mx = -INFINITY, hi_mn = INFINITY, hi_mx = -INFINITY;
        if (cp < np) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int tt = q * 8 + k;
                if (tt < n) {
                    const uint32_t w = xs[tt][cp];
                    const float x0 = bf16_lo(w), x1 = bf16_hi(w);
                    lo_mn = fminf(lo_mn, x0);
                    lo_mx = fmaxf(lo_mx, x0);
                    hi_mn = fminf(hi_mn, x1);
                    hi_mx = fmaxf(hi_mx, x1);
                }
            }
        }
#pragma unroll
        for (int o = 1; o < 4; o <<= 1) {
            lo_mn = fminf(lo_mn, __shfl_xor(lo_mn, o));
            lo_mx = fmaxf(lo_mx, __shfl_xor(lo_mx, o));
            hi_mn = fminf(hi_mn, __shfl_xor(hi_mn, o));
            hi_mx = fmaxf(hi_mx, __shfl_xor(hi_mx, o));
        }
        if (cp < np && q == 0) {
            const QParams p0 = qparams(lo_mn, lo_mx), p1 = qparams(hi_mn, hi_mx);
            pm[2 * cp] = p0.m;
            pr[2 * cp] = p0.r;
            pm[2 * cp + 1] = p1.m;
            pr[2 * cp + 1] = p1.r;
            const int64_t mo = ((int64_t)bh * ng + j) * a.D + 2 * cp;
            uint16_t* sc = static_cast<uint16_t*>(a.scale);
            uint16_t* mn = static_cast<uint16_t*>(a.minv);
            sc[mo] = p0.sc16;
            sc[mo + 1] = p1.sc16;
            mn[mo] = p0.mn16;
            mn[mo + 1] = p1.mn16;
        }
    }
    __syncthreads();
    uint32_t* codes = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(a.codes) + ((int64_t)bh * a.S + t0) * np);
    for (int e = tid; e < n * cpr; e += 256) {
        const int tt = e / cpr, c = e - (e / cpr) * cpr;
        uint32_t acc = 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t w = xs[tt][c * 4 + k];
            const int ch = c * 8 + 2 * k;
            QParams p0{}, p1{};
            p0.m = pm[ch];
            p0.r = pr[ch];
            p1.m = pm[ch + 1];
            p1.r = pr[ch + 1];
            acc |= (qcode(bf16_lo(w), p0) | (qcode(bf16_hi(w), p1) << 4)) << (8 * k);
        }
        // row tt of the group, bytes 4c..4c+3 (D/2 bytes per row: a whole number of words)
        codes[tt * (np / 4) + c] = acc;
    }
}

// Value positions inside a 32-token block: element e of word w is token
// 4w + (e % 4) + 16 (e / 4), stored in nibble e / 2 (even e) or 4 + e / 2.
__device__ __forceinline__ int vblock_pos(int tt)  // token in block -> 8w + e
{
    return tt < 16 ? 8 * (tt >> 2) + (tt & 3) : 8 * ((tt - 16) >> 2) + 4 + ((tt - 16) & 3);
}

// Values: one workgroup per (batch*head, 32-token block).  The block is
// staged in LDS as float32; one thread per (token, channel group) takes the
// group's minimum, maximum and parameters, then one thread per channel packs
// the block's 32 codes of that channel.
__global__ __launch_bounds__(256) void kivi_quant_values_kernel(const KiviQuantArgs a)
{
    constexpr int kMaxD = 128;
    __shared__ float xs[kGroup][kMaxD + 1];
    __shared__ float pm[kGroup][4], pr[kGroup][4];
    const int nb = (a.S + kGroup - 1) / kGroup, ng = (a.D + kGroup - 1) / kGroup;
    const int bh = blockIdx.x / nb, j = blockIdx.x - (blockIdx.x / nb) * nb;
    const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
    const int tid = threadIdx.x;
    const int cpr = a.D / 8;
    for (int e = tid; e < kGroup * cpr; e += 256) {
        const int tt = e / cpr, c = e - (e / cpr) * cpr;
        const int t = j * kGroup + tt;
        uint4 u = make_uint4(0u, 0u, 0u, 0u);
        if (t < a.S)
            u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.src.data) + (int64_t)b * a.src.sb +
                                                (int64_t)t * a.src.ss + (int64_t)h * a.src.sh + c * 8);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            xs[tt][c * 8 + 2 * k] = bf16_lo(w[k]);
            xs[tt][c * 8 + 2 * k + 1] = bf16_hi(w[k]);
        }
    }
    __syncthreads();
    if (tid < kGroup * ng) {
        const int tt = tid / ng, g = tid - (tid / ng) * ng;
        const int d0 = g * kGroup, n = min(kGroup, a.D - d0);
        const bool live = j * kGroup + tt < a.S;
        QParams p{};
        if (live) {
            float mn = INFINITY, mx = -INFINITY;
            for (int c = 0; c < n; ++c) {
                mn = fminf(mn, xs[tt][d0 + c]);
                mx = fmaxf(mx, xs[tt][d0 + c]);
            }
            p = qparams(mn, mx);
        }
        pm[tt][g] = live ? p.m : 0.0f;
        pr[tt][g] = live ? p.r : 0.0f;
        const int64_t mo = (((int64_t)bh * nb + j) * ng + g) * kGroup + vblock_pos(tt);
        static_cast<uint16_t*>(a.scale)[mo] = live ? p.sc16 : (uint16_t)0;
        static_cast<uint16_t*>(a.minv)[mo] = live ? p.mn16 : (uint16_t)0;
    }
    __syncthreads();
    for (int c = tid; c < a.D; c += 256) {
        const int g = c / kGroup;
        uint32_t wd[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t acc = 0u;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int tt = 4 * w + (e & 3) + 16 * (e >> 2);
                QParams p{};
                p.m = pm[tt][g];
                p.r = pr[tt][g];
                const uint32_t q = j * kGroup + tt < a.S ? qcode(xs[tt][c], p) : 0u;
                const int nib = (e & 1) ? 4 + (e >> 1) : (e >> 1);
                acc |= q << (4 * nib);
            }
            wd[w] = acc;
        }
        *reinterpret_cast<uint4*>(static_cast<uint8_t*>(a.codes) + (((int64_t)bh * nb + j) * a.D + c) * 16) =
            make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
}

typedef __attribute__((ext_vector_type(4))) float f32x4;

// 8 bytes read once per call (non-temporal)
__device__ __forceinline__ uint2 stream8(const void* p)
{
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_nontemporal_load(static_cast<const u32x2*>(p));
    return make_uint2(v[0], v[1]);
}

__device__ __forceinline__ f32x4 mma16(uint4 a, uint4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(a), as_f16x8(b), c, 0, 0, 0);
}

// Eight 4-bit codes of one word -> eight binary16 subnormals n * 2^-24, the
// pair k holding nibbles k and k + 4.
__device__ __forceinline__ uint4 codes_f16(uint32_t w)
{
    return make_uint4(w & 0x000F000Fu, (w >> 4) & 0x000F000Fu, (w >> 8) & 0x000F000Fu, (w >> 12) & 0x000F000Fu);
}

// Key codes: the same pairs with one instruction fewer; pairs 1 and 3 come
// out 16x larger (nibbles 1, 5 and 3, 7 are masked in place), which the
// query side divides out exactly.
__device__ __forceinline__ uint4 codes_f16_k(uint32_t w)
{
    const uint32_t h = w >> 8;
    return make_uint4(w & 0x000F000Fu, w & 0x00F000F0u, h & 0x000F000Fu, h & 0x00F000F0u);
}

// fp16 pairs (x_k, x_{k+4}) of eight consecutive fp16 values held as four
// words (x0 x1)(x2 x3)(x4 x5)(x6 x7): the channel order of codes_f16.
__device__ __forceinline__ uint4 pair_k4(uint4 u)
{
    return make_uint4(__builtin_amdgcn_perm(u.z, u.x, 0x05040100u), __builtin_amdgcn_perm(u.z, u.x, 0x07060302u),
                      __builtin_amdgcn_perm(u.w, u.y, 0x05040100u), __builtin_amdgcn_perm(u.w, u.y, 0x07060302u));
}

__device__ __forceinline__ uint32_t pk_mul(uint32_t x, uint32_t y)
{
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, x) * __builtin_bit_cast(f16x2, y));
}
__device__ __forceinline__ uint4 pk_mul4(uint4 x, uint4 y)
{
    return make_uint4(pk_mul(x.x, y.x), pk_mul(x.y, y.y), pk_mul(x.z, y.z), pk_mul(x.w, y.w));
}
__device__ __forceinline__ float sum4(float v)  // over the 4 lanes l, l^16, l^32, l^48
{
    v += __shfl_xor(v, 16);
    return v + __shfl_xor(v, 32);
}
__device__ __forceinline__ float max4(float v)
{
    v = fmaxf(v, __shfl_xor(v, 16));
    return fmaxf(v, __shfl_xor(v, 32));
}

constexpr float kTwo24 = 16777216.0f;

template <int D, bool FUSED, int G, int NW>
__global__ __launch_bounds__(64 * NW) void q4_decode_kernel(const KiviDecodeArgs a)
{
    constexpr int NT = 64 * NW;
    constexpr int KS = (D + 31) / 32;  // 32-channel k-steps of the score product (= value groups)
    constexpr int NVB = D / 16;        // 16-channel column blocks of the output
    constexpr int NS = FUSED ? 2 : 1;  // key (and value) sources
    static_assert(G <= 16, "heads of a KV head fit the 16 rows");

    __shared__ float s_acc[NW][G][D];
    __shared__ float s_ml[NW][G][2];
    __shared__ float s_M[NW][NS][G][KS];

    const int split = blockIdx.x;
    const int bg = blockIdx.y;  // b * Hkv + g
    const int b = bg / a.Hkv, g = bg - (bg / a.Hkv) * a.Hkv;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, hb = lane >> 4;
    const bool hv = l16 < G;  // this lane's head column holds a real head

    int len = a.seqlens ? a.seqlens[b] : a.Sk;
    len = len < 0 ? 0 : (len > a.Sk ? a.Sk : len);
    const int t_begin = split * a.chunk;
    const int t_end = min(len, t_begin + a.chunk);
    const int ngk = (a.Sk + kGroup - 1) / kGroup;
    const int64_t bh = bg;

    // q * a * scale * log2e of this lane's head, as fp16 pairs in the
    // channel order of codes_f16: k-step ks, channels 32 ks + 8 hb + {k, k+4}
    // q * a * scale * log2e of each lane's head, fp16 pairs in the channel
    // order of the codes, kept in LDS (the same for every wave): lane
    // (head l16, quarter hb), k-step ks, channels 32 ks + 8 hb + {k, k+4}
    __shared__ uint4 s_qa[NS][KS][64];
    if (wave == 0) {
        const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.Hq + (int64_t)g * G + (hv ? l16 : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c0 = ks * 32 + hb * 8;
            const bool live = hv && c0 < D;
            uint4 u = make_uint4(0u, 0u, 0u, 0u);
            if (live) u = *reinterpret_cast<const uint4*>(qp + c0);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
            float qf[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                qf[2 * k] = bf16_lo(w[k]) * a.scale_log2;
                qf[2 * k + 1] = bf16_hi(w[k]) * a.scale_log2;
            }
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                float wt[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) wt[k] = 1.0f;
                if constexpr (FUSED) {
                    const float* wp = (s == 0 ? a.kw1 : a.kwn) + (int64_t)g * D + c0;
                    if (live) {
#pragma unroll
                        for (int k = 0; k < 8; ++k) wt[k] = wp[k];
                    }
                }
                // pairs 1 and 3 meet codes held 16x larger (codes_f16_k)
                uint4 v = make_uint4(pack2(qf[0] * wt[0], qf[4] * wt[4]),
                                     pack2(qf[1] * wt[1] * 0.0625f, qf[5] * wt[5] * 0.0625f),
                                     pack2(qf[2] * wt[2], qf[6] * wt[6]),
                                     pack2(qf[3] * wt[3] * 0.0625f, qf[7] * wt[7] * 0.0625f));
                if (!live) v = make_uint4(0u, 0u, 0u, 0u);
                s_qa[s][ks][lane] = v;
            }
        }
    }
    __syncthreads();

    const Q4View* ksrc[2] = {&a.qk1, &a.qkn};
    const Q4View* vsrc[2] = {&a.qv1, &a.qvn};
    const int nbv = (a.Sk + kGroup - 1) / kGroup;

    // Per-block metadata: NC = NS * KS * 2 chunks of 16 bytes per lane
    // quarter hb (scale or minimum, of one source and one 32-channel slice),
    // each fetched by one lane (column l16 = chunk) and parked in this
    // wave's LDS area, where every lane reads the chunks it needs.
    constexpr int NC = NS * KS * 2;
    static_assert(NC <= 16, "one metadata chunk per lane column");
    __shared__ uint4 s_meta[NW][2][NC][4];  // [wave][key, value][chunk][hb]
    // key-code chunks: 16 bytes, or 8 where a row (D/2 bytes) is not a
    // multiple of 16, so that no chunk spans two rows
    constexpr int CB = (D / 2) % 16 == 0 ? 16 : 8;
    constexpr int NCS = 16 * D / CB;         // chunks per source and block
    constexpr int NKI = (NS * NCS + 63) / 64;  // loads per lane and block
    using KChunk = typename std::conditional<CB == 16, uint4, uint2>::type;
    __shared__ __attribute__((aligned(16))) uint32_t s_kc[NW][NS * 4 * D];  // [wave]: a block's key codes

    // The loads of one 32-token block: key codes (staged through LDS, see
    // below), value codes (NVB column blocks) and one key and one value
    // metadata chunk.  The next block's are in flight while this one is
    // computed.
    //
    // Key codes: a block holds 32 token rows of D/2 bytes per source, one
    // contiguous range of 16 D bytes.  The wave reads it with contiguous
    // loads of CB bytes (chunk c of the block, source c / NCS, lands at byte
    // CB c of the wave's LDS area) and takes each lane's score-product
    // operand (4 bytes of one row) from LDS.  Loading the operands straight
    // from memory (4 bytes per lane spread over 16 rows) streams at about
    // 4 TB/s on gfx950, against 6.2 for contiguous loads of the same bytes.
    struct Blk {  // key side
        KChunk kraw[NKI];
        uint4 km;
    };
    struct VBlk {  // value side
        uint32_t vc[NS][NVB];
        uint4 vm;
    };
    // Every load is unconditional: out-of-range positions are clamped into
    // the arrays and their results zeroed, so the loop has no divergent
    // branches around memory instructions.
    auto load_block = [&](int t0, Blk& x) {
#pragma unroll
        for (int i = 0; i < NKI; ++i) {
            const int c = i * 64 + lane;
            const int s = NS == 1 ? 0 : (c < NCS ? 0 : 1);
            const int cc = c - s * NCS;                 // chunk within the source's block
            const int t = t0 + (cc * CB) / (D / 2);     // its token row
            const bool ok = c < NS * NCS && t < a.Sk;   // (rows past the cache read as zero)
            const uint8_t* kcp = static_cast<const uint8_t*>(ksrc[s]->codes) + bh * a.Sk * (D / 2) +
                                 (ok ? (int64_t)t0 * (D / 2) + cc * CB : 0);
            if constexpr (CB == 16) {
                const uint4 v = stream16(kcp);
                x.kraw[i] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
            } else {
                const uint2 v = stream8(kcp);
                x.kraw[i] = ok ? v : make_uint2(0u, 0u);
            }
        }
        // metadata chunk of this lane column (columns past NC fetch a copy of
        // chunk column mod NC and are never read).  Metadata loads are plain,
        // cached loads: a block's 192-byte metadata rows share cache lines
        // with the neighbouring blocks', which other waves read at about the
        // same time (streamed past the caches, those lines were fetched
        // twice: 1.029x the algorithmic bytes against 1.000x).
        const int j = t0 / kGroup;
        const int c = l16 % NC;
        const int s = c / (2 * KS), ks = (c >> 1) - (c / (2 * KS)) * KS, sm = c & 1;
        const Q4View& kv = *ksrc[s];
        const bool chan = ks * 32 + hb * 8 < D;
        const uint4 km = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(sm ? kv.minv : kv.scale) + (bh * ngk + j) * D +
                                  (chan ? ks * 32 + hb * 8 : 0));
        x.km = chan ? km : make_uint4(0u, 0u, 0u, 0u);
    };
    auto load_values = [&](int t0, VBlk& x) {
        const int j = t0 / kGroup;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const uint8_t* vcp = static_cast<const uint8_t*>(vsrc[s]->codes) + (bh * nbv + j) * D * 16;
#pragma unroll
            for (int n = 0; n < NVB; ++n)
                x.vc[s][n] = stream4(vcp + (n * 16 + l16) * 16 + hb * 4);
        }
        const int c = l16 % NC;
        const int s = c / (2 * KS), ks = (c >> 1) - (c / (2 * KS)) * KS, sm = c & 1;
        const Q4View& vv = *vsrc[s];
        x.vm = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(sm ? vv.minv : vv.scale) + ((bh * nbv + j) * KS + ks) * kGroup +
                        hb * 8);
    };

    // oacc: O of each source (rows: heads 4 hb + i, columns: channels);
    // mp: the value-minimum terms sum_t p_t m_t of each source, one column
    // per 32-channel group (column l16 = group, rows heads 4 hb + i)
    f32x4 oacc[NS][NVB];
    f32x4 mp[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int n = 0; n < NVB; ++n) oacc[s][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        mp[s] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    float m_run = -INFINITY, l_part = 0.0f;

    // park a block's metadata chunks in this wave's LDS area (wave-private:
    // in-order LDS access within the wave orders the writes after the
    // previous block's reads).  Key chunks are stored re-paired into the
    // (c, c+4) channel order of the codes, minima of pairs 1 and 3 scaled
    // by 16 to meet the query side's 1/16.
    auto park = [&](const Blk& x) {
#pragma unroll
        for (int i = 0; i < NKI; ++i) {
            const int c = i * 64 + lane;
            if ((NS * NCS) % 64 == 0 || c < NS * NCS)
                reinterpret_cast<KChunk*>(&s_kc[wave][0])[c] = x.kraw[i];
        }
        if (l16 < NC) {
            uint4 k = pair_k4(x.km);
            if (l16 & 1) {
                const uint32_t s16 = 0x4C004C00u;  // (16, 16) in binary16
                k.y = pk_mul(k.y, s16);
                k.w = pk_mul(k.w, s16);
            }
            s_meta[wave][0][l16][hb] = k;
        }
    };
    // One block.  PART: the block holds the end of the row (tokens past
    // t_end are masked); full blocks skip every per-token test.
    constexpr bool ALLCH = D % 32 == 0;  // every lane quarter holds real channels
    auto compute = [&](const Blk& x, const VBlk& y, int t0, auto part) {
            constexpr bool PART = decltype(part)::value;
            // ---- scores: two 16-token tiles, heads on the columns ----
            // cacc: sum over channels of q a m (log2 units) per head, the
            // same in every token row: the key minima as a matrix operand
            // whose 16 rows are equal
            f32x4 sc[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
            f32x4 cacc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    #pragma unroll
            for (int s = 0; s < NS; ++s)
    #pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const uint4 ksc = s_meta[wave][0][(s * KS + ks) * 2 + 0][hb];
                    const uint4 kmn = s_meta[wave][0][(s * KS + ks) * 2 + 1][hb];
                    const uint4 qav = s_qa[s][ks][lane];
                    const uint4 u = pk_mul4(qav, ksc);
                    cacc = mma16(kmn, qav, cacc);
    #pragma unroll
                    for (int tl = 0; tl < 2; ++tl) {
                        // this lane's 8 codes: row 16 tl + l16, bytes 16 ks + 4 hb
                        const bool chan = ALLCH || ks * 32 + hb * 8 < D;
                        const bool live = chan && (!PART || t0 + tl * 16 + l16 < t_end);
                        const uint32_t kc =
                            s_kc[wave][s * 4 * D + (tl * 16 + l16) * (D / 8) + (chan ? ks * 4 + hb : 0)];
                        sc[tl] = mma16(codes_f16_k(live ? kc : 0u), u, sc[tl]);
                    }
                }
            // lane: head l16; entries: tokens t0 + 16 tl + 4 hb + i
            float sv[8];
            float bmax = -INFINITY;
    #pragma unroll
            for (int tl = 0; tl < 2; ++tl)
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = t0 + tl * 16 + hb * 4 + i;
                    const float x = (hv && (!PART || t < t_end)) ? sc[tl][i] * kTwo24 + cacc[i] : -INFINITY;
                    sv[tl * 4 + i] = x;
                    bmax = fmaxf(bmax, x);
                }
            bmax = max4(bmax);
            const float m_new = fmaxf(m_run, bmax);
            if (__any(m_new > m_run)) {
                const float corr = rel_weight(m_run, m_new);
                l_part *= corr;
                // output rows are heads 4 hb + i: fetch those heads' factors
                // (lane h holds head h's factor: l16 = h, hb = 0)
                float cr[G];
    #pragma unroll
                for (int h = 0; h < G; ++h) cr[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(corr), h));
                float rc[4];
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float r = 1.0f;
    #pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        if (q4 * 4 + i < G && hb == q4) r = cr[q4 * 4 + i];
                    rc[i] = r;
                }
    #pragma unroll
                for (int s = 0; s < NS; ++s) {
    #pragma unroll
                    for (int n = 0; n < NVB; ++n)
    #pragma unroll
                        for (int i = 0; i < 4; ++i) oacc[s][n][i] *= rc[i];
    #pragma unroll
                    for (int i = 0; i < 4; ++i) mp[s][i] *= rc[i];
                }
                m_run = m_new;
            }
            const float msub = m_run == -INFINITY ? 0.0f : m_run;
            float pv[8];
    #pragma unroll
            for (int e = 0; e < 8; ++e) {
                pv[e] = exp2_fast(sv[e] - msub);  // (2^-inf = 0: masked entries)
                l_part += pv[e];
            }
            const uint4 p16 = make_uint4(pack2(pv[0], pv[1]), pack2(pv[2], pv[3]), pack2(pv[4], pv[5]), pack2(pv[6], pv[7]));

            // ---- O += P' * codes, P' = p * (token's value scale), per group ----
        if (l16 < NC) {
            // A metadata chunk lists 8 tokens, t0 + 16 (e/4) + 4 hb + e%4 for
            // entry e.  In the block that holds the end of the row, entries of
            // tokens past it are zeroed: their p is 0, but 0 * inf or NaN
            // metadata would still reach the sums.
            uint4 vm = y.vm;
            if (PART && t0 + kGroup > t_end) {
                uint32_t w[4];
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ta = t0 + 16 * ((2 * i) >> 2) + 4 * hb + ((2 * i) & 3);
                    w[i] = (ta < t_end ? 0x0000ffffu : 0u) | (ta + 1 < t_end ? 0xffff0000u : 0u);
                }
                vm = make_uint4(vm.x & w[0], vm.y & w[1], vm.z & w[2], vm.w & w[3]);
            }
            s_meta[wave][1][l16][hb] = vm;
        }
    #pragma unroll
            for (int s = 0; s < NS; ++s) {
                // minimum terms of every group at once: column l16 = group
                // l16's minima of this lane quarter's 8 tokens
                const uint4 mcol = l16 < KS ? s_meta[wave][1][(s * KS + (l16 < KS ? l16 : 0)) * 2 + 1][hb]
                                            : make_uint4(0u, 0u, 0u, 0u);
                mp[s] = mma16(p16, mcol, mp[s]);
    #pragma unroll
                for (int k = 0; k < KS; ++k) {
                    const uint4 vsc = s_meta[wave][1][(s * KS + k) * 2 + 0][hb];
                    const uint4 pa = pk_mul4(p16, vsc);
    #pragma unroll
                    for (int n = 2 * k; n < 2 * k + 2 && n < NVB; ++n)
                        oacc[s][n] = mma16(pa, codes_f16(y.vc[s][n]), oacc[s][n]);
                }
            }
    };

    // The next block's key-side loads are in flight while a block is
    // computed.  The value side is issued when a block starts and lands
    // during its score product, except in the 8-wave four-source kernel
    // (D = 128), which prefetches it one block ahead as well: elsewhere the
    // registers that prefetch would take buy a third wave per SIMD (the
    // 12-wave four-source kernel) or a fourth (the 16-wave single-source).
    const int step = NW * kGroup;
    Blk cur;
    VBlk vcur;
    int t0 = t_begin + wave * kGroup;
    constexpr bool VPRE = FUSED && NW == 8;  // prefetch the value side one block ahead
    if (t0 < t_end) {
        load_block(t0, cur);
        if constexpr (VPRE) load_values(t0, vcur);
    }
    for (; t0 < t_end; t0 += step) {
        park(cur);
        Blk nxt;
        VBlk vnxt;
        if (t0 + step < t_end) {
            load_block(t0 + step, nxt);
            if constexpr (VPRE) load_values(t0 + step, vnxt);
        }
        if constexpr (!VPRE) load_values(t0, vcur);
        if (t0 + kGroup <= t_end)
            compute(cur, vcur, t0, std::false_type{});
        else
            compute(cur, vcur, t0, std::true_type{});
        cur = nxt;
        if constexpr (VPRE) vcur = vnxt;
    }

    // ---- wave results: (m, l) and the minimum terms per head ----
    const float l_tot = sum4(l_part);
    if (hb == 0 && hv) {
        s_ml[wave][l16][0] = m_run;
        s_ml[wave][l16][1] = l_tot;
    }
    if (l16 < KS) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * hb + i < G) s_M[wave][s][4 * hb + i][l16] = mp[s][i];
    }
    __syncthreads();
    // lane: output column c = 16 n + l16 of heads 4 hb + i
#pragma unroll
    for (int n = 0; n < NVB; ++n) {
        const int c = n * 16 + l16;
        const int k = c / kGroup;
        float w1 = 1.0f, wn = 0.0f;
        if constexpr (FUSED) {
            w1 = a.vw1[(int64_t)g * D + c];
            wn = a.vwn[(int64_t)g * D + c];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = hb * 4 + i;
            if (h < G) {
                float o = w1 * (oacc[0][n][i] * kTwo24 + s_M[wave][0][h][k]);
                if constexpr (FUSED) o += wn * (oacc[NS - 1][n][i] * kTwo24 + s_M[wave][NS - 1][h][k]);
                s_acc[wave][h][c] = o;
            }
        }
    }
    __syncthreads();

    // ---- merge the waves; write O/LSE (one split) or this split's partial row ----
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
    constexpr int NW = kivi_waves(FUSED, G, D);
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
    int64_t blocks;
    if (a.is_value) {
        blocks = (int64_t)a.B * a.H * ((a.S + kGroup - 1) / kGroup);  // one workgroup per 32-token block
    } else {
        blocks = (int64_t)a.B * a.H * ((a.S + kGroup - 1) / kGroup);  // one workgroup per 32-token group
    }
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
