// fkv_decode_mfma.hip -- FusedKV decode for high GQA ratios (G = 64 query
// heads per KV head) on gfx950 matrix cores (fp16 operands, fp32 accumulate).
//
// Pages cited (by title):
//   [Deck]  "FusedKV: Reconstructing KV Caches with Cross-Layer Fusion"
//   [Notes] "FusedKV:通过跨层融合重构 KV 缓存"
//
// What a call computes: for one new token per sequence, O = softmax(q K^T *
// scale) V for each of the G query heads of a KV head, with keys
// a(.)K1 + a'(.)Kn and values b(.)V1 + b'(.)Vn fused on the fly ([Deck] frame
// "FusedKV learns two-source, channel-wise fusion", Eqs. (4)-(5)), or one key
// and one value source (FusedKV-Lite, Eq. (6), or the plain control).  The
// pages show a second decode regime with many query heads per KV head
// ([Deck] frame "Decode cost depends on the inference regime", Fig. 5,
// right): there the work per cached token grows with G while the bytes do
// not, so the per-token dot products belong on the matrix cores and the
// fusion, done once per token for all G heads, is amortised.
//
// Layout of the work
//   * One workgroup of 4 waves per (batch, KV head, split of the key axis).
//     The 64 query heads are the columns of the matrix-core products, in two
//     blocks of 32; a wave owns one head block and one 32-key half of every
//     64-key tile, so each fused tile is used by all 64 heads.
//   * Scores S^T = K~ Q^T (v_mfma_f32_32x32x16_f16): a lane holds 16 scores of
//     one head; the row max / sum take one exchange with the lane 32 apart.
//     O^T += V~^T P^T reads V~ row-major through transposing LDS reads.
//   * Tiles are fused into double-buffered LDS; the next tile's source loads
//     are issued as the tile's score product starts.  One barrier per tile.
//   * The two key halves of a head block merge in LDS at the end; with
//     several splits, partial (max, sum, O) rows go to the workspace and a
//     second kernel merges them per group of 8 heads.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fkv_internal.h"
#include "fkv_mfma_common.h"

namespace fkv {
namespace {

using namespace dev;

constexpr int kHG = 64;               // query heads per KV head
constexpr int kHWaves = 4;            // 2 key halves x 2 head blocks
constexpr int kHThreads = 64 * kHWaves;
constexpr int kHBN = 64;              // keys per tile
constexpr int kHeadsPerCombine = 8;   // heads merged by one combine workgroup
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float rel2(float m, float M) { return m == -INFINITY ? 0.0f : exp2_fast(m - M); }

template <int D, bool FUSED>
__global__ __launch_bounds__(kHThreads, 2) void hgqa_decode_kernel(const DecodeArgs a)
{
    constexpr int DP = (D + 31) / 32 * 32;
    constexpr int KS = D / 16;           // k-steps of the score product
    constexpr int NDB = DP / 32;         // 32-channel blocks of the output
    constexpr int KP = D + 8;            // LDS row pitch of K~ (elements)
    constexpr int VP = D <= 96 ? 96 : 160;  // LDS row pitch of V~
    constexpr int CPR = D / 8;           // 16-byte chunks per key row
    constexpr int RPP = kHThreads / CPR; // key rows per staging pass
    constexpr int KPASS = (kHBN + RPP - 1) / RPP;
    constexpr int NSRC = FUSED ? 4 : 2;  // sources: keys first, then values
    constexpr int NKS = FUSED ? 2 : 1;
    constexpr int NL = NSRC * KPASS;     // 16-byte loads per thread per tile

    // K~ and V~ tile buffers (one spare row each takes the stores of idle
    // staging lanes) in one LDS block, which the final merge reuses
    constexpr int KT_ELEMS = 2 * (kHBN + 1) * KP, VT_ELEMS = 2 * (kHBN + 1) * VP;
    constexpr int MERGE_BYTES = (2 * NDB * 16 * 64 + 2 * 2 * 32) * 4;
    constexpr int SMEM_BYTES = (KT_ELEMS + VT_ELEMS) * 2 > MERGE_BYTES ? (KT_ELEMS + VT_ELEMS) * 2 : MERGE_BYTES;
    __shared__ __attribute__((aligned(16))) uint4 smem[(SMEM_BYTES + 15) / 16];
    auto& Kt = *reinterpret_cast<uint16_t(*)[2][(kHBN + 1) * KP]>(&smem[0]);
    auto& Vt = *reinterpret_cast<uint16_t(*)[2][(kHBN + 1) * VP]>(reinterpret_cast<uint16_t*>(&smem[0]) + KT_ELEMS);
    __shared__ __attribute__((aligned(16))) uint32_t Wt[FUSED ? 4 * D : 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kh = wave & 1, hb = wave >> 1;  // key half, head block
    const int l32 = lane & 31, hi = lane >> 5;

    const int split = blockIdx.x, bg = blockIdx.y;
    const int b = bg / a.Hkv, g = bg - (bg / a.Hkv) * a.Hkv;
    int len = a.seqlens ? a.seqlens[b] : a.Sk;
    len = len < 0 ? 0 : (len > a.Sk ? a.Sk : len);
    const int k0 = split * a.chunk;
    const int k1 = min(len, k0 + a.chunk);
    const int nt = k1 > k0 ? (k1 - k0 + kHBN - 1) / kHBN : 0;
    const int head = g * kHG + hb * 32 + l32;  // this lane's query head
    const bool direct = a.n_splits == 1;
    const int64_t prow = ((int64_t)bg * a.n_splits + split) * kHG + hb * 32 + l32;  // partial row

    if (nt == 0) {  // no key of this split is visible: an empty partial
        if (kh == 0) {
            if (direct) {
                uint16_t* op = static_cast<uint16_t*>(a.out) + ((int64_t)b * a.Hq + head) * D;
                for (int c = hi * (D / 2); c < (hi + 1) * (D / 2); ++c) op[c] = 0;
                if (hi == 0 && a.lse) a.lse[(int64_t)b * a.Hq + head] = -INFINITY;
            } else {
                for (int c = hi * (D / 2); c < (hi + 1) * (D / 2); ++c) a.part[prow * D + c] = 0.0f;
                if (hi == 0) {
                    a.ml[prow * 2] = -INFINITY;
                    a.ml[prow * 2 + 1] = 0.0f;
                }
            }
        }
        return;
    }

    if constexpr (DP > D) {
        for (int i = tid; i < kHBN * (DP - D); i += kHThreads) {
            const int r = i / (DP - D), c = D + i % (DP - D);
            Vt[0][r * VP + c] = 0;
            Vt[1][r * VP + c] = 0;
        }
    }
    if constexpr (FUSED) {
        // w = hi + lo with both parts bf16 (~2^-16 relative): a fused element
        // is two bf16 dot products of its (source 1, source n) pair
        for (int i = tid; i < 2 * D; i += kHThreads) {
            const int ch = i % D;
            const bool val = i >= D;
            const float x = (val ? a.vw1 : a.kw1)[g * D + ch];
            const float y = (val ? a.vwn : a.kwn)[g * D + ch];
            const uint32_t whi = pack2_bf16(x, y);
            Wt[2 * i] = whi;
            Wt[2 * i + 1] = pack2_bf16(x - bf16_lo(whi), y - bf16_hi(whi));
        }
    }

    // queries: B operand of S^T = K~ Q^T, 8 channels per lane per k-step
    f16x8 qreg[KS];
    {
        const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.Hq + head) * D + hi * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qreg[ks] = as_f16x8(bf16x8_to_f16x8(*reinterpret_cast<const uint4*>(qp + ks * 16)));
    }

    // staging: a thread owns one 16-byte chunk column of KPASS key rows
    const int kc = tid % CPR, kr = tid / CPR;
    const bool active = kr < RPP;
    __amdgpu_buffer_rsrc_t rs[NSRC];
    uint32_t loff[NSRC][KPASS], rstep[NSRC];
    {
        const View* src[4] = {&a.k1, &a.kn, &a.v1, &a.vn};
        if constexpr (!FUSED) src[1] = &a.v1;
#pragma unroll
        for (int s = 0; s < NSRC; ++s) {
            const View& v = *src[s];
            const uint16_t* base = static_cast<const uint16_t*>(v.data) + (int64_t)b * v.sb + (int64_t)g * v.sh;
            // up to the end of row len-1: rows at or past len load zeros
            rs[s] = slab_rsrc(base, len > 0 ? (uint32_t)(((int64_t)(len - 1) * v.ss + D) * 2) : 0u);
            rstep[s] = (uint32_t)v.ss * 2;
#pragma unroll
            for (int p = 0; p < KPASS; ++p)
                loff[s][p] = (active && kr + p * RPP < kHBN) ? (uint32_t)(kr * v.ss * 2 + kc * 16) : kOffNone;
        }
    }
    int srow[KPASS];
#pragma unroll
    for (int p = 0; p < KPASS; ++p) srow[p] = (active && kr + p * RPP < kHBN) ? kr + p * RPP : kHBN;

    uint4 xr[NSRC][KPASS];
    auto load_one = [&](int t, int i) {
        const int s = i / KPASS, p = i % KPASS;
        const uint32_t so = (uint32_t)(k0 + t * kHBN + p * RPP) * rstep[s];
        xr[s][p] = ld16s(rs[s], loff[s][p], so);
    };
    auto fuse8 = [&](const uint4& u1, const uint4& un, const uint4* w) {
        const uint32_t x1[4] = {u1.x, u1.y, u1.z, u1.w};
        const uint32_t xn[4] = {un.x, un.y, un.z, un.w};
        uint32_t r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r[i] = pack2(fuse_pair(pair_lo(x1[i], xn[i]), w[i].x, w[i].y), fuse_pair(pair_hi(x1[i], xn[i]), w[i].z, w[i].w));
        return make_uint4(r[0], r[1], r[2], r[3]);
    };
    auto store_tile = [&](int nb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {  // 0: keys, 1: values
            uint4 w[4];
            if constexpr (FUSED) {
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = *reinterpret_cast<const uint4*>(&Wt[half * 2 * D + kc * 16 + 4 * i]);
            }
#pragma unroll
            for (int p = 0; p < KPASS; ++p) {
                uint4 o;
                if constexpr (FUSED) o = fuse8(xr[half * 2][p], xr[half * 2 + 1][p], w);
                else o = bf16x8_to_f16x8(xr[half * NKS][p]);
                if (half == 0) *reinterpret_cast<uint4*>(&Kt[nb][srow[p] * KP + kc * 8]) = o;
                else *reinterpret_cast<uint4*>(&Vt[nb][srow[p] * VP + kc * 8]) = o;
            }
        }
    };

    // O^T += V~^T P^T: the A operand (channels x keys) of 16-key step c comes
    // from the row-major V~ tile by two transposing reads (within each
    // 16-lane group, lane r reads 4 channels of one key row and receives one
    // channel of 4 key rows); its keys follow the score layout,
    // c*16 + hi*4 + e%4 + (e/4)*8 for element e.
    typedef short v4s __attribute__((ext_vector_type(4)));
    const uint16_t* vt_lane = &Vt[0][0] + (hi * 4 + ((l32 & 15) >> 2)) * VP + (l32 >> 4) * 16 + (l32 & 3) * 4;
    auto vfrag = [&](int buf, int c, int d) {
        const uint16_t* p = vt_lane + buf * ((kHBN + 1) * VP) + c * 16 * VP + d * 32;
        const v4s x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
        const v4s x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p + 8 * VP));
        return __builtin_bit_cast(f16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    f32x16 oacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY, l_run = 0.0f, l_run2 = 0.0f;
    const float sl2 = a.scale_log2;

    __syncthreads();  // weights, V~ padding
#pragma unroll
    for (int i = 0; i < NL; ++i) load_one(0, i);
    store_tile(0);
    __syncthreads();

    for (int t = 0; t < nt; ++t) {
        const int buf = t & 1;
        const bool more = t + 1 < nt;
        const int tbase = k0 + t * kHBN;
        // S^T for this wave's 32 keys x 32 heads; the next tile's loads are
        // all issued with the first k-step, so they are in flight for the
        // whole tile (1% faster than spreading them over the k-steps)
        f32x16 sacc = f32x16{};
        const uint16_t* kt = &Kt[buf][0] + (kh * 32 + l32) * KP + hi * 8;
        uint4 kf[KS];
#pragma unroll
        for (int ks = 0; ks < KS && ks < 2; ++ks) kf[ks] = *reinterpret_cast<const uint4*>(kt + ks * 16);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (more && ks == 0) {
#pragma unroll
                for (int i = 0; i < NL; ++i) load_one(t + 1, i);
            }
            if (ks + 2 < KS) kf[ks + 2] = *reinterpret_cast<const uint4*>(kt + (ks + 2) * 16);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(kf[ks]), qreg[ks], sacc, 0, 0, 0);
        }
        // keys at or past the end of the split (or of the sequence)
        if (tbase + kHBN > k1) {
            const int lim = k1 - 1 - tbase - kh * 32 - hi * 4;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if ((i >> 2) * 8 + (i & 3) > lim) sacc[i] = -INFINITY;
        }
        // running max with lazy rescale (reference raised only when a tile max
        // exceeds it by more than 8 in log2 units: probabilities stay <= 2^8)
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
        const float m_tile = halves_max(mx) * sl2;
        if (__any(m_tile > m_run + 8.0f)) {
            const float m_new = fmaxf(m_run, m_tile);
            const float corr = rel2(m_run, m_new);
            l_run *= corr;
            l_run2 *= corr;
#pragma unroll
            for (int d = 0; d < NDB; ++d)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[d][i] *= corr;
            m_run = m_new;
        }
        const float msub = m_run == -INFINITY ? 0.0f : m_run;
        f16x8 vf[2][NDB];
#pragma unroll
        for (int d = 0; d < NDB; ++d) vf[0][d] = vfrag(buf, 2 * kh, d);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p0 = exp2_fast(sacc[c * 8 + 2 * i] * sl2 - msub);
                const float p1 = exp2_fast(sacc[c * 8 + 2 * i + 1] * sl2 - msub);
                w[i] = pack2(p0, p1);
                if (i & 1) l_run2 = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w[i]), kOnes2, l_run2, false);
                else l_run = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w[i]), kOnes2, l_run, false);
            }
            if (c == 0) {
#pragma unroll
                for (int d = 0; d < NDB; ++d) vf[1][d] = vfrag(buf, 2 * kh + 1, d);
            }
            const f16x8 pbc = as_f16x8(make_uint4(w[0], w[1], w[2], w[3]));
#pragma unroll
            for (int d = 0; d < NDB; ++d) oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[c][d], pbc, oacc[d], 0, 0, 0);
        }
        if (more) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- merge the two key halves of each head block in LDS ----
    // The tile buffers are free after the loop's last barrier.
    float* xo = reinterpret_cast<float*>(&smem[0]);  // [hb][NDB * 16][64 lanes]
    float* xm = xo + 2 * NDB * 16 * 64;               // [hb][2][32 heads]
    const float l_tot = halves_sum(l_run + l_run2);
    if (kh == 1) {
#pragma unroll
        for (int d = 0; d < NDB; ++d)
#pragma unroll
            for (int i = 0; i < 16; ++i) xo[((hb * NDB + d) * 16 + i) * 64 + lane] = oacc[d][i];
        if (hi == 0) {
            xm[(hb * 2 + 0) * 32 + l32] = m_run;
            xm[(hb * 2 + 1) * 32 + l32] = l_tot;
        }
    }
    __syncthreads();
    if (kh == 1) return;
    const float mo = xm[(hb * 2 + 0) * 32 + l32], lo = xm[(hb * 2 + 1) * 32 + l32];
    const float M = fmaxf(m_run, mo);
    const float fa = rel2(m_run, M), fb = rel2(mo, M);
    const float L = fa * l_tot + fb * lo;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[d][i] = fa * oacc[d][i] + fb * xo[((hb * NDB + d) * 16 + i) * 64 + lane];

    // lane (l32, hi) holds channels d*32 + r*8 + hi*4 + 0..3 of its head
    if (direct) {
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        uint16_t* op = static_cast<uint16_t*>(a.out) + ((int64_t)b * a.Hq + head) * D;
#pragma unroll
        for (int d = 0; d < NDB; ++d)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ch = d * 32 + r * 8 + hi * 4;
                if (ch < D) {
                    const uint32_t w0 = pack2_bf16(oacc[d][r * 4 + 0] * inv, oacc[d][r * 4 + 1] * inv);
                    const uint32_t w1 = pack2_bf16(oacc[d][r * 4 + 2] * inv, oacc[d][r * 4 + 3] * inv);
                    *reinterpret_cast<uint2*>(op + ch) = make_uint2(w0, w1);
                }
            }
        if (hi == 0 && a.lse) a.lse[(int64_t)b * a.Hq + head] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
    } else {
        float* pp = a.part + prow * D;
#pragma unroll
        for (int d = 0; d < NDB; ++d)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ch = d * 32 + r * 8 + hi * 4;
                if (ch < D)
                    *reinterpret_cast<float4*>(pp + ch) =
                        make_float4(oacc[d][r * 4 + 0], oacc[d][r * 4 + 1], oacc[d][r * 4 + 2], oacc[d][r * 4 + 3]);
            }
        if (hi == 0) {
            a.ml[prow * 2] = M;
            a.ml[prow * 2 + 1] = L;
        }
    }
}

// Merge of the split partials for kHeadsPerCombine heads of one (batch, KV
// head): M = max_s m_s, w_s = 2^(m_s - M), L = sum_s w_s l_s,
// O = sum_s w_s o_s / L, LSE = ln 2 (M + log2 L).
template <int D>
__global__ __launch_bounds__(256) void hgqa_combine_kernel(const DecodeArgs a)
{
    constexpr int GS = kHeadsPerCombine;
    constexpr int NE4 = GS * D / 4;  // float4 columns
    constexpr int NSUB = 256 / NE4;
    static_assert(NE4 <= 256 && NSUB >= 1, "merge layout");
    __shared__ float s_w[256 * GS];
    __shared__ float4 s_red[256];
    __shared__ float s_M[GS], s_L[GS];
    const int bg = blockIdx.x, h0 = blockIdx.y * GS;
    const int b = bg / a.Hkv, g = bg - (bg / a.Hkv) * a.Hkv;
    const int tid = threadIdx.x;
    const int ns = a.n_splits;
    const float* mlp = a.ml + (int64_t)bg * ns * kHG * 2;
    const float* pp = a.part + (int64_t)bg * ns * kHG * D;

    for (int i = tid; i < ns * GS; i += 256) s_w[i] = mlp[((i / GS) * kHG + h0 + i % GS) * 2];
    __syncthreads();
    if (tid < GS) {
        float M = -INFINITY;
        for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, s_w[sp * GS + tid]);
        s_M[tid] = M;
    }
    __syncthreads();
    for (int i = tid; i < ns * GS; i += 256) s_w[i] = rel2(s_w[i], s_M[i % GS]);
    __syncthreads();
    if (tid < GS) {
        float L = 0.0f;
        for (int sp = 0; sp < ns; ++sp) L += s_w[sp * GS + tid] * mlp[(sp * kHG + h0 + tid) * 2 + 1];
        s_L[tid] = L;
    }
    __syncthreads();
    if (tid < NSUB * NE4) {
        const int sub = tid / NE4, e4 = tid - (tid / NE4) * NE4;
        const int hh = (e4 * 4) / D;
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        const float4* p4 = reinterpret_cast<const float4*>(pp + (int64_t)h0 * D) + e4;
        for (int sp = sub; sp < ns; sp += NSUB) {
            const float w = s_w[sp * GS + hh];
            const float4 x = p4[(int64_t)sp * (kHG * D / 4)];
            o.x += w * x.x;
            o.y += w * x.y;
            o.z += w * x.z;
            o.w += w * x.w;
        }
        s_red[tid] = o;
    }
    __syncthreads();
    if (tid < NE4) {
        float4 o = s_red[tid];
        for (int sub = 1; sub < NSUB; ++sub) {
            const float4 x = s_red[sub * NE4 + tid];
            o.x += x.x;
            o.y += x.y;
            o.z += x.z;
            o.w += x.w;
        }
        const int hh = (tid * 4) / D, d = tid * 4 - hh * D;
        const float L = s_L[hh];
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        const int64_t row = (int64_t)b * a.Hq + (int64_t)g * kHG + h0 + hh;
        uint16_t* op = static_cast<uint16_t*>(a.out) + row * D + d;
        *reinterpret_cast<uint2*>(op) = make_uint2(pack2_bf16(o.x * inv, o.y * inv), pack2_bf16(o.z * inv, o.w * inv));
        if (d == 0 && a.lse) a.lse[row] = L > 0.0f ? (s_M[hh] + log2f(L)) * kLn2 : -INFINITY;
    }
}

template <int D, bool FUSED>
int launch_hd(const DecodeArgs& a, hipStream_t st)
{
    hipLaunchKernelGGL((hgqa_decode_kernel<D, FUSED>), dim3(a.n_splits, a.B * a.Hkv), dim3(kHThreads), 0, st, a);
    int rc = (int)hipGetLastError();
    if (rc || a.n_splits == 1) return rc;
    hipLaunchKernelGGL((hgqa_combine_kernel<D>), dim3(a.B * a.Hkv, kHG / kHeadsPerCombine), dim3(256), 0, st, a);
    return (int)hipGetLastError();
}

template <bool FUSED>
int launch_hf(const DecodeArgs& a, hipStream_t st)
{
    switch (a.D) {
    case 64: return launch_hd<64, FUSED>(a, st);
    case 80: return launch_hd<80, FUSED>(a, st);
    case 96: return launch_hd<96, FUSED>(a, st);
    case 128: return launch_hd<128, FUSED>(a, st);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace

int launch_decode_hgqa(const DecodeArgs& a, bool fused, void* stream)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (a.B == 0) return 0;
    if (a.G != kHG || a.n_splits < 1 || a.n_splits > 256 || (int64_t)a.B * a.Hkv > 65535)
        return (int)hipErrorInvalidValue;
    return fused ? launch_hf<true>(a, st) : launch_hf<false>(a, st);
}

}  // namespace fkv
