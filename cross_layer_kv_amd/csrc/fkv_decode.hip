// fkv_decode.hip -- split-K flash-decode for FusedKV reconstruction layers on
// gfx950 (CDNA4, wave64).
//
// Pages cited (by title):
//   [Deck]  "FusedKV: Reconstructing KV Caches with Cross-Layer Fusion"
//   [Notes] "FusedKV:通过跨层融合重构 KV 缓存"
//
// What a call computes: for every batch row b and query head h (KV head
// g = h / G), attention of q[b, h] over keys a(.)K1 + a'(.)Kn and values
// b(.)V1 + b'(.)Vn of KV head g ([Deck] frame "FusedKV learns two-source,
// channel-wise fusion", Eqs. (4)-(5)), or over one key and one value source
// for FusedKV-Lite / the plain control ([Deck] frame "Lite separates the key
// source from the value source", Eq. (6)).  The reconstruction is formed in
// float32 registers, tile by tile, and never stored ([Notes] section 2.3).
//
// Decode is bound by HBM: every cached element is read once and used for a
// handful of flops ([Deck] frame "Decode cost depends on the inference
// regime": memory-bound TPOT of FusedKV is about 1.5x vanilla over a model).
// The design therefore aims only at streaming the source caches at full
// bandwidth with little VALU work per byte:
//   * a workgroup owns one (batch, KV head) -- or a split of its key axis
//     when there are too few of them to fill the chip -- and all G query heads
//     of that KV head, so each fused element is built once and used G times;
//     its waves stream consecutive 16-token slices;
//   * a lane owns 8 channels (one 16-byte bf16 load, two for f32) of one
//     token; the D/8 lanes of a token form an 8- or 16-lane group, and the
//     score of that token is a DPP butterfly sum inside the group;
//   * each lane runs its own online softmax over the tokens its group sees;
//     groups (lane exchanges), waves (LDS) and splits are merged with the
//     usual (max, sum) rescaling, in the log2 domain (scale * log2 e is folded
//     into the query);
//   * with one split per (batch, KV head) the workgroup writes O and LSE
//     directly; otherwise a second, small kernel merges the splits.  No
//     workgroup waits on another, and no device-scope fence is needed: on
//     this part such a fence writes back the L2, and one per workgroup cost
//     more than a third of the kernel's time when it was measured.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "fkv_internal.h"

namespace fkv {

// ---- static scratch of the allocation-free decode entry point ----
// Split partials of fkv_decode_noalloc live here instead of in a caller
// workspace.  Each GPU the library runs on holds its own copy for the life of
// the process.  In host code the array's name is only a stand-in for the
// device symbol; its device address comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that address is handed to
// kernels.
static __device__ __attribute__((aligned(256))) unsigned char scratch[kNoallocScratchBytes];

int scratch_pointer(void** out)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        if (!p) return (int)hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return 0;
}

namespace {

constexpr int kCombineThreads = 256;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Raw bits of C channels of one row: 8 channels are one 16-byte load for
// bf16 (two for f32); 6 bf16 channels are one 12-byte load.
template <typename T, int C>
struct RawC {
    static constexpr int NW = C * (int)sizeof(T) / 4;  // 32-bit words
    uint32_t w[NW];
};

// Every source byte is read once per call: the loads are non-temporal
// ("nt"), which streams them past the caches (80% of HBM peak against 71%
// with plain loads at the 650M shape).
template <typename T, int C>
__device__ __forceinline__ void loadc(RawC<T, C>& r, const T* p, bool pred)
{
    constexpr int NW = RawC<T, C>::NW;
    if constexpr (NW % 4 == 0) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int i = 0; i < NW / 4; ++i) {
            const u32x4 v = pred ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + i) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int k = 0; k < 4; ++k) r.w[4 * i + k] = v[k];
        }
    } else {
        static_assert(NW == 3, "12-byte rows pieces");
        // 4-byte aligned 12-byte pieces (row starts are 16-byte aligned, a
        // piece starts at 12 * lane within the row)
        typedef unsigned int u32x3 __attribute__((ext_vector_type(3), aligned(4)));
        const u32x3 v = pred ? __builtin_nontemporal_load(reinterpret_cast<const u32x3*>(p)) : u32x3{0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < 3; ++k) r.w[k] = v[k];
    }
}

template <typename T, int C>
__device__ __forceinline__ void widenc(const RawC<T, C>& r, float* f)
{
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < C / 2; ++i) {
            f[2 * i] = bf16_lo(r.w[i]);
            f[2 * i + 1] = bf16_hi(r.w[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < C; ++i) f[i] = __uint_as_float(r.w[i]);
    }
}

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float x)
{
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    bf16x2 v;
    v[0] = (__bf16)x;  // round to nearest even
    v[1] = (__bf16)0.0f;
    return (uint16_t)(__builtin_bit_cast(uint32_t, v) & 0xffffu);
}

// Sum over the LPT lanes of a token group with DPP lane permutations:
// xor 1, xor 2 (quad permutes), then mirror within 8 and within 16 lanes.
// After the quad steps every lane of a quad holds the quad sum, so the
// mirrors add exactly the partner quad / partner half-row.
template <int LPT>
__device__ __forceinline__ float group_sum(float v)
{
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    if constexpr (LPT == 16)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    return v;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Weight of a partial (max m) relative to a common max M; 0 for an empty one.
__device__ __forceinline__ float rel(float m, float M) { return m == -INFINITY ? 0.0f : exp2_fast(m - M); }

template <typename T, int D, bool FUSED, int G, int NW>
__global__ __launch_bounds__(64 * NW) void decode_kernel(const DecodeArgs a)
{
    constexpr int NT = 64 * NW;
    // channels per lane: 8, or 6 for bf16 rows of 96 channels, so that the
    // 16 lanes of a token group are all busy (one 12-byte load each)
    constexpr int CPL = (sizeof(T) == 2 && D == 96) ? 6 : 8;
    constexpr int NP = D / CPL;            // pieces per row
    constexpr int LPT = NP <= 8 ? 8 : 16;  // lanes per token group
    constexpr int TPW = 64 / LPT;          // tokens per wave step
    constexpr int WT = decode_wave_tokens(sizeof(T) == 4, FUSED, G, D);  // tokens per wave per iteration
    constexpr int U = WT / TPW;            // steps per iteration

    __shared__ float s_acc[NW][G][D];
    __shared__ float s_ml[NW][G][2];

    const int split = blockIdx.x;
    const int bg = blockIdx.y;  // b * Hkv + g
    const int b = bg / a.Hkv, g = bg - (bg / a.Hkv) * a.Hkv;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int grp = lane / LPT, pc = lane % LPT;
    const bool active = pc < NP;
    const int c0 = active ? pc * CPL : 0;

    int len = a.seqlens ? a.seqlens[b] : a.Sk;
    len = len < 0 ? 0 : (len > a.Sk ? a.Sk : len);
    const int t_begin = split * a.chunk;
    const int t_end = min(len, t_begin + a.chunk);

    // Query of the G heads, pre-scaled into the log2 domain, and the lane's
    // fusion weights.
    float qs[G][CPL];
    {
        const T* qp = static_cast<const T*>(a.q) + ((int64_t)b * a.Hq + (int64_t)g * G) * D + c0;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            RawC<T, CPL> r;
            loadc(r, qp + (int64_t)hh * D, active);
            widenc(r, qs[hh]);
#pragma unroll
            for (int c = 0; c < CPL; ++c) qs[hh][c] *= a.scale_log2;
        }
    }
    float wk1[CPL], wkn[CPL], wv1[CPL], wvn[CPL];
    if constexpr (FUSED) {
        const int64_t wo = (int64_t)g * D + c0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            wk1[c] = active ? a.kw1[wo + c] : 0.0f;
            wkn[c] = active ? a.kwn[wo + c] : 0.0f;
            wv1[c] = active ? a.vw1[wo + c] : 0.0f;
            wvn[c] = active ? a.vwn[wo + c] : 0.0f;
        }
    }

    const T* k1p = static_cast<const T*>(a.k1.data) + (int64_t)b * a.k1.sb + (int64_t)g * a.k1.sh + c0;
    const T* v1p = static_cast<const T*>(a.v1.data) + (int64_t)b * a.v1.sb + (int64_t)g * a.v1.sh + c0;
    const T* knp = k1p;
    const T* vnp = v1p;
    if constexpr (FUSED) {
        knp = static_cast<const T*>(a.kn.data) + (int64_t)b * a.kn.sb + (int64_t)g * a.kn.sh + c0;
        vnp = static_cast<const T*>(a.vn.data) + (int64_t)b * a.vn.sb + (int64_t)g * a.vn.sh + c0;
    }

    float m[G], l[G], acc[G][CPL];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        m[hh] = -INFINITY;
        l[hh] = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[hh][c] = 0.0f;
    }

    // The loads of one wave step: U token slices of each source.
    struct Blk {
        RawC<T, CPL> k1[U], kn[U], v1[U], vn[U];
    };
    auto load_blk = [&](int t0, Blk& x) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t0 + u * TPW + grp;
            const bool pr = active && t < t_end;
            loadc(x.k1[u], k1p + (int64_t)t * a.k1.ss, pr);
            if constexpr (FUSED) loadc(x.kn[u], knp + (int64_t)t * a.kn.ss, pr);
            loadc(x.v1[u], v1p + (int64_t)t * a.v1.ss, pr);
            if constexpr (FUSED) loadc(x.vn[u], vnp + (int64_t)t * a.vn.ss, pr);
        }
    };
    // Single-source bf16 steps at G <= 4 keep the next step's loads in flight
    // while one is computed: the registers fit without costing a wave per
    // SIMD (+1.6% for the 650M-shape Lite layer in a same-box A/B).  The
    // four-source kernel would drop from 16 to 12 waves, which measured
    // slower, so it issues each step's loads when the step starts.
    constexpr bool PREF = !FUSED && sizeof(T) == 2 && G <= 4;
    Blk cur;
    int t0 = t_begin + wave * WT;
    if constexpr (PREF) {
        if (t0 < t_end) load_blk(t0, cur);
    }
    for (; t0 < t_end; t0 += NW * WT) {
        Blk nxt;
        if constexpr (PREF) {
            if (t0 + NW * WT < t_end) load_blk(t0 + NW * WT, nxt);
        } else {
            load_blk(t0, cur);
        }
        const RawC<T, CPL>(&rk1)[U] = cur.k1;
        const RawC<T, CPL>(&rkn)[U] = cur.kn;
        const RawC<T, CPL>(&rv1)[U] = cur.v1;
        const RawC<T, CPL>(&rvn)[U] = cur.vn;
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) ok[u] = t0 + u * TPW + grp < t_end;

        // scores of the U tokens of this lane's group, log2 domain
        float s[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[CPL];
            widenc(rk1[u], kf);
            if constexpr (FUSED) {
                float kn[CPL];
                widenc(rkn[u], kn);
#pragma unroll
                for (int c = 0; c < CPL; ++c) kf[c] = wk1[c] * kf[c] + wkn[c] * kn[c];
            }
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                float d = 0.0f;
#pragma unroll
                for (int c = 0; c < CPL; ++c) d += qs[hh][c] * kf[c];
                d = group_sum<LPT>(d);
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
                const float corr = rel(m[hh], mx);
                l[hh] *= corr;
#pragma unroll
                for (int c = 0; c < CPL; ++c) acc[hh][c] *= corr;
                m[hh] = mx;
            }
            msub[hh] = m[hh] == -INFINITY ? 0.0f : m[hh];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[CPL];
            widenc(rv1[u], vf);
            if constexpr (FUSED) {
                float vn[CPL];
                widenc(rvn[u], vn);
#pragma unroll
                for (int c = 0; c < CPL; ++c) vf[c] = wv1[c] * vf[c] + wvn[c] * vn[c];
            }
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                const float p = exp2_fast(s[u][hh] - msub[hh]);
                l[hh] += p;
#pragma unroll
                for (int c = 0; c < CPL; ++c) acc[hh][c] += p * vf[c];
            }
        }
        if constexpr (PREF) cur = nxt;
    }

    // merge the token groups of the wave (lanes with equal pc)
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const float mo = __shfl_xor(m[hh], off);
            const float lo = __shfl_xor(l[hh], off);
            const float M = fmaxf(m[hh], mo);
            const float fa = rel(m[hh], M), fb = rel(mo, M);
            l[hh] = l[hh] * fa + lo * fb;
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[hh][c] = acc[hh][c] * fa + __shfl_xor(acc[hh][c], off) * fb;
            m[hh] = M;
        }
    }
    if (grp == 0 && active) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
            for (int c = 0; c < CPL; ++c) s_acc[wave][hh][c0 + c] = acc[hh][c];
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
            const float f = rel(s_ml[w][hh][0], M);
            o += s_acc[w][hh][d] * f;
            ls += s_ml[w][hh][1] * f;
        }
        if (final_out) {
            const int64_t row = (int64_t)b * a.Hq + (int64_t)g * G + hh;
            static_cast<T*>(a.out)[row * D + d] = from_f32<T>(ls > 0.0f ? o / ls : 0.0f);
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

// Merge of the split partials of one (batch, KV head) per workgroup:
// M = max_s m_s, w_s = 2^(m_s - M), L = sum_s w_s l_s, O = sum_s w_s o_s / L.
template <typename T, int D, int G>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const DecodeArgs a)
{
    __shared__ float s_w[256 * G];
    __shared__ float4 s_red[kCombineThreads];
    __shared__ float s_M[G], s_L[G];
    const int bg = blockIdx.x;
    const int b = bg / a.Hkv, g = bg - (bg / a.Hkv) * a.Hkv;
    const int tid = threadIdx.x;
    const int ns = a.n_splits;
    const float* mlp = a.ml + (int64_t)bg * ns * G * 2;
    const float* pp = a.part + (int64_t)bg * ns * G * D;

    for (int i = tid; i < ns * G; i += kCombineThreads) s_w[i] = mlp[2 * i];
    __syncthreads();
    if (tid < G) {
        float M = -INFINITY;
        for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, s_w[sp * G + tid]);
        s_M[tid] = M;
    }
    __syncthreads();
    for (int i = tid; i < ns * G; i += kCombineThreads) s_w[i] = rel(s_w[i], s_M[i % G]);
    __syncthreads();
    if (tid < G) {
        float L = 0.0f;
        for (int sp = 0; sp < ns; ++sp) L += s_w[sp * G + tid] * mlp[2 * (sp * G + tid) + 1];
        s_L[tid] = L;
    }
    __syncthreads();

    // float4 columns; the splits are spread over NSUB threads per column so
    // that many loads are in flight
    constexpr int NE4 = G * D / 4;
    constexpr int NSUB = kCombineThreads / NE4;
    static_assert(NE4 <= kCombineThreads && NSUB >= 1, "merge layout");
    if (tid < NSUB * NE4) {
        const int sub = tid / NE4, e4 = tid - (tid / NE4) * NE4;
        const int hh = (e4 * 4) / D;
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        const float4* p4 = reinterpret_cast<const float4*>(pp) + e4;
#pragma unroll 8
        for (int sp = sub; sp < ns; sp += NSUB) {
            const float w = s_w[sp * G + hh];
            const float4 x = p4[(int64_t)sp * NE4];
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
        const int64_t row = (int64_t)b * a.Hq + (int64_t)g * G + hh;
        T* op = static_cast<T*>(a.out) + row * D + d;
        op[0] = from_f32<T>(o.x * inv);
        op[1] = from_f32<T>(o.y * inv);
        op[2] = from_f32<T>(o.z * inv);
        op[3] = from_f32<T>(o.w * inv);
        if (d == 0 && a.lse) a.lse[row] = L > 0.0f ? (s_M[hh] + log2f(L)) * kLn2 : -INFINITY;
    }
}

template <typename T, int D, bool FUSED, int G>
int launch_one(const DecodeArgs& a, int waves, hipStream_t st)
{
    constexpr int NW = decode_waves(sizeof(T) == 4, FUSED, G);
    if (waves != NW) return (int)hipErrorInvalidValue;
    const dim3 grid(a.n_splits, a.B * a.Hkv);
    hipLaunchKernelGGL((decode_kernel<T, D, FUSED, G, NW>), grid, dim3(64 * NW), 0, st, a);
    int rc = (int)hipGetLastError();
    if (rc || a.n_splits == 1) return rc;
    hipLaunchKernelGGL((combine_kernel<T, D, G>), dim3(a.B * a.Hkv), dim3(kCombineThreads), 0, st, a);
    return (int)hipGetLastError();
}

template <typename T, int D, bool FUSED>
int launch_g(const DecodeArgs& a, int waves, hipStream_t st)
{
    switch (a.G) {
    case 1: return launch_one<T, D, FUSED, 1>(a, waves, st);
    case 2: return launch_one<T, D, FUSED, 2>(a, waves, st);
    case 4: return launch_one<T, D, FUSED, 4>(a, waves, st);
    case 8: return launch_one<T, D, FUSED, 8>(a, waves, st);
    default: return (int)hipErrorInvalidValue;
    }
}

template <typename T, bool FUSED>
int launch_d(const DecodeArgs& a, int waves, hipStream_t st)
{
    switch (a.D) {
    case 64: return launch_g<T, 64, FUSED>(a, waves, st);
    case 80: return launch_g<T, 80, FUSED>(a, waves, st);
    case 96: return launch_g<T, 96, FUSED>(a, waves, st);
    case 128: return launch_g<T, 128, FUSED>(a, waves, st);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace

int launch_decode_combine_bf16(const DecodeArgs& a, void* stream)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (a.n_splits <= 1) return 0;
    switch (a.D * 16 + a.G) {
#define FKV_COMBINE_CASE(DD, GG)                                                                                 \
    case DD * 16 + GG:                                                                                           \
        hipLaunchKernelGGL((combine_kernel<uint16_t, DD, GG>), dim3(a.B * a.Hkv), dim3(kCombineThreads), 0, st, a); \
        break;
        FKV_COMBINE_CASE(64, 1) FKV_COMBINE_CASE(64, 2) FKV_COMBINE_CASE(64, 4) FKV_COMBINE_CASE(64, 8)
        FKV_COMBINE_CASE(80, 1) FKV_COMBINE_CASE(80, 2) FKV_COMBINE_CASE(80, 4) FKV_COMBINE_CASE(80, 8)
        FKV_COMBINE_CASE(96, 1) FKV_COMBINE_CASE(96, 2) FKV_COMBINE_CASE(96, 4) FKV_COMBINE_CASE(96, 8)
        FKV_COMBINE_CASE(128, 1) FKV_COMBINE_CASE(128, 2) FKV_COMBINE_CASE(128, 4) FKV_COMBINE_CASE(128, 8)
#undef FKV_COMBINE_CASE
    default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

int launch_decode(const DecodeArgs& a, bool fused, int dtype, int waves, void* stream)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (a.B == 0) return 0;
    if (a.n_splits < 1 || a.n_splits > 256 || (int64_t)a.B * a.Hkv > 65535) return (int)hipErrorInvalidValue;
    if (dtype == 0) return fused ? launch_d<float, true>(a, waves, st) : launch_d<float, false>(a, waves, st);
    return fused ? launch_d<uint16_t, true>(a, waves, st) : launch_d<uint16_t, false>(a, waves, st);
}

}  // namespace fkv
