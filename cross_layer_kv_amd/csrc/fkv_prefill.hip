// fkv_prefill.hip -- causal flash-attention prefill for FusedKV reconstruction
// layers on gfx950 matrix cores (fp16 operands, fp32 accumulate).
//
// Pages cited (by title):
//   [Deck]  "FusedKV: Reconstructing KV Caches with Cross-Layer Fusion"
//   [Notes] "FusedKV:通过跨层融合重构 KV 缓存"
//
// What a call computes: O = softmax(Q K^T * scale) V for every query row of
// the layer with keys a(.)K1 + a'(.)Kn and values b(.)V1 + b'(.)Vn ([Deck]
// frame "FusedKV learns two-source, channel-wise fusion", Eqs. (4)-(5)), or
// one key and one value source (FusedKV-Lite, [Deck] frame "Lite separates
// the key source from the value source", Eq. (6); or the plain control).
// The fusion runs on each 64-token tile as it is staged into LDS, never in
// HBM ([Notes] section 2.3).  The pages measure such a fused kernel at about
// 28% below an MHA kernel ([Deck] frame "Prefill improves while kernel
// throughput falls", Fig. 4): the extra source loads and fusion arithmetic
// are what this file keeps off the matrix-core critical path.
//
// Layout of the work
//   * A workgroup of 12 waves owns one (batch, KV head, tile of BM query
//     rows) and all G query heads of that KV head.  Waves 0-7 are the
//     matrix-core waves: 8 * 32 = 256 query columns, BM = 256 / G rows.
//     Waves 8-11, one per SIMD, stage the K/V tiles: they load the sources,
//     fuse them in float32 and store binary16 tiles in LDS, each tile once
//     for all 256 columns.  Their vector work then runs beside the other
//     waves' matrix-core products on the same SIMD instead of between them;
//     they run at a raised wave priority, because the matrix-core waves'
//     softmax would otherwise take the vector ALU first and stall staging.
//   * Scores are computed transposed, S^T = K~ Q^T, with
//     v_mfma_f32_32x32x16_f16: a lane then holds 16 scores of ONE query, so
//     the row max and row sum are lane-local except for one exchange with
//     the lane 32 apart.  The probabilities feed the P*V product straight
//     from registers: the V tile is stored transposed in LDS with its keys
//     permuted to match the accumulator layout of the score product.
//   * Tiles are double-buffered in LDS: while tile j is multiplied, tile
//     j+1 is fused into the other buffer and the loads of tile j+2 are
//     issued (one barrier per tile).
//   * Softmax is in the log2 domain with scale * log2 e folded into one FMA;
//     a row's reference max is raised only when a tile max exceeds it by more
//     than 8, so the accumulator is rarely rescaled, and the row sums are
//     float32 adds of the probabilities.
//   * Matrix-core operands are IEEE binary16: bf16 inputs (Q, unfused K/V)
//     convert to it exactly inside its range, and the float32 fused tiles and
//     probabilities keep 11 significant bits instead of bf16's 8.  The
//     v_mfma_f32_32x32x16_f16 rate equals the bf16 one, so this costs nothing
//     and cuts the rounding error of the fused tiles by 8x; magnitudes must
//     stay below 65504 (the fp16 range).
//   * Workgroups are mapped so that all query tiles of one (batch, KV head)
//     run on the same XCD (shared L2 for the K/V tiles), heaviest causal
//     tiles first.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fkv_internal.h"
#include "fkv_mfma_common.h"

namespace fkv {
namespace {

using namespace dev;


constexpr int kCWaves = 8;                 // matrix-core (consumer) waves
constexpr int kPWaves = 4;                 // staging (producer) waves
constexpr int kCThreads = 64 * kCWaves;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kThreads = kCThreads + kPThreads;
constexpr int BN = 64;  // keys per tile
constexpr float kLn2 = 0.69314718055994530942f;

// Operand modes of the attention kernel: one bf16 key and value source, or
// two bf16 sources fused per tile in the kernel.
constexpr int kModeSingle = 0;
constexpr int kModeFused = 1;

int rows_per_tile(int G) { return (G == 1 || G == 2 || G == 4 || G == 8) ? 256 / G : 0; }

template <int D, int MODE, int G>
__global__ __launch_bounds__(kThreads) void prefill_kernel(const PrefillArgs a)
{
    constexpr bool FUSED = MODE == kModeFused;
    constexpr int BM = 256 / G;          // query rows per workgroup
    constexpr int WPH = kCWaves / G;     // matrix-core waves per query head
    constexpr int DP = (D + 31) / 32 * 32;
    constexpr int KS = D / 16;           // k-steps of the score product
    constexpr int NDB = DP / 32;         // 32-channel blocks of the output
    constexpr int KROW = D + 8;          // LDS row pitch of K~ (elements)
    constexpr int VROW = BN + 8;         // LDS row pitch of V~^T
    constexpr int CPR = D / 8;           // 16-byte chunks per key row
    constexpr int RPP = kPThreads / CPR; // key rows per staging pass
    constexpr int KPASS = (BN + RPP - 1) / RPP;
    constexpr int NVITEM = (D / 2) * (BN / 8);  // (channel pair, key octet) items
    constexpr int VPASS = (NVITEM + kPThreads - 1) / kPThreads;

    __shared__ __attribute__((aligned(16))) uint16_t Kt[2][BN * KROW];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[2][DP * VROW];
    // At D = 128 the query fragments of the last QL k-steps of each wave
    // live in LDS (each wave reads back only its own): held in registers
    // they would push the matrix-core waves past their register budget.
    constexpr int QL = D >= 128 ? 2 : 0;
    constexpr int QR = KS - QL;
    __shared__ __attribute__((aligned(16))) uint4 Qs[QL > 0 ? kCWaves * QL * 64 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // the wave index is uniform: keep it (and all that derives from it) in
    // scalar registers so that per-wave branches are real branches
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;

    // ---- work item: XCD-aware, heaviest causal tile first ----
    const int nq = a.n_qtiles;
    const int items = a.B * a.Hkv * nq;
    int item = blockIdx.x;
    if ((items & 7) == 0) item = (blockIdx.x & 7) * (items >> 3) + (blockIdx.x >> 3);
    const int unit = item / nq;
    const int qt = a.causal ? nq - 1 - (item - unit * nq) : item - unit * nq;
    const int b = unit / a.Hkv, g = unit - (unit / a.Hkv) * a.Hkv;
    const int S = a.S;
    const int q0 = qt * BM;
    const int kend = a.causal ? min(S, q0 + BM) : S;
    const int nt = (kend + BN - 1) / BN;

    // zero the padded channel rows of V~^T (D < DP); they are never written
    if constexpr (DP > D) {
        for (int i = tid; i < (DP - D) * VROW; i += kThreads) {
            Vt[0][D * VROW + i] = 0;
            Vt[1][D * VROW + i] = 0;
        }
    }

    if (wave >= kCWaves) {
        // ================= staging waves =================
        // They load the sources of tile j+2 while the matrix-core waves work
        // on tile j, and fuse tile j+1 into the other LDS buffer: their
        // vector work runs beside the other waves' matrix-core products on
        // the same SIMDs instead of between them.
        const int pt = tid - kCThreads;
        __builtin_amdgcn_s_setprio(2);
        const int kc = pt % CPR, kr = pt / CPR;  // key chunk column / first row
        const bool k_active = kr < RPP;
        int vj[VPASS], vo[VPASS];
        bool v_active[VPASS];
#pragma unroll
        for (int v = 0; v < VPASS; ++v) {
            const int it = pt + v * kPThreads;
            v_active[v] = it < NVITEM;
            vj[v] = v_active[v] ? it % (D / 2) : 0;   // channel pair
            vo[v] = v_active[v] ? it / (D / 2) : 0;   // key octet
        }

        // float32 fusion weights of this thread's channels: a fused element
        // is w1 * x1 + wn * xn in float32 (a multiply and an FMA on the
        // widened bf16 sources), rounded once to binary16
        float wk1[8], wkn[8], wv1[VPASS][2], wvn[VPASS][2];
        if constexpr (FUSED) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                wk1[c] = k_active ? a.kw1[g * D + kc * 8 + c] : 0.0f;
                wkn[c] = k_active ? a.kwn[g * D + kc * 8 + c] : 0.0f;
            }
#pragma unroll
            for (int v = 0; v < VPASS; ++v)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    wv1[v][c] = v_active[v] ? a.vw1[g * D + 2 * vj[v] + c] : 0.0f;
                    wvn[v][c] = v_active[v] ? a.vwn[g * D + 2 * vj[v] + c] : 0.0f;
                }
        }
        // Per-tile buffer descriptors: the base advances by one tile of rows
        // per tile (scalar work) and the size shrinks with it, so the lanes
        // keep fixed offsets and rows past S-1 read as zero.
        const uint16_t* b_k1 = static_cast<const uint16_t*>(a.k1.data) + (int64_t)b * a.k1.sb + (int64_t)g * a.k1.sh;
        const uint16_t* b_v1 = static_cast<const uint16_t*>(a.v1.data) + (int64_t)b * a.v1.sb + (int64_t)g * a.v1.sh;
        const uint16_t* b_kn = b_k1;
        const uint16_t* b_vn = b_v1;
        if constexpr (FUSED) {
            b_kn = static_cast<const uint16_t*>(a.kn.data) + (int64_t)b * a.kn.sb + (int64_t)g * a.kn.sh;
            b_vn = static_cast<const uint16_t*>(a.vn.data) + (int64_t)b * a.vn.sb + (int64_t)g * a.vn.sh;
        }
        auto tile_rsrc = [&](const uint16_t* base, int64_t ss, int j) {
            const int64_t total = ((int64_t)(S - 1) * ss + D) * 2;
            const int64_t skip = (int64_t)j * BN * ss * 2;
            const int64_t left = total - skip;
            return slab_rsrc(base + (int64_t)j * BN * ss, (uint32_t)(left > 0 ? left : 0));
        };
        // byte offsets of this thread's rows inside a tile (kOffNone when idle)
        uint32_t koff1[KPASS], koffn[KPASS], voff1[VPASS][8], voffn[VPASS][8];
#pragma unroll
        for (int p = 0; p < KPASS; ++p) {
            const int row = kr + p * RPP;
            const bool ok = k_active && row < BN;
            koff1[p] = ok ? (uint32_t)(row * a.k1.ss * 2 + kc * 16) : kOffNone;
            koffn[p] = ok ? (uint32_t)(row * a.kn.ss * 2 + kc * 16) : kOffNone;
        }
#pragma unroll
        for (int v = 0; v < VPASS; ++v) {
            const int vkey0 = (vo[v] >> 1) * 16 + (vo[v] & 1) * 4;  // octet's first key
#pragma unroll
            for (int s8 = 0; s8 < 8; ++s8) {
                const int row = vkey0 + (s8 & 3) + (s8 >> 2) * 8;
                voff1[v][s8] = v_active[v] ? (uint32_t)(row * a.v1.ss * 2 + vj[v] * 4) : kOffNone;
                voffn[v][s8] = v_active[v] ? (uint32_t)(row * a.vn.ss * 2 + vj[v] * 4) : kOffNone;
            }
        }

        uint4 xk1[KPASS], xkn[KPASS];
        uint32_t xv1[VPASS][8], xvn[VPASS][8];
        auto issue_loads = [&](int j) {
            const __amdgpu_buffer_rsrc_t rk1 = tile_rsrc(b_k1, a.k1.ss, j);
            const __amdgpu_buffer_rsrc_t rv1 = tile_rsrc(b_v1, a.v1.ss, j);
            __amdgpu_buffer_rsrc_t rkn = rk1, rvn = rv1;
            if constexpr (FUSED) {
                rkn = tile_rsrc(b_kn, a.kn.ss, j);
                rvn = tile_rsrc(b_vn, a.vn.ss, j);
            }
#pragma unroll
            for (int p = 0; p < KPASS; ++p) {
                xk1[p] = ld16(rk1, koff1[p]);
                if constexpr (FUSED) xkn[p] = ld16(rkn, koffn[p]);
            }
#pragma unroll
            for (int v = 0; v < VPASS; ++v)
#pragma unroll
                for (int s8 = 0; s8 < 8; ++s8) {
                    xv1[v][s8] = ld4(rv1, voff1[v][s8]);
                    if constexpr (FUSED) xvn[v][s8] = ld4(rvn, voffn[v][s8]);
                }
        };
        // fuse the loaded registers (float32) and store fp16 tiles into buffer nb
        auto store_tile = [&](int nb) {
#pragma unroll
            for (int p = 0; p < KPASS; ++p) {
                const int row = kr + p * RPP;
                if (k_active && row < BN) {
                    uint4 o;
                    if constexpr (FUSED) {
                        const uint32_t x1[4] = {xk1[p].x, xk1[p].y, xk1[p].z, xk1[p].w};
                        const uint32_t xn[4] = {xkn[p].x, xkn[p].y, xkn[p].z, xkn[p].w};
                        uint32_t r[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            r[i] = pack2(fmaf(wk1[2 * i], bf16_lo(x1[i]), wkn[2 * i] * bf16_lo(xn[i])),
                                         fmaf(wk1[2 * i + 1], bf16_hi(x1[i]), wkn[2 * i + 1] * bf16_hi(xn[i])));
                        o = make_uint4(r[0], r[1], r[2], r[3]);
                    } else {
                        o = bf16x8_to_f16x8(xk1[p]);
                    }
                    *reinterpret_cast<uint4*>(&Kt[nb][row * KROW + kc * 8]) = o;
                }
            }
#pragma unroll
            for (int v = 0; v < VPASS; ++v) {
                if (v_active[v]) {
                    uint32_t lo[4], hv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if constexpr (FUSED) {
                            lo[i] = pack2(fmaf(wv1[v][0], bf16_lo(xv1[v][2 * i]), wvn[v][0] * bf16_lo(xvn[v][2 * i])),
                                          fmaf(wv1[v][0], bf16_lo(xv1[v][2 * i + 1]), wvn[v][0] * bf16_lo(xvn[v][2 * i + 1])));
                            hv[i] = pack2(fmaf(wv1[v][1], bf16_hi(xv1[v][2 * i]), wvn[v][1] * bf16_hi(xvn[v][2 * i])),
                                          fmaf(wv1[v][1], bf16_hi(xv1[v][2 * i + 1]), wvn[v][1] * bf16_hi(xvn[v][2 * i + 1])));
                        } else {
                            lo[i] = pack2(bf16_lo(xv1[v][2 * i]), bf16_lo(xv1[v][2 * i + 1]));
                            hv[i] = pack2(bf16_hi(xv1[v][2 * i]), bf16_hi(xv1[v][2 * i + 1]));
                        }
                    }
                    *reinterpret_cast<uint4*>(&Vt[nb][(2 * vj[v]) * VROW + vo[v] * 8]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
                    *reinterpret_cast<uint4*>(&Vt[nb][(2 * vj[v] + 1) * VROW + vo[v] * 8]) = make_uint4(hv[0], hv[1], hv[2], hv[3]);
                }
            }
        };

        issue_loads(0);
        store_tile(0);
        if (nt > 1) issue_loads(1);
        __syncthreads();
        for (int j = 0; j < nt; ++j) {
            if (j + 1 < nt) {
                store_tile((j + 1) & 1);
                if (j + 2 < nt) issue_loads(j + 2);
            }
            __syncthreads();
        }
        return;
    }

    // ================= matrix-core waves =================
    // this wave's 32 query rows of local head hh
    const int hh = wave / WPH;
    const int h = g * G + hh;
    const int r0 = q0 + (wave - hh * WPH) * 32;

    // msub: the running reference max, 0 while there is none.  With SPLAT the
    // queries are pre-multiplied by scale * log2(e) and the score chains start
    // from -msub, so the accumulators hold exponent arguments directly (the
    // splat changes only when the reference is raised).  That removes one VALU
    // instruction per score, which pays where the softmax weighs most against
    // the matrix-core work of a tile (D = 80, S = 16384: +4.5%).  At D = 128 it
    // measured 0.5-0.9% slower, so there the scores are scaled and shifted by
    // one FMA before each exponential.
    constexpr bool SPLAT = D <= 96;

    // ---- queries: B operand of S^T = K~ Q^T, 8 channels per lane per k-step
    f16x8 qreg[QR];
    {
        const int row = r0 + l32;
        const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (((int64_t)b * S + row) * a.Hq + h) * D + hi * 8;
        const float qs = a.scale_log2;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 u = make_uint4(0u, 0u, 0u, 0u);
            if (row < S) u = *reinterpret_cast<const uint4*>(qp + ks * 16);
            if constexpr (SPLAT) {
                const uint32_t w[4] = {u.x, u.y, u.z, u.w};
                uint32_t o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = pack2(bf16_lo(w[i]) * qs, bf16_hi(w[i]) * qs);
                const uint4 qv = make_uint4(o[0], o[1], o[2], o[3]);
                if (ks < QR) qreg[ks] = as_f16x8(qv);
                else Qs[(wave * QL + ks - QR) * 64 + lane] = qv;
            } else {
                const uint4 qv = bf16x8_to_f16x8(u);
                if (ks < QR) qreg[ks] = as_f16x8(qv);
                else Qs[(wave * QL + ks - QR) * 64 + lane] = qv;
            }
        }
    }

    f32x16 oacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY, l_run = 0.0f, l_run2 = 0.0f;  // two row-sum chains
    float msub = 0.0f;
    f32x16 msplat = f32x16{};
    const int qrow = r0 + l32;
    const float sl2 = a.scale_log2;

    __syncthreads();  // tile 0 staged

    for (int j = 0; j < nt; ++j) {
        const int buf = j & 1;
        const int kbase = j * BN;
        const bool wave_live = !a.causal || kbase <= r0 + 31;
        if (wave_live) {
            // lane terms of the LDS addresses, re-derived per tile from an
            // opaque copy of the lane index: held across the loop they would
            // be spilled, and their reloads would wait at every tile
            int lo_ = lane;
            asm volatile("" : "+v"(lo_));
            const int l32t = lo_ & 31, hit = lo_ >> 5;
            // S^T = K~ Q^T over two 32-key blocks; LDS fragments are read KA
            // k-steps ahead of the matrix-core instructions that use them
            constexpr int KA = D >= 128 ? 1 : 2;
            f32x16 sacc[2] = {SPLAT ? msplat : f32x16{}, SPLAT ? msplat : f32x16{}};
            const uint16_t* kt = &Kt[buf][0] + l32t * KROW + hit * 8;
            uint4 kf[KS][2];
            // the query fragments kept in LDS, read with the first key fragments
            uint4 qf[QL > 0 ? QL : 1];
#pragma unroll
            for (int i = 0; i < QL; ++i) qf[i] = Qs[(wave * QL + i) * 64 + lo_];
#pragma unroll
            for (int ks = 0; ks < KS && ks < KA; ++ks)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    kf[ks][kb] = *reinterpret_cast<const uint4*>(kt + kb * 32 * KROW + ks * 16);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + KA < KS) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
                        kf[ks + KA][kb] = *reinterpret_cast<const uint4*>(kt + kb * 32 * KROW + (ks + KA) * 16);
                }
                f16x8 qop;
                if (ks < QR) qop = qreg[ks < QR ? ks : 0];
                else qop = as_f16x8(qf[ks >= QR ? ks - QR : 0]);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(kf[ks][kb]), qop, sacc[kb], 0, 0, 0);
            }
            // V~^T fragments for the first 32-key block, read while softmax runs
            const uint16_t* vt = &Vt[buf][0] + l32t * VROW + hit * 8;
            uint4 vf[4][NDB];
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int d = 0; d < NDB; ++d)
                    vf[c][d] = *reinterpret_cast<const uint4*>(vt + d * 32 * VROW + c * 16);

            // mask: causal diagonal and keys past the end
            const bool need_mask = (a.causal && kbase + BN - 1 > r0) || kbase + BN > S;
            if (need_mask) {
                // key kbase + off is visible iff off <= lim; a lane's keys sit
                // at offsets kb*32 + (i/4)*8 + hi*4 + i%4
                const int lim = (a.causal ? min(qrow, S - 1) : S - 1) - kbase - hi * 4;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (kb * 32 + (i >> 2) * 8 + (i & 3) > lim) sacc[kb][i] = -INFINITY;
            }
            // tile max (log2 domain; relative to msub with SPLAT)
            float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                mx0 = fmaxf(mx0, sacc[0][i]);
                mx1 = fmaxf(mx1, sacc[1][i]);
            }
            const float mx = halves_max(fmaxf(mx0, mx1));
            // The reference max is raised only when a tile max exceeds it by
            // more than 8 (log2 units): the probabilities then stay <= 2^8,
            // exact in fp16, and the accumulator is rescaled on few tiles.
            const float m_tile = SPLAT ? msub + mx : mx * sl2;
            if (__any(m_tile > m_run + 8.0f)) {
                const float m_new = fmaxf(m_run, m_tile);
                const float corr = m_run == -INFINITY ? 0.0f : exp2_fast(m_run - m_new);
                l_run *= corr;
                l_run2 *= corr;
#pragma unroll
                for (int d = 0; d < NDB; ++d)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[d][i] *= corr;
                m_run = m_new;
                // re-base this tile's scores and the splat on the new reference
                const float msub_new = m_run == -INFINITY ? 0.0f : m_run;
                if constexpr (SPLAT) {
                    const float sh = msub_new - msub;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int i = 0; i < 16; ++i) sacc[kb][i] -= sh;
#pragma unroll
                    for (int i = 0; i < 16; ++i) msplat[i] = -msub_new;
                }
                msub = msub_new;
            }
            const float psub = SPLAT ? 0.0f : (m_run == -INFINITY ? 0.0f : m_run);
            const float pmul = SPLAT ? 1.0f : sl2;
            // per 32-key block: probabilities -> fp16 B operands, then
            // O^T += V~^T P^T; the second block's exponentials overlap the
            // first block's matrix-core work
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f16x8 pb[2];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    uint32_t w[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float p0 = exp2_fast(sacc[kb][half * 8 + 2 * i] * pmul - psub);
                        const float p1 = exp2_fast(sacc[kb][half * 8 + 2 * i + 1] * pmul - psub);
                        w[i] = pack2(p0, p1);
                        // float32 row sums in two chains: plain adds co-issue
                        // with the matrix-core products of the other block,
                        // while dot-product instructions wait for the matrix
                        // core on this part
                        l_run += p0;
                        l_run2 += p1;
                    }
                    pb[half] = as_f16x8(make_uint4(w[0], w[1], w[2], w[3]));
                }
#pragma unroll
                for (int half = 0; half < 2; ++half)
#pragma unroll
                    for (int d = 0; d < NDB; ++d)
                        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(vf[kb * 2 + half][d]), pb[half],
                                                                         oacc[d], 0, 0, 0);
                // the second block's fragments, read while its exponentials run
                if (kb == 0) {
#pragma unroll
                    for (int c = 2; c < 4; ++c)
#pragma unroll
                        for (int d = 0; d < NDB; ++d)
                            vf[c][d] = *reinterpret_cast<const uint4*>(vt + d * 32 * VROW + c * 16);
                }
            }
        }
        __syncthreads();
    }

    // ---- epilogue: O = acc / l, LSE = ln 2 * (m + log2 l) ----
    const float l_tot = halves_sum(l_run + l_run2);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (qrow < S) {
        uint16_t* op = static_cast<uint16_t*>(a.out) + (((int64_t)b * S + qrow) * a.Hq + h) * D;
#pragma unroll
        for (int d = 0; d < NDB; ++d) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ch = d * 32 + r * 8 + hi * 4;
                if (ch < D) {
                    const uint32_t w0 = pack2_bf16(oacc[d][r * 4 + 0] * inv, oacc[d][r * 4 + 1] * inv);
                    const uint32_t w1 = pack2_bf16(oacc[d][r * 4 + 2] * inv, oacc[d][r * 4 + 3] * inv);
                    *reinterpret_cast<uint2*>(op + ch) = make_uint2(w0, w1);
                }
            }
        }
        if (hi == 0 && a.lse)
            a.lse[((int64_t)b * a.Hq + h) * S + qrow] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

template <int D, int MODE>
int launch_g(const PrefillArgs& a, hipStream_t st)
{
    const dim3 grid((unsigned)a.B * a.Hkv * a.n_qtiles);
    switch (a.G) {
    case 1: hipLaunchKernelGGL((prefill_kernel<D, MODE, 1>), grid, dim3(kThreads), 0, st, a); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<D, MODE, 2>), grid, dim3(kThreads), 0, st, a); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<D, MODE, 4>), grid, dim3(kThreads), 0, st, a); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<D, MODE, 8>), grid, dim3(kThreads), 0, st, a); break;
    default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

template <int D>
int launch_mode(const PrefillArgs& a, bool fused, hipStream_t st)
{
    return fused ? launch_g<D, kModeFused>(a, st) : launch_g<D, kModeSingle>(a, st);
}

}  // namespace

int prefill_rows_per_tile(int G) { return rows_per_tile(G); }

int launch_prefill(const PrefillArgs& a, bool fused, void* stream)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (a.B == 0 || a.S == 0) return 0;
    if ((int64_t)a.B * a.Hkv * a.n_qtiles > 0x7fffffff) return (int)hipErrorInvalidValue;
    switch (a.D) {
    case 64: return launch_mode<64>(a, fused, st);
    case 80: return launch_mode<80>(a, fused, st);
    case 96: return launch_mode<96>(a, fused, st);
    case 128: return launch_mode<128>(a, fused, st);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace fkv
