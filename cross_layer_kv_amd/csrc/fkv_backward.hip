// fkv_backward.hip -- backward pass of FusedKV reconstruction-layer attention
// (causal or full, S_q == S_k) on gfx950 matrix cores, bf16 operands with
// float32 accumulation.
//
// Pages cited (by title):
//   [Deck]  "FusedKV: Reconstructing KV Caches with Cross-Layer Fusion",
//           frame "FusedKV learns two-source, channel-wise fusion"
//           (Eqs. (4)-(5)): the per-channel vectors are learned with the
//           model, trained end to end, so a training step differentiates the
//           fused attention with respect to the queries, the four source
//           caches and the four vectors.  Frame "Lite separates the key
//           source from the value source" (Eq. (6)) for one key and one value
//           source.
//   [Notes] "FusedKV:通过跨层融合重构 KV 缓存", sections 2.1-2.3.
//
// For a loss with output gradient dO (the chain rule through the fusion and
// the softmax; Kf = a K1 + a' Kn, Vf = b V1 + b' Vn per channel):
//   P = softmax(scale Q Kf^T) (recomputed from the forward LSE)
//   dVf = sum_h P^T dO,  dP = dO Vf^T,  dS = P (dP - rowsum(dO O))
//   dQ = scale dS Kf,  dKf = scale sum_h dS^T Q
//   dK1 = a dKf, dKn = a' dKf, dV1 = b dVf, dVn = b' dVf
//   da = sum_{b,t} dKf K1 (likewise a', b, b'): column sums over tokens.
// The fused tiles are rebuilt in registers / LDS and never stored in HBM,
// like the forward pass ([Notes] section 2.3: fusion on demand).
//
// Kernels
//   1. prep: per (batch, head, row) the LSE in log2 units and
//      rowsum(dO * O) (float32).
//   2. key tiles: a workgroup of 8 waves owns 128 keys of one (batch, KV
//      head): four waves accumulate dVf and four dKf of one 32-key block
//      each, keeping the block's fused keys (and values) as matrix-core
//      operands in registers, and walk the query rows of all G heads of the
//      group in 64-row LDS tiles; the value waves hand P (fp16) to the key
//      waves through LDS, so the scores are formed once.  At 128 channels
//      the Q / dO tiles are copied from memory straight into LDS (buffer
//      loads with an LDS destination), elsewhere through registers.  It
//      writes the four source gradients and its partial column sums for
//      the weight gradients.
//   3. query tiles: a workgroup of 8 waves owns 256 (query row, head)
//      columns and walks 64-key tiles staged in LDS, accumulating dQ; four
//      sources are fused as each tile is staged.  dQ is thus written once,
//      with no float atomics, and every result is run-to-run deterministic.
//   4. reduce: the weight-gradient partials summed in a fixed order.
//
// Operand layouts (v_mfma_f32_32x32x16_bf16, A 32x16, B 16x32, C 32x32): a
// lane (l32 = lane % 32, hi = lane / 32) holds row l32 of A / column l32 of B
// with K elements 8*hi .. 8*hi+7, and C entries (rows 8j + 4hi + i, column
// l32) for j, i in 0..3.  A C tile therefore serves directly as the A (or B)
// operand of the next product when that product's K index is the C row
// index, taken in the order 16c + 4hi + (e%4) + 8(e/4) for element e of
// k-step c.  The other operand of such a product reads its K rows in that
// order from a row-major LDS tile with two transposing reads
// (ds_read_b64_tr_b16), which is how Q and dO serve both as row operands
// (for the scores and dP) and as transposed operands (for dK and dV).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "fkv_internal.h"
#include "fkv_mfma_common.h"

namespace fkv {
namespace {

using namespace dev;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kKeysPerWg = kBwdKeyTile;  // key-tile kernel: 4 blocks of 32 keys
constexpr int kQRows = 64;        // key-tile kernel: query rows per LDS tile
constexpr int kKTile = 64;        // query-tile kernel: keys per LDS tile
constexpr int kDqWaves = 8;       // query-tile kernel: 8 x 32 (query row, head) columns
constexpr int kDkvThreads = 512;  // key-tile kernel: 4 value waves + 4 key waves
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kPrepRows = 4;      // prep kernel: rows per lane group

// Slot of the (batch, KV head, key tile) weight-gradient partial.
__device__ __forceinline__ int64_t item_index(int b, int g, int kt, int Hkv, int nkt)
{
    return ((int64_t)b * Hkv + g) * nkt + kt;
}

__device__ __forceinline__ f32x16 mma(uint4 a, uint4 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// Row operand: row r0 + l32 of a row-major LDS tile, channels 16 ks + 8 hi.
__device__ __forceinline__ uint4 row_frag(const uint16_t* tile, int pitch, int r0, int ks, int l32, int hi)
{
    return *reinterpret_cast<const uint4*>(tile + (r0 + l32) * pitch + ks * 16 + hi * 8);
}

// Transposed operand: column col0 + l32 of a row-major LDS tile, K rows
// krow0 + 4 hi + (e % 4) + 8 (e / 4) for elements e = 0..7.  Within each
// 16-lane group a source lane supplies 4 channels of one row and receives
// one channel of 4 rows.
__device__ __forceinline__ uint4 tr_frag(const uint16_t* tile, int pitch, int krow0, int col0, int l32, int hi)
{
    const uint16_t* p = tile + (krow0 + hi * 4 + ((l32 & 15) >> 2)) * pitch + col0 + (l32 >> 4) * 16 + (l32 & 3) * 4;
    const v4s x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
    const v4s x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p + 8 * pitch));
    return __builtin_bit_cast(uint4, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// s_waitcnt operand: vector memory count 0, the other counters at their
// maximum (no wait).
constexpr int kWaitLoads = 0x0F70;

// Unpadded 128-channel tiles (256-byte rows), filled by direct-to-LDS loads
// that write 1 KB contiguous per instruction: logical 16-byte chunk c of row
// r sits at chunk c ^ swz(r).  swz permutes the low four row bits, so 16
// consecutive rows put one chunk in 16 different chunk slots (row reads),
// and rows 4k .. 4k+3 put a chunk pair in 8 different slots (transposing
// reads).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8); }

__device__ __forceinline__ uint4 row_frag_sw(const uint16_t* tile, int r0, int ks, int l32, int hi)
{
    const int r = r0 + l32;
    return *reinterpret_cast<const uint4*>(tile + r * 128 + (((2 * ks + hi) ^ swz(r)) << 3));
}

__device__ __forceinline__ uint4 tr_frag_sw(const uint16_t* tile, int krow0, int col0, int l32, int hi)
{
    const int r = krow0 + hi * 4 + ((l32 & 15) >> 2);
    const int e = col0 + (l32 >> 4) * 16 + (l32 & 3) * 4;
    const uint16_t* p0 = tile + r * 128 + (((e >> 3) ^ swz(r)) << 3) + (e & 7);
    const uint16_t* p1 = tile + (r + 8) * 128 + (((e >> 3) ^ swz(r + 8)) << 3) + (e & 7);
    const v4s x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p0);
    const v4s x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p1);
    return __builtin_bit_cast(uint4, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// 8 channels (16 bytes) of bf16 -> fused (w1 x1 + wn xn) bf16, float32 math.
__device__ __forceinline__ uint4 fuse8_bf16(uint4 x1, uint4 xn, const float* w1, const float* wn)
{
    const uint32_t a[4] = {x1.x, x1.y, x1.z, x1.w};
    const uint32_t b[4] = {xn.x, xn.y, xn.z, xn.w};
    uint32_t r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = w1[2 * i] * bf16_lo(a[i]) + wn[2 * i] * bf16_lo(b[i]);
        const float hi = w1[2 * i + 1] * bf16_hi(a[i]) + wn[2 * i + 1] * bf16_hi(b[i]);
        r[i] = pack2_bf16(lo, hi);
    }
    return make_uint4(r[0], r[1], r[2], r[3]);
}

__device__ __forceinline__ const uint16_t* row_ptr(const View& v, int b, int t, int h)
{
    return static_cast<const uint16_t*>(v.data) + (int64_t)b * v.sb + (int64_t)t * v.ss + (int64_t)h * v.sh;
}

__device__ __forceinline__ uint16_t* out_row(const OutView& v, int b, int t, int h)
{
    return static_cast<uint16_t*>(v.data) + (int64_t)b * v.sb + (int64_t)t * v.ss + (int64_t)h * v.sh;
}

__device__ __forceinline__ void load8f(const float* p, float* w)
{
    const float4 x = *reinterpret_cast<const float4*>(p);
    const float4 y = *reinterpret_cast<const float4*>(p + 4);
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
    w[4] = y.x; w[5] = y.y; w[6] = y.z; w[7] = y.w;
}

// ---- 1. prep: LSE in log2 units and rowsum(dO * O), [B, Hq, S] ----
// A group of LPR lanes (D/8 of them active) takes one (b, t, h) row, 16 bytes
// of O and dO per lane, so each load instruction reads whole rows; the
// group's partial sums are added over the lanes in a fixed order.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const BwdArgs a)
{
    constexpr int LPR = D / 8 <= 8 ? 8 : 16;  // lanes per row
    const int64_t n = (int64_t)a.B * a.S * a.Hq;
    // a lane group takes kPrepRows consecutive rows, all loads issued first
    const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR * kPrepRows;
    const int pc = threadIdx.x % LPR;
    uint4 x[kPrepRows], y[kPrepRows];
#pragma unroll
    for (int k = 0; k < kPrepRows; ++k) {
        const int64_t i = i0 + k;
        x[k] = y[k] = make_uint4(0u, 0u, 0u, 0u);
        if (i < n && pc < D / 8) {
            x[k] = stream16(static_cast<const uint16_t*>(a.out) + i * D + pc * 8);
            y[k] = stream16(static_cast<const uint16_t*>(a.dout) + i * D + pc * 8);
        }
    }
#pragma unroll
    for (int k = 0; k < kPrepRows; ++k) {
        const int64_t i = i0 + k;
        const uint32_t xs[4] = {x[k].x, x[k].y, x[k].z, x[k].w}, ys[4] = {y[k].x, y[k].y, y[k].z, y[k].w};
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) s += bf16_lo(xs[e]) * bf16_lo(ys[e]) + bf16_hi(xs[e]) * bf16_hi(ys[e]);
#pragma unroll
        for (int o = 1; o < LPR; o <<= 1) s += __shfl_xor(s, o);
        if (i < n && pc == 0) {
            const int h = (int)(i % a.Hq);
            const int64_t bs = i / a.Hq;
            const int t = (int)(bs % a.S), b = (int)(bs / a.S);
            const int64_t r = ((int64_t)b * a.Hq + h) * a.S + t;
            a.delta[r] = s;
            a.lse2[r] = a.lse[r] * kLog2e;
        }
    }
}

// ---- 2. key tiles: dKf, dVf, source gradients, weight partials ----
// Eight waves over 128 keys: wave w < 4 takes key block w for the values
// (scores, P, dVf += P^T dO), wave w >= 4 key block w - 4 for the keys
// (dP, dS = P (dP - delta), dKf += dS^T Q) one tile later, with the value
// wave's P.  Each wave holds one accumulator and the operands it needs,
// which fits two waves per SIMD (waves w and w + 4 share one); both have
// two products per tile, and the value waves also stage the Q / dO tiles.
template <int D, bool FUSED, int G>
__global__ __launch_bounds__(kDkvThreads, 2) void bwd_dkdv_kernel(const BwdArgs a)
{
    constexpr int DP = (D + 31) / 32 * 32;  // channels padded to whole 32-column blocks
    constexpr int NDB = DP / 32;
    constexpr int KS = D / 16;
    // LDS row pitch (elements).  The Q / dO tiles are read both by rows
    // (16 bytes per lane) and by the transposing reads (8 bytes per lane, 4
    // rows per 16-lane group); at 128 channels a 152-element pitch keeps the
    // row reads conflict-free and halves the transposing reads' bank
    // conflicts against DP + 8 (17% faster in an in-bounds probe).
    // At 128 channels the Q / dO tiles arrive by direct-to-LDS loads into
    // unpadded, swizzled 256-byte rows.
    constexpr bool kDma = D == 128;
    constexpr int P = kDma ? 128 : (DP == 128 ? DP + 24 : DP + 8);
    constexpr int CPR = D / 8;              // 16-byte chunks per row
    constexpr int TILE = kQRows * P;
    constexpr int SP = DP + 4;              // pitch of the float32 transpose buffer
    constexpr int NBUF = 3;                 // Q / dO tile buffers in LDS
    static_assert(NBUF * 2 * TILE * 2 >= kKeysPerWg * SP * 4, "transpose buffer fits in the tile buffers");

    __shared__ __attribute__((aligned(16))) uint16_t smem[NBUF * 2 * TILE];  // [buf][Q, dO][row][P]
    // the P hand-off in the loop ([tile parity][key block][sub-block][chunk]
    // [lane], 16 bytes each), then the weight-gradient partials in the
    // epilogue ([key group][source][channel] floats)
    constexpr int kXpBytes = 2 * 4 * 2 * 2 * 64 * 16;
    constexpr int kRedBytes = (kKeysPerWg / 4) * 2 * D * 4;
    __shared__ __attribute__((aligned(16))) uint4 xsm[(kXpBytes > kRedBytes ? kXpBytes : kRedBytes) / 16];
    __shared__ __attribute__((aligned(16))) float Ls[NBUF][kQRows];
    __shared__ __attribute__((aligned(16))) float Dl[NBUF][kQRows];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    const bool kwave = wave >= 4;  // keys (dK) or values (dV)
    const int kb = wave & 3;

    const int nkt = a.nkt;
    const int items = a.B * a.Hkv * nkt;
    int item = blockIdx.x;
    if ((items & 7) == 0) item = (blockIdx.x & 7) * (items >> 3) + (blockIdx.x >> 3);
    const int unit = item / nkt;
    const int kt = item - unit * nkt;  // low key tiles see the most query rows: they start first
    const int b = unit / a.Hkv, g = unit - (unit / a.Hkv) * a.Hkv;
    const int S = a.S;
    const int k0 = kt * kKeysPerWg;
    const int kw = k0 + kb * 32;

    // zero the padded channels [D, DP) of every tile row (never loaded)
    if constexpr (DP > D) {
        for (int i = tid; i < NBUF * 2 * kQRows * (DP - D); i += kDkvThreads) {
            const int r = i / (DP - D), c = i - r * (DP - D);
            smem[r * P + D + c] = 0;
        }
    }

    // ---- this block's 32 fused keys (and, key waves, values) as MFMA
    // operands in registers (lane: key l32) ----
    uint4 kreg[KS], vreg[KS];  // vreg: key waves' fused values (B operands of dP)
    {
        // Four sources are fused here, one 8-channel chunk at a time, in
        // float32 and rounded to bf16: the fused rows exist only in
        // registers.  The scheduling fence after each chunk keeps the
        // compiler from hoisting every chunk's loads and weights at once.
        const int key = kw + l32;
        const bool ok = key < S;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int ch = ks * 16 + hi * 8;
            uint4 k = make_uint4(0u, 0u, 0u, 0u), v = k;
            if (ok) {
                k = *reinterpret_cast<const uint4*>(row_ptr(a.k1, b, key, g) + ch);
                if (kwave) v = *reinterpret_cast<const uint4*>(row_ptr(a.v1, b, key, g) + ch);
                if constexpr (FUSED) {
                    float w1[8], wn[8];
                    load8f(a.kw1 + g * D + ch, w1);
                    load8f(a.kwn + g * D + ch, wn);
                    k = fuse8_bf16(k, *reinterpret_cast<const uint4*>(row_ptr(a.kn, b, key, g) + ch), w1, wn);
                    if (kwave) {
                        load8f(a.vw1 + g * D + ch, w1);
                        load8f(a.vwn + g * D + ch, wn);
                        v = fuse8_bf16(v, *reinterpret_cast<const uint4*>(row_ptr(a.vn, b, key, g) + ch), w1, wn);
                    }
                }
            }
            kreg[ks] = k;
            vreg[ks] = v;
            if constexpr (FUSED) __builtin_amdgcn_sched_barrier(0);
        }
    }

    f32x16 acc[NDB];  // dKf (key waves) or dVf (value waves)
#pragma unroll
    for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};

    // query tiles: rows qb .. qb+63 of head g*G + hh; causal rows below k0
    // see none of these keys
    const int q_begin = a.causal ? (k0 / kQRows) * kQRows : 0;
    const int nqb = S > q_begin ? (S - q_begin + kQRows - 1) / kQRows : 0;
    const int nit = nqb * G;

    // register staging (below 128 channels): thread -> (row, 16-byte chunk)
    // items of Q and dO, staged by the value waves (the key waves, a tile
    // behind, measured slower with a share of the staging).
    constexpr int kStageThreads = kDkvThreads / 2;
    constexpr int NITEM = kQRows * CPR;
    constexpr int NPASS = (NITEM + kStageThreads - 1) / kStageThreads;
    uint4 xq[NPASS], xo[NPASS];
    float xl = 0.0f, xd = 0.0f;
    // Q and dO rows of one tile through buffer descriptors whose base is the
    // tile's first row (scalar work) and whose size ends at its last row
    // inside S: rows past S-1 read as zero, and the lanes keep 32-bit
    // offsets instead of 64-bit address arithmetic per load.
    auto load_tile = [&](int it, int tid) {
        const int qb = q_begin + (it / G) * kQRows;
        const int h = g * G + it % G;
        const int64_t base = (((int64_t)b * S + qb) * a.Hq + h) * D;
        const int rows = min(S - qb, kQRows);
        const uint32_t rstride = (uint32_t)a.Hq * D * 2;  // bytes between rows
        const uint32_t bytes = (uint32_t)(rows - 1) * rstride + D * 2;
        const __amdgpu_buffer_rsrc_t rq = slab_rsrc(static_cast<const uint16_t*>(a.q) + base, bytes);
        const __amdgpu_buffer_rsrc_t ro = slab_rsrc(static_cast<const uint16_t*>(a.dout) + base, bytes);
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int e = tid + p * kStageThreads;
            const int r = e / CPR, c = e - (e / CPR) * CPR;
            const uint32_t off = e < NITEM ? (uint32_t)r * rstride + c * 16 : kOffNone;
            xq[p] = ld16(rq, off);
            xo[p] = ld16(ro, off);
        }
        if (tid < kQRows) {
            const int row = qb + tid;
            const int64_t r = ((int64_t)b * a.Hq + h) * S + row;
            xl = row < S ? a.lse2[r] : 0.0f;
            xd = row < S ? a.delta[r] : 0.0f;
        }
    };
    auto store_tile = [&](int buf, int tid) {
        uint16_t* qs = smem + (buf * 2 + 0) * TILE;
        uint16_t* os = smem + (buf * 2 + 1) * TILE;
        // tid < kStageThreads: passes below NITEM / kStageThreads are whole
        // and are stored without a branch, at fixed offsets from one address
        // when CPR divides kStageThreads
        constexpr bool kEven = kStageThreads % CPR == 0;
        const int r0 = tid / CPR, c0 = tid - (tid / CPR) * CPR;
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int e = tid + p * kStageThreads;
            const int r = kEven ? r0 + p * (kStageThreads / CPR) : e / CPR;
            const int c = kEven ? c0 : e - (e / CPR) * CPR;
            if ((p + 1) * kStageThreads <= NITEM || e < NITEM) {
                *reinterpret_cast<uint4*>(qs + r * P + c * 8) = xq[p];
                *reinterpret_cast<uint4*>(os + r * P + c * 8) = xo[p];
            }
        }
        if (tid < kQRows) {
            Ls[buf][tid] = xl;
            Dl[buf][tid] = xd;
        }
    };

    // 128 channels: each value wave copies 16 of the tile's rows of Q and dO
    // straight from memory into LDS, four 1 KB load instructions per tensor
    // (lane l: 16 bytes of row 4j + l/16, placed as the swizzle puts them),
    // and value waves 0 and 1 copy the rows' LSE and delta (4 bytes a lane).
    // Rows past S read as zero.  A wave waits for its copies before the next
    // barrier.
    auto dma_tile = [&](int t, int bufi, int tid_) {
        typedef __attribute__((address_space(3))) void lds_void;
        const int qb = q_begin + (t / G) * kQRows;
        const int h = g * G + t % G;
        const int64_t base = (((int64_t)b * S + qb) * a.Hq + h) * D;
        const int rows = min(S - qb, kQRows);
        const uint32_t rstride = (uint32_t)a.Hq * D * 2;
        const uint32_t bytes = (uint32_t)(rows - 1) * rstride + D * 2;
        const __amdgpu_buffer_rsrc_t rq = slab_rsrc(static_cast<const uint16_t*>(a.q) + base, bytes);
        const __amdgpu_buffer_rsrc_t ro = slab_rsrc(static_cast<const uint16_t*>(a.dout) + base, bytes);
        // vw (LDS addresses) keeps the thread index's known range, so the
        // copies' LDS ranges stay visible to the alias analysis; vwu (the
        // same value) drives the branches and descriptors
        const int vw = tid_ >> 6, lane_ = tid_ & 63;
        const int vwu = __builtin_amdgcn_readfirstlane(tid_ >> 6);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = vw * 4 + i;
            const int r = 4 * j + (lane_ >> 4);
            const uint32_t off = (uint32_t)r * rstride + (uint32_t)(((lane_ & 15) ^ swz(r)) << 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void*)(smem + (bufi * 2 + 0) * TILE + j * 512), 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ro, (lds_void*)(smem + (bufi * 2 + 1) * TILE + j * 512), 16, off, 0, 0, 0);
        }
        const int64_t rb = ((int64_t)b * a.Hq + h) * S + qb;
        if (vwu == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(slab_rsrc(a.lse2 + rb, (uint32_t)rows * 4), (lds_void*)&Ls[bufi][0],
                                                     4, (uint32_t)lane_ * 4, 0, 0, 0);
        else if (vwu == 1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(slab_rsrc(a.delta + rb, (uint32_t)rows * 4), (lds_void*)&Dl[bufi][0],
                                                     4, (uint32_t)lane_ * 4, 0, 0, 0);
    };

    const float sl2 = a.scale_log2;
    // Register staging: tiles are loaded two iterations ahead of use and
    // stored to LDS one iteration ahead, right after the barrier, so a
    // tile's loads have a whole iteration to arrive before the store waits
    // on them.  Direct copies: tile it+1 is copied during iteration it.
    if (nit > 0 && !kwave) {
        if constexpr (kDma) {
            dma_tile(0, 0, tid);
        } else {
            load_tile(0, tid);
            store_tile(0, tid);
            if (nit > 1) load_tile(1, tid);
        }
    }
    // P hand-off from the value waves to the key waves in the shared array:
    // [tile parity][key block][sub-block][16-byte chunk][lane], fp16 (P <= 1)
    auto xp_chunk = [&](int par, int sb, int c, int lane_) { return xsm + (((par * 4 + kb) * 2 + sb) * 2 + c) * 64 + lane_; };
    // The query-tile loop, instantiated once per wave role (KW: key wave)
    // with one straight-line tile body: the accumulators then stay in one
    // register set across the loop (branches merging inside the body made
    // the compiler keep a second copy and move it every tile), and the
    // registers left over hold LDS fragments read ahead of the matrix-core
    // instructions that use them.  The value waves form the scores and P of
    // tile it and hand P to the key waves, which take tile it one iteration
    // later (dP, dS = P (dP - delta), dK): the per-tile barrier orders the
    // hand-off, and no score product is formed twice.
    auto run = [&](auto role) {
        constexpr bool KW = decltype(role)::value;
        constexpr int PF = 2;  // k-steps of fragments in flight
        // one query tile (the value waves' tile it, the key waves' tile it-1);
        // MASKED (value waves): some (row, key) pair of the tile is invisible
        // (causal diagonal, rows or keys past S)
        auto tile = [&](int it, auto masked_c, auto buf_c) {
            constexpr bool MASKED = decltype(masked_c)::value;
            // BC: the tile's LDS buffer when known at compile time (value
            // waves at 128 channels), else -1
            constexpr int BC = decltype(buf_c)::value;
            // Lane indices re-derived per tile from an opaque copy of the
            // thread index: the loop's address terms are then recomputed (a
            // few VALU instructions) instead of held in registers across the
            // loop.
            int tid_o = tid;
            asm volatile("" : "+v"(tid_o));
            const int l32 = tid_o & 31, hi = (tid_o >> 5) & 1, lane_o = tid_o & 63;
            // the direct-to-LDS copies of this wave complete before the
            // barrier (the barrier alone does not wait for them)
            if constexpr (!KW && kDma) __builtin_amdgcn_s_waitcnt(kWaitLoads);
            __syncthreads();  // tile `it` stored, P of tile it-1 handed over; older readers done
            if (!KW && !kDma && it + 1 < nit) {
                store_tile((it + 1) % NBUF, tid_o);  // tile it+1, loaded an iteration ago
                if (it + 2 < nit) load_tile(it + 2, tid_o);
            }
            if (KW && it == 0) return;  // the key waves' tile -1: the barrier only
            const int t = KW ? it - 1 : it;  // the tile this wave works on
            const int buf = BC >= 0 ? BC : t % NBUF, par = t & 1;
            // With the buffer known, the copies of tile it+1 go out first:
            // the compiler sees this tile's row reads and the P stores as
            // disjoint from them and issues them without waiting; the
            // transposing reads (intrinsics with no alias information) wait
            // for the copies, after both score chains.
            if constexpr (!KW && kDma && BC >= 0)
                if (it + 1 < nit) dma_tile(it + 1, (BC + 1) % NBUF, tid);
            const int qb = q_begin + (t / G) * kQRows;
            const uint16_t* qs = smem + (buf * 2 + 0) * TILE;
            const uint16_t* os = smem + (buf * 2 + 1) * TILE;
            const int key = kw + l32;
            // Ls (value waves) or Dl (key waves) of the rows of entries
            // 4j .. 4j+3 of sub-block sb
            auto ld_rows = [&](int sb, int j, float4& R4) {
                R4 = *reinterpret_cast<const float4*>(KW ? &Dl[buf][sb * 32 + 8 * j + 4 * hi]
                                                         : &Ls[buf][sb * 32 + 8 * j + 4 * hi]);
            };
            // entry e of sub-block sb: P (value waves, from the score) or dS
            // (key waves, from the handed-over P and dP); lane: key kw + l32,
            // entry e: query row qb + 32 sb + 8(e/4) + 4hi + e%4
            auto entry = [&](int e, const float4& R4, const f32x16& acc_s, const uint4* ph) {
                const float Rv[4] = {R4.x, R4.y, R4.z, R4.w};
                if constexpr (KW) {
                    const uint32_t w[8] = {ph[0].x, ph[0].y, ph[0].z, ph[0].w, ph[1].x, ph[1].y, ph[1].z, ph[1].w};
                    const float p = (float)__builtin_bit_cast(f16x2, w[e >> 1])[e & 1];
                    return p * (acc_s[e] - Rv[e & 3]);
                } else {
                    return exp2_fast(acc_s[e] * sl2 - Rv[e & 3]);
                }
            };
            // invisible pairs select zero (their exponentials may be infinite)
            auto mask = [&](int sb, float* xv) {
                if constexpr (!KW && MASKED) {
                    const int qs0 = qb + sb * 32;
                    const bool key_ok = key < S;
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int q = qs0 + 8 * (e >> 2) + 4 * hi + (e & 3);
                        const bool vis = key_ok & (q < S) & (!a.causal | (key <= q));
                        xv[e] = vis ? xv[e] : 0.0f;
                    }
                }
            };
            // bf16 A operands of the product; the value waves also hand P
            // over as fp16
            auto pack = [&](int sb, const float* xv, uint4* xa) {
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    xa[c] = make_uint4(pack2_bf16(xv[8 * c + 0], xv[8 * c + 1]), pack2_bf16(xv[8 * c + 2], xv[8 * c + 3]),
                                       pack2_bf16(xv[8 * c + 4], xv[8 * c + 5]), pack2_bf16(xv[8 * c + 6], xv[8 * c + 7]));
                if constexpr (!KW) {
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        uint32_t w0 = pack2(xv[8 * c + 0], xv[8 * c + 1]), w1 = pack2(xv[8 * c + 2], xv[8 * c + 3]);
                        uint32_t w2 = pack2(xv[8 * c + 4], xv[8 * c + 5]), w3 = pack2(xv[8 * c + 6], xv[8 * c + 7]);
                        // one vector store: split stores lose the array's
                        // alias information, and each then waits for the
                        // direct-to-LDS copies in flight
                        typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
                        *reinterpret_cast<u32x4v*>(xp_chunk(par, sb, c, lane_o)) = u32x4v{w0, w1, w2, w3};
                    }
                }
            };
            const uint16_t* other = KW ? qs : os;  // dK += dS^T Q, dV += P^T dO
            auto rfrag = [&](const uint16_t* t_, int r0, int ks) {
                if constexpr (kDma) return row_frag_sw(t_, r0, ks, l32, hi);
                else return row_frag(t_, P, r0, ks, l32, hi);
            };
            auto tfrag = [&](const uint16_t* t_, int krow0, int col0) {
                if constexpr (kDma) return tr_frag_sw(t_, krow0, col0, l32, hi);
                else return tr_frag(t_, P, krow0, col0, l32, hi);
            };
            // The score chain S^T = Q K~^T (value waves) or dP^T = dO V~^T
            // (key waves) of sub-block sb (32 keys x 32 rows), with the 16
            // entries of the previous sub-block psb computed a few at a time
            // between the matrix-core steps (ps: its chain accumulator, or
            // null for the first sub-block).  A scheduling fence after each
            // step keeps the vector work beside the matrix-core instructions
            // it overlaps.
            auto chain = [&](int sb, f32x16& cacc, int psb, const f32x16* ps, float* xv) {
                const uint16_t* src = KW ? os : qs;
                uint4 fr[PF + 1], ph[2];
                float4 R4[4];
#pragma unroll
                for (int ks = 0; ks < PF; ++ks) fr[ks] = rfrag(src, sb * 32, ks);
                if (ps) {
                    ld_rows(psb, 0, R4[0]);
                    if constexpr (KW) {
                        ph[0] = *xp_chunk(par, psb, 0, lane_o);
                        ph[1] = *xp_chunk(par, psb, 1, lane_o);
                    }
                }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if (ks + PF < KS) fr[(ks + PF) % (PF + 1)] = rfrag(src, sb * 32, ks + PF);
                    // the chain starts from a zero operand, not zeroed registers
                    cacc = mma(fr[ks % (PF + 1)], KW ? vreg[ks] : kreg[ks], ks == 0 ? f32x16{} : cacc);
                    if (ps) {
                        const int e0 = ks * 16 / KS, e1 = (ks + 1) * 16 / KS;
                        // the next step's row values, one step ahead
                        const int j1 = e1 < 16 ? e1 >> 2 : 3;
                        if (e1 < 16 && (e0 >> 2) != j1) ld_rows(psb, j1, R4[j1]);
#pragma unroll
                        for (int e = e0; e < e1; ++e) xv[e] = entry(e, R4[e >> 2], *ps, ph);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            // dK / dV += (dS or P)^T (Q or dO) over the 32 rows of sub-block
            // sb, with the entries of sub-block nsb computed between the
            // matrix-core steps (ns: its chain accumulator, or null)
            auto product = [&](int sb, const uint4* xa, int nsb, const f32x16* ns, float* xv) {
                constexpr int NM = 2 * NDB;
                uint4 tf[3], ph[2];
                float4 R4[4];
                tf[0] = tfrag(other, sb * 32, 0);
                if (NM > 1) tf[1] = tfrag(other, sb * 32 + (NDB > 1 ? 0 : 16), (NDB > 1 ? 32 : 0));
                if (ns) {
                    ld_rows(nsb, 0, R4[0]);
                    if constexpr (KW) {
                        ph[0] = *xp_chunk(par, nsb, 0, lane_o);
                        ph[1] = *xp_chunk(par, nsb, 1, lane_o);
                    }
                }
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    if (m + 2 < NM) {
                        const int m2 = m + 2;
                        tf[m2 % 3] = tfrag(other, sb * 32 + 16 * (m2 / NDB), (m2 % NDB) * 32);
                    }
                    acc[m % NDB] = mma(xa[m / NDB], tf[m % 3], acc[m % NDB]);
                    if (ns) {
                        const int e0 = m * 16 / NM, e1 = (m + 1) * 16 / NM;
                        const int j1 = e1 < 16 ? e1 >> 2 : 3;
                        if (e1 < 16 && (e0 >> 2) != j1) ld_rows(nsb, j1, R4[j1]);
#pragma unroll
                        for (int e = e0; e < e1; ++e) xv[e] = entry(e, R4[e >> 2], *ns, ph);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            // Two sub-blocks in a software pipeline: sub-block 1's chain runs
            // beside sub-block 0's entries, and sub-block 0's product beside
            // sub-block 1's.
            f32x16 c0, c1;
            float xv[16];
            uint4 xa[2];
            chain(0, c0, 0, nullptr, xv);
            chain(1, c1, 0, &c0, xv);
            mask(0, xv);
            pack(0, xv, xa);
            __builtin_amdgcn_sched_barrier(0);
            product(0, xa, 1, &c1, xv);
            mask(1, xv);
            pack(1, xv, xa);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (!KW && kDma && BC < 0) {
                // The last product's operands are read first, then the copies
                // of tile it+1 are issued: no LDS access of this iteration
                // follows them (each would wait for the copies), and they
                // arrive while the products and the key waves finish.
                constexpr int NM = 2 * NDB;
                uint4 tf[NM];
#pragma unroll
                for (int m = 0; m < NM; ++m) tf[m] = tfrag(other, 32 + 16 * (m / NDB), (m % NDB) * 32);
                __builtin_amdgcn_sched_barrier(0);
                if (it + 1 < nit) dma_tile(it + 1, (it + 1) % NBUF, tid_o);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int m = 0; m < NM; ++m) acc[m % NDB] = mma(xa[m / NDB], tf[m], acc[m % NDB]);
            } else {
                product(1, xa, 0, nullptr, xv);
            }
        };
        if constexpr (KW) {
            // key waves: the barrier of iteration 0, then tiles 0 .. nit-1 in
            // iterations 1 .. nit
            // (nit + 1 barriers, as the value waves)
            if (nit > 0)
                for (int it = 0; it <= nit; ++it) tile(it, std::false_type{}, std::integral_constant<int, -1>{});
        } else {
            // Iterations [it_lo, it_hi) see every (row, key) pair of this
            // wave's block: the masked tiles are a causal prefix and a tail
            // (rows past S, or every tile when the block's keys pass S).
            int it_lo = 0, it_hi = nit;
            if (kw + 31 >= S) {
                it_hi = 0;
            } else {
                if (a.causal) it_lo = min(nit, (kw + 31 - q_begin + kQRows - 1) / kQRows * G);
                it_hi = max(it_lo, (S - q_begin) / kQRows * G);
            }
            int it = 0;
            using BR = std::integral_constant<int, -1>;
            if constexpr (kDma) {
                // tiles with their buffer index (it % 3) as a constant
                using B0 = std::integral_constant<int, 0>;
                using B1 = std::integral_constant<int, 1>;
                using B2 = std::integral_constant<int, 2>;
                static_assert(NBUF == 3, "three tile buffers");
                while (it < it_lo) {  // the masked prefix starts at tile 0
                    tile(it, std::true_type{}, B0{});
                    if (++it == it_lo) break;
                    tile(it, std::true_type{}, B1{});
                    if (++it == it_lo) break;
                    tile(it, std::true_type{}, B2{});
                    ++it;
                }
                if (it < it_hi && it % 3 == 1) tile(it++, std::false_type{}, B1{});
                if (it < it_hi && it % 3 == 2) tile(it++, std::false_type{}, B2{});
                while (it < it_hi) {
                    tile(it, std::false_type{}, B0{});
                    if (++it == it_hi) break;
                    tile(it, std::false_type{}, B1{});
                    if (++it == it_hi) break;
                    tile(it, std::false_type{}, B2{});
                    ++it;
                }
            } else {
                for (; it < it_lo; ++it) tile(it, std::true_type{}, BR{});
                for (; it < it_hi; ++it) tile(it, std::false_type{}, BR{});
            }
            for (; it < nit; ++it) tile(it, std::true_type{}, BR{});
            if (nit > 0) __syncthreads();  // the key waves' last iteration
        }
    };
    if (kwave)
        run(std::true_type{});
    else
        run(std::false_type{});

    // ---- epilogue: transpose each accumulator through LDS (float32) ----
    float* st = reinterpret_cast<float*>(smem);
    float* part = nullptr;
    if constexpr (FUSED) part = a.wpart + (int64_t)item_index(b, g, kt, a.Hkv, nkt) * 4 * D;
#pragma unroll
    for (int which = 0; which < 2; ++which) {  // 0: keys, 1: values
        __syncthreads();
        if (kwave == (which == 0)) {
#pragma unroll
            for (int nb = 0; nb < NDB; ++nb)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float x = which == 0 ? acc[nb][4 * j + i] * a.scale : acc[nb][4 * j + i];
                        st[(kb * 32 + 8 * j + 4 * hi + i) * SP + nb * 32 + l32] = x;
                    }
        }
        __syncthreads();
        const OutView o1 = which == 0 ? a.dk1 : a.dv1;
        for (int e = tid; e < kKeysPerWg * CPR; e += kDkvThreads) {
            const int r = e / CPR, c = e - (e / CPR) * CPR;
            const int key = k0 + r;
            if (key >= S) continue;
            float x[8];
            load8f(st + r * SP + c * 8, x);
            if constexpr (FUSED) {
                const OutView on = which == 0 ? a.dkn : a.dvn;
                float w1[8], wn[8];
                load8f((which == 0 ? a.kw1 : a.vw1) + g * D + c * 8, w1);
                load8f((which == 0 ? a.kwn : a.vwn) + g * D + c * 8, wn);
                uint32_t r1[4], rn[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    r1[k] = pack2_bf16(w1[2 * k] * x[2 * k], w1[2 * k + 1] * x[2 * k + 1]);
                    rn[k] = pack2_bf16(wn[2 * k] * x[2 * k], wn[2 * k + 1] * x[2 * k + 1]);
                }
                *reinterpret_cast<uint4*>(out_row(o1, b, key, g) + c * 8) = make_uint4(r1[0], r1[1], r1[2], r1[3]);
                *reinterpret_cast<uint4*>(out_row(on, b, key, g) + c * 8) = make_uint4(rn[0], rn[1], rn[2], rn[3]);
            } else {
                uint32_t r1[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) r1[k] = pack2_bf16(x[2 * k], x[2 * k + 1]);
                *reinterpret_cast<uint4*>(out_row(o1, b, key, g) + c * 8) = make_uint4(r1[0], r1[1], r1[2], r1[3]);
            }
        }
        if constexpr (FUSED) {
            // column sums over this tile's keys of dKf * K1 and dKf * Kn
            // (values: dVf * V1, dVf * Vn): a thread takes 8 channels of 4
            // keys (its 8 source loads in flight together), the 32 key
            // groups' partials meet in the hand-off array, and one thread
            // per (source, channel) adds them in a fixed order
            constexpr int NCH = D / 8;
            constexpr int KPT = 4, NKG = kKeysPerWg / KPT;
            static_assert(NKG * NCH <= kDkvThreads, "one (key group, chunk) item per thread");
            static_assert(NKG * 2 * D * 4 <= (int)sizeof(xsm), "partials fit in the shared array");
            float* red = reinterpret_cast<float*>(xsm);  // [NKG][2][D]
            const View& s1 = which == 0 ? a.k1 : a.v1;
            const View& sn = which == 0 ? a.kn : a.vn;
            if (tid < NKG * NCH) {
                const int kg = tid / NCH, c8 = tid - (tid / NCH) * NCH;
                uint4 u1[KPT], un[KPT];
#pragma unroll
                for (int r = 0; r < KPT; ++r) {
                    const int key = k0 + kg * KPT + r;
                    u1[r] = make_uint4(0u, 0u, 0u, 0u);
                    un[r] = u1[r];
                    if (key < S) {
                        u1[r] = *reinterpret_cast<const uint4*>(row_ptr(s1, b, key, g) + c8 * 8);
                        un[r] = *reinterpret_cast<const uint4*>(row_ptr(sn, b, key, g) + c8 * 8);
                    }
                }
                float acc1[8], accn[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc1[e] = accn[e] = 0.0f;
#pragma unroll
                for (int r = 0; r < KPT; ++r) {
                    float x[8];
                    load8f(st + (kg * KPT + r) * SP + c8 * 8, x);  // rows past S hold zeros
                    const uint32_t w1[4] = {u1[r].x, u1[r].y, u1[r].z, u1[r].w};
                    const uint32_t wn[4] = {un[r].x, un[r].y, un[r].z, un[r].w};
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        acc1[2 * k] = fmaf(x[2 * k], bf16_lo(w1[k]), acc1[2 * k]);
                        acc1[2 * k + 1] = fmaf(x[2 * k + 1], bf16_hi(w1[k]), acc1[2 * k + 1]);
                        accn[2 * k] = fmaf(x[2 * k], bf16_lo(wn[k]), accn[2 * k]);
                        accn[2 * k + 1] = fmaf(x[2 * k + 1], bf16_hi(wn[k]), accn[2 * k + 1]);
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    red[(kg * 2 + 0) * D + c8 * 8 + e] = acc1[e];
                    red[(kg * 2 + 1) * D + c8 * 8 + e] = accn[e];
                }
            }
            __syncthreads();
            for (int i = tid; i < 2 * D; i += kDkvThreads) {
                const int src = i / D, d = i - (i / D) * D;
                float sum = 0.0f;
                for (int kg = 0; kg < NKG; ++kg) sum += red[(kg * 2 + src) * D + d];
                part[(2 * which + src) * D + d] = sum;
            }
        }
    }
}

// ---- 3. query tiles: dQ ----
// Stages each 64-key tile of the sources in LDS; with four sources the keys
// and values are fused in float32 (weights from LDS) as the tile is stored,
// rounded once to bf16 like the key-tile kernel's operands.
template <int D, int G, bool FUSED>
__global__ __launch_bounds__(kDqThreads) void bwd_dq_kernel(const BwdArgs a)
{
    constexpr int DP = (D + 31) / 32 * 32;
    constexpr int NDB = DP / 32;
    constexpr int KS = D / 16;
    constexpr int P = DP == 128 ? DP + 24 : DP + 8;  // row pitch, as in the key-tile kernel
    constexpr int CPR = D / 8;
    constexpr int TILE = kKTile * P;
    constexpr int HPW = G < kDqWaves ? G : kDqWaves;  // heads per workgroup
    constexpr int NHG = G / HPW;                      // head groups per KV head
    constexpr int RB = kDqWaves / HPW;                // 32-row blocks per workgroup
    constexpr int BM = RB * 32;              // query rows per workgroup

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * TILE];  // [buf][K~, V~][row][P]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;

    const int nqt = (a.S + BM - 1) / BM;
    const int items = a.B * a.Hkv * NHG * nqt;
    int item = blockIdx.x;
    if ((items & 7) == 0) item = (blockIdx.x & 7) * (items >> 3) + (blockIdx.x >> 3);
    const int unit = item / nqt;
    const int qt = a.causal ? nqt - 1 - (item - unit * nqt) : item - unit * nqt;  // heaviest first
    const int ug = unit / NHG, hg = unit - (unit / NHG) * NHG;
    const int b = ug / a.Hkv, g = ug - (ug / a.Hkv) * a.Hkv;
    const int S = a.S;
    const int h = g * G + hg * HPW + wave % HPW;
    const int r0 = qt * BM + (wave / HPW) * 32;  // this wave's 32 query rows

    if constexpr (DP > D) {
        for (int i = tid; i < 2 * 2 * kKTile * (DP - D); i += kDqThreads) {
            const int r = i / (DP - D), c = i - r * (DP - D);
            smem[r * P + D + c] = 0;
        }
    }

    // queries and output gradients as B operands (lane: query row r0 + l32)
    const int row = r0 + l32;
    const bool row_ok = row < S;
    uint4 qreg[KS], oreg[KS];
    {
        const int64_t off = (((int64_t)b * S + (row_ok ? row : 0)) * a.Hq + h) * D + hi * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qreg[ks] = make_uint4(0u, 0u, 0u, 0u);
            oreg[ks] = qreg[ks];
            if (row_ok) {
                qreg[ks] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + off + ks * 16);
                oreg[ks] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.dout) + off + ks * 16);
            }
        }
    }
    const int64_t lrow = ((int64_t)b * a.Hq + h) * S + (row_ok ? row : 0);
    const float lse2 = row_ok ? a.lse2[lrow] : 0.0f;
    const float dlt = row_ok ? a.delta[lrow] : 0.0f;

    f32x16 dq[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) dq[i] = f32x16{};

    const int q_last = min(S, (qt + 1) * BM) - 1;   // last row of the workgroup
    const int kend = a.causal ? q_last + 1 : S;
    const int nt = (kend + kKTile - 1) / kKTile;

    // staging: a thread owns one 16-byte chunk column (fixed channels, so
    // fixed fusion weights) of rows sr + p * RPP of each source
    constexpr int RPP = kDqThreads / CPR;
    constexpr int NPASS = (kKTile + RPP - 1) / RPP;
    constexpr int NSRC = FUSED ? 4 : 2;  // k1, v1 (, kn, vn)
    const int sc = tid % CPR, sr = tid / CPR;
    const bool s_active = sr < RPP;
    __shared__ __attribute__((aligned(16))) float Wsm[FUSED ? 4 * D : 4];  // a, a', b, b'
    if constexpr (FUSED) {
        for (int i = tid; i < 4 * D; i += kDqThreads) {
            const float* w = i < D ? a.kw1 : (i < 2 * D ? a.kwn : (i < 3 * D ? a.vw1 : a.vwn));
            Wsm[i] = w[g * D + i % D];
        }
        __syncthreads();
    }
    uint4 xr[NSRC][NPASS];
    // each source's tile through a buffer descriptor based at the tile's
    // first key and ending at its last key inside S (keys past S-1 read as
    // zero): 32-bit lane offsets instead of 64-bit address arithmetic
    auto load_tile = [&](int t) {
        const int k0t = t * kKTile;
        const int rows = min(S - k0t, kKTile);
#pragma unroll
        for (int s_ = 0; s_ < NSRC; ++s_) {
            const View& v = s_ == 0 ? a.k1 : (s_ == 1 ? a.v1 : (s_ == 2 ? a.kn : a.vn));
            const uint32_t rs = (uint32_t)v.ss * 2;  // bytes between keys
            const __amdgpu_buffer_rsrc_t rr = slab_rsrc(
                static_cast<const uint16_t*>(v.data) + (int64_t)b * v.sb + (int64_t)k0t * v.ss + (int64_t)g * v.sh,
                (uint32_t)(rows - 1) * rs + D * 2);
#pragma unroll
            for (int p = 0; p < NPASS; ++p) {
                const int r = sr + p * RPP;
                const uint32_t off = (s_active && r < kKTile) ? (uint32_t)r * rs + sc * 16 : kOffNone;
                xr[s_][p] = ld16(rr, off);
            }
        }
    };
    auto store_tile = [&](int buf) {
        uint16_t* kt_ = smem + (buf * 2 + 0) * TILE;
        uint16_t* vt_ = smem + (buf * 2 + 1) * TILE;
        if constexpr (FUSED) {
            float wk1[8], wkn[8], wv1[8], wvn[8];
            const int c0 = s_active ? sc * 8 : 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                wk1[i] = Wsm[c0 + i];
                wkn[i] = Wsm[D + c0 + i];
                wv1[i] = Wsm[2 * D + c0 + i];
                wvn[i] = Wsm[3 * D + c0 + i];
            }
#pragma unroll
            for (int p = 0; p < NPASS; ++p) {
                const int r = sr + p * RPP;
                if (!s_active || r >= kKTile) continue;
                *reinterpret_cast<uint4*>(kt_ + r * P + sc * 8) = fuse8_bf16(xr[0][p], xr[2][p], wk1, wkn);
                *reinterpret_cast<uint4*>(vt_ + r * P + sc * 8) = fuse8_bf16(xr[1][p], xr[3][p], wv1, wvn);
            }
        } else {
#pragma unroll
            for (int p = 0; p < NPASS; ++p) {
                const int r = sr + p * RPP;
                if (!s_active || r >= kKTile) continue;
                *reinterpret_cast<uint4*>(kt_ + r * P + sc * 8) = xr[0][p];
                *reinterpret_cast<uint4*>(vt_ + r * P + sc * 8) = xr[1][p];
            }
        }
    };

    const float sl2 = a.scale_log2;
    if (nt > 0) {
        load_tile(0);
        store_tile(0);
    }
    for (int t = 0; t < nt; ++t) {
        const int buf = t & 1;
        __syncthreads();
        if (t + 1 < nt) load_tile(t + 1);
        const uint16_t* kt_ = smem + (buf * 2 + 0) * TILE;
        const uint16_t* vt_ = smem + (buf * 2 + 1) * TILE;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int kk0 = t * kKTile + kb * 32;
            if (kk0 >= S || r0 >= S || (a.causal && kk0 > r0 + 31)) continue;  // wave-uniform
            // S^T and dP^T chains; LDS fragments read PF k-steps ahead of the
            // matrix-core instructions that use them
            constexpr int PF = 2;
            f32x16 st, dpt;
            uint4 fk[PF + 1], fv[PF + 1];
#pragma unroll
            for (int ks = 0; ks < PF; ++ks) {
                fk[ks] = row_frag(kt_, P, kb * 32, ks, l32, hi);
                fv[ks] = row_frag(vt_, P, kb * 32, ks, l32, hi);
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + PF < KS) {
                    fk[(ks + PF) % (PF + 1)] = row_frag(kt_, P, kb * 32, ks + PF, l32, hi);
                    fv[(ks + PF) % (PF + 1)] = row_frag(vt_, P, kb * 32, ks + PF, l32, hi);
                }
                const int c = ks % (PF + 1);
                st = mma(fk[c], qreg[ks], ks == 0 ? f32x16{} : st);
                dpt = mma(fv[c], oreg[ks], ks == 0 ? f32x16{} : dpt);
            }
            // the first half of the product's key fragments, read while the
            // exponentials run
            uint4 tf[NDB];
#pragma unroll
            for (int nb = 0; nb < NDB; ++nb) tf[nb] = tr_frag(kt_, P, kb * 32, nb * 32, l32, hi);
            // lane: query row; entries: keys kk0 + 8j + 4hi + i
            float dsv[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) dsv[e] = exp2_fast(st[e] * sl2 - lse2) * (dpt[e] - dlt);
            // blocks with an invisible (row, key) pair select zero there (the
            // exponentials may be infinite); the branch is uniform
            if ((a.causal && kk0 + 31 > r0) || kk0 + 31 >= S || r0 + 31 >= S) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = kk0 + 8 * (e >> 2) + 4 * hi + (e & 3);
                    const bool vis = row_ok && key < S && (!a.causal || key <= row);
                    dsv[e] = vis ? dsv[e] : 0.0f;
                }
            }
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const uint4 da = make_uint4(pack2_bf16(dsv[8 * c + 0], dsv[8 * c + 1]),
                                            pack2_bf16(dsv[8 * c + 2], dsv[8 * c + 3]),
                                            pack2_bf16(dsv[8 * c + 4], dsv[8 * c + 5]),
                                            pack2_bf16(dsv[8 * c + 6], dsv[8 * c + 7]));
#pragma unroll
                for (int nb = 0; nb < NDB; ++nb) {
                    const uint4 f = tf[nb];
                    if (c == 0) tf[nb] = tr_frag(kt_, P, kb * 32 + 16, nb * 32, l32, hi);
                    dq[nb] = mma(da, f, dq[nb]);
                }
            }
        }
        if (t + 1 < nt) store_tile(buf ^ 1);
    }

    // lane: channel nb*32 + l32; entries: rows r0 + 8j + 4hi + i
    uint16_t* dqp = static_cast<uint16_t*>(a.dq);
#pragma unroll
    for (int nb = 0; nb < NDB; ++nb) {
        const int ch = nb * 32 + l32;
        if (ch >= D) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0 + 8 * j + 4 * hi + i;
                if (r < S) {
                    const uint32_t pk = pack2_bf16(dq[nb][4 * j + i] * a.scale, 0.0f);
                    dqp[(((int64_t)b * S + r) * a.Hq + h) * D + ch] = (uint16_t)(pk & 0xffffu);
                }
            }
    }
}

// ---- 4. weight gradients: sum of the per-(batch, key tile) partials ----
// One workgroup per (vector w, KV head g); thread (d, part) sums every
// kRedParts-th partial of channel d in order, then the parts are added in
// order: a fixed summation order, so the result is deterministic.
constexpr int kRedParts = 8;
__global__ __launch_bounds__(256) void bwd_wreduce_kernel(const BwdArgs a)
{
    __shared__ float red[kRedParts][128];
    const int w = blockIdx.x / a.Hkv, g = blockIdx.x - (blockIdx.x / a.Hkv) * a.Hkv;
    const int n = a.B * a.nkt;
    for (int i = threadIdx.x; i < kRedParts * a.D; i += 256) {
        const int d = i % a.D, part = i / a.D;
        float s = 0.0f;
        // (unrolled so that several loads are in flight; the additions keep their order)
#pragma unroll 8
        for (int k = part; k < n; k += kRedParts) {
            const int b = k / a.nkt, kt = k - (k / a.nkt) * a.nkt;
            s += a.wpart[((int64_t)item_index(b, g, kt, a.Hkv, a.nkt) * 4 + w) * a.D + d];
        }
        red[part][d] = s;
    }
    __syncthreads();
    for (int d = threadIdx.x; d < a.D; d += 256) {
        float s = 0.0f;
        for (int part = 0; part < kRedParts; ++part) s += red[part][d];
        float* out = w == 0 ? a.dkw1 : (w == 1 ? a.dkwn : (w == 2 ? a.dvw1 : a.dvwn));
        out[g * a.D + d] = s;
    }
}

template <int D, bool FUSED, int G>
int launch_bwd3(const BwdArgs& a, hipStream_t st)
{
    const int64_t rows = (int64_t)a.B * a.S * a.Hq;
    {
        const int64_t lanes = (rows + kPrepRows - 1) / kPrepRows * (D / 8 <= 8 ? 8 : 16);
        if ((lanes + 255) / 256 > 0x7fffffff) return (int)hipErrorInvalidValue;
        hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, st, a);
    }
    int rc = (int)hipGetLastError();
    if (rc) return rc;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, FUSED, G>), dim3((unsigned)(a.B * a.Hkv * a.nkt)), dim3(kDkvThreads), 0,
                       st, a);
    if ((rc = (int)hipGetLastError())) return rc;
    constexpr int HPW = G < kDqWaves ? G : kDqWaves;
    constexpr int BM = (kDqWaves / HPW) * 32;
    const int nqt = (a.S + BM - 1) / BM;
    const dim3 qgrid((unsigned)(a.B * a.Hkv * (G / HPW) * nqt));
    hipLaunchKernelGGL((bwd_dq_kernel<D, G, FUSED>), qgrid, dim3(kDqThreads), 0, st, a);
    if ((rc = (int)hipGetLastError())) return rc;
    if constexpr (FUSED) {
        hipLaunchKernelGGL(bwd_wreduce_kernel, dim3((unsigned)(4 * a.Hkv)), dim3(256), 0, st, a);
        rc = (int)hipGetLastError();
    }
    return rc;
}

template <int D, bool FUSED>
int launch_bwd2(const BwdArgs& a, hipStream_t st)
{
    switch (a.G) {
    case 1: return launch_bwd3<D, FUSED, 1>(a, st);
    case 2: return launch_bwd3<D, FUSED, 2>(a, st);
    case 4: return launch_bwd3<D, FUSED, 4>(a, st);
    case 8: return launch_bwd3<D, FUSED, 8>(a, st);
    default: return (int)hipErrorInvalidValue;
    }
}

template <bool FUSED>
int launch_bwd1(const BwdArgs& a, hipStream_t st)
{
    switch (a.D) {
    case 64: return launch_bwd2<64, FUSED>(a, st);
    case 80: return launch_bwd2<80, FUSED>(a, st);
    case 96: return launch_bwd2<96, FUSED>(a, st);
    case 128: return launch_bwd2<128, FUSED>(a, st);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace

int launch_backward(const BwdArgs& a, bool fused, void* stream)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (a.B == 0 || a.S == 0) return 0;
    return fused ? launch_bwd1<true>(a, st) : launch_bwd1<false>(a, st);
}

}  // namespace fkv
