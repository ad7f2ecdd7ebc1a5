// fkv_internal.h -- argument blocks passed from the host dispatcher to the
// kernel launchers of libfusedkv.  Plain C++ (no HIP headers), so the host
// validation unit can include it.
#pragma once

#include <cstddef>
#include <cstdint>

namespace fkv {

// A [B, S, H, D] view in elements; channel stride 1.
struct View {
    const void* data;
    int64_t sb, ss, sh;
};

// Decode (S_q = 1).  One workgroup per (batch, kv head, split of the key
// axis); the waves of a workgroup share its tokens and merge in LDS.  With one
// split the workgroup writes O and LSE itself; with several it writes
// partial (max, sum, unnormalised O) rows and a second kernel merges them.
struct DecodeArgs {
    const void* q;          // [B, 1, Hq, D]
    View k1, kn, v1, vn;    // kn / vn unused for single-source calls
    const float* kw1;       // [Hkv, D] each; unused for single-source calls
    const float* kwn;
    const float* vw1;
    const float* vwn;
    const int32_t* seqlens; // [B] or nullptr
    void* out;              // [B, 1, Hq, D]
    float* lse;             // [B, Hq] or nullptr
    float* ml;              // [B * Hkv, n_splits, G, 2]  (running max, sum)
    float* part;            // [B * Hkv, n_splits, G, D]  (unnormalised sums)
    int32_t B, Sk, Hq, Hkv, D, G;
    int32_t n_splits, chunk; // chunk: tokens per split, a multiple of 64
    float scale_log2;       // softmax scale * log2(e)
};

struct DecodePlan {
    int32_t waves, n_splits, chunk;
    size_t ml_bytes, part_bytes, total_bytes;
};

// Waves per decode workgroup.  Chosen so that one workgroup fills a compute
// unit at the occupancy the kernel's register count allows (4 SIMDs x waves
// per SIMD): e.g. the bf16 four-source kernel with G <= 2 uses 123 VGPRs,
// 4 waves per SIMD, 16 waves.  The kernels are compiled with the matching
// launch bound, so the register budget is enforced.
// Query heads per KV head served by the matrix-core decode kernel.
constexpr int kHighGqa = 64;

constexpr int decode_waves(int dtype_f32, bool fused, int G)
{
    if (G == kHighGqa) return 4;  // 2 key halves x 2 blocks of 32 heads
    if (!dtype_f32) {
        if (fused) return G <= 2 ? 16 : (G == 4 ? 8 : 4);
        return G <= 2 ? 16 : (G == 4 ? 12 : 8);
    }
    if (fused) return G <= 4 ? 8 : 4;
    return G <= 2 ? 12 : (G == 4 ? 8 : 4);
}

// Tokens a wave takes per iteration of the decode loop.  The bf16
// four-source kernel with G <= 2 takes 8 when a lane owns 8 channels, which
// halves its load registers (123 VGPRs) so that 4 waves per SIMD fit; at
// D = 96 a lane owns 6 channels and 16 tokens fit the same budget (121);
// the others take 16.
constexpr int decode_wave_tokens(int dtype_f32, bool fused, int G, int D)
{
    return (!dtype_f32 && fused && G <= 2 && D != 96) ? 8 : 16;
}

// Waves per workgroup of the 4-bit decode kernel (a wave takes 32-token
// blocks), one workgroup per (batch, KV head) when there are enough of them.
// Up to D = 96: sixteen single-source waves (4 per SIMD, 128 VGPRs) or
// twelve four-source waves (3 per SIMD, 168 VGPRs with the value side
// loaded when a block starts).  At D = 128 neither fits: eight.
constexpr int kivi_waves(bool fused, int G, int D)
{
    (void)G;
    return D <= 96 ? (fused ? 12 : 16) : 8;
}

// Prefill (S_q == S_k), bf16 only.
struct PrefillArgs {
    const void* q;          // [B, S, Hq, D] bf16
    View k1, kn, v1, vn;
    const float* kw1;
    const float* kwn;
    const float* vw1;
    const float* vwn;
    void* out;              // [B, S, Hq, D] bf16
    float* lse;             // [B, Hq, S] or nullptr
    int32_t B, S, Hq, Hkv, D, G;
    int32_t causal;
    int32_t n_qtiles;       // ceil(S / rows per tile)
    float scale_log2;
};

// KIVI-style 4-bit cache of one source, contiguous (layout in fusedkv.h),
// NB = ceil(S/32):
//   keys    codes [B, Hkv, S, D/2] bytes (channel 2i low nibble, 2i+1 high);
//           scale / minv fp16 [B, Hkv, NB, D]
//   values  codes [B, Hkv, NB, D, 16] bytes, channel-major per 32-token block;
//           scale / minv fp16 [B, Hkv, NB, ceil(D/32), 32]
struct Q4View {
    const void* codes;
    const void* scale;
    const void* minv;
};

// Decode over 4-bit sources: the decode arguments (q, out, lse, workspace,
// weights, shape, split plan; the View members are unused) plus the sources.
struct KiviDecodeArgs : DecodeArgs {
    Q4View qk1, qkn, qv1, qvn;  // qkn / qvn unused for single-source calls
};

// Quantisation of one bf16 source into a 4-bit cache.
struct KiviQuantArgs {
    View src;       // [B, S, H, D] bf16
    void* codes;
    void* scale;
    void* minv;
    int32_t B, S, H, D;
    int32_t is_value;  // 0: per-channel groups of 32 tokens, 1: per-token groups of 32 channels
};

// A writable [B, S, H, D] view in elements; channel stride 1.
struct OutView {
    void* data;
    int64_t sb, ss, sh;
};

// Backward pass (S_q == S_k, bfloat16).  Single-source calls (Lite or the
// plain control) use k1 / v1 as the key / value source, dk1 / dv1 as their
// gradients, and leave the n-sources, the weights and their gradients unused.
struct BwdArgs {
    const void* q;          // [B, S, Hq, D]
    View k1, kn, v1, vn;
    const float* kw1;       // [Hkv, D] each
    const float* kwn;
    const float* vw1;
    const float* vwn;
    const void* out;        // forward output O [B, S, Hq, D]
    const float* lse;       // forward LSE (natural log) [B, Hq, S]
    const void* dout;       // dO [B, S, Hq, D]
    void* dq;               // [B, S, Hq, D]
    OutView dk1, dkn, dv1, dvn;
    float* dkw1;            // [Hkv, D] each
    float* dkwn;
    float* dvw1;
    float* dvwn;
    float* lse2;            // workspace [B, Hq, S]: LSE * log2(e)
    float* delta;           // workspace [B, Hq, S]: rowsum(dO * O)
    float* wpart;           // workspace [B, Hkv, nkt, 4, D]: weight-gradient partials
    int32_t B, S, Hq, Hkv, D, G, causal;
    int32_t nkt;            // key tiles of 128 per (batch, KV head)
    float scale;            // softmax scale
    float scale_log2;       // softmax scale * log2(e)
};

// Keys per workgroup of the backward key-tile kernel (sizes the workspace).
constexpr int kBwdKeyTile = 128;

// Bytes of the static device scratch behind fkv_decode_noalloc (split-K
// partials); it must match FKV_NOALLOC_SCRATCH_BYTES in fusedkv.h.
constexpr size_t kNoallocScratchBytes = (size_t)8 << 20;

// Device address of that scratch on the calling thread's current device,
// looked up once per device.  Returns 0, or the HIP error code.
int scratch_pointer(void** out);

// Launchers (device code units).  They return 0 on success, else the HIP
// error code of the failed launch.
int launch_decode(const DecodeArgs& a, bool fused, int dtype, int waves, void* stream);
// Decode with G == kHighGqa query heads per KV head (bfloat16, matrix cores).
int launch_decode_hgqa(const DecodeArgs& a, bool fused, void* stream);
// Merge of decode split partials (bfloat16 output); used by the 4-bit decode.
int launch_decode_combine_bf16(const DecodeArgs& a, void* stream);
// 4-bit KIVI-style sources: quantiser and decode (bfloat16 queries/outputs).
int launch_kivi_quantize(const KiviQuantArgs& a, void* stream);
int launch_kivi_decode(const KiviDecodeArgs& a, bool fused, int waves, void* stream);
int launch_prefill(const PrefillArgs& a, bool fused, void* stream);
int launch_backward(const BwdArgs& a, bool fused, void* stream);

// Storage-layer cache write: tokens 0..S_new-1 of k_new / v_new to cache
// positions pos0..pos0+S_new-1; elt = element bytes (2 or 4).
struct StoreArgs {
    View k_new, v_new;
    OutView k_cache, v_cache;
    int B, S_new, H, D, pos0, elt;
};
int launch_store_kv(const StoreArgs& a, void* stream);
// Query rows per prefill workgroup for a GQA ratio (0 when unsupported).
int prefill_rows_per_tile(int G);

}  // namespace fkv
