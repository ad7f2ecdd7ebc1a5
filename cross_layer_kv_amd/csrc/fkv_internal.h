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

// Decode (S_q = 1), split over the key axis.  One workgroup per
// (batch, kv head, split); the last workgroup of each (batch, kv head) to
// finish merges the splits (completion counter in the workspace).
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
    unsigned* counters;     // [B * Hkv], zero between calls
    float* ml;              // [B * Hkv, n_splits, G, 2]  (running max, sum)
    float* part;            // [B * Hkv, n_splits, G, D]  (unnormalised sums)
    int32_t B, Sk, Hq, Hkv, D, G;
    int32_t n_splits, chunk; // chunk: tokens per split, a multiple of 64
    float scale_log2;       // softmax scale * log2(e)
};

struct DecodePlan {
    int32_t n_splits, chunk;
    size_t counters_bytes, ml_bytes, part_bytes, total_bytes;
};

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

// Launchers (device code units).  They return 0 on success, else the HIP
// error code of the failed launch.
int launch_decode(const DecodeArgs& a, bool fused, int dtype, void* stream);
int launch_prefill(const PrefillArgs& a, bool fused, void* stream);
// Query rows per prefill workgroup for a GQA ratio (0 when unsupported).
int prefill_rows_per_tile(int G);

}  // namespace fkv
