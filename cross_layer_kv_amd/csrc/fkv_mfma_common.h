// fkv_mfma_common.h -- device helpers shared by the kernels that are not the
// plain decode (causal prefill, high-GQA decode, 4-bit decode and its
// quantiser, backward pass): fp16 / bf16 packing, the two-source fusion dot
// products, half-wave and token-group exchanges and buffer-descriptor loads.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fkv {
namespace dev {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed fp16 pair, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack2(float lo, float hi)
{
    f16x2 v;
    v[0] = (_Float16)lo;
    v[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi)
{
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// A packed pair of bf16 values re-encoded as fp16 (exact inside fp16 range).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) { return pack2(bf16_lo(w), bf16_hi(w)); }

__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 u)
{
    return make_uint4(bf16x2_to_f16x2(u.x), bf16x2_to_f16x2(u.y), bf16x2_to_f16x2(u.z), bf16x2_to_f16x2(u.w));
}

__device__ __forceinline__ f16x8 as_f16x8(uint4 u) { return __builtin_bit_cast(f16x8, u); }

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v;

// (source 1, source n) bf16 pairs of the low / high element of two packed
// words: low half from u1, high half from un.
__device__ __forceinline__ uint32_t pair_lo(uint32_t u1, uint32_t un) { return __builtin_amdgcn_perm(un, u1, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t u1, uint32_t un) { return __builtin_amdgcn_perm(un, u1, 0x07060302u); }

// w1 * x1 + wn * xn for a (x1, xn) bf16 pair and weights split as bf16
// (hi, lo) pairs: two dot products with float32 accumulation.
// The compiler emits the accumulate-in-place form of the product plus a
// register clear; that pair issues faster than the three-operand form with a
// zero addend, which measured at well under half rate on gfx950.
__device__ __forceinline__ float fuse_pair(uint32_t pair, uint32_t w_hi, uint32_t w_lo)
{
    const bf16x2v x = __builtin_bit_cast(bf16x2v, pair);
    const float lo = __builtin_amdgcn_fdot2_f32_bf16(x, __builtin_bit_cast(bf16x2v, w_lo), 0.0f, false);
    return __builtin_amdgcn_fdot2_f32_bf16(x, __builtin_bit_cast(bf16x2v, w_hi), lo, false);
}

// max / sum of a value and its copy in the lane 32 apart (v_permlane32_swap:
// the upper half of the first operand trades places with the lower half of
// the second), a VALU exchange instead of an LDS permute round trip
__device__ __forceinline__ float halves_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ constexpr f16x2 kOnes2 = {(_Float16)1.0f, (_Float16)1.0f};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Weight 2^(m - M) of a partial with max m against a common max M; 0 for an
// empty partial (m = -inf).
__device__ __forceinline__ float rel_weight(float m, float M) { return m == -INFINITY ? 0.0f : exp2_fast(m - M); }

// Sum over the LPT (8 or 16) lanes of a token group with DPP permutations:
// xor 1, xor 2 (quad permutes), then mirror within 8 and within 16 lanes.
template <int LPT>
__device__ __forceinline__ float token_group_sum(float v)
{
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    if constexpr (LPT == 16)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    return v;
}


// Buffer descriptor over one (batch, KV head) slab of a cache: base at token 0
// of that head, size up to the end of row S-1.  A load at an offset past the
// size returns zeros (hardware range check), which is how rows past the end
// of the sequence read as 0 without per-load predicates.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Loads of data a call reads exactly once (source rows, 4-bit codes and
// their metadata): non-temporal, so they stream through the caches without
// displacing lines that are reused.
__device__ __forceinline__ uint32_t stream4(const void* p)
{
    return __builtin_nontemporal_load(static_cast<const uint32_t*>(p));
}
__device__ __forceinline__ uint4 stream16(const void* p)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(static_cast<const u32x4*>(p)));
}

constexpr uint32_t kOffNone = 0x80000000u;  // always past the descriptor's size

__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t ld4(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
// 16 bytes at lane offset + uniform offset; the range check covers the sum
// (measured on gfx950), so either part may carry the row position.  For data
// read once per call: the load is non-temporal (cache policy bit 1, "nt").
__device__ __forceinline__ uint4 ld16s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, (int)soff, 2));
}

}  // namespace dev
}  // namespace fkv
