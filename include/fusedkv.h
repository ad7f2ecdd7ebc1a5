/*
 * fusedkv.h -- C ABI of libfusedkv: FusedKV reconstruction-layer attention on
 * AMD Instinct MI355X (gfx950).
 *
 * Pages cited (by title):
 *   [Deck]  "FusedKV: Reconstructing KV Caches with Cross-Layer Fusion"
 *           (reading slides of arXiv:2512.03870v3, Lin et al.)
 *   [Notes] "FusedKV:通过跨层融合重构 KV 缓存" (reading notes of the same paper)
 *
 * The method.  A model of L = 2n layers keeps KV caches only for its lower
 * half (storage layers 1..n).  Each upper layer i > n rebuilds its keys and
 * values from the stored post-RoPE caches of layer 1 and layer n with its own
 * per-channel vectors, broadcast over tokens ([Deck] frame "FusedKV learns
 * two-source, channel-wise fusion", Eqs. (4)-(5); [Notes] section 2.3):
 *     K^i = a  (.) K^1 + a' (.) K^n,        V^i = b (.) V^1 + b' (.) V^n
 * and runs its own layer-specific queries through grouped-query softmax
 * attention over them.  The reconstruction happens tile by tile inside the
 * attention kernels and is never written to memory ([Deck] frame "Half the
 * storage can require 50% more cache I/O"; [Notes] section 2.3).
 * FusedKV-Lite takes K^i = K^n and V^i = V^1 unchanged ([Deck] frame "Lite
 * separates the key source from the value source", Eq. (6)); the same
 * single-source entry points run plain attention of a storage layer over its
 * own caches, the control.
 *
 * Conventions shared by every entry point
 *   - One call handles one layer.  All work is enqueued on `stream` (a
 *     hipStream_t; NULL means the default stream) and the call returns after
 *     the enqueue; nothing is synchronised.
 *   - Every pointer except the host-side parameter structs is DEVICE memory
 *     owned by the caller.  The library never allocates or frees memory and
 *     keeps no pointer after returning.
 *   - Q and O are contiguous [B, S_q, H_q, D] in the data dtype.  The optional
 *     LSE output is contiguous float32 [B, H_q, S_q], natural log.
 *   - A cache is a [B, S_k, H_kv, D] view given by a base pointer and element
 *     strides for the batch, token and head axes; the channel axis is
 *     contiguous.  Head-major storage [B, H_kv, S_k, D] (stride_s = D) streams
 *     best.  Base pointers and every row start must be 16-byte aligned.
 *   - Query head h reads KV head h / G, G = H_q / H_kv (contiguous groups).
 *   - softmax scale: 0 selects 1/sqrt(D); negative scales are rejected.
 *   - Fusion weights are float32 device arrays [H_kv, D] for one layer.  Key
 *     weights must be equal on the two coordinates of each RoPE pair so that
 *     fused post-RoPE scores stay relative-position only ([Deck] frame
 *     "Post-RoPE fusion needs paired key weights", Eqs. (7)-(8); [Notes]
 *     section 2.4); the kernels do not re-check this (see fkv_check_tied).
 *
 * Errors.  Arguments are validated on the host from the parameter structs and
 * pointer values only (null, alignment, sizes); an invalid call returns a
 * non-zero status before anything is enqueued, and fkv_last_error() gives the
 * reason on that thread.  A failed launch returns FKV_ERROR_LAUNCH.  Faults
 * inside kernels surface at the caller's next synchronisation.  No C++
 * exception crosses this interface.  Calls are re-entrant.
 */
#ifndef FUSEDKV_H_
#define FUSEDKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FKV_ABI_VERSION 7

typedef enum {
    FKV_SUCCESS = 0,
    FKV_ERROR_INVALID_VALUE = 1, /* null/misaligned pointer, bad shape or stride */
    FKV_ERROR_UNSUPPORTED = 2,   /* valid request outside what the kernels cover */
    FKV_ERROR_WORKSPACE = 3,     /* workspace missing or smaller than required */
    FKV_ERROR_LAUNCH = 4         /* the HIP runtime rejected a launch */
} fkv_status;

typedef enum {
    FKV_F32 = 0, /* float32 data, float32 arithmetic */
    FKV_BF16 = 1 /* bfloat16 data, float32 accumulation */
} fkv_dtype;

/* A [B, S_k, H_kv, D] cache view: element strides for b, s, h. */
typedef struct {
    const void* data;
    int64_t stride_b, stride_s, stride_h;
} fkv_cache;

typedef struct {
    int32_t batch;        /* B >= 0 */
    int32_t seqlen_q;     /* S_q: 1 for decode; S_k for prefill */
    int32_t seqlen_k;     /* S_k >= 0: cached tokens (the cache's token extent) */
    int32_t num_q_heads;  /* H_q = G * H_kv, G in {1, 2, 4, 8}; decode also G = 64 */
    int32_t num_kv_heads; /* H_kv >= 1 */
    int32_t head_dim;     /* D in {64, 80, 96, 128} */
    int32_t dtype;        /* fkv_dtype */
    float softmax_scale;  /* 0 -> 1/sqrt(D); otherwise finite and > 0 */
    int32_t causal;       /* prefill: 1 = causal mask (query p sees keys t <= p) */
} fkv_params;

/* Per-layer fusion vectors, device float32 [H_kv, D] each:
 * k_w1 = a, k_wn = a' (keys), v_w1 = b, v_wn = b' (values). */
typedef struct {
    const float* k_w1;
    const float* k_wn;
    const float* v_w1;
    const float* v_wn;
} fkv_fusion;

/* ABI version of the loaded library (FKV_ABI_VERSION). */
int fkv_abi_version(void);

/* Static text for a status code. */
const char* fkv_status_string(fkv_status status);

/* Reason for the last non-success status returned on the calling thread. */
const char* fkv_last_error(void);

/*
 * Bytes of device workspace fkv_decode / fkv_lite_decode need for `params`:
 * the split-K partial results when the key axis is split across workgroups
 * (few batch rows x KV heads, long caches), otherwise 0.  The size covers
 * both entry points.  Returns 0 also when params is invalid.  The workspace
 * needs no initialisation; it only carries data between the two kernels of
 * one call, so calls that may run concurrently need separate workspaces.
 */
size_t fkv_decode_workspace_size(const fkv_params* params);

/*
 * fkv_decode -- one decode step (S_q = 1) of a FusedKV reconstruction layer.
 * [Deck] frame "FusedKV learns two-source, channel-wise fusion", Eqs. (4)-(5);
 * [Notes] section 2.3 (fuse inside the attention kernel, block by block).
 *
 * The query of every batch row attends to keys t in [0, len_b), len_b =
 * seqlens_k[b] clamped to [0, seqlen_k] (or seqlen_k when seqlens_k is NULL):
 * the new token's keys are already in the caches of layers 1 and n when the
 * upper layers run ([Notes] section 2.3).  Keys are a (.) K1 + a' (.) Kn and
 * values b (.) V1 + b' (.) Vn, formed in float32 in registers and never
 * stored.  An empty row yields O = 0 and LSE = -inf.
 *
 * With G = 64 query heads per KV head (bfloat16 only; float32 returns
 * FKV_ERROR_UNSUPPORTED) the dot products run on the matrix cores: the
 * many-heads decode regime of [Deck] frame "Decode cost depends on the
 * inference regime" (Fig. 5, right).  Each token is fused once for all 64
 * heads, and the fused tiles and probabilities are rounded to IEEE binary16
 * for the products, as in fkv_prefill.
 *
 *   q          device [B, 1, H_q, D]
 *   k1, kn     caches of layers 1 and n (post-RoPE keys)
 *   v1, vn     value caches of layers 1 and n
 *   fusion     device weights of this layer (all four non-NULL)
 *   seqlens_k  device int32 [B] or NULL
 *   out        device [B, 1, H_q, D], data dtype
 *   lse        device float32 [B, H_q] or NULL
 *   workspace  device, >= fkv_decode_workspace_size(params) bytes and
 *              256-byte aligned; may be NULL when that size is 0
 */
fkv_status fkv_decode(const fkv_params* params, const void* q,
                      fkv_cache k1, fkv_cache kn, fkv_cache v1, fkv_cache vn,
                      const fkv_fusion* fusion, const int32_t* seqlens_k,
                      void* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * fkv_decode_noalloc -- fkv_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops and harnesses
 * that forbid allocation.  It takes no workspace and allocates nothing: when
 * the key axis is split, the split partials go to a static device scratch of
 * FKV_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends (its device address is looked up once per device).
 * The launch plan, kernels and results are those of fkv_decode with a
 * workspace, bit for bit.  A call whose partials need more than the scratch
 * (fkv_decode_workspace_size(params) > FKV_NOALLOC_SCRATCH_BYTES) returns
 * FKV_ERROR_WORKSPACE before anything is enqueued.  The scratch needs no
 * initialisation (each call writes every partial before reading it), but all
 * calls on one GPU share it: calls that may overlap on one GPU (concurrent
 * streams or threads) race and must be serialised by the caller.  Arguments
 * and errors otherwise as fkv_decode.
 */
#define FKV_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
fkv_status fkv_decode_noalloc(const fkv_params* params, const void* q,
                              fkv_cache k1, fkv_cache kn, fkv_cache v1,
                              fkv_cache vn, const fkv_fusion* fusion,
                              const int32_t* seqlens_k, void* out, float* lse,
                              void* stream);

/*
 * fkv_lite_decode -- one decode step over a single key cache and a single
 * value cache.  FusedKV-Lite passes (K^n, V^1) ([Deck] frame "Lite separates
 * the key source from the value source", Eq. (6)); plain attention of a
 * storage layer (the control) passes that layer's own (K^i, V^i).  Arguments
 * otherwise as fkv_decode.
 */
fkv_status fkv_lite_decode(const fkv_params* params, const void* q,
                           fkv_cache k_src, fkv_cache v_src,
                           const int32_t* seqlens_k, void* out, float* lse,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * fkv_prefill -- attention of a FusedKV reconstruction layer over a whole
 * prompt (S_q == S_k), bfloat16 data.  With causal = 1, query row p sees keys
 * t <= p.  [Deck] frames "FusedKV learns two-source, channel-wise fusion"
 * (Eqs. (4)-(5)) and "Prefill improves while kernel throughput falls"
 * (the fused kernel's throughput, paper Fig. 4); [Notes] section 2.3 (the
 * reconstruction is built block by block inside the attention kernel).
 *
 * Every attention workgroup fuses the 64-token key and value tiles it reads
 * in float32 registers and keeps them in LDS only; nothing of the
 * reconstruction is written to memory.  The matrix-core operands are IEEE
 * binary16 (11 significant bits):
 *   - fused key and value tiles are rounded once from float32;
 *   - at D <= 96 the queries are multiplied by scale * log2(e) in float32 and
 *     then rounded to binary16 (one rounding per element); at D = 128 the
 *     bf16 queries convert to binary16 exactly and the scale is applied to
 *     the float32 scores;
 *   - softmax probabilities are rounded to binary16 after the exponential.
 * Softmax, row sums and accumulation are float32.
 * Limits that follow from binary16 operands:
 *   - |scale*log2(e)*q| (D <= 96) or |q| (D = 128), |fused key| and |fused
 *     value| must stay below 65504, else the call yields inf/NaN;
 *   - each operand rounding carries a relative error of up to 2^-11, so a
 *     score s (in log2 units) carries an absolute error that grows with |s|;
 *     with softmax inputs spanning up to ~30 log2 units within a row the
 *     output stays inside a 1e-2 relative error, while scores near 100 log2
 *     units (a near one-hot softmax) exceed it (measured 2.6e-2).
 *
 *   q          device [B, S, H_q, D] bfloat16
 *   out        device [B, S, H_q, D] bfloat16
 *   lse        device float32 [B, H_q, S] or NULL
 */
fkv_status fkv_prefill(const fkv_params* params, const void* q,
                       fkv_cache k1, fkv_cache kn, fkv_cache v1, fkv_cache vn,
                       const fkv_fusion* fusion, void* out, float* lse,
                       void* stream);

/*
 * fkv_lite_prefill -- prefill over one key cache and one value cache
 * (FusedKV-Lite with (K^n, V^1), or the plain control with a layer's own
 * caches).  The bf16 tiles convert to binary16 exactly (inside its range);
 * arguments, arithmetic and limits otherwise as fkv_prefill.
 */
fkv_status fkv_lite_prefill(const fkv_params* params, const void* q,
                            fkv_cache k_src, fkv_cache v_src, void* out,
                            float* lse, void* stream);

/*
 * fkv_check_tied -- host-side check that key fusion weights are tied on RoPE
 * pairs: |w[h, i] - w[h, j]| <= tol for every pair (i, j) of every head.
 * pairing 0: interleaved pairs (2j, 2j+1); 1: half-split pairs (j, j + D/2).
 * host_k_w is HOST float32 [h_kv, d].  Returns FKV_SUCCESS when tied,
 * FKV_ERROR_INVALID_VALUE when not (or on bad arguments).  [Deck] frame
 * "Post-RoPE fusion needs paired key weights"; [Notes] section 2.4 (the pair
 * to tie is the one the RoPE layout actually rotates together).
 */
fkv_status fkv_check_tied(const float* host_k_w, int32_t h_kv, int32_t d,
                          int32_t pairing, float tol);

/*
 * ---- KIVI-style 4-bit source caches ----
 * [Deck] frame "Four-bit KV quantization is the stronger combination"
 * (Tables 14-15); [Notes] section A.6.5: FusedKV composed with 4-bit KIVI
 * caches cuts the payload 4-fold on top of FusedKV's halving (1/8 of an FP16
 * vanilla cache, metadata excluded).  The pages print no format; this one is
 * the published KIVI scheme at 4 bits:
 *   keys   grouped per channel over 32 consecutive tokens,
 *   values grouped per token over 32 consecutive channels (the last group of
 *          an axis may be shorter, e.g. 16 channels for D = 80);
 *   a group keeps its minimum and scale = (max - min) / 15 as IEEE binary16;
 *   code = rint((x - min) * (1 / scale)) clamped to 0..15 (0 if scale == 0),
 *   decided in float32 with the rounded min and scale; x ~ min + scale*code.
 * Arrays of one quantised source, contiguous, S = params->seqlen_k,
 * NB = ceil(S/32):
 *   keys    codes uint8    [B, H_kv, S, D/2]   channel 2i low nibble, 2i+1 high
 *           scale binary16 [B, H_kv, NB, D]     (minv: same shape)
 *   values  codes uint8    [B, H_kv, NB, D, 16]
 *           scale binary16 [B, H_kv, NB, ceil(D/32), 32]  (minv: same shape)
 * Value codes are channel-major inside each 32-token block: the 16 bytes of
 * (block, channel) are four 4-byte words; word w holds the tokens
 * 4w + (e%4) + 16(e/4) of the block for e = 0..7, element e in nibble e/2
 * (even e) or 4 + e/2 (odd e), nibble k meaning bits 4k..4k+3.  A value
 * scale/minv row lists the block's tokens in the same order (position 8w +
 * e).  Tokens of the last block past S have code, scale and minv 0.  (This
 * is the order in which the decode kernel's matrix-core products consume the
 * codes, so that every operand is one aligned load.)
 * All three device pointers 16-byte aligned; the caller owns them.
 */
typedef struct {
    const void* codes;
    const void* scale;
    const void* minv;
} fkv_q4_cache;

/* Bytes of the codes of one quantised source, and of its scale (or minv)
 * array (is_value 0: keys, 1: values).  0 for invalid params. */
size_t fkv_kivi_codes_bytes(const fkv_params* params, int32_t is_value);
size_t fkv_kivi_meta_bytes(const fkv_params* params, int32_t is_value);

/*
 * fkv_kivi_quantize -- write the 4-bit cache of one bfloat16 source: all
 * seqlen_k tokens of every (batch row, KV head); dst arrays are overwritten.
 * params: batch, seqlen_k, num_kv_heads, head_dim and dtype = FKV_BF16 are
 * used (num_q_heads must still be a valid multiple).  src any strides with
 * 16-byte aligned rows, as fkv_cache.  Asynchronous on `stream`.
 */
fkv_status fkv_kivi_quantize(const fkv_params* params, fkv_cache src,
                             int32_t is_value, fkv_q4_cache dst, void* stream);

/*
 * fkv_kivi_decode -- fkv_decode over 4-bit sources, fused after
 * dequantisation (min + scale * code).  Both products run on the matrix
 * cores with the codes as exact binary16 values; the key scale and key
 * weight fold into the query (rounded to binary16), the value scale into
 * the probabilities (binary16), all accumulation float32.  k1/kn are key caches, v1/vn value caches in the format above.
 * bfloat16 queries and outputs, G in {1, 2, 4, 8}; other arguments,
 * workspace (fkv_decode_workspace_size covers these calls) and errors as
 * fkv_decode.
 */
fkv_status fkv_kivi_decode(const fkv_params* params, const void* q,
                           fkv_q4_cache k1, fkv_q4_cache kn, fkv_q4_cache v1,
                           fkv_q4_cache vn, const fkv_fusion* fusion,
                           const int32_t* seqlens_k, void* out, float* lse,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/* fkv_kivi_lite_decode -- one 4-bit key and one 4-bit value source
 * (FusedKV-Lite: K^n and V^1); otherwise as fkv_kivi_decode. */
fkv_status fkv_kivi_lite_decode(const fkv_params* params, const void* q,
                                fkv_q4_cache k_src, fkv_q4_cache v_src,
                                const int32_t* seqlens_k, void* out,
                                float* lse, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * ---- Backward pass (training through the fusion) ----
 * [Deck] frame "FusedKV learns two-source, channel-wise fusion" (Eqs.
 * (4)-(5)): the fusion vectors are learned with the model, end to end, so a
 * training step needs the gradients of a reconstruction layer's attention
 * with respect to its queries, the four source caches and the four vectors.
 * For a loss with output gradient dO (the LSE output is not differentiated),
 * with Kf = a*K1 + a'*Kn, Vf = b*V1 + b'*Vn and P the softmax probabilities:
 *   dVf = sum_h P^T dO, dS = P * (dO Vf^T - rowsum(dO * O)),
 *   dQ = scale dS Kf, dKf = scale sum_h dS^T Q,
 *   dK1 = a*dKf, dKn = a'*dKf, dV1 = b*dVf, dVn = b'*dVf,
 *   da[g, d] = sum over batch rows and tokens of dKf * K1 (a': Kn; b: dVf *
 *   V1; b': dVf * Vn) -- per channel; a RoPE-tied parameter's gradient is
 *   the sum over its channel pair.
 * The sum over h runs over the G query heads of KV head g.
 */

/* A writable [B, S, H_kv, D] gradient view: element strides for b, s, h;
 * channel stride 1; base and rows 16-byte aligned. */
typedef struct {
    void* data;
    int64_t stride_b, stride_s, stride_h;
} fkv_grad;

/* Gradients of the fusion vectors, device float32 [H_kv, D] each,
 * overwritten (not accumulated) by each call. */
typedef struct {
    float* k_w1;
    float* k_wn;
    float* v_w1;
    float* v_wn;
} fkv_fusion_grad;

/* Workspace bytes for fkv_prefill_backward / fkv_lite_prefill_backward with
 * these params (0 when the params are invalid or empty): per-row softmax
 * statistics (2 x B*H_q*S_q float32) and the weight-gradient partials
 * (B*H_kv*ceil(S/128) x 4 x D float32), each part 256-byte aligned.  The
 * fused keys and values are rebuilt tile by tile inside the kernels and
 * never stored. */
size_t fkv_backward_workspace_size(const fkv_params* params);

/*
 * fkv_prefill_backward -- gradients of fkv_prefill for one layer: seqlen_q ==
 * seqlen_k, bfloat16 data, G in {1, 2, 4, 8}, causal 0 or 1.  Recomputes the
 * probabilities from the forward LSE; matrix-core operands are bfloat16
 * (fused tiles, probabilities and dS rounded once from float32), all
 * accumulation float32; the key-gradient pass forms dS from the
 * probabilities rounded to binary16, which holds them because P <= 1 when
 * lse is the forward's row log-sum-exp (another lse voids the results).
 * Outputs are overwritten, not accumulated.  Every result is run-to-run
 * deterministic (no float atomics).
 *
 *   q, out, dout  device [B, S, H_q, D] bfloat16 (out: the forward output)
 *   lse           device float32 [B, H_q, S] (the forward LSE, natural log)
 *   dq            device [B, S, H_q, D] bfloat16
 *   dk1 .. dvn    gradient views of K^1, K^n, V^1, V^n (bfloat16)
 *   dfusion       device float32 gradients of (a, a', b, b')
 *   workspace     >= fkv_backward_workspace_size bytes, 256-byte aligned,
 *                 contents ignored
 * Errors as fkv_prefill; FKV_ERROR_WORKSPACE for a short workspace.
 */
fkv_status fkv_prefill_backward(const fkv_params* params, const void* q,
                                fkv_cache k1, fkv_cache kn, fkv_cache v1,
                                fkv_cache vn, const fkv_fusion* fusion,
                                const void* out, const float* lse,
                                const void* dout, void* dq, fkv_grad dk1,
                                fkv_grad dkn, fkv_grad dv1, fkv_grad dvn,
                                const fkv_fusion_grad* dfusion,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * fkv_lite_prefill_backward -- gradients of fkv_lite_prefill: one key and one
 * value source (FusedKV-Lite with (K^n, V^1), [Deck] frame "Lite separates
 * the key source from the value source", Eq. (6); or the plain control), so
 * dk and dv are the gradients of k_src and v_src.  Otherwise as
 * fkv_prefill_backward.
 */
fkv_status fkv_lite_prefill_backward(const fkv_params* params, const void* q,
                                     fkv_cache k_src, fkv_cache v_src,
                                     const void* out, const float* lse,
                                     const void* dout, void* dq, fkv_grad dk,
                                     fkv_grad dv, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * ---- Storage layers ----
 * fkv_store_kv -- write one storage layer's new keys and values into its
 * caches.  In the FusedKV schedule the lower layers 1..n run a full prefill
 * and keep their caches, which the upper layers then read: for the first
 * token an upper layer needs only the last prompt position, one decode over
 * the caches of layer 1 and layer n ([Deck] backup frame "Prefill skipping
 * has a specific scope"; [Notes] section 2.5).  This call is that cache
 * write, run before the layer's attention (fkv_lite_prefill over the written
 * caches, or a decode step's append).
 *
 *   params   batch, seqlen_q = S_new (tokens written), seqlen_k = the
 *            caches' token capacity, num_kv_heads, head_dim and dtype are
 *            used (num_q_heads must still be a valid multiple)
 *   pos0     first cache position written; pos0 + S_new <= seqlen_k
 *   k_new, v_new      [B, S_new, H_kv, D] views (fkv_cache rules), e.g. the
 *                     token-major output of the key/value projection, keys
 *                     already rotated (the caches hold post-RoPE keys)
 *   k_cache, v_cache  writable [B, seqlen_k, H_kv, D] views (fkv_grad rules)
 * Cache positions pos0 .. pos0+S_new-1 receive the new rows bit for bit;
 * every other position is left as it was.  The new rows and the caches must
 * not overlap.  Errors as fkv_decode.  Asynchronous on `stream`.
 */
fkv_status fkv_store_kv(const fkv_params* params, int32_t pos0,
                        fkv_cache k_new, fkv_cache v_new, fkv_grad k_cache,
                        fkv_grad v_cache, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FUSEDKV_H_ */
