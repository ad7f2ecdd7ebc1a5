// fkv_store.hip -- the storage-layer cache write: a layer's new keys and
// values copied, bit for bit, into its KV caches at positions pos0 ...
//
// Pages cited (by title):
//   [Deck]  "FusedKV: Reconstructing KV Caches with Cross-Layer Fusion",
//           backup frame "Prefill skipping has a specific scope": the lower
//           (storage) layers run a full prefill and keep their caches; the
//           upper layers then need only the last prompt position, reading
//           the caches of layer 1 and layer n.
//   [Notes] "FusedKV:通过跨层融合重构 KV 缓存", section 2.5.
//
// The copy is HBM-bound: 2 x (B * S_new * H_kv * D * elt) bytes read and as
// many written.  One thread moves one 16-byte chunk; the thread index runs
// over (tensor, b, h, s, chunk) with the chunk fastest, so consecutive
// lanes write consecutive bytes of a head-major cache row run.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fkv_internal.h"

namespace fkv {
namespace {

constexpr int kStoreThreads = 256;

__global__ __launch_bounds__(kStoreThreads) void store_kv_kernel(const StoreArgs a)
{
    const int cpr = a.D * a.elt / 16;  // 16-byte chunks per row
    const int epc = 16 / a.elt;        // elements per chunk
    const int64_t per = (int64_t)a.B * a.H * a.S_new * cpr;
    const int64_t stride = (int64_t)gridDim.x * kStoreThreads;
    for (int64_t i = (int64_t)blockIdx.x * kStoreThreads + threadIdx.x; i < 2 * per; i += stride) {
        const bool val = i >= per;
        int64_t j = val ? i - per : i;
        const int c = (int)(j % cpr);
        j /= cpr;
        const int s = (int)(j % a.S_new);
        j /= a.S_new;
        const int h = (int)(j % a.H);
        const int b = (int)(j / a.H);
        const View& src = val ? a.v_new : a.k_new;
        const OutView& dst = val ? a.v_cache : a.k_cache;
        const char* ps = static_cast<const char*>(src.data) +
                         ((int64_t)b * src.sb + (int64_t)s * src.ss + (int64_t)h * src.sh + (int64_t)c * epc) * a.elt;
        char* pd = static_cast<char*>(dst.data) +
                   ((int64_t)b * dst.sb + (int64_t)(a.pos0 + s) * dst.ss + (int64_t)h * dst.sh + (int64_t)c * epc) * a.elt;
        *reinterpret_cast<uint4*>(pd) = *reinterpret_cast<const uint4*>(ps);
    }
}

}  // namespace

int launch_store_kv(const StoreArgs& a, void* stream)
{
    const int64_t items = 2 * (int64_t)a.B * a.H * a.S_new * (a.D * a.elt / 16);
    if (items == 0) return 0;
    int64_t blocks = (items + kStoreThreads - 1) / kStoreThreads;
    if (blocks > 16384) blocks = 16384;  // grid-stride beyond 64 waves per CU
    hipLaunchKernelGGL(store_kv_kernel, dim3((unsigned)blocks), dim3(kStoreThreads), 0,
                       static_cast<hipStream_t>(stream), a);
    return (int)hipGetLastError();
}

}  // namespace fkv
