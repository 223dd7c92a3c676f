// Cache write: place each new token's K and V rows into their cache slots.
//
// Slot s of KV head g is row (g * num_blocks * 16 + s) of the head-major cache
// viewed as [kv_heads * num_blocks * 16, head_dim] -- one index over the
// (block, offset) slots of a head, as in "From 183 ms to 19 ms per decode
// step", "Four changes", changes 2 and 4.  One thread moves one 16-byte chunk
// of a row for both K and V; consecutive threads cover consecutive chunks of a
// row, so reads and writes are coalesced per row.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(CacheArgs a) {
  const int chunks = a.row_bytes / 16;
  const int total = a.num_tokens * a.kv_heads * chunks;  // < 2^31, checked by the host
  const int stride = gridDim.x * blockDim.x;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int ch = i % chunks;
    const int rest = i / chunks;
    const int g = rest % a.kv_heads;
    const int tok = rest / a.kv_heads;
    // The slot and the data are loaded together (one memory round trip).
    const size_t src = (size_t(tok) * a.kv_heads + g) * a.row_bytes + size_t(ch) * 16;
    const u32x4 k = load16(reinterpret_cast<const char*>(a.key) + src);
    const u32x4 v = load16(reinterpret_cast<const char*>(a.value) + src);
    const int64_t slot = a.slot_mapping[tok];
    if (slot < 0 || slot >= int64_t(a.num_blocks) * kBlockSize) continue;
    const size_t dst = (size_t(g) * a.num_blocks * kBlockSize + size_t(slot)) * a.row_bytes +
                       size_t(ch) * 16;
    *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(a.k_cache) + dst) = k;
    *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(a.v_cache) + dst) = v;
  }
}

}  // namespace

hipError_t launch_reshape_and_cache(const CacheArgs& a, hipStream_t stream) {
  const long total = long(a.num_tokens) * a.kv_heads * (a.row_bytes / 16);
  if (total == 0) return hipSuccess;
  const long want = (total + 255) / 256;
  const int blocks = int(want < 8192 ? want : 8192);
  reshape_and_cache_kernel<<<blocks, 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace pa
