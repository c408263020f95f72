// Cache append on gfx950: copy the index key and latent row of each new token
// into the preallocated caches at the sequence's next positions (HF model doc
// "DeepSeek-V3.2", section "DeepSeek Sparse Attention (DSA)": the index-key
// cache sits next to the MLA cache and grows with the tokens processed).
// One work-group per (sequence, new token); 16-byte copies when both rows are
// 16-byte aligned, 4-byte copies otherwise.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

__device__ __forceinline__ void copy_row(uint8_t* dst, const uint8_t* src, int bytes) {
  if ((((uintptr_t)dst | (uintptr_t)src | (uintptr_t)bytes) & 15u) == 0) {
    for (int o = threadIdx.x * 16; o < bytes; o += blockDim.x * 16) st16(dst + o, ld16(src + o));
  } else {
    for (int o = threadIdx.x * 4; o < bytes; o += blockDim.x * 4)
      *reinterpret_cast<uint32_t*>(dst + o) = *reinterpret_cast<const uint32_t*>(src + o);
  }
}

__global__ __launch_bounds__(128) void cache_append_kernel(CacheAppend c) {
  const int t = blockIdx.x, b = blockIdx.y;
  const int64_t src_row = (int64_t)b * c.n_new + t;
  const int64_t dst_row = (int64_t)b * c.cap + c.pos + t;
  copy_row(static_cast<uint8_t*>(c.k) + dst_row * c.k_row_bytes,
           static_cast<const uint8_t*>(c.k_new) + src_row * c.k_row_bytes, c.k_row_bytes);
  copy_row(static_cast<uint8_t*>(c.kv) + dst_row * c.kv_row_bytes,
           static_cast<const uint8_t*>(c.kv_new) + src_row * c.kv_row_bytes, c.kv_row_bytes);
  if (c.ks && threadIdx.x == 0) c.ks[dst_row] = c.ks_new[src_row];
}

}  // namespace

hipError_t launch_cache_append(const CacheAppend& c, hipStream_t s) {
  hipLaunchKernelGGL(cache_append_kernel, dim3(c.n_new, c.B), dim3(128), 0, s, c);
  return hipGetLastError();
}

}  // namespace dsa
