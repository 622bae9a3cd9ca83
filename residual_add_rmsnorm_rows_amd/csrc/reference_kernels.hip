// Measurement references launched through the same path as the normalization
// kernels: a kernel that does nothing (bare launch latency) and a plain
// streaming copy (the practical bandwidth ceiling for a stream that reads and
// writes the same number of bytes).
#include <hip/hip_runtime.h>

#include "device_common.h"

namespace rn {
namespace {
__global__ __launch_bounds__(64) void empty_kernel() {}

// Each workgroup copies one contiguous tile of kCopyThreads * 16 bytes: one
// nontemporal 16-byte load and store per lane, through a buffer resource sized
// to the tile so that a short last tile reads and writes nothing past the end.
__global__ __launch_bounds__(kCopyThreads) void copy_kernel(const char* src, char* dst, int64_t bytes) {
  constexpr int64_t kTile = static_cast<int64_t>(kCopyThreads) * 16;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kTile;
  const int64_t left = bytes - base;
  const uint32_t n = static_cast<uint32_t>(left < kTile ? left : kTile);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + base, n);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(dst + base, n);
  uint32_t v[4];
  buffer_load_words<16, true>(rs, threadIdx.x * 16u, v);
  buffer_store_words<16>(rd, threadIdx.x * 16u, v);
}
}  // namespace

const void* empty_kernel_address() { return reinterpret_cast<const void*>(&empty_kernel); }
const void* copy_kernel_address() { return reinterpret_cast<const void*>(&copy_kernel); }

}  // namespace rn
