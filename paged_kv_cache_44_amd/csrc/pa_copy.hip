// pa_copy.hip — whole-block copies inside device memory (copy-on-write of a
// shared block: "Efficient Memory Management for Large Language Model
// Serving with PagedAttention", sampling and prefix paragraphs; "Continuous
// Batching and PagedAttention", section "Sharing, the part that goes beyond
// fixing what broke").
//
// One workgroup per (pair, layer, K|V) slab of heads x slots x dim bytes,
// moved with 16-byte loads and stores. Pairs naming a block outside either
// pool are skipped.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

__global__ void __launch_bounds__(256)
copy_kernel(const CopyParams a) {
  const int pair = blockIdx.x;
  const int layer = blockIdx.y >> 1;
  const bool is_v = blockIdx.y & 1;
  const int64_t s = a.pairs[2 * pair];
  const int64_t d = a.pairs[2 * pair + 1];
  if (s < 0 || s >= a.src_num_blocks || d < 0 || d >= a.dst_num_blocks) return;
  const uint4* src = reinterpret_cast<const uint4*>(
      (is_v ? a.src_v : a.src_k) + s * a.src_block_bytes + layer * a.src_layer_bytes);
  uint4* dst = reinterpret_cast<uint4*>(
      (is_v ? a.dst_v : a.dst_k) + d * a.dst_block_bytes + layer * a.dst_layer_bytes);
  const int64_t n = a.slab_bytes / 16;
  for (int64_t i = threadIdx.x; i < n; i += 256) dst[i] = src[i];
}

hipError_t launch_copy(const CopyParams& a, hipStream_t st) {
  if (a.num_pairs == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_kernel, dim3(a.num_pairs, 2 * a.num_layers), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace pa
