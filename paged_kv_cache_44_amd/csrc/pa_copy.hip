// pa_copy.hip — whole-block copies inside device memory (copy-on-write of a
// shared block: "Efficient Memory Management for Large Language Model
// Serving with PagedAttention", sampling and prefix paragraphs; "Continuous
// Batching and PagedAttention", section "Sharing, the part that goes beyond
// fixing what broke").
//
// One workgroup per (pair, layer, K|V) slab of heads x slots x dim bytes,
// moved with 16-byte loads and stores. Pairs naming a block outside either
// pool are skipped.
//
// A second kernel takes its pairs in the launch arguments, so it can serve
// host-side pair lists:
//  * swap by kernel: blocks move between device memory and pinned host
//    memory mapped into the device's address space ("When KV Capacity Runs
//    Out", section "Restore KV stored outside the GPU"; "41 · Preemption,
//    Recomputation & KV Pressure", section 3). One launch covers every block
//    and layer, so the per-transfer cost of the DMA engines, which dominates
//    for the small slabs of small blocks, is paid once. Its host-link
//    traffic shares the memory path of every other kernel, though, so
//    memory-bound kernels beside it on other streams stall until it ends.
//  * staged swap: scattered device blocks are gathered into (or scattered
//    from) a contiguous device staging buffer, so the DMA engines move a few
//    large ranges instead of one small transfer per block and layer.
// A fixed grid walks the (pair, layer, K|V) slabs: 64 workgroups keep the
// host link saturated (fewer than 16 fall behind); device-to-device staging
// uses more.

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

__global__ void __launch_bounds__(256)
arg_copy_kernel(const ArgCopyParams a) {
  const int units = a.num_pairs * 2 * a.num_layers;
  const int64_t n = a.slab_bytes / 16;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int pair = u / (2 * a.num_layers);
    const int r = u - pair * 2 * a.num_layers;
    const int layer = r >> 1;
    const bool is_v = r & 1;
    const int64_t s = a.pairs[2 * pair];
    const int64_t d = a.pairs[2 * pair + 1];
    const uint4* src = reinterpret_cast<const uint4*>(
        (is_v ? a.src_v : a.src_k) + s * a.src_block_bytes + layer * a.src_layer_bytes);
    uint4* dst = reinterpret_cast<uint4*>(
        (is_v ? a.dst_v : a.dst_k) + d * a.dst_block_bytes + layer * a.dst_layer_bytes);
    // four 16-byte loads in flight per thread before their stores
    int64_t i = threadIdx.x;
    for (; i + 3 * 256 < n; i += 4 * 256) {
      const uint4 x0 = src[i], x1 = src[i + 256], x2 = src[i + 512], x3 = src[i + 768];
      dst[i] = x0;
      dst[i + 256] = x1;
      dst[i + 512] = x2;
      dst[i + 768] = x3;
    }
    for (; i < n; i += 256) dst[i] = src[i];
  }
}

hipError_t launch_arg_copy(const ArgCopyParams& a, hipStream_t st) {
  if (a.num_pairs == 0) return hipSuccess;
  const int units = a.num_pairs * 2 * a.num_layers;
  const int grid = units < a.max_wgs ? units : a.max_wgs;
  hipLaunchKernelGGL(arg_copy_kernel, dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_copy(const CopyParams& a, hipStream_t st) {
  if (a.num_pairs == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_kernel, dim3(a.num_pairs, 2 * a.num_layers), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace pa
