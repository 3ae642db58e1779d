// copy_blocks / swap_blocks: whole physical blocks copied between pools.
//
// Within one pool set this is the copy that a shared, partly filled block needs
// before one of its sequences writes into it (the prefix cache of the LLM
// Inference Server page, Stage 1: sequences with the same system prompt share
// its blocks).  Between a device pool set and a pinned host pool set it moves a
// preempted sequence's blocks out of HBM and back (the scheduler's preemption
// in the pipeline figure of the From Scratch page, How it works).
//
// A pool is any array whose leading axis is the physical block; block b of pool
// i is bytes [b * block_bytes[i], (b + 1) * block_bytes[i]).  One workgroup
// moves one 32 KiB slice of one block of one pool: each lane issues its eight
// 16-byte loads before any store, so a wave keeps 8 KiB in flight, and the
// slices of a block are coalesced runs.  Host pools are reached through their
// device mapping (pinned memory), so a swap is one launch over PCIe whatever
// the number of blocks, not one DMA request per block.
#include "device_common.h"
#include "launch.h"

namespace pkv {

// Every byte is read once and written once.  Between device pools both go with
// the non-temporal hint: measured on 1024 decode-shaped blocks, it halves the
// copy time (49 -> 24 us, 5.6 TB/s read + write).  Through pinned host memory
// the hint costs PCIe rate (swap of 32 MiB: 53 -> 49 GB/s), so swaps use plain
// accesses.
template <bool NT>
__device__ __forceinline__ uint4 copy_load(const uint4* p) {
  if constexpr (NT) {
    const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(x.x, x.y, x.z, x.w);
  } else {
    return *p;
  }
}
template <bool NT>
__device__ __forceinline__ void copy_store(uint4* p, const uint4& v) {
  if constexpr (NT) {
    const u32x4_t x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4_t*>(p));
  } else {
    *p = v;
  }
}

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 8;
constexpr int kCopySliceVecs = kCopyThreads * kCopyUnroll;  // 2048 vectors = 32 KiB

template <bool NT>
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    CopyPools p, const int32_t* __restrict__ pairs, int n_src_blocks, int n_dst_blocks) {
  const int pool = blockIdx.y;
  const int64_t vecs = p.vecs[pool];
  const int64_t first = (int64_t)blockIdx.z * kCopySliceVecs;
  if (first >= vecs) return;
  const int32_t src = pairs[2 * (int64_t)blockIdx.x];
  const int32_t dst = pairs[2 * (int64_t)blockIdx.x + 1];
  if (src < 0 || src >= n_src_blocks || dst < 0 || dst >= n_dst_blocks) return;
  const uint4* __restrict__ s = p.src[pool] + (int64_t)src * vecs + first;
  uint4* __restrict__ d = p.dst[pool] + (int64_t)dst * vecs + first;
  const int64_t n = vecs - first < kCopySliceVecs ? vecs - first : kCopySliceVecs;
  uint4 r[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = (int64_t)u * kCopyThreads + threadIdx.x;
    if (i < n) r[u] = copy_load<NT>(s + i);
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = (int64_t)u * kCopyThreads + threadIdx.x;
    if (i < n) copy_store<NT>(d + i, r[u]);
  }
}

hipError_t launch_copy_blocks(const CopyPools& p, int n_pools, const int32_t* pairs, int n_pairs,
                              int n_src_blocks, int n_dst_blocks, bool device_only,
                              hipStream_t stream) {
  int64_t most = 0;
  for (int i = 0; i < n_pools; ++i) most = p.vecs[i] > most ? p.vecs[i] : most;
  const int64_t slices = (most + kCopySliceVecs - 1) / kCopySliceVecs;
  if (n_pairs <= 0 || n_pools <= 0 || slices <= 0) return hipSuccess;
  if (slices > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)n_pairs, (unsigned)n_pools, (unsigned)slices);
  if (device_only)
    hipLaunchKernelGGL(copy_blocks_kernel<true>, grid, dim3(kCopyThreads), 0, stream, p, pairs,
                       n_src_blocks, n_dst_blocks);
  else
    hipLaunchKernelGGL(copy_blocks_kernel<false>, grid, dim3(kCopyThreads), 0, stream, p, pairs,
                       n_src_blocks, n_dst_blocks);
  return hipGetLastError();
}

}  // namespace pkv
