// kv_append: scatter the K/V rows of new tokens into their 16-token pool slots.
//
// The cache is pre-allocated and written in place at each token's slot instead
// of being re-concatenated (LLM Inference Server page, Stage 1 "KV-Cache
// Engine", pre-allocation task); slots address fixed 16-token physical blocks
// (same page, Paged KV-Cache Block Allocator stretch challenge).
//
// One lane moves one 16-byte vector of K and the matching vector of V.  Reads
// of k_new/v_new are fully coalesced; each (token, head) row of d_h elements is
// written as a contiguous run of d_h * elem / 16 lanes, so the scatter keeps
// whole 64- or 128-byte segments per row.
#include "device_common.h"
#include "launch.h"

namespace pkv {

__global__ __launch_bounds__(256) void kv_append_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    const int64_t* __restrict__ slot_mapping, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, int64_t total_vecs, int h_kv, int vec_per_row,
    int64_t n_slots) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total_vecs) return;
  const int64_t per_token = (int64_t)h_kv * vec_per_row;
  const int64_t tok = gid / per_token;
  const int rem = (int)(gid - tok * per_token);
  const int head = rem / vec_per_row;
  const int c = rem - head * vec_per_row;
  const int64_t slot = slot_mapping[tok];
  if (slot < 0 || slot >= n_slots) return;  // padding, or out of range: no write
  const int64_t blk = slot >> 4;
  const int off = (int)(slot & 15);
  const int64_t dst = ((blk * h_kv + head) * kBlock + off) * vec_per_row + c;
  const uint4 kv = k_new[gid];
  const uint4 vv = v_new[gid];
  k_cache[dst] = kv;
  v_cache[dst] = vv;
}

hipError_t launch_kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                            void* k_cache, void* v_cache, int T, int h_kv, int d_h,
                            int n_blocks, int elem_bytes, hipStream_t stream) {
  const int vec_per_row = d_h * elem_bytes / 16;
  const int64_t total = (int64_t)T * h_kv * vec_per_row;
  const int threads = 256;
  const int64_t grid = (total + threads - 1) / threads;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)grid), dim3(threads), 0, stream,
                     (const uint4*)k_new, (const uint4*)v_new, slot_mapping, (uint4*)k_cache,
                     (uint4*)v_cache, total, h_kv, vec_per_row, (int64_t)n_blocks * kBlock);
  return hipGetLastError();
}

}  // namespace pkv
