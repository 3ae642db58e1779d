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

// I is the index type: 32-bit when every vector index fits, which keeps the
// division by the row count short.
template <typename I>
__global__ __launch_bounds__(256) void kv_append_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    const int64_t* __restrict__ slot_mapping, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, I total_vecs, int h_kv, int vec_per_row, int64_t n_slots) {
  const I gid = (I)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total_vecs) return;
  const I per_token = (I)h_kv * vec_per_row;
  const I tok = gid / per_token;
  const int rem = (int)(gid - tok * per_token);
  const int head = rem / vec_per_row;
  const int c = rem - head * vec_per_row;
  // The rows are requested together with the slot, so that the copy waits for
  // one memory round trip, not two (the empty asm keeps all three loads above
  // the slot test).
  int64_t slot = slot_mapping[tok];
  uint4 kv = k_new[gid];
  uint4 vv = v_new[gid];
  asm volatile("" : "+v"(slot), "+v"(kv.x), "+v"(kv.y), "+v"(kv.z), "+v"(kv.w), "+v"(vv.x),
               "+v"(vv.y), "+v"(vv.z), "+v"(vv.w));
  if (slot < 0 || slot >= n_slots) return;  // padding, or out of range: no write
  const int64_t blk = slot >> 4;
  const int off = (int)(slot & 15);
  const int64_t dst = ((blk * h_kv + head) * kBlock + off) * vec_per_row + c;
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
  const int64_t n_slots = (int64_t)n_blocks * kBlock;
  if (total + threads <= INT32_MAX)
    hipLaunchKernelGGL(kv_append_kernel<uint32_t>, dim3((unsigned)grid), dim3(threads), 0,
                       stream, (const uint4*)k_new, (const uint4*)v_new, slot_mapping,
                       (uint4*)k_cache, (uint4*)v_cache, (uint32_t)total, h_kv, vec_per_row,
                       n_slots);
  else
    hipLaunchKernelGGL(kv_append_kernel<int64_t>, dim3((unsigned)grid), dim3(threads), 0,
                       stream, (const uint4*)k_new, (const uint4*)v_new, slot_mapping,
                       (uint4*)k_cache, (uint4*)v_cache, total, h_kv, vec_per_row, n_slots);
  return hipGetLastError();
}

}  // namespace pkv
