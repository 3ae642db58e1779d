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

namespace pkv {

// INT8 cache: each new (token, KV head) row is quantised on the way in, with
// the symmetric absmax rule of the LLM Inference Server page ("Required
// Mathematical Concepts"; "INT8 KV-Cache Quantization" stretch challenge, per
// token head): s = max(max|x|, 1e-8) / 127 and x_q = round(x / s), in float32,
// a true division and rounding half to even, as in the page's reference INT8
// layer.  The codes land where the bf16 row would, the scale in a float32
// pool [n_blocks, h_kv, 16].
//
// L = d_h / 8 adjacent lanes cover one row (8 values each), so a wave holds
// 64 / L rows; the row maximum is reduced across those lanes.
template <typename Src, int D>
__global__ __launch_bounds__(256) void kv_append_i8_kernel(
    const Src* __restrict__ k_new, const Src* __restrict__ v_new,
    const int64_t* __restrict__ slot_mapping, uint2* __restrict__ k_cache,
    uint2* __restrict__ v_cache, float* __restrict__ k_scale, float* __restrict__ v_scale,
    int rows, int h_kv, int64_t n_slots) {
  constexpr int L = D / 8;
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  const int row = gid / L;  // token * h_kv + head
  const int part = gid % L;
  const bool live = row < rows;
  const int r = live ? row : rows - 1;  // lanes past the end mirror the last row, write nothing
  const int tok = r / h_kv;
  const int head = r - tok * h_kv;
  float k[8], v[8];
  if constexpr (sizeof(Src) == 2) {
    const uint4 kw = reinterpret_cast<const uint4*>(k_new)[(size_t)r * L + part];
    const uint4 vw = reinterpret_cast<const uint4*>(v_new)[(size_t)r * L + part];
    const uint32_t kk[4] = {kw.x, kw.y, kw.z, kw.w}, vv[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      k[2 * i] = __uint_as_float(kk[i] << 16);
      k[2 * i + 1] = __uint_as_float(kk[i] & 0xffff0000u);
      v[2 * i] = __uint_as_float(vv[i] << 16);
      v[2 * i + 1] = __uint_as_float(vv[i] & 0xffff0000u);
    }
  } else {
    const float4* kp = reinterpret_cast<const float4*>(k_new) + ((size_t)r * L + part) * 2;
    const float4* vp = reinterpret_cast<const float4*>(v_new) + ((size_t)r * L + part) * 2;
    const float4 k0 = kp[0], k1 = kp[1], v0 = vp[0], v1 = vp[1];
    const float kk[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
    const float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      k[i] = kk[i];
      v[i] = vv[i];
    }
  }
  float km = 0.f, vm = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    km = fmaxf(km, fabsf(k[i]));
    vm = fmaxf(vm, fabsf(v[i]));
  }
#pragma unroll
  for (int o = 1; o < L; o <<= 1) {  // L adjacent lanes, aligned to L
    km = fmaxf(km, __shfl_xor(km, o));
    vm = fmaxf(vm, __shfl_xor(vm, o));
  }
  const float ks = fmaxf(km, 1e-8f) / 127.0f;
  const float vs = fmaxf(vm, 1e-8f) / 127.0f;
  uint32_t kc[2] = {0u, 0u}, vc[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int kq = (int)rintf(k[i] / ks);
    const int vq = (int)rintf(v[i] / vs);
    kc[i / 4] |= ((uint32_t)kq & 0xffu) << (8 * (i % 4));
    vc[i / 4] |= ((uint32_t)vq & 0xffu) << (8 * (i % 4));
  }
  if (!live) return;
  const int64_t slot = slot_mapping[tok];
  if (slot < 0 || slot >= n_slots) return;  // padding, or out of range: no write
  const int64_t blk = slot >> 4;
  const int off = (int)(slot & 15);
  const int64_t rh = (blk * h_kv + head) * kBlock + off;  // (block, head, slot) row
  k_cache[rh * L + part] = make_uint2(kc[0], kc[1]);
  v_cache[rh * L + part] = make_uint2(vc[0], vc[1]);
  if (part == 0) {
    k_scale[rh] = ks;
    v_scale[rh] = vs;
  }
}

hipError_t launch_kv_append_i8(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                               int8_t* k_cache, int8_t* v_cache, float* k_scale, float* v_scale,
                               int T, int h_kv, int d_h, int n_blocks, int src_bytes,
                               hipStream_t stream) {
  const int rows = T * h_kv;
  const int threads = 256;
  const int64_t lanes = (int64_t)rows * (d_h / 8);
  const unsigned grid = (unsigned)((lanes + threads - 1) / threads);
  const int64_t n_slots = (int64_t)n_blocks * kBlock;
  auto go = [&](auto kern, const auto* kn, const auto* vn) {
    hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, stream, kn, vn, slot_mapping,
                       (uint2*)k_cache, (uint2*)v_cache, k_scale, v_scale, rows, h_kv, n_slots);
  };
  if (src_bytes == 2) {
    const bf16_t* kn = (const bf16_t*)k_new;
    const bf16_t* vn = (const bf16_t*)v_new;
    if (d_h == 64) go(kv_append_i8_kernel<bf16_t, 64>, kn, vn);
    else go(kv_append_i8_kernel<bf16_t, 128>, kn, vn);
  } else {
    const float* kn = (const float*)k_new;
    const float* vn = (const float*)v_new;
    if (d_h == 64) go(kv_append_i8_kernel<float, 64>, kn, vn);
    else go(kv_append_i8_kernel<float, 128>, kn, vn);
  }
  return hipGetLastError();
}

}  // namespace pkv
