// Device pieces shared by the bf16 and INT8 prefill kernels (gfx950): tile
// geometry and swizzle, the untracked global-to-LDS copy and its waits, the
// fence-free barrier, and the longest-context-first order of sequence planes.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace pkv {

constexpr int kPfWaves = 4;
constexpr int kPfRows = 32 * kPfWaves;  // packed rows per workgroup
constexpr int kPfTile = 64;             // keys per tile
constexpr float kPfNegInf = -__builtin_huge_valf();
constexpr float kPfSlack = 8.0f;  // log2 units

#define PKV_LDS __attribute__((address_space(3)))
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

template <int D>
struct PfTile {
  static constexpr int kChunks = D / 8;              // 16-byte chunks per key row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kMatBytes = kPfTile * kRowBytes;  // K (or V) of one tile
  static constexpr int kBufBytes = 2 * kMatBytes;
  static constexpr int kRowsPerCopy = 1024 / kRowBytes;   // rows one wave-wide copy fills
  static constexpr int kCopiesPerBlock = kBlock / kRowsPerCopy;
  // Chunk swizzle: a permutation of the row's low bits into the chunk index.
  __device__ static int swz(int r) {
    if constexpr (D == 64)
      return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    else
      return ((r & 3) << 2) | ((r >> 2) & 3);
  }
  __device__ static int offset(int r, int chunk) { return r * kRowBytes + ((chunk ^ swz(r)) << 4); }
};

// Accumulator element r of a 32x32 MFMA result in lane (col, half) is row
// 8 * (r / 4) + 4 * half + r % 4.
__device__ __forceinline__ int mfma32_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

// One wave-wide 16-byte-per-lane copy from global memory straight into LDS:
// lane l's 16 bytes land at lds_addr + 16 * l.  Issued as inline assembly so
// that the compiler does not track it: it would otherwise wait for every copy
// in flight before any LDS read it cannot prove disjoint.  Completion is
// handled explicitly (wait_vm + tile_barrier).  Compiler-generated vmcnt waits
// stay correct, only stricter, because loads retire in order.
__device__ __forceinline__ void copy_to_lds(const void* src, const void* lds_dst) {
  // The destination is the same for every lane (m0): make it a scalar even
  // where the compiler computed it in vector registers.
  const unsigned lds_addr =
      __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(const PKV_LDS unsigned char*)lds_dst);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_addr)
               : "memory");
}

// The same copy with the source given as a wave-uniform base (a scalar
// register pair) plus this lane's 32-bit byte offset, so that no 64-bit
// vector address arithmetic is needed per copy.
__device__ __forceinline__ void copy_to_lds_off(const void* base, uint32_t off,
                                                const void* lds_dst) {
  const unsigned lds_addr =
      __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(const PKV_LDS unsigned char*)lds_dst);
  // readfirstlane returns int: each half goes through uint32_t so that the
  // low word is not sign-extended into the high one.
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)b);
  const uint64_t sb = ((uint64_t)hi << 32) | lo;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(sb),
               "s"(lds_addr)
               : "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  // vmcnt is 6 bits: the low 4 in bits 3:0, the high 2 in bits 15:14.
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// s_waitcnt lgkmcnt(0): this wave's LDS stores are done.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier without a memory fence: the tiles are published by the
// explicit waits above each call, and nothing else is shared, so the fence of
// __syncthreads (which would also wait for the tiles still in flight) is not
// needed.  The empty asm statements keep the compiler from moving LDS accesses
// across the barrier.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The sequence of grid plane z when the planes are taken longest context first
// (ties: lower index), for grids larger than the chip holds at once: the
// longest key walks then start in the first round instead of whenever their
// plane comes up (longest-processing-time order).  Each lane holds the lengths
// of sequences lane, lane + 64, ... (a.S <= kLptMaxSeqs) and ranks its own
// against all of them; every wave computes the same answer.
constexpr int kLptMaxSeqs = 256;
__device__ __forceinline__ int longest_first_sequence(const PrefillArgs& a, int z) {
  constexpr int kC = kLptMaxSeqs / 64;
  const int lane = threadIdx.x & 63;
  const int cap = a.max_blocks_per_seq * kBlock;
  int len[kC];
#pragma unroll
  for (int c = 0; c < kC; ++c) {
    const int j = c * 64 + lane;
    len[c] = j < a.S ? max(0, min(a.context_lens[j], cap)) : -1;
  }
  int found = z;
#pragma unroll
  for (int c = 0; c < kC; ++c) {
    if (c * 64 >= a.S) break;
    const int j = c * 64 + lane;
    int rank = 0;
#pragma unroll
    for (int ci = 0; ci < kC; ++ci) {
      if (ci * 64 >= a.S) break;
      const int n = min(64, a.S - ci * 64);
      for (int t = 0; t < n; ++t) {
        const int li = __builtin_amdgcn_readlane(len[ci], t);
        rank += (li > len[c]) || (li == len[c] && ci * 64 + t < j);
      }
    }
    const uint64_t hit = __ballot(j < a.S && rank == z);
    if (hit) {
      found = c * 64 + __builtin_ctzll(hit);
      break;
    }
  }
  return __builtin_amdgcn_readfirstlane(found);
}

}  // namespace pkv
