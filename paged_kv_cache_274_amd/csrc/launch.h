// Host-side launchers of the libpkv kernels (internal; the public C ABI is pkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Query heads handled together by one decode wavefront: the GQA group of a KV
// head is split into n_chunks chunks of at most max_chunk heads, so the per-lane
// accumulators stay in registers (fp32 with d_h = 128 holds twice as many
// accumulator words per head, so its chunks are half as large).
struct HeadChunks {
  int n_chunks;
  int per_chunk;
};
inline int max_chunk(int d_h, bool bf16) { return (!bf16 && d_h == 128) ? 4 : 8; }
inline HeadChunks chunks_of(int g, int cap) {
  HeadChunks c;
  c.n_chunks = (g + cap - 1) / cap;
  c.per_chunk = (g + c.n_chunks - 1) / c.n_chunks;
  return c;
}

// Small batches: chunks of more than 4 heads leave one wave per SIMD, and with
// few blocks per wave the call is bound by each wave's serial walk, not by HBM.
// Chunks of at most 4 heads then read every block once per chunk but give two
// waves per SIMD and lighter blocks (g = 7, d_h = 64, 60 sequences of up to
// 2048 tokens: 22.95 -> 20.2 us).  This applies when the whole line at that
// chunking holds at most kSmallLineBlocksPerWave blocks per wave of a
// 2048-wave chip; the decision uses host arguments only, so the workspace
// size and the launch agree.
constexpr int kSmallLineWaves = 2048;
constexpr int kSmallLineBlocksPerWave = 16;
inline HeadChunks head_chunks(int g, int d_h, bool bf16, int B, int h_kv, int max_context_len) {
  const int cap = max_chunk(d_h, bf16);
  if (g > 4 && cap > 4) {
    const int64_t line4 = (int64_t)B * h_kv * ((g + 3) / 4) * (((int64_t)max_context_len + 15) / 16);
    if (line4 <= (int64_t)kSmallLineWaves * kSmallLineBlocksPerWave) return chunks_of(g, 4);
  }
  return chunks_of(g, cap);
}

// Decode work line: every (sequence, KV head, head chunk) segment's blocks laid
// end to end.  Its length is at most B * h_kv * n_chunks * ceil(max_context_len / 16).
inline int64_t decode_line_upper(int B, int h_q, int h_kv, int d_h, bool bf16,
                                 int max_context_len) {
  return (int64_t)B * h_kv *
         head_chunks(h_q / h_kv, d_h, bf16, B, h_kv, max_context_len).n_chunks *
         (((int64_t)max_context_len + 15) / 16);
}

// Upper bound of the automatic split count (resident wavefronts of a full MI355X
// at two waves per SIMD is 2048; the bound leaves room for higher occupancy).
constexpr int kMaxAutoSplits = 4096;
constexpr int kMaxSplits = 1 << 16;
// Longest line the decode cuts: positions times the cut's cumulative weights
// (at most kMaxSplits * 11) stay within int64.
constexpr int64_t kMaxLineBlocks = (int64_t)1 << 40;

// Splits the workspace must hold: the explicit count, or the automatic bound.
inline int64_t decode_split_bound(int B, int h_q, int h_kv, int d_h, bool bf16,
                                  int max_context_len, int num_splits) {
  if (num_splits > 0) return num_splits;
  const int64_t up = decode_line_upper(B, h_q, h_kv, d_h, bf16, max_context_len);
  return up < 1 ? 1 : (up > kMaxAutoSplits ? kMaxAutoSplits : up);
}

// Workspace: per split, two partial states (first and last segment piece) of gc
// heads, each d_h accumulators plus the running max and sum, in fp32; then one
// descriptor per (sequence, KV head, head chunk) segment: the first and last
// wave holding a piece of it; then the line length (int64, 16 bytes reserved).
inline size_t decode_partials_bytes(int B, int h_q, int h_kv, int d_h, bool bf16,
                                    int max_context_len, int num_splits) {
  const int gc = head_chunks(h_q / h_kv, d_h, bf16, B, h_kv, max_context_len).per_chunk;
  return (size_t)decode_split_bound(B, h_q, h_kv, d_h, bf16, max_context_len, num_splits) * 2 *
         gc * (size_t)(d_h + 2) * sizeof(float);
}
inline size_t decode_workspace_bytes(int B, int h_q, int h_kv, int d_h, bool bf16,
                                     int max_context_len, int num_splits) {
  if (B <= 0) return 0;
  const size_t segs =
      (size_t)B * h_kv * head_chunks(h_q / h_kv, d_h, bf16, B, h_kv, max_context_len).n_chunks;
  return decode_partials_bytes(B, h_q, h_kv, d_h, bf16, max_context_len, num_splits) +
         ((segs * 2 * sizeof(int32_t) + 15) / 16) * 16 + 16;
}

// Workspace bound that needs neither h_kv nor the dtype: for any h_kv dividing
// h_q and any pool type, the automatic split count is at most
// min(kMaxAutoSplits, B * h_q * ceil(L / 16)) (a segment holds at least one
// query head, so there are at most B * h_q segments), a chunk holds at most
// min(8, h_q) heads, and there are at most B * h_q segment descriptors.
inline size_t decode_workspace_bound(int B, int h_q, int d_h, int max_context_len) {
  if (B <= 0) return 0;
  const int64_t segs = (int64_t)B * h_q;
  int64_t splits = segs * (((int64_t)max_context_len + 15) / 16);
  splits = splits < 1 ? 1 : (splits > kMaxAutoSplits ? kMaxAutoSplits : splits);
  const int gc = h_q < 8 ? h_q : 8;
  return (size_t)splits * 2 * gc * (size_t)(d_h + 2) * sizeof(float) +
         (((size_t)segs * 2 * sizeof(int32_t) + 15) / 16) * 16 + 16;
}

// Element type of a KV pool.  kI8: int8 codes with a float32 scale per token
// head row, read by bf16 queries.
enum class KvType { kF32, kBF16, kI8 };

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;  // kI8 only: [n_blocks, h_kv, 16]
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws;  // [num_splits][2][gc][d_h + 2]: accumulators, max (log2 units), sum
  int32_t* seg_desc;  // [B * h_kv * n_chunks][2]: first and last wave of each segment
  int64_t* line_total;  // blocks on the line, written by the first pass
  int B, h_q, h_kv, g, n_chunks, gc, n_blocks, max_blocks_per_seq, num_splits;
  float scale_log2;  // scale * log2(e)
};

// Wavefronts of the decode kernel for (d_h, dtype, gc) that the current device
// holds at once; 0 if it cannot be queried.
int decode_resident_waves(int d_h, KvType kv, int gc);

hipError_t launch_kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                            void* k_cache, void* v_cache, int T, int h_kv, int d_h,
                            int n_blocks, int elem_bytes, hipStream_t stream);

// Returns hipErrorInvalidValue for (dtype, d_h, gc) combinations without a kernel.
hipError_t launch_decode(const DecodeArgs& a, int d_h, KvType kv, hipStream_t stream);

// Quantises each new token's K and V rows to int8 with a float32 scale per
// (token, KV head) row and scatters codes and scales to their slots.  src_bytes:
// 2 (bf16 rows) or 4 (float32 rows).
hipError_t launch_kv_append_i8(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                               int8_t* k_cache, int8_t* v_cache, float* k_scale, float* v_scale,
                               int T, int h_kv, int d_h, int n_blocks, int src_bytes,
                               hipStream_t stream);

struct PrefillArgs {
  void* out;
  const void* q;
  const int32_t* cu_seqlens_q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const float* k_scale;  // INT8 cache only: [n_blocks, h_kv, 16]
  const float* v_scale;
  int S, T_q, max_q_len, h_q, h_kv, g, n_blocks, max_blocks_per_seq;
  float scale_log2;
  int longest_first;  // set by the launcher: sequence planes taken longest context first
};

hipError_t launch_prefill_bf16(const PrefillArgs& a, int d_h, hipStream_t stream);
// The bf16 prefill in 8-wave workgroups whose two wave groups alternate matrix
// and vector phases (for grids of many workgroups).
hipError_t launch_prefill_pp(const PrefillArgs& a, int d_h, hipStream_t stream);
// Prefill over an INT8 cache (codes and float32 scales), bf16 queries and output.
hipError_t launch_prefill_i8(const PrefillArgs& a, int d_h, hipStream_t stream);

// Block copies between pool sets: up to kMaxCopyPools pools (K, V, and for the
// INT8 cache their scales) share one block mapping.  src/dst are device
// addresses (a pinned host pool's device mapping included); vecs[i] is the
// 16-byte vectors per block of pool i.
constexpr int kMaxCopyPools = 8;
struct CopyPools {
  const uint4* src[kMaxCopyPools];
  uint4* dst[kMaxCopyPools];
  int64_t vecs[kMaxCopyPools];
};

// pairs: int32 [n_pairs][2] (source block, destination block), device-visible.
// A pair with an index out of range is skipped.  device_only: every pool is
// device memory (the copy then streams with the non-temporal hint).  Returns
// hipErrorInvalidValue when a block is too large for the grid (more than 65535
// slices of 32 KiB).
hipError_t launch_copy_blocks(const CopyPools& p, int n_pools, const int32_t* pairs, int n_pairs,
                              int n_src_blocks, int n_dst_blocks, bool device_only,
                              hipStream_t stream);

}  // namespace pkv
