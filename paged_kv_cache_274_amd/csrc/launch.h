// Host-side launchers of the libpkv kernels (internal; the public C ABI is pkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Query heads handled by one decode workgroup: the GQA group of a KV head is
// split into n_chunks chunks of at most 8 heads, so per-lane accumulators stay
// in registers.
struct HeadChunks {
  int n_chunks;
  int per_chunk;
};
inline HeadChunks head_chunks(int g) {
  HeadChunks c;
  c.n_chunks = (g + 7) / 8;
  c.per_chunk = (g + c.n_chunks - 1) / c.n_chunks;
  return c;
}

// Decode context split.  Picks the largest power of two in [64, 1024] such
// that, were every context half of max_context_len long, the launch would
// still hold about 2048 (sequence, KV head, partition) work units: enough to
// fill 256 CUs several times while the per-partition partial results stay a
// few percent of the KV bytes read.
inline int decode_partition_tokens(int B, int h_q, int h_kv, int max_context_len,
                                   int requested) {
  if (B < 0 || h_q <= 0 || h_kv <= 0 || h_q % h_kv != 0 || max_context_len < 0) return -1;
  if (requested != 0) {
    if (requested < 16 || requested > 1024 || requested % 16 != 0) return -1;
    return requested;
  }
  const int64_t base = (int64_t)B * h_kv * head_chunks(h_q / h_kv).n_chunks;
  const int64_t want = base * (int64_t)max_context_len / 4096;
  int p = 64;
  while (p < 1024 && 2 * p <= want) p *= 2;
  return p;
}

inline int decode_num_partitions(int max_context_len, int partition_tokens) {
  return (max_context_len + partition_tokens - 1) / partition_tokens;
}

inline size_t decode_workspace_bytes(int B, int h_q, int d_h, int max_context_len,
                                     int partition_tokens) {
  const int P = decode_num_partitions(max_context_len, partition_tokens);
  if (P <= 1 || B == 0) return 0;
  return (size_t)B * h_q * P * (size_t)(d_h + 2) * sizeof(float);
}

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_acc;   // [B, h_q, P, d_h] unnormalised partial outputs
  float* ws_ml;    // [B, h_q, P, 2]  (running max in log2 units, sum of weights)
  int B, h_q, h_kv, g, n_chunks, n_blocks, max_blocks_per_seq;
  int partition_tokens, num_partitions;
  float scale_log2;  // scale * log2(e)
};

hipError_t launch_kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                            void* k_cache, void* v_cache, int T, int h_kv, int d_h,
                            int n_blocks, int elem_bytes, hipStream_t stream);

// Returns hipErrorInvalidValue for (dtype, d_h, chunk) combinations without a kernel.
hipError_t launch_decode(const DecodeArgs& a, int d_h, bool bf16, hipStream_t stream);

struct PrefillArgs {
  void* out;
  const void* q;
  const int32_t* cu_seqlens_q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int S, T_q, max_q_len, h_q, h_kv, g, n_blocks, max_blocks_per_seq;
  float scale_log2;
};

hipError_t launch_prefill_bf16(const PrefillArgs& a, int d_h, hipStream_t stream);

}  // namespace pkv
