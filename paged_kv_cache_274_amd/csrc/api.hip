// C ABI of libpkv (declared in include/pkv.h): argument validation and dispatch.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "launch.h"
#include "line.h"
#include "pkv.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
// Widest block-table row: its token capacity (16 per block) stays an int, as
// the kernels clamp context lengths to it in 32-bit arithmetic.
constexpr int kMaxTableWidth = 0x7fffffff / 16;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(int dtype) {
  if (dtype == PKV_F32) return 4;
  if (dtype == PKV_BF16) return 2;
  return 0;
}

bool debug_checks() {
  static const bool on = [] {
    const char* e = getenv("PKV_DEBUG");
    return e && e[0] == '1';
  }();
  return on;
}

template <typename T>
bool copy_to_host(std::vector<T>& dst, const T* src, size_t n, hipStream_t stream) {
  dst.resize(n);
  if (n == 0) return true;
  if (hipStreamSynchronize(stream) != hipSuccess) return false;
  return hipMemcpy(dst.data(), src, n * sizeof(T), hipMemcpyDefault) == hipSuccess;
}

// PKV_DEBUG: context lengths and the block-table entries they reach.
int debug_check_tables(const int32_t* tables, const int32_t* lens, int n_seqs, int max_blocks,
                       int max_len, int n_blocks, hipStream_t stream) {
  std::vector<int32_t> t, l;
  if (!copy_to_host(l, lens, (size_t)n_seqs, stream)) return PKV_ERR_HIP;
  if (!copy_to_host(t, tables, (size_t)n_seqs * max_blocks, stream)) return PKV_ERR_HIP;
  for (int s = 0; s < n_seqs; ++s) {
    if (l[s] < 0 || l[s] > max_len) return PKV_ERR_INVALID_ARG;
    for (int64_t j = 0; j < ((int64_t)l[s] + 15) / 16; ++j) {
      const int32_t e = t[(size_t)s * max_blocks + j];
      if (e < 0 || e >= n_blocks) return PKV_ERR_INVALID_ARG;
    }
  }
  return PKV_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

// PKV_DEBUG: slots in range (or negative) and no slot named twice.
int debug_check_slots(const int64_t* slot_mapping, int T, int n_blocks, hipStream_t stream) {
  std::vector<int64_t> sl;
  if (!copy_to_host(sl, slot_mapping, (size_t)T, stream)) return PKV_ERR_HIP;
  std::vector<char> seen((size_t)n_blocks * 16, 0);
  for (int64_t v : sl) {
    if (v < 0) continue;
    if (v >= (int64_t)n_blocks * 16 || seen[(size_t)v]) return PKV_ERR_INVALID_ARG;
    seen[(size_t)v] = 1;
  }
  return PKV_OK;
}

// Device address of a pool the GPU can reach: device or managed memory as is,
// pinned host memory through its device mapping.  False for memory the GPU
// cannot reach (pageable host memory, unknown pointers); the runtime's error is
// cleared so that it is not reported by a later launch check.
bool device_address(const void* p, const void** out, bool* on_host) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  *on_host = false;
  if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) {
    *out = p;
    return true;
  }
  if (a.type == hipMemoryTypeHost) {
    // Only memory the runtime pinned (hipHostMalloc or registered) has flags
    // and a device mapping.
    unsigned int flags = 0;
    void* d = nullptr;
    if (hipHostGetFlags(&flags, const_cast<void*>(p)) != hipSuccess ||
        hipHostGetDevicePointer(&d, const_cast<void*>(p), 0) != hipSuccess || !d) {
      (void)hipGetLastError();
      return false;
    }
    *out = d;
    *on_host = true;
    return true;
  }
  return false;
}

// PKV_DEBUG: block pairs in range, no destination named twice and, within one
// pool set, no block both read and written.
int debug_check_pairs(const int32_t* pairs, int n_pairs, int n_src, int n_dst, bool same_set,
                      hipStream_t stream) {
  std::vector<int32_t> p;
  if (!copy_to_host(p, pairs, (size_t)n_pairs * 2, stream)) return PKV_ERR_HIP;
  std::vector<char> written((size_t)n_dst, 0), read(same_set ? (size_t)n_src : 0, 0);
  for (int i = 0; i < n_pairs; ++i) {
    const int32_t s = p[2 * (size_t)i], d = p[2 * (size_t)i + 1];
    if (s < 0 || s >= n_src || d < 0 || d >= n_dst || written[(size_t)d]) return PKV_ERR_INVALID_ARG;
    written[(size_t)d] = 1;
    if (same_set) read[(size_t)s] = 1;
  }
  if (same_set)
    for (int b = 0; b < n_src; ++b)
      if (read[(size_t)b] && written[(size_t)b]) return PKV_ERR_INVALID_ARG;
  return PKV_OK;
}

// Both block-copy entry points.  src == dst for a copy within one pool set.
int copy_call(const void* const* src, void* const* dst, const int64_t* block_bytes, int n_pools,
              int n_src, int n_dst, const int32_t* pairs, int n_pairs, bool same_set,
              hipStream_t stream) {
  if (n_pools < 1 || n_pools > pkv::kMaxCopyPools || n_src < 1 || n_dst < 1 || n_pairs < 0 ||
      !src || !dst || !block_bytes)
    return PKV_ERR_INVALID_ARG;
  for (int i = 0; i < n_pools; ++i) {
    const int64_t bb = block_bytes[i];
    if (bb <= 0 || (bb & 15) || !src[i] || !dst[i] || !aligned16(src[i]) || !aligned16(dst[i]))
      return PKV_ERR_INVALID_ARG;
    if (!same_set && src[i] == dst[i]) return PKV_ERR_INVALID_ARG;
    if (bb / 16 > (int64_t)65535 * 2048) return PKV_ERR_UNSUPPORTED;
  }
  if (n_pairs == 0) return PKV_OK;
  if (!pairs || ((uintptr_t)pairs & 3u)) return PKV_ERR_INVALID_ARG;
  pkv::CopyPools p;
  memset(&p, 0, sizeof(p));
  bool device_only = true;
  for (int i = 0; i < n_pools; ++i) {
    const void* s_dev;
    const void* d_dev;
    bool s_host, d_host;
    if (!device_address(src[i], &s_dev, &s_host) || !device_address(dst[i], &d_dev, &d_host))
      return PKV_ERR_INVALID_ARG;
    device_only = device_only && !s_host && !d_host;
    p.src[i] = (const uint4*)s_dev;
    p.dst[i] = (uint4*)d_dev;
    p.vecs[i] = block_bytes[i] / 16;
  }
  const void* pairs_dev;
  bool pairs_host;
  if (!device_address(pairs, &pairs_dev, &pairs_host)) return PKV_ERR_INVALID_ARG;
  hipStream_t s = stream;
  if (debug_checks()) {
    const int rc = debug_check_pairs(pairs, n_pairs, n_src, n_dst, same_set, s);
    if (rc != PKV_OK) return rc;
  }
  return from_hip(pkv::launch_copy_blocks(p, n_pools, (const int32_t*)pairs_dev, n_pairs, n_src,
                                          n_dst, device_only, s));
}

// Pool element type of a decode dtype code; false for an unknown code.
bool kv_type_of(int dtype, pkv::KvType* kv) {
  if (dtype == PKV_F32) *kv = pkv::KvType::kF32;
  else if (dtype == PKV_BF16) *kv = pkv::KvType::kBF16;
  else if (dtype == PKV_INT8) *kv = pkv::KvType::kI8;
  else return false;
  return true;
}
// The head chunking and workspace of an INT8 cache are those of bf16 rows.
bool chunks_as_bf16(pkv::KvType kv) { return kv != pkv::KvType::kF32; }

}  // namespace

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID_ARG: return "PKV_ERR_INVALID_ARG";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE";
    case PKV_ERR_HIP: return "PKV_ERR_HIP";
    case PKV_ERR_NO_BLOCKS: return "PKV_ERR_NO_BLOCKS";
  }
  return "PKV_UNKNOWN_STATUS";
}

int kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping, void* k_cache,
              void* v_cache, int T, int h_kv, int d_h, int n_blocks, int dtype, hipStream_t stream) {
  const int eb = elem_bytes(dtype);
  if (eb == 0) return PKV_ERR_INVALID_ARG;
  if (T < 0 || h_kv <= 0 || n_blocks <= 0) return PKV_ERR_INVALID_ARG;
  if (d_h != 64 && d_h != 128) return PKV_ERR_UNSUPPORTED;
  if (T == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PKV_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      ((uintptr_t)slot_mapping & 7u))
    return PKV_ERR_INVALID_ARG;
  hipStream_t s = stream;
  if (debug_checks()) {
    const int rc = debug_check_slots(slot_mapping, T, n_blocks, s);
    if (rc != PKV_OK) return rc;
  }
  return from_hip(pkv::launch_kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, T, h_kv, d_h,
                                        n_blocks, eb, s));
}

int kv_append_int8(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                   int8_t* k_cache, int8_t* v_cache, float* k_scale, float* v_scale, int T,
                   int h_kv, int d_h, int n_blocks, int dtype, hipStream_t stream) {
  const int eb = elem_bytes(dtype);
  if (eb == 0) return PKV_ERR_INVALID_ARG;
  if (T < 0 || h_kv <= 0 || n_blocks <= 0) return PKV_ERR_INVALID_ARG;
  if (d_h != 64 && d_h != 128) return PKV_ERR_UNSUPPORTED;
  if ((int64_t)T * h_kv * (d_h / 8) > 0x7fffffff - 256) return PKV_ERR_UNSUPPORTED;
  if (T == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache || !k_scale || !v_scale)
    return PKV_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      ((uintptr_t)k_scale & 3u) || ((uintptr_t)v_scale & 3u) || ((uintptr_t)slot_mapping & 7u))
    return PKV_ERR_INVALID_ARG;
  hipStream_t s = stream;
  if (debug_checks()) {
    const int rc = debug_check_slots(slot_mapping, T, n_blocks, s);
    if (rc != PKV_OK) return rc;
  }
  return from_hip(pkv::launch_kv_append_i8(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale,
                                           v_scale, T, h_kv, d_h, n_blocks, eb, s));
}

static bool decode_shape_ok(int B, int h_q, int h_kv, int max_context_len, int num_splits) {
  return B >= 0 && h_q > 0 && h_kv > 0 && h_q % h_kv == 0 && max_context_len >= 0 &&
         num_splits >= 0 && num_splits <= pkv::kMaxSplits;
}

// Automatic split count: one range per wavefront the device holds at once,
// but no more ranges than half the blocks of the longest possible line, so
// that a short line is not cut into one-block pieces whose partial states cost
// more to merge than their blocks cost to read (Llama-3.2-1B-shaped decode,
// 8 sequences of 512 tokens at 32/8/64: 2048 one-block ranges 12.8 us per
// call, 1024 two-block ranges 11.1 us).
static int auto_splits(int B, int h_q, int h_kv, int d_h, int max_context_len, pkv::KvType kv) {
  const bool bf16 = chunks_as_bf16(kv);
  const int gc = pkv::head_chunks(h_q / h_kv, d_h, bf16, B, h_kv, max_context_len).per_chunk;
  int waves = pkv::decode_resident_waves(d_h, kv, gc);
  if (waves <= 0) waves = 2048;
  const int64_t bound = pkv::decode_split_bound(B, h_q, h_kv, d_h, bf16, max_context_len, 0);
  const int64_t half_line =
      (pkv::decode_line_upper(B, h_q, h_kv, d_h, bf16, max_context_len) + 1) / 2;
  int64_t n = waves < bound ? waves : bound;
  if (half_line >= 1 && n > half_line) n = half_line;
  return (int)n;
}

int64_t pkv_decode_line_start(int64_t total, int splits, int w) {
  if (total < 0 || total > pkv::kMaxLineBlocks || splits < 1 || splits > pkv::kMaxSplits ||
      w < 0 || w > splits)
    return -1;
  return pkv::Line{total, splits}.start(w);
}

int pkv_decode_line_wave_of(int64_t total, int splits, int64_t p) {
  if (total < 1 || total > pkv::kMaxLineBlocks || splits < 1 || splits > pkv::kMaxSplits ||
      p < 0 || p >= total)
    return -1;
  return pkv::Line{total, splits}.wave_of(p);
}

int pkv_decode_num_splits(int B, int h_q, int h_kv, int d_h, int max_context_len, int dtype,
                          int num_splits) {
  pkv::KvType kv;
  if (!decode_shape_ok(B, h_q, h_kv, max_context_len, num_splits) || !kv_type_of(dtype, &kv) ||
      (d_h != 64 && d_h != 128))
    return -1;
  if (num_splits > 0) return num_splits;
  return auto_splits(B, h_q, h_kv, d_h, max_context_len, kv);
}

size_t pkv_decode_workspace_bytes_split(int B, int h_q, int h_kv, int d_h, int max_context_len,
                                        int dtype, int num_splits) {
  pkv::KvType kv;
  if (!decode_shape_ok(B, h_q, h_kv, max_context_len, num_splits) || d_h <= 0 ||
      !kv_type_of(dtype, &kv))
    return 0;
  return pkv::decode_workspace_bytes(B, h_q, h_kv, d_h, chunks_as_bf16(kv), max_context_len,
                                     num_splits);
}

size_t pkv_decode_workspace_bytes(int B, int h_q, int d_h, int max_context_len) {
  if (B <= 0 || h_q <= 0 || d_h <= 0 || max_context_len < 0) return 0;
  return pkv::decode_workspace_bound(B, h_q, d_h, max_context_len);
}

// Device memory of paged_decode_attention_noalloc, for callers that cannot
// allocate: the decode workspace (partial states, segment descriptors, line
// length) of one call.  Each GPU holds its own copy until the process ends.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// Device address of `scratch` on the current device, looked up once per device
// (hipGetSymbolAddress with that device current) and kept; nullptr if the
// runtime cannot provide it.  In host code `scratch` itself only names the
// symbol: its address is never passed to a kernel.
static void* static_scratch() {
  static std::mutex mu;
  static std::vector<void*> per_device;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if ((size_t)dev >= per_device.size()) per_device.resize((size_t)dev + 1, nullptr);
  if (!per_device[(size_t)dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    per_device[(size_t)dev] = p;
  }
  return per_device[(size_t)dev];
}

// Both decode entry points: validation, workspace layout and launch.  k_scale
// and v_scale are used (and required) for the INT8 cache only.
static int decode_call(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const float* k_scale, const float* v_scale, const int32_t* block_tables,
                       const int32_t* context_lens, int B, int h_q, int h_kv, int d_h,
                       int n_blocks, int max_blocks_per_seq, int max_context_len, float scale,
                       pkv::KvType kv, int num_splits, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  if (!decode_shape_ok(B, h_q, h_kv, max_context_len, num_splits) || n_blocks <= 0 ||
      max_blocks_per_seq <= 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * 16 ||
      !isfinite(scale))
    return PKV_ERR_INVALID_ARG;
  if ((d_h != 64 && d_h != 128) || max_blocks_per_seq > kMaxTableWidth) return PKV_ERR_UNSUPPORTED;
  if (B == 0) return PKV_OK;
  const bool i8 = kv == pkv::KvType::kI8;
  const bool bf16 = chunks_as_bf16(kv);
  const pkv::HeadChunks hc = pkv::head_chunks(h_q / h_kv, d_h, bf16, B, h_kv, max_context_len);
  if ((int64_t)B * h_kv * hc.n_chunks > 0x7fffffff ||
      pkv::decode_line_upper(B, h_q, h_kv, d_h, bf16, max_context_len) > pkv::kMaxLineBlocks)
    return PKV_ERR_UNSUPPORTED;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens ||
      (i8 && (!k_scale || !v_scale)))
    return PKV_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      ((uintptr_t)block_tables & 3u) || ((uintptr_t)context_lens & 3u) ||
      (i8 && (!aligned16(k_scale) || !aligned16(v_scale))))
    return PKV_ERR_INVALID_ARG;
  const size_t need =
      pkv::decode_workspace_bytes(B, h_q, h_kv, d_h, bf16, max_context_len, num_splits);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PKV_ERR_WORKSPACE;
  hipStream_t s = stream;
  if (debug_checks()) {
    const int rc = debug_check_tables(block_tables, context_lens, B, max_blocks_per_seq,
                                      max_context_len, n_blocks, s);
    if (rc != PKV_OK) return rc;
  }
  pkv::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = i8 ? k_scale : nullptr;
  a.v_scale = i8 ? v_scale : nullptr;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.ws = (float*)workspace;
  a.seg_desc = (int32_t*)((char*)workspace + pkv::decode_partials_bytes(B, h_q, h_kv, d_h, bf16,
                                                                         max_context_len, num_splits));
  a.line_total = (int64_t*)((char*)workspace + need - 16);
  a.B = B;
  a.h_q = h_q;
  a.h_kv = h_kv;
  a.g = h_q / h_kv;
  a.n_chunks = hc.n_chunks;
  a.gc = hc.per_chunk;
  a.n_blocks = n_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_splits = num_splits > 0 ? num_splits : auto_splits(B, h_q, h_kv, d_h, max_context_len, kv);
  a.scale_log2 = scale * kLog2e;
  return from_hip(pkv::launch_decode(a, d_h, kv, s));
}

int paged_decode_attention_split(void* out, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables,
                                 const int32_t* context_lens, int B, int h_q, int h_kv, int d_h,
                                 int n_blocks, int max_blocks_per_seq, int max_context_len,
                                 float scale, int dtype, int num_splits, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  if (dtype != PKV_F32 && dtype != PKV_BF16) return PKV_ERR_INVALID_ARG;
  return decode_call(out, q, k_cache, v_cache, nullptr, nullptr, block_tables, context_lens, B,
                     h_q, h_kv, d_h, n_blocks, max_blocks_per_seq, max_context_len, scale,
                     dtype == PKV_BF16 ? pkv::KvType::kBF16 : pkv::KvType::kF32, num_splits,
                     workspace, workspace_bytes, stream);
}

int paged_decode_attention(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens, int B,
                           int h_q, int h_kv, int d_h, int n_blocks, int max_blocks_per_seq,
                           int max_context_len, float scale, int dtype, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  return paged_decode_attention_split(out, q, k_cache, v_cache, block_tables, context_lens, B,
                                      h_q, h_kv, d_h, n_blocks, max_blocks_per_seq,
                                      max_context_len, scale, dtype, 0, workspace,
                                      workspace_bytes, stream);
}

int paged_decode_attention_noalloc(void* out, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, int B, int h_q, int h_kv, int d_h,
                                   int n_blocks, int max_blocks_per_seq, int max_context_len,
                                   float scale, int dtype, hipStream_t stream) {
  if (dtype != PKV_F32 && dtype != PKV_BF16) return PKV_ERR_INVALID_ARG;
  pkv::KvType kv = dtype == PKV_BF16 ? pkv::KvType::kBF16 : pkv::KvType::kF32;
  if (!decode_shape_ok(B, h_q, h_kv, max_context_len, 0) || (d_h != 64 && d_h != 128))
    return decode_call(out, q, k_cache, v_cache, nullptr, nullptr, block_tables, context_lens, B,
                       h_q, h_kv, d_h, n_blocks, max_blocks_per_seq, max_context_len, scale, kv,
                       0, nullptr, 0, stream);  // reports the argument error
  if (B == 0) return PKV_OK;
  // The automatic split, stated explicitly: the same launch as
  // paged_decode_attention, with the workspace sized for the count in use
  // rather than for the largest automatic count.
  const int splits = auto_splits(B, h_q, h_kv, d_h, max_context_len, kv);
  if (pkv::decode_workspace_bytes(B, h_q, h_kv, d_h, chunks_as_bf16(kv), max_context_len,
                                  splits) > kStaticScratchBytes)
    return PKV_ERR_WORKSPACE;
  if (stream) {
    int cur = -1, sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &sdev) != hipSuccess) {
      (void)hipGetLastError();
      return PKV_ERR_HIP;
    }
    if (cur != sdev) return PKV_ERR_INVALID_ARG;
  }
  void* ws = static_scratch();
  if (!ws) return PKV_ERR_HIP;
  return decode_call(out, q, k_cache, v_cache, nullptr, nullptr, block_tables, context_lens, B,
                     h_q, h_kv, d_h, n_blocks, max_blocks_per_seq, max_context_len, scale, kv,
                     splits, ws, kStaticScratchBytes, stream);
}

int paged_decode_attention_int8(void* out, const void* q, const int8_t* k_cache,
                                const int8_t* v_cache, const float* k_scale, const float* v_scale,
                                const int32_t* block_tables, const int32_t* context_lens, int B,
                                int h_q, int h_kv, int d_h, int n_blocks, int max_blocks_per_seq,
                                int max_context_len, float scale, int num_splits, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  return decode_call(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, B,
                     h_q, h_kv, d_h, n_blocks, max_blocks_per_seq, max_context_len, scale,
                     pkv::KvType::kI8, num_splits, workspace, workspace_bytes, stream);
}

int paged_prefill_attention(void* out, const void* q, const int32_t* cu_seqlens_q,
                            const void* k_cache, const void* v_cache, const int32_t* block_tables,
                            const int32_t* context_lens, int S, int T_q, int max_q_len, int h_q,
                            int h_kv, int d_h, int n_blocks, int max_blocks_per_seq, float scale,
                            int dtype, hipStream_t stream) {
  if (elem_bytes(dtype) == 0) return PKV_ERR_INVALID_ARG;
  if (S < 0 || T_q < 0 || max_q_len < 0 || h_q <= 0 || h_kv <= 0 || h_q % h_kv != 0 ||
      n_blocks <= 0 || max_blocks_per_seq <= 0 || !isfinite(scale))
    return PKV_ERR_INVALID_ARG;
  if ((d_h != 64 && d_h != 128) || max_blocks_per_seq > kMaxTableWidth) return PKV_ERR_UNSUPPORTED;
  if (dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (S == 0 || T_q == 0 || max_q_len == 0) return PKV_OK;
  if (S > 65535 || h_kv > 65535) return PKV_ERR_UNSUPPORTED;
  if (!out || !q || !cu_seqlens_q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PKV_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      ((uintptr_t)block_tables & 3u) || ((uintptr_t)context_lens & 3u) ||
      ((uintptr_t)cu_seqlens_q & 3u))
    return PKV_ERR_INVALID_ARG;
  hipStream_t s = stream;
  if (debug_checks()) {
    std::vector<int32_t> cu, l;
    if (!copy_to_host(cu, cu_seqlens_q, (size_t)S + 1, s)) return PKV_ERR_HIP;
    if (!copy_to_host(l, context_lens, (size_t)S, s)) return PKV_ERR_HIP;
    if (cu[0] != 0 || cu[S] != T_q) return PKV_ERR_INVALID_ARG;
    for (int i = 0; i < S; ++i) {
      const int n = cu[i + 1] - cu[i];
      if (n < 0 || n > max_q_len || n > l[i]) return PKV_ERR_INVALID_ARG;
    }
    const int rc = debug_check_tables(block_tables, context_lens, S, max_blocks_per_seq,
                                      max_blocks_per_seq * 16, n_blocks, s);
    if (rc != PKV_OK) return rc;
  }
  pkv::PrefillArgs a;
  memset(&a, 0, sizeof(a));
  a.out = out;
  a.q = q;
  a.cu_seqlens_q = cu_seqlens_q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.S = S;
  a.T_q = T_q;
  a.max_q_len = max_q_len;
  a.h_q = h_q;
  a.h_kv = h_kv;
  a.g = h_q / h_kv;
  a.n_blocks = n_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.scale_log2 = scale * kLog2e;
  return from_hip(pkv::launch_prefill_bf16(a, d_h, s));
}

int paged_prefill_attention_int8(void* out, const void* q, const int32_t* cu_seqlens_q,
                                 const int8_t* k_cache, const int8_t* v_cache,
                                 const float* k_scale, const float* v_scale,
                                 const int32_t* block_tables, const int32_t* context_lens, int S,
                                 int T_q, int max_q_len, int h_q, int h_kv, int d_h, int n_blocks,
                                 int max_blocks_per_seq, float scale, hipStream_t stream) {
  if (S < 0 || T_q < 0 || max_q_len < 0 || h_q <= 0 || h_kv <= 0 || h_q % h_kv != 0 ||
      n_blocks <= 0 || max_blocks_per_seq <= 0 || !isfinite(scale))
    return PKV_ERR_INVALID_ARG;
  if ((d_h != 64 && d_h != 128) || max_blocks_per_seq > kMaxTableWidth) return PKV_ERR_UNSUPPORTED;
  if (S == 0 || T_q == 0 || max_q_len == 0) return PKV_OK;
  if (S > 65535 || h_kv > 65535) return PKV_ERR_UNSUPPORTED;
  if (!out || !q || !cu_seqlens_q || !k_cache || !v_cache || !k_scale || !v_scale ||
      !block_tables || !context_lens)
    return PKV_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(k_scale) || !aligned16(v_scale) || ((uintptr_t)block_tables & 3u) ||
      ((uintptr_t)context_lens & 3u) || ((uintptr_t)cu_seqlens_q & 3u))
    return PKV_ERR_INVALID_ARG;
  hipStream_t s = stream;
  if (debug_checks()) {
    std::vector<int32_t> cu, l;
    if (!copy_to_host(cu, cu_seqlens_q, (size_t)S + 1, s)) return PKV_ERR_HIP;
    if (!copy_to_host(l, context_lens, (size_t)S, s)) return PKV_ERR_HIP;
    if (cu[0] != 0 || cu[S] != T_q) return PKV_ERR_INVALID_ARG;
    for (int i = 0; i < S; ++i) {
      const int n = cu[i + 1] - cu[i];
      if (n < 0 || n > max_q_len || n > l[i]) return PKV_ERR_INVALID_ARG;
    }
    const int rc = debug_check_tables(block_tables, context_lens, S, max_blocks_per_seq,
                                      max_blocks_per_seq * 16, n_blocks, s);
    if (rc != PKV_OK) return rc;
  }
  pkv::PrefillArgs a;
  memset(&a, 0, sizeof(a));
  a.out = out;
  a.q = q;
  a.cu_seqlens_q = cu_seqlens_q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.S = S;
  a.T_q = T_q;
  a.max_q_len = max_q_len;
  a.h_q = h_q;
  a.h_kv = h_kv;
  a.g = h_q / h_kv;
  a.n_blocks = n_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.scale_log2 = scale * kLog2e;
  return from_hip(pkv::launch_prefill_i8(a, d_h, s));
}

int copy_blocks(void* const* pools, const int64_t* block_bytes, int n_pools, int n_blocks,
                const int32_t* pairs, int n_pairs, hipStream_t stream) {
  return copy_call((const void* const*)pools, pools, block_bytes, n_pools, n_blocks, n_blocks,
                   pairs, n_pairs, true, stream);
}

int swap_blocks(const void* const* src_pools, void* const* dst_pools, const int64_t* block_bytes,
                int n_pools, int n_src_blocks, int n_dst_blocks, const int32_t* pairs,
                int n_pairs, hipStream_t stream) {
  return copy_call(src_pools, dst_pools, block_bytes, n_pools, n_src_blocks, n_dst_blocks, pairs,
                   n_pairs, false, stream);
}

}  // extern "C"
