// Split-context paged decode attention for gfx950.
//
// Single-token decode over the cached context of a continuous batch of
// variable-length sequences (LLM Inference Server page, Stage 1 prefill/decode
// task; "What you build" of the From Scratch page), with grouped-query heads
// and 16-token blocks behind a per-sequence block table (Paged KV-Cache Block
// Allocator stretch challenge; Block Manager box of the pipeline figure).
// Decode is bound by reading the KV cache from HBM ("What You Will Build",
// LLM Inference Server page), so the design goal is streaming every K/V byte
// exactly once at full bandwidth:
//
//  * Work unit = (sequence b, KV head, chunk of <= 8 query heads of its GQA
//    group, context partition).  A partition of P tokens is split block by block
//    over the 4 wavefronts of the workgroup; each K/V block of a KV head is read
//    once for every query head of the chunk.
//  * A wavefront streams whole 16-token blocks straight into VGPRs with 16-byte
//    loads; the next block's loads are in flight while the current block is
//    used.  A token row is covered by LPT = row_bytes / 32 adjacent lanes, so
//    one load instruction reads contiguous half-rows of 64 / LPT tokens.
//  * q.K partial sums are combined across the LPT lanes of a token with DPP row
//    permutations (no LDS).  bf16 products use v_dot2_f32_bf16.
//  * Online softmax in base 2 (scale * log2(e) folded into the score).  Every
//    lane keeps its own running reference max, sum and fp32 accumulators for
//    the tokens it owns; the reference only moves when a score exceeds it by
//    more than 2^8, so rescaling the accumulators is rare.  The per-lane states
//    are merged exactly (log-sum-exp) at the end: across lanes with DPP/
//    shuffles, across the 4 waves through LDS, and across partitions by the
//    second kernel.
//  * A context that fits one partition is normalised and stored by the first
//    kernel; the merge kernel skips it.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace pkv {

constexpr int kDecodeWaves = 4;
constexpr float kRescaleSlack = 8.0f;  // log2 units
constexpr float kNegInf = -__builtin_huge_valf();

template <typename T, int D>
struct DecodeShape {
  static constexpr int kElem = sizeof(T);
  static constexpr int kRowVec = D * kElem / 16;   // 16-byte vectors per token row
  static constexpr int kLPT = kRowVec / 2;         // lanes per token row (two vectors each)
  static constexpr int kEPV = 16 / kElem;          // elements per vector
  static constexpr int kEPL = 2 * kEPV;            // elements a lane holds of one token
  static constexpr int kTPW = kWave / kLPT;        // tokens one wave covers per pass
  static constexpr int kPasses = kBlock / kTPW;    // passes per 16-token block
  static_assert(kLPT >= 2 && kLPT <= 16, "row must span 2..16 lanes");
};

template <int NP>
struct BlockRegs {
  uint4 k[NP][2];
  uint4 v[NP][2];
};

__device__ __forceinline__ uint32_t dw(const uint4& u, int w) {
  return w == 0 ? u.x : (w == 1 ? u.y : (w == 2 ? u.z : u.w));
}

// Loads one 16-token block of one KV head: base points at its first vector.
template <typename T, int D>
__device__ __forceinline__ void load_block(BlockRegs<DecodeShape<T, D>::kPasses>& r,
                                           const uint4* __restrict__ kbase,
                                           const uint4* __restrict__ vbase, int slot, int sub) {
  using Sh = DecodeShape<T, D>;
#pragma unroll
  for (int ps = 0; ps < Sh::kPasses; ++ps) {
    const int tk = ps * Sh::kTPW + slot;
#pragma unroll
    for (int v = 0; v < 2; ++v) r.k[ps][v] = kbase[tk * Sh::kRowVec + v * Sh::kLPT + sub];
  }
#pragma unroll
  for (int ps = 0; ps < Sh::kPasses; ++ps) {
    const int tk = ps * Sh::kTPW + slot;
#pragma unroll
    for (int v = 0; v < 2; ++v) r.v[ps][v] = vbase[tk * Sh::kRowVec + v * Sh::kLPT + sub];
  }
}

// Query registers: bf16 kept packed for v_dot2, fp32 kept as floats.
template <typename T, int GC, int EPL>
struct QRegs {
  static constexpr int kWords = std::is_same<T, float>::value ? EPL : EPL / 2;
  uint32_t w[GC][kWords];
};

template <typename T, int D, int GC>
__device__ __forceinline__ float dot_lane(const QRegs<T, GC, DecodeShape<T, D>::kEPL>& q, int j,
                                          const uint4 (&k)[2]) {
  float acc = 0.f;
  if constexpr (std::is_same<T, float>::value) {
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int w = 0; w < 4; ++w)
        acc = fmaf(__uint_as_float(q.w[j][v * 4 + w]), __uint_as_float(dw(k[v], w)), acc);
  } else {
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int w = 0; w < 4; ++w)
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, dw(k[v], w)),
                                              __builtin_bit_cast(bf16x2_t, q.w[j][v * 4 + w]),
                                              acc, false);
  }
  return acc;
}

template <typename T, int EPL>
__device__ __forceinline__ void widen(const uint4 (&v)[2], float (&f)[EPL]) {
  if constexpr (std::is_same<T, float>::value) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int w = 0; w < 4; ++w) f[i * 4 + w] = __uint_as_float(dw(v[i], w));
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        f[i * 8 + 2 * w] = bf16lo_to_f32(dw(v[i], w));
        f[i * 8 + 2 * w + 1] = bf16hi_to_f32(dw(v[i], w));
      }
  }
}

// Folds one block into the lane's running (m, l, acc).  MASK: tokens at local
// index >= valid are outside the context (their scores and values are ignored,
// whatever the pool holds there).
template <typename T, int D, int GC, bool MASK>
__device__ __forceinline__ void attend_block(const BlockRegs<DecodeShape<T, D>::kPasses>& r,
                                             const QRegs<T, GC, DecodeShape<T, D>::kEPL>& q,
                                             float (&m)[GC], float (&l)[GC],
                                             float (&acc)[GC][DecodeShape<T, D>::kEPL],
                                             float scale_log2, int slot, int valid) {
  using Sh = DecodeShape<T, D>;
  constexpr int NP = Sh::kPasses;
  constexpr int EPL = Sh::kEPL;
  float s[NP][GC];
#pragma unroll
  for (int ps = 0; ps < NP; ++ps)
#pragma unroll
    for (int j = 0; j < GC; ++j) s[ps][j] = group_sum<Sh::kLPT>(dot_lane<T, D, GC>(q, j, r.k[ps])) * scale_log2;
  bool ok[NP];
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
    ok[ps] = !MASK || (ps * Sh::kTPW + slot < valid);
    if (MASK && !ok[ps]) {
#pragma unroll
      for (int j = 0; j < GC; ++j) s[ps][j] = kNegInf;
    }
  }
  float smax[GC];
  bool need = false;
#pragma unroll
  for (int j = 0; j < GC; ++j) {
    smax[j] = s[0][j];
#pragma unroll
    for (int ps = 1; ps < NP; ++ps) smax[j] = fmaxf(smax[j], s[ps][j]);
    need |= smax[j] > m[j] + kRescaleSlack;
  }
  if (__any(need)) {
#pragma unroll
    for (int j = 0; j < GC; ++j) {
      const float mn = smax[j] > m[j] + kRescaleSlack ? smax[j] : m[j];
      const float alpha = mn == m[j] ? 1.f : fast_exp2(m[j] - mn);
      m[j] = mn;
      l[j] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] *= alpha;
    }
  }
  float p[NP][GC];
#pragma unroll
  for (int ps = 0; ps < NP; ++ps)
#pragma unroll
    for (int j = 0; j < GC; ++j) {
      float w = fast_exp2(s[ps][j] - m[j]);
      if (MASK) w = ok[ps] ? w : 0.f;
      p[ps][j] = w;
      l[j] += w;
    }
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
    float vf[EPL];
    widen<T, EPL>(r.v[ps], vf);
    if (MASK && !ok[ps]) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) vf[e] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < GC; ++j)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] = fmaf(p[ps][j], vf[e], acc[j][e]);
  }
}

template <typename T>
__device__ __forceinline__ void store_elem(T* out, size_t i, float x) {
  if constexpr (std::is_same<T, float>::value) {
    out[i] = x;
  } else {
    reinterpret_cast<uint16_t*>(out)[i] = (uint16_t)f32_to_bf16_bits(x);
  }
}

template <typename T, int D, int GC>
__global__ __launch_bounds__(256) void decode_partial_kernel(DecodeArgs a) {
  using Sh = DecodeShape<T, D>;
  constexpr int NP = Sh::kPasses;
  constexpr int EPL = Sh::kEPL;
  constexpr int W = kDecodeWaves;
  __shared__ float s_acc[W][GC][D];
  __shared__ float s_m[W][GC];
  __shared__ float s_l[W][GC];

  const int part = blockIdx.x;
  const int kvh = blockIdx.y / a.n_chunks;
  const int chunk = blockIdx.y - kvh * a.n_chunks;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int sub = lane % Sh::kLPT;
  const int slot = lane / Sh::kLPT;
  const int head0 = kvh * a.g + chunk * GC;
  const int nh = min(GC, a.g - chunk * GC);
  const int P = a.partition_tokens;
  // Lengths beyond the table or beyond the launched partitions are clamped, so
  // no value in device memory can move an access outside its buffer.
  int L = a.context_lens[b];
  L = max(0, min(L, min(a.max_blocks_per_seq * kBlock, a.num_partitions * P)));
  const int n_part = (L + P - 1) / P;
  T* out = reinterpret_cast<T*>(a.out);

  if (part >= n_part) {
    if (L == 0 && part == 0) {
      for (int i = threadIdx.x; i < nh * D; i += blockDim.x)
        store_elem<T>(out, ((size_t)b * a.h_q + head0 + i / D) * D + i % D, 0.f);
    }
    return;
  }
  const int tok0 = part * P;
  const int tok1 = min(L, tok0 + P);
  const int blk0 = tok0 / kBlock;
  const int nblk = (tok1 + kBlock - 1) / kBlock - blk0;  // <= 64

  int my_tbl = 0;
  if (lane < nblk) {
    const int e = a.block_tables[(size_t)b * a.max_blocks_per_seq + blk0 + lane];
    my_tbl = (e >= 0 && e < a.n_blocks) ? e : 0;
  }

  QRegs<T, GC, EPL> q;
  {
    const uint4* qv = reinterpret_cast<const uint4*>(a.q);
#pragma unroll
    for (int j = 0; j < GC; ++j) {
      const int h = head0 + min(j, nh - 1);
      const size_t rowv = ((size_t)b * a.h_q + h) * Sh::kRowVec;
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const uint4 x = qv[rowv + v * Sh::kLPT + sub];
        if constexpr (std::is_same<T, float>::value) {
          q.w[j][v * 4 + 0] = x.x; q.w[j][v * 4 + 1] = x.y;
          q.w[j][v * 4 + 2] = x.z; q.w[j][v * 4 + 3] = x.w;
        } else {
          q.w[j][v * 4 + 0] = x.x; q.w[j][v * 4 + 1] = x.y;
          q.w[j][v * 4 + 2] = x.z; q.w[j][v * 4 + 3] = x.w;
        }
      }
    }
  }

  float m[GC], l[GC], acc[GC][EPL];
#pragma unroll
  for (int j = 0; j < GC; ++j) {
    m[j] = kNegInf;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[j][e] = 0.f;
  }

  const uint4* kc = reinterpret_cast<const uint4*>(a.k_cache);
  const uint4* vc = reinterpret_cast<const uint4*>(a.v_cache);
  const size_t head_vecs = (size_t)kBlock * Sh::kRowVec;
  auto block_base = [&](int j) -> size_t {
    const int blk = __builtin_amdgcn_readlane(my_tbl, j);
    return ((size_t)blk * a.h_kv + kvh) * head_vecs;
  };
  auto attend_tail = [&](const BlockRegs<NP>& r, int j) {
    const int valid = tok1 - (blk0 + j) * kBlock;
    if (valid >= kBlock)
      attend_block<T, D, GC, false>(r, q, m, l, acc, a.scale_log2, slot, kBlock);
    else
      attend_block<T, D, GC, true>(r, q, m, l, acc, a.scale_log2, slot, valid);
  };

  int j = wave;
  if (j < nblk) {
    BlockRegs<NP> A, Bv;
    size_t base = block_base(j);
    load_block<T, D>(A, kc + base, vc + base, slot, sub);
    // Blocks before the last one of the partition are always full.
    while (j + 2 * W < nblk) {
      base = block_base(j + W);
      load_block<T, D>(Bv, kc + base, vc + base, slot, sub);
      attend_block<T, D, GC, false>(A, q, m, l, acc, a.scale_log2, slot, kBlock);
      base = block_base(j + 2 * W);
      load_block<T, D>(A, kc + base, vc + base, slot, sub);
      attend_block<T, D, GC, false>(Bv, q, m, l, acc, a.scale_log2, slot, kBlock);
      j += 2 * W;
    }
    if (j + W < nblk) {
      base = block_base(j + W);
      load_block<T, D>(Bv, kc + base, vc + base, slot, sub);
      attend_block<T, D, GC, false>(A, q, m, l, acc, a.scale_log2, slot, kBlock);
      attend_tail(Bv, j + W);
    } else {
      attend_tail(A, j);
    }
  }

  // Merge the lanes' states: lanes with the same sub hold the same channels.
#pragma unroll
  for (int jh = 0; jh < GC; ++jh) {
    const float M = class_max<Sh::kLPT>(m[jh]);
    const float f = m[jh] == kNegInf ? 0.f : fast_exp2(m[jh] - M);
    const float ls = class_sum<Sh::kLPT>(l[jh] * f);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[jh][e] = class_sum<Sh::kLPT>(acc[jh][e] * f);
    if (slot == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int v = e / Sh::kEPV;
        const int dim = (v * Sh::kLPT + sub) * Sh::kEPV + e % Sh::kEPV;
        s_acc[wave][jh][dim] = acc[jh][e];
      }
    }
    if (lane == 0) {
      s_m[wave][jh] = M;
      s_l[wave][jh] = ls;
    }
  }
  __syncthreads();

  for (int i = threadIdx.x; i < nh * D; i += blockDim.x) {
    const int jh = i / D;
    const int dim = i - jh * D;
    float Mx = kNegInf;
#pragma unroll
    for (int w = 0; w < W; ++w) Mx = fmaxf(Mx, s_m[w][jh]);
    float o = 0.f, lt = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = s_m[w][jh];
      const float f = mw == kNegInf ? 0.f : fast_exp2(mw - Mx);
      o = fmaf(f, s_acc[w][jh][dim], o);
      lt = fmaf(f, s_l[w][jh], lt);
    }
    const size_t row = (size_t)b * a.h_q + head0 + jh;
    if (n_part == 1) {
      store_elem<T>(out, row * D + dim, o / lt);
    } else {
      const size_t pi = row * a.num_partitions + part;
      a.ws_acc[pi * D + dim] = o;
      if (dim == 0) {
        a.ws_ml[pi * 2] = Mx;
        a.ws_ml[pi * 2 + 1] = lt;
      }
    }
  }
}

// Log-sum-exp merge of the partitions of one (sequence, query head).
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  int L = a.context_lens[b];
  L = max(0, min(L, min(a.max_blocks_per_seq * kBlock, a.num_partitions * a.partition_tokens)));
  const int n_part = (L + a.partition_tokens - 1) / a.partition_tokens;
  if (n_part <= 1) return;
  const size_t row = (size_t)b * a.h_q + h;
  const float* ml = a.ws_ml + row * a.num_partitions * 2;
  const float* pacc = a.ws_acc + row * a.num_partitions * D;
  float Mx = kNegInf;
  for (int p = 0; p < n_part; ++p) Mx = fmaxf(Mx, ml[2 * p]);
  float lt = 0.f;
  for (int p = 0; p < n_part; ++p) lt = fmaf(fast_exp2(ml[2 * p] - Mx), ml[2 * p + 1], lt);
  const float inv = 1.f / lt;
  T* out = reinterpret_cast<T*>(a.out);
  for (int dim = threadIdx.x; dim < D; dim += blockDim.x) {
    float o = 0.f;
    for (int p = 0; p < n_part; ++p) o = fmaf(fast_exp2(ml[2 * p] - Mx), pacc[(size_t)p * D + dim], o);
    store_elem<T>(out, row * D + dim, o * inv);
  }
}

template <typename T, int D, int GC>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.num_partitions, a.h_kv * a.n_chunks, a.B);
  hipLaunchKernelGGL((decode_partial_kernel<T, D, GC>), grid, dim3(256), 0, stream, a);
  if (a.num_partitions > 1)
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(a.h_q, a.B), dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_gc(const DecodeArgs& a, int gc, hipStream_t stream) {
  switch (gc) {
    case 1: return launch_t<T, D, 1>(a, stream);
    case 2: return launch_t<T, D, 2>(a, stream);
    case 3: return launch_t<T, D, 3>(a, stream);
    case 4: return launch_t<T, D, 4>(a, stream);
    case 5: return launch_t<T, D, 5>(a, stream);
    case 6: return launch_t<T, D, 6>(a, stream);
    case 7: return launch_t<T, D, 7>(a, stream);
    case 8: return launch_t<T, D, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, int d_h, bool bf16, hipStream_t stream) {
  const int gc = head_chunks(a.g).per_chunk;
  if (bf16) {
    if (d_h == 64) return launch_gc<bf16_t, 64>(a, gc, stream);
    if (d_h == 128) return launch_gc<bf16_t, 128>(a, gc, stream);
  } else {
    if (d_h == 64) return launch_gc<float, 64>(a, gc, stream);
    if (d_h == 128) return launch_gc<float, 128>(a, gc, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
