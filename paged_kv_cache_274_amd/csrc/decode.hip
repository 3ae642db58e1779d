// Paged decode attention for gfx950: wave-level even split of the whole batch.
//
// Single-token decode over the cached context of a continuous batch of
// variable-length sequences (LLM Inference Server page, Stage 1 prefill/decode
// task; "What you build" of the From Scratch page), with grouped-query heads
// and 16-token blocks behind a per-sequence block table (Paged KV-Cache Block
// Allocator stretch challenge; Block Manager box of the pipeline figure).
// Decode is bound by reading the KV cache from HBM ("What You Will Build",
// LLM Inference Server page): the design streams every K/V byte once, with the
// whole chip busy from the first to the last cycle.
//
// Work decomposition
//  * A segment is (sequence b, KV head, chunk of <= 8 query heads of its GQA
//    group); it owns the ceil(L_b / 16) blocks of that KV head.  All segments'
//    blocks are laid end to end (sequence-major) and the line is cut into
//    num_splits contiguous ranges, one per wavefront, sized by the speed of
//    the XCD the wavefront runs on (line.h).  With num_splits = the number of
//    wavefronts the chip holds at once, every wave starts at once, does its
//    share of blocks whatever the length mix, and finishes with the others;
//    there is no per-partition prologue or tail.
//  * A wave walks its range block by block, crossing segment boundaries.  Each
//    K/V block of a KV head is read once for all query heads of the chunk.
//    A segment finished inside one wave is normalised and stored directly; a
//    segment cut by a range boundary leaves an unnormalised partial state
//    (max, sum, accumulator) in the workspace, at most two per wave, and the
//    combine kernel merges them with the exact log-sum-exp rule.
//
// Inside a wave
//  * kLPT adjacent lanes cover one token row with 16-byte loads (16 lanes for
//    bf16 rows of 128 channels, 8 otherwise), so a load instruction reads
//    64 / kLPT tokens and a block takes two or four passes.  The next block's
//    loads are in flight while the current one is used.
//  * An INT8 cache keeps the bf16 lane mapping with 8 code bytes per lane and
//    token, widened exactly to bf16 in registers; the token's K scale
//    multiplies its score and its V scale the softmax weight.
//  * q.K partial sums are combined across the lanes of a token by DPP row
//    permutations (no LDS).  bf16 products use v_dot2_f32_bf16; for P.V the
//    two tokens a lane holds are paired so that one v_dot2 adds both
//    (weights rounded to bf16, accumulation in fp32).  fp32 inputs use fp32 FMAs.
//  * Online softmax in base 2 (scale * log2(e) folded into the score).  Each
//    lane keeps its own reference max, sum and accumulators for its tokens; the
//    reference only moves when a score exceeds it by more than 2^8, so the
//    accumulators are rarely rescaled.  The lanes' states are merged exactly at
//    the end of each segment piece.
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "line.h"

namespace pkv {

constexpr float kRescaleSlack = 8.0f;  // log2 units

constexpr float kNegInf = -__builtin_huge_valf();

// Lane mapping.  A token row of D elements is covered by kLPT adjacent lanes,
// each holding kVPL 16-byte vectors of it; one load instruction covers kTPW
// tokens and a 16-token block takes kPasses passes.  bf16 rows of 128 channels
// use 16 lanes (8 channels per lane) so that the per-lane accumulators and
// query words stay small enough for three wavefronts per SIMD; other rows use 8.
template <typename T, int D>
struct DecodeShape {
  static constexpr int kElem = sizeof(T);
  static constexpr int kRowVec = D * kElem / 16;   // 16-byte vectors per token row
  static constexpr int kLPT = (kElem == 2 && kRowVec >= 16) ? 16 : 8;
  static constexpr int kVPL = kRowVec / kLPT;
  static constexpr int kEPV = 16 / kElem;          // elements per vector
  static constexpr int kEPL = kVPL * kEPV;         // elements a lane holds of one token
  static constexpr int kTPW = kWave / kLPT;        // tokens one wave covers per pass
  static constexpr int kPasses = kBlock / kTPW;    // passes per 16-token block (2 or 4)
  static_assert(kVPL >= 1 && kPasses % 2 == 0, "lane mapping");
};

// INT8 cache (codes with one float32 scale per token head row) read by bf16
// queries: the lane mapping, query words and accumulators are those of bf16
// rows of the same width, so a lane holds 8 channels (8 bytes) of a token row.
struct i8_t {};
template <int D>
struct DecodeShape<i8_t, D> : DecodeShape<bf16_t, D> {};

// Element type of q and out: the cache's own, bf16 for an INT8 cache.
template <typename T>
using OutOf = typename std::conditional<std::is_same<T, i8_t>::value, bf16_t, T>::type;

template <int NP, int VPL>
struct BlockRegs {
  uint4 k[NP][VPL];
  uint4 v[NP][VPL];
};

// An INT8 block as one lane holds it: 8 codes of K and of V per pass, and the
// scales of the pass's token.  In an INT8 block the lanes of slot s hold the
// NP consecutive tokens s * NP .. s * NP + NP - 1 (pass ps: token s * NP + ps),
// so their scales are one contiguous load.
template <int NP>
struct BlockRegsI8 {
  uint2 k[NP];
  uint2 v[NP];
  float ks[NP];
  float vs[NP];
};
template <typename T, int D>
__device__ __forceinline__ int token_of(int ps, int slot) {
  using Sh = DecodeShape<T, D>;
  return std::is_same<T, i8_t>::value ? slot * Sh::kPasses + ps : ps * Sh::kTPW + slot;
}

__device__ __forceinline__ uint32_t dw(const uint4& u, int w) {
  return w == 0 ? u.x : (w == 1 ? u.y : (w == 2 ? u.z : u.w));
}

// Channel held by element e of a lane with in-row index sub.
template <typename T, int D>
__device__ __forceinline__ int lane_channel(int sub, int e) {
  using Sh = DecodeShape<T, D>;
  return ((e / Sh::kEPV) * Sh::kLPT + sub) * Sh::kEPV + e % Sh::kEPV;
}

template <typename T, int D>
struct BlockSel {
  using type = BlockRegs<DecodeShape<T, D>::kPasses, DecodeShape<T, D>::kVPL>;
};
template <int D>
struct BlockSel<i8_t, D> {
  static_assert(DecodeShape<i8_t, D>::kVPL == 1, "one 8-byte chunk per lane and token");
  using type = BlockRegsI8<DecodeShape<i8_t, D>::kPasses>;
};
template <typename T, int D>
using BlockOf = typename BlockSel<T, D>::type;

// K/V are read exactly once per call, so they are loaded with the non-temporal
// hint: on MI355X this streams them past the caches' normal allocation and
// lifts the sustained read bandwidth of this access pattern by about 13%.
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}

__device__ __forceinline__ uint2 stream_load(const uint2* p) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(x.x, x.y);
}

// Loads one 16-token block of one KV head; bh = physical block * h_kv + KV head.
template <typename T, int D>
__device__ __forceinline__ void load_block(BlockOf<T, D>& r, const DecodeArgs& a, size_t bh,
                                           int slot, int sub) {
  using Sh = DecodeShape<T, D>;
  if constexpr (std::is_same<T, i8_t>::value) {
    constexpr int kRow = D / 8;  // 8-byte chunks per row of codes
    const uint2* kbase = reinterpret_cast<const uint2*>(a.k_cache) + bh * (kBlock * kRow);
    const uint2* vbase = reinterpret_cast<const uint2*>(a.v_cache) + bh * (kBlock * kRow);
#pragma unroll
    for (int ps = 0; ps < Sh::kPasses; ++ps)
      r.k[ps] = stream_load(&kbase[token_of<T, D>(ps, slot) * kRow + sub]);
#pragma unroll
    for (int ps = 0; ps < Sh::kPasses; ++ps)
      r.v[ps] = stream_load(&vbase[token_of<T, D>(ps, slot) * kRow + sub]);
    static_assert(Sh::kPasses == 2 || Sh::kPasses == 4, "scales as one 8- or 16-byte load");
    const float* ksp = a.k_scale + bh * kBlock + slot * Sh::kPasses;
    const float* vsp = a.v_scale + bh * kBlock + slot * Sh::kPasses;
    if constexpr (Sh::kPasses == 4) {
      const float4 k4 = *reinterpret_cast<const float4*>(ksp);
      const float4 v4 = *reinterpret_cast<const float4*>(vsp);
      r.ks[0] = k4.x; r.ks[1] = k4.y; r.ks[2] = k4.z; r.ks[3] = k4.w;
      r.vs[0] = v4.x; r.vs[1] = v4.y; r.vs[2] = v4.z; r.vs[3] = v4.w;
    } else {
      const float2 k2 = *reinterpret_cast<const float2*>(ksp);
      const float2 v2 = *reinterpret_cast<const float2*>(vsp);
      r.ks[0] = k2.x; r.ks[1] = k2.y;
      r.vs[0] = v2.x; r.vs[1] = v2.y;
    }
  } else {
    const size_t head_vecs = (size_t)kBlock * Sh::kRowVec;
    const uint4* __restrict__ kbase = reinterpret_cast<const uint4*>(a.k_cache) + bh * head_vecs;
    const uint4* __restrict__ vbase = reinterpret_cast<const uint4*>(a.v_cache) + bh * head_vecs;
#pragma unroll
    for (int ps = 0; ps < Sh::kPasses; ++ps)
#pragma unroll
      for (int v = 0; v < Sh::kVPL; ++v)
        r.k[ps][v] =
            stream_load(&kbase[(ps * Sh::kTPW + slot) * Sh::kRowVec + v * Sh::kLPT + sub]);
#pragma unroll
    for (int ps = 0; ps < Sh::kPasses; ++ps)
#pragma unroll
      for (int v = 0; v < Sh::kVPL; ++v)
        r.v[ps][v] =
            stream_load(&vbase[(ps * Sh::kTPW + slot) * Sh::kRowVec + v * Sh::kLPT + sub]);
  }
}

// Codes c0 (low half) and c1 (high half) as a bf16 pair, exactly: an int8 code
// converts to float32 without rounding and, being at most 7 significant bits,
// its float32 pattern ends in 16 zero bits, so the high halves are the bf16
// values.
__device__ __forceinline__ uint32_t i8_pair_bf16(int c0, int c1) {
  return __builtin_amdgcn_perm(__float_as_uint((float)c1), __float_as_uint((float)c0),
                               0x07060302u);
}
// Code k (0..7) of an 8-byte chunk, sign-extended.
__device__ __forceinline__ int i8_code(const uint2& u, int k) {
  const uint32_t w = k < 4 ? u.x : u.y;
  return (int)(int8_t)(w >> (8 * (k & 3)));
}

// Query registers: bf16 kept packed for v_dot2, fp32 kept as floats (4 words per vector).
// For an INT8 cache the words become f16 pairs of q * 2^-k (see q_for_codes),
// with the bias correction of each head and the score factor scale * log2(e) * 2^k.
template <int GC, int VPL>
struct QRegs {
  uint32_t w[GC][VPL * 4];
  float bias[GC];
  float sfac;
};

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// INT8 cache: K codes widen to f16 in one byte permutation per pair.  The
// biased byte u = c + 128 (c ^ 0x80) below an exponent byte 0x64 is the f16
// value 1024 + u = 1152 + c, exactly, so q . K = q . (1152 + c) - 1152 * sum(q):
// the scores start from the lane's share of -1152 * sum(q) instead of 0.  The
// products then need q in f16: q (bf16) is scaled by the power of two 2^-k
// that brings its largest magnitude over the wave into [2^14, 2^15), which
// keeps every bf16 value exact in f16 down to 2^-29 of that maximum, and 2^k
// joins the score factor.  (The widening through float32 conversions costs
// about twice as many instructions per code; measured on the Llama-3-8B-shaped
// batch, 77.1 -> 73.8 us per call.)
// The f16 widening is used for chunks of at most 4 heads: with more, its
// registers would cost the kernel its second wave per SIMD.
template <typename T, int GC>
constexpr bool kF16Codes = std::is_same<T, i8_t>::value && GC <= 4;

template <int GC, int VPL>
__device__ __forceinline__ void q_for_codes(QRegs<GC, VPL>& q, float scale_log2) {
  float mx = 0.f;
#pragma unroll
  for (int j = 0; j < GC; ++j)
#pragma unroll
    for (int x = 0; x < VPL * 4; ++x)
      mx = fmaxf(mx, fmaxf(fabsf(__uint_as_float(q.w[j][x] << 16)),
                           fabsf(__uint_as_float(q.w[j][x] & 0xffff0000u))));
  mx = wave_max(mx);
  const int k = mx > 0.f ? __builtin_amdgcn_frexp_expf(mx) - 15 : 0;
  const float down = __builtin_amdgcn_ldexpf(1.f, -k);
#pragma unroll
  for (int j = 0; j < GC; ++j) {
    float sum = 0.f;
#pragma unroll
    for (int x = 0; x < VPL * 4; ++x) {
      const float lo = __uint_as_float(q.w[j][x] << 16) * down;
      const float hi = __uint_as_float(q.w[j][x] & 0xffff0000u) * down;
      sum += lo + hi;
      q.w[j][x] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
    }
    q.bias[j] = -1152.f * sum;
  }
  q.sfac = __builtin_amdgcn_ldexpf(scale_log2, k);
}



// Folds one block into the lane's running (m, l, acc).  MASK: tokens at local
// index >= valid lie past the context; their scores and values are ignored,
// whatever the pool holds there.
template <typename T, int D, int GC, bool MASK>
__device__ __forceinline__ void attend_block(const BlockOf<T, D>& r,
                                             const QRegs<GC, DecodeShape<T, D>::kVPL>& q,
                                             float (&m)[GC], float (&l)[GC],
                                             float (&acc)[GC][DecodeShape<T, D>::kEPL],
                                             float scale_log2, int slot, int valid) {
  using Sh = DecodeShape<T, D>;
  constexpr int NP = Sh::kPasses;
  constexpr int VPL = Sh::kVPL;
  constexpr int EPL = Sh::kEPL;
  // q.K for the lane's NP tokens and every head: the NP * GC dot products are
  // accumulated word by word in interleaved order so that no accumulator is
  // used by two consecutive instructions, then reduced across the kLPT lanes
  // of a token step by step, again interleaved.
  float s[NP][GC];
#pragma unroll
  for (int ps = 0; ps < NP; ++ps)
#pragma unroll
    for (int j = 0; j < GC; ++j) s[ps][j] = kF16Codes<T, GC> ? q.bias[j] : 0.f;
#pragma unroll
  for (int v = 0; v < VPL; ++v)
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int ps = 0; ps < NP; ++ps) {
        uint32_t kw;
        if constexpr (kF16Codes<T, GC>)
          kw = __builtin_amdgcn_perm(0x64646464u, ((w < 2) ? r.k[ps].x : r.k[ps].y) ^ 0x80808080u,
                                     (w & 1) ? 0x04030402u : 0x04010400u);
        else if constexpr (std::is_same<T, i8_t>::value)
          kw = i8_pair_bf16(i8_code(r.k[ps], 2 * w), i8_code(r.k[ps], 2 * w + 1));
        else
          kw = dw(r.k[ps][v], w);
#pragma unroll
        for (int j = 0; j < GC; ++j) {
          if constexpr (std::is_same<T, float>::value)
            s[ps][j] = fmaf(__uint_as_float(q.w[j][v * 4 + w]), __uint_as_float(kw), s[ps][j]);
          else if constexpr (kF16Codes<T, GC>)
            s[ps][j] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, kw),
                                              __builtin_bit_cast(f16x2_t, q.w[j][v * 4 + w]),
                                              s[ps][j], false);
          else
            s[ps][j] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, kw),
                                                       __builtin_bit_cast(bf16x2_t, q.w[j][v * 4 + w]),
                                                       s[ps][j], false);
        }
      }
#pragma unroll
  for (int ps = 0; ps < NP; ++ps)
#pragma unroll
    for (int j = 0; j < GC; ++j) s[ps][j] += dpp<kDppXor1>(s[ps][j]);
#pragma unroll
  for (int ps = 0; ps < NP; ++ps)
#pragma unroll
    for (int j = 0; j < GC; ++j) s[ps][j] += dpp<kDppXor2>(s[ps][j]);
#pragma unroll
  for (int ps = 0; ps < NP; ++ps)
#pragma unroll
    for (int j = 0; j < GC; ++j) s[ps][j] += dpp<kDppRowHalfMirror>(s[ps][j]);
  if constexpr (Sh::kLPT == 16) {
#pragma unroll
    for (int ps = 0; ps < NP; ++ps)
#pragma unroll
      for (int j = 0; j < GC; ++j) s[ps][j] += dpp<kDppRowMirror>(s[ps][j]);
  }
  bool ok[NP];
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
    ok[ps] = !MASK || (token_of<T, D>(ps, slot) < valid);
    float f = scale_log2;
    if constexpr (kF16Codes<T, GC>) f = r.ks[ps] * q.sfac;  // the token's K scale
    else if constexpr (std::is_same<T, i8_t>::value) f = r.ks[ps] * scale_log2;
#pragma unroll
    for (int j = 0; j < GC; ++j) s[ps][j] = (MASK && !ok[ps]) ? kNegInf : s[ps][j] * f;
  }
  bool need = false;
  float smax[GC];
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
    }
#pragma unroll
  for (int j = 0; j < GC; ++j) {
    float t = p[0][j];
#pragma unroll
    for (int ps = 1; ps < NP; ++ps) t += p[ps][j];
    l[j] += t;
  }

  if constexpr (std::is_same<T, float>::value) {
#pragma unroll
    for (int ps = 0; ps < NP; ++ps) {
      if (MASK && !ok[ps]) continue;
#pragma unroll
      for (int v = 0; v < VPL; ++v)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float x = __uint_as_float(dw(r.v[ps][v], w));
#pragma unroll
          for (int j = 0; j < GC; ++j) acc[j][v * 4 + w] = fmaf(p[ps][j], x, acc[j][v * 4 + w]);
        }
    }
  } else if constexpr (std::is_same<T, i8_t>::value) {
    // As for bf16 rows, tokens are paired (passes 2i, 2i+1); each weight carries
    // its token's V scale (p * s_v, rounded to bf16 once), and the codes of the
    // two tokens at one channel form an exact bf16 pair.  A masked token's
    // weight is zero whatever its scale slot holds.
#pragma unroll
    for (int pr = 0; pr < NP / 2; ++pr) {
      uint32_t pp[GC];
#pragma unroll
      for (int j = 0; j < GC; ++j) {
        float p0 = p[2 * pr][j] * r.vs[2 * pr];
        float p1 = p[2 * pr + 1][j] * r.vs[2 * pr + 1];
        if (MASK) {
          p0 = ok[2 * pr] ? p0 : 0.f;
          p1 = ok[2 * pr + 1] ? p1 : 0.f;
        }
        pp[j] = pack_bf16x2(p0, p1);
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t x = i8_pair_bf16(i8_code(r.v[2 * pr], c), i8_code(r.v[2 * pr + 1], c));
#pragma unroll
        for (int j = 0; j < GC; ++j)
          acc[j][c] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pp[j]),
                                                      __builtin_bit_cast(bf16x2_t, x), acc[j][c],
                                                      false);
      }
    }
  } else {
    // Tokens are paired (passes 2i, 2i+1): word (V_t0[c], V_t1[c]) against
    // (p_t0, p_t1), so one v_dot2 adds both tokens' contributions.
#pragma unroll
    for (int pr = 0; pr < NP / 2; ++pr) {
      uint32_t pp[GC];
#pragma unroll
      for (int j = 0; j < GC; ++j) pp[j] = pack_bf16x2(p[2 * pr][j], p[2 * pr + 1][j]);
#pragma unroll
      for (int v = 0; v < VPL; ++v)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t x0 = dw(r.v[2 * pr][v], w), x1 = dw(r.v[2 * pr + 1][v], w);
          if (MASK) {
            x0 = ok[2 * pr] ? x0 : 0u;
            x1 = ok[2 * pr + 1] ? x1 : 0u;
          }
          const uint32_t lo = __builtin_amdgcn_perm(x1, x0, 0x05040100u);  // channel 2w
          const uint32_t hi = __builtin_amdgcn_perm(x1, x0, 0x07060302u);  // channel 2w+1
#pragma unroll
          for (int j = 0; j < GC; ++j) {
            acc[j][v * 8 + 2 * w] = __builtin_amdgcn_fdot2_f32_bf16(
                __builtin_bit_cast(bf16x2_t, pp[j]), __builtin_bit_cast(bf16x2_t, lo),
                acc[j][v * 8 + 2 * w], false);
            acc[j][v * 8 + 2 * w + 1] = __builtin_amdgcn_fdot2_f32_bf16(
                __builtin_bit_cast(bf16x2_t, pp[j]), __builtin_bit_cast(bf16x2_t, hi),
                acc[j][v * 8 + 2 * w + 1], false);
          }
        }
    }
  }
}

// INT8 cache, d_h = 128, chunks of 4 heads: a row of 16 lanes shares 4 tokens
// (one per pass) and forms 16 partial scores per lane, one per (pass, head).
// attend_block sums each across the row (4 DPP steps for each of the 16) and
// then every lane repeats the same scaling, exponential and sum for all 16.
// Here the row's partial scores are reduce-scattered instead, so that lane i
// of the row ends with the full score of one (pass, head) pair: 45
// instructions for the sum, then one scale, one exponential and one sum term
// per lane; the P.V weights return to every lane of the row as 8 packed bf16
// pairs by row broadcasts.  The running maximum m[j] stays replicated across
// the row; m_sel is this lane's head's copy, and l_slot the lane's share of
// its head's sum, combined into l[j] at the end of a piece (rs_finish_sum).
template <typename T, int D, int GC>
constexpr bool kScatterScores =
    (std::is_same<T, i8_t>::value || std::is_same<T, bf16_t>::value) && D == 128 && GC == 4;

// Index of the (pass ps, head j) score in the scatter order; lane i of a row
// ends with index i, so pass 2i and 2i + 1 of a head (the two weights one P.V
// word pairs) sit one lane apart.
__device__ constexpr int rs_index(int ps, int j) { return 8 * (ps >> 1) + 2 * j + (ps & 1); }

// One level of the reduce-scatter: v[0 .. 2n-1] becomes v[0 .. n-1], the half
// this lane keeps (the upper one if hi) summed with the partner's copy of it;
// the partner (DPP control CTRL) keeps the other half.
template <int CTRL, int N>
__device__ __forceinline__ void rs_level(float (&v)[16], bool hi) {
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const float keep = hi ? v[k + N] : v[k];
    const float send = hi ? v[k] : v[k + N];
    v[k] = keep + dpp<CTRL>(send);
  }
}

// The entry of four values that belongs to this lane's pass (2 * b3 + b0),
// chosen by selects on values: each passes through an empty asm first, so
// that the selects are not folded into one dynamically indexed read of the
// block's registers, which would move the whole block to scratch memory.
__device__ __forceinline__ float pick_pass(const float (&x)[4], bool b3, bool b0) {
  float x0 = x[0], x1 = x[1], x2 = x[2], x3 = x[3];
  asm("" : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3));
  return b3 ? (b0 ? x3 : x2) : (b0 ? x1 : x0);
}

template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + N, 0xf, 0xf, false));
}
template <int N>
__device__ __forceinline__ uint32_t row_bcast_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x150 + N, 0xf, 0xf, false);
}

template <typename T, int D, int GC, bool MASK>
__device__ __forceinline__ void attend_block_rs(const BlockOf<T, D>& r,
                                                const QRegs<GC, DecodeShape<T, D>::kVPL>& q,
                                                float (&m)[GC], float& m_sel, float& l_slot,
                                                float (&acc)[GC][DecodeShape<T, D>::kEPL],
                                                float scale_log2, int slot, int valid, int i16) {
  constexpr int NP = DecodeShape<T, D>::kPasses;
  constexpr bool kI8 = std::is_same<T, i8_t>::value;
  static_assert(NP == 4 && GC == 4 && DecodeShape<T, D>::kVPL == 1, "16 scores over 16 lanes");
  float v[16];
#pragma unroll
  for (int ps = 0; ps < NP; ++ps)
#pragma unroll
    for (int j = 0; j < GC; ++j) v[rs_index(ps, j)] = kI8 ? q.bias[j] : 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int ps = 0; ps < NP; ++ps) {
      if constexpr (kI8) {
        const uint32_t kw = __builtin_amdgcn_perm(
            0x64646464u, ((w < 2) ? r.k[ps].x : r.k[ps].y) ^ 0x80808080u,
            (w & 1) ? 0x04030402u : 0x04010400u);
#pragma unroll
        for (int j = 0; j < GC; ++j)
          v[rs_index(ps, j)] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, kw),
                                                      __builtin_bit_cast(f16x2_t, q.w[j][w]),
                                                      v[rs_index(ps, j)], false);
      } else {
        const uint32_t kw = dw(r.k[ps][0], w);
#pragma unroll
        for (int j = 0; j < GC; ++j)
          v[rs_index(ps, j)] = __builtin_amdgcn_fdot2_f32_bf16(
              __builtin_bit_cast(bf16x2_t, kw), __builtin_bit_cast(bf16x2_t, q.w[j][w]),
              v[rs_index(ps, j)], false);
      }
    }
  const bool b3 = i16 & 8, b2 = i16 & 4, b1 = i16 & 2, b0 = i16 & 1;
  rs_level<kDppRowMirror, 8>(v, b3);
  rs_level<kDppRowHalfMirror, 4>(v, b2);
  rs_level<kDppXor2, 2>(v, b1);
  rs_level<kDppXor1, 1>(v, b0);
  // This lane's score: pass ps = 2 * b3 + b0, head (i16 >> 1) & 3.  An INT8
  // score takes its token's K scale and the query's power of two.
  const int ps = 2 * b3 + b0;
  float x;
  if constexpr (kI8)
    x = v[0] * (pick_pass(r.ks, b3, b0) * q.sfac);
  else
    x = v[0] * scale_log2;
  const bool ok = !MASK || token_of<T, D>(ps, slot) < valid;
  if (MASK) x = ok ? x : kNegInf;
  if (__any(x > m_sel + kRescaleSlack)) {
    // The row's maximum of this lane's head over the 4 passes (lanes i, i ^ 1,
    // i ^ 8, i ^ 9), the lazy rescale of attend_block, and the new maxima and
    // factors sent to every lane of the row for the accumulators.
    float mx = fmaxf(x, dpp<kDppXor1>(x));
    mx = fmaxf(mx, dpp<kDppRowRor8>(mx));
    const float mn = mx > m_sel + kRescaleSlack ? mx : m_sel;
    const float alpha = mn == m_sel ? 1.f : fast_exp2(m_sel - mn);
    m_sel = mn;
    l_slot *= alpha;
    const float al[4] = {row_bcast<0>(alpha), row_bcast<2>(alpha), row_bcast<4>(alpha),
                         row_bcast<6>(alpha)};
    m[0] = row_bcast<0>(mn);
    m[1] = row_bcast<2>(mn);
    m[2] = row_bcast<4>(mn);
    m[3] = row_bcast<6>(mn);
#pragma unroll
    for (int j = 0; j < GC; ++j)
#pragma unroll
      for (int e = 0; e < DecodeShape<T, D>::kEPL; ++e) acc[j][e] *= al[j];
  }
  float p = fast_exp2(x - m_sel);
  if (MASK) p = ok ? p : 0.f;
  l_slot += p;
  // An INT8 weight carries the token's V scale (a masked token's weight is
  // zero whatever its scale slot holds); the weight is rounded to bf16 once,
  // in the pair with the next pass's weight; even lanes hold the pairs.
  float w = p;
  if constexpr (kI8) w = p * pick_pass(r.vs, b3, b0);
  if (MASK) w = ok ? w : 0.f;
  const uint32_t pk = pack_bf16x2(w, dpp<kDppXor1>(w));
  uint32_t pp[2][GC];
  pp[0][0] = row_bcast_u<0>(pk);
  pp[0][1] = row_bcast_u<2>(pk);
  pp[0][2] = row_bcast_u<4>(pk);
  pp[0][3] = row_bcast_u<6>(pk);
  pp[1][0] = row_bcast_u<8>(pk);
  pp[1][1] = row_bcast_u<10>(pk);
  pp[1][2] = row_bcast_u<12>(pk);
  pp[1][3] = row_bcast_u<14>(pk);
  if constexpr (kI8) {
#pragma unroll
    for (int pr = 0; pr < NP / 2; ++pr)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t xv = i8_pair_bf16(i8_code(r.v[2 * pr], c), i8_code(r.v[2 * pr + 1], c));
#pragma unroll
        for (int j = 0; j < GC; ++j)
          acc[j][c] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pp[pr][j]),
                                                      __builtin_bit_cast(bf16x2_t, xv), acc[j][c],
                                                      false);
      }
  } else {
    // Tokens of passes 2pr and 2pr + 1 paired per channel, as in attend_block;
    // V rows past the context are zeroed, since a zero weight times a NaN is NaN.
    const bool ok0 = !MASK || token_of<T, D>(0, slot) < valid;
    const bool ok1 = !MASK || token_of<T, D>(1, slot) < valid;
    const bool ok2 = !MASK || token_of<T, D>(2, slot) < valid;
    const bool ok3 = !MASK || token_of<T, D>(3, slot) < valid;
    const bool okp[4] = {ok0, ok1, ok2, ok3};
#pragma unroll
    for (int pr = 0; pr < NP / 2; ++pr)
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        uint32_t x0 = dw(r.v[2 * pr][0], w4), x1 = dw(r.v[2 * pr + 1][0], w4);
        if (MASK) {
          x0 = okp[2 * pr] ? x0 : 0u;
          x1 = okp[2 * pr + 1] ? x1 : 0u;
        }
        const uint32_t lo = __builtin_amdgcn_perm(x1, x0, 0x05040100u);  // channel 2w
        const uint32_t hi = __builtin_amdgcn_perm(x1, x0, 0x07060302u);  // channel 2w+1
#pragma unroll
        for (int j = 0; j < GC; ++j) {
          acc[j][2 * w4] = __builtin_amdgcn_fdot2_f32_bf16(
              __builtin_bit_cast(bf16x2_t, pp[pr][j]), __builtin_bit_cast(bf16x2_t, lo),
              acc[j][2 * w4], false);
          acc[j][2 * w4 + 1] = __builtin_amdgcn_fdot2_f32_bf16(
              __builtin_bit_cast(bf16x2_t, pp[pr][j]), __builtin_bit_cast(bf16x2_t, hi),
              acc[j][2 * w4 + 1], false);
        }
      }
  }
}

// The row's sums per head from the lanes' shares: l[j] on every lane of the row.
template <int GC>
__device__ __forceinline__ void rs_finish_sum(float l_slot, float (&l)[GC]) {
  float t = l_slot + dpp<kDppXor1>(l_slot);
  t += dpp<kDppRowRor8>(t);
  l[0] = row_bcast<0>(t);
  l[1] = row_bcast<2>(t);
  l[2] = row_bcast<4>(t);
  l[3] = row_bcast<6>(t);
}

template <typename T>
__device__ __forceinline__ void store_elem(T* out, size_t i, float x) {
  if constexpr (std::is_same<T, float>::value)
    out[i] = x;
  else
    reinterpret_cast<uint16_t*>(out)[i] = (uint16_t)f32_to_bf16_bits(x);
}

// Clamped context length: never beyond the block table row.
__device__ __forceinline__ int seq_len(const DecodeArgs& a, int b) {
  const int L = constant_view(a.context_lens)[b];
  return max(0, min(L, a.max_blocks_per_seq * kBlock));
}
__device__ __forceinline__ int seq_blocks(const DecodeArgs& a, int b) {
  return (seq_len(a, b) + kBlock - 1) / kBlock;
}

// Inclusive prefix sum over the wave's lanes (64-bit: 64 rows of up to 2^27
// blocks each can pass 2^31).
__device__ __forceinline__ int64_t wave_incl_scan(int64_t x, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int64_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Blocks of all sequences, read in chunks of 64 sequences (one per lane).
__device__ __forceinline__ int64_t total_blocks(const DecodeArgs& a, int lane) {
  int64_t total = 0;
  for (int c0 = 0; c0 < a.B; c0 += kWave) {
    const int bb = c0 + lane;
    const int64_t incl = wave_incl_scan(bb < a.B ? seq_blocks(a, bb) : 0, lane);
    total += uniform((int64_t)__shfl(incl, kWave - 1));
  }
  return total;
}

// Merges the partial states of head j of one segment cut by range boundaries
// with the exact log-sum-exp rule and stores the normalised result.  The pieces
// are wave wa's last-segment slot and the first-segment slots of the non-empty
// waves wa + 1 .. wb (all waves are non-empty when the line has at least three
// blocks per split).  Run by one whole wave.  The pieces' (max, sum) and the
// first kBatch pieces' accumulators are requested together, before any of them
// is used, so a merge of up to kBatch pieces costs one memory round trip
// (kBatch = 32 for a long context cut over many waves; 8 otherwise, which
// keeps the unrolled loads and sums short).
template <typename T, int D, int GC, int kBatch>
__device__ __forceinline__ void merge_segment_head(const DecodeArgs& a, const Line& line, int b,
                                                   int head0, int j, int wa, int wb, int lane) {
  const int np = wb - wa + 1;
  // Every wave's range is non-empty once the line holds 3 blocks per wave (the
  // lightest wave's share is then at least 3 * kWeightOdd / kWeightEven > 2).
  const bool all_live = line.total >= 3 * (int64_t)line.splits;
  constexpr int CPL = (D + kWave - 1) / kWave;  // channels per lane
  auto piece = [&](int k) -> const float* {
    return a.ws + ((size_t)((wa + k) * 2 + (k == 0 ? 1 : 0)) * GC + j) * (D + 2);
  };
  auto live = [&](int k) -> bool {
    return all_live || k == 0 || line.start(wa + k) < line.start(wa + k + 1);
  };
  auto load_batch = [&](int k0, uint64_t live_mask, float (&x)[kBatch][CPL]) {
#pragma unroll
    for (int t = 0; t < kBatch; ++t) {
      const bool use = k0 + t < np && ((live_mask >> (t & 63)) & 1);
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = lane + i * kWave;
        x[t][i] = (use && c < D) ? piece(k0 + t)[c] : 0.f;
      }
    }
  };
  float o[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) o[i] = 0.f;
  float inv;
  if (np <= kWave) {
    const bool lk = lane < np && live(lane);
    const uint64_t live_mask = __ballot(lk);
    const float mk = lk ? piece(lane)[D] : kNegInf;
    const float lv = lk ? piece(lane)[D + 1] : 0.f;
    float x[kBatch][CPL];
    load_batch(0, live_mask, x);
    const float M = wave_max(mk);
    const float wk = lk ? fast_exp2(mk - M) : 0.f;
    inv = 1.f / wave_sum(wk * lv);
    for (int k0 = 0; k0 < np; k0 += kBatch) {
      if (k0 > 0) load_batch(k0, live_mask >> k0, x);
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        const float w = __int_as_float(
            __builtin_amdgcn_readlane(__float_as_int(wk), min(k0 + t, kWave - 1)));
#pragma unroll
        for (int i = 0; i < CPL; ++i) o[i] = fmaf(w, x[t][i], o[i]);
      }
    }
  } else {
    float M = kNegInf;
    for (int k0 = 0; k0 < np; k0 += kWave) {
      const int k = k0 + lane;
      M = fmaxf(M, wave_max((k < np && live(k)) ? piece(k)[D] : kNegInf));
    }
    float ls = 0.f;
    for (int k0 = 0; k0 < np; k0 += kWave) {
      const int k = k0 + lane;
      const bool lk = k < np && live(k);
      const float wk = lk ? fast_exp2(piece(k)[D] - M) : 0.f;
      ls += wave_sum(lk ? wk * piece(k)[D + 1] : 0.f);
      const uint64_t live_mask = __ballot(lk);
      const int kn = min(kWave, np - k0);
      for (int t0 = 0; t0 < kn; t0 += kBatch) {
        float x[kBatch][CPL];
        load_batch(k0 + t0, t0 + kBatch <= kWave ? live_mask >> t0 : 0, x);
#pragma unroll
        for (int t = 0; t < kBatch; ++t) {
          const float w = __int_as_float(
              __builtin_amdgcn_readlane(__float_as_int(wk), min(t0 + t, kWave - 1)));
#pragma unroll
          for (int i = 0; i < CPL; ++i) o[i] = fmaf(t0 + t < kn ? w : 0.f, x[t][i], o[i]);
        }
      }
    }
    inv = 1.f / ls;
  }
  using O = OutOf<T>;
  O* out = reinterpret_cast<O*>(a.out) + ((size_t)b * a.h_q + head0 + j) * D;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + i * kWave;
    if (c < D) store_elem<O>(out, c, o[i] * inv);
  }
}

// A piece of a wave's range: blocks j0 .. j1-1 of segment (b, kc), whose block
// 0 sits at line position seg0.
struct Piece {
  int b, kc, j0, j1, nb;
  int64_t seg0;
  bool valid;
};

// The piece after p on a wave's range ending at e (wave-uniform).
__device__ __forceinline__ Piece next_piece(const DecodeArgs& a, int HC, const Piece& p, int64_t e) {
  Piece n = p;
  n.valid = false;
  if (p.seg0 + p.j1 >= e) return n;
  if (p.kc + 1 < HC) {
    n.kc = p.kc + 1;
    n.seg0 = p.seg0 + p.nb;
  } else {
    int b = p.b, nb = 0;
    do {
      ++b;
      nb = b < a.B ? seq_blocks(a, b) : 1;
    } while (nb == 0);
    if (b >= a.B) return n;  // only reachable if the lengths changed under the kernel
    n.b = b;
    n.kc = 0;
    n.nb = nb;
    n.seg0 = p.seg0 + p.nb;
  }
  n.j0 = 0;
  n.j1 = (int)min((int64_t)n.nb, e - n.seg0);
  n.valid = true;
  return n;
}

// Streams one wave's range of the line.  The K/V block pipeline runs through
// the whole range without draining at piece boundaries: the next piece's
// query registers and first table entry are requested when a piece starts, and
// its first block is loaded before the current piece's epilogue, whose
// reductions and stores then hide that load.  Table entries are read with
// scalar loads two blocks ahead, so they never hold up the vector loads.
template <typename T, int D, int GC>
struct RangeStream {
  using Sh = DecodeShape<T, D>;
  static constexpr int VPL = Sh::kVPL;
  static constexpr int EPL = Sh::kEPL;

  struct Ctx {  // per-piece constants (wave-uniform)
    int kvh, head0, nh, L;
    const int32_t* trow;
  };

  __device__ static Ctx ctx_of(const DecodeArgs& a, const Piece& p) {
    Ctx c;
    c.kvh = p.kc / a.n_chunks;
    const int chunk = p.kc - c.kvh * a.n_chunks;
    c.head0 = c.kvh * a.g + chunk * GC;
    c.nh = min(GC, a.g - chunk * GC);
    c.L = seq_len(a, p.b);
    c.trow = a.block_tables + (size_t)p.b * a.max_blocks_per_seq;
    return c;
  }

  // Raw table entry (a scalar load); clamped only where it is used, so that the
  // load has a whole block step to land.
  __device__ static int table_entry(const Ctx& c, int j) { return constant_view(c.trow)[j]; }
  __device__ static int clamp_block(const DecodeArgs& a, int e) {
    return (e >= 0 && e < a.n_blocks) ? e : 0;
  }

  __device__ static void load_q(const DecodeArgs& a, const Piece& p, const Ctx& c, int sub,
                                QRegs<GC, VPL>& q) {
    const uint4* qv = reinterpret_cast<const uint4*>(a.q);
#pragma unroll
    for (int j = 0; j < GC; ++j) {
      const int h = c.head0 + min(j, c.nh - 1);
      const size_t rowv = ((size_t)p.b * a.h_q + h) * Sh::kRowVec;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const uint4 x = qv[rowv + v * Sh::kLPT + sub];
        q.w[j][v * 4 + 0] = x.x;
        q.w[j][v * 4 + 1] = x.y;
        q.w[j][v * 4 + 2] = x.z;
        q.w[j][v * 4 + 3] = x.w;
      }
    }
  }

  // Stores a finished piece: the normalised output if it is the whole
  // segment, else a partial state in slot 0 (first piece of the wave's range)
  // or 1 (last).  The wave holding a segment's first block records which waves
  // hold its pieces, for the second pass.
  __device__ static void epilogue(const DecodeArgs& a, const Line& line, int W, const Piece& p,
                                  const Ctx& c, int lane, float (&m)[GC], float (&l)[GC],
                                  float (&acc)[GC][EPL]) {
    const int sub = lane % Sh::kLPT;
    const int slot_id = lane / Sh::kLPT;
    const bool whole = (p.j0 == 0 && p.j1 == p.nb);
    const int slot = p.j0 > 0 ? 0 : 1;
    if (p.j0 == 0 && lane == 0) {
      const int wb = whole ? W : line.wave_of(p.seg0 + p.nb - 1);
      reinterpret_cast<int2*>(a.seg_desc)[(size_t)p.b * a.h_kv * a.n_chunks + p.kc] = make_int2(W, wb);
    }
#pragma unroll
    for (int j = 0; j < GC; ++j) {
      const float M = class_max<Sh::kLPT>(m[j]);
      const float f = m[j] == kNegInf ? 0.f : fast_exp2(m[j] - M);
      const float ls = class_sum<Sh::kLPT>(l[j] * f);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] = class_sum<Sh::kLPT>(acc[j][e] * f);
      if (j >= c.nh || slot_id != 0) continue;
      if (whole) {
        const float inv = 1.f / ls;
        using O = OutOf<T>;
        O* out = reinterpret_cast<O*>(a.out) + ((size_t)p.b * a.h_q + c.head0 + j) * D;
#pragma unroll
        for (int e = 0; e < EPL; ++e) store_elem<O>(out, lane_channel<T, D>(sub, e), acc[j][e] * inv);
      } else {
        float* ws = a.ws + ((size_t)(W * 2 + slot) * GC + j) * (D + 2);
#pragma unroll
        for (int e = 0; e < EPL; ++e) ws[lane_channel<T, D>(sub, e)] = acc[j][e];
        if (sub == 0) {
          ws[D] = M;
          ws[D + 1] = ls;
        }
      }
    }
  }

  __device__ static void run(const DecodeArgs& a, const Line& line, int W, int64_t e, Piece cur,
                             int lane) {
    const int HC = a.h_kv * a.n_chunks;
    const int sub = lane % Sh::kLPT;
    const int slot_id = lane / Sh::kLPT;
    auto block_head = [&](int raw_entry, int kvh) {
      return (size_t)clamp_block(a, raw_entry) * a.h_kv + kvh;
    };

    Ctx cc = ctx_of(a, cur);
    QRegs<GC, VPL> q, qn;
    load_q(a, cur, cc, sub, q);
    int t = cur.j0;
    // Blocks walked so far, and the count after which a raised issue priority
    // (see decode_split_kernel) drops back to the default.
    int walked = 0;
    const int64_t prio_until = (e - (cur.seg0 + cur.j0)) * 3 / 4;
    // Table entries are requested two blocks (and, for the next piece, one
    // piece) ahead of their use: the entry of block t + 1 is in ent[0] at even
    // steps of the inner loop and in ent[1] at odd steps, so each scalar load
    // has two block steps to land and is never copied before use.
    int ent0 = table_entry(cc, min(t + 1, cur.j1 - 1));
    int ent1 = table_entry(cc, min(t + 2, cur.j1 - 1));
    Piece nxt = next_piece(a, HC, cur, e);
    Ctx nc = nxt.valid ? ctx_of(a, nxt) : cc;
    int nxt_blk0 = 0, nxt_blk1 = 0;
    if (nxt.valid) {
      load_q(a, nxt, nc, sub, qn);
      nxt_blk0 = table_entry(nc, 0);
      nxt_blk1 = table_entry(nc, min(1, nxt.j1 - 1));
    }

    float m[GC], l[GC], acc[GC][EPL];
    float m_sel = kNegInf, l_slot = 0.f;  // reduce-scattered scores only
    auto reset = [&]() {
      m_sel = kNegInf;
      l_slot = 0.f;
#pragma unroll
      for (int j = 0; j < GC; ++j) {
        m[j] = kNegInf;
        l[j] = 0.f;
#pragma unroll
        for (int x = 0; x < EPL; ++x) acc[j][x] = 0.f;
      }
    };
    reset();

    BlockOf<T, D> A, B;
    {
      load_block<T, D>(A, a, block_head(table_entry(cc, t), cc.kvh), slot_id, sub);
    }

    // Block t (in X) is not the piece's last: load block t + 1 (entry in E)
    // into Y, request the entry of block t + 3 into E, then attend block t.
    // A block before the last is always full.
    auto step_in = [&](BlockOf<T, D>& X, BlockOf<T, D>& Y, int& E) {
      load_block<T, D>(Y, a, block_head(E, cc.kvh), slot_id, sub);
      E = table_entry(cc, min(t + 3, cur.j1 - 1));
      if constexpr (kScatterScores<T, D, GC>)
        attend_block_rs<T, D, GC, false>(X, q, m, m_sel, l_slot, acc, a.scale_log2, slot_id, kBlock,
                                         sub);
      else
        attend_block<T, D, GC, false>(X, q, m, l, acc, a.scale_log2, slot_id, kBlock);
      ++t;
      if (++walked == prio_until) __builtin_amdgcn_s_setprio(0);
    };
    // Block t (in X) is the piece's last: load the next piece's first block
    // into Y, if there is a next piece, then attend block t, masking the tokens
    // past the context.
    auto step_last = [&](BlockOf<T, D>& X, BlockOf<T, D>& Y) {
      if (nxt.valid) {
        load_block<T, D>(Y, a, block_head(nxt_blk0, nc.kvh), slot_id, sub);
      }
      const int valid = cc.L - t * kBlock;
      if constexpr (kScatterScores<T, D, GC>) {
        if (valid >= kBlock)
          attend_block_rs<T, D, GC, false>(X, q, m, m_sel, l_slot, acc, a.scale_log2, slot_id, kBlock,
                                         sub);
        else
          attend_block_rs<T, D, GC, true>(X, q, m, m_sel, l_slot, acc, a.scale_log2, slot_id, valid,
                                        sub);
      } else {
        if (valid >= kBlock)
          attend_block<T, D, GC, false>(X, q, m, l, acc, a.scale_log2, slot_id, kBlock);
        else
          attend_block<T, D, GC, true>(X, q, m, l, acc, a.scale_log2, slot_id, valid);
      }
    };

    if constexpr (kF16Codes<T, GC>) q_for_codes(q, a.scale_log2);
    // Block t of the current piece is in A, or in B when in_b (a register copy
    // from B to A would wait for that block's loads and drain the pipeline, so
    // the roles swap instead: one step from B realigns the walk to A).
    bool in_b = false;
    while (true) {
      bool ended = false;
      if (in_b) {
        if (t + 1 < cur.j1) {
          step_in(B, A, ent0);
          const int e = ent0;
          ent0 = ent1;
          ent1 = e;
        } else {
          step_last(B, A);
          ended = true;
          in_b = false;
        }
      }
      if (!ended) {
        while (t + 2 < cur.j1) {
          step_in(A, B, ent0);
          step_in(B, A, ent1);
        }
        if (t + 1 < cur.j1) {
          step_in(A, B, ent0);
          step_last(B, A);
          in_b = false;
        } else {
          step_last(A, B);
          in_b = true;
        }
      }
      if constexpr (kScatterScores<T, D, GC>) rs_finish_sum<GC>(l_slot, l);
      epilogue(a, line, W, cur, cc, lane, m, l, acc);
      if (!nxt.valid) break;
      cur = nxt;
      cc = nc;
#pragma unroll
      for (int j = 0; j < GC; ++j)
#pragma unroll
        for (int x = 0; x < VPL * 4; ++x) q.w[j][x] = qn.w[j][x];
      if constexpr (kF16Codes<T, GC>) q_for_codes(q, a.scale_log2);
      reset();
      t = 0;
      ent0 = nxt_blk1;
      ent1 = table_entry(cc, min(2, cur.j1 - 1));
      nxt = next_piece(a, HC, cur, e);
      if (nxt.valid) {
        nc = ctx_of(a, nxt);
        load_q(a, nxt, nc, sub, qn);
        nxt_blk0 = table_entry(nc, 0);
        nxt_blk1 = table_entry(nc, min(1, nxt.j1 - 1));
      }
    }
  }
};

constexpr int kSplitWaves = 4;  // waves per workgroup of the split kernel

template <typename T, int D, int GC>
__global__ __launch_bounds__(kSplitWaves * kWave) void decode_split_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  // The wave index and the grid size come from compile-time and argument
  // values, not from the dispatch's hidden arguments, so the kernel starts
  // with a single round of scalar argument loads.
  const int W = blockIdx.x * kSplitWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const bool in_grid = W < a.num_splits;  // the last workgroup may hold spare waves
  const int HC = a.h_kv * a.n_chunks;
  // Two workgroups share each CU, and the one dispatched second is younger on
  // every SIMD it shares; issue arbitration favours the older wave, so the
  // first round would finish early and leave its CU half occupied for the
  // tail.  The second half of the grid therefore runs at a raised priority for
  // the first three quarters of its range (measured on the Llama-3-8B-shaped
  // batch: 111.4 -> 109.2 us per call; priority over the whole range, or up
  // to half of it, gained less).
  if ((int)blockIdx.x >= (a.num_splits + kSplitWaves - 1) / kSplitWaves / 2)
    __builtin_amdgcn_s_setprio(2);

  // Context lengths.  A batch of at most 64 sequences is read once, one
  // sequence per lane, and the zero-length outputs, the line length and the
  // search for the wave's first piece all take their lengths from that one
  // load instead of waiting for three loads in turn (about one memory round
  // trip less before the first block is requested).  Larger batches are read
  // in chunks of 64 sequences for each.
  const bool one_load = a.B <= kWave;
  const int len_lane = (one_load && lane < a.B) ? seq_len(a, lane) : 0;
  const int n_lane = (len_lane + kBlock - 1) / kBlock;
  const int64_t incl_lane = wave_incl_scan(n_lane, lane);

  // Sequences of length 0 get an all-zero output (sequence b by wave b mod splits).
  for (int b0 = W; in_grid && b0 < a.B; b0 += a.num_splits) {
    if ((one_load ? __builtin_amdgcn_readlane(len_lane, b0) : seq_len(a, b0)) != 0) continue;
    OutOf<T>* out = reinterpret_cast<OutOf<T>*>(a.out) + (size_t)b0 * a.h_q * D;
    for (int i = lane; i < a.h_q * D; i += kWave) store_elem<OutOf<T>>(out, i, 0.f);
  }

  const int64_t total =
      one_load ? uniform((int64_t)__shfl(incl_lane, kWave - 1)) : total_blocks(a, lane);
  const Line line{total * HC, a.num_splits};
  if (W == 0 && lane == 0) *a.line_total = line.total;  // for the second pass
  if (line.total == 0 || !in_grid) return;
  const int64_t s = line.start(W);
  const int64_t e = line.start(W + 1);
  if (s >= e) return;

  // The sequence holding position s: the first whose end lies past s.
  Piece first;
  {
    int64_t base = 0;
    int b = 0, nb = 1;
    int64_t seq0 = 0;
    for (int c0 = 0; c0 < a.B; c0 += kWave) {
      const int bb = c0 + lane;
      const int n = one_load ? n_lane : (bb < a.B ? seq_blocks(a, bb) : 0);
      const int64_t incl = one_load ? incl_lane : wave_incl_scan(n, lane);
      const uint64_t hit = __ballot(bb < a.B && (base + incl) * HC > s);
      if (hit) {
        const int f = __builtin_ctzll(hit);
        b = c0 + f;
        nb = __shfl(n, f);
        seq0 = (base + __shfl(incl, f) - nb) * HC;
        break;
      }
      base += __shfl(incl, kWave - 1);
    }
    b = uniform(b);
    nb = uniform(nb);
    seq0 = uniform(seq0);
    const int64_t r = s - seq0;
    first.b = b;
    first.nb = nb;
    first.kc = (int)(r / nb);
    first.j0 = (int)(r - (int64_t)first.kc * nb);
    first.seg0 = seq0 + (int64_t)first.kc * nb;
    first.j1 = (int)min((int64_t)nb, e - first.seg0);
    first.valid = true;
  }
  RangeStream<T, D, GC>::run(a, line, W, e, first, lane);
}

// Second pass: merges the segments cut by range boundaries.  One workgroup per
// segment; wave j takes heads j, j + 4, ...
constexpr int kCombineWaves = 4;
template <typename T, int D, int GC>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int HC = a.h_kv * a.n_chunks;
  const int seg = blockIdx.x;
  const int b = seg / HC;
  const int kc = seg - b * HC;
  const int kvh = kc / a.n_chunks;
  const int chunk = kc - kvh * a.n_chunks;
  const int head0 = kvh * a.g + chunk * GC;
  const int nh = min(GC, a.g - chunk * GC);
  const int nb = seq_blocks(a, b);
  const int2 wr = reinterpret_cast<const int2*>(a.seg_desc)[seg];
  if (nb == 0 || wr.x == wr.y) return;  // zero-filled, or stored whole, by the first pass
  const Line line{*a.line_total, a.num_splits};
  const int wa = wr.x;
  const int wb = wr.y;
  if (wb - wa < 8) {
    for (int j = wave; j < nh; j += kCombineWaves)
      merge_segment_head<T, D, GC, 8>(a, line, b, head0, j, wa, wb, lane);
  } else {
    for (int j = wave; j < nh; j += kCombineWaves)
      merge_segment_head<T, D, GC, 32>(a, line, b, head0, j, wa, wb, lane);
  }
}

template <typename T, int D, int GC>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<T, D, GC>),
                     dim3((a.num_splits + kSplitWaves - 1) / kSplitWaves),
                     dim3(kSplitWaves * kWave), 0, stream, a);
  // With one range the single wave walks every segment whole and stores (or
  // zero-fills) every output itself: no segment is cut, so no second pass.
  if (a.num_splits > 1)
    hipLaunchKernelGGL((decode_combine_kernel<T, D, GC>), dim3(a.B * a.h_kv * a.n_chunks),
                       dim3(kCombineWaves * kWave), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D, int GC>
static int occupancy_waves_t() {
  static int waves = [] {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(decode_split_kernel<T, D, GC>),
            kSplitWaves * kWave, 0) !=
            hipSuccess ||
        cus <= 0 || per_cu <= 0)
      return 0;
    return cus * per_cu * kSplitWaves;
  }();
  return waves;
}

template <typename T, int D, int GC>
static hipError_t run_or_query(const DecodeArgs& a, hipStream_t stream, int* waves_out) {
  if (waves_out) {
    *waves_out = occupancy_waves_t<T, D, GC>();
    return hipSuccess;
  }
  return launch_t<T, D, GC>(a, stream);
}

template <typename T, int D>
static hipError_t dispatch_gc(const DecodeArgs& a, hipStream_t stream, int* waves_out) {
  constexpr bool kWide = std::is_same<T, float>::value && D == 128;  // at most 4 heads per chunk
  switch (a.gc) {
    case 1: return run_or_query<T, D, 1>(a, stream, waves_out);
    case 2: return run_or_query<T, D, 2>(a, stream, waves_out);
    case 3: return run_or_query<T, D, 3>(a, stream, waves_out);
    case 4: return run_or_query<T, D, 4>(a, stream, waves_out);
  }
  if constexpr (!kWide) {
    switch (a.gc) {
      case 5: return run_or_query<T, D, 5>(a, stream, waves_out);
      case 6: return run_or_query<T, D, 6>(a, stream, waves_out);
      case 7: return run_or_query<T, D, 7>(a, stream, waves_out);
      case 8: return run_or_query<T, D, 8>(a, stream, waves_out);
    }
  }
  return hipErrorInvalidValue;
}

static hipError_t dispatch(const DecodeArgs& a, int d_h, KvType kv, hipStream_t stream,
                           int* waves_out) {
  if (kv == KvType::kI8) {
    if (d_h == 64) return dispatch_gc<i8_t, 64>(a, stream, waves_out);
    if (d_h == 128) return dispatch_gc<i8_t, 128>(a, stream, waves_out);
    return hipErrorInvalidValue;
  }
  if (kv == KvType::kBF16) {
    if (d_h == 64) return dispatch_gc<bf16_t, 64>(a, stream, waves_out);
    if (d_h == 128) return dispatch_gc<bf16_t, 128>(a, stream, waves_out);
  } else {
    if (d_h == 64) return dispatch_gc<float, 64>(a, stream, waves_out);
    if (d_h == 128) return dispatch_gc<float, 128>(a, stream, waves_out);
  }
  return hipErrorInvalidValue;
}

int decode_resident_waves(int d_h, KvType kv, int gc) {
  DecodeArgs a{};
  a.gc = gc;
  int waves = 0;
  if (dispatch(a, d_h, kv, nullptr, &waves) != hipSuccess) return 0;
  return waves;
}

hipError_t launch_decode(const DecodeArgs& a, int d_h, KvType kv, hipStream_t stream) {
  return dispatch(a, d_h, kv, stream, nullptr);
}

}  // namespace pkv
