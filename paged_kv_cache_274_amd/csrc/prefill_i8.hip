// Causal chunked prefill over an INT8 KV cache with bf16 matrix cores (gfx950).
//
// The cache holds x_hat = s * x_q: int8 codes with one float32 scale per token
// head row (LLM Inference Server page, Optional Stretch Challenges, "INT8
// KV-Cache Quantization"), and the new prompt tokens are processed in parallel
// over it with causal masking (Stage 1 prefill/decode task of the same page;
// Attention Kernel box of the pipeline figure, From Scratch page).
//
// Design: the bf16 prefill's tiling and matrix products (prefill.hip: GQA rows
// packed, 128 rows per workgroup of 4 waves, at d_h = 64 two such groups over
// alternate key tiles when the grid fits the chip, 64-key tiles, S^T = K Q^T
// and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16, lazy-rescale online
// softmax), with the cache read as codes:
//  * the codes and scales of a tile (half the bytes of a bf16 tile) are copied
//    straight from HBM into one of four LDS staging buffers, three tiles
//    ahead;
//  * the 256 threads of a group widen the tile's codes exactly to bf16
//    (|c| <= 127 needs 8 significant bits) into one of two bf16 tiles in the
//    swizzled layout the matrix reads use, once per group, and write the
//    tile's scales with the keys past the context set to 0 (their slots may
//    hold anything) and the K scales multiplied by |scale| * log2(e).  A
//    wave widens the group's next tile right after attending the current
//    one, so one barrier per step publishes both the copies and the widening.
//    (Widening in registers as each wave reads its operands, as the few-rows
//    kernel below does, repeats the work in every row wave: 4 x 4096-token
//    prompts took 17-25% longer.)
//  * the K scale multiplies each score S^T (one key per accumulator element);
//    the V scale multiplies each softmax weight before it is rounded to bf16
//    for the P^T operand (the normaliser sums the unscaled weights), so
//    attention is over x_hat exactly up to the bf16 rounding of the weights,
//    as in the bf16 and INT8 decodes.
#include "prefill_common.h"

namespace pkv {

namespace {

// Codes c0..c3 of a dword as two bf16 pairs, exactly: an int8 converts to
// float32 without rounding, and with at most 8 significant bits its float32
// pattern ends in 16 zero bits.
__device__ __forceinline__ void widen4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const float f0 = (float)(int)(int8_t)(w & 0xff);
  const float f1 = (float)(int)(int8_t)((w >> 8) & 0xff);
  const float f2 = (float)(int)(int8_t)((w >> 16) & 0xff);
  const float f3 = (float)(int)(int8_t)(w >> 24);
  lo = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  hi = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
}

// A tile of codes as staged: K codes, V codes (64 rows of D bytes each), then
// the raw K and V scales of its four blocks.
template <int D>
struct I8Stage {
  static constexpr int kCodeMat = kPfTile * D;
  static constexpr int kBytes = 2 * kCodeMat + 2 * kPfTile * 4;
  static constexpr int kCopiesPerBlock = kBlock * D / 1024;  // 1 KiB copies per block of codes
};

}  // namespace

// KS groups of 4 waves share a workgroup's 128 rows and split its key tiles,
// as in the bf16 prefill: group G takes tiles G, G + KS, ..., each group with
// its own staging buffers, bf16 tile and scales, and the groups' softmax
// states are merged at the end.  KS = 2 halves the serial key walk of the
// longest rows when the grid alone cannot fill the chip.
template <int D, int KS>
__global__ __launch_bounds__(256 * KS) void prefill_i8_kernel(PrefillArgs a) {
  using Tl = PfTile<D>;
  using St = I8Stage<D>;
  // LDS per group: four staging buffers (codes of K and V, raw K and V
  // scales) and two bf16 tiles (K then V), each with the tile's sanitised
  // scales (K, then V).
  constexpr int kBfBytes = 2 * Tl::kMatBytes + 2 * kPfTile * 4;
  constexpr int kGroupBytes = 4 * St::kBytes + 2 * kBfBytes;
  __shared__ __attribute__((aligned(16))) unsigned char lds[KS * kGroupBytes];
  constexpr int NC = D / 16;
  constexpr int NT = D / 32;
  // copies per wave per tile: its block's K and V codes, plus one for the scales
  constexpr int kCopies = 2 * St::kCopiesPerBlock + 1;

  const int bx = gridDim.x - 1 - blockIdx.x;
  const int s = a.longest_first ? longest_first_sequence(a, blockIdx.z) : (int)blockIdx.z;
  const int kvh = blockIdx.y;
  const int g = a.g;
  const int q0 = a.cu_seqlens_q[s];
  const int n = a.cu_seqlens_q[s + 1] - q0;
  int L = a.context_lens[s];
  L = max(0, min(L, a.max_blocks_per_seq * kBlock));
  const int rows = n * g;
  const int r0 = bx * kPfRows;
  if (n <= 0 || n > L || r0 >= rows || q0 < 0 || q0 + n > a.T_q) return;

  const int tid = threadIdx.x;
  const int gtid = tid & 255;  // thread index within the group
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);  // row wave in the group
  const int grp_id = __builtin_amdgcn_readfirstlane(tid >> 8);       // key-split group
  const int col = lane & 31;
  const int half = lane >> 5;
  const int first = L - n;

  const int r = r0 + wave * 32 + col;
  const bool row_ok = r < rows;
  const int tok = row_ok ? r / g : n - 1;
  const int hh = row_ok ? r - (r / g) * g : 0;
  const int pos = first + tok;
  const int wave_r0 = r0 + wave * 32;
  const bool wave_live = wave_r0 < rows;
  const int wave_pos_lo = first + wave_r0 / g;
  const int wave_pos_hi = first + (min(wave_r0 + 31, rows - 1)) / g;
  const int wg_pos_hi = first + (min(r0 + kPfRows - 1, rows - 1)) / g;
  const int n_tiles = __builtin_amdgcn_readfirstlane(wg_pos_hi / kPfTile + 1);
  const int n_steps = (n_tiles + KS - 1) / KS;  // tiles per group, rounded up
  const int Lu = __builtin_amdgcn_readfirstlane(L);
  unsigned char* const glds = lds + grp_id * kGroupBytes;
  // The group's i-th tile: codes in staging buffer i % 4, widened into bf16
  // tile i % 2.
  auto btile = [&](int i) { return glds + 4 * St::kBytes + (i & 1) * kBfBytes; };

  const float csc = fabsf(a.scale_log2);
  const uint32_t qsign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  f32x16_t o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  float m = kPfNegInf;
  float lsum = 0.f;

  const unsigned char* kc = reinterpret_cast<const unsigned char*>(a.k_cache);
  const unsigned char* vc = reinterpret_cast<const unsigned char*>(a.v_cache);
  const unsigned char* ks = reinterpret_cast<const unsigned char*>(a.k_scale);
  const unsigned char* vs = reinterpret_cast<const unsigned char*>(a.v_scale);
  const int32_t* trow = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  auto stage = [&](int i) { return glds + (i & 3) * St::kBytes; };

  // Copies block (4 * kt + wave) of tile kt, the group's i-th, into its
  // staging buffer: the K and V codes of that block (rows 16 * wave ..), and
  // its 16 K and 16 V scales (lanes 0-3 and 4-7 of one more copy) into the
  // scale area (wave w's block at floats 32 w .. 32 w + 31: K then V).
  auto issue_tile = [&](int kt, int i) {
    const int bi = min(kt * (kPfTile / kBlock) + wave, a.max_blocks_per_seq - 1);
    int blk = constant_view(trow)[bi];
    blk = (blk >= 0 && blk < a.n_blocks) ? blk : 0;
    const size_t bh = (size_t)blk * a.h_kv + kvh;
    unsigned char* st = stage(i);
#pragma unroll
    for (int c = 0; c < St::kCopiesPerBlock; ++c) {
      const size_t src = bh * (kBlock * D) + (size_t)c * 1024 + lane * 16;
      const int dst = wave * kBlock * D + c * 1024;
      copy_to_lds(kc + src, st + dst);
      copy_to_lds(vc + src, st + St::kCodeMat + dst);
    }
    if (lane < 8) {
      const unsigned char* src = (lane < 4 ? ks : vs) + bh * (kBlock * 4) + (lane & 3) * 16;
      copy_to_lds(src, st + 2 * St::kCodeMat + wave * 128);
    }
  };

  // Widens tile kt's codes (staged as the group's i-th tile) into its bf16
  // tile and writes its sanitised scales (the group's 256 threads).  Rows past
  // the context: V zero, both scales zero.
  auto convert_tile = [&](int kt, int i) {
    const unsigned char* st = stage(i);
    unsigned char* const tile = btile(i);
    float* const ksc = reinterpret_cast<float*>(tile + 2 * Tl::kMatBytes);
    float* const vsc = ksc + kPfTile;
    const int valid = Lu - kt * kPfTile;  // rows of this tile inside the context
    constexpr int kUnits = 2 * kPfTile * Tl::kChunks;  // 8-code units of K and V
#pragma unroll
    for (int u0 = 0; u0 < kUnits; u0 += 256) {
      const int u = u0 + gtid;
      const int isv = u >= kPfTile * Tl::kChunks;
      const int uu = isv ? u - kPfTile * Tl::kChunks : u;
      const int row = uu / Tl::kChunks;
      const int ch = uu - row * Tl::kChunks;
      const uint2 w = *reinterpret_cast<const uint2*>(st + isv * St::kCodeMat + row * D + ch * 8);
      uint4 x;
      widen4(w.x, x.x, x.y);
      widen4(w.y, x.z, x.w);
      if (isv && row >= valid) x = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(tile + isv * Tl::kMatBytes + Tl::offset(row, ch)) = x;
    }
    if (gtid < 2 * kPfTile) {
      const int key = gtid & (kPfTile - 1);
      const int isv = gtid >= kPfTile;
      const float* raw = reinterpret_cast<const float*>(st + 2 * St::kCodeMat);
      // raw layout: block w = key / 16 at floats 32 w (K) and 32 w + 16 (V)
      const float x = raw[(key >> 4) * 32 + isv * 16 + (key & 15)];
      const float y = key < valid ? x : 0.f;
      (isv ? vsc : ksc)[key] = isv ? y : y * csc;
    }
  };

  const int grp = lane >> 4;
  const int tr_row = 4 * (grp >> 1) + ((lane & 15) >> 2);
  const int tr_ch = 16 * (grp & 1) + 4 * (lane & 3);

  bf16x8_t qb[NC];
  {
    const uint4* qv = reinterpret_cast<const uint4*>(a.q);
    const size_t rowv = ((size_t)(q0 + tok) * a.h_q + kvh * g + hh) * (D / 8);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint4 x = row_ok ? qv[rowv + 2 * c + half] : make_uint4(0, 0, 0, 0);
      x.x ^= qsign;
      x.y ^= qsign;
      x.z ^= qsign;
      x.w ^= qsign;
      qb[c] = __builtin_bit_cast(bf16x8_t, x);
    }
  }
  // Whether the group has an i-th tile.
  auto has = [&](int i) { return i * KS + grp_id < n_tiles; };
  if (has(0)) issue_tile(grp_id, 0);
  if (has(1)) issue_tile(grp_id + KS, 1);
  if (has(2)) issue_tile(grp_id + 2 * KS, 2);
  wait_vm<0>();
  tile_barrier();
  if (has(0)) convert_tile(grp_id, 0);

  // Step i: every group attends its i-th tile, tile kt = i * KS + group, and
  // widens its next one, so one barrier per step separates each tile's
  // widening from its use; all groups pass the same barriers.
  for (int i = 0; i < n_steps; ++i) {
    const int kt = i * KS + grp_id;
    const bool mine = kt < n_tiles;
    // The group's next tile's copies have landed (own ones: all but the one
    // after it) and this tile's widening is written (own writes), then every
    // wave's (barrier); every wave is also done with the previous step's
    // tile and with this tile's codes.
    if (has(i + 2)) wait_vm<kCopies>();
    else wait_vm<0>();
    wait_lds();
    tile_barrier();
    if (has(i + 3)) issue_tile(kt + 3 * KS, i + 3);
    if (mine && wave_live && kt * kPfTile <= wave_pos_hi) {
    const unsigned char* const tile = btile(i);
    const float* const ksc = reinterpret_cast<const float*>(tile + 2 * Tl::kMatBytes);
    const float* const vsc = ksc + kPfTile;
    const int key0 = kt * kPfTile;
    f32x16_t sc[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[h2][i] = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint4 kx = *reinterpret_cast<const uint4*>(tile + Tl::offset(32 * h2 + col, 2 * c + half));
        sc[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kx), qb[c],
                                                         sc[h2], 0, 0, 0);
      }
    }
    // The keys of accumulator elements (h2, 4j .. 4j + 3): 32 h2 + 8 j + 4 half + 0..3.
    float kf[2][16], vf[2][16];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 k4 = *reinterpret_cast<const float4*>(ksc + 32 * h2 + 8 * j + 4 * half);
        const float4 v4 = *reinterpret_cast<const float4*>(vsc + 32 * h2 + 8 * j + 4 * half);
        kf[h2][4 * j + 0] = k4.x; kf[h2][4 * j + 1] = k4.y; kf[h2][4 * j + 2] = k4.z; kf[h2][4 * j + 3] = k4.w;
        vf[h2][4 * j + 0] = v4.x; vf[h2][4 * j + 1] = v4.y; vf[h2][4 * j + 2] = v4.z; vf[h2][4 * j + 3] = v4.w;
      }
    // Scores in log2 units: the K scale (times |scale| log2 e) of each key.
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[h2][i] *= kf[h2][i];
    if (key0 + kPfTile - 1 > wave_pos_lo) {
      const int lim = pos - key0 - 4 * half;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * h2 + mfma32_row(i, 0) > lim) sc[h2][i] = kPfNegInf;
    }
    float tmax = kPfNegInf;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sc[h2][i]);
    tmax = xor32_max(tmax);
    if (__any(tmax > m + kPfSlack)) {
      const float mn = tmax > m + kPfSlack ? tmax : m;
      const float alpha = mn == m ? 1.f : fast_exp2(m - mn);
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
    }
    const float mb = m == kPfNegInf ? 0.f : m;  // all scores so far masked: weight 0
    float ps = 0.f;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(sc[h2][i] - mb);
        ps += p;
        sc[h2][i] = p * vf[h2][i];  // the weight times the key's V scale
      }
    lsum += ps;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x16_t& w = sc[c >> 1];
      const int e0 = 8 * (c & 1);
      uint4 pw;
      pw.x = pack_bf16x2(w[e0 + 0], w[e0 + 1]);
      pw.y = pack_bf16x2(w[e0 + 2], w[e0 + 3]);
      pw.z = pack_bf16x2(w[e0 + 4], w[e0 + 5]);
      pw.w = pack_bf16x2(w[e0 + 6], w[e0 + 7]);
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int chn = 32 * t + tr_ch;
        const int ra = 16 * c + tr_row;
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (PKV_LDS i16x4_t*)(tile + Tl::kMatBytes + Tl::offset(ra, chn >> 3) + (chn & 4) * 2));
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (PKV_LDS i16x4_t*)(tile + Tl::kMatBytes + Tl::offset(ra + 8, chn >> 3) + (chn & 4) * 2));
        const i16x4_t lohi[2] = {lo, hi};
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, lohi), pb, o[t],
                                                       0, 0, 0);
      }
    }
    }
    if (has(i + 1)) convert_tile(kt + KS, i + 1);
  }

  if constexpr (KS == 2) {
    // Group 1 hands its state for the same rows to group 0 through LDS (field
    // f of lane l of row wave w at float (f * 4 + w) * 64 + l), which merges
    // the two with the log-sum-exp rule.
    constexpr int kFields = NT * 16 + 2;
    static_assert(kFields * 4 * 64 * 4 <= (int)sizeof(lds), "merge area");
    float* mg = reinterpret_cast<float*>(lds);
    auto at = [&](int f) -> float& { return mg[(f * 4 + wave) * 64 + lane]; };
    tile_barrier();  // every wave is done with the tiles
    if (grp_id == 1) {
      at(0) = m;
      at(1) = lsum;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) at(2 + t * 16 + e) = o[t][e];
    }
    wait_lds();
    tile_barrier();
    if (grp_id == 1) return;
    const float m1 = at(0);
    const float mm = fmaxf(m, m1);
    const float a0 = m == kPfNegInf ? 0.f : fast_exp2(m - mm);
    const float a1 = m1 == kPfNegInf ? 0.f : fast_exp2(m1 - mm);
    lsum = lsum * a0 + at(1) * a1;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[t][e] = o[t][e] * a0 + at(2 + t * 16 + e) * a1;
  }

  if (!row_ok) return;
  const float lt = xor32_sum(lsum);
  const float inv = 1.f / lt;
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  const size_t orow = ((size_t)(q0 + tok) * a.h_q + kvh * g + hh) * D;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int chn = t * 32 + 8 * gq + 4 * half;
      uint2 w;
      w.x = pack_bf16x2(o[t][4 * gq + 0] * inv, o[t][4 * gq + 1] * inv);
      w.y = pack_bf16x2(o[t][4 * gq + 2] * inv, o[t][4 * gq + 3] * inv);
      *reinterpret_cast<uint2*>(&out[orow + chn]) = w;
    }
}

// Few query rows per (sequence, KV head) (at most 32: multi-token decode), as
// prefill_few_rows_kernel in prefill.hip: the 4 waves split the key walk into
// 32-key chunks w, w + 4, ..., each wave staging its chunk's codes and scales
// in two LDS stages of its own (one in flight), so no barrier is needed until
// the states are merged.  The codes are widened to bf16 in registers on their
// way to the matrix cores: the K operand (8 channels of a key) is an 8-byte
// read of a code row, the V^T operand (8 keys of a channel) an 8-bit
// transposed read (ds_read_b64_tr_b8: in each 16-lane group, byte b of lane i
// comes from byte i % 8 of the row lane 2b + i / 8 points at).  The copies
// swizzle each code row's 16-byte chunks so that both reads spread over the
// LDS banks; the scales are read raw and the ones past the context replaced
// by 0 in registers.
constexpr int kI8FewKeys = 32;
// Two workgroups per compute unit (at most 256 VGPRs: two waves per SIMD; the
// stages take 66 KiB of LDS at d_h = 128).
template <int D>
__global__ __launch_bounds__(256, 2) void prefill_i8_few_rows_kernel(PrefillArgs a) {
  using Tl = PfTile<D>;
  constexpr int kCodes = kI8FewKeys * D;                       // codes of K (or V) of a chunk
  constexpr int kStage = 2 * kCodes + 2 * kI8FewKeys * 4;       // codes + raw K, V scales
  constexpr int kWaveBytes = 2 * kStage;
  constexpr int kRowChunks = D / 16;                           // 16-byte chunks of a code row
  constexpr int kRowsPerLine = 256 / D;                        // code rows per 64 LDS banks
  constexpr int NC = D / 16;
  constexpr int NT = D / 32;
  constexpr int kCopiesPerBlock = kBlock * D / 1024;
  constexpr int kCopies = 2 * 2 * kCopiesPerBlock + 2;         // codes of 2 blocks, 2 scale copies
  constexpr int kFields = NT * 16 + 2;
  __shared__ __attribute__((aligned(16))) unsigned char
      lds[(kPfWaves * kWaveBytes > kPfWaves * kFields * 256) ? kPfWaves * kWaveBytes
                                                             : kPfWaves * kFields * 256];

  const int s = a.longest_first ? longest_first_sequence(a, blockIdx.z) : (int)blockIdx.z;
  const int kvh = blockIdx.y;
  const int g = a.g;
  const int q0 = a.cu_seqlens_q[s];
  const int n = a.cu_seqlens_q[s + 1] - q0;
  int L = a.context_lens[s];
  L = max(0, min(L, a.max_blocks_per_seq * kBlock));
  const int rows = n * g;
  if (n <= 0 || n > L || rows > 32 || q0 < 0 || q0 + n > a.T_q) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;
  const int first = L - n;
  const bool row_ok = col < rows;
  const int tok = row_ok ? col / g : n - 1;
  const int hh = row_ok ? col - (col / g) * g : 0;
  const int pos = first + tok;
  const int Lu = __builtin_amdgcn_readfirstlane(L);
  const int n_chunks = (Lu + kI8FewKeys - 1) / kI8FewKeys;

  const float csc = fabsf(a.scale_log2);
  const uint32_t qsign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  f32x16_t o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  float m = kPfNegInf;
  float lsum = 0.f;

  const unsigned char* kc = reinterpret_cast<const unsigned char*>(a.k_cache);
  const unsigned char* vc = reinterpret_cast<const unsigned char*>(a.v_cache);
  const unsigned char* ks = reinterpret_cast<const unsigned char*>(a.k_scale);
  const unsigned char* vs = reinterpret_cast<const unsigned char*>(a.v_scale);
  const int32_t* trow = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  unsigned char* const mine = lds + wave * kWaveBytes;
  // Physical 16-byte chunk of logical chunk ch of code row r (an involution).
  auto swz = [](int r, int ch) { return ch ^ ((r / kRowsPerLine) % kRowChunks); };

  // Raw table entry of block b (0 or 1) of chunk c, a scalar load; clamped
  // where it is used, so the load has an iteration to land.
  auto entry = [&](int c, int b) {
    return constant_view(trow)[min(2 * c + b, a.max_blocks_per_seq - 1)];
  };
  // Copies a chunk (blocks with table entries e0 and e1): codes of K then V
  // (rows = keys, D bytes each), then the blocks' K and V scales (16 each,
  // lanes 0-3 / 4-7 of one copy per block: block b at floats 32 b .. 32 b + 31,
  // K then V).
  auto issue_chunk = [&](int st, int e0, int e1) {
    unsigned char* dst = mine + st * kStage;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      int blk = b == 0 ? e0 : e1;
      blk = (blk >= 0 && blk < a.n_blocks) ? blk : 0;
      const size_t bh = (size_t)blk * a.h_kv + kvh;
#pragma unroll
      for (int i = 0; i < kCopiesPerBlock; ++i) {
        // Lane l fills LDS bytes 16 l .. 16 l + 15 of this copy: row rb of
        // the block, physical chunk pc, i.e. logical chunk swz(row, pc).
        const int pos = i * 1024 + lane * 16;
        const int rb = pos / D;
        const int pc = (pos % D) / 16;
        const size_t src = bh * (kBlock * D) + (size_t)rb * D + swz(b * kBlock + rb, pc) * 16;
        const int d = b * kBlock * D + i * 1024;
        copy_to_lds(kc + src, dst + d);
        copy_to_lds(vc + src, dst + kCodes + d);
      }
      if (lane < 8) {
        const unsigned char* src = (lane < 4 ? ks : vs) + bh * (kBlock * 4) + (lane & 3) * 16;
        copy_to_lds(src, dst + 2 * kCodes + b * 128);
      }
    }
  };
  bf16x8_t qb[NC];
  {
    const uint4* qv = reinterpret_cast<const uint4*>(a.q);
    const size_t rowv = ((size_t)(q0 + tok) * a.h_q + kvh * g + hh) * (D / 8);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint4 x = row_ok ? qv[rowv + 2 * c + half] : make_uint4(0, 0, 0, 0);
      x.x ^= qsign;
      x.y ^= qsign;
      x.z ^= qsign;
      x.w ^= qsign;
      qb[c] = __builtin_bit_cast(bf16x8_t, x);
    }
  }
  // V^T operand addressing (see above): this lane points at key row
  // 8 (b / 4) + 4 h + b % 4 (b = (lane % 16) / 2, h = lane / 32) of a 16-key
  // half and at byte 8 (lane % 2) of the 16 channels of its 16-lane group, so
  // that it receives the 8 keys of channel lane % 32 in the P^T operand's key
  // order (accumulator element e: key 8 (e / 4) + 4 h + e % 4).
  const int vt_b = (lane & 15) >> 1;
  const int vt_row = 8 * (vt_b >> 2) + 4 * half + (vt_b & 3);
  const int vt_ch = 16 * ((lane >> 4) & 1) + 8 * (lane & 1);

  if (wave < n_chunks) issue_chunk(0, entry(wave, 0), entry(wave, 1));
  // Entries of the chunk after next are requested an iteration before their
  // copies are issued.
  int n0 = entry(wave + kPfWaves, 0);
  int n1 = entry(wave + kPfWaves, 1);
  for (int c = wave, st = 0; c < n_chunks; c += kPfWaves, st ^= 1) {
    const bool more = c + kPfWaves < n_chunks;
    if (more) {
      issue_chunk(st ^ 1, n0, n1);
      n0 = entry(c + 2 * kPfWaves, 0);
      n1 = entry(c + 2 * kPfWaves, 1);
    }
    if (more)
      wait_vm<kCopies>();
    else
      wait_vm<0>();
    const unsigned char* kb = mine + st * kStage;
    const unsigned char* vb = kb + kCodes;
    const float* raw = reinterpret_cast<const float*>(kb + 2 * kCodes);
    const int key0 = c * kI8FewKeys;
    const int valid = Lu - key0;
    f32x16_t sc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = 0.f;
#pragma unroll
    for (int c2 = 0; c2 < NC; ++c2) {
      // Channels 16 c2 + 8 half .. + 7 of key col: half of logical chunk c2.
      const uint2 w = *reinterpret_cast<const uint2*>(kb + col * D + swz(col, c2) * 16 + 8 * half);
      uint4 kx;
      widen4(w.x, kx.x, kx.y);
      widen4(w.y, kx.z, kx.w);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kx), qb[c2], sc, 0,
                                                   0, 0);
    }
    // Keys of accumulator elements 4j .. 4j + 3: 8 j + 4 half + 0..3, in block
    // j / 2; raw scales of block b at floats 32 b (K) and 32 b + 16 (V).  A slot
    // past the context may hold anything (NaN included): selected away.
    float kf[16], vf[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = 8 * j + 4 * half;
      const float4 k4 = *reinterpret_cast<const float4*>(raw + (key >> 4) * 32 + (key & 15));
      const float4 v4 = *reinterpret_cast<const float4*>(raw + (key >> 4) * 32 + 16 + (key & 15));
      const float kr[4] = {k4.x, k4.y, k4.z, k4.w};
      const float vr[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[4 * j + e] = key + e < valid ? kr[e] * csc : 0.f;
        vf[4 * j + e] = key + e < valid ? vr[e] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] *= kf[i];
    if (key0 + kI8FewKeys - 1 > first) {
      const int lim = pos - key0 - 4 * half;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (mfma32_row(i, 0) > lim) sc[i] = kPfNegInf;
    }
    float tmax = kPfNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sc[i]);
    tmax = xor32_max(tmax);
    if (__any(tmax > m + kPfSlack)) {
      const float mn = tmax > m + kPfSlack ? tmax : m;
      const float alpha = mn == m ? 1.f : fast_exp2(m - mn);
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
    }
    const float mb = m == kPfNegInf ? 0.f : m;  // all scores so far masked: weight 0
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(sc[i] - mb);
      ps += p;
      sc[i] = p * vf[i];
    }
    lsum += ps;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      uint4 pw;
      pw.x = pack_bf16x2(sc[8 * c2 + 0], sc[8 * c2 + 1]);
      pw.y = pack_bf16x2(sc[8 * c2 + 2], sc[8 * c2 + 3]);
      pw.z = pack_bf16x2(sc[8 * c2 + 4], sc[8 * c2 + 5]);
      pw.w = pack_bf16x2(sc[8 * c2 + 6], sc[8 * c2 + 7]);
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);
      const int vr = 16 * c2 + vt_row;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int ch = 32 * t + vt_ch;
        const i32x2_t w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (PKV_LDS i32x2_t*)(vb + vr * D + swz(vr, ch >> 4) * 16 + (ch & 8)));
        uint4 vx;
        widen4((uint32_t)w[0], vx.x, vx.y);
        widen4((uint32_t)w[1], vx.z, vx.w);
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vx), pb, o[t],
                                                       0, 0, 0);
      }
    }
    // The stage is rewritten only after every read of this iteration has
    // returned.
    wait_lds();
  }

  float* mg = reinterpret_cast<float*>(lds);
  auto at = [&](int f, int w) -> float& { return mg[(f * kPfWaves + w) * 64 + lane]; };
  tile_barrier();
  if (wave != 0) {
    at(0, wave) = m;
    at(1, wave) = lsum;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) at(2 + t * 16 + e, wave) = o[t][e];
  }
  wait_lds();
  tile_barrier();
  if (wave != 0 || !row_ok) return;
  float mm = m;
#pragma unroll
  for (int w = 1; w < kPfWaves; ++w) mm = fmaxf(mm, at(0, w));
  const float a0 = m == kPfNegInf ? 0.f : fast_exp2(m - mm);
  lsum *= a0;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[t][e] *= a0;
#pragma unroll
  for (int w = 1; w < kPfWaves; ++w) {
    const float mw = at(0, w);
    const float aw = mw == kPfNegInf ? 0.f : fast_exp2(mw - mm);
    lsum += at(1, w) * aw;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[t][e] += at(2 + t * 16 + e, w) * aw;
  }
  const float lt = xor32_sum(lsum);
  const float inv = 1.f / lt;
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  const size_t orow = ((size_t)(q0 + tok) * a.h_q + kvh * g + hh) * D;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int chn = t * 32 + 8 * gq + 4 * half;
      uint2 w;
      w.x = pack_bf16x2(o[t][4 * gq + 0] * inv, o[t][4 * gq + 1] * inv);
      w.y = pack_bf16x2(o[t][4 * gq + 2] * inv, o[t][4 * gq + 3] * inv);
      *reinterpret_cast<uint2*>(&out[orow + chn]) = w;
    }
}

static int compute_units_i8() {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    return n;
  }();
  return cus;
}

template <int D>
static hipError_t launch_i8_d(const PrefillArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.max_q_len * a.g;
  PrefillArgs args = a;
  const int cus = compute_units_i8();
  if (rows <= 32) {
    args.longest_first = a.S > 1 && a.S <= kLptMaxSeqs && cus > 0 && (int64_t)a.h_kv * a.S > cus;
    hipLaunchKernelGGL((prefill_i8_few_rows_kernel<D>), dim3(1, a.h_kv, a.S), dim3(256), 0, stream,
                       args);
    return hipGetLastError();
  }
  const int64_t gx = (rows + kPfRows - 1) / kPfRows;
  const dim3 grid((unsigned)gx, a.h_kv, a.S);
  // Sequence planes longest context first when the grid takes more than one
  // round of the chip (as for the bf16 prefill).
  args.longest_first = a.S > 1 && a.S <= kLptMaxSeqs && cus > 0 && gx * a.h_kv * a.S > cus;
  // Split the key walk over two wave groups when the grid has no more
  // workgroups than the chip has compute units (d_h = 64, as for the bf16
  // prefill).
  if constexpr (D == 64) {
    if (cus > 0 && gx * a.h_kv * a.S <= cus) {
      hipLaunchKernelGGL((prefill_i8_kernel<D, 2>), grid, dim3(512), 0, stream, args);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((prefill_i8_kernel<D, 1>), grid, dim3(256), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_prefill_i8(const PrefillArgs& a, int d_h, hipStream_t stream) {
  if (d_h == 64) return launch_i8_d<64>(a, stream);
  if (d_h == 128) return launch_i8_d<128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
