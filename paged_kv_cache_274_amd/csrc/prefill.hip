// Causal chunked prefill over paged K/V with bf16 matrix cores (gfx950).
//
// New prompt tokens are processed in parallel (LLM Inference Server page,
// Stage 1 prefill/decode task) with causal masking and grouped-query heads
// (Attention Kernel box of the pipeline figure, From Scratch page); their K/V
// were already appended to 16-token blocks reached through the block table.
// Only here is the path a dense contraction, so QK^T and PV run on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation and an fp32 online softmax.
//
// Tiling
//  * GQA rows are packed: for one KV head the g query heads of a token are
//    adjacent rows (row r = token * g + head-in-group), so one K/V tile in LDS
//    serves the whole group.  A workgroup of 4 wavefronts owns 128 packed rows;
//    each wavefront owns 32 of them.
//  * Keys are walked in tiles of 32 (two blocks), gathered through the block
//    table into LDS: K row-major, V transposed, keys past the context zeroed.
//  * The wavefront computes S^T = K . Q^T (keys x its 32 query rows), so a lane
//    holds 16 scores of one query column; the row max and sum need only one
//    exchange with the other half-wave.  The scores' accumulator layout is
//    exactly the B operand layout of the next product, O^T = V^T . P^T, once
//    the V^T operand is read with the matching key order.
//  * Key tiles past the wavefront's last query position are skipped; only
//    tiles that cross the diagonal are masked.
#include "device_common.h"
#include "launch.h"

namespace pkv {

constexpr int kPfWaves = 4;
constexpr int kPfRows = 32 * kPfWaves;  // packed rows per workgroup
constexpr int kPfKeys = 32;             // keys per tile
constexpr float kPfNegInf = -__builtin_huge_valf();

template <int D>
struct PfLds {
  static constexpr int kKStride = D + 8;        // bf16 elements per K row (16-byte pad)
  static constexpr int kVStride = kPfKeys + 4;  // bf16 elements per V^T row (8-byte pad)
  uint16_t k[kPfKeys * kKStride];
  uint16_t vt[D * kVStride];
};

// Accumulator element r of a 32x32 MFMA result in lane (col, half) is row
// 8 * (r / 4) + 4 * half + r % 4.
__device__ __forceinline__ int mfma32_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

template <int D>
__global__ __launch_bounds__(256) void prefill_bf16_kernel(PrefillArgs a) {
  __shared__ PfLds<D> lds;
  constexpr int NC = D / 16;   // 16-channel chunks (K dimension of S^T)
  constexpr int NT = D / 32;   // 32-channel tiles of O^T

  const int s = blockIdx.z;
  const int kvh = blockIdx.y;
  const int g = a.g;
  const int q0 = a.cu_seqlens_q[s];
  const int n = a.cu_seqlens_q[s + 1] - q0;
  int L = a.context_lens[s];
  L = max(0, min(L, a.max_blocks_per_seq * kBlock));
  const int rows = n * g;
  const int r0 = blockIdx.x * kPfRows;
  if (n <= 0 || n > L || r0 >= rows || q0 < 0 || q0 + n > a.T_q) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;
  const int first = L - n;  // position of query 0

  // This lane's query row.
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
  const int n_tiles = (wg_pos_hi + kPfKeys) / kPfKeys;

  // Q^T operand (B of S^T = K Q^T): lane (col, half) holds channels
  // 16c + 8*half .. +8 of its row; rows past the end are zero.
  bf16x8_t qb[NC];
  {
    const uint4* qv = reinterpret_cast<const uint4*>(a.q);
    const size_t rowv = ((size_t)(q0 + tok) * a.h_q + kvh * g + hh) * (D / 8);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint4 x = row_ok ? qv[rowv + 2 * c + half] : make_uint4(0, 0, 0, 0);
      qb[c] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  f32x16_t o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  float m = kPfNegInf;
  float lsum = 0.f;

  const uint4* kc = reinterpret_cast<const uint4*>(a.k_cache);
  const uint4* vc = reinterpret_cast<const uint4*>(a.v_cache);
  const int32_t* tbl = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  constexpr int kVecPerRow = D / 8;                   // 16-byte vectors per token row
  constexpr int kTileVecs = kPfKeys * kVecPerRow;     // vectors per K (or V) tile

  for (int kt = 0; kt < n_tiles; ++kt) {
    // Gather the K and V tiles of keys kt*32 .. kt*32+31 into LDS.
    for (int i = tid; i < kTileVecs; i += blockDim.x) {
      const int key = i / kVecPerRow;
      const int cv = i - key * kVecPerRow;
      const int kpos = kt * kPfKeys + key;
      uint4 kx = make_uint4(0, 0, 0, 0), vx = make_uint4(0, 0, 0, 0);
      if (kpos < L) {
        int blk = tbl[kpos >> 4];
        blk = (blk >= 0 && blk < a.n_blocks) ? blk : 0;
        const size_t src = (((size_t)blk * a.h_kv + kvh) * kBlock + (kpos & 15)) * kVecPerRow + cv;
        kx = kc[src];
        vx = vc[src];
      }
      *reinterpret_cast<uint4*>(&lds.k[key * PfLds<D>::kKStride + cv * 8]) = kx;
      const uint32_t vw[4] = {vx.x, vx.y, vx.z, vx.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lds.vt[(cv * 8 + 2 * e) * PfLds<D>::kVStride + key] = (uint16_t)(vw[e] & 0xffffu);
        lds.vt[(cv * 8 + 2 * e + 1) * PfLds<D>::kVStride + key] = (uint16_t)(vw[e] >> 16);
      }
    }
    __syncthreads();

    if (wave_live && kt * kPfKeys <= wave_pos_hi) {
      // S^T tile: rows = 32 keys, columns = this wave's 32 query rows.
      f32x16_t st;
#pragma unroll
      for (int i = 0; i < 16; ++i) st[i] = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint4 kx = *reinterpret_cast<const uint4*>(
            &lds.k[col * PfLds<D>::kKStride + c * 16 + half * 8]);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kx), qb[c], st, 0, 0, 0);
      }
      float sv[16];
      const bool diag = kt * kPfKeys + kPfKeys - 1 > wave_pos_lo;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = st[i] * a.scale_log2;
        if (diag && kt * kPfKeys + mfma32_row(i, half) > pos) x = kPfNegInf;
        sv[i] = x;
      }
      float tmax = sv[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, sv[i]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mn = fmaxf(m, tmax);
      const float alpha = mn == m ? 1.f : fast_exp2(m - mn);
      m = mn;
      float p[16];
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = fast_exp2(sv[i] - mn);
        ps += p[i];
      }
      lsum = lsum * alpha + ps;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] *= alpha;

      // P^T operand for key chunk c (keys 16c..16c+15): element e of lane
      // (col, half) is key 16c + 8*(e/4) + 4*half + e%4 = accumulator 8c + e.
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        uint4 pw;
        pw.x = pack_bf16x2(p[8 * c + 0], p[8 * c + 1]);
        pw.y = pack_bf16x2(p[8 * c + 2], p[8 * c + 3]);
        pw.z = pack_bf16x2(p[8 * c + 4], p[8 * c + 5]);
        pw.w = pack_bf16x2(p[8 * c + 6], p[8 * c + 7]);
        const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          // V^T operand: row = channel 32t + col, same key order as P^T.
          const uint16_t* vrow = &lds.vt[(t * 32 + col) * PfLds<D>::kVStride + 16 * c + 4 * half];
          uint4 vx;
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
          vx.x = lo.x; vx.y = lo.y; vx.z = hi.x; vx.w = hi.y;
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vx), pb, o[t], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  if (!row_ok) return;
  const float lt = lsum + __shfl_xor(lsum, 32);
  const float inv = 1.f / lt;
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  const size_t orow = ((size_t)(q0 + tok) * a.h_q + kvh * g + hh) * D;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int ch = t * 32 + 8 * grp + 4 * half;
      uint2 w;
      w.x = pack_bf16x2(o[t][4 * grp + 0] * inv, o[t][4 * grp + 1] * inv);
      w.y = pack_bf16x2(o[t][4 * grp + 2] * inv, o[t][4 * grp + 3] * inv);
      *reinterpret_cast<uint2*>(&out[orow + ch]) = w;
    }
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, int d_h, hipStream_t stream) {
  const int64_t rows = (int64_t)a.max_q_len * a.g;
  const int64_t gx = (rows + kPfRows - 1) / kPfRows;
  dim3 grid((unsigned)gx, a.h_kv, a.S);
  if (d_h == 64)
    hipLaunchKernelGGL(prefill_bf16_kernel<64>, grid, dim3(256), 0, stream, a);
  else if (d_h == 128)
    hipLaunchKernelGGL(prefill_bf16_kernel<128>, grid, dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
