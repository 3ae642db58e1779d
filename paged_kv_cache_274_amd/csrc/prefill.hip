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
//  * Keys are walked in tiles of 64 (four blocks).  Each wavefront copies one
//    block of K and of V per tile straight from HBM into LDS
//    (global_load_lds_dwordx4, no register staging), and three tile buffers
//    keep the next two tiles in flight while the current one is used.
//  * LDS rows are key-major and unpadded; the 16-byte chunk c of row r sits at
//    chunk position c ^ swz(r), chosen so that both the K operand reads (16
//    consecutive rows at one chunk) and the transposed V reads (4 rows x 64
//    bytes) touch every bank once.
//  * The wavefront computes S^T = K . Q^T (keys x its 32 query rows), so a lane
//    holds the scores of one query row; the row max and sum need one exchange
//    with the other half-wave.  The scores' accumulator layout is exactly the B
//    operand layout of the next product, O^T = V^T . P^T, with the keys of each
//    16-key chunk taken in the matching order; the V^T operand comes from the
//    key-major V rows through ds_read_b64_tr_b16, which hands each lane four
//    consecutive keys of one channel.
//  * Key tiles past the wavefront's last query position are skipped; only
//    tiles that cross the diagonal are masked.  V rows past the context (the
//    tail of the last block, or blocks beyond it) are zeroed in LDS so that
//    whatever the pool holds there never reaches the product.
#include <type_traits>

#include "prefill_common.h"

namespace pkv {

// KS wave groups of 4 share a workgroup's 128 rows and split its key tiles:
// group G takes tiles G, G + KS, G + 2 KS, ... with three buffers of its own,
// and the groups' softmax states are merged at the end.  KS = 2 halves the
// serial key walk of the longest rows when the grid alone cannot fill the chip.
template <int D, int KS>
__global__ __launch_bounds__(256 * KS) void prefill_bf16_kernel(PrefillArgs a) {
  using Tl = PfTile<D>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[KS * 3 * Tl::kBufBytes];
  constexpr int NC = D / 16;   // 16-channel chunks (K dimension of S^T)
  constexpr int NT = D / 32;   // 32-channel tiles of O^T
  constexpr int kCopies = 2 * Tl::kCopiesPerBlock;  // copies per wave per tile (K and V)

  // Workgroups with the most key tiles (the last rows of a sequence) first.
  const int bx = gridDim.x - 1 - blockIdx.x;
  const int s = a.longest_first ? longest_first_sequence(a, blockIdx.z) : (int)blockIdx.z;
  const int kvh = blockIdx.y;
  const int g = a.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);  // row wave in the group
  const int grp_id = __builtin_amdgcn_readfirstlane(tid >> 8);       // key-split group
  // Block-table entries of this wave's blocks of tile kt.  The index stays
  // inside the table row without waiting for the context length: entries past
  // the context may hold anything, so the block id is clamped into the pool
  // when used, and those rows are masked (K) or zeroed (V).  The first two
  // tiles' entries are loaded together with the sequence's offsets, one
  // memory round trip before they would be otherwise.
  const int32_t* trow = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  auto entry = [&](int kt) -> int {
    return constant_view(trow)[min(kt * (kPfTile / kBlock) + wave, a.max_blocks_per_seq - 1)];
  };
  int e_a = entry(grp_id);
  const int e_b = entry(grp_id + KS);
  const int q0 = a.cu_seqlens_q[s];
  const int n = a.cu_seqlens_q[s + 1] - q0;
  int L = a.context_lens[s];
  L = max(0, min(L, a.max_blocks_per_seq * kBlock));
  const int rows = n * g;
  const int r0 = bx * kPfRows;
  if (n <= 0 || n > L || r0 >= rows || q0 < 0 || q0 + n > a.T_q) return;

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
  const int n_tiles = uniform(wg_pos_hi / kPfTile + 1);
  const int n_steps = (n_tiles + KS - 1) / KS;  // tiles per group, rounded up
  const int Lu = uniform(L);

  bf16x8_t qb[NC];  // filled once the first tiles are in flight
  // Scores enter the softmax as s * c with c = |scale| * log2(e) > 0; a negative
  // scale flips the sign bits of Q instead (exact), so that the row maximum of
  // s * c is c times the maximum of s.
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
  const size_t head_bytes = (size_t)kBlock * Tl::kRowBytes;

  // The group's i-th tile lives in its buffer i % 3.
  auto buffer_of = [&](int group, auto B) -> unsigned char* {
    return lds + (group * 3 + decltype(B)::value) * Tl::kBufBytes;
  };
  auto buffer = [&](auto B) -> unsigned char* { return buffer_of(grp_id, B); };

  // Copies this wave's block of a tile (block id blk, block 4 * kt + wave of
  // the table row), K and V, into buffer B.  Lane l
  // of copy i fills LDS row 16 * wave + i * kRowsPerCopy + l / kChunks at chunk
  // position l % kChunks, i.e. logical chunk (l % kChunks) ^ swz(row).
  auto issue_tile = [&](auto B, int blk) {
    blk = (blk >= 0 && blk < a.n_blocks) ? blk : 0;
    const size_t gbase = ((size_t)blk * a.h_kv + kvh) * head_bytes;
    unsigned char* buf = buffer(B);
#pragma unroll
    for (int i = 0; i < Tl::kCopiesPerBlock; ++i) {
      const int rb = i * Tl::kRowsPerCopy + lane / Tl::kChunks;       // row within the block
      const int row = wave * kBlock + rb;                               // row within the tile
      const int chunk = (lane % Tl::kChunks) ^ Tl::swz(row);
      const size_t src = gbase + (size_t)rb * Tl::kRowBytes + chunk * 16;
      const int ldst = (wave * kBlock + i * Tl::kRowsPerCopy) * Tl::kRowBytes;
      copy_to_lds(kc + src, buf + ldst);
      copy_to_lds(vc + src, buf + Tl::kMatBytes + ldst);
    }
  };

  // Transposed-read addressing: within each 16-lane group, lane j points at key
  // kq + j / 4 and channel cq + 4 * (j % 4) and receives, for k = 0..3, channel
  // cq + j of key kq + k.
  const int grp = lane >> 4;
  const int tr_row = 4 * (grp >> 1) + ((lane & 15) >> 2);
  const int tr_ch = 16 * (grp & 1) + 4 * (lane & 3);

  // Attends tile kt (in buffer B): S^T, online softmax, O^T += V^T P^T.
  auto attend_tile = [&](auto B, int kt) {
    const unsigned char* kb_lds = buffer(B);
    const unsigned char* vb_lds = buffer(B) + Tl::kMatBytes;
    const int key0 = kt * kPfTile;
    f32x16_t st[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) st[h2][i] = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint4 kx = *reinterpret_cast<const uint4*>(kb_lds + Tl::offset(32 * h2 + col, 2 * c + half));
        st[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kx), qb[c],
                                                         st[h2], 0, 0, 0);
      }
    }
    // Causal mask on tiles that cross the diagonal: element (h2, i) holds key
    // key0 + 32 * h2 + mfma32_row(i, half), masked when past this row's position;
    // compared as a compile-time offset against one per-lane limit.
    if (key0 + kPfTile - 1 > wave_pos_lo) {
      const int lim = pos - key0 - 4 * half;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * h2 + mfma32_row(i, 0) > lim) st[h2][i] = kPfNegInf;
    }
    float tmax = kPfNegInf;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, st[h2][i]);
    tmax = xor32_max(tmax) * csc;
    // Lazy rescale: the reference max only moves when a score exceeds it by
    // more than 2^kPfSlack, so O^T and the sum are rarely rescaled (exact
    // either way: the weights are taken against the same reference m).
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
    // A row whose keys so far were all masked (possible for the second key
    // group, which starts at tile 1) keeps m = -inf; its scores are all -inf,
    // and a finite reference gives them weight 0 instead of -inf + inf.
    const float mn = m == kPfNegInf ? 0.f : m;
    float ps = 0.f;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(st[h2][i], csc, -mn));
        st[h2][i] = p;
        ps += p;
      }
    lsum += ps;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // P^T operand for keys 16c .. 16c + 15: element e of lane (col, half) is
      // key 16c + 8 * (e / 4) + 4 * half + e % 4 = accumulator 8 * (c % 2) + e of
      // half-tile c / 2.
      const f32x16_t& sc = st[c >> 1];
      const int e0 = 8 * (c & 1);
      uint4 pw;
      pw.x = pack_bf16x2(sc[e0 + 0], sc[e0 + 1]);
      pw.y = pack_bf16x2(sc[e0 + 2], sc[e0 + 3]);
      pw.z = pack_bf16x2(sc[e0 + 4], sc[e0 + 5]);
      pw.w = pack_bf16x2(sc[e0 + 6], sc[e0 + 7]);
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        // V^T operand: row = channel 32t + col, keys in the order of P^T.
        const int ch = 32 * t + tr_ch;
        const int ra = 16 * c + tr_row;
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (PKV_LDS i16x4_t*)(vb_lds + Tl::offset(ra, ch >> 3) + (ch & 4) * 2));
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (PKV_LDS i16x4_t*)(vb_lds + Tl::offset(ra + 8, ch >> 3) + (ch & 4) * 2));
        const i16x4_t lohi[2] = {lo, hi};
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, lohi), pb,
                                                       o[t], 0, 0, 0);
      }
    }
  };

  // Step i of the walk: every group attends its i-th tile, tile kt = i * KS +
  // group, from buffer B = i % 3; false past the last step.  All groups pass
  // the same barriers.
  auto step = [&](auto B, int i) -> bool {
    if (i >= n_steps) return false;
    const int kt = i * KS + grp_id;
    const bool mine = kt < n_tiles;
    // This wave's copies of tile kt have landed once only the group's next
    // tile's remain; after the barrier every wave's have, and every wave is
    // done with its previous tile, whose buffer the copy two tiles ahead then
    // refills.
    if (mine && kt + KS < n_tiles)
      wait_vm<kCopies>();
    else
      wait_vm<0>();
    tile_barrier();
    const int last = n_tiles - 1;  // the only tile that can reach past the context
    if (i == last / KS && (last + 1) * kPfTile > Lu) {
      // Zero its V rows past the context (all threads, in the owning group's buffer).
      unsigned char* vb = buffer_of(last % KS, B) + Tl::kMatBytes;
      const int zr = max(0, Lu - last * kPfTile);
      for (int z = tid; z < (kPfTile - zr) * Tl::kChunks; z += 256 * KS)
        *reinterpret_cast<uint4*>(vb + (zr + z / Tl::kChunks) * Tl::kRowBytes + (z % Tl::kChunks) * 16) =
            make_uint4(0, 0, 0, 0);
      wait_lds();
      tile_barrier();
    }
    if (mine && kt + 2 * KS < n_tiles)
      issue_tile(std::integral_constant<int, (decltype(B)::value + 2) % 3>{}, e_a);
    if (mine && wave_live && kt * kPfTile <= wave_pos_hi) attend_tile(B, kt);
    // The entry of the tile the next step issues, loaded after this tile's LDS
    // reads (a scalar load in flight makes every LDS wait a full wait) and
    // used one barrier later.
    __builtin_amdgcn_sched_barrier(0);
    e_a = entry(kt + 3 * KS);
    return true;
  };

  if (grp_id < n_tiles) issue_tile(std::integral_constant<int, 0>{}, e_a);
  if (grp_id + KS < n_tiles) issue_tile(std::integral_constant<int, 1>{}, e_b);
  e_a = entry(grp_id + 2 * KS);

  // Q^T operand (B of S^T = K Q^T): lane (col, half) holds channels
  // 16c + 8*half .. +8 of its row; rows past the end are zero.  The wait that
  // follows also covers the first two tiles' copies, issued just before, so
  // no load is left pending that the loop below would wait on.
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
  wait_vm<0>();
  for (int i = 0;; i += 3) {
    if (!step(std::integral_constant<int, 0>{}, i)) break;
    if (!step(std::integral_constant<int, 1>{}, i + 1)) break;
    if (!step(std::integral_constant<int, 2>{}, i + 2)) break;
  }

  if constexpr (KS == 2) {
    // Group 1 hands its state for the same rows to group 0 through LDS (field
    // f of lane l of row wave w at float (f * 4 + w) * 64 + l), which merges
    // the two with the log-sum-exp rule.
    constexpr int kFields = NT * 16 + 2;
    static_assert(kFields * 4 * 64 * 4 <= (int)sizeof(lds), "merge area");
    float* mg = reinterpret_cast<float*>(lds);
    auto at = [&](int f) -> float& { return mg[(f * 4 + wave) * 64 + lane]; };
    tile_barrier();  // every wave is done with the tile buffers
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
    const float a0 = fast_exp2(m - mm);
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
      const int ch = t * 32 + 8 * gq + 4 * half;
      uint2 w;
      w.x = pack_bf16x2(o[t][4 * gq + 0] * inv, o[t][4 * gq + 1] * inv);
      w.y = pack_bf16x2(o[t][4 * gq + 2] * inv, o[t][4 * gq + 3] * inv);
      *reinterpret_cast<uint2*>(&out[orow + ch]) = w;
    }
}

// Few query rows per (sequence, KV head): at most 32 packed rows (multi-token
// decode: a few new tokens times the GQA group), all held by every wave of the
// workgroup.  The key walk is split over the 4 waves instead of the rows: wave
// w attends the 32-key chunks w, w + 4, w + 8, ... of the context, each copied
// from HBM into the wave's own two LDS stages (one chunk in flight while the
// other is used), so the waves need no barrier until the end, where their
// softmax states are merged through LDS.  Four waves walk a context four times
// faster than the one wave that holds the rows in prefill_bf16_kernel.
constexpr int kFewKeys = 32;
template <int D>
__global__ __launch_bounds__(256) void prefill_few_rows_kernel(PrefillArgs a) {
  using Tl = PfTile<D>;
  constexpr int kStage = 2 * kFewKeys * Tl::kRowBytes;  // K then V of one chunk
  constexpr int kWaveBytes = 2 * kStage;
  constexpr int NC = D / 16;
  constexpr int NT = D / 32;
  constexpr int kCopies = 2 * 2 * Tl::kCopiesPerBlock;  // K and V of two blocks
  constexpr int kFields = NT * 16 + 2;                  // merge: O^T, m, l per lane
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
  const int Lu = uniform(L);
  const int n_chunks = (Lu + kFewKeys - 1) / kFewKeys;

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
  const int32_t* trow = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  const size_t head_bytes = (size_t)kBlock * Tl::kRowBytes;
  unsigned char* const mine = lds + wave * kWaveBytes;

  // Copies the two blocks of chunk c (keys 32c .. 32c + 31), K and V, into
  // stage st of this wave (rows = keys of the chunk, swizzled as PfTile).
  auto issue_chunk = [&](int c, int st) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int bi = min(2 * c + b, a.max_blocks_per_seq - 1);
      int blk = constant_view(trow)[bi];
      blk = (blk >= 0 && blk < a.n_blocks) ? blk : 0;
      const size_t gbase = ((size_t)blk * a.h_kv + kvh) * head_bytes;
#pragma unroll
      for (int i = 0; i < Tl::kCopiesPerBlock; ++i) {
        const int rb = i * Tl::kRowsPerCopy + lane / Tl::kChunks;  // row within the block
        const int row = b * kBlock + rb;                            // row within the chunk
        const int chunk = (lane % Tl::kChunks) ^ Tl::swz(row);
        const size_t src = gbase + (size_t)rb * Tl::kRowBytes + chunk * 16;
        const int ldst = (b * kBlock + i * Tl::kRowsPerCopy) * Tl::kRowBytes;
        copy_to_lds(kc + src, mine + st * kStage + ldst);
        copy_to_lds(vc + src, mine + st * kStage + kFewKeys * Tl::kRowBytes + ldst);
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

  const int grp = lane >> 4;
  const int tr_row = 4 * (grp >> 1) + ((lane & 15) >> 2);
  const int tr_ch = 16 * (grp & 1) + 4 * (lane & 3);

  if (wave < n_chunks) issue_chunk(wave, 0);
  for (int c = wave, st = 0; c < n_chunks; c += kPfWaves, st ^= 1) {
    const bool more = c + kPfWaves < n_chunks;
    if (more) issue_chunk(c + kPfWaves, st ^ 1);
    // This wave's copies of chunk c have landed (the next chunk's may stay in
    // flight); no other wave reads them.
    if (more)
      wait_vm<kCopies>();
    else
      wait_vm<0>();
    const unsigned char* kb = mine + st * kStage;
    unsigned char* vb = mine + st * kStage + kFewKeys * Tl::kRowBytes;
    const int key0 = c * kFewKeys;
    if (key0 + kFewKeys > Lu) {
      // V rows past the context of the last chunk are zeroed (own stage).
      const int zr = Lu - key0;
      for (int z = lane; z < (kFewKeys - zr) * Tl::kChunks; z += 64)
        *reinterpret_cast<uint4*>(vb + (zr + z / Tl::kChunks) * Tl::kRowBytes + (z % Tl::kChunks) * 16) =
            make_uint4(0, 0, 0, 0);
      wait_lds();
    }
    f32x16_t sc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = 0.f;
#pragma unroll
    for (int c2 = 0; c2 < NC; ++c2) {
      const uint4 kx = *reinterpret_cast<const uint4*>(kb + Tl::offset(col, 2 * c2 + half));
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kx), qb[c2], sc, 0,
                                                   0, 0);
    }
    if (key0 + kFewKeys - 1 > first) {
      const int lim = pos - key0 - 4 * half;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (mfma32_row(i, 0) > lim) sc[i] = kPfNegInf;
    }
    float tmax = kPfNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sc[i]);
    tmax = xor32_max(tmax) * csc;
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
    // A wave's first chunk can lie wholly past a row's position (m stays
    // -inf, all its scores -inf): a finite reference gives them weight 0.
    const float mb = m == kPfNegInf ? 0.f : m;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(fmaf(sc[i], csc, -mb));
      sc[i] = p;
      ps += p;
    }
    lsum += ps;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      // P^T for keys 16 c2 .. 16 c2 + 15: accumulator elements 8 c2 .. 8 c2 + 7.
      uint4 pw;
      pw.x = pack_bf16x2(sc[8 * c2 + 0], sc[8 * c2 + 1]);
      pw.y = pack_bf16x2(sc[8 * c2 + 2], sc[8 * c2 + 3]);
      pw.z = pack_bf16x2(sc[8 * c2 + 4], sc[8 * c2 + 5]);
      pw.w = pack_bf16x2(sc[8 * c2 + 6], sc[8 * c2 + 7]);
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int ch = 32 * t + tr_ch;
        const int ra = 16 * c2 + tr_row;
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (PKV_LDS i16x4_t*)(vb + Tl::offset(ra, ch >> 3) + (ch & 4) * 2));
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (PKV_LDS i16x4_t*)(vb + Tl::offset(ra + 8, ch >> 3) + (ch & 4) * 2));
        const i16x4_t lohi[2] = {lo, hi};
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, lohi), pb, o[t],
                                                       0, 0, 0);
      }
    }
    // Every LDS read of this stage is done before the stage is refilled by
    // the copy issued at the top of the iteration after next.
    wait_lds();
  }

  // Merge the four waves' states for the same rows through LDS (field f of
  // lane l of wave w at float (f * 4 + w) * 64 + l), in wave 0.
  float* mg = reinterpret_cast<float*>(lds);
  auto at = [&](int f, int w) -> float& { return mg[(f * kPfWaves + w) * 64 + lane]; };
  tile_barrier();  // every wave is done with its stages
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
      const int ch = t * 32 + 8 * gq + 4 * half;
      uint2 w;
      w.x = pack_bf16x2(o[t][4 * gq + 0] * inv, o[t][4 * gq + 1] * inv);
      w.y = pack_bf16x2(o[t][4 * gq + 2] * inv, o[t][4 * gq + 3] * inv);
      *reinterpret_cast<uint2*>(&out[orow + ch]) = w;
    }
}

static int compute_units() {
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
static hipError_t launch_d(const PrefillArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.max_q_len * a.g;
#ifndef PKV_PF_NO_FEW
  if (rows <= 32) {
    const dim3 grid(1, a.h_kv, a.S);
    PrefillArgs args = a;
    const int cus = compute_units();
    args.longest_first = a.S > 1 && a.S <= kLptMaxSeqs && cus > 0 && (int64_t)a.h_kv * a.S > cus;
    hipLaunchKernelGGL((prefill_few_rows_kernel<D>), grid, dim3(256), 0, stream, args);
    return hipGetLastError();
  }
#endif
#ifndef PKV_PF_NO_PP
  // Many rows per (sequence, KV head) and enough workgroups of 256 rows to
  // fill the chip: the 8-wave kernel whose wave pairs overlap one wave's MFMAs
  // with the other's softmax.
  {
    const int64_t gx8 = (rows + 255) / 256;
    const int cus = compute_units();
    if (rows >= 256 && cus > 0 && gx8 * a.h_kv * a.S >= cus) {
      PrefillArgs args = a;
      args.longest_first = a.S > 1 && a.S <= kLptMaxSeqs && gx8 * a.h_kv * a.S > cus;
      return launch_prefill_pp(args, D, stream);
    }
  }
#endif
  const int64_t gx = (rows + kPfRows - 1) / kPfRows;
  const dim3 grid((unsigned)gx, a.h_kv, a.S);
  // Order the sequence planes longest first when the grid takes more than one
  // round of the chip (one workgroup per compute unit is assumed: the tile
  // buffers of d_h = 128 fill most of its LDS) and the ranking stays cheap.
  PrefillArgs args = a;
  const int cus = compute_units();
  args.longest_first = a.S > 1 && a.S <= kLptMaxSeqs && cus > 0 && gx * a.h_kv * a.S > cus;
  // Split the key walk over two wave groups when the grid has no more
  // workgroups than the chip has compute units (d_h = 64: eight waves of this
  // kernel fit one compute unit's registers).
  if constexpr (D == 64) {
    if (gx * a.h_kv * a.S <= compute_units()) {
      hipLaunchKernelGGL((prefill_bf16_kernel<D, 2>), grid, dim3(512), 0, stream, args);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((prefill_bf16_kernel<D, 1>), grid, dim3(256), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, int d_h, hipStream_t stream) {
  if (d_h == 64) return launch_d<64>(a, stream);
  if (d_h == 128) return launch_d<128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
