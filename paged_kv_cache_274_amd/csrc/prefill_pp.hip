// Causal chunked prefill with two waves per SIMD in alternating phases (gfx950).
//
// The contraction is that of prefill_bf16_kernel: GQA rows packed (row =
// token * g + head-in-group), keys in tiles of 64 copied from the paged pool
// straight into LDS with the same swizzle, S^T = K . Q^T and O^T = V^T . P^T on
// v_mfma_f32_32x32x16_bf16, and an fp32 online softmax in base 2 with a lazy
// reference max.  What differs is how a compute unit's time is spent.
//
// A wavefront's work on one key tile is a matrix phase (the tile's scores,
// 16 MFMAs at d_h = 128, and the previous tile's P.V, 16 more) and a vector
// phase (the online softmax of the tile's scores: masking, maxima, the
// exponentials, the bf16 weights).  With one wavefront per SIMD the matrix
// cores idle through every vector phase.  Here a workgroup holds 8 wavefronts
// (256 packed rows), two on every SIMD, and wavefronts 4..7 run one phase
// behind wavefronts 0..3: while one wavefront of a SIMD issues its MFMAs, the
// other runs its softmax.  Workgroup barriers separate the phases; between two
// barriers one group is in its matrix phase and the other in its vector phase.
//
// Key and value tiles have rings of three LDS slots each.  Every wavefront
// copies 8 rows of K and 8 of V of a tile; tile t + 2's keys and tile t + 1's
// values are issued when the group ahead starts tile t's matrix phase, two
// tile periods before their first use.  Rows past the context are copied from
// the context's last row instead (finite data): their keys are masked by the
// causal rule, and their values meet a zero weight, so nothing past the
// context reaches the product whatever the pool holds there.
#include <type_traits>

#include "prefill_common.h"

namespace pkv {

constexpr int kPpWaves = 8;
constexpr int kPpRows = 32 * kPpWaves;  // packed rows per workgroup

template <int D>
__global__ __launch_bounds__(64 * kPpWaves) void prefill_pp_kernel(PrefillArgs a) {
  using Tl = PfTile<D>;
  constexpr int kMat = Tl::kMatBytes;  // one tile of K or of V
  __shared__ __attribute__((aligned(16))) unsigned char lds[6 * kMat];  // K slots 0-2, V slots 0-2
  constexpr int NC = D / 16;  // 16-channel chunks (K dimension of S^T)
  constexpr int NT = D / 32;  // 32-channel tiles of O^T
  constexpr int kRowsPerWave = kPfTile / kPpWaves;                   // rows of a tile one wave copies
  constexpr int kCopies = kRowsPerWave / Tl::kRowsPerCopy;           // copies per wave per matrix
  static_assert(kCopies >= 1 && kRowsPerWave % Tl::kRowsPerCopy == 0, "copy shape");

  // One-dimensional grid, dispatched in order: the sequence planes (KV head,
  // sequence) vary fastest and the row block slowest, last row block first, so
  // the workgroups with the most key tiles (the last rows of every sequence)
  // all start before any shorter one (longest processing time first).
  const int planes = a.h_kv * a.S;
  const int plane = blockIdx.x % planes;
  const int bx = (int)(gridDim.x / planes) - 1 - (int)(blockIdx.x / planes);
  const int s = a.longest_first ? longest_first_sequence(a, plane / a.h_kv) : plane / a.h_kv;
  const int kvh = plane % a.h_kv;
  const int g = a.g;
  const int q0 = a.cu_seqlens_q[s];
  const int n = a.cu_seqlens_q[s + 1] - q0;
  int L = a.context_lens[s];
  L = max(0, min(L, a.max_blocks_per_seq * kBlock));
  const int rows = n * g;
  const int r0 = bx * kPpRows;
  if (n <= 0 || n > L || r0 >= rows || q0 < 0 || q0 + n > a.T_q) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int phase_lag = wave >> 2;  // 0: leading group, 1: one phase behind
  const int col = lane & 31;
  const int half = lane >> 5;
  const int first = L - n;  // position of query 0

  // This lane's query row (rows past the end compute the last row's values
  // and are not stored).
  const int r = r0 + wave * 32 + col;
  const bool row_ok = r < rows;
  const int tok = row_ok ? r / g : n - 1;
  const int hh = row_ok ? r - (r / g) * g : 0;
  const int pos = first + tok;

  const int wave_r0 = r0 + wave * 32;
  const bool wave_live = wave_r0 < rows;
  const int wave_pos_lo = first + wave_r0 / g;
  const int wave_pos_hi = first + (min(wave_r0 + 31, rows - 1)) / g;
  const int wg_pos_hi = first + (min(r0 + kPpRows - 1, rows - 1)) / g;
  const int n_tiles = uniform(wg_pos_hi / kPfTile + 1);
  const int mine = uniform(wave_live ? wave_pos_hi / kPfTile + 1 : 0);  // tiles this wave attends

  const float csc = fabsf(a.scale_log2);
  const uint32_t qsign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  f32x16_t o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  float m = kPfNegInf;
  float lsum = 0.f;
  f32x16_t st[2];  // scores of the tile in flight (matrix phase -> vector phase)
  bf16x8_t pb[4];  // its weights, one 16-key chunk each (vector phase -> next matrix phase)
  bf16x8_t qb[NC];

  const unsigned char* kc = reinterpret_cast<const unsigned char*>(a.k_cache);
  const unsigned char* vc = reinterpret_cast<const unsigned char*>(a.v_cache);
  const int32_t* trow = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  const size_t head_bytes = (size_t)kBlock * Tl::kRowBytes;
  const int last_tok = L - 1;

  // Block-table entry of this wave's block of tile kt (the context's last
  // block for a tile past it), clamped into the pool.  Entries are loaded one
  // tile period before their copies are issued, so the scalar load's latency
  // stays off the walk.
  auto entry = [&](int kt) -> int {
    const int bi = min(kt * (kPfTile / kBlock) + (wave >> 1), last_tok >> 4);
    return constant_view(trow)[bi];
  };
  auto clamp_entry = [&](int blk) { return (blk >= 0 && blk < a.n_blocks) ? blk : 0; };
  // Lane part of each copy's source (row rb of the block, the chunk that lands
  // at this lane's LDS position) for blocks wholly inside the context.
  uint32_t src_off[kCopies], chunk_off[kCopies];
#pragma unroll
  for (int i = 0; i < kCopies; ++i) {
    const int rb = 8 * (wave & 1) + i * Tl::kRowsPerCopy + lane / Tl::kChunks;
    const int row = kRowsPerWave * wave + i * Tl::kRowsPerCopy + lane / Tl::kChunks;
    chunk_off[i] = ((lane % Tl::kChunks) ^ Tl::swz(row)) * 16;
    src_off[i] = rb * Tl::kRowBytes + chunk_off[i];
  }
  // Copies this wave's 8 rows of tile kt of one matrix (K or V), which live in
  // pool block blk, into its slot.  Tile row 8 * wave + j is row
  // 8 * (wave & 1) + j of the tile's block wave / 2; a row at or past the
  // context is read from the context's last row, so every address stays inside
  // the sequence's own blocks.
  auto issue = [&](const unsigned char* pool, unsigned char* slot, int kt, int blk) {
    const unsigned char* src = pool + ((size_t)blk * a.h_kv + kvh) * head_bytes;
    const int bi = kt * (kPfTile / kBlock) + (wave >> 1);
    if (bi * kBlock + kBlock <= L) {
#pragma unroll
      for (int i = 0; i < kCopies; ++i)
        copy_to_lds_off(src, src_off[i],
                        slot + (kRowsPerWave * wave + i * Tl::kRowsPerCopy) * Tl::kRowBytes);
    } else {
#pragma unroll
      for (int i = 0; i < kCopies; ++i) {
        const int rb = 8 * (wave & 1) + i * Tl::kRowsPerCopy + lane / Tl::kChunks;
        const int rbe = bi * kBlock + rb < L ? rb : (last_tok & (kBlock - 1));
        copy_to_lds_off(src, rbe * Tl::kRowBytes + chunk_off[i],
                        slot + (kRowsPerWave * wave + i * Tl::kRowsPerCopy) * Tl::kRowBytes);
      }
    }
  };
  auto kslot = [&](int kt) { return lds + (kt % 3) * kMat; };
  auto vslot = [&](int kt) { return lds + (3 + kt % 3) * kMat; };

  // LDS addresses of the operands.  In the swizzled layout, row r's 16-byte
  // chunk c sits at r * kRowBytes + ((c ^ swz(r)) << 4), and swz(r) depends on
  // r's low 4 bits only.  So a lane's K operand for channel step c (row
  // 32 h2 + col, chunk 2c + half) is kbase ^ (c << 5) plus 32 h2 rows, and its
  // V^T operand for 32-channel tile t and keys 16c + ... is vbase ^ (t << 6)
  // plus 16c rows: one XOR per read, the rest immediate offsets.
  const int grp = lane >> 4;
  const int tr_row = 4 * (grp >> 1) + ((lane & 15) >> 2);
  const int tr_ch = 16 * (grp & 1) + 4 * (lane & 3);
  const uint32_t kbase = col * Tl::kRowBytes + ((half ^ Tl::swz(col)) << 4);
  const uint32_t vbase_lo = tr_row * Tl::kRowBytes + (((tr_ch >> 3) ^ Tl::swz(tr_row)) << 4) +
                            (tr_ch & 4) * 2;
  const uint32_t vbase_hi = (tr_row + 8) * Tl::kRowBytes +
                            (((tr_ch >> 3) ^ Tl::swz(tr_row + 8)) << 4) + (tr_ch & 4) * 2;
  const PKV_LDS unsigned char* lds_as = (const PKV_LDS unsigned char*)lds;

  auto k_operand = [&](uint32_t kb, int h2, int c) {
    return *(const PKV_LDS bf16x8_t*)(lds_as + ((kb ^ (c << 5)) + h2 * 32 * Tl::kRowBytes));
  };
  auto v_operand = [&](uint32_t vlo, uint32_t vhi, int c, int t) {
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (PKV_LDS i16x4_t*)(lds_as + ((vlo ^ (t << 6)) + 16 * c * Tl::kRowBytes)));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (PKV_LDS i16x4_t*)(lds_as + ((vhi ^ (t << 6)) + 16 * c * Tl::kRowBytes)));
    const i16x4_t lohi[2] = {lo, hi};
    return __builtin_bit_cast(bf16x8_t, lohi);
  };

  // Matrix phase of tile kt: S^T of tile kt (if attended) and O^T += V^T P^T
  // of tile kt - 1 (if attended), interleaved in four steps.  Step c takes
  // the S^T products of channel chunks [NC/4 * c, NC/4 * (c + 1)) and the P.V
  // products of keys 16c .. 16c + 15; a scheduling barrier between steps keeps
  // the compiler from hoisting every step's LDS reads at once, which would
  // need more registers than two waves per SIMD have.
  // Which products a matrix phase runs: this tile's scores (kS) and the
  // previous tile's P.V (kPV).  A wave attends tiles 0 .. mine - 1, so tile 0
  // has scores only, tile mine P.V only, the tiles between both, and the tiles
  // past mine (the other waves' diagonal) neither; each case is its own
  // straight-line code so the waits on LDS reads stay exact.
  auto matrix_phase = [&](int kt, auto KS_, auto KPV_) {
    constexpr bool kS = decltype(KS_)::value, kPV = decltype(KPV_)::value;
    const uint32_t kb = (uint32_t)((kt % 3) * kMat) + kbase;
    const uint32_t vs = (uint32_t)((3 + (kt + 2) % 3) * kMat);  // slot of tile kt - 1
    const uint32_t vlo = vs + vbase_lo;
    const uint32_t vhi = vs + vbase_hi;
    constexpr int kPerStep = NC / 4;
    if constexpr (kS) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 16; ++i) st[h2][i] = 0.f;
    }
    // Operands of one step: read one step ahead, while the previous step's
    // products run.
    bf16x8_t kx[2][kPerStep][2], vx[2][NT];
    auto load = [&](int c, int b) {
      if constexpr (kS) {
#pragma unroll
        for (int k = 0; k < kPerStep; ++k)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) kx[b][k][h2] = k_operand(kb, h2, c * kPerStep + k);
      }
      if constexpr (kPV) {
#pragma unroll
        for (int t = 0; t < NT; ++t) vx[b][t] = v_operand(vlo, vhi, c, t);
      }
    };
    load(0, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int b = c & 1;
      if (c < 3) load(c + 1, b ^ 1);
      if constexpr (kS) {
#pragma unroll
        for (int k = 0; k < kPerStep; ++k)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
            st[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kx[b][k][h2], qb[c * kPerStep + k],
                                                             st[h2], 0, 0, 0);
      }
      if constexpr (kPV) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vx[b][t], pb[c], o[t], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Vector phase of tile kt: causal mask, online softmax, bf16 weights.
  auto vector_phase = [&](int kt) {
    const int key0 = kt * kPfTile;
    if (key0 + kPfTile - 1 > wave_pos_lo) {
      const int lim = pos - key0 - 4 * half;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * h2 + mfma32_row(i, 0) > lim) st[h2][i] = kPfNegInf;
    }
    // Row maximum as a tree of three-input maxima (depth 4, not a chain of 16).
    float t1[11];
#pragma unroll
    for (int j = 0; j < 10; ++j) {
      const int e = 3 * j;
      t1[j] = fmaxf(fmaxf(st[e >> 4][e & 15], st[(e + 1) >> 4][(e + 1) & 15]),
                    st[(e + 2) >> 4][(e + 2) & 15]);
    }
    t1[10] = fmaxf(st[1][14], st[1][15]);
    const float t2a = fmaxf(fmaxf(t1[0], t1[1]), t1[2]);
    const float t2b = fmaxf(fmaxf(t1[3], t1[4]), t1[5]);
    const float t2c = fmaxf(fmaxf(t1[6], t1[7]), t1[8]);
    const float t2d = fmaxf(t1[9], t1[10]);
    float tmax = fmaxf(fmaxf(t2a, t2b), fmaxf(t2c, t2d));
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
    const float mn = m == kPfNegInf ? 0.f : m;
    // The row sum adds the bf16 weights the P.V products use, two per v_dot2
    // against (1, 1), in two independent chains.
    const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // Weights of keys 16c .. 16c + 15 in the P^T operand order (see
      // prefill_bf16_kernel): accumulators 8 * (c % 2) .. + 7 of half-tile c / 2.
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(st[c >> 1][8 * (c & 1) + e], csc, -mn));
      uint32_t pw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pw[e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
      ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[0]), ones, ps0, false);
      ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[1]), ones, ps1, false);
      ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[2]), ones, ps0, false);
      ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[3]), ones, ps1, false);
      pb[c] = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
    }
    lsum += ps0 + ps1;
  };

  // Prologue: keys of tiles 0 and 1, values of tile 0, then Q; one wait for all.
  const int e0 = clamp_entry(entry(0));
  int e_v = clamp_entry(entry(1));  // entry of the tile whose values are issued next
  int e_k = clamp_entry(entry(2));  // entry of the tile whose keys are issued next
  issue(kc, kslot(0), 0, e0);
  if (n_tiles > 1) issue(kc, kslot(1), 1, e_v);
  issue(vc, vslot(0), 0, e0);
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
  tile_barrier();

  // Interval j is the time between barriers j and j + 1 (barrier 0 is the
  // prologue's).  The leading group runs tile t's matrix phase in interval 2t
  // and its vector phase in 2t + 1; the lagging group runs each phase one
  // interval later.  At the start of interval 2t every wave issues tile t + 2's
  // keys and tile t + 1's values into the slots that tiles t - 1 and t - 2
  // left (their last readers finished in interval 2t - 1); at the end of
  // interval 2t + 1 it waits for all but those copies, so tile t + 1's keys and
  // tile t's values, issued in interval 2t - 2, are published by the barrier
  // for interval 2t + 2.  The groups run separate loops whose bodies are
  // straight-line, so that the compiler keeps every accumulator in place.
  auto issue_for_interval = [&](int t) {  // the copies of interval 2t
    if (t + 2 < n_tiles) issue(kc, kslot(t + 2), t + 2, e_k);
    if (t + 1 < n_tiles) issue(vc, vslot(t + 1), t + 1, e_v);
  };
  // After interval 2t's copies: tile t + 3's entry, loaded at the start of a
  // vector phase and clamped (the first use of the loaded value, where the
  // wave waits for it) only at its end, behind a scheduling barrier, so the
  // load's latency hides under the softmax and no scalar load is in flight
  // when the next matrix phase waits on its LDS reads.
  int e_raw = 0;
  auto next_entries = [&](int t) {
    e_v = e_k;
    e_raw = entry(t + 3);
  };
  auto entries_landed = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    e_k = clamp_entry(e_raw);
  };
  auto wait_for_interval = [&](int t) {  // the wait at the end of interval 2t + 1
    const bool k = t + 2 < n_tiles, v = t + 1 < n_tiles;
    if (k && v)
      wait_vm<2 * kCopies>();
    else if (k || v)
      wait_vm<kCopies>();
    else
      wait_vm<0>();
  };
  // The entry loads go where this wave has no LDS reads in flight (before a
  // vector phase): a scalar load outstanding would make every LDS wait a
  // wait for it as well.
  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  if (phase_lag == 0) {
    // Intervals 2t (matrix phase) and 2t + 1 (vector phase).
    auto period = [&](int t, auto KS_, auto KPV_) {
      issue_for_interval(t);
      matrix_phase(t, KS_, KPV_);
      tile_barrier();
      next_entries(t);
      if constexpr (decltype(KS_)::value) vector_phase(t);
      entries_landed();
      wait_for_interval(t);
      tile_barrier();
    };
    int t = 0;
    if (mine >= 1) {
      period(0, T_{}, F_{});
      for (t = 1; t < mine; ++t) period(t, T_{}, T_{});
      period(mine, F_{}, T_{});
      t = mine + 1;
    }
    for (; t <= n_tiles; ++t) period(t, F_{}, F_{});
  } else {
    // Intervals 2t + 1 (matrix phase) and 2t + 2 (vector phase).
    issue_for_interval(0);
    next_entries(0);
    entries_landed();
    tile_barrier();
    auto period = [&](int t, auto KS_, auto KPV_) {
      matrix_phase(t, KS_, KPV_);
      wait_for_interval(t);
      tile_barrier();
      if (t == n_tiles) return;
      issue_for_interval(t + 1);
      next_entries(t + 1);
      if constexpr (decltype(KS_)::value) vector_phase(t);
      entries_landed();
      tile_barrier();
    };
    int t = 0;
    if (mine >= 1) {
      period(0, T_{}, F_{});
      for (t = 1; t < mine; ++t) period(t, T_{}, T_{});
      period(mine, F_{}, T_{});
      t = mine + 1;
    }
    for (; t <= n_tiles; ++t) period(t, F_{}, F_{});
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

hipError_t launch_prefill_pp(const PrefillArgs& a, int d_h, hipStream_t stream) {
  const int64_t rows = (int64_t)a.max_q_len * a.g;
  const int64_t gx = (rows + kPpRows - 1) / kPpRows;
  const int64_t n_wg = gx * a.h_kv * a.S;
  if (n_wg > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)n_wg);
  if (d_h == 64)
    hipLaunchKernelGGL((prefill_pp_kernel<64>), grid, dim3(64 * kPpWaves), 0, stream, a);
  else if (d_h == 128)
    hipLaunchKernelGGL((prefill_pp_kernel<128>), grid, dim3(64 * kPpWaves), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
