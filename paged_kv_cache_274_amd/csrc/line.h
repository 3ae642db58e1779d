// The decode's work line and its cut, shared by the kernels and the host (the
// host inspection calls of the C ABI and their tests).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Positions are block indices on the line of all segments laid end to end.
// The line is cut in proportion to per-wave weights: the 4 waves of a
// workgroup share a weight, and workgroups go to the 8 XCDs in turn, so waves
// 0-3 of every 8 run on an even XCD and waves 4-7 on an odd one.  Measured
// per-wave end times (several boxes, both decode shapes) put the odd XCDs
// 7-10% behind the even ones on equal shares, whichever ranges they stream,
// so even XCDs take kWeightEven / kWeightOdd times an odd XCD's share.  Any
// positive weights give a valid cut; equal weights give the even cut
// w * total / splits exactly.  total * cum(splits) must fit int64 (the host
// bounds the line at kMaxLineBlocks).
constexpr int64_t kWeightEven = 11;
constexpr int64_t kWeightOdd = 10;
struct Line {
  int64_t total;  // blocks on the line (all segments)
  int splits;
  static constexpr int64_t kPer8 = 4 * (kWeightEven + kWeightOdd);  // weight of waves 8c .. 8c + 7
  // Weight of waves 0 .. u - 1.
  __host__ __device__ static int64_t cum(int u) {
    const int r = u & 7;
    return (int64_t)(u >> 3) * kPer8 +
           (r < 4 ? r * kWeightEven : 4 * kWeightEven + (r - 4) * kWeightOdd);
  }
  // First position of wave w's range (w = splits: the line's end).
  __host__ __device__ int64_t start(int w) const { return total * cum(w) / cum(splits); }
  // The wave whose range holds position p: the smallest w with start(w + 1) > p,
  // i.e. with cum(w + 1) >= ceil((p + 1) * cum(splits) / total).
  __host__ __device__ int wave_of(int64_t p) const {
    const int64_t t = ((p + 1) * cum(splits) + total - 1) / total;
    const int64_t c = t / kPer8;
    const int64_t rem = t - c * kPer8;
    int64_t u = 8 * c;
    if (rem > 4 * kWeightEven)
      u += 4 + (rem - 4 * kWeightEven + kWeightOdd - 1) / kWeightOdd;
    else if (rem > 0)
      u += (rem + kWeightEven - 1) / kWeightEven;
    return (int)u - 1;
  }
};

}  // namespace pkv
