// FP32 log-sum-exp merge of attention partials (KV-cache engineering page,
// section "Exact recent pages, compact older pages"): partial t is weighted
// by exp(lse_t - max lse), the weighted outputs are summed and divided by the
// summed weights, and the merged log-sum-exp is max + log(sum).
//
// One kernel serves two places on the path:
//   * the final merge of every slot of a row into one output (pkv_merge_partials);
//   * the tile finalize inside pkv_decode_attention, which merges the fixed
//     groups of split partials that make up one tile.
// Two waves own one (row, output slot), 128 channels each (two per lane, so
// more of the GPU's load queues work on a row and every load is 512
// contiguous bytes), and each walks its input
// slots in increasing order with one accumulator per channel, so the result
// is independent of scheduling, an empty slot (lse = -inf) contributes
// exactly nothing and a lone slot merges to itself bit for bit.
#include "device.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kMergeThreads = 64;     // one wave; lane i owns channels 128 * half + 2i, +1
constexpr int kMergeParts = kHeadDim / 128;   // waves per (row, output slot)
constexpr int kMergeChunk = 64;       // input slots whose loads are in flight together

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
  const int row = blockIdx.x;
  const int j = blockIdx.y;
  const int part = blockIdx.z;
  const int lane = threadIdx.x;
  const int t0 = j * a.group;
  const int cnt = min(a.group, a.in_slots - t0);

  const float* lse_in = a.in_lse + (int64_t)row * a.in_slots + t0;
  const float2* o_in = reinterpret_cast<const float2*>(
      a.in_o + ((int64_t)row * a.in_slots + t0) * kHeadDim + 128 * part) + lane;

  // The output loads of the first 64 slots do not depend on the max: they go
  // out first, beside this lane's log-sum-exp, so the max and the loads
  // overlap instead of taking two round trips to memory.
  float2 o[kMergeChunk];
  const int n0 = min(kMergeChunk, cnt);
#pragma unroll
  for (int u = 0; u < kMergeChunk; ++u)
    o[u] = (u < n0) ? o_in[(int64_t)u * (kHeadDim / 2)] : make_float2(0.f, 0.f);
  const float lv = (lane < cnt) ? lse_in[lane] : -INFINITY;

  // M = max_t lse_t over the group (NaN if any slot's is: the row's result
  // then comes out NaN instead of dropping that slot).
  float m = lv;
  for (int t = lane + kMergeThreads; t < cnt; t += kMergeThreads) m = max_nan(m, lse_in[t]);
  m = wave_max_nan(m);

  const int64_t orow = (int64_t)row * a.out_slots + a.out_slot0 + j;
  float2* o_out = reinterpret_cast<float2*>(a.out_o + orow * kHeadDim + 128 * part) + lane;
  if (m == -INFINITY) {                       // every slot empty
    *o_out = make_float2(0.f, 0.f);
    if (part == 0 && lane == 0) a.out_lse[orow] = -INFINITY;
    return;
  }

  // Chunks of 64 slots: lane u computes the weight of the chunk's slot u
  // (one exp per lane, all in parallel), then the slots are summed in
  // increasing order with each weight read from its lane.
  float2 acc = make_float2(0.f, 0.f);
  float wsum = 0.f;
  for (int c0 = 0; c0 < cnt; c0 += kMergeChunk) {
    const int nc = min(kMergeChunk, cnt - c0);
    if (c0 > 0) {
#pragma unroll
      for (int u = 0; u < kMergeChunk; ++u)
        o[u] = (u < nc) ? o_in[(int64_t)(c0 + u) * (kHeadDim / 2)] : make_float2(0.f, 0.f);
    }
    const float lt = (c0 == 0) ? lv : ((lane < nc) ? lse_in[c0 + lane] : -INFINITY);
    const float wl = (lane < nc) ? expf(lt - m) : 0.f;     // 0 for an empty slot
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u));
      if (w != 0.f) {                          // uniform across the wave
        acc.x = fmaf(w, o[u].x, acc.x);
        acc.y = fmaf(w, o[u].y, acc.y);
        wsum += w;
      }
    }
  }
  *o_out = make_float2(acc.x / wsum, acc.y / wsum);
  if (part == 0 && lane == 0) a.out_lse[orow] = m + logf(wsum);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int rows, hipStream_t stream) {
  if (rows <= 0 || a.n_out <= 0) return hipSuccess;
  dim3 grid(rows, a.n_out, kMergeParts);
  hipLaunchKernelGGL(merge_kernel, grid, dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
