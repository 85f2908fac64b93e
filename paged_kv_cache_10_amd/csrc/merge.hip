// FP32 log-sum-exp merge of attention partials (KV-cache engineering page,
// section "Exact recent pages, compact older pages"): partial t is weighted
// by exp(lse_t - max lse), the weighted outputs are summed and divided by the
// summed weights, and the merged log-sum-exp is max + log(sum).
//
// One kernel serves two places on the path:
//   * the final merge of every slot of a row into one output (pkv_merge_partials);
//   * the tile finalize inside pkv_decode_attention, which merges the fixed
//     groups of split partials that make up one tile.
// A wave owns one (row, output slot) and walks its input slots in increasing
// order with one accumulator per channel, so the result is independent of
// scheduling, an empty slot (lse = -inf) contributes exactly nothing and a
// lone slot merges to itself bit for bit.
#include "device.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kMergeThreads = 64;     // one wave; lane i owns channels 4i..4i+3
constexpr int kMergeUnroll = 8;       // input slots loaded ahead of their use

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
  const int row = blockIdx.x;
  const int j = blockIdx.y;
  const int lane = threadIdx.x;
  const int t0 = j * a.group;
  const int cnt = min(a.group, a.in_slots - t0);

  const float* lse_in = a.in_lse + (int64_t)row * a.in_slots + t0;
  const float4* o_in =
      reinterpret_cast<const float4*>(a.in_o + ((int64_t)row * a.in_slots + t0) * kHeadDim) + lane;

  // M = max_t lse_t over the group.
  float m = -INFINITY;
  for (int t = lane; t < cnt; t += kMergeThreads) m = fmaxf(m, lse_in[t]);
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));

  const int64_t orow = (int64_t)row * a.out_slots + a.out_slot0 + j;
  float4* o_out = reinterpret_cast<float4*>(a.out_o + orow * kHeadDim) + lane;
  if (m == -INFINITY) {                       // every slot empty
    *o_out = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane == 0) a.out_lse[orow] = -INFINITY;
    return;
  }

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.f;
  int t = 0;
  for (; t + kMergeUnroll <= cnt; t += kMergeUnroll) {
    float4 o[kMergeUnroll];
    float l[kMergeUnroll];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      o[u] = o_in[(int64_t)(t + u) * (kHeadDim / 4)];
      l[u] = lse_in[t + u];
    }
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const float w = expf(l[u] - m);        // 0 for an empty slot
      if (w != 0.f) {                          // uniform across the wave
        acc.x = fmaf(w, o[u].x, acc.x);
        acc.y = fmaf(w, o[u].y, acc.y);
        acc.z = fmaf(w, o[u].z, acc.z);
        acc.w = fmaf(w, o[u].w, acc.w);
        wsum += w;
      }
    }
  }
  for (; t < cnt; ++t) {
    const float4 o = o_in[(int64_t)t * (kHeadDim / 4)];
    const float w = expf(lse_in[t] - m);
    if (w != 0.f) {
      acc.x = fmaf(w, o.x, acc.x);
      acc.y = fmaf(w, o.y, acc.y);
      acc.z = fmaf(w, o.z, acc.z);
      acc.w = fmaf(w, o.w, acc.w);
      wsum += w;
    }
  }
  *o_out = make_float4(acc.x / wsum, acc.y / wsum, acc.z / wsum, acc.w / wsum);
  if (lane == 0) a.out_lse[orow] = m + logf(wsum);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int rows, hipStream_t stream) {
  if (rows <= 0 || a.n_out <= 0) return hipSuccess;
  dim3 grid(rows, a.n_out);
  hipLaunchKernelGGL(merge_kernel, grid, dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
