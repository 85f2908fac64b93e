// FP32 log-sum-exp merge of attention partials (KV-cache engineering page,
// section "Exact recent pages, compact older pages"): partial t is weighted
// by exp(lse_t - max lse); the sum of weighted outputs over the total
// weight is the merged output, max + log(total) the merged log-sum-exp.
//
// The merge arithmetic (merge_slots) serves three places:
//   * the final merge of every slot of a row into one output
//     (pkv_merge_partials: merge_final_kernel for rows of at most 64 slots,
//     merge_kernel beyond);
//   * the tile finalize inside pkv_decode_attention, which merges the fixed
//     groups of split partials that make up one tile (merge_kernel);
//   * both at once for pkv_decode_attention_merged (merge2_kernel).
// In merge_kernel two waves own one (row, output slot), 128 channels each
// (two per lane, every load 512 contiguous bytes); merge_final_kernel and
// merge2_kernel give each lane one channel, so four work-groups share a row
// and its loads reach more compute units.  Every channel walks its input
// slots in increasing order with one accumulator, so the result is
// independent of scheduling and of how channels are spread over lanes, an
// empty slot (lse = -inf) contributes exactly nothing and a lone slot merges
// to itself bit for bit.
#include "device.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kMergeThreads = 64;     // one wave (merge_kernel: lane i owns channels 128 * half + 2i, +1)
constexpr int kMergeParts = kHeadDim / 128;   // merge_kernel: waves per (row, output slot)
constexpr int kMergeChunk = 64;       // input slots whose loads are in flight together

struct Merged {
  float2 o;    // this lane's two channels
  float lse;
};

// The first min(64, cnt) slots' outputs (o_in[t * 128], two channels per
// lane) into o; they do not depend on the max, so they go out first.
__device__ __forceinline__ void load_chunk(float2 (&o)[kMergeChunk], const float2* o_in, int n) {
#pragma unroll
  for (int u = 0; u < kMergeChunk; ++u)
    o[u] = (u < n) ? load_stream(o_in + (int64_t)u * (kHeadDim / 2)) : make_float2(0.f, 0.f);
}

// The merge of cnt slots: lv = this lane's slot's log-sum-exp (lane < cnt,
// else -inf), further log-sum-exps in lse_in[64 ..), outputs at o_in with
// the first 64 already in o.  M = max_t lse_t (NaN if any slot's is: the
// row's result then comes out NaN instead of dropping that slot); chunks of
// 64 slots: lane u computes the weight of the chunk's slot u (one exp per
// lane, all in parallel), then the slots are summed in increasing order with
// each weight read from its lane.  Every merge in this file goes through
// here or repeats its arithmetic step for step (merge_window,
// merge_final_kernel), so a merge gives the same bits wherever it runs.
__device__ __forceinline__ Merged merge_slots(float lv, const float* lse_in, const float2* o_in,
                                              int cnt, int lane, float2 (&o)[kMergeChunk]) {
  float m = lv;
  for (int t = lane + kMergeThreads; t < cnt; t += kMergeThreads) m = max_nan(m, lse_in[t]);
  m = wave_max_nan(m);
  if (m == -INFINITY) return Merged{make_float2(0.f, 0.f), -INFINITY};   // every slot empty
  float2 acc = make_float2(0.f, 0.f);
  float wsum = 0.f;
  for (int c0 = 0; c0 < cnt; c0 += kMergeChunk) {
    const int nc = min(kMergeChunk, cnt - c0);
    if (c0 > 0) load_chunk(o, o_in + (int64_t)c0 * (kHeadDim / 2), nc);
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
  return Merged{make_float2(acc.x / wsum, acc.y / wsum), m + logf(wsum)};
}

// Group j of row `row`: slots j*group .. of the input, into output slot j.
__device__ __forceinline__ Merged merge_group(const MergeArgs& a, int row, int j, int part,
                                              int lane) {
  const int t0 = j * a.group;
  const int cnt = min(a.group, a.in_slots - t0);
  const float* lse_in = a.in_lse + (int64_t)row * a.in_slots + t0;
  const float2* o_in = reinterpret_cast<const float2*>(
      a.in_o + ((int64_t)row * a.in_slots + t0) * kHeadDim + 128 * part) + lane;
  float2 o[kMergeChunk];
  load_chunk(o, o_in, min(kMergeChunk, cnt));
  const float lv = (lane < cnt) ? lse_in[lane] : -INFINITY;
  return merge_slots(lv, lse_in, o_in, cnt, lane, o);
}

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
  const int row = blockIdx.x, j = blockIdx.y, part = blockIdx.z, lane = threadIdx.x;
  const Merged r = merge_group(a, row, j, part, lane);
  const int64_t orow = (int64_t)row * a.out_slots + a.out_slot0 + j;
  reinterpret_cast<float2*>(a.out_o + orow * kHeadDim + 128 * part)[lane] = r.o;
  if (part == 0 && lane == 0) a.out_lse[orow] = r.lse;
}

// The final merge of rows of at most 64 slots (every slot into one output):
// one channel per lane, so four single-wave work-groups share a row and its
// loads are spread over four compute units (measured: ~0.7 µs less per
// 262K layer than two waves of two channels per lane).  Per channel the
// arithmetic is merge_slots' (the same max, the same exp per slot in the
// slot's lane, the slots summed in increasing order), so the bits are the
// ones merge_kernel gives.
__global__ __launch_bounds__(kMergeThreads) void merge_final_kernel(MergeArgs a) {
  constexpr int kChannels = kMergeThreads;          // per work-group
  const int row = blockIdx.x, part = blockIdx.z, lane = threadIdx.x;
  const int n = a.in_slots;
  const float* lse_in = a.in_lse + (int64_t)row * n;
  const float* o_in = a.in_o + (int64_t)row * n * kHeadDim + kChannels * part + lane;
  float o[kMergeChunk];
#pragma unroll
  for (int u = 0; u < kMergeChunk; ++u)
    o[u] = (u < n) ? __builtin_nontemporal_load(o_in + (int64_t)u * kHeadDim) : 0.f;
  const float lv = (lane < n) ? lse_in[lane] : -INFINITY;
  const int64_t orow = (int64_t)row * a.out_slots + a.out_slot0;
  float* out = a.out_o + orow * kHeadDim + kChannels * part + lane;
  const float m = wave_max_nan(lv);
  if (m == -INFINITY) {                        // every slot empty
    *out = 0.f;
    if (part == 0 && lane == 0) a.out_lse[orow] = -INFINITY;
    return;
  }
  const float wl = (lane < n) ? expf(lv - m) : 0.f;   // 0 for an empty slot
  float acc = 0.f, wsum = 0.f;
#pragma unroll
  for (int u = 0; u < kMergeChunk; ++u) {
    const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u));
    if (w != 0.f) {                            // uniform across the wave
      acc = fmaf(w, o[u], acc);
      wsum += w;
    }
  }
  *out = acc / wsum;
  if (part == 0 && lane == 0) a.out_lse[orow] = m + logf(wsum);
}

struct Merged1 {
  float o;     // this lane's channel
  float lse;
};

// The merge of the cnt slots lo .. lo+cnt-1 of a window of at most 64 slots
// whose log-sum-exps sit in the lanes (lv at lane u = slot u) and whose
// outputs are in LDS (win[u][lane], one channel per lane): merge_slots'
// arithmetic (the same max, the same exp per slot, the slots summed in
// increasing order), so a group merged here has the bits merge_slots gives
// it.  The outputs are read eight slots at a time, so the LDS reads of a
// batch are in flight together.
__device__ __forceinline__ Merged1 merge_window(float lv, int lo, int cnt, int lane,
                                                const float (*win)[kMergeThreads]) {
  constexpr int kBatch = 8;
  const int hi = lo + cnt;
  const bool mine = lane >= lo && lane < hi;
  const float m = wave_max_nan(mine ? lv : -INFINITY);
  if (m == -INFINITY) return Merged1{0.f, -INFINITY};   // every slot empty
  const float wl = mine ? expf(lv - m) : 0.f;
  float acc = 0.f, wsum = 0.f;
  for (int u0 = lo; u0 < hi; u0 += kBatch) {
    float ou[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) ou[i] = (u0 + i < hi) ? win[u0 + i][lane] : 0.f;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (u0 + i < hi) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u0 + i));
        if (w != 0.f) {                        // uniform: 0 for an empty slot
          acc = fmaf(w, ou[i], acc);
          wsum += w;
        }
      }
    }
  }
  return Merged1{acc / wsum, m + logf(wsum)};
}

// Tile finalize and final merge in one launch, for rows of at most 64 split
// partials.  Four waves share one (row, 64-channel quarter): together they
// load the row's split partials into LDS (slot u by wave u % 4, so every
// load is in flight at once), wave w then merges groups j = w, w + 4, ...
// into output slot j (as merge_kernel would), and wave 0 merges the group
// results, kept in LDS, into fin_o / fin_lse (as the final merge over those
// slots would), so the bits equal the two launches'.
constexpr int kMerge2Waves = 4;
constexpr int kMerge2Parts = kHeadDim / kMergeThreads;   // one channel per lane

__global__ __launch_bounds__(kMergeThreads * kMerge2Waves) void merge2_kernel(MergeArgs a,
                                                                               float* fin_o,
                                                                               float* fin_lse) {
  constexpr int kPerWave = kMergeChunk / kMerge2Waves;
  const int row = blockIdx.x, part = blockIdx.z;
  const int w = threadIdx.x / kMergeThreads, lane = threadIdx.x % kMergeThreads;
  const int c = kMergeThreads * part + lane;      // this lane's channel
  __shared__ float split_o[kMergeChunk][kMergeThreads];
  __shared__ float tile_o[kMergeChunk][kMergeThreads];
  __shared__ float tile_lse[kMergeChunk];
  const float* lse_in = a.in_lse + (int64_t)row * a.in_slots;
  const float* o_in = a.in_o + (int64_t)row * a.in_slots * kHeadDim + c;
  {
    float o[kPerWave];
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int u = kMerge2Waves * i + w;
      o[i] = (u < a.in_slots) ? __builtin_nontemporal_load(o_in + (int64_t)u * kHeadDim) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int u = kMerge2Waves * i + w;
      if (u < a.in_slots) split_o[u][lane] = o[i];
    }
  }
  const float lv = (lane < a.in_slots) ? lse_in[lane] : -INFINITY;
  __syncthreads();
  for (int j = w; j < a.n_out; j += kMerge2Waves) {
    const int lo = j * a.group;
    const Merged1 r = merge_window(lv, lo, min(a.group, a.in_slots - lo), lane, split_o);
    const int64_t orow = (int64_t)row * a.out_slots + a.out_slot0 + j;
    a.out_o[orow * kHeadDim + c] = r.o;
    if (part == 0 && lane == 0) a.out_lse[orow] = r.lse;
    tile_o[j][lane] = r.o;
    if (lane == 0) tile_lse[j] = r.lse;
  }
  __syncthreads();
  if (w != 0) return;
  const float tl = (lane < a.n_out) ? tile_lse[lane] : -INFINITY;   // lane j: group j's
  const Merged1 r = merge_window(tl, 0, a.n_out, lane, tile_o);
  fin_o[(int64_t)row * kHeadDim + c] = r.o;
  if (part == 0 && lane == 0) fin_lse[row] = r.lse;
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int rows, hipStream_t stream) {
  if (rows <= 0 || a.n_out <= 0) return hipSuccess;
  if (a.n_out == 1 && a.group >= a.in_slots && a.in_slots <= kMergeChunk) {   // a final merge
    hipLaunchKernelGGL(merge_final_kernel, dim3(rows, 1, kHeadDim / kMergeThreads),
                       dim3(kMergeThreads), 0, stream, a);
    return hipGetLastError();
  }
  dim3 grid(rows, a.n_out, kMergeParts);
  hipLaunchKernelGGL(merge_kernel, grid, dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_merge2(const MergeArgs& a, int rows, float* fin_o, float* fin_lse,
                         hipStream_t stream) {
  if (rows <= 0 || a.n_out <= 0) return hipSuccess;
  if (a.in_slots > kMergeChunk) return hipErrorInvalidValue;   // one window per row
  dim3 grid(rows, 1, kMerge2Parts);
  hipLaunchKernelGGL(merge2_kernel, grid, dim3(kMergeThreads * kMerge2Waves), 0, stream, a,
                     fin_o, fin_lse);
  return hipGetLastError();
}

}  // namespace pkv
