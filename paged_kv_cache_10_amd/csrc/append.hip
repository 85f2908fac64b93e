// KV append: write one new token's K and V rows per request into its page
// of one layer, in the pool's operand-ordered block layout, so that the next
// decode step attends over it (the newest token of the history; GPU memory
// management page, "Pages held by right, borrowed or free": the newest pages
// and the sink stay on the device).
//
// One work-group of 256 threads per (request, KV head): threads 0..31 store
// the K row as 32 pieces of 8 channels (16 bytes each); every thread stores
// its channel of the V row as one bf16 inside that channel's 8-token piece.
#include "device.h"
#include "kernels.h"

namespace pkv {

namespace {

__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int g = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int pos = a.positions[b];
  if (pos < 0) return;                                     // no token for this request
  const int lp = pos / kPageTokens;
  if (lp >= a.pt_stride) return;                           // outside the row: never written
  const int phys = a.table[(int64_t)b * a.pt_stride + lp];
  if (phys < 0 || phys >= a.num_pages) return;             // not a page of the pool
  const int j = pos % kPageTokens;
  uint16_t* page = a.arena + a.layer_off + (int64_t)phys * a.page_elems;
  uint16_t* kb = page + (int64_t)g * kPageTokens * kHeadDim;
  uint16_t* vb = page + (int64_t)(a.num_kv_heads + g) * kPageTokens * kHeadDim;
  const uint16_t* krow = a.k + ((int64_t)b * a.num_kv_heads + g) * kHeadDim;
  const uint16_t* vrow = a.v + ((int64_t)b * a.num_kv_heads + g) * kHeadDim;
  if (tid < kHeadDim / 8) {
    const uint4 piece = reinterpret_cast<const uint4*>(krow)[tid];
    reinterpret_cast<uint4*>(kb)[k_piece(j, tid)] = piece;
  }
  vb[v_piece(tid, j >> 3) * 8 + (j & 7)] = vrow[tid];
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int batch, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3(a.num_kv_heads, batch), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
