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

// One work-group of 256 threads per (KV head, row): threads 0..31 copy the
// token's 32 K pieces (16 bytes each, a piece holds 8 channels of one
// token), every thread its channel's V element (2 bytes inside the channel's
// 8-token piece).  The stores then reach system scope before the kernel
// ends, so a copy ordered after this launch reads them from host memory.
__global__ __launch_bounds__(256) void writeback_kernel(WritebackArgs a) {
  const int g = blockIdx.x;
  const TailRow r = a.rows[blockIdx.y];
  const int tid = threadIdx.x;
  if (r.src_page < 0 || r.src_page >= a.src_num_pages || r.dst_page < 0 ||
      r.dst_page >= a.dst_num_pages || r.token < 0 || r.token >= kPageTokens)
    return;                                                // not a row of either arena
  const int j = r.token;
  const int64_t kofs = (int64_t)g * kPageTokens * kHeadDim;
  const int64_t vofs = (int64_t)(a.num_kv_heads + g) * kPageTokens * kHeadDim;
  const uint16_t* sp = a.src + a.src_layer_off + (int64_t)r.src_page * a.page_elems;
  uint16_t* dp = a.dst + a.dst_layer_off + (int64_t)r.dst_page * a.page_elems;
  if (tid < kHeadDim / 8) {
    const int i = k_piece(j, tid);
    reinterpret_cast<uint4*>(dp + kofs)[i] = reinterpret_cast<const uint4*>(sp + kofs)[i];
  }
  const int e = v_piece(tid, j >> 3) * 8 + (j & 7);
  dp[vofs + e] = sp[vofs + e];
  __threadfence_system();
}

}  // namespace

hipError_t launch_writeback(const WritebackArgs& a, hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(writeback_kernel, dim3(a.num_kv_heads, a.n), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, int batch, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3(a.num_kv_heads, batch), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
