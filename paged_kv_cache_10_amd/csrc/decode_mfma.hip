// Kernel entry of the exact decode: one work-group per (split, KV head,
// request) in the launch's work order; the split itself is exact::decode_split
// (decode_exact.h).
#include "decode_exact.h"

namespace pkv {

namespace {

template <int G>
__global__ __launch_bounds__(exact::kThreads)
void decode_mfma_kernel(DecodeArgs a) {
  const WorkItem item = dense_item_grid(a.ctx_lens, a.row_split, a.token_begin, a.token_count,
                                        a.split_tokens);
  exact::decode_split<G>(a, item, (int)gridDim.x);
}


template <int G>
hipError_t launch_g(const DecodeArgs& a, int batch, hipStream_t stream) {
  const int n_split = a.token_count / a.split_tokens;
  dim3 grid(n_split, a.num_kv_heads, batch);
  hipLaunchKernelGGL((decode_mfma_kernel<G>), grid, dim3(exact::kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, int batch, int group, hipStream_t stream) {
  if (batch <= 0 || a.token_count <= 0) return hipSuccess;
  switch (group) {
    case 1: return launch_g<1>(a, batch, stream);
    case 2: return launch_g<2>(a, batch, stream);
    case 3: return launch_g<3>(a, batch, stream);
    case 4: return launch_g<4>(a, batch, stream);
    case 5: return launch_g<5>(a, batch, stream);
    case 6: return launch_g<6>(a, batch, stream);
    case 7: return launch_g<7>(a, batch, stream);
    case 8: return launch_g<8>(a, batch, stream);
    case 12: return launch_g<12>(a, batch, stream);
    case 16: return launch_g<16>(a, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
