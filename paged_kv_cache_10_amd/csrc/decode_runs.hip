// Runs of two representations in one launch: the work-groups of an older run
// read from compact pages and of a recent run from exact pages (or any two
// runs), each with its own table, lengths, tiling and output slots, share one
// grid, so the two runs fill the GPU together instead of one after the other
// (no second ramp and drain, no run waiting for the other's last
// work-group).  Every work-group runs exactly the split its own kernel would
// run (compact::decode_split, exact::decode_split), so the partials are the
// bits those kernels write.
#include "decode_compact.h"
#include "decode_exact.h"

namespace pkv {

namespace {

template <int G>
__global__ __launch_bounds__(exact::kThreads) void decode_runs_kernel(RunsArgs r) {
  unsigned lin = blockIdx.x;
  int k = 0;
  if (lin >= (unsigned)r.wgs[0]) {
    lin -= r.wgs[0];
    k = 1;
  }
  const unsigned hkv = r.num_kv_heads;
  if (r.compact[k]) {
    const CompactDecodeArgs& a = r.c[k];
    const WorkItem item = dense_item(a.ctx_lens, nullptr, a.token_begin, a.token_count,
                                     a.split_tokens, r.n_split[k], hkv, r.batch, lin);
    compact::decode_split<G>(a, item, r.n_split[k]);
  } else {
    const DecodeArgs& a = r.e[k];
    const WorkItem item = dense_item(a.ctx_lens, nullptr, a.token_begin, a.token_count,
                                     a.split_tokens, r.n_split[k], hkv, r.batch, lin);
    exact::decode_split<G>(a, item, r.n_split[k]);
  }
}

template <int G>
hipError_t launch_g(const RunsArgs& a, hipStream_t stream) {
  const int total = a.wgs[0] + (a.n_runs > 1 ? a.wgs[1] : 0);
  hipLaunchKernelGGL((decode_runs_kernel<G>), dim3(total), dim3(exact::kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_runs(const RunsArgs& a, int group, hipStream_t stream) {
  if (a.batch <= 0 || a.wgs[0] + (a.n_runs > 1 ? a.wgs[1] : 0) <= 0) return hipSuccess;
  switch (group) {
    case 1: return launch_g<1>(a, stream);
    case 2: return launch_g<2>(a, stream);
    case 3: return launch_g<3>(a, stream);
    case 4: return launch_g<4>(a, stream);
    case 5: return launch_g<5>(a, stream);
    case 6: return launch_g<6>(a, stream);
    case 7: return launch_g<7>(a, stream);
    case 8: return launch_g<8>(a, stream);
    case 12: return launch_g<12>(a, stream);
    case 16: return launch_g<16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
