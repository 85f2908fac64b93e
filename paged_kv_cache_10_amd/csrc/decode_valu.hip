// Split-KV paged decode attention on the vector ALUs (gfx950).
//
// One work-group (4 waves) owns one split of `split_tokens` tokens of one
// request for one KV head and the query group that reads it.  It walks the
// split page by page; for every page:
//   QK  wave w scores tokens 16w..16w+15.  Eight lanes share a token, each
//       taking 32 of the 256 channels so that every load instruction reads
//       whole 128-byte lines; products are bf16 x bf16 -> FP32 (v_dot2), and
//       the eight partial dots meet in a 3-step butterfly.
//   softmax  every wave reads the page's 64 x G scores from LDS and updates
//       the running max m and sum l in FP32 (base 2) with wave reductions;
//       all waves hold identical copies.
//   PV  wave w owns channels 64w..64w+63 of the output.  A V block is
//       dim-major, so eight lanes read one channel's 64 tokens (one 128-byte
//       line) and each lane accumulates its 8 tokens for all G heads.
// At the end of the split the eight token-lanes of a channel are summed, the
// output is divided by l and lse = (m + log2 l) ln 2 is stored: the split's
// normalised output and log-sum-exp (KV-cache engineering page, section
// "Exact recent pages, compact older pages").
//
// Tokens at or past the request's length score -inf and their V values are
// replaced by zero before use, so padding never enters the arithmetic even
// when it holds NaN.
#include "device.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int G>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(DecodeArgs a) {
  constexpr int D = kHeadDim;
  constexpr int PT = kPageTokens;

  const WorkItem item = dense_item_grid(a.ctx_lens, nullptr, a.token_begin, a.token_count,
                                        a.split_tokens);
  const int split = item.split;
  const int g = item.g;
  const int b = item.b;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 7;      // channel chunk (QK) / token chunk (PV)
  const int tg = lane >> 3;    // token within an 8-token step (QK) / channel row (PV)

  const int win_end = a.token_begin + a.token_count;
  const int ctx = max(0, min(item.ctx, win_end));
  const int t0 = a.token_begin + split * a.split_tokens;
  const int t1 = min(t0 + a.split_tokens, ctx);
  const int slot = a.out_slot0 + split;
  const int64_t row0 = (int64_t)b * a.num_q_heads + (int64_t)g * G;

  // a split with no key of the request: an empty partial, nothing read
  if (t1 <= t0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      a.out_o[((row0 + h) * a.out_slots + slot) * D + tid] = 0.f;
      if (tid == 0) a.out_lse[(row0 + h) * a.out_slots + slot] = -INFINITY;
    }
    return;
  }

  __shared__ float s_lds[G][PT];
  __shared__ float p_lds[kWaves][G][PT];

  // q slices: head h, channels 64i + 8c .. +8 for i = 0..3
  uint4 qv[G][4];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + row0 * D);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) qv[h][i] = qp[h * (D / 8) + 8 * i + c];
  }

  float m[G], l[G], acc[8][G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r][h] = 0.f;
  }

  const uint16_t* layer_base = a.arena + a.layer_off;
  const int32_t* trow = a.table + (int64_t)b * a.pt_stride;

  for (int tok = t0; tok < t1; tok += PT) {
    const int phys = trow[(tok - a.token_begin) / PT];
    if (phys < 0 || phys >= a.num_pages) continue;          // never dereferenced
    const int valid = min(PT, t1 - tok);
    const uint16_t* page = layer_base + (int64_t)phys * a.page_elems;
    const uint16_t* kb = page + (int64_t)g * PT * D;
    const uint16_t* vb = page + (int64_t)(a.num_kv_heads + g) * PT * D;

    // ---- QK: scores of tokens 16w .. 16w+15
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int j = 16 * w + 8 * st + tg;
      const uint4* kr = reinterpret_cast<const uint4*>(kb);
      uint4 kv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kv[i] = kr[k_piece(j, 8 * i + c)];
      float s[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float x = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x = dot2_bf16(kv[i].x, qv[h][i].x, x);
          x = dot2_bf16(kv[i].y, qv[h][i].y, x);
          x = dot2_bf16(kv[i].z, qv[h][i].z, x);
          x = dot2_bf16(kv[i].w, qv[h][i].w, x);
        }
        s[h] = x;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        s[h] = sum8(s[h]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
        if (c == h) s_lds[h][j] = (j < valid) ? s[h] * a.scale_log2 : -INFINITY;
    }
    __syncthreads();

    // ---- online softmax over the page (identical in every wave)
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float x = s_lds[h][lane];
      const float mn = fmaxf(m[h], wave_max(x));
      alpha[h] = fast_exp2(m[h] - mn);                       // 0 while m = -inf
      const float p = fast_exp2(x - mn);                     // 0 for masked tokens
      l[h] = l[h] * alpha[h] + wave_sum(p);
      m[h] = mn;
      p_lds[w][h][lane] = p;
    }
    __syncthreads();

    // ---- PV: channels 64w + 8r + tg, tokens 8c .. 8c+7
    float pv[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float4 p0 = *reinterpret_cast<const float4*>(&p_lds[w][h][8 * c]);
      const float4 p1 = *reinterpret_cast<const float4*>(&p_lds[w][h][8 * c + 4]);
      pv[h][0] = p0.x; pv[h][1] = p0.y; pv[h][2] = p0.z; pv[h][3] = p0.w;
      pv[h][4] = p1.x; pv[h][5] = p1.y; pv[h][6] = p1.z; pv[h][7] = p1.w;
    }
    const bool ragged = valid < PT;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int d = 64 * w + 8 * r + tg;
      const uint4 vv = reinterpret_cast<const uint4*>(vb)[v_piece(d, c)];
      float vf[8] = {bf16_lo(vv.x), bf16_hi(vv.x), bf16_lo(vv.y), bf16_hi(vv.y),
                     bf16_lo(vv.z), bf16_hi(vv.z), bf16_lo(vv.w), bf16_hi(vv.w)};
      if (ragged) {
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[e] = (8 * c + e < valid) ? vf[e] : 0.f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float x = acc[r][h] * alpha[h];
#pragma unroll
        for (int e = 0; e < 8; ++e) x = fmaf(pv[h][e], vf[e], x);
        acc[r][h] = x;
      }
    }
  }

  // ---- sum the eight token-lanes of each channel, normalise, store
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      acc[r][h] = sum8(acc[r][h]);
    }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (c == h) {
      const float inv = (l[h] > 0.f) ? 1.f / l[h] : 0.f;
      float* o = a.out_o + ((row0 + h) * a.out_slots + slot) * D + 64 * w + tg;
#pragma unroll
      for (int r = 0; r < 8; ++r) o[8 * r] = acc[r][h] * inv;
    }
    if (tid == h)
      a.out_lse[(row0 + h) * a.out_slots + slot] =
          (l[h] > 0.f) ? (m[h] + log2f(l[h])) * kLn2 : -INFINITY;
  }
}

template <int G>
hipError_t launch_g(const DecodeArgs& a, int batch, hipStream_t stream) {
  const int n_split = a.token_count / a.split_tokens;
  dim3 grid(n_split, a.num_kv_heads, batch);
  hipLaunchKernelGGL(decode_valu_kernel<G>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_valu(const DecodeArgs& a, int batch, int group, hipStream_t stream) {
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
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
