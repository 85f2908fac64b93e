// Split-KV paged decode attention over compact (E4M3) pages on the matrix
// cores (gfx950, v_mfma_f32_16x16x32_bf16): the older run of a history kept
// in the compact representation (KV-cache engineering, section "Exact recent
// pages, compact older pages").  Same work split, softmax and partial
// outputs as the exact kernel; half the bytes per token.
//
// One work-group (4 waves) owns one split of one KV head of one request;
// each wave takes every 4th page.  Per 64-token page, in one wave:
//   loads  16 K pieces and 16 V pieces of 1 KiB (32 KiB in flight, as the
//          exact kernel keeps per 32-token chunk);
//   QK     32 MFMAs (2 halves x 2 tiles x 8 k-steps); every E4M3 code is
//          widened to bf16 exactly (an E4M3 value has at most 4 significant
//          bits), two per instruction, right before its MFMA; the page's K
//          scale multiplies the scores;
//   softmax base-2 running max and sum over the page's 64 scores;
//   PV     64 MFMAs (2 halves x 16 channel blocks x hi/lo): P times the
//          page's V scale, split p = hi + lo in bf16, so the product keeps
//          ~2^-17 relative accuracy.
// The next page's K loads are issued after QK, its V loads after PV.
// Padding (tokens at or past the length, pages whose id is out of range)
// scores -inf and its V codes are zeroed before widening.
#pragma once

#include "compact.h"
#include "kernels.h"

namespace pkv {
namespace compact {


constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQPad = kHeadDim + 8;        // LDS row pitch of Q (bf16)

__device__ __forceinline__ f32x4_t mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Eight E4M3 codes (bytes 0..7 of w0, w1) widened to eight bf16, exactly
// (scale 1: v_cvt_scalef32_pk_bf16_fp8 converts two codes per instruction).
__device__ __forceinline__ bf16x8_t widen8(uint32_t w0, uint32_t w1) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  bf16x8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// Keep the first `live` (0..8) bytes of a two-word group, zero the rest.
__device__ __forceinline__ uint2 keep_bytes(uint32_t w0, uint32_t w1, int live) {
  const uint32_t m0 = live >= 4 ? 0xffffffffu : (live <= 0 ? 0u : (0xffffffffu >> (32 - 8 * live)));
  const int l1 = live - 4;
  const uint32_t m1 = l1 >= 4 ? 0xffffffffu : (l1 <= 0 ? 0u : (0xffffffffu >> (32 - 8 * l1)));
  return make_uint2(w0 & m0, w1 & m1);
}

struct PageRef {
  const uint8_t* k;      // compact K block
  const uint8_t* v;      // compact V block
  float sk, sv;          // the blocks' scales
  int valid;             // tokens of the page that exist (0..64)
};

__device__ __forceinline__ void load_blk(uint4 (&r)[16], const uint8_t* blk, int lane) {
  const uint4* p = reinterpret_cast<const uint4*>(blk) + lane;
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = load_stream(p + i * 64);
}

// One page: QK, online softmax, PV.  With kNext the next page's K loads
// follow QK and its V loads follow PV.
template <bool kNext>
__device__ __forceinline__ void page_step(uint4 (&kr)[16], uint4 (&vr)[16], f32x4_t (&acc)[16],
                                          float& m, float& lsum, const uint16_t* qrow,
                                          const PageRef& cur, float scale_log2, int q, int lane,
                                          const PageRef& nxt) {
  f32x4_t s[4];                                    // [h*2 + t]
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  asm volatile("" ::: "memory");
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    const bf16x8_t qb = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qrow + 32 * kb));
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      const uint4 u = kr[ht * 4 + (kb >> 1)];
      const bf16x8_t kop = (kb & 1) ? widen8(u.z, u.w) : widen8(u.x, u.y);
      s[ht] = mfma(kop, qb, s[ht]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kNext) load_blk(kr, nxt.k, lane);
  __builtin_amdgcn_sched_barrier(0);

  // lane holds tokens 32h + 8q + e (e = 0..7) of head n: e < 4 from tile 0,
  // e >= 4 from tile 1
  const float f = cur.sk * scale_log2;
  float sc[16];
  float cmax = -INFINITY;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float raw = (e < 4) ? s[h * 2][e] : s[h * 2 + 1][e - 4];
      const float x = (32 * h + 8 * q + e < cur.valid) ? raw * f : -INFINITY;
      sc[h * 8 + e] = x;
      cmax = fmaxf(cmax, x);
    }
  cmax = max_x32(max_x16(cmax));
  const float mn = fmaxf(m, cmax);
  const float mref = (mn == -INFINITY) ? 0.f : mn;
  const float alpha = fast_exp2(m - mref);
  m = mn;
  float p[16];
  float ps = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    p[e] = fast_exp2(sc[e] - mref);
    ps += p[e];
  }
  lsum = lsum * alpha + ps;
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      acc[db][0] *= alpha;
      acc[db][1] *= alpha;
      acc[db][2] *= alpha;
      acc[db][3] *= alpha;
    }
  }
  bf16x8_t phi[2], plo[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pv = p[h * 8 + e] * cur.sv;
      const __bf16 hb = (__bf16)pv;
      phi[h][e] = hb;
      plo[h][e] = (__bf16)(pv - (float)hb);
    }
  if (cur.valid < 64) {
    const int l0 = cur.valid - 8 * q, l1 = cur.valid - 32 - 8 * q;
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      const uint2 a0 = keep_bytes(vr[db].x, vr[db].y, l0);
      const uint2 a1 = keep_bytes(vr[db].z, vr[db].w, l1);
      vr[db] = make_uint4(a0.x, a0.y, a1.x, a1.y);
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      const bf16x8_t vop = h ? widen8(vr[db].z, vr[db].w) : widen8(vr[db].x, vr[db].y);
      acc[db] = mfma(vop, phi[h], acc[db]);
      acc[db] = mfma(vop, plo[h], acc[db]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kNext) load_blk(vr, nxt.v, lane);
  __builtin_amdgcn_sched_barrier(0);
}

// One work-group's split: item names the request, KV head and split;
// n_split is the number of splits in a row of the launch.
template <int G>
__device__ __forceinline__ void decode_split(const CompactDecodeArgs& a, const WorkItem& item,
                                             int n_split) {
  constexpr int D = kHeadDim;
  constexpr int PT = kPageTokens;

  const int split = item.split;
  const int g = item.g;
  const int b = item.b;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 15;
  const int q = lane >> 4;

  const int win_end = a.token_begin + a.token_count;
  const int ctx = max(0, min(item.ctx, win_end));
  const int t0 = a.token_begin + split * a.split_tokens;
  const int t1 = min(t0 + a.split_tokens, ctx);
  const int slot = a.out_slot0 + split;
  const int64_t row0 = (int64_t)b * a.num_q_heads + (int64_t)g * G;

  __shared__ __attribute__((aligned(16))) uint16_t q_lds[16 * kQPad];
  __shared__ float acc_lds[kWaves][G][D];
  __shared__ float m_lds[kWaves][16];
  __shared__ float l_lds[kWaves][16];

  if (t1 <= t0) {                      // no key of the request in this split
#pragma unroll
    for (int h = 0; h < G; ++h) {
      a.out_o[((row0 + h) * a.out_slots + slot) * D + tid] = 0.f;
      if (tid == 0) a.out_lse[(row0 + h) * a.out_slots + slot] = -INFINITY;
    }
    return;
  }

  const uint8_t* layer_base = a.codes + a.layer_off;
  const float* layer_scales = a.scales + a.scale_layer_off;
  const int32_t* trow = a.table + (int64_t)b * a.pt_stride;
  const int first_page = (t0 - a.token_begin) / PT;
  const int n_pages = (t1 - t0 + PT - 1) / PT;
  const int my_pages = (n_pages > w) ? (n_pages - w + kWaves - 1) / kWaves : 0;

  // Prologue: page ids, the query group, the pages' scales and the first
  // page's loads are issued before anything waits.  Lane j holds the id and
  // the two scales of the wave's page j (at most 64 pages per wave:
  // split_tokens <= 16384).
  int my_id = (lane < my_pages) ? trow[first_page + w + kWaves * lane] : -1;
  uint4 qv[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = tid + r * kThreads;
    const int h = i / (D / 8);
    qv[r] = (h < G) ? reinterpret_cast<const uint4*>(a.q + (row0 + h) * D)[i % (D / 8)]
                    : make_uint4(0, 0, 0, 0);
  }
  const bool id_ok = my_id >= 0 && my_id < a.num_pages;
  float my_sk = 0.f, my_sv = 0.f;
  if (id_ok) {
    const float* ps = layer_scales + (int64_t)my_id * 2 * a.num_kv_heads;
    my_sk = ps[g];
    my_sv = ps[a.num_kv_heads + g];
  } else {
    my_id = -1;
  }
  auto page_at = [&](int j) {
    PageRef pg;
    int phys = __builtin_amdgcn_readlane(my_id, j);
    pg.sk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_sk), j));
    pg.sv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_sv), j));
    pg.valid = min(PT, t1 - (t0 + (w + kWaves * j) * PT));
    if (phys < 0) { phys = 0; pg.valid = 0; }            // read page 0, mask all
    const uint8_t* page = layer_base + (int64_t)phys * a.page_bytes;
    pg.k = page + (int64_t)g * kCompactBlockBytes;
    pg.v = page + (int64_t)(a.num_kv_heads + g) * kCompactBlockBytes;
    return pg;
  };
  uint4 kr[16], vr[16];
  PageRef cur = page_at(0);
  if (my_pages > 0) {
    load_blk(kr, cur.k, lane);
    load_blk(vr, cur.v, lane);
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = tid + r * kThreads;
    *reinterpret_cast<uint4*>(&q_lds[(i / (D / 8)) * kQPad + 8 * (i % (D / 8))]) = qv[r];
  }
  __syncthreads();
  const uint16_t* qrow = &q_lds[n * kQPad + 8 * q];

  float m = -INFINITY;
  float lsum = 0.f;
  f32x4_t acc[16];
#pragma unroll
  for (int db = 0; db < 16; ++db) acc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (my_pages > 0) {
    for (int j = 0; j + 1 < my_pages; ++j) {
      const PageRef nxt = page_at(j + 1);
      page_step<true>(kr, vr, acc, m, lsum, qrow, cur, a.scale_log2, q, lane, nxt);
      cur = nxt;
    }
    page_step<false>(kr, vr, acc, m, lsum, qrow, cur, a.scale_log2, q, lane, cur);
  }

  lsum = sum_x32(sum_x16(lsum));
  if (q == 0) {
    m_lds[w][n] = m;
    l_lds[w][n] = lsum;
  }
  if (n < G) {
#pragma unroll
    for (int db = 0; db < 16; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc_lds[w][n][16 * db + 4 * q + i] = acc[db][i];
  }
  __syncthreads();

#pragma unroll 1
  for (int h = 0; h < G; ++h) {
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, m_lds[v][h]);
    float o = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const float f = fast_exp2(m_lds[v][h] - M);
        if (f != 0.f) {
          L = fmaf(f, l_lds[v][h], L);
          o = fmaf(f, acc_lds[v][h][tid], o);
        }
      }
    }
    const bool live = L > 0.f;
    a.out_o[((row0 + h) * a.out_slots + slot) * D + tid] = live ? o / L : 0.f;
    if (tid == 0)
      a.out_lse[(row0 + h) * a.out_slots + slot] = live ? (M + log2f(L)) * kLn2 : -INFINITY;
  }
}

}  // namespace compact
}  // namespace pkv
