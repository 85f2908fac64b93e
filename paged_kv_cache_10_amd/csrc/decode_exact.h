// Split-KV paged decode attention on the matrix cores (gfx950,
// v_mfma_f32_16x16x32_bf16).
//
// One work-group (4 waves) owns one split of `split_tokens` tokens of one
// request for one KV head; the KV head's query group (G <= 16 heads, padded
// with zero rows to 16) is staged in LDS once.  Each wave takes every 4th
// page of the split and keeps its own running max / sum; the four waves meet
// in LDS at the end, in a fixed order.
//
// Per 32-token chunk of a page, in one wave:
//   QK  S[token][head] = K[16 tokens x 256] . Q^T[256 x 16 heads], two MFMA
//       tiles of 16 tokens x 8 steps of 32 channels.  Tile rows are assigned
//       so that lane l ends up with the scores of tokens 8(l/16) .. +7 of
//       head l%16, exactly the operand layout PV needs next.
//   softmax  base-2 running max m and per-lane partial sum l in FP32; the
//       chunk max meets across the 4 lanes of a head by two row swaps
//       (v_permlane16_swap, v_permlane32_swap), with no LDS round trip.
//   PV  O^T[channel][head] += V^T[16 channels x 32 tokens] . P^T[32 x 16].
//       V blocks are stored dim-major, so the V^T operand is one contiguous
//       16-byte load per lane.  P is split as p = hi + lo with hi, lo bf16
//       (both round to nearest), two MFMAs per tile, so the product keeps
//       ~2^-17 relative accuracy instead of bf16's 2^-9.
// K/V loads of the next chunk are issued while the current chunk computes;
// the first chunk's loads are in flight while the query group is staged.
//
// Padding (tokens at or past the length, or pages whose id is out of range)
// scores -inf and its V values are zeroed before the MFMA, so NaN padding
// never reaches the sums.
#pragma once

#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace pkv {
namespace exact {


constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQPad = kHeadDim + 8;        // LDS row pitch of Q (bf16), breaks bank aliasing

typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4_t mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8_t, u);
}

// Zero bf16 element e of an 8-element operand when !keep[e].
__device__ __forceinline__ uint4 mask_pairs(uint4 u, int live) {
  // live = number of leading elements kept (0..8)
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (2 * i < live) ? 0x0000ffffu : 0u;
    const uint32_t hi = (2 * i + 1 < live) ? 0xffff0000u : 0u;
    w[i] &= (lo | hi);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Addresses of one page of one KV head for one wave.
struct PageRef {
  const uint16_t* k;     // K block (token-major [64][256])
  const uint16_t* v;     // V block (dim-major [256][64])
  int valid;             // tokens of the page that exist (0..64)
};

// K operand of a 32-token chunk (half `base`/32 of the page): 16 loads of
// 1 KiB, tile t and k-step kb at piece (t*8 + kb)*64 + lane.
__device__ __forceinline__ void load_k(uint4 (&kr)[2][8], const PageRef& pg, int base, int lane) {
  const uint4* p = reinterpret_cast<const uint4*>(pg.k) + (base >> 5) * 1024 + lane;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) kr[t][kb] = load_stream(p + (t * 8 + kb) * 64);
}

// V^T operand of a 32-token chunk: channel block db at piece db*64 + lane.
__device__ __forceinline__ void load_v(uint4 (&vr)[16], const PageRef& pg, int base, int lane) {
  const uint4* p = reinterpret_cast<const uint4*>(pg.v) + (base >> 5) * 1024 + lane;
#pragma unroll
  for (int db = 0; db < 16; ++db) vr[db] = load_stream(p + db * 64);
}

// One 32-token chunk: QK, online softmax, PV.  `live` = tokens of the chunk
// that exist.  With kNext, the next chunk's K loads are issued as soon as QK
// has consumed kr, and its V loads as soon as PV has consumed vr.
template <bool kNext>
__device__ __forceinline__ void chunk(uint4 (&kr)[2][8], uint4 (&vr)[16], f32x4_t (&acc)[16],
                                      float& m, float& lsum, const uint16_t* qrow, int live,
                                      float scale_log2, int q, int lane,
                                      const PageRef& nxt, int nbase) {
  f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
  asm volatile("" ::: "memory");     // keep the LDS operand reads inside the loop
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    const bf16x8_t qb = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 32 * kb));
    s0 = mfma(as_bf16x8(kr[0][kb]), qb, s0);
    s1 = mfma(as_bf16x8(kr[1][kb]), qb, s1);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kNext) load_k(kr, nxt, nbase, lane);
  __builtin_amdgcn_sched_barrier(0);

  // online softmax; lane holds tokens 8q + e, e = 0..7, of head n (base 2)
  float s[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  float cmax = -INFINITY;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    s[e] = (8 * q + e < live) ? s[e] * scale_log2 : -INFINITY;
    cmax = fmaxf(cmax, s[e]);
  }
  cmax = max_x32(max_x16(cmax));
  const float mn = fmaxf(m, cmax);
  const float mref = (mn == -INFINITY) ? 0.f : mn;
  const float alpha = fast_exp2(m - mref);
  m = mn;
  float p[8];
  float ps = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = fast_exp2(s[e] - mref);
    ps += p[e];
  }
  lsum = lsum * alpha + ps;
  if (__any(alpha != 1.f)) {           // multiplying by 1 is exact: skipping changes no bit
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      acc[db][0] *= alpha;
      acc[db][1] *= alpha;
      acc[db][2] *= alpha;
      acc[db][3] *= alpha;
    }
  }
  bf16x8_t phi, plo;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = (__bf16)p[e];
    phi[e] = h;
    plo[e] = (__bf16)(p[e] - (float)h);
  }
  if (live < 32) {
    const int vlive = max(0, min(8, live - 8 * q));
#pragma unroll
    for (int db = 0; db < 16; ++db) vr[db] = mask_pairs(vr[db], vlive);
  }
  // PV: all hi products, then all lo products (independent MFMAs back to back)
#pragma unroll
  for (int db = 0; db < 16; ++db) acc[db] = mfma(as_bf16x8(vr[db]), phi, acc[db]);
#pragma unroll
  for (int db = 0; db < 16; ++db) acc[db] = mfma(as_bf16x8(vr[db]), plo, acc[db]);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kNext) load_v(vr, nxt, nbase, lane);
  __builtin_amdgcn_sched_barrier(0);
}

// One work-group's split: item names the request, KV head and split;
// n_split is the number of splits in a row of the launch.
template <int G>
__device__ __forceinline__ void decode_split(const DecodeArgs& a, const WorkItem& item,
                                             int n_split) {
  constexpr int D = kHeadDim;
  constexpr int PT = kPageTokens;

  const int split = item.split;
  const int g = item.g;
  const int b = item.b;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 15;        // head column of every MFMA tile
  const int q = lane >> 4;        // k-group of operands / row group of results

  const int win_end = a.token_begin + a.token_count;
  const int ctx = max(0, min(item.ctx, win_end));
  const int S = item.S;
  const int t0 = a.token_begin + split * S;
  const int t1 = min(t0 + S, ctx);
  const int slot = a.out_slot0 + split;
  // per-request splits: keys past the grid row's last split (a split too
  // short for the row's slots) are not attended, and that row's last
  // partial says so with a NaN log-sum-exp
  const bool uncovered = a.row_split && split == n_split - 1 &&
                         item.ctx > a.token_begin + (split + 1) * S;
  const int64_t row0 = (int64_t)b * a.num_q_heads + (int64_t)g * G;

  __shared__ __attribute__((aligned(16))) uint16_t q_lds[16 * kQPad];
  __shared__ float acc_lds[kWaves][G][D];
  __shared__ float m_lds[kWaves][16];
  __shared__ float l_lds[kWaves][16];

  // ---- a malformed per-request split (outside 64 .. 16,384 tokens or not a
  // multiple of 64): nothing is read, and the partial says so with a NaN
  // log-sum-exp
  if (a.row_split && (S < PT || S > 64 * kWaves * PT || S % PT != 0)) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      a.out_o[((row0 + h) * a.out_slots + slot) * D + tid] = 0.f;
      if (tid == 0) a.out_lse[(row0 + h) * a.out_slots + slot] = NAN;
    }
    return;
  }

  // ---- a split with no key of the request: an empty partial, nothing read
  if (t1 <= t0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      a.out_o[((row0 + h) * a.out_slots + slot) * D + tid] = 0.f;
      if (tid == 0) a.out_lse[(row0 + h) * a.out_slots + slot] = -INFINITY;
    }
    return;
  }

  const uint16_t* layer_base = a.arena + a.layer_off;
  const int32_t* trow = a.table + (int64_t)b * a.pt_stride;
  const int first_page = (t0 - a.token_begin) / PT;
  const int n_pages = (t1 - t0 + PT - 1) / PT;
  // this wave's pages: w, w + 4, ...
  const int my_pages = (n_pages > w) ? (n_pages - w + kWaves - 1) / kWaves : 0;

  // Prologue: the page ids, the query group and the first chunk's K/V loads
  // are all issued before anything waits, so their latencies overlap.
  // Page ids of this wave's pages (at most 64: split_tokens <= 16384): lane j
  // holds the id of the wave's page j, read with readlane, so no dependent
  // global load sits in front of K/V loads inside the loop.
  const int my_id = (lane < my_pages) ? trow[first_page + w + kWaves * lane] : 0;
  // the query group: 16 rows (zero past G) x 32 pieces = 2 pieces per thread
  uint4 qv[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = tid + r * kThreads;
    const int h = i / (D / 8);
    qv[r] = (h < G) ? reinterpret_cast<const uint4*>(a.q + (row0 + h) * D)[i % (D / 8)]
                    : make_uint4(0, 0, 0, 0);
  }
  const uint16_t* stage_base = a.stage_arena + a.stage_layer_off;
  auto page_at = [&](int j) {
    PageRef pg;
    int phys = __builtin_amdgcn_readlane(my_id, j);
    pg.valid = min(PT, t1 - (t0 + (w + kWaves * j) * PT));
    const uint16_t* base = layer_base;
    if (phys >= a.num_pages && phys - a.num_pages < a.stage_pages) {   // a staged page
      phys -= a.num_pages;
      base = stage_base;
    } else if (phys < 0 || phys >= a.num_pages) {
      phys = 0;                                    // read page 0 of the pool, mask all
      pg.valid = 0;
    }
    const uint16_t* page = base + (int64_t)phys * a.page_elems;
    pg.k = page + (int64_t)g * PT * D;
    pg.v = page + (int64_t)(a.num_kv_heads + g) * PT * D;
    return pg;
  };
  // One register buffer: the next chunk's K (V) loads follow QK (PV) of
  // this chunk.
  uint4 kA[2][8], vA[16];
  const int n_chunks = 2 * my_pages;
  PageRef cur = page_at(0);
  if (n_chunks > 0) {
    load_k(kA, cur, 0, lane);
    load_v(vA, cur, 0, lane);
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = tid + r * kThreads;
    *reinterpret_cast<uint4*>(&q_lds[(i / (D / 8)) * kQPad + 8 * (i % (D / 8))]) = qv[r];
  }
  __syncthreads();

  // B operand of QK (head n, channels 32kb + 8q .. +7) is read from LDS at
  // every use rather than held in 32 registers.
  const uint16_t* qrow = &q_lds[n * kQPad + 8 * q];

  float m = -INFINITY;   // running max of head n (base 2), same in the 4 lanes of a head
  float lsum = 0.f;      // this lane's share of the running sum
  f32x4_t acc[16];       // O^T tile db: channels 16db + 4q + i, head n
#pragma unroll
  for (int db = 0; db < 16; ++db) acc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (n_chunks > 0) {
    int cbase = 0;
    for (int ci = 0; ci + 1 < n_chunks; ++ci) {
      const int ni = ci + 1;
      const PageRef nxt = (ni & 1) ? cur : page_at(ni >> 1);
      const int nbase = 32 * (ni & 1);
      chunk<true>(kA, vA, acc, m, lsum, qrow, max(0, min(32, cur.valid - cbase)), a.scale_log2,
                  q, lane, nxt, nbase);
      cur = nxt;
      cbase = nbase;
    }
    chunk<false>(kA, vA, acc, m, lsum, qrow, max(0, min(32, cur.valid - cbase)), a.scale_log2, q,
                 lane, cur, cbase);
  }

  // ---- this wave's (m, l, acc) into LDS
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

  // ---- fixed-order merge of the 4 waves; thread tid owns channel tid
#pragma unroll 1
  for (int h = 0; h < G; ++h) {
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, m_lds[v][h]);
    float o = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const float f = fast_exp2(m_lds[v][h] - M);     // 0 for a wave with no keys
        if (f != 0.f) {
          L = fmaf(f, l_lds[v][h], L);
          o = fmaf(f, acc_lds[v][h][tid], o);
        }
      }
    }
    const bool live = L > 0.f;
    a.out_o[((row0 + h) * a.out_slots + slot) * D + tid] = live ? o / L : 0.f;
    if (tid == 0)
      a.out_lse[(row0 + h) * a.out_slots + slot] =
          uncovered ? NAN : (live ? (M + log2f(L)) * kLn2 : -INFINITY);
  }
}

}  // namespace exact
}  // namespace pkv
