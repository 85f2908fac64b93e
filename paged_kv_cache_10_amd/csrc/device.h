// Device-side helpers shared by the gfx950 kernels of libpkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kHeadDim = 256;     // channels per head the kernels are built for
constexpr int kPageTokens = 64;   // tokens per page
constexpr int kMaxGroup = 16;     // query heads per KV head, at most

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Both halves of a packed bf16 pair, widened exactly to FP32.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// a.lo * b.lo + a.hi * b.hi + c, bf16 products exact, FP32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// 2^x on the transcendental unit; 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A 16-byte load marked nontemporal (the instruction's nt bit): the history
// is read once per step, so its lines are streamed past the caches instead
// of being allocated in them.  Measured on the decode kernels' access shape
// (random 32 KiB blocks, one 4-wave work-group per CU): 6.78-6.83 TB/s
// against 6.00-6.02 TB/s for ordinary loads.
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float2 load_stream(const float2* p) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(p));
  return make_float2(v.x, v.y);
}

// Pool block layout.  A (layer, page, K|V, kv head) block holds 64 tokens x
// 256 channels as 2,048 pieces of 16 bytes (8 bf16), stored in the order the
// MFMA kernel's wave loads consume them: 64 consecutive pieces (1 KiB) per
// load instruction, lane l taking piece l, so every load is one contiguous
// 1 KiB read.
//   K piece (token j, channels 8c..8c+7): h = j/32 (32-token half), within
//   the half jj = j%32 goes to MFMA tile t = (jj/4)%2, row r = 4(jj/8)+jj%4,
//   and the piece to k-step c/4, lane group c%4.
//   V piece (channel d, tokens 8u..8u+7): half u/4, channel block d/16,
//   lane group u%4, row d%16.
__device__ __forceinline__ int k_piece(int j, int c) {
  const int h = j >> 5, jj = j & 31;
  const int t = (jj >> 2) & 1, r = 4 * (jj >> 3) + (jj & 3);
  return ((h * 2 + t) * 8 + (c >> 2)) * 64 + (c & 3) * 16 + r;
}
__device__ __forceinline__ int v_piece(int d, int u) {
  return ((u >> 2) * 16 + (d >> 4)) * 64 + (u & 3) * 16 + (d & 15);
}

// Work order of a decode launch.  The grid holds one work-group per (split,
// KV head, request): gridDim = (splits per row, KV heads, requests).  The
// hardware deals work-groups to the 8 XCDs round-robin by linear id and
// starts them in that order, so the linear id decides where and when a split
// runs.  The order used: every non-empty split first, request by request, KV
// head by KV head, split by split; then the empty splits (those wholly past a
// request's length) in the same order.  Consecutive splits of a row so land
// on consecutive XCDs, the real work starts in the first rounds on all CUs,
// and the empty work-groups (which only write an empty partial) run last,
// in the gaps the finishing work leaves.  Within a row the live splits are
// rotated by (row mod 8), so the KV heads of one split, which read the same
// pages, start on different XCDs (measured: ~1 % faster than leaving them
// on one).  A split's arithmetic does not depend on which work-group runs
// it, so the order changes no result bit.
struct WorkItem {
  int b;       // request
  int g;       // KV head
  int split;   // split within the window
  int ctx;     // ctx_lens[b]
  int S;       // tokens per split of request b
};

// Splits of request b's row that hold at least one key of the window.
__device__ __forceinline__ int live_splits(int ctx, int token_begin, int token_count,
                                           int split_tokens) {
  const int c = min(ctx, token_begin + token_count) - token_begin;
  return c > 0 ? (c + split_tokens - 1) / split_tokens : 0;
}

// The item at position j of request b's items in a pass (0: its ph = live
// live splits per KV head, 1: its ph empty splits per KV head).
__device__ __forceinline__ WorkItem item_at(int b, unsigned j, unsigned ph, unsigned live,
                                            int pass, unsigned hkv, int ctx, int S) {
  WorkItem it;
  it.b = b;
  const unsigned g = j / ph;
  const unsigned pos = j - g * ph;
  it.g = (int)g;
  if (pass == 0) {
    // a row's live splits rotated by (row mod 8): the KV heads of one split
    // (the same pages) then start on different XCDs
    unsigned rot = (g + hkv * (unsigned)b) & 7u;
    if (rot >= ph) rot %= ph;
    const unsigned r = pos + ph - rot;            // < 2 ph
    it.split = (int)(r >= ph ? r - ph : r);
  } else {
    it.split = (int)(live + pos);
  }
  it.ctx = ctx;
  it.S = S;
  return it;
}

// This work-group's item.  Up to 4 requests the lengths are read with
// uniform (scalar) loads and walked in order; beyond, every wave computes the
// item in parallel (the same value): lane j holds request 64k + j of chunk
// k, and an exclusive prefix over the chunk's lanes (readlane broadcasts,
// uniform) locates the request whose items contain the linear id.
// row_split (or null) gives each request its own split length; a request
// needing more splits than the grid row holds gets the row's splits (the
// kernel flags the uncovered rest).
// The launch (or the run of a launch) has n_split splits per row, hkv KV
// heads and batch requests; lin is the work-group's linear id within it.
__device__ __forceinline__ WorkItem dense_item(const int32_t* ctx_lens, const int32_t* row_split,
                                               int token_begin, int token_count,
                                               int split_tokens, unsigned n_split, unsigned hkv,
                                               int batch, unsigned lin) {
  // live splits of a request; a malformed per-request split reads nothing
  auto live_of = [&](int ctx, int S) {
    return S >= kPageTokens ? min(live_splits(ctx, token_begin, token_count, S), (int)n_split) : 0;
  };
  if (batch <= 4) {
    int cs[4], ss[4], lv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {            // every load issued before any is used
      cs[i] = (i < batch) ? ctx_lens[i] : 0;
      ss[i] = (i < batch) ? (row_split ? row_split[i] : split_tokens) : 0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) lv[i] = (i < batch) ? live_of(cs[i], ss[i]) : 0;
    unsigned base = 0;
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= batch) break;
        const unsigned ph = pass == 0 ? (unsigned)lv[i] : n_split - (unsigned)lv[i];
        const unsigned v = ph * hkv;
        if (lin < base + v) return item_at(i, lin - base, ph, lv[i], pass, hkv, cs[i], ss[i]);
        base += v;
      }
    }
  } else {
    const int lane = threadIdx.x & 63;
    unsigned base = 0;                       // items of this pass before the chunk
    for (int pass = 0; pass < 2; ++pass) {
      for (int c0 = 0; c0 < batch; c0 += 64) {
        const int b = c0 + lane;
        const int cb = (b < batch) ? ctx_lens[b] : 0;
        const int sb = (b < batch) ? (row_split ? row_split[b] : split_tokens) : 0;
        const int live = (b < batch) ? live_of(cb, sb) : 0;
        const unsigned per_head = (b < batch) ? (pass == 0 ? live : n_split - live) : 0u;
        const unsigned v = per_head * hkv;
        const int nl = min(64, batch - c0);
        unsigned pre = 0, tot = 0;
        for (int i = 0; i < nl; ++i) {
          const unsigned x = (unsigned)__builtin_amdgcn_readlane((int)v, i);
          pre += (i < lane) ? x : 0u;
          tot += x;
        }
        const bool mine = lin >= base + pre && lin < base + pre + v;
        const unsigned long long hit = __ballot(mine);
        if (hit != 0ull) {
          const int l = __ffsll((long long)hit) - 1;
          return item_at(c0 + l, lin - base - (unsigned)__builtin_amdgcn_readlane((int)pre, l),
                         (unsigned)__builtin_amdgcn_readlane((int)per_head, l),
                         (unsigned)__builtin_amdgcn_readlane(live, l), pass, hkv,
                         __builtin_amdgcn_readlane(cb, l), __builtin_amdgcn_readlane(sb, l));
        }
        base += tot;
      }
    }
  }
  WorkItem none = {0, 0, 0, 0, split_tokens};   // not reached: the items cover the grid
  return none;
}

// The item of a launch whose grid is (splits per row, KV heads, requests).
__device__ __forceinline__ WorkItem dense_item_grid(const int32_t* ctx_lens,
                                                    const int32_t* row_split, int token_begin,
                                                    int token_count, int split_tokens) {
  // grid sizes and ids are uniform: readfirstlane keeps the walk (and its
  // loads) on the scalar unit
  const unsigned n_split = __builtin_amdgcn_readfirstlane(gridDim.x);
  const unsigned hkv = __builtin_amdgcn_readfirstlane(gridDim.y);
  const int batch = __builtin_amdgcn_readfirstlane(gridDim.z);
  const unsigned lin = blockIdx.x + n_split * (blockIdx.y + hkv * blockIdx.z);
  return dense_item(ctx_lens, row_split, token_begin, token_count, split_tokens, n_split, hkv,
                    batch, lin);
}

// ---- Wave-level reductions on the VALU's lane-crossing paths, no LDS round
// trip.  Within a 16-lane row DPP combines lanes (quad_perm [1,0,3,2] pairs
// lane i with i^1, [2,3,0,1] with i^2, row_half_mirror with the mirror lane
// of its 8-lane half, row_mirror with the mirror lane of its row);
// v_permlane16_swap and v_permlane32_swap (gfx950) exchange whole rows, so a
// value and its swapped copy hold lanes l and l^16 (l^32).  Every step
// combines two partials over disjoint sets of lanes, and both lanes of a
// pair compute the same commutative operation, so after the steps up to
// width w every lane of a w-lane group holds the same bits.
namespace dpp {
constexpr int kXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;   // row_half_mirror
constexpr int kMirror = 0x140;       // row_mirror
}  // namespace dpp

template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xf, 0xf, false));
}

// {value of lane l, value of lane l^16} in some order, at every lane l.
__device__ __forceinline__ void swap16(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
// {value of lane l, value of lane l^32} in some order, at every lane l.
__device__ __forceinline__ void swap32(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Over lanes {l, l^16}, {l, l^32}: max and sum.
__device__ __forceinline__ float max_x16(float x) { float a, b; swap16(x, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float max_x32(float x) { float a, b; swap32(x, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float sum_x16(float x) { float a, b; swap16(x, a, b); return a + b; }
__device__ __forceinline__ float sum_x32(float x) { float a, b; swap32(x, a, b); return a + b; }

// Sum over the 8-lane group of lane l (lanes 8k .. 8k+7).
__device__ __forceinline__ float sum8(float x) {
  x += dpp_mov<dpp::kXor1>(x);
  x += dpp_mov<dpp::kXor2>(x);
  return x + dpp_mov<dpp::kHalfMirror>(x);
}

// Max and sum over the whole wave.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_mov<dpp::kXor1>(x));
  x = fmaxf(x, dpp_mov<dpp::kXor2>(x));
  x = fmaxf(x, dpp_mov<dpp::kHalfMirror>(x));
  x = fmaxf(x, dpp_mov<dpp::kMirror>(x));
  return max_x32(max_x16(x));
}
__device__ __forceinline__ float wave_sum(float x) {
  x = sum8(x);
  x += dpp_mov<dpp::kMirror>(x);
  return sum_x32(sum_x16(x));
}

// Max that keeps a NaN (fmaxf drops it): a NaN log-sum-exp marks a partial
// that must not be merged away.
__device__ __forceinline__ float max_nan(float a, float b) {
  return (a != a) ? a : ((b != b) ? b : fmaxf(a, b));
}
__device__ __forceinline__ float wave_max_nan(float x) {
  x = max_nan(x, dpp_mov<dpp::kXor1>(x));
  x = max_nan(x, dpp_mov<dpp::kXor2>(x));
  x = max_nan(x, dpp_mov<dpp::kHalfMirror>(x));
  x = max_nan(x, dpp_mov<dpp::kMirror>(x));
  float a, b;
  swap16(x, a, b);
  x = max_nan(a, b);
  swap32(x, a, b);
  return max_nan(a, b);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Arguments of one decode launch: per-split partials of one layer.
struct DecodeArgs {
  const uint16_t* arena;     // bf16 arena
  int64_t page_elems;        // bf16 elements of one (layer, page): 2 x Hkv blocks
  int64_t layer_off;         // element offset of this layer's slab in the arena
  int32_t num_pages;
  int32_t num_kv_heads;
  const uint16_t* q;         // [batch][num_q_heads][256]
  const int32_t* table;      // [batch][pt_stride], entry i = logical page token_begin/64 + i
  int32_t pt_stride;
  const int32_t* ctx_lens;   // [batch]
  int32_t num_q_heads;
  int32_t token_begin;       // first token of the window (multiple of split_tokens)
  int32_t token_count;       // window length (multiple of split_tokens)
  int32_t split_tokens;      // tokens per work-group (multiple of 64)
  const int32_t* row_split;  // [batch] tokens per work-group of each request, or null
                             // (split_tokens for all); with it every split is a tile
  float scale_log2;          // softmax scale * log2(e): scores are kept in base 2
  float* out_o;              // [batch][num_q_heads][out_slots][256]
  float* out_lse;            // [batch][num_q_heads][out_slots]
  int32_t out_slots;         // slots per row of out_o / out_lse
  int32_t out_slot0;         // slot written by split 0 of this window
  // A second, staging arena (the MFMA kernel only): a table entry e with
  // num_pages <= e < num_pages + stage_pages names page e - num_pages of it,
  // read from stage_arena + stage_layer_off; every other entry outside
  // [0, num_pages) is skipped.  stage_pages = 0: no staging arena.
  const uint16_t* stage_arena = nullptr;
  int64_t stage_layer_off = 0;
  int32_t stage_pages = 0;
};

}  // namespace pkv
