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

// XCD-aware placement.  Work-groups are dealt to the 8 XCDs round-robin by
// linear id, and every (request, KV head) row of the grid starts at split 0,
// which is often the row's only non-empty split; with a row length that is a
// multiple of 8 every row's split 0 would land on one XCD.  Rotating each
// row's splits by a row-dependent amount spreads them; a split's arithmetic
// does not depend on which work-group runs it.
__device__ __forceinline__ int rotated_split() {
  const unsigned row = blockIdx.y + gridDim.y * blockIdx.z;
  const unsigned rot = (row & 7u) % gridDim.x;
  return (int)((blockIdx.x + gridDim.x - rot) % gridDim.x);
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
  float scale_log2;          // softmax scale * log2(e): scores are kept in base 2
  float* out_o;              // [batch][num_q_heads][out_slots][256]
  float* out_lse;            // [batch][num_q_heads][out_slots]
  int32_t out_slots;         // slots per row of out_o / out_lse
  int32_t out_slot0;         // slot written by split 0 of this window
};

}  // namespace pkv
