// Compact pages (KV-cache engineering, section "Exact recent pages, compact
// older pages": runs of two representations; a page is converted only after
// every layer has written all its tokens, checksummed, and served exact
// before that).
//
// Representation: E4M3 codes (OCP 8-bit float: bias 7, 3 mantissa bits,
// largest finite 448) with one FP32 scale per (layer, page, K|V, kv head)
// block; a code c stands for value(c) * scale.  scale = amax / 448 in FP32
// (1 for an all-zero block); code = E4M3 rounding (nearest, ties to even,
// saturating at 448, sign of the input kept) of the FP32 quotient x / scale.
//
// Compact arena: code region [layer][page][K|V][kv_head][16 KiB block],
// then scale region [layer][page][K|V][kv_head] FP32.
//
// Block layout: 64 tokens x 256 channels of codes as 1,024 pieces of 16
// bytes in the order the compact decode kernel's wave loads consume them,
// 64 consecutive pieces (1 KiB) per load, lane l taking piece l:
//   K piece ((h*2 + t)*4 + kk)*64 + q*16 + r holds token j = 32h + jj with
//     jj = 8(r/4) + 4t + r%4 (MFMA tile t, row r of the 32-token half h);
//     bytes 0..7 are channels 64kk + 8q .. +7, bytes 8..15 channels
//     64kk + 32 + 8q .. +7 (the lane's operands for k-steps 2kk and 2kk+1).
//   V piece (d/16)*64 + q*16 + d%16 holds channel d; bytes 0..7 are tokens
//     8q .. 8q+7, bytes 8..15 tokens 32 + 8q .. +7 (the lane's operands for
//     the two 32-token halves).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"

namespace pkv {

constexpr int kCompactBlockBytes = kPageTokens * kHeadDim;   // one byte per code
constexpr float kE4M3Max = 448.f;

// Byte offset of (token j, channel c) in a compact K block.
__host__ __device__ __forceinline__ int kc_byte(int j, int c) {
  const int h = j >> 5, jj = j & 31;
  const int t = (jj >> 2) & 1, r = 4 * (jj >> 3) + (jj & 3);
  const int kk = c >> 6, half = (c >> 5) & 1, q = (c >> 3) & 3, e = c & 7;
  return ((((h * 2 + t) * 4 + kk) * 64 + q * 16 + r) << 4) + 8 * half + e;
}
// Byte offset of (channel d, token j) in a compact V block.
__host__ __device__ __forceinline__ int vc_byte(int d, int j) {
  const int h = j >> 5, q = (j >> 3) & 3, e = j & 7;
  return ((((d >> 4) * 64) + q * 16 + (d & 15)) << 4) + 8 * h + e;
}

struct CompactDecodeArgs {
  const uint8_t* codes;      // code region of the compact arena
  const float* scales;       // scale region: [layer][page][K|V][kv_head]
  int64_t page_bytes;        // code bytes of one (layer, page): 2 x Hkv blocks
  int64_t layer_off;         // byte offset of this layer's slab in the code region
  int64_t scale_layer_off;   // float offset of this layer's scales
  int32_t num_pages;
  int32_t num_kv_heads;
  const uint16_t* q;         // [batch][num_q_heads][256] bf16
  const int32_t* table;      // [batch][pt_stride], entry i = logical page token_begin/64 + i
  int32_t pt_stride;
  const int32_t* ctx_lens;   // [batch]
  int32_t num_q_heads;
  int32_t token_begin;
  int32_t token_count;
  int32_t split_tokens;
  float scale_log2;
  float* out_o;
  float* out_lse;
  int32_t out_slots;
  int32_t out_slot0;
};

hipError_t launch_decode_fp8(const CompactDecodeArgs& a, int batch, int group, hipStream_t stream);

// Conversion of whole exact pages (all layers) into compact pages.
struct ConvertArgs {
  const uint16_t* src;       // exact arena (bf16, operand-ordered blocks)
  int64_t src_page_elems;    // bf16 elements of one exact (layer, page)
  int64_t src_num_pages;
  uint8_t* codes;            // compact code region
  float* scales;             // compact scale region
  int64_t dst_page_bytes;    // code bytes of one compact (layer, page)
  int64_t dst_num_pages;
  int32_t num_layers;
  int32_t num_kv_heads;
  const int32_t* src_pages;  // [n] device
  const int32_t* dst_pages;  // [n] device
  int32_t n;
};

hipError_t launch_convert(const ConvertArgs& a, hipStream_t stream);

// CRC-32 of whole compact pages.  The x_* constants are powers of x modulo
// the CRC polynomial (reflected), prepared on the host.
struct CrcArgs {
  const uint8_t* codes;
  const float* scales;
  int64_t page_bytes;        // code bytes of one (layer, page), a multiple of 4 KiB
  int64_t num_pages;
  int32_t num_layers;
  int32_t scale_count;       // scales per (layer, page): 2 x Hkv
  const int32_t* pages;      // [n] device
  int32_t n;
  uint32_t* crc;             // [n] device
  uint32_t x_seg[8];         // x^(8 * seg * 2^k), seg = page_bytes / 256
  uint32_t x_scales;         // x^(8 * 4 * scale_count)
  uint32_t x_layer;          // x^(8 * (page_bytes + 4 * scale_count))
  uint32_t init_term;        // 0xFFFFFFFF advanced over the whole page
};

hipError_t launch_crc(const CrcArgs& a, hipStream_t stream);

// Runs of the history decoded in one launch (KV-cache engineering, section
// "Exact recent pages, compact older pages": runs of two representations).
// Run k has wgs[k] work-groups (its splits x KV heads x requests, one split
// per tile) and is read from a compact pool (compact[k] != 0, c[k]) or an
// exact one (e[k]); the launch's linear work-group ids list run 0's, then
// run 1's, each run in its own work order.
struct RunsArgs {
  int32_t n_runs;              // 1 or 2
  int32_t compact[2];
  int32_t n_split[2];          // splits per row of each run
  int32_t wgs[2];
  int32_t num_kv_heads;
  int32_t batch;
  DecodeArgs e[2];
  CompactDecodeArgs c[2];
};

hipError_t launch_decode_runs(const RunsArgs& a, int group, hipStream_t stream);

}  // namespace pkv
