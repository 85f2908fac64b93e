// Host-side launchers of the gfx950 kernels (internal to libpkv).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"

namespace pkv {

// Segmented FP32 log-sum-exp merge: output slot j of a row merges input
// slots [j * group, min((j + 1) * group, in_slots)) of the same row.
struct MergeArgs {
  const float* in_o;     // [rows][in_slots][256]
  const float* in_lse;   // [rows][in_slots]
  int32_t in_slots;
  int32_t group;
  float* out_o;          // [rows][out_slots][256]
  float* out_lse;        // [rows][out_slots]
  int32_t out_slots;
  int32_t out_slot0;     // output slot of j = 0
  int32_t n_out;         // output slots written per row
};

hipError_t launch_merge(const MergeArgs& a, int rows, hipStream_t stream);
// The same groups of rows of at most 64 input slots, then their n_out
// results merged into fin_o [rows][256] and fin_lse [rows], in one launch.
hipError_t launch_merge2(const MergeArgs& a, int rows, float* fin_o, float* fin_lse,
                         hipStream_t stream);

// Split-KV decode: one work-group per (split, kv head, request) writes the
// normalised output and log-sum-exp of its split for the kv head's query
// group.  `group` = num_q_heads / num_kv_heads.
hipError_t launch_decode_valu(const DecodeArgs& a, int batch, int group, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeArgs& a, int batch, int group, hipStream_t stream);

// KV append: request b's token positions[b] gets rows k[b], v[b] of every KV
// head in `layer`.
struct AppendArgs {
  uint16_t* arena;
  int64_t page_elems;        // bf16 elements of one (layer, page)
  int64_t layer_off;         // element offset of the layer's slab
  int32_t num_pages;
  int32_t num_kv_heads;
  const int32_t* table;      // [batch][pt_stride]
  int32_t pt_stride;
  const int32_t* positions;  // [batch] token index to write (-1: none)
  const uint16_t* k;         // [batch][num_kv_heads][256] bf16
  const uint16_t* v;         // [batch][num_kv_heads][256] bf16
};

hipError_t launch_append(const AppendArgs& a, int batch, hipStream_t stream);

// Tail write-back: for each listed row, the K and V elements of one token
// copied from a page of one arena to the same token of a page of another
// (a host arena in pinned memory the device addresses), in the block layout,
// byte for byte: 2 x num_kv_heads x 256 bf16 per row, nothing else.
struct TailRow {
  int32_t src_page;          // page of the source arena (0..src_num_pages-1)
  int32_t dst_page;          // page of the destination arena (0..dst_num_pages-1)
  int32_t token;             // token within the page (0..63)
  int32_t unused;
};
constexpr int kMaxTailRows = 128;   // rows per launch (kernel-argument space)
struct WritebackArgs {
  const uint16_t* src;       // source arena
  int64_t src_layer_off;     // element offset of the source layer's slab
  int64_t src_num_pages;
  uint16_t* dst;             // destination arena (device address)
  int64_t dst_layer_off;
  int64_t dst_num_pages;
  int64_t page_elems;        // bf16 elements of one (layer, page), both arenas
  int32_t num_kv_heads;
  int32_t n;                 // rows used (1..kMaxTailRows)
  TailRow rows[kMaxTailRows];
};

hipError_t launch_writeback(const WritebackArgs& a, hipStream_t stream);

// Largest query group each kernel supports.
constexpr int kValuMaxGroup = 8;
constexpr int kMfmaMaxGroup = 16;

}  // namespace pkv
