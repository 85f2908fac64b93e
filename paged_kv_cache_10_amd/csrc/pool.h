// Host-side pool handle and error reporting shared by the C ABI sources.
#pragma once

#include <stdint.h>

#include "../../include/pkv.h"

struct pkv_pool {
  pkv_geom geom;
  void* base;
  uint64_t bytes;
  uint64_t page_bytes;        // one physical page, all layers
  uint64_t page_layer_bytes;  // one (layer, page)
  int64_t num_pages;
  int32_t format;             // PKV_FORMAT_BF16 or PKV_FORMAT_E4M3
  uint64_t scale_offset;      // E4M3: byte offset of the scale region in the arena
};

namespace pkv {
// Record `code` and a printf-style message for pkv_last_error(); returns code.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// A layer of a staging pool whose pages a composed table names as entries
// num_pages .. num_pages + stage pages - 1 of the decoded pool.
struct StageRef {
  const pkv_pool* pool;
  int32_t layer;
};

// pkv_decode_attention_merged over a composed table (the live pool); with
// dry_run only the argument checks run and nothing is launched.
int decode_merged_staged(const pkv_pool* pool, int32_t layer, const void* q,
                         const int32_t* dev_table, int32_t pt_stride, const int32_t* dev_ctx_lens,
                         int32_t batch, int32_t num_q_heads, int32_t token_count,
                         int32_t tile_tokens, float scale, float* part_out, float* part_lse,
                         int32_t num_slots, float* out, float* lse, void* workspace,
                         uint64_t workspace_bytes, const pkv_decode_opts* opts, void* stream,
                         const StageRef& stage, bool dry_run = false);

// One run of pkv_decode_attention_runs, with a layer of its own and, for an
// exact run, a staging pool its table may name.
struct RunSpec {
  const pkv_pool* pool;
  int32_t layer;
  const int32_t* dev_table;
  int32_t pt_stride;
  const int32_t* dev_ctx_lens;
  int32_t token_count;
  int32_t tile_tokens;
  int32_t slot_offset;
  const StageRef* stage;
};

int runs_impl(const RunSpec* runs, int32_t n_runs, const void* q, int32_t batch,
              int32_t num_q_heads, float scale, float* part_out, float* part_lse,
              int32_t num_slots, void* stream, bool dry_run);
}  // namespace pkv
