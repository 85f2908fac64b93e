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
}  // namespace pkv
