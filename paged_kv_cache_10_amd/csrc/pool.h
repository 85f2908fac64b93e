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
};

namespace pkv {
// Record `code` and a printf-style message for pkv_last_error(); returns code.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
}  // namespace pkv
