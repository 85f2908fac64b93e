// libpkv host side: the C ABI of include/pkv.h.  Every check runs on the
// host before any device work; a call that passes them only queues kernels
// on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "kernels.h"
#include "pool.h"

#define PKV_API extern "C" __attribute__((visibility("default")))

namespace {
thread_local char g_err[512] = "";
}  // namespace

namespace pkv {
int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}
void clear_error() { g_err[0] = '\0'; }
}  // namespace pkv

namespace {

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wformat-security"
template <typename... A>
int fail(int code, const char* fmt, A... args) {   // every caller passes a literal
  return pkv::set_error(code, fmt, args...);
}
#pragma clang diagnostic pop

int ok() {
  pkv::clear_error();
  return PKV_OK;
}

constexpr int kDefaultSplit = 2048;  // tokens per work-group unless the caller says otherwise

int check_geom(const pkv_geom* g) {
  if (!g) return fail(PKV_ERR_INVALID_ARG, "geom is NULL");
  if (g->num_layers < 1) return fail(PKV_ERR_GEOMETRY, "geom.num_layers = %d, need >= 1", g->num_layers);
  if (g->num_kv_heads < 1)
    return fail(PKV_ERR_GEOMETRY, "geom.num_kv_heads = %d, need >= 1", g->num_kv_heads);
  if (g->head_dim != pkv::kHeadDim)
    return fail(PKV_ERR_GEOMETRY, "geom.head_dim = %d: the kernels are built for head_dim = %d",
                g->head_dim, pkv::kHeadDim);
  if (g->page_tokens != pkv::kPageTokens)
    return fail(PKV_ERR_GEOMETRY, "geom.page_tokens = %d: the kernels are built for %d-token pages",
                g->page_tokens, pkv::kPageTokens);
  return PKV_OK;
}

uint64_t page_layer_bytes(const pkv_geom* g) {
  return 2ull * (uint64_t)g->num_kv_heads * (uint64_t)g->page_tokens * (uint64_t)g->head_dim * 2ull;
}

// Tokens per work-group for a tile length: the requested split, else the
// largest multiple of 64 that divides tile_tokens and is <= kDefaultSplit.
int split_for(int tile_tokens, const pkv_decode_opts* opts, int* split_out) {
  if (opts && opts->split_tokens > 0) {
    const int s = opts->split_tokens;
    if (s % pkv::kPageTokens || tile_tokens % s)
      return fail(PKV_ERR_INVALID_ARG,
                  "opts.split_tokens = %d must be a multiple of %d that divides tile_tokens = %d", s,
                  pkv::kPageTokens, tile_tokens);
    *split_out = s;
    return PKV_OK;
  }
  int best = pkv::kPageTokens;
  for (int s = pkv::kPageTokens; s <= kDefaultSplit && s <= tile_tokens; s += pkv::kPageTokens)
    if (tile_tokens % s == 0) best = s;
  *split_out = best;
  return PKV_OK;
}

int kernel_for(const pkv_decode_opts* opts, int group, int* kernel_out) {
  int k = opts ? opts->kernel : 0;
  if (k < 0 || k > 2) return fail(PKV_ERR_INVALID_ARG, "opts.kernel = %d, need 0, 1 or 2", k);
  if (k == 0) k = 2;                                           // MFMA is the default
  if (k == 1 && group > pkv::kValuMaxGroup)
    return fail(PKV_ERR_GEOMETRY, "query group %d exceeds the VALU kernel's %d", group,
                pkv::kValuMaxGroup);
  if (k == 2) {
    const bool built = (group >= 1 && group <= 8) || group == 12 || group == 16;
    if (!built)
      return fail(PKV_ERR_GEOMETRY, "query group %d: the MFMA kernel is built for 1..8, 12, 16",
                  group);
  }
  *kernel_out = k;
  return PKV_OK;
}

}  // namespace

PKV_API const char* pkv_last_error(void) { return g_err; }

PKV_API int32_t pkv_abi_version(void) { return PKV_ABI_VERSION; }

PKV_API int pkv_page_bytes(const pkv_geom* geom, uint64_t* page_bytes_out) {
  if (int rc = check_geom(geom)) return rc;
  if (!page_bytes_out) return fail(PKV_ERR_INVALID_ARG, "page_bytes_out is NULL");
  *page_bytes_out = page_layer_bytes(geom) * (uint64_t)geom->num_layers;
  return ok();
}

PKV_API int pkv_pool_create(const pkv_geom* geom, void* dev_arena, uint64_t arena_bytes,
                            pkv_pool** pool_out) {
  if (int rc = check_geom(geom)) return rc;
  if (!pool_out) return fail(PKV_ERR_INVALID_ARG, "pool_out is NULL");
  *pool_out = nullptr;
  const uint64_t pb = page_layer_bytes(geom) * (uint64_t)geom->num_layers;
  if (arena_bytes == 0)
    return fail(PKV_ERR_AUTO_SIZE_REFUSED,
                "arena_bytes = 0: an automatic pool size is refused; pass an explicit size, a "
                "whole number of %llu-byte pages",
                (unsigned long long)pb);
  if (arena_bytes % pb) {
    const unsigned long long lo = arena_bytes / pb;
    return fail(PKV_ERR_INVALID_ARG,
                "arena_bytes = %llu is not a whole number of %llu-byte pages; use %llu (%llu pages) "
                "or %llu (%llu pages)",
                (unsigned long long)arena_bytes, (unsigned long long)pb, lo * pb, lo,
                (lo + 1) * pb, lo + 1);
  }
  if (!dev_arena) return fail(PKV_ERR_INVALID_ARG, "dev_arena is NULL");
  if (reinterpret_cast<uintptr_t>(dev_arena) % 256)
    return fail(PKV_ERR_INVALID_ARG, "dev_arena %p is not 256-byte aligned", dev_arena);
  const uint64_t pages = arena_bytes / pb;
  if (pages > (uint64_t)INT32_MAX)
    return fail(PKV_ERR_INVALID_ARG, "arena holds %llu pages; page ids are int32",
                (unsigned long long)pages);
  pkv_pool* p = new (std::nothrow) pkv_pool;
  if (!p) return fail(PKV_ERR_INVALID_ARG, "host allocation failed");
  p->geom = *geom;
  p->base = dev_arena;
  p->bytes = arena_bytes;
  p->page_bytes = pb;
  p->page_layer_bytes = page_layer_bytes(geom);
  p->num_pages = (int64_t)pages;
  *pool_out = p;
  return ok();
}

PKV_API int pkv_pool_info(const pkv_pool* pool, int64_t* num_pages, uint64_t* page_bytes,
                          void** dev_arena) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (num_pages) *num_pages = pool->num_pages;
  if (page_bytes) *page_bytes = pool->page_bytes;
  if (dev_arena) *dev_arena = pool->base;
  return ok();
}

PKV_API int pkv_pool_destroy(pkv_pool* pool) {
  delete pool;
  return ok();
}

PKV_API int pkv_page_table_validate(const pkv_pool* pool, const int32_t* host_table,
                                    const int32_t* host_ctx_lens, int32_t batch,
                                    int32_t pt_stride) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (batch < 0) return fail(PKV_ERR_INVALID_ARG, "batch = %d is negative", batch);
  if (pt_stride < 1) return fail(PKV_ERR_INVALID_ARG, "pt_stride = %d, need >= 1", pt_stride);
  if (batch == 0) return ok();
  if (!host_table || !host_ctx_lens)
    return fail(PKV_ERR_INVALID_ARG, "host_table or host_ctx_lens is NULL");
  const int64_t P = pool->num_pages;
  const int PT = pool->geom.page_tokens;
  std::vector<int32_t> owner((size_t)P, -1);
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t ctx = host_ctx_lens[b];
    if (ctx < 0) return fail(PKV_ERR_PAGE_TABLE, "ctx_lens[%d] = %lld is negative", b, (long long)ctx);
    if (ctx > (int64_t)pt_stride * PT)
      return fail(PKV_ERR_PAGE_TABLE,
                  "ctx_lens[%d] = %lld needs %lld pages but pt_stride = %d; raise pt_stride", b,
                  (long long)ctx, (long long)((ctx + PT - 1) / PT), pt_stride);
    const int64_t need = (ctx + PT - 1) / PT;
    const int32_t* row = host_table + (int64_t)b * pt_stride;
    for (int64_t i = 0; i < pt_stride; ++i) {
      const int32_t e = row[i];
      if (i < need) {
        if (e < 0 || e >= P)
          return fail(PKV_ERR_PAGE_TABLE,
                      "table[%d][%lld] = %d is not a page of this pool (0..%lld)%s", b,
                      (long long)i, e, (long long)(P - 1),
                      i == 0 ? "; entry 0 is the request's sink page and must always be present"
                             : "");
        if (owner[(size_t)e] >= 0)
          return fail(PKV_ERR_PAGE_TABLE, "page %d appears twice (rows %d and %d)", e,
                      owner[(size_t)e], b);
        owner[(size_t)e] = b;
      } else if (e != -1) {
        return fail(PKV_ERR_PAGE_TABLE,
                    "table[%d][%lld] = %d past the request's %lld pages; padding must be -1", b,
                    (long long)i, e, (long long)need);
      }
    }
  }
  return ok();
}

PKV_API int pkv_page_table_write(const pkv_pool* pool, const int32_t* host_table,
                                 const int32_t* host_ctx_lens, int32_t batch, int32_t pt_stride,
                                 int32_t* dev_table, int32_t* dev_ctx_lens, void* stream) {
  if (int rc = pkv_page_table_validate(pool, host_table, host_ctx_lens, batch, pt_stride))
    return rc;
  if (batch == 0) return ok();
  if (!dev_table || !dev_ctx_lens) return fail(PKV_ERR_INVALID_ARG, "dev_table or dev_ctx_lens is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(dev_table, host_table, sizeof(int32_t) * (size_t)batch * pt_stride,
                                hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(dev_ctx_lens, host_ctx_lens, sizeof(int32_t) * (size_t)batch,
                       hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess)
    return fail(PKV_ERR_DEVICE, "page-table copy failed: %s", hipGetErrorString(e));
  return ok();
}

PKV_API int pkv_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                       int32_t token_count, int32_t tile_tokens,
                                       const pkv_decode_opts* opts, uint64_t* bytes_out) {
  if (!bytes_out) return fail(PKV_ERR_INVALID_ARG, "bytes_out is NULL");
  if (batch < 0 || num_q_heads < 1 || token_count < 0)
    return fail(PKV_ERR_INVALID_ARG, "batch = %d, num_q_heads = %d, token_count = %d", batch,
                num_q_heads, token_count);
  if (head_dim != pkv::kHeadDim)
    return fail(PKV_ERR_GEOMETRY, "head_dim = %d: built for %d", head_dim, pkv::kHeadDim);
  if (tile_tokens <= 0 || tile_tokens % pkv::kPageTokens)
    return fail(PKV_ERR_INVALID_ARG, "tile_tokens = %d must be a positive multiple of %d",
                tile_tokens, pkv::kPageTokens);
  int split = 0;
  if (int rc = split_for(tile_tokens, opts, &split)) return rc;
  if (split == tile_tokens) {
    *bytes_out = 0;
    return ok();
  }
  const uint64_t n_split = (uint64_t)((token_count + split - 1) / split);
  *bytes_out = (uint64_t)batch * num_q_heads * n_split * (uint64_t)(head_dim + 1) * sizeof(float);
  return ok();
}

PKV_API int pkv_decode_attention(const pkv_pool* pool, int32_t layer, const void* q,
                                 const int32_t* dev_table, int32_t pt_stride,
                                 const int32_t* dev_ctx_lens, int32_t batch, int32_t num_q_heads,
                                 int32_t token_begin, int32_t token_count, int32_t tile_tokens,
                                 float scale, float* part_out, float* part_lse, int32_t num_slots,
                                 void* workspace, uint64_t workspace_bytes,
                                 const pkv_decode_opts* opts, void* stream) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  const pkv_geom& G = pool->geom;
  if (layer < 0 || layer >= G.num_layers)
    return fail(PKV_ERR_INVALID_ARG, "layer = %d outside 0..%d", layer, G.num_layers - 1);
  if (batch < 0) return fail(PKV_ERR_INVALID_ARG, "batch = %d is negative", batch);
  if (batch > 65535) return fail(PKV_ERR_INVALID_ARG, "batch = %d exceeds 65535", batch);
  if (num_q_heads < 1 || num_q_heads % G.num_kv_heads)
    return fail(PKV_ERR_GEOMETRY, "num_q_heads = %d must be a positive multiple of num_kv_heads = %d",
                num_q_heads, G.num_kv_heads);
  const int group = num_q_heads / G.num_kv_heads;
  int kernel = 0;
  if (int rc = kernel_for(opts, group, &kernel)) return rc;
  if (tile_tokens <= 0 || tile_tokens % G.page_tokens)
    return fail(PKV_ERR_INVALID_ARG, "tile_tokens = %d must be a positive multiple of %d",
                tile_tokens, G.page_tokens);
  if (token_begin < 0 || token_begin % tile_tokens)
    return fail(PKV_ERR_INVALID_ARG, "token_begin = %d must be a non-negative multiple of tile_tokens = %d",
                token_begin, tile_tokens);
  if (token_count < 0 || token_count % tile_tokens)
    return fail(PKV_ERR_INVALID_ARG, "token_count = %d must be a non-negative multiple of tile_tokens = %d",
                token_count, tile_tokens);
  if ((int64_t)token_begin + token_count > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARG, "token_begin + token_count overflows int32");
  if ((int64_t)pt_stride * G.page_tokens < token_count)
    return fail(PKV_ERR_INVALID_ARG,
                "pt_stride = %d covers %lld tokens, less than token_count = %d", pt_stride,
                (long long)pt_stride * G.page_tokens, token_count);
  const int first_slot = token_begin / tile_tokens;
  const int n_tiles = token_count / tile_tokens;
  if (num_slots < 1 || (int64_t)first_slot + n_tiles > num_slots)
    return fail(PKV_ERR_INVALID_ARG, "slots %d..%d of this window exceed num_slots = %d",
                first_slot, first_slot + n_tiles - 1, num_slots);
  if (num_slots > 65535) return fail(PKV_ERR_INVALID_ARG, "num_slots = %d exceeds 65535", num_slots);
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale is not finite");
  if (batch == 0 || token_count == 0) return ok();
  if (!q || !dev_table || !dev_ctx_lens || !part_out || !part_lse)
    return fail(PKV_ERR_INVALID_ARG, "q, dev_table, dev_ctx_lens, part_out or part_lse is NULL");
  if (reinterpret_cast<uintptr_t>(q) % 16 || reinterpret_cast<uintptr_t>(part_out) % 16)
    return fail(PKV_ERR_INVALID_ARG, "q and part_out must be 16-byte aligned");

  int split = 0;
  if (int rc = split_for(tile_tokens, opts, &split)) return rc;
  uint64_t need = 0;
  if (int rc = pkv_decode_workspace_bytes(batch, num_q_heads, G.head_dim, token_count, tile_tokens,
                                          opts, &need))
    return rc;
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PKV_ERR_WORKSPACE, "workspace of %llu bytes given, %llu needed",
                (unsigned long long)(workspace ? workspace_bytes : 0), (unsigned long long)need);
  if (need > 0 && reinterpret_cast<uintptr_t>(workspace) % 16)
    return fail(PKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

  hipStream_t s = static_cast<hipStream_t>(stream);
  pkv::DecodeArgs a;
  a.arena = static_cast<const uint16_t*>(pool->base);
  a.page_elems = (int64_t)(pool->page_layer_bytes / 2);
  a.layer_off = (int64_t)(pool->page_layer_bytes / 2) * pool->num_pages * layer;
  a.num_pages = (int32_t)pool->num_pages;
  a.num_kv_heads = G.num_kv_heads;
  a.q = static_cast<const uint16_t*>(q);
  a.table = dev_table;
  a.pt_stride = pt_stride;
  a.ctx_lens = dev_ctx_lens;
  a.num_q_heads = num_q_heads;
  a.token_begin = token_begin;
  a.token_count = token_count;
  a.split_tokens = split;
  a.scale_log2 = scale * pkv::kLog2e;

  const int n_split = token_count / split;
  float* ws_o = nullptr;
  float* ws_lse = nullptr;
  if (split == tile_tokens) {          // splits are the tiles: write the caller's slots directly
    a.out_o = part_out;
    a.out_lse = part_lse;
    a.out_slots = num_slots;
    a.out_slot0 = first_slot;
  } else {                             // splits into the workspace, then one merge per tile
    ws_o = static_cast<float*>(workspace);
    ws_lse = ws_o + (size_t)batch * num_q_heads * n_split * G.head_dim;
    a.out_o = ws_o;
    a.out_lse = ws_lse;
    a.out_slots = n_split;
    a.out_slot0 = 0;
  }
  hipError_t e = (kernel == 1) ? pkv::launch_decode_valu(a, batch, group, s)
                               : pkv::launch_decode_mfma(a, batch, group, s);
  if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "decode launch failed: %s", hipGetErrorString(e));
  if (split != tile_tokens) {
    pkv::MergeArgs m;
    m.in_o = ws_o;
    m.in_lse = ws_lse;
    m.in_slots = n_split;
    m.group = tile_tokens / split;
    m.out_o = part_out;
    m.out_lse = part_lse;
    m.out_slots = num_slots;
    m.out_slot0 = first_slot;
    m.n_out = n_tiles;
    e = pkv::launch_merge(m, batch * num_q_heads, s);
    if (e != hipSuccess)
      return fail(PKV_ERR_LAUNCH, "tile finalize launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

PKV_API int pkv_merge_partials(const float* part_out, const float* part_lse, int32_t rows,
                               int32_t num_slots, int32_t head_dim, float* out, float* lse,
                               void* stream) {
  if (rows < 0) return fail(PKV_ERR_INVALID_ARG, "rows = %d is negative", rows);
  if (num_slots < 1) return fail(PKV_ERR_INVALID_ARG, "num_slots = %d, need >= 1", num_slots);
  if (head_dim != pkv::kHeadDim)
    return fail(PKV_ERR_GEOMETRY, "head_dim = %d: built for %d", head_dim, pkv::kHeadDim);
  if (rows == 0) return ok();
  if (!part_out || !part_lse || !out || !lse)
    return fail(PKV_ERR_INVALID_ARG, "part_out, part_lse, out or lse is NULL");
  if (reinterpret_cast<uintptr_t>(part_out) % 16 || reinterpret_cast<uintptr_t>(out) % 16)
    return fail(PKV_ERR_INVALID_ARG, "part_out and out must be 16-byte aligned");
  pkv::MergeArgs m;
  m.in_o = part_out;
  m.in_lse = part_lse;
  m.in_slots = num_slots;
  m.group = num_slots;
  m.out_o = out;
  m.out_lse = lse;
  m.out_slots = 1;
  m.out_slot0 = 0;
  m.n_out = 1;
  hipError_t e = pkv::launch_merge(m, rows, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

PKV_API int pkv_append_kv(const pkv_pool* pool, int32_t layer, const int32_t* dev_table,
                          int32_t pt_stride, const int32_t* dev_positions, int32_t batch,
                          const void* k_new, const void* v_new, void* stream) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  const pkv_geom& G = pool->geom;
  if (layer < 0 || layer >= G.num_layers)
    return fail(PKV_ERR_INVALID_ARG, "layer = %d outside 0..%d", layer, G.num_layers - 1);
  if (batch < 0 || batch > 65535) return fail(PKV_ERR_INVALID_ARG, "batch = %d outside 0..65535", batch);
  if (pt_stride < 1) return fail(PKV_ERR_INVALID_ARG, "pt_stride = %d, need >= 1", pt_stride);
  if (batch == 0) return ok();
  if (!dev_table || !dev_positions || !k_new || !v_new)
    return fail(PKV_ERR_INVALID_ARG, "dev_table, dev_positions, k_new or v_new is NULL");
  if (reinterpret_cast<uintptr_t>(k_new) % 16)
    return fail(PKV_ERR_INVALID_ARG, "k_new must be 16-byte aligned");
  pkv::AppendArgs a;
  a.arena = static_cast<uint16_t*>(pool->base);
  a.page_elems = (int64_t)(pool->page_layer_bytes / 2);
  a.layer_off = (int64_t)(pool->page_layer_bytes / 2) * pool->num_pages * layer;
  a.num_pages = (int32_t)pool->num_pages;
  a.num_kv_heads = G.num_kv_heads;
  a.table = dev_table;
  a.pt_stride = pt_stride;
  a.positions = dev_positions;
  a.k = static_cast<const uint16_t*>(k_new);
  a.v = static_cast<const uint16_t*>(v_new);
  hipError_t e = pkv::launch_append(a, batch, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "append launch failed: %s", hipGetErrorString(e));
  return ok();
}
