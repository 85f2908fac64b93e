// libpkv host side: the C ABI of include/pkv.h.  Every check runs on the
// host before any device work; a call that passes them only queues kernels
// on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "compact.h"
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
constexpr int kMaxMfmaSplit = 64 * 4 * 64;   // 64 pages per wave x 4 waves x 64 tokens
constexpr int kMaxMerge2Splits = 64;          // split partials per row one merge2 launch holds

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

// Compact (layer, page): codes of 2 x Hkv blocks, and their 2 x Hkv scales.
uint64_t compact_code_bytes(const pkv_geom* g) {
  return 2ull * (uint64_t)g->num_kv_heads * (uint64_t)pkv::kCompactBlockBytes;
}
uint64_t compact_scale_bytes(const pkv_geom* g) { return 2ull * (uint64_t)g->num_kv_heads * 4ull; }

int create_pool(const pkv_geom* geom, void* dev_arena, uint64_t arena_bytes, int32_t format,
                pkv_pool** pool_out);

// CRC-32 arithmetic on the host (reflected representation: bit 31 is the
// coefficient of x^0): a * b mod the polynomial, and x^(8 n).
constexpr uint32_t kCrcPoly = 0xEDB88320u;
uint32_t gf_mul(uint32_t a, uint32_t b) {
  uint32_t p = 0;
  for (int i = 0; i < 32; ++i) {
    if (a & (0x80000000u >> i)) p ^= b;
    b = (b & 1u) ? (b >> 1) ^ kCrcPoly : (b >> 1);
  }
  return p;
}
uint32_t x_pow_bytes(uint64_t n) {       // x^(8 n) mod P by square and multiply
  uint32_t result = 0x80000000u;          // x^0
  uint32_t base = 0x00800000u;            // x^8
  while (n) {
    if (n & 1u) result = gf_mul(result, base);
    base = gf_mul(base, base);
    n >>= 1;
  }
  return result;
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
  return create_pool(geom, dev_arena, arena_bytes, PKV_FORMAT_BF16, pool_out);
}

PKV_API int pkv_compact_pool_create(const pkv_geom* geom, void* dev_arena, uint64_t arena_bytes,
                                    pkv_pool** pool_out) {
  return create_pool(geom, dev_arena, arena_bytes, PKV_FORMAT_E4M3, pool_out);
}

PKV_API int pkv_compact_page_bytes(const pkv_geom* geom, uint64_t* page_bytes_out) {
  if (int rc = check_geom(geom)) return rc;
  if (!page_bytes_out) return fail(PKV_ERR_INVALID_ARG, "page_bytes_out is NULL");
  *page_bytes_out = (compact_code_bytes(geom) + compact_scale_bytes(geom)) * (uint64_t)geom->num_layers;
  return ok();
}

PKV_API int pkv_pool_format(const pkv_pool* pool, int32_t* format_out) {
  if (!pool || !format_out) return fail(PKV_ERR_INVALID_ARG, "pool or format_out is NULL");
  *format_out = pool->format;
  return ok();
}

namespace {
int create_pool(const pkv_geom* geom, void* dev_arena, uint64_t arena_bytes, int32_t format,
                pkv_pool** pool_out) {
  if (int rc = check_geom(geom)) return rc;
  if (!pool_out) return fail(PKV_ERR_INVALID_ARG, "pool_out is NULL");
  *pool_out = nullptr;
  const bool compact = format == PKV_FORMAT_E4M3;
  const uint64_t plb = compact ? compact_code_bytes(geom) : page_layer_bytes(geom);
  const uint64_t pb =
      (compact ? plb + compact_scale_bytes(geom) : plb) * (uint64_t)geom->num_layers;
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
  p->page_layer_bytes = plb;
  p->num_pages = (int64_t)pages;
  p->format = format;
  p->scale_offset = compact ? plb * (uint64_t)geom->num_layers * pages : 0;
  *pool_out = p;
  return ok();
}
}  // namespace

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

PKV_API int pkv_page_table_write_async(const pkv_pool* pool, const int32_t* host_table,
                                       const int32_t* host_ctx_lens, int32_t batch,
                                       int32_t pt_stride, int32_t* dev_table,
                                       int32_t* dev_ctx_lens, void* stream, void* done_event) {
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
  if (e == hipSuccess && done_event) e = hipEventRecord(static_cast<hipEvent_t>(done_event), s);
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

namespace {

// pkv_decode_attention, and with fin_out / fin_lse also the final merge of
// every slot of each row (pkv_decode_attention_merged).  With `stage`,
// table entries past the pool's pages name pages of a staging pool's layer
// (the live pool's composed tables; the MFMA kernel only).
int decode_impl(const pkv_pool* pool, int32_t layer, const void* q, const int32_t* dev_table,
                int32_t pt_stride, const int32_t* dev_ctx_lens, int32_t batch,
                int32_t num_q_heads, int32_t token_begin, int32_t token_count,
                int32_t tile_tokens, float scale, float* part_out, float* part_lse,
                int32_t num_slots, void* workspace, uint64_t workspace_bytes,
                const pkv_decode_opts* opts, void* stream, float* fin_out, float* fin_lse,
                const pkv::StageRef* stage = nullptr, bool dry_run = false) {
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
  const int slot_offset = opts ? opts->slot_offset : 0;
  if (slot_offset < 0) return fail(PKV_ERR_INVALID_ARG, "opts.slot_offset = %d is negative", slot_offset);
  if (pool->format == PKV_FORMAT_E4M3 && kernel != 2)
    return fail(PKV_ERR_INVALID_ARG, "a compact pool is read by the MFMA kernel only (opts.kernel 0 or 2)");
  const int64_t first_slot64 = (int64_t)slot_offset + token_begin / tile_tokens;
  if (first_slot64 > 65535) return fail(PKV_ERR_INVALID_ARG, "first slot %lld exceeds 65535", (long long)first_slot64);
  const int first_slot = (int)first_slot64;
  const int n_tiles = token_count / tile_tokens;
  if (num_slots < 1 || (int64_t)first_slot + n_tiles > num_slots)
    return fail(PKV_ERR_INVALID_ARG, "slots %d..%d of this window exceed num_slots = %d",
                first_slot, first_slot + n_tiles - 1, num_slots);
  if (num_slots > 65535) return fail(PKV_ERR_INVALID_ARG, "num_slots = %d exceeds 65535", num_slots);
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale is not finite");
  const bool merged = fin_out != nullptr || fin_lse != nullptr;
  if (merged && (slot_offset != 0 || n_tiles != num_slots))
    return fail(PKV_ERR_INVALID_ARG,
                "merged decode writes every slot of its rows: token_count / tile_tokens = %d must "
                "equal num_slots = %d and opts.slot_offset (%d) must be 0", n_tiles, num_slots,
                slot_offset);
  if (batch == 0 || token_count == 0) return ok();
  if (!q || !dev_table || !dev_ctx_lens || !part_out || !part_lse)
    return fail(PKV_ERR_INVALID_ARG, "q, dev_table, dev_ctx_lens, part_out or part_lse is NULL");
  if (merged && (!fin_out || !fin_lse)) return fail(PKV_ERR_INVALID_ARG, "out or lse is NULL");
  if (merged && reinterpret_cast<uintptr_t>(fin_out) % 16)
    return fail(PKV_ERR_INVALID_ARG, "out must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(q) % 16 || reinterpret_cast<uintptr_t>(part_out) % 16)
    return fail(PKV_ERR_INVALID_ARG, "q and part_out must be 16-byte aligned");

  int split = 0;
  if (int rc = split_for(tile_tokens, opts, &split)) return rc;
  // the matrix-core kernels hold one page id per lane of a wave: at most 64
  // pages per wave, 4 waves per work-group
  if (kernel == 2 && split > kMaxMfmaSplit)
    return fail(PKV_ERR_INVALID_ARG,
                "opts.split_tokens = %d exceeds %d tokens per work-group of the MFMA and compact "
                "kernels", split, kMaxMfmaSplit);
  uint64_t need = 0;
  if (int rc = pkv_decode_workspace_bytes(batch, num_q_heads, G.head_dim, token_count, tile_tokens,
                                          opts, &need))
    return rc;
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PKV_ERR_WORKSPACE, "workspace of %llu bytes given, %llu needed",
                (unsigned long long)(workspace ? workspace_bytes : 0), (unsigned long long)need);
  if (need > 0 && reinterpret_cast<uintptr_t>(workspace) % 16)
    return fail(PKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

  if (stage && (kernel != 2 || pool->format != PKV_FORMAT_BF16))
    return fail(PKV_ERR_INVALID_ARG, "staged pages are read by the MFMA kernel from bf16 pools");
  if (dry_run) return ok();

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
  a.row_split = nullptr;
  a.scale_log2 = scale * pkv::kLog2e;
  if (stage) {
    a.stage_arena = static_cast<const uint16_t*>(stage->pool->base);
    a.stage_layer_off = (int64_t)(stage->pool->page_layer_bytes / 2) * stage->pool->num_pages *
                        stage->layer;
    a.stage_pages = (int32_t)stage->pool->num_pages;
  }

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
  hipError_t e;
  if (pool->format == PKV_FORMAT_E4M3) {
    pkv::CompactDecodeArgs c;
    c.codes = static_cast<const uint8_t*>(pool->base);
    c.scales = reinterpret_cast<const float*>(static_cast<const char*>(pool->base) + pool->scale_offset);
    c.page_bytes = (int64_t)pool->page_layer_bytes;
    c.layer_off = (int64_t)pool->page_layer_bytes * pool->num_pages * layer;
    c.scale_layer_off = (int64_t)2 * G.num_kv_heads * pool->num_pages * layer;
    c.num_pages = a.num_pages;
    c.num_kv_heads = a.num_kv_heads;
    c.q = a.q;
    c.table = a.table;
    c.pt_stride = a.pt_stride;
    c.ctx_lens = a.ctx_lens;
    c.num_q_heads = a.num_q_heads;
    c.token_begin = a.token_begin;
    c.token_count = a.token_count;
    c.split_tokens = a.split_tokens;
    c.scale_log2 = a.scale_log2;
    c.out_o = a.out_o;
    c.out_lse = a.out_lse;
    c.out_slots = a.out_slots;
    c.out_slot0 = a.out_slot0;
    e = pkv::launch_decode_fp8(c, batch, group, s);
  } else {
    e = (kernel == 1) ? pkv::launch_decode_valu(a, batch, group, s)
                      : pkv::launch_decode_mfma(a, batch, group, s);
  }
  if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "decode launch failed: %s", hipGetErrorString(e));
  const int rows = batch * num_q_heads;
  bool final_done = false;
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
    if (merged && n_split <= kMaxMerge2Splits) {   // finalize and final merge in one launch
      e = pkv::launch_merge2(m, rows, fin_out, fin_lse, s);
      final_done = true;
    } else {
      e = pkv::launch_merge(m, rows, s);
    }
    if (e != hipSuccess)
      return fail(PKV_ERR_LAUNCH, "tile finalize launch failed: %s", hipGetErrorString(e));
  }
  if (merged && !final_done) {
    pkv::MergeArgs m;
    m.in_o = part_out;
    m.in_lse = part_lse;
    m.in_slots = num_slots;
    m.group = num_slots;
    m.out_o = fin_out;
    m.out_lse = fin_lse;
    m.out_slots = 1;
    m.out_slot0 = 0;
    m.n_out = 1;
    e = pkv::launch_merge(m, rows, s);
    if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "merge launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

namespace pkv {
int decode_merged_staged(const pkv_pool* pool, int32_t layer, const void* q,
                         const int32_t* dev_table, int32_t pt_stride, const int32_t* dev_ctx_lens,
                         int32_t batch, int32_t num_q_heads, int32_t token_count,
                         int32_t tile_tokens, float scale, float* part_out, float* part_lse,
                         int32_t num_slots, float* out, float* lse, void* workspace,
                         uint64_t workspace_bytes, const pkv_decode_opts* opts, void* stream,
                         const StageRef& stage, bool dry_run) {
  if (!out || !lse) return fail(PKV_ERR_INVALID_ARG, "out or lse is NULL");
  return decode_impl(pool, layer, q, dev_table, pt_stride, dev_ctx_lens, batch, num_q_heads, 0,
                     token_count, tile_tokens, scale, part_out, part_lse, num_slots, workspace,
                     workspace_bytes, opts, stream, out, lse, &stage, dry_run);
}
}  // namespace pkv

PKV_API int pkv_decode_attention(const pkv_pool* pool, int32_t layer, const void* q,
                                 const int32_t* dev_table, int32_t pt_stride,
                                 const int32_t* dev_ctx_lens, int32_t batch, int32_t num_q_heads,
                                 int32_t token_begin, int32_t token_count, int32_t tile_tokens,
                                 float scale, float* part_out, float* part_lse, int32_t num_slots,
                                 void* workspace, uint64_t workspace_bytes,
                                 const pkv_decode_opts* opts, void* stream) {
  return decode_impl(pool, layer, q, dev_table, pt_stride, dev_ctx_lens, batch, num_q_heads,
                     token_begin, token_count, tile_tokens, scale, part_out, part_lse, num_slots,
                     workspace, workspace_bytes, opts, stream, nullptr, nullptr);
}

PKV_API int pkv_decode_attention_merged(const pkv_pool* pool, int32_t layer, const void* q,
                                        const int32_t* dev_table, int32_t pt_stride,
                                        const int32_t* dev_ctx_lens, int32_t batch,
                                        int32_t num_q_heads, int32_t token_count,
                                        int32_t tile_tokens, float scale, float* part_out,
                                        float* part_lse, int32_t num_slots, float* out, float* lse,
                                        void* workspace, uint64_t workspace_bytes,
                                        const pkv_decode_opts* opts, void* stream) {
  if (!out || !lse) return fail(PKV_ERR_INVALID_ARG, "out or lse is NULL");
  return decode_impl(pool, layer, q, dev_table, pt_stride, dev_ctx_lens, batch, num_q_heads, 0,
                     token_count, tile_tokens, scale, part_out, part_lse, num_slots, workspace,
                     workspace_bytes, opts, stream, out, lse);
}

// Device scratch for pkv_decode_attention_merged_noalloc: a file-scope
// array, one copy per GPU the library runs on, held until the process ends.
// Host code never uses the array's name as an address (on the host it is a
// stand-in, not a device pointer): each device's address is looked up once
// with hipGetSymbolAddress, with that device current, and kept.
static __device__ __align__(256) unsigned char scratch[PKV_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's scratch address (the current device's), or an error code.
int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_ERR_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PKV_ERR_DEVICE, "device %d: the static scratch serves devices 0..%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PKV_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}
}  // namespace

PKV_API int pkv_decode_attention_merged_noalloc(const pkv_pool* pool, int32_t layer,
                                                const void* q, const int32_t* dev_table,
                                                int32_t pt_stride, const int32_t* dev_ctx_lens,
                                                int32_t batch, int32_t num_q_heads,
                                                int32_t token_count, int32_t tile_tokens,
                                                float scale, float* part_out, float* part_lse,
                                                int32_t num_slots, float* out, float* lse,
                                                const pkv_decode_opts* opts, void* stream) {
  if (!out || !lse) return fail(PKV_ERR_INVALID_ARG, "out or lse is NULL");
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  uint64_t need = 0;
  if (int rc = pkv_decode_workspace_bytes(batch, num_q_heads, pool->geom.head_dim, token_count,
                                          tile_tokens, opts, &need))
    return rc;
  if (need > PKV_STATIC_SCRATCH_BYTES)
    return fail(PKV_ERR_WORKSPACE,
                "this call needs %llu bytes of split partials; the static scratch holds %llu "
                "(PKV_STATIC_SCRATCH_BYTES): use pkv_decode_attention_merged with a workspace, "
                "or fewer splits per tile (opts.split_tokens = tile_tokens needs none)",
                (unsigned long long)need, (unsigned long long)PKV_STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0)
    if (int rc = scratch_for_current_device(&ws)) return rc;
  return decode_impl(pool, layer, q, dev_table, pt_stride, dev_ctx_lens, batch, num_q_heads, 0,
                     token_count, tile_tokens, scale, part_out, part_lse, num_slots, ws,
                     need > 0 ? (uint64_t)PKV_STATIC_SCRATCH_BYTES : 0, opts, stream, out, lse);
}

namespace pkv {
// pkv_decode_attention_runs with a layer of its own per run and, for an exact
// run, a staging pool whose pages its table may name (the live pool's
// composed table); with dry_run only the checks run.
int runs_impl(const RunSpec* runs, int32_t n_runs, const void* q, int32_t batch,
              int32_t num_q_heads, float scale, float* part_out, float* part_lse,
              int32_t num_slots, void* stream, bool dry_run) {
  if (n_runs < 1 || n_runs > 2) return fail(PKV_ERR_INVALID_ARG, "n_runs = %d, need 1 or 2", n_runs);
  if (!runs) return fail(PKV_ERR_INVALID_ARG, "runs is NULL");
  if (batch < 0 || batch > 65535) return fail(PKV_ERR_INVALID_ARG, "batch = %d outside 0..65535", batch);
  if (num_slots < 1 || num_slots > 65535)
    return fail(PKV_ERR_INVALID_ARG, "num_slots = %d outside 1..65535", num_slots);
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale is not finite");
  pkv::RunsArgs r;
  std::memset(&r, 0, sizeof(r));
  r.n_runs = n_runs;
  r.batch = batch;
  int group = 0;
  int lo[2] = {0, 0}, hi[2] = {0, 0};          // slots [lo, hi) of each run
  for (int k = 0; k < n_runs; ++k) {
    const RunSpec& u = runs[k];
    if (!u.pool) return fail(PKV_ERR_INVALID_ARG, "runs[%d].pool is NULL", k);
    const pkv_pool* pool = u.pool;
    const pkv_geom& G = pool->geom;
    const int32_t layer = u.layer;
    if (layer < 0 || layer >= G.num_layers)
      return fail(PKV_ERR_INVALID_ARG, "layer = %d outside 0..%d of runs[%d].pool", layer,
                  G.num_layers - 1, k);
    if (k == 0) {
      r.num_kv_heads = G.num_kv_heads;
      if (num_q_heads < 1 || num_q_heads % G.num_kv_heads)
        return fail(PKV_ERR_GEOMETRY,
                    "num_q_heads = %d must be a positive multiple of num_kv_heads = %d",
                    num_q_heads, G.num_kv_heads);
      group = num_q_heads / G.num_kv_heads;
      int kernel = 0;
      if (int rc = kernel_for(nullptr, group, &kernel)) return rc;
    } else if (G.num_kv_heads != r.num_kv_heads) {
      return fail(PKV_ERR_GEOMETRY, "runs[1].pool has %d KV heads, runs[0].pool %d",
                  G.num_kv_heads, r.num_kv_heads);
    }
    if (u.tile_tokens < G.page_tokens || u.tile_tokens > kMaxMfmaSplit ||
        u.tile_tokens % G.page_tokens)
      return fail(PKV_ERR_INVALID_ARG, "runs[%d].tile_tokens = %d must be a multiple of %d in %d..%d",
                  k, u.tile_tokens, G.page_tokens, G.page_tokens, kMaxMfmaSplit);
    if (u.token_count < 0 || u.token_count % u.tile_tokens)
      return fail(PKV_ERR_INVALID_ARG,
                  "runs[%d].token_count = %d must be a non-negative multiple of its tile_tokens",
                  k, u.token_count);
    if ((int64_t)u.pt_stride * G.page_tokens < u.token_count)
      return fail(PKV_ERR_INVALID_ARG, "runs[%d].pt_stride = %d covers less than token_count = %d",
                  k, u.pt_stride, u.token_count);
    const int n_tiles = u.token_count / u.tile_tokens;
    if (u.slot_offset < 0 || (int64_t)u.slot_offset + n_tiles > num_slots)
      return fail(PKV_ERR_INVALID_ARG, "runs[%d] slots %d..%d exceed num_slots = %d", k,
                  u.slot_offset, u.slot_offset + n_tiles - 1, num_slots);
    lo[k] = u.slot_offset;
    hi[k] = u.slot_offset + n_tiles;
    if (batch > 0 && n_tiles > 0 && (!u.dev_table || !u.dev_ctx_lens))
      return fail(PKV_ERR_INVALID_ARG, "runs[%d].dev_table or dev_ctx_lens is NULL", k);
    const int64_t wgs = (int64_t)n_tiles * G.num_kv_heads * batch;
    if (wgs > INT32_MAX / 2)
      return fail(PKV_ERR_INVALID_ARG, "runs[%d] holds %lld work-groups, more than %d", k,
                  (long long)wgs, INT32_MAX / 2);
    r.compact[k] = pool->format == PKV_FORMAT_E4M3;
    if (u.stage && (r.compact[k] || u.stage->pool->format != PKV_FORMAT_BF16))
      return fail(PKV_ERR_INVALID_ARG, "runs[%d]: staged pages are bf16 pages of an exact run", k);
    r.n_split[k] = n_tiles;
    r.wgs[k] = (int32_t)wgs;
    pkv::DecodeArgs& a = r.e[k];
    a.arena = static_cast<const uint16_t*>(pool->base);
    a.page_elems = (int64_t)(pool->page_layer_bytes / 2);
    a.layer_off = (int64_t)(pool->page_layer_bytes / 2) * pool->num_pages * layer;
    a.num_pages = (int32_t)pool->num_pages;
    a.num_kv_heads = G.num_kv_heads;
    a.q = static_cast<const uint16_t*>(q);
    a.table = u.dev_table;
    a.pt_stride = u.pt_stride;
    a.ctx_lens = u.dev_ctx_lens;
    a.num_q_heads = num_q_heads;
    a.token_begin = 0;
    a.token_count = u.token_count;
    a.split_tokens = u.tile_tokens;
    a.row_split = nullptr;
    a.scale_log2 = scale * pkv::kLog2e;
    a.out_o = part_out;
    a.out_lse = part_lse;
    a.out_slots = num_slots;
    a.out_slot0 = u.slot_offset;
    if (u.stage) {
      a.stage_arena = static_cast<const uint16_t*>(u.stage->pool->base);
      a.stage_layer_off = (int64_t)(u.stage->pool->page_layer_bytes / 2) *
                          u.stage->pool->num_pages * u.stage->layer;
      a.stage_pages = (int32_t)u.stage->pool->num_pages;
    }
    if (r.compact[k]) {
      pkv::CompactDecodeArgs& c = r.c[k];
      c.codes = static_cast<const uint8_t*>(pool->base);
      c.scales = reinterpret_cast<const float*>(static_cast<const char*>(pool->base) +
                                                pool->scale_offset);
      c.page_bytes = (int64_t)pool->page_layer_bytes;
      c.layer_off = (int64_t)pool->page_layer_bytes * pool->num_pages * layer;
      c.scale_layer_off = (int64_t)2 * G.num_kv_heads * pool->num_pages * layer;
      c.num_pages = a.num_pages;
      c.num_kv_heads = a.num_kv_heads;
      c.q = a.q;
      c.table = a.table;
      c.pt_stride = a.pt_stride;
      c.ctx_lens = a.ctx_lens;
      c.num_q_heads = a.num_q_heads;
      c.token_begin = 0;
      c.token_count = a.token_count;
      c.split_tokens = a.split_tokens;
      c.scale_log2 = a.scale_log2;
      c.out_o = part_out;
      c.out_lse = part_lse;
      c.out_slots = num_slots;
      c.out_slot0 = a.out_slot0;
    }
  }
  if (n_runs == 2 && lo[0] < hi[1] && lo[1] < hi[0])
    return fail(PKV_ERR_INVALID_ARG, "the runs' slots %d..%d and %d..%d overlap", lo[0], hi[0] - 1,
                lo[1], hi[1] - 1);
  if (batch == 0 || r.wgs[0] + (n_runs > 1 ? r.wgs[1] : 0) == 0) return ok();
  if (!q || !part_out || !part_lse)
    return fail(PKV_ERR_INVALID_ARG, "q, part_out or part_lse is NULL");
  if (reinterpret_cast<uintptr_t>(q) % 16 || reinterpret_cast<uintptr_t>(part_out) % 16)
    return fail(PKV_ERR_INVALID_ARG, "q and part_out must be 16-byte aligned");
  if (dry_run) return ok();
  hipError_t e = pkv::launch_decode_runs(r, group, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "decode launch failed: %s", hipGetErrorString(e));
  return ok();
}
}  // namespace pkv

PKV_API int pkv_decode_attention_runs(int32_t layer, const void* q, int32_t batch,
                                      int32_t num_q_heads, const pkv_decode_run* runs,
                                      int32_t n_runs, float scale, float* part_out,
                                      float* part_lse, int32_t num_slots, void* stream) {
  if (n_runs < 1 || n_runs > 2) return fail(PKV_ERR_INVALID_ARG, "n_runs = %d, need 1 or 2", n_runs);
  if (!runs) return fail(PKV_ERR_INVALID_ARG, "runs is NULL");
  pkv::RunSpec spec[2];
  for (int k = 0; k < n_runs; ++k)
    spec[k] = {runs[k].pool, layer, runs[k].dev_table, runs[k].pt_stride, runs[k].dev_ctx_lens,
               runs[k].token_count, runs[k].tile_tokens, runs[k].slot_offset, nullptr};
  return pkv::runs_impl(spec, n_runs, q, batch, num_q_heads, scale, part_out, part_lse, num_slots,
                        stream, false);
}

PKV_API int pkv_plan_tiles(const int32_t* host_ctx_lens, int32_t batch, int32_t num_kv_heads,
                           int32_t work_groups, int32_t max_tile_tokens,
                           int32_t* host_row_tile_tokens, int32_t* max_tiles_out) {
  if (batch < 0 || batch > 65535) return fail(PKV_ERR_INVALID_ARG, "batch = %d outside 0..65535", batch);
  if (num_kv_heads < 1) return fail(PKV_ERR_INVALID_ARG, "num_kv_heads = %d, need >= 1", num_kv_heads);
  if (work_groups < 1) return fail(PKV_ERR_INVALID_ARG, "work_groups = %d, need >= 1", work_groups);
  if (max_tile_tokens < pkv::kPageTokens || max_tile_tokens > kMaxMfmaSplit ||
      max_tile_tokens % pkv::kPageTokens)
    return fail(PKV_ERR_INVALID_ARG, "max_tile_tokens = %d must be a multiple of %d in %d..%d",
                max_tile_tokens, pkv::kPageTokens, pkv::kPageTokens, kMaxMfmaSplit);
  if (!max_tiles_out || (batch > 0 && (!host_ctx_lens || !host_row_tile_tokens)))
    return fail(PKV_ERR_INVALID_ARG, "host_ctx_lens, host_row_tile_tokens or max_tiles_out is NULL");
  for (int b = 0; b < batch; ++b)
    if (host_ctx_lens[b] < 0) return fail(PKV_ERR_INVALID_ARG, "ctx_lens[%d] = %d is negative", b, host_ctx_lens[b]);
  const int PT = pkv::kPageTokens;
  // work-groups with every split at most tau tokens
  auto groups = [&](int64_t tau) {
    int64_t n = 0;
    for (int b = 0; b < batch; ++b) n += (host_ctx_lens[b] + tau - 1) / tau;
    return n * num_kv_heads;
  };
  // smallest multiple of 64 (up to the maximum) whose split count fits
  int lo = 1, hi = max_tile_tokens / PT;
  while (lo < hi) {
    const int mid = lo + (hi - lo) / 2;
    if (groups((int64_t)mid * PT) <= work_groups) hi = mid;
    else lo = mid + 1;
  }
  const int64_t tau = (int64_t)lo * PT;
  int max_tiles = 1;
  for (int b = 0; b < batch; ++b) {
    const int64_t c = host_ctx_lens[b];
    const int64_t n = (c + tau - 1) / tau;                    // splits of this request
    const int64_t even = n > 0 ? (c + n - 1) / n : PT;         // equal shares of its tokens
    host_row_tile_tokens[b] = (int32_t)((even + PT - 1) / PT * PT);
    if (n > max_tiles) max_tiles = (int)n;
  }
  *max_tiles_out = max_tiles;
  return ok();
}

PKV_API int pkv_decode_attention_rows(const pkv_pool* pool, int32_t layer, const void* q,
                                      const int32_t* dev_table, int32_t pt_stride,
                                      const int32_t* dev_ctx_lens, int32_t batch,
                                      int32_t num_q_heads, const int32_t* dev_row_tile_tokens,
                                      int32_t max_row_tile_tokens, int32_t max_tiles, float scale,
                                      float* part_out, float* part_lse, int32_t num_slots,
                                      const pkv_decode_opts* opts, void* stream) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  const pkv_geom& G = pool->geom;
  if (layer < 0 || layer >= G.num_layers)
    return fail(PKV_ERR_INVALID_ARG, "layer = %d outside 0..%d", layer, G.num_layers - 1);
  if (batch < 0 || batch > 65535) return fail(PKV_ERR_INVALID_ARG, "batch = %d outside 0..65535", batch);
  if (num_q_heads < 1 || num_q_heads % G.num_kv_heads)
    return fail(PKV_ERR_GEOMETRY, "num_q_heads = %d must be a positive multiple of num_kv_heads = %d",
                num_q_heads, G.num_kv_heads);
  const int group = num_q_heads / G.num_kv_heads;
  int kernel = 0;
  if (int rc = kernel_for(opts, group, &kernel)) return rc;
  if (kernel != 2 || pool->format != PKV_FORMAT_BF16)
    return fail(PKV_ERR_INVALID_ARG, "per-request tiles are decoded by the MFMA kernel from bf16 pools only");
  if (opts && opts->split_tokens != 0)
    return fail(PKV_ERR_INVALID_ARG, "opts.split_tokens = %d: per-request tiles are their own splits",
                opts->split_tokens);
  if (max_row_tile_tokens < G.page_tokens || max_row_tile_tokens > kMaxMfmaSplit ||
      max_row_tile_tokens % G.page_tokens)
    return fail(PKV_ERR_INVALID_ARG, "max_row_tile_tokens = %d must be a multiple of %d in %d..%d",
                max_row_tile_tokens, G.page_tokens, G.page_tokens, kMaxMfmaSplit);
  if (max_tiles < 1 || max_tiles > 65535)
    return fail(PKV_ERR_INVALID_ARG, "max_tiles = %d outside 1..65535", max_tiles);
  const int64_t span = (int64_t)max_tiles * max_row_tile_tokens;
  if (span > INT32_MAX) return fail(PKV_ERR_INVALID_ARG, "max_tiles x max_row_tile_tokens overflows int32");
  if ((int64_t)pt_stride * G.page_tokens < span)
    return fail(PKV_ERR_INVALID_ARG, "pt_stride = %d covers %lld tokens, less than max_tiles x "
                "max_row_tile_tokens = %lld", pt_stride, (long long)pt_stride * G.page_tokens,
                (long long)span);
  const int slot_offset = opts ? opts->slot_offset : 0;
  if (slot_offset < 0) return fail(PKV_ERR_INVALID_ARG, "opts.slot_offset = %d is negative", slot_offset);
  if (num_slots < 1 || num_slots > 65535 || (int64_t)slot_offset + max_tiles > num_slots)
    return fail(PKV_ERR_INVALID_ARG, "slots %d..%d exceed num_slots = %d", slot_offset,
                slot_offset + max_tiles - 1, num_slots);
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale is not finite");
  if (batch == 0) return ok();
  if (!q || !dev_table || !dev_ctx_lens || !dev_row_tile_tokens || !part_out || !part_lse)
    return fail(PKV_ERR_INVALID_ARG,
                "q, dev_table, dev_ctx_lens, dev_row_tile_tokens, part_out or part_lse is NULL");
  if (reinterpret_cast<uintptr_t>(q) % 16 || reinterpret_cast<uintptr_t>(part_out) % 16)
    return fail(PKV_ERR_INVALID_ARG, "q and part_out must be 16-byte aligned");

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
  a.token_begin = 0;                   // the window: every row's max_tiles splits
  a.token_count = (int32_t)span;
  a.split_tokens = max_row_tile_tokens;   // sets the grid row: token_count / split_tokens
  a.row_split = dev_row_tile_tokens;
  a.scale_log2 = scale * pkv::kLog2e;
  a.out_o = part_out;
  a.out_lse = part_lse;
  a.out_slots = num_slots;
  a.out_slot0 = slot_offset;
  hipError_t e = pkv::launch_decode_mfma(a, batch, group, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "decode launch failed: %s", hipGetErrorString(e));
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
  if (pool->format != PKV_FORMAT_BF16)
    return fail(PKV_ERR_INVALID_ARG, "compact pages are immutable: append to the exact pool");
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

PKV_API int pkv_compact_convert(const pkv_pool* exact, const pkv_pool* compact,
                                const int32_t* dev_src_pages, const int32_t* dev_dst_pages,
                                int32_t n, uint32_t* dev_crc, void* stream) {
  if (!exact || !compact) return fail(PKV_ERR_INVALID_ARG, "exact or compact pool is NULL");
  if (exact->format != PKV_FORMAT_BF16 || compact->format != PKV_FORMAT_E4M3)
    return fail(PKV_ERR_INVALID_ARG, "convert takes an exact (bf16) pool and a compact (E4M3) pool");
  const pkv_geom& a = exact->geom;
  const pkv_geom& b = compact->geom;
  if (a.num_layers != b.num_layers || a.num_kv_heads != b.num_kv_heads ||
      a.head_dim != b.head_dim || a.page_tokens != b.page_tokens)
    return fail(PKV_ERR_GEOMETRY, "the two pools differ in geometry");
  if (n < 0) return fail(PKV_ERR_INVALID_ARG, "n = %d is negative", n);
  if (n == 0) return ok();
  if (!dev_src_pages || !dev_dst_pages || !dev_crc)
    return fail(PKV_ERR_INVALID_ARG, "dev_src_pages, dev_dst_pages or dev_crc is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t i0 = 0; i0 < n; i0 += 65535) {          // grid z is at most 65535
    const int32_t m = std::min<int32_t>(65535, n - i0);
    pkv::ConvertArgs c;
    c.src = static_cast<const uint16_t*>(exact->base);
    c.src_page_elems = (int64_t)(exact->page_layer_bytes / 2);
    c.src_num_pages = exact->num_pages;
    c.codes = static_cast<uint8_t*>(compact->base);
    c.scales = reinterpret_cast<float*>(static_cast<char*>(compact->base) + compact->scale_offset);
    c.dst_page_bytes = (int64_t)compact->page_layer_bytes;
    c.dst_num_pages = compact->num_pages;
    c.num_layers = a.num_layers;
    c.num_kv_heads = a.num_kv_heads;
    c.src_pages = dev_src_pages + i0;
    c.dst_pages = dev_dst_pages + i0;
    c.n = m;
    hipError_t e = pkv::launch_convert(c, s);
    if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "convert launch failed: %s", hipGetErrorString(e));
  }
  return pkv_compact_crc(compact, dev_dst_pages, n, dev_crc, stream);
}

PKV_API int pkv_compact_crc(const pkv_pool* compact, const int32_t* dev_pages, int32_t n,
                            uint32_t* dev_crc, void* stream) {
  if (!compact) return fail(PKV_ERR_INVALID_ARG, "compact pool is NULL");
  if (compact->format != PKV_FORMAT_E4M3) return fail(PKV_ERR_INVALID_ARG, "not a compact pool");
  if (n < 0) return fail(PKV_ERR_INVALID_ARG, "n = %d is negative", n);
  if (n == 0) return ok();
  if (!dev_pages || !dev_crc) return fail(PKV_ERR_INVALID_ARG, "dev_pages or dev_crc is NULL");
  const pkv_geom& G = compact->geom;
  pkv::CrcArgs c;
  c.codes = static_cast<const uint8_t*>(compact->base);
  c.scales = reinterpret_cast<const float*>(static_cast<const char*>(compact->base) +
                                            compact->scale_offset);
  c.page_bytes = (int64_t)compact->page_layer_bytes;
  c.num_pages = compact->num_pages;
  c.num_layers = G.num_layers;
  c.scale_count = 2 * G.num_kv_heads;
  const uint64_t seg = compact->page_layer_bytes / 256;
  for (int k = 0; k < 8; ++k) c.x_seg[k] = x_pow_bytes(seg << k);
  const uint64_t sb = 4ull * (uint64_t)c.scale_count;
  c.x_scales = x_pow_bytes(sb);
  c.x_layer = x_pow_bytes(compact->page_layer_bytes + sb);
  c.init_term = gf_mul(0xFFFFFFFFu, x_pow_bytes((compact->page_layer_bytes + sb) * G.num_layers));
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t i0 = 0; i0 < n; i0 += 1 << 20) {
    const int32_t m = std::min<int32_t>(1 << 20, n - i0);
    c.pages = dev_pages + i0;
    c.crc = dev_crc + i0;
    c.n = m;
    hipError_t e = pkv::launch_crc(c, s);
    if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "crc launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}
