// The live pool: decode steps over histories whose authoritative copy is in
// pinned host memory, with the device pool's pages handed out per step by
// the admission planner (Staging without a stall, sections "Admission that
// does arithmetic", "Two copy queues and device-side ordering" and "Leases
// instead of buffers"; GPU memory management, sections "Pages held by
// right, borrowed or free" and "Staging as a lease").
//
// Per step, on the host: admission decides which logical pages of each
// context hold pool pages (the sink and the newest pages).  Every pool page
// carries a tag naming the (context, logical page) whose bytes it holds; a
// resident page whose tag differs turned hot this step and is copied in
// once.  Every other logical page of the history is staged: given a page of
// the staging pool for this step.  The step's table is composed from both:
// entry i is the pool page of logical page i, or num_pages + s for staging
// page s.  The table, lengths and append positions go to the device through
// a small pinned ring, on the compute stream.
//
// Per layer, on the device, ordered by events only:
//   copy streams     (the caller's and the runtime's own second one, each
//                    taking half of every run of pages) wait for the
//                    previous step's write-back of this layer
//                    (its pool pages and host rows are then settled) and for
//                    the last layer that read this staging buffer; copies in
//                    the hot pages' slices of this layer and the staged pages
//                    into staging buffer layer % K;
//   compute stream   waits for the copies; appends the new token at
//                    length - 1; decodes every tile over the composed table
//                    in one launch and merges (pkv_decode_attention_merged);
//   write-back       waits for the decode; stores the new token's K and V
//                    rows into the host pages (the changed rows only).
// The host waits only when the table ring is full and in destroy.
//
// With compact pages attached (KV-cache engineering, sections "Exact recent
// pages, compact older pages" and "What the hybrid tier buys": a
// representation is worth the bus bytes per token it saves), a
// non-resident page whose compact copy the caller has published is staged
// as E4M3 codes and scales instead of bf16: its entry in the exact table is
// -1 and it joins a compact run of its own (logical order, every page full).
// The layer's decode is then one launch of both runs (the exact run over
// the composed table, the compact run from the compact staging pool) into
// disjoint slots, and one FP32 merge.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <new>
#include <vector>

#include "kernels.h"
#include "pool.h"

#define PKV_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kRing = 4;   // steps of tables in flight before the host waits

int fail(int code, const char* msg) { return pkv::set_error(code, "%s", msg); }

struct PageCopy {            // one page of one layer, host -> device
  int32_t dst;               // pool page, or staging page
  int32_t host;              // host page
};

int64_t tag_of(int32_t ctx, int32_t lp) { return ((int64_t)(uint32_t)ctx << 32) | (uint32_t)lp; }

}  // namespace

struct pkv_live {
  const pkv_pool* pool;
  const pkv_pool* stage;
  pkv_admit* admit = nullptr;
  char* host = nullptr;
  char* host_dev = nullptr;        // the host arena as the device addresses it
  int64_t host_pages = 0;
  int32_t layers = 0;
  int32_t buffers = 0;             // staging buffers (layers of the staging pool)
  int32_t max_batch = 0;
  int32_t pt_stride = 0;
  int32_t* dev_state = nullptr;    // [max_batch][pt_stride] table, [max_batch] lengths, positions
  int32_t* ring = nullptr;         // pinned: kRing slots, each dev_state's contents then dev_cstate's
  hipEvent_t ring_ev[kRing] = {};
  bool ring_used[kRing] = {};
  hipStream_t copy = nullptr, compute = nullptr, writeback = nullptr;
  hipStream_t copy2 = nullptr;          // the runtime's own second copy stream
  hipEvent_t copied = nullptr, copied2 = nullptr, consumed = nullptr;
  std::vector<hipEvent_t> layer_done;   // after the write-back of layer l
  std::vector<char> layer_done_set;
  std::vector<hipEvent_t> buf_done;     // after the write-back of the last layer using buffer k
  std::vector<char> buf_done_set;
  std::vector<int64_t> tag;             // per pool page: (context, logical page) held, or -1
  // the open step
  uint64_t steps = 0;
  bool open = false;
  int32_t n = 0;
  std::vector<char> layer_run;
  int32_t layers_run = 0;
  std::vector<PageCopy> hot;            // pool pages to fill from the host
  std::vector<PageCopy> staged;         // staging pages to fill from the host
  std::vector<pkv::TailRow> tails;      // new token rows to write back
  bool quarantined = false;
  // compact older pages (attached or not)
  const pkv_pool* cstage = nullptr;     // E4M3 staging pool: its layers are the buffers
  int32_t* dev_cstate = nullptr;        // [max_batch][pt_stride] compact table, [max_batch] lengths
  char* chost = nullptr;                // compact host arena: codes [layer][page], then scales
  uint64_t chost_scale_off = 0;
  int32_t ctile = 0;                    // tile tokens of the compact run
  std::vector<char> published;          // per host page: a compact copy exists
  std::vector<PageCopy> cstaged;        // compact staging page <- host page
  std::vector<hipEvent_t> cbuf_done;    // after the write-back of the last layer using it
  std::vector<char> cbuf_done_set;
};

namespace {

int quarantine(pkv_live* L, hipError_t e, const char* what) {
  L->quarantined = true;
  return pkv::set_error(PKV_ERR_DEVICE, "%s failed (%s): live pool quarantined", what,
                        hipGetErrorString(e));
}

// Copies of whole (layer, page) slices; runs of consecutive destination and
// host pages go as one copy, its first half on s0 and the rest on s1 (two
// copy engines, so that one's wait before a layer overlaps the other's
// transfer).
hipError_t copy_pages(const std::vector<PageCopy>& pages, char* dst_slab, const char* host_slab,
                      uint64_t plb, hipStream_t s0, hipStream_t s1) {
  size_t i = 0;
  hipError_t e = hipSuccess;
  while (i < pages.size() && e == hipSuccess) {
    size_t run = 1;
    while (i + run < pages.size() && pages[i + run].dst == pages[i].dst + (int32_t)run &&
           pages[i + run].host == pages[i].host + (int32_t)run)
      ++run;
    const size_t half = (run + 1) / 2;
    e = hipMemcpyAsync(dst_slab + (uint64_t)pages[i].dst * plb,
                       host_slab + (uint64_t)pages[i].host * plb, half * plb,
                       hipMemcpyHostToDevice, s0);
    if (e == hipSuccess && run > half)
      e = hipMemcpyAsync(dst_slab + (uint64_t)(pages[i].dst + (int32_t)half) * plb,
                         host_slab + (uint64_t)(pages[i].host + (int32_t)half) * plb,
                         (run - half) * plb, hipMemcpyHostToDevice, s1);
    i += run;
  }
  return e;
}

void destroy_events(pkv_live* L) {
  for (auto& ev : L->ring_ev) if (ev) (void)hipEventDestroy(ev);
  if (L->copied) (void)hipEventDestroy(L->copied);
  if (L->copied2) (void)hipEventDestroy(L->copied2);
  if (L->consumed) (void)hipEventDestroy(L->consumed);
  for (auto ev : L->layer_done) if (ev) (void)hipEventDestroy(ev);
  for (auto ev : L->buf_done) if (ev) (void)hipEventDestroy(ev);
  for (auto ev : L->cbuf_done) if (ev) (void)hipEventDestroy(ev);
}

}  // namespace

PKV_API int pkv_live_create(const pkv_pool* pool, const pkv_pool* stage, void* host_arena,
                            uint64_t host_bytes, int32_t max_batch, int32_t pt_stride,
                            int32_t* dev_state, void* copy_stream, void* compute_stream,
                            void* writeback_stream, pkv_live** out) {
  if (!out) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!pool || !stage) return fail(PKV_ERR_INVALID_ARG, "pool or stage is NULL");
  if (pool->format != PKV_FORMAT_BF16 || stage->format != PKV_FORMAT_BF16)
    return fail(PKV_ERR_INVALID_ARG, "the live pool and its staging pool hold bf16 pages");
  if (stage->geom.num_kv_heads != pool->geom.num_kv_heads)
    return fail(PKV_ERR_GEOMETRY, "the staging pool's KV heads differ from the pool's");
  if ((int64_t)pool->num_pages + stage->num_pages > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARG, "pool + staging pages exceed int32 page ids");
  if (!host_arena || !dev_state) return fail(PKV_ERR_INVALID_ARG, "host_arena or dev_state is NULL");
  const uint64_t plb = pool->page_layer_bytes;
  const uint64_t hpb = plb * (uint64_t)pool->geom.num_layers;
  if (host_bytes == 0 || host_bytes % hpb)
    return pkv::set_error(PKV_ERR_INVALID_ARG,
                          "host_bytes = %llu must be a positive whole number of %llu-byte pages",
                          (unsigned long long)host_bytes, (unsigned long long)hpb);
  if (host_bytes / hpb > (uint64_t)INT32_MAX) return fail(PKV_ERR_INVALID_ARG, "too many host pages");
  if (max_batch < 1 || max_batch > 65535) return fail(PKV_ERR_INVALID_ARG, "max_batch outside 1..65535");
  if (pt_stride < 1) return fail(PKV_ERR_INVALID_ARG, "pt_stride must be >= 1");
  pkv_live* L = new (std::nothrow) pkv_live;
  if (!L) return fail(PKV_ERR_INVALID_ARG, "host allocation failed");
  L->pool = pool;
  L->stage = stage;
  L->host = static_cast<char*>(host_arena);
  L->host_pages = (int64_t)(host_bytes / hpb);
  L->layers = pool->geom.num_layers;
  L->buffers = stage->geom.num_layers;
  L->max_batch = max_batch;
  L->pt_stride = pt_stride;
  L->dev_state = dev_state;
  L->copy = static_cast<hipStream_t>(copy_stream);
  L->compute = static_cast<hipStream_t>(compute_stream);
  L->writeback = static_cast<hipStream_t>(writeback_stream);
  L->layer_done.assign((size_t)L->layers, nullptr);
  L->layer_done_set.assign((size_t)L->layers, 0);
  L->buf_done.assign((size_t)L->buffers, nullptr);
  L->buf_done_set.assign((size_t)L->buffers, 0);
  L->layer_run.assign((size_t)L->layers, 0);
  L->tag.assign((size_t)pool->num_pages, -1);
  int rc = pkv_admit_create(pool->num_pages, pool->geom.page_tokens, &L->admit);
  if (rc != PKV_OK) {
    delete L;
    return rc;
  }
  void* dev = nullptr;
  hipError_t e = hipHostGetDevicePointer(&dev, host_arena, 0);
  L->host_dev = static_cast<char*>(dev);
  // each ring slot: the dev_state image, then the compact run's table and lengths
  const size_t slot = (size_t)max_batch * (size_t)(2 * pt_stride + 3);
  if (e == hipSuccess)
    e = hipHostMalloc(reinterpret_cast<void**>(&L->ring), sizeof(int32_t) * slot * kRing,
                      hipHostMallocDefault);
  for (auto& ev : L->ring_ev)
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&L->copied, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&L->copied2, hipEventDisableTiming);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&L->copy2, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&L->consumed, hipEventDisableTiming);
  for (auto& ev : L->layer_done)
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
  for (auto& ev : L->buf_done)
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
  if (e != hipSuccess) {
    destroy_events(L);
    if (L->copy2) (void)hipStreamDestroy(L->copy2);
    if (L->ring) (void)hipHostFree(L->ring);
    pkv_admit_destroy(L->admit);
    delete L;
    return pkv::set_error(PKV_ERR_DEVICE,
                          "live pool setup failed: %s (host_arena must be pinned host memory the "
                          "device can address)", hipGetErrorString(e));
  }
  *out = L;
  pkv::clear_error();
  return PKV_OK;
}

PKV_API int pkv_live_add(pkv_live* L, int32_t ctx, int32_t target_pages, int32_t burst_pages) {
  if (!L) return fail(PKV_ERR_INVALID_ARG, "live pool is NULL");
  return pkv_admit_add(L->admit, ctx, target_pages, burst_pages);
}

PKV_API int pkv_live_set_target(pkv_live* L, int32_t ctx, int32_t target_pages,
                                int32_t burst_pages) {
  if (!L) return fail(PKV_ERR_INVALID_ARG, "live pool is NULL");
  return pkv_admit_set_target(L->admit, ctx, target_pages, burst_pages);
}

PKV_API int pkv_live_remove(pkv_live* L, int32_t ctx) {
  if (!L) return fail(PKV_ERR_INVALID_ARG, "live pool is NULL");
  if (L->open) return fail(PKV_ERR_LEASE, "a step is open: run its layers before removing a context");
  const int rc = pkv_admit_remove(L->admit, ctx);
  if (rc != PKV_OK) return rc;
  // its pages keep their bytes, but no later context of the same id may
  // take them for its own
  for (auto& t : L->tag)
    if (t >= 0 && (int32_t)(t >> 32) == ctx) t = -1;
  return PKV_OK;
}

PKV_API int pkv_live_admission(pkv_live* L, pkv_admit** out) {
  if (!L || !out) return fail(PKV_ERR_INVALID_ARG, "live pool or out is NULL");
  *out = L->admit;
  pkv::clear_error();
  return PKV_OK;
}

PKV_API int pkv_live_attach_compact(pkv_live* L, const pkv_pool* cstage, void* compact_host,
                                    uint64_t compact_host_bytes, int32_t compact_tile_tokens,
                                    int32_t* dev_cstate) {
  if (!L || !cstage || !compact_host || !dev_cstate)
    return fail(PKV_ERR_INVALID_ARG, "live pool, cstage, compact_host or dev_cstate is NULL");
  if (L->cstage) return fail(PKV_ERR_INVALID_ARG, "compact pages are already attached");
  if (L->open) return fail(PKV_ERR_LEASE, "a step is open: attach between steps");
  if (cstage->format != PKV_FORMAT_E4M3)
    return fail(PKV_ERR_INVALID_ARG, "cstage must be a compact (E4M3) pool");
  if (cstage->geom.num_kv_heads != L->pool->geom.num_kv_heads)
    return fail(PKV_ERR_GEOMETRY, "the compact staging pool's KV heads differ from the pool's");
  const uint64_t cplb = cstage->page_layer_bytes;                  // codes of one (layer, page)
  const uint64_t csb = 2ull * (uint64_t)cstage->geom.num_kv_heads * 4ull;
  const uint64_t want = (cplb + csb) * (uint64_t)L->layers * (uint64_t)L->host_pages;
  if (compact_host_bytes != want)
    return pkv::set_error(PKV_ERR_INVALID_ARG,
                          "compact_host_bytes = %llu; the compact copy of %lld host pages of %d "
                          "layers takes %llu", (unsigned long long)compact_host_bytes,
                          (long long)L->host_pages, L->layers, (unsigned long long)want);
  const int PT = L->pool->geom.page_tokens;
  if (compact_tile_tokens < PT || compact_tile_tokens > 64 * 4 * PT || compact_tile_tokens % PT ||
      ((int64_t)L->pt_stride * PT) % compact_tile_tokens)
    return fail(PKV_ERR_INVALID_ARG, "compact_tile_tokens must be a multiple of 64 in 64..16384 "
                "that divides pt_stride x 64");
  if ((int64_t)L->pool->num_pages + cstage->num_pages > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARG, "too many pages");
  L->cbuf_done.assign((size_t)cstage->geom.num_layers, nullptr);
  L->cbuf_done_set.assign((size_t)cstage->geom.num_layers, 0);
  hipError_t e = hipSuccess;
  for (auto& ev : L->cbuf_done)
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
  if (e != hipSuccess) {
    for (auto& ev : L->cbuf_done) if (ev) (void)hipEventDestroy(ev);
    L->cbuf_done.clear();
    return pkv::set_error(PKV_ERR_DEVICE, "attach failed: %s", hipGetErrorString(e));
  }
  L->cstage = cstage;
  L->dev_cstate = dev_cstate;
  L->chost = static_cast<char*>(compact_host);
  L->chost_scale_off = cplb * (uint64_t)L->layers * (uint64_t)L->host_pages;
  L->ctile = compact_tile_tokens;
  L->published.assign((size_t)L->host_pages, 0);
  pkv::clear_error();
  return PKV_OK;
}

namespace {
int set_published(pkv_live* L, const int32_t* host_pages, int32_t n, char value) {
  if (!L) return fail(PKV_ERR_INVALID_ARG, "live pool is NULL");
  if (!L->cstage) return fail(PKV_ERR_INVALID_ARG, "no compact pages are attached");
  if (n < 0 || (n > 0 && !host_pages)) return fail(PKV_ERR_INVALID_ARG, "bad host page list");
  for (int32_t i = 0; i < n; ++i)
    if (host_pages[i] < 0 || host_pages[i] >= L->host_pages)
      return pkv::set_error(PKV_ERR_INVALID_ARG, "host_pages[%d] = %d is not a host page", i,
                            host_pages[i]);
  for (int32_t i = 0; i < n; ++i) L->published[(size_t)host_pages[i]] = value;
  pkv::clear_error();
  return PKV_OK;
}
}  // namespace

PKV_API int pkv_live_publish(pkv_live* L, const int32_t* host_pages, int32_t n) {
  return set_published(L, host_pages, n, 1);
}

PKV_API int pkv_live_retract(pkv_live* L, const int32_t* host_pages, int32_t n) {
  return set_published(L, host_pages, n, 0);
}

PKV_API int pkv_live_step_begin(pkv_live* L, int32_t n, const int32_t* ctx_ids,
                                const int64_t* lengths, const int32_t* host_rows,
                                int32_t host_stride, int32_t* status, pkv_live_info* info) {
  if (!L) return fail(PKV_ERR_INVALID_ARG, "live pool is NULL");
  if (L->quarantined) return fail(PKV_ERR_QUARANTINED, "live pool is quarantined; destroy it");
  if (L->open)
    return pkv::set_error(PKV_ERR_LEASE, "step %llu has run %d of %d layers; every layer runs "
                          "once per step before the next step begins",
                          (unsigned long long)L->steps, L->layers_run, L->layers);
  if (n < 1 || n > L->max_batch) return fail(PKV_ERR_INVALID_ARG, "n outside 1..max_batch");
  if (!ctx_ids || !lengths || !host_rows || !status)
    return fail(PKV_ERR_INVALID_ARG, "ctx_ids, lengths, host_rows or status is NULL");
  if (host_stride < 1) return fail(PKV_ERR_INVALID_ARG, "host_stride must be >= 1");
  const int PT = L->pool->geom.page_tokens;
  for (int32_t i = 0; i < n; ++i) {
    if (lengths[i] < 1 || lengths[i] > (int64_t)L->pt_stride * PT ||
        lengths[i] > (int64_t)host_stride * PT)
      return pkv::set_error(PKV_ERR_INVALID_ARG, "lengths[%d] = %lld outside 1..%lld", i,
                            (long long)lengths[i],
                            (long long)std::min(L->pt_stride, host_stride) * PT);
    const int64_t need = (lengths[i] + PT - 1) / PT;
    for (int64_t lp = 0; lp < need; ++lp) {
      const int32_t hp = host_rows[(int64_t)i * host_stride + lp];
      if (hp < 0 || hp >= L->host_pages)
        return pkv::set_error(PKV_ERR_PAGE_TABLE, "host_rows[%d][%lld] = %d is not a host page "
                              "(0..%lld)", i, (long long)lp, hp, (long long)(L->host_pages - 1));
    }
  }
  // the ring slot for this step's table: wait only if the GPU is kRing steps behind
  const int k = (int)(L->steps % kRing);
  if (L->ring_used[k]) {
    const hipError_t e = hipEventSynchronize(L->ring_ev[k]);
    if (e != hipSuccess) return quarantine(L, e, "wait for the table ring");
  }
  std::vector<int32_t> rows((size_t)n * L->pt_stride);
  int rc = pkv_admit_step(L->admit, n, ctx_ids, lengths, rows.data(), L->pt_stride, status);
  if (rc != PKV_OK) return rc;
  // compose the step's table; hot pages and staged pages
  const int32_t P = (int32_t)L->pool->num_pages;
  const size_t slot = (size_t)L->max_batch * (size_t)(2 * L->pt_stride + 3);
  const size_t state = (size_t)L->max_batch * (size_t)(L->pt_stride + 2);
  int32_t* tab = L->ring + slot * (size_t)k;
  int32_t* lens = tab + (size_t)L->max_batch * L->pt_stride;
  int32_t* pos = lens + L->max_batch;
  int32_t* ctab = pos + L->max_batch;                    // the compact run's rows
  int32_t* clens = ctab + (size_t)L->max_batch * L->pt_stride;
  std::fill(ctab, ctab + (size_t)L->max_batch * L->pt_stride, -1);
  std::fill(clens, clens + L->max_batch, 0);
  L->hot.clear();
  L->staged.clear();
  L->cstaged.clear();
  L->tails.clear();
  int32_t refused = 0, resident = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t* out = tab + (size_t)i * L->pt_stride;
    const int32_t* arow = rows.data() + (size_t)i * L->pt_stride;
    const int32_t* hrow = host_rows + (int64_t)i * host_stride;
    std::fill(out, out + L->pt_stride, -1);
    if (status[i] == PKV_ADMIT_REFUSED_STEP) {
      lens[i] = 0;
      pos[i] = -1;
      ++refused;
      continue;
    }
    const int32_t need = (int32_t)((lengths[i] + PT - 1) / PT);
    int32_t nc = 0;
    for (int32_t lp = 0; lp < need; ++lp) {
      const int32_t d = arow[lp];
      const bool full = (int64_t)(lp + 1) * PT <= lengths[i];
      if (d < 0 && L->cstage && full && L->published[(size_t)hrow[lp]]) {   // staged compact
        const int32_t c = (int32_t)L->cstaged.size();
        if (c >= L->cstage->num_pages) {
          L->quarantined = true;
          return pkv::set_error(PKV_ERR_PAGE_TABLE,
                                "the step stages more than the compact staging pool's %lld "
                                "pages; raise it (live pool quarantined)",
                                (long long)L->cstage->num_pages);
        }
        L->cstaged.push_back({c, hrow[lp]});
        ctab[(size_t)i * L->pt_stride + nc++] = c;
        continue;                                        // its exact entry stays -1
      }
      if (d >= 0) {
        out[lp] = d;
        ++resident;
        if (L->tag[(size_t)d] != tag_of(ctx_ids[i], lp)) {     // turned hot: copy in once
          L->hot.push_back({d, hrow[lp]});
          L->tag[(size_t)d] = tag_of(ctx_ids[i], lp);
        }
      } else {
        const int32_t s = (int32_t)L->staged.size();
        if (s >= L->stage->num_pages) {
          L->quarantined = true;           // admission moved on; the tags are no longer known good
          return pkv::set_error(PKV_ERR_PAGE_TABLE,
                                "the step stages more than the staging pool's %lld pages; "
                                "raise the staging pool (live pool quarantined)",
                                (long long)L->stage->num_pages);
        }
        L->staged.push_back({s, hrow[lp]});
        out[lp] = P + s;
      }
    }
    const int32_t tail = need - 1;                      // the newest page: always resident
    if (arow[tail] < 0) {
      L->quarantined = true;
      return fail(PKV_ERR_DEVICE, "admission left a tail page out (internal error)");
    }
    lens[i] = (int32_t)lengths[i];
    pos[i] = (int32_t)lengths[i] - 1;
    clens[i] = nc * PT;
    L->tails.push_back({arow[tail], hrow[tail], (int32_t)((lengths[i] - 1) % PT), 0});
  }
  for (int32_t i = n; i < L->max_batch; ++i) {
    std::fill(tab + (size_t)i * L->pt_stride, tab + (size_t)(i + 1) * L->pt_stride, -1);
    lens[i] = 0;
    pos[i] = -1;
  }
  // the table, lengths and positions to the device, in stream order
  hipError_t e = hipMemcpyAsync(L->dev_state, tab, sizeof(int32_t) * state,
                                hipMemcpyHostToDevice, L->compute);
  if (e == hipSuccess && L->cstage)
    e = hipMemcpyAsync(L->dev_cstate, ctab, sizeof(int32_t) * (slot - state),
                       hipMemcpyHostToDevice, L->compute);
  if (e == hipSuccess) e = hipEventRecord(L->ring_ev[k], L->compute);
  if (e != hipSuccess) return quarantine(L, e, "table copy");
  L->ring_used[k] = true;
  ++L->steps;
  L->open = true;
  L->n = n;
  std::fill(L->layer_run.begin(), L->layer_run.end(), 0);
  L->layers_run = 0;
  if (info) {
    info->copied_in_pages = (int64_t)L->hot.size();
    info->staged_pages = (int64_t)L->staged.size();
    info->compact_staged_pages = (int64_t)L->cstaged.size();
    info->refused = refused;
    info->resident_pages = resident;
  }
  pkv::clear_error();
  return PKV_OK;
}

PKV_API int pkv_live_layer(pkv_live* L, int32_t layer, const void* q, const void* k_new,
                           const void* v_new, int32_t num_q_heads, int32_t tile_tokens,
                           float scale, float* part_out, float* part_lse, int32_t num_slots,
                           float* out, float* lse, void* workspace, uint64_t workspace_bytes,
                           const pkv_decode_opts* opts) {
  if (!L) return fail(PKV_ERR_INVALID_ARG, "live pool is NULL");
  if (L->quarantined) return fail(PKV_ERR_QUARANTINED, "live pool is quarantined; destroy it");
  if (!L->open) return fail(PKV_ERR_LEASE, "no step is open: call pkv_live_step_begin");
  if (layer < 0 || layer >= L->layers) return fail(PKV_ERR_INVALID_ARG, "layer out of range");
  if (L->layer_run[(size_t)layer])
    return pkv::set_error(PKV_ERR_LEASE, "layer %d already ran in this step", layer);
  if (!k_new || !v_new) return fail(PKV_ERR_INVALID_ARG, "k_new or v_new is NULL");
  if (!L->cstage &&
      (int64_t)num_slots * tile_tokens > (int64_t)L->pt_stride * L->pool->geom.page_tokens)
    return fail(PKV_ERR_INVALID_ARG, "num_slots x tile_tokens exceeds the table's pages");
  if (reinterpret_cast<uintptr_t>(k_new) % 16)
    return fail(PKV_ERR_INVALID_ARG, "k_new must be 16-byte aligned");
  const int32_t* dev_table = L->dev_state;
  const int32_t* dev_lens = dev_table + (size_t)L->max_batch * L->pt_stride;
  const int32_t* dev_pos = dev_lens + L->max_batch;
  const int32_t* dev_ctable = L->dev_cstate;
  const int32_t* dev_clens = dev_ctable + (size_t)L->max_batch * L->pt_stride;
  const int32_t buf = layer % L->buffers;
  const pkv::StageRef st{L->stage, buf};
  // with compact pages: both runs in one launch (exact tiles first, then the
  // compact run's), one merge over every slot
  const int PTk = L->pool->geom.page_tokens;
  const int32_t cbuf = L->cstage ? layer % L->cstage->geom.num_layers : 0;
  pkv::RunSpec runs[2];
  int32_t n_exact = 0;
  if (L->cstage) {
    if (tile_tokens <= 0 || ((int64_t)L->pt_stride * PTk) % tile_tokens)
      return fail(PKV_ERR_INVALID_ARG, "tile_tokens must divide pt_stride x 64 with compact pages");
    if (opts && opts->split_tokens != 0 && opts->split_tokens != tile_tokens)
      return fail(PKV_ERR_INVALID_ARG, "with compact pages every exact tile is one split");
    n_exact = L->pt_stride * PTk / tile_tokens;
    const int32_t n_compact = L->pt_stride * PTk / L->ctile;
    if (num_slots != n_exact + n_compact)
      return pkv::set_error(PKV_ERR_INVALID_ARG, "num_slots = %d; with compact pages it is %d "
                            "exact tiles + %d compact tiles", num_slots, n_exact, n_compact);
    runs[0] = {L->pool, layer, dev_table, L->pt_stride, dev_lens, n_exact * tile_tokens,
               tile_tokens, 0, &st};
    runs[1] = {L->cstage, cbuf, dev_ctable, L->pt_stride, dev_clens, n_compact * L->ctile,
               L->ctile, n_exact, nullptr};
    if (int rc = pkv::runs_impl(runs, 2, q, L->n, num_q_heads, scale, part_out, part_lse,
                                num_slots, L->compute, true))
      return rc;
    if (!out || !lse || reinterpret_cast<uintptr_t>(out) % 16)
      return fail(PKV_ERR_INVALID_ARG, "out or lse is NULL, or out is not 16-byte aligned");
  } else if (int rc = pkv::decode_merged_staged(L->pool, layer, q, dev_table, L->pt_stride,
                                                dev_lens, L->n, num_q_heads,
                                                num_slots * tile_tokens, tile_tokens, scale,
                                                part_out, part_lse, num_slots, out, lse,
                                                workspace, workspace_bytes, opts, L->compute, st,
                                                true)) {
    return rc;                           // every argument checked before anything is queued
  }
  const uint64_t plb = L->pool->page_layer_bytes;
  // 1. copies of this layer's hot and staged pages, after their last readers
  hipError_t e = hipSuccess;
  for (hipStream_t cs : {L->copy, L->copy2}) {
    if (e == hipSuccess && L->layer_done_set[(size_t)layer])
      e = hipStreamWaitEvent(cs, L->layer_done[(size_t)layer], 0);
    if (e == hipSuccess && L->buf_done_set[(size_t)buf])
      e = hipStreamWaitEvent(cs, L->buf_done[(size_t)buf], 0);
    if (e == hipSuccess && L->cstage && L->cbuf_done_set[(size_t)cbuf])
      e = hipStreamWaitEvent(cs, L->cbuf_done[(size_t)cbuf], 0);
  }
  const char* hslab = L->host + (uint64_t)layer * (uint64_t)L->host_pages * plb;
  char* pslab = static_cast<char*>(L->pool->base) + (uint64_t)layer * (uint64_t)L->pool->num_pages * plb;
  char* sslab = static_cast<char*>(L->stage->base) + (uint64_t)buf * (uint64_t)L->stage->num_pages * plb;
  if (e == hipSuccess) e = copy_pages(L->hot, pslab, hslab, plb, L->copy, L->copy2);
  if (e == hipSuccess) e = copy_pages(L->staged, sslab, hslab, plb, L->copy, L->copy2);
  if (e == hipSuccess && L->cstage && !L->cstaged.empty()) {
    // compact pages: codes (two halves on two engines) and scales of this layer
    const uint64_t cplb = L->cstage->page_layer_bytes;
    const uint64_t csb = 2ull * (uint64_t)L->cstage->geom.num_kv_heads * 4ull;
    const uint64_t cpages = (uint64_t)L->cstage->num_pages;
    char* cbase = static_cast<char*>(L->cstage->base);
    e = copy_pages(L->cstaged, cbase + (uint64_t)cbuf * cpages * cplb,
                   L->chost + (uint64_t)layer * (uint64_t)L->host_pages * cplb, cplb, L->copy,
                   L->copy2);
    if (e == hipSuccess)
      e = copy_pages(L->cstaged, cbase + L->cstage->scale_offset + (uint64_t)cbuf * cpages * csb,
                     L->chost + L->chost_scale_off +
                         (uint64_t)layer * (uint64_t)L->host_pages * csb,
                     csb, L->copy, L->copy2);
  }
  if (e == hipSuccess) e = hipEventRecord(L->copied, L->copy);
  if (e == hipSuccess) e = hipEventRecord(L->copied2, L->copy2);
  if (e == hipSuccess) e = hipStreamWaitEvent(L->compute, L->copied, 0);
  if (e == hipSuccess) e = hipStreamWaitEvent(L->compute, L->copied2, 0);
  if (e != hipSuccess) return quarantine(L, e, "layer copies");
  // 2. append the new token, decode over the composed table, merge
  int rc = pkv_append_kv(L->pool, layer, dev_table, L->pt_stride, dev_pos, L->n, k_new, v_new,
                         L->compute);
  if (rc == PKV_OK && L->cstage) {
    rc = pkv::runs_impl(runs, 2, q, L->n, num_q_heads, scale, part_out, part_lse, num_slots,
                        L->compute, false);
    if (rc == PKV_OK)
      rc = pkv_merge_partials(part_out, part_lse, L->n * num_q_heads, num_slots,
                              L->pool->geom.head_dim, out, lse, L->compute);
  } else if (rc == PKV_OK) {
    rc = pkv::decode_merged_staged(L->pool, layer, q, dev_table, L->pt_stride, dev_lens, L->n,
                                   num_q_heads, num_slots * tile_tokens, tile_tokens, scale,
                                   part_out, part_lse, num_slots, out, lse, workspace,
                                   workspace_bytes, opts, L->compute, st);
  }
  if (rc != PKV_OK) {             // a launch failed after the copies were queued
    L->quarantined = true;
    return rc;
  }
  e = hipEventRecord(L->consumed, L->compute);
  // 3. the new token's rows back to the host pages, after the decode
  if (e == hipSuccess) e = hipStreamWaitEvent(L->writeback, L->consumed, 0);
  const int64_t pe = (int64_t)(plb / 2);
  pkv::WritebackArgs w;
  w.src = static_cast<const uint16_t*>(L->pool->base);
  w.src_layer_off = pe * L->pool->num_pages * layer;
  w.src_num_pages = L->pool->num_pages;
  w.dst = reinterpret_cast<uint16_t*>(L->host_dev);
  w.dst_layer_off = pe * L->host_pages * layer;
  w.dst_num_pages = L->host_pages;
  w.page_elems = pe;
  w.num_kv_heads = L->pool->geom.num_kv_heads;
  size_t i = 0;
  while (e == hipSuccess && i < L->tails.size()) {
    w.n = 0;
    for (; i < L->tails.size() && w.n < pkv::kMaxTailRows; ++i) w.rows[w.n++] = L->tails[i];
    e = pkv::launch_writeback(w, L->writeback);
  }
  if (e == hipSuccess) e = hipEventRecord(L->layer_done[(size_t)layer], L->writeback);
  if (e == hipSuccess) e = hipEventRecord(L->buf_done[(size_t)buf], L->writeback);
  if (e == hipSuccess && L->cstage) e = hipEventRecord(L->cbuf_done[(size_t)cbuf], L->writeback);
  if (e != hipSuccess) return quarantine(L, e, "layer write-back");
  L->layer_done_set[(size_t)layer] = 1;
  L->buf_done_set[(size_t)buf] = 1;
  if (L->cstage) L->cbuf_done_set[(size_t)cbuf] = 1;
  L->layer_run[(size_t)layer] = 1;
  if (++L->layers_run == L->layers) L->open = false;     // every layer queued: the step is done
  pkv::clear_error();
  return PKV_OK;
}

PKV_API int pkv_live_destroy(pkv_live* L) {
  if (!L) return PKV_OK;
  // the streams may still read the ring and the host rows: wait for them
  (void)hipStreamSynchronize(L->copy);
  (void)hipStreamSynchronize(L->copy2);
  (void)hipStreamSynchronize(L->compute);
  (void)hipStreamSynchronize(L->writeback);
  destroy_events(L);
  (void)hipStreamDestroy(L->copy2);
  if (L->ring) (void)hipHostFree(L->ring);
  pkv_admit_destroy(L->admit);
  delete L;
  pkv::clear_error();
  return PKV_OK;
}
