// Staged tiles under a lease: the history of a layer lives in pinned host
// memory and is brought into a staging buffer on the device one window at a
// time (Staging without a stall, sections "Two copy queues and device-side
// ordering" and "Leases instead of buffers"; KV-cache engineering, "Staging
// layers under a lease"; GPU memory management, "Staging as a lease").
//
// Ordering is on the device: the copy streams wait for the previous readers
// of the buffer they overwrite and for any write-back still landing in a
// host page they read, the compute stream waits for the copies, the
// write-back stream waits for the compute stream's consumer event.  Nothing
// but the appended token's rows goes back to the host (one per request), by a kernel
// that stores them into the pinned host pages.  Each
// window's copy is split in two halves, one on the caller's copy stream and
// one on a second copy stream the stager owns (default priority), so that one
// copy engine's wait before a window overlaps the other's transfer.  The host
// blocks only in pkv_stager_retire.  Any HIP failure quarantines the stager:
// new leases are refused and nothing is released until a drain proves that
// every queued copy and kernel finished.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <new>
#include <unordered_set>
#include <vector>

#include "kernels.h"
#include "pool.h"

#define PKV_API extern "C" __attribute__((visibility("default")))

namespace {

int fail(int code, const char* msg) { return pkv::set_error(code, "%s", msg); }

struct Buffer {
  hipEvent_t copied = nullptr;     // H2D copy of the window's first half done (copy stream)
  hipEvent_t copied2 = nullptr;    // and of its second half (the stager's own copy stream)
  hipEvent_t consumed = nullptr;   // work of the lease on the compute stream done
  hipEvent_t written = nullptr;    // tail write-back done (write-back stream)
  bool has_readers = false;        // consumed / written recorded by a sealed lease
  bool wrote_back = false;
};

struct Tail {                      // a changed tail row to copy back at seal
  int64_t staging_page;
  int64_t host_page;
  int32_t token;                   // token within the page
};

}  // namespace

struct pkv_stager {
  const pkv_pool* staging;
  char* host;                      // pinned host arena, layout of a pool of host_pages pages
  char* host_dev = nullptr;        // the same memory as the device addresses it
  int64_t host_pages;
  int32_t host_layers;
  int32_t max_batch;
  int32_t window_tokens;
  int32_t window_pages;
  int32_t num_buffers;
  int32_t* dev_tables;             // [num_buffers][max_batch][window_pages]
  bool compact = false;            // compact (E4M3) pages: codes, plus a scale run per copy
  uint64_t scale_bytes = 0;        // scales of one compact (layer, page)
  char* host_scales = nullptr;     // scale region of the host arena
  char* staging_scales = nullptr;  // scale region of the staging pool (its layer 0)
  hipStream_t copy, compute, writeback;
  hipStream_t copy2 = nullptr;     // the stager's own second copy stream
  std::vector<Buffer> buffers;
  uint64_t generation = 0;         // leases begun so far
  bool open = false;               // a lease is begun and not yet sealed
  uint64_t open_generation = 0;
  int32_t open_buffer = -1;
  std::vector<Tail> open_tails;
  int64_t sealed_unretired = 0;    // leases sealed since the last retire
  bool quarantined = false;
  // Host pages (layer * host_pages + page) written back since the last
  // retire, and an event after the latest write-back: the write-back stream
  // runs in order, so a copy that waits for it reads every earlier row too.
  std::unordered_set<int64_t> wb_pending;
  hipEvent_t wb_last = nullptr;
};

namespace {

int quarantine(pkv_stager* st, hipError_t e, const char* what) {
  st->quarantined = true;
  return pkv::set_error(PKV_ERR_DEVICE, "%s failed (%s): stager quarantined", what,
                        hipGetErrorString(e));
}

}  // namespace

PKV_API int pkv_stager_create(const pkv_pool* staging, void* host_arena, uint64_t host_bytes,
                              int32_t host_layers, int32_t max_batch, int32_t window_tokens,
                              int32_t num_buffers, int32_t* dev_tables, void* copy_stream,
                              void* compute_stream, void* writeback_stream, pkv_stager** out) {
  if (!out) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!staging) return fail(PKV_ERR_INVALID_ARG, "staging pool is NULL");
  if (!host_arena || !dev_tables) return fail(PKV_ERR_INVALID_ARG, "host_arena or dev_tables is NULL");
  if (host_layers < 1) return fail(PKV_ERR_INVALID_ARG, "host_layers must be >= 1");
  const bool compact = staging->format == PKV_FORMAT_E4M3;
  const uint64_t plb = staging->page_layer_bytes;   // codes only, for a compact pool
  const uint64_t sb = compact ? 2ull * (uint64_t)staging->geom.num_kv_heads * 4ull : 0ull;
  const uint64_t host_page_bytes = (plb + sb) * (uint64_t)host_layers;
  if (host_bytes == 0 || host_bytes % host_page_bytes)
    return pkv::set_error(PKV_ERR_INVALID_ARG,
                          "host_bytes = %llu must be a positive whole number of %llu-byte pages",
                          (unsigned long long)host_bytes, (unsigned long long)host_page_bytes);
  if (max_batch < 1 || max_batch > 65535) return fail(PKV_ERR_INVALID_ARG, "max_batch outside 1..65535");
  if (window_tokens < staging->geom.page_tokens || window_tokens % staging->geom.page_tokens)
    return fail(PKV_ERR_INVALID_ARG, "window_tokens must be a positive multiple of page_tokens");
  if (num_buffers < 1 || num_buffers > 64) return fail(PKV_ERR_INVALID_ARG, "num_buffers outside 1..64");
  const int32_t wpp = window_tokens / staging->geom.page_tokens;
  const int64_t need = (int64_t)num_buffers * max_batch * wpp;
  if (need > staging->num_pages)
    return pkv::set_error(PKV_ERR_INVALID_ARG,
                          "staging pool holds %lld pages; %d buffers x %d requests x %d pages "
                          "need %lld",
                          (long long)staging->num_pages, num_buffers, max_batch, wpp,
                          (long long)need);
  pkv_stager* st = new (std::nothrow) pkv_stager;
  if (!st) return fail(PKV_ERR_INVALID_ARG, "host allocation failed");
  st->staging = staging;
  st->host = static_cast<char*>(host_arena);
  st->host_pages = (int64_t)(host_bytes / host_page_bytes);
  st->host_layers = host_layers;
  st->max_batch = max_batch;
  st->window_tokens = window_tokens;
  st->window_pages = wpp;
  st->num_buffers = num_buffers;
  st->dev_tables = dev_tables;
  st->compact = compact;
  st->scale_bytes = sb;
  if (compact) {
    st->host_scales = st->host + (uint64_t)host_layers * (uint64_t)st->host_pages * plb;
    st->staging_scales = static_cast<char*>(staging->base) + staging->scale_offset;
  }
  st->copy = static_cast<hipStream_t>(copy_stream);
  st->compute = static_cast<hipStream_t>(compute_stream);
  st->writeback = static_cast<hipStream_t>(writeback_stream);
  st->buffers.resize(num_buffers);
  // Every lease's staging table is fixed: buffer k, request b, window page i
  // lives in staging page (k * max_batch + b) * window_pages + i.
  std::vector<int32_t> t((size_t)need);
  for (int64_t i = 0; i < need; ++i) t[(size_t)i] = (int32_t)i;
  hipError_t e = hipMemcpy(dev_tables, t.data(), sizeof(int32_t) * (size_t)need, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&st->copy2, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&st->wb_last, hipEventDisableTiming);
  if (e == hipSuccess && !compact) {
    // the tail write-back kernel stores into the host pages directly
    void* dev = nullptr;
    e = hipHostGetDevicePointer(&dev, host_arena, 0);
    st->host_dev = static_cast<char*>(dev);
  }
  for (auto& bf : st->buffers) {
    if (e == hipSuccess) e = hipEventCreateWithFlags(&bf.copied, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&bf.copied2, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&bf.consumed, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&bf.written, hipEventDisableTiming);
  }
  if (e != hipSuccess) {
    for (auto& bf : st->buffers) {
      if (bf.copied) (void)hipEventDestroy(bf.copied);
      if (bf.copied2) (void)hipEventDestroy(bf.copied2);
      if (bf.consumed) (void)hipEventDestroy(bf.consumed);
      if (bf.written) (void)hipEventDestroy(bf.written);
    }
    if (st->copy2) (void)hipStreamDestroy(st->copy2);
    if (st->wb_last) (void)hipEventDestroy(st->wb_last);
    delete st;
    return pkv::set_error(PKV_ERR_DEVICE,
                          "stager setup failed: %s (host_arena must be pinned host memory, "
                          "e.g. hipHostMalloc, which the device can address)",
                          hipGetErrorString(e));
  }
  *out = st;
  pkv::clear_error();
  return PKV_OK;
}

PKV_API int pkv_lease_begin(pkv_stager* st, int32_t layer, const int32_t* host_table,
                            int32_t pt_stride, const int32_t* host_ctx_lens, int32_t batch,
                            int32_t window_begin, pkv_lease* lease) {
  if (!st || !lease) return fail(PKV_ERR_INVALID_ARG, "stager or lease is NULL");
  if (st->quarantined) return fail(PKV_ERR_QUARANTINED, "stager is quarantined; retire it");
  if (st->open)
    return pkv::set_error(PKV_ERR_LEASE, "lease %llu is not sealed; seal it before beginning "
                          "another",
                          (unsigned long long)st->open_generation);
  if (layer < 0 || layer >= st->host_layers) return fail(PKV_ERR_INVALID_ARG, "layer out of range");
  if (batch < 1 || batch > st->max_batch) return fail(PKV_ERR_INVALID_ARG, "batch outside 1..max_batch");
  if (window_begin < 0 || window_begin % st->window_tokens)
    return fail(PKV_ERR_INVALID_ARG, "window_begin must be a non-negative multiple of window_tokens");
  if (!host_table || !host_ctx_lens) return fail(PKV_ERR_INVALID_ARG, "host_table or host_ctx_lens is NULL");
  const int PT = st->staging->geom.page_tokens;
  const int first = window_begin / PT;
  // validate every host page the window reads before queueing anything
  for (int b = 0; b < batch; ++b) {
    const int64_t ctx = host_ctx_lens[b];
    if (ctx < 0 || ctx > (int64_t)pt_stride * PT)
      return pkv::set_error(PKV_ERR_PAGE_TABLE, "ctx_lens[%d] = %lld outside 0..%lld", b,
                            (long long)ctx, (long long)pt_stride * PT);
    const int64_t end = std::min<int64_t>(ctx, (int64_t)window_begin + st->window_tokens);
    for (int64_t lp = first; lp * PT < end; ++lp) {
      const int32_t hp = host_table[(int64_t)b * pt_stride + lp];
      if (hp < 0 || hp >= st->host_pages)
        return pkv::set_error(PKV_ERR_PAGE_TABLE, "host_table[%d][%lld] = %d is not a host page "
                              "(0..%lld)", b, (long long)lp, hp, (long long)(st->host_pages - 1));
    }
  }
  // a host page this window reads may still be receiving an earlier lease's
  // tail row: then the copies also wait for the latest write-back
  bool reads_pending = false;
  if (!st->wb_pending.empty()) {
    const int64_t lbase = (int64_t)layer * st->host_pages;
    for (int b = 0; b < batch && !reads_pending; ++b) {
      const int64_t end = std::min<int64_t>(host_ctx_lens[b], (int64_t)window_begin + st->window_tokens);
      for (int64_t lp = first; lp * PT < end && !reads_pending; ++lp)
        reads_pending = st->wb_pending.count(lbase + host_table[(int64_t)b * pt_stride + lp]) > 0;
    }
  }
  const int32_t k = (int32_t)(st->generation % (uint64_t)st->num_buffers);
  Buffer& bf = st->buffers[k];
  hipError_t e = hipSuccess;
  // the previous readers of buffer k must finish before the copies overwrite it
  for (hipStream_t cs : {st->copy, st->copy2}) {
    if (e == hipSuccess && bf.has_readers) e = hipStreamWaitEvent(cs, bf.consumed, 0);
    if (e == hipSuccess && bf.has_readers && bf.wrote_back) e = hipStreamWaitEvent(cs, bf.written, 0);
    if (e == hipSuccess && reads_pending) e = hipStreamWaitEvent(cs, st->wb_last, 0);
  }
  if (e != hipSuccess) return quarantine(st, e, "wait for the buffer's readers");
  const uint64_t plb = st->staging->page_layer_bytes;
  char* slab = static_cast<char*>(st->staging->base);        // staging layer 0
  const char* hslab = st->host + (uint64_t)layer * (uint64_t)st->host_pages * plb;
  std::vector<Tail> tails;
  for (int b = 0; b < batch; ++b) {
    const int64_t ctx = host_ctx_lens[b];
    const int64_t end = std::min<int64_t>(ctx, (int64_t)window_begin + st->window_tokens);
    const int64_t npg = end > window_begin ? (end - window_begin + PT - 1) / PT : 0;
    const int64_t dst0 = ((int64_t)k * st->max_batch + b) * st->window_pages;
    int64_t i = 0;
    while (i < npg && e == hipSuccess) {                     // one copy per run of host pages
      const int32_t h0 = host_table[(int64_t)b * pt_stride + first + i];
      int64_t run = 1;
      while (i + run < npg && host_table[(int64_t)b * pt_stride + first + i + run] == h0 + run) ++run;
      // first half of the run on the copy stream, the rest on the second one
      const int64_t half = (run + 1) / 2;
      e = hipMemcpyAsync(slab + (uint64_t)(dst0 + i) * plb, hslab + (uint64_t)h0 * plb,
                         (size_t)(half * (int64_t)plb), hipMemcpyHostToDevice, st->copy);
      if (e == hipSuccess && run > half)
        e = hipMemcpyAsync(slab + (uint64_t)(dst0 + i + half) * plb,
                           hslab + (uint64_t)(h0 + half) * plb,
                           (size_t)((run - half) * (int64_t)plb), hipMemcpyHostToDevice, st->copy2);
      if (e == hipSuccess && st->compact)                    // the run's scales
        e = hipMemcpyAsync(st->staging_scales + (uint64_t)(dst0 + i) * st->scale_bytes,
                           st->host_scales + ((uint64_t)layer * (uint64_t)st->host_pages +
                                              (uint64_t)h0) * st->scale_bytes,
                           (size_t)((uint64_t)run * st->scale_bytes), hipMemcpyHostToDevice,
                           st->copy);
      i += run;
    }
    if (ctx > window_begin && ctx <= (int64_t)window_begin + st->window_tokens) {
      const int64_t lp = (ctx - 1) / PT;                     // the request's tail page is here
      tails.push_back({dst0 + (lp - first), host_table[(int64_t)b * pt_stride + lp],
                       (int32_t)((ctx - 1) % PT)});
    }
  }
  if (e == hipSuccess) e = hipEventRecord(bf.copied, st->copy);
  if (e == hipSuccess) e = hipEventRecord(bf.copied2, st->copy2);
  if (e == hipSuccess) e = hipStreamWaitEvent(st->compute, bf.copied, 0);
  if (e == hipSuccess) e = hipStreamWaitEvent(st->compute, bf.copied2, 0);
  if (e != hipSuccess) return quarantine(st, e, "window copy");
  st->open = true;
  st->open_generation = ++st->generation;
  st->open_buffer = k;
  st->open_tails = std::move(tails);
  lease->generation = st->open_generation;
  lease->layer = layer;
  lease->window_begin = window_begin;
  lease->buffer = k;
  lease->staging_layer = 0;
  lease->dev_table = st->dev_tables + (int64_t)k * st->max_batch * st->window_pages;
  lease->pt_stride = st->window_pages;
  pkv::clear_error();
  return PKV_OK;
}

PKV_API int pkv_lease_seal(pkv_stager* st, const pkv_lease* lease, int32_t write_back_tail) {
  if (!st || !lease) return fail(PKV_ERR_INVALID_ARG, "stager or lease is NULL");
  if (st->quarantined) return fail(PKV_ERR_QUARANTINED, "stager is quarantined; retire it");
  if (!st->open || lease->generation != st->open_generation || lease->buffer != st->open_buffer)
    return pkv::set_error(PKV_ERR_LEASE, "lease %llu is not the open lease; a lease is sealed "
                          "only by its own handle", (unsigned long long)lease->generation);
  if (write_back_tail && st->compact)
    return fail(PKV_ERR_INVALID_ARG, "compact pages are immutable: nothing to write back");
  Buffer& bf = st->buffers[st->open_buffer];
  hipError_t e = hipEventRecord(bf.consumed, st->compute);
  bool wrote = false;
  if (e == hipSuccess && write_back_tail && !st->open_tails.empty()) {
    // the changed rows only: one token of K and V per request whose tail is
    // in the window, 2 x Hkv x 256 bf16 each, stored into the host page
    e = hipStreamWaitEvent(st->writeback, bf.consumed, 0);
    const int64_t page_elems = (int64_t)(st->staging->page_layer_bytes / 2);
    pkv::WritebackArgs w;
    w.src = static_cast<const uint16_t*>(st->staging->base);
    w.src_layer_off = 0;
    w.src_num_pages = st->staging->num_pages;
    w.dst = reinterpret_cast<uint16_t*>(st->host_dev);
    w.dst_layer_off = page_elems * st->host_pages * lease->layer;
    w.dst_num_pages = st->host_pages;
    w.page_elems = page_elems;
    w.num_kv_heads = st->staging->geom.num_kv_heads;
    const int64_t lbase = (int64_t)lease->layer * st->host_pages;
    size_t i = 0;
    while (e == hipSuccess && i < st->open_tails.size()) {
      w.n = 0;
      for (; i < st->open_tails.size() && w.n < pkv::kMaxTailRows; ++i, ++w.n) {
        const Tail& t = st->open_tails[i];
        w.rows[w.n] = {(int32_t)t.staging_page, (int32_t)t.host_page, t.token, 0};
        st->wb_pending.insert(lbase + t.host_page);
      }
      e = pkv::launch_writeback(w, st->writeback);
    }
    if (e == hipSuccess) e = hipEventRecord(bf.written, st->writeback);
    if (e == hipSuccess) e = hipEventRecord(st->wb_last, st->writeback);
    wrote = true;
  }
  if (e != hipSuccess) return quarantine(st, e, "seal");
  bf.has_readers = true;
  bf.wrote_back = wrote;
  st->open = false;
  st->open_tails.clear();
  ++st->sealed_unretired;
  pkv::clear_error();
  return PKV_OK;
}

PKV_API int pkv_stager_retire(pkv_stager* st, int64_t* receipts) {
  if (!st) return fail(PKV_ERR_INVALID_ARG, "stager is NULL");
  if (st->open) return fail(PKV_ERR_LEASE, "a lease is open; seal it before retiring");
  hipError_t e = hipSuccess;
  if (st->quarantined) {
    // drain: the copy and write-back queues, the compute queue, then the device
    e = hipStreamSynchronize(st->copy);
    if (e == hipSuccess) e = hipStreamSynchronize(st->copy2);
    if (e == hipSuccess) e = hipStreamSynchronize(st->writeback);
    if (e == hipSuccess) e = hipStreamSynchronize(st->compute);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess)
      return pkv::set_error(PKV_ERR_DEVICE, "drain failed (%s): everything stays retained",
                            hipGetErrorString(e));
  } else {
    for (auto& bf : st->buffers) {
      if (!bf.has_readers) continue;
      e = hipEventSynchronize(bf.copied);
      if (e == hipSuccess) e = hipEventSynchronize(bf.copied2);
      if (e == hipSuccess) e = hipEventSynchronize(bf.consumed);
      if (e == hipSuccess && bf.wrote_back) e = hipEventSynchronize(bf.written);
      if (e != hipSuccess) {
        st->quarantined = true;
        return pkv::set_error(PKV_ERR_DEVICE, "wait on a lease failed (%s): quarantined",
                              hipGetErrorString(e));
      }
    }
  }
  if (receipts) *receipts = st->sealed_unretired;
  st->sealed_unretired = 0;
  st->wb_pending.clear();            // every write-back has landed
  st->quarantined = false;
  for (auto& bf : st->buffers) bf.has_readers = bf.wrote_back = false;
  pkv::clear_error();
  return PKV_OK;
}

PKV_API int pkv_stager_info(const pkv_stager* st, uint64_t* generation, int64_t* unretired,
                            int32_t* open, int32_t* quarantined) {
  if (!st) return fail(PKV_ERR_INVALID_ARG, "stager is NULL");
  if (generation) *generation = st->generation;
  if (unretired) *unretired = st->sealed_unretired;
  if (open) *open = st->open ? 1 : 0;
  if (quarantined) *quarantined = st->quarantined ? 1 : 0;
  pkv::clear_error();
  return PKV_OK;
}

PKV_API int pkv_stager_fail(pkv_stager* st) {
  if (!st) return fail(PKV_ERR_INVALID_ARG, "stager is NULL");
  st->quarantined = true;
  st->open = false;                // an open lease is abandoned, its buffer still retained
  st->open_tails.clear();
  pkv::clear_error();
  return PKV_OK;
}

PKV_API int pkv_stager_destroy(pkv_stager* st) {
  if (!st) return PKV_OK;
  if (st->open || st->sealed_unretired > 0 || st->quarantined)
    return fail(PKV_ERR_BUSY, "leases are outstanding; retire the stager first (destroy never waits)");
  for (auto& bf : st->buffers) {
    (void)hipEventDestroy(bf.copied);
    (void)hipEventDestroy(bf.copied2);
    (void)hipEventDestroy(bf.consumed);
    (void)hipEventDestroy(bf.written);
  }
  (void)hipStreamDestroy(st->copy2);
  (void)hipEventDestroy(st->wb_last);
  delete st;
  pkv::clear_error();
  return PKV_OK;
}
