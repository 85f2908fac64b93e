// Device page admission: which logical pages of which contexts hold device
// pages, decided at step boundaries by explicit arithmetic (Staging without
// a stall, section "Admission that does arithmetic"; GPU memory management,
// section "Pages held by right, borrowed or free").
//
// Every context holds its attention-sink page (logical page 0) and as many
// of its newest pages as its allowance permits: `target` pages by right,
// plus up to `burst` pages borrowed while the pool has free pages.  Its floor
// is the sink plus one page.  Pages outside a context's resident set are
// served from the host copy (staged).
//
// Per step, for each active context in the order given, the sink first and
// then the newest pages downward; a missing page is filled by, in order:
//   1. a page the context already holds outside its window (its oldest
//      non-sink page below the window, or past the end of a history that
//      got shorter);
//   2. the lowest-numbered free page, while the context holds fewer than
//      target + burst (borrowed if it already holds its target);
//   3. while below target, a page reclaimed from other contexts, least
//      recently active first (ties: lower id): their borrowed pages, then
//      pages above their (possibly lowered) target, then whole idle
//      contexts; a victim gives its oldest non-sink page;
//   4. the context's own oldest non-sink page older than the one wanted
//      (the history gives up its oldest pages so the newest stay resident);
// and when none of these exists the context is refused for the step if it
// lacks its sink or floor, else its window simply stays shorter.  Borrowing
// is a count per context (never above its pages over target); moving a page
// inside a context leaves it unchanged.  Every fill and reclamation is
// counted and logged.  No HIP call is made here.
#include <algorithm>
#include <cstdio>
#include <functional>
#include <map>
#include <new>
#include <queue>
#include <set>
#include <vector>

#include "pool.h"

#define PKV_API extern "C" __attribute__((visibility("default")))

namespace {

int fail(int code, const char* msg) { return pkv::set_error(code, "%s", msg); }

constexpr int32_t kFloor = 2;   // sink + 1

struct Ctx {
  int32_t id;
  int32_t target;
  int32_t burst;
  int64_t last_active = 0;      // step it was last active (0 = never)
  std::map<int32_t, int32_t> pages;   // logical page -> device page, oldest first
  std::vector<int32_t> where;         // the same as a dense index (-1: not resident)
  int32_t borrowed = 0;               // pages held beyond target via burst
  int32_t held() const { return (int32_t)pages.size(); }
  bool has(int32_t lp) const { return lp < (int32_t)where.size() && where[(size_t)lp] >= 0; }
  void put(int32_t lp, int32_t page) {
    if (lp >= (int32_t)where.size()) where.resize((size_t)lp + 1, -1);
    where[(size_t)lp] = page;
    pages[lp] = page;
  }
};

}  // namespace

struct pkv_admit {
  int64_t num_pages;
  int32_t page_tokens;
  // free device pages, lowest first
  std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free_pages;
  std::map<int32_t, Ctx> ctxs;
  int64_t step = 0;
  pkv_admit_counts counts{};
  std::vector<pkv_admit_event> log;
};

namespace {

void event(pkv_admit* A, int32_t kind, int32_t ctx, int32_t victim, int32_t page, int32_t logical) {
  pkv_admit_event e;
  e.step = A->step;
  e.kind = kind;
  e.context = ctx;
  e.victim = victim;
  e.page = page;
  e.logical = logical;
  A->log.push_back(e);
  switch (kind) {
    case PKV_ADMIT_REUSE_OWN: ++A->counts.reuse_own; break;
    case PKV_ADMIT_TAKE_FREE: ++A->counts.take_free; break;
    case PKV_ADMIT_RECLAIM_BORROWED: ++A->counts.reclaim_borrowed; break;
    case PKV_ADMIT_RECLAIM_ABOVE_TARGET: ++A->counts.reclaim_above_target; break;
    case PKV_ADMIT_RECLAIM_IDLE: ++A->counts.reclaim_idle; break;
    case PKV_ADMIT_SHRINK_OWN: ++A->counts.shrink_own; break;
    case PKV_ADMIT_REFUSED: ++A->counts.refused; break;
  }
}

// Remove logical page `lp` of context c, returning its device page.
int32_t drop(Ctx& c, int32_t lp) {
  auto it = c.pages.find(lp);
  const int32_t page = it->second;
  c.pages.erase(it);
  c.where[(size_t)lp] = -1;
  return page;
}

int32_t pop_free(pkv_admit* A) {
  const int32_t page = A->free_pages.top();
  A->free_pages.pop();
  return page;
}

// Other contexts, least recently active first (ties: lower id first).
std::vector<Ctx*> victims_lra(pkv_admit* A, int32_t self) {
  std::vector<Ctx*> v;
  for (auto& kv : A->ctxs)
    if (kv.first != self) v.push_back(&kv.second);
  std::stable_sort(v.begin(), v.end(), [](const Ctx* a, const Ctx* b) {
    return a->last_active < b->last_active;
  });
  return v;
}

// Oldest non-sink logical page of c below `limit`, or -1 (O(1): the map is
// ordered by logical page).
int32_t oldest_non_sink_below(const Ctx& c, int32_t limit) {
  auto it = c.pages.upper_bound(0);
  return (it != c.pages.end() && it->first < limit) ? it->first : -1;
}

// Oldest non-sink logical page of c outside the window [lo, need), or -1.
int32_t oldest_outside(const Ctx& c, int32_t lo, int32_t need) {
  const int32_t below = oldest_non_sink_below(c, lo);
  if (below >= 0) return below;
  auto it = c.pages.lower_bound(std::max(need, 1));
  return it != c.pages.end() ? it->first : -1;
}

// A page for logical page lp of context c (see the file comment), or -1.
int32_t acquire(pkv_admit* A, Ctx& c, int32_t lp, int32_t window_lo, int32_t need) {
  // 1. own page outside the window
  const int32_t out = oldest_outside(c, window_lo, need);
  if (out >= 0) {
    const int32_t page = drop(c, out);
    event(A, PKV_ADMIT_REUSE_OWN, c.id, c.id, page, lp);
    return page;
  }
  // 2. the lowest free page, within target + burst
  if (!A->free_pages.empty() && c.held() < c.target + c.burst) {
    if (c.held() >= c.target) ++c.borrowed;
    const int32_t page = pop_free(A);
    event(A, PKV_ADMIT_TAKE_FREE, c.id, -1, page, lp);
    return page;
  }
  // 3. reclaim while below target: borrowed, above target, idle contexts
  if (c.held() < c.target) {
    for (Ctx* v : victims_lra(A, c.id)) {
      if (v->borrowed == 0) continue;
      const int32_t vl = oldest_non_sink_below(*v, INT32_MAX);
      if (vl < 0) continue;
      const int32_t page = drop(*v, vl);
      --v->borrowed;
      event(A, PKV_ADMIT_RECLAIM_BORROWED, c.id, v->id, page, lp);
      return page;
    }
    for (Ctx* v : victims_lra(A, c.id)) {
      if (v->held() <= v->target) continue;
      const int32_t vl = oldest_non_sink_below(*v, INT32_MAX);
      if (vl < 0) continue;
      const int32_t page = drop(*v, vl);
      event(A, PKV_ADMIT_RECLAIM_ABOVE_TARGET, c.id, v->id, page, lp);
      return page;
    }
    for (Ctx* v : victims_lra(A, c.id)) {
      if (v->last_active == A->step || v->pages.empty()) continue;   // active now, or empty
      // evict the whole idle context; its pages become free
      for (const auto& kv : v->pages) A->free_pages.push(kv.second);
      v->pages.clear();
      v->where.clear();
      v->borrowed = 0;
      event(A, PKV_ADMIT_RECLAIM_IDLE, c.id, v->id, -1, -1);
      const int32_t page = pop_free(A);
      event(A, PKV_ADMIT_TAKE_FREE, c.id, -1, page, lp);
      return page;
    }
  }
  // 4. shrink from the own oldest non-sink page older than lp
  const int32_t old = oldest_non_sink_below(c, lp);
  if (old >= 0) {
    const int32_t page = drop(c, old);
    event(A, PKV_ADMIT_SHRINK_OWN, c.id, c.id, page, lp);
    return page;
  }
  return -1;
}

}  // namespace

PKV_API int pkv_admit_create(int64_t num_pages, int32_t page_tokens, pkv_admit** out) {
  if (!out) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (num_pages == 0)
    return fail(PKV_ERR_AUTO_SIZE_REFUSED, "num_pages = 0: the pool size must be explicit");
  if (num_pages < 0 || num_pages > INT32_MAX) return fail(PKV_ERR_INVALID_ARG, "num_pages out of range");
  if (page_tokens < 1) return fail(PKV_ERR_INVALID_ARG, "page_tokens must be >= 1");
  pkv_admit* A = new (std::nothrow) pkv_admit;
  if (!A) return fail(PKV_ERR_INVALID_ARG, "host allocation failed");
  A->num_pages = num_pages;
  A->page_tokens = page_tokens;
  std::vector<int32_t> all((size_t)num_pages);
  for (int64_t p = 0; p < num_pages; ++p) all[(size_t)p] = (int32_t)p;
  A->free_pages = decltype(A->free_pages)(std::greater<int32_t>(), std::move(all));
  A->counts.free_pages = num_pages;
  *out = A;
  pkv::clear_error();
  return PKV_OK;
}

PKV_API int pkv_admit_add(pkv_admit* A, int32_t ctx, int32_t target_pages, int32_t burst_pages) {
  if (!A) return fail(PKV_ERR_INVALID_ARG, "admission is NULL");
  if (A->ctxs.count(ctx)) return pkv::set_error(PKV_ERR_INVALID_ARG, "context %d exists", ctx);
  if (target_pages < kFloor)
    return pkv::set_error(PKV_ERR_INVALID_ARG, "target_pages = %d below the floor of %d (sink + 1)",
                          target_pages, kFloor);
  if (burst_pages < 0) return fail(PKV_ERR_INVALID_ARG, "burst_pages must be >= 0");
  Ctx c;
  c.id = ctx;
  c.target = target_pages;
  c.burst = burst_pages;
  A->ctxs.emplace(ctx, std::move(c));
  pkv::clear_error();
  return PKV_OK;
}

PKV_API int pkv_admit_set_target(pkv_admit* A, int32_t ctx, int32_t target_pages,
                                 int32_t burst_pages) {
  if (!A) return fail(PKV_ERR_INVALID_ARG, "admission is NULL");
  auto it = A->ctxs.find(ctx);
  if (it == A->ctxs.end()) return pkv::set_error(PKV_ERR_INVALID_ARG, "no context %d", ctx);
  if (target_pages < kFloor || burst_pages < 0)
    return fail(PKV_ERR_INVALID_ARG, "target below the floor or negative burst");
  Ctx& c = it->second;
  c.target = target_pages;   // pages above it become reclaimable
  c.burst = burst_pages;
  // pages held within the new target are held by right, not borrowed
  c.borrowed = std::min(c.borrowed, std::max(0, c.held() - c.target));
  pkv::clear_error();
  return PKV_OK;
}

PKV_API int pkv_admit_remove(pkv_admit* A, int32_t ctx) {
  if (!A) return fail(PKV_ERR_INVALID_ARG, "admission is NULL");
  auto it = A->ctxs.find(ctx);
  if (it == A->ctxs.end()) return pkv::set_error(PKV_ERR_INVALID_ARG, "no context %d", ctx);
  for (const auto& kv : it->second.pages) A->free_pages.push(kv.second);
  A->ctxs.erase(it);
  A->counts.free_pages = (int64_t)A->free_pages.size();
  pkv::clear_error();
  return PKV_OK;
}

PKV_API int pkv_admit_step(pkv_admit* A, int32_t n, const int32_t* ctx_ids,
                           const int64_t* lengths, int32_t* table, int32_t pt_stride,
                           int32_t* status) {
  if (!A) return fail(PKV_ERR_INVALID_ARG, "admission is NULL");
  if (n < 0) return fail(PKV_ERR_INVALID_ARG, "n must be >= 0");
  if (n > 0 && (!ctx_ids || !lengths || !table || !status))
    return fail(PKV_ERR_INVALID_ARG, "ctx_ids, lengths, table or status is NULL");
  if (pt_stride < 1) return fail(PKV_ERR_INVALID_ARG, "pt_stride must be >= 1");
  std::set<int32_t> seen;
  for (int32_t i = 0; i < n; ++i) {
    auto it = A->ctxs.find(ctx_ids[i]);
    if (it == A->ctxs.end()) return pkv::set_error(PKV_ERR_INVALID_ARG, "no context %d", ctx_ids[i]);
    if (!seen.insert(ctx_ids[i]).second)
      return pkv::set_error(PKV_ERR_INVALID_ARG, "context %d listed twice", ctx_ids[i]);
    if (lengths[i] < 1) return pkv::set_error(PKV_ERR_INVALID_ARG, "lengths[%d] must be >= 1", i);
    const int64_t need = (lengths[i] + A->page_tokens - 1) / A->page_tokens;
    if (need > pt_stride)
      return pkv::set_error(PKV_ERR_INVALID_ARG, "context %d needs %lld pages > pt_stride %d",
                            ctx_ids[i], (long long)need, pt_stride);
  }
  ++A->step;
  ++A->counts.steps;
  for (int32_t i = 0; i < n; ++i) A->ctxs[ctx_ids[i]].last_active = A->step;
  // Phase 1: place pages, in priority order.  A context served earlier in
  // the step may still lose borrowed or above-target pages to a later one
  // below its target, so rows and status are written only in phase 2.
  std::vector<int32_t> lo_of(n), need_of(n);
  std::vector<char> refused(n, 0);
  for (int32_t i = 0; i < n; ++i) {
    Ctx& c = A->ctxs[ctx_ids[i]];
    const int32_t need = (int32_t)((lengths[i] + A->page_tokens - 1) / A->page_tokens);
    const int32_t allow = c.target + c.burst;
    const int32_t lo = std::max(1, need - (allow - 1));     // oldest page of the window
    need_of[i] = need;
    lo_of[i] = lo;
    // the sink, then the newest pages downward
    std::vector<int32_t> want{0};
    for (int32_t lp = need - 1; lp >= lo; --lp) want.push_back(lp);
    for (int32_t lp : want) {
      if (c.has(lp)) continue;
      const int32_t page = acquire(A, c, lp, lo, need);
      if (page < 0) {
        if (lp == 0) {
          refused[i] = 1;
          event(A, PKV_ADMIT_REFUSED, c.id, -1, -1, lp);
        }
        break;
      }
      c.put(lp, page);
    }
    if (!refused[i] && c.held() < std::min(kFloor, need)) {
      refused[i] = 1;
      event(A, PKV_ADMIT_REFUSED, c.id, -1, -1, -1);
    }
  }
  // Phase 2: table rows and status from the final placement.
  for (int32_t i = 0; i < n; ++i) {
    const Ctx& c = A->ctxs[ctx_ids[i]];
    int32_t* row = table + (int64_t)i * pt_stride;
    const int32_t known = std::min<int32_t>(pt_stride, (int32_t)c.where.size());
    std::copy(c.where.begin(), c.where.begin() + known, row);
    std::fill(row + known, row + pt_stride, -1);
    bool whole = row[0] >= 0;
    for (int32_t lp = lo_of[i]; lp < need_of[i] && whole; ++lp) whole = row[lp] >= 0;
    status[i] = refused[i] ? PKV_ADMIT_REFUSED_STEP : whole ? PKV_ADMIT_FULL : PKV_ADMIT_PARTIAL;
  }
  A->counts.free_pages = (int64_t)A->free_pages.size();
  pkv::clear_error();
  return PKV_OK;
}

PKV_API int pkv_admit_get_counts(const pkv_admit* A, pkv_admit_counts* out) {
  if (!A || !out) return fail(PKV_ERR_INVALID_ARG, "admission or out is NULL");
  *out = A->counts;
  pkv::clear_error();
  return PKV_OK;
}

PKV_API int pkv_admit_events(pkv_admit* A, pkv_admit_event* out, int32_t cap, int32_t* n_out) {
  if (!A || !n_out) return fail(PKV_ERR_INVALID_ARG, "admission or n_out is NULL");
  if (cap < 0 || (cap > 0 && !out)) return fail(PKV_ERR_INVALID_ARG, "bad event buffer");
  const int32_t n = std::min<int32_t>(cap, (int32_t)A->log.size());
  for (int32_t i = 0; i < n; ++i) out[i] = A->log[(size_t)i];
  A->log.erase(A->log.begin(), A->log.begin() + n);
  *n_out = n;
  pkv::clear_error();
  return PKV_OK;
}

PKV_API int pkv_admit_destroy(pkv_admit* A) {
  delete A;
  pkv::clear_error();
  return PKV_OK;
}
