"""Plain reference planner for device page admission.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see the package docstring for who may
call it).  Plain Python dictionaries, sets and loops; nothing is indexed,
cached or batched beyond what the rules below state, so that each rule can
be checked against the pages by eye.

Sources, by page and section:
  * Staging without a stall, "Admission that does arithmetic": the pool's
    size is set explicitly by the operator.  A context is entitled to a
    target number of pages, may borrow up to a burst more while free pages
    exist, and never drops below a floor (its sink page and one more).  At
    each step the planner decides which newest pages a context should hold,
    always including the sink, and sources every missing page in a fixed
    order: a page the context already holds outside that window, then a
    free page, then a page reclaimed while the context is under its target,
    and last its own oldest page moved up so the newest stay resident.
    Reclamation visits the contexts that were active longest ago first and
    takes, in turn, borrowed pages, pages over target, and whole idle
    contexts; if nothing remains the request is refused.  The layout only
    changes between steps and each reclamation is logged in order.
  * GPU memory management, "Pages held by right, borrowed or free": the same
    three limits per context, sink and newest pages resident, reclamation
    ordered by last activity with every step of it logged.

Readings where the pages leave a step open (each is listed in the design
notes):
  R1  The window of a context with n pages of history is its sink (logical
      page 0) and its newest target + burst - 1 pages: logical pages
      [lo, n) with lo = max(1, n - (target + burst - 1)).
  R2  Within a step, contexts are served in the order given.  A context
      wants its sink first, then its window pages from the newest down; the
      first page it cannot fill ends its turn.
  R3  Reuse of a page of its own that lies outside its window: the oldest
      such non-sink page (outside [lo, n): below lo in a growing history,
      past the end only if the history got shorter) moves to the wanted
      logical page.
  R4  A free page: the lowest-numbered free device page, taken only while
      the context holds fewer than target + burst pages.  Taken while it
      already holds its target or more, the page is borrowed: the
      context's borrowed count rises by one.
  R5  Reclamation inside the target: only a context holding fewer pages than
      its target reclaims.  Victims are the other contexts ordered by the
      step they were last active (earliest first; never active counts as
      step 0), ties by lower context id.  First pass: the first victim with
      a borrowed page gives its oldest non-sink page, and its borrowed
      count falls by one.  Second pass: the first victim holding more pages
      than its target gives its oldest non-sink page.  Third pass: the first
      victim not active in this step that holds any page is evicted whole
      (all its pages become free, its borrowed count 0), then R4's lowest
      free page is taken.
  R6  Shrinking from its oldest end so that its newest pages stay
      resident: the context's own oldest non-sink page below the wanted
      page moves to it.
  R7  A context that cannot get its sink is refused for the step; so is one
      left holding fewer than min(2, n) pages (its floor).  Otherwise a
      window that could not be filled stays short: status partial.
  R8  Borrowing is a count per context, never more than its pages above
      target.  Moving a page between two logical pages of one context
      (R3, R6) does not change it.  Changing the target clamps it to the
      pages now above the new target.
  R9  Table rows and statuses are written after every context of the step
      has been served, because a context served earlier can still lose
      borrowed or above-target pages to a later one below its target.
      Row entry i is the device page of logical page i, -1 if none.
Pins: tests/test_oracle_admission.py (hand-derived cases and planted
mistakes).
"""

KINDS = ("reuse_own", "take_free", "reclaim_borrowed", "reclaim_above_target",
         "reclaim_idle", "shrink_own", "refused")
FLOOR = 2   # the sink plus one page


class Context:
    def __init__(self, cid, target, burst):
        self.id = cid
        self.target = target
        self.burst = burst
        self.last_active = 0
        self.pages = {}      # logical page -> device page
        self.borrowed = 0

    def held(self):
        return len(self.pages)

    def oldest_non_sink_below(self, limit):
        below = [lp for lp in self.pages if 0 < lp < limit]
        return min(below) if below else None

    def oldest_outside(self, lo, need):
        out = [lp for lp in self.pages if 0 < lp and not lo <= lp < need]
        return min(out) if out else None


class Admission:
    """Host-side admission of one device pool of `num_pages` pages."""

    def __init__(self, num_pages, page_tokens=64):
        if num_pages == 0:
            raise ValueError("an automatic pool size is refused: give the page count")
        if num_pages < 0 or page_tokens < 1:
            raise ValueError("num_pages and page_tokens must be positive")
        self.page_tokens = page_tokens
        self.free = set(range(num_pages))
        self.contexts = {}
        self.step_no = 0
        self.log = []
        self.tally = {k: 0 for k in KINDS}

    # -- contexts ----------------------------------------------------------

    def add(self, cid, target, burst=0):
        if cid in self.contexts:
            raise ValueError(f"context {cid} exists")
        if target < FLOOR or burst < 0:
            raise ValueError("target below the floor (sink + 1) or negative burst")
        self.contexts[cid] = Context(cid, target, burst)

    def set_target(self, cid, target, burst=0):
        if cid not in self.contexts:
            raise ValueError(f"no context {cid}")
        if target < FLOOR or burst < 0:
            raise ValueError("target below the floor (sink + 1) or negative burst")
        c = self.contexts[cid]
        c.target = target
        c.burst = burst
        c.borrowed = min(c.borrowed, max(0, c.held() - c.target))          # R8

    def remove(self, cid):
        if cid not in self.contexts:
            raise ValueError(f"no context {cid}")
        self.free |= set(self.contexts.pop(cid).pages.values())

    # -- one step ----------------------------------------------------------

    def _event(self, kind, ctx, victim, page, logical):
        self.log.append(dict(step=self.step_no, kind=kind, context=ctx, victim=victim,
                             page=page, logical=logical))
        self.tally[kind] += 1

    def _victims(self, cid):
        others = [c for c in self.contexts.values() if c.id != cid]
        return sorted(others, key=lambda c: (c.last_active, c.id))          # R5

    def _take_free(self, c, lp):
        page = min(self.free)                                               # R4
        self.free.remove(page)
        self._event("take_free", c.id, -1, page, lp)
        return page

    # The sources of a missing page, one method each, tried in the order of
    # SOURCES; each returns a device page (recording its event) or None.

    def _own_outside_window(self, c, lp, lo, need):      # R3
        old = c.oldest_outside(lo, need)
        if old is None:
            return None
        page = c.pages.pop(old)
        self._event("reuse_own", c.id, c.id, page, lp)
        return page

    def _free_page(self, c, lp, lo, need):             # R4
        if not self.free or c.held() >= c.target + c.burst:
            return None
        if c.held() >= c.target:
            c.borrowed += 1
        return self._take_free(c, lp)

    def _reclaim_borrowed(self, c, lp, lo, need):      # R5, first pass
        if c.held() >= c.target:
            return None
        for v in self._victims(c.id):
            if v.borrowed > 0:
                page = v.pages.pop(v.oldest_non_sink_below(float("inf")))
                v.borrowed -= 1
                self._event("reclaim_borrowed", c.id, v.id, page, lp)
                return page
        return None

    def _reclaim_above_target(self, c, lp, lo, need):  # R5, second pass
        if c.held() >= c.target:
            return None
        for v in self._victims(c.id):
            if v.held() > v.target:
                page = v.pages.pop(v.oldest_non_sink_below(float("inf")))
                self._event("reclaim_above_target", c.id, v.id, page, lp)
                return page
        return None

    def _reclaim_idle(self, c, lp, lo, need):          # R5, third pass
        if c.held() >= c.target:
            return None
        for v in self._victims(c.id):
            if v.last_active != self.step_no and v.pages:
                self.free |= set(v.pages.values())
                v.pages = {}
                v.borrowed = 0
                self._event("reclaim_idle", c.id, v.id, -1, -1)
                return self._take_free(c, lp)
        return None

    def _shrink_from_oldest(self, c, lp, lo, need):    # R6
        old = c.oldest_non_sink_below(lp)
        if old is None:
            return None
        page = c.pages.pop(old)
        self._event("shrink_own", c.id, c.id, page, lp)
        return page

    SOURCES = ("_own_outside_window", "_free_page", "_reclaim_borrowed",
               "_reclaim_above_target", "_reclaim_idle", "_shrink_from_oldest")

    def _acquire(self, c, lp, lo, need):
        """A device page for logical page lp of context c, or None."""
        for name in self.SOURCES:
            page = getattr(self, name)(c, lp, lo, need)
            if page is not None:
                return page
        return None

    def step(self, ids, lengths, pt_stride):
        """Serve the contexts `ids` (in priority order) with histories of
        `lengths` tokens.  Returns (rows, status): rows[i] is a list of
        pt_stride device pages (-1 where not resident), status[i] one of
        'full', 'partial', 'refused'."""
        ids = [int(x) for x in ids]
        lengths = [int(x) for x in lengths]
        if len(set(ids)) != len(ids):
            raise ValueError("a context is listed twice")
        for cid, n_tok in zip(ids, lengths):
            if cid not in self.contexts:
                raise ValueError(f"no context {cid}")
            if n_tok < 1:
                raise ValueError("a history must hold at least one token")
            if -(-n_tok // self.page_tokens) > pt_stride:
                raise ValueError("a history needs more pages than a row holds")
        self.step_no += 1
        for cid in ids:
            self.contexts[cid].last_active = self.step_no
        windows = []
        refused = []
        for cid, n_tok in zip(ids, lengths):
            c = self.contexts[cid]
            need = -(-n_tok // self.page_tokens)
            lo = max(1, need - (c.target + c.burst - 1))                    # R1
            windows.append((need, lo))
            is_refused = False
            for lp in [0] + list(range(need - 1, lo - 1, -1)):              # R2
                if lp in c.pages:
                    continue
                page = self._acquire(c, lp, lo, need)
                if page is None:
                    if lp == 0:                                             # R7
                        is_refused = True
                        self._event("refused", c.id, -1, -1, 0)
                    break
                c.pages[lp] = page
            if not is_refused and c.held() < min(FLOOR, need):              # R7
                is_refused = True
                self._event("refused", c.id, -1, -1, -1)
            refused.append(is_refused)
        rows, status = [], []
        for cid, (need, lo), is_refused in zip(ids, windows, refused):      # R9
            c = self.contexts[cid]
            row = [c.pages.get(lp, -1) for lp in range(pt_stride)]
            rows.append(row)
            window = [0] + list(range(lo, need))
            if is_refused:
                status.append("refused")
            elif all(row[lp] >= 0 for lp in window):
                status.append("full")
            else:
                status.append("partial")
        return rows, status

    # -- what happened -----------------------------------------------------

    def events(self):
        out, self.log = self.log, []
        return out

    def counts(self):
        out = dict(steps=self.step_no, **self.tally)
        out["free_pages"] = len(self.free)
        return out
