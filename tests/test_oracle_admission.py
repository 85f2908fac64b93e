"""Pins for the admission oracle (oracle/admission.py), on the CPU.

Each hand case below was worked out from the rules of Staging without a
stall, section "Admission that does arithmetic", and GPU memory management,
section "Pages held by right, borrowed or free" (with the readings R1-R9
listed in the oracle), not from any implementation.  The cases run on the
oracle (its pins), on planted mistakes of the oracle (each must fail at
least one case) and, from tests/test_admit.py, on the library's planner.

An implementation is a factory `make(num_pages)` of objects with add,
set_target, remove, step(ids, lengths, pt_stride) -> (rows, status),
events() and counts().
"""

import numpy as np
import pytest

from oracle import admission as OA

T = 64   # tokens per page


def toks(pages):
    return pages * T


def kinds(events):
    return [e["kind"] for e in events]


def step(a, ids, lengths, pt_stride):
    rows, st = a.step(ids, lengths, pt_stride)
    return np.asarray(rows, dtype=np.int64).reshape(len(ids), pt_stride), list(st)


# ----------------------------------------------------------------------------
# hand cases (each raises AssertionError when the implementation is wrong)


def case_free_pages_fill_sink_then_newest(make):
    a = make(8)
    a.add(7, 4)
    tab, st = step(a, [7], [toks(6) - 5], 8)
    # 6 pages needed, 4 by right: the sink and the newest three, each the
    # lowest free page at the time (R2, R4)
    assert st == ["full"]
    assert list(tab[0]) == [0, -1, -1, 3, 2, 1, -1, -1]
    ev = a.events()
    assert kinds(ev) == ["take_free"] * 4
    assert [e["logical"] for e in ev] == [0, 5, 4, 3]
    c = a.counts()
    assert c["take_free"] == 4 and c["free_pages"] == 4 and c["steps"] == 1


def case_sliding_window_reuses_own_page_and_keeps_sink(make):
    a = make(4)
    a.add(1, 3)
    tab, _ = step(a, [1], [toks(3)], 4)
    held = {lp: p for lp, p in enumerate(tab[0]) if p >= 0}
    assert sorted(held) == [0, 1, 2]
    a.events()
    tab, st = step(a, [1], [toks(3) + 1], 4)          # a fourth page opens
    ev = a.events()
    assert kinds(ev) == ["reuse_own"] and ev[0]["logical"] == 3
    assert ev[0]["page"] == held[1]                   # the page that left the window
    assert st == ["full"] and tab[0][0] == held[0] and tab[0][1] == -1
    assert tab[0][2] == held[2] and tab[0][3] == held[1]
    assert a.counts()["free_pages"] == 1              # the window never grew


def case_burst_borrows_only_while_free_and_is_reclaimed_first(make):
    a = make(10)
    a.add(1, 3, 4)
    tab, st = step(a, [1], [toks(20)], 20)
    assert st == ["full"] and (tab[0] >= 0).sum() == 7      # target + burst
    a.events()
    a.add(2, 5)
    tab, st = step(a, [2], [toks(5)], 20)
    ev = a.events()
    # three free pages, then two of context 1's borrowed pages, its oldest
    # non-sink pages first
    assert kinds(ev) == ["take_free"] * 3 + ["reclaim_borrowed"] * 2
    assert all(e["victim"] == 1 for e in ev[3:])
    assert [e["page"] for e in ev[3:]] == [6, 5]     # 1's logical pages 14, 15
    assert st == ["full"]
    tab1, st1 = step(a, [1], [toks(20)], 20)
    ev = a.events()
    # context 1 is now at 5 pages: no free page, above its target, so it
    # cannot reclaim; it keeps sink + newest 4 and the window is partial
    assert st1 == ["partial"] and (tab1[0] >= 0).sum() == 5
    assert tab1[0][0] >= 0 and (tab1[0][16:20] >= 0).all()
    assert "reclaim_borrowed" not in kinds(ev)


def case_reclaim_least_recently_active_first(make):
    a = make(12)
    for c in (1, 2, 3):
        a.add(c, 2, 2)
    step(a, [3], [toks(8)], 16)    # step 1
    step(a, [1], [toks(8)], 16)    # step 2
    step(a, [2], [toks(8)], 16)    # step 3: the pool is full, 2 borrowed each
    a.events()
    a.add(4, 4)
    tab, st = step(a, [4], [toks(4)], 16)
    ev = a.events()
    # borrowed pages of the least recently active context first (3, then 1)
    assert [(e["kind"], e["victim"]) for e in ev] == \
        [("reclaim_borrowed", 3)] * 2 + [("reclaim_borrowed", 1)] * 2
    assert st == ["full"] and a.counts()["reclaim_borrowed"] == 4
    # a context active in the same step, served earlier, still gives up its
    # borrowed pages to one below target; its row then shows them missing
    a.add(5, 2)
    tab, st = step(a, [2, 5], [toks(8), toks(2)], 16)
    ev = a.events()
    assert [(e["kind"], e["victim"]) for e in ev] == [("reclaim_borrowed", 2)] * 2
    assert st == ["partial", "full"]
    assert (tab[0] >= 0).sum() == 2 and tab[0][0] >= 0 and tab[0][7] >= 0
    assert not set(tab[0][tab[0] >= 0]) & set(tab[1][tab[1] >= 0])


def case_above_target_after_borrowed_then_idle_then_refuse(make):
    a = make(8)
    a.add(1, 6)
    a.add(2, 2)
    step(a, [1], [toks(6)], 8)                 # 1 holds 6 by right
    step(a, [2], [toks(2)], 8)                 # 2 holds 2
    a.events()
    a.set_target(1, 3)                         # operator lowers 1's right
    a.add(3, 4)
    tab, st = step(a, [2, 3], [toks(2), toks(4)], 8)
    ev = a.events()
    assert st == ["full", "full"]
    # pool is full: 3 pages above target from context 1 (now at its target),
    # then context 1 is idle and evicted whole for the last one
    k = kinds(ev)
    assert k[:3] == ["reclaim_above_target"] * 3 and all(e["victim"] == 1 for e in ev[:3])
    assert k[3:5] == ["reclaim_idle", "take_free"] and ev[3]["victim"] == 1
    assert a.counts()["free_pages"] == 2        # the rest of 1's pages
    # a new context that needs more than what is left, with both others
    # active: it takes the two free pages (sink + 1: its floor) and runs
    a.add(4, 4)
    tab, st = step(a, [2, 3, 4], [toks(2), toks(4), toks(4)], 8)
    assert st == ["full", "full", "partial"]
    a.events()
    # one more, with everyone active and nothing free or reclaimable: refused
    a.add(5, 2)
    tab, st = step(a, [2, 3, 4, 5], [toks(2), toks(4), toks(4), toks(2)], 8)
    assert st[3] == "refused" and (tab[3] == -1).all()
    ev = a.events()
    assert kinds(ev) == ["refused"] and a.counts()["refused"] == 1


def case_shrink_from_oldest_keeps_the_tail(make):
    a = make(4)
    a.add(1, 8)
    tab, st = step(a, [1], [toks(4)], 8)
    held = {lp: p for lp, p in enumerate(tab[0]) if p >= 0}
    a.events()
    tab, st = step(a, [1], [toks(5)], 8)
    ev = a.events()
    # no page outside the window, none free, none to reclaim: the oldest
    # non-sink page (logical 1) goes to the new tail page
    assert kinds(ev) == ["shrink_own"] and ev[0]["page"] == held[1] and ev[0]["logical"] == 4
    assert st == ["partial"]
    assert list(tab[0][:5]) == [held[0], -1, held[2], held[3], held[1]]


def case_floor_refuses_a_context_with_only_its_sink(make):
    a = make(3)
    a.add(1, 2)
    a.add(2, 2)
    step(a, [1], [toks(2)], 4)
    tab, st = step(a, [1, 2], [toks(2), toks(3)], 4)
    # context 2 gets the last free page as its sink, then finds nothing for
    # a second page: below its floor, refused for the step
    assert st == ["full", "refused"]
    # a single-page history needs only its sink
    a.add(3, 2)
    a.remove(2)
    tab, st = step(a, [3], [10], 4)
    assert st == ["full"]


def case_remove_returns_pages_lowest_first(make):
    a = make(6)
    a.add(1, 4)
    step(a, [1], [toks(4)], 4)
    assert a.counts()["free_pages"] == 2
    a.remove(1)
    a.add(2, 6)
    tab, st = step(a, [2], [toks(6)], 8)
    # every page is free again; the sink takes 0 and the newest pages
    # downward take 1, 2, ... (R4)
    assert st == ["full"] and list(tab[0][:6]) == [0, 5, 4, 3, 2, 1]


def case_raised_target_turns_borrowed_pages_into_right(make):
    a = make(5)
    a.add(1, 2, 3)
    tab, st = step(a, [1], [toks(5)], 8)       # 2 by right, 3 borrowed
    assert st == ["full"] and (tab[0] >= 0).sum() == 5
    a.set_target(1, 4)                         # now 4 by right: 1 borrowed left (R8)
    a.add(2, 2)
    a.events()
    tab, st = step(a, [2], [toks(2)], 8)
    ev = a.events()
    # the one borrowed page (1's oldest non-sink), then 1 holds exactly its
    # target and is idle, so it is evicted whole for the second page
    assert [(e["kind"], e["victim"]) for e in ev] == \
        [("reclaim_borrowed", 1), ("reclaim_idle", 1), ("take_free", -1)]
    assert ev[0]["logical"] == 0 and ev[2]["logical"] == 1
    assert st == ["full"]


def case_shorter_history_reuses_pages_past_its_end(make):
    a = make(8)
    a.add(1, 2)
    tab, st = step(a, [1], [toks(4)], 8)       # sink and logical page 3
    assert list(tab[0][:4]) == [0, -1, -1, 1]
    a.events()
    tab, st = step(a, [1], [toks(2)], 8)       # the history is now 2 pages long
    ev = a.events()
    # logical page 3 is outside the window [1, 2): its page moves to 1 (R3)
    assert kinds(ev) == ["reuse_own"] and ev[0]["page"] == 1 and ev[0]["logical"] == 1
    assert st == ["full"] and list(tab[0][:4]) == [0, 1, -1, -1]
    assert a.counts()["free_pages"] == 6


CASES = [case_free_pages_fill_sink_then_newest,
         case_sliding_window_reuses_own_page_and_keeps_sink,
         case_burst_borrows_only_while_free_and_is_reclaimed_first,
         case_reclaim_least_recently_active_first,
         case_above_target_after_borrowed_then_idle_then_refuse,
         case_shrink_from_oldest_keeps_the_tail,
         case_floor_refuses_a_context_with_only_its_sink,
         case_remove_returns_pages_lowest_first,
         case_raised_target_turns_borrowed_pages_into_right,
         case_shorter_history_reuses_pages_past_its_end]


# ----------------------------------------------------------------------------
# planted mistakes in the oracle


class MostRecentVictim(OA.Admission):
    """Victims most recently active first."""

    def _victims(self, cid):
        return list(reversed(super()._victims(cid)))


class AboveTargetBeforeBorrowed(OA.Admission):
    SOURCES = ("_own_outside_window", "_free_page", "_reclaim_above_target",
               "_reclaim_borrowed", "_reclaim_idle", "_shrink_from_oldest")


class ShrinkDropsTheTail(OA.Admission):
    """Shrink moves the newest page below the wanted one, not the oldest."""

    def _shrink_from_oldest(self, c, lp, lo, need):
        below = [x for x in c.pages if 0 < x < lp]
        if not below:
            return None
        page = c.pages.pop(max(below))
        self._event("shrink_own", c.id, c.id, page, lp)
        return page


class WindowIgnoresBurst(OA.Admission):
    """The window holds the target only, never the burst."""

    def add(self, cid, target, burst=0):
        super().add(cid, target, 0)


class ReuseOnlyBelowWindow(OA.Admission):
    """A page past the end of a shortened history is not outside the window."""

    def _own_outside_window(self, c, lp, lo, need):
        old = c.oldest_non_sink_below(lo)
        if old is None:
            return None
        page = c.pages.pop(old)
        self._event("reuse_own", c.id, c.id, page, lp)
        return page


class IdleEvictsActive(OA.Admission):
    """The third pass also evicts contexts active in this step."""

    def _reclaim_idle(self, c, lp, lo, need):
        if c.held() >= c.target:
            return None
        for v in self._victims(c.id):
            if v.pages:
                self.free |= set(v.pages.values())
                v.pages = {}
                v.borrowed = 0
                self._event("reclaim_idle", c.id, v.id, -1, -1)
                return self._take_free(c, lp)
        return None


class NoFloor(OA.Admission):
    """A context holding only its sink runs anyway."""

    def step(self, ids, lengths, pt_stride):
        saved, OA.FLOOR = OA.FLOOR, 1
        try:
            return super().step(ids, lengths, pt_stride)
        finally:
            OA.FLOOR = saved


class BorrowNotCounted(OA.Admission):
    """Pages taken beyond the target are not marked borrowed."""

    def _free_page(self, c, lp, lo, need):
        if not self.free or c.held() >= c.target + c.burst:
            return None
        return self._take_free(c, lp)


class TargetNotClamped(OA.Admission):
    """A raised target leaves the borrowed count as it was."""

    def set_target(self, cid, target, burst=0):
        c = self.contexts[cid]
        c.target, c.burst = target, burst


class HighestFreePage(OA.Admission):
    def _take_free(self, c, lp):
        page = max(self.free)
        self.free.remove(page)
        self._event("take_free", c.id, -1, page, lp)
        return page


MUTANTS = [MostRecentVictim, AboveTargetBeforeBorrowed, ShrinkDropsTheTail, WindowIgnoresBurst,
           ReuseOnlyBelowWindow,
           IdleEvictsActive, NoFloor, BorrowNotCounted, TargetNotClamped, HighestFreePage]


# ----------------------------------------------------------------------------
# tests


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.__name__)
def test_oracle_pin(case):
    case(OA.Admission)


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_planted_mistake_is_caught(mutant):
    caught = []
    for case in CASES:
        try:
            case(mutant)
        except AssertionError:
            caught.append(case.__name__)
    assert caught, f"{mutant.__name__} passed every hand case"


def test_refusals():
    with pytest.raises(ValueError):
        OA.Admission(0)                       # an automatic size is refused
    a = OA.Admission(8)
    with pytest.raises(ValueError):
        a.add(1, 1)                           # below the floor
    a.add(1, 2)
    for ids, lens in (([2], [10]), ([1, 1], [10, 10]), ([1], [0]), ([1], [toks(9)])):
        with pytest.raises(ValueError):
            a.step(ids, lens, 8)
    assert a.counts()["steps"] == 0
