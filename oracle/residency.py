"""Oracle for the online precision-residency policy -- TEST INFRASTRUCTURE.

Only the tests may import this module; the GPU library never does, and this
module imports nothing from it.

Page "Dynamic Expert Quantization for Scalable Mixture-of-Experts Inference"
(DynaExq):
  * section 2.5 / 3.5 "online scheduling policy": per-expert counters of
    router selections over an update interval are folded into a smoothed
    score S <- alpha S + (1 - alpha) c; the high-precision set is the top
    n_hi experts by score (n_hi fixed by the memory budget); promotion
    candidates are the target set minus the current set, demotion candidates
    the reverse;
  * "stability hysteresis": an expert enters only if its score beats the
    lowest-ranked member of the current set by a margin, and a member leaves
    only if its score is below the highest-ranked outsider by the same
    margin; the budget constraint is unchanged.
  * section 2.3 / 3.3 "budget model": a promotion is admitted only after an
    explicit reservation succeeds against the capacity left once the fixed
    part is set aside.

Readings (the pages give the rules in words only):
  * ranking ties go to the lower expert index ("hottest" = highest score,
    then lowest index; "coldest" = lowest score, then highest index);
  * while the current set has free capacity, the hottest outsiders with a
    positive score fill it without a margin (no member has to leave, so
    nothing can oscillate); only swaps against members need the margin;
  * swaps pair the j-th hottest outsider with the j-th coldest member and stop
    at the first pair that fails the margin test, which is both conditions of
    the page at once: S_out > S_mem + margin;
  * if the capacity shrank below the set's size, the coldest members leave
    first;
  * experts whose transition is still in flight ("locked") keep their
    membership and are never paired;
  * the margin test runs in fp32 (the scores are fp32 on the device), so
    S_mem + margin is rounded to fp32 before the comparison.

Parity status: pinned in tests/test_oracle_pins.py against brute force over
all sets of tiny N (fewest swaps to a state with no pair violating the
margin), a plain numpy top-n for margin 0, and a hand-worked example in
tests/golden/residency_hysteresis.json.
"""
from __future__ import annotations

import numpy as np


def ema_fold(S, counts, alpha: float) -> np.ndarray:
    """S <- alpha S + (1 - alpha) c with c = the counts summed over the
    interval's steps (counts: iterable of [N] integer arrays), in float64."""
    c = np.zeros(len(S), dtype=np.float64)
    for cnt in counts:
        c += np.asarray(cnt, dtype=np.float64)
    return alpha * np.asarray(S, dtype=np.float64) + (1.0 - alpha) * c


def _hotter(S, a: int, b: int) -> bool:
    """True when expert a ranks above expert b (score desc, index asc)."""
    return S[a] > S[b] or (S[a] == S[b] and a < b)


def _sort_hottest_first(S, experts):
    # a plain insertion sort keeps the rank rule explicit
    out = []
    for e in experts:
        j = len(out)
        out.append(e)
        while j > 0 and _hotter(S, out[j], out[j - 1]):
            out[j], out[j - 1] = out[j - 1], out[j]
            j -= 1
    return out


def select(S, in_hi, n_hi: int, margin: float, locked=None):
    """One policy update.

    S      : [N] fp32 scores
    in_hi  : [N] bool, membership of the current high-precision set (experts
             being promoted count as members)
    n_hi   : capacity in experts
    margin : additive hysteresis margin (>= 0)
    locked : [N] bool or None, experts whose membership may not change now

    Returns (target [N] bool, promote list, demote list); promote lists the
    experts in the order they should be admitted (hottest first), demote the
    coldest first.
    """
    S = np.asarray(S, dtype=np.float32)
    N = len(S)
    in_hi = np.asarray(in_hi, dtype=bool)
    locked = np.zeros(N, dtype=bool) if locked is None else np.asarray(locked, dtype=bool)
    members = [e for e in range(N) if in_hi[e]]
    promote, demote = [], []

    # capacity shrink: the coldest movable members leave first
    size = len(members)
    movable_cold_first = list(reversed(_sort_hottest_first(S, [e for e in members if not locked[e]])))
    while size > n_hi and movable_cold_first:
        demote.append(movable_cold_first.pop(0))
        size -= 1

    outsiders = _sort_hottest_first(S, [e for e in range(N) if not in_hi[e] and not locked[e] and S[e] > 0])
    free = n_hi - size
    while free > 0 and outsiders:
        promote.append(outsiders.pop(0))
        free -= 1

    # hysteresis swaps: j-th hottest outsider against j-th coldest member
    m32 = np.float32(margin)
    for o, m in zip(outsiders, movable_cold_first):
        if S[o] > np.float32(S[m] + m32):
            promote.append(o)
            demote.append(m)
        else:
            break

    target = in_hi.copy()
    target[demote] = False
    target[promote] = True
    return target, promote, demote


class Budget:
    """The budget tracker as the page defines it: reservations succeed only
    while they fit in the capacity (total minus the fixed part)."""

    def __init__(self, total: int, fixed: int):
        self.capacity = total - fixed
        self.used = 0

    def try_reserve(self, nbytes: int) -> bool:
        if self.used + nbytes > self.capacity:
            return False
        self.used += nbytes
        return True

    def release(self, nbytes: int) -> None:
        assert nbytes <= self.used
        self.used -= nbytes
