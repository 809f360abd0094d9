"""Host model of the token-commit protocol (plain Python, no GPU).

TEST INFRASTRUCTURE ONLY: like ``oracle/sampler.py``, only ``tests/`` may use
it; the product never does.

Arc PR #217 ("device decode loop"), "What this does", step 3, and the fault
handling that follows it describe what one decode step commits: the step's
tokens go into the input buffer of the next step, the device position moves
on, and the tokens are published into a pinned host ring that the host drains
with plain loads; the commit checks the tokens and the position before it
writes anything and reports a refusal through a sticky fault word instead of
blocking.  This model restates that protocol, with the readings the library
documents for what the page leaves open:

* a token of -1 (the sampler's mark for a row it refused, whose reason is in
  that row's status) is published as -1 and is not a fault;
* any other token outside [0, V) refuses the step with FAULT_TOKEN_RANGE;
* the step is refused with FAULT_RING_OVERRUN when its slot, position % capacity,
  still holds a step the host has not drained (position - drained >= capacity);
* while the fault word is set every step is refused and nothing is written;
  the first fault code stays until the host clears the word;
* otherwise next_input = ids, ring[position % capacity] = ids, then
  published = position + 1 and position = position + 1.
"""

from __future__ import annotations

from typing import List, Optional

FAULT_NONE = 0
FAULT_TOKEN_RANGE = 1
FAULT_RING_OVERRUN = 2
REFUSED_ROW = -1


class CommitModel:
    def __init__(self, B: int, V: int, capacity: int, fill: int = -7):
        self.B, self.V, self.capacity = B, V, capacity
        self.position = 0
        self.published = 0
        self.drained = 0           # written by the host
        self.fault = FAULT_NONE    # written by the commit, cleared by the host
        self.ring: List[List[int]] = [[fill] * B for _ in range(capacity)]
        self.next_input: Optional[List[int]] = None

    def commit(self, ids) -> bool:
        """One commit; returns whether the step was published."""
        ids = [int(t) for t in ids]
        assert len(ids) == self.B
        bad = any((t < 0 and t != REFUSED_ROW) or t >= self.V for t in ids)
        code = FAULT_NONE
        if bad:
            code = FAULT_TOKEN_RANGE
        elif self.position - self.drained >= self.capacity:
            code = FAULT_RING_OVERRUN
        latched = self.fault
        if latched == FAULT_NONE and code != FAULT_NONE:
            self.fault = code
        if latched != FAULT_NONE or code != FAULT_NONE:
            return False
        self.next_input = list(ids)
        self.ring[self.position % self.capacity] = list(ids)
        self.published = self.position + 1
        self.position += 1
        return True
