"""Oracle of the expert slot bank (test infrastructure only).

The pages keep routed experts outside the dense model and page them through
a bounded cache of expert slots whose size trades memory for fewer reads
(Anemll/ds4-ssd README, section "Run SSD Sidecar Mode": --moe-slot-bank caps
the resident routed-expert slots, --ssd-cache sizes them in bytes; the
10100.com article on ds4-ssd, section 核心功能).  They name no replacement
policy.  The reading taken: least recently used, with these rules for one
pass over a set of wanted experts (at most N of them, N = slots):

* a wanted expert already in a slot is a hit;
* each miss, in the order the pass lists them, goes to the lowest-numbered
  empty slot, else to the slot whose expert was used longest ago among the
  experts this pass does not want (lowest slot number on a tie; ties cannot
  happen once every slot has been used, since uses are numbered);
* after the misses, the pass's experts are marked used, in the pass's order.

A layer call routes its tokens, takes the experts with at least one routed
pair -- the resident ones first, then the others, each group in id order --
and splits them into passes of at most N experts.

Everything here is plain Python over lists, written to be read against the
rules above.
"""

from __future__ import annotations


class SlotBank:
    """State of an N-slot bank over E experts: which expert each slot holds
    (None when empty) and the use number of the slot's last use."""

    def __init__(self, E: int, N: int):
        if not (1 <= E <= 64 and 1 <= N <= E):
            raise ValueError("need 1 <= N <= E <= 64")
        self.E, self.N = E, N
        self.holder = [None] * N          # slot -> expert
        self.used_at = [0] * N            # slot -> use number of its last use
        self.uses = 0                     # use numbers handed out so far

    def slot_of(self, e: int):
        for s in range(self.N):
            if self.holder[s] == e:
                return s
        return None

    def plan(self, want: list[int]) -> list[tuple[int, int]]:
        """One pass: returns the loads [(expert, slot), ...] in miss order and
        updates the state."""
        if len(want) > self.N or len(set(want)) != len(want):
            raise ValueError("a pass wants at most N distinct experts")
        if any(not (0 <= e < self.E) for e in want):
            raise ValueError("expert id out of range")
        loads = []
        for e in want:
            if self.slot_of(e) is not None:
                continue
            empty = [s for s in range(self.N) if self.holder[s] is None]
            if empty:
                slot = empty[0]
            else:
                candidates = [s for s in range(self.N) if self.holder[s] not in want]
                oldest = min(self.used_at[s] for s in candidates)
                slot = [s for s in candidates if self.used_at[s] == oldest][0]
            self.holder[slot] = e
            loads.append((e, slot))
        for e in want:
            self.uses += 1
            self.used_at[self.slot_of(e)] = self.uses
        return loads


def layer_passes(bank: SlotBank, active: list[int]) -> list[list[int]]:
    """The passes of one layer call over the experts `active` (those with at
    least one routed pair): resident ones first, then the others, each in id
    order, cut into groups of at most N."""
    resident = sorted(e for e in set(active) if bank.slot_of(e) is not None)
    others = sorted(e for e in set(active) if bank.slot_of(e) is None)
    order = resident + others
    if not order:
        return [[]]
    return [order[i:i + bank.N] for i in range(0, len(order), bank.N)]


def run_layer_calls(E: int, N: int, calls: list[list[int]]) -> list[dict]:
    """Replays a sequence of layer calls (each the list of routed expert ids
    of that call, repeats allowed) on a fresh bank; per call, the hits
    (active experts resident at the start), the loads of every pass and the
    slot each active expert was computed from."""
    bank = SlotBank(E, N)
    out = []
    for ids in calls:
        active = sorted(set(ids))
        passes = layer_passes(bank, active)
        hits = sum(1 for e in active if bank.slot_of(e) is not None)
        loads, slot_used = [], {}
        for want in passes:
            loads.append(bank.plan(want))
            for e in want:
                slot_used[e] = bank.slot_of(e)
        out.append(dict(active=len(active), hits=hits, passes=len(passes), loads=loads, slot_used=slot_used,
                        holder=list(bank.holder)))
    return out
