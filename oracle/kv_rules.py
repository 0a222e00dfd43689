"""Plain reference model of the dual-pool KV manager's rules.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): only the tests may
import it.  It shares no code with the HIP library and never imports it.

Every rule is written the slow, obvious way -- the full-attention pool as one
owner entry per row, scanned from row 0; the reuse length by trying every
length -- so that it can be checked by eye against the pages:

* gokawiil "Full-Pipeline Inference Optimization for MiMo-V2.5 Series",
  section 2.1 "SWA KVCache Management": full-attention layers keep O(N) rows
  per sequence, windowed layers O(W) (the ring); a request is admitted only if
  BOTH pools have room (admission checks the capacity of each pool, not
  one combined figure); prefix reuse is clipped to the
  "window-safe length", the longest matched prefix whose last W positions the
  windowed layers still hold (anything beyond is a miss).
* colibri "MiMo-V2.6 (Xiaomi)", section "System One mode and prompt reuse":
  a snapshot leaves the full layers' rows in place and records the token ids
  they hold; a prompt that diverged below the snapshot rewrote them and the
  snapshot is released; the windowed layers' rings are copied into the
  snapshot and back, and the snapshot's position is its length.

Readings where the pages leave a step open:
* pool rows are handed out as one contiguous run per sequence (the attention
  calls address rows as seq_base + position), at the lowest row where
  ``max_len`` free rows start; the ring slot is the lowest free one;
* every ring slot holds one position (colibri "System One mode": position p
  lives in slot p mod W).  Appending tokens means the caller runs the
  attention calls over them, which write each appended position into its
  slot; a truncate writes nothing; a restore brings back the slots the
  snapshot copied.  The model records, per sequence, the position each slot
  holds, and nothing else about the rings;
* the windowed state at length L exists when the rings hold the positions the
  next token's window reads from them, max(0, L - W + 1) .. L - 1 (the token
  at L goes into its own slot first).  Live candidates are the lengths up to
  the live length (a truncate reaches them); a snapshot is a candidate at its
  own position when its copied slots hold that window.  Of equal lengths the
  live state is preferred, then the lowest snapshot id;
* a snapshot is released as soon as an append writes a token id different
  from the one its row held at a position below the snapshot's, and never
  comes back.
"""
from __future__ import annotations


class KvModel:
    CAPACITY, STALE, SHAPE = "capacity", "stale", "shape"

    def __init__(self, ring_seqs: int, pool_rows: int, max_snapshots: int, window: int = 128):
        self.window = window
        self.owner = [None] * pool_rows          # sequence owning each pool row
        self.ring = [False] * ring_seqs          # ring slot taken?
        self.seqs = {}                           # seq -> dict(base, max_len, len, rows, slots)
        self.snap_slots = [False] * max_snapshots
        self.snaps = {}                          # id -> dict(seq, pos, slot, slots)
        self.next_id = 0

    # -- admission / release --------------------------------------------
    def first_run(self, n: int):
        """Lowest row where n consecutive free rows start, or None."""
        for start in range(0, len(self.owner) - n + 1):
            if all(self.owner[r] is None for r in range(start, start + n)):
                return start
        return None

    def admit(self, max_len: int):
        if max_len < 1:
            return self.SHAPE
        slot = next((i for i, t in enumerate(self.ring) if not t), None)
        start = self.first_run(max_len)
        if slot is None or start is None:      # both pools checked, nothing taken
            return self.CAPACITY
        self.ring[slot] = True
        for r in range(start, start + max_len):
            self.owner[r] = slot
        # slots: the position each ring slot holds (None: nothing written yet)
        self.seqs[slot] = dict(base=start, max_len=max_len, len=0, rows=[], slots=[None] * self.window)
        return slot, start

    def release(self, seq: int):
        if seq not in self.seqs:
            return self.SHAPE
        s = self.seqs.pop(seq)
        for r in range(s["base"], s["base"] + s["max_len"]):
            self.owner[r] = None
        self.ring[seq] = False
        for sid in [k for k, v in self.snaps.items() if v["seq"] == seq]:
            self._drop(sid)
        return None

    # -- token record ----------------------------------------------------
    def append(self, seq: int, tokens):
        if seq not in self.seqs:
            return self.SHAPE
        s = self.seqs[seq]
        if s["len"] + len(tokens) > s["max_len"]:
            return self.CAPACITY
        start = s["len"]
        for i, t in enumerate(tokens):
            p = start + i
            if p < len(s["rows"]):
                if s["rows"][p] != t:
                    # row p now holds another history: snapshots above it go
                    for sid in [k for k, v in self.snaps.items() if v["seq"] == seq and v["pos"] > p]:
                        self._drop(sid)
                    s["rows"][p] = t
            else:
                s["rows"].append(t)
            s["slots"][p % self.window] = p    # the attention calls write position p's K/V
        s["len"] = start + len(tokens)
        return start

    def truncate(self, seq: int, new_len: int):
        if seq not in self.seqs or not 0 <= new_len <= self.seqs[seq]["len"]:
            return self.SHAPE
        self.seqs[seq]["len"] = new_len
        return None

    def info(self, seq: int):
        if seq not in self.seqs:
            return self.SHAPE
        s = self.seqs[seq]
        return s["len"], s["base"], s["max_len"]

    def free_space(self):
        run = best = 0
        for o in self.owner:
            run = run + 1 if o is None else 0
            best = max(best, run)
        return self.ring.count(False), best, self.snap_slots.count(False)

    # -- snapshots -------------------------------------------------------
    def snapshot(self, seq: int):
        if seq not in self.seqs:
            return self.SHAPE
        slot = next((i for i, t in enumerate(self.snap_slots) if not t), None)
        if slot is None:
            return self.CAPACITY
        self.snap_slots[slot] = True
        sid = self.next_id
        self.next_id += 1
        self.snaps[sid] = dict(seq=seq, pos=self.seqs[seq]["len"], slot=slot,
                               slots=list(self.seqs[seq]["slots"]))
        return sid

    def _drop(self, sid: int):
        self.snap_slots[self.snaps[sid]["slot"]] = False
        del self.snaps[sid]

    def drop_snapshot(self, sid: int):
        if sid not in self.snaps:
            return self.STALE
        self._drop(sid)
        return None

    def restore(self, sid: int):
        if sid not in self.snaps:
            return self.STALE
        sn = self.snaps[sid]
        self.seqs[sn["seq"]]["len"] = sn["pos"]
        self.seqs[sn["seq"]]["slots"] = list(sn["slots"])
        return sn["seq"], sn["slot"]

    # -- reuse -----------------------------------------------------------
    def holds_window(self, slots, L: int) -> bool:
        """Do these slots hold every position the window of the token at L
        reads from the ring, max(0, L - W + 1) .. L - 1?"""
        return all(slots[p % self.window] == p for p in range(max(0, L - self.window + 1), L))

    def window_safe_length(self, seq: int, tokens):
        """Brute force over every length L: the first L ids must equal the
        ids the rows hold, and the windowed state must exist at L."""
        if seq not in self.seqs:
            return None
        s = self.seqs[seq]
        best, snap = 0, -1
        for L in range(0, len(tokens) + 1):
            if L > len(s["rows"]) or list(tokens[:L]) != s["rows"][:L]:
                continue
            if L <= s["len"] and self.holds_window(s["slots"], L) and L > best:
                best, snap = L, -1
            for sid in sorted(self.snaps):
                sn = self.snaps[sid]
                if sn["seq"] == seq and sn["pos"] == L and self.holds_window(sn["slots"], L) and L > best:
                    best, snap = L, sid
        return best, snap
