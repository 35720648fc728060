"""Integer model of the ring cursors (test infrastructure only).

Three int32 cursors per slot, shared by every layer (replayssm(B)SpecDecode
App. A.1: block-keyed write_pos / cache_base / is_flush_flags):

* ``cache_base`` - physical start of the committed history, the ring's head
  (replayssm(B)SpecDecode §10.1-10.2);
* ``write_pos``  - number of committed records after the checkpoint, also the
  logical position of the next window (§4.1, §10.2);
* ``is_flush``   - the next verify must fold the history into the checkpoint.

Logical position j of a slot lives at (cache_base + j) & (L - 1) (§10.1).

Advance by the accept count a (§4.2, §8.1-8.2, §9.3):
  if is_flush: cache_base = (cache_base + write_pos) & (L-1); write_pos = a
  else:        write_pos += a
  is_flush = (write_pos + 2 * max_spec_len) > L        (strict, early flush)

Reset at the prefill -> decode handoff (App. A.2): write_pos = 0,
cache_base = 0, is_flush = INIT_FLUSH.

Shared conventions with the library: rows whose slot is outside
[0, num_slots) are padding and change nothing; the accept count is clamped to
[0, T]; write_pos is clamped to [0, L - T] before use, which never binds while
the early-flush invariant holds.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class CursorState:
    write_pos: np.ndarray
    cache_base: np.ndarray
    is_flush: np.ndarray

    @staticmethod
    def zeros(num_slots: int) -> "CursorState":
        z = lambda: np.zeros(num_slots, dtype=np.int32)  # noqa: E731
        return CursorState(z(), z(), z())

    def copy(self) -> "CursorState":
        return CursorState(self.write_pos.copy(), self.cache_base.copy(), self.is_flush.copy())


def phys(cache_base: int, logical: int, L: int) -> int:
    return (int(cache_base) + int(logical)) & (L - 1)


def clamp_write_pos(wp: int, L: int, T: int) -> int:
    return min(max(int(wp), 0), L - T)


def history_len(cur: CursorState, slot: int, L: int, T: int) -> int:
    """Committed records a verify replays: none for a flagged slot."""
    if cur.is_flush[slot]:
        return 0
    return clamp_write_pos(cur.write_pos[slot], L, T)


def advance(cur: CursorState, slot_idx, accept, L: int, T: int, max_spec: int) -> None:
    num_slots = cur.write_pos.shape[0]
    for row, s in enumerate(np.asarray(slot_idx).tolist()):
        if not (0 <= s < num_slots):
            continue
        a = min(max(int(accept[row]), 0), T)
        wp = clamp_write_pos(cur.write_pos[s], L, T)
        if cur.is_flush[s]:
            cur.cache_base[s] = (int(cur.cache_base[s]) + wp) & (L - 1)
            wp = a
        else:
            wp = wp + a
        cur.write_pos[s] = wp
        cur.is_flush[s] = 1 if wp + 2 * max_spec > L else 0


def reset(cur: CursorState, slots, init_flush: int = 0) -> None:
    num_slots = cur.write_pos.shape[0]
    for s in np.asarray(slots).tolist():
        if 0 <= s < num_slots:
            cur.write_pos[s] = 0
            cur.cache_base[s] = 0
            cur.is_flush[s] = int(init_flush)
