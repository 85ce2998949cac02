"""Block arena bookkeeping of the oracle: LIFO free-list and frame registry.

"Rebuilding Kshipra Around Memory", §1 (Block-Arena KV Cache): KV memory is
reserved once as fixed-size blocks; the free-list is a Python list initialised
to range(num_blocks), so ``pop()`` hands out the highest id first and a freed
block is appended and reused by the very next allocation (LIFO).

"Can an LLM Forget the Right Things?", §5: frames are the unit of eviction;
the FIFO baseline evicts until enough slots are free and reports failure when
no frame is left; the semantic policy removes a frame and shifts the retained
frames down (keys keep their rotation: nothing is recomputed).

Readings fixed here (the pages are silent): a frame is one prefill chunk or one
raw append and always starts on a fresh block; decode tokens form a
non-evictable tail segment that also starts on a fresh block; eviction pushes a
frame's blocks in logical order, so the next pops return them reversed;
positions come from a monotonic counter and are never reused.
"""
from __future__ import annotations

from dataclasses import dataclass, field


class NoBlocks(Exception):
    """Not enough free blocks; the state is left unchanged."""


class NothingToEvict(Exception):
    """Fewer than two evictable frames."""


class BlockPool:
    """LIFO free-list over block ids 0..n-1."""

    def __init__(self, num_blocks: int, initial=None):
        self.num_blocks = num_blocks
        # initial free-list order; default range(n) so pop() returns n-1 first
        self.free = list(range(num_blocks)) if initial is None else list(initial)

    def alloc(self, n: int) -> list[int]:
        if n > len(self.free):
            raise NoBlocks(f"need {n} blocks, {len(self.free)} free")
        return [self.free.pop() for _ in range(n)]

    def release(self, blocks) -> None:
        for b in blocks:
            self.free.append(b)


@dataclass
class Segment:
    kind: str              # "frame" or "tail"
    frame_id: int          # -1 for a decode tail
    start_pos: int         # absolute RoPE position of the first token
    ntok: int
    blocks: list = field(default_factory=list)

    @property
    def positions(self):
        return list(range(self.start_pos, self.start_pos + self.ntok))
