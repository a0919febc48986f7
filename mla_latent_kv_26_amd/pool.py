"""Paged latent-cache pool with a host-side block allocator.

The pool is one device tensor [num_blocks, block_size, R + Dr]; sequences own
lists of physical blocks handed out by a free list, and a page table row
lists a sequence's blocks in logical order (the ticket "MLA + KV cache
(Tier 3 #5)", "Description": a PagedKVCache pool with a block allocator).
The allocator is bookkeeping only; rows are written by the library
(mla_cache_append / mla_prefill).
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional

import torch

from .api import MLAConfig


class LatentKVPool:
    def __init__(self, cfg: MLAConfig, num_blocks: int, device="cuda", zero: bool = True):
        if num_blocks <= 0:
            raise ValueError("num_blocks must be positive")
        self.cfg = cfg
        self.num_blocks = num_blocks
        shape = (num_blocks, cfg.block_size, cfg.pool_row)
        alloc = torch.zeros if zero else torch.empty
        self.data = alloc(shape, dtype=cfg.pool_dtype, device=device)
        self._free: List[int] = list(range(num_blocks - 1, -1, -1))
        self._blocks: Dict[int, List[int]] = {}
        self._len: Dict[int, int] = {}

    # -- allocator ---------------------------------------------------------
    @property
    def free_blocks(self) -> int:
        return len(self._free)

    def blocks(self, seq_id: int) -> List[int]:
        return list(self._blocks.get(seq_id, []))

    def length(self, seq_id: int) -> int:
        return self._len.get(seq_id, 0)

    def reserve(self, seq_id: int, new_len: int) -> List[int]:
        """Grow sequence seq_id to hold new_len tokens; returns its blocks."""
        bs = self.cfg.block_size
        blocks = self._blocks.setdefault(seq_id, [])
        need = -(-new_len // bs) - len(blocks)
        if need > len(self._free):
            raise MemoryError(f"pool exhausted: need {need} blocks, {len(self._free)} free")
        for _ in range(max(need, 0)):
            blocks.append(self._free.pop())
        self._len[seq_id] = max(self._len.get(seq_id, 0), new_len)
        return list(blocks)

    def release(self, seq_id: int) -> None:
        for b in self._blocks.pop(seq_id, []):
            self._free.append(b)
        self._len.pop(seq_id, None)

    # -- tables ------------------------------------------------------------
    def block_table(self, seq_ids: Iterable[int], max_blocks: Optional[int] = None,
                    device=None) -> torch.Tensor:
        ids = list(seq_ids)
        mb = max_blocks or max(1, max(len(self._blocks.get(s, [])) for s in ids))
        t = torch.zeros((len(ids), mb), dtype=torch.int32)
        for i, s in enumerate(ids):
            bl = self._blocks.get(s, [])
            if len(bl) > mb:
                raise ValueError(f"sequence {s} has {len(bl)} blocks > max_blocks {mb}")
            t[i, :len(bl)] = torch.tensor(bl, dtype=torch.int32)
        return t.to(device or self.data.device)

    def seq_lens(self, seq_ids: Iterable[int], device=None) -> torch.Tensor:
        return torch.tensor([self._len.get(s, 0) for s in seq_ids], dtype=torch.int32,
                            device=device or self.data.device)

    def slot_mapping(self, seq_id: int, positions: Iterable[int], device=None) -> torch.Tensor:
        bs = self.cfg.block_size
        bl = self._blocks[seq_id]
        slots = [bl[p // bs] * bs + p % bs for p in positions]
        return torch.tensor(slots, dtype=torch.int32, device=device or self.data.device)
