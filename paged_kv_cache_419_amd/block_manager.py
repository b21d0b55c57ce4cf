"""The control-plane block manager (C++ in libpagedkv.so), wrapped for Python.

It turns sequences of token ids into the block tables, slot mappings and
lengths the data-plane calls take ("Nano-vLLM part 1", sections 3.2 and 4):
fixed-size blocks, prefix caching through chained block hashes with reference
counts, a free list whose blocks keep their content until handed out again,
and "no space" answers on which the caller preempts a sequence.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Sequence

import numpy as np

from . import binding

NO_SPACE = -1
ERR_ARG = -2


def _ints(values: Sequence[int]):
    a = np.ascontiguousarray(np.asarray(values, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


class NoSpace(RuntimeError):
    """Not enough free blocks; the manager is unchanged (preempt a sequence)."""


def _library() -> ctypes.CDLL:
    # PKV_BM_LIBRARY names a host-only build of the same C++ source (the CPU tests
    # load one built with AddressSanitizer and UndefinedBehaviorSanitizer)
    path = os.environ.get("PKV_BM_LIBRARY")
    return binding.load_block_manager(path) if path else binding.load()


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int = 256):
        self._lib = _library()
        self._h = self._lib.pkv_bm_create(num_blocks, block_size)
        if not self._h:
            raise ValueError(f"bad sizes: {num_blocks} blocks of {block_size} tokens")
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self) -> None:
        if self._h:
            self._lib.pkv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def _check(self, r: int, what: str) -> int:
        if r == NO_SPACE:
            raise NoSpace(what)
        if r == ERR_ARG:
            raise ValueError(f"{what}: invalid argument or sequence id")
        return r

    @property
    def num_free(self) -> int:
        return self._lib.pkv_bm_num_free(self._h)

    def allocate(self, seq_id: int, tokens: Sequence[int]) -> int:
        """Admit a sequence; returns how many leading tokens are already cached."""
        a, p = _ints(tokens)
        return self._check(self._lib.pkv_bm_allocate(self._h, seq_id, p, len(a)), "allocate")

    def append(self, seq_id: int, token: int) -> None:
        self._check(self._lib.pkv_bm_append(self._h, seq_id, int(token)), "append")

    def free(self, seq_id: int) -> None:
        self._check(self._lib.pkv_bm_free(self._h, seq_id), "free")

    def seq_len(self, seq_id: int) -> int:
        return self._check(self._lib.pkv_bm_seq_len(self._h, seq_id), "seq_len")

    def block_table(self, seq_id: int, width: int = 0) -> np.ndarray:
        n = self._check(self._lib.pkv_bm_block_table(self._h, seq_id, None, 0), "block_table")
        out = np.full(max(width, n), -1, dtype=np.int32)
        self._lib.pkv_bm_block_table(self._h, seq_id, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                     len(out))
        return out

    def slots(self, seq_id: int, start: int, stop: int) -> np.ndarray:
        out = np.empty(max(stop - start, 0), dtype=np.int32)
        self._check(self._lib.pkv_bm_slots(self._h, seq_id, start, stop,
                                           out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))),
                    "slots")
        return out

    def ref_count(self, block_id: int) -> int:
        return self._check(self._lib.pkv_bm_ref_count(self._h, block_id), "ref_count")

    def tables(self, seq_ids: Sequence[int], width: int = 0) -> np.ndarray:
        """Block tables of several sequences, padded with -1 to a common width."""
        rows: List[np.ndarray] = [self.block_table(s) for s in seq_ids]
        w = max([width] + [len(r) for r in rows])
        out = np.full((len(rows), w), -1, dtype=np.int32)
        for i, r in enumerate(rows):
            out[i, :len(r)] = r
        return out
