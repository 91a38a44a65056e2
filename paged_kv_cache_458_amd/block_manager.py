"""Python wrapper of the native block manager (include/paged_block_manager.h): argument marshalling only.

The manager hands out cache slots, copy-on-write pairs and block tables; the decode kernels move the bytes.
"""

from __future__ import annotations

import ctypes

import numpy as np

from . import PagedAttentionError, load_library

PA_ERR_NOMEM = -8
PA_ERR_SEQ = -9

STAT_NAMES = ("free_blocks", "used_blocks", "shared_blocks", "sequences", "tokens", "slots_in_used_blocks",
              "slots_holding_tokens", "cow_copies")


def _bind(lib):
    if getattr(lib, "_pa_bm_bound", False):
        return lib
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.pa_bm_create.argtypes, lib.pa_bm_create.restype = [i32, i32, i32, i32], P
    lib.pa_bm_destroy.argtypes, lib.pa_bm_destroy.restype = [P], None
    lib.pa_bm_add_sequence.argtypes, lib.pa_bm_add_sequence.restype = [P, i64, P, i32, P], i32
    lib.pa_bm_fork.argtypes, lib.pa_bm_fork.restype = [P, i64, i64], i32
    lib.pa_bm_append_slots.argtypes, lib.pa_bm_append_slots.restype = [P, P, i32, P], i32
    lib.pa_bm_take_copies.argtypes, lib.pa_bm_take_copies.restype = [P, P, i32], i32
    lib.pa_bm_free_sequence.argtypes, lib.pa_bm_free_sequence.restype = [P, i64], i32
    lib.pa_bm_block_tables.argtypes, lib.pa_bm_block_tables.restype = [P, P, i32, P, P, i32], i32
    lib.pa_bm_stats.argtypes, lib.pa_bm_stats.restype = [P, P], i32
    lib.pa_bm_set_host_pool.argtypes, lib.pa_bm_set_host_pool.restype = [P, i32], i32
    lib.pa_bm_swap_out.argtypes, lib.pa_bm_swap_out.restype = [P, i64, P, i32], i32
    lib.pa_bm_swap_in.argtypes, lib.pa_bm_swap_in.restype = [P, i64, P, i32], i32
    lib.pa_bm_swap_stats.argtypes, lib.pa_bm_swap_stats.restype = [P, P], i32
    lib._pa_bm_bound = True
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class BlockManager:
    """Refcounted pool of `num_blocks` blocks of `block_size` slots; block `reserved_block` pads tables."""

    def __init__(self, num_blocks: int, block_size: int, max_blocks_per_seq: int, reserved_block: int = -1):
        self._lib = _bind(load_library())
        self._h = self._lib.pa_bm_create(num_blocks, block_size, max_blocks_per_seq, reserved_block)
        if not self._h:
            raise ValueError("invalid block manager sizes")
        self.num_blocks, self.block_size, self.max_blocks_per_seq = num_blocks, block_size, max_blocks_per_seq
        self.reserved_block = reserved_block

    def close(self):
        if self._h:
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _check(fn, status):
        if status < 0:
            raise PagedAttentionError(fn, status)
        return status

    def add_sequence(self, seq_id: int, num_tokens: int, tokens=None) -> np.ndarray:
        """Slots of the prompt tokens (-1 where the token lives in a shared prefix block)."""
        slots = np.empty(max(num_tokens, 1), dtype=np.int32)
        tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
        if tok is not None and tok.size != num_tokens:
            raise ValueError("tokens must hold num_tokens ids")
        self._check("pa_bm_add_sequence", self._lib.pa_bm_add_sequence(
            self._h, seq_id, None if tok is None else _ptr(tok), num_tokens, _ptr(slots)))
        return slots[:num_tokens]

    def fork(self, parent_id: int, child_id: int):
        self._check("pa_bm_fork", self._lib.pa_bm_fork(self._h, parent_id, child_id))

    def append_slots(self, seq_ids) -> np.ndarray:
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        slots = np.empty(max(ids.size, 1), dtype=np.int32)
        self._check("pa_bm_append_slots", self._lib.pa_bm_append_slots(self._h, _ptr(ids), ids.size, _ptr(slots)))
        return slots[: ids.size]

    def take_copies(self) -> np.ndarray:
        """Pending copy-on-write pairs [P, 2] = (src, dst), in the order they arose."""
        cap = self.num_blocks
        buf = np.empty((cap, 2), dtype=np.int32)
        n = self._check("pa_bm_take_copies", self._lib.pa_bm_take_copies(self._h, _ptr(buf), cap))
        return buf[:n].copy()

    def free_sequence(self, seq_id: int):
        self._check("pa_bm_free_sequence", self._lib.pa_bm_free_sequence(self._h, seq_id))

    def block_tables(self, seq_ids, pad: int | None = None):
        """(tables int32 [n, max_blocks_per_seq], context lengths int32 [n])."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = ids.size
        tables = np.empty((max(n, 1), self.max_blocks_per_seq), dtype=np.int32)
        lens = np.empty(max(n, 1), dtype=np.int32)
        pad = self.reserved_block if pad is None else pad
        self._check("pa_bm_block_tables", self._lib.pa_bm_block_tables(self._h, _ptr(ids), n, _ptr(tables),
                                                                         _ptr(lens), pad))
        return tables[:n], lens[:n]

    def set_host_pool(self, num_host_blocks: int):
        """Host blocks [0, num_host_blocks) of the caller's pinned host pools receive swapped-out sequences."""
        self._check("pa_bm_set_host_pool", self._lib.pa_bm_set_host_pool(self._h, num_host_blocks))
        self.num_host_blocks = num_host_blocks

    def _swap(self, fn, seq_id: int) -> np.ndarray:
        cap = self.max_blocks_per_seq
        buf = np.empty((cap, 2), dtype=np.int32)
        n = self._check(fn, getattr(self._lib, fn)(self._h, seq_id, _ptr(buf), cap))
        return buf[:n].copy()

    def swap_out(self, seq_id: int) -> np.ndarray:
        """Move a sequence to host blocks: pairs [n, 2] = (device block, host block), in logical order."""
        return self._swap("pa_bm_swap_out", seq_id)

    def swap_in(self, seq_id: int) -> np.ndarray:
        """Bring a swapped-out sequence back: pairs [n, 2] = (host block, device block), in logical order."""
        return self._swap("pa_bm_swap_in", seq_id)

    def swap_stats(self) -> dict:
        out = np.zeros(4, dtype=np.int64)
        self._check("pa_bm_swap_stats", self._lib.pa_bm_swap_stats(self._h, _ptr(out)))
        return dict(zip(("free_host_blocks", "used_host_blocks", "swapped_sequences", "blocks_moved"),
                        (int(x) for x in out)))

    def stats(self) -> dict:
        out = np.zeros(8, dtype=np.int64)
        self._check("pa_bm_stats", self._lib.pa_bm_stats(self._h, _ptr(out)))
        d = dict(zip(STAT_NAMES, (int(x) for x in out)))
        d["internal_fragmentation"] = (1.0 - d["slots_holding_tokens"] / d["slots_in_used_blocks"]
                                       if d["slots_in_used_blocks"] else 0.0)
        return d
