"""A multi-step decode loop over the paged KV cache: the native block manager decides where every token goes,
the HIP kernels move and read the bytes.

Each step appends one token to every running sequence (vLLM PagedAttention, page 3 section 2.1: forward,
sample, update the KV cache, forward again): the block manager hands out the new tokens' slots and any
copy-on-write pairs; copy_blocks applies the copies, and paged_attention_decode_append writes the new K/V
into their slots and attends over each sequence's whole cache (in one launch where its plan allows). Sequences join (with a prompt whose full
blocks may be shared with earlier prompts), fork (sharing every block, page 1 section 3.2) and finish
(their blocks return to the pool) between steps. With a host pool (page 1 section 5: swap space; page 2
section 7.2: inactive blocks to host memory) a step that runs out of blocks swaps the most recently admitted
sequence out to pinned host memory, and swapped-out sequences come back, oldest first, once blocks are free.

K/V values are synthetic. A prompt token's K/V is a fixed function of the prompt up to and including it, so
two prompts with a common prefix would write identical rows there -- which is what makes sharing their
blocks correct. Generated tokens get fresh random K/V from the device generator.
"""

from __future__ import annotations

import numpy as np

from . import (PA_BF16, PA_F32, PagedAttentionError, copy_blocks, paged_attention_decode_append,
               reshape_and_cache, swap_blocks, workspace_bytes)
from .block_manager import PA_ERR_NOMEM, BlockManager


def _prefix_seed(seed: int, tokens: np.ndarray) -> int:
    """A 63-bit seed determined by the token prefix (FNV-1a over the ids)."""
    h = 1469598103934665603 ^ (seed & 0xFFFFFFFF)
    for t in tokens.tolist():
        h = ((h ^ (t & 0xFFFFFFFF)) * 1099511628211) & 0xFFFFFFFFFFFFFFFF
    return h & 0x7FFFFFFFFFFFFFFF


class DecodeLoop:
    """Paged KV pools on one GPU plus the block manager that fills them.

    The pools hold `num_blocks` blocks; the last one is never handed out and pads the block tables. Every slot
    that holds no token is NaN, so a kernel that reads one shows it.
    """

    def __init__(self, *, num_blocks: int, block_size: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 max_blocks_per_seq: int, dtype: str = "bf16", device="cuda", seed: int = 0, scale=None,
                 partition_size: int = -1, record: bool = False, prompt_kv: str = "prefix",
                 host_blocks: int = 0):
        import torch

        self.torch = torch
        self.dev = torch.device(device)
        self.dt = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.kv_code = PA_BF16 if dtype == "bf16" else PA_F32
        self.bs, self.hq, self.hkv, self.d = block_size, num_q_heads, num_kv_heads, head_dim
        self.mbs = max_blocks_per_seq
        self.pad_block = num_blocks - 1
        self.seed = seed
        self.scale = float(scale) if scale is not None else head_dim ** -0.5
        self.partition_size = partition_size
        self.bm = BlockManager(num_blocks, block_size, max_blocks_per_seq, reserved_block=self.pad_block)
        shape = (num_blocks, block_size, num_kv_heads, head_dim)
        self.key_cache = torch.full(shape, float("nan"), dtype=self.dt, device=self.dev)
        self.value_cache = torch.full(shape, float("nan"), dtype=self.dt, device=self.dev)
        self.gen = torch.Generator(device=self.dev)
        self.gen.manual_seed(seed)
        self.running: list[int] = []
        self.swapped: list[int] = []  # swapped-out sequences, oldest first
        self.lengths: dict[int, int] = {}
        # pinned host pools that swapped-out sequences live in (NaN until written, like the device pools)
        self.host_key = self.host_value = None
        if host_blocks:
            self.bm.set_host_pool(host_blocks)
            hshape = (host_blocks, block_size, num_kv_heads, head_dim)
            self.host_key = torch.full(hshape, float("nan"), dtype=self.dt).pin_memory()
            self.host_value = torch.full(hshape, float("nan"), dtype=self.dt).pin_memory()
        self._ws = None
        # with record=True every cache write and copy is kept on the host so that a test can rebuild the pools
        self.log: list | None = [] if record else None
        # "prefix": prompt K/V is a function of the token prefix (host generator, for checking shared blocks);
        # "random": fresh device-generated rows (for timing, where only the access pattern matters)
        if prompt_kv not in ("prefix", "random"):
            raise ValueError("prompt_kv must be 'prefix' or 'random'")
        self.prompt_kv = prompt_kv
        # a list to collect ((start, end) HIP events, context lengths) of every attention call, or None
        self.attention_events: list | None = None

    # ------------------------------------------------------------------------------------------------------
    def _rows(self, n: int):
        t = self.torch
        k = t.randn((n, self.hkv, self.d), generator=self.gen, device=self.dev, dtype=t.float32).to(self.dt)
        v = t.randn((n, self.hkv, self.d), generator=self.gen, device=self.dev, dtype=t.float32).to(self.dt)
        return k, v

    def prompt_rows(self, tokens: np.ndarray):
        """K/V of every prompt position: row t depends only on tokens[: t + 1] (host numpy, then the device)."""
        t = self.torch
        n = len(tokens)
        k = np.empty((n, self.hkv, self.d), np.float32)
        v = np.empty((n, self.hkv, self.d), np.float32)
        for i in range(n):
            rng = np.random.default_rng(_prefix_seed(self.seed, tokens[: i + 1]))
            k[i] = rng.standard_normal((self.hkv, self.d), dtype=np.float32)
            v[i] = rng.standard_normal((self.hkv, self.d), dtype=np.float32)
        return (t.from_numpy(k).to(self.dev).to(self.dt), t.from_numpy(v).to(self.dev).to(self.dt))

    def _to_device(self, a: np.ndarray):
        # through pinned memory without blocking: the host can prepare the next step while the GPU works, and
        # torch's pinned-memory allocator does not hand the staging buffer out again before the copy has run
        return self.torch.from_numpy(np.ascontiguousarray(a)).pin_memory().to(self.dev, non_blocking=True)

    def _write(self, k, v, slots: np.ndarray):
        sm = self._to_device(np.asarray(slots, dtype=np.int32))
        reshape_and_cache(k, v, self.key_cache, self.value_cache, sm)
        if self.log is not None:
            self.log.append(("write", slots.copy(), k.cpu(), v.cpu()))

    def _apply_copies(self):
        pairs = self.bm.take_copies()
        if len(pairs):
            copy_blocks(self.key_cache, self.value_cache, self._to_device(pairs))
            if self.log is not None:
                self.log.append(("copy", pairs.copy()))
        return pairs

    # ------------------------------------------------------------------------------------------------------
    def add_sequence(self, seq_id: int, tokens) -> np.ndarray:
        """Admit a sequence with its prompt; returns the prompt slots (-1 where a shared block already has it)."""
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        slots = self.bm.add_sequence(seq_id, len(tokens), tokens)
        fresh = slots >= 0
        if fresh.any():
            if self.prompt_kv == "random":
                k, v = self._rows(int(fresh.sum()))
            else:
                k, v = self.prompt_rows(tokens)
                idx = self._to_device(np.nonzero(fresh)[0])
                k, v = k[idx].contiguous(), v[idx].contiguous()
            self._write(k, v, slots[fresh])
        self.running.append(seq_id)
        self.lengths[seq_id] = len(tokens)
        return slots

    def fork(self, parent_id: int, child_id: int):
        self.bm.fork(parent_id, child_id)
        self.running.append(child_id)
        self.lengths[child_id] = self.lengths[parent_id]

    def finish(self, seq_id: int):
        self.bm.free_sequence(seq_id)
        (self.swapped if seq_id in self.swapped else self.running).remove(seq_id)
        del self.lengths[seq_id]

    def swap_out(self, seq_id: int):
        """Move a running sequence to the host pool (the copy is enqueued before anything reuses its blocks)."""
        pairs = self.bm.swap_out(seq_id)
        if len(pairs):
            swap_blocks(self.host_key, self.host_value, self.key_cache, self.value_cache, self._to_device(pairs))
        self.running.remove(seq_id)
        self.swapped.append(seq_id)
        if self.log is not None:
            self.log.append(("swap_out", pairs.copy()))

    def swap_in(self, seq_id: int):
        """Bring a swapped-out sequence back into fresh device blocks."""
        pairs = self.bm.swap_in(seq_id)
        if len(pairs):
            swap_blocks(self.key_cache, self.value_cache, self.host_key, self.host_value, self._to_device(pairs))
        self.swapped.remove(seq_id)
        self.running.append(seq_id)
        if self.log is not None:
            self.log.append(("swap_in", pairs.copy()))

    def _schedule(self):
        """Swap sequences back in while the free blocks also leave one per running sequence for this step's
        tokens; then take this step's slots, swapping the most recently admitted sequence out while they do not
        fit. Returns the slots of the running sequences, in order."""
        bs = self.bs
        while self.swapped:
            sid = self.swapped[0]
            need = -(-self.lengths[sid] // bs) + len(self.running) + 1
            if self.bm.stats()["free_blocks"] < need:
                break
            self.swap_in(sid)
        while True:
            try:
                return self.bm.append_slots(self.running)
            except PagedAttentionError as e:
                if e.status != PA_ERR_NOMEM or self.host_key is None or len(self.running) <= 1:
                    raise
                self.swap_out(self.running[-1])

    def step(self, query=None, new_kv=None):
        """One decode step for every running sequence; returns (seq_ids, out [n, Hq, D] fp32, copy pairs).

        query defaults to random rows; new_kv (k, v) of shape [n, Hkv, D] to random rows.
        """
        t = self.torch
        if not self.running and not self.swapped:
            return [], None, np.zeros((0, 2), np.int32)
        slots = self._schedule()
        ids = list(self.running)
        n = len(ids)
        if n == 0:  # everything is swapped out and nothing fits back in yet
            return [], None, np.zeros((0, 2), np.int32)
        pairs = self._apply_copies()  # copy-on-write before the new tokens land in the copies
        k, v = self._rows(n) if new_kv is None else new_kv
        slots_d = self._to_device(np.asarray(slots, dtype=np.int32))
        if self.log is not None:
            self.log.append(("write", slots.copy(), k.cpu(), v.cpu()))
        for s in ids:
            self.lengths[s] += 1
        if query is None:
            query = t.randn((n, self.hq, self.d), generator=self.gen, device=self.dev,
                            dtype=t.float32).to(self.dt)
        tables, lens = self.bm.block_tables(ids)
        mcl = int(lens.max())
        need = workspace_bytes(n, self.hq, self.hkv, self.d, mcl, self.bs, self.kv_code, self.partition_size)
        if need and (self._ws is None or self._ws.numel() < need):
            self._ws = t.empty(need, dtype=t.uint8, device=self.dev)
        out = t.empty((n, self.hq, self.d), dtype=t.float32, device=self.dev)
        # the step's tables go up before the attention call's events: the upload is host bookkeeping
        tables_d, lens_d = self._to_device(tables), self._to_device(lens)
        ev = None
        if self.attention_events is not None:
            ev = (t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True))
            ev[0].record(t.cuda.current_stream(self.dev))
        paged_attention_decode_append(out, query, k.contiguous(), v.contiguous(), self.key_cache, self.value_cache,
                                      tables_d, lens_d, slots_d, self.scale, max_context_len=mcl,
                                      partition_size=self.partition_size, workspace=self._ws if need else None)
        if ev is not None:
            ev[1].record(t.cuda.current_stream(self.dev))
            self.attention_events.append((ev, lens.copy(), tables.copy()))
        self.last_query = query
        return ids, out, pairs

    def stats(self) -> dict:
        return self.bm.stats()
