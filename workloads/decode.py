"""Seeded structure and values for the five synthetic paged decode workloads.

Structure (context lengths, the block tables of the paged pool, the slot of each sequence's new token, copy
pairs) comes from numpy's PCG64 generator; values come from torch's generator on the requested device. The
pool layout is the paged one the pages sketch (vLLM PagedAttention, page 1 section 3.2): one tensor per K and V
of shape [num_blocks, block_size, num_kv_heads, head_dim], with a per-sequence table that maps logical block j
to a physical block id (page 3 section 2.2 gives the example logical 0 -> physical 7). A sequence of length L
uses ceil(L / block_size) blocks (page 2 section 4.2, the block-per-sequence loop of its pseudocode).

With dtype "fp8" the caches hold OCP FP8 E4M3 codes (torch.float8_e4m3fn) read as code value x k_scale
(keys) and x v_scale (values); the query and the step's new rows stay bfloat16. The codes are torch's
float8 rounding of N(0, 1) / scale draws (clamped to the format's +-448), the scales 1/64 (a power of two, so
that N(0, 1) data spans most of the E4M3 range without saturating).

Every slot that holds no live token -- free blocks, the unused tail of a sequence's last block, a dedicated
poison block that pads the tables -- is filled with NaN, so a kernel that reads a slot it should not read
produces a NaN that a parity test sees.

Nothing in here computes attention, writes a cache slot or copies a block.
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field

import numpy as np

CONFIG_NAMES = ("tiny_fp32", "llama2_7b", "mixed_len", "mistral_gqa_prefix", "llama2_70b_gqa", "llama2_7b_fp8",
                "llama2_70b_gqa_fp8")
# further batches beside the configurations: grouped heads at head_dim 256 (8 query heads per KV head)
EXTRA_NAMES = ("gqa_d256", "gqa_d256_fp8")

_ESIZE = {"f32": 4, "bf16": 2, "fp8": 1}
FP8_KV_SCALE = 1.0 / 64


@dataclass
class DecodeStructure:
    """Host-side description of one decode batch over a paged KV pool."""

    name: str
    seed: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str  # "f32" or "bf16" (query and caches), or "fp8" (bf16 query, E4M3 caches); the output is fp32
    scale: float
    max_context_len: int
    max_blocks_per_seq: int
    num_blocks: int
    poison_block: int
    context_lens: np.ndarray  # int32 [num_seqs]
    block_tables: np.ndarray  # int32 [num_seqs, max_blocks_per_seq]; the tables attention reads
    block_tables_pre: np.ndarray  # tables before the copy-on-write repointing (== block_tables without CoW)
    slot_mapping: np.ndarray  # int32 [num_seqs]; slot of the new token (position L-1), -1 when L == 0
    copy_pairs: np.ndarray  # int32 [num_pairs, 2] = (src, dst)
    partition_size: int  # 0 = single pass, -1 = library default, > 0 = split-context partition in tokens
    notes: dict = field(default_factory=dict)
    k_scale: float = 1.0  # dequantisation scales of an E4M3 cache (1.0 otherwise)
    v_scale: float = 1.0

    @property
    def esize(self) -> int:
        """Bytes per cached K/V element."""
        return _ESIZE[self.dtype]

    @property
    def q_esize(self) -> int:
        """Bytes per query element (and per element of the step's new K/V rows)."""
        return 2 if self.dtype == "fp8" else _ESIZE[self.dtype]

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def blocks_per_seq(self) -> np.ndarray:
        return (self.context_lens.astype(np.int64) + self.block_size - 1) // self.block_size


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def custom_structure(
    name: str,
    seed: int,
    context_lens,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_size: int,
    dtype: str,
    *,
    pool_factor: float = 1.1,
    free_fraction: float | None = None,
    pool_blocks: int | None = None,
    shared_prefix_blocks: int = 0,
    cow_seqs: int = 0,
    partition_size: int = -1,
    max_context_len: int | None = None,
    scale: float | None = None,
    rng: np.random.Generator | None = None,
) -> DecodeStructure:
    """Lay out a decode batch in a randomly permuted paged pool.

    Physical ids are a seeded permutation of all non-poison blocks, taken in this order: shared prefix blocks,
    then each sequence's private blocks in sequence order, then fresh copy-on-write destinations. The pool has
    ``pool_blocks`` blocks if given, else ceil(need / (1 - free_fraction)) + 1 or ceil(pool_factor * need) + 1,
    the +1 being the poison block (the last id) that pads every table.
    """
    rng = rng if rng is not None else np.random.default_rng(seed)
    lens = np.asarray(context_lens, dtype=np.int64)
    if lens.ndim != 1 or lens.size == 0 or (lens < 0).any():
        raise ValueError("context_lens must be a non-empty 1-D array of non-negative lengths")
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    bs = int(block_size)
    num_seqs = int(lens.size)
    max_len = int(max_context_len) if max_context_len is not None else int(max(1, lens.max()))
    if lens.max() > max_len:
        raise ValueError("a context length exceeds max_context_len")
    mb = max(1, _ceil_div(max_len, bs))
    nblk = (lens + bs - 1) // bs
    if shared_prefix_blocks:
        # the shared blocks must be full and must not hold any sequence's new token (position L-1)
        if ((lens - 1) // bs < shared_prefix_blocks).any():
            raise ValueError("every sequence must extend past its shared prefix")
    if cow_seqs > num_seqs or (cow_seqs and not shared_prefix_blocks):
        raise ValueError("copy-on-write needs a shared prefix and at most num_seqs sequences")

    private = nblk - shared_prefix_blocks
    need = shared_prefix_blocks + int(private.sum()) + cow_seqs
    if pool_blocks is not None:
        num_blocks = int(pool_blocks)
        if num_blocks < need + 1:
            raise ValueError("pool too small")
    elif free_fraction is not None:
        num_blocks = _ceil_div(need * 1000, int(round((1.0 - free_fraction) * 1000))) + 1
    else:
        num_blocks = int(math.ceil(pool_factor * need - 1e-9)) + 1
    poison = num_blocks - 1
    perm = rng.permutation(num_blocks - 1).astype(np.int64)

    cursor = 0
    shared_ids = perm[cursor:cursor + shared_prefix_blocks]
    cursor += shared_prefix_blocks
    tables = np.full((num_seqs, mb), poison, dtype=np.int64)
    for s in range(num_seqs):
        n = int(nblk[s])
        tables[s, :shared_prefix_blocks] = shared_ids
        k = n - shared_prefix_blocks
        tables[s, shared_prefix_blocks:n] = perm[cursor:cursor + k]
        cursor += k
    cow_ids = perm[cursor:cursor + cow_seqs]
    cursor += cow_seqs
    assert cursor == need

    tables_pre = tables.copy()
    pairs = np.zeros((cow_seqs, 2), dtype=np.int64)
    for i in range(cow_seqs):
        j = shared_prefix_blocks - 1
        pairs[i] = (tables[i, j], cow_ids[i])
        tables[i, j] = cow_ids[i]

    slots = np.full(num_seqs, -1, dtype=np.int64)
    for s in range(num_seqs):
        L = int(lens[s])
        if L > 0:
            slots[s] = tables[s, (L - 1) // bs] * bs + (L - 1) % bs

    if dtype not in _ESIZE:
        raise ValueError(f"dtype must be one of {tuple(_ESIZE)}")
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    kv_scale = FP8_KV_SCALE if dtype == "fp8" else 1.0
    return DecodeStructure(
        name=name, seed=seed, num_seqs=num_seqs, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, block_size=bs, dtype=dtype, scale=float(scale), max_context_len=max_len,
        max_blocks_per_seq=mb, num_blocks=num_blocks, poison_block=poison,
        context_lens=lens.astype(np.int32), block_tables=tables.astype(np.int32),
        block_tables_pre=tables_pre.astype(np.int32), slot_mapping=slots.astype(np.int32),
        copy_pairs=pairs.astype(np.int32), partition_size=partition_size,
        notes={"need_blocks": need, "shared_prefix_blocks": shared_prefix_blocks}, k_scale=kv_scale,
        v_scale=kv_scale,
    )


def build_structure(name: str, seed: int | None = None) -> DecodeStructure:
    """The synthetic decode workloads at their full sizes (seeds 1..7 by default). A name ending in "_fp8" is
    the structure of the workload without the suffix (same seed, same lengths and tables) over E4M3 caches."""
    names = CONFIG_NAMES + EXTRA_NAMES
    if name not in names:
        raise KeyError(f"unknown workload {name!r}; known: {names}")
    idx = names.index(name)
    if name.endswith("_fp8"):
        base = build_structure(name[: -len("_fp8")], seed)
        return dataclasses.replace(base, name=name, seed=idx + 1 if seed is None else seed, dtype="fp8",
                                   k_scale=FP8_KV_SCALE, v_scale=FP8_KV_SCALE)
    seed = idx + 1 if seed is None else seed
    rng = np.random.default_rng(seed)
    if name == "tiny_fp32":
        # 4 sequences, MHA 4 x 64, fp32, block 16, a 64-block pool
        return custom_structure(name, seed, [5, 17, 33, 64], 4, 4, 64, 16, "f32", pool_blocks=64,
                                max_context_len=64, rng=rng)
    if name == "llama2_7b":
        lens = rng.integers(128, 2048, size=64, endpoint=True)
        return custom_structure(name, seed, lens, 32, 32, 128, 16, "bf16", pool_factor=1.1,
                                max_context_len=2048, rng=rng)
    if name == "mixed_len":
        # exact 70/30 split of 256 sequences into short (32..500) and long (1024..4096), then shuffled
        short = rng.integers(32, 500, size=179, endpoint=True)
        long_ = rng.integers(1024, 4096, size=77, endpoint=True)
        lens = np.concatenate([short, long_])
        rng.shuffle(lens)
        return custom_structure(name, seed, lens, 32, 32, 128, 16, "bf16", free_fraction=0.2,
                                max_context_len=4096, rng=rng)
    if name == "mistral_gqa_prefix":
        # The caller knows that every sequence shares the first 1024 tokens, which the library cannot see from
        # the host: it asks for 1024-token partitions, whose first spans run together in dispatch order and read
        # the shared blocks through L2 (the library's own choice for such a grid is the balanced split).
        lens = np.full(128, 4096)
        return custom_structure(name, seed, lens, 32, 8, 128, 16, "bf16", pool_factor=1.1,
                                shared_prefix_blocks=64, cow_seqs=32, partition_size=1024, max_context_len=4096,
                                rng=rng)
    if name == "gqa_d256":
        # 64 sequences of 1024..4096 tokens, 32 query heads on 4 KV heads of 256 dims, 16-token blocks
        lens = rng.integers(1024, 4096, size=64, endpoint=True)
        return custom_structure(name, seed, lens, 32, 4, 256, 16, "bf16", pool_factor=1.1, max_context_len=4096,
                                rng=rng)
    # llama2_70b_gqa
    lens = rng.integers(2048, 4096, size=64, endpoint=True)
    return custom_structure(name, seed, lens, 64, 8, 128, 256, "bf16", pool_factor=1.1,
                            partition_size=512, max_context_len=4096, rng=rng)


def live_slot_mask(st: DecodeStructure, include_new_token: bool = True, tables: np.ndarray | None = None):
    """bool [num_blocks, block_size]: the slots that hold a token of some sequence.

    With ``include_new_token`` False the slot of each sequence's position L-1 is left out (it is written by
    the step's cache update). The mask is taken under ``tables`` (default: the pre-copy tables).
    """
    tables = st.block_tables_pre if tables is None else tables
    bs = st.block_size
    mask = np.zeros((st.num_blocks, bs), dtype=bool)
    for s in range(st.num_seqs):
        L = int(st.context_lens[s]) - (0 if include_new_token else 1)
        if L <= 0:
            continue
        full, rem = divmod(L, bs)
        ids = tables[s, :full]
        mask[ids, :] = True
        if rem:
            mask[tables[s, full], :rem] = True
    return mask


def materialize(st: DecodeStructure, device="cpu", include_new_token: bool = True, chunk_blocks: int = 2048):
    """Draw the tensors of one batch on ``device``.

    Returns a dict with ``query`` [B, Hq, D], ``key_cache`` / ``value_cache`` [NB, bs, Hkv, D], ``new_key`` /
    ``new_value`` [B, Hkv, D] (the step's new token), all in the structure's dtype, N(0, 1) then rounded to the
    dtype, and NaN in every slot that is not live. For "fp8" the query and new rows are bfloat16 and the caches
    float8_e4m3fn codes of N(0, 1) / scale (NaN code 0x7F in the slots that are not live). With ``include_new_token`` True the position-(L-1) slots
    already hold random values (attention-only use, read through ``block_tables_pre``); with False they hold
    NaN and the caller writes ``new_key``/``new_value`` there and copies the copy-on-write pairs before
    attending through ``block_tables``.
    """
    import torch

    dt = torch.float32 if st.dtype == "f32" else torch.bfloat16
    fp8 = st.dtype == "fp8"
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(st.seed))
    B, Hq, Hkv, D, bs, NB = (st.num_seqs, st.num_q_heads, st.num_kv_heads, st.head_dim, st.block_size,
                             st.num_blocks)

    def draw(shape):
        return torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(dt)

    query = draw((B, Hq, D))
    new_key = draw((B, Hkv, D))
    new_value = draw((B, Hkv, D))
    mask = torch.from_numpy(live_slot_mask(st, include_new_token)).to(dev)
    nan = float("nan")
    caches = []
    for scale in (st.k_scale, st.v_scale):
        cache = torch.empty((NB, bs, Hkv, D), dtype=torch.float8_e4m3fn if fp8 else dt, device=dev)
        for b0 in range(0, NB, chunk_blocks):
            b1 = min(NB, b0 + chunk_blocks)
            if fp8:
                part = torch.randn((b1 - b0, bs, Hkv, D), generator=gen, device=dev, dtype=torch.float32)
                part = (part / scale).clamp_(-448.0, 448.0)
            else:
                part = draw((b1 - b0, bs, Hkv, D))
            part[~mask[b0:b1]] = nan
            cache[b0:b1] = part.to(cache.dtype)
        caches.append(cache)
    return {"query": query, "key_cache": caches[0], "value_cache": caches[1], "new_key": new_key,
            "new_value": new_value}


def query_rows(st: DecodeStructure, query_lens, device="cpu", seed: int | None = None):
    """Query rows for several new tokens per sequence: ``query_lens[s]`` rows for sequence s, packed in sequence
    order. Returns (query [T, Hq, D] in the query dtype, N(0, 1) then rounded; query_start int32 [B + 1] with
    query_start[s] the first row of sequence s).
    """
    import torch

    ql = np.asarray(query_lens, dtype=np.int64)
    if ql.shape != (st.num_seqs,) or (ql < 0).any():
        raise ValueError("query_lens must hold one non-negative count per sequence")
    query_start = np.zeros(st.num_seqs + 1, dtype=np.int32)
    query_start[1:] = np.cumsum(ql)
    dt = torch.float32 if st.dtype == "f32" else torch.bfloat16
    gen = torch.Generator(device=torch.device(device))
    gen.manual_seed(int(st.seed if seed is None else seed) + 7919)
    T = int(query_start[-1])
    q = torch.randn((T, st.num_q_heads, st.head_dim), generator=gen, device=torch.device(device),
                    dtype=torch.float32).to(dt)
    return q, query_start


def algorithmic_bytes(st: DecodeStructure, query_len: int = 1) -> dict:
    """Bytes a decode call must move at minimum: every live K and V element once, the query, the fp32 output,
    the live table entries and the lengths. ``kv_unique`` counts shared prefix blocks once. With ``query_len``
    new tokens per sequence the query and output rows multiply; K and V are still needed once."""
    lens = st.context_lens.astype(np.int64)
    row = st.num_kv_heads * st.head_dim * st.esize
    kv = int(lens.sum()) * row * 2
    q = st.num_seqs * query_len * st.num_q_heads * st.head_dim * st.q_esize
    out = st.num_seqs * query_len * st.num_q_heads * st.head_dim * 4
    tbl = int(st.blocks_per_seq().sum()) * 4 + 4 * st.num_seqs
    shared = st.notes.get("shared_prefix_blocks", 0)
    kv_unique = kv - max(0, st.num_seqs - 1) * shared * st.block_size * row * 2 if shared else kv
    return {"kv": kv, "kv_unique": kv_unique, "query": q, "out": out, "tables": tbl,
            "total": kv + q + out + tbl}
