"""The C ABI on the host: the library loads, exports what the header declares, and rejects invalid calls before
anything reaches the device (these calls never launch a kernel, so they run without a GPU)."""

from __future__ import annotations

import ctypes
import re

import pytest

import paged_kv_cache_458_amd as pa

PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP, PA_ERR_ALIGN = (
    -1, -2, -3, -4, -5, -6, -7)

FAKE = 1 << 20  # a 16-byte-aligned address that is never dereferenced: validation fails first


def header_functions():
    text = "".join(open(p).read() for p in (pa.HEADER_PATH, pa.DIAG_HEADER_PATH, pa.BM_HEADER_PATH))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = pa.load_library()
    names = header_functions()
    assert {"paged_attention_decode", "reshape_and_cache", "copy_blocks", "paged_gather",
            "paged_attention_workspace_bytes", "paged_attention_partition_size", "pa_strerror",
            "pa_abi_version", "pa_stream_read", "pa_stream_copy", "pa_bm_create", "pa_bm_append_slots",
            "paged_attention_decode_scaled", "reshape_and_cache_fp8", "paged_attention_decode_multi",
            "paged_attention_multi_workspace_bytes", "paged_attention_multi_partition_size",
            "swap_blocks", "paged_attention_decode_noalloc"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"
    assert lib.pa_abi_version() == pa.ABI_VERSION


def header_prototypes():
    """name -> list of parameter names, for every function the three headers declare."""
    text = "".join(open(p).read() for p in (pa.HEADER_PATH, pa.DIAG_HEADER_PATH, pa.BM_HEADER_PATH))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    protos = {}
    for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(([^)]*)\)\s*;", text, flags=re.M):
        params = [q.strip() for q in m.group(2).replace("\n", " ").split(",") if q.strip() and q.strip() != "void"]
        protos[m.group(1)] = [re.findall(r"(\w+)\s*$", q)[0] for q in params]
    return protos


def test_binding_matches_header_prototypes():
    # every binding that sets argtypes passes as many arguments as the header declares; the sizing calls keep
    # max_context_len before block_size (the order the decode call's documentation of them uses)
    lib = pa.load_library()
    protos = header_prototypes()
    checked = 0
    for name, params in protos.items():
        fn = getattr(lib, name)
        if fn.argtypes is not None:
            assert len(fn.argtypes) == len(params), f"{name}: {len(fn.argtypes)} argtypes, header has {len(params)}"
            checked += 1
    assert checked >= 15
    for name in ("paged_attention_workspace_bytes", "paged_attention_partition_size",
                 "paged_attention_multi_workspace_bytes", "paged_attention_multi_partition_size"):
        params = protos[name]
        assert params.index("max_context_len") + 1 == params.index("block_size"), name
        assert params[-1] == "partition_size" and params[-2] == "kv_dtype", name


def append_call(**over):
    args = dict(out=FAKE, query=FAKE, key=FAKE, value=FAKE, key_cache=FAKE, value_cache=FAKE, block_tables=FAKE,
                context_lens=FAKE, slot_mapping=FAKE, scale=0.1, k_scale=1.0, v_scale=1.0, block_size=16,
                num_seqs=4, num_q_heads=8,
                num_kv_heads=8, head_dim=128, num_blocks=100, max_blocks_per_seq=8, max_context_len=128,
                q_dtype=pa.PA_BF16, kv_dtype=pa.PA_BF16, partition_size=-1, workspace=None, workspace_bytes=0,
                stream=None)
    args.update(over)
    return pa.load_library().paged_attention_decode_append(*args.values())


@pytest.mark.parametrize("over,status", [
    (dict(kv_dtype=7), PA_ERR_DTYPE),
    (dict(kv_dtype=pa.PA_FP8_E4M3, q_dtype=7), PA_ERR_DTYPE),          # the quantising write's source dtype
    (dict(kv_dtype=pa.PA_FP8_E4M3, q_dtype=pa.PA_F32), PA_ERR_DTYPE),  # the decode takes E4M3 under bf16 only
    (dict(kv_dtype=pa.PA_FP8_E4M3, k_scale=0.0), PA_ERR_SHAPE),
    (dict(kv_dtype=pa.PA_FP8_E4M3, v_scale=float("inf")), PA_ERR_SHAPE),
    (dict(kv_dtype=pa.PA_FP8_E4M3, key=None), PA_ERR_NULL),
    (dict(key=None), PA_ERR_NULL),
    (dict(slot_mapping=None), PA_ERR_NULL),
    (dict(value=FAKE + 8), PA_ERR_ALIGN),
    (dict(num_kv_heads=0), PA_ERR_SHAPE),
    (dict(head_dim=100), PA_ERR_UNSUPPORTED),           # the decode's own checks follow the cache write's
    (dict(workspace=None, workspace_bytes=0, partition_size=64), PA_ERR_WORKSPACE),
])
def test_append_rejects_before_launch(over, status):
    assert append_call(**over) == status


def test_append_no_sequences_is_a_no_op():
    assert append_call(num_seqs=0, key=None, value=None, slot_mapping=None) == 0


def test_strerror_names_every_status():
    for code in (0, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP,
                 PA_ERR_ALIGN, -10, pa.PA_ERR_SCRATCH):
        assert pa.strerror(code) != "unknown status"
    assert pa.strerror(123) == "unknown status"


def decode_call(**over):
    args = dict(out=FAKE, query=FAKE, key_cache=FAKE, value_cache=FAKE, block_tables=FAKE, context_lens=FAKE,
                scale=0.1, block_size=16, num_seqs=4, num_q_heads=8, num_kv_heads=2, head_dim=128, num_blocks=100,
                max_blocks_per_seq=8, max_context_len=128, q_dtype=pa.PA_BF16, kv_dtype=pa.PA_BF16,
                partition_size=0, workspace=None, workspace_bytes=0, stream=None)
    args.update(over)
    return pa.load_library().paged_attention_decode(*args.values())


@pytest.mark.parametrize("over,status", [
    (dict(head_dim=100), PA_ERR_UNSUPPORTED),
    (dict(head_dim=48), PA_ERR_UNSUPPORTED),
    (dict(block_size=4), PA_ERR_UNSUPPORTED),
    (dict(block_size=48), PA_ERR_UNSUPPORTED),
    (dict(block_size=512, max_context_len=128), PA_ERR_UNSUPPORTED),
    (dict(num_q_heads=6, num_kv_heads=4), PA_ERR_SHAPE),
    (dict(num_kv_heads=0), PA_ERR_SHAPE),
    (dict(num_seqs=-1), PA_ERR_SHAPE),
    (dict(num_seqs=70000), PA_ERR_UNSUPPORTED),
    (dict(q_dtype=pa.PA_F32), PA_ERR_DTYPE),
    (dict(kv_dtype=7, q_dtype=7), PA_ERR_DTYPE),
    (dict(max_context_len=129), PA_ERR_SHAPE),
    (dict(num_blocks=0), PA_ERR_SHAPE),
    (dict(num_blocks=1 << 31), PA_ERR_SHAPE),
    (dict(num_blocks=(1 << 28) + 1), PA_ERR_UNSUPPORTED),  # 2^32 + 16 slots: beyond a 32-bit slot index
    (dict(num_blocks=1 << 28, num_seqs=0), 0),           # exactly 2^32 slots
    (dict(partition_size=24), PA_ERR_SHAPE),
    (dict(partition_size=-2), PA_ERR_SHAPE),
    (dict(out=None), PA_ERR_NULL),
    (dict(block_tables=None), PA_ERR_NULL),
    (dict(query=FAKE + 8), PA_ERR_ALIGN),
    (dict(context_lens=FAKE + 2), PA_ERR_ALIGN),
    (dict(partition_size=32), PA_ERR_WORKSPACE),
    (dict(partition_size=32, workspace=FAKE, workspace_bytes=100), PA_ERR_WORKSPACE),
])
def test_decode_rejects_before_launch(over, status):
    assert decode_call(**over) == status


def scaled_call(**over):
    args = dict(out=FAKE, query=FAKE, key_cache=FAKE, value_cache=FAKE, block_tables=FAKE, context_lens=FAKE,
                scale=0.1, k_scale=0.5, v_scale=0.25, block_size=16, num_seqs=4, num_q_heads=8, num_kv_heads=2,
                head_dim=128, num_blocks=100, max_blocks_per_seq=8, max_context_len=128, q_dtype=pa.PA_BF16,
                kv_dtype=pa.PA_FP8_E4M3, partition_size=0, workspace=None, workspace_bytes=0, stream=None)
    args.update(over)
    return pa.load_library().paged_attention_decode_scaled(*args.values())


@pytest.mark.parametrize("over,status", [
    (dict(q_dtype=pa.PA_F32), PA_ERR_DTYPE),  # an E4M3 cache takes a bf16 query
    (dict(q_dtype=pa.PA_FP8_E4M3), PA_ERR_DTYPE),
    (dict(q_dtype=pa.PA_F32, kv_dtype=pa.PA_BF16), PA_ERR_DTYPE),
    (dict(k_scale=0.0), PA_ERR_SHAPE),
    (dict(v_scale=float("nan")), PA_ERR_SHAPE),
    (dict(k_scale=float("inf")), PA_ERR_SHAPE),
    (dict(head_dim=100), PA_ERR_UNSUPPORTED),
    (dict(head_dim=48), PA_ERR_UNSUPPORTED),
    (dict(head_dim=64, block_size=8, max_context_len=64), PA_ERR_UNSUPPORTED),  # 16 E4M3 rows per load
    (dict(partition_size=32), PA_ERR_WORKSPACE),
    (dict(out=None), PA_ERR_NULL),
])
def test_scaled_decode_rejects_before_launch(over, status):
    assert scaled_call(**over) == status


def multi_call(**over):
    args = dict(out=FAKE, query=FAKE, key_cache=FAKE, value_cache=FAKE, block_tables=FAKE, context_lens=FAKE,
                query_start=FAKE, scale=0.1, k_scale=1.0, v_scale=1.0, block_size=16, num_seqs=4,
                num_query_tokens=10, max_query_len=4, num_q_heads=8, num_kv_heads=2, head_dim=128, num_blocks=100,
                max_blocks_per_seq=8, max_context_len=128, q_dtype=pa.PA_BF16, kv_dtype=pa.PA_BF16,
                partition_size=0, workspace=None, workspace_bytes=0, stream=None)
    args.update(over)
    return pa.load_library().paged_attention_decode_multi(*args.values())


@pytest.mark.parametrize("over,status", [
    (dict(query_start=None), PA_ERR_NULL),
    (dict(query_start=FAKE + 2), PA_ERR_ALIGN),
    (dict(num_query_tokens=17), PA_ERR_SHAPE),  # more rows than num_seqs * max_query_len
    (dict(max_query_len=0), PA_ERR_SHAPE),
    (dict(num_query_tokens=-1), PA_ERR_SHAPE),
    (dict(num_query_tokens=70000, num_seqs=20000), PA_ERR_UNSUPPORTED),
    (dict(q_dtype=pa.PA_F32), PA_ERR_DTYPE),
    (dict(partition_size=32), PA_ERR_WORKSPACE),
])
def test_multi_rejects_before_launch(over, status):
    assert multi_call(**over) == status


def test_multi_no_rows_is_a_no_op_and_plans_match_decode():
    assert multi_call(num_query_tokens=0, out=None, query=None, query_start=None) == 0
    # one row per sequence plans exactly like decode
    for args in ((64, 32, 32, 128, 2048, 16, pa.PA_BF16, -1), (64, 64, 8, 128, 4096, 256, pa.PA_BF16, 512)):
        B, Hq, Hkv, D, L, bs, kd, part = args
        assert pa.multi_workspace_bytes(B, B, 1, Hq, Hkv, D, L, bs, kd, part) == pa.workspace_bytes(*args)
        assert pa.multi_partition_size_for(B, B, 1, Hq, Hkv, D, L, bs, kd, part) == pa.partition_size_for(*args)
    # the workspace holds one partial per query row and wave span: a matrix-core wave covers two 512-token
    # partitions and merges them itself
    B, T = 8, 24
    w = pa.multi_workspace_bytes(B, T, 3, 8, 2, 64, 4096, 16, pa.PA_BF16, 512)
    pm = 4096 // 1024
    assert w == (T * 8 * pm * 64 * 4 + 255) // 256 * 256 + T * 8 * pm * 2 * 4


def test_unscaled_decode_refuses_an_fp8_cache():
    assert decode_call(kv_dtype=pa.PA_FP8_E4M3) == PA_ERR_DTYPE


@pytest.mark.parametrize("over,status", [
    (dict(src_dtype=pa.PA_FP8_E4M3), PA_ERR_DTYPE),
    (dict(src_dtype=7), PA_ERR_DTYPE),
    (dict(k_scale=0.0), PA_ERR_SHAPE),
    (dict(v_scale=float("-inf")), PA_ERR_SHAPE),
    (dict(num_kv_heads=1, head_dim=8), PA_ERR_UNSUPPORTED),
    (dict(num_tokens=-1), PA_ERR_SHAPE),
    (dict(value_cache=None), PA_ERR_NULL),
    (dict(key_cache=FAKE + 8), PA_ERR_ALIGN),
])
def test_fp8_cache_write_rejects(over, status):
    args = dict(key=FAKE, value=FAKE, key_cache=FAKE, value_cache=FAKE, slot_mapping=FAKE, num_tokens=4,
                num_kv_heads=2, head_dim=64, block_size=16, num_blocks=10, src_dtype=pa.PA_BF16, k_scale=0.1,
                v_scale=0.1, stream=None)
    args.update(over)
    assert pa.load_library().reshape_and_cache_fp8(*args.values()) == status
    if over.get("num_tokens", 4) > 0:
        args.update(num_tokens=0, key=None, value=None, key_cache=None, value_cache=None, slot_mapping=None)
        expect_noop = status in (PA_ERR_NULL, PA_ERR_ALIGN)
        assert (pa.load_library().reshape_and_cache_fp8(*args.values()) == 0) == expect_noop


def test_decode_with_no_sequences_is_a_no_op():
    assert decode_call(num_seqs=0, out=None, query=None) == 0


def test_workspace_and_partition_plan():
    lib = pa.load_library()
    # single pass needs no workspace
    assert pa.workspace_bytes(64, 32, 32, 128, 2048, 16, pa.PA_BF16, 0) == 0
    assert pa.partition_size_for(64, 32, 32, 128, 2048, 16, pa.PA_BF16, 0) == 0
    # an explicit split: o [B, Hq, PM, D] fp32, then (m, l) pairs, 256-byte aligned; PM counts wave spans, and a
    # matrix-core wave covers two 512-token partitions
    B, Hq, D, P, L = 64, 64, 128, 512, 4096
    pm = L // (2 * P)
    o = B * Hq * pm * D * 4
    want = (o + 255) // 256 * 256 + B * Hq * pm * 2 * 4
    assert pa.workspace_bytes(B, Hq, 8, D, L, 256, pa.PA_BF16, P) == want
    assert pa.partition_size_for(B, Hq, 8, D, L, 256, pa.PA_BF16, P) == P
    # a partition that covers the longest context is a single pass
    assert pa.workspace_bytes(4, 4, 4, 64, 64, 16, pa.PA_F32, 64) == 0
    # the library's own choice is consistent with its workspace size
    for args in ((64, 64, 8, 128, 4096, 256, pa.PA_BF16), (4, 4, 4, 64, 64, 16, pa.PA_F32)):
        p = pa.partition_size_for(*args, -1)
        assert p == 0 or p % 16 == 0
        assert (pa.workspace_bytes(*args, -1) > 0) == (p > 0)
    assert lib.paged_attention_workspace_bytes(4, 8, 3, 128, 64, 16, 1, -1) == 0  # invalid -> 0
    assert lib.paged_attention_partition_size(4, 8, 3, 128, 64, 16, 1, -1) == PA_ERR_SHAPE


def test_grouped_query_default_counts_waves_per_span():
    # the partition rule, seen where the balanced split does not apply (8 new tokens per sequence x 4 heads = 32
    # columns per KV head: two column groups, which one wave serves, so 8 waves per sequence, and partitions one
    # to a wave since that wave holds two accumulators): 1024 halves while the grid holds fewer than 2048 waves
    def multi(B, *args):
        return pa.multi_partition_size_for(B, 8 * B, 8, *args)
    assert multi(32, 32, 8, 128, 2048, 16, pa.PA_BF16, -1) == 256
    assert multi(8, 32, 8, 128, 2048, 16, pa.PA_BF16, -1) == 64
    assert multi(64, 32, 8, 128, 2048, 16, pa.PA_BF16, -1) == 512
    # 1024-token partitions that already give 2048 waves stay; 2048 (sequence, KV head, wave) triples run single
    # pass
    assert multi(128, 32, 8, 128, 2048, 16, pa.PA_BF16, -1) == 1024
    assert multi(256, 32, 8, 128, 2048, 16, pa.PA_BF16, -1) == 0
    # at head_dim 256 a wave serves one column group: 16 waves per sequence
    assert multi(8, 32, 8, 256, 2048, 16, pa.PA_BF16, -1) == 128
    assert pa.load_library().paged_attention_multi_partition_size(
        32, 256, 8, 32, 8, 128, 2048, 16, pa.PA_BF16, pa.PA_PARTITION_BALANCED) == PA_ERR_UNSUPPORTED


def test_several_tokens_per_sequence_take_the_balanced_split_where_measured():
    B = pa.PA_PARTITION_BALANCED
    # one column group: beyond one round of partitions, as in decode
    assert pa.multi_partition_size_for(64, 128, 2, 32, 8, 128, 2048, 16, pa.PA_BF16, -1) == B
    # 64 sequences x 32 heads x 4 rows (MHA): a single pass of 2048 unequal waves -> balanced
    assert pa.multi_partition_size_for(64, 256, 4, 32, 32, 128, 2048, 16, pa.PA_BF16, -1) == B
    assert pa.multi_partition_size_for(64, 256, 4, 32, 32, 128, 2048, 16, pa.PA_FP8_E4M3, -1) == B
    # 70B shape, 2 rows: one round of partitions keeps them (partitions measured faster there)
    assert pa.multi_partition_size_for(64, 128, 2, 64, 8, 128, 4096, 256, pa.PA_BF16, -1) == 1024
    # decode keeps its single pass where it fills a round
    assert pa.partition_size_for(256, 32, 8, 128, 1024, 16, pa.PA_BF16, -1) == 0


def test_grouped_query_decode_default_takes_the_balanced_split_beyond_one_round():
    B = pa.PA_PARTITION_BALANCED
    # partitions of 256 tokens would launch 64 x 8 x 8 = 4096 waves, two rounds: balanced
    assert pa.partition_size_for(64, 32, 8, 128, 2048, 16, pa.PA_BF16, -1) == B
    assert pa.partition_size_for(128, 32, 8, 128, 4096, 16, pa.PA_FP8_E4M3, -1) == B
    # one round of 2048 waves (64 x 8 x 4 spans of 1024 tokens) keeps its partitions; so does single pass
    assert pa.partition_size_for(64, 64, 8, 128, 4096, 256, pa.PA_BF16, -1) == 1024
    assert pa.partition_size_for(16, 64, 8, 128, 16384, 16, pa.PA_BF16, -1) == 1024
    assert pa.partition_size_for(256, 32, 8, 128, 2048, 16, pa.PA_BF16, -1) == 0
    # more than 16 heads per KV head (two column groups): partitions
    assert pa.partition_size_for(64, 64, 2, 128, 2048, 16, pa.PA_BF16, -1) % 16 == 0


def balanced_ws(T, Hq, D, hpw=1):
    runs = max(1, 1024 // (((Hq + hpw - 1) // hpw + 1) // 2))
    o = (Hq * runs * 2 * D * 4 + 255) // 256 * 256
    ml = (Hq * runs * 2 * 2 * 4 + 255) // 256 * 256
    return o + ml + (T + 1) * 4


def gqa_balanced_ws(B, Hq, Hkv, D, ql=1):
    # B sequences (the tile list's items), ql partial slots per (head, run, side): the most rows of a sequence
    w = 8 if Hkv >= 8 else 4 if Hkv >= 4 else 2 if Hkv >= 2 else 1
    runs = max(1, 2048 // ((Hkv + w - 1) // w * w))
    o = (Hq * runs * 2 * ql * D * 4 + 255) // 256 * 256
    ml = (Hq * runs * 2 * ql * 2 * 4 + 255) // 256 * 256
    return o + ml + (B + 1) * 4


def test_balanced_split_plan():
    lib = pa.load_library()
    B = pa.PA_PARTITION_BALANCED
    # the library takes the balanced split where the single-head kernel would split its contexts
    assert pa.partition_size_for(64, 32, 32, 128, 2048, 16, pa.PA_BF16, -1) == B
    # (bf16 rows of 256 bytes: two heads per wave, half the waves per run, twice the runs)
    assert pa.workspace_bytes(64, 32, 32, 128, 2048, 16, pa.PA_BF16, -1) == balanced_ws(64, 32, 128, 2)
    assert pa.workspace_bytes(7, 5, 5, 80, 900, 16, pa.PA_FP8_E4M3, B) == balanced_ws(7, 5, 80)
    assert pa.workspace_bytes(3, 4096, 4096, 64, 900, 16, pa.PA_F32, B) == balanced_ws(3, 4096, 64)  # one run
    # two heads per wave where head rows are 64 or 128 bytes (or 256 bytes of bf16) and every query head has its
    # own KV head: half the waves per run, twice the runs
    assert pa.workspace_bytes(64, 32, 32, 128, 2048, 16, pa.PA_FP8_E4M3, B) == balanced_ws(64, 32, 128, 2)
    assert pa.workspace_bytes(9, 5, 5, 64, 900, 16, pa.PA_BF16, B) == balanced_ws(9, 5, 64, 2)
    assert pa.workspace_bytes(9, 8, 4, 64, 900, 16, pa.PA_F32, B) == balanced_ws(9, 8, 64)
    # several tokens per sequence (fp32: the per-head kernel): one tile count per query row
    assert pa.multi_partition_size_for(64, 256, 4, 32, 32, 128, 2048, 16, pa.PA_F32, -1) == B
    assert pa.multi_workspace_bytes(64, 256, 4, 32, 32, 128, 2048, 16, pa.PA_F32, -1) == balanced_ws(256, 32, 128)
    # contexts that fit one partition stay single pass; grouped heads on the matrix cores whose partitions fit
    # one round of waves keep them by default ...
    assert pa.partition_size_for(4, 4, 4, 64, 64, 16, pa.PA_F32, -1) == 0
    assert pa.partition_size_for(64, 64, 8, 128, 4096, 256, pa.PA_BF16, -1) % 16 == 0
    # ... and take the balanced split when asked: runs = 2048 waves / (KV heads rounded to whole workgroups of
    # up to 8), partials per query head and run
    assert pa.partition_size_for(64, 64, 8, 128, 4096, 256, pa.PA_BF16, B) == B
    assert pa.workspace_bytes(64, 64, 8, 128, 4096, 256, pa.PA_BF16, B) == gqa_balanced_ws(64, 64, 8, 128)
    assert pa.workspace_bytes(5, 24, 12, 64, 4096, 32, pa.PA_FP8_E4M3, B) == gqa_balanced_ws(5, 24, 12, 64)
    assert pa.workspace_bytes(3, 16, 1, 128, 900, 16, pa.PA_BF16, B) == gqa_balanced_ws(3, 16, 1, 128)
    # beyond 2048 query rows, or 2^30 row-positions, the default falls back to partitions ...
    assert pa.partition_size_for(4096, 32, 32, 128, 2048, 16, pa.PA_BF16, -1) % 16 == 0
    assert pa.partition_size_for(2048, 32, 32, 128, 1 << 20, 16, pa.PA_BF16, -1) % 16 == 0
    # ... and an explicit request is refused, on either kernel; so is one for the matrix-core kernel with more
    # than 16 (query row, head) columns per KV head
    for args in ((2049, 32, 32, 128, 2048, 16, pa.PA_BF16), (2048, 32, 32, 128, 1 << 20, 16, pa.PA_BF16),
                 (2049, 64, 8, 128, 4096, 256, pa.PA_BF16), (64, 64, 2, 128, 2048, 16, pa.PA_BF16)):
        assert lib.paged_attention_partition_size(*args, B) == PA_ERR_UNSUPPORTED
        assert lib.paged_attention_workspace_bytes(*args, B) == 0
    # several new tokens per sequence on the matrix cores: one column group takes it, with partial slots for
    # every row of a sequence; more columns are refused
    assert lib.paged_attention_multi_partition_size(64, 128, 2, 64, 8, 128, 4096, 256, pa.PA_BF16, B) == B
    assert lib.paged_attention_multi_workspace_bytes(64, 128, 2, 64, 8, 128, 4096, 256, pa.PA_BF16, B) == \
        gqa_balanced_ws(64, 64, 8, 128, ql=2)
    assert lib.paged_attention_multi_partition_size(64, 192, 3, 64, 8, 128, 4096, 256, pa.PA_BF16,
                                                    B) == PA_ERR_UNSUPPORTED
    assert pa.multi_partition_size_for(64, 128, 2, 64, 8, 128, 4096, 256, pa.PA_BF16, -1) % 16 == 0
    # partition sizes between the balanced code and 16 are not multiples of 16
    assert lib.paged_attention_partition_size(64, 32, 32, 128, 2048, 16, pa.PA_BF16, 2) == PA_ERR_SHAPE


@pytest.mark.parametrize("over,status", [
    (dict(num_kv_heads=0), PA_ERR_SHAPE),
    (dict(kv_dtype=5), PA_ERR_DTYPE),
    (dict(head_dim=3, kv_dtype=pa.PA_BF16, num_kv_heads=1), PA_ERR_UNSUPPORTED),
    (dict(slot_mapping=None), PA_ERR_NULL),
    (dict(key=FAKE + 4), PA_ERR_ALIGN),
])
def test_reshape_and_cache_rejects(over, status):
    args = dict(key=FAKE, value=FAKE, key_cache=FAKE, value_cache=FAKE, slot_mapping=FAKE, num_tokens=4,
                num_kv_heads=2, head_dim=64, block_size=16, num_blocks=10, kv_dtype=pa.PA_F32, stream=None)
    args.update(over)
    assert pa.load_library().reshape_and_cache(*args.values()) == status


def test_cache_ops_with_nothing_to_do_are_no_ops():
    lib = pa.load_library()
    assert lib.reshape_and_cache(None, None, None, None, None, 0, 2, 64, 16, 10, pa.PA_F32, None) == 0
    assert lib.copy_blocks(None, None, None, 0, 16, 2, 64, 10, pa.PA_F32, None) == 0


@pytest.mark.parametrize("over,status", [
    (dict(num_pairs=-1), PA_ERR_SHAPE),
    (dict(kv_dtype=9), PA_ERR_DTYPE),
    (dict(block_pairs=None), PA_ERR_NULL),
    (dict(block_pairs=FAKE + 1), PA_ERR_ALIGN),
])
def test_copy_blocks_rejects(over, status):
    args = dict(key_cache=FAKE, value_cache=FAKE, block_pairs=FAKE, num_pairs=3, block_size=16, num_kv_heads=2,
                head_dim=64, num_blocks=10, kv_dtype=pa.PA_BF16, stream=None)
    args.update(over)
    assert pa.load_library().copy_blocks(*args.values()) == status


@pytest.mark.parametrize("over,status", [
    (dict(num_pairs=-1), PA_ERR_SHAPE),
    (dict(src_num_blocks=0), PA_ERR_SHAPE),
    (dict(kv_dtype=9), PA_ERR_DTYPE),
    (dict(head_dim=3, num_kv_heads=1, block_size=2, kv_dtype=pa.PA_BF16), PA_ERR_UNSUPPORTED),
    (dict(block_pairs=None), PA_ERR_NULL),
    (dict(src_key_cache=FAKE + 8), PA_ERR_ALIGN),
    # an address HIP does not know is refused on the host, before any launch (here: no device at all)
    (dict(), -10),
])
def test_swap_blocks_rejects(over, status):
    args = dict(dst_key_cache=FAKE, dst_value_cache=FAKE, dst_num_blocks=10, src_key_cache=FAKE,
                src_value_cache=FAKE, src_num_blocks=20, block_pairs=FAKE, num_pairs=3, block_size=16, num_kv_heads=2,
                head_dim=64, kv_dtype=pa.PA_BF16, stream=None)
    args.update(over)
    assert pa.load_library().swap_blocks(*args.values()) == status


def test_gather_rejects():
    lib = pa.load_library()
    base = [FAKE] * 6 + [16, 2, 2, 64, 10, 4, 64, pa.PA_BF16, None]
    bad_bs = list(base)
    bad_bs[6] = 24
    assert lib.paged_gather(*bad_bs) == PA_ERR_UNSUPPORTED
    too_long = list(base)
    too_long[12] = 65
    assert lib.paged_gather(*too_long) == PA_ERR_SHAPE
    null = list(base)
    null[4] = None
    assert lib.paged_gather(*null) == PA_ERR_NULL
    huge_pool = list(base)
    huge_pool[10] = (1 << 28) + 1  # 16-slot blocks: 2^32 + 16 slots
    assert lib.paged_gather(*huge_pool) == PA_ERR_UNSUPPORTED


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        pa.load_library(str(tmp_path / "nope.so"))


def test_stream_diagnostics_reject():
    lib = pa.load_library()
    assert lib.pa_stream_read(FAKE, 100, FAKE, None) == PA_ERR_SHAPE
    assert lib.pa_stream_read(None, 1024, FAKE, None) == PA_ERR_NULL
    assert lib.pa_stream_read(FAKE + 8, 1024, FAKE, None) == PA_ERR_ALIGN
    assert lib.pa_stream_copy(FAKE, FAKE, 0, None) == PA_ERR_SHAPE
    assert lib.pa_stream_copy(FAKE + 4, FAKE, 1024, None) == PA_ERR_ALIGN


def noalloc_call(**over):
    args = dict(out=FAKE, query=FAKE, key_cache=FAKE, value_cache=FAKE, block_tables=FAKE, context_lens=FAKE,
                scale=0.1, k_scale=1.0, v_scale=1.0, block_size=16, num_seqs=4, num_q_heads=8, num_kv_heads=2,
                head_dim=128, num_blocks=100, max_blocks_per_seq=8, max_context_len=128, q_dtype=pa.PA_BF16,
                kv_dtype=pa.PA_BF16, partition_size=32, stream=None)
    args.update(over)
    return pa.load_library().paged_attention_decode_noalloc(*args.values())


@pytest.mark.parametrize("over,status", [
    (dict(head_dim=100), PA_ERR_UNSUPPORTED),
    (dict(num_q_heads=6, num_kv_heads=4), PA_ERR_SHAPE),
    (dict(q_dtype=pa.PA_F32), PA_ERR_DTYPE),
    (dict(v_scale=0.0), PA_ERR_SHAPE),
    (dict(max_context_len=129), PA_ERR_SHAPE),
    (dict(partition_size=24), PA_ERR_SHAPE),
    (dict(out=None), PA_ERR_NULL),
    (dict(query=FAKE + 8), PA_ERR_ALIGN),
    # 256 sequences x 32 heads x 256 partitions of 16 tokens x 128 dims of fp32 partials: 1 GiB > 32 MiB
    (dict(num_seqs=256, num_q_heads=32, num_kv_heads=32, max_blocks_per_seq=256, max_context_len=4096,
          partition_size=16), pa.PA_ERR_SCRATCH),
])
def test_noalloc_decode_rejects_before_launch(over, status):
    # every rejection comes before the static scratch is looked up (no device is touched here)
    assert noalloc_call(**over) == status


def test_noalloc_scratch_limit_matches_the_workspace_rule():
    lib = pa.load_library()
    # the largest plan that fits: the workspace size function gives the same bytes the no-alloc call needs
    need = lib.paged_attention_workspace_bytes(256, 32, 32, 128, 4096, 16, pa.PA_BF16, 16)
    assert need > pa.PA_STATIC_SCRATCH_BYTES
    fits = lib.paged_attention_workspace_bytes(64, 64, 8, 128, 4096, 256, pa.PA_BF16, 512)
    assert 0 < fits <= pa.PA_STATIC_SCRATCH_BYTES
    assert "PA_STATIC_SCRATCH_BYTES" in pa.strerror(pa.PA_ERR_SCRATCH)
    assert noalloc_call(num_seqs=0) == 0  # nothing to do: no-op


def test_grouped_query_default_partitions_within_one_round():
    lib = pa.load_library()
    # 64 sequences of up to 4096 tokens, 32 query heads on 4 KV heads of 256 dims: 512-token partitions (one per
    # wave at head_dim > 128) fill one round of workgroups, which the kernel spreads over the XCDs by sequence
    assert lib.paged_attention_partition_size(64, 32, 4, 256, 4096, 16, pa.PA_BF16, -1) == 512
    # the 70B shape: 1024-token spans, one round of 2048 waves
    assert lib.paged_attention_partition_size(64, 64, 8, 128, 4096, 256, pa.PA_BF16, -1) == 1024
    # grouped heads at every served head dim plan on the matrix cores (workspace of the balanced split with
    # one partial slot per query head and run, not per query row)
    for d in (64, 80, 96, 112, 128, 192, 256):
        for kd in (pa.PA_BF16, pa.PA_FP8_E4M3):
            assert lib.paged_attention_partition_size(4, 16, 2, d, 4096, 16, kd, pa.PA_PARTITION_BALANCED) == 1
    # at head_dim > 128 a grouped-query wave covers one partition: 512-token partitions need a partial each
    ws_128 = lib.paged_attention_workspace_bytes(8, 16, 2, 128, 4096, 16, pa.PA_BF16, 512)
    ws_256 = lib.paged_attention_workspace_bytes(8, 16, 2, 256, 4096, 16, pa.PA_BF16, 512)
    assert ws_256 > 2 * ws_128 * 1.9
