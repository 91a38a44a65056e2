"""paged_attention_decode_append: one decode step's cache write and attention in one call, against the two
separate calls (reshape_and_cache, then paged_attention_decode) and the oracle.

The pools must end byte for byte as the separate cache write leaves them. The single-head kernels add the new
token to its row's softmax after the pool rows of its tile or partition, so their output equals the separate
calls' up to the order of floating-point additions; the matrix-core kernels stage the new row in place of the
pool's, and must match the separate calls bit for bit (as must a call with max_context_len 0, which launches
the cache write first). All are also compared with the fp64 oracle over the updated pools."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_458_amd as pa
from tests._host import to_host
from tests.test_gpu_parity import assert_attention_close, decode, dev_i32, oracle_decode
from workloads import build_structure, custom_structure, materialize

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


def appended(st, t, pools, tables, slots, partition_size, context_lens=None, max_context_len=None):
    out = torch.empty((st.num_seqs, st.num_q_heads, st.head_dim), dtype=torch.float32, device=DEV)
    cl = st.context_lens if context_lens is None else context_lens
    pa.paged_attention_decode_append(out, t["query"], t["new_key"], t["new_value"], pools[0], pools[1],
                                     dev_i32(tables), dev_i32(cl), dev_i32(slots), st.scale,
                                     max_context_len=st.max_context_len if max_context_len is None
                                     else max_context_len, partition_size=partition_size, k_scale=st.k_scale,
                                     v_scale=st.v_scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def write_separately(st, t, pools, slots):
    """The step's cache write as its own call (quantising for E4M3 caches)."""
    pa.reshape_and_cache(t["new_key"], t["new_value"], pools[0], pools[1], dev_i32(slots), k_scale=st.k_scale,
                         v_scale=st.v_scale)


def write_on_host(st, h, slots):
    if st.dtype == "fp8":
        oracle.reshape_and_cache_e4m3(h["key_cache"], h["value_cache"], h["new_key"], h["new_value"], slots,
                                      st.k_scale, st.v_scale)
    else:
        oracle.reshape_and_cache(h["key_cache"], h["value_cache"], h["new_key"], h["new_value"], slots)


def fused_here(st, partition_size) -> str:
    """Which decode kernel appends the new tokens itself (each of them does)."""
    kd = {"f32": pa.PA_F32, "bf16": pa.PA_BF16, "fp8": pa.PA_FP8_E4M3}[st.dtype]
    part = pa.partition_size_for(st.num_seqs, st.num_q_heads, st.num_kv_heads, st.head_dim, st.max_context_len,
                                 st.block_size, kd, partition_size)
    mfma = st.dtype in ("bf16", "fp8") and st.num_q_heads != st.num_kv_heads
    if part == pa.PA_PARTITION_BALANCED:
        return "matrix-core balanced" if mfma else "single-head balanced"
    return "matrix-core partitions" if mfma else "single-head partitions"


def reordered(st, partition_size) -> bool:
    """Whether the appended output may differ from the separate calls' in the order of its additions."""
    return fused_here(st, partition_size).startswith("single-head")


def compare(st, fused, separate, ref, what, exact):
    if exact:
        np.testing.assert_array_equal(fused, separate, err_msg=what)
    else:
        np.testing.assert_allclose(fused, separate, rtol=1e-5, atol=1e-6, err_msg=what)
    return assert_attention_close(fused, ref, st.dtype, what)


@pytest.mark.parametrize("name", ["llama2_7b", "mixed_len", "llama2_70b_gqa", "mistral_gqa_prefix", "llama2_7b_fp8",
                                  "llama2_70b_gqa_fp8"])
def test_full_size_step(name):
    # the benchmark's step: copy-on-write pairs, then the new tokens appended and attended over
    st = build_structure(name)
    t = materialize(st, DEV, include_new_token=False)
    pools = (t["key_cache"].clone(), t["value_cache"].clone())
    h = {k: to_host(v) for k, v in t.items()}
    # the separate calls, on the device and on the host copies
    if len(st.copy_pairs):
        pa.copy_blocks(t["key_cache"], t["value_cache"], dev_i32(st.copy_pairs))
        pa.copy_blocks(pools[0], pools[1], dev_i32(st.copy_pairs))
        oracle.copy_blocks(h["key_cache"], h["value_cache"], st.copy_pairs)
    write_separately(st, t, (t["key_cache"], t["value_cache"]), st.slot_mapping)
    write_on_host(st, h, st.slot_mapping)
    separate = decode(st, t, st.block_tables, st.partition_size)
    fused = appended(st, t, pools, st.block_tables, st.slot_mapping, st.partition_size)
    for got, want, which in ((pools[0], t["key_cache"], "key"), (pools[1], t["value_cache"], "value")):
        assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"{name}: {which} pool differs"
    del pools
    ref = oracle_decode(st, h, st.block_tables)
    err = compare(st, fused, separate, ref, name, exact=not reordered(st, st.partition_size))
    sys.__stderr__.write(f"[{name}] appended in the launch: {fused_here(st, st.partition_size)}, "
                         f"max abs err {err:.3e}\n")


# lengths with the new token alone in its tile (9 and 17 with 8- and 16-token tiles), a one-token context, rows
# cut across the balanced split's runs; bf16 two heads per wave (head_dim 128 and 64), fp32 one head per wave,
# grouped fp32 heads (one wave per KV head writes the rows), 8-slot blocks; grouped bf16 heads on the matrix
# cores (new token first or last in a 32-token tile, two partitions per wave, head dims with padded lanes,
# phased K/V at head_dim 256, two column groups per wave at 32 heads per KV head)
SMALL = [
    # (seed, lens, Hq, Hkv, D, bs, dtype)
    (601, [1, 8, 9, 16, 17, 300, 1000], 8, 8, 128, 16, "bf16"),
    (602, [9, 1, 17, 2049, 33, 700], 4, 4, 64, 16, "bf16"),
    (603, [1, 5, 16, 17, 129, 900], 4, 4, 128, 16, "f32"),
    (604, [17, 1, 400, 9, 63], 8, 2, 64, 8, "f32"),
    (605, [1000, 3, 8, 9, 250, 1], 16, 16, 128, 8, "bf16"),
    (606, [1, 32, 33, 64, 1024, 1025, 2000, 513], 32, 8, 128, 16, "bf16"),
    (607, [31, 97, 1500, 1, 600], 8, 2, 80, 16, "bf16"),
    (608, [700, 1, 65, 2048, 129], 16, 4, 256, 16, "bf16"),
    (609, [40, 1300, 1, 257], 64, 2, 64, 8, "bf16"),
    (611, [3000, 45, 800, 1], 32, 4, 112, 32, "bf16"),
    # E4M3 caches from bf16 rows: the kernels that append quantise the new row where they use it
    (612, [1, 32, 33, 1024, 1025, 2000, 513], 32, 8, 128, 16, "fp8"),
    (613, [31, 97, 1500, 1, 600], 8, 2, 80, 16, "fp8"),
    (614, [700, 1, 65, 2048, 129], 16, 4, 256, 16, "fp8"),
    (615, [9, 1, 300, 17, 1000], 8, 8, 128, 16, "fp8"),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"seed{c[0]}" for c in SMALL])
def test_small_cases(case):
    seed, lens, hq, hkv, d, bs, dt = case
    st = custom_structure(f"a{seed}", seed, lens, hq, hkv, d, bs, dt)
    assert len(st.copy_pairs) == 0  # the tables before and after the step are the same
    # the new tokens' slots hold data already (read where a token is not appended) ...
    t = materialize(st, DEV, include_new_token=True)
    tables = st.block_tables_pre
    slots = st.slot_mapping.copy()
    slots[1] = -1  # this sequence's token is not written: the pool is read as it was
    # ... and NaN where one is: a kernel that read such a slot instead of the new row would show it
    for pool in (t["key_cache"], t["value_cache"]):
        rows = pool.view(torch.uint8).view(-1, hkv * d * pool.element_size())
        nan = torch.tensor([float("nan")], dtype=pool.dtype, device=DEV).view(torch.uint8)
        rows[torch.from_numpy(slots[slots >= 0].astype(np.int64)).to(DEV)] = nan.repeat(hkv * d)
    kd = {"f32": pa.PA_F32, "bf16": pa.PA_BF16, "fp8": pa.PA_FP8_E4M3}[dt]
    for part in (-1, pa.PA_PARTITION_BALANCED, 0, 64):
        if part == pa.PA_PARTITION_BALANCED and not pa.workspace_bytes(st.num_seqs, hq, hkv, d, st.max_context_len,
                                                                       bs, kd, part):
            continue  # no balanced split for these sizes (more than 16 columns per KV head on the matrix cores)
        ref_pools = (t["key_cache"].clone(), t["value_cache"].clone())
        pools = (t["key_cache"].clone(), t["value_cache"].clone())
        h = {k: to_host(v) for k, v in t.items()}
        write_separately(st, t, ref_pools, slots)
        write_on_host(st, h, slots)
        tref = dict(t, key_cache=ref_pools[0], value_cache=ref_pools[1])
        separate = decode(st, tref, tables, part)
        fused = appended(st, t, pools, tables, slots, part)
        assert torch.equal(pools[0].view(torch.uint8), ref_pools[0].view(torch.uint8)), f"key pool, part {part}"
        assert torch.equal(pools[1].view(torch.uint8), ref_pools[1].view(torch.uint8)), f"value pool, part {part}"
        ref = oracle_decode(st, h, tables)
        compare(st, fused, separate, ref, f"seed {seed} partition {part}", exact=not reordered(st, part))


@pytest.mark.parametrize("hq,part", [(8, -1), (32, 512), (32, 0)],
                         ids=["single-head balanced", "matrix-core partitions", "matrix-core single pass"])
def test_length_beyond_max_context_len_is_written_not_attended(hq, part):
    # the caller's max_context_len clamps the longest sequence: its new token is written (as the cache write
    # does) but lies past the positions attended over, in both forms
    st = custom_structure("a610", 610, [700, 33, 1200, 90], hq, 8, 128, 16, "bf16")
    t = materialize(st, DEV, include_new_token=True)
    mcl = 1100
    cl = st.context_lens  # sequence 2 (1200 positions) is beyond it
    pools = (t["key_cache"].clone(), t["value_cache"].clone())
    ref_pools = (t["key_cache"].clone(), t["value_cache"].clone())
    pa.reshape_and_cache(t["new_key"], t["new_value"], ref_pools[0], ref_pools[1], dev_i32(st.slot_mapping))
    separate = decode(st, dict(t, key_cache=ref_pools[0], value_cache=ref_pools[1]), st.block_tables_pre, part,
                      context_lens=cl, max_context_len=mcl)
    fused = appended(st, t, pools, st.block_tables_pre, st.slot_mapping, part, context_lens=cl,
                     max_context_len=mcl)
    assert torch.equal(pools[0].view(torch.uint8), ref_pools[0].view(torch.uint8))
    assert torch.equal(pools[1].view(torch.uint8), ref_pools[1].view(torch.uint8))
    if reordered(st, part):
        np.testing.assert_allclose(fused, separate, rtol=1e-5, atol=1e-6)
    else:
        np.testing.assert_array_equal(fused, separate)


@pytest.mark.parametrize("hq,part", [(8, pa.PA_PARTITION_BALANCED), (32, pa.PA_PARTITION_BALANCED), (32, -1)],
                         ids=["single-head balanced", "matrix-core balanced", "matrix-core default"])
def test_zero_max_context_len_still_writes(hq, part):
    # nothing is attended over (zero rows), and every new token still lands in its slot
    st = custom_structure("a616", 616, [300, 1, 45, 1000], hq, 8, 128, 16, "bf16")
    t = materialize(st, DEV, include_new_token=True)
    pools = (t["key_cache"].clone(), t["value_cache"].clone())
    ref_pools = (t["key_cache"].clone(), t["value_cache"].clone())
    write_separately(st, t, ref_pools, st.slot_mapping)
    fused = appended(st, t, pools, st.block_tables_pre, st.slot_mapping, part, max_context_len=0)
    assert torch.equal(pools[0].view(torch.uint8), ref_pools[0].view(torch.uint8))
    assert torch.equal(pools[1].view(torch.uint8), ref_pools[1].view(torch.uint8))
    np.testing.assert_array_equal(fused, np.zeros_like(fused))


@pytest.mark.parametrize("scale", [1 / 64, 0.3, 1.5 * 2.0 ** 33, 1.37 * 2.0 ** -40],
                         ids=["2^-6", "0.3", "above the kernels' range", "below the kernels' range"])
@pytest.mark.parametrize("hq,part", [(8, pa.PA_PARTITION_BALANCED), (32, 512)],
                         ids=["single-head balanced", "matrix-core partitions"])
def test_e4m3_scales_inside_and_outside_the_kernels_range(scale, hq, part):
    # the decode kernels quantise an appended row without a division, for |scale| in [2^-32, 2^32]; a call with a
    # scale outside that range writes the rows with the quantising cache write first and then attends. Either way
    # the pools end as reshape_and_cache_fp8 leaves them, and the output is the two calls' (bit for bit where the
    # cache write runs first, or on the matrix cores)
    st = custom_structure("a617", 617, [700, 33, 1200, 90, 2], hq, 8, 128, 16, "fp8")
    t = materialize(st, DEV, include_new_token=True)  # pool codes drawn for the default scale
    # the same codes read with the scale under test (the logits as before, so that the softmax stays as peaked
    # as the oracle comparison expects); the new rows are quantised with it
    st.scale = st.scale * st.k_scale / scale
    st.k_scale, st.v_scale = scale, scale * 0.75
    pools = (t["key_cache"].clone(), t["value_cache"].clone())
    ref_pools = (t["key_cache"].clone(), t["value_cache"].clone())
    write_separately(st, t, ref_pools, st.slot_mapping)
    h = {k: to_host(v) for k, v in t.items()}
    write_on_host(st, h, st.slot_mapping)
    separate = decode(st, dict(t, key_cache=ref_pools[0], value_cache=ref_pools[1]), st.block_tables_pre, part)
    fused = appended(st, t, pools, st.block_tables_pre, st.slot_mapping, part)
    assert torch.equal(pools[0].view(torch.uint8), ref_pools[0].view(torch.uint8))
    assert torch.equal(pools[1].view(torch.uint8), ref_pools[1].view(torch.uint8))
    np.testing.assert_array_equal(to_host(pools[0]).view(np.uint8), h["key_cache"].view(np.uint8))
    np.testing.assert_array_equal(to_host(pools[1]).view(np.uint8), h["value_cache"].view(np.uint8))
    inside = 2.0 ** -32 <= scale * 0.75 and scale <= 2.0 ** 32
    # the outputs scale with v_scale: compared in units of v_scale * 64, in which they are of order one (the unit
    # is 1 at the default scale) as the tolerances expect
    unit = st.v_scale * 64
    if inside and reordered(st, part):
        np.testing.assert_allclose(fused, separate, rtol=1e-5, atol=1e-6 * unit)
    else:
        np.testing.assert_array_equal(fused, separate)
    assert_attention_close(fused / unit, oracle_decode(st, h, st.block_tables_pre) / unit, st.dtype, f"scale {scale}")
