"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on the same seeded inputs.

Bar: bit-exact for reshape_and_cache (also its quantising FP8 form), copy_blocks and the block-table gather
(whole pools compared byte for byte, so untouched blocks, NaN-poisoned free slots and tails are covered);
attention within 1e-5 absolute for fp32 and within 2e-3 absolute + 1e-2 relative for bf16 or E4M3 K/V under a
bf16 query (fp32 accumulation), element by element.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_458_amd as pa
from tests._host import f64, to_host
from workloads import CONFIG_NAMES, build_structure, custom_structure, materialize

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


def assert_attention_close(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    err = np.abs(gpu.astype(np.float64) - ref)
    if dtype == "f32":
        bad = err > 1e-5
    else:  # bf16, or fp8 (E4M3 caches, bf16 query): both multiply bf16 operands with fp32 accumulation
        bad = err > 2e-3 + 1e-2 * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance, max err {err.max():.3e}"
    return float(err.max())


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def decode(st, t, tables, partition_size, context_lens=None, max_context_len=None):
    out = torch.empty((st.num_seqs, st.num_q_heads, st.head_dim), dtype=torch.float32, device=DEV)
    cl = st.context_lens if context_lens is None else context_lens
    pa.paged_attention_decode(out, t["query"], t["key_cache"], t["value_cache"], dev_i32(tables), dev_i32(cl),
                              st.scale, st.block_size, partition_size=partition_size,
                              max_context_len=st.max_context_len if max_context_len is None else max_context_len,
                              k_scale=st.k_scale, v_scale=st.v_scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def balanced_ok(st) -> bool:
    """Whether the library runs the balanced split for these sizes (either kernel)."""
    kd = {"f32": pa.PA_F32, "bf16": pa.PA_BF16, "fp8": pa.PA_FP8_E4M3}[st.dtype]
    return pa.load_library().paged_attention_partition_size(
        st.num_seqs, st.num_q_heads, st.num_kv_heads, st.head_dim, st.max_context_len, st.block_size, kd,
        pa.PA_PARTITION_BALANCED) == pa.PA_PARTITION_BALANCED


def oracle_decode(st, h, tables, context_lens=None, rows=None):
    cl = st.context_lens if context_lens is None else context_lens
    return oracle.decode(h["query"], h["key_cache"], h["value_cache"], tables, cl, st.scale, rows=rows,
                         k_scale=st.k_scale, v_scale=st.v_scale)


def step_writes(st, t, h):
    """The step's cache update on the device pools and on their host copies: copy-on-write pairs, then the
    new token's K/V (quantised into an E4M3 cache)."""
    if len(st.copy_pairs):
        pa.copy_blocks(t["key_cache"], t["value_cache"], dev_i32(st.copy_pairs))
        oracle.copy_blocks(h["key_cache"], h["value_cache"], st.copy_pairs)
    pa.reshape_and_cache(t["new_key"], t["new_value"], t["key_cache"], t["value_cache"], dev_i32(st.slot_mapping),
                         k_scale=st.k_scale, v_scale=st.v_scale)
    if st.dtype == "fp8":
        oracle.reshape_and_cache_e4m3(h["key_cache"], h["value_cache"], h["new_key"], h["new_value"],
                                      st.slot_mapping, st.k_scale, st.v_scale)
    else:
        oracle.reshape_and_cache(h["key_cache"], h["value_cache"], h["new_key"], h["new_value"], st.slot_mapping)


# --------------------------------------------------------------------------------------------------------
# small seeded cases: several tiles, ragged tails, every supported dtype / head_dim / group / block size

SMALL = [
    # (seed, lens, Hq, Hkv, D, bs, dtype)
    (201, [5, 17, 33, 64], 4, 4, 64, 16, "f32"),
    (202, [1, 16, 31, 100, 255], 8, 8, 128, 16, "f32"),
    (203, [7, 300, 129, 1000, 16], 32, 32, 128, 16, "bf16"),
    (204, [513, 2, 77, 1030], 16, 16, 64, 16, "bf16"),
    (205, [700, 1200, 45, 1], 32, 8, 128, 16, "bf16"),
    (206, [2050, 999, 513, 300], 64, 8, 128, 256, "bf16"),
    (207, [90, 33, 257, 16], 8, 2, 64, 32, "bf16"),
    (208, [600, 129, 64, 3], 16, 1, 128, 128, "bf16"),
    (209, [100, 45, 1, 65], 6, 3, 64, 64, "f32"),
    (210, [5, 17, 300, 64, 1030], 8, 8, 128, 16, "fp8"),
    (211, [100, 1, 65, 513], 4, 4, 64, 16, "fp8"),
    (212, [700, 1200, 45, 1], 32, 8, 128, 16, "fp8"),
    (213, [90, 33, 257, 16], 8, 2, 64, 32, "fp8"),
    (214, [2050, 999, 513, 300], 64, 8, 128, 256, "fp8"),
    # 8-slot blocks (page 1 section 5): a 16-token tile spans two blocks
    (215, [5, 17, 100, 64, 300, 8], 8, 8, 128, 8, "bf16"),
    (216, [90, 33, 257, 16, 1], 16, 4, 64, 8, "bf16"),
    (217, [700, 45, 513, 9], 32, 8, 128, 8, "fp8"),
    (218, [33, 64, 7, 200], 4, 4, 64, 8, "f32"),
    (219, [1100, 24, 520], 64, 8, 128, 8, "bf16"),
    # other head dims: row groups padded to a power of two of 16-byte chunks, tiles of 4..16 tokens (per-head
    # kernel); the grouped bf16 and E4M3 cases among them (222, 224) run on the matrix cores
    (220, [5, 17, 100, 300], 8, 8, 80, 16, "bf16"),
    (221, [33, 64, 129], 4, 2, 96, 16, "f32"),
    (222, [90, 513, 7], 16, 4, 112, 32, "fp8"),
    (223, [700, 45, 1], 8, 8, 192, 16, "bf16"),
    (224, [260, 33, 1000], 8, 2, 256, 16, "bf16"),
    (225, [100, 17, 70], 4, 4, 256, 8, "f32"),
    (226, [300, 8, 65], 4, 4, 80, 8, "fp8"),
    (227, [129, 64, 3], 4, 4, 192, 16, "f32"),
    (228, [515, 31, 2], 8, 8, 96, 16, "fp8"),
    (229, [400, 77], 8, 8, 256, 32, "fp8"),
    # two heads per wave in the balanced split (64- and 128-byte head rows), 8-slot blocks
    (230, [90, 33, 257, 16, 1], 8, 8, 128, 8, "fp8"),
    (231, [300, 8, 65, 1000], 4, 4, 64, 8, "bf16"),
    # grouped heads on the matrix cores at every head dim: rows padded to whole 16-byte pieces per power of two of
    # lanes, the score contraction zero-padded to 32-dim chunks (80, 112), K and V taking turns through one
    # register set and LDS slice for bf16 rows over 256 bytes (192, 256)
    (232, [700, 45, 1, 300], 32, 8, 80, 16, "bf16"),
    (233, [513, 90, 1030], 16, 4, 96, 16, "bf16"),
    (234, [260, 33, 1000, 7], 16, 2, 112, 32, "bf16"),
    (235, [700, 1200, 45, 1], 32, 4, 192, 16, "bf16"),
    (236, [2050, 999, 513, 300], 16, 2, 256, 256, "bf16"),
    (237, [90, 33, 257, 16, 1], 8, 2, 256, 8, "bf16"),
    (238, [700, 45, 1, 300], 32, 8, 80, 16, "fp8"),
    (239, [513, 90, 1030], 16, 4, 96, 8, "fp8"),
    (240, [260, 33, 1000, 7], 16, 2, 192, 32, "fp8"),
    (241, [2050, 999, 513, 300], 16, 2, 256, 256, "fp8"),
    (242, [129, 64, 3, 517], 24, 3, 112, 16, "fp8"),
    (243, [1500, 2, 64], 12, 6, 80, 64, "bf16"),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"seed{c[0]}" for c in SMALL])
def test_small_attention_parity(case):
    seed, lens, hq, hkv, d, bs, dt = case
    st = custom_structure(f"s{seed}", seed, lens, hq, hkv, d, bs, dt)
    t = materialize(st, DEV)
    h = {k: to_host(v) for k, v in t.items()}
    ref = oracle_decode(st, h, st.block_tables_pre)
    # 16 cuts GQA tiles across partitions; 32, 64, 96 and 512 let one GQA wave cover several partitions
    parts = (0, 16, 32, 64, 96, 512, -1) + ((pa.PA_PARTITION_BALANCED,) if balanced_ok(st) else ())
    for part in parts:
        gpu = decode(st, t, st.block_tables_pre, part)
        assert_attention_close(gpu, ref, dt, f"partition {part}")


@pytest.mark.parametrize("dt,bs,d", [("f32", 16, 64), ("bf16", 16, 64), ("fp8", 16, 64), ("bf16", 8, 64),
                                     ("fp8", 8, 128), ("bf16", 16, 80), ("fp8", 16, 112), ("f32", 8, 192)])
def test_small_cache_ops_bit_exact(dt, bs, d):
    # (E4M3 rows of 64 dims need blocks of >= 16 slots)
    st = custom_structure("ops", 301, [65, 77, 96, 100, 130, 81], 8, 2, d, bs, dt, shared_prefix_blocks=4,
                          cow_seqs=3, pool_factor=1.5)
    t = materialize(st, DEV, include_new_token=False)
    h = {k: to_host(v) for k, v in t.items()}
    step_writes(st, t, h)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(t["key_cache"]).view(np.uint8), h["key_cache"].view(np.uint8))
    np.testing.assert_array_equal(to_host(t["value_cache"]).view(np.uint8), h["value_cache"].view(np.uint8))
    gpu = decode(st, t, st.block_tables, -1)
    assert_attention_close(gpu, oracle_decode(st, h, st.block_tables), dt)


@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_fp8_quantiser_special_values_bit_exact(src):
    # every E4M3 code value, the midpoints between neighbours (ties to even), values past the largest finite
    # code (saturation), NaN, infinities, signed zeros, tiny values, then random data, at several scales
    vals = oracle.e4m3_values()
    fin = vals[~np.isnan(vals)]
    pos = np.sort(vals[(vals >= 0) & ~np.isnan(vals)])
    special = np.concatenate([fin, (pos[:-1] + pos[1:]) / 2, -(pos[:-1] + pos[1:]) / 2,
                              [464.0, 479.0, 480.0, 1e6, -1e6, np.inf, -np.inf, np.nan, -np.nan, 0.0, -0.0, 1e-30,
                               -1e-30, 2.0 ** -10, 3 * 2.0 ** -11]])
    rng = np.random.default_rng(501)
    x = np.concatenate([special, rng.standard_normal(4096) * rng.choice([1e-3, 1.0, 100.0, 1e4], 4096)])
    x = x.astype(np.float32)
    hkv, d = 2, 32
    x = np.concatenate([x, np.zeros((-x.size) % (hkv * d), np.float32)]).reshape(-1, hkv, d)
    n = x.shape[0]
    src_t = torch.from_numpy(x)
    if src == "bf16":
        src_t = src_t.to(torch.bfloat16)
    host_src = to_host(src_t)
    nb, bs = -(-n // 16) + 1, 16
    slots = np.random.default_rng(502).permutation(nb * bs)[:n].astype(np.int32)
    for ks, vs in ((1.0, 1.0), (0.0125, 3.0), (2.0 ** -6, 0.3)):
        kc = torch.full((nb, bs, hkv, d), float("nan"), device=DEV).to(torch.float8_e4m3fn)
        vc = kc.clone()
        k_dev = src_t.to(DEV)
        v_dev = (-src_t).to(DEV)
        pa.reshape_and_cache(k_dev, v_dev, kc, vc, dev_i32(slots), k_scale=ks, v_scale=vs)
        torch.cuda.synchronize()
        hk = np.full((nb, bs, hkv, d), 0x7F, np.uint8)
        hv = hk.copy()
        oracle.reshape_and_cache_e4m3(hk, hv, host_src, to_host(-src_t), slots, ks, vs)
        np.testing.assert_array_equal(to_host(kc), hk, err_msg=f"k_scale {ks}")
        np.testing.assert_array_equal(to_host(vc), hv, err_msg=f"v_scale {vs}")


@pytest.mark.parametrize("scale", [0.0125, 1 / 3, 0.3, 7.0, -0.7, 1.37 * 2.0 ** -40, 2.0 ** -32, 1.999 * 2.0 ** 31,
                                   1.5 * 2.0 ** 32])
def test_fp8_quantiser_every_bf16_value(scale):
    # the quantiser divides by the scale without a division per value (a reciprocal and one fma correction) for
    # scales of magnitude 2^-32 .. 2^32 and divides outside that range: every finite and non-finite bf16 bit
    # pattern as key, its negation as value, and for a float32 source the values whose quotient lies at or one
    # ulp either side of every E4M3 code and every midpoint between neighbouring codes
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    vals = oracle.e4m3_values()
    pos = np.sort(vals[(vals >= 0) & ~np.isnan(vals)])
    targets = np.concatenate([pos, (pos[:-1] + pos[1:]) / 2, [464.0, 480.0]])
    targets = np.concatenate([targets, -targets])
    near = (targets * np.float64(np.float32(scale))).astype(np.float32)
    near = np.concatenate([near, np.nextafter(near, np.float32(np.inf)), np.nextafter(near, np.float32(-np.inf))])
    hkv, d = 2, 32
    for src, data in (("bf16", x), ("f32", near)):
        data = np.concatenate([data, np.zeros((-data.size) % (hkv * d), np.float32)]).reshape(-1, hkv, d)
        n = data.shape[0]
        src_t = torch.from_numpy(data)
        if src == "bf16":
            src_t = src_t.to(torch.bfloat16)
        host_src = to_host(src_t)
        nb, bs = -(-n // 16) + 1, 16
        slots = np.random.default_rng(503).permutation(nb * bs)[:n].astype(np.int32)
        kc = torch.full((nb, bs, hkv, d), float("nan"), device=DEV).to(torch.float8_e4m3fn)
        vc = kc.clone()
        pa.reshape_and_cache(src_t.to(DEV), (-src_t).to(DEV), kc, vc, dev_i32(slots), k_scale=scale, v_scale=scale)
        torch.cuda.synchronize()
        hk = np.full((nb, bs, hkv, d), 0x7F, np.uint8)
        hv = hk.copy()
        oracle.reshape_and_cache_e4m3(hk, hv, host_src, to_host(-src_t), slots, scale, scale)
        np.testing.assert_array_equal(to_host(kc), hk, err_msg=f"{src} scale {scale}")
        np.testing.assert_array_equal(to_host(vc), hv, err_msg=f"{src} scale {scale}")


def test_reshape_skips_padding_and_out_of_pool_slots():
    st = custom_structure("skip", 302, [20, 40, 9], 4, 4, 64, 16, "bf16")
    t = materialize(st, DEV, include_new_token=False)
    before_k, before_v = to_host(t["key_cache"]), to_host(t["value_cache"])
    slots = st.slot_mapping.copy()
    slots[1] = -1
    slots[2] = st.num_blocks * st.block_size  # one past the pool
    pa.reshape_and_cache(t["new_key"], t["new_value"], t["key_cache"], t["value_cache"], dev_i32(slots))
    torch.cuda.synchronize()
    oracle_slots = slots.copy()
    oracle_slots[2] = -1  # the kernel skips it; the oracle would reject it
    oracle.reshape_and_cache(before_k, before_v, to_host(t["new_key"]), to_host(t["new_value"]), oracle_slots)
    np.testing.assert_array_equal(to_host(t["key_cache"]), before_k)
    np.testing.assert_array_equal(to_host(t["value_cache"]), before_v)


@pytest.mark.parametrize("bs,dt", [(16, "bf16"), (256, "bf16"), (32, "f32"), (16, "fp8"), (8, "bf16"), (8, "fp8")])
def test_gather_bit_exact(bs, dt):
    st = custom_structure("gather", 303, [1, 15, 16, 17, 300, 513], 8, 4, 128, bs, dt)
    t = materialize(st, DEV)
    mcl = st.max_context_len
    ok = torch.full((st.num_seqs, mcl, st.num_kv_heads, st.head_dim), float("nan"),
                    device=DEV).to(t["key_cache"].dtype)
    ov = ok.clone()
    pa.paged_gather(ok, ov, t["key_cache"], t["value_cache"], dev_i32(st.block_tables_pre), dev_i32(st.context_lens))
    torch.cuda.synchronize()
    gk, gv = to_host(ok), to_host(ov)
    hk, hv = to_host(t["key_cache"]), to_host(t["value_cache"])
    rk = oracle.gather(hk, st.block_tables_pre, st.context_lens)
    rv = oracle.gather(hv, st.block_tables_pre, st.context_lens)
    r = 0
    for s, L in enumerate(st.context_lens):
        np.testing.assert_array_equal(gk[s, :L].view(np.uint8), rk[r:r + L].view(np.uint8))
        np.testing.assert_array_equal(gv[s, :L].view(np.uint8), rv[r:r + L].view(np.uint8))
        if dt == "fp8":
            assert (gk[s, L:] == 0x7F).all()  # rows past the length untouched (the NaN code)
        else:
            assert np.isnan(f64(gk[s, L:])).all()  # rows past the length untouched
        r += L


# --------------------------------------------------------------------------------------------------------
# invariants on the GPU


def test_permutation_and_determinism_bit_identical():
    st = custom_structure("perm", 401, [700, 33, 1500, 260], 32, 8, 128, 16, "bf16", pool_factor=1.5)
    t = materialize(st, DEV)
    a = decode(st, t, st.block_tables_pre, -1)
    b = decode(st, t, st.block_tables_pre, -1)
    np.testing.assert_array_equal(a, b)
    perm = torch.from_numpy(np.random.default_rng(402).permutation(st.num_blocks)).to(DEV)
    t2 = dict(t)
    t2["key_cache"] = torch.empty_like(t["key_cache"])
    t2["value_cache"] = torch.empty_like(t["value_cache"])
    t2["key_cache"][perm] = t["key_cache"]
    t2["value_cache"][perm] = t["value_cache"]
    tables = perm.cpu().numpy()[st.block_tables_pre]
    c = decode(st, t2, tables, -1)
    np.testing.assert_array_equal(a, c)


def test_single_token_is_exact_value_row():
    for dt, hq, hkv in (("f32", 4, 4), ("bf16", 32, 32), ("bf16", 32, 8), ("bf16", 64, 8), ("fp8", 32, 32),
                        ("fp8", 32, 8)):
        st = custom_structure("one", 411, [1, 1, 1], hq, hkv, 128, 16, dt)
        t = materialize(st, DEV)
        gpu = decode(st, t, st.block_tables_pre, -1)
        hv = to_host(t["value_cache"])
        # with a power-of-two v_scale the output row is code value x v_scale exactly
        v = oracle.e4m3_values()[hv] * st.v_scale if dt == "fp8" else f64(hv)
        G = hq // hkv
        for s in range(3):
            b = st.block_tables_pre[s, 0]
            for hh in range(hq):
                np.testing.assert_array_equal(gpu[s, hh], v[b, 0, hh // G].astype(np.float32))


def test_one_hot_locates_a_single_position():
    st = custom_structure("hot", 421, [1000, 77], 8, 8, 128, 16, "bf16")
    t = materialize(st, DEV)
    for s, pos in ((0, 613), (1, 76)):
        b, off = st.block_tables_pre[s, pos // 16], pos % 16
        t["key_cache"][b, off] = t["query"][s]
    h = {k: to_host(v) for k, v in t.items()}
    st.scale = 4.0
    gpu = decode(st, t, st.block_tables_pre, 64)
    ref = oracle_decode(st, h, st.block_tables_pre)
    assert_attention_close(gpu, ref, "bf16")
    for s, pos in ((0, 613), (1, 76)):
        b, off = st.block_tables_pre[s, pos // 16], pos % 16
        np.testing.assert_allclose(gpu[s], f64(h["value_cache"][b, off]), atol=2e-3)


def test_empty_context_bad_entries_and_clamped_lengths():
    st = custom_structure("edge", 431, [0, 40, 300, 500], 8, 8, 64, 16, "bf16", max_context_len=512)
    t = materialize(st, DEV)
    h = {k: to_host(v) for k, v in t.items()}
    tables = st.block_tables_pre.copy()
    tables[2, 3] = st.num_blocks + 7  # a live entry outside the pool: that sequence's rows become NaN
    lens = st.context_lens.copy()
    lens[3] = 600  # past max_context_len (512): clamped
    for part in (0, 64, -1):
        gpu = decode(st, t, tables, part, context_lens=lens)
        assert (gpu[0] == 0).all()
        assert np.isnan(gpu[2]).all()
        # positions 500..511 read slots that the generator poisoned: clamping to 512 must surface them as NaN
        assert np.isnan(gpu[3]).all()
        ref = oracle_decode(st, h, st.block_tables_pre)
        assert_attention_close(gpu[[1]], ref[[1]], "bf16", f"partition {part}")


# --------------------------------------------------------------------------------------------------------
# the balanced split: equal runs of tiles cut rows anywhere; rows that attend over nothing get zero rows


@pytest.mark.parametrize("lens,hq,d,dt", [
    ([0, 0, 700, 1, 0, 3000, 45, 0, 0], 8, 128, "bf16"),   # empty rows before, between and after
    ([5000], 2, 64, "f32"),                                # one row cut into about a thousand runs
    ([3, 1, 2, 17, 16, 15, 33] * 9, 32, 80, "fp8"),        # many short rows per run
    ([900, 1300, 20, 2500], 16, 256, "bf16"),              # few rows, 512-byte head rows
    # two adjacent heads per wave where head rows are 64 or 128 bytes
    ([0, 0, 700, 1, 0, 3000, 45, 0, 0], 8, 128, "fp8"),    # empty rows, E4M3 128-byte rows
    ([3, 1, 2, 17, 16, 15, 33] * 9, 5, 128, "fp8"),        # odd head count: the last wave holds one head
    ([900, 1300, 20, 2500], 6, 64, "bf16"),                # bf16 128-byte rows
    ([5000], 2, 64, "fp8"),                                # E4M3 64-byte rows, one row cut into many runs
    ([3, 1, 2, 17, 16, 15, 33] * 9, 5, 128, "bf16"),       # bf16 256-byte rows, odd head count: 8-token tiles
    ([4000, 1, 0, 900], 4, 128, "bf16"),                   # a row cut into many runs, 512-byte pieces
])
def test_balanced_split_parity(lens, hq, d, dt):
    st = custom_structure("bal", 441, lens, hq, hq, d, 16, dt, pool_factor=1.2)
    assert balanced_ok(st)
    t = materialize(st, DEV)
    h = {k: to_host(v) for k, v in t.items()}
    ref = oracle_decode(st, h, st.block_tables_pre)
    a = decode(st, t, st.block_tables_pre, pa.PA_PARTITION_BALANCED)
    assert_attention_close(a, ref, dt, "balanced")
    empty = np.asarray(lens) == 0
    assert (a[empty] == 0).all()
    np.testing.assert_array_equal(a, decode(st, t, st.block_tables_pre, pa.PA_PARTITION_BALANCED))


@pytest.mark.parametrize("dt", ["bf16", "fp8"])  # fp8: two heads per wave
def test_balanced_split_edge_cases(dt):
    # a bad table entry in a row that several runs cut poisons that row only, through the merge
    st = custom_structure("baledge", 442, [4000, 64, 2500, 0], 4, 4, 128, 16, dt, max_context_len=4096)
    t = materialize(st, DEV)
    h = {k: to_host(v) for k, v in t.items()}
    tables = st.block_tables_pre.copy()
    tables[2, 100] = -3
    lens = st.context_lens.copy()
    lens[1] = 9000  # clamped to max_context_len: positions past the sequence's own blocks are poisoned slots
    gpu = decode(st, t, tables, pa.PA_PARTITION_BALANCED, context_lens=lens)
    assert np.isnan(gpu[2]).all() and np.isnan(gpu[1]).all() and (gpu[3] == 0).all()
    ref = oracle_decode(st, h, st.block_tables_pre)
    assert_attention_close(gpu[[0]], ref[[0]], dt, "balanced")
    # every row empty: zero rows, no tile to read
    z = decode(st, t, tables, pa.PA_PARTITION_BALANCED, context_lens=np.zeros(4, np.int32))
    assert (z == 0).all()


# the matrix-core kernel's balanced split (grouped heads at head_dim 64 / 128, bf16 or E4M3 caches): runs of
# 32-token tiles cut sequences anywhere; the partials share the single-head split's layout and merge


@pytest.mark.parametrize("lens,hq,hkv,d,bs,dt", [
    ([0, 0, 700, 1, 0, 3000, 45, 0, 0], 32, 8, 128, 16, "bf16"),       # empty sequences before, between, after
    ([20000], 16, 2, 64, 16, "bf16"),                                  # one sequence cut into 625 one-tile runs
    ([3, 1, 2, 17, 16, 15, 33, 64, 65] * 40, 8, 4, 128, 8, "fp8"),     # many short sequences, 8-slot blocks
    ([2050, 999, 513, 300, 4096, 1], 64, 8, 128, 256, "bf16"),         # 256-slot blocks, 8 heads per KV head
    ([900, 1300, 20, 2500], 16, 1, 128, 128, "fp8"),                   # 16 heads on one KV head
    ([129, 4000, 31, 777, 64], 24, 12, 64, 32, "bf16"),                # 12 KV heads: two workgroups per run
    ([0, 2300, 1, 700, 45, 0], 32, 4, 256, 16, "bf16"),                # K and V take turns through one slice
    ([3, 1, 2, 17, 16, 15, 33, 64, 65] * 20, 16, 4, 192, 8, "fp8"),    # padded row lanes, many short sequences
    ([900, 1300, 20, 2500], 16, 2, 80, 32, "bf16"),                    # zero-padded score contraction
])
def test_gqa_balanced_split_parity(lens, hq, hkv, d, bs, dt):
    st = custom_structure("gbal", 443, lens, hq, hkv, d, bs, dt, pool_factor=1.2)
    assert balanced_ok(st)
    t = materialize(st, DEV)
    h = {k: to_host(v) for k, v in t.items()}
    ref = oracle_decode(st, h, st.block_tables_pre)
    a = decode(st, t, st.block_tables_pre, pa.PA_PARTITION_BALANCED)
    assert_attention_close(a, ref, dt, "balanced")
    empty = np.asarray(lens) == 0
    assert (a[empty] == 0).all()
    np.testing.assert_array_equal(a, decode(st, t, st.block_tables_pre, pa.PA_PARTITION_BALANCED))
    # permuting the physical blocks leaves the output bit for bit the same
    perm = np.random.default_rng(444).permutation(st.num_blocks)
    kp, vp = torch.empty_like(t["key_cache"]), torch.empty_like(t["value_cache"])
    idx = torch.from_numpy(perm).to(DEV)
    kp[idx], vp[idx] = t["key_cache"], t["value_cache"]
    tp = dict(t, key_cache=kp, value_cache=vp)
    np.testing.assert_array_equal(a, decode(st, tp, perm[st.block_tables_pre], pa.PA_PARTITION_BALANCED))


def test_gqa_balanced_split_at_its_row_limit():
    # 2048 sequences, the most the workgroups' tile-count scan takes (the one beyond is refused)
    lens = np.random.default_rng(446).integers(0, 300, size=2048)
    st = custom_structure("gbalmax", 446, lens, 16, 4, 128, 16, "bf16", pool_factor=1.05)
    assert balanced_ok(st)
    t = materialize(st, DEV)
    h = {k: to_host(v) for k, v in t.items()}
    gpu = decode(st, t, st.block_tables_pre, pa.PA_PARTITION_BALANCED)
    ref = oracle_decode(st, h, st.block_tables_pre)
    assert_attention_close(gpu, ref, "bf16", "2048 sequences")
    assert (gpu[lens == 0] == 0).all()
    np.testing.assert_allclose(gpu, decode(st, t, st.block_tables_pre, 256), rtol=1e-2, atol=2e-3)


def test_gqa_balanced_split_edge_cases():
    st = custom_structure("gbaledge", 445, [4000, 64, 2500, 0, 3000], 32, 8, 128, 16, "bf16", max_context_len=4096)
    assert balanced_ok(st)
    t = materialize(st, DEV)
    h = {k: to_host(v) for k, v in t.items()}
    tables = st.block_tables_pre.copy()
    tables[2, 100] = -3  # a bad entry in a sequence that several runs cut poisons that sequence only
    lens = st.context_lens.copy()
    lens[1] = 9000  # clamped to max_context_len: positions past the sequence's own blocks are poisoned slots
    gpu = decode(st, t, tables, pa.PA_PARTITION_BALANCED, context_lens=lens)
    assert np.isnan(gpu[2]).all() and np.isnan(gpu[1]).all() and (gpu[3] == 0).all()
    ref = oracle_decode(st, h, st.block_tables_pre)
    assert_attention_close(gpu[[0, 4]], ref[[0, 4]], "bf16", "balanced")
    z = decode(st, t, tables, pa.PA_PARTITION_BALANCED, context_lens=np.zeros(5, np.int32))
    assert (z == 0).all()
    # several new tokens per sequence take it while grouped heads x rows fill one column group of 16, and are
    # refused beyond that
    lib = pa.load_library()
    assert lib.paged_attention_multi_partition_size(
        5, 20, 4, 32, 8, 128, 4096, 16, pa.PA_BF16, pa.PA_PARTITION_BALANCED) == pa.PA_PARTITION_BALANCED
    assert lib.paged_attention_multi_partition_size(
        5, 40, 8, 32, 8, 128, 4096, 16, pa.PA_BF16, pa.PA_PARTITION_BALANCED) == -4  # PA_ERR_UNSUPPORTED


# --------------------------------------------------------------------------------------------------------
# the five workloads at full size, in the launch configuration the benchmark times


@pytest.mark.parametrize("name", CONFIG_NAMES)
def test_full_workload_step(name):
    st = build_structure(name)
    t = materialize(st, DEV, include_new_token=False)
    h = {k: to_host(v) for k, v in t.items()}
    step_writes(st, t, h)
    gpu = decode(st, t, st.block_tables, st.partition_size)
    gk, gv = to_host(t["key_cache"]), to_host(t["value_cache"])
    assert np.array_equal(gk.view(np.uint8), h["key_cache"].view(np.uint8)), "key pool differs after the step"
    assert np.array_equal(gv.view(np.uint8), h["value_cache"].view(np.uint8)), "value pool differs after the step"
    del gk, gv
    ref = oracle_decode(st, h, st.block_tables)
    err = assert_attention_close(gpu, ref, st.dtype, name)
    sys.__stderr__.write(f"[{name}] max abs err {err:.3e}\n")
    if len(st.copy_pairs):
        # copy-on-write leaves every output unchanged (bit for bit) against reading the shared blocks
        pre = decode(st, t, st.block_tables_pre, st.partition_size)
        np.testing.assert_array_equal(gpu, pre)


@pytest.mark.parametrize("name", ["gqa_d256", "gqa_d256_fp8"])
def test_full_size_head_dim_256(name):
    # 64 sequences of 1k-4k tokens, 8 query heads per KV head of 256 dims, on the matrix cores, every output
    # element against the oracle, for the library's plan and explicit partitions
    st = build_structure(name)
    t = materialize(st, DEV)
    h = {k: to_host(v) for k, v in t.items()}
    ref = oracle_decode(st, h, st.block_tables_pre)
    for part in (-1, 512, pa.PA_PARTITION_BALANCED):
        gpu = decode(st, t, st.block_tables_pre, part)
        err = assert_attention_close(gpu, ref, st.dtype, f"{name} partition {part}")
        sys.__stderr__.write(f"[{name} partition {part}] max abs err {err:.3e}\n")


# --------------------------------------------------------------------------------------------------------
# maximum sizes: very long contexts (thousands of partitions, 64-bit pool offsets) and the grid's sequence limit


@pytest.mark.parametrize("hq,hkv,dt", [(8, 8, "bf16"), (32, 8, "bf16"), (16, 4, "fp8")])
def test_very_long_contexts(hq, hkv, dt):
    st = custom_structure("long", 451, [131072, 70001, 5], hq, hkv, 128, 16, dt, pool_factor=1.02)
    t = materialize(st, DEV, chunk_blocks=4096)
    h = {k: to_host(v) for k, v in t.items()}
    ref = oracle_decode(st, h, st.block_tables_pre)  # every (sequence, head) row
    for part in (-1, 4096):
        gpu = decode(st, t, st.block_tables_pre, part)
        err = assert_attention_close(gpu, ref, dt, f"partition {part}")
        sys.__stderr__.write(f"[long {hq}/{hkv} {dt} partition {part}] max abs err {err:.3e}\n")


def test_grid_limit_of_sequences():
    # 65535 sequences (the grid's z limit) of 0..3 tokens each, one head of 64 dims
    B = 65535
    lens = np.random.default_rng(452).integers(0, 4, size=B)
    st = custom_structure("many", 452, lens, 1, 1, 64, 16, "bf16", pool_factor=1.0)
    t = materialize(st, DEV)
    h = {k: to_host(v) for k, v in t.items()}
    gpu = decode(st, t, st.block_tables_pre, -1)
    ref = oracle_decode(st, h, st.block_tables_pre)
    assert_attention_close(gpu, ref, "bf16", "65535 sequences")
    assert (gpu[lens == 0] == 0).all()
