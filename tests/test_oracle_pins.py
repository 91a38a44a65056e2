"""Pins for the CPU oracle: values fixed by the pages and by mathematics, not by the oracle itself.

Each pin is a function of the oracle library so that ``test_pins_catch_planted_mistakes`` can run the same pins
against copies of the oracle with a mistake planted in them (on the CPU) and show that each mistake is caught.
"""

from __future__ import annotations

import json
import math
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from oracle import brute
from tests._host import f64, small_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _val(x, dtype):
    if dtype == "bf16":
        return np.uint16(int(x, 16)) if x is not None else np.uint16(0x7FC0)
    return np.float32(np.nan if x is None else x)


def _arr(nested, dtype):
    a = np.array(nested, dtype=object)
    npdt = np.uint16 if dtype == "bf16" else np.float32
    return np.vectorize(lambda x: _val(x, dtype), otypes=[npdt])(a) if a.size else np.zeros(a.shape, npdt)


def _empty_pool(c):
    npdt = np.uint16 if c["dtype"] == "bf16" else np.float32
    shape = (c["num_blocks"], c["block_size"], c["num_kv_heads"], c["head_dim"])
    fill = 0x7FC0 if c["dtype"] == "bf16" else np.nan
    return np.full(shape, fill, dtype=npdt)


def _golden_decode_inputs(c):
    kc, vc = _empty_pool(c), _empty_pool(c)
    for pool, key in ((kc, "key_blocks"), (vc, "value_blocks")):
        for b, rows in c[key].items():
            r = _arr(rows, c["dtype"])
            pool[int(b), : r.shape[0]] = r
    q = _arr(c["query"], c["dtype"])
    scale = math.log(3.0) if c["scale"] == "ln3" else float(c["scale"])
    return q, kc, vc, np.array(c["block_tables"], np.int32), np.array(c["context_lens"], np.int32), scale


# ----------------------------------------------------------------------------------------------------------
# pins, each a function of the oracle library


def pin_golden_decode(lib):
    for c in _golden_cases():
        if c["kind"] != "decode":
            continue
        q, kc, vc, bt, cl, scale = _golden_decode_inputs(c)
        out = oracle.decode(q, kc, vc, bt, cl, scale, lib=lib)
        np.testing.assert_allclose(out, np.array(c["expected"]), rtol=0, atol=4e-15, err_msg=c["name"])


def pin_golden_cache_ops(lib):
    for c in _golden_cases():
        if c["kind"] == "reshape":
            kc, vc = _empty_pool(c), _empty_pool(c)
            kc[:] = 0
            vc[:] = 0
            oracle.reshape_and_cache(kc, vc, _arr(c["key"], c["dtype"]), _arr(c["value"], c["dtype"]),
                                     np.array(c["slot_mapping"], np.int32), lib=lib)
            for pool, key in ((kc, "expected_key_blocks"), (vc, "expected_value_blocks")):
                want = np.zeros_like(pool)
                for b, slots in c[key].items():
                    for off, row in slots.items():
                        want[int(b), int(off)] = _arr(row, c["dtype"])
                np.testing.assert_array_equal(pool, want, err_msg=c["name"])
        elif c["kind"] == "copy":
            kc, vc = _arr(c["key_pool"], c["dtype"]), _arr(c["value_pool"], c["dtype"])
            oracle.copy_blocks(kc, vc, np.array(c["pairs"], np.int32), lib=lib)
            np.testing.assert_array_equal(kc, _arr(c["expected_key_pool"], c["dtype"]), err_msg=c["name"])
            np.testing.assert_array_equal(vc, _arr(c["expected_value_pool"], c["dtype"]), err_msg=c["name"])


BRUTE_SWEEP = [
    # (seed, lens, Hq, Hkv, D, bs, dtype)
    (11, [1, 7, 40], 2, 2, 8, 1, "f32"),
    (12, [5, 16, 17, 33], 4, 2, 16, 2, "f32"),
    (13, [40, 3], 4, 1, 8, 16, "bf16"),
    (14, [31, 32, 1, 2], 8, 2, 16, 16, "bf16"),
    (15, [9, 0, 23], 4, 4, 8, 2, "bf16"),
    (16, [40, 39, 38, 37], 4, 4, 4, 16, "f32"),
]


def pin_brute_force(lib):
    for seed, lens, hq, hkv, d, bs, dt in BRUTE_SWEEP:
        st, h = small_case(seed, lens, hq, hkv, d, bs, dt, scale=0.7)
        a = oracle.decode(h["query"], h["key_cache"], h["value_cache"], st.block_tables_pre, st.context_lens,
                          st.scale, lib=lib)
        b = brute.decode(h["query"], h["key_cache"], h["value_cache"], st.block_tables_pre, st.context_lens,
                         st.scale)
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12, err_msg=f"seed {seed}")


def pin_paged_equals_contiguous(lib):
    rng = np.random.default_rng(21)
    B, Hkv, G, D, bs, max_len = 3, 2, 2, 16, 4, 23
    lens = np.array([23, 1, 10], np.int32)
    kcont = rng.standard_normal((B, Hkv, max_len, D)).astype(np.float32)
    vcont = rng.standard_normal((B, Hkv, max_len, D)).astype(np.float32)
    q = rng.standard_normal((B, Hkv * G, D)).astype(np.float32)
    mb = -(-max_len // bs)
    nb = B * mb + 1
    ids = rng.permutation(nb - 1)
    tables = ids.reshape(B, mb).astype(np.int32)
    kc = np.full((nb, bs, Hkv, D), np.nan, np.float32)
    vc = np.full((nb, bs, Hkv, D), np.nan, np.float32)
    pad = mb * bs
    for s in range(B):
        # [Hkv, L, D] -> [L_pad, Hkv, D] -> [blocks, bs, Hkv, D], scattered by numpy reshape, not by index math
        for src, dst in ((kcont, kc), (vcont, vc)):
            seq = np.full((pad, Hkv, D), np.nan, np.float32)
            seq[: lens[s]] = src[s, :, : lens[s]].transpose(1, 0, 2)
            dst[tables[s]] = seq.reshape(mb, bs, Hkv, D)
    a = oracle.decode(q, kc, vc, tables, lens, 0.3, lib=lib)
    b = brute.contiguous_decode(q, kcont, vcont, lens, 0.3)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def pin_permutation_invariance(lib):
    st, h = small_case(31, [17, 33, 5, 48], 4, 2, 16, 16, "bf16", pool_factor=2.0)
    ref = oracle.decode(h["query"], h["key_cache"], h["value_cache"], st.block_tables_pre, st.context_lens,
                        st.scale, lib=lib)
    perm = np.random.default_rng(32).permutation(st.num_blocks)
    kc, vc = np.empty_like(h["key_cache"]), np.empty_like(h["value_cache"])
    kc[perm] = h["key_cache"]
    vc[perm] = h["value_cache"]
    tables = perm[st.block_tables_pre].astype(np.int32)
    out = oracle.decode(h["query"], kc, vc, tables, st.context_lens, st.scale, lib=lib)
    np.testing.assert_array_equal(out, ref)


def pin_shared_equals_copied(lib):
    st, h = small_case(41, [70, 65, 80], 4, 2, 8, 16, "f32", shared_prefix_blocks=4)
    ref = oracle.decode(h["query"], h["key_cache"], h["value_cache"], st.block_tables_pre, st.context_lens,
                        st.scale, lib=lib)
    # give every sequence private copies of the shared prefix blocks (numpy fancy indexing)
    shared = st.block_tables_pre[0, :4]
    nb = st.num_blocks
    extra = st.num_seqs * 4
    kc = np.concatenate([h["key_cache"], np.zeros((extra,) + h["key_cache"].shape[1:], np.float32)])
    vc = np.concatenate([h["value_cache"], np.zeros((extra,) + h["value_cache"].shape[1:], np.float32)])
    tables = st.block_tables_pre.copy()
    for s in range(st.num_seqs):
        new = np.arange(nb + 4 * s, nb + 4 * s + 4)
        kc[new] = h["key_cache"][shared]
        vc[new] = h["value_cache"][shared]
        tables[s, :4] = new
    out = oracle.decode(h["query"], kc, vc, tables, st.context_lens, st.scale, lib=lib)
    np.testing.assert_array_equal(out, ref)


def pin_single_token(lib):
    for dt in ("f32", "bf16"):
        st, h = small_case(51, [1, 1, 1], 4, 2, 16, 16, dt)
        out = oracle.decode(h["query"], h["key_cache"], h["value_cache"], st.block_tables_pre, st.context_lens,
                            st.scale, lib=lib)
        v = f64(h["value_cache"])
        for s in range(st.num_seqs):
            b = st.block_tables_pre[s, 0]
            for hh in range(4):
                np.testing.assert_array_equal(out[s, hh], v[b, 0, hh // 2])


def pin_identical_keys_and_positions(lib):
    st, h = small_case(61, [40, 17, 3], 2, 2, 8, 4, "f32")
    kc, vc = h["key_cache"].copy(), h["value_cache"].copy()
    live = ~np.isnan(kc[:, :, 0, 0])
    kc[live] = kc[st.block_tables_pre[0, 0], 0]  # one key everywhere: every weight equal
    # value dim 0 holds the logical position t of its slot, so the mean over 0..L-1 is (L-1)/2
    for s in range(st.num_seqs):
        for t in range(int(st.context_lens[s])):
            vc[st.block_tables_pre[s, t // 4], t % 4, :, 0] = t
    out = oracle.decode(h["query"], kc, vc, st.block_tables_pre, st.context_lens, st.scale, lib=lib)
    for s in range(st.num_seqs):
        L = int(st.context_lens[s])
        np.testing.assert_allclose(out[s, :, 0], (L - 1) / 2.0, rtol=0, atol=1e-12)
    # scale 0 with random keys gives the same mean of V
    out0 = oracle.decode(h["query"], h["key_cache"], vc, st.block_tables_pre, st.context_lens, 0.0, lib=lib)
    np.testing.assert_allclose(out0, out, rtol=0, atol=1e-12)


def pin_gqa_replication(lib):
    for g in (2, 4, 8):
        st, h = small_case(70 + g, [33, 20], 2 * g, 2, 16, 16, "bf16")
        gqa = oracle.decode(h["query"], h["key_cache"], h["value_cache"], st.block_tables_pre, st.context_lens,
                            st.scale, lib=lib)
        kc = np.repeat(h["key_cache"], g, axis=2)  # KV head j becomes MHA heads j*g .. j*g+g-1
        vc = np.repeat(h["value_cache"], g, axis=2)
        mha = oracle.decode(h["query"], kc, vc, st.block_tables_pre, st.context_lens, st.scale, lib=lib)
        np.testing.assert_array_equal(gqa, mha)


def pin_block_size_invariance(lib):
    rng = np.random.default_rng(81)
    lens = np.array([300, 17, 256], np.int32)
    Hkv, D = 2, 8
    seqk = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    seqv = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    q = rng.standard_normal((3, 4, D)).astype(np.float32)
    outs = []
    for bs in (1, 16, 256):
        mb = -(-300 // bs)
        nb = 3 * mb + 1
        ids = np.random.default_rng(bs).permutation(nb - 1).reshape(3, mb).astype(np.int32)
        kc = np.full((nb, bs, Hkv, D), np.nan, np.float32)
        vc = np.full((nb, bs, Hkv, D), np.nan, np.float32)
        for s, L in enumerate(lens):
            for src, dst in ((seqk[s], kc), (seqv[s], vc)):
                seq = np.full((mb * bs, Hkv, D), np.nan, np.float32)
                seq[:L] = src
                dst[ids[s]] = seq.reshape(mb, bs, Hkv, D)
        outs.append(oracle.decode(q, kc, vc, ids, lens, 0.4, lib=lib))
    np.testing.assert_array_equal(outs[0], outs[1])
    np.testing.assert_array_equal(outs[0], outs[2])


def pin_one_hot(lib):
    st, h = small_case(91, [64, 50], 2, 2, 16, 16, "f32")
    kc = h["key_cache"].copy()
    for s, pos in ((0, 37), (1, 5)):
        b, off = st.block_tables_pre[s, pos // 16], pos % 16
        kc[b, off, :, :] = h["query"][s]  # the key at `pos` equals the query: by far the largest logit
    out = oracle.decode(h["query"], kc, h["value_cache"], st.block_tables_pre, st.context_lens, 1e3, lib=lib)
    for s, pos in ((0, 37), (1, 5)):
        b, off = st.block_tables_pre[s, pos // 16], pos % 16
        np.testing.assert_allclose(out[s], h["value_cache"][b, off].astype(np.float64), rtol=0, atol=1e-12)


def pin_cache_write(lib):
    st, h = small_case(101, [5, 17, 32, 1], 4, 2, 8, 16, "bf16", include_new_token=False)
    kc, vc = h["key_cache"].copy(), h["value_cache"].copy()
    oracle.reshape_and_cache(kc, vc, h["new_key"], h["new_value"], st.slot_mapping, lib=lib)
    # the slot as a flat row index of the [NB * bs] view, independent of the oracle's block/offset split
    flat_k = kc.reshape(-1, *kc.shape[2:])
    flat_v = vc.reshape(-1, *vc.shape[2:])
    np.testing.assert_array_equal(flat_k[st.slot_mapping], h["new_key"])
    np.testing.assert_array_equal(flat_v[st.slot_mapping], h["new_value"])
    untouched = np.ones(flat_k.shape[0], bool)
    untouched[st.slot_mapping] = False
    np.testing.assert_array_equal(flat_k[untouched], h["key_cache"].reshape(flat_k.shape)[untouched])
    np.testing.assert_array_equal(flat_v[untouched], h["value_cache"].reshape(flat_v.shape)[untouched])
    # read back through the inverse-map route: position L-1 of every sequence is the new token
    for s in range(st.num_seqs):
        L = int(st.context_lens[s])
        k, v = brute.dense_kv(kc, vc, st.block_tables[s], L)
        np.testing.assert_array_equal(k[L - 1], f64(h["new_key"][s]))
        np.testing.assert_array_equal(v[L - 1], f64(h["new_value"][s]))


def pin_copy_on_write(lib):
    st, h = small_case(111, [70, 66, 90], 4, 2, 8, 16, "bf16", shared_prefix_blocks=4, cow_seqs=2)
    kc, vc = h["key_cache"].copy(), h["value_cache"].copy()
    oracle.copy_blocks(kc, vc, st.copy_pairs, lib=lib)
    for src, dst in st.copy_pairs:
        np.testing.assert_array_equal(kc[dst], h["key_cache"][src])
        np.testing.assert_array_equal(vc[dst], h["value_cache"][src])
    others = np.setdiff1d(np.arange(st.num_blocks), st.copy_pairs[:, 1])
    np.testing.assert_array_equal(kc[others], h["key_cache"][others])
    np.testing.assert_array_equal(vc[others], h["value_cache"][others])
    before = oracle.decode(h["query"], h["key_cache"], h["value_cache"], st.block_tables_pre, st.context_lens,
                           st.scale, lib=lib)
    after = oracle.decode(h["query"], kc, vc, st.block_tables, st.context_lens, st.scale, lib=lib)
    np.testing.assert_array_equal(after, before)


def pin_gather(lib):
    st, h = small_case(121, [17, 3, 40], 2, 2, 8, 16, "bf16")
    g = oracle.gather(h["key_cache"], st.block_tables_pre, st.context_lens, lib=lib)
    r = 0
    for s in range(st.num_seqs):
        L = int(st.context_lens[s])
        k, _ = brute.dense_kv(h["key_cache"], h["value_cache"], st.block_tables_pre[s], L)
        np.testing.assert_array_equal(f64(g[r:r + L]), k)
        r += L
    assert r == g.shape[0]


def _log_sum_exp_scores(h, st, s, hh, t0, t1):
    """log of sum_t exp(scale * q . k_t) over positions t0..t1-1 of sequence s, head hh (numpy, fp64)."""
    g = hh // (st.num_q_heads // st.num_kv_heads)
    q = f64(h["query"][s, hh])
    ks = []
    for t in range(t0, t1):
        b = st.block_tables_pre[s, t // st.block_size]
        ks.append(f64(h["key_cache"][b, t % st.block_size, g]))
    z = st.scale * (np.array(ks) @ q)
    zmax = z.max()
    return zmax + math.log(np.exp(z - zmax).sum())


def pin_split_merge(lib):
    # Cutting a context into partitions and merging the partitions' normalised outputs o_p with weights
    # w_p = exp(lse_p), lse_p = log sum_{t in p} exp(z_t), is exact in real arithmetic. The partition outputs
    # come from the oracle itself over block-aligned sub-contexts (the table shifted by t0 / block_size); the
    # weights from an independent numpy sum of the same scores.
    st, h = small_case(31, [70, 16, 33, 1], 4, 2, 8, 4, "bf16", scale=0.4)
    full = oracle.decode(h["query"], h["key_cache"], h["value_cache"], st.block_tables_pre, st.context_lens,
                         st.scale, lib=lib)
    for part in (4, 8, 32):
        for s, L in enumerate(st.context_lens):
            L = int(L)
            bounds = [(t0, min(L, t0 + part)) for t0 in range(0, L, part)]
            for hh in range(st.num_q_heads):
                outs, lses = [], []
                for t0, t1 in bounds:
                    tbl = np.zeros((1, st.max_blocks_per_seq), np.int32)
                    shifted = st.block_tables_pre[s, t0 // st.block_size:]
                    tbl[0, : shifted.size] = shifted
                    o = oracle.decode(h["query"][s:s + 1], h["key_cache"], h["value_cache"], tbl,
                                      np.array([t1 - t0], np.int32), st.scale, rows=np.array([[0, hh]]), lib=lib)
                    outs.append(o[0, hh])
                    lses.append(_log_sum_exp_scores(h, st, s, hh, t0, t1))
                lse = np.array(lses)
                w = np.exp(lse - lse.max())
                merged = (w[:, None] * np.array(outs)).sum(0) / w.sum()
                np.testing.assert_allclose(merged, full[s, hh], rtol=0, atol=1e-12,
                                           err_msg=f"partition {part}, seq {s}, head {hh}")


PINS = [pin_golden_decode, pin_golden_cache_ops, pin_brute_force, pin_paged_equals_contiguous,
        pin_permutation_invariance, pin_shared_equals_copied, pin_single_token, pin_identical_keys_and_positions,
        pin_gqa_replication, pin_block_size_invariance, pin_one_hot, pin_cache_write, pin_copy_on_write,
        pin_gather, pin_split_merge]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.load())


def test_brute_force_matches_golden():
    for c in _golden_cases():
        if c["kind"] != "decode":
            continue
        q, kc, vc, bt, cl, scale = _golden_decode_inputs(c)
        np.testing.assert_allclose(brute.decode(q, kc, vc, bt, cl, scale), np.array(c["expected"]), rtol=0,
                                   atol=4e-15, err_msg=c["name"])


def test_rejects_bad_live_table_entry_but_ignores_padding():
    st, h = small_case(131, [17, 3], 2, 2, 8, 16, "f32")
    bt = st.block_tables_pre.copy()
    bt[1, 1:] = 10**6  # padding beyond ceil(3 / 16) = 1 live block: never read
    oracle.decode(h["query"], h["key_cache"], h["value_cache"], bt, st.context_lens, 1.0)
    bt[0, 1] = st.num_blocks  # live entry out of the pool
    with pytest.raises(ValueError):
        oracle.decode(h["query"], h["key_cache"], h["value_cache"], bt, st.context_lens, 1.0)


# ----------------------------------------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail

MUTANTS = {
    "dropped_scale": ("z[t] = scale * acc;", "z[t] = acc;"),
    "wrong_kv_head": ("const int32_t g = h / G;", "const int32_t g = h % num_kv_heads;"),
    "offset_off_by_one": ("const int64_t off = t % block_size;", "const int64_t off = (t + 1) % block_size;"),
    "k_v_swapped": ("k[t * head_dim + d] = k_scale * elem(key_cache", "k[t * head_dim + d] = k_scale * elem(value_cache"),
    "bf16_misdecoded": ("<< 16;", "<< 15;"),
    "no_normalisation": ("o[d] /= sum;", "o[d] /= 1.0;"),
    "table_row_stride": ("block_tables[(int64_t)s * max_blocks_per_seq + t / block_size]",
                         "block_tables[(int64_t)s + t / block_size]"),
    "cache_write_offset": ("const int64_t off = slot % block_size;", "const int64_t off = 0;"),
    "copy_direction": ("memmove((char *)key_cache + dst * block_bytes, (const char *)key_cache + src * block_bytes",
                       "memmove((char *)key_cache + src * block_bytes, (const char *)key_cache + dst * block_bytes"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name, tmp_path):
    old, new = MUTANTS[name]
    with open(oracle._SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    so = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", so, str(mutated), "-lm"], check=True)
    lib = oracle.load(so)
    caught = []
    for pin in PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
