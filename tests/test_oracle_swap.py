"""Pins for the oracle's block swap between two pools (page 1 section 5: swap space on the host; page 2
section 7.2: inactive blocks moved to host memory): whole blocks copied from one pool to another, checked
against numpy indexing and by a round trip that must restore a sequence's blocks exactly."""

from __future__ import annotations

import subprocess

import numpy as np
import pytest

import oracle


def pools(rng, nb, bs, hkv, d, dtype):
    if dtype == np.uint16:
        k = rng.integers(0, 1 << 16, size=(nb, bs, hkv, d)).astype(np.uint16)
        v = rng.integers(0, 1 << 16, size=(nb, bs, hkv, d)).astype(np.uint16)
    else:
        k = rng.standard_normal((nb, bs, hkv, d)).astype(dtype)
        v = rng.standard_normal((nb, bs, hkv, d)).astype(dtype)
    return k, v


def pin_numpy_indexing(lib):
    rng = np.random.default_rng(71)
    for dtype, (nd, ns) in ((np.float32, (20, 12)), (np.uint16, (9, 30))):
        dk, dv = pools(rng, nd, 4, 2, 8, dtype)
        sk, sv = pools(rng, ns, 4, 2, 8, dtype)
        n = 7
        pairs = np.stack([rng.choice(ns, n, replace=False), rng.choice(nd, n, replace=False)], 1).astype(np.int32)
        want_k, want_v = dk.copy(), dv.copy()
        want_k[pairs[:, 1]] = sk[pairs[:, 0]]
        want_v[pairs[:, 1]] = sv[pairs[:, 0]]
        oracle.swap_blocks(dk, dv, sk, sv, pairs, lib=lib)
        assert np.array_equal(dk, want_k) and np.array_equal(dv, want_v)


def pin_round_trip(lib):
    # a sequence's blocks go out to a host pool and come back into other device blocks: its logical K/V, read
    # through the rewritten table row, are unchanged, and the host pool holds exactly what left
    rng = np.random.default_rng(72)
    dk, dv = pools(rng, 16, 4, 2, 8, np.uint16)
    hk, hv = np.zeros((6, 4, 2, 8), np.uint16), np.zeros((6, 4, 2, 8), np.uint16)
    table = np.array([3, 11, 7, 0], np.int32)
    before_k, before_v = dk[table].copy(), dv[table].copy()
    host_ids = np.array([5, 1, 2, 4], np.int32)
    oracle.swap_blocks(hk, hv, dk, dv, np.stack([table, host_ids], 1), lib=lib)
    assert np.array_equal(hk[host_ids], before_k) and np.array_equal(hv[host_ids], before_v)
    dk[table] = 0  # the device blocks are reused meanwhile
    dv[table] = 0
    new_table = np.array([9, 2, 14, 6], np.int32)
    oracle.swap_blocks(dk, dv, hk, hv, np.stack([host_ids, new_table], 1), lib=lib)
    assert np.array_equal(dk[new_table], before_k) and np.array_equal(dv[new_table], before_v)
    with pytest.raises(ValueError):
        oracle.swap_blocks(dk, dv, hk, hv, np.array([[6, 0]], np.int32), lib=lib)  # source block outside its pool


PINS = [pin_numpy_indexing, pin_round_trip]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.load())


MUTANTS = {
    # (mutants stay inside the pools: the test process must not read out of bounds)
    "source_block_off_by_one": ("memcpy((char *)dst_key + dst * block_bytes, (const char *)src_key + src * block_bytes,",
                                "memcpy((char *)dst_key + dst * block_bytes, (const char *)src_key + (src > 0 ? src - 1 : 1) * block_bytes,"),
    "value_from_key_pool": ("memcpy((char *)dst_value + dst * block_bytes, (const char *)src_value + src * block_bytes,",
                            "memcpy((char *)dst_value + dst * block_bytes, (const char *)src_key + src * block_bytes,"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_swap_pins_catch_planted_mistakes(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found once"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    so = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", so, str(mutated), "-lm"], check=True)
    lib = oracle.load(so)
    caught = []
    for pin in PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no swap pin catches the planted mistake {name}"
