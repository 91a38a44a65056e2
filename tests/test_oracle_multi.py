"""Pins for the oracle's several-new-tokens attention (speculative verification, page 1 section 6; a prompt
chunk): sequence s's QL newest tokens attend causally -- token j at position L - QL + j over positions
0 .. L - QL + j -- through the same block table (page 1 section 3.2).

The pins fix the oracle against what does not depend on it: the numpy pool-scanning route, torch's fp64
scaled_dot_product_attention with an explicit bottom-right causal mask over K/V gathered by numpy indexing
(and its own is_causal mask when the whole sequence is the query), and plain decode when QL = 1.
"""

from __future__ import annotations

import subprocess

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from tests._host import f64, to_host
from workloads import custom_structure, materialize, query_rows


def multi_case(seed, lens, qls, hq, hkv, d, bs, dtype):
    st = custom_structure(f"multi{seed}", seed, lens, hq, hkv, d, bs, dtype, pool_factor=1.5)
    t = materialize(st, "cpu")
    q, qs = query_rows(st, qls)
    h = {k: to_host(v) for k, v in t.items()}
    return st, to_host(q), qs, h


CASES = [
    # (seed, lens, query lens, Hq, Hkv, D, bs, dtype)
    (61, [9, 17, 4, 33], [3, 1, 4, 0], 4, 2, 8, 4, "f32"),
    (62, [5, 40, 16], [5, 7, 2], 4, 4, 16, 16, "bf16"),  # QL = L for the first sequence
    (63, [3, 21, 30], [5, 8, 1], 6, 3, 8, 1, "bf16"),  # QL > L: the first two rows of sequence 0 are zero
    (64, [12, 0, 26], [2, 0, 6], 8, 2, 8, 8, "fp8"),
]


def pin_against_brute(lib):
    for seed, lens, qls, hq, hkv, d, bs, dt in CASES:
        st, q, qs, h = multi_case(seed, lens, qls, hq, hkv, d, bs, dt)
        a = oracle.decode_multi(q, h["key_cache"], h["value_cache"], st.block_tables_pre, st.context_lens, qs,
                                st.scale, k_scale=st.k_scale, v_scale=st.v_scale, lib=lib)
        b = brute.decode_multi(q, h["key_cache"], h["value_cache"], st.block_tables_pre, st.context_lens, qs,
                               st.scale, st.k_scale, st.v_scale)
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12, err_msg=f"seed {seed}")
        if seed == 63:
            assert (a[0] == 0).all() and (a[1] == 0).all() and np.abs(a[2]).max() > 0


def _dense_by_indexing(cache, table_row, L, scale_factor):
    """[L, Hkv, D] fp64 rows of one sequence gathered with numpy fancy indexing of the flattened pool."""
    NB, bs, Hkv, D = cache.shape
    pos = np.arange(L)
    slots = np.asarray(table_row)[pos // bs].astype(np.int64) * bs + pos % bs
    return brute.to_f64(cache.reshape(NB * bs, Hkv, D)[slots]) * scale_factor


def pin_against_sdpa(lib):
    for seed, lens, qls, hq, hkv, d, bs, dt in CASES[:2] + [(65, [24, 13, 50], [24, 3, 9], 8, 4, 16, 8, "bf16")]:
        st, q, qs, h = multi_case(seed, lens, qls, hq, hkv, d, bs, dt)
        a = oracle.decode_multi(q, h["key_cache"], h["value_cache"], st.block_tables_pre, st.context_lens, qs,
                                st.scale, k_scale=st.k_scale, v_scale=st.v_scale, lib=lib)
        qf = f64(q)
        G = hq // hkv
        for s, L in enumerate(st.context_lens):
            L = int(L)
            QL = int(qs[s + 1] - qs[s])
            if QL == 0 or L == 0:
                continue
            k = _dense_by_indexing(h["key_cache"], st.block_tables_pre[s], L, st.k_scale)
            v = _dense_by_indexing(h["value_cache"], st.block_tables_pre[s], L, st.v_scale)
            kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, dim=0)  # [Hq, L, D]
            vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, dim=0)
            qt = torch.from_numpy(qf[qs[s]:qs[s + 1]]).permute(1, 0, 2)  # [Hq, QL, D]
            if QL == L:
                ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=st.scale)
            else:
                mask = torch.arange(L)[None, :] <= (L - QL + torch.arange(QL))[:, None]
                ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=st.scale)
            np.testing.assert_allclose(a[qs[s]:qs[s + 1]], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12,
                                       err_msg=f"seed {seed} sequence {s}")


def pin_one_token_is_decode(lib):
    st, q, qs, h = multi_case(66, [7, 33, 1, 20], [1, 1, 1, 1], 4, 2, 16, 4, "bf16")
    a = oracle.decode_multi(q, h["key_cache"], h["value_cache"], st.block_tables_pre, st.context_lens, qs,
                            st.scale, lib=lib)
    b = brute.decode(q, h["key_cache"], h["value_cache"], st.block_tables_pre, st.context_lens, st.scale)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def pin_sampled_rows(lib):
    seed, lens, qls, hq, hkv, d, bs, dt = CASES[0]
    st, q, qs, h = multi_case(seed, lens, qls, hq, hkv, d, bs, dt)
    full = oracle.decode_multi(q, h["key_cache"], h["value_cache"], st.block_tables_pre, st.context_lens, qs,
                               st.scale, lib=lib)
    rows = np.array([[0, 1], [4, 3], [7, 0], [4, 3], [0, 1], [4, 3]], np.int32)  # repeated rows are computed once
    part = oracle.decode_multi(q, h["key_cache"], h["value_cache"], st.block_tables_pre, st.context_lens, qs,
                               st.scale, rows=rows, lib=lib)
    for t, hh in rows:
        np.testing.assert_array_equal(part[t, hh], full[t, hh])
    assert np.isnan(part[1, 0]).all()
    with pytest.raises(ValueError):
        oracle.decode_multi(q, h["key_cache"], h["value_cache"], st.block_tables_pre, st.context_lens,
                            qs[::-1].copy(), st.scale, lib=lib)


def pin_golden_multi(lib):
    # hand-computed closed forms (tests/golden/hand_examples.json, kind "multi")
    from tests.test_oracle_pins import _golden_cases, _golden_decode_inputs

    n = 0
    for c in _golden_cases():
        if c["kind"] != "multi":
            continue
        q, kc, vc, bt, cl, scale = _golden_decode_inputs(c)
        out = oracle.decode_multi(q, kc, vc, bt, cl, np.array(c["query_start"], np.int32), scale, lib=lib)
        np.testing.assert_allclose(out, np.array(c["expected"]), rtol=0, atol=4e-15, err_msg=c["name"])
        n += 1
    assert n > 0


PINS = [pin_against_brute, pin_against_sdpa, pin_one_token_is_decode, pin_sampled_rows, pin_golden_multi]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.load())


MUTANTS = {
    "causal_off_by_one": ("const int64_t E = (int64_t)context_lens[s] - QL + j + 1;",
                          "const int64_t E = (int64_t)context_lens[s] - QL + j;"),
    "top_left_causal": ("const int64_t E = (int64_t)context_lens[s] - QL + j + 1;", "const int64_t E = j + 1;"),
    "row_index_in_sequence": ("const int64_t j = t - query_start[s];", "const int64_t j = t;"),
    "query_row_of_sequence": ("const int rc = attend_row(o, query, q_dtype, t,",
                              "const int rc = attend_row(o, query, q_dtype, s,"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_multi_pins_catch_planted_mistakes(name, tmp_path):
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
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no multi-token pin catches the planted mistake {name}"
