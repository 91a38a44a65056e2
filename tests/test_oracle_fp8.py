"""Pins for the oracle's FP8 (OCP E4M3) KV cache: values fixed by the format and by an independent library.

The format (OCP 8-bit floating point, E4M3): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no
infinities, NaN = exponent 15 with mantissa 7, largest finite value 448. torch's float8_e4m3fn type is an
independent implementation of it. The cache write quantises x / scale (fp32 division) with saturation to
+-448 and round-to-nearest-even, NaN to 0x7F (a reading: the pages fix no quantisation rule; page 1 section
4.1 and page 3 section 2.3 only name FP8 among the quantised formats). Dequantised K and V are code value x
scale.
"""

from __future__ import annotations

import subprocess

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from tests._host import small_case


def torch_values():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def same(a, b):
    return np.array_equal(np.nan_to_num(a, nan=12345.0), np.nan_to_num(b, nan=12345.0)) and np.array_equal(
        np.isnan(a), np.isnan(b))


def pin_values(lib):
    v = oracle.e4m3_values(lib=lib)
    assert same(v, torch_values()), "code values differ from torch.float8_e4m3fn"
    assert same(v, brute.to_f64(np.arange(256, dtype=np.uint8))), "code values differ from the bit construction"
    assert v[0x7E] == 448.0 and v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9 and np.isnan(v[0xFF])


def pin_quantize(lib):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * rng.choice([1e-4, 1e-2, 1.0, 30.0, 500.0], 20000)).astype(np.float32)
    for scale in (1.0, 0.0125, 3.0):
        ours = oracle.quantize_e4m3(x, scale, lib=lib)
        ref = (torch.from_numpy(x) / torch.tensor(scale, dtype=torch.float32)).clamp(-448, 448)
        ref = ref.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(ours, ref), f"scale {scale}: {np.sum(ours != ref)} codes differ from torch"
    # every finite code round-trips; every midpoint between neighbouring codes goes to the even mantissa
    v = oracle.e4m3_values(lib=lib)
    codes = np.array([c for c in range(256) if not np.isnan(v[c])], np.uint8)
    assert np.array_equal(oracle.quantize_e4m3(v[codes].astype(np.float32), 1.0, lib=lib), codes)
    pos = np.arange(0, 0x7E + 1)
    mid = ((v[pos[:-1]] + v[pos[1:]]) / 2).astype(np.float32)  # exact in fp32
    got = oracle.quantize_e4m3(mid, 1.0, lib=lib)
    want = np.where(pos[:-1] % 2 == 0, pos[:-1], pos[1:])
    assert np.array_equal(got, want.astype(np.uint8)), "ties do not go to the even mantissa"
    special = np.array([np.nan, np.inf, -np.inf, 1e9, -1e9, 464.0, -0.0], np.float32)
    assert oracle.quantize_e4m3(special, 1.0, lib=lib).tolist() == [0x7F, 0x7E, 0xFE, 0x7E, 0xFE, 0x7E, 0x80]
    # bf16 input quantises as its float32 value
    b = torch.from_numpy(x[:1000]).to(torch.bfloat16)
    bits = b.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.quantize_e4m3(bits, 0.5, lib=lib),
                          oracle.quantize_e4m3(b.to(torch.float32).numpy(), 0.5, lib=lib))


def fp8_case(seed, lens, hq, hkv, d, bs):
    st, h = small_case(seed, lens, hq, hkv, d, bs, "f32", include_new_token=True)
    rng = np.random.default_rng(seed)
    kc = rng.integers(0, 256, size=h["key_cache"].shape).astype(np.uint8)
    vc = rng.integers(0, 256, size=h["value_cache"].shape).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x3C  # keep the live codes finite
    vc[(vc & 0x7F) == 0x7F] = 0x44
    return st, h["query"], kc, vc


def pin_fp8_attention(lib):
    for seed, lens, hq, hkv, d, bs in ((41, [5, 17, 33], 4, 2, 16, 4), (42, [1, 40, 9], 6, 3, 8, 16)):
        st, q, kc, vc = fp8_case(seed, lens, hq, hkv, d, bs)
        for ks, vs in ((1.0, 1.0), (0.0125, 0.03), (2.0 ** -5, 0.25)):
            a = oracle.decode(q, kc, vc, st.block_tables_pre, st.context_lens, st.scale, k_scale=ks, v_scale=vs,
                              lib=lib)
            b = brute.decode(q, kc, vc, st.block_tables_pre, st.context_lens, st.scale, ks, vs)
            np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
        # with power-of-two scales the fp8 cache equals a float32 cache holding value x scale, exactly
        vals = oracle.e4m3_values(lib=lib)
        kf = (vals[kc] * 2.0 ** -5).astype(np.float32)
        vf = (vals[vc] * 0.25).astype(np.float32)
        a = oracle.decode(q, kc, vc, st.block_tables_pre, st.context_lens, st.scale, k_scale=2.0 ** -5,
                          v_scale=0.25, lib=lib)
        c = oracle.decode(q, kf, vf, st.block_tables_pre, st.context_lens, st.scale, lib=lib)
        np.testing.assert_allclose(a, c, rtol=0, atol=1e-12)
        # k_scale only rescales the logits, v_scale only the output
        d1 = oracle.decode(q, kc, vc, st.block_tables_pre, st.context_lens, st.scale * 0.7, k_scale=1.0,
                           v_scale=3.0, lib=lib)
        d2 = oracle.decode(q, kc, vc, st.block_tables_pre, st.context_lens, st.scale, k_scale=0.7, v_scale=1.0,
                           lib=lib)
        np.testing.assert_allclose(d1, 3.0 * d2, rtol=1e-12, atol=1e-12)


def pin_fp8_cache_write(lib):
    st, h = small_case(43, [5, 17, 32, 1], 4, 2, 8, 16, "bf16", include_new_token=False)
    NB, bs, hkv, d = h["key_cache"].shape
    kc = np.full((NB, bs, hkv, d), 0x7F, np.uint8)
    vc = kc.copy()
    oracle.reshape_and_cache_e4m3(kc, vc, h["new_key"], h["new_value"], st.slot_mapping, 0.05, 0.02, lib=lib)
    # placement by flat row index, values by the quantiser
    want_k = np.full((NB * bs, hkv, d), 0x7F, np.uint8)
    want_v = want_k.copy()
    want_k[st.slot_mapping] = oracle.quantize_e4m3(h["new_key"], 0.05, lib=lib)
    want_v[st.slot_mapping] = oracle.quantize_e4m3(h["new_value"], 0.02, lib=lib)
    assert np.array_equal(kc.reshape(-1, hkv, d), want_k) and np.array_equal(vc.reshape(-1, hkv, d), want_v)


PINS = [pin_values, pin_quantize, pin_fp8_attention, pin_fp8_cache_write]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.load())


MUTANTS = {
    "subnormal_scale": ("return sign * ldexp((double)m, -9);", "return sign * ldexp((double)m, -10);"),
    "exponent_bias": ("return sign * ldexp(1.0 + m / 8.0, e - 7);", "return sign * ldexp(1.0 + m / 8.0, e - 8);"),
    "truncating_quantiser": ("double q = nearbyint(ldexp(a, 3 - e));", "double q = floor(ldexp(a, 3 - e));"),
    "no_saturation": ("        a = 448.0;\n", "        a = a;\n"),
    "k_scale_dropped": ("k[t * head_dim + d] = k_scale * elem(key_cache",
                        "k[t * head_dim + d] = 1.0 * elem(key_cache"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_fp8_pins_catch_planted_mistakes(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle._SRC).read()
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
    assert caught, f"no FP8 pin catches the planted mistake {name}"
