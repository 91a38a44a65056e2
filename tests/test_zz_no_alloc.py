"""GPU test of paged_attention_decode_noalloc, the decode call for callers that cannot allocate: through the C ABI
it must give, bit for bit, what paged_attention_decode_scaled gives with a caller workspace (same plan, same
kernels), on consecutive calls that reuse the library's static scratch -- the second with a smaller input --
for every kind of plan that uses scratch (partitions with the log-sum-exp merge, the single-head and the
matrix-core balanced splits) and for a single pass, which uses none. (Calls that need more scratch than the
static buffer holds are refused on the host before any launch: tests/test_abi_host.py.)
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_458_amd as pa
from tests._host import to_host
from workloads import build_structure, custom_structure, materialize

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def kv_code(st):
    return {"f32": pa.PA_F32, "bf16": pa.PA_BF16, "fp8": pa.PA_FP8_E4M3}[st.dtype]


def run_both(st, t, part):
    """(no-alloc output, workspace output, launched partition) for one batch."""
    tables, lens = dev_i32(st.block_tables_pre), dev_i32(st.context_lens)
    shape = (st.num_seqs, st.num_q_heads, st.head_dim)
    a = torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
    b = torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
    pa.paged_attention_decode_noalloc(a, t["query"], t["key_cache"], t["value_cache"], tables, lens, st.scale,
                                      max_context_len=st.max_context_len, partition_size=part, k_scale=st.k_scale,
                                      v_scale=st.v_scale)
    torch.cuda.synchronize()
    got = a.cpu().numpy()
    # the existing entry point on the same inputs, with a workspace of its own
    pa.paged_attention_decode(b, t["query"], t["key_cache"], t["value_cache"], tables, lens, st.scale,
                              max_context_len=st.max_context_len, partition_size=part, k_scale=st.k_scale,
                              v_scale=st.v_scale)
    torch.cuda.synchronize()
    launched = pa.partition_size_for(st.num_seqs, st.num_q_heads, st.num_kv_heads, st.head_dim, st.max_context_len,
                                     st.block_size, kv_code(st), part)
    return got, b.cpu().numpy(), launched


# (large batch, smaller batch, partition argument): the smaller call reuses the scratch the large one filled
PAIRS = [
    ("llama2_70b_gqa", ("g", 71, [700, 45, 1300], 16, 2, 128, 16, "bf16"), 512),   # matrix cores, partitions
    ("llama2_7b", ("m", 72, [33, 900, 5, 260], 8, 8, 128, 16, "bf16"), -1),         # single-head balanced split
    ("mistral_gqa_prefix", ("p", 73, [1500, 20, 640], 32, 8, 128, 16, "bf16"), -1),  # matrix-core balanced split
    ("llama2_70b_gqa_fp8", ("e", 74, [3000, 17], 64, 8, 128, 256, "fp8"), -1),      # E4M3, matrix cores
    ("tiny_fp32", ("f", 75, [5, 40], 4, 4, 64, 16, "f32"), 16),                      # fp32 partitions
    ("llama2_7b", ("s", 76, [100, 7], 4, 4, 128, 16, "bf16"), 0),                    # single pass: no scratch
]


@pytest.mark.parametrize("big,small,part", PAIRS, ids=[p[0] + "_" + str(p[2]) for p in PAIRS])
def test_noalloc_matches_workspace_call(big, small, part):
    st_big = build_structure(big)
    t_big = materialize(st_big, DEV)
    got, ref, launched = run_both(st_big, t_big, part)
    np.testing.assert_array_equal(got, ref)
    assert np.isfinite(got).all()
    need = pa.workspace_bytes(st_big.num_seqs, st_big.num_q_heads, st_big.num_kv_heads, st_big.head_dim,
                              st_big.max_context_len, st_big.block_size, kv_code(st_big), part)
    sys.__stderr__.write(f"[{big}] partition {launched}, scratch {need} B: identical\n")
    del t_big

    name, seed, lens, hq, hkv, d, bs, dt = small
    st = custom_structure(name, seed, lens, hq, hkv, d, bs, dt)
    t = materialize(st, DEV)
    got, ref, launched_small = run_both(st, t, part)
    np.testing.assert_array_equal(got, ref)
    # and against the oracle, to the tolerance of the cache's type
    h = {k: to_host(v) for k, v in t.items()}
    exp = oracle.decode(h["query"], h["key_cache"], h["value_cache"], st.block_tables_pre, st.context_lens, st.scale,
                        k_scale=st.k_scale, v_scale=st.v_scale)
    err = np.abs(got.astype(np.float64) - exp)
    tol = 1e-5 if dt == "f32" else 2e-3 + 1e-2 * np.abs(exp)
    assert (err <= tol).all(), f"max err {err.max():.3e}"
    sys.__stderr__.write(f"[{name}] partition {launched_small}: identical, max err vs oracle {err.max():.2e}\n")
