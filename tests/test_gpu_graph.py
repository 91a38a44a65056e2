"""Decode steps captured into a HIP graph and replayed.

The library allocates nothing, clears nothing with memsets and never synchronises, so a whole decode step --
the slot-mapped write of the new token's K/V, then paged attention with its merge kernel -- can be captured
once (torch.cuda.graph) and replayed; so can the call that does both, paged_attention_decode_append. Each replay
starts from the pristine pools and a NaN-filled output, with eager work and host synchronisations between
replays, and must reproduce the eager step bit for bit: output and both pools.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_458_amd as pa
from workloads import custom_structure, materialize

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


def i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


CASES = [
    # (Hq, Hkv, partition_size, cache dtype, what runs)
    (8, 8, -1, "bf16", "single-head balanced split + merge"),
    (8, 8, 0, "bf16", "single-head single pass"),
    (32, 8, 512, "bf16", "matrix-core partitions, two per wave, + log-sum-exp merge"),
    (32, 8, pa.PA_PARTITION_BALANCED, "bf16", "matrix-core balanced split + merge"),
    (8, 8, -1, "fp8", "E4M3: quantising cache write, balanced split with two heads per wave + merge"),
    (8, 8, -1, "bf16+append", "one call: new rows written by the balanced split's launch + merge"),
    (32, 8, 512, "bf16+append", "one call: new rows written by the matrix-core partition kernel + merge"),
    (32, 8, pa.PA_PARTITION_BALANCED, "fp8+append",
     "one call, E4M3: new rows quantised by the matrix-core balanced split + merge"),
]


@pytest.mark.parametrize("hq,hkv,part,dt,what", CASES, ids=[c[4] for c in CASES])
def test_captured_decode_step_replays_bit_for_bit(hq, hkv, part, dt, what):
    append = dt.endswith("+append")
    dt = dt.split("+")[0]
    st = custom_structure("graph", 461, [700, 1500, 33, 2048, 1, 900], hq, hkv, 128, 16, dt)
    t = materialize(st, DEV, include_new_token=False)
    kc, vc = t["key_cache"], t["value_cache"]
    kc0, vc0 = kc.clone(), vc.clone()
    tables, lens, slots = i32(st.block_tables_pre), i32(st.context_lens), i32(st.slot_mapping)
    kd = pa.PA_FP8_E4M3 if dt == "fp8" else pa.PA_BF16
    need = pa.workspace_bytes(st.num_seqs, hq, hkv, st.head_dim, st.max_context_len, st.block_size, kd, part)
    assert (need > 0) == (part != 0)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    out = torch.empty((st.num_seqs, hq, st.head_dim), dtype=torch.float32, device=DEV)

    def step():
        if append:
            pa.paged_attention_decode_append(out, t["query"], t["new_key"], t["new_value"], kc, vc, tables, lens,
                                             slots, st.scale, max_context_len=st.max_context_len,
                                             partition_size=part, workspace=ws, k_scale=st.k_scale,
                                             v_scale=st.v_scale)
            return
        pa.reshape_and_cache(t["new_key"], t["new_value"], kc, vc, slots, k_scale=st.k_scale, v_scale=st.v_scale)
        pa.paged_attention_decode(out, t["query"], kc, vc, tables, lens, st.scale, st.block_size,
                                  max_context_len=st.max_context_len, partition_size=part, workspace=ws,
                                  k_scale=st.k_scale, v_scale=st.v_scale)

    step()
    torch.cuda.synchronize()
    want_out, want_k, want_v = out.clone(), kc.clone(), vc.clone()
    assert torch.isfinite(want_out).all()

    g = torch.cuda.CUDAGraph()
    kc.copy_(kc0)
    vc.copy_(vc0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        kc.copy_(kc0)
        vc.copy_(vc0)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), want_out.view(torch.int32)), f"{what}: replay {rep} output"
        assert torch.equal(kc.view(torch.uint8), want_k.view(torch.uint8)), f"{what}: replay {rep} key pool"
        assert torch.equal(vc.view(torch.uint8), want_v.view(torch.uint8)), f"{what}: replay {rep} value pool"
