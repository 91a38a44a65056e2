#!/usr/bin/env python3
"""Benchmark of the paged decode hot path on one MI355X.

A step is one decode step of a batch over its paged KV pool: copy-on-write block copies (the workload with a
shared prefix), the slot-mapped write of every sequence's new K/V, then paged decode attention over the whole
context (single pass, split-context partitions or the balanced split, plus the log-sum-exp reduce). Inputs are
seeded synthetic tensors already resident in HBM; consecutive steps read different replicas of the pools so
that no step can be served from the 256 MB last-level cache left warm by the previous one.

Prints one JSON line: whole-step achieved GB/s (algorithmic bytes / step time), decode queries/s, a roofline
entry for the attention call (HIP events on the stream it runs on; the bytes HBM must deliver, a block shared by
several sequences counted once) and the CPU oracle's rate on the host cores. The default (headline) run also
measures every other synthetic workload, each in a fresh child process, and reports them under "configs".

    python bench.py [--workload llama2_7b] [--steps 100] [--warmup 10] [--no-configs]
    python bench.py --workload configs    (one line per synthetic decode workload, each in a fresh process)
    python bench.py --workload decode_loop --steps 100 --warmup 50   (continuous batching, block manager)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "paged decode attention achieved HBM GB/s (% of peak) + decode queries/sec"


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# the sources that define or launch the attention kernels whose HBM traffic is counted (partition kernels, the
# log-sum-exp reduce, the launch plan); a change to any of them makes stored counter readings stale
ATTENTION_SOURCES = ("decode_valu.hip", "decode_gqa_mfma.hip", "pa_device.h", "pa_kernels.h", "pa_abi.hip")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(os.path.join(ROOT, "paged_kv_cache_458_amd", "csrc", f) for f in ATTENTION_SOURCES):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + f.read())
    return h.hexdigest()[:16]


def step_appends(query_len: int, max_context_len: int, separate_write: bool = False) -> bool:
    """Whether the benchmark's step writes the new tokens inside the decode launch: paged_attention_decode_append
    does so under every plan of a decode step, except with max_context_len 0 (where it launches the cache write
    first)."""
    return query_len == 1 and not separate_write and max_context_len >= 1


def appended_row_bytes(st) -> int:
    """The new rows a decode step reads from its input and writes to both pools (sequences with a slot)."""
    return 2 * int((st.slot_mapping >= 0).sum()) * st.num_kv_heads * st.head_dim * (st.q_esize + st.esize)


TRAFFIC_TAG = "<!-- traffic "
COPY_BYTES = 1 << 31  # bytes the calibration copy reads and writes per dispatch (stream_copy over 2 GiB)


def traffic_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.md")


def load_traffic(workload: str):
    """Counter-measured HBM bytes per attention call, if taken on the current kernel sources."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith(TRAFFIC_TAG):
                rec = json.loads(line[len(TRAFFIC_TAG):].rsplit("-->", 1)[0])
    if rec is None or rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_call")


def _counter_means(db: str, counter: str) -> dict:
    """Mean value of `counter` per dispatch, by kernel name, from a rocprofv3 database."""
    import sqlite3

    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, dispatch_id, sum(value) from counters_collection where counter_name = ? "
                       "group by kernel_name, dispatch_id", (counter,)).fetchall()
    con.close()
    acc = {}
    for name, _, v in rows:
        acc.setdefault(name, []).append(float(v))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def write_traffic_summary(workload: str, fetch_db: str, write_db: str, cmd_fetch: str, cmd_write: str,
                          query_len: int = 1) -> str:
    """Turn the FETCH_SIZE and WRITE_SIZE runs of this benchmark into bytes per attention call.

    Each counter is scaled by what it reads for the streaming copy kernel, whose traffic is known exactly
    (COPY_BYTES read and COPY_BYTES written per dispatch). The attention call is the decode kernel (partition
    or balanced split) plus, when the context is split, its log-sum-exp merge kernel: their per-dispatch means
    are added.
    """
    fetch, write = _counter_means(fetch_db, "FETCH_SIZE"), _counter_means(write_db, "WRITE_SIZE")

    def pick(d, key):
        hits = [k for k in d if key in k]
        return hits[0] if hits else None

    copy_f, copy_w = pick(fetch, "stream_copy_kernel"), pick(write, "stream_copy_kernel")
    f_scale, w_scale = COPY_BYTES / fetch[copy_f][0], COPY_BYTES / write[copy_w][0]
    rows, fb, wb = [], 0.0, 0.0
    for key in ("decode_valu_kernel", "decode_valu_balanced_kernel", "decode_gqa_mfma_kernel",
                "decode_gqa_mfma_balanced_kernel", "lse_reduce_kernel", "balanced_reduce_kernel"):
        kf, kw = pick(fetch, key), pick(write, key)
        if kf is None:
            continue
        f, w = fetch[kf][0] * f_scale, write[kw][0] * w_scale
        fb, wb = fb + f, wb + w
        rows.append((kf, fetch[kf][1], fetch[kf][0], write[kw][0], f, w))
    from workloads import algorithmic_bytes, build_structure

    st = build_structure(workload)
    alg = algorithmic_bytes(st, query_len)["total"]
    if step_appends(query_len, st.max_context_len):  # the counted call also reads and writes the new rows
        alg += appended_row_bytes(st)
    label = workload if query_len == 1 else f"{workload}_q{query_len}"
    lines = [f"# HBM traffic per attention call: {label}", "",
             "Two counter runs of the benchmark (run from the repository root on one MI355X):", "", "```",
             cmd_fetch, cmd_write, "```", "",
             f"Calibration: the streaming copy kernel moves {COPY_BYTES} B each way per dispatch; it reads "
             f"FETCH_SIZE = {fetch[copy_f][0]:.0f} and WRITE_SIZE = {write[copy_w][0]:.0f} per dispatch, so the "
             f"scale factors are {f_scale:.3f} B per FETCH_SIZE unit and {w_scale:.3f} B per WRITE_SIZE unit.", "",
             "| kernel | dispatches | FETCH_SIZE | WRITE_SIZE | fetched B | written B |", "|---|---|---|---|---|---|"]
    for k, n, f0, w0, f, w in rows:
        lines.append(f"| `{k[:90]}` | {n} | {f0:.0f} | {w0:.0f} | {f:.4g} | {w:.4g} |")
    lines += ["", f"Per call: {fb + wb:.4g} B of HBM traffic against {alg} algorithmic bytes "
                  f"(ratio {(fb + wb) / alg:.3f}).", "",
              TRAFFIC_TAG + json.dumps({"kernel_source_hash": kernel_source_hash(), "fetch_bytes_per_call": round(fb),
                                        "write_bytes_per_call": round(wb), "bytes_per_call": round(fb + wb),
                                        "algorithmic_bytes": alg}) + " -->"]
    path = traffic_path(label)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def unique_slots(tables, lens, bs: int) -> int:
    """Distinct pool slots that one decode call reads: a physical block referenced by several sequences counts
    once, with the most rows any of them uses in it."""
    import numpy as np

    lens = np.asarray(lens, dtype=np.int64)
    nblk = (lens + bs - 1) // bs
    seq = np.repeat(np.arange(len(lens)), nblk)
    j = np.arange(int(nblk.sum())) - np.repeat(np.cumsum(nblk) - nblk, nblk)  # logical block within its sequence
    ids = np.asarray(tables)[seq, j].astype(np.int64)
    rows = np.minimum(bs, lens[seq] - j * bs)
    most = {}
    for b, r in zip(ids.tolist(), rows.tolist()):
        if r > most.get(b, 0):
            most[b] = r
    return int(sum(most.values()))


def run_decode_loop(args) -> int:
    """Continuous-batching decode over a request stream: the block manager places every token, the kernels
    move and read them. Llama-2-7B-shaped attention (32 heads x 128, bf16, 16-token blocks), up to 256
    sequences, prompts of the mixed-length workload (30% of the long ones open with a shared 1024-token
    system prompt), 32..256 new tokens each, 5% of requests sampled twice (a fork). Finished sequences free
    their blocks and are replaced at once. A step is one decode step of every running sequence, host
    bookkeeping included; the timed steps run after the batch has filled."""
    import numpy as np
    import torch

    import paged_kv_cache_458_amd as pa
    from paged_kv_cache_458_amd.block_manager import PA_ERR_NOMEM
    from paged_kv_cache_458_amd.decode_loop import DecodeLoop
    from workloads import request_stream

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pa.load_library()
    max_batch, hq, hkv, d, bs, max_len = 256, 32, 32, 128, 16, 4096 + 256
    num_blocks = 40000  # about 1.6x what 256 sequences of the mix hold on average; plus the padding block
    loop = DecodeLoop(num_blocks=num_blocks, block_size=bs, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                      max_blocks_per_seq=-(-max_len // bs), dtype="bf16", seed=6, prompt_kv="random",
                      partition_size=-1 if args.partition_size is None else args.partition_size)
    stream = request_stream(6)
    remaining: dict[int, int] = {}
    pending = []
    next_id = 0
    admitted = finished = deferred = 0

    def refill():
        nonlocal next_id, admitted, deferred
        while len(loop.running) < max_batch:
            req = pending.pop() if pending else next(stream)
            try:
                loop.add_sequence(next_id, req.prompt)
            except pa.PagedAttentionError as e:
                if e.status != PA_ERR_NOMEM:
                    raise
                pending.append(req)
                deferred += 1
                return
            remaining[next_id] = req.max_new_tokens
            next_id += 1
            admitted += 1
            if req.parallel > 1 and len(loop.running) < max_batch:
                loop.fork(next_id - 1, next_id)
                remaining[next_id] = req.max_new_tokens
                next_id += 1

    def step():
        nonlocal finished
        refill()
        ids, _, _ = loop.step()
        for s in ids:
            remaining[s] -= 1
            if remaining[s] == 0:
                loop.finish(s)
                del remaining[s]
                finished += 1

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize(dev)
    loop.attention_events = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    events = loop.attention_events
    loop.attention_events = None
    stats = []  # occupancy, sampled over further steps outside the timed region
    for _ in range(min(args.steps, 20)):
        step()
        stats.append(loop.stats())
    row = hkv * d * 2
    attn_s, attn_bytes, unique_bytes, stepped = 0.0, 0, 0, 0
    for (e0, e1), lens, tables in events:
        attn_s += e0.elapsed_time(e1) * 1e-3
        lens = lens.astype(np.int64)
        nb = int(((lens + bs - 1) // bs).sum())
        # query in, fp32 out, live table entries, lengths; the new rows read from the input and written to the
        # pools by the same call
        other = len(lens) * hq * d * (2 + 4) + nb * 4 + 4 * len(lens) + 2 * row * len(lens)
        attn_bytes += int(lens.sum()) * row * 2 + other
        unique_bytes += unique_slots(tables, lens, bs) * row * 2 + other
        stepped += len(lens)
    frag = float(np.mean([s["internal_fragmentation"] for s in stats]))
    contiguous_slots = float(np.mean([s["sequences"] for s in stats])) * max_len
    rec = {
        "metric": METRIC,
        "value": round(attn_bytes / wall / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "accumulate": "f32",
        "data": "synthetic",
        "config": {"workload": "decode_loop", "max_batch": max_batch, "num_q_heads": hq, "num_kv_heads": hkv,
                   "head_dim": d, "block_size": bs, "pool_blocks": num_blocks, "seed": 6},
        "decode_queries_per_s": round(stepped / wall, 1),
        "attention": {"us_mean": round(attn_s / len(events) * 1e6, 2),
                      "gb_per_s": round(attn_bytes / attn_s / 1e9, 1),
                      "gb_per_s_unique": round(unique_bytes / attn_s / 1e9, 1),
                      "share_of_step": round(attn_s / wall, 3)},
        "decode_loop": {
            "admitted": admitted, "finished": finished, "deferred_for_memory": deferred,
            "mean_running": round(stepped / len(events), 1),
            "internal_fragmentation": round(frag, 4),
            "used_slots_vs_contiguous_max_len": round(float(np.mean([s["slots_in_used_blocks"] for s in stats]))
                                                      / contiguous_slots, 4),
            "shared_blocks_mean": round(float(np.mean([s["shared_blocks"] for s in stats])), 1),
            "cow_copies": stats[-1]["cow_copies"],
        },
        # unique bytes: blocks shared by several sequences (prompt prefixes, forks) count once per call
        "roofline": {"bound": "hbm", "kernel": "paged_attention_decode_append within the loop",
                     "achieved": round(unique_bytes / attn_s / 1e9, 1),
                     "achieved_logical": round(attn_bytes / attn_s / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(unique_bytes / attn_s / 1e9 / PEAK_HBM_GBS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)
    return 0


def run_swap(args) -> int:
    """Block swap between the device pool and a pinned host pool (page 1 section 5: swap space): the 7B shape
    (32 KV heads x 128, bf16, 16-token blocks: 256 KiB of K and V per block), 2048 random blocks out to the host
    pool and 2048 back in per step. Reference: torch's DMA copy of the same bytes between pinned host memory
    and the device, and the host link's nominal 64 GB/s per direction (PCIe 5.0 x16)."""
    import numpy as np
    import torch

    import paged_kv_cache_458_amd as pa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pa.load_library()
    nb_dev, nb_host, n, bs, hkv, d = 8192, 4096, 2048, 16, 32, 128
    shape = (bs, hkv, d)
    kc = torch.randn((nb_dev,) + shape, device=dev).to(torch.bfloat16)
    vc = torch.randn((nb_dev,) + shape, device=dev).to(torch.bfloat16)
    hk = torch.empty((nb_host,) + shape, dtype=torch.bfloat16).pin_memory()
    hv = torch.empty((nb_host,) + shape, dtype=torch.bfloat16).pin_memory()
    rng = np.random.default_rng(7)
    out_pairs = torch.from_numpy(np.stack([rng.choice(nb_dev, n, replace=False), rng.choice(nb_host, n, replace=False)],
                                          1).astype(np.int32)).to(dev)
    in_pairs = torch.from_numpy(np.stack([out_pairs[:, 1].cpu().numpy(), rng.choice(nb_dev, n, replace=False)],
                                         1).astype(np.int32)).to(dev)
    moved = 2 * n * kc[0].nbytes  # K and V, one direction
    stream = torch.cuda.current_stream(dev)

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / reps

    ms_out = timed(lambda: pa.swap_blocks(hk, hv, kc, vc, out_pairs), args.steps)
    ms_in = timed(lambda: pa.swap_blocks(kc, vc, hk, hv, in_pairs), args.steps)
    flat_h = torch.empty(moved, dtype=torch.uint8).pin_memory()
    flat_d = torch.empty(moved, dtype=torch.uint8, device=dev)
    ms_dma_h2d = timed(lambda: flat_d.copy_(flat_h, non_blocking=True), args.steps)
    ms_dma_d2h = timed(lambda: flat_h.copy_(flat_d, non_blocking=True), args.steps)
    gbs = lambda ms: round(moved / (ms * 1e-3) / 1e9, 2)
    value = 2 * moved / ((ms_out + ms_in) * 1e-3) / 1e9
    rec = {
        "metric": "block swap GB/s between device pool and pinned host pool",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": 2,
        "ms_per_step": round(ms_out + ms_in, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "swap", "blocks_per_direction": n, "block_bytes_kv": 2 * kc[0].nbytes,
                   "device_pool_blocks": nb_dev, "host_pool_blocks": nb_host},
        "swap_out_gbs": gbs(ms_out),
        "swap_in_gbs": gbs(ms_in),
        "dma_copy_d2h_gbs": gbs(ms_dma_d2h),
        "dma_copy_h2d_gbs": gbs(ms_dma_h2d),
        "roofline": {"bound": "host link", "achieved": round(value, 2), "peak": 64.0, "unit": "GB/s",
                     "frac": round(value / 64.0, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)
    return 0


HEADLINE = "llama2_7b"


def config_summary(rec: dict) -> dict:
    """The per-workload figures the headline line carries for each synthetic workload."""
    att, roof = rec["attention"], rec["roofline"]
    traffic = roof.get("traffic")
    out = {
        "attention_us": {"mean": att["us_mean"], "median": att["us_median"], "min": att["us_min"]},
        "gb_per_s": att["gb_per_s"],
        "gb_per_s_unique": att["gb_per_s_unique"],
        "frac": roof["frac"],
        "traffic_over_unique": round(traffic / att["unique_bytes_per_call"], 4) if traffic else None,
        "traffic_over_logical": round(traffic / att["bytes_per_call"], 4) if traffic else None,
        "decode_queries_per_s": att["queries_per_s"],
        "step_ms": rec["ms_per_step"],
        "bytes_per_call": att["bytes_per_call"],
        "unique_bytes_per_call": att["unique_bytes_per_call"],
        "kv_cache_dtype": rec["config"]["kv_cache_dtype"],
        "partition_size": rec["config"]["partition_size"],
        "cpu_baseline": rec["cpu_baseline"],
    }
    return out


def run_config_children(args) -> dict:
    """Every synthetic workload but the headline, each measured by this script in a fresh process of its own (run
    before this process touches the GPU), summarised per workload."""
    import subprocess

    from workloads import CONFIG_NAMES

    res = {}
    # at least 100 timed steps and 200 warmup steps each: the shortest calls (about 70 us) are the noisiest, and
    # their means settle only after tens of milliseconds of work
    steps, warmup = max(args.steps, 100), max(args.warmup, 200)
    for name in CONFIG_NAMES:
        if name == HEADLINE:
            continue
        cmd = [sys.executable, os.path.abspath(__file__), "--workload", name, "--steps", str(steps),
               "--warmup", str(warmup), "--replicas", str(args.replicas), "--cpu-seconds",
               str(args.config_cpu_seconds), "--no-configs"]
        log(f"configs: {name}")
        r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=600)
        lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
        if r.returncode != 0 or not lines:
            raise RuntimeError(f"bench.py --workload {name} failed (exit {r.returncode}); no further GPU runs")
        res[name] = config_summary(json.loads(lines[-1]))
        log(f"configs: {name}: attention {res[name]['attention_us']['mean']} us, frac {res[name]['frac']}")
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--partition-size", type=int, default=None, help="override the workload's partition size")
    ap.add_argument("--query-len", type=int, default=1,
                    help="new tokens per sequence (> 1: a verification batch through paged_attention_decode_multi)")
    ap.add_argument("--replicas", type=int, default=2, help="pool replicas cycled by consecutive steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle timing budget (0 = skip)")
    ap.add_argument("--separate-write", action="store_true",
                    help="time the cache write and the attention as two calls even where the library appends the "
                         "new tokens in its decode launch")
    ap.add_argument("--no-configs", action="store_true",
                    help="headline run only: skip measuring the other synthetic workloads in child processes")
    ap.add_argument("--config-cpu-seconds", type=float, default=2.0,
                    help="CPU oracle budget of each other workload's child run")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="summarise two rocprofv3 --pmc databases (FETCH_SIZE, WRITE_SIZE) of this benchmark "
                         "into profiles/traffic_<workload>.md and exit")
    ap.add_argument("--traffic-cmds", nargs=2, default=("", ""), help="the two profiling commands, for the record")
    args = ap.parse_args()

    if args.traffic_from:
        print(write_traffic_summary(args.workload, *args.traffic_from, *args.traffic_cmds,
                                    query_len=args.query_len))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py runs on one GPU only: this library has no multi-GPU path (each GPU would run the "
                  "same kernels on its own share of sequences or KV heads); use --gpus 1", flush=True)
        return 2

    if args.workload == "configs":
        # every synthetic decode workload, one JSON line each, each run in a process of its own (this one never
        # touches the GPU)
        import subprocess

        from workloads import CONFIG_NAMES

        rc = 0
        for name in CONFIG_NAMES:
            cmd = [sys.executable, os.path.abspath(__file__), "--workload", name, "--steps", str(args.steps),
                   "--warmup", str(args.warmup), "--replicas", str(args.replicas), "--cpu-seconds",
                   str(args.cpu_seconds), "--no-configs"]
            log(f"configs: {name}")
            rc = rc or subprocess.run(cmd).returncode
        return rc

    # the headline run also reports every other synthetic workload, each measured in a fresh child process
    # before this one touches the GPU
    configs = None
    if args.workload == HEADLINE and args.query_len == 1 and not args.no_configs:
        configs = run_config_children(args)

    import numpy as np
    import torch

    import paged_kv_cache_458_amd as pa
    from workloads import CONFIG_NAMES, EXTRA_NAMES, algorithmic_bytes, build_structure, materialize, query_rows

    if args.workload == "decode_loop":
        return run_decode_loop(args)
    if args.workload == "swap":
        return run_swap(args)
    if args.workload not in CONFIG_NAMES + EXTRA_NAMES:
        ap.error(f"--workload must be one of {CONFIG_NAMES + EXTRA_NAMES}, configs, decode_loop or swap")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pa.load_library()

    st = build_structure(args.workload)
    part = st.partition_size if args.partition_size is None else args.partition_size
    B, Hq, Hkv, D, bs = st.num_seqs, st.num_q_heads, st.num_kv_heads, st.head_dim, st.block_size
    kv_code = {"f32": pa.PA_F32, "bf16": pa.PA_BF16, "fp8": pa.PA_FP8_E4M3}[st.dtype]
    Q = args.query_len
    if Q < 1 or (st.context_lens < Q).any():
        ap.error("--query-len must be >= 1 and at most every context length")
    T = B * Q  # query rows
    label = args.workload if Q == 1 else f"{args.workload}_q{Q}"
    if Q == 1:
        launched_part = pa.partition_size_for(B, Hq, Hkv, D, st.max_context_len, bs, kv_code, part)
    else:
        launched_part = pa.multi_partition_size_for(B, T, Q, Hq, Hkv, D, st.max_context_len, bs, kv_code, part)
    append = step_appends(Q, st.max_context_len, args.separate_write)

    t = materialize(st, dev, include_new_token=False)
    pools = [(t["key_cache"], t["value_cache"])]
    for _ in range(1, max(1, args.replicas)):
        pools.append((t["key_cache"].clone(), t["value_cache"].clone()))
    log(f"{args.workload}: {len(pools)} pool replicas of {2 * t['key_cache'].nbytes / 2**30:.2f} GiB")

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    tables, lens, slots = i32(st.block_tables), i32(st.context_lens), i32(st.slot_mapping)
    pairs = i32(st.copy_pairs) if len(st.copy_pairs) else None
    out = torch.empty((T, Hq, D), dtype=torch.float32, device=dev)
    query, new_key, new_value = t["query"], t["new_key"], t["new_value"]
    if Q > 1:
        # a verification batch: each sequence's last Q positions are new; their K/V are written, then all Q
        # rows attend (host-side slot list of those positions, prepared outside the timed region)
        query, query_start = query_rows(st, np.full(B, Q), dev)
        qstart = i32(query_start)
        pos = (st.context_lens[:, None].astype(np.int64) - Q + np.arange(Q)[None, :]).reshape(-1)
        seq = np.repeat(np.arange(B), Q)
        if (pos // bs < st.notes.get("shared_prefix_blocks", 0)).any():
            ap.error("--query-len reaches into the shared prefix blocks")
        slots = i32(st.block_tables[seq, pos // bs].astype(np.int64) * bs + pos % bs)
        gen = torch.Generator(device=dev)
        gen.manual_seed(st.seed + 104729)
        kdt = torch.float32 if st.dtype == "f32" else torch.bfloat16
        new_key = torch.randn((T, Hkv, D), generator=gen, device=dev).to(kdt)
        new_value = torch.randn((T, Hkv, D), generator=gen, device=dev).to(kdt)
        ws_bytes = pa.multi_workspace_bytes(B, T, Q, Hq, Hkv, D, st.max_context_len, bs, kv_code, part)
    else:
        ws_bytes = pa.workspace_bytes(B, Hq, Hkv, D, st.max_context_len, bs, kv_code, part)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    # Each step's library calls are bound once per pool replica, straight to the C ABI (which still checks every
    # argument on each call): with the Python binding's per-call checks, a step's host work outlasts the short
    # steps' GPU time and the events would time the GPU waiting for the host.
    import ctypes
    import functools

    lib = pa.load_library()
    sp = ctypes.c_void_p(stream.cuda_stream)
    qd = pa.PA_F32 if st.dtype == "f32" else pa.PA_BF16
    NB, MB, mcl = st.num_blocks, st.block_tables.shape[1], st.max_context_len
    nk = new_key.shape[0]

    def bound_calls(kc, vc):
        writes = []
        if pairs is not None:
            writes.append(functools.partial(lib.copy_blocks, kc.data_ptr(), vc.data_ptr(), pairs.data_ptr(),
                                            pairs.shape[0], bs, Hkv, D, NB, kv_code, sp))
        if append:
            attn = functools.partial(lib.paged_attention_decode_append, out.data_ptr(), query.data_ptr(),
                                     new_key.data_ptr(), new_value.data_ptr(), kc.data_ptr(), vc.data_ptr(),
                                     tables.data_ptr(), lens.data_ptr(), slots.data_ptr(), st.scale, st.k_scale,
                                     st.v_scale, bs, B, Hq, Hkv, D, NB, MB, mcl, qd, kv_code, part, ws.data_ptr(),
                                     ws.numel(), sp)
            return writes, attn
        if st.dtype == "fp8":
            writes.append(functools.partial(lib.reshape_and_cache_fp8, new_key.data_ptr(), new_value.data_ptr(),
                                            kc.data_ptr(), vc.data_ptr(), slots.data_ptr(), nk, Hkv, D, bs, NB,
                                            pa.PA_BF16, st.k_scale, st.v_scale, sp))
        else:
            writes.append(functools.partial(lib.reshape_and_cache, new_key.data_ptr(), new_value.data_ptr(),
                                            kc.data_ptr(), vc.data_ptr(), slots.data_ptr(), nk, Hkv, D, bs, NB,
                                            kv_code, sp))
        if Q == 1:
            attn = functools.partial(lib.paged_attention_decode_scaled, out.data_ptr(), query.data_ptr(),
                                     kc.data_ptr(), vc.data_ptr(), tables.data_ptr(), lens.data_ptr(), st.scale,
                                     st.k_scale, st.v_scale, bs, B, Hq, Hkv, D, NB, MB, mcl, qd, kv_code, part,
                                     ws.data_ptr(), ws.numel(), sp)
        else:
            attn = functools.partial(lib.paged_attention_decode_multi, out.data_ptr(), query.data_ptr(),
                                     kc.data_ptr(), vc.data_ptr(), tables.data_ptr(), lens.data_ptr(),
                                     qstart.data_ptr(), st.scale, st.k_scale, st.v_scale, bs, B, T, Q, Hq, Hkv, D,
                                     NB, MB, mcl, qd, kv_code, part, ws.data_ptr(), ws.numel(), sp)
        return writes, attn

    bound = [bound_calls(kc, vc) for kc, vc in pools]

    def run(fn):
        status = fn()
        if status != pa.PA_OK:
            raise pa.PagedAttentionError(fn.func.__name__, status)

    def step(i):
        writes, attn = bound[i % len(bound)]
        for fn in writes:  # copy-on-write pairs, then the step's new K/V
            run(fn)
        run(attn)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize(dev)
    log(f"warmup done ({args.warmup} steps)")

    # The timed region: the K steps back to back, one event pair around them. (An event pair around every step
    # added about 7 us per step on MI355X: the event records, not the work.)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    end.record(stream)
    torch.cuda.synchronize(dev)
    ms_step = start.elapsed_time(end) / args.steps

    # The attention call alone, for its duration. Where the step is that call (the appending call, no copies),
    # the timed steps give it. Otherwise K calls back to back, one event pair around them (the step's writes left
    # out: the decode gives the same result on every repetition over the same inputs). The spread comes from
    # blocks of a few calls with an event pair around each block, so its median and minimum include a share of
    # the pair's cost (about 7 us per pair on MI355X) and can read above the mean.
    def call_loop(idx):
        for i in idx:
            run(bound[(args.warmup + i) % len(bound)][1])

    if not bound[0][0]:
        attn_avg_ms = ms_step
    else:
        torch.cuda.synchronize(dev)
        start.record(stream)
        call_loop(range(args.steps))
        end.record(stream)
        torch.cuda.synchronize(dev)
        attn_avg_ms = start.elapsed_time(end) / args.steps
    block = max(1, min(5, args.steps))
    blocks = [list(range(b, min(b + block, args.steps))) for b in range(0, args.steps, block)]
    bevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in blocks]
    torch.cuda.synchronize(dev)
    for (e0, e1), idx in zip(bevs, blocks):
        e0.record(stream)
        call_loop(idx)
        e1.record(stream)
    torch.cuda.synchronize(dev)
    attn_ms = [a.elapsed_time(b) / len(idx) for (a, b), idx in zip(bevs, blocks)]
    log(f"timed {args.steps} steps: {ms_step * 1e3:.1f} us/step; attention call {attn_avg_ms * 1e3:.1f} us "
        f"(blocks of {block}: median {np.median(attn_ms) * 1e3:.1f}, min {np.min(attn_ms) * 1e3:.1f})")

    # the practical ceiling: a plain streaming read (same 16-byte loads) and copy over 4 GiB on this device
    big = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
    big2 = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
    sink = torch.empty(pa.STREAM_SINK_FLOATS, dtype=torch.float32, device=dev)
    for _ in range(3):
        pa.stream_read(big, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        pa.stream_read(big, sink)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    read_gbs = 10 * big.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    e0.record(stream)
    for _ in range(10):
        pa.stream_copy(big2, big[: big2.numel()])
    e1.record(stream)
    torch.cuda.synchronize(dev)
    copy_gbs = 10 * 2 * big2.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del big, big2
    log(f"streaming read {read_gbs:.0f} GB/s, copy {copy_gbs:.0f} GB/s (read + write)")

    ab = algorithmic_bytes(st, Q)
    row_bytes = Hkv * D * st.esize
    # K and V: read the new row (query dtype), write it into the cache (cache dtype)
    new_rows = int((st.slot_mapping >= 0).sum()) if Q == 1 else T
    cache_write_bytes = 2 * new_rows * Hkv * D * (st.q_esize + st.esize)
    copy_bytes = 2 * 2 * len(st.copy_pairs) * bs * row_bytes
    step_bytes = ab["total"] + cache_write_bytes + copy_bytes
    value = step_bytes / (ms_step * 1e-3) / 1e9
    # the timed call's bytes: the attention's, plus the new rows read and written when the call appends them
    call_bytes = ab["total"] + (cache_write_bytes if append else 0)
    attn_gbs = call_bytes / (attn_avg_ms * 1e-3) / 1e9
    # bytes HBM must deliver: a block that several sequences share (a common prefix) counts once per call
    unique_bytes = ab["kv_unique"] + ab["query"] + ab["out"] + ab["tables"] + (cache_write_bytes if append else 0)
    attn_gbs_unique = unique_bytes / (attn_avg_ms * 1e-3) / 1e9
    traffic = load_traffic(label)

    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # an E4M3 cache is widened to bf16 for the products: the arithmetic is bf16 x bf16 -> f32
        "dtype": "bf16" if st.dtype == "fp8" else st.dtype,
        "accumulate": "f32",
        "data": "synthetic",
        "config": {
            "workload": label,
            "num_seqs": B,
            "query_len": Q,
            "num_q_heads": Hq,
            "num_kv_heads": Hkv,
            "head_dim": D,
            "block_size": bs,
            "kv_cache_dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8_e4m3"}[st.dtype],
            "context_len_mean": float(st.context_lens.mean()),
            "context_len_max": int(st.context_lens.max()),
            "partition_size": "balanced" if launched_part == pa.PA_PARTITION_BALANCED else launched_part,
            "step": "appended in the decode launch" if append else "cache write, then attention",
            "pool_blocks": st.num_blocks,
            "replicas": len(pools),
            "seed": st.seed,
        },
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "decode_queries_per_s": round(T / (ms_step * 1e-3), 1),  # query rows (tokens), B * query_len
        "attention": {
            "us_mean": round(attn_avg_ms * 1e3, 2),
            "us_median": round(float(np.median(attn_ms)) * 1e3, 2),
            "us_min": round(float(np.min(attn_ms)) * 1e3, 2),
            "gb_per_s": round(attn_gbs, 1),
            "gb_per_s_unique": round(attn_gbs_unique, 1),
            "queries_per_s": round(T / (attn_avg_ms * 1e-3), 1),
            "bytes_per_call": call_bytes,
            "unique_bytes_per_call": unique_bytes,
            "kv_unique_bytes": ab["kv_unique"],
        },
        "step_bytes": step_bytes,
        "device_stream_read_gbs": round(read_gbs, 1),
        "device_stream_copy_gbs": round(copy_gbs, 1),
        "roofline": {
            "bound": "hbm",
            "kernel": ("paged_attention_decode_append (decode kernel appending the new tokens + log-sum-exp "
                       "reduce when split)" if append else
                       ("paged_attention_decode" if Q == 1 else "paged_attention_decode_multi") +
                       " (partition or balanced-split kernel + log-sum-exp reduce when split)"),
            # unique bytes (shared blocks once); the logical count of the metric's byte formula beside it
            "achieved": round(attn_gbs_unique, 1),
            "achieved_logical": round(attn_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(attn_gbs_unique / PEAK_HBM_GBS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": None,
    }

    if args.cpu_seconds > 0:
        import oracle

        kc, vc = pools[0]
        host = {}
        for name, tt in (("query", query), ("key_cache", kc), ("value_cache", vc)):
            tt = tt.contiguous().cpu()
            if tt.dtype == torch.bfloat16:
                host[name] = tt.view(torch.int16).numpy().view(np.uint16)
            elif tt.dtype == torch.float8_e4m3fn:
                host[name] = tt.view(torch.uint8).numpy()
            else:
                host[name] = tt.numpy()
        lib = oracle.load()
        reps, t0, last = 0, time.perf_counter(), 0.0
        while True:
            if Q == 1:
                oracle.decode(host["query"], host["key_cache"], host["value_cache"], st.block_tables,
                              st.context_lens, st.scale, k_scale=st.k_scale, v_scale=st.v_scale, lib=lib)
            else:
                oracle.decode_multi(host["query"], host["key_cache"], host["value_cache"], st.block_tables,
                                    st.context_lens, query_start, st.scale, k_scale=st.k_scale, v_scale=st.v_scale,
                                    lib=lib)
            reps += 1
            el = time.perf_counter() - t0
            if el - last >= 5.0:
                log(f"cpu oracle: {reps} calls in {el:.1f} s")
                last = el
            if el >= args.cpu_seconds or reps >= 1000:
                break
        log(f"cpu oracle: {reps} calls in {el:.1f} s")
        rec["cpu_baseline"] = {
            "value": round(T * reps / el, 2),
            "unit": "decode queries/s",
            "gb_per_s": round(ab["total"] * reps / el / 1e9, 3),
            "cores": oracle.num_threads(lib),
            "nproc": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"the whole {label} batch ({T} query rows x {Hq} heads, fp64 C oracle with OpenMP), "
                      f"{reps} call(s) in {el:.1f} s",
        }
    if configs is not None:
        rec["configs"] = {HEADLINE: config_summary(rec), **configs}
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
