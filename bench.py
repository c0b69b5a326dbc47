"""Benchmark: one rank's causal bf16 ring of attention on one MI355X.

A "step" is one whole emulated ring of the rank: state init, the P ring steps
(side-stream staging of the next key/value block, double-buffered swaps, one
ra_step launch per non-skipped block) and the finalize; by default the init
and the finalize are fused into the first and the last launched step
(ra_step_ex; --unfused launches them separately).  Inputs are seeded
synthetic blocks already resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--rank I]
                    [--partition contiguous|zigzag] [--decode-rows R] [--backward]
                    [--unfused] [--no-cpu-baseline]

Prints ONE JSON line.  FLOPs count 4*head_dim per unmasked (query, key) pair
per head (the diagonal block counts c(c+1)/2 pairs, skipped blocks none).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from ring_attention_block_amd import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_FP32_VECTOR_TFLOPS = 157.3
PEAK_HBM_BYTES = 8.0e12     # MI355X HBM3E, bytes/s
HBM_GBPS = 8000.0
DEFAULT_WORKLOAD = "causal_bf16_h32_d128_c4096_p8"
DEFAULT_RANK = 7


def unmasked_pairs(wl, rank, rows=None):
    """Unmasked (query, key) pairs of one head for `rank` (optionally only `rows`)."""
    c = wl.rows
    rows = np.arange(c) if rows is None else np.asarray(rows)
    if not wl.causal:
        return int(len(rows) * c * wl.blocks)
    return int(np.sum(rank * c + rows + 1))


def ring_flops(wl, rank):
    return 4 * wl.head_dim * wl.heads * unmasked_pairs(wl, rank)


def full_step_flops(wl):
    return 4 * wl.head_dim * wl.heads * wl.rows * wl.rows


def generate(wl, rank, threads=16, q_blocks=None):
    """Seeded blocks of the workload (Q of the rank's blocks, every K and V), in
    parallel; each block has its own seed, so threading does not change any value."""
    import concurrent.futures as cf
    q_blocks = (rank,) if q_blocks is None else tuple(q_blocks)
    jobs = [(synth.ROLE_Q, b) for b in q_blocks] + [(r, j) for j in range(wl.blocks)
                                                    for r in (synth.ROLE_K, synth.ROLE_V)]
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        arrs = list(ex.map(lambda rj: synth.block(wl, *rj), jobs))
    return dict(zip(jobs, arrs))


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles",
                               "ra_step_bf16_full_causal_h32_d128_c4096_hbm_traffic.md")
BWD_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles",
                                   "ra_bwd_step_bf16_full_causal_h32_d128_c4096_hbm_traffic.md")
DEC_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles",
                                   "ra_step_bf16_decode_h32_d128_shards8x4096_q16_hbm_traffic.md")
DEC_TRAFFIC_ROWS = 16   # the query-block length the decode counters were taken at


def software_versions() -> dict:
    """ROCm, HIP runtime, torch and device identity of the run."""
    import torch
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    props = torch.cuda.get_device_properties(0)
    return {"rocm": rocm, "hip": torch.version.hip, "torch": torch.__version__,
            "numpy": np.__version__, "device": props.name,
            "arch": getattr(props, "gcnArchName", None), "compute_units": props.multi_processor_count}


def device_memory() -> dict:
    """Peak device memory the run held through torch's caching allocator (the
    library allocates nothing: every buffer of the emulated rank, the blocks
    of the other ranks included, is a torch tensor)."""
    import torch
    return {"peak_allocated_bytes": int(torch.cuda.max_memory_allocated()),
            "peak_reserved_bytes": int(torch.cuda.max_memory_reserved()),
            "note": "whole process: inputs of every emulated rank, receive buffers, states, "
                    "outputs, graph pools"}


COUNTER_PROFILE = "ra_step_bf16_causal_h32_d128_c4096_counters.md"
COUNTER_KEYS = ("sclk_mhz", "mfma_busy_pct", "valu_busy_pct", "lds_bank_conflict_pct")


def profile_fields(name, keys):
    """Machine-readable `key: value` lines of profiles/<name>, only while the
    kernel source still hashes to the recorded kernel_source_sha256; else None."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        key, sep, val = line.strip().partition(": ")
        if sep and (key in keys or key in ("kernel_source", "kernel_source_sha256")):
            fields[key] = val.strip()
    if "kernel_source" not in fields or "kernel_source_sha256" not in fields:
        return None
    src = os.path.join(ROOT, fields["kernel_source"])
    if not os.path.exists(src):
        return None
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != fields["kernel_source_sha256"]:
            return None
    return fields


def measured_counters(case):
    """Shader clock and MFMA, VALU and LDS-conflict occupancy of the full
    ("full") or diagonal ("diag") step kernel of the headline ring, from the
    committed counter summary; `current` false (no figures) once the kernel
    source has changed since the counters were taken."""
    keys = tuple(f"{case}.{k}" for k in COUNTER_KEYS)
    f = profile_fields(COUNTER_PROFILE, keys)
    if not f:
        return {"profile": "profiles/" + COUNTER_PROFILE, "current": False}
    out = {"profile": "profiles/" + COUNTER_PROFILE, "current": True}
    for k in COUNTER_KEYS:
        v = f.get(f"{case}.{k}")
        out[k] = float(v) if v else None
    return out


def host_info() -> dict:
    """The host the oracle runs on: `cores` is the thread count the oracle
    actually uses for its products (numpy's BLAS threads; the exponentials run
    on one thread), `affinity_cores` the CPUs this process may run on
    (os.sched_getaffinity), plus the CPU model and the BLAS library."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, blas_threads = None, None
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
            blas_threads = max(i.get("num_threads", 1) for i in libs)
    except Exception:  # noqa: BLE001
        pass
    return {"cores": blas_threads, "affinity_cores": len(os.sched_getaffinity(0)),
            "cpu_model": model, "blas": blas}


def capture_ring(one_ring, copy_stream, compute, outs):
    """See _capture; copy_stream None: the ring runs on the compute stream
    alone (staging carried by the step launches), nothing to join."""
    return _capture(one_ring, copy_stream, compute, outs)


def _capture(one_ring, copy_stream, compute, outs):
    """One untimed ring captured as a HIP graph on the compute stream (the
    copy stream forks from it through the ring's first event and is joined
    back at the end), for the untimed rings of the timed region: one graph
    launch per ring instead of the host enqueueing every copy, wait and step.
    The graph is used only if its replay reproduces the eager ring's outputs
    bit for bit, twice, with an eager ring in between; otherwise (None,
    reason) and every ring runs eagerly."""
    import torch
    from ring_attention_block_amd.hip_events import Event

    join = Event()

    def joined():
        one_ring()
        if copy_stream is not None:
            join.record(copy_stream)
            join.wait(compute)

    try:
        joined()
        torch.cuda.synchronize()
        want = [t.clone() for pair in outs for t in pair]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=compute):
            joined()
        torch.cuda.synchronize()
        for _ in range(2):
            for pair in outs:
                for t in pair:
                    t.fill_(float("nan"))
            torch.cuda.synchronize()
            with torch.cuda.stream(compute):
                g.replay()
            torch.cuda.synchronize()
            got = [t for pair in outs for t in pair]
            if not all(torch.equal(a, b) for a, b in zip(got, want)):
                return None, "off: the replay differed from the eager ring"
            joined()
            torch.cuda.synchronize()
        return g, "untimed rings replay one captured ring"
    except Exception as e:  # capture unsupported here: every ring runs eagerly
        torch.cuda.synchronize()
        return None, f"off: capture failed ({type(e).__name__}: {e})"


def timed_rings(args) -> int:
    """Timed rings whose step launches carry timing events (every time_every-th)."""
    return (args.steps + args.time_every - 1) // args.time_every


def measured_traffic(wl, profile=TRAFFIC_PROFILE, require=None):
    """HBM bytes per full-step launch from a committed FETCH_SIZE/WRITE_SIZE summary.

    Only for the workload the counters were taken on, only while the kernel
    source still hashes to the value recorded with them, and only if every
    `require` key is recorded there with the given value; else None.
    """
    if wl.name != DEFAULT_WORKLOAD:
        return None
    require = require or {}
    f = profile_fields(os.path.basename(profile), ("traffic_bytes_per_launch", *require))
    if not f or "traffic_bytes_per_launch" not in f:
        return None
    if any(f.get(k) != str(v) for k, v in require.items()):
        return None
    return int(f["traffic_bytes_per_launch"])


def cpu_baseline(wl, rank, blocks, target_s=15.0):
    """The CPU fp64 oracle, as it stands, on a bounded sample of query rows."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from _helpers import oracle_rank          # test plumbing around oracle/
    host = host_info()
    cache = dict(blocks)
    kv_blocks = list(range(rank + 1)) if wl.causal else list(range(wl.blocks))
    n = 4
    while True:
        rows = synth.sample_rows(wl.seed, wl.rows, n)
        t0 = time.perf_counter()
        oracle_rank(wl, rank, kv_blocks, wl.causal, row_sel=rows, cache=cache)
        dt = time.perf_counter() - t0
        if dt >= target_s / 3 or n >= wl.rows:
            break
        n = min(wl.rows, int(n * max(2.0, target_s / 3 / max(dt, 1e-3))))
    flops = 4 * wl.head_dim * wl.heads * unmasked_pairs(wl, rank, rows)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": host["cores"],
            "kind": "oracle", **{k: v for k, v in host.items() if k != "cores"},
            "sample": f"{len(rows)} seeded query rows x {wl.heads} heads of rank {rank} "
                      f"({flops / 1e9:.1f} GFLOP fp64, {dt:.1f} s; numpy BLAS threads for the "
                      f"products, one thread for exp)"}


def cpu_baseline_decode(wl, blocks, rq, target_s=15.0):
    """The CPU fp64 oracle on the decode step, head by head (each head: the
    rq query rows against all P x c keys, inputs converted to fp64 as the
    oracle takes them) until about target_s / 3 seconds; the rate is the
    key/value bytes of the heads done per second."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from _helpers import oracle_values        # test plumbing around oracle/
    from oracle import dense
    host = host_info()
    P, c = wl.blocks, wl.rows
    qh = synth.block(wl, synth.ROLE_Q, P, rows=rq)
    kp, qp = np.arange(P * c), np.full(rq, P * c)
    esize = 2 if wl.dtype == "bf16" else 4
    done, t0 = 0, time.perf_counter()
    while done < wl.heads:
        h = done
        k = np.concatenate([oracle_values(blocks[(synth.ROLE_K, j)][h:h + 1], wl) for j in range(P)],
                           axis=1)
        v = np.concatenate([oracle_values(blocks[(synth.ROLE_V, j)][h:h + 1], wl) for j in range(P)],
                           axis=1)
        dense.attention(oracle_values(qh[h:h + 1], wl), k, v, qp, kp, False, wl.scale)
        done += 1
        if time.perf_counter() - t0 >= target_s / 3:
            break
    dt = time.perf_counter() - t0
    nbytes = 2 * P * c * wl.head_dim * esize * done
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": host["cores"], "kind": "oracle",
            **{k: v for k, v in host.items() if k != "cores"},
            "sample": f"{rq} query rows x {done} of {wl.heads} heads against {P} x {c} keys "
                      f"({nbytes / 1e6:.0f} MB of keys and values, {dt:.1f} s; numpy BLAS threads "
                      f"for the products, one thread for exp)"}


def bench_decode(args, wl):
    """Decode: args.decode_rows query rows (the tokens after the sequence)
    against the workload's P blocks as key/value shards, each shard laid out
    as S chunks of consecutive keys along the batch axis (ring.split_keys;
    S from --decode-splits, by default decode.splits_for) (ChunkedDecode: one
    ra_step launch over all chunks reading the one query block, one
    ra_merge_finalize over the P*S partial states).  Memory-bound: the figure
    of merit is the key/value bytes read per second."""
    import torch
    from ring_attention_block_amd.decode import ChunkedDecode, splits_for
    from ring_attention_block_amd.ring import split_keys
    from ring_attention_block_amd.hip_events import Event

    rq, P, c = args.decode_rows, wl.blocks, wl.rows
    blocks = generate(wl, P - 1)
    dev = "cuda"

    def to_dev(x):
        t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if wl.dtype == "bf16" \
            else torch.from_numpy(x)
        return t.reshape(1, *x.shape).to(dev)

    S = splits_for(P, wl.heads, c, rq) if args.decode_splits == "auto" else int(args.decode_splits)
    if S < 1 or c % S:
        raise SystemExit(f"--decode-splits {S} must divide the shard length {c}")
    q = to_dev(synth.block(wl, synth.ROLE_Q, P, rows=rq))   # the tokens after the cache
    k = torch.cat([split_keys(to_dev(blocks[(synth.ROLE_K, j)]), S) for j in range(P)], dim=0)
    v = torch.cat([split_keys(to_dev(blocks[(synth.ROLE_V, j)]), S) for j in range(P)], dim=0)
    compute = torch.cuda.Stream()
    dec = ChunkedDecode(q.shape, P * S, dev, compute_stream=compute)
    o = torch.empty(q.shape, dtype=torch.float32, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    # The step kernel of one timed step in time_every carries timing events
    # bound to its dispatch.
    n_timed = len(range(0, args.steps, args.time_every))
    pool = iter([Event(timing=True) for _ in range(2 * n_timed)])
    timers = []
    e0, e1 = Event(timing=True), Event(timing=True)
    for _ in range(args.warmup):
        dec.run(q, k, v, wl.scale, o_out=o, lse_out=lse)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(compute)
    for s in range(args.steps):
        ev = (next(pool), next(pool)) if s % args.time_every == 0 else (None, None)
        dec.run(q, k, v, wl.scale, o_out=o, lse_out=lse, start=ev[0], stop=ev[1])
        if ev[0] is not None:
            timers.append(ev)
    e1.record(compute)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed / args.steps * 1e3
    esize = 2 if wl.dtype == "bf16" else 4
    kv_bytes = 2 * P * c * wl.heads * wl.head_dim * esize
    flops = 4 * wl.head_dim * wl.heads * rq * P * c
    # Algorithmic bytes of the fold launch: the cache and the query block as
    # the P*S chunks' workgroups read it, the P*S partial states written (m, l, O
    # in fp32; the fresh fold reads no state).
    step_bytes = kv_bytes + P * S * wl.heads * rq * (wl.head_dim * esize + (wl.head_dim + 2) * 4)
    step_ms = float(np.mean([a.elapsed_time(b) for a, b in timers]))
    achieved = step_bytes / (step_ms / 1e3) / 1e9
    peak = PEAK_HBM_BYTES / 1e9
    line = {
        "metric": "decode key/value read rate (GB/s)", "value": round(kv_bytes / (ms / 1e3) / 1e9, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) blocks rounded to bf16, resident in HBM)",
        "config": {"workload": wl.name, "mode": "decode", "query_rows": rq, "shards": P,
                   "shard_rows": c, "heads": wl.heads, "head_dim": wl.head_dim,
                   "splits_per_shard": S,
                   "layout": f"each shard as {S} chunk(s) of {c // S} keys along the batch axis",
                   "kv_bytes": kv_bytes, "flop_per_step": flops,
                   "tflops": round(flops / (ms / 1e3) / 1e12, 2),
                   "pct_of_hbm_peak": round(100 * kv_bytes / (ms / 1e3) / PEAK_HBM_BYTES, 2)},
        "roofline": {"bound": "hbm", "kernel": "ra_step decode fold", "achieved": round(achieved, 1),
                     "peak": peak, "unit": "GB/s", "frac": round(achieved / peak, 4),
                     "traffic": (measured_traffic(wl, DEC_TRAFFIC_PROFILE, {"splits_per_shard": S})
                                 if rq == DEC_TRAFFIC_ROWS else None),
                     "bytes_per_launch": step_bytes,
                     "avg_launch_ms": round(step_ms, 5), "launches": len(timers),
                     "timed_steps": f"1 in {args.time_every} of the {args.steps} timed steps"},
        "compute_stream_ms": round(e0.elapsed_time(e1) / args.steps, 4),
        "env": software_versions(),
        "memory": device_memory(),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(wl, blocks, rq)
    print(json.dumps(line), flush=True)


def cpu_baseline_backward(wl, rank, blocks, target_s=15.0):
    """The CPU fp64 oracle's dense attention backward (dQ, dK, dV), as it
    stands, on a bounded sample of rank's query rows against the key blocks
    its backward ring visits, every head; FLOPs as for the GPU line (10 x
    head_dim per unmasked pair per head)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from _helpers import oracle_values        # test plumbing around oracle/
    from oracle import backward, dense
    host = host_info()
    kv_blocks = list(range(rank + 1)) if wl.causal else list(range(wl.blocks))
    kp = np.concatenate([dense.ring_positions(j, wl.rows) for j in kv_blocks])
    n = 4
    while True:
        rows = synth.sample_rows(wl.seed, wl.rows, n)
        qp = dense.ring_positions(rank, wl.rows)[rows]
        t0 = time.perf_counter()
        for h in range(wl.heads):
            kh = np.concatenate([oracle_values(blocks[(synth.ROLE_K, j)][h:h + 1], wl)
                                 for j in kv_blocks], axis=1)
            vh = np.concatenate([oracle_values(blocks[(synth.ROLE_V, j)][h:h + 1], wl)
                                 for j in kv_blocks], axis=1)
            backward.attention_backward(oracle_values(blocks[(synth.ROLE_Q, rank)][h:h + 1, rows], wl),
                                        kh, vh,
                                        oracle_values(blocks[(synth.ROLE_DO, rank)][h:h + 1, rows], wl),
                                        qp, kp, wl.causal, wl.scale)
        dt = time.perf_counter() - t0
        if dt >= target_s / 3 or n >= wl.rows:
            break
        n = min(wl.rows, int(n * max(2.0, target_s / 3 / max(dt, 1e-3))))
    flops = 10 * wl.head_dim * wl.heads * unmasked_pairs(wl, rank, rows)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": host["cores"],
            "kind": "oracle", **{k: v for k, v in host.items() if k != "cores"},
            "sample": f"{len(rows)} seeded query rows x {wl.heads} heads of rank {rank}, backward "
                      f"({flops / 1e9:.1f} GFLOP fp64, {dt:.1f} s; numpy BLAS threads for the "
                      f"products, one thread for exp)"}


def bench_backward(args, wl, rank):
    """Backward ring of `rank`: D = rowsum(dO * O) (ra_bwd_prepare), then the P
    ring steps with dK, dV travelling with the visiting block (staged in,
    updated, sent on).  The forward that provides O and the LSE runs once,
    before the timed region.  FLOPs count 10*head_dim per unmasked (query, key)
    pair per head: the five products of the gradients (S, dP, dV, dQ, dK)."""
    import torch
    from ring_attention_block_amd import _lib
    from ring_attention_block_amd.hip_events import Event
    from ring_attention_block_amd.ring import RingEmulator, ZigzagRing, zigzag_blocks, zigzag_plan

    dev = "cuda"
    zigzag = args.partition == "zigzag"
    step_wl = synth.zigzag_workload(wl) if zigzag else wl
    mine = zigzag_blocks(rank, wl.blocks) if zigzag else (rank,)
    blocks = generate(step_wl, rank, q_blocks=mine)
    for b in mine:
        blocks[(synth.ROLE_DO, b)] = synth.block(step_wl, synth.ROLE_DO, b)

    def to_dev(x):
        t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if wl.dtype == "bf16" \
            else torch.from_numpy(x)
        return t.reshape(1, *x.shape).to(dev)

    qs = [to_dev(blocks[(synth.ROLE_Q, b)]) for b in mine]
    dos = [to_dev(blocks[(synth.ROLE_DO, b)]) for b in mine]
    kv = {j: (to_dev(blocks[(synth.ROLE_K, j)]), to_dev(blocks[(synth.ROLE_V, j)]))
          for j in range(step_wl.blocks)}
    shape = tuple(qs[0].shape)
    compute = torch.cuda.Stream()
    states = [_lib.State(*shape, device=dev) for _ in mine]
    grads = {j: (torch.zeros(shape, dtype=torch.float32, device=dev),
                 torch.zeros(shape, dtype=torch.float32, device=dev)) for j in range(step_wl.blocks)}
    dqs = [torch.zeros(shape, dtype=torch.float32, device=dev) for _ in mine]
    deltas = [torch.empty(shape[:3], dtype=torch.float32, device=dev) for _ in mine]
    if zigzag:
        ring = ZigzagRing(shape, qs[0].dtype, dev, compute_stream=compute, backward=True)

        def source(j):
            a, b = zigzag_blocks(j, wl.blocks)
            return (kv[a][0], kv[b][0], kv[a][1], kv[b][1], grads[a][0], grads[b][0],
                    grads[a][1], grads[b][1])

        ring.run(states, qs, lambda j: source(j)[:4], rank, wl.blocks, wl.causal, wl.scale)
        cases = [c for _, prods in zigzag_plan(rank, wl.blocks, wl.causal) for _, _, c in prods]
    else:
        ring = RingEmulator(shape, qs[0].dtype, dev, compute_stream=compute,
                            extra_specs=[(shape, torch.float32), (shape, torch.float32)])
        source = lambda j: (kv[j][0], kv[j][1], grads[j][0], grads[j][1])
        ring.run(states[0], qs[0], lambda j: source(j)[:2], rank, wl.blocks, wl.causal, wl.scale)
        cases = [_lib.step_case(rank, j, wl.blocks, wl.causal) for j in range(wl.blocks)]
    outs = [_lib.finalize(st, torch.float32, compute) for st in states]
    torch.cuda.synchronize()
    del states

    def one_ring(timers=None, pool=None):
        for (o, _), do, delta, dq in zip(outs, dos, deltas, dqs):
            _lib.bwd_prepare(o, do, delta, stream=compute, dq=dq)   # also zeroes dQ
        lses = [lse for _, lse in outs]
        if zigzag:
            ring.run_backward(qs, dos, lses, deltas, dqs, source, rank, wl.blocks, wl.causal,
                              wl.scale, step_timers=timers, timer_events=pool)
        else:
            ring.run_backward(qs[0], dos[0], lses[0], deltas[0], dqs[0], source, rank, wl.blocks,
                              wl.causal, wl.scale, step_timers=timers, timer_events=pool)

    launched = sum(c != _lib.RA_CASE_SKIP for c in cases)
    pool = iter([Event(timing=True) for _ in range(2 * launched * timed_rings(args))])
    timers = []
    for _ in range(args.warmup):
        one_ring()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in range(args.steps):
        one_ring(*((timers, pool) if r % args.time_every == 0 else ()))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed / args.steps * 1e3
    c2 = step_wl.rows
    pairs = (cases.count(_lib.RA_CASE_FULL) * c2 * c2 + cases.count(_lib.RA_CASE_DIAG) * c2 * (c2 + 1) // 2)
    flops = 10 * wl.head_dim * wl.heads * pairs
    tflops = flops / (ms / 1e3) / 1e12
    full = [a.elapsed_time(b) for c, a, b in timers if c == _lib.RA_CASE_FULL]
    diag = [a.elapsed_time(b) for c, a, b in timers if c == _lib.RA_CASE_DIAG]
    if full:
        dom_ms, dom_flops = float(np.mean(full)), 10 * wl.head_dim * wl.heads * c2 * c2
        dom = "ra_bwd_step full (bwd_dq + bwd_dkdv kernels)"
    else:
        dom_ms = float(np.mean(diag))
        dom_flops = 10 * wl.head_dim * wl.heads * (c2 * (c2 + 1) // 2)
        dom = "ra_bwd_step diagonal (bwd_dq + bwd_dkdv kernels)"
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_VECTOR_TFLOPS
    achieved = dom_flops / (dom_ms / 1e3) / 1e12
    line = {
        "metric": (f"{'causal' if wl.causal else 'non-causal'} {wl.dtype} ring-step attention backward "
                   f"TFLOP/s (c={wl.rows}, d={wl.head_dim})"),
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) blocks rounded to bf16, resident in HBM)",
        "config": {"workload": wl.name, "mode": "backward", "rank": rank,
                   "partition": args.partition, "heads": wl.heads,
                   "head_dim": wl.head_dim, "rows_per_block": wl.rows, "blocks": wl.blocks,
                   "causal": wl.causal, "tokens": wl.tokens, "flop_per_step": flops,
                   "pct_of_mfma_peak": round(100 * tflops / peak, 2)},
        "roofline": {"bound": "mfma" if wl.dtype == "bf16" else "alu", "kernel": dom,
                     "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": (measured_traffic(wl, BWD_TRAFFIC_PROFILE)
                                 if full and not zigzag else None),
                     "avg_launch_ms": round(dom_ms, 5),
                     "launches": len(full) if full else len(diag),
                     "timed_rings": f"1 in {args.time_every} of the {args.steps} timed rings",
                     "diag_avg_launch_ms": round(float(np.mean(diag)), 5) if diag else None},
        "ring": {"cases": {"skip": cases.count(_lib.RA_CASE_SKIP),
                           "diag": cases.count(_lib.RA_CASE_DIAG),
                           "full": cases.count(_lib.RA_CASE_FULL)}},
        "env": software_versions(),
        "memory": device_memory(),
    }
    if not args.no_cpu_baseline and not zigzag:
        line["cpu_baseline"] = cpu_baseline_backward(wl, rank, blocks)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # 30 untimed rings: with 3 the clocks have not settled and the timed
    # rings of the 32-head causal workload ran 1-2% slower.
    ap.add_argument("--warmup", type=int, default=30)
    # Each timing event costs the compute stream a few microseconds between two
    # step kernels (a bound start event about 8 us, a stop event about 4 us), so
    # the kernel durations are sampled: the launches of every K-th timed ring
    # carry events (all rings with K = 1).  At the defaults two of the 20 timed
    # rings are sampled (14 full-step launches of the headline ring).
    ap.add_argument("--time-every", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(synth.WORKLOADS))
    ap.add_argument("--rank", type=int, default=None)
    ap.add_argument("--partition", default="contiguous", choices=("contiguous", "zigzag"),
                    help="contiguous: rank i holds block i; zigzag: the sequence in 2P pieces, "
                         "rank i holds pieces i and 2P-1-i")
    ap.add_argument("--decode-rows", type=int, default=None,
                    help="instead of the ring: decode this many query rows against the "
                         "workload's P blocks as key/value shards (all shards folded by one "
                         "launch along the batch axis, one merge-and-finalize launch)")
    ap.add_argument("--decode-splits", default="auto",
                    help="with --decode-rows: lay each shard out as this many chunks of "
                         "consecutive keys along the batch axis (more workgroups per fold); "
                         "auto: decode.splits_for")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the forward ring: the rank's backward ring (D, then the "
                         "P gradient steps with dK, dV travelling with the blocks)")
    ap.add_argument("--unfused", action="store_true",
                    help="separate init and finalize launches instead of fusing them into the "
                         "first and last ring steps")
    ap.add_argument("--key-split", default="auto", choices=("auto", "1", "2", "4"),
                    help="key ranges per visiting block (no causal mask only): auto splits when "
                         "the query block alone would leave compute units idle")
    ap.add_argument("--staging", default="auto", choices=("auto", "side", "fused"),
                    help="forward rings: stage the next block with copy kernels on a side stream "
                         "ordered by events (side), or inside the step launches on the compute "
                         "stream alone (fused, ra_step_staged); auto: ring.staging_for")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="enqueue every untimed ring eagerly instead of replaying a captured one")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.time_every < 1:
        ap.error("--time-every must be >= 1")

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the ring of one rank is emulated on a "
              "single MI355X; the library has no multi-GPU ring (no collectives).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from ring_attention_block_amd import _lib
    from ring_attention_block_amd.hip_events import Event
    from ring_attention_block_amd.ring import (RingEmulator, ZigzagRing, key_split_for, launch_pairs,
                                               split_keys, staging_for, zigzag_blocks,
                                               zigzag_fused_launches)

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    _lib.lib()   # fails loudly if libra.so is missing

    wl = synth.WORKLOADS[args.workload]
    if args.decode_rows is not None:
        bench_decode(args, wl)
        return
    rank = args.rank if args.rank is not None else (
        DEFAULT_RANK if wl.name == DEFAULT_WORKLOAD else wl.ranks[-1])
    if args.backward:
        bench_backward(args, wl, rank)
        return
    dev = "cuda"
    compute = torch.cuda.Stream()

    def to_dev(x, w):
        if w.dtype == "bf16":
            t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(x)
        return t.reshape(1, *x.shape).to(dev)

    if args.partition == "contiguous":
        step_wl = wl
        blocks = generate(wl, rank)
        q = to_dev(blocks[(synth.ROLE_Q, rank)], wl)
        kv = {j: (to_dev(blocks[(synth.ROLE_K, j)], wl), to_dev(blocks[(synth.ROLE_V, j)], wl))
              for j in range(wl.blocks)}
        # Without the causal mask a small query block may fold each visiting
        # block as key ranges into partial states merged at the end.
        ks = (key_split_for(wl.heads, wl.rows, wl.rows, wl.causal) if args.key_split == "auto"
              else int(args.key_split))
        if ks > 1:
            kv = {j: (split_keys(k, ks), split_keys(v, ks)) for j, (k, v) in kv.items()}
        states = [_lib.State(ks, wl.heads, wl.rows, wl.head_dim, device=dev)]
        cases = [_lib.step_case(rank, j, wl.blocks, wl.causal) for j in range(wl.blocks)]
        staging = (staging_for(ks * wl.heads, wl.rows, wl.rows // ks, wl.head_dim,
                               cases.count(_lib.RA_CASE_SKIP))
                   if args.staging == "auto" else args.staging)
        emu = RingEmulator(kv[0][0].shape, q.dtype, dev, compute_stream=compute, staging=staging)
        flops = ring_flops(wl, rank)
        baseline_q = rank

        fused = not args.unfused or ks > 1
        copy_stream = emu.copy if staging == "side" else None

        def fold(timers, pool):
            emu.run(states[0], q, lambda j: kv[j], rank, wl.blocks, wl.causal, wl.scale,
                    step_timers=timers, timer_events=pool,
                    finalize_out=outs[0] if fused else None, key_split=ks)
    else:
        ks = 1
        # Zigzag: the sequence in 2P pieces of c/2 tokens; the rank holds
        # pieces (rank, 2P-1-rank), both in one block in position order (and
        # so does every visiting rank's block); each visit is one launch on
        # row ranges of these blocks, the own visit one causal diagonal launch
        # (ZigzagRing.run_block), split per piece where a fused init or
        # finalize needs it.
        step_wl = synth.zigzag_workload(wl)
        mine = zigzag_blocks(rank, wl.blocks)
        blocks = generate(step_wl, rank, q_blocks=mine)
        q = torch.cat([to_dev(blocks[(synth.ROLE_Q, b)], step_wl) for b in mine], dim=2)
        kv = {}
        for j in range(wl.blocks):
            pieces = zigzag_blocks(j, wl.blocks)
            kv[j] = tuple(torch.cat([to_dev(blocks[(role, b)], step_wl) for b in pieces], dim=2)
                          for role in (synth.ROLE_K, synth.ROLE_V))
        states = [_lib.State(1, wl.heads, 2 * step_wl.rows, wl.head_dim, device=dev)]
        fused = not args.unfused
        zplan = zigzag_fused_launches(rank, wl.blocks, wl.causal)
        if not fused:
            from ring_attention_block_amd.ring import zigzag_launches
            zplan = zigzag_launches(rank, wl.blocks, wl.causal)
        launches = [l for _, ls in zplan for l in ls]
        cases = [l[4] for l in launches]
        c2 = step_wl.rows
        launch_flops = [4 * wl.head_dim * wl.heads * launch_pairs(l, c2) for l in launches]
        flops = sum(launch_flops)
        # the visit with the least matrix work decides the staging mode
        lightest = min(sum(launch_pairs(l, c2) for l in ls) for _, ls in zplan)
        staging = (staging_for(wl.heads, lightest, 1, wl.head_dim, 0)
                   if args.staging == "auto" else args.staging)
        zz = ZigzagRing((1, wl.heads, c2, wl.head_dim), q.dtype, dev, compute_stream=compute,
                        staging=staging)
        copy_stream = zz.emu.copy if staging == "side" else None
        baseline_q = mine[1]

        def fold(timers, pool):
            zz.run_block(states[0], q, lambda j: kv[j], rank, wl.blocks, wl.causal, wl.scale,
                         step_timers=timers, timer_events=pool,
                         finalize_out=outs[0] if fused else None)

    outs = [(torch.empty((1, *st.o.shape[1:]), dtype=torch.float32, device=dev),
             torch.empty((1, *st.m.shape[1:]), dtype=torch.float32, device=dev)) for st in states]

    def one_ring(timers=None, pool=None):
        fold(timers, pool)
        if not fused:
            for st, (o_out, lse_out) in zip(states, outs):
                _lib.finalize(st, stream=compute, o_out=o_out, lse_out=lse_out)

    # Timing events for every launched step of the sampled timed rings,
    # created before the timed region.
    launched = sum(c != _lib.RA_CASE_SKIP for c in cases)
    pool = iter([Event(timing=True) for _ in range(2 * launched * timed_rings(args))])
    timers = []
    for _ in range(args.warmup):
        one_ring()
    torch.cuda.synchronize()
    graph, graph_note = (capture_ring(one_ring, copy_stream, compute, outs) if args.graph
                         else (None, "off (--no-graph)"))

    def untimed_ring():
        if graph is None:
            one_ring()
        else:
            with torch.cuda.stream(compute):
                graph.replay()

    for _ in range(args.warmup):
        untimed_ring()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in range(args.steps):
        if r % args.time_every == 0:
            one_ring(timers, pool)
        else:
            untimed_ring()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    ms = elapsed / args.steps * 1e3
    tflops = flops / (ms / 1e3) / 1e12

    full = [a.elapsed_time(b) for c, a, b in timers if c == _lib.RA_CASE_FULL]
    diag = [a.elapsed_time(b) for c, a, b in timers if c == _lib.RA_CASE_DIAG]
    if full and args.partition == "zigzag":
        # launches of unequal sizes: the full launches' FLOP over their time
        per = [(f, a.elapsed_time(b)) for (c, a, b), f in
               zip(timers, launch_flops * (len(timers) // len(launch_flops)))
               if c == _lib.RA_CASE_FULL]
        dom_ms = float(np.mean([t for _, t in per]))
        dom_flops = sum(f for f, _ in per) / len(per)
        dom = "ra_step full (zigzag row ranges, mean launch)"
    elif full:
        dom_ms, dom_flops, dom = float(np.mean(full)), full_step_flops(step_wl), "ra_step full"
    else:
        dom_ms = float(np.mean(diag))
        dom_flops = 4 * wl.head_dim * wl.heads * (step_wl.rows * (step_wl.rows + 1) // 2)
        dom = "ra_step diagonal"
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_VECTOR_TFLOPS
    achieved = dom_flops / (dom_ms / 1e3) / 1e12
    n_full, n_diag = cases.count(_lib.RA_CASE_FULL), cases.count(_lib.RA_CASE_DIAG)
    kernel_ms = n_full * (float(np.mean(full)) if full else 0.0) + \
        n_diag * (float(np.mean(diag)) if diag else 0.0)
    esize = 2 if wl.dtype == "bf16" else 4
    staged = (wl.blocks - 1) * 2 * wl.heads * wl.rows * wl.head_dim * esize

    line = {
        "metric": (f"{'causal' if wl.causal else 'non-causal'} {wl.dtype} ring-step attention "
                   f"TFLOP/s + % of MFMA peak (c={wl.rows}, d={wl.head_dim})"),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) blocks rounded to bf16, resident in HBM)",
        "config": {"workload": wl.name, "rank": rank, "partition": args.partition,
                   "fused_init_finalize": fused, "key_split": ks, "staging": staging,
                   "graph": graph_note,
                   "heads": wl.heads, "head_dim": wl.head_dim, "rows_per_block": wl.rows,
                   "blocks": wl.blocks, "causal": wl.causal, "tokens": wl.tokens,
                   "flop_per_step": flops,
                   "pct_of_mfma_peak": round(100 * tflops / peak, 2)},
        "roofline": {"bound": "mfma" if wl.dtype == "bf16" else "alu", "kernel": dom,
                     "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": (measured_traffic(wl) if full and args.partition == "contiguous"
                                 else None),
                     "avg_launch_ms": round(dom_ms, 5),
                     "launches": len(full) if full else len(diag),
                     "timed_rings": f"1 in {args.time_every} of the {args.steps} timed rings",
                     "diag_avg_launch_ms": round(float(np.mean(diag)), 5) if diag else None},
        "ring": {"cases": {"skip": cases.count(_lib.RA_CASE_SKIP), "diag": n_diag, "full": n_full},
                 "step_kernel_ms": round(kernel_ms, 5),
                 "exposed_ms": round(ms - kernel_ms, 5),
                 "exposed_note": "ring time minus the step kernels' event-timed average durations: "
                                 "launch gaps, cross-stream waits (side staging) and copies that "
                                 "overlap no step (skipped blocks) on the compute stream",
                 "bytes_staged": staged,
                 "staged_GBps": round(staged / (ms / 1e3) / 1e9, 1)},
        "counters": ({"full": measured_counters("full"), "diag": measured_counters("diag")}
                     if wl.name == DEFAULT_WORKLOAD and args.partition == "contiguous" else None),
        "env": software_versions(),
        "memory": device_memory(),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(step_wl, baseline_q, blocks)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
