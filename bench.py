"""Benchmark: one weighted block-sparse attention layer per step on one MI355X.

A step is the whole sparse pass -- bsa_score, bsa_select, bsa_attend, preceded
on a permuted sequence by bsa_permute_rows of K and V -- over a synthetic
clustered-token layer shaped like Wan2.1-T2V-14B at 720p (B=1, H=40,
N=75,600 -> 75,648, d=128, bf16, 128-token blocks, 20 exact + 40 sampled key
blocks per query block, ~10% density). Inputs are resident in HBM before the
timed region. The dense flash-attention kernel of the same library is timed
separately for the speedup.

Prints one JSON line. `value` is milliseconds per layer (lower is better),
warm: the timed steps run back to back. `cold` times each call on its own
after 512 MB of writes have evicted the caches; `plan_reuse` times one
score + select followed by r attend calls that reuse its lists; `ibcs` times
the intra-block clustering scorer in place of bsa_score, `stats` the
statistics-aware scorer.
`roofline` describes bsa_attend (bf16 MFMA bound), timed with HIP events on
the stream it runs on; `mfma_ceiling` is the rate a register-only MFMA loop
sustains on the same chip (below the top clock under a long matrix load), and
`attend_frac_of_ceiling` bsa_attend's rate against it; `mfma_ceiling_random`
and `attend_frac_of_random_ceiling` the same for the loop on operands that
change from one product to the next (bsa_mfma_ceiling_random: data that toggles
bits costs energy, and energy sets the clock at the power limit); with --power,
`power` gives the socket power (amd-smi) while bsa_attend, then both loops, run
back to back, and the energy per floating-point operation of each; `cpu_baseline` is the fp64 CPU oracle timed on a
bounded sample of the same workload on this host's cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
CSRC = os.path.join(ROOT, "block_sparse_attention_27_amd", "csrc")


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def attend_source_hash() -> str:
    """Hash of the attention kernel sources (the attend_* headers and units, in name order)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.startswith("attend_") and name.endswith((".hpp", ".hip")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _traffic(workload: str):
    """HBM bytes per bsa_attend launch from the committed counter summary, if it is current."""
    path = os.path.join(ROOT, "profiles", f"attend_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("attend_source_sha256_16") != attend_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def _socket_power_w():
    """Current socket power in watts from amd-smi (None when the tool or the field is missing)."""
    import re
    import shutil
    import subprocess
    tool = shutil.which("amd-smi") or ("/opt/rocm/bin/amd-smi" if os.path.exists("/opt/rocm/bin/amd-smi") else None)
    if tool is None:
        return None
    try:
        out = subprocess.run([tool, "metric", "-p", "-g", "0"], capture_output=True, text=True, timeout=10).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    m = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", out)
    return float(m.group(1)) if m else None


def power_under_load(torch, call, flop_per_call: float, seconds: float = 10.0) -> dict:
    """Socket power while `call` runs back to back for about `seconds` (median of samples taken from
    the middle of the run), the rate it sustains meanwhile, and the energy per floating-point operation."""
    import threading
    samples, stop = [], threading.Event()

    def sampler():
        time.sleep(min(3.0, seconds / 3))  # let the clock and power settle first
        while not stop.is_set():
            v = _socket_power_w()
            if v is not None:
                samples.append(v)
            time.sleep(0.5)

    call()
    torch.cuda.synchronize()
    th = threading.Thread(target=sampler)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0, n = time.perf_counter(), 0
    th.start()
    e0.record()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            call()
        n += 10
        torch.cuda.synchronize()
    e1.record()
    torch.cuda.synchronize()
    stop.set()
    th.join()
    ms = e0.elapsed_time(e1) / n
    tf = flop_per_call / (ms * 1e-3) / 1e12
    w = statistics.median(samples) if samples else None
    return {"watts": w, "samples": len(samples), "ms_per_call": round(ms, 3), "tflops": round(tf, 1),
            "pj_per_flop": None if w is None else round(w / (tf * 1e12) * 1e12, 3)}


def power_report(bsa, torch, attend_call, exec_flops: float) -> dict:
    """Idle socket power, then bsa_attend and both MFMA loops each run back to back with power sampled.

    The idle figure is the lowest of samples taken over 4 s with the GPU idle: the reading averages over a
    window, so one taken right after a load still carries it."""
    torch.cuda.synchronize()
    idle_samples = []
    for _ in range(8):
        time.sleep(0.5)
        v = _socket_power_w()
        if v is not None:
            idle_samples.append(v)
    idle = min(idle_samples) if idle_samples else None
    att = power_under_load(torch, attend_call, exec_flops)
    cout = torch.empty(512 * 256, dtype=torch.float32, device="cuda")
    ceil = power_under_load(torch, lambda: bsa.bsa_mfma_ceiling(cout, 40000, 512),
                            512 * 4 * 40000 * bsa.MFMA_CEILING_FLOP)
    ceil_r = power_under_load(torch, lambda: bsa.bsa_mfma_ceiling_random(cout, 40000, 512),
                              512 * 4 * 40000 * bsa.MFMA_CEILING_FLOP)
    return {"idle_watts": idle, "bsa_attend": att, "mfma_ceiling": ceil, "mfma_ceiling_random": ceil_r}


def cpu_baseline(w, g, budget_s: float = 20.0):
    """Time the oracle on a bounded sample and scale it to one layer (ms/layer)."""
    import numpy as np
    import oracle
    from block_sparse_attention_27_amd.inputs import as_float32
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    h = 0
    q = as_float32(g["q"][:, h:h + 1]).astype(np.float64)
    k = as_float32(g["k"][:, h:h + 1]).astype(np.float64)
    v = as_float32(g["v"][:, h:h + 1]).astype(np.float64)
    t0 = time.perf_counter()
    S, _, _ = oracle.score(q, k, w.N, w.block_q, w.block_k, w.sm_scale, g["perm"])
    t_score_head = time.perf_counter() - t0
    # selection: query blocks of head 0 in a spread order, for up to a quarter of the budget
    order = list(range(0, w.n_qblocks, 7)) + [i for i in range(w.n_qblocks) if i % 7]
    idx = np.zeros((1, 1, w.n_qblocks, w.list_len), np.int32)
    wt = np.ones((1, 1, w.n_qblocks, w.list_len), np.float32)
    t0 = time.perf_counter()
    rows = []
    for i in order:
        (ri, rw), = oracle.select(S, w.N, w.block_k, w.k_exact, w.m_sample, w.select_seed, rows=[(0, 0, i)])
        idx[0, 0, i], wt[0, 0, i] = ri, rw
        rows.append(i)
        if time.perf_counter() - t0 > budget_s / 4:
            break
    t_select_row = (time.perf_counter() - t0) / len(rows)
    # attention: the same query blocks, for the rest of the budget
    t0 = time.perf_counter()
    done = 0
    for i in rows:
        oracle.attend(q, k, v, w.N, w.block_q, w.block_k, w.sm_scale, idx, wt, g["perm"], blocks=[(0, 0, i)])
        done += 1
        if time.perf_counter() - t0 > budget_s * 3 / 4:
            break
    t_attend_block = (time.perf_counter() - t0) / done
    n_rows_total = w.B * w.H * w.n_qblocks
    ms = 1e3 * (t_score_head * w.B * w.H + (t_select_row + t_attend_block) * n_rows_total)
    sample = (f"head 0 of {w.H}: full score; select on {len(rows)} of {w.n_qblocks} query blocks; "
              f"attend on {done} query blocks; scaled by (b,h) and query-block counts to the whole layer")
    return {"value": round(ms, 1), "unit": "ms/layer", "cores": int(cores), "kind": "oracle",
            "sample": sample,
            "parts_s": {"score_per_head": round(t_score_head, 4), "select_per_block": round(t_select_row, 5),
                        "attend_per_block": round(t_attend_block, 5)}}


def mfma_ceiling(bsa, torch, iters: int = 40000, n_wg: int = 512, reps: int = 5, random: bool = False) -> dict:
    """Sustained bf16 MFMA rate of this chip: bsa_mfma_ceiling, 2 workgroups per CU, ~10 ms per launch.

    Under a long matrix load the clock stays well below the top clock (the chip
    runs at or near its power limit), so this register-only loop is the
    ceiling any matrix-bound kernel meets here. random=True times
    bsa_mfma_ceiling_random, whose operands change from one product to the
    next as real data does (iters must then be a multiple of 4).
    """
    stream = torch.cuda.current_stream()
    out = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")
    probe = bsa.bsa_mfma_ceiling_random if random else bsa.bsa_mfma_ceiling
    for _ in range(2):
        probe(out, iters, n_wg)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for e in ev:
        e[0].record(stream)
        probe(out, iters, n_wg)
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = statistics.mean(e[0].elapsed_time(e[1]) for e in ev)
    flop = n_wg * 4 * iters * bsa.MFMA_CEILING_FLOP
    tf = flop / (ms * 1e-3) / 1e12
    return {"tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4), "ms_per_launch": round(ms, 3),
            "kernel": f"{'bsa_mfma_ceiling_random' if random else 'bsa_mfma_ceiling'}: {n_wg} workgroups of 4 waves, "
                      f"{iters} rounds of 8 register-only v_mfma_f32_32x32x16_bf16 per wave"
                      + (" on operands that change from one product to the next" if random else
                         " on constant operands")}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="wan14b_720p")
    ap.add_argument("--seed", type=int, default=None, help="generator seed of the synthetic inputs (preset: 0)")
    ap.add_argument("--select-seed", type=int, default=None, help="Philox key of the selection (preset: 0)")
    ap.add_argument("--temperature", type=float, default=None,
                    help="logit temperature, sm_scale = 1 / temperature (preset: the config's)")
    ap.add_argument("--heads", type=int, default=None, help="number of heads H (preset: the config's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the sustained-MFMA-rate measurement")
    ap.add_argument("--ceiling-only", action="store_true",
                    help="only measure the sustained MFMA rate (bsa_mfma_ceiling) and print it")
    ap.add_argument("--power", action="store_true",
                    help="also sample socket power (amd-smi) under bsa_attend and under bsa_mfma_ceiling")
    ap.add_argument("--power-only", action="store_true",
                    help="only the power samples: bsa_attend on the config's lists, then bsa_mfma_ceiling")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU: this path has no multi-GPU mode (--gpus {args.gpus} asked). "
              "Heads shard across GPUs with no communication; run one process per GPU instead.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import block_sparse_attention_27_amd as bsa
    from block_sparse_attention_27_amd.inputs import WORKLOADS, generate

    if args.ceiling_only:
        print(json.dumps({"mfma_ceiling": mfma_ceiling(bsa, torch),
                          "mfma_ceiling_random": mfma_ceiling(bsa, torch, random=True)}), flush=True)
        return 0

    w = WORKLOADS[args.config]
    overrides = {name: val for name, val in (("seed", args.seed), ("select_seed", args.select_seed),
                                             ("temperature", args.temperature), ("H", args.heads))
                 if val is not None}
    if overrides:
        w = w.replace(**overrides)
    _log(f"generating {w.name} inputs")
    g = generate(w)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    q, k, v = dev(g["q"]), dev(g["k"]), dev(g["v"])
    perm = torch.from_numpy(g["perm"]).cuda() if g["perm"] is not None else None
    p = bsa.problem_for(w, out_fp32=1)   # the parity-checked variant: fp32 output
    p16 = bsa.problem_for(w)             # same kernel, bf16 output (RNE of the fp32 result)
    S = torch.empty((w.B, w.H, w.n_qblocks, w.n_units), dtype=torch.float32, device="cuda")
    qm = torch.empty((w.B, w.H, w.n_qblocks, w.d), dtype=torch.float32, device="cuda")
    km = torch.empty((w.B, w.H, w.n_units, w.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.B, w.H, w.n_qblocks, w.list_len), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.B, w.H, w.n_qblocks, w.list_len), dtype=torch.float32, device="cuda")
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    # A permuted sequence: K and V are put into the permuted order once per
    # pass (bsa_permute_rows) and the steps run with kv_permuted = 1, so the
    # attention pass reads every key unit as contiguous rows; Q is gathered and
    # out scattered inside the kernels.
    if perm is not None:
        kk, vv = torch.empty_like(k), torch.empty_like(v)
        pp, pp16 = bsa.with_kv_permuted(p), bsa.with_kv_permuted(p16)
    else:
        kk, vv, pp, pp16 = k, v, p, p16

    def permute():
        if perm is not None:
            bsa.bsa_permute_rows(p, k, perm, kk)
            bsa.bsa_permute_rows(p, v, perm, vv)

    def step(ev=None):
        if ev: ev[0].record(stream)
        permute()
        if ev: ev[4].record(stream)
        bsa.bsa_score(pp, q, kk, perm, S, qm, km)
        if ev: ev[1].record(stream)
        bsa.bsa_select(pp, S, idx, wt)
        if ev: ev[2].record(stream)
        bsa.bsa_attend(pp, q, kk, vv, perm, idx, wt, out, None)
        if ev: ev[3].record(stream)

    _log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def attend_call():
        bsa.bsa_attend(pp, q, kk, vv, perm, idx, wt, out, None)

    if args.power_only:
        _log("sampling socket power under bsa_attend, then under both MFMA loops")
        print(json.dumps({"config": w.name, "power": power_report(bsa, torch, attend_call, w.executed_flops())}),
              flush=True)
        return 0

    _log(f"timing {args.steps} steps")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    t_permute = statistics.mean(e[0].elapsed_time(e[4]) for e in evs)
    t_score = statistics.mean(e[4].elapsed_time(e[1]) for e in evs)
    t_select = statistics.mean(e[1].elapsed_time(e[2]) for e in evs)
    t_attend = statistics.mean(e[2].elapsed_time(e[3]) for e in evs)
    t_pass = statistics.mean(e[0].elapsed_time(e[3]) for e in evs)

    # cold caches: 512 MB written before every call evicts L2 and the 256 MB
    # Infinity Cache; each call is timed on its own
    n_cold = max(3, min(args.steps, 5))
    flush = torch.empty(1 << 27, dtype=torch.float32, device="cuda")
    cold = {"permute": [], "score": [], "select": [], "attend": []}
    calls = (("permute", permute),
             ("score", lambda: bsa.bsa_score(pp, q, kk, perm, S, qm, km)),
             ("select", lambda: bsa.bsa_select(pp, S, idx, wt)),
             ("attend", lambda: bsa.bsa_attend(pp, q, kk, vv, perm, idx, wt, out, None)))
    for _ in range(n_cold):
        for name, call in calls:
            flush.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            cold[name].append((e0, e1))
    torch.cuda.synchronize()
    t_cold = {n: statistics.median(a.elapsed_time(b) for a, b in ev) for n, ev in cold.items()}
    del flush

    # sampling-plan reuse: one score + select, then r attend calls with that plan
    # (each on its own step's K and V, so a permuted sequence permutes them each time)
    reuse_r = 4
    re = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    re[0].record(stream)
    permute()
    bsa.bsa_score(pp, q, kk, perm, S, qm, km)
    bsa.bsa_select(pp, S, idx, wt)
    for i in range(reuse_r):
        if i:
            permute()
        bsa.bsa_attend(pp, q, kk, vv, perm, idx, wt, out, None)
    re[1].record(stream)
    torch.cuda.synchronize()
    t_reuse = re[0].elapsed_time(re[1]) / reuse_r

    # intra-block clustering scorer (4 groups, 3 k-means iterations) in place of bsa_score
    ib_g, ib_t = 4, 3
    qc = torch.empty((w.B, w.H, w.n_qblocks, ib_g, w.d), dtype=torch.float32, device="cuda")
    qs = torch.empty((w.B, w.H, w.n_qblocks, ib_g), dtype=torch.int32, device="cuda")
    for _ in range(2):
        bsa.bsa_score_ibcs(pp, ib_g, ib_t, q, kk, perm, S, qc, qs, km)
    ie = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(max(3, min(args.steps, 10)))]
    for e in ie:
        e[0].record(stream)
        bsa.bsa_score_ibcs(pp, ib_g, ib_t, q, kk, perm, S, qc, qs, km)
        e[1].record(stream)
    torch.cuda.synchronize()
    t_ibcs = statistics.mean(e[0].elapsed_time(e[1]) for e in ie)
    del qc, qs

    # statistics-aware scorer (key-unit variances) in place of bsa_score
    kv = torch.empty_like(km)
    for _ in range(2):
        bsa.bsa_score_stats(pp, q, kk, perm, S, qm, km, kv)
    se = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(max(3, min(args.steps, 10)))]
    for e in se:
        e[0].record(stream)
        bsa.bsa_score_stats(pp, q, kk, perm, S, qm, km, kv)
        e[1].record(stream)
    torch.cuda.synchronize()
    t_stats = statistics.mean(e[0].elapsed_time(e[1]) for e in se)
    del kv

    # bsa_attend with a bf16 output, same lists
    out16 = torch.empty_like(q)
    be = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(max(3, min(args.steps, 10)))]
    for e in be:
        e[0].record(stream)
        bsa.bsa_attend(pp16, q, kk, vv, perm, idx, wt, out16, None)
        e[1].record(stream)
    torch.cuda.synchronize()
    t_attend16 = statistics.mean(e[0].elapsed_time(e[1]) for e in be)
    del out16

    # the same lists with K and V gathered inside the attention pass (kv_permuted = 0)
    t_attend_gather = None
    if perm is not None:
        ge = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(max(3, min(args.steps, 10)))]
        bsa.bsa_attend(p, q, k, v, perm, idx, wt, out, None)
        for e in ge:
            e[0].record(stream)
            bsa.bsa_attend(p, q, k, v, perm, idx, wt, out, None)
            e[1].record(stream)
        torch.cuda.synchronize()
        t_attend_gather = statistics.mean(e[0].elapsed_time(e[1]) for e in ge)

    t_dense = None
    if not args.no_dense:
        _log("timing the dense kernel")
        outd = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        for _ in range(2):
            bsa.bsa_attend_dense(p, q, k, v, perm, outd, None)
        n_dense = max(3, min(args.steps, 10))
        de = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_dense)]
        for e in de:
            e[0].record(stream)
            bsa.bsa_attend_dense(p, q, k, v, perm, outd, None)
            e[1].record(stream)
        torch.cuda.synchronize()
        t_dense = statistics.mean(e[0].elapsed_time(e[1]) for e in de)
        del outd

    exec_flops = w.executed_flops()
    dense_flops = w.dense_flops()
    ach = exec_flops / (t_attend * 1e-3) / 1e12
    elem = 2 if w.dtype == "bf16" else 4
    score_bytes = 2 * w.B * w.H * w.N * w.d * elem + 4 * w.B * w.H * w.n_qblocks * w.n_units
    select_bytes = 4 * w.B * w.H * w.n_qblocks * (w.n_valid_units + 2 * w.list_len)

    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    power = None
    if args.power:
        _log("sampling socket power under bsa_attend, then under both MFMA loops")
        power = power_report(bsa, torch, attend_call, exec_flops)

    ceiling = ceiling_r = None
    if not args.no_ceiling:
        _log("measuring the sustained MFMA rate")
        ceiling = mfma_ceiling(bsa, torch)
        ceiling_r = mfma_ceiling(bsa, torch, random=True)

    cpu = None
    if not args.no_cpu_baseline:
        _log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(w, g)

    rec = {
        "metric": "sparse-attn ms/layer + executed MFMA TFLOP/s (% peak), Wan-14B shape, 10% density",
        "value": round(t_pass, 4),
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic clustered tokens (seeded), inputs resident in HBM",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "N_pad": w.N_pad, "d": w.d,
                   "block_q": w.block_q, "block_k": w.block_k, "k_exact": w.k_exact,
                   "m_sample": w.m_sample, "density": round(w.density, 4), "temperature": w.temperature,
                   "permuted": w.permute, "seed": w.seed, "select_seed": w.select_seed,
                   "parallelism": "single GPU"},
        "device": {"name": torch.cuda.get_device_name(0), "hip": torch.version.hip,
                   "arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", None)},
        "t_permute_ms": round(t_permute, 4) if perm is not None else None,
        "t_score_ms": round(t_score, 4),
        "t_select_ms": round(t_select, 4),
        "t_attend_ms": round(t_attend, 4),
        "t_attend_bf16_out_ms": round(t_attend16, 4),
        "t_attend_gather_inside_ms": None if t_attend_gather is None else round(t_attend_gather, 4),
        "t_dense_ms": None if t_dense is None else round(t_dense, 4),
        "score_select_share": round((t_score + t_select) / t_pass, 4),
        "cold": {"t_permute_ms": round(t_cold["permute"], 4) if perm is not None else None,
                 "t_score_ms": round(t_cold["score"], 4), "t_select_ms": round(t_cold["select"], 4),
                 "t_attend_ms": round(t_cold["attend"], 4),
                 "t_pass_ms": round(sum(t_cold.values()), 4), "calls": n_cold,
                 "flush": "512 MB written before every call"},
        "ibcs": {"groups": ib_g, "iters": ib_t, "t_score_ms": round(t_ibcs, 4),
                 "score_select_share": round((t_ibcs + t_select) / (t_ibcs + t_select + t_attend), 4)},
        "stats": {"t_score_ms": round(t_stats, 4),
                  "score_select_share": round((t_stats + t_select) / (t_stats + t_select + t_attend), 4)},
        "plan_reuse": {"r": reuse_r, "ms_per_layer": round(t_reuse, 4),
                       "score_select_share": round((t_score + t_select) / reuse_r / t_reuse, 4)},
        "executed_tflops": round(ach, 1),
        "executed_frac_peak": round(ach / PEAK_BF16_TFLOPS, 4),
        "dense_equiv_tflops": round(dense_flops / (t_pass * 1e-3) / 1e12, 1),
        "dense_equiv_frac_peak": round(dense_flops / (t_pass * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "dense_kernel_tflops": None if t_dense is None else round(dense_flops / (t_dense * 1e-3) / 1e12, 1),
        "speedup_vs_dense": None if t_dense is None else round(t_dense / t_pass, 3),
        "speedup_attend_vs_dense": None if t_dense is None else round(t_dense / t_attend, 3),
        "score_hbm_gbs": round(score_bytes / (t_score * 1e-3) / 1e9, 1),
        "select_hbm_gbs": round(select_bytes / (t_select * 1e-3) / 1e9, 1),
        "mfma_ceiling": ceiling,
        "power": power,
        "attend_frac_of_ceiling": None if ceiling is None else round(ach / ceiling["tflops"], 4),
        "mfma_ceiling_random": ceiling_r,
        "attend_frac_of_random_ceiling": None if ceiling_r is None else round(ach / ceiling_r["tflops"], 4),
        "roofline": {"kernel": "bsa_attend", "bound": "mfma", "achieved": round(ach, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                     "traffic": None if overrides else _traffic(w.name)},  # counters were taken on the preset
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
