"""Benchmark of the serial Markov draft walk on one MI355X.

One "step" of this benchmark is one round of the walk: one dsw_walk call over
one seeded synthetic round (base logits, anchor, temperatures, uniforms) of
the chosen workload.  Default: vocabulary 151,936, r = 256, gamma = 7, one
greedy request (the Qwen3-size configuration), 1000 distinct seeded rounds
resident in HBM before timing starts.

Prints ONE JSON line.  `value` is microseconds per round over K back-to-back
rounds, bracketed by device synchronisation (lower is better).  Extra fields:
per-launch kernel time from HIP events (the roofline's denominator), a
cold-cache leg (L2 and the 256 MB Infinity Cache flushed before each round),
gamma = 16 at the same vocabulary, the step-wise torch loop (the pages'
default walk: gamma x {GEMV, add, argmax}), a short timing of every other
checked configuration (more requests, gamma = 16, V = 248,320 in bf16 and
int8, the batched kernel up to 253 requests) and the CPU oracle on a bounded
sample of the same rounds.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "serial_draft_head_amd", "csrc")
COPY_BYTES = 256 << 20  # known-size copy that calibrates the HBM byte counters


def kernel_source_hash():
    """Hash of the HIP/C++ sources: counter records are valid only for these."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload_name, B, gamma, cold=False):
    """HBM bytes per launch from the committed counter record (warm, or with L2
    and the Infinity Cache flushed before each launch), if it was taken on the
    current kernel sources; else None."""
    path = os.path.join(PROFILES, f"counters_{workload_name}_b{B}_g{gamma}{'_cold' if cold else ''}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


READ_COUNTERS = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_BUBBLE_sum")
WRITE_COUNTERS = ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum")


def summarize_counters(outdir, workload_name, V, B, gamma, cold, dest_dir=PROFILES):
    """The counter record of one workload from rocprofv3 --pmc CSV output
    under `outdir` (any number of runs of --pmc-mode, each with some of
    READ_COUNTERS / WRITE_COUNTERS): per-dispatch means for the walk kernel
    and for the 256 MiB calibration copy, and the bytes they stand for.

    L2-to-fabric requests: reads of 32 B (RDREQ_32B), 128 B (BUBBLE) and
    64 B (the rest); writes of 64 B (WRREQ_64B) and 32 B (the rest).  Each
    direction is scaled by what the same sum reads for the copy of known
    size.  With L2 and the Infinity Cache flushed before each launch these
    are HBM bytes; warm they count L2 misses, some of which the Infinity
    Cache serves."""
    import csv
    import glob
    walk_names, w_vals, cp = set(), {}, {}  # walk: counter -> [per dispatch]; copy: counter -> value
    for path in glob.glob(os.path.join(outdir, "**", "*counter_collection.csv"), recursive=True):
        disp = {}  # dispatch id -> (kernel, {counter: value summed over rows})
        with open(path) as f:
            for row in csv.DictReader(f):
                d = disp.setdefault(int(row["Dispatch_Id"]), (row["Kernel_Name"], {}))[1]
                d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
        for kname, d in disp.values():
            if "dsw::walk_" in kname:
                walk_names.add(kname)
                for c, v in d.items():
                    w_vals.setdefault(c, []).append(v)
        # the calibration copy: the last copy dispatch of real size in this run
        # (earlier ones upload the inputs, a later tiny one reads the status back)
        big = [i for i, (kname, d) in disp.items()
               if "copy" in kname.lower() and "dsw::" not in kname and sum(d.values()) > 10_000]
        if big:
            cp.update(disp[max(big)][1])
    if len(walk_names) != 1 or not cp:
        raise SystemExit(f"expected one walk kernel and the calibration copy, found {sorted(walk_names)}")
    w = {c: sum(v) / len(v) for c, v in w_vals.items()}

    def rd(m):
        if not all(c in m for c in READ_COUNTERS):
            return None
        req, r32, r128 = (m[c] for c in READ_COUNTERS)
        return r32 * 32 + r128 * 128 + (req - r32 - r128) * 64

    def wr(m):
        if not all(c in m for c in WRITE_COUNTERS):
            return None
        req, w64 = (m[c] for c in WRITE_COUNTERS)
        return w64 * 64 + (req - w64) * 32

    rec = {"kernel": walk_names.pop(), "workload": workload_name, "B": B, "gamma": gamma, "cold": bool(cold),
           "kernel_source_hash": kernel_source_hash(), "dispatches": {c: len(v) for c, v in w_vals.items()},
           "walk_counters_per_dispatch": {c: round(v, 1) for c, v in sorted(w.items())},
           "copy_bytes": COPY_BYTES,
           "copy_counters": {c: round(v, 1) for c, v in sorted(cp.items())},
           "algorithmic_bytes_per_launch": algorithmic_bytes(V, B, gamma)}
    total = 0.0
    for name, f in (("read", rd), ("write", wr)):
        raw, ref = f(w), f(cp)
        if raw is None or not ref:
            rec[name + "_bytes_per_launch"] = None
            continue
        scale = COPY_BYTES / ref
        rec[name + "_bytes_raw"] = round(raw)
        rec[name + "_scale"] = round(scale, 4)
        rec[name + "_bytes_per_launch"] = round(raw * scale)
        total += raw * scale
    if rec["read_bytes_per_launch"] is not None and rec["write_bytes_per_launch"] is not None:
        rec["hbm_bytes_per_launch"] = round(total)
    path = os.path.join(dest_dir, f"counters_{workload_name}_b{B}_g{gamma}{'_cold' if cold else ''}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def algorithmic_bytes(V, B, gamma, want_logits=False, r=256):
    """Bytes one round must move at minimum: W2 once, base, the gathered W1
    rows, tokens, anchors, temperatures and uniforms (+ logits if written)."""
    n = V * r * 2 + B * gamma * V * 2 + B * gamma * r * 2 + B * gamma * 4 + B * 8 + B * gamma * 4
    if want_logits:
        n += B * gamma * V * 2
    return n


def make_rounds(index, n, B, gamma, V, temps):
    import workloads
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        return list(ex.map(lambda r: workloads.round_inputs(index, r, B=B, gamma=gamma, V=V,
                                                            temps=temps), range(n)))


def to_device(rounds, torch, dev):
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)  # noqa: E731
    base = torch.stack([bf(r["base"]) for r in rounds]).to(dev)
    anchor = torch.stack([torch.from_numpy(r["anchor"]) for r in rounds]).to(dev)
    T = torch.stack([torch.from_numpy(r["T"]) for r in rounds]).to(dev)
    uni = torch.stack([torch.from_numpy(r["uniforms"]) for r in rounds]).to(dev)
    return base, anchor, T, uni


def time_walk(torch, walker, W1d, W2d, dev_rounds, K, W, per_launch=False, flush=None):
    base, anchor, T, uni = dev_rounds
    n = base.shape[0]
    B, gamma = base.shape[1], base.shape[2]
    tokens = torch.empty((B, gamma), dtype=torch.int32, device=W1d.device)
    for i in range(W):
        j = i % n
        walker.walk(W1d, W2d, base[j], anchor[j], T[j], uni[j], tokens=tokens)
    torch.cuda.synchronize()
    if not per_launch and flush is None:
        t0 = time.perf_counter()
        for i in range(K):
            j = (W + i) % n
            walker.walk(W1d, W2d, base[j], anchor[j], T[j], uni[j], tokens=tokens)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / K * 1e6, None
    if flush is None:
        # one event pair on the launch stream around K back-to-back launches:
        # the mean launch duration without an event between launches
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(K):
            j = (W + i) % n
            walker.walk(W1d, W2d, base[j], anchor[j], T[j], uni[j], tokens=tokens)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / K, None
    durs = []
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for i in range(K):
        j = (W + i) % n
        if flush is not None:
            flush()
        ev[i][0].record()
        walker.walk(W1d, W2d, base[j], anchor[j], T[j], uni[j], tokens=tokens)
        ev[i][1].record()
    torch.cuda.synchronize()
    durs = [a.elapsed_time(b) * 1e3 for a, b in ev]
    return statistics.fmean(durs), durs


def stepwise_torch(torch, W1d, W2d, dev_rounds, K):
    """The pages' default walk as separate library ops per step (re-reads W2 every step)."""
    base, anchor, T, uni = dev_rounds
    n, B, gamma, V = base.shape

    def one(j):
        prev = anchor[j].long()
        out = []
        for k in range(gamma):
            u = W1d[prev]                                  # [B, 256]
            bias = torch.matmul(u, W2d.t())                # bf16 out: rounded once
            logit = base[j][:, k] + bias                   # bf16 add: rounded again
            prev = torch.argmax(logit, dim=-1)
            out.append(prev)
        return out

    for j in range(3):
        one(j)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        one(i % n)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / K * 1e6


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(index, B, gamma, V, W1, W2, n_rounds=1000, budget_s=30.0, one_thread_s=10.0):
    """The oracle as it stands, on the host cores: the same seeded rounds as
    the workload (all n_rounds of them unless the budget runs out first),
    median wall time per round with every OpenMP thread, then a shorter
    sample with one thread."""
    import oracle
    import workloads

    def timed(limit_s, max_rounds):
        times = []
        t_start = time.perf_counter()
        r = 0
        while r < max_rounds:
            inp = workloads.round_inputs(index, r, B=B, gamma=gamma, V=V)
            t0 = time.perf_counter()
            oracle.walk(W1, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], W2_bits=W2,
                        want_logits=False)
            times.append(time.perf_counter() - t0)
            r += 1
            if time.perf_counter() - t_start > limit_s:
                break
        return times

    n_threads = oracle.threads()
    times = timed(budget_s, n_rounds)
    oracle.set_threads(1)
    try:
        one = timed(one_thread_s, n_rounds)
    finally:
        oracle.set_threads(n_threads)
    return {"value": statistics.median(times) * 1e6, "unit": "us/round", "cores": n_threads,
            "kind": "oracle", "cpu_model": cpu_model(), "rounds": len(times),
            "one_thread_us": statistics.median(one) * 1e6, "one_thread_rounds": len(one),
            "sample": f"{len(times)} of the workload's {n_rounds} seeded rounds (rounds 0..{len(times) - 1}) with "
                      f"{n_threads} OpenMP threads, then rounds 0..{len(one) - 1} with one thread; median wall "
                      f"time per round of the binary64 C oracle"}


MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix peak, published


def gamma_sweep(torch, dsw, W1d, W2d, V, gammas=(1, 4, 7, 10, 16), rounds=60, K=200):
    """Walk time against gamma, fitted as t = entry + gamma * step by least
    squares, once with the shard resident and once with nothing on chip
    (DSW_FLAG_FORCE_STREAM: W2 re-read every step inside the one launch).
    The resident entry is the one-time shard load; the difference between the
    two per-step costs is what residency saves on each step."""
    out = {}
    for name, flags in (("resident", 0), ("streamed", dsw.FLAG_FORCE_STREAM)):
        walker = dsw.Walker(V, gamma_max=max(gammas), B_max=1, flags=flags)
        pts = []
        for g in gammas:
            d = to_device(make_rounds(1, rounds, 1, g, V, "greedy"), torch, W1d.device)
            us, _ = time_walk(torch, walker, W1d, W2d, d, K, 10)
            pts.append((g, us))
            del d
        st = walker.status()
        walker.close()
        x = np.array([p[0] for p in pts], dtype=np.float64)
        y = np.array([p[1] for p in pts], dtype=np.float64)
        step, entry = np.polyfit(x, y, 1)
        out[name] = {"us_per_round": {int(g): round(u, 2) for g, u in pts},
                     "entry_us": round(float(entry), 2), "us_per_step": round(float(step), 3),
                     "status": st}
    return out

def cold_gamma_sweep(torch, dsw, W1d, W2d, V, flush, gammas=(1, 4, 7, 10, 16), rounds=30):
    """The resident walk with L2 and the Infinity Cache flushed before each
    round (outside the events), against gamma, fitted as entry + gamma * step:
    the entry is then the shard load from HBM."""
    walker = dsw.Walker(V, gamma_max=max(gammas), B_max=1)
    try:
        pts = []
        for g in gammas:
            d = to_device(make_rounds(1, rounds, 1, g, V, "greedy"), torch, W1d.device)
            mean, durs = time_walk(torch, walker, W1d, W2d, d, rounds, 2, flush=flush)
            pts.append((g, statistics.median(durs)))
            del d
        st = walker.status()
    finally:
        walker.close()
    x = np.array([p[0] for p in pts], dtype=np.float64)
    y = np.array([p[1] for p in pts], dtype=np.float64)
    step, entry = np.polyfit(x, y, 1)
    return {"us_per_round_median": {int(g): round(u, 2) for g, u in pts}, "entry_us": round(float(entry), 2),
            "us_per_step": round(float(step), 3), "status": st}


def grid_sweep(torch, dsw, grids=(8, 16, 32, 64, 128, 256), rounds=20, K=200):
    """The rendezvous against the number of workgroups (dsw_set_grid): at
    V = 2,048 (shards of 8 to 256 rows, so that the GEMV stays small) the
    per-step cost of a greedy walk, fitted over gamma in {1, 9, 17}, is the
    exchange, the gather and a few MFMA tiles; then the V = 32,000 walk
    (gamma = 7) at the grids whose shards fit on chip."""
    import workloads
    dev = torch.device("cuda", 0)
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    out = {"exchange_v2048": {}, "toy_v32000_g7": {}}
    V = 2048
    W1, W2 = workloads.weights(0, V=V)
    W1d, W2d = bf(W1), bf(W2)
    for G in grids:
        walker = dsw.Walker(V, gamma_max=17, B_max=1)
        try:
            walker.set_grid(G)
            pts = []
            for g in (1, 9, 17):
                d = to_device(make_rounds(0, rounds, 1, g, V, "greedy"), torch, dev)
                us, _ = time_walk(torch, walker, W1d, W2d, d, K, 10)
                pts.append((g, us))
            st = walker.status()
        finally:
            walker.close()
        step, entry = np.polyfit([p[0] for p in pts], [p[1] for p in pts], 1)
        out["exchange_v2048"][G] = {"us_per_round": {g: round(u, 2) for g, u in pts},
                                    "us_per_step": round(float(step), 3), "entry_us": round(float(entry), 2),
                                    "status": st}
        log("grid", G, out["exchange_v2048"][G])
    V = 32_000
    W1, W2 = workloads.weights(0, V=V)
    W1d, W2d = bf(W1), bf(W2)
    d = to_device(make_rounds(0, rounds, 1, 7, V, "greedy"), torch, dev)
    for G in grids:
        if -(-V // G) > 1024:  # more rows than the compiled shapes hold on chip
            continue
        walker = dsw.Walker(V, gamma_max=7, B_max=1)
        try:
            walker.set_grid(G)
            us, _ = time_walk(torch, walker, W1d, W2d, d, K, 10)
            out["toy_v32000_g7"][G] = {"us_per_round": round(us, 2), "status": walker.status(),
                                       "plan": {k: v for k, v in walker.query_plan(1).as_dict().items()
                                                if k in ("rows_per_wg", "reg_tiles", "max_tiles", "lds_tiles")}}
        finally:
            walker.close()
        log("toy grid", G, out["toy_v32000_g7"][G])
    return out


# Every configuration the walk is checked on, timed briefly after the headline
# line's own measurements: (workload, requests, gamma, W2 storage).
SWEEP = [(0, 1, 7, "bf16"), (2, 1, 16, "bf16"), (2, 4, 16, "bf16"), (2, 16, 16, "bf16"),
         (3, 1, 16, "bf16"), (3, 1, 16, "int8"), (4, 64, 5, "bf16"), (4, 64, 5, "int8"), (4, 128, 5, "bf16"),
         (4, 253, 5, "bf16"),
         # the mixed-temperature walks again, sampled by Gumbel-max (DSW_FLAG_GUMBEL)
         (2, 1, 16, "bf16", "gumbel"), (2, 4, 16, "bf16", "gumbel"), (2, 16, 16, "bf16", "gumbel"),
         # the GRU serial head (DSW_FLAG_GRU) on the headline and the long walk
         (1, 1, 7, "bf16", "inverse_cdf", "gru"), (2, 1, 16, "bf16", "inverse_cdf", "gru"),
         (1, 1, 7, "bf16", "inverse_cdf", "rnn"),
         # DSpark's gated head (DSW_FLAG_GATED) on the headline and the long walk
         (1, 1, 7, "bf16", "inverse_cdf", "gated"), (2, 1, 16, "bf16", "inverse_cdf", "gated"),
         # Domino's head (DSW_FLAG_DOMINO; hidden width 2560) on the headline and the long walk
         (1, 1, 7, "bf16", "inverse_cdf", "domino"), (2, 1, 16, "bf16", "inverse_cdf", "domino"),
         # one GPU's share of a two-GPU vocabulary split (the kernel at its real shape;
         # the cross-GPU exchange is not built): half of V = 151,936 and of V = 248,320
         (1, 1, 7, "bf16", "inverse_cdf", "markov", 75_968), (3, 1, 16, "bf16", "inverse_cdf", "markov", 124_160)]


def sweep_one(torch, dsw, index, B, gamma, dtype, sampler="inverse_cdf", head="markov", V=None):
    import workloads
    wl = workloads.WORKLOADS[index]
    V = wl.V if V is None else V
    dev = torch.device("cuda", 0)
    W1, W2 = workloads.weights(index, V=V)
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    W1d = bf(W1)
    scale = None
    if dtype == "int8":
        Q, sc = workloads.quantize_int8(W2)
        W2d = torch.from_numpy(Q).to(dev)
        scale = torch.from_numpy(sc).to(dev)
        w2_bytes = V * 256 + V * 4
    else:
        W2d = bf(W2)
        w2_bytes = V * 256 * 2
    big = B * gamma * V > 50_000_000
    rounds = make_rounds(index, 3 if big else 8, B, gamma, V, wl.temps)
    base, anchor, T, uni = to_device(rounds, torch, dev)
    del rounds
    walker = dsw.Walker(V, gamma_max=gamma, B_max=B, w2_dtype=dsw.INT8 if dtype == "int8" else dsw.BF16,
                        flags=(dsw.FLAG_GUMBEL if sampler == "gumbel" else 0) |
                              (dsw.FLAG_GRU if head == "gru" else 0) | (dsw.FLAG_RNN if head == "rnn" else 0) |
                              (dsw.FLAG_GATED if head == "gated" else 0) |
                              (dsw.FLAG_DOMINO if head == "domino" else 0))
    if sampler == "gumbel":
        walker.set_seed(0x5EED + index)
    plan = walker.query_plan(B)
    tokens = torch.empty((B, gamma), dtype=torch.int32, device=dev)
    n = base.shape[0]

    if head in ("gru", "rnn"):  # synthetic cell and initial state (no checkpoint uses these heads)
        cw = workloads.gru_cell_weights(index, gates=3 if head == "gru" else 1)
        celld = (bf(cw[0]), bf(cw[1]), torch.from_numpy(cw[2]).to(dev), torch.from_numpy(cw[3]).to(dev))
        h0 = torch.from_numpy(workloads.gru_h0(index, 0, 1)[0]).to(dev)
    if head == "domino":
        cw = workloads.domino_cell_weights(index)
        celld = (bf(cw[0]), bf(cw[1]), torch.from_numpy(cw[2]).to(dev), torch.from_numpy(cw[3]).to(dev))
        hid = bf(workloads.domino_hidden(index, 0, 1, gamma)[0])
        h0 = torch.from_numpy(workloads.gru_h0(index, 0, 1)[0]).to(dev)
    if head == "gated":
        gw = workloads.gated_weights(index)
        gated = tuple(torch.from_numpy(a).to(dev) for a in gw)
        h0 = torch.from_numpy(workloads.gru_h0(index, 0, 1)[0]).to(dev)

    def go(j):
        if head == "domino":
            walker.walk_domino(W1d, W2d, celld, hid, h0, base[j % n], anchor[j % n], T[j % n], uni[j % n],
                               tokens=tokens)
            return
        if head == "gated":
            walker.walk_gated(W1d, W2d, gated, h0, base[j % n], anchor[j % n], T[j % n], uni[j % n], tokens=tokens)
            return
        if head in ("gru", "rnn"):
            (walker.walk_gru if head == "gru" else walker.walk_rnn)(
                W1d, W2d, celld, h0, base[j % n], anchor[j % n], T[j % n], uni[j % n], tokens=tokens)
            return
        walker.walk(W1d, W2d, base[j % n], anchor[j % n], T[j % n], uni[j % n], w2_scale=scale,
                    tokens=tokens)
    # warm up for about 0.1 s: the first milliseconds of a burst of launches
    # run slower (at B = 253, ~300 against ~285 us per round) while clocks
    # settle
    t_w = time.perf_counter()
    j = 0
    while j < 5 or time.perf_counter() - t_w < 0.1:
        go(j)
        j += 1
        if j % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    K = 60 if big else 200
    t0 = time.perf_counter()
    for j in range(K):
        go(j)
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / K * 1e6
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for j in range(K):
        go(j)
    e1.record()
    torch.cuda.synchronize()
    launch = e0.elapsed_time(e1) * 1e3 / K
    st = walker.status()
    walker.close()
    abytes = algorithmic_bytes(V, B, gamma) - V * 256 * 2 + w2_bytes
    stepwise = (gamma * w2_bytes + B * gamma * V * 2) / (HBM_PEAK_GBS * 1e9) * 1e6
    flops = 2.0 * B * 256 * V * gamma
    out = {"workload": wl.name, "V": V, "B": B, "gamma": gamma, "w2": dtype, "temps": wl.temps, "sampler": sampler,
           "head": head,
           "us_per_round": round(us, 2), "launch_us": round(launch, 2),
           "kernel": "batched" if plan.batch_tile == 256 else
                     ("valu" if plan.engine == dsw.ENGINE_VALU else "mfma"),
           "path": "resident" if plan.stream_rows == 0 else f"partial ({plan.stream_rows} rows/wg streamed)",
           "hbm_gbs": round(abytes / (launch * 1e-6) / 1e9, 1),
           "hbm_frac": round(abytes / (launch * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "stepwise_bound_us": round(stepwise, 2),
           "vs_stepwise_bound": round(us / stepwise, 3), "status": st}
    if B >= 16:
        tfs = flops / (launch * 1e-6) / 1e12
        out["mfma_tfs"] = round(tfs, 1)
        out["mfma_frac"] = round(tfs / MFMA_BF16_PEAK_TFS, 4)
    del base, anchor, T, uni, W1d, W2d
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=1)
    ap.add_argument("--B", type=int, default=None)
    ap.add_argument("--gamma", type=int, default=None)
    ap.add_argument("--rounds", type=int, default=1000, help="distinct seeded rounds resident in HBM")
    ap.add_argument("--cold-rounds", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="only the timed walk (for profiling)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the other configurations")
    ap.add_argument("--pmc-mode", action="store_true",
                    help="for counter runs: --pmc-walks walks, then one 256 MiB device copy of known size")
    ap.add_argument("--pmc-walks", type=int, default=50)
    ap.add_argument("--pmc-cold", action="store_true", help="with --pmc-mode: a 1 GiB flush before each walk")
    ap.add_argument("--heads-only", action="store_true",
                    help="only the recurrent heads' configurations of the sweep (for profiling)")
    ap.add_argument("--stepwise-only", action="store_true",
                    help="for counter runs: only the step-wise library-op loop, then the same copy")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="write the counter record of --workload/--B/--gamma (cold with --pmc-cold) "
                         "from the rocprofv3 --pmc CSV output under DIR; no GPU")
    ap.add_argument("--grid-sweep", action="store_true",
                    help="only the rendezvous cost against the number of workgroups (8 .. 256)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the walk runs on one GPU; --gpus must be 1 (the multi-GPU split is a design, not built)"}))
        sys.exit(2)

    if args.summarize_counters:
        import workloads
        wl = workloads.WORKLOADS[args.workload]
        B = args.B if args.B is not None else wl.batches[0]
        gamma = args.gamma if args.gamma is not None else wl.gamma
        print(json.dumps(summarize_counters(args.summarize_counters, wl.name, wl.V, B, gamma, args.pmc_cold)))
        return

    import torch

    import serial_draft_head_amd as dsw
    import workloads

    if args.grid_sweep:
        print(json.dumps({"grid_sweep": grid_sweep(torch, dsw)}))
        return
    if args.heads_only:
        heads = [sweep_one(torch, dsw, *cfg) for cfg in SWEEP if len(cfg) > 5 and cfg[5] != "markov"]
        print(json.dumps({"heads_only": True, "configs": heads}))
        return

    wl = workloads.WORKLOADS[args.workload]
    B = args.B if args.B is not None else wl.batches[0]
    gamma = args.gamma if args.gamma is not None else wl.gamma
    V = wl.V
    dev = torch.device("cuda", 0)
    log(f"workload {wl.name} V={V} B={B} gamma={gamma}: generating inputs")
    W1, W2 = workloads.weights(args.workload)
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    W1d, W2d = bf(W1), bf(W2)
    n_rounds = min(args.rounds, args.steps + args.warmup)
    rounds = make_rounds(args.workload, n_rounds, B, gamma, V, wl.temps)
    dev_rounds = to_device(rounds, torch, dev)
    del rounds
    walker = dsw.Walker(V, gamma_max=max(gamma, 16), B_max=B)
    try:
        result = headline(args, torch, dsw, wl, walker, W1d, W2d, dev_rounds, B, gamma, V, n_rounds)
    finally:
        walker.close()   # every path: no handle outlives main()
    if result is None:
        return
    del dev_rounds
    torch.cuda.empty_cache()
    if not args.no_extras:
        extras(args, torch, dsw, result, W1d, W2d, B, V)
        del W1d, W2d
        torch.cuda.empty_cache()
        if not args.no_sweep:
            result["configs"] = []
            for (index, b, g, dt, *smp) in SWEEP:
                log(f"sweep: workload {index} B={b} gamma={g} {dt} {smp}")
                r = sweep_one(torch, dsw, index, b, g, dt, *smp)
                log(r)
                result["configs"].append(r)
        if not args.no_cpu_baseline:
            log("cpu baseline (oracle)")
            result["cpu_baseline"] = cpu_baseline(args.workload, B, gamma, V, W1, W2)
    print(json.dumps(result), flush=True)


def flusher(torch, dev, write=False):
    """Evicts L2 and the 256 MB Infinity Cache before a launch: a read of
    1 GiB (a sum over it), which leaves the caches holding clean lines of
    another buffer.  write=True zeroes the 1 GiB instead, which also evicts
    them but leaves up to the caches' size in dirty lines whose write-back
    the next launch pays for."""
    scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)

    def flush():
        if write:
            scratch.zero_()
        else:
            scratch.sum()
    return flush


def headline(args, torch, dsw, wl, walker, W1d, W2d, dev_rounds, B, gamma, V, n_rounds):
    """The timed walk and its roofline; None for the profiling-only modes."""
    dev = W1d.device
    plan = walker.query_plan(B).as_dict()
    log("plan", plan)

    if args.stepwise_only:
        sw = stepwise_torch(torch, W1d, W2d, dev_rounds, 20)
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"stepwise_only": True, "rounds": 23, "us_per_round": round(sw, 3),
                          "copy_bytes": COPY_BYTES}))
        return None
    if args.pmc_mode:
        # counter runs: args.pmc_walks walks (each after a 1 GiB flush with
        # --pmc-cold), then one device copy of known size to calibrate the counters
        base, anchor, T, uni = dev_rounds
        flush = flusher(torch, dev) if args.pmc_cold else None
        for i in range(args.pmc_walks):
            j = i % base.shape[0]
            if flush is not None:
                flush()
            walker.walk(W1d, W2d, base[j], anchor[j], T[j], uni[j])
        torch.cuda.synchronize()
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_mode": True, "walks": args.pmc_walks, "cold": bool(args.pmc_cold),
                          "copy_bytes": COPY_BYTES, "kernel_source_hash": kernel_source_hash(),
                          "status": walker.status()}))
        return None
    us_round, _ = time_walk(torch, walker, W1d, W2d, dev_rounds, args.steps, args.warmup)
    st = walker.status()
    if st != 0:
        raise SystemExit(f"device status {st} during the timed walk")
    log(f"warm: {us_round:.2f} us/round")
    result = {
        "metric": "Markov-walk µs/round (γ=7,16; bs=1) and HBM bytes/round vs streaming roofline",
        "value": round(us_round, 3), "unit": "us/round", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us_round / 1e3, 6), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "V": V, "r": 256, "gamma": gamma, "B": B,
                   "temps": wl.temps, "rounds_resident": n_rounds, "w2": "bf16"},
    }
    if args.no_extras:
        return result

    # per-launch kernel time (HIP events on the launch stream)
    k_launch = min(args.steps, 300)
    mean_launch, _ = time_walk(torch, walker, W1d, W2d, dev_rounds, k_launch, 10, per_launch=True)
    abytes = algorithmic_bytes(V, B, gamma)
    achieved = abytes / (mean_launch * 1e-6) / 1e9
    w2_bytes = V * 256 * 2
    stepwise_bound = gamma * w2_bytes / (HBM_PEAK_GBS * 1e9) * 1e6
    kernel = (f"walk_kernel<{plan['engine']}, "
              f"{plan['reg_tiles'] if plan['engine'] == dsw.ENGINE_MFMA else plan['reg_slots']}, "
              f"{plan['max_tiles'] if plan['engine'] == dsw.ENGINE_MFMA else 0}, {plan['batch_tile']}>")
    result["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                          "traffic": recorded_traffic(wl.name, B, gamma),
                          "kernel": kernel, "algorithmic_bytes_per_launch": abytes,
                          "launch_us_mean": round(mean_launch, 3),
                          "launches_timed": k_launch}
    result["stepwise_hbm_bound_us"] = round(stepwise_bound, 3)
    result["frac_of_stepwise_bound"] = round(us_round / stepwise_bound, 4)
    result["one_w2_read_floor_us"] = round(w2_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 3)
    log(f"per launch {mean_launch:.2f} us, {achieved:.0f} GB/s algorithmic")

    # cold: flush L2 + Infinity Cache before each round (outside the events)
    flush = flusher(torch, dev)
    kc = min(args.cold_rounds, n_rounds)
    cold_mean, cold = time_walk(torch, walker, W1d, W2d, dev_rounds, kc, 2, flush=flush)
    cold.sort()
    cold_med = statistics.median(cold)
    result["cold_us_per_round"] = {"median": round(cold_med, 3), "p10": round(cold[len(cold) // 10], 3),
                                   "p90": round(cold[(9 * len(cold)) // 10], 3), "rounds": kc}
    cold_ach = abytes / (cold_med * 1e-6) / 1e9
    result["roofline"].update({"cold_launch_us_median": round(cold_med, 3), "cold_achieved": round(cold_ach, 1),
                               "cold_frac": round(cold_ach / HBM_PEAK_GBS, 4),
                               "cold_traffic": recorded_traffic(wl.name, B, gamma, cold=True)})
    result["cold_frac_of_stepwise_bound"] = round(cold_med / stepwise_bound, 4)
    log("cold", result["cold_us_per_round"])
    wflush = flusher(torch, dev, write=True)
    _, cold_w = time_walk(torch, walker, W1d, W2d, dev_rounds, min(kc, 40), 2, flush=wflush)
    result["cold_after_write_flush_us"] = round(statistics.median(cold_w), 3)
    log("cold after a write flush", result["cold_after_write_flush_us"])
    del wflush
    if B == 1 and V == 151_936 and not args.no_sweep:
        result["cold_gamma_sweep"] = cold_gamma_sweep(torch, dsw, W1d, W2d, V, flush)
        log("cold gamma sweep", result["cold_gamma_sweep"])
    del flush
    torch.cuda.empty_cache()

    # gamma = 16 at the same vocabulary (the metric's second walk length)
    if gamma != 16 and V == 151_936:
        r16 = make_rounds(2, 100, 1, 16, V, "greedy")
        d16 = to_device(r16, torch, dev)
        us16, _ = time_walk(torch, walker, W1d, W2d, d16, 300, 20)
        result["gamma16_us_per_round"] = round(us16, 3)
        result["gamma16_stepwise_hbm_bound_us"] = round(16 * w2_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 3)
        log(f"gamma16: {us16:.2f} us/round")
        del d16

    # the step-wise loop of library ops (re-reads W2 every step)
    if B <= 16:
        sw = stepwise_torch(torch, W1d, W2d, dev_rounds, 100)
        result["stepwise_torch_us_per_round"] = round(sw, 3)
        result["stepwise_torch_w2_gbs"] = round(gamma * w2_bytes / (sw * 1e-6) / 1e9, 1)
        log(f"step-wise torch: {sw:.2f} us/round")
    return result


def extras(args, torch, dsw, result, W1d, W2d, B, V):
    # gamma sweep at this vocabulary: one-time entry vs per-step cost, resident vs streamed
    if B == 1 and V == 151_936 and not args.no_sweep:
        result["gamma_sweep"] = gamma_sweep(torch, dsw, W1d, W2d, V)
        log("gamma sweep", result["gamma_sweep"])

if __name__ == "__main__":
    main()
