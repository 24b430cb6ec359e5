"""Throughput of the verification hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py ... --copy-calibration      (also runs a plain device copy of known size)
    python bench.py --traffic-from FETCH.csv WRITE.csv   (no GPU: turns two rocprofv3 --pmc
                                                          counter files into profiles/traffic_*.json)
    python bench.py --workload ssd_build_b16x12_k4_v128256_bf16   (an SSD round: every stage of it)
    python bench.py --ablation fanout   (cache hit rate of geometric against uniform fan-out over
                                         temperatures; one JSON object)
    python bench.py --trace-timeline [--workload NAME]   (needs libssd_trace.so: per-phase times
                                         of every verification workgroup, summarised)

A step is one verification round over one batch: every draft and target logit row of the batch
is streamed once (temperature softmax statistics, fused top-F guesses), the accept decisions and
first rejection are taken, the residual is formed and normalised and the bonus token is drawn by
inverse CDF. Inputs are seeded synthetic logits (see synth/gen.py) resident in HBM before timing;
the timed loop rotates over enough input replicas (>= 512 MB per cycle) that the 256 MB Infinity
Cache cannot serve them. Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified logit rows/sec and achieved HBM GB/s (B=16,K=4,V=128256)"
HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 512 << 20
COPY_BYTES = 256 << 20  # calibration copy: reads and writes exactly this many bytes per launch
VERIFY_KERNEL = "verify_kernel"
SPLIT_KERNELS = "verify_kernel (streaming) + resid_kernel"
KERNEL_SOURCES = ["draft_verification_ssd_amd/csrc/ssd_verify.hip",
                  "draft_verification_ssd_amd/csrc/ssd_device.hpp",
                  "draft_verification_ssd_amd/csrc/ssd_plan.hpp"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="b16_k4_v128256_bf16_top3")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed loop, copy COPY_BYTES device-to-device a few times so a "
                         "counter run sees the copy kernel beside the verification kernel")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--ablation", choices=["fanout"])
    ap.add_argument("--trace-timeline", action="store_true")
    ap.add_argument("--trace-out", default=None, help="with --trace-timeline: save the raw timestamps (.npy)")
    ap.add_argument("--wait-polls", type=int, default=None,
                    help="ssd_verify's wait_polls option (default: the library's)")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle worker processes for cpu_baseline (0: the usable cores, at most 16)")
    ap.add_argument("--temps", default="0.5,0.75,1.0,1.5,2.0")
    ap.add_argument("--ablation-batch", type=int, default=128)
    ap.add_argument("--ablation-seeds", type=int, default=4)
    ap.add_argument("--ablation-budget", type=int, default=12)
    ap.add_argument("--ablation-C", type=float, default=1.0,
                    help="Saguaro factor of the verification (the sets are the top-F_max of each draft row)")
    ap.add_argument("--ablation-rows", default="zipf,gauss",
                    help="row shapes: zipf (rank^-1.1 profile, noise 0.8, as the large-batch workload) "
                         "and/or gauss (N(0, 2^2), noise 0.5, as the cache-build workload)")
    return ap.parse_args()


def uniform_fanout(K, budget):
    """The budget split evenly over the K+1 outcomes' positions, the remainder to the smallest k."""
    base, left = divmod(budget, K + 1)
    return [base + (1 if k < left else 0) for k in range(K + 1)]


def fanout_ablation(args):
    """Geometric against uniform fan-out ([SSD] "消融实验": geometric fan-out keeps a higher cache hit
    rate, the more so at high temperature). For each temperature, seeded synthetic batches of the
    cache-build shape (K=4, V=128256 bf16, budget 12 unless given, C=1 unless given: only the fan-out
    differs between the two caches), with
    Zipf-shaped or Gaussian rows, are
    verified on the GPU with top-F_max guesses at every position; the geometric fan-out uses the
    acceptance rate measured in that batch (mean accept probability of the drafted tokens) and r=1;
    each fan-out's cache keys are built from the same guesses and the batch's outcomes looked up."""
    import numpy as np
    import torch

    import draft_verification_ssd_amd as ssd
    import synth

    B, K, V, dtype, budget, r = args.ablation_batch, 4, 128256, "bf16", args.ablation_budget, 1.0
    C = args.ablation_C
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    shapes = {"zipf": dict(zipf_s=1.1, noise_sigma=0.8), "gauss": dict(draft_sigma=2.0, noise_sigma=0.5)}
    rows = []
    for shape, T in [(sh, float(t)) for sh in args.ablation_rows.split(",") for t in args.temps.split(",")]:
        hits = {"geometric": 0, "uniform": 0}
        a_sum, n_seq, fans = 0.0, 0, {}
        for seed in range(args.ablation_seeds):
            lg = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
            Gm = 16

            def outcome(bt, C_run):
                """verify the batch (Saguaro sets = its own, when C < 1); the guesses of every position"""
                draft, target = lg(bt.draft), lg(bt.target)
                ap = torch.empty((B, K), device=dev)
                sets = torch.from_numpy(bt.sets).to(dev) if bt.sets is not None else None
                out = ssd.ssd_verify(draft[:, :K], target, torch.from_numpy(bt.x).to(dev),
                                     torch.from_numpy(bt.u).to(dev), T, sag_set=sets, sag_C=C_run,
                                     topf_F_max=Gm, accept_prob=ap)
                return out, ssd.ssd_topf_guess(draft[:, K, :], Gm), float(ap.mean().item())

            bt0 = synth.make_verify_batch(B, K, V, dtype, args.seed * 1000 + seed, T=T, **shapes[shape])
            out0, last0, a_hat = outcome(bt0, 1.0)  # the acceptance rate the geometric fan-out uses
            fans = {"geometric": ssd.ssd_fanout_alloc(K, min(max(a_hat, 1e-3), 1 - 1e-3), r, budget)[0],
                    "uniform": uniform_fanout(K, budget)}
            for name, fan in fans.items():
                assert max(fan) <= Gm
                if C < 1.0:  # each cache's own guesses are the Saguaro sets its drafts were drawn with
                    bt = synth.make_verify_batch(B, K, V, dtype, args.seed * 1000 + seed, T=T, **shapes[shape],
                                                 sag_sizes=fan[:K], C=C)
                    out, last, _ = outcome(bt, C)
                else:
                    out, last = out0, last0
                ck, ct = ssd.ssd_cache_keys(out["topf"], fan, guesses_last=last)
                _, miss = ssd.ssd_cache_lookup(ck, ct, out["accepted_len"], out["bonus_token"])
                hits[name] += B - int(miss.item())
            a_sum += a_hat * B
            n_seq += B
        rows.append({"rows": shape, "T": T, "acceptance_rate": round(a_sum / n_seq, 4), "sequences": n_seq,
                     "fanout_geometric_last_batch": fans["geometric"], "fanout_uniform": fans["uniform"],
                     "hit_rate_geometric": round(hits["geometric"] / n_seq, 4),
                     "hit_rate_uniform": round(hits["uniform"] / n_seq, 4)})
        print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
    print(json.dumps({"ablation": "fanout", "K": K, "V": V, "dtype": dtype, "budget": budget, "r": r, "C": C,
                      "data": "synthetic: zipf = -1.1 ln(rank) + N(0,1) draft, target + N(0, 0.8^2); "
                              "gauss = N(0, 2^2) draft, target + N(0, 0.5^2)", "results": rows}))


TRACE_SLOTS = 16
TRACE_PHASES = [  # slot: what the workgroup has just finished
    (1, "statistics of every row computed"),
    (2, "statistics published, arrived (role known)"),
    (3, "closer: every tile's statistics merged"),
    (11, "waves 1-3: the tile's guesses published"),
    (4, "decision published (closer) / guesses out and decision read (others)"),
    (5, "residual mass published"),
    (10, "merger (tile r mod T): guess row r merged"),
    (6, "others: every residual mass seen"),
    (7, "closer: every residual mass in"),
    (8, "bonus token drawn (the tile that drew it)"),
    (9, "end"),
]


def trace_timeline(args):
    """Per-phase timestamps of every verification workgroup (libssd_trace.so), relative to the
    earliest start of the launch, over several launches: percentiles per phase, for all tiles and
    for the closers (the last tile of each sequence)."""
    import numpy as np
    import torch

    import draft_verification_ssd_amd as ssd
    import synth

    ssd._lib.use_trace_library()
    spec = synth.workload(args.workload)
    B, K, V, dtype = spec["B"], spec["K"], spec["V"], spec["dtype"]
    topf = spec.get("topf", 0)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bt = synth.make_verify_batch(B, K, V, dtype, args.seed, T=spec["T"],
                                 noise_sigma=spec.get("noise_sigma", 0.5), zipf_s=spec.get("zipf_s"))
    esize = 2 if dtype == "bf16" else 4
    n_rep = max(1, math.ceil(ROTATE_BYTES / ((2 * K + 1) * B * V * esize)))
    ws = ssd.Workspace(ssd.ssd_verify_workspace_bytes(B, K, V, topf), dev)
    calls = [make_replica(bt, dev, topf, ws, args.wait_polls) for _ in range(n_rep)]
    T = ssd.ssd_verify_tiles(B, K, V, ssd.SSD_BF16 if dtype == "bf16" else ssd.SSD_F32)
    nwg = B * T
    buf = torch.zeros(nwg * TRACE_SLOTS, dtype=torch.int64, device=dev)
    ssd.lib().ssd_set_trace_buffer(buf.data_ptr())
    for i in range(args.warmup):
        calls[i % n_rep]()
    torch.cuda.synchronize()
    rows = []
    for i in range(args.steps):
        buf.zero_()
        calls[i % n_rep]()
        torch.cuda.synchronize()
        rows.append(buf.view(nwg, TRACE_SLOTS).cpu().numpy().copy())
    ssd.lib().ssd_set_trace_buffer(None)
    if args.trace_out:
        np.save(args.trace_out, np.stack(rows))
    out = {"workload": args.workload, "launches": args.steps, "workgroups": nwg, "tiles_per_row": T,
           "clock": "s_memrealtime, 100 MHz (10 ns)", "phases": []}
    rel_all = {slot: [] for slot, _ in TRACE_PHASES}
    rel_cl = {slot: [] for slot, _ in TRACE_PHASES}
    ends, gave_up = [], 0
    for r in rows:
        t0 = r[:, 0].min()
        role = r[:, 12]
        closer = (role & 1) != 0
        gave_up += int((((role >> 8) & 1) == 0).sum())
        ends.append((r[:, 9].max() - t0) * 10)
        for slot, _ in TRACE_PHASES:
            v = r[:, slot]
            ok = v > 0
            rel_all[slot].extend(((v[ok] - t0) * 10).tolist())
            rel_cl[slot].extend(((v[ok & closer] - t0) * 10).tolist())
    pct = lambda a, q: float(np.percentile(a, q)) if len(a) else None
    for slot, name in TRACE_PHASES:
        a, c = rel_all[slot], rel_cl[slot]
        out["phases"].append({"slot": slot, "phase": name, "ns_p10": pct(a, 10), "ns_p50": pct(a, 50),
                              "ns_p90": pct(a, 90), "ns_max": pct(a, 100), "closer_ns_p50": pct(c, 50),
                              "closer_ns_max": pct(c, 100)})
    out["launch_ns_p50"] = pct(ends, 50)
    out["tiles_that_gave_up_waiting"] = gave_up
    print(json.dumps(out), flush=True)


def algorithmic_bytes(B, K, V, esize, topf):
    logits = (2 * K + 1) * B * V * esize          # every draft (K) and target (K+1) row read once
    small = B * K * 4 + B * (K + 1) * 4           # draft tokens, uniforms
    outs = 2 * B * 4 + B * K * topf * 4           # accepted length, bonus, guesses
    return logits + small + outs


def make_replica(bt, dev, topf, workspace, wait_polls=None):
    import numpy as np
    import torch

    import draft_verification_ssd_amd as ssd

    def lg(a):
        a = np.ascontiguousarray(a)
        if bt.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    draft = lg(bt.draft[:, : bt.K])
    target = lg(bt.target)
    x = torch.from_numpy(bt.x).to(dev)
    u = torch.from_numpy(bt.u).to(dev)
    aprob = torch.empty((bt.B, bt.K), dtype=torch.float32, device=dev)
    return ssd.VerifyCall(draft, target, x, u, bt.T, topf_F_max=topf, accept_prob=aprob, workspace=workspace,
                          wait_polls=wait_polls)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_workers(requested: int) -> int:
    """Oracle worker processes: the host's cores, at most 16 (one GPU's share of the box)."""
    if requested > 0:
        return requested
    return max(1, min(os.cpu_count() or 1, 16))


def _one_thread():
    for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[v] = "1"


def _oracle_verify_worker(job):
    """One worker of the CPU baseline: whole sequences of the batch through the float64 oracle
    (verification and top-F guesses) for `seconds`, starting at sequence `first`."""
    import oracle as O

    draft, target, dtype, x, u, T, topf, first, seconds = job
    B, K = x.shape
    t0 = time.perf_counter()
    seqs = 0
    while True:
        b = (first + seqs) % B
        zq = O.logits_f64(draft[b, :K], dtype)
        zp = O.logits_f64(target[b], dtype)
        O.verify_sequence(zq, zp, x[b], u[b], T)
        for i in range(K):
            O.topf(zq[i], topf, int(x[b, i]))
        seqs += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return seqs, seqs * (2 * K + 1), el


def _oracle_round_worker(job):
    """One worker of the round's CPU baseline: whole sequences of the round (verification, guesses,
    keys, lookup and the branch rows' draft step) for `seconds`."""
    import oracle as O

    draft, target, dtype, x, u, T, sets, C, fan, branch, branch_u, first, seconds = job
    B, K = x.shape
    nbr = branch.shape[1]
    t0 = time.perf_counter()
    seqs = 0
    while True:
        b = (first + seqs) % B
        O.ssd_round(draft[b:b + 1], target[b:b + 1], dtype, x[b:b + 1], u[b:b + 1], T, sets[b:b + 1], C, fan,
                    branch=branch[b:b + 1], branch_u=branch_u[b:b + 1])
        seqs += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return seqs, seqs * ((2 * K + 2) + nbr * K), el


def _run_workers(fn, jobs):
    """The jobs in fresh interpreter processes (spawned: nothing of this process's GPU state is
    inherited), one per job, each single-threaded."""
    import multiprocessing as mp

    with mp.get_context("spawn").Pool(len(jobs), initializer=_one_thread) as pool:
        res = pool.map(fn, jobs)
    return sum(r[0] for r in res), sum(r[1] for r in res), max(r[2] for r in res)


def cpu_baseline(bt, topf, seconds, workers):
    """The float64 oracle on a bounded sample of the same workload, over `workers` processes."""
    K = bt.K
    jobs = [(bt.draft[:, :K], bt.target, bt.dtype, bt.x, bt.u, bt.T, topf, (w * bt.B) // workers, seconds)
            for w in range(workers)]
    seqs, rows, el = _run_workers(_oracle_verify_worker, jobs)
    return dict(value=round(rows / el, 1), unit="rows/s", cores=workers, kind="oracle", cpu=cpu_model(),
                sample=f"{seqs} sequences of the workload (seed 0) over {workers} processes, {rows} logit "
                       f"rows, float64 NumPy oracle verify + top-{topf} guesses, {el:.1f} s each")


def cpu_baseline_round(bt, branch, branch_u, fan, seconds, workers):
    """The float64 oracle on a bounded sample of an SSD round, over `workers` processes: whole
    sequences, each with its verification, guesses, keys, lookup and its branch rows' draft step."""
    jobs = [(bt.draft, bt.target, bt.dtype, bt.x, bt.u, bt.T, bt.sets, bt.C, fan, branch, branch_u,
             (w * bt.B) // workers, seconds) for w in range(workers)]
    seqs, rows, el = _run_workers(_oracle_round_worker, jobs)
    nbr = branch.shape[1]
    return dict(value=round(rows / el, 1), unit="rows/s", cores=workers, kind="oracle", cpu=cpu_model(),
                sample=f"{seqs} whole sequences of the round (seed 0) with their {nbr} branches over "
                       f"{workers} processes, {rows} logit rows, float64 NumPy oracle, {el:.1f} s each")


def load_traffic(workload, khash):
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("kernel_hash") != khash:
        return None
    return d.get("bytes_per_launch")


def _counter_rows(path):
    """(kernel name, counter name, value in KiB) per dispatch from a rocprofv3 counter CSV."""
    import csv
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])))
    return rows


def summarize_traffic(fetch_csv, write_csv, workload):
    """HBM bytes per launch of the verification kernel, each counter scaled by what it reads for
    the calibration copy (COPY_BYTES read and COPY_BYTES written per launch)."""
    import statistics
    out = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _counter_rows(path) if r[1] == name]
        ver = [v for k, _, v in rows if VERIFY_KERNEL in k]
        # the copy is the launch whose counter comes closest to COPY_BYTES (torch names it
        # differently across versions); it must be one of the non-verification kernels
        other = [v for k, _, v in rows if VERIFY_KERNEL not in k]
        if not ver or not other:
            raise SystemExit(f"{path}: no {name} rows for the verification kernel or the copy")
        copy_kib = min(other, key=lambda v: abs(v * 1024 - COPY_BYTES))
        scale = COPY_BYTES / (copy_kib * 1024)
        out[name] = dict(raw_kib_per_launch=statistics.median(ver), copy_raw_kib=copy_kib, scale=scale,
                         bytes_per_launch=statistics.median(ver) * 1024 * scale, launches=len(ver))
    total = out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"]
    d = dict(workload=workload, kernel=VERIFY_KERNEL, kernel_hash=kernel_hash(), bytes_per_launch=round(total),
             fetch=out["FETCH_SIZE"], write=out["WRITE_SIZE"],
             note="median over dispatches; each counter scaled by its reading for a plain "
                  f"{COPY_BYTES >> 20} MiB device copy")
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(d, f, indent=1)
    print(json.dumps(d))


class _Stage:
    def __init__(self, name, nbytes, fn):
        self.name, self.nbytes, self.fn = name, nbytes, fn


def pipeline_bench(args, spec):
    """One SSD round per step (the cache build and the full round): verification with Saguaro sets
    and per-position top-F guesses, draft row K's guesses in the same pass, cache keys and the lookup
    of the outcome in one launch,
    and, for the speculation-cache branches, the draft step of every branch row in one pass: its
    top-F set, Saguaro mass and normaliser, and a token drawn from q' (ssd_saguaro_sample). Each stage
    is timed on the GPU with an event pair per step; its algorithmic bytes (every logit it reads,
    once, plus its small inputs and outputs) over that time give its bandwidth."""
    import numpy as np
    import torch

    import draft_verification_ssd_amd as ssd
    import synth

    B, K, V, dtype, T = spec["B"], spec["K"], spec["V"], spec["dtype"], spec["T"]
    es = 2 if dtype == "bf16" else 4
    fan, _ = ssd.ssd_fanout_alloc(K, spec["a"], spec["r"], spec["budget"])
    budget, Gm = sum(fan), max(fan)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    bt = synth.make_verify_batch(B, K, V, dtype, args.seed, T=T, sag_sizes=fan[:K], C=spec["C"])
    branch = synth.make_branch_rows(B, budget, K, V, dtype, args.seed)
    branch_u = synth.make_branch_uniforms(B, budget, K, args.seed)
    Rb = B * budget * K  # branch rows

    def lg(a):
        a = np.ascontiguousarray(a)
        if dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    # every logit row of the outer batch once (K + 1 draft rows, the extra one for its guesses, and
    # K + 1 target rows), tokens, uniforms and sets in; k, bonus, top-F and row-K guesses out
    b_verify = ((2 * K + 2) * B * V * es + B * K * 4 + B * (K + 1) * 4 + B * K * Gm * 4 + 2 * B * 4
                + B * K * Gm * 4 + B * fan[K] * 4)
    # one read of every branch row; F and u in; set, sigma, N, token and q'(token) out
    b_branch = Rb * V * es + 2 * Rb * 4 + Rb * Gm * 4 + 4 * Rb * 4
    # guesses and outcomes in; keys, slots and the miss count out
    b_keys_lookup = B * K * Gm * 4 + B * fan[K] * 4 + 2 * B * 4 + 2 * B * budget * 4 + B * 4 + 4
    total_logit_bytes = ((2 * K + 2) * B + Rb) * V * es
    n_rep = max(1, math.ceil(ROTATE_BYTES / total_logit_bytes))

    reps = []
    ws_v = ssd.Workspace(ssd.ssd_verify_workspace_bytes(B, K, V, Gm), dev)
    ws_b = ssd.Workspace(ssd.ssd_saguaro_sample_workspace_bytes(Rb, V, Gm), dev)
    ub = torch.from_numpy(branch_u.reshape(-1)).to(dev)
    Fr = torch.tensor(fan[:K], dtype=torch.int32, device=dev).repeat(B * budget)
    for _ in range(n_rep):
        r = {}
        r["draft"] = lg(bt.draft)                      # [B, K+1, V]
        r["target"] = lg(bt.target)
        r["bd"] = lg(branch).view(Rb, V)
        r["topf"] = torch.empty((B, K, Gm), dtype=torch.int32, device=dev)
        r["gk"] = torch.empty((B, fan[K]), dtype=torch.int32, device=dev)
        r["bsets"] = torch.empty((Rb, Gm), dtype=torch.int32, device=dev)
        r["sig"] = torch.empty(Rb, dtype=torch.float32, device=dev)
        r["N"] = torch.empty(Rb, dtype=torch.float32, device=dev)
        r["btok"] = torch.empty(Rb, dtype=torch.int32, device=dev)
        r["bprob"] = torch.empty(Rb, dtype=torch.float32, device=dev)
        r["ck"] = torch.empty((B, budget), dtype=torch.int32, device=dev)
        r["ct"] = torch.empty((B, budget), dtype=torch.int32, device=dev)
        r["slot"] = torch.empty(B, dtype=torch.int32, device=dev)
        r["miss"] = torch.empty(1, dtype=torch.int32, device=dev)
        r["verify"] = ssd.VerifyCall(r["draft"], r["target"], torch.from_numpy(bt.x).to(dev),
                                     torch.from_numpy(bt.u).to(dev), T,
                                     sag_set=torch.from_numpy(bt.sets).to(dev), sag_C=bt.C, topf_F=fan[:K],
                                     topf_F_max=Gm, topf_out=r["topf"], topf_last_F=fan[K],
                                     topf_last_out=r["gk"], workspace=ws_v)
        reps.append(r)

    def stages(r):
        out = r["verify"].outputs

        def keys_lookup():  # straight from ssd_verify's top-F outputs and its outcome
            ssd.ssd_cache_keys_lookup(r["topf"], fan, out["accepted_len"], out["bonus_token"], guesses_last=r["gk"],
                                      cache_k=r["ck"], cache_tok=r["ct"], out_slot=r["slot"],
                                      out_miss_count=r["miss"])

        return [
            _Stage("verify (ssd_verify, fused top-F of rows 0..K and Saguaro)", b_verify, r["verify"]),
            _Stage("cache keys + lookup (ssd_cache_keys_lookup)", b_keys_lookup, keys_lookup),
            _Stage("branch draft step (ssd_saguaro_sample)", b_branch,
                   lambda: ssd.ssd_saguaro_sample(r["bd"], T, Gm, bt.C, ub, F_per_row=Fr, out_token=r["btok"],
                                                  out_prob=r["bprob"], out_set=r["bsets"], out_set_mass=r["sig"],
                                                  out_norm=r["N"], workspace=ws_b)),
        ]

    plans = [stages(r) for r in reps]
    for i in range(args.warmup):
        for st in plans[i % n_rep]:
            st.fn()
    torch.cuda.synchronize()
    nst = len(plans[0])
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        e = ev[i]
        e[0].record(stream)
        for j, st in enumerate(plans[i % n_rep]):
            st.fn()
            e[j + 1].record(stream)
    torch.cuda.synchronize()
    stage_ms = [float(np.median([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)]))
                for j in range(nst)]
    serial_ms = float(np.median([ev[i][0].elapsed_time(ev[i][nst]) for i in range(args.steps)]))
    # The branch rows' draft step does not depend on the outer verification (the branches are
    # drafted for every outcome before it is known), so a round can run it on a second stream
    # beside the verification and the lookup: fork, both, join, per step.
    side = torch.cuda.Stream(device=dev)
    ev2 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True), torch.cuda.Event())
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        e0, e1, ej = ev2[i]
        plan = plans[i % n_rep]
        e0.record(stream)
        side.wait_event(e0)
        with torch.cuda.stream(side):
            plan[-1].fn()  # the branch draft step
            ej.record(side)
        for st in plan[:-1]:
            st.fn()
        stream.wait_event(ej)
        e1.record(stream)
    torch.cuda.synchronize()
    overlapped_ms = float(np.median([a.elapsed_time(b) for a, b, _ in ev2]))
    step_ms = serial_ms
    flags = ssd.ssd_read_flags(ws_v) | ssd.ssd_read_flags(ws_b)
    if flags:
        print(f"device flags {flags:#x}", file=sys.stderr)
        sys.exit(3)
    rows = (2 * K + 2) * B + Rb
    algo = b_verify + b_keys_lookup + b_branch
    miss = int(reps[0]["miss"].item())
    st_out = {}
    for st, ms in zip(plans[0], stage_ms):
        st_out[st.name] = {"ms": round(ms, 5), "algorithmic_bytes": st.nbytes,
                           "GB/s": round(st.nbytes / (ms * 1e-3) / 1e9, 1)}
    dom = max(range(nst), key=lambda j: stage_ms[j])
    cpu = None if args.no_cpu_baseline else cpu_baseline_round(bt, branch, branch_u, fan, args.cpu_seconds, cpu_workers(args.cpu_workers))
    line = {
        "metric": METRIC,
        "value": round(rows / (step_ms * 1e-3), 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "K": K, "V": V, "T": T, "fanout": fan,
                   "C": spec["C"], "branch_rows": Rb, "rows_per_step": rows,
                   "algorithmic_bytes_per_step": algo, "input_replicas": n_rep},
        "roofline": {"bound": "hbm", "achieved": st_out[plans[0][dom].name]["GB/s"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(st_out[plans[0][dom].name]["GB/s"] / HBM_PEAK_GBS, 4),
                     "traffic": None, "kernel": plans[0][dom].name,
                     "note": "median stage time per step from HIP event pairs on the launch stream"},
        "stages": st_out,
        "overlapped_ms_per_step": round(overlapped_ms, 6),
        "schedule": "stages one after another on one stream (ms_per_step, stages); overlapped: the branch "
                    "draft step on a second stream beside verification and lookup",
        "step_GB/s": round(algo / (step_ms * 1e-3) / 1e9, 1),
        "cache": {"misses": miss, "hits": B - miss, "path": "zero-wait" if miss == 0 else "fallback"},
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.traffic_from:
        summarize_traffic(args.traffic_from[0], args.traffic_from[1], args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path would shard "
              f"by sequence, each GPU verifying its own sequences with no exchange)", file=sys.stderr)
        sys.exit(2)
    if args.ablation == "fanout":
        fanout_ablation(args)
        return
    if args.trace_timeline:
        trace_timeline(args)
        return
    import numpy as np
    import torch

    import draft_verification_ssd_amd as ssd
    import synth

    spec = synth.workload(args.workload)
    if "budget" in spec:  # an SSD round (cache build, full round)
        pipeline_bench(args, spec)
        return
    B, K, V, dtype = spec["B"], spec["K"], spec["V"], spec["dtype"]
    topf = spec.get("topf", 0)
    esize = 2 if dtype == "bf16" else 4
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    bt = synth.make_verify_batch(B, K, V, dtype, args.seed, T=spec["T"],
                                 noise_sigma=spec.get("noise_sigma", 0.5), zipf_s=spec.get("zipf_s"))
    step_bytes = algorithmic_bytes(B, K, V, esize, topf)
    logit_bytes = (2 * K + 1) * B * V * esize
    n_rep = max(1, math.ceil(ROTATE_BYTES / logit_bytes))
    ws = ssd.Workspace(ssd.ssd_verify_workspace_bytes(B, K, V, topf), dev)
    calls = [make_replica(bt, dev, topf, ws, args.wait_polls) for _ in range(n_rep)]

    for i in range(args.warmup):
        calls[i % n_rep]()
    torch.cuda.synchronize()

    # whole-loop throughput: K back-to-back steps bracketed by one event pair
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        calls[i % n_rep]()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps

    # per-launch duration of the kernel over the timed region: every step issues the same number of
    # launches of it (rounds of resident sequences), back to back on this stream
    n_launch = ssd.ssd_verify_launches(B, K, V, ssd.SSD_BF16 if dtype == "bf16" else ssd.SSD_F32, topf)
    if n_launch < 1:
        sys.exit(f"ssd_verify_launches returned {n_launch}")
    launch_ms = ms_per_step / n_launch

    # the same launch alone between an event pair (includes the event and dispatch overhead)
    n_ev = min(args.steps, 500)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_ev)]
    torch.cuda.synchronize()
    for i in range(n_ev):
        e0, e1 = evs[i]
        e0.record(stream)
        calls[i % n_rep]()
        e1.record(stream)
    torch.cuda.synchronize()
    # a whole step alone, per launch
    isolated_ms = float(np.mean([a.elapsed_time(b) for a, b in evs])) / n_launch

    # context: what a plain device-to-device copy reaches on this GPU (outside the timed region),
    # read + write bytes over its event-pair time, best of a few 512 MiB copies (not in counter
    # runs, whose calibration copy must be the only large copy)
    copy_gbs = None
    if not args.copy_calibration:
        csrc = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cdst = torch.empty_like(csrc)
        copy_ms = []
        for _ in range(6):
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            cdst.copy_(csrc)
            c1.record(stream)
            torch.cuda.synchronize()
            copy_ms.append(c0.elapsed_time(c1))
        copy_gbs = round(2 * csrc.numel() / (min(copy_ms[1:]) * 1e-3) / 1e9, 1)
        del csrc, cdst

    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    flags = ssd.ssd_read_flags(ws)
    if flags:
        print(f"device flags {flags:#x}", file=sys.stderr)
        sys.exit(3)

    # the read-only streaming ceiling at this footprint: a plain read of as many bytes as the step's
    # logits, rotating over as many buffers, timed the same way (outside the timed region above)
    read_ceiling = None
    if not args.copy_calibration:
        bufs = [torch.empty(logit_bytes, dtype=torch.uint8, device=dev) for _ in range(n_rep)]
        sink = torch.zeros(8192, dtype=torch.int32, device=dev)
        for i in range(2 * n_rep):
            ssd.ssd_stream_read(bufs[i % n_rep], sink, stream=stream)
        n_read = max(n_rep * 20, 200)
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        r0.record(stream)
        for i in range(n_read):
            ssd.ssd_stream_read(bufs[i % n_rep], sink, stream=stream)
        r1.record(stream)
        torch.cuda.synchronize()
        read_ms = r0.elapsed_time(r1) / n_read
        read_ceiling = round(logit_bytes / (read_ms * 1e-3) / 1e9, 1)
        del bufs, sink

    rows = (2 * K + 1) * B
    value = rows / (ms_per_step * 1e-3)
    # algorithmic bytes (every logit once) over the time they take: with one launch per step, that
    # launch's bytes over its duration; with two (statistics and guesses, then decision, the residual
    # rows read again and the bonus), the step's bytes over both launches' time
    achieved = step_bytes / (ms_per_step * 1e-3) / 1e9
    khash = kernel_hash()
    traffic = load_traffic(args.workload, khash)

    k_all = calls[0].outputs["accepted_len"].cpu().numpy()  # the replicas hold copies of one batch
    a_all = calls[0].outputs["accept_prob"].cpu().numpy().ravel()
    k_hist = np.bincount(k_all, minlength=K + 1).tolist()
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "K": K, "V": V, "T": spec["T"], "topf": topf,
                   "rows_per_step": rows, "algorithmic_bytes_per_step": step_bytes,
                   "input_replicas": n_rep, "sequences_per_s": round(B / (ms_per_step * 1e-3), 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": VERIFY_KERNEL if n_launch == 1 else SPLIT_KERNELS,
                     "launch_ms": round(launch_ms, 6), "launches_per_step": n_launch,
                     "isolated_launch_ms": round(isolated_ms, 6), "kernel_hash": khash,
                     "read_ceiling_GBps": read_ceiling,
                     "frac_of_read_ceiling": None if read_ceiling is None else round(achieved / read_ceiling, 4),
                     "device_copy_GBps": copy_gbs},
        # [SD7.3] 7.3.7: the acceptance rate and the accepted length, over the replicas' sequences
        "acceptance": {"alpha": round(float(a_all.mean()), 4), "mean_k": round(float(k_all.mean()), 4),
                       "accepted_len_hist": k_hist},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(bt, topf, args.cpu_seconds, cpu_workers(args.cpu_workers))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
