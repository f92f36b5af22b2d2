#!/usr/bin/env python3
"""Throughput of the speculative-decoding verify step on one MI355X.

One step = one verify round of the B=64, K=8, V=128256 bf16 workload (T = 1.0):
both launches of spec_verify_sample (pass 1: row statistics, accept tests and
the first rejection; pass 2: the residual / bonus draw). Inputs are seeded
synthetic logits already resident in HBM. The timed steps cycle through
several copies of the inputs (together more than twice the 256 MB Infinity
Cache), so each step reads its logits from HBM rather than from the cache.
Steps are launched from HIP graphs that each hold a run of consecutive steps
(a graph launch costs about as much as a short kernel); the timed region, exactly
--steps steps, is bracketed by HIP events on the stream the kernels run on.

Prints ONE JSON line. Also reported: the pass-1 kernel alone (the dominant
kernel, for the roofline), the same round with early exit (pass 1 in stages,
spec_verify_sample_staged, which gives the same outputs), the same round
verified on top-k 50 / top-p 0.9 filtered laws (spec_verify_sample_filtered),
the n-gram pool (insert + lookup), the greedy verify and the sampling verify
of greedy-drafted n-grams on their own workload (B=32 G=7 N=5 V=32000 bf16),
and the CPU oracle on a bounded sample of the same round.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, AMD published peak
CACHE_BYTES = 256 * 2 ** 20  # MI355X Infinity Cache
METRIC = "verify rounds/s + achieved HBM GB/s (% peak), B=64 K=8 V=128256 bf16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = ["common.hpp", "params.hpp", "rowstats.hpp", "search.hpp", "sample.hip", "filter.hip",
                  "greedy.hip"]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--rotate", type=int, default=0, help="input copies (0: enough to exceed 2x the cache)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="bound on the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-greedy", action="store_true")
    ap.add_argument("--no-filtered", action="store_true", help="skip the top-k / top-p filtered leg")
    ap.add_argument("--no-staged", action="store_true", help="skip the early-exit (staged pass 1) leg")
    ap.add_argument("--no-pool", action="store_true", help="skip the n-gram pool leg")
    ap.add_argument("--no-ngram-sample", action="store_true", help="skip the one-hot n-gram sampling verify leg")
    ap.add_argument("--eager", action="store_true", help="launch through the Python binding instead of graphs")
    ap.add_argument("--counters", action="store_true",
                    help="short run for rocprofv3 --pmc: a 256 MiB copy (calibration), then 3 eager verify rounds "
                         "and 3 greedy rounds; prints nothing else")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/hbm_traffic.json from the counter_collection.csv files of two "
                         "rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of --counters; no GPU needed")
    return ap.parse_args()


def counters_run() -> int:
    """A few dispatches of each kernel for hardware-counter collection (no timing)."""
    import torch

    import rejection_sampling_verify_sample_amd as rsv
    from workloads import make_greedy_inputs, make_sample_inputs
    from workloads.torch_io import greedy_tensors, sample_tensors

    dev = torch.device("cuda:0")
    n = 256 * 2 ** 20
    src = torch.full((n // 4,), 1.5, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)  # calibration: reads and writes exactly n bytes
    torch.cuda.synchronize()
    del src, dst
    s = make_sample_inputs(3, 0)
    t = sample_tensors(s, dev)
    for _ in range(3):
        rsv.verify_sample(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"])
    torch.cuda.synchronize()
    del t
    g = greedy_tensors(make_greedy_inputs(0), dev)
    for _ in range(3):
        rsv.verify_greedy(g["logits"], g["cand"])
    torch.cuda.synchronize()
    del g
    from workloads import make_filter_params, make_ngram_sample_inputs
    t = sample_tensors(s, dev)
    fk, fp = make_filter_params(s.shape[0], top_k=FILTER_K, top_p=FILTER_P)
    fk, fp = torch.from_numpy(fk).to(dev), torch.from_numpy(fp).to(dev)
    for _ in range(3):
        rsv.verify_sample_filtered(t["target"], t["draft"], t["draft_tokens"], t["uniforms"], t["temperature"], fk, fp)
    torch.cuda.synchronize()
    del t
    ns = make_ngram_sample_inputs(0, peak=10.0)
    nlg = torch.from_numpy(ns.logits).to(dev).view(torch.bfloat16)
    ncand, nuni = torch.from_numpy(ns.cand).to(dev), torch.from_numpy(ns.uniforms).to(dev)
    for _ in range(3):
        rsv.verify_ngram_sample(nlg, ncand, nuni, ns.temperature)
    torch.cuda.synchronize()
    print("counters run done", file=sys.stderr)
    return 0


TRAFFIC_KERNELS = ["k_sample_rowstats", "k_sample_mass", "k_sample_draw", "k_greedy_argmax", "k_greedy_select",
                   "k_filter_fast", "k_filter_rows", "k_sample_mass_filtered", "k_sample_draw_filtered",
                   "k_ngs_rowstats", "k_ngs_verify"]
CALIBRATION_KERNEL = "__amd_rocclr_copyBuffer"
CALIBRATION_KIB = 256 * 1024


def _counter_means(path: str, counter: str) -> dict:
    """Mean counter value (KiB) per kernel family over its dispatches in one rocprofv3 CSV."""
    import csv
    acc = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            key = next((k for k in TRAFFIC_KERNELS + [CALIBRATION_KERNEL] if k in name), None)
            if key is None:
                continue
            if key in ("k_sample_mass", "k_sample_draw") and name.split(">(")[0].endswith("true"):
                key += "_filtered"  # the filtered round's variant (last template argument)
            acc.setdefault(key, []).append(float(row["Counter_Value"]))
    if CALIBRATION_KERNEL in acc:
        # the calibration copies come first; later copy dispatches are the small host-to-device input uploads
        acc[CALIBRATION_KERNEL] = acc[CALIBRATION_KERNEL][:3]
    return {k: sum(v) / len(v) for k, v in acc.items()}


def ingest_counters(fetch_csv: str, write_csv: str) -> int:
    """Scale the two counters by what they read for a copy of known size and store bytes per launch."""
    fetch, write = _counter_means(fetch_csv, "FETCH_SIZE"), _counter_means(write_csv, "WRITE_SIZE")
    if CALIBRATION_KERNEL not in fetch or CALIBRATION_KERNEL not in write:
        log("no calibration copy in the counter files")
        return 1
    fs = round(CALIBRATION_KIB / fetch[CALIBRATION_KERNEL], 5)
    ws = round(CALIBRATION_KIB / write[CALIBRATION_KERNEL], 5)
    sha = kernel_source_sha()
    out = {
        "about": "HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch, mean over "
                 "the dispatches of bench.py --counters), scaled by the factors a 256 MiB device copy gives "
                 "(copy bytes / counter bytes). source_sha: the kernel sources the counters were taken on "
                 "(bench.py reports null once they change).",
        "fetch_scale": fs, "write_scale": ws,
        "workloads": {"k_sample_*": "B=64 K=8 V=128256 bf16", "k_greedy_*": "B=32 G=7 N=5 V=32000 bf16",
                      "k_filter_*, *_filtered": "B=64 K=8 V=128256 bf16, top-k 50 and top-p 0.9 on every row",
                      "k_ngs_*": "n-gram sampling verify B=32 G=7 N=5 V=32000 bf16, peaked rows"},
    }
    for k in TRAFFIC_KERNELS:
        if k in fetch and k in write:
            out[k] = {"source_sha": sha, "fetch_kib": round(fetch[k], 1), "write_kib": round(write[k], 1),
                      "bytes_per_launch": round(1024 * (fetch[k] * fs + write[k] * ws))}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))
    return 0


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "rejection_sampling_verify_sample_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from rocprofv3 counters, if taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    ent = d.get(kernel)
    if not ent or ent.get("source_sha") != kernel_source_sha():
        return None
    return ent.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


CHUNK_STEPS = 48   # verify steps per HIP graph (a graph launch costs about as much as a short kernel)
FILTER_K, FILTER_P = 50, 0.9
STAGES = [3, 8]  # early-exit leg: pass 1 reads positions 0..2, then 3..7 of the rows still walking


class GraphSteps:
    """Runs verify steps step_fn(i, phases) from HIP graphs holding a run of consecutive steps.

    Steps cycle over the M input copies; a graph holds a whole number of cycles
    (about CHUNK_STEPS steps), and a remainder graph makes any count exact.
    """

    def __init__(self, torch, step_fn, M: int, eager: bool):
        self.torch, self.step_fn, self.M, self.eager = torch, step_fn, M, eager
        self.chunk = M * max(1, CHUNK_STEPS // M)
        self.graphs: dict = {}

    def _capture(self, phases, count):
        g = self.torch.cuda.CUDAGraph()
        with self.torch.cuda.graph(g):
            for j in range(count):
                self.step_fn(j, phases)
        return g

    def prepare(self, phases, n_list) -> None:
        if self.eager:
            return
        t = self.torch
        if phases not in self.graphs:
            side = t.cuda.Stream()
            side.wait_stream(t.cuda.current_stream())
            with t.cuda.stream(side):
                for j in range(self.M):
                    self.step_fn(j, phases)
            t.cuda.current_stream().wait_stream(side)
            t.cuda.synchronize()
            self.graphs[phases] = (self._capture(phases, self.chunk), {})
        tails = self.graphs[phases][1]
        for n in n_list:
            r = n % self.chunk
            if r and r not in tails:
                tails[r] = self._capture(phases, r)

    def run(self, phases, n: int) -> None:
        """Exactly n steps: whole graphs, then the remainder graph."""
        if self.eager:
            for i in range(n):
                self.step_fn(i, phases)
            return
        g, tails = self.graphs[phases]
        q, r = divmod(n, self.chunk)
        for _ in range(q):
            g.replay()
        if r:
            tails[r].replay()

    def timed(self, phases, n: int) -> float:
        """Seconds for n steps, between HIP events on the stream the graphs run on."""
        t = self.torch
        t.cuda.synchronize()
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        self.run(phases, n)
        b.record()
        t.cuda.synchronize()
        return a.elapsed_time(b) / 1e3


class Timer:
    def __init__(self, torch):
        self.torch = torch

    def time(self, fn, n: int) -> float:
        """Seconds for n calls of fn(i), bracketed by events on the current stream."""
        t = self.torch
        t.cuda.synchronize()
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        for i in range(n):
            fn(i)
        b.record()
        t.cuda.synchronize()
        return a.elapsed_time(b) / 1e3


def main() -> int:
    args = parse_args()
    if args.counters:
        return counters_run()
    if args.ingest_counters:
        return ingest_counters(*args.ingest_counters)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import rejection_sampling_verify_sample_amd as rsv
    from workloads import WORKLOAD_NAMES, make_greedy_inputs, make_sample_inputs
    from workloads.torch_io import greedy_tensors, sample_tensors

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    timer = Timer(torch)

    # ---------------------------------------------------------------- sampling verify, B=64 K=8 V=128256 bf16
    t0 = time.time()
    s = make_sample_inputs(3, 0)
    B, K, V = s.shape
    esz = 2
    base = sample_tensors(s, dev)
    set_bytes = (base["target"].numel() + base["draft"].numel()) * esz
    M = args.rotate or max(2, math.ceil(2 * CACHE_BYTES / set_bytes) + 1)
    log(f"inputs generated in {time.time() - t0:.1f}s; {M} copies of {set_bytes / 1e6:.1f} MB")
    sets = []
    for m in range(M):
        sets.append(dict(target=base["target"].clone(), draft=base["draft"].clone(),
                         draft_tokens=base["draft_tokens"].clone(), uniforms=base["uniforms"].clone(),
                         out_tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
                         out_n=torch.empty((B,), dtype=torch.int32, device=dev)))
    del base
    ws = torch.zeros(rsv.sample_workspace_size(B, K, V), dtype=torch.uint8, device=dev)

    def call(st, phases=rsv.PHASE_ALL):
        rsv.verify_sample(st["target"], st["draft"], st["draft_tokens"], st["uniforms"], s.temperature,
                          out_tokens=st["out_tokens"], out_num_accepted=st["out_n"], workspace=ws, phases=phases)

    for i in range(3):
        call(sets[i % M])
    torch.cuda.synchronize()
    steps = GraphSteps(torch, lambda i, ph: call(sets[i % M], ph), M, args.eager)
    n_list = [args.warmup, args.steps]
    steps.prepare(rsv.PHASE_ALL, n_list)
    steps.prepare(rsv.PHASE_ROW_STATS, n_list)
    steps.timed(rsv.PHASE_ALL, args.warmup)
    t_step = steps.timed(rsv.PHASE_ALL, args.steps) / args.steps
    steps.timed(rsv.PHASE_ROW_STATS, args.warmup)
    t_pass1 = steps.timed(rsv.PHASE_ROW_STATS, args.steps) / args.steps
    # outputs of the last full step of each copy (identical inputs -> identical outputs)
    for st in sets:
        call(st)
    torch.cuda.synchronize()
    n_acc = sets[0]["out_n"].cpu().numpy()
    assert np.all(n_acc >= 0) and np.all(n_acc <= K), "invalid accepted counts"
    tok = sets[0]["out_tokens"].cpu().numpy()
    assert np.all((tok[np.arange(B), n_acc] >= 0) & (tok[np.arange(B), n_acc] < V))

    # algorithmic bytes. Row statistics (pass 1): the 2K logit rows of every batch
    # row, read once. Pass 2: target + draft row n after a rejection, or the bonus
    # row. Plus the draft tokens, the uniforms and the outputs.
    row_bytes = V * esz
    pass1_bytes = B * 2 * K * row_bytes
    pass2_bytes = int(sum(2 * row_bytes if n < K else row_bytes for n in n_acc))
    small_bytes = B * K * 4 + B * (K + 1) * 2 * 4 + B * (K + 1) * 4 + B * 4
    step_bytes = pass1_bytes + pass2_bytes + small_bytes
    rounds_per_s = 1.0 / t_step
    step_gbps = step_bytes / t_step / 1e9
    pass1_gbps = pass1_bytes / t_pass1 / 1e9
    traffic = measured_traffic("k_sample_rowstats")
    log(f"step {t_step * 1e6:.2f} us ({rounds_per_s:.0f} rounds/s, {step_gbps:.0f} GB/s); "
        f"pass 1 {t_pass1 * 1e6:.2f} us ({pass1_gbps:.0f} GB/s); mean accepted {n_acc.mean():.3f}")
    del steps
    # the same round on one input copy every step ("hot": part of it may stay in the
    # 256 MB Infinity Cache); labelled apart from the rotated measurement above
    hsteps = GraphSteps(torch, lambda i, ph: call(sets[0], ph), 1, args.eager)
    hn = max(CHUNK_STEPS, min(args.steps, 500))
    hsteps.prepare(rsv.PHASE_ALL, [hn])
    hsteps.timed(rsv.PHASE_ALL, hn)
    t_hot = hsteps.timed(rsv.PHASE_ALL, hn) / hn
    hot = {"workload": WORKLOAD_NAMES[3] + "; one input copy reused every step", "steps": hn,
           "us_per_round": round(t_hot * 1e6, 3), "rounds_per_s": round(1.0 / t_hot, 1)}
    log(f"hot (one copy): {t_hot * 1e6:.2f} us per round")
    del hsteps

    # ---------------------------------------------------------------- the same round with early exit (pass 1 in stages)
    staged = None
    if not args.no_staged:
        stages = STAGES

        def scall(st, phases=rsv.PHASE_ALL):
            rsv.verify_sample_staged(st["target"], st["draft"], st["draft_tokens"], st["uniforms"], s.temperature,
                                     stages, out_tokens=st["out_tokens"], out_num_accepted=st["out_n"], workspace=ws)

        for st in sets:
            scall(st)
        torch.cuda.synchronize()
        sn = sets[0]["out_n"].cpu().numpy()
        # the outputs match the one-pass verify's except where a decision sits within rounding of
        # its boundary (the stages split rows into other segments); the parity tests hold both to the oracle
        same = bool(np.array_equal(sn, n_acc) and np.array_equal(sets[0]["out_tokens"].cpu().numpy(), tok))
        ssteps = GraphSteps(torch, lambda i, ph: scall(sets[i % M], ph), M, args.eager)
        ssteps.prepare(rsv.PHASE_ALL, n_list)
        ssteps.timed(rsv.PHASE_ALL, args.warmup)
        ts_step = ssteps.timed(rsv.PHASE_ALL, args.steps) / args.steps
        del ssteps
        # bytes this design reads: pass 1 through the stage holding each row's first
        # rejection (every stage when all K are accepted), then pass 2 as before
        read_pos = [next(e for e in stages if int(n) < e) if int(n) < K else K for n in n_acc]
        sbytes = int(sum(2 * p * row_bytes for p in read_pos)) + pass2_bytes + small_bytes
        staged = {"workload": f"{WORKLOAD_NAMES[3]}; pass 1 in stages ending at positions {stages}",
                  "rounds_per_s": round(1.0 / ts_step, 1), "us_per_round": round(ts_step * 1e6, 3),
                  "speedup_vs_one_pass": round(t_step / ts_step, 4), "same_outputs_as_one_pass": same,
                  "algorithmic_bytes_per_step": sbytes, "bytes_vs_one_pass": round(sbytes / step_bytes, 4),
                  "achieved_gbps": round(sbytes / ts_step / 1e9, 1),
                  "frac_of_hbm_peak": round(sbytes / ts_step / 1e9 / HBM_PEAK_GBPS, 4)}
        log(f"staged {stages}: {ts_step * 1e6:.2f} us ({1.0 / ts_step:.0f} rounds/s), "
            f"{sbytes / 1e6:.1f} MB read ({sbytes / step_bytes:.2f} of one pass)")

    # ---------------------------------------------------------------- the same round, top-k 50 / top-p 0.9 filtered
    filtered = None
    if not args.no_filtered:
        from workloads import make_filter_params
        fk, fp = make_filter_params(B, top_k=FILTER_K, top_p=FILTER_P)
        topk = torch.from_numpy(fk).to(dev)
        topp = torch.from_numpy(fp).to(dev)
        fws = torch.zeros(rsv.sample_filtered_workspace_size(B, K, V), dtype=torch.uint8, device=dev)
        kept = torch.empty((B, 2 * K + 1), dtype=torch.int32, device=dev)

        def fcall(st, phases=rsv.PHASE_ALL):
            rsv.verify_sample_filtered(st["target"], st["draft"], st["draft_tokens"], st["uniforms"], s.temperature,
                                       topk, topp, out_tokens=st["out_tokens"], out_num_accepted=st["out_n"],
                                       out_kept=kept, workspace=fws, phases=phases)

        for st in sets:
            fcall(st)
        torch.cuda.synchronize()
        fsteps = GraphSteps(torch, lambda i, ph: fcall(sets[i % M], ph), M, args.eager)
        fn = max(CHUNK_STEPS, args.steps // 4)
        fsteps.prepare(rsv.PHASE_ALL, [fn])
        fsteps.prepare(rsv.PHASE_ROW_STATS, [fn])
        fsteps.timed(rsv.PHASE_ALL, fn)
        tf_step = fsteps.timed(rsv.PHASE_ALL, fn) / fn
        fsteps.timed(rsv.PHASE_ROW_STATS, fn)
        tf_filter = fsteps.timed(rsv.PHASE_ROW_STATS, fn) / fn
        fcall(sets[0])
        torch.cuda.synchronize()
        fn_acc = sets[0]["out_n"].cpu().numpy()
        assert np.all(fn_acc >= 0) and np.all(fn_acc <= K), "invalid accepted counts (filtered)"
        rows = B * (2 * K + 1)
        one_read = rows * row_bytes
        # top-k 50 takes the one-pass path (k <= 64): each row is read once
        passes = 1
        filtered = {"workload": f"{WORKLOAD_NAMES[3]}; top-k {FILTER_K} and top-p {FILTER_P} on every row",
                    "rounds_per_s": round(1.0 / tf_step, 1), "us_per_round": round(tf_step * 1e6, 3),
                    "filter_kernel_us": round(tf_filter * 1e6, 3), "rows_filtered": rows,
                    "one_read_bytes": one_read, "filter_gbps_one_read": round(one_read / tf_filter / 1e9, 1),
                    "filter_passes_per_row": passes,
                    "filter_frac_of_hbm_peak": round(one_read / tf_filter / 1e9 / HBM_PEAK_GBPS, 4),
                    "mean_kept": round(float(kept.float().mean().item()), 2),
                    "mean_accepted": round(float(fn_acc.mean()), 4),
                    "filter_traffic": measured_traffic("k_filter_fast")}
        log(f"filtered step {tf_step * 1e6:.2f} us; filter kernel {tf_filter * 1e6:.2f} us "
            f"({one_read / tf_filter / 1e9:.0f} GB/s on one read of {rows} rows)")
        del fsteps
    del sets

    # ---------------------------------------------------------------- n-gram pool, B=32 V=32000 G=7 N=5, W=15 per call
    pool_leg = None
    if not args.no_pool:
        from workloads.ngram import lookup_tokens, ngram_steps
        PB, PV, PG, PN, PW = 32, 32000, 7, 5, 15
        pool = rsv.NgramPool(PB, PV, PG, PN, dev)
        host = ngram_steps(3, 16, PB, PW, PN, PV)
        grams = [torch.from_numpy(g).to(dev) for g in host]
        lasts = [torch.from_numpy(lookup_tokens(i, PB, PV, host)).to(dev) for i in range(16)]
        skipped = torch.empty((PB,), dtype=torch.int32, device=dev)
        pcand = torch.empty((PB, PG, PN - 1), dtype=torch.int32, device=dev)
        pcount = torch.empty((PB,), dtype=torch.int32, device=dev)

        def pstep(i):
            pool.insert(grams[i % 16], out_skipped=skipped)
            pool.lookup(lasts[i % 16], out_cand=pcand, out_count=pcount)

        for i in range(16):
            pstep(i)
        torch.cuda.synchronize()
        psteps = 48
        if args.eager:
            pfn = pstep
            pcalls = 1
        else:
            pgraph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(pgraph):
                for j in range(psteps):
                    pstep(j)
            pfn = lambda i: pgraph.replay()  # noqa: E731
            pcalls = psteps
        n_rep = max(1, args.steps // pcalls)
        timer.time(pfn, max(1, args.warmup // pcalls))
        t_pool = timer.time(pfn, n_rep) / (n_rep * pcalls)
        pool_leg = {"workload": f"n-gram pool B={PB} V={PV} G={PG} N={PN}: insert W={PW} n-grams per sequence, "
                                "then look up each sequence's last token",
                    "us_per_step": round(t_pool * 1e6, 3), "steps_per_s": round(1.0 / t_pool, 1),
                    "mean_candidates": round(float(pcount.float().mean().item()), 3)}
        log(f"n-gram pool insert + lookup: {t_pool * 1e6:.2f} us per step")
        del pool

    # ---------------------------------------------------------------- greedy verify, B=32 G=7 N=5 V=32000 bf16
    greedy = None
    if not args.no_greedy:
        g5 = make_greedy_inputs(0)
        gb, gg, gn, gv = g5.shape
        gt = greedy_tensors(g5, dev)
        gbytes = gt["logits"].numel() * 2
        M5 = max(2, math.ceil(2 * CACHE_BYTES / gbytes) + 1)
        gsets = [dict(logits=gt["logits"].clone(), cand=gt["cand"].clone(),
                      ot=torch.empty((gb, gn), dtype=torch.int32, device=dev),
                      ol=torch.empty((gb,), dtype=torch.int32, device=dev),
                      ob=torch.empty((gb,), dtype=torch.int32, device=dev)) for _ in range(M5)]
        gws = torch.zeros(rsv.greedy_workspace_size(gb, gg, gn, gv), dtype=torch.uint8, device=dev)

        def gcall(st):
            rsv.verify_greedy(st["logits"], st["cand"], out_tokens=st["ot"], out_accept_len=st["ol"],
                              out_best=st["ob"], workspace=gws)

        for st in gsets:
            gcall(st)
        torch.cuda.synchronize()
        L5 = M5 * max(1, 48 // M5)
        if args.eager:
            gstep = lambda i: gcall(gsets[i % M5])   # noqa: E731
            per_call = 1
        else:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for j in range(L5):
                    gcall(gsets[j % M5])
            gstep = lambda i: graph.replay()         # noqa: E731
            per_call = L5
        reps = max(1, args.steps // per_call)
        timer.time(gstep, max(1, args.warmup // per_call))
        per = (timer.time(gstep, reps) / reps) / per_call
        gal = gbytes + gb * gg * (gn - 1) * 4 + gb * (gn + 2) * 4
        greedy = {"workload": WORKLOAD_NAMES[5], "rounds_per_s": round(1.0 / per, 1),
                  "us_per_round": round(per * 1e6, 3), "achieved_gbps": round(gal / per / 1e9, 1),
                  "frac_of_hbm_peak": round(gal / per / 1e9 / HBM_PEAK_GBPS, 4), "rotate": M5,
                  "algorithmic_bytes": gal, "argmax_traffic": measured_traffic("k_greedy_argmax")}
        log(f"greedy {per * 1e6:.2f} us/round ({gal / per / 1e9:.0f} GB/s)")

    # ---------------------------------------------------------------- sampling verify of one-hot n-grams, same shape
    ngs = None
    if not args.no_ngram_sample:
        from workloads import make_ngram_sample_inputs
        ns = make_ngram_sample_inputs(0, peak=10.0)
        nb, ng, nn, nv = ns.shape
        nlg = torch.from_numpy(ns.logits).to(dev).view(torch.bfloat16)
        nbytes_set = nlg.numel() * 2
        MN = max(2, math.ceil(2 * CACHE_BYTES / nbytes_set) + 1)
        nsets = [dict(lg=nlg.clone(), cand=torch.from_numpy(ns.cand).to(dev), uni=torch.from_numpy(ns.uniforms).to(dev),
                      ot=torch.empty((nb, nn), dtype=torch.int32, device=dev),
                      ol=torch.empty((nb,), dtype=torch.int32, device=dev),
                      orow=torch.empty((nb,), dtype=torch.int32, device=dev)) for _ in range(MN)]
        del nlg
        nws = torch.zeros(rsv.ngram_sample_workspace_size(nb, ng, nn, nv), dtype=torch.uint8, device=dev)

        def ncall(st):
            rsv.verify_ngram_sample(st["lg"], st["cand"], st["uni"], ns.temperature, out_tokens=st["ot"],
                                    out_accept_len=st["ol"], out_rows=st["orow"], workspace=nws)

        for st in nsets:
            ncall(st)
        torch.cuda.synchronize()
        LN = MN * max(1, 48 // MN)
        if args.eager:
            nstep, ncalls = (lambda i: ncall(nsets[i % MN])), 1  # noqa: E731
        else:
            ngraph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(ngraph):
                for j in range(LN):
                    ncall(nsets[j % MN])
            nstep, ncalls = (lambda i: ngraph.replay()), LN  # noqa: E731
        nrep = max(1, args.steps // ncalls)
        timer.time(nstep, max(1, args.warmup // ncalls))
        tn = timer.time(nstep, nrep) / (nrep * ncalls)
        nL = nsets[0]["ol"].cpu().numpy()
        # pass 1 reads every row once; the draw reads one row per sequence (twice, the second time from cache)
        nalg = nbytes_set + nb * nv * 2
        ngs = {"workload": f"sampling verify of greedy-drafted n-grams B={nb} G={ng} N={nn} V={nv} bf16 T=1.0, "
                           "peaked rows, candidates on the peak w.p. 0.6",
               "rounds_per_s": round(1.0 / tn, 1), "us_per_round": round(tn * 1e6, 3),
               "achieved_gbps": round(nalg / tn / 1e9, 1), "frac_of_hbm_peak": round(nalg / tn / 1e9 / HBM_PEAK_GBPS, 4),
               "algorithmic_bytes": nalg, "mean_accepted": round(float(nL.mean()), 4), "rotate": MN,
               "pass1_traffic": measured_traffic("k_ngs_rowstats")}
        log(f"n-gram sampling verify {tn * 1e6:.2f} us/round ({nalg / tn / 1e9:.0f} GB/s), mean accepted {nL.mean():.3f}")
        del nsets

    # ---------------------------------------------------------------- CPU oracle on a bounded sample
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        tgt, drf = s.target_f32(), s.draft_f32()
        rows = 0
        t1 = time.perf_counter()
        while time.perf_counter() - t1 < args.cpu_seconds:
            b = rows % B
            oracle.oracle_sample(tgt[b:b + 1], drf[b:b + 1], s.draft_tokens[b:b + 1], s.uniforms[b:b + 1],
                                 s.temperature, with_probs=False)
            rows += 1
        el = time.perf_counter() - t1
        cpu = {"value": round(rows / el / B, 4), "unit": "verify rounds/s", "cores": 1, "kind": "oracle",
               "sample": f"{rows} batch rows of the B=64 K=8 V=128256 bf16 round (float64 NumPy, one thread), "
                         f"{el:.1f} s, scaled to rounds of 64 rows",
               "host_cpu": cpu_model(), "host_logical_cpus": os.cpu_count()}
        log(f"cpu oracle {rows} rows in {el:.1f}s")

    out = {
        "metric": METRIC,
        "value": round(rounds_per_s, 2),
        "unit": "verify rounds/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[3], "B": B, "K": K, "V": V, "T": s.temperature,
                   "input_copies": M, "graph": not args.eager},
        "draft_tokens_per_s": round(B * K * rounds_per_s, 1),
        "achieved_gbps": round(step_gbps, 1),
        "frac_of_hbm_peak": round(step_gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": step_bytes,
        "mean_accepted": round(float(n_acc.mean()), 4),
        "roofline": {"kernel": "k_sample_rowstats", "bound": "hbm", "achieved": round(pass1_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(pass1_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes": pass1_bytes,
                     "us_per_launch": round(t_pass1 * 1e6, 3)},
        "cpu_baseline": cpu,
        "hot_single_copy": hot,
        "staged": staged,
        "ngram_pool": pool_leg,
        "greedy": greedy,
        "ngram_sample": ngs,
        "filtered": filtered,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
