"""Benchmark of the DeltaLog decode path on one MI355X.

One bench "step" is one merge cycle: C decode tokens for every head of the
batch (C-1 appends and the fused decode + fold), i.e. one pass over every
stage of the path.  The headline value is the amortised time per token
(cycle time / C) of GDN at B=128, H=32, d=128, C=8 with bf16 q/k/v and an fp32
state, inputs resident in HBM.

Printed: ONE JSON line.  Besides the contract fields it carries
  roofline      the dominant kernel (the append) against 8 TB/s HBM:
                algorithmic bytes per launch / mean launch time from HIP
                events recorded around every launch of the timed region
  cpu_baseline  the fp64 oracle timed on the host cores on a bounded sample
  eager         this library's eager dense kernel on the same inputs
  cold          every launch of a few cycles timed alone after the 256 MB
                Infinity Cache was refilled with another buffer (the state of
                the other layers of a model would pass through it between two
                launches of one layer)
  ceilings      what the GPU streams at the kernels' own access pattern: a read,
                an in-place copy and a write of every head with the decode
                kernels' workgroup shape, mapping and loads, back to back and
                cold
Usage: python bench.py [--steps K] [--warmup W] [--workload NAME] [--C c]
                       [--no-cold] [--report PATH] [--no-cpu] [--capacity-study]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, vendor figure
METRIC_TEMPLATE = "amortized µs/token + achieved HBM GB/s, {op} B={B} H={H} d={d} C={C}"


def metric_name(op, B, H, dk, dv, C):
    """The metric string of the workload actually run (the headline run, GDN
    B=128 H=32 d=128 C=8, gives the headline metric's exact name)."""
    d = str(dk) if dk == dv else f"{dk}x{dv}"
    return METRIC_TEMPLATE.format(op=op.upper(), B=B, H=H, d=d, C=C)


# committed counter summaries of the append, per serving-shape workload at C = 8
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "append_{workload}_c8_traffic.md")
# the sources each kind of counter summary is tied to
KERNEL_SOURCES = ["recurrent_state_updates_amd/csrc/step_kernel.h",
                  "recurrent_state_updates_amd/csrc/step_launch.h",
                  "recurrent_state_updates_amd/csrc/launch.h"]
CHUNK_SOURCES = KERNEL_SOURCES + ["recurrent_state_updates_amd/csrc/chunk_kernel.h"]


def kernel_source_hash(sources=None):
    """First 16 hex digits of the SHA-256 of the kernel sources with comments
    and blank space removed: the counters are tied to the code, not to its
    commentary.  The single-token summaries hash step_kernel.h, step_launch.h
    (which decides the launch shape) and launch.h,
    the multi-token ones chunk_kernel.h as well (CHUNK_SOURCES)."""
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(ln.strip() for ln in text.splitlines() if ln.strip()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per append launch from the committed rocprofv3 counter summary
    of the workload at C = 8, or None when there is none or the kernel source
    changed since."""
    path = TRAFFIC_PROFILE.format(workload=workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        text = f.read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]{16})", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


# Untimed warm-up before every timed region, in ms of back-to-back launches.
# Measured on MI355X: the first ~25 ms of load after an idle spell run up to
# a few percent slower (per-slot multi-token calls up to 18 %), then the
# times settle.
WARM_MS = 40


def warm_up(run_batch, sync, at_least=3):
    """Call run_batch() (which launches some work and returns how many units
    it launched) until at least WARM_MS of it has run and at least at_least
    units were launched; synchronises after each batch.  Returns the units."""
    n = 0
    t0 = time.perf_counter()
    while n < at_least or (time.perf_counter() - t0) * 1e3 < WARM_MS:
        n += run_batch()
        sync()
    return n


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40, help="timed merge cycles")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed merge cycles (default: whole cycles until %d ms of them have run, at "
                         "least 3; the clocks settle over the first few tens of ms of load)" % WARM_MS)
    ap.add_argument("--workload", default="gdn_b128_h32_d128")
    ap.add_argument("--C", type=int, default=8, help="log capacity = merge interval")
    ap.add_argument("--B", type=int, default=None, help="override the batch (sweep)")
    ap.add_argument("--cold", action="store_true",
                    help="(the default) time each launch of a few cycles alone after refilling the 256 MB "
                         "Infinity Cache with another buffer")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache timing and the ceilings")
    ap.add_argument("--capacity-study", action="store_true",
                    help="also time C=8, 16 and 32 (one capacity per kernel family), scale the measured "
                         "ceilings by each family's modelled over measured time, and time the capacity "
                         "dl_choose_capacity_bounds picks with those rates (and dl_choose_capacity's pick with "
                         "the bare ceilings) against the model's predictions")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-eager", action="store_true", help="skip the eager GPU kernel")
    ap.add_argument("--cpu-tokens", type=int, default=256, help="tokens in the CPU-baseline sample")
    ap.add_argument("--report", default=None, help="also append the JSON line to this file")
    ap.add_argument("--tokens", type=int, default=8,
                    help="also time multi-token decode: K tokens per dl_decode_tokens call (0: skip)")
    ap.add_argument("--staggered", action="store_true",
                    help="also time per-slot logs with slot b starting at token b mod C, so that "
                         "1/C of the slots fold at every step (continuous batching); with --tokens K "
                         "also K tokens per call on those slots")
    ap.add_argument("--split-ablation", action="store_true",
                    help="also time the fused and the split replay preparation, each launched call by "
                         "call and replayed as a captured merge-cycle graph")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 268 MB device-to-device copy (the reference kernel "
                         "for scaling hardware byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the decode path needs no exchange between GPUs "
              "(heads are independent), so there is no multi-GPU run to time. Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import recurrent_state_updates_amd as dl
    import workloads
    from recurrent_state_updates_amd import traffic

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dl.load_library()
    dev = torch.device("cuda:0")
    w = workloads.WORKLOADS[args.workload]
    Bsz = args.B or w.B
    C = args.C
    print(f"# generating {w.name} B={Bsz} T={w.T}", file=sys.stderr, flush=True)
    x = workloads.generate_workload(w, B=Bsz)
    d = {k: (None if v is None else v.to(dev)) for k, v in x.items()}
    T, H, D = w.T, w.H, w.d
    sh = traffic.Shape(w.op, Bsz, H, D, 2 if w.in_dtype == "bf16" else 4)
    outs = torch.empty((T, Bsz, H, D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    base = d["S0"].clone()
    st = dl.DeltaLogState(w.op, w.in_dtype, base, C)
    tok_args = [st.step_args(d["q"][t], d["k"][t], d["v"][t],
                             None if d["beta"] is None else d["beta"][t], d["decay"][t], d["bonus"],
                             outs[t]) for t in range(T)]
    lib = dl.load_library()
    step_fn = lib.dl_decode_step
    handle = st.handle
    import ctypes
    arg_refs = [ctypes.byref(a) for a in tok_args]

    def run_cycles(ncyc, tok0, marks=None):
        """Launch ncyc merge cycles.  marks maps a cycle index to three events,
        recorded before its first launch, before its fold and after it."""
        tok = tok0
        for c in range(ncyc):
            m = None if marks is None else marks.get(c)
            if m is not None:
                m[0].record(stream)
            for i in range(C):
                if m is not None and i == C - 1:
                    m[1].record(stream)
                rc = step_fn(handle, arg_refs[tok % T], sptr)
                if rc != 0:
                    raise dl.DeltaLogError(rc, dl.dl_last_error())
                tok += 1
            if m is not None:
                m[2].record(stream)
        return tok

    # warm-up, then the timed region: K merge cycles of back-to-back launches.
    # Every fifth cycle carries events (an event pair costs several
    # microseconds of GPU time here, so instrumenting every cycle would
    # distort the wall-clock value); C = 1 has events around the whole region.
    if args.warmup is None:
        box = [0]

        def warm_batch():
            box[0] = run_cycles(4, box[0])
            return 4
        nwarm = warm_up(warm_batch, torch.cuda.synchronize)
        tok = box[0]
    else:
        nwarm = args.warmup
        tok = run_cycles(nwarm, 0)
    assert st.log_length == 0
    K = args.steps
    torch.cuda.synchronize()
    if C > 1:
        every = 5
        marks = {c: [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                 for c in range(0, K, every)}
        t0 = time.perf_counter()
        tok = run_cycles(K, tok, marks)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        appends = np.array([m[0].elapsed_time(m[1]) * 1e3 for m in marks.values()])
        folds = np.array([m[1].elapsed_time(m[2]) * 1e3 for m in marks.values()])
    else:
        m0 = torch.cuda.Event(enable_timing=True)
        m1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        m0.record(stream)
        tok = run_cycles(K, tok)
        m1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        appends = np.zeros(1)
        folds = np.array([m0.elapsed_time(m1) * 1e3 / K])
    ms_per_cycle = wall * 1e3 / K
    us_per_token = wall * 1e6 / (K * C)
    kern_per_cycle = appends + folds
    us_tok_events = float(np.median(kern_per_cycle)) / C

    # the same region without any event, for the event-overhead check
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    tok = run_cycles(K, tok)
    torch.cuda.synchronize()
    us_per_token_noev = (time.perf_counter() - t1) * 1e6 / (K * C)

    append_mean_us = float(np.mean(appends)) / max(1, C - 1)
    merge_us = float(np.mean(folds))
    cyc_bytes = traffic.cycle_bytes(sh, C)
    tok_bytes = cyc_bytes / C
    if C > 1:
        app_bytes = [traffic.append_bytes(sh, L) for L in range(C - 1)]
        dom_bytes = float(np.mean(app_bytes))
        dom_us = append_mean_us
        dom_name = "append"
    else:
        dom_bytes = float(traffic.merge_bytes(sh, 1))
        dom_us = merge_us
        dom_name = "decode_fold"
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    measured = measured_traffic(w.name) if (C == 8 and Bsz == w.B) else None

    result = {
        "metric": metric_name(w.op, Bsz, H, D, D, C),
        "value": round(us_per_token, 3),
        "unit": "us/token",
        "n_gpus": 1,
        "steps": K,
        "warmup": nwarm,
        "ms_per_step": round(ms_per_cycle, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "op": w.op, "B": Bsz, "H": H, "dk": D, "dv": D, "C": C,
                   "in_dtype": w.in_dtype, "state_dtype": "f32", "tokens_per_step": C,
                   "seed": w.seed},
        "achieved_GBps": round(tok_bytes / (us_per_token * 1e-6) / 1e9, 1),
        "model_MB_per_token": round(tok_bytes / 1e6, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": measured, "kernel": dom_name,
                     "algorithmic_bytes_per_launch": int(dom_bytes),
                     "mean_launch_us": round(dom_us, 3)},
        "kernels_us": {"append_mean": round(append_mean_us, 2), "decode_fold": round(merge_us, 2),
                       "cycle_median_events": round(float(np.median(kern_per_cycle)), 2)},
        "us_per_token_kernel_events": round(us_tok_events, 3),
        "us_per_token_without_events": round(us_per_token_noev, 3),
    }
    # standalone fold (dl_merge mid-cycle) and materialise at L = C/2
    if C > 1:
        Lm = C // 2
        while st.log_length != Lm:
            rc = step_fn(handle, arg_refs[tok % T], sptr)
            if rc != 0:
                raise dl.DeltaLogError(rc, dl.dl_last_error())
            tok += 1
        dst = torch.empty_like(base)
        reps = 10
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            dl.dl_materialize(handle, dst.data_ptr(), sptr)
        e1.record(stream)
        torch.cuda.synchronize()
        mat_us = e0.elapsed_time(e1) * 1e3 / reps
        e0.record(stream)
        dl.dl_merge(handle, sptr)  # one early fold: L becomes 0
        e1.record(stream)
        torch.cuda.synchronize()
        merge_only_us = e0.elapsed_time(e1) * 1e3
        fb = traffic.fold_bytes(sh, Lm)
        result["fold_kernels"] = {
            "L": Lm, "materialize_us": round(mat_us, 2),
            "materialize_GBps": round(fb / (mat_us * 1e-6) / 1e9, 1),
            "merge_us": round(merge_only_us, 2),
            "merge_GBps": round(fb / (merge_only_us * 1e-6) / 1e9, 1)}
        del dst
    st.close()
    del st

    if not args.no_eager:
        state = d["S0"].clone()
        cfg = dl.make_config(w.op, w.in_dtype, Bsz, H, D, D, 1)
        eargs = [ctypes.byref(dl.state.make_step_args(
            w.op, w.in_dtype, Bsz, H, D, D, dev, d["q"][t], d["k"][t], d["v"][t],
            None if d["beta"] is None else d["beta"][t], d["decay"][t], d["bonus"], outs[t]))
            for t in range(T)]
        efn = lib.dl_eager_step
        cref = ctypes.byref(cfg)
        sp = state.data_ptr()
        for t in range(nwarm * C):
            efn(cref, sp, eargs[t % T], sptr)
        ne = K * C
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        e0.record(stream)
        for t in range(ne):
            rc = efn(cref, sp, eargs[t % T], sptr)
            if rc != 0:
                raise dl.DeltaLogError(rc, dl.dl_last_error())
        e1.record(stream)
        torch.cuda.synchronize()
        e_wall_us = (time.perf_counter() - t2) * 1e6 / ne
        e_us = e0.elapsed_time(e1) * 1e3 / ne
        eb = traffic.eager_bytes(sh)
        result["eager"] = {"us_per_token": round(e_wall_us, 3), "mean_launch_us": round(e_us, 3),
                           "achieved_GBps": round(eb / (e_us * 1e-6) / 1e9, 1),
                           "model_MB_per_token": round(eb / 1e6, 2)}
        result["speedup_vs_eager"] = round(e_wall_us / us_per_token, 3)

    if args.tokens > 0:
        result["multi_token"] = multi_token_times(dl, d, w, Bsz, C, sh, traffic, dev, stream, outs, K,
                                                  args.tokens)

    if args.split_ablation and C > 1:
        result["split_replay_ablation"] = split_ablation(dl, d, w, Bsz, C, dev, stream, outs, K)

    if args.staggered and C > 1:
        result["staggered"] = staggered_times(dl, d, w, Bsz, C, sh, traffic, dev, stream, outs, K)
        if args.tokens > 1:
            result["staggered"]["multi_token"] = staggered_multi_token_times(
                dl, d, w, Bsz, C, sh, traffic, dev, stream, outs, K, args.tokens)

    if args.calibrate_copy:
        src = torch.empty(sh.heads * D * D, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["calibration_copy_bytes"] = int(src.numel() * 4)
        del src, dst

    if not args.no_cold:
        flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
        ceil = stream_ceilings(dl, d["S0"], Bsz, H, D, D, stream, flush, K)
        result["ceilings"] = ceil
        cold = cold_cache_times(dl, d, w, Bsz, C, sh, traffic, dev, stream, outs, args.tokens, flush)
        cold["frac_of_peak"] = round(cold["achieved_GBps"] / PEAK_HBM_GBPS, 4)
        cold["isolated"]["frac_of_peak"] = round(cold["isolated"]["achieved_GBps"] / PEAK_HBM_GBPS, 4)
        # fractions of the ceilings are rates: the kernel's algorithmic bytes per
        # microsecond over the probe's (the append also moves its tokens and log)
        if C > 1:
            app_cold = float(np.mean(cold["append_by_L"]))
            cold["append_mean_us"] = round(app_cold, 2)
            cold["append_frac_of_read_ceiling"] = round(
                (dom_bytes / app_cold) / (ceil["read"]["bytes"] / ceil["read"]["cold_us"]), 4)
        cold["decode_fold_frac_of_copy_ceiling"] = round(
            (traffic.merge_bytes(sh, C) / cold["decode_fold"]) / (ceil["copy"]["bytes"] / ceil["copy"]["cold_us"]), 4)
        result["cold"] = cold
        if C > 1:
            result["roofline"]["frac_of_read_ceiling"] = round(
                (dom_bytes / dom_us) / (ceil["read"]["bytes"] / ceil["read"]["warm_us"]), 4)
        del flush

    if args.capacity_study and not args.no_cold:
        result["capacity_study"] = capacity_study(dl, d, w, Bsz, sh, traffic, stream, outs, K, ceil)

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(x, w, Bsz, args.cpu_tokens)

    line = json.dumps(result)
    print(line, flush=True)
    if args.report:
        with open(args.report, "a") as f:
            f.write(line + "\n")


def multi_token_times(dl, d, w, Bsz, C, sh, traffic, dev, stream, outs, K, ntok):
    """About K cycles of C tokens, decoded ntok per dl_decode_tokens call (a
    call that passes the log's end folds there and goes on in the same
    launch)."""
    import torch
    base = d["S0"].clone()
    st = dl.DeltaLogState(w.op, w.in_dtype, base, C)
    T = w.T
    one = [st.step_args(d["q"][t], d["k"][t], d["v"][t], None if d["beta"] is None else d["beta"][t],
                        d["decay"][t], d["bonus"], outs[t]) for t in range(T)]
    fn = dl.load_library().dl_decode_tokens
    sptr = stream.cuda_stream
    # every call's argument array is built before the timed region
    ntimed = -(-K * C // ntok)
    schedule, tok = [], 0
    for _ in range(ntimed):
        schedule.append((dl.StepArgs * ntok)(*[one[(tok + i) % T] for i in range(ntok)]))
        tok += ntok

    def run(arrs):
        for arr in arrs:
            assert fn(st.handle, arr, ntok, sptr) == 0
        return len(arrs)

    warm_up(lambda: run(schedule[:8]), torch.cuda.synchronize, at_least=-(-3 * C // ntok))
    L0 = st.log_length  # the log length when the timed calls start
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    run(schedule)
    e1.record(stream)
    torch.cuda.synchronize()
    ntokens = ntimed * ntok
    wall_us = (time.perf_counter() - t0) * 1e6 / ntokens
    st.close()
    nbytes = traffic.multi_token_bytes(sh, C, ntok, ntokens, L0)
    return {"tokens_per_call": ntok, "us_per_token": round(wall_us, 3),
            "events_us_per_token": round(e0.elapsed_time(e1) * 1e3 / ntokens, 3),
            "model_MB_per_token": round(nbytes / ntokens / 1e6, 2),
            "achieved_GBps": round(nbytes / ntokens / (wall_us * 1e-6) / 1e9, 1)}


def split_ablation(dl, d, w, Bsz, C, dev, stream, outs, K):
    """Amortised time per token over K merge cycles for the fused and the split
    replay preparation, launched call by call and replayed from one captured
    cycle.  The graph replays decode the same C tokens again (the work per
    replay does not depend on the values), so no refill runs in the region."""
    import ctypes
    import torch
    T = w.T
    fn = dl.load_library().dl_decode_step
    sptr = stream.cuda_stream
    res = {}

    def timed(body, ncyc):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        body(ncyc)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e6 / (ncyc * C)
        return {"us_per_token": round(wall, 3),
                "events_us_per_token": round(e0.elapsed_time(e1) * 1e3 / (ncyc * C), 3)}

    for split in (False, True):
        name = "split" if split else "fused"
        base = d["S0"].clone()
        st = dl.DeltaLogState(w.op, w.in_dtype, base, C, split_replay=split)
        refs = [ctypes.byref(st.step_args(d["q"][t], d["k"][t], d["v"][t],
                                          None if d["beta"] is None else d["beta"][t], d["decay"][t],
                                          d["bonus"], outs[t])) for t in range(T)]

        def calls(ncyc):
            for i in range(ncyc * C):
                assert fn(st.handle, refs[i % T], sptr) == 0

        calls(3)
        res[f"{name}_launches"] = timed(calls, K)
        tokens = [dict(q=d["q"][t], k=d["k"][t], v=d["v"][t],
                       beta=None if d["beta"] is None else d["beta"][t], decay=d["decay"][t],
                       bonus=d["bonus"], out=outs[t]) for t in range(C)]
        graph = st.capture_cycle(tokens)

        def replays(ncyc):
            for _ in range(ncyc):
                graph.launch(sptr)

        replays(3)
        res[f"{name}_graph"] = timed(replays, K)
        graph.close()
        st.close()
    return res


def staggered_times(dl, d, w, Bsz, C, sh, traffic, dev, stream, outs, K):
    """Per-slot logs, slot b started at token b mod C: every step then folds
    the 1/C of the slots whose log fills and appends for the rest."""
    import ctypes
    import numpy as np
    import torch
    base = d["S0"].clone()
    st = dl.DeltaLogState(w.op, w.in_dtype, base, C, slots=True)
    T = w.T
    args = [ctypes.byref(st.step_args(d["q"][t], d["k"][t], d["v"][t],
                                      None if d["beta"] is None else d["beta"][t], d["decay"][t],
                                      d["bonus"], outs[t])) for t in range(T)]
    fn = dl.load_library().dl_decode_step
    sptr = stream.cuda_stream
    tok = 0
    for s_ in range(C):  # staggered starts
        for b in range(s_, Bsz, C):
            st.activate(b)
        assert fn(st.handle, args[tok % T], sptr) == 0
        tok += 1
    for _ in range(3 * C):
        assert fn(st.handle, args[tok % T], sptr) == 0
        tok += 1
    steps = K * C
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        assert fn(st.handle, args[tok % T], sptr) == 0
        tok += 1
    e1.record(stream)
    torch.cuda.synchronize()
    wall_us = (time.perf_counter() - t0) * 1e6 / steps
    ev_us = e0.elapsed_time(e1) * 1e3 / steps
    st.close()
    tok_bytes = traffic.per_token_bytes(sh, C)
    return {"us_per_token": round(wall_us, 3), "events_us_per_token": round(ev_us, 3),
            "achieved_GBps": round(tok_bytes / (wall_us * 1e-6) / 1e9, 1),
            "note": "one launch per step; each slot appends, or folds when its token fills its log"}


def staggered_multi_token_times(dl, d, w, Bsz, C, sh, traffic, dev, stream, outs, K, ntok):
    """Per-slot logs started as in staggered_times, decoded ntok tokens per
    dl_decode_tokens call: one launch, in which each slot folds when its log
    fills and goes on from there."""
    import ctypes
    import torch
    base = d["S0"].clone()
    st = dl.DeltaLogState(w.op, w.in_dtype, base, C, slots=True)
    T = w.T
    one = [st.step_args(d["q"][t], d["k"][t], d["v"][t], None if d["beta"] is None else d["beta"][t],
                        d["decay"][t], d["bonus"], outs[t]) for t in range(T)]
    lib = dl.load_library()
    sptr = stream.cuda_stream
    start, tok = {}, 0
    for s_ in range(C):  # staggered starts, one token apart
        for b in range(s_, Bsz, C):
            st.activate(b)
            start[b] = tok
        assert lib.dl_decode_step(st.handle, ctypes.byref(one[tok % T]), sptr) == 0
        tok += 1
    ncalls = max(1, (K * C) // ntok)
    warm_arrs = [(dl.StepArgs * ntok)(*[one[(i * ntok + j) % T] for j in range(ntok)]) for i in range(8)]

    def warm_batch():
        for arr in warm_arrs:
            assert lib.dl_decode_tokens(st.handle, arr, ntok, sptr) == 0
        return len(warm_arrs)
    tok += ntok * warm_up(warm_batch, torch.cuda.synchronize)
    calls = []
    for _ in range(ncalls):
        calls.append((tok, (dl.StepArgs * ntok)(*[one[(tok + i) % T] for i in range(ntok)])))
        tok += ntok
    # modelled bytes of the timed calls: one launch per call, each slot from
    # its own log length
    sh1 = traffic.Shape(sh.op, 1, sh.H, sh.d, sh.in_bytes)
    nbytes = 0
    for t0, _ in calls:
        for b in range(Bsz):
            nbytes += traffic.call_bytes(sh1, (t0 - start[b]) % C, ntok, C) - sh1.shared()
        nbytes += sh.shared()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _, arr in calls:
        assert lib.dl_decode_tokens(st.handle, arr, ntok, sptr) == 0
    e1.record(stream)
    torch.cuda.synchronize()
    ntoks = ncalls * ntok
    wall_us = (time.perf_counter() - t0) * 1e6 / ntoks
    st.close()
    return {"tokens_per_call": ntok, "us_per_token": round(wall_us, 3),
            "events_us_per_token": round(e0.elapsed_time(e1) * 1e3 / ntoks, 3),
            "model_MB_per_token": round(nbytes / ntoks / 1e6, 2),
            "achieved_GBps": round(nbytes / ntoks / (wall_us * 1e-6) / 1e9, 1)}


def stream_ceilings(dl, S0, Bsz, H, dk, dv, stream, flush, K):
    """The read, the in-place copy and the write of every head at the decode
    kernels' access pattern (dl_probe_stream), on a copy of the state: back
    to back (mean over 4 K launches between two events, as the timed region
    runs the kernels) and cold, in sequence and isolated (ColdTimer, medians
    of 24)."""
    import numpy as np
    import torch
    state = S0.clone()
    sink = torch.zeros(1, dtype=torch.float32, device=S0.device)
    sptr = stream.cuda_stream
    nbytes = Bsz * H * dk * dv * 4
    timer = ColdTimer(torch, stream, flush)
    res = {"state_bytes": nbytes}
    def measure(name, mode, moved):
        def launch():
            dl.dl_probe_stream(mode, state.data_ptr(), Bsz, H, dk, dv, sink.data_ptr(), sptr)
        for _ in range(3):
            launch()
        n = 4 * K
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        warm = e0.elapsed_time(e1) * 1e3 / n
        iso = float(np.median([timer.isolated(launch) for _ in range(24)]))
        raw = float(np.median([timer.paired(launch) for _ in range(24)]))
        cold = raw - timer.refill_cost()
        res[name] = {"bytes": moved, "warm_us": round(warm, 2), "warm_GBps": round(moved / (warm * 1e-6) / 1e9, 1),
                     "cold_us": round(cold, 2), "cold_GBps": round(moved / (cold * 1e-6) / 1e9, 1),
                     "isolated_cold_us": round(iso, 2),
                     "isolated_cold_GBps": round(moved / (iso * 1e-6) / 1e9, 1)}

    measure("read", dl.DL_PROBE_READ, nbytes)
    measure("copy", dl.DL_PROBE_COPY, 2 * nbytes)
    assert torch.equal(state, S0), "the copy probe must leave the state unchanged"
    # the write side alone (overwrites this copy of the state)
    measure("write", dl.DL_PROBE_WRITE, nbytes)
    # the fixed cost of a launch: the read probe over one head, back to back and isolated
    def one():
        dl.dl_probe_stream(dl.DL_PROBE_READ, state.data_ptr(), 1, 1, dk, dv, sink.data_ptr(), sptr)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(50):
        one()
    e1.record(stream)
    torch.cuda.synchronize()
    res["one_head_launch_us"] = {"back_to_back": round(e0.elapsed_time(e1) * 1e3 / 50, 2),
                                 "isolated_cold": round(float(np.median([timer.isolated(one) for _ in range(24)])), 2)}
    del state
    return res


def capacity_study(dl, d, w, Bsz, sh, traffic, stream, outs, K, ceil):
    """NEXT-3 checked on the GPU.  The byte model prices appends at the read
    ceiling and the fold at the copy ceiling measured in this run; it cannot
    see that the kernels built for 16- and 32-entry logs hold more registers
    than those for 8.  So one capacity of each family (C = 8, 16, 32) is timed
    -- back to back, whole cycles -- and each family's rates are the ceilings
    scaled by its modelled over measured time.  dl_choose_capacity_bounds
    picks with those rates, dl_choose_capacity with the bare ceilings; both
    picks are timed beside the three calibration capacities."""
    import ctypes
    import torch
    read_gbps = ceil["read"]["warm_GBps"]
    copy_gbps = ceil["copy"]["warm_GBps"]
    fn = dl.load_library().dl_decode_step
    sptr = stream.cuda_stream

    def cfg_c(C):
        return dl.make_config(w.op, w.in_dtype, Bsz, w.H, w.d, w.d, C)

    def time_c(C):
        base = d["S0"].clone()
        st = dl.DeltaLogState(w.op, w.in_dtype, base, C)
        refs = [ctypes.byref(st.step_args(d["q"][t], d["k"][t], d["v"][t],
                                          None if d["beta"] is None else d["beta"][t], d["decay"][t],
                                          d["bonus"], outs[t])) for t in range(w.T)]
        ntok = C * max(K, -(-64 // C))  # whole cycles, at least 64 tokens
        for i in range(2 * C):
            assert fn(st.handle, refs[i % w.T], sptr) == 0
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(ntok):
            assert fn(st.handle, refs[i % w.T], sptr) == 0
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) * 1e6 / ntok
        st.close()
        return us

    measured = {C: time_c(C) for C in (8, 16, 32)}
    model = {C: dl.dl_predict_token_us(cfg_c(C), read_gbps, copy_gbps) for C in measured}
    eff = [model[C] / measured[C] for C in (8, 16, 32)]
    fam_read = [e * read_gbps for e in eff]
    fam_copy = [e * copy_gbps for e in eff]
    pick_one = dl.dl_choose_capacity(cfg_c(8), dl.DL_MAX_CAPACITY, read_gbps, copy_gbps)
    pick = dl.dl_choose_capacity_bounds(cfg_c(8), fam_read, fam_copy)
    for C in (pick, pick_one):
        if C not in measured:
            measured[C] = time_c(C)
    rows = {}
    for C in sorted(measured):
        one = dl.dl_predict_token_us(cfg_c(C), read_gbps, copy_gbps)
        fam = dl.dl_predict_token_us_bounds(cfg_c(C), fam_read, fam_copy)
        rows[str(C)] = {"measured_us_per_token": round(measured[C], 3), "model_us_per_token": round(one, 3),
                        "family_model_us_per_token": round(fam, 3),
                        "measured_over_model": round(measured[C] / one, 4)}
    fastest = min(rows, key=lambda c: rows[c]["measured_us_per_token"])
    return {"bandwidths_GBps": {"append_read": read_gbps, "fold_copy": copy_gbps},
            "family_efficiency": {"8": round(eff[0], 4), "16": round(eff[1], 4), "32": round(eff[2], 4)},
            "chosen_C": pick, "chosen_C_one_rate": pick_one, "by_C": rows,
            "chosen_is_fastest_measured": fastest == str(pick),
            "one_rate_pick_is_fastest_measured": fastest == str(pick_one)}


class ColdTimer:
    """Launch times with the 256 MB Infinity Cache refilled before each launch
    by a 512 MB read of another buffer (a read leaves only clean lines, so the
    launch pays no write-back of the refill).  Two measures:

      isolated     refill, then events around the launch alone: the launch
                   then also pays the idle GPU's wake-up from the events
                   (an empty kernel costs about 6 us this way, against about
                   2 us back to back)
      in sequence  events around [refill, launch], less the median of events
                   around [refill] alone (measured after every pair): the
                   launch's cold cost inside a stream of other work, as a
                   layer of a model meets it
    """

    def __init__(self, torch, stream, flush):
        self.torch, self.stream, self.flush = torch, stream, flush
        self.sink = torch.empty((), dtype=torch.float32, device=flush.device)
        self.refill_alone = []
        self.refill()
        torch.cuda.synchronize()

    def refill(self):
        self.torch.sum(self.flush, dim=0, out=self.sink)

    def _events(self):
        return (self.torch.cuda.Event(enable_timing=True), self.torch.cuda.Event(enable_timing=True))

    def isolated(self, launch):
        a, b = self._events()
        self.refill()
        a.record(self.stream)
        launch()
        b.record(self.stream)
        self.torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3

    def paired(self, launch):
        """Raw time of [refill, launch]; call refill_cost() at the end."""
        a, b = self._events()
        a.record(self.stream)
        self.refill()
        launch()
        b.record(self.stream)
        self.torch.cuda.synchronize()
        raw = a.elapsed_time(b) * 1e3
        c, d = self._events()
        c.record(self.stream)
        self.refill()
        d.record(self.stream)
        self.torch.cuda.synchronize()
        self.refill_alone.append(c.elapsed_time(d) * 1e3)
        return raw

    def refill_cost(self):
        import numpy as np
        return float(np.median(self.refill_alone))


def cold_cache_times(dl, d, w, Bsz, C, sh, traffic, dev, stream, outs, ntok=0, flush=None):
    """Every launch of a few merge cycles with the Infinity Cache refilled
    before it (ColdTimer): in sequence (the headline cold figure) and
    isolated; the same for calls of ntok tokens."""
    import numpy as np
    import torch
    if flush is None:
        flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    timer = ColdTimer(torch, stream, flush)
    base = d["S0"].clone()
    st = dl.DeltaLogState(w.op, w.in_dtype, base, C)
    ncyc = 20  # a 14 us launch after a 150 us refill: enough cycles that the median settles
    iso = np.zeros((ncyc, C))
    raw = np.zeros((ncyc, C))
    tok = 0
    for c in range(2 * ncyc):
        for i in range(C):
            t = tok % w.T

            def launch():
                st.step(d["q"][t], d["k"][t], d["v"][t], None if d["beta"] is None else d["beta"][t],
                        d["decay"][t], d["bonus"], outs[t])
            if c < ncyc:
                iso[c, i] = timer.isolated(launch)
            else:
                raw[c - ncyc, i] = timer.paired(launch)
            tok += 1
    st.close()
    seq = raw - timer.refill_cost()
    per_tok = float(np.median(seq.sum(axis=1))) / C
    per_tok_iso = float(np.median(iso.sum(axis=1))) / C
    tok_bytes = traffic.per_token_bytes(sh, C)
    result = {"us_per_token": round(per_tok, 3),
              "achieved_GBps": round(tok_bytes / (per_tok * 1e-6) / 1e9, 1),
              "append_by_L": [round(float(np.median(seq[:, L])), 2) for L in range(C - 1)],
              "decode_fold": round(float(np.median(seq[:, C - 1])), 2),
              "refill_us": round(timer.refill_cost(), 2),
              "isolated": {"us_per_token": round(per_tok_iso, 3),
                           "achieved_GBps": round(tok_bytes / (per_tok_iso * 1e-6) / 1e9, 1),
                           "append_by_L": [round(float(np.median(iso[:, L])), 2) for L in range(C - 1)],
                           "decode_fold": round(float(np.median(iso[:, C - 1])), 2)}}
    if ntok > 1:
        # the same for calls of ntok tokens, one launch each, in sequence
        base = d["S0"].clone()
        st = dl.DeltaLogState(w.op, w.in_dtype, base, C)
        fn = dl.load_library().dl_decode_tokens
        one = [st.step_args(d["q"][t], d["k"][t], d["v"][t], None if d["beta"] is None else d["beta"][t],
                            d["decay"][t], d["bonus"], outs[t]) for t in range(w.T)]
        ncalls = max(4, ncyc * C // ntok)
        raw_mt, tok, L = [], 0, 0
        nbytes = 0
        for _ in range(ncalls):
            arr = (dl.StepArgs * ntok)(*[one[(tok + i) % w.T] for i in range(ntok)])
            raw_mt.append(timer.paired(lambda: fn(st.handle, arr, ntok, stream.cuda_stream)))
            nbytes += traffic.call_bytes(sh, L, ntok, C)
            L = (L + ntok) % C
            tok += ntok
        st.close()
        per_tok_mt = (float(np.sum(raw_mt)) - ncalls * timer.refill_cost()) / (ncalls * ntok)
        result["multi_token"] = {"tokens_per_call": ntok, "us_per_token": round(per_tok_mt, 3),
                                 "achieved_GBps": round(nbytes / (ncalls * ntok) / (per_tok_mt * 1e-6) / 1e9, 1)}
    return result


def cpu_baseline(x, w, Bsz, tokens):
    """The fp64 oracle on the host cores: all heads of the batch, the first ``tokens`` tokens.
    A batch of fewer heads than threads also gets a one-thread figure (``one_thread``)."""
    import oracle
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    threads = max(1, min(16, ncpu))
    T = min(tokens, w.T)
    N = Bsz * w.H
    D = w.d

    def flat(t, width):
        return t[:T].reshape(T, N, width).double().numpy()

    beta = None if w.op == "rwkv6" else x["beta"][:T].reshape(T, N).double().numpy()
    decay = x["decay"][:T].reshape(T, N).double().numpy() if w.op == "gdn" else flat(x["decay"], D)
    bonus = None
    if w.op == "rwkv6":
        import numpy as np
        bonus = x["bonus"].double().numpy()[np.arange(N) % w.H]
    S0 = x["S0"].reshape(N, D, D).double().numpy()
    q, k, v = flat(x["q"], D), flat(x["k"], D), flat(x["v"], D)
    t0 = time.perf_counter()
    oracle.eager_run(w.op, q, k, v, beta, decay, bonus, S0, nthreads=threads)
    wall = time.perf_counter() - t0
    one_thread = None
    if N < threads:
        # fewer heads than threads, where the pool cannot help: the one-thread
        # figure too, repeated for at least 0.2 s of wall time
        reps, t1 = 0, time.perf_counter()
        while True:
            oracle.eager_run(w.op, q, k, v, beta, decay, bonus, S0, nthreads=1)
            reps += 1
            el = time.perf_counter() - t1
            if el >= 0.2:
                break
        one_thread = {"value": round(el * 1e6 / (reps * T), 2), "unit": "us/token", "cores": 1,
                      "repeats": reps}
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
    except OSError:
        pass
    res = {"value": round(wall * 1e6 / T, 1), "unit": "us/token", "cores": threads, "kind": "oracle",
           "sample": f"all {N} heads of {w.name} (B={Bsz}), first {T} tokens, fp64, "
                     f"{threads} threads; wall {wall:.2f} s",
           "cpu_model": model, "host_cpus_available": ncpu}
    if one_thread is not None:
        res["one_thread"] = one_thread
    return res


if __name__ == "__main__":
    main()
