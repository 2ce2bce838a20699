#!/usr/bin/env python3
"""Benchmark of batched verification steps on one MI355X.

Headline workload (the confidence-scheduled block with every drafted position
verified): B = 256 sequences, K = 16 drafted positions, V = 129280, bf16
target and draft logits (target 2*N(0,1), draft = target + N(0, sigma_j) with
sigma_j rising 0.3 -> 1.5 along the block), T = 1, confidence c_j = max draft
probability, tau = 0 for every sequence, so L_b = 16.  Inputs are synthetic,
seeded, and resident in HBM before timing; two input sets alternate between
steps.

Printed: one JSON line with the metric (verified draft positions per second),
the step time, the roofline of the dominant kernel on the bytes the outputs
depend on, a "configs" object with every workload of the suite (each config as
written, plus the tau = 0 shadows of the two confidence-scheduled ones), the
later rows' legs, and the CPU oracle timed on this host as a baseline.

Timing: before each timed region's warm-up steps, about 50 ms of plain device
copies (on other buffers) are enqueued with no host wait in between.  After a
few ms idle the GPU runs the next ~10 ms of work 8-17% slower, every kernel
alike (a power-state effect; measured by --idle-probe and recorded in the
"idle_start_ms_per_step" field); the copies keep the timed steps out of that
window.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--only headline]
    python bench.py --copy-calibration     # plain 1 GiB copy, for counter scaling
    python bench.py --idle-probe 0,5,20    # step times after idle gaps of 0, 5, 20 ms
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft positions/sec and achieved HBM GB/s at V=129280 (1 MI355X)"
PEAK_HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_sv_stream_B256_K16_V129280_bf16_tau0.json")
KERNEL_SRC = os.path.join(ROOT, "draft_verification_amd", "csrc", "spec_verify.hip")
DOMINANT = "sv_stream"
HEADLINE = "sched256_tau0"

# key, synthetic workload, tau override (None: as written), description
CONFIGS = [
    ("tiny", "tiny", None,
     "tiny verify: B=4 K=4 V=1024 fp32, target 2*N(0,1), draft = target + N(0,0.5), T=1, L=K"),
    ("zipf64", "zipf64", None,
     "B=64 K=8 V=129280 bf16, target -1.1 ln(rank) + N(0,0.3), draft = target + N(0,0.7), T=1, L=8"),
    ("sched256", "sched256", None,
     "confidence-scheduled as written: B=256 K=16 V=129280 bf16, target 2*N(0,1), draft noise 0.3 -> 1.5, "
     "T=1, c = max draft prob, tau=0.3"),
    ("sched256_tau0", "sched256", 0.0,
     "the same tensors with tau=0 (every position verified, L=16): the headline workload"),
    ("greedy1024", "greedy1024", None,
     "greedy verify: B=1024 K=8 V=129280 bf16, N(0,1) with one planted max per row, draft = argmax w.p. 0.8, T=0"),
    ("peaked512", "peaked512", None,
     "peaked: B=512 K=16 V=129280 fp32, target -1.3 ln(rank) + N(0,0.3) at T=0.7, draft = target + N(0,0.2), "
     "c = max draft prob, tau in {0.2, 0.4, 0.6} per sequence"),
    ("peaked512_tau0", "peaked512", 0.0,
     "the same tensors with tau=0 (every position verified, L=16)"),
]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def workload(synth, base: str, tau, seed_shift=0):
    w = synth.WORKLOADS[base]
    w = w.with_(seed=w.seed + seed_shift)
    if tau is not None:
        w = w.with_(tau_choices=(float(tau),))
    return w


def with_tau(prob, tau: float):
    """The same problem with every sequence's threshold set to tau."""
    import dataclasses
    return dataclasses.replace(prob, w=prob.w.with_(tau_choices=(float(tau),)),
                               tau=np.full_like(prob.tau, np.float32(tau)))


def open_walk(prob) -> np.ndarray:
    """Sequences whose verify length the device finds by walking the block:
    derived confidences (c = max draft prob) with 0 < tau <= 1."""
    w = prob.w
    B = prob.tokens.shape[0]
    if w.length_mode != 1 or prob.confidence is not None or w.temperature == 0 or getattr(w, "draft_mode", 0) == 1:
        return np.zeros(B, bool)
    return (prob.tau > 0) & (prob.tau <= 1)


def byte_counts(res, prob) -> dict:
    """Bytes of one step, summed over the batch.

    needed:   the rows the outputs depend on, each read once -- target rows
              1..a+1, the draft rows of the tested positions (1..min(a+1, L)),
              and with an open length walk the draft rows the length rule
              reads (1..min(L+1, K)) -- plus the per-position inputs and the
              outputs.
    window:   every row up to L+1 (with an open walk every draft row), the
              same inputs and outputs: what a kernel without early exit reads.
    streamed: the logit bytes the step actually streamed (the library's
              bytes_read), same inputs and outputs."""
    w = prob.w
    K, V = w.K, w.V
    es = 2 if w.dtype == 1 else 4
    greedy = w.temperature == 0
    no_draft_rows = greedy or getattr(w, "draft_mode", 0) == 1
    a = res["accepted_len"].astype(np.int64)
    L = res["verify_len_out"].astype(np.int64)
    ok = np.array([res["out_tokens"][b][min(int(a[b]), K)] >= 0 for b in range(len(a))])
    ow = open_walk(prob)
    tested = np.minimum(a + 1, L)
    t_rows = np.where(ok, a + 1, 0)
    d_rows = np.zeros_like(a) if no_draft_rows else np.where(ok, np.maximum(tested, np.where(ow, np.minimum(L + 1, K), 0)), 0)
    per_pos_in = 4 if greedy else 8                      # drafted token (+ uniform)
    io = tested * per_pos_in + (0 if greedy else 4) + (K + 1) * 4 + 8
    io_total = int(io.sum())
    win_d = np.zeros_like(a) if no_draft_rows else np.where(ow, K, L)
    out = {
        "needed": int((t_rows + d_rows).sum()) * V * es + io_total,
        "window": int(((L + 1) + win_d).sum()) * V * es + io_total,
        "needed_rows": int((t_rows + d_rows).sum()),
    }
    if res.get("bytes_read") is not None and res["bytes_read"][0] >= 0:
        out["streamed"] = int(res["bytes_read"].astype(np.int64).sum()) + io_total
        out["streamed_rows"] = int(res["rows_read"].astype(np.int64).sum())
    return out


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    with open(KERNEL_SRC, "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def traffic_entry(src_hash: str, leg: str = None):
    """HBM bytes of one step's sv_stream launches from committed counter runs,
    if they were taken on this kernel source: the headline workload, or a
    later leg ("onehot", "packed")."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_src_sha") != src_hash:
        return None
    if leg is not None:
        return t.get("legs", {}).get(leg, {}).get("hbm_bytes_per_launch")
    return t.get("hbm_bytes_per_launch")


class Prewarm:
    """Plain device copies between two buffers of its own, enqueued right
    before a timed region's warm-up steps (no host wait in between), so that
    the GPU is out of its idle power state when the timed steps start.  The
    copies also evict the inputs from the on-die cache."""

    def __init__(self, torch, ms: float = 50.0, nbytes: int = 1 << 29):
        self.torch = torch
        self.ms = ms
        self.src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.dst = torch.empty_like(self.src)
        self.src.fill_(1)
        for _ in range(3):
            self.dst.copy_(self.src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(8):
            self.dst.copy_(self.src)
        e1.record()
        torch.cuda.synchronize()
        self.n = max(1, int(math.ceil(ms / (e0.elapsed_time(e1) / 8))))

    def enqueue(self):
        for _ in range(self.n):
            self.dst.copy_(self.src)

    def describe(self):
        return {"ms": self.ms, "copies": self.n, "bytes_per_copy": int(self.src.numel()),
                "what": "device copies between two buffers of their own, enqueued just before the warm-up steps"}

    def close(self):
        del self.src, self.dst


def time_block(torch, sv, argv, steps, warmup, pw):
    """W warm-up steps (after the pre-warm copies), then exactly K steps
    between two events on the launch stream, synchronised on both sides."""
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    pw.enqueue()
    for i in range(warmup):
        sv.run(argv[i % len(argv)], stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        sv.run(argv[i % len(argv)], stream)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def kernel_times(torch, sv, argv, steps, pw):
    """Average ms per step of each kernel, from events attached to each
    dispatch (a separate pass)."""
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    pw.enqueue()
    sv.timing_begin(steps)
    for i in range(steps):
        sv.run(argv[i % len(argv)], stream)
    torch.cuda.synchronize()
    kms, nruns = sv.timing_end()
    return {k: v / max(nruns, 1) for k, v in kms.items()}


def count_pass(torch, sv, dps):
    """One untimed step per input set with the stream counts requested; its
    outputs (all but the counts) equal the timed steps'."""
    outs = []
    stream = torch.cuda.current_stream().cuda_stream
    for d in dps:
        sv.run(d.args(counts=True), stream)
        outs.append(d.fetch())
    return outs


def measure(torch, B, D, probs, steps, warmup, pw, *, dominant=DOMINANT, extra=False):
    """Time one workload's step over its two input sets; returns the config
    entry and the outputs of the timed steps (for the oracle check)."""
    w = probs[0].w
    dps = [D.from_problem(p, diagnostics=False) for p in probs]
    sv = B.SpecVerify(w.B, w.K, w.V, w.dtype, 0)
    argv = [d.args(counts=False) for d in dps]
    ms = time_block(torch, sv, argv, steps, warmup, pw)
    timed_outs = [d.fetch() for d in dps]   # the last timed step of each set
    kt = kernel_times(torch, sv, argv, steps, pw)
    outs = count_pass(torch, sv, dps)
    for o, t in zip(outs, timed_outs):
        for k in ("accepted_len", "verify_len_out", "out_tokens", "device_status"):
            assert np.array_equal(o[k], t[k]), f"{k}: the counted step differs from the timed one"
        assert int(o["device_status"][0]) == 0, "the device reported a bad input or an incomplete walk"
    extras = {}
    if extra:
        extras = headline_extras(torch, sv, argv, steps, pw)
    sv.close()
    del dps, argv
    torch.cuda.empty_cache()

    bc = [byte_counts(o, p) for o, p in zip(outs, probs)]
    mean = lambda k: sum(c[k] for c in bc) / len(bc)
    positions = float(np.mean([o["verify_len_out"].sum() for o in outs]))
    emitted = float(np.mean([o["accepted_len"].sum() + (o["out_tokens"][:, 0] >= 0).sum() for o in outs]))
    needed, streamed, window = mean("needed"), mean("streamed"), mean("window")
    dom_ms = kt.get(dominant, 0.0)
    entry = {
        "B": w.B, "K": w.K, "V": w.V, "logits": "bf16" if w.dtype == 1 else "fp32", "temperature": w.temperature,
        "tau": None if probs[0].tau is None else sorted({float(x) for x in np.unique(probs[0].tau)}),
        "ms_per_step": ms,
        "value": positions / (ms / 1e3), "unit": "verified draft positions/s",
        "emitted_tokens_per_s": emitted / (ms / 1e3),
        "verified_positions_per_step": positions,
        "mean_L": float(np.mean([o["verify_len_out"].mean() for o in outs])),
        "mean_accepted": float(np.mean([o["accepted_len"].mean() for o in outs])),
        "needed_bytes_per_step": needed,
        "streamed_bytes_per_step": streamed,
        "streamed_over_needed": streamed / needed,
        "window_bytes_per_step": window,
        "kernel_avg_ms": kt,
        "dominant_kernel": dominant,
        "frac": needed / (dom_ms / 1e3) / 1e9 / PEAK_HBM_GBPS if dom_ms > 0 else None,
        "step_frac": needed / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS,
        "oracle_agreement": None,
    }
    entry.update(extras)
    return entry, outs


def headline_extras(torch, sv, argv, steps, pw):
    """Headline only: the step-time distribution, the time when the steps
    start from idle, and HIP graph replay."""
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    pw.enqueue()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        sv.run(argv[i % 2], stream)
        evs[i + 1].record()
    torch.cuda.synchronize()
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)])
    dist = {"p10": float(np.percentile(per_step, 10)), "p50": float(np.median(per_step)),
            "p90": float(np.percentile(per_step, 90)), "n": int(steps), "unit": "ms",
            "method": "HIP events between consecutive steps on the launch stream (a separate pass)"}
    # the same K steps started after 20 ms of idle GPU, no pre-warm
    time.sleep(0.02)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        sv.run(argv[i % 2], stream)
    e1.record()
    torch.cuda.synchronize()
    idle_ms = e0.elapsed_time(e1) / steps
    graph_ms = time_graph_replay(torch, sv, argv, steps, pw)
    return {"step_ms_distribution": dist, "idle_start_ms_per_step": idle_ms, "graph_replay_ms_per_step": graph_ms}


def time_graph_replay(torch, sv, argv, steps, pw):
    """Time per step when each input set's step is captured once in a HIP graph
    and replayed (no host launch cost per kernel): a step is only kernel
    launches on the caller's stream, so a serving loop can capture it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for a in argv:
            sv.run(a)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for a in argv:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sv.run(a)
        graphs.append(g)
    torch.cuda.synchronize()
    pw.enqueue()
    for i in range(4):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del graphs
    return ms


# ---------------------------------------------------------------- CPU-baseline leg
# Everything below that touches oracle/ runs only in this leg.

def cpu_baseline(prob, L_total, seconds=10.0, max_reps=200):
    from oracle import oracle as O
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    threads = max(1, min(threads, len(os.sched_getaffinity(0))))
    reps, t0 = 0, time.perf_counter()
    while True:
        O.verify_problem(prob, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= max_reps:
            break
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": reps * L_total / el, "unit": "verified draft positions/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the full headline step ({prob.w.B} sequences, {L_total} verified positions) run {reps} times "
                      f"in {el:.2f} s on the host CPU ({cpu_model})"}


def timed_inputs_check(probs, outs):
    """The oracle on the exact inputs that were timed: emitted tokens, accepted
    and verify lengths must match for every sequence outside the oracle's
    margins (a margin sequence is counted; at a CDF-gap margin the final token
    may be either one across the step)."""
    from oracle import oracle as O
    n = mism = margin = 0
    for prob, g in zip(probs, outs):
        orc = O.verify_problem(prob)
        for i, b in enumerate(orc.seq):
            n += 1
            a, tok = int(orc.accepted_len[i]), orc.out_tokens[i]
            lengths = (int(g["accepted_len"][b]) == a and int(g["verify_len_out"][b]) == int(orc.verify_len[i]))
            m = int(orc.margin[i])
            if m == 0:
                same = lengths and np.array_equal(g["out_tokens"][b], tok)
            elif m == O.MARGIN_CDF:
                margin += 1
                gt = g["out_tokens"][b]
                same = (lengths and np.array_equal(gt[:a], tok[:a]) and np.all(gt[a + 1:] == -1)
                        and int(gt[a]) in (int(tok[a]), int(orc.alt_token[i])))
            else:
                margin += 1
                continue
            mism += 0 if same else 1
    return {"sequences": n, "margin_cases": margin, "mismatches": mism,
            "rule": "outside the oracle's margins emitted tokens and lengths equal; at a CDF-gap margin "
                    "lengths and prefix equal and the final token is one of the two across the step"}


# inputs and GPU outputs of the later legs, for the oracle in the CPU-baseline leg
LEG_DATA = {}


def _timed(fn, seconds):
    reps, t0 = 0, time.perf_counter()
    while True:
        r = fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            return r, el / reps


def next_rows_oracle(seconds=2.0):
    """The oracle on each later leg's inputs (the one-hot and packed verify
    steps, the admission decision, the calibrated confidences): its time per
    call on the host, and whether the GPU's outputs match it."""
    from oracle import oracle as O
    threads = len(os.sched_getaffinity(0))
    res = {}
    if "onehot" in LEG_DATA:
        probs, outs = LEG_DATA["onehot"]
        chk = timed_inputs_check(probs, outs)
        _, sec = _timed(lambda: O.verify_problem(probs[0], threads=threads), seconds)
        L = int(outs[0]["verify_len_out"].sum())
        res["onehot"] = {"value": L / sec, "unit": "verified draft positions/s", "s_per_step": sec,
                         "cores": threads, "vs_gpu": chk}
    if "packed" in LEG_DATA:
        probs, outs = LEG_DATA["packed"]
        chk = timed_inputs_check(probs, outs)
        _, sec = _timed(lambda: O.verify_problem(probs[0], threads=threads), seconds)
        L = float(outs[0]["verify_len_out"].sum())
        res["packed"] = {"value": L / sec, "unit": "verified draft positions/s", "s_per_step": sec,
                         "cores": threads, "vs_gpu": chk}
    if "admission" in LEG_DATA:
        conf, speed, vl, adm = LEG_DATA["admission"]
        r, sec = _timed(lambda: O.schedule(conf, speed), seconds)
        res["admission"] = {"us_per_call": sec * 1e6, "cores": 1, "margin": bool(r.margin),
                            "vs_gpu": {"verify_len_equal": bool(np.array_equal(r.verify_len, vl)),
                                       "admitted_equal": int(r.admitted) == adm}}
    if "confidence" in LEG_DATA:
        z, T, got = LEG_DATA["confidence"]
        steps = [z.astype(np.float32)] * 3
        r, sec = _timed(lambda: O.calibrated_confidence_steps(steps, T, delay=2, c_default=0.0), seconds)
        _, handed, _ = r
        want = np.asarray(handed[-1], np.float32)  # the third call hands over the first call's value
        ulp = np.abs(got.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
        res["confidence"] = {"us_per_call": sec * 1e6 / 3, "cores": 1,
                             "vs_gpu": {"max_ulp": int(ulp.max()), "within_1_ulp": bool(ulp.max() <= 1)}}
    return res


def cpu_single_thread(seconds=2.0):
    """The oracle on one host thread for the two small workloads (tiny: B=4
    K=4 V=1024 fp32; zipf64: B=64 K=8 V=129280 bf16), about `seconds` each."""
    from oracle import oracle as O
    from synth import synth
    out = {}
    for name in ("tiny", "zipf64"):
        prob = synth.make_problem(synth.WORKLOADS[name])
        reps, t0 = 0, time.perf_counter()
        while True:
            r = O.verify_problem(prob, threads=1)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds or reps >= 2000:
                break
        L = int(np.asarray(r.verify_len).sum())
        w = prob.w
        out[name] = {"us_per_step": el / reps * 1e6, "verified_positions_per_s": reps * L / el, "threads": 1,
                     "B": w.B, "K": w.K, "V": w.V, "steps": reps}
    return out


# ---------------------------------------------------------------- later rows' legs

def time_onehot(torch, B, D, synth, steps, warmup, pw):
    """One-hot drafts (q_j = point mass at x_j; no draft logits handed over) on
    peaked rows where a greedy drafter is worth verifying: B=256 K=16 V=129280
    bf16, target -1.3 ln(rank) + N(0, 0.3) at T = 0.7, drafted token = the
    largest value of target + N(0, 0.2), every position verified."""
    base = synth.WORKLOADS["peaked512"].with_(B=256, dtype=synth.BF16, length_mode=0, token_mode=2, draft_mode=1)
    probs = [synth.make_problem(base.with_(seed=7 + s)) for s in (0, 1000)]
    entry, outs = measure(torch, B, D, probs, steps, warmup, pw)
    entry["traffic"] = traffic_entry(kernel_source_hash(), "onehot")
    entry["workload"] = ("one-hot drafts (greedy drafter) on peaked rows: B=256 K=16 V=129280 bf16, "
                         "Zipf(1.3)+N(0,0.3) at T=0.7, draft noise 0.2, L=16; target rows only")
    LEG_DATA["onehot"] = (probs, outs)
    return entry


def time_packed(torch, B, D, synth, steps, warmup, pw):
    """Admission then verification, as an engine would chain them: the GPU
    scheduler picks L_b from seeded confidences (same shape as the headline
    workload), the target and draft logits then hold only the admitted rows
    (packed, with row offsets), and the verify step runs on them.  The dense
    layout at the same L_b is timed beside it."""
    base = synth.WORKLOADS["sched256"].with_(length_mode=0, tau_choices=())
    Bn, K = base.B, base.K
    conf, speed = synth.admission_inputs(0, Bn, K)
    sv = B.SpecVerify(Bn, K, base.V, base.dtype, 0)
    dev = torch.device("cuda")
    vl = torch.empty(Bn, dtype=torch.int32, device=dev)
    sv.schedule(B.make_sched_args(Bn, K, confidence=torch.from_numpy(conf).to(dev),
                                  speed=torch.from_numpy(speed).to(dev), n_speed=speed.size, verify_len_out=vl))
    L = vl.cpu().numpy()
    sv.close()
    out = {"admitted": int(L.sum()), "mean_L": float(L.mean())}
    probs = []
    for s in (0, 1000):
        prob = synth.make_problem(base.with_(seed=3 + s))
        prob.verify_len = L.astype(np.int32)
        probs.append(prob)
    # the engine knows its lengths once it has built the verify batch: every
    # call but "packed_no_bound" passes their maximum as max_verify_len
    out["max_verify_len"] = int(L.max())
    for layout in ("packed", "dense", "packed_no_bound"):
        dps = [D.packed_from_problem(p, L, diagnostics=False) if layout != "dense"
               else D.from_problem(p, diagnostics=False) for p in probs]
        for d in dps:
            d.max_verify_len = 0 if layout == "packed_no_bound" else int(L.max())
        sv = B.SpecVerify(Bn, K, base.V, base.dtype, 0)
        argv = [d.args(counts=False) for d in dps]
        ms = time_block(torch, sv, argv, steps, warmup, pw)
        kt = kernel_times(torch, sv, argv, steps, pw)
        outs = count_pass(torch, sv, dps)
        sv.close()
        if layout == "packed_no_bound":
            out[layout] = {"ms_per_step": ms, "kernel_avg_ms": kt}
            del dps, argv, outs
            torch.cuda.empty_cache()
            continue
        bc = [byte_counts(o, p) for o, p in zip(outs, probs)]
        needed = sum(c["needed"] for c in bc) / 2.0
        streamed = sum(c["streamed"] for c in bc) / 2.0
        if layout == "packed":
            LEG_DATA["packed"] = (probs, outs)
        out[layout] = {"ms_per_step": ms, "value": float(L.sum()) / (ms / 1e3),
                       "needed_bytes_per_step": needed, "streamed_bytes_per_step": streamed,
                       "frac": needed / (kt[DOMINANT] / 1e3) / 1e9 / PEAK_HBM_GBPS,
                       "step_frac": needed / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS,
                       "kernel_avg_ms": kt,
                       "traffic": traffic_entry(kernel_source_hash(),
                                                "packed" if layout == "packed" else "dense_same_lengths"),
                       "logit_bytes_held": sum(int(d.target.numel() * d.target.element_size()) + (
                           int(d.draft.numel() * d.draft.element_size()) if d.draft is not None else 0)
                           for d in dps) / 2.0}
        del dps, argv, outs
        torch.cuda.empty_cache()
    out["unit"] = "verified draft positions/s"
    out["workload"] = ("B=256 K=16 V=129280 bf16 rows as the headline workload; L_b chosen by spec_verify_schedule "
                       "from seeded confidences and step time 20 + 0.05 n")
    return out


def time_confidence(sv, torch, B, synth, Bn, K, steps, warmup):
    """Time one step of calibrated, causally delayed confidences
    (spec_verify_confidence, delay 2) on the same batch shape."""
    dev = torch.device("cuda")
    z = torch.from_numpy((4.0 * synth.uniforms(600, Bn * K) - 2.0).reshape(Bn, K)).to(dev)
    T = torch.from_numpy(np.linspace(0.8, 1.6, K).astype(np.float32)).to(dev)
    out = torch.empty((Bn, K), dtype=torch.float32, device=dev)
    a = B.make_conf_args(Bn, K, conf_logits=z, temperature=T, conf_out=out, delay=2, c_default=0.0)
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(max(warmup, 3)):
        sv.confidence(a, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        sv.confidence(a, stream)
    e1.record()
    torch.cuda.synchronize()
    LEG_DATA["confidence"] = (z.cpu().numpy(), T.cpu().numpy(), out.cpu().numpy())
    return {"us_per_call": e0.elapsed_time(e1) / steps * 1e3, "B": Bn, "K": K, "delay": 2,
            "inputs": "logits uniform in [-2, 2) (Philox key 600), temperatures 0.8 .. 1.6"}


def time_admission(sv, torch, B, synth, Bn, K, steps, warmup):
    """Time the load-aware admission decision (spec_verify_schedule) on the
    same batch shape: seeded confidences and a linear step-time curve."""
    conf, speed = synth.admission_inputs(0, Bn, K)
    dev = torch.device("cuda")
    c_d = torch.from_numpy(conf).to(dev)
    s_d = torch.from_numpy(speed).to(dev)
    vl = torch.empty(Bn, dtype=torch.int32, device=dev)
    adm = torch.empty(1, dtype=torch.int32, device=dev)
    a = B.make_sched_args(Bn, K, confidence=c_d, speed=s_d, n_speed=speed.size, verify_len_out=vl, admitted=adm)
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(max(warmup, 3)):
        sv.schedule(a, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        sv.schedule(a, stream)
    e1.record()
    torch.cuda.synchronize()
    LEG_DATA["admission"] = (conf, speed, vl.cpu().numpy(), int(adm.item()))
    return {"us_per_call": e0.elapsed_time(e1) / steps * 1e3, "B": Bn, "K": K, "candidates": Bn * K,
            "admitted": int(adm.item()),
            "inputs": "confidences uniform in [0.3, 1) (Philox key 500), step time 20 + 0.05 n"}


def copy_rate(torch, n=1 << 30, reps=10):
    """A plain device copy of n bytes (torch's copy kernel): bytes read and
    written per ms, a measured ceiling beside the published 8 TB/s."""
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del src, dst
    return {"copy_bytes_read": n, "copy_bytes_written": n, "ms": ms, "gbps_rw": 2 * n / ms / 1e6}


def idle_probe(gaps, steps):
    """Step times of the headline workload in ranges of consecutive steps, each
    burst started after the given idle gap (ms) following 50 ms of copies."""
    import torch
    from draft_verification_amd import binding as B
    from draft_verification_amd import device as D
    from synth import synth
    probs = [synth.make_problem(workload(synth, "sched256", 0.0, s)) for s in (0, 1000)]
    w = probs[0].w
    dps = [D.from_problem(p, diagnostics=False) for p in probs]
    argv = [d.args(counts=False) for d in dps]
    sv = B.SpecVerify(w.B, w.K, w.V, w.dtype, 0)
    stream = torch.cuda.current_stream().cuda_stream
    sv.run(argv[0], stream)
    torch.cuda.synchronize()
    pw = Prewarm(torch)
    ranges = [(0, 5), (5, 25), (25, 50), (50, 100), (100, steps)]
    out = []
    for gap in gaps:
        pw.enqueue()
        torch.cuda.synchronize()
        time.sleep(gap / 1e3)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        evs[0].record()
        for i in range(steps):
            sv.run(argv[i % 2], stream)
            evs[i + 1].record()
        torch.cuda.synchronize()
        t = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(steps)])
        row = {"idle_gap_ms": gap, "mean_us": {f"{lo}-{hi}": float(t[lo:hi].mean()) for lo, hi in ranges if hi > lo}}
        log(f"[idle-probe] {json.dumps(row)}")
        out.append(row)
    sv.close()
    print(json.dumps({"idle_probe": out, "steps": steps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=("all", "headline"), default="all")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--idle-probe", type=str, default=None)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(sequences are independent, so a batch would shard across GPUs with no exchange; this run has one GPU).",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        import torch
        print(json.dumps(copy_rate(torch)))
        return
    if args.idle_probe is not None:
        idle_probe([float(x) for x in args.idle_probe.split(",")], max(args.steps, 100))
        return

    import torch
    from draft_verification_amd import binding as B
    from draft_verification_amd import device as D
    from synth import synth

    cpu = not args.no_cpu_baseline
    pw = Prewarm(torch)
    configs = {}
    head_probs = head_outs = None
    order = [c for c in CONFIGS if args.only == "all" or c[0] in (HEADLINE,)]
    # the headline first; then the rest, reusing the tensors of a config and its tau = 0 shadow
    order.sort(key=lambda c: c[0] != HEADLINE)
    cache = {}  # base workload -> its two input sets as written (a config and its tau = 0 shadow share them)
    for n, (key, base, tau, desc) in enumerate(order):
        t0 = time.perf_counter()
        if base not in cache:
            cache[base] = [synth.make_problem(workload(synth, base, None, s)) for s in (0, 1000)]
        probs = [with_tau(p, tau) for p in cache[base]] if tau is not None else cache[base]
        if not any(c[1] == base for c in order[n + 1:]):
            del cache[base]
        log(f"[bench] {key}: inputs ready in {time.perf_counter() - t0:.1f} s")
        entry, outs = measure(torch, B, D, probs, args.steps, args.warmup, pw, extra=(key == HEADLINE))
        entry["workload"] = desc
        if cpu:
            entry["oracle_agreement"] = timed_inputs_check(probs, outs)
        configs[key] = entry
        log(f"[bench] {key}: {entry['ms_per_step'] * 1e3:.1f} us/step, frac {entry['frac']:.3f}, "
            f"step_frac {entry['step_frac']:.3f}")
        if key == HEADLINE:
            head_probs, head_outs = probs, outs
        del probs, outs
    head = configs[HEADLINE]

    legs = {}
    if args.only == "all":
        w = head_probs[0].w
        sv = B.SpecVerify(w.B, w.K, w.V, w.dtype, 0)
        legs["admission"] = time_admission(sv, torch, B, synth, w.B, w.K, args.steps, args.warmup)
        legs["confidence"] = time_confidence(sv, torch, B, synth, w.B, w.K, args.steps, args.warmup)
        sv.close()
        legs["onehot"] = time_onehot(torch, B, D, synth, args.steps, args.warmup, pw)
        legs["packed"] = time_packed(torch, B, D, synth, args.steps, args.warmup, pw)
    ceiling = copy_rate(torch)
    pw_desc = pw.describe()
    pw.close()

    src_hash = kernel_source_hash()
    dom_ms = head["kernel_avg_ms"][DOMINANT]
    needed = head["needed_bytes_per_step"]
    achieved = needed / (dom_ms / 1e3) / 1e9
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "verified draft positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded generator; no dataset)",
        "config": {"workload": "confidence-scheduled verify, every position verified: B=256 K=16 V=129280 "
                               "bf16 logits, T=1, c=max draft prob, tau=0 (L=16)",
                   "B": head["B"], "K": head["K"], "V": head["V"], "logits": "bf16",
                   "arithmetic": "fp32 per-token exponentials, fp64 merges, ratios and prefix sums",
                   "temperature": head["temperature"], "tau": 0.0, "input_sets": 2},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic_entry(src_hash),
                     "kernel": DOMINANT, "kernel_avg_ms": dom_ms, "launches_per_step": 1,
                     "algorithmic_bytes_per_launch": needed,
                     "algorithmic_bytes": "the bytes the outputs depend on: target rows 1..a+1, the draft rows "
                                          "of the tested positions and those the length rule reads, each once, "
                                          "plus per-position inputs and the outputs",
                     "step_frac": head["step_frac"],
                     "step_achieved": needed / (head["ms_per_step"] / 1e3) / 1e9,
                     "streamed_bytes_per_launch": head["streamed_bytes_per_step"],
                     "streamed_over_needed": head["streamed_over_needed"],
                     "window_bytes_per_launch": head["window_bytes_per_step"],
                     "traffic_source": "rocprofv3 FETCH_SIZE + WRITE_SIZE of the sv_stream launch, copy-"
                                       "calibrated, bytes per step; null when the kernel source changed since "
                                       "the counters were taken"},
        "step_ms_distribution": head.get("step_ms_distribution"),
        "idle_start_ms_per_step": head.get("idle_start_ms_per_step"),
        "graph_replay_ms_per_step": head.get("graph_replay_ms_per_step"),
        "prewarm": pw_desc,
        "copy_ceiling": {"gbps_rw": ceiling["gbps_rw"], "bytes": 2 * ceiling["copy_bytes_read"],
                         "what": "torch device copy of 1 GiB, (read + write bytes) / time"},
        "emitted_tokens_per_s": head["emitted_tokens_per_s"],
        "mean_accepted": head["mean_accepted"],
        "kernel_avg_ms": head["kernel_avg_ms"],
        "kernel_src_sha": src_hash,
        "configs": {k: {kk: vv for kk, vv in v.items()
                        if kk not in ("step_ms_distribution", "idle_start_ms_per_step", "graph_replay_ms_per_step")}
                    for k, v in configs.items()},
    }
    out.update(legs)
    if cpu:
        log("[bench] timing the CPU oracle on the headline workload ...")
        L_total = int(head_outs[0]["verify_len_out"].sum()) if head_outs is not None else 0
        out["cpu_baseline"] = cpu_baseline(head_probs[0], L_total)
        out["cpu_baseline"]["single_thread"] = cpu_single_thread()
        out["cpu_baseline"]["next_rows"] = next_rows_oracle()
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
