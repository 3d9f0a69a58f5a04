#!/usr/bin/env python3
"""Benchmark of the Mamba-2 streaming-state hot path on one MI355X.

One bench step is one pass of every path over one batch of synthetic input:
  decode   256 slots x (H=128, P=64, N=128) fp32 state, one token each, seeded
           per-slot resets (p = 0.02)                                  [headline]
  replay   ReplaySSM verify of 5 in-flight tokens (real + 4 drafts, p = 0.7)
           per slot, window 16, then commit
  copy     the copy-state-per-draft baseline of the same verify, then commit
  prefill  one 65,536-token chunk of 8 packed bf16 sequences (H=128, P=64,
           N=128), resets at sequence starts, final states as checkpoints
The K timed steps run path by path (K decode steps, then K verify steps, and
so on: the same work as K interleaved steps), so that every path is timed in
its own steady state.  Each path is timed with events on the stream it runs
on; ``value`` is the decode state bandwidth (algorithmic state + input + output bytes per step
divided by the decode kernel time).  Replay windows 8 and 32, the
Mamba-130M-shaped chunked streaming layer and the CPU oracle are measured
beside the steps.  Prints ONE JSON line.
"""
import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MIB = 1 << 20


# HBM bytes of the decode kernel from two rocprofv3 --pmc passes (FETCH_SIZE,
# then WRITE_SIZE, KiB per dispatch, mean of the 6 dispatches of
# `bench.py --only decode --steps 5 --warmup 1`), each scaled by what the same
# counter reads for a plain copy kernel of known size (ssm_state_init: 4 MiB
# read + 4 MiB written per dispatch, `bench.py --only calib`).  Valid only for
# the kernel sources they were taken on: a change to any of them turns the
# figure into null until the counters are taken again.
DECODE_COUNTERS = {
    "sources": ["ssm_decode.hip", "ssm_device.h", "ssm_internal.h"],
    "sha256": "621f66d038b53276cb419095e90120d9d758a8fb2d947a36d25f9d51f82fb833",
    "fetch_kib": 519888.57, "write_kib": 1056770.82,
    "calib_fetch_kib": 2059.01, "calib_write_kib": 4096.0, "calib_true_kib": 4096.0,
    "algorithmic_kib": 1035989.33 + 1056768.0,
}


# The same for scan_ssd_pair_kernel on the 65,536-token prefill (mean per dispatch
# over 6 dispatches): MFMA busy cycles summed over all SIMDs, GPU-active
# cycles summed over the 8 XCDs, bf16 MFMA operations (x512 = flops), and the
# HBM counters with the copy calibration above.
PREFILL_COUNTERS = {
    "sources": ["ssm_ssd_pair.hip", "ssm_device.h", "ssm_internal.h"],
    "sha256": "832afb19a52f45ded11133edf7e26b117602a38b8376c7a08f3164a611369340",
    "mfma_busy_cycles": 361070592.0, "gui_active_cycles": 13773072.5, "xcds": 8, "simds": 1024,
    "mfma_mops_bf16": 722141184.0,
    "fetch_kib": 721082.55, "write_kib": 1114124.34,
    # x in and y out (bf16), dt, B, C (bf16), and each sequence's final state
    # twice (into its slot and as a checkpoint)
    "algorithmic_bytes": 2 * 2**30 + 3 * 2**24 + 2 * 2**25,
}

# The same for replay_kernel at W = 16 (mean over the 6 verify steps of
# "--only replay --steps 5 --warmup 1"; the algorithmic bytes of exactly those
# steps, from the log lengths, averaged).
REPLAY_COUNTERS = {
    "sources": ["ssm_kernels.hip", "ssm_device.h", "ssm_internal.h"],
    "sha256": "d751269df3d1ca1d99cee37bfc9298555699eb0ea15f7e508e31d311448b2f61",
    "fetch_kib": 577003.33, "write_kib": 208613.47,
    "algorithmic_bytes": 1375888554.67,
}


def _sources_match(c):
    import hashlib
    h = hashlib.sha256()
    for f in c["sources"]:
        with open(os.path.join(ROOT, "streaming_state_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest() == c["sha256"]


def prefill_counters():
    """MFMA utilisation and scaled HBM bytes of one prefill launch from the
    recorded counters, or None if the kernel changed since they were taken."""
    c, d = PREFILL_COUNTERS, DECODE_COUNTERS
    if not _sources_match(c):
        return None
    per_xcd = c["gui_active_cycles"] / c["xcds"]
    kib = (c["fetch_kib"] * d["calib_true_kib"] / d["calib_fetch_kib"]
           + c["write_kib"] * d["calib_true_kib"] / d["calib_write_kib"])
    return {"mfma_busy_frac": round(c["mfma_busy_cycles"] / (per_xcd * c["simds"]), 4),
            "mfma_flops_executed": c["mfma_mops_bf16"] * 512,
            "traffic": round(kib * 1024),
            "traffic_over_algorithmic": round(kib * 1024 / c["algorithmic_bytes"], 4)}


def replay_counter_traffic():
    """Scaled HBM bytes per replay_kernel launch over its algorithmic bytes,
    or None if the kernel changed since the counters were taken."""
    c, d = REPLAY_COUNTERS, DECODE_COUNTERS
    if not _sources_match(c):
        return None
    kib = (c["fetch_kib"] * d["calib_true_kib"] / d["calib_fetch_kib"]
           + c["write_kib"] * d["calib_true_kib"] / d["calib_write_kib"])
    return round(kib * 1024 / c["algorithmic_bytes"], 4)


def counter_traffic():
    """Scaled HBM bytes per decode launch, or None if the kernel changed."""
    c = DECODE_COUNTERS
    if not _sources_match(c):
        return None, None
    kib = (c["fetch_kib"] * c["calib_true_kib"] / c["calib_fetch_kib"]
           + c["write_kib"] * c["calib_true_kib"] / c["calib_write_kib"])
    return round(kib * 1024), round(kib / c["algorithmic_kib"], 4)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--only", default="", help="comma list of decode,replay,copy,prefill,conv,gdn (profiling)")
    ap.add_argument("--skip-extras", action="store_true")
    return ap.parse_args()


class Timer:
    """Events around launches on the current stream; mean of the recorded pairs."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, e0):
        e1 = self.torch.cuda.Event(enable_timing=True)
        e1.record()
        self.pairs.append((e0, e1))

    def ms(self):
        return [a.elapsed_time(b) for a, b in self.pairs]


class LogMirror:
    """Replay log lengths per slot, mirrored on the host from the accept
    counts (the library's rule: a step whose committed entries plus its n_in
    in-flight tokens exceed W folds the log first and restarts it empty), so
    that a step's algorithmic bytes need no library query between timed
    launches.  check() compares the mirror with the library afterwards."""

    def __init__(self, n_slots, W, n_in):
        self.W, self.n_in = W, n_in
        self.lens = np.zeros(n_slots, np.int64)

    def step_bytes(self, state_b, entry_b, io_b):
        """Checkpoint read; the committed log read (a fold reads it to fold
        it, otherwise the outputs read it); on a fold the checkpoint written;
        the n_in in-flight entries appended; in-flight inputs and outputs."""
        fold = self.lens + self.n_in > self.W
        per = state_b + (self.lens + self.n_in) * entry_b + io_b + fold * state_b
        return int(per.sum())

    def commit(self, acc):
        fold = self.lens + self.n_in > self.W
        self.lens = np.where(fold, 0, self.lens) + np.asarray(acc, np.int64)

    def check(self, r):
        got = np.array([r.log_state(b)[0] for b in range(len(self.lens))])
        assert (got == self.lens).all(), "log length mirror disagrees with the library"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(decode and replay would shard by batch or head with no exchange; one GPU's "
              "share is the workload measured here)",
              file=sys.stderr)
        sys.exit(2)
    # child processes that use the GPU run before this process initialises it
    devinfo = device_info()
    abi_lat = None if (args.skip_extras or args.only) else abi_latency()
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from streaming_state_amd import inputs
    from streaming_state_amd import ssm
    only = set(filter(None, args.only.split(",")))
    want = (lambda k: (not only and k != "calib") or k in only)
    if want("calib"):
        return calib_copy(torch, ssm, args)
    K, Wm = args.steps, args.warmup
    dev = "cuda"

    # ------------------------------------------------------------ decode setup
    w2 = inputs.W2
    Bd, H, P, N, G = w2["batch"], w2["H"], w2["P"], w2["N"], w2["G"]
    A2, D2 = inputs.params(2, H)
    dec = ssm.StreamState(H, P, N, Bd, torch.from_numpy(A2).to(dev),
                          torch.from_numpy(D2).to(dev), G=G)
    dec.init(np.arange(Bd), inputs.device_state(2, Bd, H, P, N))
    dec_slots = inputs.slot_permutation(2, Bd, Bd)
    n_dec_inputs = w2["steps"]
    dec_in = [inputs.device_tokens(2, Bd, H, P, N, G, seed_extra=s) for s in range(n_dec_inputs)]
    dec_reset = [inputs.device_resets(2, s, Bd) for s in range(n_dec_inputs)]
    state_b = H * P * N * 4

    def dec_bytes(reset):
        nr = int(reset.sum())
        st = (Bd - nr) * state_b + Bd * state_b
        io = Bd * (H * P * 4 * 2 + H * 4 + 2 * G * N * 4)
        return st + io, st

    # ------------------------------------------------------------ replay setup
    w3 = inputs.W3
    n_in = w3["T"] + 1
    A3, D3 = inputs.params(3, H)
    acc_all = inputs.acceptances(w3["steps"], Bd, T=w3["T"], p=w3["p"])
    spec_in = []
    for s in range(8):
        x, dt, B, C = inputs.device_tokens(3, Bd * n_in, H, P, N, G, seed_extra=s)
        spec_in.append((x.view(Bd, n_in, H, P), dt.view(Bd, n_in, H), B.view(Bd, n_in, G, N),
                        C.view(Bd, n_in, G, N)))
    init3 = inputs.device_state(3, Bd, H, P, N)

    def make_replay(W):
        r = ssm.StreamState(H, P, N, Bd, torch.from_numpy(A3).to(dev),
                            torch.from_numpy(D3).to(dev), G=G)
        r.init(np.arange(Bd), init3)
        r.replay_attach(W)
        return r

    rep16 = make_replay(16) if want("replay") else None
    cop = None
    if want("copy"):
        cop = ssm.StreamState(H, P, N, Bd, torch.from_numpy(A3).to(dev),
                              torch.from_numpy(D3).to(dev), G=G)
        cop.init(np.arange(Bd), init3)
        cop.copy_attach(n_in)
    slots3 = np.arange(Bd, dtype=np.int32)

    # ----------------------------------------------------------- prefill setup
    w4 = inputs.W4
    L4 = w4["L"]
    pre = None
    if want("prefill"):
        d4 = inputs.device_prefill(L4, H, P, N, G)
        lengths = inputs.sequence_lengths()
        reset4, cu4, ends4 = inputs.packed_layout(lengths)
        nseq4 = len(lengths)
        pre = ssm.StreamState(H, P, N, nseq4, d4["A"], d4["D"], G=G, io_dtype="bf16")
        pre.reset(list(range(nseq4)))
        slots4 = np.arange(nseq4, dtype=np.int32)
        cu4 = cu4.astype(np.int32)
        y4 = torch.empty((L4, H, P), dtype=torch.bfloat16, device=dev)
        ck4 = torch.empty((nseq4, H, P, N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log("setup done")

    t_dec, t_rep, t_cop, t_pre = (Timer(torch) for _ in range(4))
    y_dec = torch.empty((Bd, H, P), dtype=torch.float32, device=dev)
    y_spec = torch.empty((Bd, n_in, H, P), dtype=torch.float32, device=dev)
    step_bytes, step_state_bytes = [], []
    flushes_before = 0

    rep_bytes, rep_bytes_all = [], []
    entry_b = (H + H * P + G * N) * 4   # one log entry: dt[H], x[H,P], B[G,N]
    io_b = n_in * (2 * H * P + H + 2 * G * N) * 4  # in-flight x, dt, B, C in; y out

    mir16 = LogMirror(Bd, 16, n_in)

    # One step runs every path once.  The K timed steps run path by path
    # (K decode steps, then K verify steps, ...) so that each path is timed in
    # its own steady state rather than behind another path's memory traffic;
    # the work timed is the same K passes of every path.
    def run_decode(s, timed):
        i = s % n_dec_inputs
        e = t_dec.start() if timed else None
        dec.decode_step(dec_slots, *dec_in[i], reset=dec_reset[i], y=y_dec)
        if timed:
            t_dec.stop(e)
            b, sb = dec_bytes(dec_reset[i])
            step_bytes.append(b)
            step_state_bytes.append(sb)

    def run_replay(s, timed):
        a = acc_all[s % len(acc_all)]
        sp = spec_in[s % len(spec_in)]
        # algorithmic bytes of this verify step, from the log lengths
        rep_bytes_all.append(mir16.step_bytes(state_b, entry_b, io_b))
        if timed:
            rep_bytes.append(rep_bytes_all[-1])
        e = t_rep.start() if timed else None
        rep16.replay_step(slots3, *sp, y=y_spec)
        if timed:
            t_rep.stop(e)
        rep16.replay_commit(slots3, a)
        mir16.commit(a)

    def run_copy(s, timed):
        a = acc_all[s % len(acc_all)]
        sp = spec_in[s % len(spec_in)]
        e = t_cop.start() if timed else None
        cop.copy_step(slots3, *sp, y=y_spec)
        if timed:
            t_cop.stop(e)
        cop.copy_commit(slots3, a)

    def run_prefill(s, timed):
        e = t_pre.start() if timed else None
        # each sequence starts a fresh stream in its own slot; final states
        # land there and, as checkpoints, in ck4
        pre.scan_packed(cu4, slots4, d4["x"], d4["dt"], d4["B"], d4["C"], y=y4, final=ck4)
        if timed:
            t_pre.stop(e)

    paths = [fn for want_it, fn in ((want("decode"), run_decode), (rep16 is not None, run_replay),
                                    (cop is not None, run_copy), (pre is not None, run_prefill))
             if want_it]
    for fn in paths:
        for s in range(Wm):
            fn(s, False)
    torch.cuda.synchronize()
    log(f"warmup {Wm} done")
    if rep16 is not None:
        flushes_before = rep16.counters()["replay_flushes"]
    t0 = time.perf_counter()
    for fn in paths:
        for s in range(Wm, Wm + K):
            fn(s, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {K} steps in {wall:.3f} s")
    if rep16 is not None:
        mir16.check(rep16)

    out = {}
    comp = {}
    if want("decode"):
        ms = np.array(t_dec.ms())
        # whole-run rate: every timed step's bytes over every timed step's time
        gbps = float(np.sum(step_bytes) / (ms.sum() * 1e-3) / 1e9)
        state_gbps = float(np.sum(step_state_bytes) / (ms.sum() * 1e-3) / 1e9)
        comp["decode"] = dict(ms_mean=float(ms.mean()), ms_median=float(np.median(ms)),
                              GBps=gbps, state_GBps=state_gbps,
                              frac_hbm=gbps / HBM_PEAK_GBPS,
                              bytes_per_step=float(np.mean(step_bytes)))
    if rep16 is not None:
        ms = np.array(t_rep.ms())
        rate = float(np.sum(rep_bytes) / (ms.sum() * 1e-3))
        comp["replay_W16"] = dict(ms_mean=float(ms.mean()), ms_median=float(np.median(ms)),
                                  flushes=int(rep16.counters()["replay_flushes"] - flushes_before),
                                  bytes_per_step=float(np.mean(rep_bytes)),
                                  GBps=rate / 1e9,
                                  bytes_each_step_with_warmup=[int(b) for b in rep_bytes_all],
                                  frac_hbm=rate / 8e12,
                                  traffic_over_algorithmic_counters=replay_counter_traffic())
    if cop is not None:
        ms = np.array(t_cop.ms())
        cbytes = Bd * state_b * (1 + n_in) + Bd * n_in * (H * P * 8 + H * 4 + 2 * G * N * 4)
        comp["copy"] = dict(ms_mean=float(ms.mean()), ms_median=float(np.median(ms)),
                            GBps=float(cbytes / (ms.mean() * 1e-3) / 1e9))
        if rep16 is not None:
            comp["replay_vs_copy_speedup_W16"] = comp["copy"]["ms_mean"] / comp["replay_W16"]["ms_mean"]
    if pre is not None:
        ms = np.array(t_pre.ms())
        comp["prefill"] = dict(ms_mean=float(ms.mean()), tokens_per_s=float(L4 / (ms.mean() * 1e-3)),
                               algorithmic_GFLOP=415.1)
        tf = 415.1e9 / (ms.mean() * 1e-3) / 1e12
        comp["prefill"]["TFLOPs_algorithmic"] = tf
        pc = prefill_counters()
        comp["prefill"]["roofline"] = {
            "bound": "mfma", "kernel": "scan_ssd_pair_kernel", "achieved": round(tf, 1),
            "peak": 2500.0, "unit": "TFLOP/s", "frac": round(tf / 2500.0, 4),
            "mfma_busy_frac_counter": pc and pc["mfma_busy_frac"],
            "mfma_flops_executed": pc and pc["mfma_flops_executed"],
            "traffic": pc and pc["traffic"],
            "traffic_over_algorithmic": pc and pc["traffic_over_algorithmic"]}

    # ------------------------------------------------------------- extras
    extras = {}
    if "conv" in only:  # the steps around the scan alone (for profiling)
        extras["conv_and_gate"] = conv_gate_bench(torch, ssm, inputs, H, P, N, G, dev)
    if "gdn" in only:  # Gated DeltaNet verify alone (for profiling)
        extras["gdn_replay_vs_copy"] = gdn_bench(torch, ssm, inputs, dev)
    if not args.skip_extras and not only:
        # replay at W = 8 and 32 against the same copy baseline
        for W in (8, 32):
            r = make_replay(W)
            tm = Timer(torch)
            nst, warm = 48, 4
            wbytes = []
            mir = LogMirror(Bd, W, n_in)
            for s in range(nst + warm):
                sp = spec_in[s % len(spec_in)]
                if s >= warm:
                    wbytes.append(mir.step_bytes(state_b, entry_b, io_b))
                e = tm.start() if s >= warm else None
                r.replay_step(slots3, *sp, y=y_spec)
                if s >= warm:
                    tm.stop(e)
                r.replay_commit(slots3, acc_all[s])
                mir.commit(acc_all[s])
            torch.cuda.synchronize()
            mir.check(r)
            wms = np.array(tm.ms())
            ms = float(wms.mean())
            rate = float(np.sum(wbytes) / (wms.sum() * 1e-3))
            extras[f"replay_W{W}"] = dict(ms_mean=ms, ms_median=float(np.median(wms)),
                                          flushes=r.counters()["replay_flushes"],
                                          steps=nst + warm, timed_steps=nst,
                                          bytes_per_step=float(np.mean(wbytes)),
                                          GBps=rate / 1e9, frac_hbm=rate / 8e12)
            if cop is not None:
                extras[f"replay_vs_copy_speedup_W{W}"] = comp["copy"]["ms_mean"] / ms
            r.destroy()
            del r
        # Mamba-130M-shaped streaming layer: chunk sizes 1, 17, 64, 256 and full
        w1 = inputs.W1
        L1, H1 = w1["L"], w1["H"]
        A1, D1 = inputs.params(1, H1)
        x1, dt1, B1, C1 = inputs.device_tokens(1, L1, H1, P, N, G, seed_extra=0)
        s1 = ssm.StreamState(H1, P, N, 1, torch.from_numpy(A1).to(dev),
                             torch.from_numpy(D1).to(dev), G=G)
        y1 = torch.empty((L1, H1, P), dtype=torch.float32, device=dev)
        stream1 = {}
        for chunk, wsm in ((L1, None), (256, None), (64, None), (17, None), (1, None),
                           (L1, "serial"), (256, "serial"), (64, "serial")):
            s1.reset([0])
            sizes = [chunk] * (L1 // chunk) + ([L1 % chunk] if L1 % chunk else [])
            for rep in range(2):  # the first run warms caches
                s1.reset([0])
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                tw = time.perf_counter()
                e0.record()
                t = 0
                for q, sz in enumerate(sizes):
                    s1.scan_chunk(0, q, x1[t:t + sz], dt1[t:t + sz], B1[t:t + sz], C1[t:t + sz],
                                  y=y1[t:t + sz], workspace=wsm)
                    t += sz
                e1.record()
                torch.cuda.synchronize()
                wall1 = time.perf_counter() - tw
            gpu_ms = e0.elapsed_time(e1)
            stream1[str(chunk) + ("_serial" if wsm else "")] = dict(calls=len(sizes), tokens_per_s=L1 / (gpu_ms * 1e-3),
                                       us_per_call=gpu_ms * 1e3 / len(sizes),
                                       host_wall_us_per_call=wall1 * 1e6 / len(sizes))
        extras["stream_130m"] = stream1
        # the same calls through the C ABI with no binding in the loop
        extras["stream_130m_abi"] = abi_lat
        extras["replay_alone_vs_decode"] = replay_alone_sweep(torch, ssm, inputs, H, P, N, G, dev)
        extras["conv_and_gate"] = conv_gate_bench(torch, ssm, inputs, H, P, N, G, dev)
        extras["gdn_replay_vs_copy"] = gdn_bench(torch, ssm, inputs, dev)
        # plain device copy of 1 GiB for the achievable-bandwidth context
        a = torch.empty(256 * MIB, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        tm = Timer(torch)
        for _ in range(10):
            e = tm.start()
            b.copy_(a)
            tm.stop(e)
        torch.cuda.synchronize()
        extras["torch_copy_1GiB_GBps"] = 2 * a.numel() * 4 / (np.mean(tm.ms()) * 1e-3) / 1e9
        del a, b

    # --------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu_baseline and want("decode"):
        cpu = cpu_baseline(inputs, dec_in, dec_reset, A2, D2, Bd, H, P, N, G, args.cpu_seconds,
                           torch)

    dec_c = comp.get("decode", {})
    traffic, traffic_ratio = counter_traffic()
    total_ms = sum(v["ms_mean"] for k, v in comp.items() if isinstance(v, dict) and "ms_mean" in v)
    line = {
        "metric": "decode state GB/s (% of HBM peak) at B=256; prefill tokens/s; replay vs copy speedup",
        "value": round(dec_c.get("GBps", 0.0), 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode B=256 H=128 P=64 N=128 fp32 state, reset p=0.02; "
                               "replay/copy verify n_in=5 W=16; prefill 65536 tokens bf16",
                   "batch": Bd, "H": H, "P": P, "N": N, "prefill_tokens": L4},
        "components": comp,
        "frac_of_hbm_peak": round(dec_c.get("frac_hbm", 0.0), 4),
        "prefill_tokens_per_s": comp.get("prefill", {}).get("tokens_per_s"),
        "replay_vs_copy_speedup": {"W16": comp.get("replay_vs_copy_speedup_W16"),
                                   "W8": extras.get("replay_vs_copy_speedup_W8"),
                                   "W32": extras.get("replay_vs_copy_speedup_W32")},
        "sum_of_path_ms": round(total_ms, 4),
        "roofline": {"bound": "hbm", "achieved": round(dec_c.get("GBps", 0.0), 2),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(dec_c.get("GBps", 0.0) / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": "decode_kernel<float>",
                     "algorithmic_bytes_per_launch": dec_c.get("bytes_per_step"),
                     "traffic_over_algorithmic": traffic_ratio},
        "cpu_baseline": cpu,
        "extras": extras,
        "device": dict(devinfo, name=torch.cuda.get_device_name(0),
                       arch=getattr(torch.cuda.get_device_properties(0), "gcnArchName", None),
                       torch_multiprocessors=torch.cuda.get_device_properties(0).multi_processor_count),
    }
    print(json.dumps(line), flush=True)


def device_info():
    """Compute units and peak engine clock of the first GPU agent, as rocminfo
    reports them (the denominators of the roofline fractions assume 256 CUs at
    2.4 GHz)."""
    import subprocess
    info = {"compute_units": None, "max_clock_mhz": None, "agent": None}
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return info
    for block in out.split("*******"):
        if "Device Type:" in block and "GPU" in block.split("Device Type:", 1)[1][:40]:
            for ln in block.splitlines():
                ln = ln.strip()
                if ln.startswith("Name:") and info["agent"] is None:
                    info["agent"] = ln.split(":", 1)[1].strip()
                elif ln.startswith("Compute Unit:"):
                    info["compute_units"] = int(ln.split(":", 1)[1])
                elif ln.startswith("Max Clock Freq. (MHz):"):
                    info["max_clock_mhz"] = int(ln.split(":", 1)[1])
            break
    return info


def abi_latency():
    """Run the C-ABI latency probe (ssm_abi_latency) as a child process: per
    call of ssm_scan_chunk on the Mamba-130M-shaped layer, host time inside
    the call, host wall time to completion and device time."""
    import subprocess
    exe = os.path.join(ROOT, "streaming_state_amd", "ssm_abi_latency")
    if not os.path.exists(exe):
        return None
    try:
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    except subprocess.SubprocessError as e:
        return {"error": str(e)}
    if r.returncode != 0:
        return {"error": r.stderr.strip()[-500:]}
    return json.loads(r.stdout)


def conv_gate_bench(torch, ssm, inputs, H, P, N, G, dev, reps=10):
    """The steps around the scan at the workloads' shapes: the conv over the
    packed prefill (65,536 bf16 tokens, C = H*P + 2*G*N channels, K = 4, a
    reset at each sequence start), the conv decode step for 256 slots (fp32),
    and the gated group RMS norm over the prefill's y (bf16, one group of H*P
    channels).  Algorithmic bytes: every input read once and every output and
    state written once."""
    C, K, L, Bd = H * P + 2 * G * N, 4, 65536, 256
    A, D = inputs.params(4, H)
    At, Dt = torch.from_numpy(A).to(dev), torch.from_numpy(D).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(4)
    w = torch.randn((C, K), generator=g, device=dev) * 0.5
    b = torch.randn(C, generator=g, device=dev) * 0.1

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def line(ms, nbytes):
        return dict(ms=ms, bytes=int(nbytes), GBps=nbytes / (ms * 1e-3) / 1e9,
                    frac_hbm=nbytes / (ms * 1e-3) / 8e12)

    out = {"channels": C, "K": K}
    h = ssm.StreamState(H, P, N, 1, At, Dt, G=G, io_dtype="bf16")
    h.conv_attach(C, K, w, b, act=True)
    x = torch.randn((L, C), generator=g, device=dev).to(torch.bfloat16)
    y = torch.empty_like(x)
    lengths = inputs.sequence_lengths()
    rs = np.zeros(L, np.uint8)
    rs[np.concatenate([[0], np.cumsum(lengths)[:-1]])] = 1
    ms = timed(lambda: h.conv_chunk(0, x, reset=rs, y=y))
    out["conv_chunk_prefill"] = line(ms, 2 * L * C * 2 + 2 * C * (K - 1) * 4 + C * (K + 1) * 4)
    # gated RMS norm over y[L, H*P] with z of the same shape
    yz = torch.randn((2, L, H * P), generator=g, device=dev).to(torch.bfloat16)
    nw = torch.randn(H * P, generator=g, device=dev)
    og = torch.empty_like(yz[0])
    ms = timed(lambda: ssm.gate(yz[0], yz[1], nw, group=H * P, out=og))
    out["gate_norm_prefill"] = line(ms, 3 * L * H * P * 2 + H * P * 4)
    del x, y, yz, og
    h.destroy()
    hd = ssm.StreamState(H, P, N, Bd, At, Dt, G=G)
    hd.conv_attach(C, K, w, b, act=True)
    xd = torch.randn((Bd, C), generator=g, device=dev)
    yd = torch.empty_like(xd)
    slots = np.arange(Bd, dtype=np.int32)
    ms = timed(lambda: hd.conv_decode(slots, xd, y=yd))
    out["conv_decode_256"] = line(ms, 2 * Bd * C * (K - 1) * 4 + 2 * Bd * C * 4 + C * (K + 1) * 4)
    hd.destroy()
    return out


def gdn_bench(torch, ssm, inputs, dev, steps=48, warm=4, copy_steps=16):
    """Gated DeltaNet verify at B=256 (32 value heads over 16 key groups,
    P = N = 128, fp32 state 2 MiB per slot), n_in = 5 (p = 0.7): ReplaySSM at
    W = 8, 16, 32 against the copy-state-per-draft baseline on the same
    inputs.  Algorithmic bytes per replay step, from the log lengths: the
    checkpoint read, the checkpoint write of folding slots, the committed
    entries read (dt, beta, v, k) and the in-flight ones appended, in-flight
    inputs and outputs; per copy step: one state read and n_in state writes
    plus the same inputs and outputs."""
    w5 = inputs.W5
    Bd, H, P, N, G, T = w5["batch"], w5["H"], w5["P"], w5["N"], w5["G"], w5["T"]
    n_in = T + 1
    A = torch.from_numpy(inputs.params(5, H)[0]).to(dev)
    init = inputs.device_state(5, Bd, H, P, N)
    acc = inputs.acceptances(steps + warm, Bd, T=T, p=w5["p"], workload=5)
    toks = []
    for s in range(8):
        v, dt, beta, k, q = inputs.device_gdn_tokens(5, Bd * n_in, H, P, N, G, seed_extra=s)
        toks.append((v.view(Bd, n_in, H, P), dt.view(Bd, n_in, H), beta.view(Bd, n_in, H),
                     k.view(Bd, n_in, G, N), q.view(Bd, n_in, G, N)))
    slots = np.arange(Bd, dtype=np.int32)
    y = torch.empty((Bd, n_in, H, P), dtype=torch.float32, device=dev)
    state_b = H * P * N * 4
    entry_b = (2 * H + H * P + G * N) * 4
    io_b = n_in * (H * P + 2 * H + 2 * G * N) * 4 + n_in * H * P * 4
    out = {"batch": Bd, "H": H, "G": G, "P": P, "N": N, "n_in": n_in}
    c = ssm.StreamState(H, P, N, Bd, A, None, G=G, recurrence="gated_delta")
    c.init(slots, init)
    c.copy_attach(n_in)
    tc = Timer(torch)
    for s in range(warm + copy_steps):
        e = tc.start() if s >= warm else None
        c.gdn_copy_step(slots, *toks[s % len(toks)], y=y)
        if e is not None:
            tc.stop(e)
        c.copy_commit(slots, acc[s])
    torch.cuda.synchronize()
    cms = np.array(tc.ms())
    cbytes = Bd * (state_b * (1 + n_in) + io_b)
    out["copy"] = dict(ms_mean=float(cms.mean()), bytes_per_step=cbytes,
                       GBps=cbytes / (cms.mean() * 1e-3) / 1e9,
                       frac_hbm=cbytes / (cms.mean() * 1e-3) / 8e12)
    c.destroy()
    del c
    for W in (8, 16, 32):
        r = ssm.StreamState(H, P, N, Bd, A, None, G=G, recurrence="gated_delta")
        r.init(slots, init)
        r.replay_attach(W)
        tm, nbytes = Timer(torch), []
        mir = LogMirror(Bd, W, n_in)
        for s in range(warm + steps):
            if s >= warm:
                nbytes.append(mir.step_bytes(state_b, entry_b, io_b))
            e = tm.start() if s >= warm else None
            r.gdn_replay_step(slots, *toks[s % len(toks)], y=y)
            if e is not None:
                tm.stop(e)
            r.replay_commit(slots, acc[s])
            mir.commit(acc[s])
        torch.cuda.synchronize()
        mir.check(r)
        ms = np.array(tm.ms())
        rate = float(np.sum(nbytes) / (ms.sum() * 1e-3))
        out[f"replay_W{W}"] = dict(ms_mean=float(ms.mean()), bytes_per_step=float(np.mean(nbytes)),
                                   GBps=rate / 1e9, frac_hbm=rate / 8e12,
                                   flushes=r.counters()["replay_flushes"],
                                   speedup_vs_copy=float(cms.mean() / ms.mean()))
        r.destroy()
        del r
    del init, toks
    return out


def replay_alone_sweep(torch, ssm, inputs, H, P, N, G, dev, W=16, steps=32, warm=16):
    """ReplaySSM with one token per step (no drafts) against plain decode on the
    same inputs, per batch size: mean step time of each over `steps` steps after
    `warm` (two full windows, so the fold every W steps is included).  State
    traffic per token: decode reads and writes the state, replay reads the
    checkpoint and writes it once per window."""
    A, D = inputs.params(2, H)
    At, Dt = torch.from_numpy(A).to(dev), torch.from_numpy(D).to(dev)
    out = {}
    for Bs in (1, 16, 64, 128, 256, 512):
        init = inputs.device_state(2, Bs, H, P, N)
        dec = ssm.StreamState(H, P, N, Bs, At, Dt, G=G)
        rep = ssm.StreamState(H, P, N, Bs, At, Dt, G=G)
        dec.init(np.arange(Bs), init)
        rep.init(np.arange(Bs), init)
        rep.replay_attach(W)
        del init
        toks = [inputs.device_tokens(2, Bs, H, P, N, G, seed_extra=500 + s) for s in range(4)]
        slots = np.arange(Bs, dtype=np.int32)
        ones = np.ones(Bs, np.int32)
        yd = torch.empty((Bs, H, P), dtype=torch.float32, device=dev)
        yr = torch.empty((Bs, 1, H, P), dtype=torch.float32, device=dev)
        td, tr = Timer(torch), Timer(torch)
        for i in range(warm + steps):
            x, dt, B, C = toks[i % len(toks)]
            e = td.start() if i >= warm else None
            dec.decode_step(slots, x, dt, B, C, y=yd)
            if e is not None:
                td.stop(e)
            e = tr.start() if i >= warm else None
            rep.replay_step(slots, x.view(Bs, 1, H, P), dt.view(Bs, 1, H), B.view(Bs, 1, G, N),
                            C.view(Bs, 1, G, N), y=yr)
            if e is not None:
                tr.stop(e)
            rep.replay_commit(slots, ones)
        torch.cuda.synchronize()
        md, mr = float(np.mean(td.ms())), float(np.mean(tr.ms()))
        st = Bs * H * P * N * 4
        out[str(Bs)] = dict(decode_ms=md, replay_ms=mr, speedup=md / mr,
                            decode_state_GBps=2 * st / (md * 1e-3) / 1e9,
                            replay_state_GBps=st * (1 + 1 / W) / (mr * 1e-3) / 1e9)
        dec.destroy()
        rep.destroy()
        del dec, rep, toks, yd, yr
    out["model_state_traffic_ratio"] = 2 / (1 + 1 / W)
    return out


def calib_copy(torch, ssm, args):
    """Counter calibration: the library's state copy (ssm_state_init) of 256
    slots x 4 MiB = 1 GiB read + 1 GiB write, a plain copy kernel of known
    size.  Prints the mean kernel time; counters are read by the profiler."""
    H, P, N, S = 128, 64, 128, 256
    A = torch.full((H,), -1.0, device="cuda")
    D = torch.zeros(H, device="cuda")
    h = ssm.StreamState(H, P, N, S, A, D)
    src = torch.ones((S, H, P, N), device="cuda")
    tm = Timer(torch)
    for i in range(args.warmup + args.steps):
        e = tm.start() if i >= args.warmup else None
        h.init(list(range(S)), src)
        if e is not None:
            tm.stop(e)
    torch.cuda.synchronize()
    ms = float(np.mean(tm.ms()))
    print(json.dumps({"calib": "copy_f32_kernel", "bytes_read": S * H * P * N * 4,
                      "bytes_written": S * H * P * N * 4, "ms": ms,
                      "GBps": 2 * S * H * P * N * 4 / (ms * 1e-3) / 1e9}), flush=True)


def cpu_baseline(inputs, dec_in, dec_reset, A, D, Bd, H, P, N, G, seconds, torch):
    """The fp64 oracle's decode on host cores over whole decode steps of the same
    workload (all 256 slots, all heads), as many as fit in ``seconds``."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    state = np.zeros((Bd, H, P, N))
    pos = np.zeros(Bd, np.int64)
    slots = np.arange(Bd, dtype=np.int32)
    done, bytes_, t_used = 0, 0.0, 0.0
    host_in = {}
    # cycle through the workload's decode steps until the time budget is used
    while t_used < seconds and done < 100000:
        i = done % len(dec_in)
        if i not in host_in:
            host_in[i] = tuple(t.cpu().numpy() for t in dec_in[i])
        x, dt, B, C = host_in[i]
        reset = dec_reset[i]
        t0 = time.perf_counter()
        oracle.decode(state, pos, slots, x, dt, B, C, A, D, reset=reset, n_threads=cores)
        t_used += time.perf_counter() - t0
        nr = int(reset.sum())
        bytes_ += (Bd - nr) * H * P * N * 4 + Bd * H * P * N * 4 + \
            Bd * (H * P * 8 + H * 4 + 2 * G * N * 4)
        done += 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(bytes_ / t_used / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{done} full decode steps (256 slots x 128 heads, fp64; the workload's "
                      f"{len(dec_in)} step inputs cycled) in {t_used:.1f} s; "
                      f"fp32-equivalent state bytes; {model}; {platform.machine()}"}


if __name__ == "__main__":
    main()
