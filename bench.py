#!/usr/bin/env python3
"""Benchmark of the GDN ring spec-verify step on one MI355X.

Workload: one Qwen3-Next-shaped GDN layer, B=256 rows over 512 state slots
(fp32 checkpoint S[512,32,128,128] = 1.07 GB), H=16 qk-heads, HV=32 value
heads, K=V=128, T=4 drafts, ring L=64, bf16 activations; seeded synthetic
inputs with random ring cursors (history pre-filled through the library's own
verify).  A step is the whole hot path for one batch: exact fold of the rows
flagged for flush, the ring verify (outputs of all T drafts + ring write),
and the cursor advance by synthetic accept counts U{0..T}.

Prints one JSON line: draft tokens/s per layer, the verify kernel's achieved
HBM GB/s against the 8 TB/s peak (algorithmic bytes / event-timed duration),
the snapshot baseline, the fold-every-commit and d-cache designs for
comparison, the per-channel-gate (KDA) layer on the same workload (bound by
the fp32 vector ALU), the 48-layer B=128 stack's whole-step latency and
memory, and the fp64 CPU oracle's rate at B=256 and B=32.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "qwen3next_b256"
HBM_PEAK_GBS = 8000.0
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "verify_kernel_qwen3next_b256.md")
VERIFY_SRC = os.path.join(ROOT, "linear_attention_speculative_spec_amd", "csrc", "gdn_verify.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # long enough for the clocks to settle (the first few milliseconds of
    # work run measurably slower)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=1002)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-snapshot", action="store_true")
    ap.add_argument("--no-dcache", action="store_true",
                    help="skip the comparison with the d-cache verify")
    ap.add_argument("--no-fold-every-commit", action="store_true",
                    help="skip the comparison with the fold-every-commit design")
    ap.add_argument("--no-kda", action="store_true",
                    help="skip the per-channel-gate (KDA) layer leg")
    ap.add_argument("--no-chain", action="store_true",
                    help="skip the 48-layer whole-stack leg")
    ap.add_argument("--no-interleaved", action="store_true",
                    help="skip the raw-replay / d-cache comparison on fixed state that follows "
                         "the d-cache leg")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall-clock budget of the CPU oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run a plain device copy of COPY_BYTES "
                         "(the reference for scaling the HBM byte counters)")
    ap.add_argument("--summarize-kda-profile", metavar="DIR",
                    help="no GPU work: write the KDA kernel's profile summary from the rocprofv3 "
                         "CSVs under DIR/kt and DIR/alu")
    ap.add_argument("--summarize-dcache-profile", metavar="DIR",
                    help="no GPU work: write the d-cache verify's profile summary from the rocprofv3 "
                         "CSVs under DIR/kt, DIR/fetch, DIR/write and DIR/alu")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="no GPU work: write the profile summary from the rocprofv3 CSVs "
                         "under DIR/kt, DIR/fetch and DIR/write")
    return ap.parse_args()


def record_bytes(sh) -> int:
    eb = 2 if sh.act == "bf16" else 4
    return sh.H * sh.K * eb + sh.HV * (sh.V * eb + 8)


def verify_alg_bytes(sh, hist: np.ndarray) -> int:
    """Bytes the verify must move for one call (each counted once).

    S0 rows read + committed history read + window in + outputs + ring write
    of the window + slot indices and cursors."""
    eb = 2 if sh.act == "bf16" else 4
    B, T = sh.B, sh.T
    s0 = B * sh.HV * sh.V * sh.K * 4
    win = B * T * (2 * sh.H * sh.K + sh.HV * sh.V + 2 * sh.HV) * eb
    out = B * T * sh.HV * sh.V * eb
    ring_w = B * T * record_bytes(sh)
    hist_r = int(hist.sum()) * record_bytes(sh)
    return s0 + hist_r + win + out + ring_w + B * 16


def dcache_alg_bytes(sh, hist: np.ndarray) -> int:
    """Bytes the d-cache verify must move for one call (each counted once).

    As the raw-replay verify, except that a committed record is read as its
    key, gate and fp32 corrected delta (not its raw value), and the window's
    deltas are written beside its raw records."""
    eb = 2 if sh.act == "bf16" else 4
    B, T = sh.B, sh.T
    s0 = B * sh.HV * sh.V * sh.K * 4
    win = B * T * (2 * sh.H * sh.K + sh.HV * sh.V + 2 * sh.HV) * eb
    out = B * T * sh.HV * sh.V * eb
    dvec = sh.HV * sh.V * 4
    ring_w = B * T * (record_bytes(sh) + dvec)
    hist_r = int(hist.sum()) * (sh.H * sh.K * eb + sh.HV * 8 + dvec)
    return s0 + hist_r + win + out + ring_w + B * 16


def fold_alg_bytes(sh, folded_records: np.ndarray) -> int:
    n = len(folded_records)
    return n * 2 * sh.HV * sh.V * sh.K * 4 + int(folded_records.sum()) * record_bytes(sh)


def snapshot_alg_bytes(sh) -> int:
    eb = 2 if sh.act == "bf16" else 4
    B, T = sh.B, sh.T
    return (B * sh.HV * sh.V * sh.K * 4 + B * T * sh.HV * sh.V * sh.K * 4 +
            B * T * (2 * sh.H * sh.K + sh.HV * sh.V + 2 * sh.HV) * eb + B * T * sh.HV * sh.V * eb)


def kda_record_bytes(sh) -> int:
    eb = 2 if sh.act == "bf16" else 4
    return sh.H * sh.K * eb + sh.HV * (sh.V * eb + sh.K * 4 + 4)


def kda_alg(sh, replayed: int, flagged: int):
    """(flops, bytes) one KDA verify launch must do and move.

    Flops: a state-row step is a decay multiply, a dot and an update over K
    columns (5K flops; an FMA counts 2), for every replayed record and window
    token of every (row, value head, value row); the readout adds 2K per
    window token.  Bytes: checkpoints read (and written for flagged rows),
    replayed records, window in, outputs, the window's ring records."""
    eb = 2 if sh.act == "bf16" else 4
    B, T = sh.B, sh.T
    rows = sh.HV * sh.V
    flops = (replayed + B * T) * rows * 5 * sh.K + B * T * rows * 2 * sh.K
    state = sh.HV * sh.V * sh.K * 4
    byts = (B * state + flagged * state + replayed * kda_record_bytes(sh) +
            B * T * (2 * sh.H * sh.K + sh.HV * sh.V + sh.HV * sh.K + sh.HV) * eb +
            B * T * sh.HV * sh.V * eb + B * T * kda_record_bytes(sh) + B * 16)
    return flops, byts


# fp32 vector rate without packed fp32 instructions (which this library does not
# emit): 256 CUs x 4 SIMDs x 16 lanes x 1 FMA (2 flops) per clock x 2.4 GHz
ALU_F32_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12


def traffic_from_profile():
    """HBM bytes per verify launch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        text = open(PROFILE_SUMMARY).read()
    except OSError:
        return None
    src_hash = hashlib.sha256(open(VERIFY_SRC, "rb").read()).hexdigest()[:16]
    m_hash = re.search(r"source sha256\[:16\]: `([0-9a-f]{16})`", text)
    m_bytes = re.search(r"HBM bytes per launch \(scaled\): ([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != src_hash:
        return None
    return float(m_bytes.group(1))


def interleaved_verifies(args, sh, gs, gv, params, slots, cd, w, bf, f32, i32, rounds=8, calls=20):
    """Median launch time of the raw-replay verify and of the d-cache verify,
    timed in alternating blocks on identical state (rings of both designs
    filled with the same records by one-token verifies).  The first two
    rounds are dropped (clocks settling)."""
    import torch
    dev = "cuda:0"
    n_hist = int(cd.write_pos[slots].max())
    hw = synth_history(sh, args.seed + 1, n_hist)
    A_log, dt_bias = f32(params.A_log), f32(params.dt_bias)

    def rings():
        return [torch.zeros(sh.num_slots, sh.H, sh.L, sh.K, dtype=torch.bfloat16, device=dev),
                torch.zeros(sh.num_slots, sh.HV, sh.L, sh.V, dtype=torch.bfloat16, device=dev),
                torch.zeros(sh.num_slots, sh.HV, sh.L, dtype=torch.float32, device=dev),
                torch.zeros(sh.num_slots, sh.HV, sh.L, dtype=torch.float32, device=dev)]

    Sr, Sd = f32(params.S0), f32(params.S0)
    rr, rd4 = rings(), rings()
    rd = torch.zeros(sh.num_slots, sh.HV, sh.L, sh.V, dtype=torch.float32, device=dev)
    dslots = i32(slots)
    gs1 = gs.replace(T=1)
    scratch = torch.empty(sh.B, sh.HV, sh.V, dtype=torch.bfloat16, device=dev)
    zeros = i32(np.zeros(sh.num_slots))
    base = i32(cd.cache_base)
    for r, x in enumerate(hw):
        sl = i32(np.where(cd.write_pos[slots] > r, slots, -1).astype(np.int32))
        xw = [bf(y) for y in (x.q, x.k, x.v, x.a, x.b)]
        wpr = i32(np.full(sh.num_slots, r))
        gv.gdn_spec_verify_ring(gs1, *xw, A_log, dt_bias, Sr, sl, wpr, base, zeros, *rr, 1, 0, scratch)
        gv.gdn_spec_verify_dcache(gs1, *xw, A_log, dt_bias, Sd, sl, wpr, base, zeros, *rd4, rd, 1, 0,
                                  scratch)
    wp0 = cd.write_pos.astype(np.int32)
    cur = [i32(wp0), i32(cd.cache_base), i32((wp0 + 2 * sh.max_spec > sh.L).astype(np.int32))]
    o = torch.empty(sh.B * sh.T, sh.HV, sh.V, dtype=torch.bfloat16, device=dev)
    fns = {"raw": lambda: gv.gdn_spec_verify_ring(gs, *w, A_log, dt_bias, Sr, dslots, *cur, *rr, 1, 0, o),
           "dcache": lambda: gv.gdn_spec_verify_dcache(gs, *w, A_log, dt_bias, Sd, dslots, *cur, *rd4,
                                                       rd, 1, 0, o)}
    res = {k: [] for k in fns}
    for _ in range(rounds + 2):
        for k, fn in fns.items():
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(calls)]
            for e0, e1 in evs:
                e0.record()
                fn()
                e1.record()
            torch.cuda.synchronize()
            res[k].append(float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]) * 1e3))
    del Sr, Sd, rr, rd4, rd
    return {"rounds": rounds, "calls_per_round": calls,
            "raw_verify_us": float(np.median(res["raw"][2:])),
            "dcache_verify_us": float(np.median(res["dcache"][2:])),
            "raw_rounds_us": [round(x, 1) for x in res["raw"][2:]],
            "dcache_rounds_us": [round(x, 1) for x in res["dcache"][2:]]}


def synth_history(sh, seed, n):
    from linear_attention_speculative_spec_amd import synth
    return synth.history_windows(synth.make_rng(seed), sh, n)


def cpu_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    cap = int(os.environ.get("OMP_NUM_THREADS", n) or n)
    return max(1, min(n, cap))


def main():
    args = parse()
    if args.summarize_profile:
        summarize_profile(args.summarize_profile)
        return
    if args.summarize_kda_profile:
        summarize_kda_profile(args.summarize_kda_profile)
        return
    if args.summarize_dcache_profile:
        summarize_dcache_profile(args.summarize_dcache_profile)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not "
              "supported (the path shards by rows and value heads with no exchange; "
              "see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    from linear_attention_speculative_spec_amd import gdnverify as gv
    from linear_attention_speculative_spec_amd import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    sh = synth.CONFIGS[WORKLOAD]
    gs = gv.GdnShape.from_layer(sh)
    gv.lib()   # fail loudly if the HIP library is missing
    rng = synth.make_rng(args.seed)

    t0 = time.time()
    log(f"[bench] generating {WORKLOAD} inputs")
    params = synth.layer_params(rng, sh)
    slots = synth.slot_choice(rng, sh)
    cd = synth.random_cursors(rng, sh)
    n_hist = int(cd.write_pos[slots].max())
    hist_windows = synth.history_windows(rng, sh, n_hist)
    n_pool = 4
    pool = [synth.window(rng, sh) for _ in range(n_pool)]
    n_steps = args.warmup + args.steps
    accepts = synth.accept_counts(rng, sh.B, sh.T, n_steps)

    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    f32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)  # noqa: E731
    i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(dev)    # noqa: E731

    S = f32(params.S0)
    A_log, dt_bias = f32(params.A_log), f32(params.dt_bias)
    rawk = torch.zeros(sh.num_slots, sh.H, sh.L, sh.K, dtype=torch.bfloat16, device=dev)
    rawv = torch.zeros(sh.num_slots, sh.HV, sh.L, sh.V, dtype=torch.bfloat16, device=dev)
    rg = torch.zeros(sh.num_slots, sh.HV, sh.L, dtype=torch.float32, device=dev)
    rb = torch.zeros_like(rg)
    dslots = i32(slots)
    wins = [[bf(x) for x in (w.q, w.k, w.v, w.a, w.b)] for w in pool]

    # pre-fill the rings: one recorded token per call through the verify itself
    log(f"[bench] pre-filling rings with up to {n_hist} records ({time.time() - t0:.1f}s)")
    gs1 = gs.replace(T=1)
    scratch = torch.empty(sh.B, sh.HV, sh.V, dtype=torch.bfloat16, device=dev)
    zeros = i32(np.zeros(sh.num_slots))
    base_d = i32(cd.cache_base)
    for r, w in enumerate(hist_windows):
        sl = np.where(cd.write_pos[slots] > r, slots, -1).astype(np.int32)
        wp_r = i32(np.full(sh.num_slots, r))
        gv.gdn_spec_verify_ring(gs1, *[bf(x) for x in (w.q, w.k, w.v, w.a, w.b)], A_log,
                                dt_bias, S, i32(sl), wp_r, base_d, zeros, rawk, rawv, rg, rb,
                                1, 0, scratch)
    del hist_windows
    wp0 = cd.write_pos.astype(np.int32)
    fl0 = (wp0 + 2 * sh.max_spec > sh.L).astype(np.int32)
    cur = [i32(wp0), i32(cd.cache_base), i32(fl0)]
    acc_d = [i32(a) for a in accepts]
    o = torch.empty(sh.B * sh.T, sh.HV, sh.V, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def step(i, ev=None):
        w = wins[i % n_pool]
        if ev is not None:
            ev[0].record()
        gv.gdn_exact_fold(gs, 1, 0, 0, S, rawk, rawv, rg, rb, dslots, cur[0], cur[1], cur[2], 1)
        if ev is not None:
            ev[1].record()
        gv.gdn_spec_verify_ring(gs, *w, A_log, dt_bias, S, dslots, cur[0], cur[1], cur[2],
                                rawk, rawv, rg, rb, 1, 0, o)
        if ev is not None:
            ev[2].record()
        gv.gdn_advance_cursors(gs, dslots, acc_d[i], cur[0], cur[1], cur[2])

    # dry run of the same trajectory to learn each step's history lengths
    saved = [S.clone(), rawk.clone(), rawv.clone(), rg.clone(), rb.clone(),
             [c.clone() for c in cur]]
    hist_per_step, fold_per_step = [], []
    for i in range(n_steps):
        wp = cur[0].cpu().numpy()[slots]
        fl = cur[2].cpu().numpy()[slots]
        hist_per_step.append(np.where(fl != 0, 0, np.clip(wp, 0, sh.L - sh.T)))
        fold_per_step.append(np.clip(wp[fl != 0], 0, sh.L - sh.T))
        step(i)
    torch.cuda.synchronize()

    def restore():
        S.copy_(saved[0]), rawk.copy_(saved[1]), rawv.copy_(saved[2])
        rg.copy_(saved[3]), rb.copy_(saved[4])
        for c, s0 in zip(cur, saved[5]):
            c.copy_(s0)
        torch.cuda.synchronize()

    restore()
    log(f"[bench] warmup {args.warmup} steps ({time.time() - t0:.1f}s)")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    start.record()
    for j in range(args.steps):
        step(args.warmup + j, evs[j])
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps
    verify_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    fold_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    timed = range(args.warmup, n_steps)
    vbytes = np.array([verify_alg_bytes(sh, hist_per_step[i]) for i in timed], dtype=np.float64)
    fbytes = np.array([fold_alg_bytes(sh, fold_per_step[i]) for i in timed], dtype=np.float64)
    v_avg_us = float(verify_ms.mean() * 1e3)
    achieved = float(vbytes.mean() / (verify_ms.mean() * 1e-3) / 1e9)
    tokens = sh.B * sh.T
    log(f"[bench] step {ms_step * 1e3:.1f} us, verify {v_avg_us:.1f} us "
        f"({achieved:.0f} GB/s), fold {fold_ms.mean() * 1e3:.1f} us")

    traffic = traffic_from_profile()
    result = {
        "metric": "GDN verify draft tokens/s per layer",
        "value": tokens / (ms_step * 1e-3),
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; random cursors, ring pre-filled by the library's verify)",
        "config": {"workload": "GDN layer B=256 rows, 512 slots, H=16, HV=32, K=V=128, "
                               "T=4, L=64, bf16 act, fp32 state",
                   "global_batch": sh.B, "draft_tokens": sh.T, "ring_len": sh.L,
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm",
            "kernel": "verify_kernel",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "traffic_GBs": (traffic / (v_avg_us * 1e-6) / 1e9) if traffic else None,
            "alg_bytes_per_launch": float(vbytes.mean()),
            "avg_launch_us": v_avg_us,
        },
        "fold": {"avg_launch_us": float(fold_ms.mean() * 1e3),
                 "alg_bytes_per_launch": float(fbytes.mean()),
                 "flagged_rows_per_step": float(np.mean([len(fold_per_step[i]) for i in timed]))},
        "memory": {"ring_bytes_per_layer": gv.gdn_ring_bytes(gs),
                   "snapshot_bytes_per_layer": gv.gdn_snapshot_bytes(gs),
                   "checkpoint_bytes_per_layer": sh.num_slots * sh.HV * sh.V * sh.K * 4},
    }

    if args.copy_calibration:
        x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        del x, y

    if not args.no_snapshot:
        snap = torch.empty(sh.B, sh.T, sh.HV, sh.V, sh.K, dtype=torch.float32, device=dev)
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        for i in range(3):
            gv.gdn_recurrent_verify_snapshot(gs, *wins[i % n_pool], A_log, dt_bias, S, dslots,
                                             snap, o)
        torch.cuda.synchronize()
        reps = 10
        e0.record()
        for i in range(reps):
            gv.gdn_recurrent_verify_snapshot(gs, *wins[i % n_pool], A_log, dt_bias, S, dslots,
                                             snap, o)
        e1.record()
        for i in range(reps):
            gv.gdn_snapshot_commit(gs, snap, dslots, acc_d[i % n_steps], saved[0])
        e2.record()
        torch.cuda.synchronize()
        snap_us = e0.elapsed_time(e1) / reps * 1e3
        commit_us = e1.elapsed_time(e2) / reps * 1e3
        sb = snapshot_alg_bytes(sh)
        result["snapshot_baseline"] = {
            "verify_us": snap_us, "commit_us": commit_us,
            "alg_bytes_per_launch": sb, "achieved_GBs": sb / (snap_us * 1e-6) / 1e9,
            "draft_tokens_per_s": tokens / ((snap_us + commit_us) * 1e-6)}
        del snap

    if not args.no_fold_every_commit:
        # The other design the method admits: the ring holds only the window
        # (2T records), every commit is folded into the checkpoint at once and
        # the cursors are reset, so the verify never replays a history.  Same
        # checkpoint, windows and accept counts; its own ring.
        gsf = gs.replace(L=2 * sh.max_spec)
        rkf = torch.zeros(sh.num_slots, sh.H, gsf.L, sh.K, dtype=torch.bfloat16, device=dev)
        rvf = torch.zeros(sh.num_slots, sh.HV, gsf.L, sh.V, dtype=torch.bfloat16, device=dev)
        rgf = torch.zeros(sh.num_slots, sh.HV, gsf.L, dtype=torch.float32, device=dev)
        rbf = torch.zeros_like(rgf)
        Sf = saved[0].clone()
        curf = [i32(np.zeros(sh.num_slots)) for _ in range(3)]

        def step_f(i, ev=None):
            w = wins[i % n_pool]
            if ev is not None:
                ev[0].record()
            gv.gdn_spec_verify_ring(gsf, *w, A_log, dt_bias, Sf, dslots, *curf, rkf, rvf, rgf, rbf,
                                    1, 0, o)
            if ev is not None:
                ev[1].record()
            gv.gdn_advance_cursors(gsf, dslots, acc_d[i % n_steps], *curf)
            gv.gdn_exact_fold(gsf, 1, 0, 0, Sf, rkf, rvf, rgf, rbf, dslots, *curf, 0)
            if ev is not None:
                ev[2].record()
            gv.gdn_reset_cursors(gsf, dslots, sh.B, 0, *curf)

        for i in range(args.warmup):
            step_f(i)
        evf = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for j in range(args.steps):
            step_f(args.warmup + j, evf[j])
        e1.record()
        torch.cuda.synchronize()
        f_step = e0.elapsed_time(e1) / args.steps * 1e3
        result["fold_every_commit"] = {
            "ring_len": gsf.L,
            "step_us": f_step,
            "verify_us": float(np.mean([e[0].elapsed_time(e[1]) for e in evf]) * 1e3),
            "fold_us": float(np.mean([e[1].elapsed_time(e[2]) for e in evf]) * 1e3),
            "draft_tokens_per_s": tokens / (f_step * 1e-6),
            "ring_bytes_per_layer": gv.gdn_ring_bytes(gsf)}
        log(f"[bench] fold every commit: step {f_step:.1f} us")
        del rkf, rvf, rgf, rbf, Sf

    if not args.no_dcache:
        # The d-cache design: the verify reads the committed history through
        # the corrected deltas earlier verifies recorded.  Same checkpoint,
        # cursors, windows and accept counts; its own rings, pre-filled by
        # one-token d-cache verifies of history records drawn the same way.
        rkd = torch.zeros_like(rawk)
        rvd = torch.zeros_like(rawv)
        rgd = torch.zeros_like(rg)
        rbd = torch.zeros_like(rb)
        rdd = torch.zeros(sh.num_slots, sh.HV, sh.L, sh.V, dtype=torch.float32, device=dev)
        Sd = f32(params.S0)
        hw = synth.history_windows(synth.make_rng(args.seed + 1), sh, n_hist)
        for r, w in enumerate(hw):
            sl = np.where(cd.write_pos[slots] > r, slots, -1).astype(np.int32)
            gv.gdn_spec_verify_dcache(gs1, *[bf(x) for x in (w.q, w.k, w.v, w.a, w.b)], A_log,
                                      dt_bias, Sd, i32(sl), i32(np.full(sh.num_slots, r)), base_d,
                                      zeros, rkd, rvd, rgd, rbd, rdd, 1, 0, scratch)
        del hw
        curd = [i32(wp0), i32(cd.cache_base), i32(fl0)]

        def step_d(i, ev=None):
            w = wins[i % n_pool]
            if ev is not None:
                ev[0].record()
            gv.gdn_exact_fold(gs, 1, 0, 0, Sd, rkd, rvd, rgd, rbd, dslots, *curd, 1)
            if ev is not None:
                ev[1].record()
            gv.gdn_spec_verify_dcache(gs, *w, A_log, dt_bias, Sd, dslots, *curd, rkd, rvd, rgd,
                                      rbd, rdd, 1, 0, o)
            if ev is not None:
                ev[2].record()
            gv.gdn_advance_cursors(gs, dslots, acc_d[i], *curd)

        for i in range(args.warmup):
            step_d(i)
        evd = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for j in range(args.steps):
            step_d(args.warmup + j, evd[j])
        e1.record()
        torch.cuda.synchronize()
        d_step = e0.elapsed_time(e1) / args.steps * 1e3
        d_ver = float(np.mean([e[1].elapsed_time(e[2]) for e in evd]) * 1e3)
        dbytes = float(np.mean([dcache_alg_bytes(sh, hist_per_step[i]) for i in timed]))
        result["dcache"] = {
            "step_us": d_step,
            "verify_us": d_ver,
            "fold_us": float(np.mean([e[0].elapsed_time(e[1]) for e in evd]) * 1e3),
            "alg_bytes_per_launch": dbytes,
            "achieved_GBs": dbytes / (d_ver * 1e-6) / 1e9,
            "draft_tokens_per_s": tokens / (d_step * 1e-6),
            "dring_bytes_per_layer": gv.gdn_dring_bytes(gs)}
        log(f"[bench] d-cache: step {d_step:.1f} us, verify {d_ver:.1f} us "
            f"({dbytes / (d_ver * 1e-6) / 1e9:.0f} GB/s)")
        del rkd, rvd, rgd, rbd, rdd, Sd

        # The two verifies on a fixed state: fresh rings of both designs
        # filled with the same records, the same checkpoint, cursors and
        # window, timed in alternating blocks of repeated calls in this one
        # process (the trajectory legs above step each design on its own).
        if not args.no_interleaved:
            result["dcache"]["interleaved"] = interleaved_verifies(args, sh, gs, gv, params, slots, cd,
                                                                   wins[0], bf, f32, i32)
            log(f"[bench] interleaved: raw replay {result['dcache']['interleaved']['raw_verify_us']:.1f} us, "
                f"d-cache {result['dcache']['interleaved']['dcache_verify_us']:.1f} us")

    if not args.no_kda:
        traj = [int(hist_per_step[i].sum() + fold_per_step[i].sum()) for i in range(n_steps)]
        nflag = [len(fold_per_step[i]) for i in range(n_steps)]
        result["kda"] = kda_leg(args, sh, saved[0], params.A_log, slots, cd, acc_d, traj, nflag)
        del saved
    if not args.no_chain:
        del S, rawk, rawv, rg, rb
        torch.cuda.empty_cache()
        result["chain"] = chain_leg(args)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(sh, args.seed, args.cpu_seconds)
        b32 = synth.CONFIGS["qwen3next_b32"]
        result["cpu_baseline"]["qwen3next_b32"] = cpu_baseline(b32, args.seed, args.cpu_seconds / 3)

    print(json.dumps(result), flush=True)


def kda_leg(args, sh, S0, A_log_h, slots, cd, acc_d, traj, nflag):
    """The per-channel-gate (KDA) layer on the same workload: same slots,
    initial cursors and accept counts (so the same history lengths), a
    checkpoint copied from the GDN leg's, K gate values per record.  A step is
    the one verify launch (flagged rows fold on the way) plus the cursor
    advance."""
    import torch

    from linear_attention_speculative_spec_amd import gdnverify as gv
    from linear_attention_speculative_spec_amd import synth

    dev = "cuda:0"
    gs = gv.GdnShape.from_layer(sh)
    t0 = time.time()
    rng = synth.make_rng(args.seed + 2)
    dt_bias = torch.from_numpy(rng.normal(0.0, 0.1, (sh.HV, sh.K)).astype(np.float32)).to(dev)
    A_log = torch.from_numpy(np.ascontiguousarray(A_log_h, np.float32)).to(dev)
    i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(dev)    # noqa: E731
    S = S0.clone()
    rawk = torch.zeros(sh.num_slots, sh.H, sh.L, sh.K, dtype=torch.bfloat16, device=dev)
    rawv = torch.zeros(sh.num_slots, sh.HV, sh.L, sh.V, dtype=torch.bfloat16, device=dev)
    rg = torch.zeros(sh.num_slots, sh.HV, sh.L, sh.K, dtype=torch.float32, device=dev)
    rb = torch.zeros(sh.num_slots, sh.HV, sh.L, dtype=torch.float32, device=dev)
    dslots = i32(slots)
    dw = synth.DeviceWindows(args.seed + 2, sh, kda=True)
    pool = [dw.draw() for _ in range(4)]
    dw1 = synth.DeviceWindows(args.seed + 3, sh.replace(T=1), kda=True)
    gs1 = gs.replace(T=1)
    scratch = torch.empty(sh.B, sh.HV, sh.V, dtype=torch.bfloat16, device=dev)
    zeros, base_d = i32(np.zeros(sh.num_slots)), i32(cd.cache_base)
    n_hist = int(cd.write_pos[slots].max())
    for r in range(n_hist):
        w = dw1.draw()
        sl = np.where(cd.write_pos[slots] > r, slots, -1).astype(np.int32)
        gv.gdn_kda_spec_verify_ring(gs1, w["q"], w["k"], w["v"], w["a"], w["b"], A_log, dt_bias,
                                    S, i32(sl), i32(np.full(sh.num_slots, r)), base_d, zeros,
                                    rawk, rawv, rg, rb, 1, 0, scratch)
    wp0 = cd.write_pos.astype(np.int32)
    cur = [i32(wp0), i32(cd.cache_base), i32((wp0 + 2 * sh.max_spec > sh.L).astype(np.int32))]
    o = torch.empty(sh.B * sh.T, sh.HV, sh.V, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] kda: rings pre-filled with up to {n_hist} records ({time.time() - t0:.1f}s)")

    def step(i, ev=None):
        w = pool[i % len(pool)]
        if ev is not None:
            ev[0].record()
        gv.gdn_kda_spec_verify_ring(gs, w["q"], w["k"], w["v"], w["a"], w["b"], A_log, dt_bias,
                                    S, dslots, *cur, rawk, rawv, rg, rb, 1, 1, o)
        if ev is not None:
            ev[1].record()
        gv.gdn_advance_cursors(gs, dslots, acc_d[i], *cur)

    for i in range(args.warmup):
        step(i)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for j in range(args.steps):
        step(args.warmup + j, evs[j])
    e1.record()
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) / args.steps * 1e3
    ver = np.array([e[0].elapsed_time(e[1]) * 1e3 for e in evs])
    timed = range(args.warmup, args.warmup + args.steps)
    fl, by = np.mean([kda_alg(sh, traj[i], nflag[i]) for i in timed], axis=0)
    v_us = float(ver.mean())
    tflops = fl / (v_us * 1e-6) / 1e12
    log(f"[bench] kda: step {step_us:.1f} us, verify {v_us:.1f} us ({tflops:.1f} TFLOP/s fp32)")
    return {
        "step_us": step_us,
        "draft_tokens_per_s": sh.B * sh.T / (step_us * 1e-6),
        "roofline": {"bound": "alu", "kernel": "kda_kernel (verify)", "achieved": tflops,
                     "peak": ALU_F32_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / ALU_F32_PEAK_TFLOPS, "traffic": None,
                     "alg_flops_per_launch": float(fl), "alg_bytes_per_launch": float(by),
                     "achieved_GBs": by / (v_us * 1e-6) / 1e9, "avg_launch_us": v_us},
        "replayed_records_per_step": float(np.mean([traj[i] for i in timed])),
        "ring_bytes_per_layer": gv.gdn_kda_ring_bytes(gs),
        "snapshot_bytes_per_layer": gv.gdn_snapshot_bytes(gs)}


def chain_leg(args):
    """The 48-layer stack of Qwen3-Next-shaped GDN layers at B=128 (T=4,
    L=64, 256 slots): one whole-stack verify step is the all-layer fold of the
    flagged rows (one launch), then the 48 layers' ring verifies, then one
    cursor advance.  Each layer reads a pre-drawn window (the glue between
    layers is not part of the path); its own checkpoint and ring."""
    import torch

    from linear_attention_speculative_spec_amd import gdnverify as gv
    from linear_attention_speculative_spec_amd import synth

    dev = "cuda:0"
    sh = synth.CONFIGS["layer_chain_b128"]
    NL = 48
    gs = gv.GdnShape.from_layer(sh)
    t0 = time.time()
    dw = synth.DeviceWindows(args.seed + 10, sh)
    gen = dw.gen
    A_log = torch.log(torch.rand((NL, sh.HV), generator=gen, device=dev) * 15.0 + 1.0)
    dt_bias = torch.randn((NL, sh.HV), generator=gen, device=dev) * 0.1
    S = torch.empty((NL, sh.num_slots, sh.HV, sh.V, sh.K), dtype=torch.float32, device=dev)
    for l in range(NL):
        S[l].normal_(0.0, 0.02, generator=gen)
    rawk = torch.zeros((NL, sh.num_slots, sh.H, sh.L, sh.K), dtype=torch.bfloat16, device=dev)
    rawv = torch.zeros((NL, sh.num_slots, sh.HV, sh.L, sh.V), dtype=torch.bfloat16, device=dev)
    rg = torch.zeros((NL, sh.num_slots, sh.HV, sh.L), dtype=torch.float32, device=dev)
    rb = torch.zeros_like(rg)
    i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(dev)    # noqa: E731
    rng = synth.make_rng(args.seed + 10)
    slots = synth.slot_choice(rng, sh)
    cd = synth.random_cursors(rng, sh)
    dslots = i32(slots)
    gs1 = gs.replace(T=1)
    dw1 = synth.DeviceWindows(args.seed + 11, sh.replace(T=1))
    scratch = torch.empty((sh.B, sh.HV, sh.V), dtype=torch.bfloat16, device=dev)
    zeros, base_d = i32(np.zeros(sh.num_slots)), i32(cd.cache_base)
    n_hist = int(cd.write_pos[slots].max())
    for r in range(n_hist):
        sl = i32(np.where(cd.write_pos[slots] > r, slots, -1))
        wp_r = i32(np.full(sh.num_slots, r))
        w = dw1.draw()
        for l in range(NL):
            gv.gdn_spec_verify_ring(gs1, w["q"], w["k"], w["v"], w["a"], w["b"], A_log[l],
                                    dt_bias[l], S[l], sl, wp_r, base_d, zeros, rawk[l], rawv[l],
                                    rg[l], rb[l], 1, 0, scratch)
    wp0 = cd.write_pos.astype(np.int32)
    cur = [i32(wp0), i32(cd.cache_base), i32((wp0 + 2 * sh.max_spec > sh.L).astype(np.int32))]
    pool = [dw.draw() for _ in range(4)]
    o = torch.empty((sh.B * sh.T, sh.HV, sh.V), dtype=torch.bfloat16, device=dev)
    warm, steps = 3, 10
    accepts = [i32(a) for a in synth.accept_counts(rng, sh.B, sh.T, warm + steps)]
    torch.cuda.synchronize()
    log(f"[bench] chain: {NL} layers pre-filled with up to {n_hist} records "
        f"({time.time() - t0:.1f}s)")

    def step(i, ev=None):
        if ev is not None:
            ev[0].record()
        gv.gdn_exact_fold(gs, NL, 0, 0, S, rawk, rawv, rg, rb, dslots, *cur, 1)
        if ev is not None:
            ev[1].record()
        for l in range(NL):
            w = pool[(i + l) % len(pool)]
            gv.gdn_spec_verify_ring(gs, w["q"], w["k"], w["v"], w["a"], w["b"], A_log[l],
                                    dt_bias[l], S[l], dslots, *cur, rawk[l], rawv[l], rg[l], rb[l],
                                    1, 0, o)
        if ev is not None:
            ev[2].record()
        gv.gdn_advance_cursors(gs, dslots, accepts[i], *cur)

    for i in range(warm):
        step(i)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for j in range(steps):
        step(warm + j, evs[j])
    e1.record()
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / steps
    fold_us = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]) * 1e3)
    ver_us = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]) * 1e3)
    log(f"[bench] chain: step {step_ms:.3f} ms (fold {fold_us:.1f} us, {NL} verifies "
        f"{ver_us:.1f} us)")
    return {
        "workload": f"{NL} GDN layers, B={sh.B}, {sh.num_slots} slots, H={sh.H}, HV={sh.HV}, "
                    f"K=V={sh.K}, T={sh.T}, L={sh.L}, bf16 act, fp32 state",
        "step_ms": step_ms,
        "all_layer_fold_us": fold_us,
        "verify_us_per_layer": ver_us / NL,
        "draft_tokens_per_s": sh.B * sh.T / (step_ms * 1e-3),
        "ring_bytes_stack": NL * gv.gdn_ring_bytes(gs),
        "snapshot_bytes_stack": NL * gv.gdn_snapshot_bytes(gs),
        "checkpoint_bytes_stack": NL * sh.num_slots * sh.HV * sh.V * sh.K * 4}


COPY_BYTES = 256 << 20
PROFILE_CMDS = [
    "cd /tmp && export TMPDIR=/tmp",
    "rocprofv3 --kernel-trace --stats -d $R/gpurun_out/prof/kt -o run --output-format csv -- "
    "python3 $R/bench.py --steps 50 --warmup 20 --no-cpu-baseline --no-snapshot --no-fold-every-commit --no-dcache --no-kda --no-chain "
    "--copy-calibration "
    "> $R/gpurun_out/prof/kt.log 2>&1",
    "rocprofv3 --pmc FETCH_SIZE -d $R/gpurun_out/prof/fetch -o run --output-format csv -- "
    "python3 $R/bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-snapshot --no-fold-every-commit "
    "--no-dcache --no-kda --no-chain --copy-calibration",
    "rocprofv3 --pmc WRITE_SIZE -d $R/gpurun_out/prof/write -o run --output-format csv -- "
    "python3 $R/bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-snapshot --no-fold-every-commit "
    "--no-dcache --no-kda --no-chain --copy-calibration",
    "rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_VALU_MFMA_BUSY_CYCLES "
    "SQ_INSTS_VALU_MFMA_BF16 SQ_INSTS_VALU_MFMA_F32 GRBM_GUI_ACTIVE -d $R/gpurun_out/prof/mfma -o run "
    "--output-format csv -- python3 $R/bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-snapshot "
    "--no-fold-every-commit --no-dcache --no-kda --no-chain",
    "cd $R && python3 bench.py --summarize-profile gpurun_out/prof",
]
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense MFMA peaks of the part
SIMDS = 256 * 4
XCDS = 8    # GRBM_GUI_ACTIVE is reported summed over the accelerator dies


def _csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_profile(d):
    """Profile summary (markdown) from one kernel-trace run and two counter\n    runs of this script: the verify kernel's average duration over the timed\n    steps, and its HBM bytes from FETCH_SIZE / WRITE_SIZE scaled by what the\n    same counters read for a plain copy of COPY_BYTES."""
    steps_kt, steps_pmc = 50, 5
    trace = [r for r in _csv(os.path.join(d, "kt", "run_kernel_trace.csv"))]
    stats = _csv(os.path.join(d, "kt", "run_kernel_stats.csv"))
    ver = [r for r in trace if "verify_kernel" in r["Kernel_Name"]]
    timed = ver[-steps_kt:]
    dur = np.array([int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in timed]) * 1e-3
    vname = timed[-1]["Kernel_Name"]

    def counter(sub, name):
        rows = _csv(os.path.join(d, sub, "run_counter_collection.csv"))
        rows = [r for r in rows if r["Counter_Name"] == name]
        v = [float(r["Counter_Value"]) for r in rows if "verify_kernel" in r["Kernel_Name"]][-steps_pmc:]
        c = [float(r["Counter_Value"]) for r in rows if "copy" in r["Kernel_Name"].lower()][-3:]
        return float(np.mean(v)), float(np.mean(c))

    fv, fc = counter("fetch", "FETCH_SIZE")
    wv, wc = counter("write", "WRITE_SIZE")
    kib = COPY_BYTES / 1024.0
    f_fetch, f_write = kib / fc, kib / wc
    hbm = (fv * f_fetch + wv * f_write) * 1024.0
    alg = None
    try:
        for line in open(os.path.join(d, "kt.log")):
            if line.startswith("{"):
                alg = json.loads(line)["roofline"]["alg_bytes_per_launch"]
    except OSError:
        pass
    src_hash = hashlib.sha256(open(VERIFY_SRC, "rb").read()).hexdigest()[:16]
    out = []
    out.append("# verify_kernel, GDN layer B=256 (qwen3next_b256 workload)\n")
    out.append("Commands (from the repository root on the GPU host, `R=$PWD`; each profiler run under "
               "its own `timeout`):\n")
    out.append("```\n" + "\n".join(PROFILE_CMDS) + "\n```\n")
    out.append(f"- kernel source: `linear_attention_speculative_spec_amd/csrc/gdn_verify.hip`, "
               f"source sha256[:16]: `{src_hash}`")
    out.append(f"- dispatch: `{vname}`")
    out.append(f"- timed steps (last {steps_kt} verify dispatches of the kernel-trace run): "
               f"average {dur.mean():.1f} us, min {dur.min():.1f} us, max {dur.max():.1f} us\n")
    out.append("## --kernel-trace --stats (all dispatches of the run)\n")
    out.append("| kernel | calls | average us | total ms | % |")
    out.append("|---|---|---|---|---|")
    for r in stats[:8]:
        out.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) * 1e-3:.1f} | "
                   f"{float(r['TotalDurationNs']) * 1e-6:.2f} | {float(r['Percentage']):.1f} |")
    out.append("\nThe verify's stats line also averages the ring pre-fill calls (one-token windows) and "
               "the dry run; the timed-step average above is the figure bench.py's HIP events report.\n")
    out.append("## HBM bytes (--pmc FETCH_SIZE, then --pmc WRITE_SIZE)\n")
    out.append("| | FETCH_SIZE KiB | WRITE_SIZE KiB |")
    out.append("|---|---|---|")
    out.append(f"| verify_kernel, mean of the last {steps_pmc} dispatches | {fv:.0f} | {wv:.0f} |")
    out.append(f"| plain copy of {COPY_BYTES >> 20} MiB (mean of 3) | {fc:.0f} | {wc:.0f} |")
    out.append(f"\nScale factors (copy bytes / counter): fetch {f_fetch:.4f}, write {f_write:.4f}.\n")
    out.append(f"HBM bytes per launch (scaled): {hbm:.6e}")
    if alg:
        out.append(f"\nAlgorithmic bytes per launch (bench.py accounting): {alg:.6e} "
                   f"(counter / algorithmic = {hbm / alg:.3f})")
    mdir = os.path.join(d, "mfma", "run_counter_collection.csv")
    if os.path.exists(mdir):
        rows = _csv(mdir)

        def mc(name):
            v = [float(r["Counter_Value"]) for r in rows
                 if r["Counter_Name"] == name and "verify_kernel" in r["Kernel_Name"]][-steps_pmc:]
            return float(np.mean(v))
        mops_bf16, mops_f32 = mc("SQ_INSTS_VALU_MFMA_MOPS_BF16"), mc("SQ_INSTS_VALU_MFMA_MOPS_F32")
        busy, gui = mc("SQ_VALU_MFMA_BUSY_CYCLES"), mc("GRBM_GUI_ACTIVE")
        n_bf16, n_f32 = mc("SQ_INSTS_VALU_MFMA_BF16"), mc("SQ_INSTS_VALU_MFMA_F32")
        fl_bf16, fl_f32 = mops_bf16 * 512, mops_f32 * 512
        t = dur.mean() * 1e-6
        out.append("\n## MFMA use (--pmc SQ_INSTS_VALU_MFMA_MOPS_*, SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE)\n")
        out.append("The window algebra (Gram tiles in bf16; Z, the value part and S0 Z in fp32) is small "
                   "beside the checkpoint stream; these counters show how much of the matrix units it "
                   "occupies.\n")
        out.append("| | bf16 | fp32 |")
        out.append("|---|---|---|")
        out.append(f"| MFMA instructions per launch | {n_bf16:.0f} | {n_f32:.0f} |")
        out.append(f"| MFMA flops per launch (MOPS x 512) | {fl_bf16:.4e} | {fl_f32:.4e} |")
        out.append(f"| achieved at the timed average ({dur.mean():.1f} us), TFLOP/s | "
                   f"{fl_bf16 / t / 1e12:.2f} | {fl_f32 / t / 1e12:.2f} |")
        out.append(f"| fraction of the dense peak ({MFMA_PEAK_TFLOPS['bf16']:.0f} / "
                   f"{MFMA_PEAK_TFLOPS['f32']:.1f} TFLOP/s) | {fl_bf16 / t / 1e12 / MFMA_PEAK_TFLOPS['bf16']:.4f} | "
                   f"{fl_f32 / t / 1e12 / MFMA_PEAK_TFLOPS['f32']:.4f} |")
        out.append(f"\nSQ_VALU_MFMA_BUSY_CYCLES {busy:.4e}, GRBM_GUI_ACTIVE {gui:.4e} per launch "
                   f"(summed over {XCDS} dies: {gui / XCDS:.4e} cycles each): matrix units busy "
                   f"{100.0 * busy / (gui / XCDS * SIMDS):.2f}% of SIMD-cycles "
                   f"(busy / (GRBM_GUI_ACTIVE / {XCDS} x {SIMDS} SIMDs)).")
    path = PROFILE_SUMMARY
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


KDA_PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "kda_kernel_qwen3next_b256.md")
KDA_SRC = os.path.join(ROOT, "linear_attention_speculative_spec_amd", "csrc", "gdn_kda.hip")
KDA_PROFILE_CMDS = [
    "cd /tmp && export TMPDIR=/tmp",
    "rocprofv3 --kernel-trace --stats -d $R/gpurun_out/kprof/kt -o run --output-format csv -- "
    "python3 $R/bench.py --steps 20 --warmup 5 --no-cpu-baseline --no-snapshot --no-fold-every-commit "
    "--no-dcache --no-chain > $R/gpurun_out/kprof/kt.log 2>&1",
    "rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_LDS SQ_INSTS_SALU SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES "
    "SQ_ACTIVE_INST_VALU GRBM_GUI_ACTIVE -d $R/gpurun_out/kprof/alu -o run --output-format csv -- "
    "python3 $R/bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-snapshot --no-fold-every-commit "
    "--no-dcache --no-chain",
    "cd $R && python3 bench.py --summarize-kda-profile gpurun_out/kprof",
]


def summarize_kda_profile(d):
    """Profile summary (markdown) of the KDA verify kernel: its average
    duration over the timed steps of the KDA leg, and its instruction
    counters against the fp32 vector issue rate."""
    steps_kt, steps_pmc = 20, 3
    is_ver = lambda name: "kda_kernel" in name and ("true" in name or "Lb1E" in name)   # noqa: E731
    trace = _csv(os.path.join(d, "kt", "run_kernel_trace.csv"))
    stats = _csv(os.path.join(d, "kt", "run_kernel_stats.csv"))
    ver = [r for r in trace if is_ver(r["Kernel_Name"])]
    timed = ver[-steps_kt:]
    dur = np.array([int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in timed]) * 1e-3
    kname = timed[-1]["Kernel_Name"]
    flops = None
    try:
        for line in open(os.path.join(d, "kt.log")):
            if line.startswith("{"):
                flops = json.loads(line)["kda"]["roofline"]["alg_flops_per_launch"]
    except (OSError, KeyError):
        pass
    rows = _csv(os.path.join(d, "alu", "run_counter_collection.csv"))

    def cval(name):
        v = [float(r["Counter_Value"]) for r in rows
             if r["Counter_Name"] == name and is_ver(r["Kernel_Name"])][-steps_pmc:]
        return float(np.mean(v)) if v else float("nan")

    valu, lds, salu = cval("SQ_INSTS_VALU"), cval("SQ_INSTS_LDS"), cval("SQ_INSTS_SALU")
    waves, gui = cval("SQ_WAVES"), cval("GRBM_GUI_ACTIVE")
    t = dur.mean() * 1e-6
    clock = gui / XCDS / t
    issue = valu * 4 / SIMDS / clock            # a wave's VALU instruction takes 4 cycles of its SIMD
    src_hash = hashlib.sha256(open(KDA_SRC, "rb").read()).hexdigest()[:16]
    out = ["# kda_kernel (verify), KDA layer B=256 (qwen3next_b256 workload shape)\n",
           "Commands (from the repository root on the GPU host, `R=$PWD`; each profiler run under "
           "its own `timeout`):\n",
           "```\n" + "\n".join(KDA_PROFILE_CMDS) + "\n```\n",
           f"- kernel source: `linear_attention_speculative_spec_amd/csrc/gdn_kda.hip`, "
           f"source sha256[:16]: `{src_hash}`",
           f"- dispatch: `{kname}`",
           f"- timed steps (last {steps_kt} KDA verify dispatches of the kernel-trace run): "
           f"average {dur.mean():.1f} us, min {dur.min():.1f} us, max {dur.max():.1f} us\n",
           "## --kernel-trace --stats (all dispatches of the run)\n",
           "| kernel | calls | average us | total ms | % |", "|---|---|---|---|---|"]
    for r in stats[:8]:
        out.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) * 1e-3:.1f} | "
                   f"{float(r['TotalDurationNs']) * 1e-6:.2f} | {float(r['Percentage']):.1f} |")
    out.append("\nThe KDA kernel's stats line also averages the ring pre-fill calls (one-token windows); "
               "the timed-step average above is the figure bench.py's HIP events report.\n")
    out.append(f"## Instructions per launch (--pmc, mean of the last {steps_pmc} KDA verify dispatches)\n")
    out.append("| SQ_INSTS_VALU | SQ_INSTS_LDS | SQ_INSTS_SALU | SQ_WAVES | GRBM_GUI_ACTIVE |")
    out.append("|---|---|---|---|---|")
    out.append(f"| {valu:.4e} | {lds:.4e} | {salu:.4e} | {waves:.0f} | {gui:.4e} |")
    out.append(f"\nClock over the timed average: GRBM_GUI_ACTIVE / {XCDS} dies / {dur.mean():.1f} us = "
               f"{clock / 1e9:.2f} GHz.")
    out.append(f"VALU issue time: SQ_INSTS_VALU x 4 cycles / {SIMDS} SIMDs / clock = {issue * 1e6:.1f} us, "
               f"{100.0 * issue / t:.0f}% of the kernel's time (100% would mean every SIMD issues a "
               f"vector instruction every 4 cycles).")
    if flops:
        out.append(f"\nAlgorithmic flops per launch (bench.py accounting): {flops:.4e}; "
                   f"{flops / t / 1e12:.1f} TFLOP/s at the timed average, "
                   f"{flops / t / 1e12 / ALU_F32_PEAK_TFLOPS:.3f} of the non-packed fp32 peak "
                   f"({ALU_F32_PEAK_TFLOPS:.1f} TFLOP/s at 2.4 GHz); "
                   f"{flops / valu:.1f} flops per wave-level VALU instruction (at most 128).")
    os.makedirs(os.path.dirname(KDA_PROFILE_SUMMARY), exist_ok=True)
    with open(KDA_PROFILE_SUMMARY, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


DCACHE_PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "dcache_verify_kernel_qwen3next_b256.md")
DCACHE_SRC = os.path.join(ROOT, "linear_attention_speculative_spec_amd", "csrc", "gdn_dcache.hip")
_DC_LEG = "--no-cpu-baseline --no-snapshot --no-fold-every-commit --no-kda --no-chain --no-interleaved --copy-calibration"
DCACHE_PROFILE_CMDS = [
    "cd /tmp && export TMPDIR=/tmp",
    "rocprofv3 --kernel-trace --stats -d $R/gpurun_out/dcprof/kt -o run --output-format csv -- "
    f"python3 $R/bench.py --steps 50 --warmup 20 {_DC_LEG} > $R/gpurun_out/dcprof/kt.log 2>&1",
    "rocprofv3 --pmc FETCH_SIZE -d $R/gpurun_out/dcprof/fetch -o run --output-format csv -- "
    f"python3 $R/bench.py --steps 5 --warmup 2 {_DC_LEG}",
    "rocprofv3 --pmc WRITE_SIZE -d $R/gpurun_out/dcprof/write -o run --output-format csv -- "
    f"python3 $R/bench.py --steps 5 --warmup 2 {_DC_LEG}",
    "rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_WAVES SQ_WAVE_CYCLES SQ_WAIT_INST_ANY "
    "SQ_WAIT_ANY GRBM_GUI_ACTIVE -d $R/gpurun_out/dcprof/alu -o run --output-format csv -- "
    f"python3 $R/bench.py --steps 5 --warmup 2 {_DC_LEG}",
    "cd $R && python3 bench.py --summarize-dcache-profile gpurun_out/dcprof",
]


def summarize_dcache_profile(d):
    """Profile summary (markdown) of the d-cache verify kernel: its average
    duration over the timed steps of the d-cache leg, its HBM bytes from the
    byte counters (scaled by a plain copy's), and its instruction counters
    against the vector issue rate."""
    steps_kt, steps_pmc = 50, 5

    def is_dc(r):
        return "dcache_verify_kernel" in r["Kernel_Name"]

    trace = [r for r in _csv(os.path.join(d, "kt", "run_kernel_trace.csv")) if is_dc(r)]
    stats = _csv(os.path.join(d, "kt", "run_kernel_stats.csv"))
    big = max(int(r["Grid_Size_X"]) for r in trace)          # the B=256 windows (the pre-fill runs T=1)
    timed = [r for r in trace if int(r["Grid_Size_X"]) == big][-steps_kt:]
    dur = np.array([int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in timed]) * 1e-3
    kname = timed[-1]["Kernel_Name"]

    def counter(sub, name, copy=True):
        rows = [r for r in _csv(os.path.join(d, sub, "run_counter_collection.csv")) if r["Counter_Name"] == name]
        g = max(int(r["Grid_Size"]) for r in rows if is_dc(r))
        v = [float(r["Counter_Value"]) for r in rows if is_dc(r) and int(r["Grid_Size"]) == g][-steps_pmc:]
        # the calibration copies: the first three copy dispatches after the
        # headline leg's last verify (the d-cache leg that follows restores its
        # state with copies of its own)
        last_v = max(int(r["Dispatch_Id"]) for r in rows
                     if "verify_kernel" in r["Kernel_Name"] and not is_dc(r))
        cr = sorted((int(r["Dispatch_Id"]), float(r["Counter_Value"])) for r in rows
                    if "copy" in r["Kernel_Name"].lower() and int(r["Dispatch_Id"]) > last_v)[:3]
        c = [x for _, x in cr]
        return float(np.mean(v)), float(np.mean(c if copy else [1.0]))

    fv, fc = counter("fetch", "FETCH_SIZE")
    wv, wc = counter("write", "WRITE_SIZE")
    kib = COPY_BYTES / 1024.0
    f_fetch, f_write = kib / fc, kib / wc
    hbm = (fv * f_fetch + wv * f_write) * 1024.0
    alg = None
    try:
        for line in open(os.path.join(d, "kt.log")):
            if line.startswith("{"):
                alg = json.loads(line)["dcache"]["alg_bytes_per_launch"]
    except (OSError, KeyError):
        pass
    src_hash = hashlib.sha256(open(DCACHE_SRC, "rb").read()).hexdigest()[:16]
    t = dur.mean() * 1e-6
    out = ["# dcache_verify_kernel, GDN layer B=256 (qwen3next_b256 workload)\n",
           "The d-cache verify (`gdn_spec_verify_dcache`): history read through stored corrected deltas. "
           "It is timed in `bench.py`'s `dcache` leg on the same checkpoint, cursors, windows and accept "
           "counts as the headline.\n",
           "Commands (from the repository root on the GPU host, `R=$PWD`; each profiler run under "
           "its own `timeout`):\n",
           "```\n" + "\n".join(DCACHE_PROFILE_CMDS) + "\n```\n",
           f"- kernel source: `linear_attention_speculative_spec_amd/csrc/gdn_dcache.hip`, "
           f"source sha256[:16]: `{src_hash}`",
           f"- dispatch: `{kname}`, grid {big} threads",
           f"- timed steps (last {steps_kt} d-cache verify dispatches of the kernel-trace run): "
           f"average {dur.mean():.1f} us, min {dur.min():.1f} us, max {dur.max():.1f} us\n",
           "## --kernel-trace --stats (all dispatches of the run)\n",
           "| kernel | calls | average us | total ms | % |", "|---|---|---|---|---|"]
    for r in stats[:8]:
        out.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) * 1e-3:.1f} | "
                   f"{float(r['TotalDurationNs']) * 1e-6:.2f} | {float(r['Percentage']):.1f} |")
    out.append("\nThe d-cache line's stats average includes the ring pre-fill calls with one-token "
               "windows; the timed-step average above is the figure to use.\n")
    out.append("## HBM bytes (--pmc FETCH_SIZE, then --pmc WRITE_SIZE)\n")
    out.append("| | FETCH_SIZE KiB | WRITE_SIZE KiB |")
    out.append("|---|---|---|")
    out.append(f"| dcache_verify_kernel, mean of the last {steps_pmc} dispatches | {fv:.0f} | {wv:.0f} |")
    out.append(f"| plain copy of {COPY_BYTES >> 20} MiB (mean of 3) | {fc:.0f} | {wc:.0f} |")
    out.append(f"\nScale factors (copy bytes / counter): fetch {f_fetch:.4f}, write {f_write:.4f}.\n")
    out.append(f"HBM bytes per launch (scaled): {hbm:.4e} (fetch {fv * f_fetch * 1024:.4e}, "
               f"write {wv * f_write * 1024:.4e})")
    if alg:
        out.append(f"\nAlgorithmic bytes per launch (bench.py `dcache_alg_bytes`): {alg:.4e}; "
                   f"{alg / t / 1e9:.0f} GB/s at the timed average, {alg / t / 1e9 / 8000.0:.3f} of 8 TB/s; "
                   f"counter / algorithmic = {hbm / alg:.3f}.")
    rows = _csv(os.path.join(d, "alu", "run_counter_collection.csv"))

    def cval(name):
        g = max(int(r["Grid_Size"]) for r in rows if is_dc(r))
        v = [float(r["Counter_Value"]) for r in rows
             if r["Counter_Name"] == name and is_dc(r) and int(r["Grid_Size"]) == g][-steps_pmc:]
        return float(np.mean(v)) if v else float("nan")

    valu, salu, lds = cval("SQ_INSTS_VALU"), cval("SQ_INSTS_SALU"), cval("SQ_INSTS_LDS")
    waves, wcyc, wissue, wany, gui = (cval("SQ_WAVES"), cval("SQ_WAVE_CYCLES"), cval("SQ_WAIT_INST_ANY"),
                                      cval("SQ_WAIT_ANY"), cval("GRBM_GUI_ACTIVE"))
    clock = gui / XCDS / t
    issue = valu * 4 / SIMDS / clock
    out.append(f"\n## Instructions and wave states per launch (--pmc, mean of the last {steps_pmc} "
               "dispatches)\n")
    out.append("| SQ_INSTS_VALU | SQ_INSTS_SALU | SQ_INSTS_LDS | SQ_WAVES | GRBM_GUI_ACTIVE |")
    out.append("|---|---|---|---|---|")
    out.append(f"| {valu:.4e} | {salu:.4e} | {lds:.4e} | {waves:.0f} | {gui:.4e} |")
    out.append(f"\nPer wave: {valu / waves:.0f} VALU, {salu / waves:.0f} SALU and {lds / waves:.0f} LDS "
               f"instructions. Clock over the timed average: GRBM_GUI_ACTIVE / {XCDS} dies / "
               f"{dur.mean():.1f} us = {clock / 1e9:.2f} GHz. VALU issue time (SQ_INSTS_VALU x 4 cycles / "
               f"{SIMDS} SIMDs / clock) = {issue * 1e6:.1f} us, {100.0 * issue / t:.0f}% of the kernel's time.")
    out.append(f"Of the waves' cycles (SQ_WAVE_CYCLES), {100.0 * wissue / wcyc:.0f}% were spent ready but "
               f"waiting for an issue slot (SQ_WAIT_INST_ANY) and {100.0 * wany / wcyc:.0f}% waiting on "
               "loads, LDS or barriers (SQ_WAIT_ANY).")
    os.makedirs(os.path.dirname(DCACHE_PROFILE_SUMMARY), exist_ok=True)
    with open(DCACHE_PROFILE_SUMMARY, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def cpu_baseline(sh, seed, budget_s):
    """The fp64 oracle on the same workload: the same seeded layer, cursors
    and pre-filled history, verifying whole batches of rows on the host."""
    import oracle
    from oracle.cursors import CursorState
    from linear_attention_speculative_spec_amd import synth

    rng = synth.make_rng(seed)
    params = synth.layer_params(rng, sh)
    slots = synth.slot_choice(rng, sh)
    cd = synth.random_cursors(rng, sh)
    n_hist = int(cd.write_pos[slots].max())
    hist_windows = synth.history_windows(rng, sh, n_hist)
    win = synth.window(rng, sh)
    rows = np.arange(sh.B)
    osh = sh.replace(num_slots=sh.B)
    orc = oracle.OracleLayer(osh, params.A_log, params.dt_bias, params.S0[slots])
    del params
    oslots = np.arange(sh.B, dtype=np.int32)
    cur = CursorState(np.zeros(sh.B, np.int32), cd.cache_base[slots].copy(),
                      np.zeros(sh.B, np.int32))
    to64 = lambda w: tuple(synth.act_to_f64(x, sh.act) for x in (w.q, w.k, w.v, w.a, w.b))  # noqa: E731
    for r, w in enumerate(hist_windows):
        cur.write_pos[:] = r
        sl = np.where(cd.write_pos[slots] > r, oslots, -1).astype(np.int32)
        orc.write_ring(cur, sl, to64(w), T=1)
    del hist_windows
    wp = cd.write_pos[slots].astype(np.int32)
    cur = CursorState(wp, cd.cache_base[slots].copy(),
                      (wp + 2 * sh.max_spec > sh.L).astype(np.int32))
    w64 = to64(win)
    nt = cpu_threads()
    # only unflagged rows so the oracle's checkpoint stays as generated
    cur.is_flush[:] = 0
    reps, t_used = 0, 0.0
    while t_used < budget_s:
        t1 = time.perf_counter()
        orc.verify(cur, oslots, w64, write_ring=False, fold_flagged=False, nthreads=nt)
        t_used += time.perf_counter() - t1
        reps += 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"value": reps * sh.B * sh.T / t_used, "unit": "draft tokens/s", "cores": nt,
            "os_cpu_count": os.cpu_count(), "affinity_cpus": affinity,
            "kind": "oracle",
            "sample": f"{reps} full verifies of the B={sh.B} batch (all {sh.HV} value heads, "
                      f"history replay + {sh.T} drafts, fp64), {t_used:.1f} s wall on {nt} threads"}


if __name__ == "__main__":
    main()
