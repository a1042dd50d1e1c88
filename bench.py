#!/usr/bin/env python3
"""Throughput of one rank's ZeRO-DP shard step on one MI355X.

Workload (the 13B-parameter, N = 64 ZeRO-3 rank shard): a GPT-style model of
40 layers, hidden 5120, FFN 20480, vocabulary 50257 (Psi = 12,848,143,360)
cut into 64 shards; rank 63 owns S = 200,752,240 elements.  Per step it
reduces R = 2 fp16 gradient contributions, unscales them with the overflow
check, applies Adam to its fp32 master/momentum/variance shard and writes the
fp16 parameters into its slot of a 64-slot gather buffer (25.7 GB).  All
inputs are synthetic and resident in HBM before the timed region.

A timed step is one zero_shard_step call through a PreparedStep (arguments
checked once; fused kernel, the overflow decision that its last block
publishes to the host, loss-scale control).  `value` comes from exactly K
timed steps; the kernel time behind the roofline from K more, with HIP
events that each launch records at its kernel's start and end.  The same
run also reports
  * the partition layout of the 484-tensor model (host, once per model),
  * the rank's whole local share of an iteration: its full gradient stream
    packed through a 2^26 bucket, then the shard step,
  * the bucket pack of the 20,000-tensor stream (82 fills of 2^26),
  * the owners' share of the bucketed reduce of two ranks' copies of that
    stream into the 16 owners' fp16 gradient shards,
  * the owner step: rank 63's shard step fed straight from two ranks' whole
    gradient streams of the 13B model (reduce and update in one pass),
  * the kernel's HBM roofline (algorithmic bytes per launch over the kernel's
    HIP-event time on its stream) and, when the counter profile under
    profiles/ was taken from the current kernel source, its measured traffic,
  * the achievable line: the step's own access pattern with none of its
    arithmetic (libzero_probe: same tile-per-wave schedule, 5 read and 4
    write streams) on the step's own buffers, and a plain copy of the same
    number of bytes, each timed like the step kernel,
  * torch's device copy of 2 GiB for comparison (a library copy kernel),
  * the CPU oracle timed on the host on the same shard: all of the host's
    CPU share in threads (the reported baseline) and one thread.

With --shard-workloads it instead times the fused step on every shard
workload (tiny, GPT-2 1.5B, 13B, 1T) and reports each.

Prints one JSON line.  Usage: python bench.py [--steps K] [--warmup W] [--shard-workloads]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("fused shard-step elements/s and achieved HBM GB/s (% of peak) per rank shard")
HBM_PEAK_GBS = 8000.0
PMC_PROFILE = os.path.join(ROOT, "profiles", "shard_step_zero3_13b_pmc.json")
KERNEL_SOURCES = [os.path.join(ROOT, "sharded_zero_partition_amd", "csrc", f)
                  for f in ("shard_step.hip", "zp_internal.hpp", "vec16.hpp", "adam.hpp")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(shard_elems: int):
    """HBM bytes per launch from the committed counter profile, or None when
    there is none or it was taken from another version of the kernel."""
    if not os.path.exists(PMC_PROFILE):
        return None
    with open(PMC_PROFILE) as f:
        prof = json.load(f)
    if prof.get("kernel_source_sha") != kernel_source_hash() or prof.get("shard_elems") != shard_elems:
        return None
    return int(round((prof["fetch_kib_per_dispatch"] * prof["fetch_scale"] +
                      prof["write_kib_per_dispatch"] * prof["write_scale"]) * 1024))


def host_cpu_share():
    """(threads, how, cpu_count, model): the CPUs this process may use -- the
    affinity set, limited by a cgroup CPU quota when there is one, and by the
    CPU share of one GPU on the GPU machines (16) -- and the CPU model."""
    count = os.cpu_count() or 1
    n, how = count, "os.cpu_count()"
    try:
        aff = len(os.sched_getaffinity(0))
        if aff < n:
            n, how = aff, "sched_getaffinity"
    except (AttributeError, OSError):
        pass
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        if quota != "max" and int(quota) // int(period) < n:
            n, how = max(1, int(quota) // int(period)), "cgroup cpu.max quota"
    except (OSError, ValueError):
        pass
    if n > 16:
        n, how = 16, "the CPU share of one GPU on the GPU boxes (16 CPUs)"
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, how, count, model


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--mode", choices=["pingpong", "inplace"], default="pingpong")
    ap.add_argument("--shard-workloads", action="store_true",
                    help="instead of the default measurement: the fused step on each shard workload "
                         "(tiny, GPT-2 1.5B, 13B, 1T), K timed steps each, one JSON line")
    ap.add_argument("--no-pack", action="store_true", help="skip the bucket-pack measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="three more plain 2 GiB device copies after the library copy (the "
                         "scale reference of the HBM counter runs)")
    ap.add_argument("--no-rank-iteration", action="store_true",
                    help="skip the 13B rank's full gradient-stream pack + step measurement")
    ap.add_argument("--no-placement-spread", action="store_true",
                    help="skip re-timing the step on re-allocated buffers")
    ap.add_argument("--no-owner-step", action="store_true",
                    help="skip the owner-step measurement (shard step fed from the ranks' tensor lists)")
    ap.add_argument("--pack-views", action="store_true",
                    help="pack sources as views of one buffer instead of 20,000 allocations")
    ap.add_argument("--arena", action="store_true",
                    help="carve the shard state, its alternate set and the contributions out of "
                         "one contiguous block (zero_arena_plan_for) instead of separate allocations")
    return ap.parse_args()


def shard_workload_step(w, steps: int, warmup: int) -> dict:
    """The fused ping-pong step on workload `w` (its shard, R contributions of
    step 1, its scale, the slot at the rank's offset of the workload's gather
    buffer): wall time per step over `steps` steps, then kernel time over
    `steps` more by HIP events the launches record at their kernels' start
    and end, and algorithmic bytes (26 + 2R per element) over the kernel
    time."""
    import numpy as np
    import torch

    import sharded_zero_partition_amd as zp
    from sharded_zero_partition_amd import workloads as W

    dev = "cuda"
    S, R = w.shard, w.n_contrib
    gather = torch.empty(w.gather_slots * S, dtype=torch.int16, device=dev)
    off = (w.rank if w.gather_slots == w.n_ranks else 0) * S
    slot = gather[off:off + S]
    p0 = W.master_init(w, device=dev)
    slot.copy_(p0.to(torch.float16).view(torch.int16))
    st = zp.ShardState(p0, torch.zeros_like(p0), torch.zeros_like(p0),
                       torch.empty_like(p0), torch.empty_like(p0), torch.empty_like(p0))
    grads = [W.grad_contribution(w, 1, r, w.scale, device=dev) for r in range(R)]
    hp = zp.AdamHParams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay)
    step = zp.PreparedStep(st, grads, hp, zp.LossScaler.make(w.scale), slot)
    flags = 0
    for _ in range(warmup):
        flags += step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        flags += step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    zp.set_kernel_timing(True)
    for _ in range(steps):
        flags += step()
    torch.cuda.synchronize()
    kms = zp.kernel_times()
    zp.set_kernel_timing(False)
    assert len(kms) == steps and flags == 0, "unexpected overflow in the benchmark inputs"
    kern = float(np.mean(kms)) * 1e-3
    gbs = (26 + 2 * R) * S / kern / 1e9
    row = {"workload": w.name, "shard_elems": S, "contributions": R, "rank": w.rank,
           "slot_offset_elems": off, "ms_per_step": round(wall * 1e3, 4),
           "elements_per_s": round(S / wall, 1), "kernel_ms": round(kern * 1e3, 4),
           "kernel_ms_min": round(float(np.min(kms)), 4),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    if w.special_step is not None:
        # the overflow step, reported apart: an inf in one contribution makes
        # every step skip (the fused pass raises the flag, the slot is then
        # restored from the master; the state does not change)
        grads[0][0] = 0x7C00
        assert step() == 1
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        skipped = sum(step() for _ in range(steps))
        torch.cuda.synchronize()
        assert skipped == steps
        row["overflow_step"] = {
            "ms_per_step": round((time.perf_counter() - t0) / steps * 1e3, 4),
            "what": "fused pass that raises the flag, then the slot restored from the master "
                    "(6 B per element); wall clock per step, state unchanged"}
    del step, st, grads, gather, slot, p0
    torch.cuda.empty_cache()
    return row


def shard_workloads_main(args):
    """One JSON line: the fused step on every shard workload, in order tiny,
    GPT-2 1.5B, 13B, 1T (each allocated, timed and freed in turn)."""
    import torch

    from sharded_zero_partition_amd import workloads as W

    torch.cuda.set_device(0)
    rows = [shard_workload_step(make(), args.steps, args.warmup)
            for make in (W.tiny, W.gpt2_1p5b, W.zero3_13b, W.zero3_1t)]
    main_row = rows[2]
    out = {"metric": METRIC, "value": main_row["elements_per_s"], "unit": "elements/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": main_row["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": "every shard workload, the 13B rank-63 shard as value",
                      "mode": "pingpong", "state_allocation": "separate buffers"},
           "roofline": main_row["roofline"],
           "workloads": rows,
           "note": "the tiny shard (8.9 MB of traffic) stays in the 256 MB last-level cache and "
                   "is launch-bound: its figure is latency, not HBM bandwidth"}
    print(json.dumps(out), flush=True)


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one rank's shard step on a single GPU; the library has no "
              "multi-GPU exchange, so --gpus above 1 (or a multi-process launch) is not supported",
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.steps > 4096 or args.warmup < 0:
        sys.exit("--steps must be in 1..4096 (one kernel-timing pair per step) and --warmup >= 0")

    if args.shard_workloads:
        shard_workloads_main(args)
        return

    import numpy as np
    import torch

    import sharded_zero_partition_amd as zp
    from sharded_zero_partition_amd import workloads as W

    torch.cuda.set_device(0)
    dev = "cuda"
    w = W.zero3_13b()
    S, R = w.shard, w.n_contrib

    # a1: the partition layout of the model (host; once per model).  The first
    # call also loads the library (the binding is imported lazily), so it is
    # left out; layout_ms is the median of five calls after it.
    zp.partition_layout(w.numels, w.n_ranks, stage=w.stage).close()
    lt = []
    for _ in range(5):
        t0 = time.perf_counter()
        lay = zp.partition_layout(w.numels, w.n_ranks, stage=w.stage)
        lt.append((time.perf_counter() - t0) * 1e3)
        lay.close()
    layout_ms = float(np.median(lt))
    lay = zp.partition_layout(w.numels, w.n_ranks, stage=w.stage)
    assert lay.info.shard_elems == S
    begin, _, _ = lay.rank_range(w.rank)
    lay.close()

    # inputs resident in HBM
    gather = torch.empty(w.gather_slots * S, dtype=torch.int16, device=dev)
    slot = gather[w.rank * S:(w.rank + 1) * S]
    p0 = W.master_init(w, device=dev)
    slot.copy_(p0.to(torch.float16).view(torch.int16))
    arena = None
    if args.arena:
        alay = zp.partition_layout(w.numels, w.n_ranks, stage=w.stage)
        arena = zp.carve_arena(alay.arena_plan(pingpong=args.mode == "pingpong", n_contrib=R))
        alay.close()
        arena["master"].copy_(p0)
        arena["momentum"].zero_()
        arena["variance"].zero_()
        del p0
        p0 = arena["master"]
        alt = [arena.get(k) for k in ("master_alt", "momentum_alt", "variance_alt")]
        st = zp.ShardState(p0, arena["momentum"], arena["variance"], *alt)
        grads = []
        for r in range(R):
            arena[f"contrib{r}"].copy_(W.grad_contribution(w, 1, r, w.scale, device=dev))
            grads.append(arena[f"contrib{r}"])
    elif args.mode == "pingpong":
        st = zp.ShardState(p0, torch.zeros_like(p0), torch.zeros_like(p0),
                           torch.empty_like(p0), torch.empty_like(p0), torch.empty_like(p0))
        grads = [W.grad_contribution(w, 1, r, w.scale, device=dev) for r in range(R)]
    else:
        st = zp.ShardState(p0, torch.zeros_like(p0), torch.zeros_like(p0))
        grads = [W.grad_contribution(w, 1, r, w.scale, device=dev) for r in range(R)]
    hp = zp.AdamHParams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay)
    scaler = zp.LossScaler.make(w.scale)

    # host copy of the sample the CPU oracle will take (before any update)
    cpu_n = S                    # the whole shard, one step (~10 s on one core)
    cpu_inputs = None
    if not args.no_cpu_baseline:
        cpu_inputs = (p0[:cpu_n].cpu().numpy().copy(),
                      [g[:cpu_n].cpu().numpy().view(np.uint16).copy() for g in grads])

    step = zp.PreparedStep(st, grads, hp, scaler, slot)   # arguments checked once
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps (no kernel timing, which would add to the
    # host's critical path)
    flags = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        flags += step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # kernel time: K more steps, each launch recording HIP events at its
    # kernel's start and end on the launch stream (read after the loop)
    zp.set_kernel_timing(True)
    for _ in range(args.steps):
        flags += step()
    torch.cuda.synchronize()
    kernel_ms = zp.kernel_times()
    zp.set_kernel_timing(False)
    assert len(kernel_ms) == args.steps
    assert flags == 0, "unexpected overflow in the benchmark inputs"

    step_ms = elapsed / args.steps * 1e3
    value = S * args.steps / elapsed
    # ping-pong: one pass; in place: the check pass reads the contributions once more
    bytes_per_elem = 26 + 2 * R if args.mode == "pingpong" else 26 + 4 * R
    alg_bytes = bytes_per_elem * S
    kern_avg_ms = float(np.mean(kernel_ms))
    achieved = alg_bytes / (kern_avg_ms * 1e-3) / 1e9
    traffic = measured_traffic(S) if args.mode == "pingpong" else None   # profile is of the fused pass
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}

    # The achievable line on the step's own buffers: the step kernel's access
    # pattern with none of its arithmetic (reads the contributions and the
    # live p/m/v, writes the alternate set and the slot: the same 9 streams
    # and 30 B per element), then a plain copy of the same number of bytes.
    # Both record HIP events at their kernels' start and end, like the step.
    achievable = None
    if args.mode == "pingpong":
        from sharded_zero_partition_amd import probe
        lp, lm, lv = st.live()
        ap, am, av = st.p_alt if st.cur == 0 else st.p, st.m_alt if st.cur == 0 else st.m, \
            st.v_alt if st.cur == 0 else st.v
        probe.step_pattern(grads, lp, lm, lv, ap, am, av, slot, reps=2)          # warm-up
        pat_ms = probe.step_pattern(grads, lp, lm, lv, ap, am, av, slot, reps=args.steps)
        half = (alg_bytes // 2) // 16 * 16
        csrc = torch.empty(half, dtype=torch.uint8, device=dev).fill_(7)
        cdst = torch.empty_like(csrc)
        probe.copy(csrc, cdst, reps=2)
        copy_probe_ms = probe.copy(csrc, cdst, reps=args.steps)
        del csrc, cdst
        pat_gbs = alg_bytes / (pat_ms * 1e-3) / 1e9
        cp_gbs = 2 * half / (copy_probe_ms * 1e-3) / 1e9
        achievable = {
            "step_pattern": {"ms": round(pat_ms, 4), "achieved": round(pat_gbs, 1), "unit": "GB/s",
                             "frac_of_peak": round(pat_gbs / HBM_PEAK_GBS, 4),
                             "what": "zero_probe_step_pattern on the step's own buffers: its "
                                     "tile-per-wave schedule, 2 fp16 + 3 fp32 read and 3 fp32 + 1 fp16 "
                                     "written streams (30 B per element), no arithmetic; mean kernel "
                                     f"time of {args.steps} launches"},
            "copy": {"ms": round(copy_probe_ms, 4), "achieved": round(cp_gbs, 1), "unit": "GB/s",
                     "frac_of_peak": round(cp_gbs / HBM_PEAK_GBS, 4),
                     "what": f"zero_probe_copy of {half} bytes into fresh buffers ({2 * half} bytes "
                             f"moved, the step's algorithmic bytes); mean kernel time of {args.steps} launches"},
            "step_over_pattern": round(achieved / pat_gbs, 4),
            "step_over_copy": round(achieved / cp_gbs, 4)}

    # The rank's whole local share of one iteration at 13B: its full fp16
    # gradient stream (the model's 484 tensors, packed bucket by bucket for the
    # reduce-scatter) through a 2^26-element bucket, then the shard step.
    rank_iteration = None
    if not args.no_pack and not args.no_rank_iteration:
        gB = 1 << 26
        glay = zp.partition_layout(w.numels, w.n_ranks, stage=w.stage, bucket=gB)
        gstream = [torch.empty(n, dtype=torch.float16, device=dev).normal_(0.0, 1e-3 * w.scale)
                   .view(torch.int16) for n in w.numels]
        glay.bind_tensors(gstream)
        gbucket = torch.empty(gB, dtype=torch.int16, device=dev)
        n_fills = glay.info.n_fills

        def iteration():
            for k in range(n_fills):
                glay.pack_bucket(k, gbucket)
            return step()

        flags += iteration()
        torch.cuda.synchronize()
        iters = 3
        t0 = time.perf_counter()
        for _ in range(iters):
            flags += iteration()
        torch.cuda.synchronize()
        it_s = (time.perf_counter() - t0) / iters
        assert flags == 0, "unexpected overflow in the benchmark inputs"
        psi = sum(w.numels)
        it_bytes = 4 * psi + 2 * (n_fills * gB - psi) + bytes_per_elem * S
        rank_iteration = {
            "workload": f"zero3_13b rank 63: the full fp16 gradient stream ({len(w.numels)} tensors, "
                        f"{psi} elements) packed through a 2^26 bucket ({n_fills} fills), then the "
                        "shard step",
            "ms": round(it_s * 1e3, 3),
            "algorithmic_gbs": round(it_bytes / it_s / 1e9, 1),
            "frac": round(it_bytes / it_s / 1e9 / HBM_PEAK_GBS, 4)}
        glay.close()
        del gstream, gbucket

    del step, st, grads, gather, slot, p0, arena
    torch.cuda.empty_cache()

    # The same step on freshly allocated buffers placed behind padding
    # allocations of several sizes: the kernel's time follows where its nine
    # buffers land physically.  Reported beside `value`, which is the first
    # measurement above and is never replaced by these.
    placement = None
    if not args.no_placement_spread:
        spread = []
        for pad_gb in (0, 7, 19, 31, 43):
            torch.cuda.empty_cache()
            pad = torch.empty(pad_gb << 30, dtype=torch.uint8, device=dev) if pad_gb else None
            pp0 = W.master_init(w, device=dev)
            pst = zp.ShardState(pp0, torch.zeros_like(pp0), torch.zeros_like(pp0),
                                torch.empty_like(pp0), torch.empty_like(pp0), torch.empty_like(pp0))
            pgr = [W.grad_contribution(w, 1, r, w.scale, device=dev) for r in range(R)]
            pslot = torch.empty(S, dtype=torch.int16, device=dev)
            pstep = zp.PreparedStep(pst, pgr, hp, zp.LossScaler.make(w.scale), pslot)
            for _ in range(3):
                pstep()
            torch.cuda.synchronize()
            zp.set_kernel_timing(True)
            for _ in range(args.steps):
                assert pstep() == 0
            torch.cuda.synchronize()
            spread.append(round(float(np.mean(zp.kernel_times())), 4))
            zp.set_kernel_timing(False)
            del pstep, pst, pgr, pslot, pp0, pad
        torch.cuda.empty_cache()
        placement = {"kernel_ms": spread, "padding_gb": [0, 7, 19, 31, 43],
                     "frac": [round(alg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) for ms in spread],
                     "what": f"the same step re-timed ({args.steps} steps each) on freshly allocated "
                             "buffers behind padding allocations of these sizes; value and roofline "
                             "are the first measurement"}

    # NEXT: the owner step -- the same rank's shard step with its sum taken
    # straight from R = 2 ranks' whole gradient streams of the model (484
    # tensors each, one buffer per rank with 0..7-element gaps), so the
    # Stage 2 reduce of its partition and the update are one pass
    owner = None
    if not args.no_owner_step:
        olay = zp.partition_layout(w.numels, w.n_ranks, stage=w.stage, bucket=1 << 26)
        streams = [W.gradient_stream(w.numels, w.wid, r, w.scale, 1, dev) for r in range(R)]
        olay.bind_contributions([views for _, _, views in streams])
        n_real = max(0, min(S, sum(w.numels) - w.rank * S))
        op0 = W.master_init(w, device=dev)
        ost = zp.ShardState(op0, torch.zeros_like(op0), torch.zeros_like(op0),
                            torch.empty_like(op0), torch.empty_like(op0), torch.empty_like(op0))
        oslot = torch.empty(S, dtype=torch.int16, device=dev)
        oscaler = zp.LossScaler.make(w.scale)
        oflags = 0
        for _ in range(args.warmup):
            oflags += olay.owner_step(w.rank, ost, hp, oscaler, oslot)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            oflags += olay.owner_step(w.rank, ost, hp, oscaler, oslot)
        torch.cuda.synchronize()
        o_wall = (time.perf_counter() - t0) / args.steps
        zp.set_kernel_timing(True)
        for _ in range(args.steps):
            oflags += olay.owner_step(w.rank, ost, hp, oscaler, oslot)
        torch.cuda.synchronize()
        o_ms = zp.kernel_times()
        zp.set_kernel_timing(False)
        assert len(o_ms) == args.steps and oflags == 0
        o_kern = float(np.mean(o_ms)) * 1e-3
        o_bytes = (26 + 2 * R) * n_real           # R fp16 reads, p/m/v in and out, fp16 slot
        o_gbs = o_bytes / o_kern / 1e9
        # the fused step on these same state and slot buffers (its own dense
        # contributions): the kernels' times follow where the buffers land,
        # so this is the comparison that holds the placement fixed
        sgr = [W.grad_contribution(w, 1, r, w.scale, device=dev) for r in range(R)]
        sstep = zp.PreparedStep(ost, sgr, hp, zp.LossScaler.make(w.scale), oslot)
        for _ in range(args.warmup):
            sstep()
        torch.cuda.synchronize()
        zp.set_kernel_timing(True)
        for _ in range(args.steps):
            assert sstep() == 0
        torch.cuda.synchronize()
        s_ms = zp.kernel_times()
        zp.set_kernel_timing(False)
        del sstep, sgr
        owner = {
            "workload": f"zero3_13b rank 63: R = {R} ranks' whole fp16 gradient streams "
                        f"({len(w.numels)} tensors each, misaligned in one buffer per rank) "
                        "reduced straight into the ping-pong Adam step of the rank's "
                        f"{n_real} real elements",
            "elements": n_real,
            "ms_per_step": round(o_wall * 1e3, 4),
            "kernel_ms": round(o_kern * 1e3, 4),
            "kernel_ms_min": round(float(np.min(o_ms)), 4),
            "fused_step_kernel_ms": round(kern_avg_ms, 4),
            "fused_step_same_buffers_kernel_ms": round(float(np.mean(s_ms)), 4),
            "roofline": {"bound": "hbm", "achieved": round(o_gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(o_gbs / HBM_PEAK_GBS, 4)}}
        olay.close()
        del streams, ost, op0, oslot
        torch.cuda.empty_cache()

    # a library copy for comparison: torch's copy_ of 2 GiB (read 2 GiB, write
    # 2 GiB), timed with HIP events; also the reference dispatch for the
    # counter scale
    a = torch.empty(1 << 30, dtype=torch.int16, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    copy_ms = []
    for _ in range(5 + (3 if args.calibration_copy else 0)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        e1.synchronize()
        copy_ms.append(e0.elapsed_time(e1))
    del a, b
    copy_gbs = 2 * 2 * (1 << 30) / (float(np.median(copy_ms)) * 1e-3) / 1e9
    library_copy = {"achieved": round(copy_gbs, 1), "unit": "GB/s",
                    "what": "torch copy_ of a 2 GiB tensor into another (4 GiB moved), median "
                            f"of {len(copy_ms)}, HIP events",
                    "step_over_copy": round(achieved / copy_gbs, 4)}

    # a2: bucket pack of the 20,000-tensor stream
    pack = None
    reduce_owner = None
    if not args.no_pack:
        pw = W.pack_20k()
        tensors = W.pack_sources(pw, device=dev, views=args.pack_views)
        play = zp.partition_layout(pw.numels, pw.n_ranks, stage=2, bucket=pw.bucket)
        play.bind_tensors(tensors)
        bucket = torch.empty(pw.bucket, dtype=torch.int16, device=dev)
        for k in range(pw.n_fills):                                   # warm-up pass
            play.pack_bucket(k, bucket)
        torch.cuda.synchronize()
        t0 = time.perf_counter()                                      # wall pass, no events
        for k in range(pw.n_fills):
            play.pack_bucket(k, bucket)
        torch.cuda.synchronize()
        pack_wall = time.perf_counter() - t0
        zp.set_kernel_timing(True)                                    # per-launch event pairs
        for k in range(pw.n_fills):
            play.pack_bucket(k, bucket)
        torch.cuda.synchronize()
        fill_ms = zp.kernel_times()
        zp.set_kernel_timing(False)
        assert len(fill_ms) == pw.n_fills
        # kernel time: one event pair around a pass of back-to-back launches
        # on the launch stream (no host wait between fills), which leaves out
        # the per-pair overhead a short kernel would otherwise carry
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for k in range(pw.n_fills):
            play.pack_bucket(k, bucket)
        e1.record()
        e1.synchronize()
        kernel_total = e0.elapsed_time(e1) * 1e-3
        pack_bytes = 4 * pw.psi + 2 * (pw.n_fills * pw.bucket - pw.psi)
        pack_gbs = pack_bytes / kernel_total / 1e9
        pack = {"workload": "pack_20k: 20,000 fp16 tensors, log-uniform sizes in [1, 2^22], "
                            "bucket 2^26, 82 fills",
                "elements": pw.psi, "fills": pw.n_fills,
                "elements_per_s": round(pw.psi / pack_wall, 1),
                "ms_total": round(pack_wall * 1e3, 3),
                "kernel_ms_per_fill": round(kernel_total * 1e3 / pw.n_fills, 4),
                "kernel_ms_per_fill_event_pairs": round(float(np.mean(fill_ms)), 4),
                "timing": "kernel_ms_per_fill and roofline: one HIP-event pair around a pass of the "
                          "82 back-to-back launches on the launch stream; event_pairs: one pair per "
                          "launch, recorded by the launch at its kernel's start and end",
                "roofline": {"bound": "hbm", "achieved": round(pack_gbs, 1), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(pack_gbs / HBM_PEAK_GBS, 4)}}
        play.close()
        del bucket

        # NEXT: the owners' share of the bucketed reduce of two ranks' gradient
        # tensors (this stream and a second draw), every fill and owner
        lists = [tensors, W.pack_sources(pw, device=dev, views=args.pack_views, draw=1)]
        rlay = zp.partition_layout(pw.numels, pw.n_ranks, stage=2, bucket=pw.bucket)
        rlay.bind_contributions(lists)
        S4 = rlay.info.shard_elems
        flat = torch.empty(pw.n_ranks * S4, dtype=torch.int16, device=dev)
        pairs = [(k, r) for k in range(pw.n_fills) for r in range(pw.n_ranks)
                 if max(k * pw.bucket, r * S4) < min((k + 1) * pw.bucket, (r + 1) * S4, pw.psi)]
        for k, r in pairs:                                             # warm-up pass
            rlay.reduce_to_owner(k, r, flat[r * S4:(r + 1) * S4])
        torch.cuda.synchronize()
        t0 = time.perf_counter()                                      # wall pass, no events
        for k, r in pairs:
            rlay.reduce_to_owner(k, r, flat[r * S4:(r + 1) * S4])
        torch.cuda.synchronize()
        red_wall = time.perf_counter() - t0
        zp.set_kernel_timing(True)                                    # per-launch event pairs
        for k, r in pairs:
            rlay.reduce_to_owner(k, r, flat[r * S4:(r + 1) * S4])
        torch.cuda.synchronize()
        red_ms = zp.kernel_times()
        zp.set_kernel_timing(False)
        assert len(red_ms) == len(pairs)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()                                                   # one pair around the pass
        for k, r in pairs:
            rlay.reduce_to_owner(k, r, flat[r * S4:(r + 1) * S4])
        e1.record()
        e1.synchronize()
        red_kernel = e0.elapsed_time(e1) * 1e-3
        red_bytes = 6 * pw.psi                        # 2 x 2 B read + 2 B written
        red_gbs = red_bytes / red_kernel / 1e9
        reduce_owner = {
            "workload": "pack_20k stream, R = 2 ranks' gradient tensors, reduced into the "
                        "fp16 gradient shards of its 16 owners, all 82 fills",
            "elements": pw.psi, "launches": len(pairs),
            "elements_per_s": round(pw.psi / red_wall, 1),
            "ms_total": round(red_wall * 1e3, 3),
            "kernel_ms_total": round(red_kernel * 1e3, 3),
            "kernel_ms_total_event_pairs": round(float(np.sum(red_ms)), 3),
            "timing": "kernel_ms_total and roofline: one HIP-event pair around the pass of "
                      "back-to-back launches on the launch stream; event_pairs: the sum of one "
                      "pair per launch",
            "roofline": {"bound": "hbm", "achieved": round(red_gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(red_gbs / HBM_PEAK_GBS, 4)}}
        rlay.close()
        del tensors, lists, flat
        torch.cuda.empty_cache()

    # CPU oracle on a bounded sample of the same shard (first step's inputs)
    cpu = None
    cpu_one = None
    if cpu_inputs is not None:
        import oracle
        p_host, c_host = cpu_inputs
        ost = oracle.ShardState(p_host)
        out16 = np.empty(cpu_n, np.uint16)
        t0 = time.perf_counter()
        oracle.shard_step(ost, c_host, oracle.LossScaler(w.scale),
                          oracle.AdamHP(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay), out16)
        cpu_s = time.perf_counter() - t0
        cpu_one = {"value": round(cpu_n / cpu_s, 1), "unit": "elements/s", "cores": 1,
                   "kind": "oracle",
                   "sample": f"the whole rank-63 shard ({cpu_n} elements), first step "
                             f"(scalar C oracle, one thread, {cpu_s:.1f} s)"}

        # The same C functions over contiguous chunks in parallel threads (the
        # calls release the GIL), one per CPU of the host's share: the
        # overflow flag over every chunk first, then Adam on every chunk when
        # no chunk overflowed.
        from concurrent.futures import ThreadPoolExecutor
        n_threads, share_how, cpu_count, cpu_model = host_cpu_share()
        bounds = np.linspace(0, cpu_n, n_threads + 1).astype(np.int64)
        par = oracle.ShardState(p_host)
        par_out = np.empty(cpu_n, np.uint16)
        ohp = oracle.AdamHP(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay)
        parts = [(int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
        t0 = time.perf_counter()
        with ThreadPoolExecutor(n_threads) as pool:
            flags_par = list(pool.map(lambda ab: oracle.overflow_flag([c[ab[0]:ab[1]] for c in c_host]), parts))
            if not any(flags_par):
                list(pool.map(lambda ab: oracle.adam_apply(
                    [c[ab[0]:ab[1]] for c in c_host], par.p[ab[0]:ab[1]], par.m[ab[0]:ab[1]],
                    par.v[ab[0]:ab[1]], par_out[ab[0]:ab[1]], w.scale, 1, ohp), parts))
        par_s = time.perf_counter() - t0
        assert np.array_equal(par_out, out16) and np.array_equal(par.p.view(np.uint32), ost.p.view(np.uint32))
        cpu = {"value": round(cpu_n / par_s, 1), "unit": "elements/s", "cores": n_threads,
               "kind": "oracle",
               "sample": f"the whole rank-63 shard ({cpu_n} elements), first step: the oracle's C "
                         f"functions over {len(parts)} contiguous chunks in {n_threads} threads "
                         f"({par_s:.2f} s); results equal to the one-thread run",
               "cpu_model": cpu_model, "cpu_count": cpu_count,
               "threads_from": share_how}

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "zero3_13b: rank 63 of 64, 13B-param GPT-style model "
                               "(40 layers, hidden 5120, FFN 20480, vocab 50257)",
                   "shard_elems": S, "contributions": R, "mode": args.mode,
                   "state_allocation": "one contiguous arena" if args.arena else "separate buffers",
                   "gather_slots": w.gather_slots, "slot_offset_elems": begin},
        "algorithmic_gbs_per_step": round(alg_bytes / (step_ms * 1e-3) / 1e9, 1),
        "kernel_ms": round(kern_avg_ms, 4),
        "kernel_ms_min": round(float(np.min(kernel_ms)), 4),
        "kernel_ms_median": round(float(np.median(kernel_ms)), 4),
        "roofline": roofline,
        "achievable": achievable,
        "placement_spread": placement,
        "library_copy": library_copy,
        "rank_iteration": rank_iteration,
        "layout_ms": round(layout_ms, 3),
        "pack": pack,
        "reduce_to_owner": reduce_owner,
        "owner_step": owner,
        "cpu_baseline": cpu,
        "cpu_baseline_one_thread": cpu_one,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
