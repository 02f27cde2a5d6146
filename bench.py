#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet chunked forward on one MI355X.

One step = one gdn_chunk_fwd call over one batch of the workload's synthetic
inputs (decay cumsum, UT transform, WY pair, the sequential chunk walk or the
chunk-group fold / prefix / replay, and the outputs), with inputs, outputs
and workspace resident in HBM before the timed region starts.

Timing: each of the K timed steps runs after a 512 MB read that evicts the
memory-side cache (MALL, 256 MB), and is bracketed by its own HIP events on
the stream the library launches on (torch's current stream); `ms_per_step` is
the median.  The same K steps each after a 512 MB write instead are reported
as `after_write_flush` (the cache then holds ~256 MB of that buffer's dirty
lines, whose write-back lands in the step), and back to back (cache warm) as
`warm`.

Prints ONE JSON line.  `value` is tokens/s (B*T per step).  `roofline`
relates the whole step to the method's own algorithmic HBM bytes (inputs read
once, o and h_T written once; the long path's fold re-read, pairs and
incoming states), with `traffic` the HBM bytes per step that the rocprofv3
counters measured for the same kernels (when taken on the current sources);
`dominant_kernel` gives the longest kernel against the bytes this design
makes it move.  `cpu_baseline` times the fp64 oracle on this host's cores
over a bounded sample of the workload (and on one thread for the small
workloads).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12            # bytes/s, MI355X HBM3E
BF16_PEAK = 2.5e15           # dense bf16 MFMA FLOP/s
METRIC = "GDN fwd tokens/sec (all heads) at T=4096/262144; MFMA util % vs gfx950 peak"


def algorithmic(w, o_bytes=4):
    """The method's own FLOPs and HBM bytes per step (inputs read once, o and
    h_T written once; the long path adds the fold's re-read of k, v, g, beta,
    the pairs and the incoming states)."""
    C, dk, dv = w.chunk, w.dk, w.dv
    tok = w.B * w.T
    s = 2 if w.dtype == "bf16" else 4
    per_qk = 2 * C * dk
    per_v = (C - 1) * (dk + dv) + (C + 1) * dv + 6 * dk * dv + C * C / 3
    flops = tok * (w.Hqk * per_qk + w.Hv * per_v)
    nbytes = tok * (2 * w.Hqk * dk * s + w.Hv * dv * s + 8 * w.Hv + w.Hv * dv * o_bytes)
    nbytes += w.B * w.Hv * dk * dv * 4 * (2 if w.h0_std > 0 else 1)
    J = max(w.n_groups, 1)
    if J > 1:
        flops += tok * w.Hv * 4 * dk * (dk + dv)
        flops += w.B * w.Hv * J * 2 * dk * dk * dv
        nbytes += tok * (w.Hqk * dk * s + w.Hv * dv * s + 8 * w.Hv)
        nbytes += w.B * w.Hv * J * (dk * dk + dk * dv) * 4 * 2 + w.B * w.Hv * J * dk * dv * 4 * 2
    return flops, nbytes


def bwd_algorithmic(w):
    """FLOPs and HBM bytes of one backward call (gdn_chunk_bwd).  FLOPs: the
    products of the chunked backward per chunk and value head -- the
    intra-chunk transform (K K^T, the triangular inverse, W and U), the
    forward-state walk (W h, K_g^T X), the reverse walk and its chunk term
    (K dh, W^T X, Q K^T, P W, Qeff^T dO) and the chunk gradients (the adjoint
    of every line of the chunk's forward: 5 products of C x d x d, 12 of
    C x C x d, 2 of C x C x C) -- counted dense, as launched.  Bytes: the
    inputs and cotangents read once, the gradients written once."""
    C, d = w.chunk, w.dk
    N = -(-w.T // C)
    units = w.B * w.Hv * N
    cdd, ccd, ccc = 2 * C * d * d, 2 * C * C * d, 2 * C * C * C
    per = (ccd / 2 + ccc / 6 + 2 * ccd) + 2 * cdd + (3 * cdd + 2 * ccd) + (5 * cdd + 12 * ccd + 2 * ccc)
    flops = units * per
    tok = w.B * w.T
    s = 2 if w.dtype == "bf16" else 4
    nbytes = tok * (2 * w.Hqk * d * s + w.Hv * d * s + 8 * w.Hv + w.Hv * d * 4)      # q, k, v, g, beta, dO
    nbytes += tok * (2 * w.Hqk * d * 4 + w.Hv * d * 4 + 8 * w.Hv)                    # dq, dk, dv, dg, dbeta
    nbytes += w.B * w.Hv * d * d * 4 * 3                                              # h0, dh_T, dh0
    return flops, nbytes


def measure_backward(w, x, steps, warmup, torch, gdn, with_cpu=True):
    """Time gdn_chunk_bwd on the workload's inputs (random dO and dh_T), as
    the forward: median of `steps` calls after a cache-evicting write, and
    back to back."""
    gen = torch.Generator(device="cuda").manual_seed(5)
    dO = torch.randn((w.B, w.T, w.Hv, w.dv), generator=gen, device="cuda")
    dhT = torch.randn((w.B, w.Hv, w.dk, w.dv), generator=gen, device="cuda") * 0.1
    shape = gdn.make_shape(w.B, w.T, w.Hqk, w.Hv, w.dk, w.dv, w.chunk, 0, x["k"].dtype, torch.float32)
    ws = torch.empty(gdn.workspace_size_bwd_grads(shape), dtype=torch.uint8, device="cuda")
    out = gdn.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], dO, h0=x["h0"], dh_T=dhT, chunk=w.chunk,
                        workspace=ws)

    def step():
        gdn.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], dO, h0=x["h0"], dh_T=dhT, chunk=w.chunk,
                      workspace=ws, out=out)
    tm = time_steps(step, steps, warmup)
    flops, nbytes = bwd_algorithmic(w)
    t = tm["cold"] * 1e-3
    res = {"workload": w.name, "ms_per_step": tm["cold"], "warm_ms_per_step": tm["warm"],
           "after_write_flush_ms_per_step": tm["dirty"],
           "value": w.tokens / t, "unit": "tokens/s",
           "roofline": {"bound": "mfma", "achieved": flops / t / 1e12, "peak": BF16_PEAK / 1e12,
                        "unit": "TFLOP/s", "frac": flops / t / BF16_PEAK,
                        "hbm_frac": nbytes / t / HBM_PEAK, "algorithmic_flops": flops,
                        "algorithmic_bytes": nbytes,
                        "note": "bf16 inputs: every product runs as three bf16 matrix-core passes "
                                "(hi/lo split operands)"},
           "workspace_bytes": ws.numel()}
    if with_cpu:
        res["cpu_baseline"] = cpu_baseline_bwd(w, x, dO, dhT)
    del ws, out, dO, dhT
    return res


def cpu_baseline_bwd(w, x, dO, dhT, budget_s=10.0):
    """The oracle's per-token reverse pass (numpy fp64, as it stands) over the
    first T_s tokens of batch row 0, all value heads."""
    from oracle import backward

    cpu = {kk: (None if vv is None else vv[:1].cpu()) for kk, vv in x.items()}
    dOc, dhc = dO[:1].cpu(), dhT[:1].cpu()

    def run(T_s):
        t0 = time.perf_counter()
        backward.bwd(*[cpu[kk][:, :T_s] for kk in ("q", "k", "v", "g", "beta")], cpu["h0"],
                     do=dOc[:, :T_s], dhT=dhc)
        return time.perf_counter() - t0
    T_s = min(w.T, 64)
    dt = run(T_s)
    T_s = max(T_s, min(w.T, int(T_s * budget_s / max(dt, 1e-6)) // 64 * 64))
    dt = run(T_s)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or None
    return {"value": T_s / dt, "unit": "tokens/s", "cores": threads or os.cpu_count(), "kind": "oracle",
            "sample": f"first {T_s} of {w.T} tokens of batch row 0, all {w.Hv} value heads; numpy fp64 "
                      f"per-token reverse pass, {dt:.2f} s (threads: numpy's BLAS default)"}


FUSED_MIN_WALKS = 128   # the library's GDN_FUSED_MIN_WALKS


def fused_walk(w):
    """Whether the library runs the walk that forms the outputs itself (no
    separate output stage) for this workload: as many walks as
    FUSED_MIN_WALKS or more (batch rows x value heads x groups)."""
    return w.B * w.Hv * max(w.n_groups, 1) >= FUSED_MIN_WALKS


def stage_bytes(w, o_bytes=4):
    """Minimum HBM bytes each kernel must move in this design (its inputs read
    once, its outputs written once)."""
    C, dk, dv = w.chunk, w.dk, w.dv
    tok = w.B * w.T
    s = 2 if w.dtype == "bf16" else 4
    N = -(-w.T // C)   # chunks (a partial last chunk counts whole)
    J = max(w.n_groups, 1)
    BHv = w.B * w.Hv
    k_b = tok * w.Hqk * dk * s
    q_b = k_b
    v_b = tok * w.Hv * dv * s
    gb_b = 8 * tok * w.Hv
    G_b = 4 * tok * w.Hv
    W_b = s * tok * w.Hv * dk
    U_b = 4 * tok * w.Hv * dv
    Hs_b = 4 * BHv * N * dk * dv
    Vn_b = 4 * tok * w.Hv * dv
    st = 4 * BHv * dk * dv
    h0_b = st if w.h0_std > 0 else 0
    pairs = 4 * BHv * J * (dk * dk + dk * dv)
    hin = 4 * BHv * J * dk * dv
    Kt_b = k_b                      # K^T per chunk and query/key head, input dtype
    out = {
        "prep": k_b + v_b + gb_b + G_b + W_b + Kt_b + U_b,
        "out": q_b + k_b + G_b + Hs_b + Vn_b + tok * w.Hv * dv * o_bytes,
    }
    init = h0_b if J == 1 else hin
    if J > 1:
        out["fold"] = W_b + U_b + G_b + Kt_b + pairs
        out["prefix"] = pairs + h0_b + hin + st
    if fused_walk(w):   # the walk reads q and k and writes o itself; no handoff
        del out["out"]
        out["walk"] = W_b + U_b + G_b + Kt_b + init + q_b + k_b + tok * w.Hv * dv * o_bytes + st
    else:
        out["walk"] = W_b + U_b + G_b + Kt_b + init + Hs_b + Vn_b + (st if J == 1 else 0)
    return out


def kernel_source_sha():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "linear_attention_rnn_gdn_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".h", ".hip")):
            h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernels):
    """HBM bytes per step of `kernels` (one launch each) from the committed
    rocprofv3 counter summary, if it was taken on the current kernel sources
    and covers every kernel; else None."""
    p = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha") != kernel_source_sha():
        return None
    per = d.get("workloads", {}).get(workload, {})
    try:
        return sum(per[k]["bytes_per_launch"] for k in kernels)
    except (KeyError, TypeError):
        return None


def _stage_of(kernel_name):
    """Map a demangled kernel name to its stage."""
    n = kernel_name
    if "prep_kernel" in n:
        return "prep"
    if "prefix_kernel" in n or "pair_walk_kernel" in n:   # (the blocked prefix's block passes)
        return "prefix"
    if "walk_out_kernel" in n:   # the walk that forms the outputs itself
        return "walk"
    if "out_kernel" in n:
        return "out"
    if "walk_pair_kernel" in n:   # (walk only; no KIND argument)
        return "walk"
    if "walk_ring_kernel" in n or "walk_shared_kernel" in n:
        # walk_*_kernel<C, TI, MODE, KIND[, WPG]>: KIND 1 = fold (demangled or
        # mangled name; TI is not an integer argument in the mangled form)
        import re
        tail = n.split("_kernel", 1)[1]
        if tail.startswith("<"):
            kind = tail[1:].split(">", 1)[0].split(",")[3].strip()
        else:
            kind = re.findall(r"Li(\d+)E", tail)[2]
        return "fold" if kind == "1" else "walk"
    if "copy" in n.lower():
        return "copy"
    return None


def _pmc_rows(d, counter):
    import csv
    import glob

    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection*.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r.get("Counter_Name") == counter:
                rows.append((int(r.get("Dispatch_Id", 0) or 0), r.get("Kernel_Name", ""),
                             float(r["Counter_Value"])))
    rows.sort()
    return [(name, val) for _, name, val in rows]


def summarize_pmc(fetch_dir, write_dir, workload, copy_bytes):
    """Per-launch HBM bytes per kernel from two rocprofv3 --pmc runs of
    `bench.py --profile-run` (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch),
    each scaled by what the counter reads for the calibration copy of
    `copy_bytes` bytes.  Writes profiles/hbm_traffic.json."""
    out = {}
    scale = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = {}
        for name, val in _pmc_rows(d, counter):
            st = _stage_of(name)
            if st:
                per.setdefault(st, []).append(val * 1024.0)
        # the calibration copies are the first three copy kernels of the run
        copy = sorted(per.get("copy", [])[:3])
        if len(copy) < 3:
            raise SystemExit(f"no calibration copy kernels found for {counter} in {d}")
        med = copy[1]
        scale[counter] = copy_bytes / med
        for st, vals in per.items():
            if st != "copy":
                out.setdefault(st, {})[counter] = sum(vals) / len(vals) * scale[counter]
    p = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        d = {}
    if d.get("kernel_source_sha") != kernel_source_sha():
        d = {"workloads": {}}
    d["kernel_source_sha"] = kernel_source_sha()
    d["note"] = ("bytes_per_launch = mean FETCH_SIZE + WRITE_SIZE per dispatch (KiB x 1024), each "
                 "scaled by copy_bytes / (what that counter reads for one torch copy of copy_bytes)")
    d["scale"] = scale
    d["workloads"][workload] = {st: {"fetch_bytes": v.get("FETCH_SIZE"),
                                     "write_bytes": v.get("WRITE_SIZE"),
                                     "bytes_per_launch": (v.get("FETCH_SIZE") or 0)
                                     + (v.get("WRITE_SIZE") or 0)}
                                for st, v in out.items()}
    json.dump(d, open(p, "w"), indent=1)
    print(json.dumps(d, indent=1))


def cpu_baseline(w, x, budget_s=15.0, one_thread=False):
    """Time the fp64 oracle (as it stands) on this host over a bounded sample:
    the first T_s tokens of every head of the workload, on all host cores
    (and, if `one_thread`, also on one thread over a shorter sample)."""
    import oracle

    nthreads = oracle.default_threads()
    cpu = {kk: (None if vv is None else vv.cpu()) for kk, vv in x.items()}

    def run(T_s, nt):
        sub = {kk: (vv[:, :T_s].contiguous() if kk != "h0" else vv) for kk, vv in cpu.items()}
        t0 = time.perf_counter()
        oracle.fwd(**sub, nthreads=nt)
        return time.perf_counter() - t0

    def measure(nt, budget):
        T_s = min(w.T, 256)
        dt = run(T_s, nt)
        if dt * w.T / T_s <= 2 * budget:
            T_s = w.T
        else:
            T_s = max(min(w.T, 256), min(w.T, int(T_s * budget / max(dt, 1e-6)) // 256 * 256))
        # repeat short samples until about 5 s of CPU work for a steady figure
        reps, total = 0, 0.0
        while reps == 0 or (total < 5.0 and reps < 50):
            total += run(T_s, nt)
            reps += 1
        return T_s, total / reps, reps

    T_s, dt, reps = measure(nthreads, budget_s)
    out = {"value": w.B * T_s / dt, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
           "sample": f"first {T_s} of {w.T} tokens x batch {w.B}, all {w.Hv} value heads, "
                     f"all {w.dv} state columns; fp64 per-token rule in C, {nthreads} threads; "
                     f"mean of {reps} runs, {dt:.2f} s each"}
    if one_thread:
        T1, dt1, reps1 = measure(1, budget_s / 3)
        out["one_thread"] = {"value": w.B * T1 / dt1, "unit": "tokens/s", "cores": 1,
                             "sample": f"first {T1} of {w.T} tokens x batch {w.B}, all heads and "
                                       f"columns; mean of {reps1} runs, {dt1:.2f} s each"}
    return out


def ramp_clocks(fn, seconds=0.5):
    """Untimed steps for `seconds` of wall time before the warm-up proper: a
    short burst of kernels leaves the GPU below its working clocks, and the
    first few hundred microseconds of work run measurably slower."""
    import torch

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


FLUSH_BYTES = 512 << 20   # twice the 256 MB memory-side cache (MALL)


def time_steps(fn, steps, warmup):
    """K steps, each after reading a 512 MB buffer, which evicts the
    memory-side cache and leaves it holding clean lines only, timed alone with
    HIP events on the current stream (median: `cold`); the same K steps each
    after a 512 MB write instead (median: `dirty`: the step then also writes
    back the cache's dirty lines of that buffer, about 256 MB, which is not its
    own work); then the K steps back to back (mean: `warm`).  Returns ms per
    step."""
    import statistics

    import torch

    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    flush.fill_(1.0)
    sink = torch.empty(1, dtype=torch.float32, device="cuda")
    ramp_clocks(fn)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()

    def timed(evict):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            evict(i)
            ev[i][0].record()
            fn()
            ev[i][1].record()
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(b) for a, b in ev)

    cold = timed(lambda i: sink.copy_(flush.sum().view(1)))
    dirty = timed(lambda i: flush.fill_(float(i)))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    del flush
    return {"cold": cold, "dirty": dirty, "warm": e0.elapsed_time(e1) / steps}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen3next_8b_layer")
    ap.add_argument("--secondary", default="long_256k",
                    help="second workload timed for context ('' to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward (gdn_chunk_bwd) timed at the headline workload")
    ap.add_argument("--n-groups", type=int, default=None,
                    help="override the workload's chunk-group count (0 = one sequential walk)")
    ap.add_argument("--packed", default="packed_8b_mix",
                    help="packed variable-length workload reported beside the headline ('' = none)")
    ap.add_argument("--profile-run", action="store_true",
                    help="counter-collection run: calibration copies, then the workload's steps")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/hbm_traffic.json from two --pmc runs of --profile-run")
    args = ap.parse_args()
    copy_bytes = 1 << 30
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload, copy_bytes)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import linear_attention_rnn_gdn_amd as gdn
    from workloads import WORKLOADS, make_inputs

    stage_bits = {"prep": gdn.STAGE_PREP, "fold": gdn.STAGE_FOLD, "prefix": gdn.STAGE_PREFIX,
                  "walk": gdn.STAGE_WALK, "out": gdn.STAGE_OUT}

    def setup(w):
        x = make_inputs(w, device="cuda")
        shape = gdn.make_shape(w.B, w.T, w.Hqk, w.Hv, w.dk, w.dv, w.chunk, w.n_groups,
                               x["k"].dtype, torch.float32)
        ws = torch.empty(gdn.workspace_size(shape), dtype=torch.uint8, device="cuda")
        o = torch.empty((w.B, w.T, w.Hv, w.dv), dtype=torch.float32, device="cuda")
        hT = torch.empty((w.B, w.Hv, w.dk, w.dv), dtype=torch.float32, device="cuda")

        def step(stages=None, events=None):
            gdn.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], chunk=w.chunk,
                          n_groups=w.n_groups, workspace=ws, out=o, final_state=hT, stages=stages,
                          events=events)
        return x, step

    w = WORKLOADS[args.workload]
    if args.n_groups is not None:
        w = w.replace(n_groups=args.n_groups)
    if args.profile_run:
        a = torch.empty(copy_bytes // 4, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1.0)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    x, step = setup(w)
    tm = time_steps(step, args.steps, args.warmup)
    if args.profile_run:
        print(json.dumps({"profile_run": w.name, "ms_per_step": tm}), flush=True)
        return
    line = measure(w, step, tm, args.steps, args.warmup, stage_bits, torch)
    if not args.no_backward:
        line["backward"] = measure_backward(w, x, max(5, args.steps // 5), 2, torch, gdn,
                                            with_cpu=not args.no_cpu_baseline)
        torch.cuda.empty_cache()
    if args.secondary and args.secondary != w.name:
        del x, step
        torch.cuda.empty_cache()
        w2 = WORKLOADS[args.secondary]
        x2, step2 = setup(w2)
        tm2 = time_steps(step2, max(3, args.steps // 4), 1)
        sec = measure(w2, step2, tm2, max(3, args.steps // 4), 1, stage_bits, torch)
        line["secondary"] = {kk: sec[kk] for kk in ("value", "unit", "ms_per_step", "warm", "after_write_flush", "roofline",
                                                    "mfma_util_pct", "stages_ms", "dominant_kernel")}
        line["secondary"]["workload"] = w2.name
        if not args.no_cpu_baseline:
            line["secondary"]["cpu_baseline"] = cpu_baseline(w2, x2)
        del x2, step2
        torch.cuda.empty_cache()
        x = make_inputs(w, device="cuda")
    if args.packed:
        # packed variable-length sequences (gdn_chunk_fwd_varlen), inputs and
        # workspace resident; reported beside the headline, not as `value`
        from workloads import make_packed_inputs
        del x
        torch.cuda.empty_cache()
        wp, xp, cu = make_packed_inputs(args.packed, device="cuda")
        shp = gdn.make_shape(len(cu) - 1, wp.T, wp.Hqk, wp.Hv, 128, 128, wp.chunk, 0, xp["k"].dtype,
                             torch.float32)
        wsp = torch.empty(gdn.workspace_size_varlen(shp), dtype=torch.uint8, device="cuda")
        op = torch.empty((1, wp.T, wp.Hv, 128), dtype=torch.float32, device="cuda")
        hp = torch.empty_like(xp["h0"])

        def step_p(stages=None, events=None):
            gdn.chunk_fwd_varlen(xp["q"], xp["k"], xp["v"], xp["g"], xp["beta"], cu, xp["h0"],
                                 chunk=wp.chunk, workspace=wsp, out=op, final_state=hp)
        tmp = time_steps(step_p, max(5, args.steps // 4), 2)
        line["packed"] = {"workload": args.packed, "sequences": len(cu) - 1, "tokens": wp.T,
                          "value": wp.T / (tmp["cold"] * 1e-3), "unit": "tokens/s",
                          "ms_per_step": tmp["cold"], "warm_ms_per_step": tmp["warm"]}
        del xp, op, hp, wsp
        torch.cuda.empty_cache()
        x = make_inputs(w, device="cuda")
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, x, one_thread=w.name in SMALL)
    print(json.dumps(line), flush=True)


SMALL = ("tiny", "qwen3next_8b_layer", "dense_d4096_layer")   # 1-thread oracle times too


def stage_times(w, step, steps, stage_bits, torch):
    """Per-kernel times: the steps again, each kernel launched with a pair of
    HIP events that record its own start and end on the launch stream
    (gdn_chunk_fwd_timed), all steps queued back to back, the first dropped."""
    names = [n for n in ("prep", "fold", "prefix", "walk", "out")
             if (w.n_groups > 1 or n not in ("fold", "prefix")) and not (n == "out" and fused_walk(w))]
    bit = {n: stage_bits[n].bit_length() - 1 for n in names}
    nst = steps + 1
    ev = [[[None] * 5, [None] * 5] for _ in range(nst)]
    for k in range(nst):
        for n in names:
            for side in (0, 1):
                e = torch.cuda.Event(enable_timing=True)
                e.record()   # creates the event
                ev[k][side][bit[n]] = e
    torch.cuda.synchronize()
    for k in range(nst):
        step(events=(ev[k][0], ev[k][1]))
    torch.cuda.synchronize()
    return {n: sum(ev[k][0][bit[n]].elapsed_time(ev[k][1][bit[n]]) for k in range(1, nst)) / steps
            for n in names}


def measure(w, step, tm, steps, warmup, stage_bits, torch):
    stage_ms = stage_times(w, step, steps, stage_bits, torch)
    flops, nbytes = algorithmic(w)
    t = tm["cold"] * 1e-3
    achieved = nbytes / t
    traffic = measured_traffic(w.name, list(stage_ms))
    # the whole step against the method's own bytes (HBM binds at every bf16
    # workload: its FLOP per byte is below the bf16 ridge of ~315)
    roof = {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
            "frac": achieved / HBM_PEAK, "traffic": traffic,
            "traffic_ratio": None if traffic is None else traffic / nbytes,
            "scope": "whole step (all kernels of one gdn_chunk_fwd call)",
            "algorithmic_bytes": nbytes, "step_ms": tm["cold"],
            "kernels_ms_sum": sum(stage_ms.values())}
    sb = stage_bytes(w)
    dom = max(stage_ms, key=stage_ms.get)
    dom_s = stage_ms[dom] * 1e-3
    dominant = {"kernel": dom, "avg_launch_ms": stage_ms[dom], "design_bytes_per_launch": sb[dom],
                "design_bytes_frac": sb[dom] / dom_s / HBM_PEAK,
                "algorithmic_bytes_frac": nbytes / dom_s / HBM_PEAK}
    return {
        "metric": METRIC,
        "value": w.tokens / t,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": tm["cold"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H_qk": w.Hqk, "H_v": w.Hv,
                   "d_k": w.dk, "d_v": w.dv, "chunk": w.chunk, "n_groups": w.n_groups,
                   "o_dtype": "f32", "parallelism": "single GPU"},
        "warm": {"ms_per_step": tm["warm"], "value": w.tokens / (tm["warm"] * 1e-3),
                 "hbm_frac": nbytes / (tm["warm"] * 1e-3) / HBM_PEAK},
        "after_write_flush": {"ms_per_step": tm["dirty"], "value": w.tokens / (tm["dirty"] * 1e-3),
                              "hbm_frac": nbytes / (tm["dirty"] * 1e-3) / HBM_PEAK},
        "mfma_util_pct": 100.0 * flops / t / BF16_PEAK,
        "roofline": roof,
        "algorithmic": {"flops": flops, "bytes": nbytes, "mfma_frac": flops / t / BF16_PEAK},
        "stages_ms": stage_ms,
        "dominant_kernel": dominant,
    }


if __name__ == "__main__":
    main()
