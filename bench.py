"""Benchmark of the attention forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-extra]
                [--cpu-seconds S] [--no-cpu] [--copy-calibration-mib M]

A step is one fa_fwd call over one batch of the workload's seeded synthetic
input, resident in HBM before timing starts.  The headline workload is the
largest single-GPU configuration, the long-context causal GQA forward
B=1, Hq=32, Hkv=8, Lq=Lk=16384, D=128 (Q x4 on every 8th head).  The tiny,
1K prefill, causal 4K and split-KV decode workloads, and the follow-on
variants (the GQA workload under a causal window of 4096 keys; the decode
workload served from a shuffled paged cache with 16-token pages; the
backward of the causal 4K and 1K prefill workloads, one fa_bwd call per
step; the causal 4K and GQA 16K forward with FP8 scores, one fa_fwd_fp8 call
per step on Q and K quantized beforehand, the quantization timed separately
and added for the end-to-end figure, and the other end-to-end form timed
too: K quantized, then fa_fwd_fp8_q quantizing Q inside the forward; the causal 4K forward with ALiBi biases
and the 1K prefill with soft-capped scores, one fa_fwd_mod call per step;
the causal GQA forward over 16 packed sequences of 128-8192 tokens, one
fa_fwd_varlen call per step with the longest-tile-first schedule computed
once for the batch and its kernel timed separately), are reported under
"workloads".

Timing: W untimed warmup steps, then exactly K steps between two HIP events
on the stream the kernels are launched on (torch's current stream),
bracketed by device synchronisation; that gives ``ms_per_step`` and
``value``.  The other workloads are warmed for at least 100 ms of calls
before their K steps (the clock settles under a sustained load).  Every workload is also timed in at least five trials of at least
50 ms each (back-to-back calls between events); their median and minimum
per-call times are reported under ``trials``.

Printed: one JSON line with the metric, throughput, a roofline object for the
dominant kernel of the headline workload and a CPU baseline (the fp64 oracle
timed on this host's cores on a bounded sample of the same workload); the
other forward workloads of the five carry their own CPU-baseline figure.
"""
from __future__ import annotations

import argparse
import hashlib
import itertools
import json
import glob
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s & % of MI355X bf16 MFMA peak; decode HBM GB/s & % peak"
PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0       # HBM3E, 8 TB/s
PEAK_FP8_TFLOPS = 5033.2    # dense fp8 MFMA, twice the bf16 rate
# FP8-score forward: half the algorithmic FLOPs (S = QK^T) at the fp8 rate and
# half (PV) at the bf16 rate, so its peak is the harmonic combination.
PEAK_FP8_SCORES_TFLOPS = 2.0 / (1.0 / PEAK_FP8_TFLOPS + 1.0 / PEAK_BF16_TFLOPS)
HEADLINE = "gqa_causal_b1_hq32_hkv8_l16384_d128"
# The five workloads the metric is stated for (the others are follow-on variants).
FIVE = ["tiny_b1_h2_l256_d64", "prefill_b4_h16_l1024_d64", "causal_b2_h16_l4096_d128",
        "gqa_causal_b1_hq32_hkv8_l16384_d128", "decode_b64_hq32_hkv8_d128_ragged"]
TRIAL_MS = 50.0
TRIALS = 5
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


# The sources a profiled kernel is built and launched from: its own file plus
# the shared device and launch headers and the C ABI that sizes its launch.
KERNEL_SOURCES = {
    "prefill_kernel": ["fa_prefill.hip"],
    "splitkv_kernel": ["fa_splitkv.hip"],
    "combine_kernel": ["fa_splitkv.hip"],
    "bwd_dkdv_split_kernel": ["fa_backward.hip"],
    "bwd_dkdv_kernel": ["fa_backward.hip"],
    "bwd_dq_kernel": ["fa_backward.hip"],
    "quantize_fp8_kernel": ["fa_fp8.hip"],
    "varlen_schedule_kernel": ["fa_varlen.hip"],
}
KERNEL_COMMON = ["fa_device.h", "fa_internal.h", "fa_api.hip"]


def kernel_source_hash(kernel: str = None) -> str:
    """Hash of the kernel sources (all of them, or those of one kernel); a
    stored traffic figure is only reported for the exact sources its counters
    were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_attention_07_amd", "csrc")
    if kernel is None:
        paths = sorted(glob.glob(os.path.join(csrc, "*")))
    else:
        paths = [os.path.join(csrc, f) for f in sorted(KERNEL_SOURCES[kernel] + KERNEL_COMMON)]
    for path in paths:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    try:
        with open(PROFILE_TRAFFIC) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(workload)
    if not entry or entry.get("kernel") not in KERNEL_SOURCES or \
            entry.get("source_hash") != kernel_source_hash(entry["kernel"]):
        return None
    return entry.get("bytes_per_launch")


def timed_trials(call, est_ms):
    """At least TRIALS trials of back-to-back calls, each lasting at least
    TRIAL_MS (the call count per trial follows from ``est_ms``, one call's
    time); returns the median and minimum per-call time over the trials."""
    import statistics

    import torch
    reps = max(1, int(math.ceil(TRIAL_MS / max(est_ms, 1e-4))))
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per_call = []
    for _ in range(TRIALS):
        torch.cuda.synchronize()
        start.record()
        for _ in range(reps):
            call()
        end.record()
        torch.cuda.synchronize()
        per_call.append(start.elapsed_time(end) / reps)
    return {"median_ms": statistics.median(per_call), "min_ms": min(per_call), "trials": TRIALS,
            "calls_per_trial": reps, "trial_ms": statistics.median(per_call) * reps}


def time_workload(w, steps, warmup, dev, trials=True, warm_ms=0.0):
    import torch
    from exact_attention_07_amd import binding, workloads as W

    inp = W.make_inputs(w)
    q = inp.q.to(dev)
    kl = None if inp.kv_lens is None else inp.kv_lens.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    lens = None
    # Arguments are checked and marshalled once; each step is one C-ABI call,
    # so host overhead stays below the kernel time.
    if w.varlen is not None:
        # Packed batch: the longest-tile-first schedule is computed once for the
        # batch layout (as a serving loop reuses it); the step is one
        # fa_fwd_varlen.  The schedule kernel is timed separately below.
        k, v = inp.k.to(dev), inp.v.to(dev)
        cq, ck = inp.meta["cu_seqlens_q"].to(dev), inp.meta["cu_seqlens_k"].to(dev)
        call = binding.PreparedVarlenCall(q, k, v, cq, ck, o, lse, causal=w.causal, scale=w.scale)
        lens = list(zip(inp.meta["lens_q"], inp.meta["lens_k"]))
        sched = call.schedule
        lib = binding.load_library()
        sargs = (cq.data_ptr(), ck.data_ptr(), w.B, q.shape[1], k.shape[1], sched.data_ptr(),
                 torch.cuda.current_stream(dev).cuda_stream)

        def schedule():
            lib.fa_varlen_schedule(*sargs)
    elif w.backward:
        k, v = inp.k.to(dev), inp.v.to(dev)
        fwd = binding.PreparedCall(q, k, v, o, lse, causal=w.causal, scale=w.scale, kv_lens=kl,
                                   window=w.window if w.window else None)
        fwd()                                   # the forward's o and lse are the backward's inputs
        call = binding.PreparedBwdCall(q, k, v, o, lse, inp.meta["dout"].to(dev), causal=w.causal,
                                       window=w.window, scale=w.scale, kv_lens=kl)
    elif w.alibi or w.softcap:
        k, v = inp.k.to(dev), inp.v.to(dev)
        sl = inp.meta["alibi_slopes"].to(dev) if w.alibi else None
        call = binding.PreparedModCall(q, k, v, o, lse, causal=w.causal, scale=w.scale, kv_lens=kl,
                                       alibi_slopes=sl, softcap=w.softcap)
    elif w.fp8:
        # Q and K quantized (after the random-sign Hadamard transform) before
        # timing, as an FP8 cache would hold them; the step is one fa_fwd_fp8.
        # The quantizer is timed separately below.
        k, v = inp.k.to(dev), inp.v.to(dev)
        sg = inp.meta["signs"].to(dev)
        q8, qs = binding.quantize_fp8(q, binding.FP8_Q_BLOCK, sg)
        k8, ks = binding.quantize_fp8(k, binding.FP8_K_BLOCK, sg)
        call = binding.PreparedFp8Call(q8, k8, v, qs, ks, causal=w.causal, scale=w.scale / w.D, kv_lens=kl)

        lib = binding.load_library()
        st = torch.cuda.current_stream(dev).cuda_stream
        qargs = (q.data_ptr(), q8.data_ptr(), qs.data_ptr(), w.B * w.Hq, w.Lq, w.D, binding.FP8_Q_BLOCK,
                 sg.data_ptr(), st)
        kargs = (k.data_ptr(), k8.data_ptr(), ks.data_ptr(), w.B * w.Hkv, w.Lk, w.D, binding.FP8_K_BLOCK,
                 sg.data_ptr(), st)

        def quantize():                     # one ctypes call each, arguments marshalled once
            lib.fa_quantize_fp8(*qargs)
            lib.fa_quantize_fp8(*kargs)

        # The other end-to-end form: K quantized, Q quantized inside the
        # forward (fa_fwd_fp8_q, bit for bit the same result).
        fused_q = binding.PreparedFp8QCall(q, k8, v, ks, sg, causal=w.causal, scale=w.scale / w.D, kv_lens=kl)

        def quantize_k_fused():
            lib.fa_quantize_fp8(*kargs)
            fused_q()
    elif w.page_size:
        # Only the paged copy of K and V is resident for a paged workload.
        kc, vc, table = (t.to(dev) for t in inp.meta["paged"])
        k, v = kc, vc
        call = binding.PreparedPagedCall(q, kc, vc, table.contiguous(), kl, o, lse, causal=w.causal,
                                         window=w.window, scale=w.scale)
    else:
        k, v = inp.k.to(dev), inp.v.to(dev)
        call = binding.PreparedCall(q, k, v, o, lse, causal=w.causal, scale=w.scale, kv_lens=kl,
                                    window=w.window if w.window else None)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    # Optionally keep warming for warm_ms of wall time (clocks settle under a
    # sustained load; a few short calls from idle run at a lower clock).
    t_warm = time.perf_counter()
    while (time.perf_counter() - t_warm) * 1e3 < warm_ms:
        for _ in range(8):
            call()
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        call()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    flops = W.algorithmic_flops(w, inp.kv_lens, lens=lens)
    nbytes = W.compulsory_bytes(w, inp.kv_lens, lens=lens)
    rec = {"ms_per_step": ms, "flops": flops, "bytes": nbytes,
           "tflops": flops / (ms * 1e-3) / 1e12, "gbs": nbytes / (ms * 1e-3) / 1e9}
    if trials:
        rec["trials"] = timed_trials(call, ms)
    if w.Lq == 1 and not w.backward:
        rec.update(bound="hbm", frac=rec["gbs"] / PEAK_HBM_GBS)
    elif w.fp8:
        rec.update(bound="mfma", frac=rec["tflops"] / PEAK_FP8_SCORES_TFLOPS, peak=PEAK_FP8_SCORES_TFLOPS)
        quantize()
        torch.cuda.synchronize()
        start.record()
        for _ in range(steps):
            quantize()
        end.record()
        torch.cuda.synchronize()
        rec["quantize_ms"] = start.elapsed_time(end) / steps
        e2e = ms + rec["quantize_ms"]
        rec["end_to_end_ms"] = e2e
        rec["end_to_end_tflops"] = flops / (e2e * 1e-3) / 1e12
        quantize_k_fused()
        torch.cuda.synchronize()
        start.record()
        for _ in range(steps):
            quantize_k_fused()
        end.record()
        torch.cuda.synchronize()
        rec["fused_q_end_to_end_ms"] = start.elapsed_time(end) / steps
    else:
        rec.update(bound="mfma", frac=rec["tflops"] / PEAK_BF16_TFLOPS)
    if w.varlen is not None:
        schedule()
        torch.cuda.synchronize()
        start.record()
        for _ in range(steps):
            schedule()
        end.record()
        torch.cuda.synchronize()
        rec["schedule_ms"] = start.elapsed_time(end) / steps
        # Ablation of the sort: the same call with the sequences in the order
        # given (a schedule in the same layout without the sort).
        nqb = [-(-n // 256) for n in inp.meta["lens_q"]]
        plain = torch.tensor(list(range(w.B)) + [0] + list(itertools.accumulate(nqb)), dtype=torch.int32,
                             device=dev)
        if trials:
            unsorted = binding.PreparedVarlenCall(q, k, v, cq, ck, o, lse, schedule=plain, causal=w.causal,
                                                  scale=w.scale)
            rec["unsorted_trials"] = timed_trials(unsorted, ms)
            del unsorted
        rec["sequence_lengths"] = inp.meta["lens_q"]
        rec["total_tokens"] = int(q.shape[1])
    if w.name in FIVE:
        torch.cuda.synchronize()
        inp.meta["gpu_out"] = (o.cpu(), lse.cpu())   # compared with the oracle's sample in cpu_baseline
    del call, q, k, v, o, lse, kl
    torch.cuda.empty_cache()
    return rec, inp


def host_cores() -> int:
    """The cores this process may run on (its CPU affinity)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(w, inp, seconds, chunk=512):
    """Time the fp64 oracle, as it stands, on the workload's host cores:
    (batch, query head, chunk of up to ``chunk`` query rows) units in order,
    one per thread of a pool of ``host_cores()`` threads (numpy's matrix
    products and elementwise loops release the interpreter lock; BLAS is held
    to one thread per worker), until about ``seconds`` of wall time; report
    the algorithmic TFLOP/s of the completed units (GB/s of compulsory bytes
    for decode)."""
    from concurrent.futures import ThreadPoolExecutor, FIRST_COMPLETED, wait

    import numpy as np
    import torch
    import oracle
    from exact_attention_07_amd import workloads as W
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover - part of the image
        threadpool_limits = None
    cores = host_cores()
    ns = W.valid_lengths(w, inp.kv_lens)
    units = [(b, h, r0, min(r0 + chunk, w.Lq)) for b in range(w.B) for h in range(w.Hq)
             for r0 in range(0, w.Lq, chunk)]

    got = inp.meta.get("gpu_out")

    def unit_work(u):
        b, h, r0, r1 = u
        rows = np.arange(r0, r1)
        ro, rl = oracle.attention_rows(inp.q, inp.k, inp.v, w.scale, w.causal, inp.kv_lens, b, h, rows,
                                       window=w.window)
        if got is not None:
            # The same rows of the timed kernel's output against the oracle's.
            go = got[0][b, h, r0:r1].double().numpy()
            gl = got[1][b, h, r0:r1].double().numpy()
            ro, rl = np.asarray(ro, np.float64), np.asarray(rl, np.float64)
            d = np.abs(go - ro)
            both_inf = np.isneginf(gl) & np.isneginf(rl)
            dl = np.where(both_inf, 0.0, np.abs(gl - rl))
            # Elements that no bf16 value can bring within 1e-2 (|O| >= 4, O
            # more than 1e-2 from both bf16 neighbours) must be one of those
            # neighbours: an error below one bf16 spacing of O.
            floor = np.abs(torch.from_numpy(ro).to(torch.bfloat16).double().numpy() - ro)
            unrep = floor > 1e-2
            spacing = np.ldexp(1.0, np.frexp(np.abs(ro))[1] - 8)
            bad_unrep = int(np.count_nonzero(unrep & (d >= spacing)))
            err.append((float(np.where(unrep, 0.0, d).max(initial=0.0)), float((d * d).sum()), float((ro * ro).sum()),
                        float(dl.max(initial=0.0)), u, float(d.max(initial=0.0)), int(np.count_nonzero(unrep)),
                        bad_unrep))
        n = ns[b]
        off = n - w.Lq
        pairs = 0
        for i in range(r0, r1):
            p = off + i
            hi = min(p + 1, n) if w.causal else n
            lo = max(p - w.window + 1, 0) if w.window > 0 else 0
            pairs += max(hi - lo, 0)
        kv_bytes = 2 * n * w.D * 2 // (w.Hq // w.Hkv) if r0 == 0 else 0
        return 4 * w.D * pairs, (r1 - r0) * (2 * w.D * 2 + 4) + kv_bytes

    done_flops = done_bytes = done = 0
    err = []
    ctx = threadpool_limits(limits=1, user_api="blas") if threadpool_limits else None
    t0 = time.perf_counter()
    try:
        with ThreadPoolExecutor(max_workers=cores) as ex:
            nxt = 0
            running = set()
            while True:
                while len(running) < cores and time.perf_counter() - t0 < seconds:
                    running.add(ex.submit(unit_work, units[nxt % len(units)]))
                    nxt += 1
                if not running:
                    break
                fin, running = wait(running, return_when=FIRST_COMPLETED)
                for f in fin:
                    fl, by = f.result()
                    done_flops += fl
                    done_bytes += by
                    done += 1
    finally:
        if ctx is not None:
            ctx.restore_original_limits()
    dt = time.perf_counter() - t0
    sample = (f"{done} (batch, query head, {chunk}-row) units of {len(units)} in the workload "
              f"({done / len(units):.3f} passes) on {cores} threads, fp64 dense S, P, O, {dt:.1f} s")
    if w.Lq == 1:
        res = {"value": done_bytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
               "sample": sample}
    else:
        res = {"value": done_flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
               "sample": sample}
    if err:
        # Parity of the timed output on the oracle's sample, against the
        # forward's bar: max |dO| <= 1e-2 wherever a bf16 value can meet it
        # (elsewhere one of O's two bf16 neighbours), relative L2 of O <= 4e-3,
        # max |dLSE| <= 1e-3.
        seen = {}
        for e in err:
            seen[e[4]] = e                  # units timed more than once: count each once
        err = list(seen.values())
        max_rep = max(e[0] for e in err)
        rel_l2 = math.sqrt(sum(e[1] for e in err) / max(sum(e[2] for e in err), 1e-300))
        dlse = max(e[3] for e in err)
        bad = sum(e[7] for e in err)
        res["parity"] = {"rows": sum(e[4][3] - e[4][2] for e in err), "max_abs": max(e[5] for e in err),
                         "max_abs_representable": max_rep, "unrepresentable": sum(e[6] for e in err),
                         "unrepresentable_off_neighbours": bad, "rel_l2": rel_l2, "max_abs_dlse": dlse,
                         "bar": {"max_abs": 1e-2, "rel_l2": 4e-3, "max_abs_dlse": 1e-3},
                         "within_bar": bool(max_rep <= 1e-2 and bad == 0 and rel_l2 <= 4e-3 and dlse <= 1e-3)}
    return res


def print_parity(name, cpu):
    par = cpu.get("parity")
    if par:
        print(f"[bench] parity of {name} on the oracle's {par['rows']} sampled rows: max |dO| {par['max_abs']:.3e} "
              f"({par['max_abs_representable']:.3e} where bf16 can meet 1e-2; {par['unrepresentable']} elements "
              f"where it cannot, {par['unrepresentable_off_neighbours']} of them off O's bf16 neighbours), "
              f"rel L2 {par['rel_l2']:.3e}, max |dLSE| {par['max_abs_dlse']:.3e}, "
              f"{'within' if par['within_bar'] else 'OUTSIDE'} the forward's bar", flush=True)


def copy_calibration(mib, dev):
    """A plain device-to-device copy of known size, for scaling HBM counters."""
    import torch
    n = mib * (1 << 20)
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(f"[bench] copy calibration: {n} bytes read, {n} bytes written", flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-extra", action="store_true", help="time only the headline workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall time of the oracle baseline on the headline workload")
    ap.add_argument("--cpu-seconds-each", type=float, default=6.0,
                    help="wall time of the oracle baseline on each other workload of the five")
    ap.add_argument("--no-trials", action="store_true",
                    help="skip the 5 x 50 ms trials (profiling runs)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the forward of one GPU's share is the unit measured; "
              "multi-GPU runs are not part of this library", file=sys.stderr)
        sys.exit(2)

    import torch
    from exact_attention_07_amd import binding, workloads as W

    binding.load_library()   # raises if libfa.so is not built: there is no fallback path
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib, dev)

    head = W.BY_NAME[args.workload]
    print(f"[bench] timing {head.name}: warmup {args.warmup}, steps {args.steps}", flush=True)
    rec, inp = time_workload(head, args.steps, args.warmup, dev, trials=not args.no_trials)
    tr = rec.get("trials")
    print(f"[bench] {head.name}: {rec['ms_per_step'] * 1e3:.1f} us/step"
          + (f" (trials: median {tr['median_ms'] * 1e3:.1f}, min {tr['min_ms'] * 1e3:.1f} us)" if tr else "")
          + f", {100 * rec['frac']:.1f}% of peak"
          + (f", quantizing Q and K {rec['quantize_ms'] * 1e3:.1f} us" if "quantize_ms" in rec else ""), flush=True)

    def rounded(r):
        return {k: (round(v, 6) if isinstance(v, float) else (rounded(v) if isinstance(v, dict) else v))
                for k, v in r.items()}

    extra = {}
    if not args.no_extra:
        for w in W.WORKLOADS:
            if w.name == head.name:
                continue
            steps = max(3, min(args.steps, 20))
            r, winp = time_workload(w, steps, max(2, min(args.warmup, 5)), dev, trials=not args.no_trials,
                                    warm_ms=100.0)
            if w.name in FIVE and not args.no_cpu:
                print(f"[bench] CPU oracle baseline on {w.name} (~{args.cpu_seconds_each:.0f} s)", flush=True)
                r["cpu_baseline"] = cpu_baseline(w, winp, args.cpu_seconds_each)
                print_parity(w.name, r["cpu_baseline"])
            del winp
            r["traffic"] = stored_traffic(w.name)
            extra[w.name] = rounded(r)
            tr = r.get("trials")
            print(f"[bench] {w.name}: {r['ms_per_step'] * 1e3:.1f} us/step"
                  + (f" (trials: median {tr['median_ms'] * 1e3:.1f}, min {tr['min_ms'] * 1e3:.1f} us)" if tr else "")
                  + f", {r['tflops']:.1f} TFLOP/s, {r['gbs']:.0f} GB/s, {100 * r['frac']:.1f}% of peak"
                  + (f", quantizing Q and K {r['quantize_ms'] * 1e3:.1f} us" if "quantize_ms" in r else "")
                  + (f", K quantized and Q in the kernel (fa_fwd_fp8_q) {r['fused_q_end_to_end_ms'] * 1e3:.1f} us"
                     if "fused_q_end_to_end_ms" in r else "")
                  + (f", schedule {r['schedule_ms'] * 1e3:.1f} us" if "schedule_ms" in r else "")
                  + (f", unsorted order median {r['unsorted_trials']['median_ms'] * 1e3:.1f} us"
                     if "unsorted_trials" in r else ""), flush=True)

    decode = head.Lq == 1
    value = rec["gbs"] if decode else rec["tflops"]
    unit = "GB/s" if decode else "TFLOP/s"
    traffic = stored_traffic(head.name)
    roof = {"bound": rec["bound"], "achieved": round(value, 3),
            "peak": PEAK_HBM_GBS if decode else rec.get("peak", PEAK_BF16_TFLOPS),
            "unit": unit, "frac": round(rec["frac"], 4), "traffic": traffic}
    cpu = None
    if not args.no_cpu and head.varlen is None:   # the oracle baseline is for the batched layout
        print(f"[bench] CPU oracle baseline on {head.name} (~{args.cpu_seconds:.0f} s)", flush=True)
        cpu = cpu_baseline(head, inp, args.cpu_seconds)
        print_parity(head.name, cpu)
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(rec["ms_per_step"], 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 scores, bf16 PV" if head.fp8 else "bf16",
        "data": "synthetic (seeded N(0,1) bf16 inputs)",
        "config": {"workload": head.name, "B": head.B, "Hq": head.Hq, "Hkv": head.Hkv,
                   "Lq": head.Lq, "Lk": head.Lk, "D": head.D, "causal": head.causal,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "trials": rounded(rec["trials"]) if "trials" in rec else None,
        "workloads": extra,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
