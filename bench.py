"""Decode benchmark: ResidualQuant fused decode attention on one MI355X.

Default workload (the metric's configuration): one layer, batch 16, 16 heads,
head_dim 128, 4 loops (loop 3 the BF16 reference, loops 0-2 INT2 residuals,
g = 32, Hadamard rotation), 8192-token context.  One step = one
rq_decode_attn call over all four loops (a single kernel launch), on seeded
synthetic KV already encoded in HBM.  Two cache replicas alternate so that
consecutive steps cannot be served from the 256 MB Infinity Cache.

Prints one JSON line: decode tokens/s (batch / step time), the roofline of the
decode kernel (algorithmic bytes / mean launch time, from two HIP events on
the launch stream around the timed steps), and the CPU oracle timed on a
bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published
SETTLE_MS = 250.0       # untimed work before every timed measurement (see parse)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=5)
    # From idle the GPU's clocks take ~200 ms of back-to-back work to reach
    # their steady state: interleaved rounds of 90 int2-8k steps (~25 ms
    # each) run ~9 % slower in the first round and ~3 % slower in rounds
    # 2-4 than from round 5 on.  So after the warm-up steps every timed
    # measurement first runs untimed steps until this much work is done,
    # whatever --warmup says.
    p.add_argument("--settle-ms", type=float, default=250.0)
    p.add_argument("--trials", type=int, default=3,
                   help="trials of --trial-steps steps after the timed steps (the pages' protocol: "
                        "one warm-up, three trials, averaged)")
    p.add_argument("--trial-steps", type=int, default=127)
    p.add_argument("--cpu-threads", type=int, default=0, help="host threads of the oracle fan-out (0 = all)")
    p.add_argument("--workload", default="int2-8k")
    p.add_argument("--splits", type=int, default=0, help="token splits (0 = library's choice)")
    p.add_argument("--replicas", type=int, default=2)
    p.add_argument("--cpu-sample", type=int, default=256, help="(batch, head) pairs the oracle decodes")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-bf16-baseline", action="store_true")
    p.add_argument("--no-sdpa", action="store_true",
                   help="int2-8k: skip timing torch's SDPA (flash / memory-efficient backends) on the BF16 "
                        "baseline's shapes")
    p.add_argument("--graphs", action="store_true",
                   help="grid workloads: time each step as a replayed HIP graph (both RQ and BF16)")
    p.add_argument("--contexts", default="",
                   help="grid workloads: comma-separated context lengths to run (default: the workload's)")
    p.add_argument("--batches", default="",
                   help="grid workloads: comma-separated batches to run at each context (default: powers of "
                        "two up to the largest that fits, and that largest)")
    p.add_argument("--mode", default="decode", choices=["decode", "copy", "split-sweep", "stream", "encode"],
                   help="copy: a plain 1 GiB device copy, the reference for HBM counter scaling; "
                        "split-sweep: every token-split count against the automatic one; "
                        "stream: the attainable HBM read rate (128-bit read-stream kernel); "
                        "encode: the prefill rq_encode of the workload's layer alone")
    a = p.parse_args()
    global SETTLE_MS
    SETTLE_MS = a.settle_ms
    a.steps_given = a.steps is not None
    if a.steps is None:
        a.steps = 127
    return a


def layout_bytes_per_token(n_loops: int, bits, g: int, d: int, ref_bits: int = 0,
                           ref_group: int = 0) -> int:
    """Bytes per (batch, head, token), K plus V, of the cache layout in
    include/rq.h: the reference (BF16 rows, or anchor codes plus an FP16
    scale and zero per group of ref_group) and, per residual loop, its codes,
    an FP16 scale and zero per group of g and an FP16 LS coefficient."""
    ref = 2 * d if not ref_bits else d * ref_bits // 8 + 4 * (d // (ref_group or g))
    return 2 * (ref + sum(d * bits[l] // 8 + 4 * (d // g) + 2 for l in range(n_loops - 1)))


def loop_read_bytes_per_token(bits: int, g: int, d: int, ref_bits: int = 0, ref_group: int = 0) -> int:
    """Bytes per (batch, head, token), K plus V, that attending over ONE
    residual loop on its own reads: the reference and that loop's planes."""
    ref = 2 * d if not ref_bits else d * ref_bits // 8 + 4 * (d // (ref_group or g))
    return 2 * (ref + d * bits // 8 + 4 * (d // g) + 2)


def algorithmic_bytes_per_token(w) -> int:
    """Bytes one fused decode step must read per (batch, head, token): the
    reference K and V once, and every residual loop's planes."""
    return layout_bytes_per_token(w.n_loops, w.bits, w.g, w.d, w.ref_bits, w.ref_group)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("rq_decode.hip", "rq_decode_kernel.hpp", "rq_device.hpp", "rq_internal.hpp"):
        h.update(open(os.path.join(ROOT, "decode_attention_rq_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when they were taken on different kernel source."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    if t.get("kernel_source_sha") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def host_threads(requested: int = 0) -> int:
    """Host threads for the oracle fan-out: the request, else the CPUs this
    process may run on, at most 16 (a one-GPU share of a GPU host)."""
    if requested > 0:
        return requested
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_layer(w, n_pairs: int, n_ctx: int, seed: int):
    """n_pairs (batch, head) pairs of workload w's layout, drawn and encoded
    by the oracle (one head per pair: layout batch = n_pairs, heads = 1)."""
    import synth
    from oracle import rq_oracle as orc
    from synth import bf16_bits

    g = synth.generator(seed)
    kstd, vstd = synth.channel_std(g, 1, w.d), synth.channel_std(g, 1, w.d)
    kr, kl = synth.draw_kv(g, w.n_loops, n_pairs, 1, n_ctx, w.d, w.c, w.sigma, kstd)
    vr, vl = synth.draw_kv(g, w.n_loops, n_pairs, 1, n_ctx, w.d, w.c, w.sigma, vstd)
    q = synth.draw_queries(g, w.n_loops, n_pairs, 1, w.d)
    lay = dict(n_loops=w.n_loops, batch=n_pairs, heads=1, d=w.d, g=w.g, cap=n_ctx,
               rotate=w.rotate, bits=w.bits)
    kp = orc.Planes(w.n_loops, n_pairs, 1, w.d, w.g, n_ctx, w.bits)
    vp = orc.Planes(w.n_loops, n_pairs, 1, w.d, w.g, n_ctx, w.bits)
    kp.ref[:] = bf16_bits(kr)
    vp.ref[:] = bf16_bits(vr)
    kin, vin = bf16_bits(kl), bf16_bits(vl)
    return lay, kp, vp, kin, vin, bf16_bits(q)


def oracle_decode_timing(w, lay, kp, vp, qb, n_pairs: int, n_ctx: int, threads: int, single_pairs: int):
    """Seconds per (batch, head) pair (all loops over n_ctx tokens) of the
    oracle's decode (FP64 reconstruction + FP64 attention): single-threaded
    over single_pairs pairs, and fanned out over `threads` host threads, one
    (loop, batch, head) row per task, over all n_pairs pairs.  The oracle
    is plain C called through ctypes, which releases the GIL during the
    call, so the rows run in parallel."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    from oracle import rq_oracle as orc

    scale = 1.0 / np.sqrt(w.d)
    rows = [(l, b) for b in range(n_pairs) for l in range(w.n_loops)]
    run = lambda r: orc.decode_row(lay, kp, vp, qb, r[0], r[1], 0, n_ctx, scale)
    run(rows[0])                                   # loads the library
    t0 = time.perf_counter()
    for r in rows[:single_pairs * w.n_loops]:
        run(r)
    one = (time.perf_counter() - t0) / single_pairs
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(run, rows))
    many = (time.perf_counter() - t0) / n_pairs
    return one, many


def cpu_baseline(w, n_pairs: int, threads: int = 0, single_pairs: int = 48, n_ctx: int = 0,
                 batch: int = 0, what: str = ""):
    """The oracle's decode (FP64 reconstruction + FP64 attention) on n_pairs
    (batch, head) pairs of workload w at n_ctx tokens, all loops, scaled to
    a full step of `batch` x heads x layers pairs: on all host threads (the
    reported value) and on one.  The oracle's encode of the sample (one
    thread) is timed too."""
    threads = host_threads(threads)
    single_pairs = min(single_pairs, n_pairs)
    n_ctx = n_ctx or w.n_ctx
    batch = batch or w.batch
    lay, kp, vp, kin, vin, qb = oracle_layer(w, n_pairs, n_ctx, w.seed + 1000)
    from oracle import rq_oracle as orc
    t0 = time.perf_counter()
    orc.encode(lay, kp, kin, 0, n_ctx)
    orc.encode(lay, vp, vin, 0, n_ctx)
    enc = (time.perf_counter() - t0) / n_pairs
    one, many = oracle_decode_timing(w, lay, kp, vp, qb, n_pairs, n_ctx, threads, single_pairs)
    pairs = batch * w.heads * w.layers
    step_many, step_one = many * pairs, one * pairs
    return {"value": batch / step_many, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_pairs} of {pairs} (batch, head) pairs x {w.n_loops} loops x {n_ctx} tokens "
                      f"decoded in {many * n_pairs:.1f} s on {threads} host threads (one (loop, batch, head) "
                      f"row per task), scaled x{pairs / n_pairs:.2f} to the full step{what}",
            "ms_per_step": step_many * 1e3, "host_cpu": cpu_model(),
            "single_thread": {"value": batch / step_one, "unit": "tokens/s", "cores": 1,
                              "ms_per_step": step_one * 1e3,
                              "sample": f"{single_pairs} pairs x {w.n_loops} loops in {one * single_pairs:.1f} s"},
            "encode_single_thread": {"s_per_pair": enc, "tokens_per_s": n_ctx / enc,
                                     "sample": f"{n_pairs} pairs x {n_ctx} tokens, K and V, "
                                               f"{w.n_loops - 1} residual loops, one thread"}}


def bf16_baseline(w, n, steps, warmup, splits_rq, trials_n=0, trial_steps=127):
    """The same decode step on a BF16 KV cache (every loop its own BF16 K, V),
    timed the same way; the comparison the pages normalise against."""
    import numpy as np
    import torch
    import decode_attention_rq_amd as rq
    import synth

    dev = "cuda"
    lay = rq.Layout(w.n_loops, w.batch, w.heads, w.d, w.g, n, w.rotate, w.bits)
    reps = []
    for r in range(2):
        d = synth.draw_layer(w, seed=w.seed + 17 * r, device=dev)
        ks = [d["k_loops"][l] for l in range(w.n_loops - 1)] + [d["k_ref"]]
        vs = [d["v_loops"][l] for l in range(w.n_loops - 1)] + [d["v_ref"]]
        reps.append((ks, vs, d["q"].contiguous()))
    splits = rq.rq_decode_splits(lay, n)
    ws = rq.workspace_for(lay, n, splits, dev)
    out = torch.empty(w.n_loops, w.batch, w.heads, w.d, device=dev)
    mask = (1 << w.n_loops) - 1

    def step(i):
        ks, vs, q = reps[i % 2]
        rq.rq_bf16_decode_attn(lay, ks, vs, q, mask, n, 1.0 / np.sqrt(w.d), out, ws, splits)

    for i in range(warmup):
        step(i)
    settled = settle(step, warmup)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = w.batch * w.heads * n * 2 * w.n_loops * w.d * 2
    trials = run_trials(step, trials_n, trial_steps)
    del reps
    torch.cuda.empty_cache()
    return {"value": round(w.batch / (ms / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4),
            "hbm_gbs": round(nbytes / (ms / 1e3) / 1e9, 1), "bytes_per_step": nbytes,
            "settle_steps": settled, "trials": trials_summary(trials, w.batch, nbytes),
            "kernel": "rq_bf16_decode_attn: the same split-K kernel over BF16 K/V, one launch per loop"}


def copy_probe():
    """A plain device copy of 1 GiB, five times: its rocprofv3 FETCH_SIZE /
    WRITE_SIZE per dispatch against the known 1 GiB gives the counter scale."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy", "bytes_read_per_copy": n, "bytes_written_per_copy": n, "copies": 5}))


def stream_probe(args):
    """The attainable HBM read rate: rq_probe_read_stream over a 4 GiB buffer
    (16x the 256 MB Infinity Cache), grid-stride, chunked and 20-plane
    patterns, default and non-temporal loads, 2 / 4 / 8 / 16 workgroups of
    256 lanes per compute unit.  One JSON line per point, then a summary
    line."""
    import torch
    import decode_attention_rq_amd as rq
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    steps = args.steps if args.steps_given else 20
    best = {}
    for pattern in (0, 1, 2):
        for nt in (0, 1):
            for per_cu in (2, 4, 8, 16):
                blocks = cus * per_cu
                sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
                ms = timed(lambda i: rq.rq_probe_read_stream(buf, nt, sink, pattern), steps, 2)
                read = nbytes
                if pattern == 2:     # whole 4 KiB segments of each of the 20 planes' chunks
                    read = 20 * 4096 * (nbytes // 20 // 16 // blocks // 256) * blocks
                gbs = read / (ms / 1e3) / 1e9
                row = {"mode": "stream", "pattern": ["grid-stride", "chunked", "planes-20"][pattern], "nontemporal": nt,
                       "workgroups_per_cu": per_cu, "ms_per_read": round(ms, 4), "gbs": round(gbs, 1),
                       "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
                print(json.dumps(row), flush=True)
                key = "nontemporal" if nt else "default"
                if gbs > best.get(key, {}).get("gbs", 0):
                    best[key] = row
    print(json.dumps({"mode": "stream", "bytes_per_read": nbytes, "best": best, "system": system_info()}), flush=True)


def sdpa_baseline(w, n, steps, warmup, ours):
    """torch's scaled_dot_product_attention (flash or memory-efficient
    backend only; the math backend is never allowed) on the BF16 baseline's
    shapes: one call per loop, q [B, H, 1, d] against that loop's BF16 K, V
    [B, H, n, d].  A sanity check that the BF16 baseline kernel is not a
    straw man.  `ours` = the baseline kernel's output on the same inputs
    (f32 [L, B, H, d]), compared with the SDPA output."""
    import numpy as np
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    import synth

    d = synth.draw_layer(w, seed=w.seed, device="cuda")
    ks = [d["k_loops"][l] for l in range(w.n_loops - 1)] + [d["k_ref"]]
    vs = [d["v_loops"][l] for l in range(w.n_loops - 1)] + [d["v_ref"]]
    q = d["q"].contiguous()
    scale = 1.0 / np.sqrt(w.d)
    res = {"kernel": "torch.nn.functional.scaled_dot_product_attention, one call per loop"}
    for name, be in (("flash", SDPBackend.FLASH_ATTENTION), ("efficient", SDPBackend.EFFICIENT_ATTENTION)):
        try:
            with sdpa_kernel([be]):
                outs = [None] * w.n_loops

                def step(i):
                    for l in range(w.n_loops):
                        outs[l] = F.scaled_dot_product_attention(q[l][:, :, None, :], ks[l], vs[l], scale=scale)
                ms = timed(step, steps, warmup)
            got = torch.stack([o[:, :, 0, :].float() for o in outs]).cpu().numpy()
            ref = ours(ks, vs, q)
            err = float((np.abs(got - ref).max(-1) / np.abs(ref).max(-1)).max())
            nbytes = w.batch * w.heads * n * 2 * w.n_loops * w.d * 2
            res[name] = {"value": round(w.batch / (ms / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4),
                         "hbm_gbs": round(nbytes / (ms / 1e3) / 1e9, 1),
                         "max_row_rel_diff_vs_bf16_baseline_kernel": err}
        except Exception as e:       # backend unavailable on this build
            res[name] = {"error": f"{type(e).__name__}: {str(e).splitlines()[0][:200]}"}
    del d, ks, vs, q
    torch.cuda.empty_cache()
    return res


def encode_bytes_per_token(w) -> int:
    """Bytes one rq_encode of a token moves per (batch, head): every loop's
    BF16 K and V read once (the reference included), and every encoded
    plane written (codes, FP16 scale and zero per group, FP16 LS
    coefficient; a quantized anchor's codes and its scale and zero)."""
    read = 2 * w.n_loops * w.d * 2
    write = 2 * sum(w.d * b // 8 + 4 * (w.d // w.g) + 2 for b in w.bits[:w.n_loops - 1])
    if w.ref_bits:
        write += 2 * (w.d * w.ref_bits // 8 + 4 * (w.d // (w.ref_group or w.g)))
    return read + write


def encode_bench(args):
    """The prefill write path alone: rq_encode of all n_ctx tokens of the
    workload's layer (every loop, K and V) from inputs already in HBM,
    after the settling work, mean over --steps calls.  Each call rewrites
    the same slots with the same bytes."""
    import torch
    import decode_attention_rq_amd as rq
    import synth
    w = synth.WORKLOADS[args.workload]
    n = w.n_ctx
    lay = rq.Layout(w.n_loops, w.batch, w.heads, w.d, w.g, n, w.rotate, w.bits, ref_bits=w.ref_bits,
                    ref_group=w.ref_group, group_loops=w.group_loops, ref_first=w.ref_first,
                    alpha_mode=w.alpha_mode, ref_chain=w.ref_chain)
    d = synth.draw_layer(w, device="cuda")
    k, v = rq.Cache(lay, "cuda", zero=False), rq.Cache(lay, "cuda", zero=False)
    if w.ref_bits:
        kin = torch.cat([d["k_loops"], d["k_ref"][None]]).contiguous()
        vin = torch.cat([d["v_loops"], d["v_ref"][None]]).contiguous()
    else:
        k.ref.copy_(d["k_ref"])
        v.ref.copy_(d["v_ref"])
        kin, vin = d["k_loops"], d["v_loops"]
    del d
    torch.cuda.empty_cache()
    steps = args.steps if args.steps_given else 10
    ms = timed(lambda i: rq.rq_encode(lay, k, v, kin, vin, 0, n), steps, 2)
    nbytes = w.batch * w.heads * n * encode_bytes_per_token(w)
    gbs = nbytes / (ms / 1e3) / 1e9
    print(json.dumps({"mode": "encode", "workload": w.name, "tokens": w.batch * w.heads * n,
                      "bits": w.bits, "ref_bits": w.ref_bits, "group": w.g, "ms_per_call": round(ms, 4),
                      "algorithmic_bytes": nbytes, "bytes_per_token": encode_bytes_per_token(w),
                      "hbm_gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                      "system": system_info()}), flush=True)


def system_info():
    """Device and software versions the numbers were taken with."""
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"device": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2**30, 1), "hip": torch.version.hip, "torch": torch.__version__}


def layout_of(w, batch, cap):
    import decode_attention_rq_amd as rq
    return rq.Layout(w.n_loops, batch, w.heads, w.d, w.g, cap, w.rotate, w.bits)


def settle(fn, start=0, settle_ms=None):
    """Run fn(start), fn(start+1), ... untimed until about settle_ms of GPU
    work is done (the clocks ramp up over the first ~10 ms of back-to-back
    work after an idle period).  The first three calls, bracketed by HIP
    events, give the per-call time that sizes the rest.  Returns the number
    of calls made."""
    import torch
    settle_ms = SETTLE_MS if settle_ms is None else settle_ms
    if settle_ms <= 0:
        return 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(3):
        fn(start + i)
    e1.record()
    torch.cuda.synchronize()
    done = e0.elapsed_time(e1)
    per = max(done / 3, 1e-3)
    more = min(5000, max(0, int((settle_ms - done) / per) + 1))
    for i in range(more):
        fn(start + 3 + i)
    torch.cuda.synchronize()
    return 3 + more


def timed(fn, steps, warmup):
    """Mean ms per call of fn(i) over `steps` calls after `warmup` calls and
    the settling work, bracketed by device synchronisation (HIP events on the
    current stream)."""
    import torch
    for i in range(warmup):
        fn(i)
    settle(fn, warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def run_trials(fn, trials, steps):
    """The pages' protocol (a warm-up, then three trials of 127 decode steps,
    averaged): `trials` back-to-back trials of `steps` calls of fn, each
    bracketed by two HIP events.  Returns ms per call of each trial."""
    import torch
    out = []
    for t in range(trials):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / steps)
    return out


def trials_summary(ms, batch, nbytes):
    """Mean and spread of the trials' step times, as tokens/s and GB/s."""
    import numpy as np
    if not ms:
        return None
    a = np.array(ms)
    return {"n": len(ms), "ms_per_step": [round(float(x), 4) for x in ms],
            "ms_mean": round(float(a.mean()), 4), "ms_spread": round(float(a.max() - a.min()), 4),
            "tokens_per_s_mean": round(float(np.mean(batch / (a / 1e3))), 1),
            "hbm_gbs_mean": round(float(np.mean(nbytes / (a / 1e3) / 1e9)), 1),
            "frac_of_peak_mean": round(float(np.mean(nbytes / (a / 1e3) / 1e9)) / HBM_PEAK_GBS, 4)}


def timed_graph(fn, steps, warmup, settle_ms=None):
    """Mean ms per step of fn, captured once into a HIP graph (torch's
    CUDAGraph on the current stream) and replayed `steps` times after
    `warmup` replays, and after as many more as make ~settle_ms of work (the
    clocks settle only after a stretch of back-to-back work, see parse;
    short steps would otherwise be timed on the ramp); HIP events bracket the
    replays."""
    settle_ms = SETTLE_MS if settle_ms is None else settle_ms
    import torch
    fn(0)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(warmup):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    per = max(e0.elapsed_time(e1) / max(warmup, 1), 1e-3)
    for i in range(min(5000, int(settle_ms / per))):
        g.replay()
    torch.cuda.synchronize()
    e0.record()
    for i in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / steps


def append_bench(args, w):
    """Mixed-precision 8k workload: rq_encode prefill of 8192 tokens (mean of
    three timed calls after three untimed ones), then `steps` append steps, each
    rq_encode of one new token per (batch, head, loop) plus rq_decode_attn
    over the n+1 tokens.  The
    reference slots (the final loop's own KV write) are in place beforehand."""
    import numpy as np
    import torch
    import decode_attention_rq_amd as rq
    import synth

    dev = "cuda"
    n0, steps = w.n_ctx, w.steps
    # capacity for the prefill and the appends, rounded up to a multiple of
    # 256 tokens (per-(batch, head) plane strides that are not slow the
    # decode by 5-10 %; see include/rq.h)
    cap = -(-(n0 + steps) // 256) * 256
    lay = layout_of(w, w.batch, cap)
    data = synth.draw_layer(w, n=cap, device=dev)
    k, v = rq.Cache(lay, dev), rq.Cache(lay, dev)
    k.ref.copy_(data["k_ref"])
    v.ref.copy_(data["v_ref"])
    kin, vin, q = data["k_loops"], data["v_loops"], data["q"].contiguous()
    pre_k, pre_v = kin[:, :, :, :n0].contiguous(), vin[:, :, :, :n0].contiguous()
    step_in = [(kin[:, :, :, t:t + 1].contiguous(), vin[:, :, :, t:t + 1].contiguous()) for t in range(n0, n0 + steps)]
    del data, kin, vin
    torch.cuda.empty_cache()
    # prefill: untimed encodes of all n0 tokens until the clocks have
    # settled, then the mean of three timed ones (each writes the same slots
    # with the same values)
    settle(lambda i: rq.rq_encode(lay, k, v, pre_k, pre_v, 0, n0))
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        rq.rq_encode(lay, k, v, pre_k, pre_v, 0, n0)
    e1.record()
    torch.cuda.synchronize()
    pre_ms = e0.elapsed_time(e1) / 3
    res_bits = [b for b in w.bits]
    enc_bytes_tok = 2 * (w.n_loops * w.d * 2) + 2 * sum(w.d * b // 8 + 4 * (w.d // w.g) + 2 for b in res_bits)
    pre_bytes = w.batch * w.heads * n0 * enc_bytes_tok
    del pre_k, pre_v
    mask = (1 << w.n_loops) - 1
    out = torch.empty(w.n_loops, w.batch, w.heads, w.d, device=dev)
    ws = rq.workspace_for(lay, cap, rq.rq_decode_splits(lay, cap), dev)
    scale = 1.0 / np.sqrt(w.d)
    def append_step(s_):
        t = n0 + s_
        rq.rq_encode(lay, k, v, step_in[s_][0], step_in[s_][1], t, 1)
        return t

    # The step rate: two events around the steps (an event marker between two
    # kernels idles the GPU for ~5 us).
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for s_ in range(steps):
        t = append_step(s_)
        rq.rq_decode_attn(lay, k, v, q, mask, t + 1, scale, out, ws, rq.rq_decode_splits(lay, t + 1))
    e1.record()
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / steps
    # The same steps again (each append rewrites its slot with the same bytes)
    # with events between the phases: the append and decode durations.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for s_ in range(steps):
        ev[s_][0].record()
        t = append_step(s_)
        ev[s_][1].record()
        rq.rq_decode_attn(lay, k, v, q, mask, t + 1, scale, out, ws, rq.rq_decode_splits(lay, t + 1))
        ev[s_][2].record()
    torch.cuda.synchronize()
    enc_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])
    per_tok = layout_bytes_per_token(w.n_loops, w.bits, w.g, w.d)
    dec_bytes = w.batch * w.heads * (n0 + steps / 2) * per_tok
    res = {"metric": "decode tokens/s with one-token append per step, mixed INT4/INT2 residual KV, 8k ctx",
           "value": round(w.batch / (step_ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": steps, "warmup": 0, "ms_per_step": round(step_ms, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"{w.name}: batch {w.batch}, {w.heads} heads, head_dim {w.d}, bits {w.bits} "
                                  f"+ BF16 reference, g={w.g}, prefill {n0} tokens then {steps} append steps"},
           "decode_ms_mean": round(float(dec_ms.mean()), 4),
           "decode_hbm_gbs": round(dec_bytes / (dec_ms.mean() / 1e3) / 1e9, 1),
           "append_encode_us_mean": round(float(enc_ms.mean()) * 1e3, 2),
           "prefill_encode": {"ms": round(pre_ms, 3), "tokens": w.batch * w.heads * n0,
                              "algorithmic_bytes": pre_bytes,
                              "hbm_gbs": round(pre_bytes / (pre_ms / 1e3) / 1e9, 1),
                              "frac_of_peak": round(pre_bytes / (pre_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}}
    del k, v, step_in
    torch.cuda.empty_cache()
    if not args.no_bf16_baseline:
        # BF16 decode over the same growing context (no encode needed)
        d2 = synth.draw_layer(w, n=cap, device=dev)
        ks = [d2["k_loops"][l] for l in range(w.n_loops - 1)] + [d2["k_ref"]]
        vs = [d2["v_loops"][l] for l in range(w.n_loops - 1)] + [d2["v_ref"]]
        lay_b = layout_of(w, w.batch, cap)
        # step i attends n0 + (i mod steps) + 1 tokens (the settling calls
        # cycle through the same context lengths)
        ms = timed(lambda i: rq.rq_bf16_decode_attn(lay_b, ks, vs, d2["q"], mask, n0 + i % steps + 1, scale, out,
                                                    ws, rq.rq_decode_splits(lay_b, n0 + i % steps + 1)), steps, 3)
        res["bf16_baseline"] = {"value": round(w.batch / (ms / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4)}
        res["speedup_vs_bf16"] = round(res["value"] / res["bf16_baseline"]["value"], 3)
    if not args.no_cpu_baseline:
        # the oracle on 8 (batch, head) pairs: its decode at 8k (threads) plus
        # its encode of one token per pair (one append step), scaled to B x H
        cb = cpu_baseline(w, 8, args.cpu_threads, 4,
                          what="; an append step adds the oracle's one-token encode of every pair, one thread")
        pairs = w.batch * w.heads
        enc_step_s = pairs * cb["encode_single_thread"]["s_per_pair"] / w.n_ctx
        step_s = cb["ms_per_step"] / 1e3 + enc_step_s
        cb["value"] = w.batch / step_s
        cb["ms_per_step"] = step_s * 1e3
        cb["prefill_encode_s"] = pairs * cb["encode_single_thread"]["s_per_pair"]
        res["cpu_baseline"] = cb
    return res


def layers_bench(args, w):
    """32k context over 24 layers: one step = 24 sequential rq_decode_attn
    calls, each layer with its own caches and queries."""
    import numpy as np
    import torch
    import decode_attention_rq_amd as rq
    import synth

    dev, n = "cuda", w.n_ctx
    lay = layout_of(w, w.batch, n)
    layers = []
    for li in range(w.layers):
        d = synth.draw_layer(w, seed=w.seed * 100 + li, device=dev)
        k, v = rq.Cache(lay, dev, zero=False), rq.Cache(lay, dev, zero=False)
        k.ref.copy_(d["k_ref"])
        v.ref.copy_(d["v_ref"])
        rq.rq_encode(lay, k, v, d["k_loops"], d["v_loops"], 0, n)
        layers.append((k, v, d["q"].contiguous()))
        del d
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    mask = (1 << w.n_loops) - 1
    splits = rq.rq_decode_splits(lay, n)
    ws = rq.workspace_for(lay, n, splits, dev)
    out = torch.empty(w.n_loops, w.batch, w.heads, w.d, device=dev)
    scale = 1.0 / np.sqrt(w.d)

    def step(i):
        for k, v, q in layers:
            rq.rq_decode_attn(lay, k, v, q, mask, n, scale, out, ws, splits)

    steps = args.steps if args.steps_given else 20
    ms = timed(step, steps, 3)
    nbytes = w.layers * w.batch * w.heads * n * layout_bytes_per_token(w.n_loops, w.bits, w.g, w.d)
    res = {"metric": "decode tokens/s + achieved HBM GB/s, INT2 residual KV, 32k ctx, 24 layers",
           "value": round(w.batch / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
           "warmup": 3, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"{w.name}: {w.layers} layers x (batch {w.batch}, {w.heads} heads, head_dim {w.d}, "
                                  f"{w.n_loops} loops, bits {w.bits} + BF16 reference), {n}-token context",
                      "splits": splits},
           "hbm_gbs": round(nbytes / (ms / 1e3) / 1e9, 1),
           "frac_of_peak": round(nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4), "bytes_per_step": nbytes}
    del layers
    torch.cuda.empty_cache()
    if not args.no_bf16_baseline:
        bl = []
        for li in range(w.layers):
            d = synth.draw_layer(w, seed=w.seed * 100 + li, device=dev)
            ks = [d["k_loops"][l].clone() for l in range(w.n_loops - 1)] + [d["k_ref"]]
            vs = [d["v_loops"][l].clone() for l in range(w.n_loops - 1)] + [d["v_ref"]]
            bl.append((ks, vs, d["q"].contiguous()))
            del d
            torch.cuda.empty_cache()

        def bstep(i):
            for ks, vs, q in bl:
                rq.rq_bf16_decode_attn(lay, ks, vs, q, mask, n, scale, out, ws, splits)

        bms = timed(bstep, max(3, steps // 2), 2)
        bbytes = w.layers * w.batch * w.heads * n * 2 * w.n_loops * w.d * 2
        res["bf16_baseline"] = {"value": round(w.batch / (bms / 1e3), 1), "unit": "tokens/s",
                                "ms_per_step": round(bms, 4), "hbm_gbs": round(bbytes / (bms / 1e3) / 1e9, 1)}
        res["speedup_vs_bf16"] = round(res["value"] / res["bf16_baseline"]["value"], 3)
        del bl
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, w.heads, args.cpu_threads, 4, n_ctx=n,
                                           what=" (one layer x one batch element sampled, extrapolated "
                                                "linearly over layers and batch)")
    return res


def peak_batch_bench(args, w, budget=250e9):
    """8k context, 24 layers: the largest batch whose KV cache fits the budget,
    for this layout and for BF16 KV, and decode tokens/s over a batch sweep up
    to each maximum (batch-prefix views of one allocation)."""
    import numpy as np
    import torch
    import decode_attention_rq_amd as rq
    import synth

    dev, n, L = "cuda", w.n_ctx, w.layers
    rq_per_b = L * w.heads * n * layout_bytes_per_token(w.n_loops, w.bits, w.g, w.d)
    bf_per_b = L * w.heads * n * 2 * w.n_loops * w.d * 2
    bmax_rq, bmax_bf = int(budget // rq_per_b), int(budget // bf_per_b)
    mask = (1 << w.n_loops) - 1
    scale = 1.0 / np.sqrt(w.d)
    steps = args.steps if args.steps_given else 10

    def sweep(bmax):
        bs = [b for b in (1, 2, 4, 8, 16, 32, 64, 128) if b < bmax] + [bmax]
        return bs

    # ---- ResidualQuant caches at the maximum batch, encoded chunk by chunk
    lay_max = layout_of(w, bmax_rq, n)
    layers = [(rq.Cache(lay_max, dev, zero=False), rq.Cache(lay_max, dev, zero=False)) for _ in range(L)]
    chunk = 8
    for b0 in range(0, bmax_rq, chunk):
        b1 = min(bmax_rq, b0 + chunk)
        d = synth.draw_layer(w, seed=w.seed * 1000 + b0, batch=b1 - b0, device=dev)
        lay_c = layout_of(w, b1 - b0, n)
        for k, v in layers:
            kc, vc = k.batch_view(b0, b1, lay_c), v.batch_view(b0, b1, lay_c)
            kc.ref.copy_(d["k_ref"])
            vc.ref.copy_(d["v_ref"])
            rq.rq_encode(lay_c, kc, vc, d["k_loops"], d["v_loops"], 0, n)
        del d
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    qall = synth.draw_queries(synth.generator(w.seed, dev), w.n_loops, bmax_rq, w.heads, w.d)
    rq_rows = []
    for B in sweep(bmax_rq):
        lay_b = layout_of(w, B, n)
        views = [(k.batch_view(0, B, lay_b), v.batch_view(0, B, lay_b)) for k, v in layers]
        q = qall[:, :B].contiguous()
        splits = rq.rq_decode_splits(lay_b, n)
        ws = rq.workspace_for(lay_b, n, splits, dev)
        out = torch.empty(w.n_loops, B, w.heads, w.d, device=dev)

        def step(i):
            for kv_, vv_ in views:
                rq.rq_decode_attn(lay_b, kv_, vv_, q, mask, n, scale, out, ws, splits)

        ms = timed(step, steps, 2)
        rq_rows.append({"batch": B, "ms_per_step": round(ms, 3), "tokens_per_s": round(B / (ms / 1e3), 1),
                        "hbm_gbs": round(B * rq_per_b / (ms / 1e3) / 1e9, 1)})
    del layers, views
    torch.cuda.empty_cache()
    # ---- BF16 caches at their maximum batch (values do not affect timing;
    # the memory is left as allocated)
    bf_rows = []
    if not args.no_bf16_baseline:
        lay_bf = layout_of(w, bmax_bf, n)
        bl = [([torch.empty(bmax_bf, w.heads, n, w.d, dtype=torch.bfloat16, device=dev) for _ in range(w.n_loops)],
               [torch.empty(bmax_bf, w.heads, n, w.d, dtype=torch.bfloat16, device=dev) for _ in range(w.n_loops)])
              for _ in range(L)]
        for B in sweep(bmax_bf):
            lay_b = layout_of(w, B, n)
            q = qall[:, :B].contiguous()
            splits = rq.rq_decode_splits(lay_b, n)
            ws = rq.workspace_for(lay_b, n, splits, dev)
            out = torch.empty(w.n_loops, B, w.heads, w.d, device=dev)
            views = [([t[:B] for t in ks], [t[:B] for t in vs]) for ks, vs in bl]

            def bstep(i):
                for ks, vs in views:
                    rq.rq_bf16_decode_attn(lay_b, ks, vs, q, mask, n, scale, out, ws, splits)

            ms = timed(bstep, steps, 2)
            bf_rows.append({"batch": B, "ms_per_step": round(ms, 3), "tokens_per_s": round(B / (ms / 1e3), 1),
                            "hbm_gbs": round(B * bf_per_b / (ms / 1e3) / 1e9, 1)})
        del bl, views
        torch.cuda.empty_cache()
    peak_rq = max(r["tokens_per_s"] for r in rq_rows)
    res = {"metric": "peak decode tokens/s and largest feasible batch at 8k ctx, 24 layers, 250 GB KV budget",
           "value": peak_rq, "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": 2,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"{w.name}: {L} layers x ({w.heads} heads, head_dim {w.d}, {w.n_loops} loops, "
                                  f"bits {w.bits} + BF16 reference), {n}-token context, KV budget {budget / 1e9:.0f} GB"},
           "max_batch": {"residualquant": bmax_rq, "bf16": bmax_bf, "gain": round(bmax_rq / bmax_bf, 3)},
           "max_pow2_batch": {"residualquant": 2 ** int(np.log2(bmax_rq)), "bf16": 2 ** int(np.log2(bmax_bf))},
           "kv_bytes_per_batch_entry": {"residualquant": rq_per_b, "bf16": bf_per_b},
           "sweep_residualquant": rq_rows}
    if bf_rows:
        peak_bf = max(r["tokens_per_s"] for r in bf_rows)
        res["sweep_bf16"] = bf_rows
        res["peak_gain_vs_bf16"] = round(peak_rq / peak_bf, 3)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, w.heads, args.cpu_threads, 4, batch=bmax_rq,
                                           what=f" at batch {bmax_rq} (one layer x one batch element "
                                                f"sampled, extrapolated linearly over layers and batch)")
    return res


def anchor_bench(args, w):
    """Per-loop decode with a quantized anchor (the pages' [2,2,2,4]: INT4
    anchor at g=32, INT2 residuals at g=16) and the most recent tokens in
    BF16.  A looped model runs its loops in sequence, so one decode step of a
    layer is one attention call per loop, in loop order, each over the cached
    tokens plus the tail: rq_decode_attn_tail with one loop in the mask.
    Compared with BF16 per-loop decode over the same tokens (each loop's own
    BF16 K and V), and with the fused call over all four loops."""
    import numpy as np
    import torch
    import decode_attention_rq_amd as rq
    import synth

    dev, n, T, L = "cuda", w.n_ctx, w.extra["tail"], w.n_loops
    B, H, d = w.batch, w.heads, w.d
    lay = rq.Layout(L, B, H, d, w.g, n, w.rotate, w.bits, ref_bits=w.ref_bits, ref_group=w.ref_group,
                    ref_chain=w.ref_chain)
    scale = 1.0 / np.sqrt(d)
    reps = []
    for r in range(args.replicas):
        dl = synth.draw_layer(w, seed=w.seed + 17 * r, device=dev)
        k, v = rq.Cache(lay, dev, zero=False), rq.Cache(lay, dev, zero=False)
        rq.rq_encode(lay, k, v, torch.cat([dl["k_loops"], dl["k_ref"][None]]),
                     torch.cat([dl["v_loops"], dl["v_ref"][None]]), 0, n)
        tl = synth.draw_tail(w, seed=w.seed + 17 * r + 1, n=T, device=dev)
        tail = rq.Tail([tl["k"][l].contiguous() for l in range(L)], [tl["v"][l].contiguous() for l in range(L)], T)
        reps.append((k, v, tail, dl["q"].contiguous()))
        del dl, tl
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    splits = args.splits or rq.rq_decode_splits(lay, n)
    ws = rq.workspace_for(lay, n, splits, dev)
    out = torch.empty(L, B, H, d, device=dev)

    def step(i):
        k, v, tail, q = reps[i % len(reps)]
        for l in range(L):
            rq.rq_decode_attn_tail(lay, k, v, tail, q, 1 << l, n, scale, out, ws, splits)

    def call(i, l):
        k, v, tail, q = reps[i % len(reps)]
        rq.rq_decode_attn_tail(lay, k, v, tail, q, 1 << l, n, scale, out, ws, splits)

    steps = args.steps
    for i in range(args.warmup):
        step(i)
    settled = settle(step, args.warmup)
    # The step rate: two events around the steps (an event marker between two
    # kernels idles the GPU for ~5 us, so the calls are not timed one by one
    # here).
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    span_ms = e0.elapsed_time(e1)
    ms = span_ms / steps
    # The calls of each loop on their own, back to back (same events): the
    # mean duration of a residual loop's call, the dominant kernel, and of
    # the anchor loop's call.
    call_ms = np.zeros((1, L))
    for l in range(L):
        settle(lambda i: call(i, l), settle_ms=SETTLE_MS / 4)
        e0.record()
        for i in range(steps):
            call(i, l)
        e1.record()
        torch.cuda.synchronize()
        call_ms[0, l] = e0.elapsed_time(e1) / steps
    tail_bytes = B * H * T * 2 * d * 2
    anchor_tok = 2 * (d * w.ref_bits // 8 + 4 * (d // w.ref_group))
    res_tok = 2 * (d * w.bits[0] // 8 + 4 * (d // w.g) + 2)
    # residual planes one loop's call reads: its own; with chained references
    # also every link between it and the anchor (loop L-1 - l of them)
    links = [(L - 1 - l) if w.ref_chain else 1 for l in range(L - 1)] + [0]
    call_bytes = [B * H * n * (anchor_tok + links[l] * res_tok) + tail_bytes + B * H * d * 6 for l in range(L)]
    step_bytes = sum(call_bytes)
    res_call = sum(call_bytes[:L - 1]) / (L - 1)
    res_us = float(call_ms[:, :L - 1].mean()) * 1e3
    roof = {"bound": "hbm", "achieved": round(res_call / (res_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(res_call / (res_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "a residual loop's call (mean over the three): decode_kernel against the INT4 anchor"
                      + (" along the reference chain" if w.ref_chain else "")
                      + " and the BF16 tail (with two splits over these 256 batch*heads the call runs as one"
                        " workgroup per (b,h) over all tokens and the tail; with more, each split takes a share"
                        " of the tail and decode_merge_kernel merges the split records)",
            "algorithmic_bytes_per_launch": res_call, "launch_us_mean": round(res_us, 2),
            "anchor_loop_call_us_mean": round(float(call_ms[:, L - 1].mean()) * 1e3, 2)}
    res = {"metric": "per-loop decode tokens/s, [2,2,2,4] INT4 anchor + INT2 residuals g=16, 8k ctx + 64 BF16 tail"
                     + (", Next-loop chained references" if w.ref_chain else ""),
           "value": round(B / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"{w.name}: 1 layer, batch {B}, {H} heads, head_dim {d}, {L} loops "
                                  f"(INT{w.ref_bits} anchor g={w.ref_group}, residual bits {w.bits} g={w.g}), "
                                  f"{n} cached tokens + {T} BF16 tail tokens, one call per loop",
                      "splits": splits, "replicas": args.replicas},
           "bytes_per_step": step_bytes, "hbm_gbs": round(step_bytes / (ms / 1e3) / 1e9, 1),
           "frac_of_peak": round(step_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4), "roofline": roof,
           "settle": {"steps": settled, "target_ms": SETTLE_MS}}
    # all four loops in one call (when every loop's query is known at once)
    def fstep(i):
        k, v, tail, q = reps[i % len(reps)]
        rq.rq_decode_attn_tail(lay, k, v, tail, q, (1 << L) - 1, n, scale, out, ws, splits)
    fms = timed(fstep, steps, 3)
    fbytes = B * H * n * layout_bytes_per_token(L, w.bits, w.g, d, w.ref_bits, w.ref_group) + L * tail_bytes
    res["fused_all_loops"] = {"ms_per_step": round(fms, 4), "tokens_per_s": round(B / (fms / 1e3), 1),
                              "hbm_gbs": round(fbytes / (fms / 1e3) / 1e9, 1), "bytes_per_step": fbytes}
    del reps
    torch.cuda.empty_cache()
    if not args.no_bf16_baseline:
        nb = n + T
        blay = layout_of(w, B, nb)
        dl = synth.draw_layer(w, seed=w.seed + 999, n=nb, device=dev)
        ks = [dl["k_loops"][l].clone() for l in range(L - 1)] + [dl["k_ref"]]
        vs = [dl["v_loops"][l].clone() for l in range(L - 1)] + [dl["v_ref"]]
        q = dl["q"].contiguous()
        del dl
        torch.cuda.empty_cache()
        bsplits = rq.rq_decode_splits(blay, nb)
        bws = rq.workspace_for(blay, nb, bsplits, dev)

        def bstep(i):
            for l in range(L):
                rq.rq_bf16_decode_attn(blay, ks, vs, q, 1 << l, nb, scale, out, bws, bsplits)
        bms = timed(bstep, steps, 3)
        bbytes = L * B * H * nb * 2 * d * 2
        res["bf16_baseline"] = {"value": round(B / (bms / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(bms, 4),
                                "hbm_gbs": round(bbytes / (bms / 1e3) / 1e9, 1), "bytes_per_step": bbytes,
                                "kernel": "rq_bf16_decode_attn, one call per loop over its own BF16 K/V"}
        res["speedup_vs_bf16"] = round(bms / ms, 3)
        res["kv_bytes_ratio_vs_bf16"] = round(2 * L * d * 2 / layout_bytes_per_token(
            L, w.bits, w.g, d, w.ref_bits, w.ref_group), 3)
    return res


def grid_bench(args, w, budget=250e9):
    """The pages' decode-throughput grid: for each context length, the largest
    batch whose KV cache (all layers, cache plus BF16 tail) fits the budget,
    and per-loop decode tokens/s over power-of-two batches up to it (plus the
    maximum), for this layout with a quantized anchor and for BF16 KV.  One
    step = every layer's four per-loop attention calls.  Batch-prefix views of
    one allocation per context; every layer has its own planes (encoded from
    the same draws) so nothing is served from cache."""
    import numpy as np
    import torch
    import decode_attention_rq_amd as rq
    import synth

    dev, L, H, d, T, NL = "cuda", w.n_loops, w.heads, w.d, w.extra["tail"], w.layers
    scale = 1.0 / np.sqrt(d)
    steps = args.steps if args.steps_given else 8
    per_tok_rq = layout_bytes_per_token(L, w.bits, w.g, d, w.ref_bits, w.ref_group)
    rows = []
    contexts = [int(x) for x in args.contexts.split(",")] if args.contexts else w.extra["contexts"]
    only = [int(x) for x in args.batches.split(",")] if args.batches else None
    for n in contexts:
        rq_per_b = NL * H * (n * per_tok_rq + T * L * 2 * d * 2)
        bf_per_b = NL * H * (n + T) * L * 2 * d * 2
        fit_rq, fit_bf = int(budget // rq_per_b), int(budget // bf_per_b)
        bmax_rq, bmax_bf = fit_rq, fit_bf
        if only:           # allocate and run only the batches asked for
            bmax_rq, bmax_bf = min(bmax_rq, max(only)), min(bmax_bf, max(only))
            sweep = lambda bm: [b for b in only if b <= bm]
        else:
            sweep = lambda bm: [b for b in (1, 2, 4, 8, 16, 32, 64, 128, 256) if b < bm] + [bm]
        lay_max = rq.Layout(L, bmax_rq, H, d, w.g, n, w.rotate, w.bits, ref_bits=w.ref_bits,
                            ref_group=w.ref_group)
        layers = [(rq.Cache(lay_max, dev, zero=False), rq.Cache(lay_max, dev, zero=False)) for _ in range(NL)]
        chunk = max(1, min(bmax_rq, (8 * 8192) // n))
        for b0 in range(0, bmax_rq, chunk):
            b1 = min(bmax_rq, b0 + chunk)
            dl = synth.draw_layer(w, seed=w.seed * 1000 + b0, batch=b1 - b0, n=n, device=dev)
            kin = torch.cat([dl["k_loops"], dl["k_ref"][None]])
            vin = torch.cat([dl["v_loops"], dl["v_ref"][None]])
            del dl
            lay_c = rq.Layout(L, b1 - b0, H, d, w.g, n, w.rotate, w.bits, ref_bits=w.ref_bits,
                              ref_group=w.ref_group)
            for k, v in layers:
                rq.rq_encode(lay_c, k.batch_view(b0, b1, lay_c), v.batch_view(b0, b1, lay_c), kin, vin, 0, n)
            del kin, vin
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        tl = synth.draw_tail(w, seed=w.seed + n, batch=bmax_rq, n=T, device=dev)
        tails = [(tl["k"].clone(), tl["v"].clone()) for _ in range(NL)]
        del tl
        qall = synth.draw_queries(synth.generator(w.seed, dev), L, bmax_rq, H, d)
        rq_rows = []
        for B in sweep(bmax_rq):
            lay_b = rq.Layout(L, B, H, d, w.g, n, w.rotate, w.bits, ref_bits=w.ref_bits, ref_group=w.ref_group)
            views = [(k.batch_view(0, B, lay_b), v.batch_view(0, B, lay_b),
                      rq.Tail([tk[l, :B] for l in range(L)], [tv[l, :B] for l in range(L)], T))
                     for (k, v), (tk, tv) in zip(layers, tails)]
            q = qall[:, :B].contiguous()
            splits = rq.rq_decode_splits(lay_b, n)
            ws = rq.workspace_for(lay_b, n, splits, dev)
            out = torch.empty(L, B, H, d, device=dev)

            def step(i):
                for kv_, vv_, tv_ in views:
                    for l in range(L):
                        rq.rq_decode_attn_tail(lay_b, kv_, vv_, tv_, q, 1 << l, n, scale, out, ws, splits)
            ms = (timed_graph if args.graphs else timed)(step, steps, 2)
            rq_rows.append({"batch": B, "ms_per_step": round(ms, 3), "tokens_per_s": round(B / (ms / 1e3), 1)})
        del layers, tails, views
        torch.cuda.empty_cache()
        bf_rows = []
        if not args.no_bf16_baseline:
            nb = n + T
            bl = [([torch.empty(bmax_bf, H, nb, d, dtype=torch.bfloat16, device=dev) for _ in range(L)],
                   [torch.empty(bmax_bf, H, nb, d, dtype=torch.bfloat16, device=dev) for _ in range(L)])
                  for _ in range(NL)]
            for ks, vs in bl:          # finite values (timing does not depend on them)
                for t in ks + vs:
                    t.fill_(0.01)
            for B in sweep(bmax_bf):
                blay = rq.Layout(L, B, H, d, w.g, nb, w.rotate, w.bits)
                q = qall[:, :B].contiguous() if B <= bmax_rq else torch.zeros(L, B, H, d, dtype=torch.bfloat16, device=dev)
                splits = rq.rq_decode_splits(blay, nb)
                ws = rq.workspace_for(blay, nb, splits, dev)
                out = torch.empty(L, B, H, d, device=dev)
                views = [([t[:B] for t in ks], [t[:B] for t in vs]) for ks, vs in bl]

                def bstep(i):
                    for ks, vs in views:
                        for l in range(L):
                            rq.rq_bf16_decode_attn(blay, ks, vs, q, 1 << l, nb, scale, out, ws, splits)
                ms = (timed_graph if args.graphs else timed)(bstep, steps, 2)
                bf_rows.append({"batch": B, "ms_per_step": round(ms, 3), "tokens_per_s": round(B / (ms / 1e3), 1)})
            del bl, views
            torch.cuda.empty_cache()
        row = {"n_ctx": n, "max_batch": {"residualquant": fit_rq, "bf16": fit_bf},
               "max_pow2_batch": {"residualquant": 2 ** int(np.log2(fit_rq)), "bf16": 2 ** int(np.log2(fit_bf))},
               "residualquant": rq_rows}
        if bf_rows:
            pr, pb = max(r["tokens_per_s"] for r in rq_rows), max(r["tokens_per_s"] for r in bf_rows)
            same = {r["batch"]: r["tokens_per_s"] for r in bf_rows}
            row.update(bf16=bf_rows, peak_gain=round(pr / pb, 3),
                       fixed_batch_gain={str(r["batch"]): round(r["tokens_per_s"] / same[r["batch"]], 3)
                                         for r in rq_rows if r["batch"] in same})
        rows.append(row)
        print(json.dumps({"progress": row}), file=sys.stderr, flush=True)
    peak8k = [r for r in rows if r["n_ctx"] == 8192]
    value = max(x["tokens_per_s"] for x in (peak8k or rows)[0]["residualquant"])
    return {"metric": f"per-loop decode tokens/s across batch and context, [2,2,2,4] INT4 anchor g={w.ref_group}, "
                      f"INT2 residuals g={w.g}, 24 layers, 250 GB KV budget (value: peak at 8k)",
            "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": 2,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic",
            "config": {"workload": f"{w.name}: {NL} layers x ({H} heads, head_dim {d}, {L} loops, INT{w.ref_bits} "
                                   f"anchor g={w.ref_group}, residual bits {w.bits} g={w.g}, {T} BF16 tail tokens), "
                                   f"contexts {contexts}"
                                   + (f", batches {only} only" if only else ""),
                       "timing": "HIP graph replay" if args.graphs else "eager launches"},
            "grid": rows}


def split_sweep():
    """Time every candidate token-split count against rq_decode_splits' choice,
    interleaved (median of 4 rounds), for a fused call over all four loops (3
    INT2 g=32 residuals + BF16 reference) and for per-loop calls over the
    anchored [2,2,2,4] layout (INT4 anchor g=32, INT2 g=16): contexts x
    batches, 16 heads, head_dim 128.  One JSON line per point on stdout."""
    import numpy as np
    import torch
    import decode_attention_rq_amd as rq
    import synth
    for kind, base, points in (
            ("fused", synth.WORKLOADS["int2-8k"], [(n, B) for n in (2048, 8192, 32768)
                                                   for B in (1, 2, 4, 8, 16, 24, 32, 48, 64)]),
            ("per-loop", synth.WORKLOADS["anchor-8k-perloop"], [(n, B) for n in (2048, 8192)
                                                                for B in (1, 2, 4, 8, 16, 32, 64, 128)])):
        for n, B in points:
            if B * n > 64 * 8192:
                continue
            w = synth.Workload("sweep", n_loops=4, batch=B, heads=16, d=128, g=base.g, n_ctx=n, bits=[2, 2, 2],
                               c=base.c, sigma=base.sigma, rotate=1, seed=3, ref_bits=base.ref_bits,
                               ref_group=base.ref_group)
            lay = rq.Layout(4, B, 16, 128, w.g, n, 1, [2, 2, 2], ref_bits=w.ref_bits, ref_group=w.ref_group)
            d = synth.draw_layer(w, batch=B, n=n, device="cuda")
            k, v = rq.Cache(lay), rq.Cache(lay)
            if k.ref is not None:
                k.ref.copy_(d["k_ref"])
                v.ref.copy_(d["v_ref"])
                kin, vin = d["k_loops"], d["v_loops"]
            else:
                kin = torch.cat([d["k_loops"], d["k_ref"].unsqueeze(0)]).contiguous()
                vin = torch.cat([d["v_loops"], d["v_ref"].unsqueeze(0)]).contiguous()
            rq.rq_encode(lay, k, v, kin, vin, 0, n)
            q = d["q"].contiguous()
            del d, kin, vin
            auto = rq.rq_decode_splits(lay, n)
            cands = [S for S in (1, 2, 4, 8, 16, 32) if n // S >= 256]
            wss = {S: rq.workspace_for(lay, n, S) for S in cands}
            out = torch.empty(4, B, 16, 128, device="cuda")
            masks = [15] if kind == "fused" else [1, 2, 4, 8]
            scale = 1.0 / np.sqrt(128)

            def call(S):
                for m in masks:
                    rq.rq_decode_attn(lay, k, v, q, m, n, scale, out, wss[S], S)
            iters = max(3, min(20, int(2e5 // (B * n // 64 + 1000))))
            res = {S: [] for S in cands}
            for _ in range(4):
                for S in cands:
                    call(S)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(iters):
                        call(S)
                    e1.record()
                    torch.cuda.synchronize()
                    res[S].append(e0.elapsed_time(e1) / iters * 1e3)
            med = {S: round(float(np.median(t)), 1) for S, t in res.items()}
            best = min(med, key=med.get)
            print(json.dumps({"mode": "split-sweep", "pass": kind, "n_ctx": n, "batch": B, "auto_splits": auto,
                              "auto_us": med.get(auto), "best_splits": best, "best_us": med[best],
                              "us_per_step_by_splits": med}), flush=True)
            del k, v, wss
            torch.cuda.empty_cache()


def main():
    args = parse()
    if args.mode == "copy":
        copy_probe()
        return
    if args.mode == "stream":
        stream_probe(args)
        return
    if args.mode == "encode":
        encode_bench(args)
        return
    if args.mode == "split-sweep":
        split_sweep()
        return
    if args.gpus != 1:
        print("bench.py: runs on one GPU; --gpus must be 1 (the per-(batch, head) "
              "work shards across GPUs without exchange, but no multi-GPU path is built)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import decode_attention_rq_amd as rq
    import synth

    w = synth.WORKLOADS[args.workload]
    if args.workload == "mixed-8k-append":
        print(json.dumps(append_bench(args, w)), flush=True)
        return
    if args.workload == "int2-32k-24l":
        print(json.dumps(layers_bench(args, w)), flush=True)
        return
    if args.workload == "peak-batch-8k":
        print(json.dumps(peak_batch_bench(args, w)), flush=True)
        return
    if args.workload in ("anchor-8k-perloop", "chain-8k-perloop"):
        print(json.dumps(anchor_bench(args, w)), flush=True)
        return
    if args.workload.startswith("grid-"):
        print(json.dumps(grid_bench(args, w)), flush=True)
        return
    dev = "cuda"
    lay = rq.Layout(w.n_loops, w.batch, w.heads, w.d, w.g, w.n_ctx, w.rotate, w.bits)
    n = w.n_ctx
    mask = (1 << w.n_loops) - 1
    scale = 1.0 / np.sqrt(w.d)

    # ---- set-up: encode the replicas (not timed) ---------------------------
    reps = []
    for r in range(args.replicas):
        data = synth.draw_layer(w, seed=w.seed + 17 * r, device=dev)
        k, v = rq.Cache(lay, dev), rq.Cache(lay, dev)
        k.ref.copy_(data["k_ref"])
        v.ref.copy_(data["v_ref"])
        rq.rq_encode(lay, k, v, data["k_loops"], data["v_loops"], 0, n)
        reps.append((k, v, data["q"].contiguous()))
        del data
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    splits = args.splits or rq.rq_decode_splits(lay, n)
    ws = rq.workspace_for(lay, n, splits, dev)
    out = torch.empty(w.n_loops, w.batch, w.heads, w.d, device=dev)

    def step(i):
        k, v, q = reps[i % len(reps)]
        rq.rq_decode_attn(lay, k, v, q, mask, n, scale, out, ws, splits)

    for i in range(args.warmup):
        step(i)
    settled = settle(step, args.warmup)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` decode steps -----------------------
    # Two HIP events on the launch stream bracket the steps: an event marker
    # between two kernels leaves the GPU idle for ~5 us (kernel traces), so
    # the launches are not timed one by one; a launch's mean duration is the
    # span over the steps (it includes the ~1-2 us between back-to-back
    # launches).
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    span_ms = e0.elapsed_time(e1)
    launch_ms = np.array([span_ms / args.steps])
    ms_per_step = span_ms / args.steps
    tokens_per_s = w.batch / (ms_per_step / 1e3)
    trials = run_trials(step, args.trials, args.trial_steps)

    per_tok = algorithmic_bytes_per_token(w)
    rows = w.n_loops * w.batch * w.heads
    alg_bytes = w.batch * w.heads * n * per_tok + rows * w.d * 2 + rows * w.d * 4   # cache + q + out
    achieved = alg_bytes / (launch_ms.mean() / 1e3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.workload),
                "kernel": "decode step: decode_kernel (+ decode_merge_kernel when the step has more than one "
                          "workgroup per (b,h))",
                "algorithmic_bytes_per_launch": alg_bytes,
                "launch_us_mean": round(float(launch_ms.mean()) * 1e3, 2)}

    res = {
        "metric": "decode tokens/s + achieved HBM GB/s (% of peak), INT2 residual KV, 8k ctx",
        "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded looped-model KV, LogNormal channel scales)",
        "config": {"workload": f"{w.name}: 1 layer, batch {w.batch}, {w.heads} heads, head_dim {w.d}, "
                               f"{w.n_loops} loops (bits {w.bits} + BF16 reference), g={w.g}, "
                               f"rotate={w.rotate}, {n}-token context",
                   "batch": w.batch, "heads": w.heads, "head_dim": w.d, "loops": w.n_loops,
                   "n_ctx": n, "splits": splits, "replicas": args.replicas},
        "hbm_gbs": round(achieved, 1),
        "roofline": roofline,
        "wall_s": round(wall, 3),
        "settle": {"steps": settled, "target_ms": SETTLE_MS},
        "trials": trials_summary(trials, w.batch, alg_bytes),
        "system": system_info(),
    }
    if not args.no_bf16_baseline:
        del reps
        torch.cuda.empty_cache()
        bf = bf16_baseline(w, n, args.steps, args.warmup, splits, args.trials, args.trial_steps)
        res["bf16_baseline"] = bf
        res["speedup_vs_bf16"] = round(tokens_per_s / bf["value"], 3)
        # KV bytes per (batch, head, token): BF16 for every loop vs this layout;
        # at equal KV memory the feasible batch grows by their ratio
        res["batch_gain_at_equal_kv_memory"] = round(2 * w.n_loops * w.d * 2 / per_tok, 3)
        if bf.get("trials") and trials:
            res["speedup_vs_bf16_trials_mean"] = round(bf["trials"]["ms_mean"] / float(np.mean(trials)), 3)
    if not args.no_sdpa and not args.no_bf16_baseline:
        lay_b = rq.Layout(w.n_loops, w.batch, w.heads, w.d, w.g, n, w.rotate, w.bits)
        ws_b = rq.workspace_for(lay_b, n, splits, dev)

        def ours(ks, vs, q):
            o = torch.empty(w.n_loops, w.batch, w.heads, w.d, device=dev)
            rq.rq_bf16_decode_attn(lay_b, ks, vs, q, mask, n, scale, o, ws_b, splits)
            torch.cuda.synchronize()
            return o.cpu().numpy()
        res["sdpa_baseline"] = sdpa_baseline(w, n, args.steps, args.warmup, ours)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, min(args.cpu_sample, w.batch * w.heads), args.cpu_threads)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
