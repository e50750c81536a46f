"""Decode benchmark: ResidualQuant fused decode attention on one MI355X.

Default workload (the metric's configuration): one layer, batch 16, 16 heads,
head_dim 128, 4 loops (loop 3 the BF16 reference, loops 0-2 INT2 residuals,
g = 32, Hadamard rotation), 8192-token context.  One step = one
rq_decode_attn call over all four loops (a single kernel launch), on seeded
synthetic KV already encoded in HBM.  Two cache replicas alternate so that
consecutive steps cannot be served from the 256 MB Infinity Cache.

Prints one JSON line: decode tokens/s (batch / step time), the roofline of the
decode kernel (algorithmic bytes / per-launch time from HIP events), and the
CPU oracle timed on a bounded sample of the same step.
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=127)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="int2-8k")
    p.add_argument("--splits", type=int, default=0, help="token splits (0 = library's choice)")
    p.add_argument("--replicas", type=int, default=2)
    p.add_argument("--cpu-sample", type=int, default=256, help="(batch, head) pairs the oracle decodes")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-bf16-baseline", action="store_true")
    p.add_argument("--mode", default="decode", choices=["decode", "copy"],
                   help="copy: a plain 1 GiB device copy, the reference for HBM counter scaling")
    return p.parse_args()


def algorithmic_bytes_per_token(w) -> int:
    """Bytes one decode step must read per (batch, head, token): the BF16
    reference K and V once, and for each residual loop its codes, FP16
    scale/zero per group and FP16 LS coefficient, for K and for V."""
    from oracle.storage import layout_bytes_per_token
    return layout_bytes_per_token(w.n_loops, w.bits, w.g, w.d)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("rq_decode.hip", "rq_device.hpp", "rq_internal.hpp"):
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


def cpu_baseline(w, n_pairs: int):
    """The oracle's decode (FP64 reconstruction + FP64 attention), single
    thread, on n_pairs (batch, head) pairs of the same workload, all loops;
    scaled to the full step."""
    import numpy as np
    import synth
    from oracle import rq_oracle as orc
    from synth import bf16_bits

    g = synth.generator(w.seed + 1000)
    kstd, vstd = synth.channel_std(g, 1, w.d), synth.channel_std(g, 1, w.d)
    kr, kl = synth.draw_kv(g, w.n_loops, n_pairs, 1, w.n_ctx, w.d, w.c, w.sigma, kstd)
    vr, vl = synth.draw_kv(g, w.n_loops, n_pairs, 1, w.n_ctx, w.d, w.c, w.sigma, vstd)
    q = synth.draw_queries(g, w.n_loops, n_pairs, 1, w.d)
    lay = dict(n_loops=w.n_loops, batch=n_pairs, heads=1, d=w.d, g=w.g, cap=w.n_ctx,
               rotate=w.rotate, bits=w.bits)
    kp = orc.Planes(w.n_loops, n_pairs, 1, w.d, w.g, w.n_ctx, w.bits)
    vp = orc.Planes(w.n_loops, n_pairs, 1, w.d, w.g, w.n_ctx, w.bits)
    kp.ref[:] = bf16_bits(kr)
    vp.ref[:] = bf16_bits(vr)
    orc.encode(lay, kp, bf16_bits(kl), 0, w.n_ctx)
    orc.encode(lay, vp, bf16_bits(vl), 0, w.n_ctx)
    qb = bf16_bits(q)
    mask = (1 << w.n_loops) - 1
    t0 = time.perf_counter()
    orc.decode(lay, kp, vp, qb, mask, w.n_ctx, 1.0 / np.sqrt(w.d))
    dt = time.perf_counter() - t0
    step_s = dt * (w.batch * w.heads) / n_pairs
    return {"value": w.batch / step_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_pairs} of {w.batch * w.heads} (batch, head) pairs x {w.n_loops} loops x "
                      f"{w.n_ctx} tokens decoded in {dt:.1f} s on one core, scaled x"
                      f"{w.batch * w.heads / n_pairs:.2f} to the full step",
            "ms_per_step": step_s * 1e3}


def bf16_baseline(w, n, steps, warmup, splits_rq):
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
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = w.batch * w.heads * n * 2 * w.n_loops * w.d * 2
    del reps
    torch.cuda.empty_cache()
    return {"value": round(w.batch / (ms / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4),
            "hbm_gbs": round(nbytes / (ms / 1e3) / 1e9, 1), "bytes_per_step": nbytes,
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


def main():
    args = parse()
    if args.mode == "copy":
        copy_probe()
        return
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU; --gpus must be 1 (the per-(batch, head) "
              "work shards across GPUs without exchange, but no multi-GPU path is built)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import decode_attention_rq_amd as rq
    import synth

    w = synth.WORKLOADS[args.workload]
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
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` decode steps -----------------------
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record()
        step(i)
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    span_ms = starts[0].elapsed_time(ends[-1])
    ms_per_step = span_ms / args.steps
    tokens_per_s = w.batch / (ms_per_step / 1e3)

    per_tok = algorithmic_bytes_per_token(w)
    rows = w.n_loops * w.batch * w.heads
    alg_bytes = w.batch * w.heads * n * per_tok + rows * w.d * 2 + rows * w.d * 4   # cache + q + out
    achieved = alg_bytes / (launch_ms.mean() / 1e3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.workload),
                "kernel": "decode_kernel (one launch per step)",
                "algorithmic_bytes_per_launch": alg_bytes,
                "launch_us_mean": round(float(launch_ms.mean()) * 1e3, 2),
                "launch_us_min": round(float(launch_ms.min()) * 1e3, 2)}

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
    }
    if not args.no_bf16_baseline:
        del reps
        torch.cuda.empty_cache()
        bf = bf16_baseline(w, n, args.steps, args.warmup, splits)
        res["bf16_baseline"] = bf
        res["speedup_vs_bf16"] = round(tokens_per_s / bf["value"], 3)
        # KV bytes per (batch, head, token): BF16 for every loop vs this layout;
        # at equal KV memory the feasible batch grows by their ratio
        res["batch_gain_at_equal_kv_memory"] = round(2 * w.n_loops * w.d * 2 / per_tok, 3)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, min(args.cpu_sample, w.batch * w.heads))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
