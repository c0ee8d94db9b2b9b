#!/usr/bin/env python3
"""Benchmark of the column-sparse delta hot path on one MI355X.

One step = one sparse diffusion step of a DiT block: the sparse MLP delta over
the top-k hidden units of each 128-token block (gathered GEMM1 + GELU + delta +
fused cache writeback, gathered GEMM2 into y) and the sparse attention delta
over the top-k keys of every (head, query block).  Both index sets are found at
the refresh, from the refresh's scores; with --mlp-rescore the MLP's scores
change every step, and each step identifies its units first.  The block is taken as
a parallel block (attention and MLP both read the block's input), so by default
the MLP's GEMM2 and the attention delta share one kernel grid (--separate: one
call each).

Default workload: HunyuanVideo 720x1280x129 (118 800 tokens: 33x45x80 latent
patches), MLP d 3072 / h 12288 keeping 860 hidden units per block (93% sparse),
attention 24 heads x 128 keeping 8316 keys per query block (93% sparse).  The
metric times K sparse steps back to back; then one whole 50-step loop runs with
its own schedule (MLP refresh every 10 steps; attention refresh at t mod 9 = 0,
6 of 50) and is timed step by step.  `--workload flux` runs the FLUX.1-dev
1280x768 shape (4352 tokens, keep 3686 units and 718 keys; 10-step loop with a
refresh at step 0).

Inputs are seeded synthetic tensors of the real shapes (random-init weights,
drifting activations).  A few distinct diffusion steps of inputs are generated
and kept in HBM; the loops cycle through them.  Everything is resident before
a timed region starts.

Prints one JSON line (last line of stdout).  Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E bandwidth (published)
HEAD_DIM = 128
RB = 128

# loop: steps of the sampler loop; mlp_every / attn_every: a layer refreshes at
# the steps t with t % every == 0; inputs: distinct diffusion steps of inputs
# kept in HBM (loop step t uses input t % inputs); mlp_sample / attn_sample:
# the oracle sample of cpu_baseline (row blocks; (head, query block) pairs),
# None = whole units until the time budget is used.
WORKLOADS = {
    # HunyuanVideo 720x1280x129: 33x45x80 latent patches, 93% sparse on the
    # sparse steps; MLP refresh every 10 steps, attention 6 dense of 50.
    "hunyuan": dict(n=118800, d=3072, h=12288, k=860, heads=24, kk=8316, loop=50, mlp_every=10, attn_every=9,
                    inputs=10, mlp_sample=32, attn_sample=4, steps=20),
    "hunyuan_mlp": dict(n=118800, d=3072, h=12288, k=860, heads=0, kk=0, loop=50, mlp_every=10, attn_every=9,
                        inputs=10, mlp_sample=32, attn_sample=0, steps=50),
    "hunyuan_attn": dict(n=118800, d=0, h=0, k=0, heads=24, kk=8316, loop=50, mlp_every=10, attn_every=9,
                         inputs=10, mlp_sample=0, attn_sample=4, steps=20),
    # FLUX.1-dev at 1280x768: 3840 image + 512 text tokens; MLP 70% sparse (keep
    # 3686 of 12288), attention 83.5% sparse (keep 718 of 4352 keys); 10 steps,
    # refresh at step 0.
    "flux": dict(n=4352, d=3072, h=12288, k=3686, heads=24, kk=718, loop=10, mlp_every=10, attn_every=10,
                 inputs=10, mlp_sample=None, attn_sample=None, steps=200),
    # FLUX.1-dev at 2304x1280: 144x80 = 11520 image + 512 text tokens, the same
    # sparsities (keep 3686 of 12288 hidden units, 16.5% = 1985 of 12032 keys).
    "flux_2304": dict(n=12032, d=3072, h=12288, k=3686, heads=24, kk=1985, loop=10, mlp_every=10, attn_every=10,
                      inputs=10, mlp_sample=None, attn_sample=None, steps=100),
    "tiny": dict(n=256, d=128, h=512, k=128, heads=0, kk=0, loop=2, mlp_every=2, attn_every=2, inputs=2,
                 mlp_sample=None, attn_sample=0, steps=200),
}
WORKLOAD_NAMES = {
    "hunyuan": "HunyuanVideo-shaped sparse step (MLP + attention delta)",
    "hunyuan_mlp": "HunyuanVideo-shaped MLP delta",
    "hunyuan_attn": "HunyuanVideo-shaped attention delta",
    "flux": "FLUX.1-dev-shaped sparse step (MLP + attention delta)",
    "flux_2304": "FLUX.1-dev-shaped sparse step at 2304x1280 (MLP + attention delta)",
    "tiny": "tiny MLP delta",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def flops_mlp(w):
    return 4.0 * w["n"] * w["d"] * w["k"]


def flops_attn(w, reident=False):
    # With per-step re-identification the delta computes two shares of the
    # chosen keys (the previous step's, taken out, and this step's, put in).
    return (8.0 if reident else 4.0) * w["n"] * w["kk"] * HEAD_DIM * w["heads"]


def kernel_work(name, w, reident=False, fp8=False, fp8_w2=False, rescore=False):
    """(amount, bound) of algorithmic work in ONE launch of kernel `name`
    (bound "mfma": bf16 matrix cores; "mfma_fp8": fp8 matrix cores; a
    ("mfma_mix", fp8 flops) bound: part of the flops on fp8 matrix cores)."""
    n, d, h, k, H, kk = w["n"], w["d"], w["h"], w["k"], w["heads"], w["kk"]
    nb = (n + RB - 1) // RB
    if name == "mlp_gemm1_sparse":
        return 2.0 * n * d * k, ("mfma_fp8" if fp8 else "mfma")
    if name == "mlp_gemm2_sparse":
        return 2.0 * n * k * d, ("mfma_fp8" if fp8_w2 else "mfma")
    if name == "sparse_step_reident_fused":
        f8 = 2.0 * n * k * d
        total = f8 + 8.0 * n * kk * HEAD_DIM * H
        return total, (("mfma_mix", f8) if fp8_w2 else "mfma")
    if name == "sparse_step_fused" and fp8_w2:
        return 2.0 * n * k * d + 4.0 * n * kk * HEAD_DIM * H, ("mfma_mix", 2.0 * n * k * d)
    if name == "quantize_fp8":
        return float(n * d * 2 + n * d + n), "hbm"
    if name == "attn_sparse":
        return 4.0 * n * kk * HEAD_DIM * H, "mfma"
    if name == "attn_reident":
        return 8.0 * n * kk * HEAD_DIM * H, "mfma"
    if name == "sparse_step_fused":
        return 2.0 * n * k * d + 4.0 * n * kk * HEAD_DIM * H, "mfma"
    if name == "topk_rows":
        # score rows read + index rows written, averaged over the step's
        # launches: the MLP's when it rescores every step, and the
        # attention's when it re-identifies (otherwise both run at the refresh)
        parts = (([nb * h * 4 + nb * k * 4] if k and rescore else []) +
                 ([H * nb * n * 4 + H * nb * kk * 4] if reident else []))
        return (float(sum(parts)) / len(parts), "hbm") if parts else (None, None)
    return None, None


def peak_for(bound, amount):
    """Matrix-core peak (TFLOP/s) for a kernel's bound: bf16, fp8, or a mix in
    which the fp8 flops run at the fp8 peak and the rest at the bf16 peak (the
    peak is then the total flops over the shortest time for both parts)."""
    if bound == "mfma_fp8":
        return PEAK_FP8_TFLOPS
    if isinstance(bound, tuple):
        f8 = bound[1]
        return amount / (f8 / PEAK_FP8_TFLOPS + (amount - f8) / PEAK_BF16_TFLOPS)
    return PEAK_BF16_TFLOPS


def source_digest():
    from dynamic_column_sparse_amd.digest import source_digest as sd
    return sd()


def traffic_for(kernel, workload):
    """HBM bytes per launch of `kernel`, from the committed counter summary
    profiles/traffic_<workload>.md, if it was taken on the current kernel
    sources (its source digest matches); else None.  Table rows read
    | kernel | source digest | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled bytes per launch |."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    digest = source_digest()
    try:
        with open(path) as f:
            for line in f:
                cells = [c.strip() for c in line.strip().strip("|").split("|")]
                if len(cells) >= 5 and cells[0] == kernel and cells[1] == digest:
                    return int(float(cells[4]))
    except (OSError, ValueError):
        return None
    return None


def copy_calibration(mib=256, reps=5):
    """A plain elementwise copy of known size (out = in + 1 over `mib` MiB of
    fp32), for scaling the HBM byte counters: each launch reads and writes
    exactly mib MiB."""
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.rand(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.add(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": n * 4, "bytes_written": n * 4, "launches": reps,
                                           "kernel": "elementwise add (torch)"}}), flush=True)


def window_sweep(workload, reps=5):
    """The sparse attention delta of the workload's shape on index sets drawn
    from the first W keys of each head, for a few W: the same kernel, the same
    flops and instruction stream, only the span of key rows the gathers touch
    changes (W keys x 512 bytes of K and V per head).  Prints one JSON line per
    W and a summary line.  Inputs are seeded Gaussian q, k, v; the index sets
    are uniform random subsets of [0, W), ascending."""
    import torch
    from dynamic_column_sparse_amd.layers import AttnDelta
    w = WORKLOADS[workload]
    n, H, kk = w["n"], w["heads"], w["kk"]
    if not kk:
        sys.exit(f"--window-sweep needs a workload with attention; {workload} has none")
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    q, k, v = (torch.randn(H, n, HEAD_DIM, generator=gen, device=dev).to(torch.bfloat16) for _ in range(3))
    att = AttnDelta(n, H, kk, dev)
    att.m.fill_(4.0)
    att.den.fill_(10.0)
    rows = H * att.nb
    windows = sorted({min(n, kk * f) for f in (1, 2, 4, 8)} | {n})
    flops = flops_attn(w)
    out = []
    for W in windows:
        for r0 in range(0, rows, 256):
            r1 = min(rows, r0 + 256)
            sc = torch.rand(r1 - r0, W, generator=gen, device=dev)
            att.idx[r0:r1] = sc.topk(kk, dim=1).indices.sort(dim=1).values.int()
        del sc
        for _ in range(2):
            att.sparse(q, k, v)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            att.sparse(q, k, v)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gathered = rows * kk * 2 * HEAD_DIM * 2
        rec = {"window_keys": W, "window_mib_per_head": round(W * 2 * HEAD_DIM * 2 / 2 ** 20, 1),
               "ms": round(ms, 3), "tflops": round(flops / ms / 1e9, 1),
               "gathered_gb": round(gathered / 1e9, 2), "gathered_tb_per_s": round(gathered / ms / 1e9, 2),
               "launches": reps + 2}
        out.append(rec)
        print(json.dumps({"window_sweep": rec}), flush=True)
    print(json.dumps({"window_sweep_summary": {"workload": WORKLOAD_NAMES[workload], "heads": H, "tokens": n, "keys_kept": kk,
                                               "windows": [r["window_keys"] for r in out],
                                               "ms": [r["ms"] for r in out]}}), flush=True)


def blas_info():
    """(threads, description) of the BLAS the oracle's NumPy runs on."""
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                desc = f"{i.get('internal_api')} {i.get('version')} ({i.get('architecture')}, " \
                       f"{i.get('threading_layer')})"
                return int(i.get("num_threads", 1)), desc
    except Exception:
        pass
    return len(os.sched_getaffinity(0)), "unknown"


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def pct(vals, q):
    return float(np.percentile(np.asarray(vals), q)) if len(vals) else None


def stats_ms(vals):
    if not vals:
        return None
    return {"count": len(vals), "median": round(pct(vals, 50), 4), "p10": round(pct(vals, 10), 4),
            "p90": round(pct(vals, 90), 4), "mean": round(float(np.mean(vals)), 4)}


def cpu_baseline(w, host, budget_s, reident=False, fp8=False, fp8_w2=False, rescore=False):
    """The CPU oracle, as it stands, on a bounded sample of the same sparse step
    (in the fp8 modes, on the fp8 operands: the weights' fp8 values are taken
    once, outside the timed part, as the layer takes them at set-up).  The
    refresh state of each sampled unit is built outside the timed part; the
    timed part is the step: the delta, per MLP row block and per attention
    (head, query block), whose index sets belong to the refresh (the MLP's
    identification is timed with the step when it rescores every step).  MLP: the workload's seeded row blocks, or whole blocks in order
    until half the budget is used; attention: the workload's seeded (head,
    query block) pairs, or pairs in order until the rest is used.  A fixed
    sample is timed repeatedly until half the budget is used.  The time per
    block / pair scales to the full step."""
    import oracle
    t_mlp = t_att = 0.0
    n_mlp = n_att = 0
    desc = []
    n = w["n"]
    nb = (n + RB - 1) // RB
    g = np.random.default_rng(1234)
    half = budget_s / 2
    if w["k"]:
        h, k = w["h"], w["k"]
        w1t = oracle.from_bf16_bits(host["w1t"])
        w2 = oracle.from_bf16_bits(host["w2"])
        if fp8:
            w1t = oracle.fp8_rows(w1t)
        w2_sparse = oracle.fp8_cols(w2) if fp8_w2 else w2
        x0, x1 = host["x"][0], host["x"][1]
        fixed = bool(w["mlp_sample"])
        blocks = sorted(g.choice(nb, size=min(nb, w["mlp_sample"]), replace=False).tolist()) if fixed else range(nb)

        def prep(b):
            r0, r1 = b * RB, min(n, b * RB + RB)
            xd = oracle.from_bf16_bits(x0[r0:r1])
            xd = oracle.fp8_rows(xd) if fp8 else xd
            a0, y0, sc = oracle.mlp_dense(xd, w1t, None, w2, None, np.zeros((r1 - r0, h)))
            idx = None if rescore else oracle.identify_topk(sc.astype(np.float32), k)
            return oracle.from_bf16_bits(x1[r0:r1]), a0, y0, sc, idx

        def run(st):
            xs1, a0, y0, sc, idx = st
            t0 = time.perf_counter()
            if rescore:
                idx = oracle.identify_topk(sc.astype(np.float32), k)
            xs1 = oracle.fp8_rows(xs1) if fp8 else xs1
            oracle.mlp_sparse(xs1, w1t, None, w2_sparse, a0, y0, idx, d_fp8=fp8_w2)
            return time.perf_counter() - t0

        if fixed:
            states = [prep(b) for b in blocks]
            reps = 0
            while reps == 0 or t_mlp < half:
                for st in states:
                    t_mlp += run(st)
                n_mlp += len(states)
                reps += 1
            desc.append(f"MLP {len(states)}/{nb} seeded row blocks, timed {reps}x")
        else:
            for b in blocks:
                t_mlp += run(prep(b))
                n_mlp += 1
                if t_mlp > half:
                    break
            desc.append(f"MLP {n_mlp}/{nb} row blocks")
    if w["kk"]:
        H, kk = w["heads"], w["kk"]
        scale = 1.0 / np.sqrt(HEAD_DIM)
        fixed = bool(w["attn_sample"])
        if fixed:
            side = int(round(np.sqrt(w["attn_sample"])))
            heads = sorted(g.choice(H, size=side, replace=False).tolist())
            qblocks = sorted(g.choice(nb, size=side, replace=False).tolist())
            pairs = [(hh, b) for hh in heads for b in qblocks]
        else:
            pairs = [(hh, b) for hh in range(H) for b in range(nb)]
        cache = {}

        def prep(hh, b):
            if cache.get("h") != hh:
                cache["h"] = hh
                cache["kv0"] = [oracle.from_bf16_bits(a[hh]) for a in host["qkv"][0][1:]]
                cache["kv1"] = [oracle.from_bf16_bits(a[hh]) for a in host["qkv"][1][1:]]
            (k0, v0), (k1, v1) = cache["kv0"], cache["kv1"]
            r0, r1 = b * RB, min(n, b * RB + RB)
            q0 = oracle.from_bf16_bits(host["qkv"][0][0][hh, r0:r1])
            q1 = oracle.from_bf16_bits(host["qkv"][1][0][hh, r0:r1])
            m, den, num, o, sc = oracle.attn_dense(q0, k0, v0, scale)
            if reident:
                return (q0, k0, v0, q1, k1, v1, m, num, den, sc)
            idx = oracle.identify_topk(sc.astype(np.float32), kk)
            nr, dr = oracle.attn_rest(q0, k0, v0, m, idx, scale)
            return (q1, k1, v1, m, nr, dr, idx)

        def run(st):
            t0 = time.perf_counter()
            if reident:
                q0, k0, v0, q1, k1, v1, m, num, den, sc = st
                idx = oracle.identify_topk(sc.astype(np.float32), kk)
                oracle.attn_reident(q0, k0, v0, q1, k1, v1, m, num, den, sc, idx, scale)
            else:
                q1, k1, v1, m, nr, dr, idx = st
                oracle.attn_sparse(q1, k1, v1, m, nr, dr, idx, scale)
            return time.perf_counter() - t0

        if fixed:
            states = [prep(hh, b) for hh, b in pairs]
            reps = 0
            while reps == 0 or t_att < half:
                for st in states:
                    t_att += run(st)
                n_att += len(states)
                reps += 1
            desc.append(f"attention {len(states)}/{H * nb} seeded (head, query block) pairs "
                        f"(2 heads x 2 query blocks), timed {reps}x")
        else:
            for hh, b in pairs:
                t_att += run(prep(hh, b))
                n_att += 1
                if t_att > half:
                    break
            desc.append(f"attention {n_att}/{H * nb} (head, query block) pairs")
    t_full = 0.0
    if n_mlp:
        t_full += t_mlp / n_mlp * nb
    if n_att:
        t_full += t_att / n_att * (w["heads"] * nb)
    extrapolated = bool(w.get("mlp_sample") or w.get("attn_sample")) or \
        (n_mlp and n_mlp < nb) or (n_att and n_att < w["heads"] * nb)
    fl = flops_mlp(w) + flops_attn(w, reident)
    threads, blas = blas_info()
    return {"value": round(fl / t_full / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "; ".join(desc) + f" of one sparse step, fp64 NumPy, scaled to the full step "
                      f"({t_full * 1e3:.0f} ms/step{' extrapolated' if extrapolated else ''}; "
                      f"sampled {t_mlp + t_att:.1f} s)",
            "ms_per_step": round(t_full * 1e3, 3), "extrapolated": bool(extrapolated),
            "cpu_model": cpu_model(), "blas": blas}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="timed sparse steps (0: the workload's default, enough steps of a short workload to make "
                         "the first step's ramp negligible)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="hunyuan", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-loop", action="store_true", help="skip the whole-loop timing (profiler runs)")
    ap.add_argument("--inputs", type=int, default=0, help="distinct input steps kept in HBM (0: the workload's)")
    ap.add_argument("--separate", action="store_true",
                    help="run the MLP and attention deltas as separate calls instead of the shared-grid step")
    ap.add_argument("--mlp-rescore", action="store_true",
                    help="every sparse step rescores the MLP units it recomputed, so S can change each step")
    ap.add_argument("--fp8", action="store_true",
                    help="the MLP's first product (dense and sparse) on fp8 e4m3 operands with per-row "
                         "power-of-two scales; x is quantized every step")
    ap.add_argument("--fp8-w2", action="store_true",
                    help="the sparse MLP delta's second product on fp8 operands (D per row and 32 units, W2 per "
                         "column)")
    ap.add_argument("--attn-reident", action="store_true",
                    help="attention identifies its keys anew every step (the cache keeps totals; each step swaps "
                         "the chosen keys' previous-step share for this step's)")
    ap.add_argument("--graph", action="store_true",
                    help="replay each sparse step as a captured HIP graph in the timed loop (eager launches are "
                         "as fast on this path)")
    ap.add_argument("--cache-every", type=int, default=0,
                    help="step caching in the timed loop: every C-th sparse step is cached (both layers recompute "
                         "nothing and keep their outputs); 0 = off")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain copy of known size (for scaling HBM byte counters)")
    ap.add_argument("--window-sweep", action="store_true",
                    help="only time the workload's sparse attention delta on index sets drawn from the first W keys "
                         "of each head, for several W (how the span of gathered rows sets the kernel's time)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return
    if args.window_sweep:
        window_sweep(args.workload)
        return

    import torch

    import synthetic as syn
    from dynamic_column_sparse_amd import lib
    from dynamic_column_sparse_amd.layers import AttnDelta, MLPDelta, sparse_step

    w = WORKLOADS[args.workload]
    if args.steps <= 0:
        args.steps = w["steps"]
    dev = torch.device("cuda:0")
    T = w["loop"]
    D = max(2, min(T, args.inputs or w["inputs"]))
    log(f"library sources {lib.chipmunk_source_digest()}")

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    t0 = time.time()
    host = {}
    mlp = att = None
    xs, qkv = [], []
    if w["k"]:
        host["w1t"], host["w2"] = syn.mlp_weights(0, w["d"], w["h"])
        mlp = MLPDelta(up(host["w1t"]), up(host["w2"]), w["n"], w["k"], rescore=args.mlp_rescore,
                       fp8=args.fp8, fp8_w2=args.fp8_w2)
        walk = syn.Walk(0, "X", 1, w["n"], w["d"])
        host["x"] = []
        for s in range(D):
            xb = walk.advance()[0]
            xs.append(up(xb))
            if s < 2:
                host["x"].append(xb)
        del walk
    if w["kk"]:
        walks = [syn.Walk(0, t, w["heads"], w["n"], HEAD_DIM) for t in "QKV"]
        host["qkv"] = []
        for s in range(D):
            st = [wk.advance() for wk in walks]
            qkv.append([up(a) for a in st])
            if s < 2:
                host["qkv"].append(st)
        del walks
        att = AttnDelta(w["n"], w["heads"], w["kk"], dev, reident=args.attn_reident)
    torch.cuda.synchronize()
    log(f"inputs ready ({time.time() - t0:.1f} s): workload {args.workload} {w}, {D} distinct input steps")

    fused = bool(mlp and att) and not args.separate

    def step(t_in, mlp_dense, attn_dense):
        if fused and not mlp_dense and not attn_dense:
            sparse_step(mlp, att, xs[t_in], *qkv[t_in])
            return
        if mlp:
            mlp.step(xs[t_in], refresh=mlp_dense)
        if att:
            att.step(*qkv[t_in], refresh=attn_dense)

    def sparse(t_in):
        step(t_in, False, False)

    def metric_input(i):
        return 1 + i % (D - 1)

    step(0, True, True)
    for i in range(args.warmup):
        sparse(metric_input(i))
    torch.cuda.synchronize()

    # One HIP graph per step input: the step's kernels replay back to back
    # without per-launch host work.  Capturing records the launches without
    # running them, so the layer state is unchanged.
    graphs = {}
    if args.graph:
        side = torch.cuda.Stream()
        for t in range(1, D):
            g = torch.cuda.CUDAGraph()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    sparse(t)
            torch.cuda.current_stream().wait_stream(side)
            graphs[t] = g
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[metric_input(i)].replay()
        torch.cuda.synchronize()

    def run_sparse(t_in):
        if graphs:
            graphs[t_in].replay()
        else:
            sparse(t_in)

    log("warmup done")

    # The metric: K whole sparse steps, nothing recorded between kernels.
    torch.cuda.synchronize()
    ts = time.perf_counter()
    for i in range(args.steps):
        run_sparse(metric_input(i))
    torch.cuda.synchronize()
    te = time.perf_counter()
    ms_per_step = (te - ts) * 1e3 / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step")

    # The spread: the same K steps with an event pair around each step.
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record(stream)
        run_sparse(metric_input(i))
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    step_ms = [a.elapsed_time(b) for a, b in evs]

    # Per-kernel durations: the same steps again, with HIP events recorded by the
    # library around every launch, on the stream the kernel runs on.
    lib.chipmunk_timing_enable(True)
    for i in range(args.steps):
        sparse(metric_input(i))
    torch.cuda.synchronize()
    lib.chipmunk_timing_enable(False)
    names = lib.kernel_names()
    kern = {}
    for kid, name in enumerate(names):
        tot, cnt = lib.chipmunk_timing_read(kid)
        if cnt:
            kern[name] = {"ms_total": tot, "launches": cnt, "avg_us": tot / cnt * 1e3}

    # The sampler loop as the workload schedules it, timed step by step: a
    # refresh of each layer where its schedule puts one, sparse steps elsewhere.
    loop = None
    if not args.no_loop:
        torch.cuda.synchronize()
        levs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(T)]
        kinds = []
        nsparse = 0
        tl = time.perf_counter()
        for t in range(T):
            md = bool(mlp) and t % w["mlp_every"] == 0
            ad = bool(att) and t % w["attn_every"] == 0
            kind = "sparse" if not (md or ad) else "dense"
            if kind == "sparse":
                nsparse += 1
                if args.cache_every and nsparse % args.cache_every == 0:
                    kind = "cached"
            kinds.append(kind)
            levs[t][0].record(stream)
            if kind != "cached":    # a cached step recomputes nothing: the output buffers stand
                step(t % D, md, ad)
            levs[t][1].record(stream)
        torch.cuda.synchronize()
        total_ms = (time.perf_counter() - tl) * 1e3
        lms = [a.elapsed_time(b) for a, b in levs]
        sp = [v for v, kd in zip(lms, kinds) if kd == "sparse"]
        dn = [v for v, kd in zip(lms, kinds) if kd == "dense"]
        ncached = sum(kd == "cached" for kd in kinds)
        loop = {"steps": T, "total_ms": round(total_ms, 3),
                "mlp_refresh_at": f"t % {w['mlp_every']} == 0" if mlp else None,
                "attn_refresh_at": f"t % {w['attn_every']} == 0" if att else None,
                "steps_with_a_refresh": len(dn), "sparse_steps": len(sp), "cached_steps": ncached,
                "sparse_step_ms": stats_ms(sp), "refresh_step_ms": stats_ms(dn),
                "distinct_inputs": D}
        log(f"loop of {T} steps: {total_ms:.1f} ms ({len(dn)} with a refresh, {ncached} cached)")

    # The outputs the timed steps left behind must be finite: a NaN or an Inf in
    # y or o marks a broken step, whatever its speed (checked after the timing).
    finite = {}
    if mlp:
        finite["y"] = bool(torch.isfinite(mlp.y).all().item())
    if att:
        finite["o"] = bool(torch.isfinite(att.o).all().item())

    fl = flops_mlp(w) + flops_attn(w, args.attn_reident)
    tflops = fl / (ms_per_step * 1e-3) / 1e12

    table = {}
    for name, r in kern.items():
        amount, bound = kernel_work(name, w, args.attn_reident, args.fp8, args.fp8_w2, args.mlp_rescore)
        ent = {"avg_us": round(r["avg_us"], 3), "launches": r["launches"],
               "share": round(r["ms_total"] / max(1e-12, sum(v["ms_total"] for v in kern.values())), 4)}
        if amount is not None:
            ach = amount / (r["avg_us"] * 1e-6)
            if bound in ("mfma", "mfma_fp8") or isinstance(bound, tuple):
                peak = peak_for(bound, amount)
                ent.update(achieved=round(ach / 1e12, 2), unit="TFLOP/s", frac=round(ach / 1e12 / peak, 4))
                if bound != "mfma":
                    ent["peak"] = round(peak, 1)
            else:
                ent.update(achieved=round(ach / 1e9, 1), unit="GB/s", frac=round(ach / 1e9 / PEAK_HBM_GBS, 4))
        table[name] = ent
    dom = max((n for n in kern if kernel_work(n, w, args.attn_reident, args.fp8, args.fp8_w2, args.mlp_rescore)[0] is not None),
              key=lambda n: kern[n]["ms_total"])
    amount, bound = kernel_work(dom, w, args.attn_reident, args.fp8, args.fp8_w2, args.mlp_rescore)
    avg_s = kern[dom]["avg_us"] * 1e-6
    if bound in ("mfma", "mfma_fp8") or isinstance(bound, tuple):
        peak = round(peak_for(bound, amount), 1)
        roof = {"bound": "mfma", "achieved": round(amount / avg_s / 1e12, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(amount / avg_s / 1e12 / peak, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(amount / avg_s / 1e9, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(amount / avg_s / 1e9 / PEAK_HBM_GBS, 4)}
    roof["kernel"] = dom
    roof["avg_us"] = round(kern[dom]["avg_us"], 3)
    roof["traffic"] = traffic_for(dom, args.workload)

    out = {
        "metric": "ms/step and effective TFLOP/s (% bf16 MFMA peak) for sparse MLP/attn delta",
        "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("bf16, fp8 e4m3 in the MLP's " + " and ".join(
            p for p, on in (("first product", args.fp8), ("second product", args.fp8_w2)) if on))
        if (args.fp8 or args.fp8_w2) else "bf16",
        "data": "synthetic (seeded Gaussian weights and drifting activations, real shapes)",
        "config": {"workload": WORKLOAD_NAMES[args.workload],
                   "tokens": w["n"], "d_model": w["d"], "d_hidden": w["h"], "mlp_keep": w["k"],
                   "heads": w["heads"], "head_dim": HEAD_DIM if w["heads"] else 0, "attn_keep": w["kk"],
                   "row_block": RB, "launch": ("hip graph per step" if args.graph else "eager")
                   + ("; MLP phase 2 and attention share one kernel" if fused else ""),
                   "mlp_set": "rescored every step" if args.mlp_rescore else "fixed between refreshes",
                   "attn_set": "re-identified every step" if args.attn_reident else "fixed between refreshes",
                   "mlp_first_product": "fp8 e4m3, per-row power-of-two scales" if args.fp8 else "bf16",
                   "mlp_second_product": "fp8 e4m3, D per (row, 32 units), W2 per column" if args.fp8_w2
                   else "bf16"},
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "flop_per_step": fl,
        "step_ms": stats_ms(step_ms),
        "roofline": roof,
        "kernels": table,
        "loop": loop,
        "outputs_finite": finite,
        "source_digest": source_digest(),
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(w, host, args.cpu_budget, args.attn_reident, args.fp8, args.fp8_w2,
                                          args.mlp_rescore)
    print(json.dumps(out), flush=True)
    if not all(finite.values()):
        print(f"bench.py: non-finite values in the step outputs {finite}", file=sys.stderr)
        sys.exit(3)


if __name__ == "__main__":
    main()
