#!/usr/bin/env python3
"""Benchmark of the sliced-precision quantized linear layer on one MI355X.

Workload (one step): the Llama-3.1-8B FFN projections (gate and up 4096->14336,
down 14336->4096) at decode batch M = 1, fp16 activations, one int8 parent
per matrix (g = 128, fp16 scale/zero, W ~ N(0, 0.02^2) with 0.1% outliers x10),
sliced with the true-prefix rule at every width r in {2, 3, 4, 6, 8}: 15 layer
calls, issued as one mixed-width call list.  Each projection reads a fixed
seeded input and writes its own output, so the 15 calls are independent and
the library runs them as one GEMV launch.

Inputs are resident in HBM before timing.  Each step reads a different copy of
the parents from a ring sized so that every timed piece reads more than 1 GiB
per pass through it (four times the 256 MB MALL): weight reads come from HBM,
not the last-level cache.

Timing (one declared mode): the calls are captured in HIP graphs (checked bit
for bit against eager calls first) and replayed, up to 40 decode steps per
graph (the default run: one graph of all timed steps); HIP events on the launch
stream bracket the replays.
  value        algorithmic bytes of all calls of the timed steps / their time
               (GB/s).  Algorithmic bytes per call = bit planes the width reads
               + 4 B (fp16 scale + zero) per group + X (2*M*K) + Y (2*M*N).
  per_r        per width: the one launch of the step (gate, up and down), and
               the two launches a dependent FFN block needs (gate+up, then
               down reading their product), each averaged over >= 200 launches.
  roofline     the step's one launch (the 15 calls of every width together),
               averaged over >= 200 launches; traffic from the committed
               counter run of that launch.
  attention    the Llama-3.1-8B attention projections (q, o 4096->4096; k, v
               4096->1024) at M = 1 (one launch per width, and the q/k/v then
               o launches of a dependent block) and M = 16, 64.
  prefill      the M = 2048 bf16 GEMM (same shapes, r in {2, 4, 8}).
  skinny       decode batches M in {8, 16, 32, 64} at r in {2, 3, 4, 8}
               against max(HBM time, MFMA time).
  mixnmatch    one pass over 42 Gemma-2-9B FFN blocks (gate/up 3584->14336,
               down 14336->3584, g = 128) at the seeded per-block widths (14
               each of 2, 3 and 4 bits), M = 1 (fp16) and M = 256 (bf16); each
               call reads a fixed input and writes its own output.
  cpu_baseline the CPU oracle on all three matrices at every width.
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
# fp32 vector operations per second: the published 157.3 TFLOP/s fp32 vector
# peak counts an FMA as two flops, i.e. 256 CUs x 4 SIMDs x 32 lanes per clock x
# 2.4 GHz operations
ALU_PEAK_OPS = 256 * 4 * 32 * 2.4e9
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
WIDTHS = (2, 3, 4, 6, 8)
PREFILL_WIDTHS = (2, 4, 8)
GROUP = 128
RING_BYTES = 1 << 30           # bytes each timed piece reads per pass through the ring
MIN_LAUNCHES = 200             # launches averaged per per-launch figure
GRAPH_STEPS = 40               # decode steps per graph in the timed region (the default --steps: one graph)
METRIC = "sliced W·X: decode GB/s (packed bytes, %HBM peak) + prefill TFLOP/s (%MFMA) per r"
PLANE_BITS = (2, 1, 1, 2, 2)
PLANES_FOR_R = {2: 1, 3: 2, 4: 3, 6: 4, 8: 5}
DECODE_KERNEL_SRC = os.path.join(ROOT, "nested_integer_weight_amd", "csrc", "mq_gemv.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_step_llama8b_ffn_m1.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def alg_bytes(m, n, k, r, group=GROUP):
    planes = sum(n * k * PLANE_BITS[p] // 8 for p in range(PLANES_FOR_R[r]))
    return planes + 4 * n * (k // group) + 2 * m * k + 2 * m * n


def src_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-steps", type=int, default=3, help="workload steps the CPU oracle baseline times")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill GEMM lines")
    ap.add_argument("--prefill-iters", type=int, default=10)
    ap.add_argument("--no-skinny", action="store_true", help="skip the M in {8,16,32,64} lines")
    ap.add_argument("--no-mix", action="store_true", help="skip the 42-block Mix'n'Match stack lines")
    ap.add_argument("--no-pieces", action="store_true", help="skip the per-launch figures")
    ap.add_argument("--no-attn", action="store_true", help="skip the attention-projection lines")
    ap.add_argument("--no-produce", action="store_true", help="skip the parent-producer lines")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (this build has no "
              "multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch
    from nested_integer_weight_amd import mq, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # ---------------- inputs (resident before timing) ----------------
    # ring: distinct parent copies, enough that the smallest timed piece (the
    # r = 2 down projection, 16.5 MB) reads > RING_BYTES per pass
    min_piece = min(alg_bytes(1, n, k, 2) for _, n, k in synth.LLAMA8B_FFN)
    ring = max(8, math.ceil(RING_BYTES / min_piece))
    if ring % len(WIDTHS) == 0:
        ring += 1  # steps walk the ring in strides of len(WIDTHS): keep them coprime
    mats = []
    for tid, (name, n, k) in enumerate(synth.LLAMA8B_FFN):
        t0 = time.time()
        lay = synth.make_layer(cfg_id=2, tensor_id=tid, n=n, k=k, m=0, group=GROUP, outlier_frac=1e-3)
        x = synth.activations(synth.rng_for(2, 100 + tid), 1, k, "f16")
        q = torch.from_numpy(lay.q).to(dev)
        s = torch.from_numpy(lay.scales).to(dev)
        z = torch.from_numpy(lay.zeros).to(dev)
        base = mq.pack_parent(q)
        copies = []
        for c in range(ring):
            planes = [p.clone() for p in base.planes]
            copies.append((mq.Packed(n, k, planes), s.clone(), z.clone()))
        del q
        mats.append(dict(name=name, n=n, k=k, lay=lay, x=x, xd=x.to(dev), copies=copies,
                         y={r: torch.empty((1, n), dtype=torch.float16, device=dev) for r in WIDTHS}))
        log(f"[bench] {name} {n}x{k}: parent packed, {ring} copies ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()

    def calls_for(step, r, idx=(0, 1, 2)):
        ri = WIDTHS.index(r)
        c = (step * len(WIDTHS) + ri) % ring
        out = []
        for i in idx:
            mt = mats[i]
            pk, s, z = mt["copies"][c]
            out.append(mq.Call(x=mt["xd"], packed=pk.truncated(r), r=r, rule="prefix", group=GROUP,
                               scales=s, zeros=z, out=mt["y"][r]))
        return out

    bytes_r = {r: sum(alg_bytes(1, mt["n"], mt["k"], r) for mt in mats) for r in WIDTHS}
    bytes_step = sum(bytes_r.values())
    log(f"[bench] bytes/step {bytes_step / 1e6:.1f} MB; ring of {ring} copies: "
        f"{ring * bytes_r[2] / 1e9:.2f} GB per pass at r=2, {ring * bytes_r[8] / 1e9:.2f} GB at r=8")

    def step_calls(step):
        # the 15 calls of a step are independent: one mq_linear_mixed call,
        # which puts them all into one GEMV launch
        mq.linear_mixed([c for r in WIDTHS for c in calls_for(step, r)])

    # ---------------- warmup ----------------
    for i in range(args.warmup):
        step_calls(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    def outputs():
        return [mt["y"][r].clone() for mt in mats for r in WIDTHS]

    def check_replay(g, eager_fn):
        """The graph must reproduce the eager calls bit for bit, replay after
        replay, with eager work and synchronisation in between."""
        eager_fn()
        torch.cuda.synchronize()
        ref = outputs()
        for _ in range(2):
            for mt in mats:
                for r in WIDTHS:
                    mt["y"][r].zero_()
            g.replay()
            torch.cuda.synchronize()
            if not all(torch.equal(a, b) for a, b in zip(outputs(), ref)):
                return False
            eager_fn()
            torch.cuda.synchronize()
        return True

    # ---------------- timed steps: HIP graph replay ----------------
    # Graphs of GRAPH_STEPS consecutive steps each (one launch per step),
    # covering the timed steps in order, so exactly --steps steps are timed and
    # consecutive steps read different parent copies.  While the GPU runs one
    # graph the host submits the next.  A replay costs the host tens of
    # microseconds, which graphs of a few 100-us steps do not hide (graphs of
    # five steps timed 4.5 us per step above the same launches in a graph of
    # 66), so the default run replays a single graph of all 40 timed steps.
    segs = [(a, min(a + GRAPH_STEPS, args.steps)) for a in range(0, args.steps, GRAPH_STEPS)]
    step_graphs = [capture(lambda a=a, b=b: [step_calls(i) for i in range(a, b)]) for a, b in segs]
    for gi in sorted({0, len(segs) - 1}):
        a, b = segs[gi]
        if not check_replay(step_graphs[gi], lambda a=a, b=b: [step_calls(i) for i in range(a, b)]):
            raise RuntimeError("graph replay of the decode step differs from the eager calls")
    torch.cuda.synchronize()
    t0_, t1_ = ev(), ev()
    t0_.record(stream)
    for g in step_graphs:
        g.replay()
    t1_.record(stream)
    torch.cuda.synchronize()
    step_ms = t0_.elapsed_time(t1_) / args.steps
    value = bytes_step / (step_ms * 1e-3) / 1e9
    log(f"[bench] {args.steps} steps (graph replay): {step_ms * 1e3:.1f} us/step, {value:.1f} GB/s")
    del step_graphs

    # secondary: the same steps issued as eager C-ABI calls (host gaps included)
    torch.cuda.synchronize()
    t0_.record(stream)
    for i in range(args.steps):
        step_calls(args.warmup + i)
    t1_.record(stream)
    torch.cuda.synchronize()
    eager_ms = t0_.elapsed_time(t1_) / args.steps
    eager = {"value": round(bytes_step / (eager_ms * 1e-3) / 1e9, 1), "ms_per_step": round(eager_ms, 5)}
    log(f"[bench] eager: {eager_ms * 1e3:.1f} us/step")
    # and with the call lists checked and marshalled once (mq.PreparedCalls):
    # one C-ABI call per step, the host cost of a serving loop without graphs
    prepared = [mq.PreparedCalls([c for r in WIDTHS for c in calls_for(i, r)]) for i in range(min(args.steps, ring))]
    prepared[0].run()
    torch.cuda.synchronize()
    t0_.record(stream)
    for i in range(args.steps):
        prepared[i % len(prepared)].run()
    t1_.record(stream)
    torch.cuda.synchronize()
    prep_ms = t0_.elapsed_time(t1_) / args.steps
    eager["prepared_ms_per_step"] = round(prep_ms, 5)
    eager["prepared_value"] = round(bytes_step / (prep_ms * 1e-3) / 1e9, 1)
    log(f"[bench] eager, prepared call lists: {prep_ms * 1e3:.1f} us/step")
    del prepared

    # ---------------- per-launch figures ----------------
    # The fused launch of each width (gate, up and down), and for comparison the
    # two launches of a dependent FFN block, where down reads what gate and up
    # produced and so cannot share their launch: gate and up, then down alone.
    # Graphs of `ring` launches over the whole ring, replayed until >= 200.
    def piece(fn_for_step, nbytes):
        g = capture(lambda: [fn_for_step(i) for i in range(ring)])
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, math.ceil(MIN_LAUNCHES / ring))
        a_, b_ = ev(), ev()
        a_.record(stream)
        for _ in range(reps):
            g.replay()
        b_.record(stream)
        torch.cuda.synchronize()
        us = a_.elapsed_time(b_) * 1e3 / (reps * ring)
        del g
        gbs = nbytes / (us * 1e-6) / 1e9
        return {"us_per_launch": round(us, 3), "bytes_per_launch": int(nbytes), "GB/s": round(gbs, 1),
                "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "launches_timed": reps * ring}

    per_r = {}
    step_launch = None
    if not args.no_pieces:
        step_launch = piece(step_calls, bytes_step)
        log(f"[bench] step as one launch: {step_launch['us_per_launch']} us "
            f"({step_launch['frac_hbm'] * 100:.1f}% HBM)")
        for r in WIDTHS:
            d = {}
            d["gate_up_down"] = piece(lambda i: mq.linear_mixed(calls_for(i, r)), bytes_r[r])
            gu = sum(alg_bytes(1, mats[i]["n"], mats[i]["k"], r) for i in (0, 1))
            d["gate_up"] = piece(lambda i: mq.linear_mixed(calls_for(i, r, (0, 1))), gu)
            d["down"] = piece(lambda i: mq.linear_mixed(calls_for(i, r, (2,))), bytes_r[r] - gu)
            dep_us = d["gate_up"]["us_per_launch"] + d["down"]["us_per_launch"]
            d["dependent_ffn_block"] = {"us": round(dep_us, 3),
                                        "frac_hbm": round(bytes_r[r] / (dep_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            per_r[str(r)] = d
            log(f"[bench] r={r}: one launch {d['gate_up_down']['us_per_launch']} us "
                f"({d['gate_up_down']['frac_hbm'] * 100:.1f}% HBM); dependent block {dep_us:.2f} us")

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            t = json.load(open(TRAFFIC_FILE))
            if t.get("kernel_src_sha256_16") == src_hash(DECODE_KERNEL_SRC):
                traffic = t.get("hbm_bytes_per_launch")
        except Exception:
            traffic = None
    roofline = None
    if step_launch:
        dom = step_launch
        roofline = {"bound": "hbm", "achieved": dom["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(dom["GB/s"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "kernel": "mq::gemv_multi_kernel<prefix, m=1, fp16>: gate, up (14336x4096) and down "
                              "(4096x14336) at r = 2, 3, 4, 6 and 8, the 15 calls in one launch "
                              "(mq_linear_mixed decode path)",
                    "bytes_per_launch": dom["bytes_per_launch"], "us_per_launch": dom["us_per_launch"]}

    # ---------------- attention projections (Llama-3.1-8B q, k, v, o) ----------------
    # Decode at M = 1: the four projections of a width in one launch (each reads
    # a fixed input, as the FFN calls do), and the two launches a dependent
    # attention block needs (q, k and v, then o); M = 16 and 64 through the
    # skinny path.  Own ring: its smallest piece is ~10 MB.
    attn = None
    if not args.no_attn:
        attn = {}
        amin = sum(alg_bytes(1, n, k, 2) for _, n, k in synth.LLAMA8B_ATTN)
        aring = math.ceil(RING_BYTES / amin)
        amats = []
        for tid, (name, n, k) in enumerate(synth.LLAMA8B_ATTN):
            lay = synth.make_layer(cfg_id=12, tensor_id=tid, n=n, k=k, m=0, group=GROUP, outlier_frac=1e-3)
            q = torch.from_numpy(lay.q).to(dev)
            s = torch.from_numpy(lay.scales).to(dev)
            z = torch.from_numpy(lay.zeros).to(dev)
            base = mq.pack_parent(q)
            copies = [(mq.Packed(n, k, [p.clone() for p in base.planes]), s.clone(), z.clone())
                      for _ in range(aring)]
            del q, base
            xa = {m: synth.activations(synth.rng_for(12, 200 + tid, m), m, k, "f16").to(dev) for m in (1, 16, 64)}
            ya = {m: torch.empty((m, n), dtype=torch.float16, device=dev) for m in (1, 16, 64)}
            amats.append(dict(name=name, n=n, k=k, copies=copies, x=xa, y=ya))
        torch.cuda.synchronize()
        log(f"[bench] attention: 4 parents, {aring} copies")

        def attn_calls(i, r, m, idx=(0, 1, 2, 3)):
            c = i % aring
            return [mq.Call(x=amats[j]["x"][m], packed=amats[j]["copies"][c][0].truncated(r), r=r, rule="prefix",
                            group=GROUP, scales=amats[j]["copies"][c][1], zeros=amats[j]["copies"][c][2],
                            out=amats[j]["y"][m]) for j in idx]

        def apiece(fn, nbytes, nflop=0.0):
            fn(0)  # eager first: any workspace is allocated outside the capture
            torch.cuda.synchronize()
            g = capture(lambda: [fn(i) for i in range(aring)])
            g.replay()
            torch.cuda.synchronize()
            reps = max(1, math.ceil(MIN_LAUNCHES / aring))
            a_, b_ = ev(), ev()
            a_.record(stream)
            for _ in range(reps):
                g.replay()
            b_.record(stream)
            torch.cuda.synchronize()
            us = a_.elapsed_time(b_) * 1e3 / (reps * aring)
            del g
            d = {"us": round(us, 3), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                 "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            if nflop:
                d["TFLOP/s"] = round(nflop / (us * 1e-6) / 1e12, 1)
            return d

        for r in WIDTHS:
            ab4 = sum(alg_bytes(1, mt["n"], mt["k"], r) for mt in amats)
            d = {"qkvo_one_launch": apiece(lambda i: mq.linear_mixed(attn_calls(i, r, 1)), ab4)}
            qkv = apiece(lambda i: mq.linear_mixed(attn_calls(i, r, 1, (0, 1, 2))),
                         sum(alg_bytes(1, amats[j]["n"], amats[j]["k"], r) for j in (0, 1, 2)))
            o = apiece(lambda i: mq.linear_mixed(attn_calls(i, r, 1, (3,))), alg_bytes(1, 4096, 4096, r))
            d["dependent_block_us"] = round(qkv["us"] + o["us"], 3)
            if r in (2, 4, 8):
                for m in (16, 64):
                    # the four skinny calls one after another (each a launch of its own)
                    byt = sum(alg_bytes(m, mt["n"], mt["k"], r) for mt in amats)
                    fl = 2.0 * m * sum(mt["n"] * mt["k"] for mt in amats)
                    d[f"m{m}_four_calls"] = apiece(lambda i: mq.linear_mixed(attn_calls(i, r, m)), byt, fl)
            attn[str(r)] = d
            log(f"[bench] attention r={r}: one launch {d['qkvo_one_launch']['us']} us "
                f"({d['qkvo_one_launch']['frac_hbm'] * 100:.1f}% HBM), dependent block {d['dependent_block_us']} us")
        del amats

    # ---------------- prefill (M = 2048, bf16) ----------------
    prefill = None
    if not args.no_prefill:
        prefill = {}
        xs = {k: synth.activations(synth.rng_for(4, 7, k), 2048, k, "bf16").to(dev) for k in (4096, 14336)}
        for r in PREFILL_WIDTHS:
            rows = []
            for mt in mats:
                x = xs[mt["k"]]
                y = torch.empty((2048, mt["n"]), dtype=torch.bfloat16, device=dev)
                for c in range(2):
                    pk, s, z = mt["copies"][c]
                    mq.linear(x, pk, r, "prefix", GROUP, s, z, out=y)
                torch.cuda.synchronize()
                a, b = ev(), ev()
                a.record(stream)
                for it in range(args.prefill_iters):
                    pk, s, z = mt["copies"][it % ring]
                    mq.linear(x, pk, r, "prefix", GROUP, s, z, out=y)
                b.record(stream)
                torch.cuda.synchronize()
                us = a.elapsed_time(b) * 1e3 / args.prefill_iters
                flops = 2.0 * 2048 * mt["n"] * mt["k"]
                rows.append((mt["name"], us, flops))
            tot_us = sum(u for _, u, _ in rows)
            tot_f = sum(f for _, _, f in rows)
            tf = tot_f / (tot_us * 1e-6) / 1e12
            prefill[str(r)] = {"TFLOP/s": round(tf, 1), "frac_mfma_bf16": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                               "us_per_matrix": {nm: round(u, 1) for nm, u, _ in rows}}
            log(f"[bench] prefill r={r}: {tf:.1f} TFLOP/s")

    # ---------------- skinny decode batches (M = 8..64, fp16) ----------------
    # gate, up and down (separate outputs) through mq_linear_mixed, so calls of
    # one launch shape share a launch; figures are per call (a third of a step)
    skinny = None
    if not args.no_skinny:
        skinny = {}
        for m in (8, 16, 32, 64):
            xs_m = {k: synth.activations(synth.rng_for(3, m, k), m, k, "f16").to(dev) for k in (4096, 14336)}
            # one output per matrix (gate and up must not share one, or they could not share a launch)
            ys_m = {mt["name"]: torch.empty((m, mt["n"]), dtype=torch.float16, device=dev) for mt in mats}
            for r in (2, 3, 4, 8):
                def sk_calls(it):
                    c = it % ring
                    return [mq.Call(x=xs_m[mt["k"]], packed=mt["copies"][c][0].truncated(r), r=r, rule="prefix",
                                    group=GROUP, scales=mt["copies"][c][1], zeros=mt["copies"][c][2],
                                    out=ys_m[mt["name"]]) for mt in mats]
                def one_by_one(cl):
                    for c in cl:
                        mq.linear(c.x, c.packed, c.r, c.rule, c.group, c.scales, c.zeros, out=c.out)

                iters = max(ring, math.ceil(MIN_LAUNCHES / len(mats)))
                per_call = {}
                for mode, issue in (("shared", mq.linear_mixed), ("one_by_one", one_by_one)):
                    for i in range(3):
                        issue(sk_calls(i))
                    torch.cuda.synchronize()
                    a_, b_ = ev(), ev()
                    a_.record(stream)
                    for i in range(iters):
                        issue(sk_calls(3 + i))
                    b_.record(stream)
                    torch.cuda.synchronize()
                    per_call[mode] = a_.elapsed_time(b_) * 1e3 / (iters * len(mats))
                us = per_call["shared"]
                byt = sum(alg_bytes(m, mt["n"], mt["k"], r) for mt in mats) / len(mats)
                fl = 2.0 * m * sum(mt["n"] * mt["k"] for mt in mats) / len(mats)
                t_hbm = byt / (HBM_PEAK_GBS * 1e9)
                t_mfma = fl / (BF16_MFMA_PEAK_TFLOPS * 1e12)
                skinny[f"m{m}_r{r}"] = {"us_per_call": round(us, 2),
                                        "us_per_call_one_launch_each": round(per_call["one_by_one"], 2),
                                        "GB/s": round(byt / (us * 1e-6) / 1e9, 1),
                                        "TFLOP/s": round(fl / (us * 1e-6) / 1e12, 1),
                                        "roofline_frac": round(max(t_hbm, t_mfma) / (us * 1e-6), 4)}
            log(f"[bench] skinny m={m} (us per call, shared launches / one launch each): " +
                ", ".join(f"r{r} {skinny[f'm{m}_r{r}']['us_per_call']} / "
                          f"{skinny[f'm{m}_r{r}']['us_per_call_one_launch_each']}" for r in (2, 3, 4, 8)))

    # ---------------- Mix'n'Match stack: 42 Gemma-2-9B FFN blocks ----------------
    mix = None
    if not args.no_mix:
        t0 = time.time()
        widths = synth.mixnmatch_widths()
        blocks = []
        for blk in range(synth.GEMMA9B_BLOCKS):
            for tid, (name, n, k) in enumerate(synth.GEMMA9B_FFN):
                q, s_, z_ = synth.device_parent(1000 * (blk + 1) + tid, n, k, GROUP, dev)
                pk = mq.pack_parent(q)
                del q
                blocks.append((blk, name, n, k, widths[blk], pk.truncated(widths[blk]), s_, z_))
        torch.cuda.synchronize()
        log(f"[bench] mixnmatch: {len(blocks)} parents drawn and packed ({time.time() - t0:.1f}s)")
        mix = {"widths": widths, "mean_bits": sum(widths) / len(widths)}
        for m, dt, tdt in ((1, "f16", torch.float16), (256, "bf16", torch.bfloat16)):
            xk = {k: synth.activations(synth.rng_for(5, 77, k, m), m, k, dt).to(dev) for k in (3584, 14336)}
            ys = [torch.empty((m, n), dtype=tdt, device=dev) for (_, _, n, _, _, _, _, _) in blocks]
            calls = [mq.Call(x=xk[k], packed=pk, r=r, rule="prefix", group=GROUP, scales=s_, zeros=z_, out=y)
                     for (blk, name, n, k, r, pk, s_, z_), y in zip(blocks, ys)]
            mq.linear_mixed(calls)
            torch.cuda.synchronize()
            ref = [y.clone() for y in ys]
            g = capture(lambda: mq.linear_mixed(calls))
            for y in ys:
                y.zero_()
            g.replay()
            torch.cuda.synchronize()
            if not all(torch.equal(a, b) for a, b in zip(ys, ref)):
                raise RuntimeError("graph replay of the Mix'n'Match pass differs from the eager calls")
            passes = 5 if m == 1 else 3
            a_, b_ = ev(), ev()
            a_.record(stream)
            for _ in range(passes):
                g.replay()
            b_.record(stream)
            torch.cuda.synchronize()
            us = a_.elapsed_time(b_) * 1e3 / passes
            del g
            byt = sum(alg_bytes(m, n, k, r) for (blk, name, n, k, r, pk, s_, z_) in blocks)
            fl = 2.0 * m * sum(n * k for (blk, name, n, k, r, pk, s_, z_) in blocks)
            if m == 1:
                mix["m1"] = {"us_per_pass": round(us, 1), "GB/s": round(byt / (us * 1e-6) / 1e9, 1),
                             "frac_hbm": round(byt / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "bytes": int(byt)}
            else:
                mix["m256"] = {"us_per_pass": round(us, 1), "TFLOP/s": round(fl / (us * 1e-6) / 1e12, 1),
                               "frac_mfma_bf16": round(fl / (us * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                               "flop": fl}
            log(f"[bench] mixnmatch m={m}: {us:.1f} us per pass of {len(blocks)} calls (graph replay)")
            del ys, calls, ref
        del blocks

    # ---------------- parent producer (scale search + cross-width code choice) ----------------
    # MatGPTQ's target set {3, 4, 8}, equal lambdas, 80 shrink candidates of the
    # min-max range (p = 1 - i/100), on the three FFN matrices of the 8B model.
    # Algorithmic fp32 operations per weight: per (weight, candidate) 3 (divide,
    # round, add the zero point) + 6 per width (two to reconstruct, difference,
    # square, weight, accumulate); per weight 5 per distinct level of each width
    # + 2^8 x |R| (|R| - 1 additions and one comparison per code).
    producer = None
    if not args.no_produce:
        pw, pl, pgrid, pden = [3, 4, 8], [1.0, 1.0, 1.0], 80, 100
        levels = sum(2 ** r for r in pw)  # true prefix: 2^r levels per width (2^8 at r = 8)
        ops_per_weight = pgrid * (3 + 6 * len(pw)) + 5 * levels + 256 * len(pw)
        producer = {"widths": pw, "lambdas": pl, "n_grid": pgrid, "grid_den": pden, "group": GROUP,
                    "rule": "prefix", "alg_ops_per_weight": ops_per_weight, "alu_peak_Tops": ALU_PEAK_OPS / 1e12}
        tot_ms, tot_w = 0.0, 0
        for i, (name, n, k) in enumerate(synth.LLAMA8B_FFN):
            w = synth.device_weights(500 + i, n, k, dev)
            mq.produce_parent(w, GROUP, pw, pl, "prefix", pgrid, pden)
            torch.cuda.synchronize()
            reps = 3
            a_, b_ = ev(), ev()
            a_.record(stream)
            for _ in range(reps):
                mq.produce_parent(w, GROUP, pw, pl, "prefix", pgrid, pden)
            b_.record(stream)
            torch.cuda.synchronize()
            ms = a_.elapsed_time(b_) / reps
            tot_ms += ms
            tot_w += n * k
            producer[name] = {"ms": round(ms, 3), "Gweights/s": round(n * k / (ms * 1e-3) / 1e9, 3)}
            del w
        producer["ffn_ms"] = round(tot_ms, 3)
        producer["Gweights/s"] = round(tot_w / (tot_ms * 1e-3) / 1e9, 3)
        producer["alu_frac"] = round(tot_w * ops_per_weight / (tot_ms * 1e-3) / ALU_PEAK_OPS, 4)
        log(f"[bench] producer: 8B FFN (3 matrices) in {tot_ms:.2f} ms, {producer['Gweights/s']} Gweights/s, "
            f"{producer['alu_frac'] * 100:.1f}% of the fp32 VALU issue rate")

    # ---------------- reference: device copies at the decode launch sizes ----------------
    # torch's device copy over a ring of buffers (> 1 GiB per pass): read and
    # write bytes over the copy time, the streaming rate one launch of that size
    # reaches without any arithmetic
    copy_ref = None
    if not args.no_pieces:
        copy_ref = {}
        for name, nbytes in (("r2_step_launch", bytes_r[2]), ("r8_step_launch", bytes_r[8])):
            half = (nbytes // 2 + 4095) // 4096 * 4096
            nbuf = max(4, math.ceil(RING_BYTES / (2 * half)))
            src = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
            dst = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
            for i in range(nbuf):
                dst[i].copy_(src[i])
            torch.cuda.synchronize()
            reps = max(nbuf, MIN_LAUNCHES)
            a_, b_ = ev(), ev()
            a_.record(stream)
            for i in range(reps):
                dst[i % nbuf].copy_(src[i % nbuf])
            b_.record(stream)
            torch.cuda.synchronize()
            us = a_.elapsed_time(b_) * 1e3 / reps
            copy_ref[name] = {"bytes_moved": 2 * half, "us": round(us, 3),
                              "GB/s": round(2 * half / (us * 1e-6) / 1e9, 1),
                              "frac_hbm": round(2 * half / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            del src, dst
        log(f"[bench] device copy reference: " + ", ".join(f"{k} {v['us']} us ({v['frac_hbm'] * 100:.1f}%)"
                                                           for k, v in copy_ref.items()))

    if args.copy_calib_mib > 0:
        nb = args.copy_calib_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {nb} bytes done")

    # ---------------- CPU oracle baseline ----------------
    cpu = None
    if not args.no_cpu:
        from threadpoolctl import threadpool_info, threadpool_limits

        from oracle import mq_oracle as O

        def oracle_calls(n_steps):
            done = 0
            for _ in range(n_steps):
                for mt in mats:
                    lay = mt["lay"]
                    x64 = mt["x"].double().numpy()
                    for r in WIDTHS:
                        O.linear(x64, lay.q, lay.scales, lay.zeros, r, O.PREFIX, GROUP)
                        done += alg_bytes(1, mt["n"], mt["k"], r)
            return done

        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        t0 = time.perf_counter()
        done = oracle_calls(args.cpu_steps)
        dt = time.perf_counter() - t0
        # single thread: config 1 (512 x 512, g = 64, both rules at r in {8, 4, 2}) and one step of config 2
        with threadpool_limits(limits=1):
            c1 = synth.make_layer(cfg_id=1, tensor_id=0, n=512, k=512, m=1, group=64, x_dtype="f16")
            x1 = c1.x.double().numpy()
            t1 = time.perf_counter()
            for r in (8, 4, 2):
                for rule in (O.PREFIX, O.ROUND):
                    O.linear(x1, c1.q, c1.scales, c1.zeros, r, rule, 64)
            c1_s = time.perf_counter() - t1
            t2 = time.perf_counter()
            done1 = oracle_calls(1)
            st_dt = time.perf_counter() - t2
        cpu = {"value": round(done / dt / 1e9, 4), "unit": "GB/s", "cores": int(blas_threads), "kind": "oracle",
               "sample": f"oracle (numpy fp64 slice + dequant + matmul) on {args.cpu_steps} steps of the "
                         f"workload: gate, up and down at M=1 for r in {list(WIDTHS)} "
                         f"({15 * args.cpu_steps} calls), {dt:.1f} s; elementwise numpy on one thread, "
                         f"BLAS on {blas_threads}",
               "host_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
               "single_thread": {"config1_s_for_6_calls": round(c1_s, 4),
                                 "config2_GB/s": round(done1 / st_dt / 1e9, 4)}}
        log(f"[bench] cpu oracle: {cpu['value']} GB/s in {dt:.1f}s ({blas_threads} BLAS threads)")

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "llama3.1-8b-ffn decode: gate/up 4096->14336 + down 14336->4096, M=1, g=128, "
                               "true-prefix, r in {2,3,4,6,8}: the 15 calls of a step in one mq_linear_mixed call",
                   "global_batch": 1, "widths": list(WIDTHS), "ring_copies": ring},
        "timing": "hip_graph_replay",
        "roofline": roofline,
        "frac_hbm_per_r": {r: v["gate_up_down"]["frac_hbm"] for r, v in per_r.items()},
        "frac_hbm_step": round(value / HBM_PEAK_GBS, 4),
        "step_one_launch": step_launch,
        "prefill": prefill,
        "per_r": per_r,
        "attention": attn,
        "copy_reference": copy_ref,
        "producer": producer,
        "eager": eager,
        "skinny": skinny,
        "mixnmatch": mix,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
