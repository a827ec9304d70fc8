"""Benchmark of the speculative-decoding verify hot path on one MI355X.

One step = one pass of the whole hot path over resident synthetic inputs:
  * verify qmv: the MLP block of a 5120-hidden decoder (gate and up
    5120 -> 17408, down 17408 -> 5120, W4 group 64) at every verify width
    M = 1..8.  Gate and up share their input, so they are packed as one
    5120 -> 34816 matrix and computed by one launch (its outputs are bitwise
    those of two separate launches); down is a second launch.  Each M uses
    its own copy of the weights, so one step streams 1.2 GB of distinct
    weights -- far beyond the 256 MB last-level cache -- and nothing is
    served from cache across steps either.
  * verification: probability-ratio acceptance with residual / bonus draws
    for B = 256 sequences of depth D = 5 over a 151936-token vocabulary
    (fp32 logits, T = 0.6), i.e. 1536 verify positions.

Launches go through pre-marshalled calls (`bind_qmv`, `bind_verify_accept`),
so the host queues them far faster than the GPU runs them.  The same qmv
work with gate and up as separate launches is timed as well and reported
under `variants`.  (Replaying the step from a HIP graph measured slower than
these eager launches on this system -- 359 vs 322 us for the qmv part -- so
graphs are not used here; the library's calls are capture-safe all the same.)

Greedy verification (`bind_verify_greedy`: match the greedy draft's tokens
against the target's argmax, reading only the target logits) of the same
block is timed on its own after the steps and reported under
`accept_greedy`; it is not part of the step.

Printed: one JSON line.  `value` is the verify qmv throughput in HBM GB/s
(algorithmic bytes / time of the qmv part of the steps); the acceptance
throughput (verify positions per second) and per-M figures ride along.

`roofline` covers qmv_kernel, the kernel with the most time per step (16
launches): algorithmic bytes per launch over the average launch duration,
the qmv part of the timed steps (HIP events on the launch stream around the
16 back-to-back launches) divided by 16.  A second set of timed steps with
events around every launch splits the time by shape and M.  `traffic` is the HBM bytes per
launch from the committed counter summary under profiles/ (FETCH_SIZE +
WRITE_SIZE scaled by a plain-copy calibration), and null when qmv.hip or the
step's launches have changed since those counters were taken.

`--copy-probe` runs only a plain read-once / write-once elementwise kernel
over 1 GiB (the calibration kernel for those counters) and exits.
`--shapes` times qmv alone per layer shape and M (rotating >= 1.1 GB of
weight copies) plus an N sweep that splits a launch's time into a fixed
cost and an incremental bandwidth, prints one JSON line each, and exits.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

METRIC = ("verify qmv HBM GB/s (% of peak) at M=1..8; "
          "accept positions/sec @152k vocab")
HIDDEN, FFN = 5120, 17408
GROUP = 64
MS = list(range(1, 9))
ACC_B, ACC_D, ACC_V, ACC_T = 256, 5, 151936, 0.6
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qmv_kernel_w4_mlp_block_hbm_traffic.txt")
QMV_SOURCE = os.path.join(ROOT, "speculative_decoding_spec_amd", "csrc", "qmv.hip")
COPY_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of each oracle sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run the 1 GiB copy kernel used to calibrate HBM counters")
    ap.add_argument("--shapes", action="store_true",
                    help="only time qmv per layer shape and M (one JSON line each) and exit")
    return ap.parse_args()


# Layer shapes of the verify pass (N, K): a 5120-hidden decoder with 48 query
# and 8 key/value heads of 128, a 17408-wide MLP and a 151936-token head.
SHAPES = {
    "gate_up (fused 5120->34816)": (4, 2 * FFN, HIDDEN),
    "gate or up 5120->17408": (4, FFN, HIDDEN),
    "down 17408->5120": (4, HIDDEN, FFN),
    "q 5120->6144": (4, 6144, HIDDEN),
    "k or v 5120->1024": (4, 1024, HIDDEN),
    "qkv (fused 5120->8192)": (4, 8192, HIDDEN),
    "o 6144->5120": (4, HIDDEN, 6144),
    "lm_head 5120->151936": (4, 151936, HIDDEN),
    "gate or up W8": (8, FFN, HIDDEN),
    "down W8": (8, HIDDEN, FFN),
    "lm_head W8": (8, 151936, HIDDEN),
}
# N sweep at K = 5120, M = 1: time per launch against bytes per launch.
SWEEP_N = [2176, 4352, 8704, 17408, 34816, 69632]


def shapes(dev, steps):
    """Microseconds per launch of qmv at each layer shape and M = 1, 4, 8, 16:
    back-to-back launches over enough weight copies (at least 1.1 GB) that
    nothing is served from the 256 MB last-level cache; then a least-squares
    line through the N sweep, whose slope is the incremental bandwidth and
    whose intercept the fixed cost of one launch."""
    import torch
    import speculative_decoding_spec_amd as spec
    from speculative_decoding_spec_amd import roofline, synth

    def timed(bits, N, K, Ms):
        nb1 = roofline.qmv_bytes(bits, 1, N, K)
        nc = min(400, max(2, -(-int(1.1e9) // nb1)))
        pk = spec.spec_pack_w4 if bits == 4 else spec.spec_pack_w8
        copies = [pk(*synth.torch_qweights(bits, N, K, GROUP, 5000 + c, dev), G=GROUP)
                  for c in range(nc)]
        res = {}
        for M in Ms:
            x = synth.torch_activations(M, K, 5100 + M, dev)
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
            calls = [spec.bind_qmv(w, x, y) for w in copies]
            reps = max(steps * 3, 2 * nc)
            for c in calls:      # touch every copy once before timing
                c()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(reps):
                calls[i % nc]()
            e1.record()
            torch.cuda.synchronize()
            res[M] = (e0.elapsed_time(e1) * 1e3 / reps, roofline.qmv_bytes(bits, M, N, K), nc)
        del copies
        torch.cuda.empty_cache()
        return res

    for name, (bits, N, K) in SHAPES.items():
        for M, (us, nb, nc) in timed(bits, N, K, (1, 4, 8, 16)).items():
            print(json.dumps({"shape": name, "bits": bits, "N": N, "K": K, "M": M,
                              "us_per_launch": round(us, 2), "GB/s": round(nb / us / 1e3, 1),
                              "frac": round(nb / us / 1e3 / 8000.0, 4), "weight_copies": nc}),
                  flush=True)
    xs, ys = [], []
    for N in SWEEP_N:
        us, nb, _ = timed(4, N, HIDDEN, (1,))[1]
        xs.append(nb)
        ys.append(us)
        print(json.dumps({"sweep": "W4 K=5120 M=1", "N": N, "bytes": nb,
                          "us_per_launch": round(us, 2)}), flush=True)
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    slope = sum((a - mx) * (b - my) for a, b in zip(xs, ys)) / sum((a - mx) ** 2 for a in xs)
    icpt = my - slope * mx
    print(json.dumps({"fit": "us = intercept + bytes / rate over the N sweep",
                      "intercept_us": round(icpt, 2),
                      "incremental_GB/s": round(1e-3 / slope, 1),
                      "incremental_frac": round(1e-3 / slope / 8000.0, 4)}), flush=True)


def copy_probe(dev):
    """A plain elementwise kernel that reads COPY_BYTES once and writes them once."""
    import torch
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_BYTES, "launches": 3}), flush=True)


def measured_traffic(bytes_per_launch):
    """HBM bytes per qmv launch from the committed counter summary, or None
    when the summary is missing, belongs to another qmv.hip, or was taken on
    another mix of launches (other algorithmic bytes per launch)."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        with open(QMV_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
        if kv.get("source_sha256") != sha:
            return None, "qmv.hip changed since the counters were taken"
        if int(kv.get("algorithmic_bytes_per_launch", -1)) != round(bytes_per_launch):
            return None, "the step's launches changed since the counters were taken"
        return float(kv["traffic_bytes_per_launch"]), kv
    except (OSError, KeyError, ValueError):
        return None, "no counter summary"


def build_inputs(dev):
    """Packed W4 weights (packing is a load-time step, outside the timing):
    per M, the fused gate/up matrix, the down matrix, and gate and up packed
    separately (for the unfused comparison)."""
    import torch
    import speculative_decoding_spec_amd as spec
    from speculative_decoding_spec_amd import synth

    blocks = []
    for i, M in enumerate(MS):
        g = synth.torch_qweights(4, FFN, HIDDEN, GROUP, 1000 + 10 * i, dev)
        u = synth.torch_qweights(4, FFN, HIDDEN, GROUP, 1001 + 10 * i, dev)
        d = synth.torch_qweights(4, HIDDEN, FFN, GROUP, 1002 + 10 * i, dev)
        gate_up = spec.spec_pack_w4(*[torch.cat([a, b]) for a, b in zip(g, u)], G=GROUP)
        gate, up = spec.spec_pack_w4(*g, G=GROUP), spec.spec_pack_w4(*u, G=GROUP)
        down = spec.spec_pack_w4(*d, G=GROUP)
        del g, u, d
        x = synth.torch_activations(M, HIDDEN, 1003 + 10 * i, dev)
        h = synth.torch_activations(M, FFN, 1004 + 10 * i, dev)
        ygu = torch.empty((M, 2 * FFN), dtype=torch.float32, device=dev)
        yg = torch.empty((M, FFN), dtype=torch.float32, device=dev)
        yu = torch.empty((M, FFN), dtype=torch.float32, device=dev)
        yd = torch.empty((M, HIDDEN), dtype=torch.float32, device=dev)
        blocks.append(dict(M=M, gate_up=gate_up, gate=gate, up=up, down=down, x=x, h=h,
                           ygu=ygu, yg=yg, yu=yu, yd=yd))
    torch.cuda.synchronize()
    return blocks


def build_accept(dev):
    import torch
    import speculative_decoding_spec_amd as spec
    from speculative_decoding_spec_amd import synth
    t, d = synth.torch_logits_pair(ACC_B, ACC_D, ACC_V, 4242, dev)
    ud = synth.torch_uniforms((ACC_B * ACC_D,), 4243, dev)
    # Drafts are drawn from the draft distributions (the draft side of the
    # cycle), so acceptance rates are those of the rule, not of random tokens.
    toks = spec.spec_sample_tokens(d.view(ACC_B * ACC_D, ACC_V), ud, ACC_T).view(ACC_B, ACC_D)
    u = synth.torch_uniforms((ACC_B, ACC_D + 1), 4244, dev)
    acc = torch.empty(ACC_B, dtype=torch.int32, device=dev)
    nxt = torch.empty(ACC_B, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    return dict(t=t, d=d, toks=toks.contiguous(), u=u, acc=acc, nxt=nxt)


def run_accept(a):
    import speculative_decoding_spec_amd as spec
    spec.spec_verify_accept(a["t"], a["d"], a["toks"], a["u"], ACC_T,
                            out=(a["acc"], a["nxt"], None, None))


def cpu_baseline(seconds):
    """The fp64 oracle, as it stands, on a bounded sample of the step.

    qmv: the step's 24 products (gate, up and down at M = 1..8) with one
    seeded weight set per shape, rows split over the host threads, stopping
    once `seconds` have passed; acceptance: the 256-sequence batch, drafts
    drawn from the draft rows as on the GPU, likewise bounded.  Rates use the
    GPU figure's algorithmic bytes (GB/s) and verify positions per second."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    from speculative_decoding_spec_amd import roofline, synth
    threads = min(16, os.cpu_count() or 1)
    shapes = {"gate_up": (FFN, HIDDEN), "down": (HIDDEN, FFN)}
    weights = {k: synth.qweights(1, 4, N, K, GROUP, salt=N) for k, (N, K) in shapes.items()}
    work = []
    for M in MS:
        for name in ("gate_up", "gate_up", "down"):
            work.append((name, M))
    chunk = 256
    done_bytes, products, t0 = 0, 0, time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        for name, M in work:
            if time.perf_counter() - t0 >= seconds:
                break
            N, K = shapes[name]
            w, s, b = weights[name]
            x = synth.activations(1, M, K, salt=M)
            spans = [(r, min(N, r + chunk)) for r in range(0, N, chunk)]
            list(ex.map(lambda sp: oracle.qmv(4, w, s, b, x, GROUP, rows=sp), spans))
            done_bytes += roofline.qmv_bytes(4, M, N, K, GROUP)
            products += 1
    dt = time.perf_counter() - t0
    tl, dl = synth.logits_pair(4, ACC_B, ACC_D, ACC_V)
    ud = synth.uniforms(4, synth.U_DRAFT, ACC_B * ACC_D)
    toks = oracle.sample_rows(dl.reshape(ACC_B * ACC_D, ACC_V), ACC_T, 0, 1.0, ud).reshape(ACC_B, ACC_D)
    u = synth.uniforms(4, synth.U_ACCEPT, (ACC_B, ACC_D + 1))
    nseq, t1 = 0, time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        while nseq < ACC_B and time.perf_counter() - t1 < seconds:
            idx = range(nseq, min(ACC_B, nseq + threads))
            list(ex.map(lambda i: oracle.accept(tl[i:i + 1], dl[i:i + 1], toks[i:i + 1],
                                                u[i:i + 1], ACC_T), idx))
            nseq = idx[-1] + 1
    at = time.perf_counter() - t1
    return {
        "value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": (f"W4 g64 qmv: {products} of the step's 24 products (gate/up 5120->17408, "
                   f"down 17408->5120, M=1..8), {done_bytes / 1e6:.0f} MB algorithmic in {dt:.1f} s; "
                   f"acceptance: {nseq} of 256 sequences (D=5, V=151936, T=0.6) in {at:.2f} s"),
        "accept_positions_per_s": round(nseq * (ACC_D + 1) / at, 1),
        "cpu": platform.processor() or platform.machine(),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; "
                          f"--gpus {args.gpus} is not supported (use --gpus 1)"}))
        sys.exit(2)
    import torch
    import speculative_decoding_spec_amd as spec
    from speculative_decoding_spec_amd import roofline

    if not os.path.exists(spec.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    dev = torch.device("cuda:0")
    if args.copy_probe:
        copy_probe(dev)
        return
    if args.shapes:
        shapes(dev, args.steps)
        return
    blocks = build_inputs(dev)
    acc = build_accept(dev)
    stream = torch.cuda.current_stream(dev)

    acc_bytes = roofline.accept_bytes(ACC_B, ACC_D, ACC_V)

    def pair():
        return (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))

    def fused_launches():
        """(bound call, shape name, algorithmic bytes) of the 16 launches."""
        out = []
        for b in blocks:
            out.append((spec.bind_qmv(b["gate_up"], b["x"], b["ygu"]), "gate_up",
                        roofline.qmv_bytes(4, b["M"], 2 * FFN, HIDDEN)))
            out.append((spec.bind_qmv(b["down"], b["h"], b["yd"]), "down",
                        roofline.qmv_bytes(4, b["M"], HIDDEN, FFN)))
        return out

    def unfused_launches():
        out = []
        for b in blocks:
            out.append((spec.bind_qmv(b["gate"], b["x"], b["yg"]), "gate",
                        roofline.qmv_bytes(4, b["M"], FFN, HIDDEN)))
            out.append((spec.bind_qmv(b["up"], b["x"], b["yu"]), "up",
                        roofline.qmv_bytes(4, b["M"], FFN, HIDDEN)))
            out.append((spec.bind_qmv(b["down"], b["h"], b["yd"]), "down",
                        roofline.qmv_bytes(4, b["M"], HIDDEN, FFN)))
        return out

    launches = fused_launches()
    unfused = unfused_launches()
    accept_call = spec.bind_verify_accept(acc["t"], acc["d"], acc["toks"], acc["u"], ACC_T,
                                          out=(acc["acc"], acc["nxt"], None, None))
    qmv_bytes_step = sum(l[2] for l in launches)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev["q"][0].record(stream)
        for call, _, _ in launches:
            call()
        if ev is not None:
            ev["q"][1].record(stream)
            ev["a"][0].record(stream)
        accept_call()
        if ev is not None:
            ev["a"][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed steps: events around the qmv part and the acceptance call.
    ev = [{"q": pair(), "a": pair()} for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    qspan_ms = sum(e["q"][0].elapsed_time(e["q"][1]) for e in ev) / args.steps
    acc_ms = sum(e["a"][0].elapsed_time(e["a"][1]) for e in ev) / args.steps
    qmv_gbs = qmv_bytes_step / (qspan_ms * 1e-3) / 1e9

    def eager(calls, per_launch):
        """K eager steps of `calls`: the span of each step and, if asked, the
        duration of every launch (events around it)."""
        evs = [(pair(), [pair() for _ in calls]) for _ in range(args.steps)]
        accept_call()          # untimed: the queue is busy at the first event
        for span, each in evs:
            span[0].record(stream)
            for i, (call, _, _) in enumerate(calls):
                if per_launch:
                    each[i][0].record(stream)
                call()
                if per_launch:
                    each[i][1].record(stream)
            span[1].record(stream)
            accept_call()
        torch.cuda.synchronize()
        span_ms = sum(s[0].elapsed_time(s[1]) for s, _ in evs) / args.steps
        each_ms = ([sum(e[i][0].elapsed_time(e[i][1]) for _, e in evs) / args.steps
                    for i in range(len(calls))] if per_launch else None)
        return span_ms, each_ms

    # Greedy verification of the same block (target logits only), drafts
    # from the greedy draft (argmax of each draft row).
    g_toks = torch.argmax(acc["d"], dim=2).to(torch.int32).contiguous()
    g_out = (torch.empty(ACC_B, dtype=torch.int32, device=dev),
             torch.empty(ACC_B, dtype=torch.int32, device=dev))
    greedy_call = spec.bind_verify_greedy(acc["t"], g_toks, out=g_out)
    for _ in range(args.warmup):
        greedy_call()
    g_ev = [pair() for _ in range(args.steps)]
    for e in g_ev:
        e[0].record(stream)
        greedy_call()
        e[1].record(stream)
    torch.cuda.synchronize()
    g_ms = sum(e[0].elapsed_time(e[1]) for e in g_ev) / args.steps
    g_bytes = roofline.greedy_bytes(ACC_B, ACC_D, ACC_V)

    eager_unfused_ms, _ = eager(unfused, False)
    _, q_ms = eager(launches, True)
    per_m = {}
    for j, b in enumerate(blocks):
        ms = sum(q_ms[2 * j:2 * j + 2])
        nb = sum(l[2] for l in launches[2 * j:2 * j + 2])
        per_m[str(b["M"])] = {"us": round(ms * 1e3, 2), "GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
                              "frac": round(nb / (ms * 1e-3) / roofline.HBM_PEAK_BYTES_PER_S, 4)}
    per_shape = {}
    for name in ("gate_up", "down"):
        idx = [i for i, l in enumerate(launches) if l[1] == name]
        ms = sum(q_ms[i] for i in idx) / len(idx)
        nb = sum(launches[i][2] for i in idx) / len(idx)
        per_shape[name] = {"us_per_launch": round(ms * 1e3, 2),
                           "GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
                           "frac": round(nb / (ms * 1e-3) / roofline.HBM_PEAK_BYTES_PER_S, 4)}
    unfused_bytes = sum(l[2] for l in unfused)
    variants = {
        "fused gate/up, 16 launches (value)": {"qmv_us_per_step": round(qspan_ms * 1e3, 2),
                                               "GB/s": round(qmv_gbs, 1)},
        "separate gate and up, 24 launches": {"qmv_us_per_step": round(eager_unfused_ms * 1e3, 2),
                                              "GB/s": round(unfused_bytes / (eager_unfused_ms * 1e-3) / 1e9, 1)},
    }
    positions = ACC_B * (ACC_D + 1)
    acc_gbs = acc_bytes / (acc_ms * 1e-3) / 1e9
    accept = {"positions_per_s": round(positions / (acc_ms * 1e-3), 1), "us": round(acc_ms * 1e3, 2),
              "GB/s": round(acc_gbs, 1), "frac": round(acc_gbs * 1e9 / roofline.HBM_PEAK_BYTES_PER_S, 4),
              "algorithmic_bytes": acc_bytes,
              "mean_accepted": float(acc["acc"].float().mean().item())}

    greedy = {"positions_per_s": round(positions / (g_ms * 1e-3), 1), "us": round(g_ms * 1e3, 2),
              "GB/s": round(g_bytes / (g_ms * 1e-3) / 1e9, 1),
              "frac": round(g_bytes / (g_ms * 1e-3) / roofline.HBM_PEAK_BYTES_PER_S, 4),
              "algorithmic_bytes": g_bytes,
              "mean_accepted": float(g_out[0].float().mean().item())}

    # Roofline of qmv_kernel: algorithmic bytes per launch over the average
    # launch duration, i.e. the qmv part of a step (16 launches back to back,
    # no events between them) divided by 16.  The per-launch events of the
    # second set of steps add about 2 us of marker time to each launch, so
    # they only split the time by shape.
    bytes_per_launch = qmv_bytes_step / len(launches)
    launch_us = qspan_ms / len(launches) * 1e3
    achieved = bytes_per_launch / (launch_us * 1e-6) / 1e9
    traffic, tinfo = measured_traffic(bytes_per_launch)
    roof = {"kernel": "qmv_kernel (W4; 16 launches per step: fused gate/up and down at M=1..8)",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": 8000.0, "unit": "GB/s",
            "frac": round(achieved / 8000.0, 4),
            "traffic": None if traffic is None else round(traffic),
            "algorithmic_bytes_per_launch": round(bytes_per_launch),
            "avg_launch_us": round(launch_us, 2),
            "traffic_source": (os.path.relpath(TRAFFIC_FILE, ROOT) if traffic is not None else tinfo)}
    other = {"qmv_kernel": {"achieved": round(achieved, 1), "frac": round(achieved / 8000.0, 4),
                            "per_shape (per-launch events)": per_shape},
             "accept (row_chunk + draw_sums + draw_final)": {
                 "achieved": round(acc_gbs, 1), "frac": round(acc_gbs / 8000.0, 4),
                 "us_per_call": round(acc_ms * 1e3, 2)}}

    out = {
        "metric": METRIC, "value": round(qmv_gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "w4-bf16xfp32 qmv; fp32 accept",
        "data": "synthetic (seeded, on-device generators)",
        "config": {"workload": ("verify MLP block W4 g64 (gate/up 5120->17408 packed as one "
                                "5120->34816 launch, down 17408->5120) at M=1..8 on distinct "
                                "weight copies + batched acceptance B=256 D=5 V=151936 T=0.6"),
                   "qmv_bytes_per_step": qmv_bytes_step, "accept_bytes_per_step": acc_bytes},
        "qmv_frac_of_peak": round(qmv_gbs / 8000.0, 4),
        "qmv_us_per_step": round(qspan_ms * 1e3, 2), "variants": variants,
        "per_M (per-launch events)": per_m, "accept": accept,
        "accept_greedy (same block, target logits only; not part of the step)": greedy,
        "roofline": roof, "roofline_parts": other,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
