"""Benchmark of the speculative-decoding verify hot path on one MI355X.

One step = one pass of the whole hot path over resident synthetic inputs:
  * verify qmv: the MLP block of a 5120-hidden decoder (gate and up
    5120 -> 17408, down 17408 -> 5120, W4 group 64) at every verify width
    M = 1..8.  Each M uses its own copy of the weights, so one step streams
    1.2 GB of distinct weights -- far beyond the 256 MB last-level cache --
    and nothing is served from cache across steps either.
  * verification: probability-ratio acceptance with residual / bonus draws
    for B = 256 sequences of depth D = 5 over a 151936-token vocabulary
    (fp32 logits, T = 0.6), i.e. 1536 verify positions.

Printed: one JSON line.  `value` is the verify qmv throughput in HBM GB/s
(algorithmic bytes / time of the qmv part of the steps); the acceptance
throughput (verify positions per second) and per-M figures ride along.
"""
from __future__ import annotations

import argparse
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of each oracle sample")
    return ap.parse_args()


def build_inputs(dev):
    """Packed W4 weights (packing is a load-time step, outside the timing)."""
    import torch
    import speculative_decoding_spec_amd as spec
    from speculative_decoding_spec_amd import synth

    def packed(N, K, seed):
        w, s, b = synth.torch_qweights(4, N, K, GROUP, seed, dev)
        return spec.spec_pack_w4(w, s, b, G=GROUP)

    blocks = []
    for i, M in enumerate(MS):
        gate = packed(FFN, HIDDEN, 1000 + 10 * i)
        up = packed(FFN, HIDDEN, 1001 + 10 * i)
        down = packed(HIDDEN, FFN, 1002 + 10 * i)
        x = synth.torch_activations(M, HIDDEN, 1003 + 10 * i, dev)
        h = synth.torch_activations(M, FFN, 1004 + 10 * i, dev)
        yg = torch.empty((M, FFN), dtype=torch.float32, device=dev)
        yu = torch.empty((M, FFN), dtype=torch.float32, device=dev)
        yd = torch.empty((M, HIDDEN), dtype=torch.float32, device=dev)
        blocks.append(dict(M=M, gate=gate, up=up, down=down, x=x, h=h, yg=yg, yu=yu, yd=yd))
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


def run_qmv(b):
    import speculative_decoding_spec_amd as spec
    spec.spec_qmv_w4(b["gate"], b["x"], y=b["yg"])
    spec.spec_qmv_w4(b["up"], b["x"], y=b["yu"])
    spec.spec_qmv_w4(b["down"], b["h"], y=b["yd"])


def run_accept(a):
    import speculative_decoding_spec_amd as spec
    spec.spec_verify_accept(a["t"], a["d"], a["toks"], a["u"], ACC_T,
                            out=(a["acc"], a["nxt"], None, None))


def cpu_baseline(seconds):
    """The fp64 oracle, as it stands, on a bounded sample of the workload.

    qmv: rows of the gate projection (M = 8, K = 5120) in chunks over the host
    threads until about `seconds` have passed; acceptance: sequences of the
    batched workload likewise.  Rates are scaled to GB/s (same algorithmic
    bytes as the GPU figure) and verify positions per second."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    from speculative_decoding_spec_amd import synth
    threads = min(16, os.cpu_count() or 1)
    M = 8
    w, s, b = synth.qweights(1, 4, FFN, HIDDEN, GROUP)
    x = synth.activations(1, M, HIDDEN)
    chunk = 64
    done, t0 = 0, time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        while done < FFN and time.perf_counter() - t0 < seconds:
            spans = [(r, min(FFN, r + chunk)) for r in range(done, min(FFN, done + chunk * threads), chunk)]
            list(ex.map(lambda sp: oracle.qmv(4, w, s, b, x, GROUP, rows=sp), spans))
            done = spans[-1][1]
    dt = time.perf_counter() - t0
    qbytes = done * (HIDDEN * 4 // 8 + (HIDDEN // GROUP) * 4) + M * HIDDEN * 2 + M * done * 4
    tl, dl = synth.logits_pair(4, threads, ACC_D, ACC_V)
    toks = np.zeros((threads, ACC_D), np.int32)
    u = synth.uniforms(4, synth.U_ACCEPT, (threads, ACC_D + 1))
    nseq, t1 = 0, time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        while nseq < ACC_B and time.perf_counter() - t1 < seconds:
            list(ex.map(lambda i: oracle.accept(tl[i:i + 1], dl[i:i + 1], toks[i:i + 1],
                                                u[i:i + 1], ACC_T), range(threads)))
            nseq += threads
    at = time.perf_counter() - t1
    return {
        "value": round(qbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": (f"W4 g64 qmv M=8 K=5120: {done} of the 17408 gate rows "
                   f"({qbytes / 1e6:.1f} MB algorithmic) in {dt:.1f} s; acceptance: "
                   f"{nseq} sequences of D=5 V=151936 T=0.6 in {at:.1f} s"),
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
    blocks = build_inputs(dev)
    acc = build_accept(dev)
    stream = torch.cuda.current_stream(dev)

    qmv_bytes_step = sum(roofline.qmv_bytes(4, b["M"], FFN, HIDDEN) * 2 +
                         roofline.qmv_bytes(4, b["M"], HIDDEN, FFN) for b in blocks)
    acc_bytes = roofline.accept_bytes(ACC_B, ACC_D, ACC_V)

    def step(events=None):
        for i, b in enumerate(blocks):
            if events is not None:
                events[i][0].record(stream)
            run_qmv(b)
            if events is not None:
                events[i][1].record(stream)
        if events is not None:
            events[-1][0].record(stream)
        run_accept(acc)
        if events is not None:
            events[-1][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(len(blocks) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per_m_ms = [sum(ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(args.steps)) / args.steps
                for i in range(len(blocks))]
    acc_ms = sum(ev[k][-1][0].elapsed_time(ev[k][-1][1]) for k in range(args.steps)) / args.steps
    qmv_ms = sum(per_m_ms)
    qmv_gbs = qmv_bytes_step / (qmv_ms * 1e-3) / 1e9
    per_m = {}
    for b, ms in zip(blocks, per_m_ms):
        nb = roofline.qmv_bytes(4, b["M"], FFN, HIDDEN) * 2 + roofline.qmv_bytes(4, b["M"], HIDDEN, FFN)
        per_m[str(b["M"])] = {"us": round(ms * 1e3, 2), "GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
                              "frac": round(nb / (ms * 1e-3) / roofline.HBM_PEAK_BYTES_PER_S, 4)}
    positions = ACC_B * (ACC_D + 1)
    acc_gbs = acc_bytes / (acc_ms * 1e-3) / 1e9
    accept = {"positions_per_s": positions / (acc_ms * 1e-3), "us": round(acc_ms * 1e3, 2),
              "GB/s": round(acc_gbs, 1), "frac": round(acc_gbs * 1e9 / roofline.HBM_PEAK_BYTES_PER_S, 4),
              "algorithmic_bytes": acc_bytes,
              "mean_accepted": float(acc["acc"].float().mean().item())}

    # Dominant kernel by time: report its roofline.
    if qmv_ms >= acc_ms:
        roof = {"kernel": "qmv_kernel<4> (all 24 launches of a step)", "bound": "hbm",
                "achieved": round(qmv_gbs, 1), "peak": 8000.0, "unit": "GB/s",
                "frac": round(qmv_gbs / 8000.0, 4), "traffic": None}
    else:
        roof = {"kernel": "row_stats_kernel + accept_kernel", "bound": "hbm",
                "achieved": round(acc_gbs, 1), "peak": 8000.0, "unit": "GB/s",
                "frac": round(acc_gbs / 8000.0, 4), "traffic": None}
    other = {"qmv": {"achieved": round(qmv_gbs, 1), "frac": round(qmv_gbs / 8000.0, 4)},
             "accept": {"achieved": round(acc_gbs, 1), "frac": round(acc_gbs / 8000.0, 4)}}

    out = {
        "metric": METRIC, "value": round(qmv_gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "w4-bf16xfp32 qmv; fp32 accept",
        "data": "synthetic (seeded, on-device generators)",
        "config": {"workload": ("verify MLP block W4 g64 (gate/up 5120->17408, down 17408->5120) "
                                "at M=1..8 on distinct weight copies + batched acceptance "
                                "B=256 D=5 V=151936 T=0.6"),
                   "qmv_bytes_per_step": qmv_bytes_step, "accept_bytes_per_step": acc_bytes},
        "qmv_frac_of_peak": round(qmv_gbs / 8000.0, 4),
        "per_M": per_m, "accept": accept, "roofline": roof, "roofline_parts": other,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
