"""Benchmark of the speculative-decoding verify hot path on one MI355X.

One step = one pass of the whole hot path over resident synthetic inputs:
  * verify qmv: the MLP block of a 5120-hidden decoder (gate and up
    5120 -> 17408, down 17408 -> 5120, W4 group 64) at every verify width
    M = 1..8, chained as the model runs it: gate and up share their input,
    so they stream as one launch that also applies the SiLU-gated
    activation and writes h = bf16(silu(g) * u); the down projection reads
    that h.  Two launches per M, 16 per step.  Each M uses its own copy of
    the weights, so one step streams 1.2 GB of distinct weights -- far
    beyond the 256 MB last-level cache -- and nothing is served from cache
    across steps either.
  * verification: probability-ratio acceptance with residual / bonus draws
    for B = 256 sequences of depth D = 5 over a 151936-token vocabulary
    (fp32 logits, T = 0.6), i.e. 1536 verify positions.

Launches go through pre-marshalled calls (`bind_qmv_gate_up_silu`,
`bind_qmv`, `bind_verify_accept`), so the host queues them far faster than
the GPU runs them.  HIP events on the launch stream bracket the qmv part and
the acceptance call of every timed step; `value` and the acceptance figures
come from the median step, with p10 and p90 beside them.

Printed: one JSON line.  `value` is the verify qmv throughput in HBM GB/s
(algorithmic bytes of the 16 launches / the median time of the qmv part).
Beside it, after the timed steps (none of it inside the steps):
  * `variants`: the same MLP weights read as stored (spec_qmv_w4 on the
    interchange layout, gate/up fused into one fp32 launch), as one plain
    gate/up launch from the packed copy, and as 24 separate launches;
  * `per_M`: the step's time split by M (events around each launch);
  * `configs`: every other workload of the verify hot path --
      pr1_reference   W4 g64 qmv M=4 K=1024 N=4096 and acceptance B=1 D=3
                      V=32768 T=0.6 (latency, us);
      lm_head_accept  the W4 LM head 5120->151936 at M=6, then acceptance of
                      its logits with top-k 20 / top-p 0.95 (B=1, D=5);
      w8_lm_head      the W8 g64 LM head at M=8;
      verify_pass_64_layers  the projections of a 64-layer 5120-hidden
                      decoder (12.3 GB of W4 weights) at M=3..6, four
                      launches per layer as the model runs them;
  * `accept_greedy`: greedy verification of the step's block (target logits
    only);
  * `stream_read`: a plain streaming read of 2 GiB (`spec_stream_read`), of
    which `qmv_frac_of_stream` and `accept.frac_of_stream` are the shares;
  * `cpu_baseline`: the fp64 oracle on the host, all threads and one.

`roofline` covers qmv_kernel, the kernel with the most time per step (16
launches): algorithmic bytes per launch over the average launch duration,
i.e. the median qmv part of a step divided by 16.  `traffic` is the HBM
bytes per launch from the committed counter summary under profiles/
(FETCH_SIZE + WRITE_SIZE scaled by a plain-copy calibration), and null when
qmv.hip or the step's launches have changed since those counters were taken.

`--step-only` times the steps alone (no variants, configs or CPU baseline):
the form the counter runs use.
`--copy-probe` runs only a plain read-once / write-once elementwise kernel
over 1 GiB (the calibration kernel for those counters) and exits.
`--lmhead`, `--depth` (also as 7 separate launches per layer), `--draft`,
`--gdn` and `--shapes` time one part each and print one JSON line (per
shape for `--shapes`, with an N sweep that splits a launch's time into a
fixed cost and an incremental bandwidth), and exit.
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
PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="target CPU time of each oracle sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run the 1 GiB copy kernel used to calibrate HBM counters")
    ap.add_argument("--step-only", action="store_true",
                    help="time the steps only (no variants, configs or CPU baseline)")
    ap.add_argument("--lmhead", action="store_true",
                    help="only time the LM head at M=6 plus acceptance with top-k/top-p (B=1) and exit")
    ap.add_argument("--depth", action="store_true",
                    help="only time the verify pass of a 64-layer decoder at M=3..6 and exit")
    ap.add_argument("--draft", action="store_true",
                    help="only time the draft step (4-bit LM head copy + sampling) and exit")
    ap.add_argument("--gdn", action="store_true",
                    help="only time the recurrent-state capture and commit and exit")
    ap.add_argument("--shapes", action="store_true",
                    help="only time qmv per layer shape and M (one JSON line each) and exit")
    ap.add_argument("--valu", action="store_true",
                    help="only time the chained MLP block at M=1..4 on the vector ALU against MFMA and exit")
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


def pct(values):
    """(median, p10, p90) of a list."""
    import numpy as np
    a = np.asarray(values, dtype=np.float64)
    return float(np.median(a)), float(np.percentile(a, 10)), float(np.percentile(a, 90))


def spread_us(values_us):
    med, p10, p90 = pct(values_us)
    return {"us": round(med, 2), "p10_us": round(p10, 2), "p90_us": round(p90, 2)}


def rate(nbytes, us):
    gbs = nbytes / us / 1e3
    return {"GB/s": round(gbs, 1), "frac": round(gbs / PEAK_GBS, 4)}


def timed_each(calls, reps, stream):
    """Microseconds of each of `reps` back-to-back calls (cycling through
    `calls`), with HIP events on `stream` around every call."""
    import torch
    for c in calls:
        c()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        calls[i % len(calls)]()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in ev]


def pr1_reference(dev, steps):
    """The smallest workload: W4 g64 qmv at M=4, K=1024, N=4096 (read as
    stored and from the packed copy) and acceptance of B=1, D=3 over a
    32768-token vocabulary at T=0.6.  Latency-bound, so reported in us."""
    import torch
    import speculative_decoding_spec_amd as spec
    from speculative_decoding_spec_amd import roofline, synth
    stream = torch.cuda.current_stream(dev)
    M, N, K = 4, 4096, 1024
    raw = [synth.torch_qweights(4, N, K, GROUP, 8600 + c, dev) for c in range(64)]
    x = synth.torch_activations(M, K, 8690, dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    # 64 weight copies (155 MB) so the launches do not stream from cache
    packed = [spec.bind_qmv(spec.spec_pack_w4(*r, G=GROUP), x, y) for r in raw]
    inter = [spec.bind_qmv(spec.QWeights(4, *r, G=GROUP), x, y) for r in raw]
    B, D, V = 1, 3, 32768
    t, d = synth.torch_logits_pair(B, D, V, 8691, dev)
    toks = spec.spec_sample_tokens(d.view(B * D, V), synth.torch_uniforms((B * D,), 8692, dev),
                                   ACC_T).view(B, D).contiguous()
    u = synth.torch_uniforms((B, D + 1), 8693, dev)
    out = (torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev),
           None, None)
    accept = spec.bind_verify_accept(t, d, toks, u, ACC_T, out=out)
    qb = roofline.qmv_bytes(4, M, N, K)
    ab = roofline.accept_bytes(B, D, V)
    # one untimed round of both first: the first launches after the copies
    # are allocated and packed ran up to twice as long in some runs
    timed_each(packed + inter, steps, stream)
    pk = spread_us(timed_each(packed, steps, stream))
    it = spread_us(timed_each(inter, steps, stream))
    ac = spread_us(timed_each([accept], steps, stream))
    return {"workload": "W4 g64 qmv M=4 K=1024 N=4096; acceptance B=1 D=3 V=32768 T=0.6",
            "qmv_packed": {**pk, **rate(qb, pk["us"])},
            "qmv_interchange": {**it, **rate(qb, it["us"])},
            "accept": {**ac, **rate(ab, ac["us"]), "positions_per_s": round(B * (D + 1) / ac["us"] * 1e6, 1)},
            "algorithmic_bytes": {"qmv": qb, "accept": ab}}


def lmhead_accept(dev, steps):
    """The end of a verify pass for one sequence at depth D = 5: the W4 LM
    head at M = 6 writes the target logits, and the acceptance (T = 0.6,
    top-k 20, top-p 0.95) runs on them; the draft logits are the target's
    minus N(0, 0.5) noise and the drafts are drawn from them.  Head copies
    rotate beyond the last-level cache."""
    import torch
    import speculative_decoding_spec_amd as spec
    from speculative_decoding_spec_amd import roofline, synth
    stream = torch.cuda.current_stream(dev)
    V, K, D = 151936, HIDDEN, 5
    heads = [spec.spec_pack_w4(*synth.torch_qweights(4, V, K, GROUP, 8400 + c, dev), G=GROUP)
             for c in range(3)]
    x = synth.torch_activations(D + 1, K, 8410, dev)
    logits = torch.empty((D + 1, V), dtype=torch.float32, device=dev)
    spec.spec_qmv_w4_packed(heads[0], x, logits)
    g = torch.Generator(device=dev)
    g.manual_seed(8411)
    draft = (logits[:D] - torch.randn((D, V), generator=g, device=dev) * 0.5).contiguous()
    ud = synth.torch_uniforms((D,), 8412, dev)
    toks = spec.spec_sample_tokens(draft, ud, ACC_T, 20, 0.95).view(1, D).contiguous()
    u = synth.torch_uniforms((1, D + 1), 8413, dev)
    out = (torch.empty(1, dtype=torch.int32, device=dev), torch.empty(1, dtype=torch.int32, device=dev),
           None, None)
    accept = spec.bind_verify_accept(logits.view(1, D + 1, V), draft.view(1, D, V), toks, u, ACC_T,
                                     20, 0.95, out=out)
    calls = [spec.bind_qmv(h, x, logits) for h in heads]
    head = spread_us(timed_each(calls, steps, stream))
    acc = spread_us(timed_each([accept], steps, stream))
    nb = roofline.qmv_bytes(4, D + 1, V, K)
    return {"workload": ("W4 g64 LM head 5120->151936 at M=6, then acceptance of D=5 drafts "
                         "(T=0.6, top-k 20, top-p 0.95) for one sequence"),
            "head": {**head, **rate(nb, head["us"]), "algorithmic_bytes": nb},
            "accept": acc,
            "accepted_len": int(out[0].item()), "next_token": int(out[1].item())}


def w8_lm_head(dev, steps):
    """The W8 g64 LM head 5120->151936 at M=8 (two copies, 1.66 GB)."""
    import torch
    import speculative_decoding_spec_amd as spec
    from speculative_decoding_spec_amd import roofline, synth
    stream = torch.cuda.current_stream(dev)
    V, K, M = 151936, HIDDEN, 8
    heads = [spec.spec_pack_w8(*synth.torch_qweights(8, V, K, GROUP, 8500 + c, dev), G=GROUP)
             for c in range(2)]
    x = synth.torch_activations(M, K, 8510, dev)
    y = torch.empty((M, V), dtype=torch.float32, device=dev)
    t = spread_us(timed_each([spec.bind_qmv(h, x, y) for h in heads], steps, stream))
    nb = roofline.qmv_bytes(8, M, V, K)
    return {"workload": "W8 g64 LM head 5120->151936 at M=8", **t, **rate(nb, t["us"]),
            "algorithmic_bytes": nb}


DEPTH_LAYERS, Q_N, KV_N, O_K = 64, 6144, 1024, 6144


def verify_pass(dev, steps, Ms=(3, 4, 5, 6), separate=False):
    """The linear projections of a whole verify pass: 64 decoder layers of
    q 5120->6144, k and v 5120->1024, o 6144->5120, gate and up
    5120->17408, down 17408->5120, all W4 g64 with each layer's own weights
    (12.3 GB), at M = 3..6 (depths D2..D5).  Streamed as the model runs it:
    q, k and v as one launch (they share x), o, gate/up with the gated
    activation, and down on that activation, 4 launches per layer; with
    `separate`, also the same weights as 7 separate launches per layer."""
    import torch
    import speculative_decoding_spec_amd as spec
    from speculative_decoding_spec_amd import roofline, synth
    stream = torch.cuda.current_stream(dev)
    fused, sep = [], []
    for li in range(DEPTH_LAYERS):
        sd = 9000 + 10 * li
        q = synth.torch_qweights(4, Q_N, HIDDEN, GROUP, sd, dev)
        k = synth.torch_qweights(4, KV_N, HIDDEN, GROUP, sd + 1, dev)
        v = synth.torch_qweights(4, KV_N, HIDDEN, GROUP, sd + 2, dev)
        o = synth.torch_qweights(4, HIDDEN, O_K, GROUP, sd + 3, dev)
        g = synth.torch_qweights(4, FFN, HIDDEN, GROUP, sd + 4, dev)
        u = synth.torch_qweights(4, FFN, HIDDEN, GROUP, sd + 5, dev)
        d = synth.torch_qweights(4, HIDDEN, FFN, GROUP, sd + 6, dev)
        qkv = spec.spec_pack_w4(*[torch.cat(t) for t in zip(q, k, v)], G=GROUP)
        po, pd = spec.spec_pack_w4(*o, G=GROUP), spec.spec_pack_w4(*d, G=GROUP)
        fused.append((qkv, po, spec.spec_pack_gate_up(4, g, u, G=GROUP), pd))
        if separate:
            sep.append(tuple(spec.spec_pack_w4(*t, G=GROUP) for t in (q, k, v, o, g, u, d)))
        del q, k, v, o, g, u, d
    torch.cuda.synchronize()
    res = {}
    for M in Ms:
        x = synth.torch_activations(M, HIDDEN, 9500 + M, dev)
        a = synth.torch_activations(M, O_K, 9510 + M, dev)          # attention output
        yqkv = torch.empty((M, Q_N + 2 * KV_N), device=dev)
        yo = torch.empty((M, HIDDEN), device=dev)
        h = torch.empty((M, FFN), dtype=torch.bfloat16, device=dev)
        yd = torch.empty((M, HIDDEN), device=dev)
        f_calls, f_bytes = [], 0
        for (qkv, po, glu, pd) in fused:
            f_calls += [spec.bind_qmv(qkv, x, yqkv), spec.bind_qmv(po, a, yo),
                        spec.bind_qmv_gate_up_silu(glu, x, h), spec.bind_qmv(pd, h, yd)]
            f_bytes += (roofline.qmv_bytes(4, M, Q_N + 2 * KV_N, HIDDEN)
                        + roofline.qmv_bytes(4, M, HIDDEN, O_K)
                        + roofline.gate_up_silu_bytes(4, M, FFN, HIDDEN)
                        + roofline.qmv_bytes(4, M, HIDDEN, FFN))

        def pass_us(calls):
            """Microseconds of each of `steps` whole passes (events around each)."""
            for c in calls:
                c()
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
            for e0, e1 in ev:
                e0.record(stream)
                for c in calls:
                    c()
                e1.record(stream)
            torch.cuda.synchronize()
            return [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]

        fu = spread_us(pass_us(f_calls))
        res[str(M)] = {"fused_4_launches_per_layer": {**fu, "bytes": f_bytes, **rate(f_bytes, fu["us"])}}
        if separate:
            yq = torch.empty((M, Q_N), device=dev)
            ykv = torch.empty((M, KV_N), device=dev)
            yg = torch.empty((M, FFN), device=dev)
            s_calls, s_bytes = [], 0
            for (q, k, v, o, g, u, d) in sep:
                s_calls += [spec.bind_qmv(q, x, yq), spec.bind_qmv(k, x, ykv), spec.bind_qmv(v, x, ykv),
                            spec.bind_qmv(o, a, yo), spec.bind_qmv(g, x, yg), spec.bind_qmv(u, x, yg),
                            spec.bind_qmv(d, h, yd)]
                s_bytes += (roofline.qmv_bytes(4, M, Q_N, HIDDEN) + 2 * roofline.qmv_bytes(4, M, KV_N, HIDDEN)
                            + roofline.qmv_bytes(4, M, HIDDEN, O_K) + 2 * roofline.qmv_bytes(4, M, FFN, HIDDEN)
                            + roofline.qmv_bytes(4, M, HIDDEN, FFN))
            su = spread_us(pass_us(s_calls))
            res[str(M)]["separate_7_launches_per_layer"] = {**su, "bytes": s_bytes, **rate(s_bytes, su["us"])}
    del fused, sep
    torch.cuda.empty_cache()
    return {"workload": (f"verify-pass projections of a {DEPTH_LAYERS}-layer 5120-hidden decoder, "
                         "W4 g64, each layer its own weights, per M"), "per_M": res}


def draft(dev, steps):
    """The draft side of a cycle (one drafted token): the LM head at M = 1,
    then one draw from its distribution (T = 0.6).  The draft-only 4-bit head
    is built from a bf16 head by spec_requantize_w4 (a load-time step, timed
    once); the comparison keeps the head at 8 bits, standing in for the
    target's model-precision head.  Weight copies rotate so that nothing is
    served from the 256 MB last-level cache."""
    import torch
    import speculative_decoding_spec_amd as spec
    from speculative_decoding_spec_amd import roofline, synth
    V, K = 151936, HIDDEN
    g = torch.Generator(device=dev)
    g.manual_seed(8100)
    heads4 = []
    req_us = None
    for c in range(3):
        w = (torch.randn((V, K), generator=g, device=dev) * 0.02).to(torch.bfloat16)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        q4 = spec.spec_requantize_w4(w)
        e1.record()
        torch.cuda.synchronize()
        if req_us is None:
            req_us = e0.elapsed_time(e1) * 1e3
        del w
        heads4.append(spec.spec_pack_w4(*q4, G=GROUP))
        del q4
    heads8 = [spec.spec_pack_w8(*synth.torch_qweights(8, V, K, GROUP, 8200 + c, dev), G=GROUP)
              for c in range(2)]
    x = synth.torch_activations(1, K, 8300, dev)
    logits = torch.empty((1, V), dtype=torch.float32, device=dev)
    u = synth.torch_uniforms((1,), 8301, dev)
    sample = spec.bind_sample_tokens(logits, u, ACC_T)

    def timed(heads):
        calls = [spec.bind_qmv(h, x, logits) for h in heads]
        for c in calls:
            c()
            sample()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i, (a, b_, c_) in enumerate(ev):
            a.record()
            calls[i % len(calls)]()
            b_.record()
            sample()
            c_.record()
        torch.cuda.synchronize()
        head = sum(a.elapsed_time(b_) for a, b_, _ in ev) / steps * 1e3
        samp = sum(b_.elapsed_time(c_) for _, b_, c_ in ev) / steps * 1e3
        return head, samp

    h4, s4 = timed(heads4)
    h8, s8 = timed(heads8)
    b4 = roofline.qmv_bytes(4, 1, V, K)
    b8 = roofline.qmv_bytes(8, 1, V, K)
    out = {"draft": f"LM head {K}->{V} at M=1, then one draw (T={ACC_T}) from its logits",
           "w4_draft_head": {"head_us": round(h4, 2), "sample_us": round(s4, 2),
                             "step_us": round(h4 + s4, 2), "head_GB/s": round(b4 / h4 / 1e3, 1),
                             "head_frac": round(b4 / h4 / 1e3 / 8000.0, 4)},
           "w8_head": {"head_us": round(h8, 2), "sample_us": round(s8, 2),
                       "step_us": round(h8 + s8, 2), "head_GB/s": round(b8 / h8 / 1e3, 1),
                       "head_frac": round(b8 / h8 / 1e3 / 8000.0, 4)},
           "draft_step_reduction": round(1.0 - (h4 + s4) / (h8 + s8), 4),
           "requantize_us_once": round(req_us, 1)}
    print(json.dumps(out), flush=True)


# Recurrent layers of the target: 36 gated-delta-rule layers of 32 heads
# (dk = dv = 128), 8 sequences, one verify block of T = 6 positions (D = 5).
GDN_LAYERS, GDN_B, GDN_H, GDN_T = 36, 8, 32, 6


def gdn(dev, steps):
    """The recurrent-state kernels of one verify cycle: per layer, the capture
    over the T verify positions (spec_gdn_record) and, after acceptance, the
    commit of the accepted steps (spec_gdn_commit, n = accepted + 1 drawn
    uniformly from 1..T).  Each layer has its own state (36 x 8 x 32 heads x
    64 KB = 604 MB, beyond the 256 MB last-level cache); one timed pass runs
    all 36 layers back to back."""
    import numpy as np
    import torch
    import speculative_decoding_spec_amd as spec
    from speculative_decoding_spec_amd import roofline, synth
    layers = []
    for li in range(GDN_LAYERS):
        S0, q, k, v, a, b = synth.torch_gdn_inputs(GDN_B, GDN_T, GDN_H, 7000 + li, dev)
        layers.append(dict(S=S0, q=q, k=k, v=v, a=a, b=b,
                           o=torch.empty_like(v), d=torch.empty_like(v)))
    n_host = np.random.default_rng(7).integers(1, GDN_T + 1, size=GDN_B).astype(np.int32)
    n = torch.from_numpy(n_host).to(dev)

    # pre-marshalled launches, so the host stays ahead of the GPU
    rec_calls = [spec.bind_gdn_record(L["S"], L["q"], L["k"], L["v"], L["a"], L["b"], L["o"], L["d"])
                 for L in layers]
    com_calls = [spec.bind_gdn_commit(L["S"], L["a"], L["k"], L["d"], n) for L in layers]

    def timed(calls):
        for c in calls:
            c()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            for c in calls:
                c()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (steps * len(calls))

    rec_us = timed(rec_calls)
    com_us = timed(com_calls)
    # The same boundary in one pass per layer: the commit of the tape just
    # recorded and the capture of the next block (here the same step inputs)
    # from the committed state, the new tape in buffers of its own.
    for L in layers:
        L["o2"], L["d2"] = torch.empty_like(L["v"]), torch.empty_like(L["v"])
    cr_calls = [spec.bind_gdn_commit_record(L["S"], L["a"], L["k"], L["d"], n, L["q"], L["k"],
                                            L["v"], L["a"], L["b"], L["o2"], L["d2"])
                for L in layers]
    cr_us = timed(cr_calls)
    # After verification the commits of all layers are independent: with the
    # layers' states and tapes laid out [layer][sequence], one launch commits
    # the whole model (sequence index layer * B + b, step counts repeated).
    allS = torch.empty((GDN_LAYERS * GDN_B, GDN_H, 128, 128), dtype=torch.float32, device=dev)
    allA = torch.empty((GDN_LAYERS * GDN_B, GDN_T, GDN_H), dtype=torch.float32, device=dev)
    allK = torch.empty((GDN_LAYERS * GDN_B, GDN_T, GDN_H, 128), dtype=torch.float32, device=dev)
    allD = torch.empty((GDN_LAYERS * GDN_B, GDN_T, GDN_H, 128), dtype=torch.float32, device=dev)
    for li, L in enumerate(layers):
        sl = slice(li * GDN_B, (li + 1) * GDN_B)
        allS[sl].copy_(L["S"]); allA[sl].copy_(L["a"]); allK[sl].copy_(L["k"]); allD[sl].copy_(L["d"])
    del layers, rec_calls, com_calls, cr_calls
    n_all = n.repeat(GDN_LAYERS)
    all_us = timed([spec.bind_gdn_commit(allS, allA, allK, allD, n_all)]) 
    rb = roofline.gdn_record_bytes(GDN_B, GDN_T, GDN_H)
    cb = roofline.gdn_commit_bytes(n_host.tolist(), GDN_H)
    crb = roofline.gdn_commit_record_bytes(n_host.tolist(), GDN_T, GDN_H)
    out = {"gdn": (f"{GDN_LAYERS} layers x {GDN_B} sequences x {GDN_H} heads, dk=dv=128, "
                   f"T={GDN_T} verify positions; commit steps {n_host.tolist()}"),
           "record": {"us_per_layer": round(rec_us, 2), "bytes_per_layer": rb,
                      "GB/s": round(rb / rec_us / 1e3, 1), "frac": round(rb / rec_us / 1e3 / 8000.0, 4)},
           "commit": {"us_per_layer": round(com_us, 2), "bytes_per_layer": cb,
                      "GB/s": round(cb / com_us / 1e3, 1), "frac": round(cb / com_us / 1e3 / 8000.0, 4)},
           "commit_record": {"us_per_layer": round(cr_us, 2), "bytes_per_layer": crb,
                             "GB/s": round(crb / cr_us / 1e3, 1),
                             "frac": round(crb / cr_us / 1e3 / 8000.0, 4),
                             "vs_two_calls_us": round(rec_us + com_us, 2)},
           "commit_all_layers_one_launch": {
               "us": round(all_us, 2), "bytes": cb * GDN_LAYERS,
               "GB/s": round(cb * GDN_LAYERS / all_us / 1e3, 1),
               "frac": round(cb * GDN_LAYERS / all_us / 1e3 / 8000.0, 4)},
           "snapshot_alternative_bytes_per_layer": GDN_B * GDN_H * 128 * 128 * 4 * (GDN_T + 1)}
    print(json.dumps(out), flush=True)


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


STREAM_BYTES = 2 << 30


def stream_read_rate(dev, reps=10):
    """GB/s of a plain streaming read of STREAM_BYTES (spec_stream_read: every
    byte once, 16-byte non-temporal loads), 8x the last-level cache."""
    import torch
    import speculative_decoding_spec_amd as spec
    src = torch.zeros(STREAM_BYTES // 4, dtype=torch.int32, device=dev)
    sink = torch.empty(spec.STREAM_READ_GROUPS, dtype=torch.int32, device=dev)
    call = spec.bind_stream_read(src, sink)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    gbs = STREAM_BYTES / (us * 1e-6) / 1e9
    del src
    return {"bytes": STREAM_BYTES, "us": round(us, 2), "GB/s": round(gbs, 1),
            "frac": round(gbs / 8000.0, 4)}


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


def valu_compare(blocks, stream, steps):
    """The chained MLP block at M = 1..4 with the products on the vector ALU
    (spec_qmv_gate_up_silu_w4_valu, spec_qmv_w4_packed_valu) and on the
    matrix cores: median (p10, p90) of each M's two launches back to back."""
    import torch
    import speculative_decoding_spec_amd as spec
    from speculative_decoding_spec_amd import roofline
    res = {}
    for b in blocks:
        M = b["M"]
        if M > 4:
            continue
        nb = roofline.gate_up_silu_bytes(4, M, FFN, HIDDEN) + roofline.qmv_bytes(4, M, HIDDEN, FFN)
        row = {}
        for path, valu in (("mfma", False), ("valu", True)):
            calls = [spec.bind_qmv_gate_up_silu(b["glu"], b["x"], b["h"], valu=valu),
                     spec.bind_qmv(b["down"], b["h"], b["yd"], valu=valu)]
            for c in calls:
                c()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(steps)]
            for e0, e1 in evs:
                e0.record(stream)
                for c in calls:
                    c()
                e1.record(stream)
            torch.cuda.synchronize()
            t = spread_us([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
            row[path] = {"us": t["us"], "p10_us": t["p10_us"], "p90_us": t["p90_us"], **rate(nb, t["us"])}
        res[str(M)] = row
    return res


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



def build_inputs(dev, variants=True):
    """W4 weights per M: gate/up packed for the gated launch and the down
    matrix (packing is a load-time step, outside the timing); for the
    variants also the weights as stored (read by spec_qmv_w4 directly, gate
    and up concatenated) and gate/up packed as one plain matrix and as two."""
    import torch
    import speculative_decoding_spec_amd as spec
    from speculative_decoding_spec_amd import synth

    blocks = []
    for i, M in enumerate(MS):
        g = synth.torch_qweights(4, FFN, HIDDEN, GROUP, 1000 + 10 * i, dev)
        u = synth.torch_qweights(4, FFN, HIDDEN, GROUP, 1001 + 10 * i, dev)
        d = synth.torch_qweights(4, HIDDEN, FFN, GROUP, 1002 + 10 * i, dev)
        glu = spec.spec_pack_gate_up(4, g, u, G=GROUP)
        down = spec.spec_pack_w4(*d, G=GROUP)
        blk = dict(M=M, glu=glu, down=down)
        if variants:
            gu = [torch.cat([a, b]) for a, b in zip(g, u)]
            blk["gate_up"] = spec.spec_pack_w4(*gu, G=GROUP)
            blk["gate"], blk["up"] = spec.spec_pack_w4(*g, G=GROUP), spec.spec_pack_w4(*u, G=GROUP)
            blk["gate_up_as_stored"] = spec.QWeights(4, *gu, G=GROUP)
            blk["down_as_stored"] = spec.QWeights(4, *d, G=GROUP)
        del g, u, d
        blk["x"] = synth.torch_activations(M, HIDDEN, 1003 + 10 * i, dev)
        blk["h"] = torch.empty((M, FFN), dtype=torch.bfloat16, device=dev)
        blk["ygu"] = torch.empty((M, 2 * FFN), dtype=torch.float32, device=dev)
        blk["yg"] = torch.empty((M, FFN), dtype=torch.float32, device=dev)
        blk["yu"] = torch.empty((M, FFN), dtype=torch.float32, device=dev)
        blk["yd"] = torch.empty((M, HIDDEN), dtype=torch.float32, device=dev)
        blocks.append(blk)
    torch.cuda.synchronize()
    return blocks


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(seconds):
    """The fp64 oracle, as it stands, on a bounded sample of the step, with
    all host threads (16 at most: the box's share) and with one.

    qmv: the step's MLP chain at M = 1..8 (the gated gate/up activation,
    then down on the oracle's own bf16 h) with one seeded weight set per
    shape, rows split over the threads, stopping once `seconds` have passed;
    acceptance: the 256-sequence batch, drafts drawn from the draft rows as
    on the GPU, likewise bounded.  Rates use the GPU figure's algorithmic
    bytes (GB/s) and verify positions per second."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    from speculative_decoding_spec_amd import roofline, synth
    gate = synth.qweights(1, 4, FFN, HIDDEN, GROUP, salt=1)
    up = synth.qweights(1, 4, FFN, HIDDEN, GROUP, salt=2)
    down = synth.qweights(1, 4, HIDDEN, FFN, GROUP, salt=3)
    tl, dl = synth.logits_pair(4, ACC_B, ACC_D, ACC_V)
    ud = synth.uniforms(4, synth.U_DRAFT, ACC_B * ACC_D)
    toks = oracle.sample_rows(dl.reshape(ACC_B * ACC_D, ACC_V), ACC_T, 0, 1.0, ud).reshape(ACC_B, ACC_D)
    u = synth.uniforms(4, synth.U_ACCEPT, (ACC_B, ACC_D + 1))

    def run(threads, budget):
        chunk = 256
        done_bytes, launches, t0 = 0, 0, time.perf_counter()
        with ThreadPoolExecutor(threads) as ex:
            for M in MS:
                if time.perf_counter() - t0 >= budget:
                    break
                x = synth.activations(1, M, HIDDEN, salt=M)
                spans = [(r, min(FFN, r + chunk)) for r in range(0, FFN, chunk)]
                parts = list(ex.map(lambda sp: oracle.gate_up_silu(4, gate, up, x, GROUP, rows=sp), spans))
                hb = np.ascontiguousarray(np.concatenate([p[1] for p in parts], axis=1))
                done_bytes += roofline.gate_up_silu_bytes(4, M, FFN, HIDDEN, GROUP)
                launches += 1
                if time.perf_counter() - t0 >= budget:
                    break
                spans = [(r, min(HIDDEN, r + chunk)) for r in range(0, HIDDEN, chunk)]
                list(ex.map(lambda sp: oracle.qmv(4, *down, hb, GROUP, rows=sp), spans))
                done_bytes += roofline.qmv_bytes(4, M, HIDDEN, FFN, GROUP)
                launches += 1
        dt = time.perf_counter() - t0
        nseq, t1 = 0, time.perf_counter()
        with ThreadPoolExecutor(threads) as ex:
            while nseq < ACC_B and time.perf_counter() - t1 < budget:
                idx = range(nseq, min(ACC_B, nseq + threads))
                list(ex.map(lambda i: oracle.accept(tl[i:i + 1], dl[i:i + 1], toks[i:i + 1],
                                                    u[i:i + 1], ACC_T), idx))
                nseq = idx[-1] + 1
        at = time.perf_counter() - t1
        return {"GB/s": round(done_bytes / dt / 1e9, 4), "launches": launches,
                "MB": round(done_bytes / 1e6), "qmv_s": round(dt, 2),
                "accept_positions_per_s": round(nseq * (ACC_D + 1) / at, 1), "sequences": nseq,
                "accept_s": round(at, 2)}

    threads = min(16, os.cpu_count() or 1)
    allc = run(threads, seconds)
    one = run(1, seconds / 2)
    return {
        "value": allc["GB/s"], "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": (f"W4 g64 MLP chain: {allc['launches']} of the step's 16 launches (gated gate/up "
                   f"5120->2x17408, down 17408->5120, M=1..8), {allc['MB']} MB algorithmic in "
                   f"{allc['qmv_s']} s; acceptance: {allc['sequences']} of 256 sequences (D=5, "
                   f"V=151936, T=0.6) in {allc['accept_s']} s"),
        "accept_positions_per_s": allc["accept_positions_per_s"],
        "single_thread": {"GB/s": one["GB/s"], "accept_positions_per_s": one["accept_positions_per_s"],
                          "sample": (f"{one['launches']} launches, {one['MB']} MB in {one['qmv_s']} s; "
                                     f"{one['sequences']} sequences in {one['accept_s']} s")},
        "cpu": cpu_model(), "host_threads": os.cpu_count(),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; "
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
    if args.gdn:
        gdn(dev, args.steps)
        return
    if args.draft:
        draft(dev, args.steps)
        return
    if args.depth:
        print(json.dumps({"depth": verify_pass(dev, min(args.steps, 20), separate=True)}), flush=True)
        return
    if args.lmhead:
        print(json.dumps({"lmhead": lmhead_accept(dev, args.steps)}), flush=True)
        return
    full = not args.step_only
    blocks = build_inputs(dev, variants=full)
    if args.valu:
        print(json.dumps({"mfma_vs_valu": valu_compare(blocks, torch.cuda.current_stream(dev),
                                                       args.steps)}), flush=True)
        return
    acc = build_accept(dev)
    stream = torch.cuda.current_stream(dev)
    acc_bytes = roofline.accept_bytes(ACC_B, ACC_D, ACC_V)

    def pair():
        return (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))

    def mlp_launches(kind):
        """(bound call, shape name, algorithmic bytes) per launch of the MLP
        blocks: 'chain' = gated gate/up then down on its h (the step);
        'plain' = gate/up as one fp32 launch, then down; 'separate' = gate,
        up and down; 'as_stored' = 'plain' read from the interchange layout."""
        out = []
        for b in blocks:
            M = b["M"]
            if kind == "chain":
                out.append((spec.bind_qmv_gate_up_silu(b["glu"], b["x"], b["h"]), "gate_up_silu",
                            roofline.gate_up_silu_bytes(4, M, FFN, HIDDEN)))
            elif kind == "plain":
                out.append((spec.bind_qmv(b["gate_up"], b["x"], b["ygu"]), "gate_up",
                            roofline.qmv_bytes(4, M, 2 * FFN, HIDDEN)))
            elif kind == "as_stored":
                out.append((spec.bind_qmv(b["gate_up_as_stored"], b["x"], b["ygu"]), "gate_up",
                            roofline.qmv_bytes(4, M, 2 * FFN, HIDDEN)))
            else:
                out.append((spec.bind_qmv(b["gate"], b["x"], b["yg"]), "gate",
                            roofline.qmv_bytes(4, M, FFN, HIDDEN)))
                out.append((spec.bind_qmv(b["up"], b["x"], b["yu"]), "up",
                            roofline.qmv_bytes(4, M, FFN, HIDDEN)))
            down = b["down_as_stored"] if kind == "as_stored" else b["down"]
            out.append((spec.bind_qmv(down, b["h"], b["yd"]), "down", roofline.qmv_bytes(4, M, HIDDEN, FFN)))
        return out

    launches = mlp_launches("chain")
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

    # Timed steps: events around the qmv part and the acceptance call of each.
    ev = [{"q": pair(), "a": pair()} for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    q_us = [e["q"][0].elapsed_time(e["q"][1]) * 1e3 for e in ev]
    a_us = [e["a"][0].elapsed_time(e["a"][1]) * 1e3 for e in ev]
    qmed, qp10, qp90 = pct(q_us)
    amed, ap10, ap90 = pct(a_us)
    qmv_gbs = qmv_bytes_step / qmed / 1e3
    positions = ACC_B * (ACC_D + 1)
    acc_gbs = acc_bytes / amed / 1e3
    accept = {"positions_per_s": round(positions / amed * 1e6, 1),
              "us": round(amed, 2), "p10_us": round(ap10, 2), "p90_us": round(ap90, 2),
              "positions_per_s_p10_p90": [round(positions / ap90 * 1e6, 1), round(positions / ap10 * 1e6, 1)],
              "GB/s": round(acc_gbs, 1), "frac": round(acc_gbs / PEAK_GBS, 4),
              "algorithmic_bytes": acc_bytes,
              "mean_accepted": float(acc["acc"].float().mean().item())}

    # Roofline of qmv_kernel: algorithmic bytes per launch over the average
    # launch duration, i.e. the median qmv part of a step (16 launches back
    # to back, no events between them) divided by 16.
    bytes_per_launch = qmv_bytes_step / len(launches)
    launch_us = qmed / len(launches)
    achieved = bytes_per_launch / launch_us / 1e3
    traffic, tinfo = measured_traffic(bytes_per_launch)
    roof = {"kernel": ("qmv_kernel (W4; 16 launches per step: gate/up with the gated activation, "
                       "and down, at M=1..8)"),
            "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_GBS, 4),
            "traffic": None if traffic is None else round(traffic),
            "algorithmic_bytes_per_launch": round(bytes_per_launch),
            "avg_launch_us": round(launch_us, 2),
            "traffic_source": (os.path.relpath(TRAFFIC_FILE, ROOT) if traffic is not None else tinfo)}
    out = {
        "metric": METRIC, "value": round(qmv_gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "w4-bf16xfp32 qmv; fp32 accept",
        "data": "synthetic (seeded, on-device generators)",
        "config": {"workload": ("verify MLP block W4 g64 (gate/up 5120->2x17408 as one launch "
                                "applying silu(gate)*up, down 17408->5120 on that activation) at "
                                "M=1..8 on distinct weight copies + batched acceptance B=256 D=5 "
                                "V=151936 T=0.6"),
                   "qmv_bytes_per_step": qmv_bytes_step, "accept_bytes_per_step": acc_bytes},
        "qmv_frac_of_peak": round(qmv_gbs / PEAK_GBS, 4),
        "qmv_us_per_step": round(qmed, 2), "qmv_us_p10": round(qp10, 2), "qmv_us_p90": round(qp90, 2),
        "value_p10_p90": [round(qmv_bytes_step / qp90 / 1e3, 1), round(qmv_bytes_step / qp10 / 1e3, 1)],
        "accept": accept, "roofline": roof,
    }
    if not full:
        print(json.dumps(out), flush=True)
        return

    steps = args.steps

    def span_us(calls):
        """Median (p10, p90) microseconds of `steps` passes over `calls`."""
        for c, _, _ in calls:
            c()
        accept_call()          # untimed: the queue is busy at the first event
        evs = [pair() for _ in range(steps)]
        for e0, e1 in evs:
            e0.record(stream)
            for c, _, _ in calls:
                c()
            e1.record(stream)
            accept_call()
        torch.cuda.synchronize()
        return spread_us([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])

    variants = {}
    for kind, label in (("chain", "chained MLP: gate/up with the gated activation, then down on its h (value)"),
                        ("as_stored", ("weights read as stored (spec_qmv_w4, interchange layout): gate/up as "
                                       "one fp32 launch, then down")),
                        ("plain", "packed: gate/up as one launch with fp32 outputs, no activation; down"),
                        ("separate", "packed: separate gate, up and down launches (24)")):
        calls = launches if kind == "chain" else mlp_launches(kind)
        t = span_us(calls)
        nb = sum(l[2] for l in calls)
        variants[label] = {"qmv_us_per_step": t["us"], "p10_us": t["p10_us"], "p90_us": t["p90_us"],
                           **rate(nb, t["us"])}
    out["variants"] = variants

    out["mfma_vs_valu (chained MLP block at M=1..4, us per block)"] = valu_compare(blocks, stream, steps)

    # Per M and per shape: events around every launch (about 2 us of marker
    # time each, so these only split the step).
    evs = [[pair() for _ in launches] for _ in range(steps)]
    accept_call()
    for each in evs:
        for i, (call, _, _) in enumerate(launches):
            each[i][0].record(stream)
            call()
            each[i][1].record(stream)
        accept_call()
    torch.cuda.synchronize()
    l_us = [pct([e[i][0].elapsed_time(e[i][1]) * 1e3 for e in evs])[0] for i in range(len(launches))]
    per_m = {}
    for j, b in enumerate(blocks):
        us = l_us[2 * j] + l_us[2 * j + 1]
        nb = launches[2 * j][2] + launches[2 * j + 1][2]
        per_m[str(b["M"])] = {"us": round(us, 2), **rate(nb, us)}
    per_shape = {}
    for name in ("gate_up_silu", "down"):
        idx = [i for i, l in enumerate(launches) if l[1] == name]
        us = sum(l_us[i] for i in idx) / len(idx)
        nb = sum(launches[i][2] for i in idx) / len(idx)
        per_shape[name] = {"us_per_launch": round(us, 2), **rate(nb, us)}
    out["per_M (per-launch events, median)"] = per_m
    out["roofline_parts"] = {
        "qmv_kernel": {"achieved": round(achieved, 1), "frac": round(achieved / PEAK_GBS, 4),
                       "per_shape (per-launch events)": per_shape},
        "accept (row statistics pass + fused decide/sum/draw)": {
            "achieved": round(acc_gbs, 1), "frac": round(acc_gbs / PEAK_GBS, 4), "us_per_call": round(amed, 2)}}

    # Greedy verification of the same block (target logits only), drafts
    # from the greedy draft (argmax of each draft row).
    g_toks = torch.argmax(acc["d"], dim=2).to(torch.int32).contiguous()
    g_out = (torch.empty(ACC_B, dtype=torch.int32, device=dev),
             torch.empty(ACC_B, dtype=torch.int32, device=dev))
    greedy_call = spec.bind_verify_greedy(acc["t"], g_toks, out=g_out)
    g = spread_us(timed_each([greedy_call], steps, stream))
    g_bytes = roofline.greedy_bytes(ACC_B, ACC_D, ACC_V)
    out["accept_greedy (same block, target logits only; not part of the step)"] = {
        "positions_per_s": round(positions / g["us"] * 1e6, 1), **g, **rate(g_bytes, g["us"]),
        "algorithmic_bytes": g_bytes, "mean_accepted": float(g_out[0].float().mean().item())}
    del blocks, launches
    torch.cuda.empty_cache()

    # The other workloads of the verify hot path.
    out["configs"] = {"pr1_reference": pr1_reference(dev, steps),
                      "lm_head_accept": lmhead_accept(dev, steps),
                      "w8_lm_head": w8_lm_head(dev, steps),
                      "verify_pass_64_layers": verify_pass(dev, min(steps, 20))}

    # The attainable read rate beside the published peak: a plain streaming
    # read of 2 GiB (spec_stream_read), and each part's share of it.
    sr = stream_read_rate(dev)
    out["stream_read"] = sr
    out["qmv_frac_of_stream"] = round(qmv_gbs / sr["GB/s"], 4)
    out["accept"]["frac_of_stream"] = round(acc_gbs / sr["GB/s"], 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
