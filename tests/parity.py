"""Shared helpers for the GPU parity tests: moving synthetic inputs to the
device, running the oracle on host threads, and the comparison rules.

Comparison rules (fixed before any kernel was written):
  qmv      |gpu - oracle| <= 1e-3 * |oracle| + 2^-20 * sum_k |x * w|  per output;
           the second term only matters for outputs near zero and the tests
           report how many outputs needed it.
  probs    |gpu - oracle| <= 1e-5 absolute.
  decisions and tokens   bit-exact, except counted ties:
           - a ratio test with |u_i - a_i| < 1e-5 (a_i from the oracle);
           - a draw whose target mass u * W lies within 1e-5 * W of a
             cumulative boundary the two sides could resolve differently;
           - a row whose top-p cut has cumulative mass within 1e-5 of top_p.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

TIE = 1e-5
THREADS = min(16, os.cpu_count() or 1)


# ------------------------------------------------------------- devices ----
def dev_qweights(w, s, b, device):
    import torch
    wt = torch.from_numpy(w.view(np.int32) if w.dtype == np.uint32 else w).to(device)
    st = torch.from_numpy(s.view(np.float16)).to(device)
    bt = torch.from_numpy(b.view(np.float16)).to(device)
    return wt, st, bt


def dev_x(x, device):
    import torch
    return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)


# ------------------------------------------------------------- oracle ----
def oracle_qmv_threaded(bits, w, s, b, x, G):
    """Full oracle output and magnitudes, rows split over host threads."""
    N = w.shape[0]
    edges = np.linspace(0, N, THREADS * 4 + 1).astype(int)
    spans = [(int(a), int(c)) for a, c in zip(edges[:-1], edges[1:]) if c > a]
    with ThreadPoolExecutor(THREADS) as ex:
        parts = list(ex.map(lambda r: oracle.qmv(bits, w, s, b, x, G, rows=r, with_abs=True), spans))
    y = np.concatenate([p[0] for p in parts], axis=1) if parts else np.zeros((x.shape[0], 0))
    a = np.concatenate([p[1] for p in parts], axis=1) if parts else np.zeros((x.shape[0], 0))
    return y, a


def oracle_accept_threaded(t, d, toks, u, T, k=0, p=1.0):
    B = t.shape[0]
    edges = np.linspace(0, B, min(B, THREADS * 2) + 1).astype(int)
    spans = [(int(a), int(c)) for a, c in zip(edges[:-1], edges[1:]) if c > a]

    def run(sp):
        a, c = sp
        return oracle.accept(t[a:c], None if d is None else d[a:c],
                             None if toks is None else toks[a:c], u[a:c], T, k, p)
    with ThreadPoolExecutor(THREADS) as ex:
        parts = list(ex.map(run, spans))
    return {key: np.concatenate([q[key] for q in parts]) for key in parts[0]}


# ---------------------------------------------------------------- qmv ----
def check_qmv(got, ref, mag, rtol=1e-3):
    """Returns (n_fail, n_abs_only, worst_rel)."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    bound = rtol * np.abs(ref) + 2.0**-20 * mag
    fail = ~(err <= bound)
    abs_only = (~fail) & (err > rtol * np.abs(ref))
    rel = err / np.maximum(np.abs(ref), 1e-30)
    worst = float(np.max(np.where(np.abs(ref) > 1e-6 * mag, rel, 0.0))) if got.size else 0.0
    return int(fail.sum()), int(abs_only.sum()), worst


def abs_only_limit(n_outputs):
    """Outputs allowed to pass only through the absolute term of the qmv rule:
    at most 0.1% of those compared (and at least one).  The term stands for
    outputs whose exact value nearly cancels; on the synthetic weights that
    is rare, so a larger count means a real loss of accuracy."""
    return max(1, int(0.001 * n_outputs))


# ------------------------------------------------------------- accept ----
def top_p_tie(z, T, k, p):
    """True if the row's top-p cut is within TIE of top_p (oracle side)."""
    if p >= 1.0 or not (T > 0) or k == 1:
        return False
    pk = oracle.probs(z, T, k, 1.0)
    if pk is None:
        return False
    order = np.lexsort((np.arange(z.shape[0]), -z.astype(np.float64)))
    cum = np.cumsum(pk[order])
    kept = int((pk > 0).sum())
    return bool(np.any(np.abs(cum[:kept] - p) < TIE))


def draw_tie(w, u, x_gpu, x_ref):
    """Whether two inverse-CDF picks differ only at a near-boundary."""
    c = np.cumsum(w)
    W = c[-1]
    t = float(np.float32(u)) * W
    if x_gpu < 0 or x_gpu >= w.shape[0]:
        return False
    if x_gpu > x_ref:
        return c[x_gpu - 1] <= t + TIE * W
    return c[x_gpu] >= t - TIE * W


def compare_accept(gpu, ref, t, d, toks, u, T, k=0, p=1.0):
    """Compares a GPU verification with the oracle's.

    Bit-exact apart from counted ties, and a tie excuses only a mismatch
    that depends on it:
      - accepted_len differs at position i = min(L_gpu, L_oracle): a ratio
        tie at i, or a top-p tie on target row i or draft row i (the rows
        P_i(d_i) and Q_i(d_i) come from);
      - same accepted_len, different token: a draw tie (the oracle's
        draw_margin below TIE: some inverse-CDF draw or candidate test on the
        way to its token lay within TIE of a boundary), or a top-p tie on the
        rows of the draw (target row L, and draft row L below D).
    A validity mismatch (one side -1, the other not) is always a failure.
    p_draft / q_draft are checked at every position whose two rows have no
    top-p tie.

    Returns dict(exact, ties, bad=[...], prob_err)."""
    acc_g, nxt_g = gpu["accepted_len"], gpu["next_token"]
    acc_o, nxt_o = ref["accepted_len"], ref["next_token"]
    B = acc_o.shape[0]
    D = t.shape[1] - 1
    exact, ties, bad = 0, 0, []
    prob_err = 0.0
    for b in range(B):
        tt = [p < 1.0 and top_p_tie(t[b, i], T, k, p) for i in range(D + 1)]
        dt = [p < 1.0 and top_p_tie(d[b, i], T, k, p) for i in range(D)]
        if (acc_o[b] < 0) != (acc_g[b] < 0):
            bad.append((b, "validity", int(acc_g[b]), int(acc_o[b])))
            continue
        if D > 0 and acc_o[b] >= 0 and "p_draft" in gpu:
            for i in range(D):
                if tt[i] or dt[i]:
                    continue
                e = max(abs(float(gpu["p_draft"][b, i]) - float(ref["p_draft"][b, i])),
                        abs(float(gpu["q_draft"][b, i]) - float(ref["q_draft"][b, i])))
                prob_err = max(prob_err, e)
        if acc_g[b] == acc_o[b] and nxt_g[b] == nxt_o[b]:
            exact += 1
            continue
        if acc_g[b] != acc_o[b]:
            i = int(min(acc_g[b], acc_o[b]))
            pf = np.float32(ref["p_draft"][b, i])
            qf = np.float32(ref["q_draft"][b, i])
            a = np.float32(0) if pf == 0 else np.float32(pf / qf)
            if abs(float(u[b, i]) - float(a)) < TIE or tt[i] or dt[i]:
                ties += 1
            else:
                bad.append((b, "decision", i, int(acc_g[b]), int(acc_o[b]), float(u[b, i]), float(a)))
            continue
        L = int(acc_o[b])
        if tt[L] or (L < D and dt[L]):
            ties += 1
            continue
        if float(ref["draw_margin"][b]) < TIE:
            ties += 1
        else:
            bad.append((b, "draw", L, int(nxt_g[b]), int(nxt_o[b]), float(ref["draw_margin"][b])))
    return {"exact": exact, "ties": ties, "bad": bad, "prob_err": prob_err}
