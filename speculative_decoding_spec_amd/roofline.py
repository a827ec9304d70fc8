"""Bandwidth roofline bookkeeping for the verify qmv and the acceptance step.

Decoding is memory bound: the bound on tokens per second is the memory
bandwidth divided by the bytes of parameters every token has to stream
(savepearlharbor.com article on MTP in llama.cpp, section on the theoretical
maximum of token generation, with its RTX 4060 Ti worked example).  The same
bookkeeping gives a kernel's achieved fraction of HBM peak: algorithmic bytes
per launch divided by the launch's duration, over the published peak.
"""
from __future__ import annotations

#: MI355X published HBM3E peak, bytes/s.
HBM_PEAK_BYTES_PER_S = 8.0e12


def decode_bound_tokens_per_s(bandwidth_bytes_per_s: float, weight_bytes: float) -> float:
    """Upper bound on decode tokens/s when every token streams all weights once."""
    return bandwidth_bytes_per_s / weight_bytes


def qmv_bytes(bits: int, M: int, N: int, K: int, group: int = 64) -> int:
    """Bytes one qmv must move: packed weights, fp16 scales and biases, bf16
    activations in, fp32 outputs out."""
    return N * K * bits // 8 + N * (K // group) * 4 + M * K * 2 + M * N * 4


def gate_up_silu_bytes(bits: int, M: int, F: int, K: int, group: int = 64) -> int:
    """Bytes of the gated gate/up launch: both packed matrices with their
    scale/bias words, bf16 x in, bf16 h [M][F] out."""
    return 2 * F * K * bits // 8 + 2 * F * (K // group) * 4 + M * K * 2 + M * F * 2


def gdn_record_bytes(B: int, T: int, H: int, d: int = 128) -> int:
    """Bytes of the recurrent capture over T steps: each head's state read
    once, q, k, v, alpha, beta read, o and the tape delta written."""
    return B * H * d * d * 4 + B * T * H * (3 * d + 2) * 4 + 2 * B * T * H * d * 4


def gdn_commit_bytes(n_steps, H: int, d: int = 128) -> int:
    """Bytes of the commit: for every sequence with n >= 1 steps, its heads'
    states read and written once and n steps of (alpha, k, delta) read; the
    step counts themselves."""
    total = 4 * len(n_steps)
    for n in n_steps:
        if n > 0:
            total += 2 * H * d * d * 4 + n * H * (2 * d + 1) * 4
    return total


def gdn_commit_record_bytes(n_steps, T: int, H: int, d: int = 128) -> int:
    """Bytes of the cycle boundary in one pass: every head's state read once
    and, for sequences with n >= 1 steps, written back committed; n steps of
    (alpha, k, delta) of the previous tape read; the step counts; then the
    capture's step inputs read and its o and delta written (the state is
    already in registers)."""
    B = len(n_steps)
    total = B * H * d * d * 4 + 4 * B
    for n in n_steps:
        if n > 0:
            total += H * d * d * 4 + n * H * (2 * d + 1) * 4
    return total + B * T * H * (3 * d + 2) * 4 + 2 * B * T * H * d * 4


def qmv_flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def accept_bytes(B: int, D: int, V: int) -> int:
    """Bytes the acceptance must move: every fp32 logit once (D + 1 target and
    D draft rows per sequence), the draft tokens, D + 1 uniforms, two int32
    outputs per sequence."""
    return B * (2 * D + 1) * V * 4 + B * D * 4 + B * (D + 1) * 4 + B * 8


def greedy_bytes(B: int, D: int, V: int) -> int:
    """Bytes greedy verification must move: every fp32 target logit once
    (D + 1 rows per sequence), the draft tokens, two int32 outputs per
    sequence.  The draft logits are not needed."""
    return B * (D + 1) * V * 4 + B * D * 4 + B * 8


def fraction_of_peak(nbytes: float, seconds: float,
                     peak: float = HBM_PEAK_BYTES_PER_S) -> float:
    return nbytes / seconds / peak
