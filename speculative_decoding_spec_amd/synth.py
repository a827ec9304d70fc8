"""Seeded synthetic inputs for the verify qmv and the acceptance step.

Random numbers only: this module holds none of the method's arithmetic (no
dequantization, no softmax, no sampling), so the HIP path and the oracle can
both be fed from it without sharing any of the computation under test.

Every tensor is drawn from ``numpy.random.default_rng(SeedSequence([cfg, tid]))``
with a fixed tensor id per role, so a (config, role) pair always yields the
same values:

    0 weights   uniform codes: W4 as random uint32 words (8 independent
                uniform nibbles each), W8 as random bytes
    1 scales    U(0.01, 0.05), rounded to fp16 (round-to-nearest-even)
    2 biases    N(0, 0.1) (second parameter = standard deviation) -> fp16
    3 x         N(0, 1) -> fp32 -> bf16 (round-to-nearest-even)
    4 draft logits  N(0, 2) fp32
    5 noise         N(0, 0.5) fp32; target = draft + noise
    6 draft-sampling uniforms
    7 acceptance uniforms

Uniforms are k * 2^-24 with k uniform in {0, ..., 2^24 - 1}: exact fp32
values in [0, 1).
"""
from __future__ import annotations

import numpy as np

W, SCALES, BIASES, X, DRAFT, NOISE, U_DRAFT, U_ACCEPT = range(8)


def rng(cfg: int, tid: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(cfg), int(tid)]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even; NaN kept."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(a)
    out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def qweights(cfg: int, bits: int, N: int, K: int, group: int = 64, salt: int = 0):
    """Packed weights, fp16 scales and fp16 biases for an [N][K] matrix.

    W4: uint32 [N][K/8] (element k at bits 4*(k%8) of word k/8); W8: uint8
    [N][K].  Scales/biases: fp16 bit patterns as uint16 [N][K/group].
    ``salt`` separates several matrices drawn under one config.
    """
    assert K % group == 0
    r = rng(cfg * 1000 + salt, W)
    if bits == 4:
        assert K % 8 == 0
        w = r.integers(0, 2**32, size=(N, K // 8), dtype=np.uint32)
    elif bits == 8:
        w = r.integers(0, 256, size=(N, K), dtype=np.uint8)
    else:
        raise ValueError(bits)
    ng = K // group
    s = rng(cfg * 1000 + salt, SCALES).uniform(0.01, 0.05, size=(N, ng))
    b = rng(cfg * 1000 + salt, BIASES).normal(0.0, 0.1, size=(N, ng))
    s16 = s.astype(np.float16).view(np.uint16)
    b16 = b.astype(np.float16).view(np.uint16)
    return w, np.ascontiguousarray(s16), np.ascontiguousarray(b16)


def activations(cfg: int, M: int, K: int, salt: int = 0) -> np.ndarray:
    """bf16 bit patterns uint16 [M][K], values N(0, 1)."""
    x = rng(cfg * 1000 + salt, X).normal(0.0, 1.0, size=(M, K)).astype(np.float32)
    return f32_to_bf16_bits(x)


def uniforms(cfg: int, tid: int, shape) -> np.ndarray:
    k = rng(cfg, tid).integers(0, 2**24, size=shape, dtype=np.int64)
    return (k.astype(np.float64) * 2.0**-24).astype(np.float32)


def logits_pair(cfg: int, B: int, D: int, V: int, draft_sd: float = 2.0,
                noise_sd: float = 0.5):
    """(target [B][D+1][V], draft [B][D][V]) fp32.

    Draft rows are N(0, draft_sd); the target row at the same position is the
    draft row plus N(0, noise_sd); the bonus position D has a fresh draft-like
    row plus noise (there is no draft distribution there)."""
    r = rng(cfg, DRAFT)
    base = r.normal(0.0, draft_sd, size=(B, D + 1, V)).astype(np.float32)
    noise = rng(cfg, NOISE).normal(0.0, noise_sd, size=(B, D + 1, V)).astype(np.float32)
    target = (base + noise).astype(np.float32)
    draft = np.ascontiguousarray(base[:, :D, :])
    return target, draft


GDN = 8   # tensor id of the recurrent-layer inputs


def gdn_inputs(cfg: int, B: int, T: int, H: int, dk: int = 128, dv: int = 128):
    """Inputs of T recurrent (gated delta rule) steps for B sequences x H heads,
    fp32: S0 [B][H][dv][dk] ~ N(0, 0.1); q, k [B][T][H][dk] unit vectors
    (normal draws scaled to length 1, as the layer normalizes them); v
    [B][T][H][dv] ~ N(0, 1); alpha [B][T][H] ~ U(0.8, 1) (decay gates near
    one); beta [B][T][H] ~ U(0, 1)."""
    r = rng(cfg, GDN)
    S0 = r.normal(0.0, 0.1, size=(B, H, dv, dk)).astype(np.float32)
    q = r.normal(size=(B, T, H, dk))
    k = r.normal(size=(B, T, H, dk))
    q = (q / np.linalg.norm(q, axis=-1, keepdims=True)).astype(np.float32)
    k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    v = r.normal(size=(B, T, H, dv)).astype(np.float32)
    alpha = r.uniform(0.8, 1.0, size=(B, T, H)).astype(np.float32)
    beta = r.uniform(0.0, 1.0, size=(B, T, H)).astype(np.float32)
    return S0, q, k, v, alpha, beta


# ---- device-side generators for benchmark working sets -------------------
# Large working sets (hundreds of MB to GB) are drawn on the GPU with torch's
# seeded generator instead: the values differ from the numpy streams above,
# but the distributions are the same.  They feed timing only, never a parity
# comparison.

def torch_qweights(bits: int, N: int, K: int, group: int, seed: int, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    if bits == 4:
        w = torch.randint(-2**31, 2**31, (N, K // 8), generator=g, device=device,
                          dtype=torch.int64).to(torch.int32)
    else:
        w = torch.randint(0, 256, (N, K), generator=g, device=device,
                          dtype=torch.int32).to(torch.uint8)
    ng = K // group
    s = (torch.rand((N, ng), generator=g, device=device) * 0.04 + 0.01).to(torch.float16)
    b = (torch.randn((N, ng), generator=g, device=device) * 0.1).to(torch.float16)
    return w, s, b


def torch_activations(M: int, K: int, seed: int, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((M, K), generator=g, device=device).to(torch.bfloat16)


def torch_logits_pair(B: int, D: int, V: int, seed: int, device,
                      draft_sd: float = 2.0, noise_sd: float = 0.5):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    base = torch.randn((B, D + 1, V), generator=g, device=device) * draft_sd
    target = base + torch.randn((B, D + 1, V), generator=g, device=device) * noise_sd
    draft = base[:, :D, :].contiguous()
    return target.contiguous(), draft


def torch_uniforms(shape, seed: int, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    k = torch.randint(0, 2**24, shape, generator=g, device=device, dtype=torch.int64)
    return (k.to(torch.float64) * 2.0**-24).to(torch.float32)


def torch_gdn_inputs(B: int, T: int, H: int, seed: int, device, dk: int = 128, dv: int = 128):
    """gdn_inputs' distributions drawn on the device (timing only)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    S0 = torch.randn((B, H, dv, dk), generator=g, device=device) * 0.1
    q = torch.randn((B, T, H, dk), generator=g, device=device)
    k = torch.randn((B, T, H, dk), generator=g, device=device)
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    v = torch.randn((B, T, H, dv), generator=g, device=device)
    alpha = torch.rand((B, T, H), generator=g, device=device) * 0.2 + 0.8
    beta = torch.rand((B, T, H), generator=g, device=device)
    return S0, q.contiguous(), k.contiguous(), v, alpha, beta
