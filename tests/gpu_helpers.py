"""Helpers shared by the GPU parity tests: error metrics and device plumbing."""
import sys

import numpy as np
import torch

from diffusion_transformer_image_mm_amd import binding as B
from diffusion_transformer_image_mm_amd.device import DeviceArena, dims_for, to_numpy_f32  # noqa: F401

# Bar for floating-point parity: max |gpu - oracle| / RMS(oracle).
TOL = 2e-2


def rel_err(gpu, ref) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "non-finite GPU output"
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(gpu - ref)) / max(rms, 1e-30))


def ulp(ref, fmt: str) -> np.ndarray:
    """Spacing of bf16 (8-bit significand) or fp16 (11-bit) numbers at |ref|."""
    a = np.abs(np.asarray(ref, dtype=np.float64))
    if fmt == "bf16":
        return 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - 7)
    assert fmt == "f16"
    return np.where(a < 2.0 ** -14, 2.0 ** -24, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -14))) - 10))


def bf16_ulp(ref) -> np.ndarray:
    return ulp(ref, "bf16")


def rel_err_rounded_out(gpu, ref, fmt: str) -> float:
    """rel_err for a kernel whose output is stored in a 16-bit format: the
    part of |gpu - ref| beyond half a step of that format at ref (the
    representation band every such output must lose), over RMS(ref).
    Rounding alone can reach ~2.5e-2 of the RMS for heavy-tailed bf16
    outputs; this measures the arithmetic error."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape and np.all(np.isfinite(g))
    excess = np.maximum(np.abs(g - r) - 0.5 * ulp(r, fmt), 0.0)
    return float(np.max(excess) / max(np.sqrt(np.mean(r * r)), 1e-30))


def rel_err_bf16_out(gpu, ref) -> float:
    return rel_err_rounded_out(gpu, ref, "bf16")


def within_one_ulp(gpu, ref, fmt: str, abs_floor=1e-6) -> float:
    """Largest |gpu - ref| in units of the format's step at ref."""
    d = np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64))
    return float(np.max(d / (ulp(ref, fmt) + abs_floor)))


def within_one_bf16_ulp(gpu, ref, abs_floor=1e-6) -> float:
    """Largest |gpu - ref| in units of bf16 ulp(ref) (1 = one rounding step)."""
    d = np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64))
    return float(np.max(d / (bf16_ulp(ref) + abs_floor)))


def vt_layout(vt):
    """V^T [..., l_pad] rearranged into the attention kernel's key order: in
    each aligned group of 16 keys the quads are stored 0, 2, 1, 3 (stored
    position p holds key 16*(p//16) + 4*swap(p//4 % 4) + p%4, swap exchanging
    quads 1 and 2)."""
    n = vt.shape[-1]
    assert n % 16 == 0
    p = np.arange(n)
    quad = (p >> 2) & 3
    key = (p & ~15) | ((((quad & 1) << 1) | (quad >> 1)) << 2) | (p & 3)
    return vt[..., key]


def say(*a):
    """Print a progress line that names the case (flushed before GPU work)."""
    print(*a, file=sys.stderr, flush=True)


def sync():
    torch.cuda.synchronize()


def stream():
    return torch.cuda.current_stream()


# The fp8 matrix cores do not sum exactly: products far below the largest one
# of a dot product lose their low bits (measured on the GPU with exact e4m3
# operands: up to 2.4e-4 of the largest product, exact when all products share
# an exponent). With sharp attention a logit moved that much flips the e4m3
# code of a dominant probability by a whole step (6-12% of it).
MFMA_F8_SUM_ERR = 2.5e-4


def attention_fp8_perturbed(q, k, v, heads, eq, ek, rows=None, rng=None, bf16_inputs=True, bf16_qk=True):
    """The oracle's fp8 attention (oracle.attention_fp8, SGLang-AMD
    "Architecture Deep Dive": fp8 on CDNA) with the perturbations the HIP
    path applies to it: v (and, where q and k are not quantised in the QKV
    projection's epilogue, q and k) stored in bf16 ahead of the quantiser,
    and every logit moved uniformly within the fp8 matrix cores' summation
    error. Built from the oracle's own quantisers; how far it lands from the
    plain oracle is the method's sensitivity to that arithmetic."""
    import math
    import oracle as O
    from diffusion_transformer_image_mm_amd import synth
    rng = rng or np.random.default_rng(0)
    bf = lambda a: synth.bf16_exact(np.asarray(a, np.float32)).astype(np.float64)
    if bf16_inputs:
        v = bf(v)
        if bf16_qk:
            q, k = bf(q), bf(k)
    qc, kc = O.quantize_pow2_fp8(q, eq), O.quantize_pow2_fp8(k, ek)
    vc, sv = O.quantize_cols_fp8(v)
    L, HD = kc.shape
    D = HD // heads
    r = np.arange(qc.shape[0]) if rows is None else np.asarray(rows)
    c = math.log2(math.e) / math.sqrt(D) * 2.0 ** (eq + ek)
    out = np.empty((len(r), HD))
    for h in range(heads):
        sl = slice(h * D, (h + 1) * D)
        qs, ks = qc[r, sl], kc[:, sl]
        big = np.abs(qs[:, None, :].astype(np.float32) * ks[None, :, :].astype(np.float32)).max(-1)
        t = (qs @ ks.T + rng.uniform(-1.0, 1.0, big.shape) * MFMA_F8_SUM_ERR * big) * c
        pp = np.exp2(t - np.ceil(t.max(axis=1, keepdims=True)) + 8.0)
        out[:, sl] = (O.e4m3_round(pp) @ (vc[:, sl] * sv[sl][None, :])) / pp.sum(axis=1, keepdims=True)
    return out
