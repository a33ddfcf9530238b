"""Seeded synthetic inputs for the MM-DiT block workloads.

This module is shared by the tests, the benchmark and the smoke check: it is
the one thing the HIP path and the CPU oracle both consume. It holds none of
the method's arithmetic. It only draws random numbers, rounds them to
bf16-representable values (so that both sides read the same numbers), lays
them out, and builds the integer position ids of the joint token sequence.

Recipe (every tensor has its own seed stream, so adding a tensor never moves
the values of another):

* base seed 42, the seed the Luminal blog ("Reducing image generation cost
  with...", section "Setup") used on both GPUs;
* stream of tensor ``tid`` in workload ``cid`` = ``default_rng([42, cid,
  tid, chunk])`` over chunks of ``_CHUNK`` values, generated in a thread pool
  (the result does not depend on the number of threads);
* linear weights and biases N(0, 0.02); RMSNorm scales U(0.5, 1.5);
  residual activations, the conditioning vector, text states and the latent
  N(0, 1); every value rounded to bf16 (round to nearest even) and handed to
  both sides as float32 (oracle) and as raw bf16 bits (GPU);
* int8 weights: N(0, 0.02) draws quantised once here, symmetrically per
  output channel, s_n = max_k |W_nk| / 127, q = rint(W / s) clamped to
  [-127, 127]; both sides consume the same (q, s).

Position ids follow the axial (t, h, w) layout: text tokens sit at (0, 0, 0),
the image token at latent-patch grid cell (r, c) sits at (0, r, c), row-major,
and the joint sequence holds the text tokens first.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Tuple

import numpy as np

BASE_SEED = 42
_CHUNK = 1 << 22


# --------------------------------------------------------------------------
# workload shapes
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Shape:
    """Sizes of one MM-DiT workload (batch 1)."""

    name: str
    cid: int                # seed-stream id of the workload
    hidden: int             # H
    heads: int              # N_h
    head_dim: int           # D, H = N_h * D
    mlp: int                # MLP hidden width
    txt_len: int            # L_t
    grid: Tuple[int, int]   # latent patch grid (rows, cols); L_i = rows * cols
    axes: Tuple[int, int, int]  # RoPE axis widths (t, h, w), summing to D
    in_channels: int = 64   # latent channels per patch token
    n_double: int = 1
    n_single: int = 0
    theta: float = 10000.0
    ln_eps: float = 1e-6
    rms_eps: float = 1e-6
    mlp_act: str = "gelu"        # "gelu" (tanh form) or "swiglu" (fc1 rows [gate | up])
    guidance_embed: bool = True  # False: guidance-free conditioning (step-distilled)
    ref: bool = False            # image editing: a reference image of the same grid
    shared_mod: bool = False     # one set of modulation weights per block type

    @property
    def ref_len(self) -> int:
        return self.grid[0] * self.grid[1] if self.ref else 0

    @property
    def img_len(self) -> int:
        """Image-stream tokens: the output image, then the reference image."""
        return self.grid[0] * self.grid[1] + self.ref_len

    @property
    def mlp_out(self) -> int:
        """Output width of fc1 (and of linear1's MLP part)."""
        return 2 * self.mlp if self.mlp_act == "swiglu" else self.mlp

    @property
    def seq_len(self) -> int:
        return self.txt_len + self.img_len


def _axes_for(head_dim: int) -> Tuple[int, int, int]:
    """Axis widths (t, h, w): D/8 for time, the rest split evenly between the
    two spatial axes: (16, 56, 56) at D = 128, (8, 28, 28) at D = 64."""
    t = head_dim // 8
    hw = (head_dim - t) // 2
    assert t % 2 == 0 and hw % 2 == 0 and t + 2 * hw == head_dim, head_dim
    return (t, hw, hw)


TINY = Shape("tiny-double-h256-L320", 1, 256, 4, 64, 1024, 64, (16, 16), _axes_for(64))
FLUX_DOUBLE = Shape("flux-double-h3072-L4608", 2, 3072, 24, 128, 12288, 512, (64, 64), _axes_for(128))
FLUX_SINGLE = Shape("flux-single-h3072-L4608", 3, 3072, 24, 128, 12288, 512, (64, 64), _axes_for(128),
                    n_double=0, n_single=1)
QWEN_DOUBLE = Shape("qwen-double-h3072-L7145", 4, 3072, 24, 128, 12288, 256, (83, 83), _axes_for(128))
FLUX_STEP = Shape("flux-dev-step-19d38s-int8", 5, 3072, 24, 128, 12288, 512, (64, 64), _axes_for(128),
                  n_double=19, n_single=38)

# Flux.2 Klein 9B-shaped (Luminal blog, "Flux.2 Klein 9B"): H 4096, 32 heads,
# 8 double + 24 single blocks, SwiGLU MLP, 4 guidance-free steps, image-to-
# image editing with a 512-token prompt; the latent is 1/16 of the image per
# side with 128 channels, and the encoded input image (same size as the
# output) is appended to the image stream. MLP width 3H and modulation
# shared by the blocks of one type are readings (with them the parameter
# count comes to ~9 B).
KLEIN_KW = dict(mlp_act="swiglu", guidance_embed=False, ref=True, shared_mod=True, in_channels=128)
KLEIN_TINY = Shape("klein-tiny-h256-L192", 6, 256, 4, 64, 768, 64, (8, 8), _axes_for(64), n_double=1,
                   **KLEIN_KW)
KLEIN_512 = Shape("klein-double-h4096-512x512-L2560", 7, 4096, 32, 128, 12288, 512, (32, 32), _axes_for(128),
                  **KLEIN_KW)
KLEIN_704x864 = Shape("klein-double-h4096-704x864-L5264", 8, 4096, 32, 128, 12288, 512, (54, 44),
                      _axes_for(128), **KLEIN_KW)
KLEIN_1200x800 = Shape("klein-double-h4096-1200x800-L8012", 9, 4096, 32, 128, 12288, 512, (50, 75),
                       _axes_for(128), **KLEIN_KW)
KLEIN_STEP_512 = Shape("klein-step-8d24s-512x512", 10, 4096, 32, 128, 12288, 512, (32, 32), _axes_for(128),
                       n_double=8, n_single=24, **KLEIN_KW)

SHAPES = {s.name: s for s in (TINY, FLUX_DOUBLE, FLUX_SINGLE, QWEN_DOUBLE, FLUX_STEP, KLEIN_TINY, KLEIN_512,
                              KLEIN_704x864, KLEIN_1200x800, KLEIN_STEP_512)}


def custom_shape(name: str, cid: int, hidden: int, heads: int, mlp: int, txt_len: int,
                 grid: Tuple[int, int], **kw) -> Shape:
    """A shape for edge-case tests (ragged lengths, tiny sequences)."""
    d = hidden // heads
    return Shape(name, cid, hidden, heads, d, mlp, txt_len, grid, kw.pop("axes", _axes_for(d)), **kw)


# --------------------------------------------------------------------------
# bf16 helpers (data preparation only)
# --------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + r) >> 16).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bits to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_exact(x: np.ndarray) -> np.ndarray:
    """float32 array holding the bf16-rounded values of ``x``."""
    return bits_to_f32(bf16_bits(x))


def f16_exact(x: np.ndarray) -> np.ndarray:
    """float32 array holding the IEEE fp16-rounded values of ``x``."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


# --------------------------------------------------------------------------
# seeded draws
# --------------------------------------------------------------------------
def _workers() -> int:
    """Threads for the draws: the CPUs this process may run on, at most 16.
    Results do not depend on it (every chunk has its own seed stream)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _draw(cid: int, tid: int, n: int, kind: str, a: float, b: float) -> np.ndarray:
    """n seeded draws, each rounded to bf16 (elementwise, so the chunking
    and the thread count do not change the values)."""
    out = np.empty(n, dtype=np.float32)
    n_chunks = (n + _CHUNK - 1) // _CHUNK

    def fill(c: int) -> None:
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        rng = np.random.default_rng([BASE_SEED, cid, tid, c])
        if kind == "normal":
            v = rng.standard_normal(hi - lo, dtype=np.float32)
            if b != 1.0:
                v *= np.float32(b)
            if a != 0.0:
                v += np.float32(a)
        else:
            v = rng.uniform(a, b, hi - lo).astype(np.float32)
        out[lo:hi] = bf16_exact(v)

    if n_chunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(max_workers=_workers()) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


def normal(cid: int, tid: int, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    n = int(np.prod(shape))
    return _draw(cid, tid, n, "normal", mean, std).reshape(shape)


def uniform(cid: int, tid: int, shape, lo: float, hi: float) -> np.ndarray:
    n = int(np.prod(shape))
    return _draw(cid, tid, n, "uniform", lo, hi).reshape(shape)


def quantize_int8(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric per-output-channel int8 codes and fp32 scales of ``w`` [N, K]
    (row by row, so blocks of rows are done in parallel)."""
    N = w.shape[0]
    q = np.empty(w.shape, dtype=np.int8)
    s = np.empty(N, dtype=np.float32)

    def rows(r0: int) -> None:
        r1 = min(N, r0 + 1024)
        blk = w[r0:r1]
        amax = np.abs(blk).max(axis=1).astype(np.float32)
        sc = np.where(amax > 0, amax / np.float32(127.0), np.float32(1.0)).astype(np.float32)
        q[r0:r1] = np.clip(np.rint(blk / sc[:, None]), -127, 127).astype(np.int8)
        s[r0:r1] = sc

    starts = range(0, N, 1024)
    if N <= 1024:
        rows(0)
    else:
        with ThreadPoolExecutor(max_workers=_workers()) as ex:
            list(ex.map(rows, starts))
    return q, s


# --------------------------------------------------------------------------
# tensors of a workload
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Linear:
    """One linear layer: weight [out, in] and bias [out].

    ``w`` holds float32 bf16-exact values for a bf16 layer. For an int8 layer
    ``q`` holds the int8 codes and ``s`` the fp32 per-output-channel scale, and
    ``w`` is None (the oracle forms diag(s)·q itself).
    """

    w: Optional[np.ndarray]
    b: np.ndarray
    q: Optional[np.ndarray] = None
    s: Optional[np.ndarray] = None

    @property
    def out_features(self) -> int:
        return self.b.shape[0]

    @property
    def in_features(self) -> int:
        return (self.w if self.w is not None else self.q).shape[1]

    @property
    def is_int8(self) -> bool:
        return self.q is not None


class _Ids:
    """Hands out consecutive tensor ids within one workload."""

    def __init__(self, start: int = 0):
        self.next = start

    def __call__(self) -> int:
        t = self.next
        self.next += 1
        return t


def make_linear(cid: int, ids: _Ids, n_out: int, n_in: int, int8: bool = False,
                std: float = 0.02) -> Linear:
    w = normal(cid, ids(), (n_out, n_in), std)
    b = normal(cid, ids(), (n_out,), std)
    if int8:
        q, s = quantize_int8(w)
        return Linear(None, b, q, s)
    return Linear(w, b)


def stream_weights(cid: int, ids: _Ids, shp: Shape, int8: bool = False) -> Dict[str, object]:
    """Weights of one stream of a double-stream block."""
    H, M, D = shp.hidden, shp.mlp, shp.head_dim
    return {
        "mod": make_linear(cid, ids, 6 * H, H, int8),
        "qkv": make_linear(cid, ids, 3 * H, H, int8),
        "proj": make_linear(cid, ids, H, H, int8),
        "fc1": make_linear(cid, ids, shp.mlp_out, H, int8),
        "fc2": make_linear(cid, ids, H, M, int8),
        "q_norm": uniform(cid, ids(), (D,), 0.5, 1.5),
        "k_norm": uniform(cid, ids(), (D,), 0.5, 1.5),
    }


def double_weights(cid: int, ids: _Ids, shp: Shape, int8: bool = False) -> Dict[str, Dict[str, object]]:
    return {"txt": stream_weights(cid, ids, shp, int8), "img": stream_weights(cid, ids, shp, int8)}


def single_weights(cid: int, ids: _Ids, shp: Shape, int8: bool = False) -> Dict[str, object]:
    H, M, D = shp.hidden, shp.mlp, shp.head_dim
    return {
        "mod": make_linear(cid, ids, 3 * H, H, int8),
        "linear1": make_linear(cid, ids, 3 * H + shp.mlp_out, H, int8),
        "linear2": make_linear(cid, ids, H, H + M, int8),
        "q_norm": uniform(cid, ids(), (D,), 0.5, 1.5),
        "k_norm": uniform(cid, ids(), (D,), 0.5, 1.5),
    }


def position_ids(shp: Shape) -> np.ndarray:
    """int32 [L, 3] axial (t, h, w) ids: text at (0,0,0), image cell (r,c) at
    (0,r,c); the cells of a reference image (editing) at (1,r,c)."""
    rows, cols = shp.grid
    ids = np.zeros((shp.seq_len, 3), dtype=np.int32)
    r, c = np.meshgrid(np.arange(rows, dtype=np.int32), np.arange(cols, dtype=np.int32), indexing="ij")
    n = rows * cols
    for k in range(2 if shp.ref else 1):
        sl = slice(shp.txt_len + k * n, shp.txt_len + (k + 1) * n)
        ids[sl, 0] = k
        ids[sl, 1] = r.reshape(-1)
        ids[sl, 2] = c.reshape(-1)
    return ids


def block_inputs(shp: Shape, kind: str = "double", int8: bool = False,
                 variant: int = 0) -> Dict[str, object]:
    """Inputs of one block forward: residual x [L, H], conditioning vec [H],
    position ids, and the block's weights. ``variant`` selects a different
    seed stream (second draw of the same shape)."""
    cid = shp.cid * 16 + variant
    ids = _Ids()
    x = normal(cid, ids(), (shp.seq_len, shp.hidden))
    vec = normal(cid, ids(), (shp.hidden,))
    ids.next = 16
    if kind == "double":
        w = double_weights(cid, ids, shp, int8)
    elif kind == "single":
        w = single_weights(cid, ids, shp, int8)
    else:
        raise ValueError(kind)
    return {"shape": shp, "kind": kind, "x": x, "vec": vec, "ids": position_ids(shp), "w": w}


def model_weights(shp: Shape, int8: bool = True, variant: int = 0, progress=None) -> Dict[str, object]:
    """Weights of a whole denoiser: embedders, blocks and the final layer.
    ``progress(kind, i, n)``, if given, is called after each block."""
    cid = shp.cid * 16 + variant
    ids = _Ids(100)
    H, C = shp.hidden, shp.in_channels

    def blocks(kind, make, n):
        out = []
        for i in range(n):
            out.append(make(cid, ids, shp, int8))
            if progress is not None:
                progress(kind, i + 1, n)
        return out

    m = {
        "img_in": make_linear(cid, ids, H, C, int8),
        "time_in": [make_linear(cid, ids, H, 256, int8), make_linear(cid, ids, H, H, int8)],
        "guid_in": ([make_linear(cid, ids, H, 256, int8), make_linear(cid, ids, H, H, int8)]
                    if shp.guidance_embed else None),
        "final_mod": make_linear(cid, ids, 2 * H, H, int8),
        "final_out": make_linear(cid, ids, C, H, int8),
        "double": blocks("double", double_weights, shp.n_double),
        "single": blocks("single", single_weights, shp.n_single),
    }
    if shp.shared_mod:
        # every block of a type uses the first block's modulation weights
        for w in m["double"][1:]:
            w["txt"]["mod"], w["img"]["mod"] = m["double"][0]["txt"]["mod"], m["double"][0]["img"]["mod"]
        for w in m["single"][1:]:
            w["mod"] = m["single"][0]["mod"]
    return m


def step_inputs(shp: Shape, variant: int = 0) -> Dict[str, object]:
    """Latent z0 [L_i, C] (with the reference rows last when editing) and
    text states [L_t, H] of a denoise step."""
    cid = shp.cid * 16 + variant
    ids = _Ids(90)
    z = normal(cid, ids(), (shp.img_len, shp.in_channels))
    txt = normal(cid, ids(), (shp.txt_len, shp.hidden))
    return {"z": z, "txt": txt, "ids": position_ids(shp)}


def sigma_schedule(n_steps: int) -> List[float]:
    """Time grid t_i = 1 - i / n_steps, i = 0..n_steps (linear, no shift)."""
    return [1.0 - i / n_steps for i in range(n_steps + 1)]


def rand_array(cid: int, tid: int, shape, std: float = 1.0) -> np.ndarray:
    """A generic seeded N(0, std^2) bf16-exact array (per-kernel tests)."""
    return normal(cid, tid, shape, std)
