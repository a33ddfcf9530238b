"""CPU oracle of the MM-DiT block, the single-stream block and the denoise step.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module. The product path (the
HIP library and its binding) never calls it, and shares no code with it.

Plain, slow, obviously correct numpy in float64: every dot product, mean and
softmax sum is taken in fp64 from the bf16-exact inputs, with no intermediate
rounding, no tiling and no fusion. A numpy matrix product is used as the one
library primitive (the definition of a linear layer).

Sources (cited by page title and section):

* Luminal blog, "Reducing image generation cost with...":
  - section "What the compiler found on its own": a matrix product is a
    broadcast multiply and a sum; attention is two such products, a scale, a
    max, an exponent, a sum and a divide; RMSNorm is a square, a sum, a
    reciprocal square root and a multiply; LayerNorm adds a mean and a
    subtraction; the adaLN modulation after it is a scale and a shift; RoPE
    multiplies each element and its partner against cosine and sine tables;
    a gate-and-residual add follows each branch; the text and image streams
    are concatenated; a timestep embedding conditions the blocks.
  - section "Flux.2 Klein 9B": a double-stream block has its own projections
    before the attention and its own norm and feed-forward network after it,
    per stream; a single-stream block shares them.
  - section "The AMD MI300X pipeline": bf16 GEMMs accumulate in fp32 (here:
    fp64, a superset); the Euler sampler integrates the latent in fp32.
* flux-amd-rocm benchmarks page (header): FLUX.1-dev at 28 steps, guidance
  3.5, int8 weight-only linears.

Readings where the pages are silent (each one is also listed in the design
notes): GELU in its tanh form; LayerNorm without affine, biased variance,
eps 1e-6; adaLN as (1 + scale) * LN(x) + shift; SiLU on the conditioning
vector before every modulation linear; RoPE on adjacent pairs (2j, 2j+1),
axes (t, h, w) in that order, theta 1e4, applied after RMSNorm; no attention
mask; text tokens first in the joint sequence; a bias on every linear;
timestep embedding of width 256 over 1000 * t, max period 1e4, [cos | sin].

Chunk orders (conventions, weights are random): double-block modulation
[shift1, scale1, gate1, shift2, scale2, gate2]; single-block [shift, scale,
gate]; final layer [shift, scale]; qkv columns [q | k | v], each head-major
(column h * D + d); linear1 columns [q | k | v | mlp]; linear2 input
[attention | GELU(mlp)].
"""
from __future__ import annotations

import math
from collections import Counter
from typing import Optional, Sequence

import numpy as np

# Counts how many times each normalisation / attention site runs, so that a
# test can compare the block structure with the launch counts the Luminal
# blog reports per diffusion step.
SITE_COUNTS: Counter = Counter()


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# elementwise functions
# --------------------------------------------------------------------------
def silu(x):
    """SiLU(x) = x / (1 + e^-x)."""
    x = _f64(x)
    return x / (1.0 + np.exp(-x))


def gelu_tanh(x):
    """GELU, tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    x = _f64(x)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


# --------------------------------------------------------------------------
# linear layers ("What the compiler found on its own": multiply then sum)
# --------------------------------------------------------------------------
def swiglu(u) -> np.ndarray:
    """Gated linear unit with SiLU (the fused SwiGLU activation that the
    Luminal blog's section "What the compiler found on its own" names for
    Flux.2 Klein): u = [gate | up] (two halves of the columns) ->
    SiLU(gate) * up."""
    u = _f64(u)
    m = u.shape[-1] // 2
    return silu(u[..., :m]) * u[..., m:]


def mlp_activation(u, act: str) -> np.ndarray:
    return swiglu(u) if act == "swiglu" else gelu_tanh(u)


def weight_matrix(lin) -> np.ndarray:
    """The layer's weight as fp64: W itself, or diag(s) Q for an int8 layer
    (flux-amd-rocm benchmarks page: int8 weight-only linears)."""
    if lin.q is not None:
        return _f64(lin.s)[:, None] * _f64(lin.q)
    return _f64(lin.w)


def linear(x, lin) -> np.ndarray:
    """y = x W^T + b, for x [..., in]."""
    return _f64(x) @ weight_matrix(lin).T + _f64(lin.b)


# --------------------------------------------------------------------------
# normalisations ("What the compiler found on its own")
# --------------------------------------------------------------------------
def layer_norm(x, eps: float) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) over the last axis, biased var, no affine."""
    x = _f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    d = x - mu
    var = (d * d).mean(axis=-1, keepdims=True)
    return d / np.sqrt(var + eps)


def modulate(y, shift, scale) -> np.ndarray:
    """adaLN modulation: y * (1 + scale) + shift."""
    return _f64(y) * (1.0 + _f64(scale)) + _f64(shift)


def ln_modulate(x, shift, scale, eps: float) -> np.ndarray:
    """One LayerNorm + modulate site."""
    SITE_COUNTS["ln_modulate"] += 1
    return modulate(layer_norm(x, eps), shift, scale)


def rms_norm(u, g, eps: float) -> np.ndarray:
    """u / sqrt(mean(u^2) + eps) * g over the last axis (one head's D values)."""
    u = _f64(u)
    ms = (u * u).mean(axis=-1, keepdims=True)
    return u / np.sqrt(ms + eps) * _f64(g)


# --------------------------------------------------------------------------
# axial rotary embedding ("What the compiler found on its own": a partner
# gather and a multiply-add against cosine and sine tables)
# --------------------------------------------------------------------------
def rope_angles(ids, axes: Sequence[int], theta: float) -> np.ndarray:
    """Angles phi [L, D/2]. Pair p belongs to axis a (segments t, h, w of the
    head dim in that order); its j-th pair in that axis turns by
    pos_a * theta^(-2j / d_a)."""
    ids = np.asarray(ids)
    cols = []
    for a, d_a in enumerate(axes):
        j = np.arange(d_a // 2, dtype=np.float64)
        freq = theta ** (-2.0 * j / d_a)
        cols.append(ids[:, a].astype(np.float64)[:, None] * freq[None, :])
    return np.concatenate(cols, axis=1)


def apply_rope(u, phi) -> np.ndarray:
    """Rotate adjacent pairs (u_2j, u_2j+1) of u [L, D] by phi [L, D/2]."""
    u = _f64(u)
    u0, u1 = u[:, 0::2], u[:, 1::2]
    c, s = np.cos(phi), np.sin(phi)
    out = np.empty_like(u)
    out[:, 0::2] = u0 * c - u1 * s
    out[:, 1::2] = u0 * s + u1 * c
    return out


def qk_norm_rope(u, g, phi, eps: float) -> np.ndarray:
    """One fused RMSNorm + RoPE site: per token, RMSNorm over the head dim, then
    the rotation. u [L, D] for one head."""
    return apply_rope(rms_norm(u, g, eps), phi)


# --------------------------------------------------------------------------
# attention ("What the compiler found on its own": two multiply-sums, a scale,
# a max, an exponent, another sum and a divide; no mask in the transformer)
# --------------------------------------------------------------------------
def softmax_rows(s) -> np.ndarray:
    s = _f64(s)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def attention_head(q, k, v, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """softmax(q k^T / sqrt(D)) v for one head; q, k, v [L, D]. With ``rows``
    only those query rows are evaluated (each output row depends on its own
    query and on every key and value)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    if rows is not None:
        q = q[rows]
    s = (q @ k.T) / math.sqrt(q.shape[-1])
    return softmax_rows(s) @ v


def attention(q, k, v, heads: int, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Multi-head attention over [L, heads*D] tensors, heads side by side."""
    SITE_COUNTS["attention"] += 1
    L, HD = _f64(k).shape
    D = HD // heads
    n = L if rows is None else len(rows)
    out = np.empty((n, HD), dtype=np.float64)
    for h in range(heads):
        sl = slice(h * D, (h + 1) * D)
        out[:, sl] = attention_head(q[:, sl], k[:, sl], v[:, sl], rows)
    return out


# --------------------------------------------------------------------------
# block pieces
# --------------------------------------------------------------------------
def modulation(vec, lin, chunks: int):
    """SiLU(vec) W^T + b, split into ``chunks`` equal parts of width H."""
    m = linear(silu(vec)[None, :], lin)[0]
    return np.split(m, chunks)


def norm_rope_heads(u, g, phi, heads: int, eps: float) -> np.ndarray:
    """Apply RMSNorm + RoPE to every head of u [L, heads*D] (one site)."""
    SITE_COUNTS["rmsnorm_rope"] += 1
    L, HD = u.shape
    D = HD // heads
    out = np.empty((L, HD), dtype=np.float64)
    for h in range(heads):
        sl = slice(h * D, (h + 1) * D)
        out[:, sl] = qk_norm_rope(u[:, sl], g, phi, eps)
    return out


def double_block(x, vec, ids, w, shp, rows: Optional[np.ndarray] = None,
                 return_stages: bool = False, fp8: bool = False):
    """Double-stream block ("Flux.2 Klein 9B" and "What the compiler found on
    its own" sections of the Luminal blog).

    x [L, H] holds the text rows first, then the image rows. For each stream s
    with its own weights:
      m_s = modulation(vec) -> shift1, scale1, gate1, shift2, scale2, gate2
      h_s = LN(x_s) * (1 + scale1) + shift1
      q_s, k_s, v_s = split(h_s W_qkv^T + b)
      q_s, k_s = RMSNorm per head (per-stream scales)
    then over the joint sequence: RoPE, attention; then per stream
      x_s += gate1 * (O_s W_proj^T + b)
      x_s += gate2 * (GELU(LN(x_s) * (1 + scale2) + shift2) W_fc1^T + b) W_fc2^T + b)
    With ``rows`` only those output rows are returned (all keys and values
    are still computed). With ``fp8`` every linear takes its fp8 form
    (``fp8_weights``, ``linear_act_fp8``): projections on per-token fp8
    activations, the modulation on the fp8 weights alone; the attention is
    ``attention_fp8`` with the power-of-two scales the two streams' q and k
    norm scales bound (``qk_fp8_exponent``).
    """
    H, heads, L_t = shp.hidden, shp.heads, shp.txt_len
    lin = linear_act_fp8 if fp8 else linear
    if fp8:
        w = fp8_weights(w)
    x = _f64(x)
    L = x.shape[0]
    phi = rope_angles(ids, shp.axes, shp.theta)
    seg = {"txt": slice(0, L_t), "img": slice(L_t, L)}
    mods = {s: modulation(vec, w[s]["mod"], 6) for s in seg}
    q = np.empty((L, H)); k = np.empty((L, H)); v = np.empty((L, H))
    stages = {}
    for s, sl in seg.items():
        sh1, sc1 = mods[s][0], mods[s][1]
        h = ln_modulate(x[sl], sh1, sc1, shp.ln_eps)
        qkv = lin(h, w[s]["qkv"])
        q[sl], k[sl], v[sl] = qkv[:, :H], qkv[:, H:2 * H], qkv[:, 2 * H:]
        stages[f"h1_{s}"] = h
        stages[f"qkv_{s}"] = qkv
    # RMSNorm + RoPE: q and k of each stream are normalised with that stream's
    # scales; the rotation uses the joint positions.
    for s, sl in seg.items():
        q[sl] = norm_rope_heads(q[sl], w[s]["q_norm"], phi[sl], heads, shp.rms_eps)
        k[sl] = norm_rope_heads(k[sl], w[s]["k_norm"], phi[sl], heads, shp.rms_eps)
    stages["q"], stages["k"], stages["v"] = q, k, v
    out_rows = np.arange(L) if rows is None else np.asarray(rows)
    if fp8:
        D = H // heads
        eq = qk_fp8_exponent([w["txt"]["q_norm"], w["img"]["q_norm"]], D)
        ek = qk_fp8_exponent([w["txt"]["k_norm"], w["img"]["k_norm"]], D)
        o = attention_fp8(q, k, v, heads, eq, ek, out_rows)
    else:
        o = attention(q, k, v, heads, out_rows)
    stages["attn"] = o
    xo = x[out_rows].copy()
    is_txt = out_rows < L_t
    for s, mask in (("txt", is_txt), ("img", ~is_txt)):
        if not mask.any():
            continue
        sh1, sc1, g1, sh2, sc2, g2 = mods[s]
        xs = xo[mask] + g1 * lin(o[mask], w[s]["proj"])
        h2 = ln_modulate(xs, sh2, sc2, shp.ln_eps)
        a = mlp_activation(lin(h2, w[s]["fc1"]), shp.mlp_act)
        xs = xs + g2 * lin(a, w[s]["fc2"])
        xo[mask] = xs
    if return_stages:
        stages["mods"] = mods
        return xo, stages
    return xo


def single_block(x, vec, ids, w, shp, rows: Optional[np.ndarray] = None,
                 return_stages: bool = False, fp8: bool = False):
    """Single-stream block: one set of weights over the joint sequence.
      shift, scale, gate = modulation(vec)
      u = (LN(x) * (1 + scale) + shift) W_1^T + b_1 -> q | k | v | m
      q, k = RMSNorm per head, then RoPE; O = attention(q, k, v)
      x += gate * ([O | GELU(m)] W_2^T + b_2)
    ``fp8`` as for ``double_block``.
    """
    H, heads = shp.hidden, shp.heads
    lin = linear_act_fp8 if fp8 else linear
    if fp8:
        w = fp8_weights(w)
    x = _f64(x)
    L = x.shape[0]
    phi = rope_angles(ids, shp.axes, shp.theta)
    sh, sc, g = modulation(vec, w["mod"], 3)
    h = ln_modulate(x, sh, sc, shp.ln_eps)
    u = lin(h, w["linear1"])
    q, k, v, m = u[:, :H], u[:, H:2 * H], u[:, 2 * H:3 * H], u[:, 3 * H:]
    q = norm_rope_heads(q, w["q_norm"], phi, heads, shp.rms_eps)
    k = norm_rope_heads(k, w["k_norm"], phi, heads, shp.rms_eps)
    out_rows = np.arange(L) if rows is None else np.asarray(rows)
    if fp8:
        D = H // heads
        o = attention_fp8(q, k, v, heads, qk_fp8_exponent([w["q_norm"]], D),
                          qk_fp8_exponent([w["k_norm"]], D), out_rows)
    else:
        o = attention(q, k, v, heads, out_rows)
    cat = np.concatenate([o, mlp_activation(m[out_rows], shp.mlp_act)], axis=1)
    xo = x[out_rows] + g * lin(cat, w["linear2"])
    if return_stages:
        return xo, {"h": h, "u": u, "q": q, "k": k, "v": v, "attn": o, "mod": (sh, sc, g)}
    return xo


# --------------------------------------------------------------------------
# denoise step
# --------------------------------------------------------------------------
def timestep_embedding(t: float, dim: int = 256, max_period: float = 10000.0,
                       time_factor: float = 1000.0) -> np.ndarray:
    """Sinusoidal embedding of a scalar: [cos(1000 t f_k) | sin(1000 t f_k)],
    f_k = exp(-ln(max_period) k / (dim/2)), k < dim/2."""
    half = dim // 2
    f = np.exp(-math.log(max_period) * np.arange(half, dtype=np.float64) / half)
    a = time_factor * float(t) * f
    return np.concatenate([np.cos(a), np.sin(a)])


def mlp_embedder(e, lins) -> np.ndarray:
    """Linear(256 -> H), SiLU, Linear(H -> H)."""
    return linear(silu(linear(e[None, :], lins[0])), lins[1])[0]


def conditioning(t: float, guidance: float, m) -> np.ndarray:
    """vec = MLP_t(emb(t)) + MLP_g(emb(guidance)); a guidance-free model
    (m["guid_in"] None: the step-distilled Flux.2 Klein of the Luminal blog)
    has only the time term."""
    vec = mlp_embedder(timestep_embedding(t), m["time_in"])
    if m.get("guid_in") is not None:
        vec = vec + mlp_embedder(timestep_embedding(guidance), m["guid_in"])
    return vec


def euler(z, v, t_cur: float, t_next: float) -> np.ndarray:
    """Flow-matching Euler update z <- z + (t_next - t_cur) v."""
    return _f64(z) + (float(t_next) - float(t_cur)) * _f64(v)


def velocity(z, txt, ids, m, shp, t_cur: float, guidance: float, fp8: bool = False) -> np.ndarray:
    """The denoiser's prediction v for latent z [L_i, C] and text states
    txt [L_t, H]: embed, run the double then the single blocks, and apply the
    final modulated LayerNorm and projection to the image rows. When editing,
    the last ``shp.ref_len`` rows of z are the encoded reference image: they
    are embedded and attended to like the others, and v covers only the rows
    before them. With ``fp8`` every linear takes its fp8 form
    (``fp8_weights``): the blocks' projections on per-token fp8 activations
    (``double_block`` / ``single_block`` with ``fp8``), the embedders, the
    modulations and the final projection on the fp8 weights alone."""
    if fp8:
        m = fp8_weights(m)
    vec = conditioning(t_cur, guidance, m)
    x = np.concatenate([_f64(txt), linear(z, m["img_in"])], axis=0)
    for wd in m["double"]:
        x = double_block(x, vec, ids, wd, shp, fp8=fp8)
    for ws in m["single"]:
        x = single_block(x, vec, ids, ws, shp, fp8=fp8)
    sh, sc = modulation(vec, m["final_mod"], 2)
    n = shp.img_len - shp.ref_len
    h = ln_modulate(x[shp.txt_len:shp.txt_len + n], sh, sc, shp.ln_eps)
    return linear(h, m["final_out"])


def denoise_step(z, txt, ids, m, shp, t_cur: float, t_next: float, guidance: float, fp8: bool = False):
    """One flow-matching Euler step of the latent; returns (z_next, v). The
    reference rows of an edit (the last shp.ref_len) are carried unchanged.
    ``fp8`` as for ``velocity``."""
    v = velocity(z, txt, ids, m, shp, t_cur, guidance, fp8=fp8)
    z_next = _f64(z).copy()
    n = shp.img_len - shp.ref_len
    z_next[:n] = euler(z[:n], v, t_cur, t_next)
    return z_next, v


# --------------------------------------------------------------------------
# fp8 (OCP e4m3) quantisation: the fp8 variant of the linears
# --------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_round(x) -> np.ndarray:
    """Round to the nearest OCP fp8 e4m3 value, ties to the even mantissa.
    e4m3: 4 exponent bits (bias 7), 3 mantissa bits; normal values
    (1 + m/8) 2^(e-7) for e = 1..15 (e = 15, m = 7 is NaN, so the largest
    finite value is 1.75 * 2^8 = 448); subnormals (m/8) 2^-6, a step of 2^-9.
    Inputs must lie within +-(448 + half a step), the quantiser's range."""
    x = _f64(x)
    a = np.abs(x)
    assert np.all(a < 464.0), "outside the e4m3 range this quantiser produces"
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)          # below 2^-6 the spacing stays 2^-9
    step = np.exp2(e - 3.0)
    return np.round(x / step) * step  # np.round: half to even; x / step is exact


def quantize_rows_fp8(x):
    """Per-row fp8 quantisation as the fp8 linears use it: the row's scale is
    max|x| / 448 and its codes e4m3(x / scale), both divisions in fp32 (the
    precision the kernels take these decisions in); an all-zero row gets scale
    0 and zero codes. Returns (code values [rows, cols] float64, scales fp32)."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=1).astype(np.float32)
    sc = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(sc > 0, sc, np.float32(1.0)).astype(np.float32)
    q = (x32 / safe[:, None]).astype(np.float32)
    codes = np.where(sc[:, None] > 0, e4m3_round(q), 0.0)
    return codes, sc


def linear_fp8(a_codes, a_scale, w_codes, w_scale, bias) -> np.ndarray:
    """y = (diag(a_scale) A) (diag(w_scale) W)^T + b from the decoded fp8
    codes, in fp64."""
    a = _f64(a_scale)[:, None] * _f64(a_codes)
    w = _f64(w_scale)[:, None] * _f64(w_codes)
    return a @ w.T + _f64(bias)[None, :]


class Fp8Linear:
    """A linear layer in its fp8 form: e4m3 code values q [out, in] (decoded,
    float64) with one fp32 scale per output channel s, and the layer's bias.
    ``weight_matrix`` reads it as diag(s) q."""

    def __init__(self, q, s, b):
        self.w, self.q, self.s, self.b = None, q, s, b


def fp8_weights(w):
    """The fp8 form of a block's weights ("Architecture Deep Dive": fp8 on
    CDNA): every 16-bit weight matrix quantised per output channel exactly as
    activations are per token (``quantize_rows_fp8``); biases and norm scales
    stay as they are. Nested dicts and lists are mapped; layers already in
    fp8 form (and int8 layers) pass through unchanged."""
    if isinstance(w, dict):
        return {k: fp8_weights(v) for k, v in w.items()}
    if isinstance(w, list):
        return [fp8_weights(v) for v in w]
    if getattr(w, "w", None) is None or not hasattr(w, "b"):
        return w
    codes, sc = quantize_rows_fp8(w.w)
    return Fp8Linear(codes, sc, w.b)


def linear_act_fp8(x, lin) -> np.ndarray:
    """A projection of the fp8 path: the activation rows x (the oracle's own
    fp64 values) quantised per token (``quantize_rows_fp8``: scale and code
    decided in fp32, the precision the kernels decide them in), times the fp8
    weights."""
    codes, sc = quantize_rows_fp8(np.asarray(x, dtype=np.float64))
    return linear_fp8(codes, sc, lin.q, lin.s, lin.b)


# --------------------------------------------------------------------------
# fp8 attention (SGLang-AMD, "Architecture Deep Dive": fp8 on CDNA; the
# fp8 path runs the attention products on fp8 operands as well)
# --------------------------------------------------------------------------
def qk_fp8_exponent(norm_scales, head_dim: int) -> int:
    """Exponent e of the power-of-two per-tensor scale 2^e of the fp8
    queries (or keys). After RMSNorm a row's mean square is below 1, so its
    2-norm is below sqrt(D); the norm scale g multiplies each element by at
    most max|g|, and RoPE rotates pairs without changing the norm. Every
    element therefore satisfies |x_d| <= sqrt(D) max|g|, and e is the
    smallest integer with 2^e >= b, b = fl32(fl32(sqrt(D) / 448) * max|g|)
    over all the given norm-scale vectors (both streams of a double block):
    no code can exceed 448."""
    gmax = np.float32(max(float(np.max(np.abs(_f64(g)))) for g in norm_scales))
    f = np.float32(math.sqrt(head_dim) / E4M3_MAX)
    b = float(np.float32(f * gmax))
    m, e = math.frexp(b)            # b = m 2^e, 0.5 <= m < 1 (m = 0 for b = 0)
    return e - 1 if m == 0.5 else e


def quantize_pow2_fp8(x, e: int) -> np.ndarray:
    """e4m3 code values of x at the scale 2^e: e4m3(x 2^-e), the scaling exact
    (x taken as fp32, the precision the kernels hold it in before this)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    return e4m3_round(x * 2.0 ** (-e))


def quantize_cols_fp8(v):
    """Per-channel fp8 quantisation of v [L, C]: one scale per column,
    max over the column's rows of |v| / 448, codes e4m3(v / scale) (both in
    fp32, as ``quantize_rows_fp8`` on v^T). Returns (codes [L, C], scales [C])."""
    codes, sc = quantize_rows_fp8(np.asarray(v, dtype=np.float64).T)
    return codes.T, sc


def attention_fp8(q, k, v, heads: int, eq: int, ek: int,
                  rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Multi-head attention of the fp8 path over [L, heads*D] tensors:
      * q and k as e4m3 codes at the per-tensor scales 2^eq and 2^ek
        (``quantize_pow2_fp8``), v as e4m3 codes with one fp32 scale per
        channel (``quantize_cols_fp8``);
      * logits in log2 units t_ij = (q8_i . k8_j) 2^(eq+ek) log2(e) / sqrt(D);
      * the exponentials p_ij = 2^(t_ij - M_i + 8), M_i the smallest integer
        >= max_j t_ij, so p lies in [0, 256]; the probabilities enter the
        second product as their e4m3 code values P8 = e4m3(p);
      * O_i = sum_j P8_ij v8_j diag(sv) / sum_j p_ij, the row sum over the
        unquantised exponentials.
    Reading: the pages name fp8 only as a capability of the stack; the integer
    reference M_i makes the codes independent of which integer at or above
    the maximum a tiled evaluation uses (scaling by a power of two commutes
    with e4m3 rounding in its normal range)."""
    SITE_COUNTS["attention"] += 1
    qc, kc = quantize_pow2_fp8(q, eq), quantize_pow2_fp8(k, ek)
    vc, sv = quantize_cols_fp8(v)
    L, HD = kc.shape
    D = HD // heads
    r = np.arange(qc.shape[0]) if rows is None else np.asarray(rows)
    c = math.log2(math.e) / math.sqrt(D) * 2.0 ** (eq + ek)
    out = np.empty((len(r), HD), dtype=np.float64)
    for h in range(heads):
        sl = slice(h * D, (h + 1) * D)
        t = (qc[r, sl] @ kc[:, sl].T) * c
        M = np.ceil(t.max(axis=1, keepdims=True))
        p = np.exp2(t - M + 8.0)
        out[:, sl] = (e4m3_round(p) @ (vc[:, sl] * _f64(sv[sl])[None, :])) / p.sum(axis=1, keepdims=True)
    return out
