"""Per-kernel parity of the HIP path against the CPU oracle, through the C ABI.

Every case feeds both sides the same seeded bf16-exact inputs. Sizes span
several tiles and ragged tails; the full-size cases check sampled outputs."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from diffusion_transformer_image_mm_amd import binding as B
from diffusion_transformer_image_mm_amd import synth
from gpu_helpers import (TOL, DeviceArena, rel_err, rel_err_bf16_out, rel_err_rounded_out, say, stream, sync,
                         to_numpy_f32, vt_layout, within_one_bf16_ulp, within_one_ulp)

pytestmark = pytest.mark.gpu
CID = 700


def rnd(tid, shape, std=1.0, cid=CID):
    return synth.rand_array(cid, tid, shape, std)


# ------------------------------------------------------------------ LN + modulate
@pytest.mark.parametrize("rows,hidden,split", [(320, 256, 64), (7, 64, 3), (1000, 3072, 512), (4608, 3072, 512),
                                               (9, 960, 4), (257, 1536, 100), (5, 2048, 2),
                                               (33, 4096, 40)])
def test_ln_modulate(rows, hidden, split):
    say(f"ln_modulate rows={rows} hidden={hidden} split={split}")
    A = DeviceArena()
    x = rnd(1, (rows, hidden)) * 3 + rnd(2, (rows, 1))
    sh = rnd(3, (2, hidden), 0.7)
    sc = rnd(4, (2, hidden), 0.7)
    dx, dsh, dsc = A.f32(x), A.f32(sh), A.f32(sc)
    out = A.empty_f16(rows, hidden)
    B.check(B.mmdit_k_ln_modulate(dx, rows, hidden, split, dsh[0], dsc[0], dsh[1], dsc[1], 1e-6, out, stream()))
    sync()
    g = to_numpy_f32(out)
    ref = np.empty((rows, hidden))
    s = min(split, rows)
    ref[:s] = O.ln_modulate(x[:s], sh[0], sc[0], 1e-6)
    ref[s:] = O.ln_modulate(x[s:], sh[1], sc[1], 1e-6)
    assert rel_err(g, ref) <= TOL
    assert rel_err_rounded_out(g, ref, "f16") <= 1e-4
    assert within_one_ulp(g, ref, "f16") <= 1.0  # one rounding of an fp32 result


def test_ln_modulate_fp16_range_overflows_to_inf():
    """The projections' activation operands are fp16 (range +-65504): a
    LayerNorm output pushed past it by a huge modulation scale is stored as
    +-inf (IEEE round to nearest: |y| >= 65520), not clamped, so the overflow
    shows downstream as a non-finite result. Values inside the range stay
    within one fp16 step of the oracle."""
    say("ln_modulate fp16 range")
    rows, hidden = 8, 256
    A = DeviceArena()
    x = rnd(1, (rows, hidden))
    sh = np.zeros((2, hidden))
    sc = np.zeros((2, hidden))
    sc[:, :32] = 1e5                       # (1 + scale) * LN(x): up to ~3e5 in these columns
    dx, dsh, dsc = A.f32(x), A.f32(sh), A.f32(sc)
    out = A.empty_f16(rows, hidden)
    B.check(B.mmdit_k_ln_modulate(dx, rows, hidden, rows, dsh[0], dsc[0], dsh[1], dsc[1], 1e-6, out, stream()))
    sync()
    g = to_numpy_f32(out)
    ref = O.ln_modulate(x, sh[0], sc[0], 1e-6)
    over = np.abs(ref) >= 65520.0 * (1 + 1e-6)
    under = np.abs(ref) <= 65504.0 * (1 - 1e-6)
    assert over.sum() > 10 and under.sum() > 0
    assert np.all(np.isinf(g[over])) and np.all(np.sign(g[over]) == np.sign(ref[over]))
    assert np.all(np.isfinite(g[under]))
    assert within_one_ulp(g[under], ref[under], "f16") <= 1.0


# ------------------------------------------------------------------ RoPE table
@pytest.mark.parametrize("shape", [synth.TINY, synth.QWEN_DOUBLE])
def test_rope_table(shape):
    say(f"rope_table {shape.name}")
    A = DeviceArena()
    from diffusion_transformer_image_mm_amd.device import dims_for
    d = dims_for(shape)
    ids = synth.position_ids(shape)
    dids = A.i32(ids)
    rope = A.empty_f32(shape.seq_len, shape.head_dim // 2, 2)
    B.check(B.mmdit_rope_table(d, dids, rope, stream()))
    sync()
    g = rope.cpu().numpy()
    phi = O.rope_angles(ids, shape.axes, shape.theta)
    np.testing.assert_allclose(g[..., 0], np.cos(phi), rtol=0, atol=2e-7)
    np.testing.assert_allclose(g[..., 1], np.sin(phi), rtol=0, atol=2e-7)


# ------------------------------------------------------------------ QK norm + RoPE
def _rope_host(ids, axes, theta):
    phi = O.rope_angles(ids, axes, theta)
    return np.stack([np.cos(phi), np.sin(phi)], axis=-1).astype(np.float32)


@pytest.mark.parametrize("D,heads,txt,grid", [(64, 4, 64, (16, 16)), (128, 3, 5, (7, 9)), (128, 24, 512, (64, 64)),
                                              (64, 2, 1, (1, 1))])
def test_qknorm_rope(D, heads, txt, grid):
    say(f"qknorm_rope D={D} heads={heads} txt={txt} grid={grid}")
    A = DeviceArena()
    shp = synth.custom_shape("qk", CID, heads * D, heads, 64, txt, grid)
    L, H = shp.seq_len, shp.hidden
    l_pad = (L + 127) // 128 * 128
    qkv = rnd(10, (L, 3 * H))
    norms = [synth.uniform(CID, 11 + i, (D,), 0.5, 1.5) for i in range(4)]  # q0 k0 q1 k1
    ids = synth.position_ids(shp)
    rope = _rope_host(ids, shp.axes, shp.theta)
    dq = A.bf16(qkv)
    dn = [A.bf16(n) for n in norms]
    qo, ko, vo = (A.empty_bf16(heads, l_pad, D), A.empty_bf16(heads, l_pad, D), A.empty_bf16(heads, D, l_pad))
    for t in (qo, ko, vo):
        t.fill_(float("nan"))  # padding must be overwritten with zeros
    B.check(B.mmdit_k_qknorm_rope(dq, 3 * H, L, heads, D, txt, dn[0], dn[1], dn[2], dn[3], A.f32(rope), 1e-6,
                                  l_pad, qo, ko, vo, stream()))
    sync()
    gq, gk, gv = to_numpy_f32(qo), to_numpy_f32(ko), to_numpy_f32(vo)
    phi = O.rope_angles(ids, shp.axes, shp.theta)
    for which, g, n_t, n_i in (("q", gq, norms[0], norms[2]), ("k", gk, norms[1], norms[3])):
        off = 0 if which == "q" else H
        for h in range(heads):
            u = qkv[:, off + h * D: off + (h + 1) * D]
            ref = np.empty((L, D))
            ref[:txt] = O.qk_norm_rope(u[:txt], n_t, phi[:txt], 1e-6)
            ref[txt:] = O.qk_norm_rope(u[txt:], n_i, phi[txt:], 1e-6)
            assert rel_err_bf16_out(g[h, :L], ref) <= TOL
            # the fp32 rotation of an fp32-normalised value, rounded once; the
            # fp32 cos/sin table adds < 1e-7 relative
            assert within_one_bf16_ulp(g[h, :L], ref, abs_floor=1e-5) <= 1.0, (which, h)
        assert np.all(g[:, L:] == 0)
    v = np.zeros((heads, D, l_pad), np.float32)
    v[:, :, :L] = qkv[:, 2 * H:].reshape(L, heads, D).transpose(1, 2, 0)
    np.testing.assert_array_equal(gv, vt_layout(v))


# ------------------------------------------------------------------ attention
def _attention_case(D, heads, L, q_scale=1.0, rows=None, tid=20):
    A = DeviceArena()
    l_pad = (L + 127) // 128 * 128
    q = rnd(tid, (heads, L, D)) * q_scale
    k = rnd(tid + 1, (heads, L, D))
    v = rnd(tid + 2, (heads, L, D))
    qp = np.zeros((heads, l_pad, D), np.float32); qp[:, :L] = synth.bf16_exact(q)
    kp = np.zeros((heads, l_pad, D), np.float32); kp[:, :L] = k
    vt = np.zeros((heads, D, l_pad), np.float32); vt[:, :, :L] = v.transpose(0, 2, 1)
    vt = vt_layout(vt)
    H = heads * D
    out = A.empty_f16(L, H)
    B.check(B.mmdit_k_attention(A.bf16(qp), A.bf16(kp), A.bf16(vt), heads, L, D, l_pad, out, H, stream()))
    sync()
    g = to_numpy_f32(out)
    qe = synth.bf16_exact(q)
    sel = np.arange(L) if rows is None else rows
    worst = 0.0
    for h in range(heads):
        ref = O.attention_head(qe[h], k[h], v[h], rows=None if rows is None else rows)
        worst = max(worst, rel_err_rounded_out(g[sel, h * D:(h + 1) * D], ref, "f16"))
    return worst


@pytest.mark.parametrize("D,heads,L", [(64, 4, 320), (128, 2, 333), (128, 3, 64), (64, 2, 1), (128, 1, 129),
                                       (64, 1, 700)])
def test_attention_small(D, heads, L):
    say(f"attention D={D} heads={heads} L={L}")
    err = _attention_case(D, heads, L)
    assert err <= TOL, err


@pytest.mark.parametrize("D,heads,L", [(128, 2, 333), (64, 4, 320)])
def test_attention_sharp(D, heads, L):
    """Queries scaled x6: scores with std ~6, so a few keys dominate each row
    and a wrong key/value pairing would show."""
    say(f"attention sharp D={D} heads={heads} L={L}")
    err = _attention_case(D, heads, L, q_scale=6.0, tid=30)
    assert err <= TOL, err


@pytest.mark.parametrize("D,L,slope", [(64, 700, 0.5), (128, 333, 0.25), (128, 300, 0.01)])
def test_attention_growing_scores(D, L, slope):
    """Scores that grow along the key axis: with a large slope every key tile
    raises the row maximum by far more than 2^8 (the rescaling path runs on
    every tile); with a small one the running maximum stays stale for many
    tiles. Both must give the exact softmax."""
    say(f"attention growing scores D={D} L={L} slope={slope}")
    A = DeviceArena()
    heads, l_pad = 2, (L + 127) // 128 * 128
    base = rnd(50, (heads, L, D), 0.3)
    u = np.zeros(D, np.float32); u[0] = 1.0
    q = synth.bf16_exact(base + 4.0 * u)
    k = synth.bf16_exact(base[::-1] * 0.5 + (slope * np.arange(L, dtype=np.float32))[None, :, None] * u)
    v = rnd(52, (heads, L, D))
    qp = np.zeros((heads, l_pad, D), np.float32); qp[:, :L] = q
    kp = np.zeros((heads, l_pad, D), np.float32); kp[:, :L] = k
    vt = np.zeros((heads, D, l_pad), np.float32); vt[:, :, :L] = v.transpose(0, 2, 1)
    vt = vt_layout(vt)
    out = A.empty_f16(L, heads * D)
    B.check(B.mmdit_k_attention(A.bf16(qp), A.bf16(kp), A.bf16(vt), heads, L, D, l_pad, out, heads * D, stream()))
    sync()
    g = to_numpy_f32(out)
    for h in range(heads):
        ref = O.attention_head(q[h], k[h], v[h])
        assert rel_err_rounded_out(g[:, h * D:(h + 1) * D], ref, "f16") <= TOL


@pytest.mark.parametrize("L", [4608, 7145])
def test_attention_full_size_sampled_rows(L):
    say(f"attention full heads=24 D=128 L={L}")
    rng = np.random.default_rng(L)
    rows = np.unique(np.r_[0, 1, 127, 128, L - 129, L - 1, rng.integers(0, L, 90)])
    err = _attention_case(128, 24, L, rows=rows, tid=40)
    assert err <= TOL, err


# ------------------------------------------------------------------ GEMM
def _lin(tid, n, k, int8):
    w = rnd(tid, (n, k), 0.02)
    b = rnd(tid + 1, (n,), 0.02)
    if int8:
        q, s = synth.quantize_int8(w)
        return synth.Linear(None, b, q, s)
    return synth.Linear(w, b)


GEMM_CASES = [
    # m, n, k, epilogue, int8
    (320, 768, 256, B.MMDIT_EPI_BIAS, False),
    (1000, 320, 1280, B.MMDIT_EPI_BIAS, False),
    (513, 1024, 256, B.MMDIT_EPI_BIAS_GELU, False),
    (700, 256, 1024, B.MMDIT_EPI_GATE_RESID, False),
    (320, 1792, 256, B.MMDIT_EPI_SPLIT_GELU, False),
    (4096, 3072, 64, B.MMDIT_EPI_BIAS_F32, False),
    (4096, 64, 3072, B.MMDIT_EPI_EULER, False),
    (1, 128, 64, B.MMDIT_EPI_BIAS, False),
    (320, 768, 256, B.MMDIT_EPI_BIAS, True),
    (700, 256, 1024, B.MMDIT_EPI_GATE_RESID, True),
    (513, 1024, 256, B.MMDIT_EPI_BIAS_GELU, True),
    (4096, 64, 3072, B.MMDIT_EPI_EULER, True),
    (320, 1792, 256, B.MMDIT_EPI_SPLIT_GELU, True),
    # one k-step (K = 64): the int8 loop's prologue conversion and a single stage
    (513, 1024, 64, B.MMDIT_EPI_BIAS_GELU, True),
    (257, 3072, 64, B.MMDIT_EPI_GATE_RESID, True),
]


_RESID = [None]


def _run_gemm(m, n, k, epi, int8, rows=None, tid=50, f16=False):
    A = DeviceArena(f16_weights=f16)
    a = synth.f16_exact(rnd(tid, (m, k)))  # the fp16 activation operand both sides read
    lin = _lin(tid + 2, n, k, int8)
    da = A.f16(a)
    wt = B.MMDIT_INT8 if int8 else (B.MMDIT_F16 if f16 else B.MMDIT_BF16)
    g = B.mmdit_gemm(m=m, n=n, k=k, weight_dtype=wt, a=da.data_ptr(), lda=k, w=A.linear(lin), epilogue=epi)
    swiglu = epi in (B.MMDIT_EPI_SWIGLU, B.MMDIT_EPI_SPLIT_SWIGLU)
    if epi == B.MMDIT_EPI_SPLIT_GELU:
        split = 3 * n // 7 // 64 * 64
    elif epi == B.MMDIT_EPI_SPLIT_SWIGLU:
        split = (n // 3) // 256 * 256       # q|k|v part; the rest is [gate | up]
    elif epi == B.MMDIT_EPI_SWIGLU:
        split = n // 2                      # output width M
    else:
        split = n
    _SPLIT[0] = split
    gate = rnd(tid + 5, (n,), 0.7)
    resid = rnd(tid + 6, (m, n))
    f32out = epi in (B.MMDIT_EPI_GATE_RESID, B.MMDIT_EPI_BIAS_F32, B.MMDIT_EPI_EULER)
    if f32out:
        out = A.f32(resid) if epi == B.MMDIT_EPI_EULER else A.empty_f32(m, n)
    else:
        f16out = epi in (B.MMDIT_EPI_BIAS_GELU, B.MMDIT_EPI_SWIGLU)
        out = A.empty_f16(m, split) if f16out else A.empty_bf16(m, split)
    g.out, g.ldo = out.data_ptr(), (n if f32out else split)
    out2 = None
    if epi == B.MMDIT_EPI_GATE_RESID:
        g.gate, g.resid, g.ldr = A.f32(gate).data_ptr(), A.f32(resid).data_ptr(), n
    if epi in (B.MMDIT_EPI_SPLIT_GELU, B.MMDIT_EPI_SPLIT_SWIGLU):
        w2 = (n - split) // 2 if swiglu else n - split
        out2 = A.empty_f16(m, 64 + w2)
        g.split_n, g.out2, g.ldo2, g.out2_col = split, out2.data_ptr(), 64 + w2, 64
    if epi == B.MMDIT_EPI_EULER:
        g.alpha = -1.0 / 28
    B.check(B.mmdit_k_gemm(g, stream()))
    sync()
    sel = np.arange(m) if rows is None else rows
    _RESID[0] = resid[sel]
    y = O.linear(a[sel], lin)
    if epi == B.MMDIT_EPI_BIAS:
        return to_numpy_f32(out)[sel], y
    if epi == B.MMDIT_EPI_BIAS_GELU:
        return to_numpy_f32(out)[sel], O.gelu_tanh(y)
    if epi == B.MMDIT_EPI_GATE_RESID:
        return to_numpy_f32(out)[sel], resid[sel] + gate * y
    if epi == B.MMDIT_EPI_BIAS_F32:
        return to_numpy_f32(out)[sel], y
    if epi == B.MMDIT_EPI_EULER:
        return to_numpy_f32(out)[sel], O.euler(resid[sel], y, 1.0, 1.0 - 1.0 / 28)
    if epi == B.MMDIT_EPI_SWIGLU:
        return to_numpy_f32(out)[sel], O.swiglu(y)
    # split: first columns plain, the rest GELU (or SwiGLU) at column offset 64 of out2
    g1 = to_numpy_f32(out)[sel]
    g2 = to_numpy_f32(out2)[sel][:, 64:]
    act = O.swiglu if swiglu else O.gelu_tanh
    return np.concatenate([g1, g2], axis=1), np.concatenate([y[:, :split], act(y[:, split:])], axis=1)


def _gemm_err(g, ref, epi, k):
    """Output error over the output's own storage format: fp32 outputs are
    compared as they are; bf16 (q, k, v) and fp16 (GELU hidden) outputs beyond
    half a step of their format; a split output in two column blocks."""
    if epi in (B.MMDIT_EPI_GATE_RESID, B.MMDIT_EPI_EULER, B.MMDIT_EPI_BIAS_F32):
        return rel_err(g, ref)
    if epi == B.MMDIT_EPI_BIAS:
        return rel_err_rounded_out(g, ref, "bf16")
    if epi in (B.MMDIT_EPI_BIAS_GELU, B.MMDIT_EPI_SWIGLU):
        return rel_err_rounded_out(g, ref, "f16")
    s = _SPLIT[0]
    return max(rel_err_rounded_out(g[:, :s], ref[:, :s], "bf16"), rel_err_rounded_out(g[:, s:], ref[:, s:], "f16"))


_SPLIT = [0]


@pytest.mark.parametrize("m,n,k,epi,int8", GEMM_CASES)
def test_gemm(m, n, k, epi, int8):
    say(f"gemm m={m} n={n} k={k} epi={epi} int8={int8}")
    g, ref = _run_gemm(m, n, k, epi, int8)
    assert _gemm_err(g, ref, epi, k) <= TOL
    if epi in (B.MMDIT_EPI_GATE_RESID, B.MMDIT_EPI_EULER, B.MMDIT_EPI_BIAS_F32):
        # fp32 outputs: bf16 x bf16 products are exact in fp32 and the sums
        # round in fp32, so the branch itself (output minus the residual the
        # epilogue adds) matches far inside the bar
        base = _RESID[0] if epi != B.MMDIT_EPI_BIAS_F32 else 0.0
        assert rel_err(g - base, ref - base) <= 1e-3


@pytest.mark.parametrize("m,n,k,epi", [(4608, 9216, 3072, B.MMDIT_EPI_BIAS), (4096, 3072, 12288, B.MMDIT_EPI_GATE_RESID),
                                       (4608, 21504, 3072, B.MMDIT_EPI_SPLIT_GELU), (6889, 12288, 3072,
                                                                                   B.MMDIT_EPI_BIAS_GELU)])
def test_gemm_full_size_sampled_rows(m, n, k, epi):
    say(f"gemm full m={m} n={n} k={k} epi={epi}")
    rows = np.unique(np.r_[0, 255, 256, m - 1, np.random.default_rng(m).integers(0, m, 40)])
    g, ref = _run_gemm(m, n, k, epi, False, rows=rows, tid=60)
    assert _gemm_err(g, ref, epi, k) <= TOL


@pytest.mark.parametrize("m,n,k,epi", [(4608, 12288, 3072, B.MMDIT_EPI_BIAS_GELU), (4096, 3072, 12288, B.MMDIT_EPI_GATE_RESID),
                                       (4608, 21504, 3072, B.MMDIT_EPI_SPLIT_GELU)])
def test_gemm_int8_full_size_sampled_rows(m, n, k, epi):
    """int8 weight-only projections at FLUX sizes (the four-wavefront loop with
    in-loop code conversion and the staged epilogues), on sampled rows."""
    say(f"gemm int8 full m={m} n={n} k={k} epi={epi}")
    rows = np.unique(np.r_[0, 255, 256, m - 1, np.random.default_rng(m + 1).integers(0, m, 40)])
    g, ref = _run_gemm(m, n, k, epi, True, rows=rows, tid=62)
    assert _gemm_err(g, ref, epi, k) <= TOL


@pytest.mark.parametrize("m,n,k,epi,wt", [
    (513, 1024, 256, B.MMDIT_EPI_SWIGLU, "bf16"), (300, 512, 448, B.MMDIT_EPI_SWIGLU, "int8"),
    (77, 2048, 320, B.MMDIT_EPI_SWIGLU, "f16"), (1, 256, 64, B.MMDIT_EPI_SWIGLU, "bf16"),
    (320, 1280, 256, B.MMDIT_EPI_SPLIT_SWIGLU, "bf16"), (257, 2816, 512, B.MMDIT_EPI_SPLIT_SWIGLU, "int8"),
    (130, 1280, 256, B.MMDIT_EPI_SPLIT_SWIGLU, "f16")])
def test_gemm_swiglu(m, n, k, epi, wt):
    """SwiGLU epilogues: W rows [gate | up] in their natural layout; the
    kernel pairs them per feature in registers."""
    say(f"gemm swiglu m={m} n={n} k={k} epi={epi} weights={wt}")
    g, ref = _run_gemm(m, n, k, epi, wt == "int8", tid=110, f16=wt == "f16")
    assert _gemm_err(g, ref, epi, k) <= TOL
    assert within_one_ulp(g[:, _SPLIT[0]:] if epi == B.MMDIT_EPI_SPLIT_SWIGLU else g,
                          ref[:, _SPLIT[0]:] if epi == B.MMDIT_EPI_SPLIT_SWIGLU else ref, "f16", 1e-3) <= 8


@pytest.mark.parametrize("m,n,k,epi", [(2560, 24576, 4096, B.MMDIT_EPI_SWIGLU),
                                       (2560, 36864, 4096, B.MMDIT_EPI_SPLIT_SWIGLU)])
def test_gemm_swiglu_klein_size_sampled_rows(m, n, k, epi):
    """Flux.2 Klein-shaped MLP-in (fc1, 4096 -> 2 x 12288) and single-block
    linear1 (4096 -> 3 x 4096 + 2 x 12288) at 512x512 editing (2560 tokens)."""
    say(f"gemm swiglu full m={m} n={n} k={k} epi={epi}")
    rows = np.unique(np.r_[0, 255, 256, m - 1, np.random.default_rng(n).integers(0, m, 40)])
    g, ref = _run_gemm(m, n, k, epi, False, rows=rows, tid=120)
    assert _gemm_err(g, ref, epi, k) <= TOL


@pytest.mark.parametrize("n,k,epi,wt", [(4032, 256, B.MMDIT_EPI_BIAS, "bf16"), (4096, 320, B.MMDIT_EPI_GATE_RESID, "int8"),
                                       (4096, 256, B.MMDIT_EPI_BIAS_GELU, "f16"),
                                       (4032, 192, B.MMDIT_EPI_SPLIT_GELU, "bf16"),
                                       (4096, 128, B.MMDIT_EPI_EULER, "f16")])
def test_gemm_tail_tiles(n, k, epi, wt):
    """4400 rows = 18 row tiles x 16 column tiles = 288 tiles: the last two
    row tiles run as 128-wide tail tiles (as in the FLUX MLP-in projection).
    Against the oracle on every element, and bit for bit against the same
    product computed as two calls (rows 0-4095 and 4096-4399) that use
    256-wide tiles only: the tile width does not change any element's sums."""
    say(f"gemm tail tiles m=4400 n={n} k={k} epi={epi} weights={wt}")
    m = 4400
    g, ref = _run_gemm(m, n, k, epi, wt == "int8", tid=130, f16=wt == "f16")
    assert _gemm_err(g, ref, epi, k) <= TOL
    A = DeviceArena(f16_weights=wt == "f16")
    a = synth.f16_exact(rnd(130, (m, k)))
    lin = _lin(132, n, k, wt == "int8")
    da = A.f16(a)
    wl = A.linear(lin)
    wtype = B.MMDIT_INT8 if wt == "int8" else (B.MMDIT_F16 if wt == "f16" else B.MMDIT_BF16)
    f32out = epi in (B.MMDIT_EPI_GATE_RESID, B.MMDIT_EPI_BIAS_F32, B.MMDIT_EPI_EULER)
    split = _SPLIT[0]
    outs = []
    for rows in ((0, m), (0, 4096), (4096, m)):
        r0, r1 = rows
        gate = rnd(135, (n,), 0.7)
        resid = rnd(136, (m, n))
        if f32out:
            out = A.f32(resid) if epi == B.MMDIT_EPI_EULER else A.empty_f32(m, n)
        else:
            out = A.empty_f16(m, split) if epi == B.MMDIT_EPI_BIAS_GELU else A.empty_bf16(m, split)
        outs.append(out)
    full, part = outs[0], outs[1]
    for (r0, r1), out in (((0, m), full), ((0, 4096), part), ((4096, m), part)):
        gm = B.mmdit_gemm(m=r1 - r0, n=n, k=k, weight_dtype=wtype, a=da[r0:].data_ptr(), lda=k, w=wl, epilogue=epi)
        f32 = out.dtype == torch.float32
        gm.out, gm.ldo = out[r0:].data_ptr(), (n if f32 else split)
        out2 = None
        if epi == B.MMDIT_EPI_GATE_RESID:
            gr = A.f32(rnd(135, (n,), 0.7))
            rs = A.f32(rnd(136, (m, n)))
            gm.gate, gm.resid, gm.ldr = gr.data_ptr(), rs[r0:].data_ptr(), n
        if epi == B.MMDIT_EPI_SPLIT_GELU:
            key = "o2_full" if out is full else "o2_part"
            if key not in _O2:
                _O2[key] = A.empty_f16(m, 64 + n - split)
            out2 = _O2[key]
            gm.split_n, gm.out2, gm.ldo2, gm.out2_col = split, out2[r0:].data_ptr(), 64 + n - split, 64
        if epi == B.MMDIT_EPI_EULER:
            gm.alpha = -1.0 / 28
        B.check(B.mmdit_k_gemm(gm, stream()))
    sync()
    np.testing.assert_array_equal(to_numpy_f32(full), to_numpy_f32(part))
    if epi == B.MMDIT_EPI_SPLIT_GELU:
        # columns 0-63 of out2 are never written (out2_col = 64)
        np.testing.assert_array_equal(to_numpy_f32(_O2["o2_full"])[:, 64:], to_numpy_f32(_O2["o2_part"])[:, 64:])
    _O2.clear()


_O2 = {}


def test_gemm_int8_rerun_bit_exact():
    say("gemm int8 rerun")
    a1, _ = _run_gemm(700, 256, 1024, B.MMDIT_EPI_GATE_RESID, True, tid=70)
    a2, _ = _run_gemm(700, 256, 1024, B.MMDIT_EPI_GATE_RESID, True, tid=70)
    np.testing.assert_array_equal(a1, a2)


@pytest.mark.parametrize("m,n,k,epi", [(513, 1024, 256, B.MMDIT_EPI_BIAS_GELU), (700, 256, 1024, B.MMDIT_EPI_GATE_RESID),
                                       (320, 1792, 256, B.MMDIT_EPI_SPLIT_GELU), (1, 128, 64, B.MMDIT_EPI_BIAS),
                                       (4608, 3072, 12288, B.MMDIT_EPI_GATE_RESID),
                                       (300, 320, 8256, B.MMDIT_EPI_BIAS_GELU), (77, 512, 8192, B.MMDIT_EPI_SWIGLU),
                                       (513, 256, 8320, B.MMDIT_EPI_GATE_RESID)])
def test_gemm_f16_weights_bit_identical(m, n, k, epi):
    """Weights re-encoded once by mmdit_weights_to_f16 give the bf16 path's
    results bit for bit (same fp16 values reach the matrix cores). With
    K >= 8192 the fp16-weight GEMM runs its pipelined main loop (odd and even
    k-step counts here), so this also pins that loop to the plain one."""
    say(f"gemm f16 weights m={m} n={n} k={k} epi={epi}")
    rows = None if m < 4096 else np.unique(np.r_[0, 255, 256, m - 1, np.arange(0, m, 97)])
    a, ref = _run_gemm(m, n, k, epi, False, rows=rows, tid=90)
    b, _ = _run_gemm(m, n, k, epi, False, rows=rows, tid=90, f16=True)
    np.testing.assert_array_equal(a, b)
    assert _gemm_err(b, ref, epi, k) <= TOL


def test_weights_to_f16_exhaustive():
    """Every bf16 bit pattern (plus a ragged tail) against numpy's
    round-to-nearest-even float32 -> float16 conversion: subnormal results,
    overflow to infinity, signed zeros; NaN stays NaN."""
    say("weights_to_f16 all bf16 patterns")
    bits = np.r_[np.arange(65536, dtype=np.uint32), np.array([0x3f80, 0x0001, 0x8001, 0x477f, 0x4780], np.uint32)]
    bits = bits.astype(np.uint16)
    src = torch.from_numpy(bits.view(np.int16)).cuda()
    dst = torch.empty(bits.size, dtype=torch.int16, device="cuda")
    B.check(B.mmdit_weights_to_f16(src, dst, bits.size, stream()))
    sync()
    got = dst.cpu().numpy().view(np.uint16)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = synth.bits_to_f32(bits).astype(np.float16).view(np.uint16)
    nan = np.isnan(synth.bits_to_f32(bits))
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(got[nan].view(np.float16)))


# ------------------------------------------------------------------ GEMV
@pytest.mark.parametrize("n,k,wt,silu_in,acc", [(1536, 256, "bf16", 1, 0), (18432, 3072, "bf16", 1, 0),
                                                (18432, 3072, "int8", 1, 0), (3072, 256, "int8", 0, 1),
                                                (100, 64, "bf16", 0, 1), (18432, 3072, "f16", 1, 0),
                                                (100, 64, "f16", 0, 1), (101, 4096, "bf16", 1, 0),
                                                (7, 1024, "int8", 1, 1), (9, 4096, "int8", 0, 0),
                                                (18432, 3072, "fp8", 1, 0), (9216, 3072, "fp8", 1, 1),
                                                (33, 64, "fp8", 0, 1), (101, 4096, "fp8", 1, 0)])
def test_gemv(n, k, wt, silu_in, acc):
    """fp8 weights: against the fp64 product with the decoded codes (the
    activation stays fp32 in the modulation GEMV)."""
    say(f"gemv n={n} k={k} weights={wt}")
    int8, f16, fp8 = wt == "int8", wt == "f16", wt == "fp8"
    A = DeviceArena(f16_weights=f16, fp8_weights=fp8)
    x = rnd(80, (k,))
    lin = _lin(81, n, k, int8)
    base = rnd(83, (n,))
    out = A.f32(base)
    dt = B.MMDIT_INT8 if int8 else (B.MMDIT_F16 if f16 else B.MMDIT_FP8 if fp8 else B.MMDIT_BF16)
    B.check(B.mmdit_k_gemv(A.f32(x), k, A.linear(lin), n, dt, silu_in, acc, out, stream()))
    sync()
    xin = O.silu(x) if silu_in else x
    ref = O.linear(xin[None, :], O.fp8_weights(lin) if fp8 else lin)[0] + (base if acc else 0)
    assert rel_err(out.cpu().numpy(), ref) <= 1e-4


# ------------------------------------------------------------------ time embedding / Euler
@pytest.mark.parametrize("t,gd,int8", [(1.0, 3.5, False), (0.37, 3.5, True), (0.0, 1.0, False)])
def test_time_embed(t, gd, int8):
    say(f"time_embed t={t} g={gd} int8={int8}")
    A = DeviceArena()
    shp = synth.custom_shape("te", CID + 1, 256, 4, 1024, 8, (2, 2), n_double=0, n_single=0)
    m = synth.model_weights(shp, int8=int8)
    from diffusion_transformer_image_mm_amd.device import dims_for
    d = dims_for(shp, int8)
    mm = A.model(m)
    vec = A.empty_f32(shp.hidden)
    ws = A.workspace(4 * (512 + 2 * shp.hidden))
    B.check(B.mmdit_k_time_embed(d, mm, t, gd, vec, ws, ws.numel(), stream()))
    sync()
    assert rel_err(vec.cpu().numpy(), O.conditioning(t, gd, m)) <= 1e-4


def test_euler():
    say("euler")
    A = DeviceArena()
    z = rnd(90, (4096, 64))
    v = rnd(91, (4096, 64))
    dz = A.f32(z)
    B.check(B.mmdit_k_euler(dz, A.f32(v), z.size, -1.0 / 28, stream()))
    sync()
    np.testing.assert_allclose(dz.cpu().numpy(), O.euler(z, v, 1.0, 1.0 - 1.0 / 28), rtol=0, atol=1e-6)



# ------------------------------------------------------------------ fp8 (OCP e4m3)
def _e4m3_table() -> np.ndarray:
    t = np.empty(256)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 0x7
        if e == 0xF and m == 0x7:
            t[c] = np.nan
        elif e == 0:
            t[c] = sign * (m / 8.0) * 2.0 ** -6
        else:
            t[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


E4M3 = _e4m3_table()


def _quantize_gpu(A, x, dtype, ldx=None, ldc=None):
    """Upload x (16-bit exact values) and quantise it per row on the GPU."""
    rows, cols = x.shape
    ldx = ldx or cols
    ldc = ldc or cols
    xp = np.zeros((rows, ldx), dtype=np.float32)
    xp[:, :cols] = x
    dx = A.f16(xp) if dtype == "f16" else A.bf16(xp)
    codes = A._hold(torch.zeros(rows, ldc, dtype=torch.uint8, device="cuda"))
    scales = A.empty_f32(rows)
    xd = B.MMDIT_F16 if dtype == "f16" else B.MMDIT_BF16
    B.check(B.mmdit_quantize_fp8_rows(dx, xd, rows, cols, ldx, codes, ldc, scales, stream()), "quantize")
    return codes, scales


@pytest.mark.parametrize("rows,cols,ldx,ldc,dt", [(37, 3072, 3072, 3072, "f16"), (5, 256, 264, 272, "bf16"),
                                               (300, 12288, 12288, 12288, "f16"), (1, 16, 16, 16, "bf16")])
def test_quantize_fp8_rows_bit_exact(rows, cols, ldx, ldc, dt):
    """Scales and codes equal the oracle's bit for bit: both take the
    decisions in fp32 (scale = max|x| / 448, x / scale, round to nearest even)."""
    say(f"quantize fp8 rows={rows} cols={cols} {dt}")
    A = DeviceArena()
    x = rnd(150, (rows, cols), 3.0)
    x = synth.f16_exact(x) if dt == "f16" else x
    if rows > 2:
        x[2] = 0.0
    codes, scales = _quantize_gpu(A, x, dt, ldx, ldc)
    sync()
    c = codes.cpu().numpy()[:, :cols]
    ref_codes, ref_sc = O.quantize_rows_fp8(x)
    np.testing.assert_array_equal(scales.cpu().numpy(), ref_sc)
    np.testing.assert_array_equal(E4M3[c], ref_codes)


def _run_gemm_fp8(m, n, k, epi, rows=None, tid=140):
    A = DeviceArena()
    a = synth.f16_exact(rnd(tid, (m, k)))
    w = rnd(tid + 1, (n, k), 0.02)
    b = rnd(tid + 2, (n,), 0.02)
    ac, asc = _quantize_gpu(A, a, "f16")
    wc, wsc = _quantize_gpu(A, w, "bf16")
    db = A.bf16(b)
    g = B.mmdit_gemm(m=m, n=n, k=k, weight_dtype=B.MMDIT_FP8, a=ac.data_ptr(), lda=k,
                     w=B.mmdit_linear(wc.data_ptr(), wsc.data_ptr(), db.data_ptr()), epilogue=epi)
    g.a_scale = asc.data_ptr()
    f32out = epi in (B.MMDIT_EPI_GATE_RESID, B.MMDIT_EPI_BIAS_F32)
    gate = rnd(tid + 5, (n,), 0.7)
    resid = rnd(tid + 6, (m, n))
    if f32out:
        out = A.empty_f32(m, n)
    else:
        out = A.empty_f16(m, n) if epi == B.MMDIT_EPI_BIAS_GELU else A.empty_bf16(m, n)
    g.out, g.ldo = out.data_ptr(), n
    if epi == B.MMDIT_EPI_GATE_RESID:
        g.gate, g.resid, g.ldr = A.f32(gate).data_ptr(), A.f32(resid).data_ptr(), n
    B.check(B.mmdit_k_gemm(g, stream()), "gemm fp8")
    sync()
    # the GPU's codes are the oracle's (bit-exact quantisation), so the
    # reference is the fp64 product of the decoded operands
    sel = np.arange(m) if rows is None else rows
    ref_ac, ref_as = O.quantize_rows_fp8(a[sel])
    ref_wc, ref_ws = O.quantize_rows_fp8(w)
    np.testing.assert_array_equal(E4M3[ac.cpu().numpy()[sel]], ref_ac)
    np.testing.assert_array_equal(E4M3[wc.cpu().numpy()], ref_wc)
    y = O.linear_fp8(ref_ac, ref_as, ref_wc, ref_ws, b)
    exact = O.linear(a[sel], synth.Linear(w, b))
    got = to_numpy_f32(out)[sel]
    if epi == B.MMDIT_EPI_BIAS_GELU:
        ref = O.gelu_tanh(y)
    elif epi == B.MMDIT_EPI_GATE_RESID:
        ref = resid[sel] + gate * y
    else:
        ref = y
    return got, ref, y, exact


@pytest.mark.parametrize("m,n,k,epi", [(513, 1024, 256, B.MMDIT_EPI_BIAS_F32), (300, 320, 1024, B.MMDIT_EPI_BIAS_GELU),
                                       (77, 512, 384, B.MMDIT_EPI_GATE_RESID), (1, 256, 128, B.MMDIT_EPI_BIAS),
                                       (700, 256, 3072, B.MMDIT_EPI_BIAS_F32)])
def test_gemm_fp8(m, n, k, epi):
    """fp8 matrix cores: against the fp64 product of the decoded operands.
    The products of two e4m3 values are exact; the matrix cores' own sums over
    a 128-deep fp8 block are not fp32-exact (measured ~1e-4 of the RMS), so
    the bar is 2e-3 of the RMS: far below the quantisation itself, far above
    the O(1) errors of a wrong lane layout or scale."""
    say(f"gemm fp8 m={m} n={n} k={k} epi={epi}")
    got, ref, y, exact = _run_gemm_fp8(m, n, k, epi)
    if epi in (B.MMDIT_EPI_BIAS_F32, B.MMDIT_EPI_GATE_RESID):
        e = rel_err(got, ref)
        say(f"  rel_err vs decoded-operand product {e:.3e}")
        assert e <= 2e-3, e
    elif epi == B.MMDIT_EPI_BIAS_GELU:
        assert rel_err_rounded_out(got, ref, "f16") <= 2e-3
    else:
        assert rel_err_rounded_out(got, ref, "bf16") <= 2e-3
    # against the unquantised product: each e4m3 rounding is at most 2^-4 of
    # its value (RMS ~2^-4/sqrt(3) = 3.6%); two of them per product term leave
    # an error of ~5% of the output's RMS in RMS, a few times that at the
    # maximum over ~10^5 outputs
    d = y - exact
    rms = float(np.sqrt(np.mean(d * d)) / np.sqrt(np.mean(exact * exact)))
    eq = rel_err(y, exact)
    say(f"  fp8 quantisation error vs the exact product: rms {rms:.3e}, max {eq:.3e}")
    assert rms <= 0.08 and eq <= 0.4, (rms, eq)


def test_gemm_fp8_mlp_in_size_sampled_rows():
    m, n, k = 4608, 12288, 3072
    say(f"gemm fp8 full m={m} n={n} k={k}")
    rows = np.unique(np.r_[0, 255, 256, m - 1, np.random.default_rng(7).integers(0, m, 40)])
    got, ref, y, exact = _run_gemm_fp8(m, n, k, B.MMDIT_EPI_BIAS_GELU, rows=rows, tid=160)
    e = rel_err_rounded_out(got, ref, "f16")
    say(f"  rel_err beyond the fp16 output rounding {e:.3e}; quantisation error {rel_err(y, exact):.3e}")
    assert e <= 2e-3, e
