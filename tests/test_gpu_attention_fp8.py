"""fp8 attention through the C ABI against the oracle's fp8 attention.

SGLang-AMD blog, "Architecture Deep Dive": fp8 quantisation on the CDNA stack.
The quantiser's decisions (power-of-two exponents from the RMSNorm scales,
codes, per-channel value scales, the operand key order) are compared bit for
bit; the attention output element by element, at sizes spanning several key
tiles and ragged tails, and on sampled rows at the FLUX size."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from diffusion_transformer_image_mm_amd import binding as B
from diffusion_transformer_image_mm_amd import synth
from gpu_helpers import (TOL, DeviceArena, attention_fp8_perturbed, rel_err_rounded_out, say, stream, sync,
                         to_numpy_f32, vt_layout)

pytestmark = pytest.mark.gpu
CID = 720


def rnd(tid, shape, std=1.0):
    return synth.rand_array(CID, tid, shape, std)


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


def _slot_keys():
    """key held by slot p of a 64-key tile in the fp8 v^T order:
    slot 32g + 16s + 4a + b holds key 32s + 8a + 4g + b."""
    p = np.arange(64)
    g, s, a, b = p >> 5, (p >> 4) & 1, (p >> 2) & 3, p & 3
    return 32 * s + 8 * a + 4 * g + b


def _normed(tid, heads, L, D, g):
    """Rows RMS-normalised per head, times the norm scale g [D] (what the
    QK-RMSNorm hands to the attention; RoPE would only rotate pairs)."""
    x = rnd(tid, (heads, L, D)).astype(np.float64)
    x = x / np.sqrt((x ** 2).mean(-1, keepdims=True) + 1e-6)
    return synth.bf16_exact((x * g[None, None, :]).astype(np.float32))


def _fp8_sensitivity(qf, kf, vf, heads, eq, ek, rows, draws=3, seed=0):
    """How far the oracle's fp8 attention moves (max |diff| / RMS) when each
    logit is perturbed within the matrix cores' summation error
    (gpu_helpers.attention_fp8_perturbed; the inputs are bf16 already): an
    implementation that sums like the hardware is one more such draw."""
    g = np.random.default_rng(seed)
    base = O.attention_fp8(qf, kf, vf, heads, eq, ek, rows=rows)
    rms = np.sqrt((base ** 2).mean())
    return max(float(np.abs(attention_fp8_perturbed(qf, kf, vf, heads, eq, ek, rows, g, bf16_inputs=False)
                            - base).max() / rms) for _ in range(draws))


def _case(D, heads, L, gq=(1.0, 1.0), gk=(1.0, 1.0), tid=10, rows=None, q=None, k=None, check_codes=True,
          norms=None, v=None):
    """Runs the quantiser and the fp8 attention; checks the quantiser's
    decisions bit for bit and returns (error of the output against the
    oracle's fp8 attention, the bar for it, the GPU output rows). The bar is
    2e-2, or twice the oracle's own movement under the matrix cores' summation
    error where that is larger (an implementation that sums like the
    hardware is one more such draw)."""
    """norms: the four RMSNorm scale vectors (q text, q image, k text, k
    image) that q and k were normalised with; by default drawn around gq, gk."""
    A = DeviceArena()
    l_pad = (L + 127) // 128 * 128
    H = heads * D
    if norms is None:
        gq0 = synth.bf16_exact(gq[0] * (0.5 + rnd(tid, (D,), 0.25) ** 2).astype(np.float32))
        gq1 = synth.bf16_exact(gq[1] * (0.5 + rnd(tid + 1, (D,), 0.25) ** 2).astype(np.float32))
        gk0 = synth.bf16_exact(gk[0] * (0.5 + rnd(tid + 2, (D,), 0.25) ** 2).astype(np.float32))
        gk1 = synth.bf16_exact(gk[1] * (0.5 + rnd(tid + 3, (D,), 0.25) ** 2).astype(np.float32))
    else:
        gq0, gq1, gk0, gk1 = (synth.bf16_exact(np.asarray(n, np.float32)) for n in norms)
    if q is None:
        q = _normed(tid + 4, heads, L, D, gq0)
    if k is None:
        k = _normed(tid + 5, heads, L, D, gk1)
    if v is None:
        v = rnd(tid + 6, (heads, L, D))
    qp = np.zeros((heads, l_pad, D), np.float32); qp[:, :L] = q
    kp = np.zeros((heads, l_pad, D), np.float32); kp[:, :L] = k
    vt = np.zeros((heads, D, l_pad), np.float32); vt[:, :, :L] = v.transpose(0, 2, 1)
    q8 = A._hold(torch.zeros(heads, l_pad, D, dtype=torch.uint8, device="cuda"))
    k8 = A._hold(torch.zeros(heads, l_pad, D, dtype=torch.uint8, device="cuda"))
    vt8 = A._hold(torch.zeros(heads, D, l_pad, dtype=torch.uint8, device="cuda"))
    sv = A.empty_f32(H)
    exps = A.i32(np.zeros(2))
    B.check(B.mmdit_k_quantize_attention_fp8(A.bf16(qp), A.bf16(kp), A.bf16(vt_layout(vt)), heads, D, l_pad,
                                             A.bf16(gq0), A.bf16(gq1), A.bf16(gk0), A.bf16(gk1),
                                             q8, k8, vt8, sv, exps, stream()), "quantize attention fp8")
    out = A.empty_f16(L, H)
    B.check(B.mmdit_k_attention_fp8(q8, k8, vt8, sv, exps, heads, L, D, l_pad, out, H, stream()), "attention fp8")
    sync()
    eq, ek = (int(e) for e in exps.cpu().numpy())
    assert eq == O.qk_fp8_exponent([gq0, gq1], D) and ek == O.qk_fp8_exponent([gk0, gk1], D), (eq, ek)
    # [L, heads*D] views for the oracle
    qf = q.transpose(1, 0, 2).reshape(L, H)
    kf = k.transpose(1, 0, 2).reshape(L, H)
    vf = v.transpose(1, 0, 2).reshape(L, H)
    if check_codes:
        qc = E4M3[q8.cpu().numpy()[:, :L]].transpose(1, 0, 2).reshape(L, H)
        kc = E4M3[k8.cpu().numpy()[:, :L]].transpose(1, 0, 2).reshape(L, H)
        np.testing.assert_array_equal(qc, O.quantize_pow2_fp8(qf, eq))
        np.testing.assert_array_equal(kc, O.quantize_pow2_fp8(kf, ek))
        assert np.all(q8.cpu().numpy()[:, L:] == 0) and np.all(k8.cpu().numpy()[:, L:] == 0)
        vcodes, vsc = O.quantize_cols_fp8(vf)
        np.testing.assert_array_equal(sv.cpu().numpy(), vsc)
        g8 = vt8.cpu().numpy().reshape(heads, D, l_pad // 64, 64)
        keys = _slot_keys()
        dec = np.empty_like(g8, dtype=np.float64)
        dec[..., keys] = E4M3[g8]                   # back to key order
        dec = dec.reshape(heads, D, l_pad)
        np.testing.assert_array_equal(dec[:, :, :L].transpose(2, 0, 1).reshape(L, H), vcodes)
        assert np.all(dec[:, :, L:] == 0)
    g = to_numpy_f32(out)
    sel = np.arange(L) if rows is None else np.asarray(rows)
    ref = O.attention_fp8(qf, kf, vf, heads, eq, ek, rows=None if rows is None else sel)
    err = rel_err_rounded_out(g[sel], ref, "f16")
    sens = _fp8_sensitivity(qf, kf, vf, heads, eq, ek, sel, draws=3 if len(sel) * L * heads < 4e7 else 2)
    say(f"  error {err:.3g}, oracle movement under the summation error {sens:.3g}")
    return err, max(TOL, 2.0 * sens), g[sel]


@pytest.mark.parametrize("D,heads,L", [(64, 4, 320), (128, 2, 333), (128, 3, 64), (64, 2, 1), (128, 1, 129),
                                       (64, 1, 700), (128, 2, 63)])
def test_attention_fp8_small(D, heads, L):
    say(f"attention fp8 D={D} heads={heads} L={L}")
    err, bar, _ = _case(D, heads, L)
    assert err <= bar, (err, bar)


@pytest.mark.parametrize("D,heads,L,gs", [(128, 2, 333, 3.0), (64, 3, 320, 4.0)])
def test_attention_fp8_sharp(D, heads, L, gs):
    """Norm scales of 3-4: logits with a spread of tens (log2 units), so a few
    keys dominate each row; the quantiser's exponent follows the larger scale
    (the image-stream scale here) and the two streams differ."""
    say(f"attention fp8 sharp D={D} heads={heads} L={L} g={gs}")
    err, bar, _ = _case(D, heads, L, gq=(1.0, gs), gk=(gs, 1.0), tid=30)
    assert err <= bar, (err, bar)


@pytest.mark.parametrize("D,L", [(128, 333), (64, 700)])
def test_attention_fp8_growing_scores(D, L):
    """Keys that turn towards the query along the key axis: the row maximum
    grows tile after tile, so the integer reference moves (and the running
    sums are rescaled) on many tiles; the result must still equal the
    definition against the final maximum. The logits reach ~60 (log2 units):
    there the matrix cores' summation error flips probability codes of the
    dominant keys, so the bar is twice the oracle's own movement under that
    error (and 2e-2 where that is smaller)."""
    say(f"attention fp8 growing scores D={D} L={L}")
    heads = 2
    g = np.full(D, 2.0, np.float32)
    u = np.zeros(D); u[0] = 1.0
    base = rnd(50, (heads, L, D), 0.6).astype(np.float64)
    q = base[:, :1] * 0.2 + 3.0 * u
    q = np.repeat(q, L, axis=1) + 0.05 * base
    k = base[:, ::-1] + (np.linspace(0.0, 6.0, L)[None, :, None]) * u
    nrm = lambda x: synth.bf16_exact((x / np.sqrt((x ** 2).mean(-1, keepdims=True)) * g).astype(np.float32))
    err, bar, _ = _case(D, heads, L, q=nrm(q), k=nrm(k), tid=60, norms=(g, g, g, g))
    assert err <= bar, (err, bar)


@pytest.mark.parametrize("L", [4608, 7145])
def test_attention_fp8_full_size_sampled_rows(L):
    say(f"attention fp8 full heads=24 D=128 L={L}")
    rng = np.random.default_rng(L)
    rows = np.unique(np.r_[0, 1, 127, 128, L - 129, L - 1, rng.integers(0, L, 60)])
    err, bar, _ = _case(128, 24, L, rows=rows, tid=80)
    assert err <= bar, (err, bar)


def test_attention_fp8_close_to_bf16_attention():
    """The fp8 result against the exact attention of the same (unquantised)
    inputs: the price of rounding q, k, v and the probabilities to 3
    mantissa bits, a few percent of the output RMS on these inputs; the GPU
    lands as close to the exact attention as the oracle's fp8 attention."""
    say("attention fp8 vs exact")
    D, heads, L = 128, 2, 700
    gq = synth.bf16_exact(np.ones(D, np.float32))
    q = _normed(91, heads, L, D, gq)
    k = _normed(92, heads, L, D, gq)
    v = rnd(93, (heads, L, D))
    H = heads * D
    e = O.qk_fp8_exponent([gq], D)
    flat = lambda x: x.transpose(1, 0, 2).reshape(L, H)
    exact = O.attention(flat(q), flat(k), flat(v), heads)
    f8 = O.attention_fp8(flat(q), flat(k), flat(v), heads, e, e)
    rms = np.sqrt((exact ** 2).mean())
    e_oracle = np.sqrt(((f8 - exact) ** 2).mean()) / rms
    err, bar, gout = _case(D, heads, L, tid=90, q=q, k=k, v=v, norms=(gq, gq, gq, gq))
    assert err <= bar, (err, bar)
    e_gpu = np.sqrt(((gout - exact) ** 2).mean()) / rms
    say(f"  RMS distance from the exact attention: oracle fp8 {e_oracle:.3g}, GPU {e_gpu:.3g}")
    assert 5e-3 < e_oracle < 0.1, e_oracle
    assert e_gpu <= 1.1 * e_oracle + 2e-3, (e_gpu, e_oracle)
