"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test checks one oracle function against something other than itself: an
invariant, a closed form, a special case that reduces to a textbook routine,
brute force on tiny inputs, or the structure the Luminal blog reports. The
cases are chosen so that a dropped term, a wrong sign, a swapped operand or a
wrong index in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import erf, expit

import oracle as O
from diffusion_transformer_image_mm_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


# ---------------------------------------------------------------- softmax / attention
def test_softmax_rows_sum_to_one():
    s = rng.standard_normal((37, 53)) * 30
    p = O.softmax_rows(s)
    assert np.all(p >= 0)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-12


def test_attention_identical_keys_is_mean_of_values():
    L, D = 29, 16
    q = rng.standard_normal((L, D))
    k = np.tile(rng.standard_normal((1, D)), (L, 1))
    v = rng.standard_normal((L, D))
    o = O.attention_head(q, k, v)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (L, 1)), rtol=0, atol=1e-13)


def test_attention_single_token_returns_v():
    q, k, v = rng.standard_normal((3, 1, 8))
    np.testing.assert_array_equal(O.attention_head(q, k, v), v)


def _attention_brute(q, k, v):
    """Attention by explicit Python loops and math.exp, no numpy reductions."""
    L, D = len(q), len(q[0])
    out = []
    for i in range(L):
        s = [sum(q[i][d] * k[j][d] for d in range(D)) / math.sqrt(D) for j in range(L)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = math.fsum(e)
        out.append([math.fsum(e[j] * v[j][d] for j in range(L)) / z for d in range(D)])
    return np.array(out)


@pytest.mark.parametrize("L,D", [(1, 4), (5, 8), (17, 6), (32, 16)])
def test_attention_brute_force_tiny(L, D):
    q, k, v = (rng.standard_normal((L, D)) * 2 for _ in range(3))
    np.testing.assert_allclose(O.attention_head(q, k, v), _attention_brute(q.tolist(), k.tolist(), v.tolist()),
                               rtol=0, atol=1e-12)


def test_attention_sharp_key_selects_its_value():
    L, D = 40, 16
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    q = 200.0 * k[7:8] / np.linalg.norm(k[7])  # query aligned with key 7 only
    o = O.attention_head(q, k, v)
    np.testing.assert_allclose(o[0], v[7], atol=1e-6)


def test_softmax_large_logits_stay_finite():
    # logits far past exp's fp64 range (e^710 overflows): the max-subtracted
    # softmax stays finite and still sums to one
    s = np.array([[1000.0, 999.0, -1000.0], [5000.0, 5000.0, 0.0]])
    p = O.softmax_rows(s)
    assert np.all(np.isfinite(p))
    np.testing.assert_allclose(p[0], [1 / (1 + math.exp(-1)), math.exp(-1) / (1 + math.exp(-1)), 0], atol=1e-15)
    np.testing.assert_allclose(p[1], [0.5, 0.5, 0], atol=1e-15)


def test_attention_multihead_heads_independent_and_rows_subset():
    L, heads, D = 23, 3, 8
    q, k, v = (rng.standard_normal((L, heads * D)) for _ in range(3))
    full = O.attention(q, k, v, heads)
    for h in range(heads):
        sl = slice(h * D, (h + 1) * D)
        np.testing.assert_allclose(full[:, sl], _attention_brute(q[:, sl].tolist(), k[:, sl].tolist(),
                                                                 v[:, sl].tolist()), atol=1e-12)
    rows = np.array([0, 5, 22])
    np.testing.assert_allclose(O.attention(q, k, v, heads, rows), full[rows], atol=1e-13)


def test_attention_permutation_equivariant():
    L, D = 31, 8
    q, k, v = (rng.standard_normal((L, D)) for _ in range(3))
    perm = rng.permutation(L)
    o = O.attention_head(q, k, v)
    op = O.attention_head(q[perm], k[perm], v[perm])
    np.testing.assert_allclose(op, o[perm], atol=1e-13)


# ---------------------------------------------------------------- norms
def test_layer_norm_closed_form_moments():
    x = rng.standard_normal((11, 64)) * np.array([1e-4, 1e-3, 1e-2, 0.1, 1, 3, 10, 1e2, 1, 1, 1])[:, None] + 5
    eps = 1e-6
    y = O.layer_norm(x, eps)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-9)
    # the biased variance of the output is var / (var + eps): catches a dropped
    # eps, an unbiased (n - 1) divisor or a missing mean subtraction
    np.testing.assert_allclose((y * y).mean(axis=1), var / (var + eps), rtol=1e-10)


def test_layer_norm_two_values_closed_form():
    # a row of +a and -a (mean 0, var a^2): LN gives +-a / sqrt(a^2 + eps)
    a, eps = 0.003, 1e-6
    x = np.array([[a, -a] * 8])
    y = O.layer_norm(x, eps)
    np.testing.assert_allclose(y[0, 0], a / math.sqrt(a * a + eps), rtol=1e-14)
    assert y[0, 1] == -y[0, 0]


def test_modulate_identity_scale_and_shift():
    x = rng.standard_normal((5, 32))
    y = O.layer_norm(x, 1e-6)
    z = np.zeros(32)
    np.testing.assert_array_equal(O.modulate(y, z, z), y)
    c = np.full(32, 0.75)
    np.testing.assert_allclose(O.modulate(y, z, c), 1.75 * y, rtol=1e-15)      # (1 + scale)
    np.testing.assert_allclose(O.modulate(y, c, z).mean(axis=1), 0.75, atol=1e-12)  # + shift
    idx = np.arange(32.0)
    np.testing.assert_allclose(O.modulate(y, z, idx), y * (1 + idx), rtol=1e-15)  # per column


def test_rms_norm_closed_forms():
    eps = 1e-6
    u = rng.standard_normal((7, 64)) * 3
    y = O.rms_norm(u, np.ones(64), eps)
    ms = (u * u).mean(axis=1)
    np.testing.assert_allclose((y * y).mean(axis=1), ms / (ms + eps), rtol=1e-12)
    # one-hot input c e_i: output g_i c / sqrt(c^2 / D + eps) at i, zero elsewhere
    g = np.linspace(0.5, 1.5, 64)
    for i in (0, 17, 63):
        e = np.zeros((1, 64)); e[0, i] = 2.5
        y = O.rms_norm(e, g, eps)
        want = np.zeros(64); want[i] = g[i] * 2.5 / math.sqrt(2.5 ** 2 / 64 + eps)
        np.testing.assert_allclose(y[0], want, rtol=1e-14, atol=0)


# ---------------------------------------------------------------- rope
AXES = (16, 56, 56)


def _ids(L, hi=90):
    return rng.integers(0, hi, size=(L, 3)).astype(np.int32)


def test_rope_zero_position_is_identity():
    u = rng.standard_normal((4, 128))
    phi = O.rope_angles(np.zeros((4, 3), np.int32), AXES, 1e4)
    np.testing.assert_array_equal(O.apply_rope(u, phi), u)


def test_rope_preserves_pair_and_vector_norms():
    u = rng.standard_normal((20, 128))
    r = O.apply_rope(u, O.rope_angles(_ids(20), AXES, 1e4))
    pair = lambda a: a[:, 0::2] ** 2 + a[:, 1::2] ** 2
    np.testing.assert_allclose(pair(r), pair(u), rtol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(r, axis=1), np.linalg.norm(u, axis=1), rtol=1e-13)


def test_rope_relative_position_property():
    # <R_m q, R_n k> = <q, R_(n-m) k> for every axis
    q, k = rng.standard_normal((2, 1, 128))
    for m, n in [((0, 3, 5), (0, 7, 2)), ((2, 0, 40), (5, 63, 1))]:
        pm = O.rope_angles(np.array([m], np.int32), AXES, 1e4)
        pn = O.rope_angles(np.array([n], np.int32), AXES, 1e4)
        pd = O.rope_angles(np.array([np.subtract(n, m)], np.int32), AXES, 1e4)
        lhs = (O.apply_rope(q, pm) * O.apply_rope(k, pn)).sum()
        rhs = (q * O.apply_rope(k, pd)).sum()
        assert abs(lhs - rhs) < 1e-12


def test_rope_axis_segments_and_unit_frequency():
    # the first pair of each axis turns by exactly its position (frequency 1);
    # the t axis owns pairs [0, 8), h [8, 36), w [36, 64)
    ids = np.array([[3, 5, 7]], np.int32)
    phi = O.rope_angles(ids, AXES, 1e4)[0]
    assert phi[0] == 3 and phi[8] == 5 and phi[36] == 7
    only_h = O.rope_angles(np.array([[0, 5, 0]], np.int32), AXES, 1e4)[0]
    assert np.all(only_h[:8] == 0) and np.all(only_h[36:] == 0) and np.all(only_h[8:36] > 0)
    # frequencies fall geometrically within an axis: ratio theta^(-2/d_a)
    np.testing.assert_allclose(only_h[9:36] / only_h[8:35], 1e4 ** (-2 / 56), rtol=1e-13)
    # unit vector e_0 at t-position 1 turns to (cos 1, sin 1)
    e = np.zeros((1, 128)); e[0, 0] = 1
    r = O.apply_rope(e, O.rope_angles(np.array([[1, 0, 0]], np.int32), AXES, 1e4))
    np.testing.assert_allclose(r[0, :2], [math.cos(1), math.sin(1)], rtol=1e-15)


# ---------------------------------------------------------------- elementwise
def test_gelu_against_erf_form_and_identities():
    x = np.linspace(-8, 8, 2001)
    g = O.gelu_tanh(x)
    exact = 0.5 * x * (1 + erf(x / math.sqrt(2)))
    assert np.max(np.abs(g - exact)) < 5e-4  # the tanh form is within 4.7e-4 of the erf form
    np.testing.assert_allclose(g - O.gelu_tanh(-x), x, atol=1e-13)  # GELU(x) - GELU(-x) = x
    assert O.gelu_tanh(np.array([0.0]))[0] == 0
    assert abs(O.gelu_tanh(np.array([12.0]))[0] - 12.0) < 1e-12


def test_silu_against_logistic():
    x = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(O.silu(x), x * expit(x), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(O.silu(x) - O.silu(-x), x, atol=1e-12)


def test_swiglu_closed_forms_and_operand_order():
    """SwiGLU (the gated MLP activation of Flux.2 Klein): the first half of
    the columns is the gate, the second the value."""
    g = np.linspace(-20, 20, 81)
    u = rng.standard_normal(81)
    np.testing.assert_allclose(O.swiglu(np.c_[g, np.ones(81)]), (g * expit(g))[:, None],
                               rtol=1e-14, atol=1e-300)
    np.testing.assert_array_equal(O.swiglu(np.c_[np.zeros(81), u]), np.zeros((81, 1)))
    # hand value: SiLU(1) * 2 = 2 / (1 + e^-1)
    assert abs(O.swiglu(np.array([[1.0, 2.0]]))[0, 0] - 2.0 / (1.0 + math.exp(-1.0))) < 1e-15
    # gate first: swapping the halves changes the result
    assert abs(O.swiglu(np.array([[2.0, 1.0]]))[0, 0] - 2.0 / (1.0 + math.exp(-2.0))) < 1e-15
    # several features: column f pairs gate f with value M + f
    x = rng.standard_normal((3, 8))
    np.testing.assert_allclose(O.swiglu(x), x[:, :4] * expit(x[:, :4]) * x[:, 4:], rtol=1e-13)


# ---------------------------------------------------------------- linear
def test_linear_brute_force_tiny_rectangular():
    x = rng.standard_normal((3, 5))
    lin = synth.Linear(rng.standard_normal((4, 5)), rng.standard_normal(4))
    y = O.linear(x, lin)
    want = [[math.fsum([x[i][k] * lin.w[n][k] for k in range(5)]) + lin.b[n] for n in range(4)] for i in range(3)]
    np.testing.assert_allclose(y, want, rtol=0, atol=1e-14)


def test_linear_int8_is_scale_after_integer_product():
    q = rng.integers(-127, 128, size=(6, 9)).astype(np.int8)
    s = rng.uniform(1e-4, 1e-2, 6).astype(np.float32)
    b = rng.standard_normal(6)
    x = rng.standard_normal((4, 9))
    lin = synth.Linear(None, b, q, s)
    y = O.linear(x, lin)
    want = [[math.fsum([x[i][k] * int(q[n][k]) for k in range(9)]) * float(s[n]) + b[n] for n in range(6)]
            for i in range(4)]
    np.testing.assert_allclose(y, want, rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- time embedding / euler
def test_timestep_embedding_closed_forms():
    e0 = O.timestep_embedding(0.0)
    np.testing.assert_array_equal(e0, np.concatenate([np.ones(128), np.zeros(128)]))
    t = 0.37
    e = O.timestep_embedding(t)
    assert e.shape == (256,)
    assert abs(e[0] - math.cos(370.0)) < 1e-12 and abs(e[128] - math.sin(370.0)) < 1e-12
    # lowest frequency: 1e4^(-127/128)
    f = 1e4 ** (-127 / 128)
    assert abs(e[127] - math.cos(370.0 * f)) < 1e-12 and abs(e[255] - math.sin(370.0 * f)) < 1e-12
    np.testing.assert_allclose(e[:128] ** 2 + e[128:] ** 2, 1.0, rtol=1e-14)


def test_euler_closed_form_multi_step():
    z0 = rng.standard_normal((10, 4))
    c = rng.standard_normal(4)
    ts = synth.sigma_schedule(28)
    z = z0
    for i in range(28):
        z = O.euler(z, np.tile(c, (10, 1)), ts[i], ts[i + 1])
    np.testing.assert_allclose(z, z0 - c, atol=1e-13)


# ---------------------------------------------------------------- blocks
TINY = synth.custom_shape("pin-tiny", 900, 64, 2, 128, 8, (4, 6))


def _zero(lin, rows=None):
    w = lin.w.copy(); b = lin.b.copy()
    if rows is None:
        w[:] = 0; b[:] = 0
    else:
        w[rows] = 0; b[rows] = 0
    return synth.Linear(w, b)


def test_double_block_zero_gate_identity():
    d = synth.block_inputs(TINY, "double")
    H = TINY.hidden
    w = d["w"]
    gates = np.r_[2 * H:3 * H, 5 * H:6 * H]
    for s in ("txt", "img"):
        w[s]["mod"] = _zero(w[s]["mod"], gates)
    out = O.double_block(d["x"], d["vec"], d["ids"], w, TINY)
    np.testing.assert_array_equal(out, d["x"].astype(np.float64))


def test_double_block_constant_branch_closed_form():
    """With zero qkv and fc1 weights (biases kept), every key and value is the
    bias, attention returns the v-bias, and each stream's update is
    gate1 * (W_o b_v + b_o) + gate2 * (W_2 GELU(b_1) + b_2): a closed form that
    pins the gate chunks, the [q|k|v] split and the proj / fc2 wiring."""
    d = synth.block_inputs(TINY, "double", variant=1)
    H = TINY.hidden
    w = d["w"]
    x = d["x"].astype(np.float64)
    want = x.copy()
    silu_vec = d["vec"] / (1 + np.exp(-d["vec"].astype(np.float64)))
    for s, sl in (("txt", slice(0, TINY.txt_len)), ("img", slice(TINY.txt_len, None))):
        w[s]["qkv"] = synth.Linear(np.zeros_like(w[s]["qkv"].w), w[s]["qkv"].b)
        w[s]["fc1"] = synth.Linear(np.zeros_like(w[s]["fc1"].w), w[s]["fc1"].b)
    # both streams get one v-bias, so every value is that bias and attention
    # returns it whatever the (RoPE-dependent) attention weights are
    bq = w["img"]["qkv"].b.copy(); bq[2 * H:] = w["txt"]["qkv"].b[2 * H:]
    w["img"]["qkv"] = synth.Linear(w["img"]["qkv"].w, bq)
    o = w["txt"]["qkv"].b[2 * H:].astype(np.float64)
    for s, sl in (("txt", slice(0, TINY.txt_len)), ("img", slice(TINY.txt_len, None))):
        m = w[s]["mod"].w.astype(np.float64) @ silu_vec + w[s]["mod"].b
        g1, g2 = m[2 * H:3 * H], m[5 * H:6 * H]
        c1 = w[s]["proj"].w.astype(np.float64) @ o + w[s]["proj"].b
        b1 = w[s]["fc1"].b.astype(np.float64)
        gb1 = 0.5 * b1 * (1 + erf(b1 / math.sqrt(2)))  # erf GELU, tanh form within 5e-4
        c2 = w[s]["fc2"].w.astype(np.float64) @ gb1 + w[s]["fc2"].b
        want[sl] += g1 * c1 + g2 * c2
    out = O.double_block(x, d["vec"], d["ids"], w, TINY)
    # the only slack is the gap between the tanh and erf forms of GELU, at most
    # 4.8e-4 per element, carried through |W_2| and |gate2|
    for s, sl in (("txt", slice(0, TINY.txt_len)), ("img", slice(TINY.txt_len, None))):
        m = w[s]["mod"].w.astype(np.float64) @ silu_vec + w[s]["mod"].b
        bound = np.abs(m[5 * H:6 * H]) * 4.8e-4 * np.abs(w[s]["fc2"].w.astype(np.float64)).sum(axis=1) + 1e-12
        assert np.all(np.abs(out[sl] - want[sl]) <= bound[None, :])


def test_double_block_norm_scales_wired_per_tensor_and_stream():
    """RoPE keeps each (2j, 2j+1) pair's norm, so the pair norms of the block's
    q and k equal those of the RMSNorm (already pinned) of the raw projections
    with that tensor's and that stream's own scale."""
    d = synth.block_inputs(TINY, "double", variant=4)
    H, D = TINY.hidden, TINY.head_dim
    _, st = O.double_block(d["x"], d["vec"], d["ids"], d["w"], TINY, return_stages=True)
    pair = lambda a: a[:, 0::2] ** 2 + a[:, 1::2] ** 2
    for s, sl in (("txt", slice(0, TINY.txt_len)), ("img", slice(TINY.txt_len, None))):
        raw = st[f"qkv_{s}"]
        for name, off in (("q", 0), ("k", H)):
            for h in range(TINY.heads):
                cols = slice(h * D, (h + 1) * D)
                want = O.rms_norm(raw[:, off + h * D: off + (h + 1) * D], d["w"][s][f"{name}_norm"], TINY.rms_eps)
                np.testing.assert_allclose(pair(st[name][sl][:, cols]), pair(want), rtol=1e-10, atol=1e-14)


def test_double_block_within_stream_permutation_equivariance():
    """Permuting tokens inside each stream together with their position ids
    permutes the output the same way (attention has no mask and RoPE travels
    with the ids)."""
    d = synth.block_inputs(TINY, "double", variant=2)
    L_t, L = TINY.txt_len, TINY.seq_len
    perm = np.r_[rng.permutation(L_t), L_t + rng.permutation(L - L_t)]
    out = O.double_block(d["x"], d["vec"], d["ids"], d["w"], TINY)
    outp = O.double_block(d["x"][perm], d["vec"], d["ids"][perm], d["w"], TINY)
    np.testing.assert_allclose(outp, out[perm], atol=1e-11)
    # and it is not invariant to moving a token's position id alone
    ids2 = d["ids"].copy(); ids2[[L_t, L_t + 1]] = ids2[[L_t + 1, L_t]]
    out2 = O.double_block(d["x"], d["vec"], ids2, d["w"], TINY)
    assert np.max(np.abs(out2 - out)) > 1e-6


def test_double_block_rows_subset_matches_full():
    d = synth.block_inputs(TINY, "double", variant=3)
    out = O.double_block(d["x"], d["vec"], d["ids"], d["w"], TINY)
    rows = np.array([0, 3, TINY.txt_len, TINY.seq_len - 1])
    np.testing.assert_allclose(O.double_block(d["x"], d["vec"], d["ids"], d["w"], TINY, rows=rows), out[rows],
                               atol=1e-12)


def test_single_block_zero_gate_and_constant_branch():
    d = synth.block_inputs(TINY, "single")
    H, M = TINY.hidden, TINY.mlp
    w = d["w"]
    w0 = dict(w); w0["mod"] = _zero(w["mod"], np.r_[2 * H:3 * H])
    np.testing.assert_array_equal(O.single_block(d["x"], d["vec"], d["ids"], w0, TINY), d["x"].astype(np.float64))
    # zero linear1 weight: q, k, v, m are the bias chunks; attention returns b_v
    w1 = dict(w); w1["linear1"] = synth.Linear(np.zeros_like(w["linear1"].w), w["linear1"].b)
    b = w["linear1"].b.astype(np.float64)
    bm = b[3 * H:]
    cat = np.concatenate([b[2 * H:3 * H], 0.5 * bm * (1 + np.tanh(math.sqrt(2 / math.pi) * (bm + 0.044715 * bm ** 3)))])
    v = d["vec"].astype(np.float64)
    mod = w["mod"].w.astype(np.float64) @ (v * expit(v)) + w["mod"].b
    gate = mod[2 * H:]
    want = d["x"] + gate * (w["linear2"].w.astype(np.float64) @ cat + w["linear2"].b)
    np.testing.assert_allclose(O.single_block(d["x"], d["vec"], d["ids"], w1, TINY), want, atol=1e-11)


def test_single_block_permutation_equivariance():
    d = synth.block_inputs(TINY, "single", variant=1)
    perm = rng.permutation(TINY.seq_len)
    out = O.single_block(d["x"], d["vec"], d["ids"], d["w"], TINY)
    outp = O.single_block(d["x"][perm], d["vec"], d["ids"][perm], d["w"], TINY)
    np.testing.assert_allclose(outp, out[perm], atol=1e-11)


def test_denoise_step_closed_form_zero_final_weight():
    shp = synth.custom_shape("pin-step", 901, 64, 2, 128, 8, (4, 4), n_double=1, n_single=1, in_channels=16)
    m = synth.model_weights(shp, int8=False)
    c = rng.standard_normal(16)
    m["final_out"] = synth.Linear(np.zeros((16, 64)), c)
    s = synth.step_inputs(shp)
    z1, v = O.denoise_step(s["z"], s["txt"], s["ids"], m, shp, 1.0, 1.0 - 1 / 28, 3.5)
    np.testing.assert_allclose(v, np.tile(c, (shp.img_len, 1)), atol=1e-14)
    np.testing.assert_allclose(z1, s["z"] - c / 28, atol=1e-14)


def test_block_structure_matches_reported_launch_counts():
    """A Klein-structured step (8 double + 24 single blocks and a final layer)
    runs exactly the per-step fused-kernel counts the Luminal blog reports."""
    with open(os.path.join(GOLDEN, "klein_structure.json")) as f:
        g = json.load(f)
    shp = synth.custom_shape("pin-klein", 902, 64, 2, 64, 4, (2, 2), n_double=g["double_blocks"],
                             n_single=g["single_blocks"], in_channels=8)
    m = synth.model_weights(shp, int8=False)
    s = synth.step_inputs(shp)
    O.SITE_COUNTS.clear()
    O.velocity(s["z"], s["txt"], s["ids"], m, shp, 0.5, 3.5)
    assert O.SITE_COUNTS["rmsnorm_rope"] == g["rmsnorm_rope_per_step"]
    assert O.SITE_COUNTS["ln_modulate"] == g["ln_modulate_per_step"]
    assert O.SITE_COUNTS["attention"] == g["attention_sites_per_step"]


def test_consistency_int8_step_equals_step_on_dequantised_weights():
    """Consistency check, not a pin (it compares the oracle with itself): an
    int8 model and the same model with W := diag(s) Q stored as float weights
    give the same velocity, i.e. the int8 layers reach the linears only
    through weight_matrix. The int8 linear itself is pinned by
    test_linear_int8_is_scale_after_integer_product."""
    shp = synth.custom_shape("pin-int8", 903, 64, 2, 128, 8, (4, 4), n_double=1, n_single=1, in_channels=16)
    m8 = synth.model_weights(shp, int8=True)

    def deq(l):
        return synth.Linear(l.s.astype(np.float64)[:, None] * l.q.astype(np.float64), l.b)

    def walk(o):
        if isinstance(o, synth.Linear):
            return deq(o)
        if isinstance(o, dict):
            return {k: walk(v) for k, v in o.items()}
        if isinstance(o, list):
            return [walk(v) for v in o]
        return o
    mf = walk(m8)
    s = synth.step_inputs(shp)
    v8 = O.velocity(s["z"], s["txt"], s["ids"], m8, shp, 0.8, 3.5)
    vf = O.velocity(s["z"], s["txt"], s["ids"], mf, shp, 0.8, 3.5)
    np.testing.assert_array_equal(v8, vf)


def _param_count(shp) -> int:
    """Parameters of a model of this shape, from the layer sizes that
    synth.model_weights draws (biases and norm scales included)."""
    H, D, C = shp.hidden, shp.head_dim, shp.in_channels

    def lin(o, i):
        return o * i + o
    dbl = 2 * (lin(3 * H, H) + lin(H, H) + lin(shp.mlp_out, H) + lin(H, shp.mlp) + 2 * D)
    sgl = lin(3 * H + shp.mlp_out, H) + lin(H, H + shp.mlp) + 2 * D
    mod_d, mod_s = 2 * lin(6 * H, H), lin(3 * H, H)
    emb = lin(H, C) + lin(H, 256) + lin(H, H) + lin(2 * H, H) + lin(C, H)
    if shp.guidance_embed:
        emb += lin(H, 256) + lin(H, H)
    if shp.shared_mod:
        return shp.n_double * dbl + shp.n_single * sgl + mod_d + mod_s + emb
    return shp.n_double * (dbl + mod_d) + shp.n_single * (sgl + mod_s) + emb


def test_klein_shape_readings_give_nine_billion_parameters():
    """The Luminal blog names the model Flux.2 Klein 9B and gives H 4096, 32
    heads, 8 double and 24 single blocks, SwiGLU. The pages leave the MLP width
    and the modulation layout open; the readings taken (MLP width 3H, one
    modulation per block type) give 9.03 B parameters. The alternatives miss
    the name: width 4H gives 11.0 B, per-block modulation 11.6 B, width 8H/3
    8.3 B."""
    shp = synth.KLEIN_STEP_512
    assert (shp.hidden, shp.heads, shp.n_double, shp.n_single, shp.mlp_act) == (4096, 32, 8, 24, "swiglu")
    n = _param_count(shp)
    assert abs(n - 9.0e9) < 0.02 * 9.0e9, n
    import dataclasses
    for alt in (dataclasses.replace(shp, mlp=4 * 4096), dataclasses.replace(shp, shared_mod=False),
                dataclasses.replace(shp, mlp=10880)):
        assert abs(_param_count(alt) - 9.0e9) > 0.05 * 9.0e9


def test_klein_step_structure_matches_reported_launch_counts():
    """The Klein-shaped step (SwiGLU, guidance-free, reference image appended,
    shared modulation) runs the per-step fused-kernel counts of the Luminal
    blog too: the editing tokens change lengths, not the block structure."""
    with open(os.path.join(GOLDEN, "klein_structure.json")) as f:
        g = json.load(f)
    shp = synth.custom_shape("pin-klein-edit", 904, 64, 2, 128, 4, (2, 2), n_double=g["double_blocks"],
                             n_single=g["single_blocks"], **synth.KLEIN_KW)
    m = synth.model_weights(shp, int8=False)
    s = synth.step_inputs(shp)
    O.SITE_COUNTS.clear()
    O.velocity(s["z"], s["txt"], s["ids"], m, shp, 0.5, 0.0)
    assert O.SITE_COUNTS["rmsnorm_rope"] == g["rmsnorm_rope_per_step"]
    assert O.SITE_COUNTS["ln_modulate"] == g["ln_modulate_per_step"]
    assert O.SITE_COUNTS["attention"] == g["attention_sites_per_step"]


def test_edit_step_reference_rows_and_guidance_free_conditioning():
    """Editing: the reference latent rows ride along unchanged, sit at time
    index 1 of the position ids, and are attended to (changing them changes
    the prediction). Guidance-free: the guidance value has no effect."""
    shp = synth.custom_shape("pin-edit", 905, 64, 2, 128, 4, (3, 3), n_double=1, n_single=1, **synth.KLEIN_KW)
    m = synth.model_weights(shp, int8=False)
    s = synth.step_inputs(shp)
    n, r = shp.img_len - shp.ref_len, shp.ref_len
    assert (n, r) == (9, 9)
    ids = s["ids"]
    np.testing.assert_array_equal(ids[shp.txt_len:shp.txt_len + n, 0], 0)
    np.testing.assert_array_equal(ids[shp.txt_len + n:, 0], 1)
    np.testing.assert_array_equal(ids[shp.txt_len:shp.txt_len + n, 1:], ids[shp.txt_len + n:, 1:])
    z1, v = O.denoise_step(s["z"], s["txt"], ids, m, shp, 1.0, 0.75, 3.5)
    assert v.shape == (n, shp.in_channels)
    np.testing.assert_array_equal(z1[n:], s["z"][n:])
    np.testing.assert_allclose(z1[:n], s["z"][:n] - 0.25 * v, atol=1e-14)
    z2, v2 = O.denoise_step(s["z"], s["txt"], ids, m, shp, 1.0, 0.75, -7.0)
    np.testing.assert_array_equal(v2, v)
    zr = s["z"].copy()
    zr[n:] = rng.standard_normal((r, shp.in_channels))
    _, v3 = O.denoise_step(zr, s["txt"], ids, m, shp, 1.0, 0.75, 3.5)
    assert np.max(np.abs(v3 - v)) > 1e-6
    # shared modulation: every block of a type holds the same weights
    assert m["single"][0]["mod"] is m["single"][-1]["mod"]



def _e4m3_decode(code: int) -> float:
    """OCP e4m3 bit pattern -> value, straight from the field layout."""
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def test_e4m3_round_against_the_bit_level_format():
    """The oracle's e4m3 rounding reproduces the format's 253 distinct finite
    values, fixes every one of them, and sends each midpoint to the neighbour
    with the even code (round to nearest even); 448 is the largest value."""
    vals = sorted({_e4m3_decode(c) for c in range(256) if not math.isnan(_e4m3_decode(c))})
    assert len(vals) == 253 and vals[-1] == 448.0 and vals[0] == -448.0
    np.testing.assert_array_equal(O.e4m3_round(np.array(vals)), np.array(vals))
    pos = [v for v in vals if v >= 0]
    code_of = {}
    for c in range(128):
        v = _e4m3_decode(c)
        if not math.isnan(v):
            code_of.setdefault(v, c)
    for lo, hi in zip(pos[:-1], pos[1:]):
        mid = (lo + hi) / 2
        even = lo if code_of[lo] % 2 == 0 else hi
        assert O.e4m3_round(np.array([mid]))[0] == even, (lo, hi)
        assert O.e4m3_round(np.array([-mid]))[0] == -even
        # just off the midpoint: the nearer neighbour
        assert O.e4m3_round(np.array([mid - (hi - lo) / 64]))[0] == lo
        assert O.e4m3_round(np.array([mid + (hi - lo) / 64]))[0] == hi
    assert O.e4m3_round(np.array([2.0 ** -9]))[0] == 2.0 ** -9          # smallest subnormal
    assert O.e4m3_round(np.array([2.0 ** -10]))[0] == 0.0               # tie to 0 (even)


def test_fp8_row_quantisation_closed_forms():
    x = rng.standard_normal((6, 96)).astype(np.float32)
    x[3] = 0.0
    codes, sc = O.quantize_rows_fp8(x)
    assert sc.dtype == np.float32 and sc[3] == 0 and np.all(codes[3] == 0)
    for r in (0, 1, 2, 4, 5):
        assert sc[r] == np.float32(np.max(np.abs(x[r])) / np.float32(448.0))
        assert np.max(np.abs(codes[r])) == 448.0        # the largest element maps to the top code
        # dequantisation error: at most half a step, i.e. 2^-4 of the value for normal codes
        deq = sc[r].astype(np.float64) * codes[r]
        err = np.abs(deq - x[r])
        normal = np.abs(codes[r]) >= 2.0 ** -6
        assert np.all(err[normal] <= np.abs(x[r][normal]) * 2.0 ** -4 * (1 + 1e-6))
        assert np.all(err[~normal] <= sc[r] * 2.0 ** -10 * (1 + 1e-6))
    # a linear over dequantised operands is the plain product of the dequantised matrices
    w = rng.standard_normal((8, 96)).astype(np.float32)
    wc, ws = O.quantize_rows_fp8(w)
    b = rng.standard_normal(8)
    y = O.linear_fp8(codes, sc, wc, ws, b)
    brute = np.array([[sum(float(sc[i]) * codes[i, k] * float(ws[j]) * wc[j, k] for k in range(96)) + b[j]
                       for j in range(8)] for i in range(6)])
    np.testing.assert_allclose(y, brute, rtol=1e-12, atol=1e-12)


def _fp8_exact_rows(shape, seed):
    """Rows of e4m3 values times a power of two per row, with the top code
    (448) in every row: per-row quantisation is the identity on them."""
    g = np.random.default_rng(seed)
    vals = np.array(sorted({_e4m3_decode(c) for c in range(256) if not math.isnan(_e4m3_decode(c))}))
    r = g.choice(vals, size=shape)
    r[:, 0] = 448.0
    return r * np.exp2(g.integers(-12, -4, size=(shape[0], 1)))


def test_fp8_linear_identity_on_fp8_exact_operands_and_error_bound():
    """linear_act_fp8 on the fp8 form of a layer: exactly the plain linear
    when both operands are already fp8-exact with a power-of-two row scale,
    and otherwise within the elementwise bound that half a code step on each
    operand gives (2^-4 of a normal value, 2^-10 of the row scale below it),
    plus the fp32 rounding of the quotient the code is decided on (2^-24 of
    it)."""
    x = _fp8_exact_rows((5, 128), 1)
    w = _fp8_exact_rows((7, 128), 2)
    b = rng.standard_normal(7)
    lin = synth.Linear(w.astype(np.float32), b)
    q = O.fp8_weights(lin)
    np.testing.assert_array_equal(q.q * q.s[:, None].astype(np.float64), w)
    np.testing.assert_array_equal(O.linear_act_fp8(x, q), O.linear(x, lin))
    # generic operands
    x = rng.standard_normal((6, 256)).astype(np.float32)
    x[2] *= 1e-3                                       # a row deep in its own scale
    w = (0.02 * rng.standard_normal((9, 256))).astype(np.float32)
    lin = synth.Linear(w, b[:9] if len(b) >= 9 else rng.standard_normal(9))
    q = O.fp8_weights(lin)
    y8 = O.linear_act_fp8(x, q)
    y = O.linear(x, lin)
    sx = np.max(np.abs(x), axis=1) / 448.0
    sw = np.max(np.abs(w), axis=1) / 448.0
    ex = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * sx[:, None]) * (1 + 2.0 ** -20)
    ew = np.maximum(2.0 ** -4 * np.abs(w), 2.0 ** -10 * sw[:, None]) * (1 + 1e-6)
    ax, aw = np.abs(x).astype(np.float64), np.abs(w).astype(np.float64)
    bound = ex @ aw.T + ax @ ew.T + ex @ ew.T
    assert np.all(np.abs(y8 - y) <= bound + 1e-12)
    assert np.max(np.abs(y8 - y)) > 0                  # the quantisation is applied


@pytest.mark.parametrize("kind", ["double", "single"])
def test_fp8_block_close_to_exact_block_and_gate_identity(kind):
    """The fp8 block moves the block's update by the quantisation noise of its
    projections, no more: a few percent of the update, and not nothing.
    Rounding to 3 mantissa bits leaves an RMS error of 2^-4..2^-3 / sqrt(12)
    of a value (~2.7% on average); a product of two quantised operands ~3.8%,
    and a chain of two projections (fc1 -> GELU -> fc2, or qkv -> attention
    -> proj) ~5.5%: measured ~5.8% on both block kinds. Zeroed gates still
    return the input exactly."""
    inp = synth.block_inputs(synth.TINY, kind, variant=3)
    f = O.double_block if kind == "double" else O.single_block
    args = (inp["x"], inp["vec"], inp["ids"], inp["w"], synth.TINY)
    exact = f(*args)
    q8 = f(*args, fp8=True)
    d = exact - inp["x"]
    e = np.sqrt(np.mean((q8 - exact) ** 2)) / np.sqrt(np.mean(d ** 2))
    assert 2e-2 < e < 1e-1, e
    # pre-quantised weights pass through fp8_weights unchanged
    w8 = O.fp8_weights(inp["w"])
    np.testing.assert_array_equal(f(inp["x"], inp["vec"], inp["ids"], w8, synth.TINY, fp8=True), q8)
    H = synth.TINY.hidden
    mods = [inp["w"][s]["mod"] for s in ("txt", "img")] if kind == "double" else [inp["w"]["mod"]]
    for lin in mods:
        rows = (2 * H, 5 * H) if kind == "double" else (2 * H,)
        for r0 in rows:
            lin.w[r0:r0 + H] = 0
            lin.b[r0:r0 + H] = 0
    np.testing.assert_array_equal(f(*args, fp8=True), inp["x"])


@pytest.mark.parametrize("kind", ["double", "single"])
def test_sharp_update_detects_rope_mistakes(kind):
    """The GPU test of the block update under sharp attention
    (test_gpu_blocks.py::test_block_sharp_attention_update, bound 2e-2) would
    catch a mistake in the RoPE stage: planted here in the oracle's inputs,
    on the CPU — image positions with the h and w axes swapped, or no
    rotation at all (every position 0) — the update moves by far more than
    that bound."""
    from sharp_inputs import sharp_block_inputs, update_rms_err

    shp = synth.custom_shape("ragged-h256-d128-L203", 711, 256, 2, 512, 3, (10, 20))
    inp = sharp_block_inputs(shp, kind)
    f = O.double_block if kind == "double" else O.single_block
    ref = f(inp["x"], inp["vec"], inp["ids"], inp["w"], shp)
    swapped = inp["ids"].copy()
    swapped[:, [1, 2]] = swapped[:, [2, 1]]
    zero = np.zeros_like(inp["ids"])
    for ids in (swapped, zero):
        bad = f(inp["x"], inp["vec"], ids, inp["w"], shp)
        assert update_rms_err(bad, ref, inp["x"]) > 0.3


# ---------------------------------------------------------------- conditioning, embedder, final layer, residual order
# Closed forms of a block and of a whole step in which the attention branch is
# a constant (zero q/k/v weights: every value is the v-bias, so attention
# returns it whatever its weights are). What is left is a composition of
# textbook layers, computed here with PyTorch's own float64 CPU routines
# (F.linear, F.silu, F.gelu, F.layer_norm), independent of the oracle's numpy
# code. The Luminal blog ("What the compiler found on its own") fixes the
# pieces: a timestep embedding conditions the blocks, a LayerNorm followed by
# a scale-and-shift modulation, and a gate-and-residual add after each branch.
def _t(a):
    import torch
    return torch.as_tensor(np.asarray(a, dtype=np.float64))


def _lin_t(x, lin):
    import torch.nn.functional as F
    return F.linear(x, _t(lin.w), _t(lin.b))


def _emb_brute(t, dim=256):
    """Sinusoidal embedding by plain loops (its own closed forms are pinned in
    test_timestep_embedding_closed_forms)."""
    half = dim // 2
    f = [math.exp(-math.log(1e4) * k / half) for k in range(half)]
    return [math.cos(1000.0 * t * fk) for fk in f] + [math.sin(1000.0 * t * fk) for fk in f]


def _scaled(lin, f):
    return synth.Linear(lin.w * f, lin.b * f)


def _constant_attention(w, H):
    """Zero the q/k/v weights of a double block (both streams share one
    v-bias) so that attention returns that v-bias for every token. The
    modulation, output projection and MLP weights are scaled up (N(0, 0.02)
    layers of width 64 would leave each branch at ~1e-3 of x, too small for
    the residual order to show)."""
    bv = w["txt"]["qkv"].b[2 * H:].copy() * 50.0
    for s in ("txt", "img"):
        b = w[s]["qkv"].b.copy()
        b[2 * H:] = bv
        w[s]["qkv"] = synth.Linear(np.zeros_like(w[s]["qkv"].w), b)
        w[s]["mod"] = _scaled(w[s]["mod"], 10.0)
        w[s]["proj"] = _scaled(w[s]["proj"], 25.0)
        w[s]["fc1"] = _scaled(w[s]["fc1"], 25.0)
        w[s]["fc2"] = _scaled(w[s]["fc2"], 25.0)
    return bv


def _double_stream_closed_form(x_s, sv, ws, bv, H, eps):
    """One stream of a double block whose attention output is the constant bv:
    x1 = x + gate1 (W_o bv + b_o); x2 = x1 + gate2 fc2(GELU(fc1(LN(x1)(1+scale2)+shift2)))."""
    import torch.nn.functional as F
    m = _lin_t(sv, ws["mod"])
    sh2, sc2, g1, g2 = m[3 * H:4 * H], m[4 * H:5 * H], m[2 * H:3 * H], m[5 * H:6 * H]
    x1 = _t(x_s) + g1 * _lin_t(_t(bv), ws["proj"])
    h2 = F.layer_norm(x1, (H,), eps=eps) * (1 + sc2) + sh2
    return x1 + g2 * _lin_t(F.gelu(_lin_t(h2, ws["fc1"]), approximate="tanh"), ws["fc2"])


def test_double_block_residual_order_closed_form():
    """LN2 reads the residual after the attention branch's gated add (x +
    gate1 * proj(O)), not the block input: with a constant attention output
    and a non-zero fc1 the MLP branch depends on which one it reads (the
    constant-branch pin above zeroes fc1, which hides that)."""
    import torch.nn.functional as F
    d = synth.block_inputs(TINY, "double", variant=5)
    H, Lt = TINY.hidden, TINY.txt_len
    w = d["w"]
    bv = _constant_attention(w, H)
    out = O.double_block(d["x"], d["vec"], d["ids"], w, TINY)
    sv = F.silu(_t(d["vec"]))
    for s, sl in (("txt", slice(0, Lt)), ("img", slice(Lt, None))):
        want = _double_stream_closed_form(d["x"][sl], sv, w[s], bv, H, TINY.ln_eps).numpy()
        np.testing.assert_allclose(out[sl], want, rtol=1e-9, atol=1e-11)
        # the other order (LN2 of the block input) is far from it
        m = _lin_t(sv, w[s]["mod"])
        x0 = _t(d["x"][sl])
        x1 = x0 + m[2 * H:3 * H] * _lin_t(_t(bv), w[s]["proj"])
        h2 = F.layer_norm(x0, (H,), eps=TINY.ln_eps) * (1 + m[4 * H:5 * H]) + m[3 * H:4 * H]
        wrong = (x1 + m[5 * H:] * _lin_t(F.gelu(_lin_t(h2, w[s]["fc1"]), approximate="tanh"), w[s]["fc2"])).numpy()
        assert np.max(np.abs(wrong - want)) > 0.1


STEP_CF = synth.custom_shape("pin-step-cf", 906, 64, 2, 128, 8, (4, 4), n_double=1, n_single=1, in_channels=16)


def _step_closed_form_model():
    m = synth.model_weights(STEP_CF, int8=False)
    H = STEP_CF.hidden
    bv = _constant_attention(m["double"][0], H)
    ws = m["single"][0]
    ws["linear1"] = synth.Linear(np.zeros_like(ws["linear1"].w), ws["linear1"].b)
    return m, bv


def _step_closed_form_velocity(m, bv, z, t, guidance):
    """v of a step whose double block has a constant attention output and
    whose single block has a zero linear1 weight, by textbook layers:
      vec   = L2_t(SiLU(L1_t(emb(t)))) + L2_g(SiLU(L1_g(emb(guidance))))
      x_img = img_in(z), then the double block's image stream (closed form
              above), then + gate (linear2([b_v | GELU(b_m)])) of the single block
      v     = final_out(LN(x_img)(1 + scale) + shift), (shift, scale) = final_mod(SiLU(vec))."""
    import torch
    import torch.nn.functional as F
    H, eps = STEP_CF.hidden, STEP_CF.ln_eps
    vec = (_lin_t(F.silu(_lin_t(_t(_emb_brute(t)), m["time_in"][0])), m["time_in"][1])
           + _lin_t(F.silu(_lin_t(_t(_emb_brute(guidance)), m["guid_in"][0])), m["guid_in"][1]))
    sv = F.silu(vec)
    x = _lin_t(_t(z), m["img_in"])
    x = _double_stream_closed_form(x, sv, m["double"][0]["img"], bv, H, eps)
    ws = m["single"][0]
    gate = _lin_t(sv, ws["mod"])[2 * H:]
    b1 = _t(ws["linear1"].b)
    cat = torch.cat([b1[2 * H:3 * H], F.gelu(b1[3 * H:], approximate="tanh")])
    x = x + gate * _lin_t(cat, ws["linear2"])
    fm = _lin_t(sv, m["final_mod"])
    h = F.layer_norm(x, (H,), eps=eps) * (1 + fm[H:]) + fm[:H]
    return _lin_t(h, m["final_out"]).numpy()


def _step_closed_form_gap(t0=0.8, t1=0.8 - 1 / 28, guidance=3.5):
    """Max |oracle - closed form| over v and z_next, and the RMS of v."""
    m, bv = _step_closed_form_model()
    s = synth.step_inputs(STEP_CF)
    z1, v = O.denoise_step(s["z"], s["txt"], s["ids"], m, STEP_CF, t0, t1, guidance)
    want = _step_closed_form_velocity(m, bv, s["z"], t0, guidance)
    gap = max(np.max(np.abs(v - want)), np.max(np.abs(z1 - (s["z"] + (t1 - t0) * want))))
    return gap, float(np.sqrt(np.mean(want * want)))


def test_denoise_step_closed_form_conditioning_embedder_final_layer():
    """The whole step against its closed form: pins the timestep and
    guidance embedders (Linear-SiLU-Linear each, summed), the latent's patch
    embedding, the image rows the final layer reads, its modulated LayerNorm
    and projection, and the Euler update (flux-amd-rocm: guidance 3.5)."""
    gap, rms = _step_closed_form_gap()
    assert rms > 0.1
    assert gap <= 1e-10 * max(rms, 1.0), gap


def _planted(monkeypatch, name, fn):
    from oracle import mmdit_oracle as M
    monkeypatch.setattr(M, name, fn)


def test_step_closed_form_catches_planted_mistakes(monkeypatch):
    """Plausible mistakes planted in the oracle's conditioning, embedder,
    final layer and residual order each move the step far from its closed
    form (so the pin above would fail on them)."""
    from oracle import mmdit_oracle as M
    good = {k: getattr(M, k) for k in ("mlp_embedder", "conditioning", "velocity", "ln_modulate", "linear")}

    def emb_no_inner_silu(e, lins):
        return good["linear"](good["linear"](e[None, :], lins[0]), lins[1])[0]

    def cond_no_guidance(t, g, m):
        return good["mlp_embedder"](M.timestep_embedding(t), m["time_in"])

    def cond_guidance_from_t(t, g, m):
        return good["conditioning"](t, t, m)

    def velocity_wrong_rows(z, txt, ids, m, shp, t, g, fp8=False):
        vec = M.conditioning(t, g, m)
        x = np.concatenate([M._f64(txt), M.linear(z, m["img_in"])], axis=0)
        for wd in m["double"]:
            x = M.double_block(x, vec, ids, wd, shp)
        for ws in m["single"]:
            x = M.single_block(x, vec, ids, ws, shp)
        sh, sc = M.modulation(vec, m["final_mod"], 2)
        h = M.ln_modulate(x[-shp.img_len:][::-1], sh, sc, shp.ln_eps)   # rows reversed
        return M.linear(h, m["final_out"])

    def velocity_swapped_shift_scale(z, txt, ids, m, shp, t, g, fp8=False):
        orig = M.modulation

        def swapped(vec, lin, chunks):
            parts = orig(vec, lin, chunks)
            return parts[::-1] if chunks == 2 else parts
        try:
            M.modulation = swapped
            return good["velocity"](z, txt, ids, m, shp, t, g)
        finally:
            M.modulation = orig

    cases = [("mlp_embedder", emb_no_inner_silu), ("conditioning", cond_no_guidance),
             ("conditioning", cond_guidance_from_t), ("velocity", velocity_wrong_rows),
             ("velocity", velocity_swapped_shift_scale)]
    for name, fn in cases:
        with monkeypatch.context() as mp:
            mp.setattr(M, name, fn)
            gap, rms = _step_closed_form_gap()
            assert gap > 1e-3 * rms, (name, fn.__name__, gap)
    # residual order: the double block with LN2 reading the block input
    src = M.double_block

    def double_ln2_of_input(x, vec, ids, w, shp, **kw):
        x0 = M._f64(x)
        orig_ln = M.ln_modulate
        seen = []

        def ln(xs, sh, sc, eps):
            seen.append(xs)
            if len(seen) > 2:      # LN2 sites (after the two LN1 sites): block input rows instead
                Lt = shp.txt_len
                xs = x0[:Lt] if len(seen) == 3 else x0[Lt:]
            return orig_ln(xs, sh, sc, eps)
        try:
            M.ln_modulate = ln
            return src(x, vec, ids, w, shp, **kw)
        finally:
            M.ln_modulate = orig_ln
    with monkeypatch.context() as mp:
        mp.setattr(M, "double_block", double_ln2_of_input)
        gap, rms = _step_closed_form_gap()
        assert gap > 1e-3 * rms, gap
    # and the unplanted oracle is back on the closed form
    gap, rms = _step_closed_form_gap()
    assert gap <= 1e-10 * max(rms, 1.0)


def test_fp8_step_with_identity_blocks_is_the_step_on_decoded_weights():
    """The fp8 denoise step (SGLang-AMD, Architecture Deep Dive: fp8 on CDNA):
    with every block's gates zeroed the blocks return their input, and what
    is left (embedders, patch embedding, modulations, final layer) runs on the
    fp8 weights alone, so the step equals the plain step on the decoded
    weights diag(s) e4m3(W / s). With the gates on, the blocks' per-token
    activation quantisation moves v by a few percent of its RMS, not more."""
    shp = synth.custom_shape("pin-fp8-step", 907, 128, 2, 256, 8, (4, 4), n_double=1, n_single=1, in_channels=16)
    H = shp.hidden
    s = synth.step_inputs(shp)
    m = synth.model_weights(shp, int8=False)
    exact = O.denoise_step(s["z"], s["txt"], s["ids"], m, shp, 0.9, 0.9 - 1 / 28, 3.5)[1]
    q8 = O.denoise_step(s["z"], s["txt"], s["ids"], m, shp, 0.9, 0.9 - 1 / 28, 3.5, fp8=True)[1]
    e = np.sqrt(np.mean((q8 - exact) ** 2)) / np.sqrt(np.mean(exact ** 2))
    assert 1e-3 < e < 0.1, e
    for wd in m["double"]:
        for st in ("txt", "img"):
            m_ = wd[st]["mod"]
            for r0 in (2 * H, 5 * H):
                m_.w[r0:r0 + H] = 0
                m_.b[r0:r0 + H] = 0
    for ws in m["single"]:
        ws["mod"].w[2 * H:] = 0
        ws["mod"].b[2 * H:] = 0

    def decoded(o):
        if isinstance(o, dict):
            return {k: decoded(v) for k, v in o.items()}
        if isinstance(o, list):
            return [decoded(v) for v in o]
        if isinstance(o, O.Fp8Linear):
            return synth.Linear(np.asarray(o.s, np.float64)[:, None] * o.q, o.b)
        return o
    md = decoded(O.fp8_weights(m))
    z8, v8 = O.denoise_step(s["z"], s["txt"], s["ids"], m, shp, 0.9, 0.9 - 1 / 28, 3.5, fp8=True)
    z1, v1 = O.denoise_step(s["z"], s["txt"], s["ids"], md, shp, 0.9, 0.9 - 1 / 28, 3.5)
    np.testing.assert_allclose(v8, v1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z8, z1, rtol=1e-12, atol=1e-12)
    assert np.max(np.abs(md["img_in"].w - m["img_in"].w)) > 0      # the weights were quantised


# With a zero query projection (weights and bias) every query is the zero
# vector after RMSNorm, every logit is 0 and attention is the plain mean of the
# values over the whole joint sequence, whatever the keys and RoPE. The blocks
# then have closed forms through their LayerNorm + modulation, value columns,
# output projection and gates (Luminal blog, "What the compiler found on its
# own": LN then a scale and a shift; joint attention over the concatenated
# streams; a gate-and-residual add after each branch).
def _double_value_path_gap():
    """max |oracle - closed form| of the double block with uniform attention,
    and the size of the branch."""
    import torch.nn.functional as F
    d = synth.block_inputs(TINY, "double", variant=6)
    H, Lt = TINY.hidden, TINY.txt_len
    w = d["w"]
    for s in ("txt", "img"):
        qkv = w[s]["qkv"]
        wq, bq = qkv.w.copy(), qkv.b.copy()
        wq[:H] = 0
        bq[:H] = 0
        w[s]["qkv"] = synth.Linear(wq, bq)
        w[s]["mod"] = _scaled(w[s]["mod"], 10.0)
        w[s]["mod"].w[5 * H:] = 0
        w[s]["mod"].b[5 * H:] = 0
        w[s]["proj"] = _scaled(w[s]["proj"], 25.0)
    out = O.double_block(d["x"], d["vec"], d["ids"], w, TINY)
    sv = F.silu(_t(d["vec"]))
    x = _t(d["x"])
    mods, vs = {}, []
    for s, sl in (("txt", slice(0, Lt)), ("img", slice(Lt, None))):
        m = _lin_t(sv, w[s]["mod"])
        mods[s] = m
        h = F.layer_norm(x[sl], (H,), eps=TINY.ln_eps) * (1 + m[H:2 * H]) + m[:H]
        vs.append(_lin_t(h, w[s]["qkv"])[:, 2 * H:])
    o = torch_cat(vs).mean(dim=0)
    want = np.empty_like(out)
    for s, sl in (("txt", slice(0, Lt)), ("img", slice(Lt, None))):
        m = mods[s]
        want[sl] = (x[sl] + m[2 * H:3 * H] * _lin_t(o, w[s]["proj"])).numpy()
    return float(np.max(np.abs(out - want))), float(np.max(np.abs(want - d["x"])))


def _single_uniform_gap():
    import torch.nn.functional as F
    d = synth.block_inputs(TINY, "single", variant=6)
    H = TINY.hidden
    w = d["w"]
    l1 = w["linear1"]
    w1, b1 = l1.w.copy() * 25.0, l1.b.copy() * 25.0
    w1[:H] = 0
    b1[:H] = 0
    w["linear1"] = synth.Linear(w1, b1)
    w["mod"] = _scaled(w["mod"], 10.0)
    w["linear2"] = _scaled(w["linear2"], 25.0)
    out = O.single_block(d["x"], d["vec"], d["ids"], w, TINY)
    m = _lin_t(F.silu(_t(d["vec"])), w["mod"])
    x = _t(d["x"])
    h = F.layer_norm(x, (H,), eps=TINY.ln_eps) * (1 + m[H:2 * H]) + m[:H]
    u = _lin_t(h, w["linear1"])
    o = u[:, 2 * H:3 * H].mean(dim=0, keepdim=True).expand(x.shape[0], H)
    cat = torch_cat([o, F.gelu(u[:, 3 * H:], approximate="tanh")], dim=1)
    want = (x + m[2 * H:3 * H] * _lin_t(cat, w["linear2"])).numpy()
    return float(np.max(np.abs(out - want))), float(np.max(np.abs(want - d["x"])))


def test_double_block_value_path_closed_form():
    """LN1 with shift1/scale1 per stream, the v columns of the qkv projection,
    attention over both streams jointly, the out-projection and gate1
    (MLP gate zeroed): x + gate1 (W_o mean_j v_j + b_o)."""
    gap, size = _double_value_path_gap()
    assert size > 0.05                      # the branch is not negligible
    assert gap <= 1e-10 * max(size, 1.0), gap


def test_single_block_closed_form_with_uniform_attention():
    """The single block with a zero query projection: LN with (shift, scale),
    linear1's v and MLP columns, attention as the mean of v, GELU on the MLP
    columns, linear2 over [attention | GELU(mlp)] and the gate."""
    gap, size = _single_uniform_gap()
    assert size > 0.05
    assert gap <= 1e-10 * max(size, 1.0), gap


def test_block_closed_forms_catch_planted_mistakes(monkeypatch):
    """Plausible mistakes planted in the oracle's blocks move them far from
    the closed forms above: shift and scale swapped in the LayerNorm
    modulation, attention restricted to each token's own stream, the
    single block's linear2 input order swapped."""
    from oracle import mmdit_oracle as M
    ln_orig, att_orig, act_orig = M.ln_modulate, M.attention, M.mlp_activation

    def ln_swapped(x, shift, scale, eps):
        return ln_orig(x, scale, shift, eps)

    def att_per_stream(q, k, v, heads, rows=None):
        Lt = TINY.txt_len
        r = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
        out = np.empty((len(r), q.shape[1]))
        for sl in (slice(0, Lt), slice(Lt, None)):
            idx = np.arange(q.shape[0])[sl]
            sel = np.isin(r, idx)
            out[sel] = att_orig(q[sl], k[sl], v[sl], heads, rows=r[sel] - idx[0])
        return out
    for name, fn, which in (("ln_modulate", ln_swapped, "both"), ("attention", att_per_stream, "double")):
        with monkeypatch.context() as mp:
            mp.setattr(M, name, fn)
            for gapf in ([_double_value_path_gap, _single_uniform_gap] if which == "both"
                         else [_double_value_path_gap]):
                gap, size = gapf()
                assert gap > 1e-3 * size, (name, gapf.__name__, gap, size)
    # the single block's [attention | GELU(mlp)] input read in the other order
    src = M.single_block

    def single_swapped(x, vec, ids, w, shp, **kw):
        H = shp.hidden
        w2 = dict(w)
        lw = w["linear2"].w
        w2["linear2"] = synth.Linear(np.concatenate([lw[:, H:2 * H], lw[:, :H], lw[:, 2 * H:]], axis=1),
                                     w["linear2"].b)
        return src(x, vec, ids, w2, shp, **kw)
    with monkeypatch.context() as mp:
        mp.setattr(M, "single_block", single_swapped)
        mp.setattr(O, "single_block", single_swapped)
        gap, size = _single_uniform_gap()
        assert gap > 1e-3 * size, gap


def torch_cat(ts, dim=0):
    import torch
    return torch.cat(ts, dim=dim)


# ---------------------------------------------------------------- fp8 attention
def _e4m3_nearest(x: float) -> float:
    """Nearest finite e4m3 value by a search over the code table, ties to the
    even code (independent of the oracle's arithmetic rounding)."""
    best = None
    for c in range(127):                 # 0x00 .. 0x7e: the non-negative finite codes
        v = _e4m3_decode(c)
        d = abs(abs(x) - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c, v)
    return math.copysign(best[2], x)


def _rms_rows(x, heads):
    """Rows normalised to unit mean square per head (what RMSNorm with g = 1
    hands to the attention)."""
    L = x.shape[0]
    y = x.reshape(L, heads, -1)
    return (y / np.sqrt((y ** 2).mean(-1, keepdims=True))).reshape(L, -1)


def _attention_fp8_brute(q, k, v, heads, eq, ek, rows):
    """Scalar loops, math.ceil / 2.0 ** / math.fsum and the table rounding."""
    f32 = np.float32
    L, HD = k.shape
    D = HD // heads
    qc = {(i, j): _e4m3_nearest(float(f32(q[i, j])) * 2.0 ** -eq) for i in rows for j in range(HD)}
    kc = [[_e4m3_nearest(float(f32(k[i, j])) * 2.0 ** -ek) for j in range(HD)] for i in range(L)]
    sv, vc = [], [[0.0] * HD for _ in range(L)]
    for j in range(HD):
        amax = max(abs(f32(v[i, j])) for i in range(L))
        s = f32(f32(amax) / f32(448.0))
        sv.append(float(s))
        for i in range(L):
            vc[i][j] = _e4m3_nearest(float(f32(f32(v[i, j]) / s))) if s > 0 else 0.0
    out = np.zeros((len(rows), HD))
    for h in range(heads):
        for n, i in enumerate(rows):
            t = [math.fsum(qc[i, h * D + d] * kc[j][h * D + d] for d in range(D))
                 * 2.0 ** (eq + ek) * math.log2(math.e) / math.sqrt(D) for j in range(L)]
            M = math.ceil(max(t))
            p = [2.0 ** (tj - M + 8) for tj in t]
            den = math.fsum(p)
            for d in range(D):
                col = h * D + d
                out[n, col] = math.fsum(_e4m3_nearest(p[j]) * vc[j][col] * sv[col] for j in range(L)) / den
    return out


def test_attention_fp8_brute_force_tiny():
    """attention_fp8 against scalar loops on a tiny case (SGLang-AMD,
    Architecture Deep Dive: fp8 on CDNA): codes of q and k at power-of-two
    scales, per-channel v codes (an all-zero channel gets scale 0 and zero
    output), logits in log2 units, exponentials against the integer ceiling
    of the row maximum, their e4m3 codes in the value product and their exact
    sum in the denominator; a row subset equals the same rows of the whole."""
    g = np.random.default_rng(71)
    L, heads, D = 9, 2, 8
    q = _rms_rows(g.standard_normal((L, heads * D)), heads) * 1.3
    k = _rms_rows(g.standard_normal((L, heads * D)), heads) * 0.7
    v = g.standard_normal((L, heads * D))
    v[:, 5] = 0.0
    eq = O.qk_fp8_exponent([np.full(D, 1.3)], D)
    ek = O.qk_fp8_exponent([np.full(D, 0.7)], D)
    rows = [0, 3, 8]
    got = O.attention_fp8(q, k, v, heads, eq, ek)
    np.testing.assert_allclose(got[rows], _attention_fp8_brute(q, k, v, heads, eq, ek, rows), rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(O.attention_fp8(q, k, v, heads, eq, ek, rows=np.array(rows)), got[rows])
    assert np.all(got[:, 5] == 0.0)


def _fp8_exact_channels(L, C, g):
    """v whose every channel is e4m3 values times a power of two, with the top
    code in each channel: per-channel quantisation is the identity on it."""
    vals = np.array(sorted({_e4m3_decode(c) for c in range(256) if not math.isnan(_e4m3_decode(c))}))
    v = g.choice(vals, size=(L, C))
    v[g.integers(0, L, size=C), np.arange(C)] = 448.0
    return v * np.exp2(g.integers(-9, -3, size=(1, C)))


def test_attention_fp8_zero_queries_give_the_mean_of_the_values():
    """q = 0: every logit is 0, M = 0, every exponential is exactly 256 (an
    e4m3 value), so the output is the plain mean of the values over the keys
    when v is fp8-exact per channel."""
    g = np.random.default_rng(72)
    L, heads, D = 37, 3, 64
    v = _fp8_exact_channels(L, heads * D, g)
    k = _rms_rows(g.standard_normal((L, heads * D)), heads)
    out = O.attention_fp8(np.zeros((L, heads * D)), k, v, heads, -3, -3)
    np.testing.assert_allclose(out, np.tile(v.mean(axis=0), (L, 1)), rtol=1e-14, atol=0)


def test_attention_fp8_single_key_closed_form():
    """L = 1: t = c q.k, M = ceil(t), p = 2^(8 + t - M) in (128, 256], whose
    e4m3 code lies on the grid of step 16 there; the output is v * code / p.
    The integer reference and the exact denominator are what set the factor."""
    heads, D = 1, 64
    g = np.random.default_rng(73)
    for trial in range(20):
        q = g.choice([-1.0, -0.5, 0.5, 1.0, 2.0], size=(1, D)) * 2.0 ** -3
        k = g.choice([-1.0, 0.5, 1.0, 1.5], size=(1, D)) * 2.0 ** -2
        v = _fp8_exact_channels(1, D, g)
        t = float(np.dot(q[0], k[0])) * math.log2(math.e) / math.sqrt(D)
        p = 2.0 ** (8 + t - math.ceil(t))
        code = round(p / 16.0) * 16.0 if abs(p / 16.0 - math.floor(p / 16.0) - 0.5) > 1e-12 else None
        if code is None:
            continue
        want = v * code / p
        np.testing.assert_allclose(O.attention_fp8(q, k, v, heads, -3, -2), want, rtol=1e-13)


def test_attention_fp8_invariances_and_distance_from_exact_attention():
    """Doubling one value channel doubles that output channel exactly (its
    scale doubles, its codes stay); permuting the keys with their values
    leaves the output unchanged; the result stays within the fp8 noise of the
    exact attention (each operand rounded to 3 mantissa bits: a few percent
    of the output RMS here) and is not the exact attention."""
    g = np.random.default_rng(74)
    L, heads, D = 96, 2, 64
    q = _rms_rows(g.standard_normal((L, heads * D)), heads)
    k = _rms_rows(g.standard_normal((L, heads * D)), heads)
    v = g.standard_normal((L, heads * D))
    e = O.qk_fp8_exponent([np.ones(D)], D)
    base = O.attention_fp8(q, k, v, heads, e, e)
    v2 = v.copy(); v2[:, 17] *= 2.0
    o2 = O.attention_fp8(q, k, v2, heads, e, e)
    np.testing.assert_array_equal(o2[:, 17], 2.0 * base[:, 17])
    np.testing.assert_array_equal(np.delete(o2, 17, axis=1), np.delete(base, 17, axis=1))
    perm = g.permutation(L)
    np.testing.assert_allclose(O.attention_fp8(q, k[perm], v[perm], heads, e, e), base, rtol=1e-12, atol=1e-14)
    exact = O.attention(q, k, v, heads)
    rms = np.sqrt((exact ** 2).mean())
    err = np.sqrt(((base - exact) ** 2).mean()) / rms
    assert 5e-3 < err < 0.1, err


def test_qk_fp8_exponent_is_the_smallest_safe_power_of_two():
    """After RMSNorm and a norm scale g, even a row with all its energy in one
    element (|x_d| = sqrt(D) |g_d|) quantises within 448 at 2^e, and 2^(e-1)
    would not be safe for the bound; both streams' scales are covered."""
    g = np.random.default_rng(75)
    for D in (64, 128):
        for trial in range(6):
            ga = (g.uniform(0.2, 3.0, D) * g.choice([-1, 1], D)).astype(np.float32)
            gb = (g.uniform(0.2, 3.0, D)).astype(np.float32)
            e = O.qk_fp8_exponent([ga, gb], D)
            gmax = max(np.max(np.abs(ga)), np.max(np.abs(gb)))
            bound = float(np.float32(np.float32(math.sqrt(D) / 448.0) * np.float32(gmax)))
            assert 2.0 ** (e - 1) < bound <= 2.0 ** e
            d = int(np.argmax(np.abs(np.concatenate([ga, gb]))) % D)
            gsel = ga if np.max(np.abs(ga)) >= np.max(np.abs(gb)) else gb
            x = np.zeros((1, D)); x[0, d] = math.sqrt(D) * float(gsel[d])
            codes = O.quantize_pow2_fp8(x, e)
            assert np.max(np.abs(codes)) <= 448.0
    assert O.qk_fp8_exponent([np.full(64, 0.5)], 64) == -6       # 8 * 0.5 / 448 = 2^-6.807...
    assert O.qk_fp8_exponent([np.full(16, 112.0)], 16) == 0      # 4 * 112 / 448 = 1 exactly


def test_attention_fp8_pins_catch_planted_mistakes():
    """Mistaken versions of the fp8 attention (floor for the integer ceiling,
    the exact maximum as reference, quantised exponentials in the
    denominator, one scale for all value channels, the scale exponent's sign
    flipped) each fail one of the closed forms above."""
    def make(mut):
        def att(q, k, v, heads, eq, ek, rows=None):
            if mut == "sign":     # codes taken at 2^-e instead of 2^e
                qc = O.quantize_pow2_fp8(q, -eq) if abs(eq) < 4 else O.quantize_pow2_fp8(q * 0, 0)
                kc = O.quantize_pow2_fp8(k, -ek) if abs(ek) < 4 else O.quantize_pow2_fp8(k * 0, 0)
            else:
                qc, kc = O.quantize_pow2_fp8(q, eq), O.quantize_pow2_fp8(k, ek)
            if mut == "tensor_v":
                s = np.float32(np.max(np.abs(v)) / 448.0)
                vc, sv = O.e4m3_round(np.asarray(v, np.float32) / s), np.full(v.shape[1], s)
            else:
                vc, sv = O.quantize_cols_fp8(v)
            L, HD = kc.shape
            D = HD // heads
            r = np.arange(qc.shape[0]) if rows is None else np.asarray(rows)
            c = math.log2(math.e) / math.sqrt(D) * 2.0 ** (eq + ek)
            out = np.empty((len(r), HD))
            for h in range(heads):
                sl = slice(h * D, (h + 1) * D)
                t = (qc[r, sl] @ kc[:, sl].T) * c
                M = {"floor": np.floor, "exact": lambda a: a}.get(mut, np.ceil)(t.max(axis=1, keepdims=True))
                p = np.exp2(t - M + 8.0)
                p8 = O.e4m3_round(np.minimum(p, 448.0))
                den = p8.sum(axis=1, keepdims=True) if mut == "den" else p.sum(axis=1, keepdims=True)
                out[:, sl] = (p8 @ (vc[:, sl] * sv[sl][None, :])) / den
            return out
        return att

    def fails(fn):
        try:
            with pytest.MonkeyPatch.context() as mp:
                mp.setattr(O, "attention_fp8", fn)
                for t in (test_attention_fp8_zero_queries_give_the_mean_of_the_values,
                          test_attention_fp8_single_key_closed_form,
                          test_attention_fp8_brute_force_tiny):
                    t()
        except AssertionError:
            return True
        return False
    assert not fails(O.attention_fp8)
    for mut in ("floor", "exact", "den", "tensor_v", "sign"):
        assert fails(make(mut)), mut
