"""The full FLUX.1-dev-shaped denoise step at its real size against the CPU
oracle: 19 double + 38 single blocks at hidden 3072 (512 text + 4096 image
tokens), int8 weight-only linears everywhere (per-output-channel scales from
the quantiser of the input generator), guidance 3.5, step 0 of 28
(t 1 -> 1 - 1/28); the flux-amd-rocm benchmarks page header fixes 28 steps,
guidance 3.5 and int8 weight-only linears.

The oracle's velocity for this step (about 74 TFLOP in fp64, 15-30 minutes
on a CPU) is stored in tests/golden/flux_step_int8_step0.npz, written by
tests/golden/make_flux_step_golden.py, which calls only the oracle and the
input generator. This test regenerates the same seeded weights (checking
their fingerprints first), runs mmdit_denoise_step through the C ABI, and
compares the updated latent z and the velocity v = (z1 - z0) / (t1 - t0)
with the oracle's, to the 2e-2 bar; then reruns the step bit for bit.
"""
import hashlib
import json
import os
import time

import numpy as np
import pytest

import oracle as O
from diffusion_transformer_image_mm_amd import binding as B
from diffusion_transformer_image_mm_amd import synth
from diffusion_transformer_image_mm_amd.device import dims_for
from gpu_helpers import TOL, DeviceArena, rel_err, say, stream, sync

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fingerprint(lin) -> str:
    h = hashlib.sha256()
    for a in (lin.q, lin.s, lin.b):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()[:16]


def test_flux_step_int8_full_shape_matches_oracle():
    with open(os.path.join(GOLDEN, "flux_step_int8_step0.json")) as f:
        meta = json.load(f)
    with np.load(os.path.join(GOLDEN, "flux_step_int8_step0.npz"), allow_pickle=False) as g:
        v_ref = g["v"].astype(np.float64)
        t0, t1, guidance = float(g["t0"]), float(g["t1"]), float(g["guidance"])
    shp = synth.FLUX_STEP
    assert meta["shape"] == shp.name and v_ref.shape == (shp.img_len, shp.in_channels)
    say(f"flux step int8 full shape: generating {shp.n_double} + {shp.n_single} blocks of seeded int8 weights")
    t = time.time()

    def progress(kind, i, n):
        if i == n or i % 8 == 0:
            say(f"  {kind} blocks {i}/{n} ({time.time() - t:.0f} s)")
    m = synth.model_weights(shp, int8=True, progress=progress)
    fps = {"img_in": m["img_in"], "time_in.1": m["time_in"][1], "double.0.img.fc1": m["double"][0]["img"]["fc1"],
           "double.18.txt.qkv": m["double"][18]["txt"]["qkv"], "single.37.linear2": m["single"][37]["linear2"],
           "final_out": m["final_out"]}
    for k, lin in fps.items():
        assert _fingerprint(lin) == meta["weight_fingerprints"][k], f"generated weights differ from the golden's: {k}"
    s = synth.step_inputs(shp)
    say("  uploading the int8 model")
    A = DeviceArena()
    d = dims_for(shp, int8=True)
    mm = A.model(m)
    del m
    rope = A.empty_f32(shp.seq_len, shp.head_dim // 2, 2)
    B.check(B.mmdit_rope_table(d, A.i32(s["ids"]), rope, stream()), "rope")
    txt = A.f32(s["txt"])
    ws = A.workspace(B.mmdit_workspace_bytes(d, B.MMDIT_WS_STEP))
    outs = []
    for rep in range(2):
        z = A.f32(s["z"])
        say(f"  mmdit_denoise_step run {rep}")
        B.check(B.mmdit_denoise_step(d, mm, z, txt, rope, t0, t1, guidance, ws, ws.numel(), stream()), "step")
        sync()
        outs.append(z.cpu().numpy())
    g1 = outs[0]
    z_ref = O.euler(s["z"], v_ref, t0, t1)
    v_gpu = (g1.astype(np.float64) - s["z"]) / (t1 - t0)
    ez, ev = rel_err(g1, z_ref), rel_err(v_gpu, v_ref)
    say(f"  full FLUX int8 step: rel_err(z)={ez:.3e} rel_err(v)={ev:.3e} (bar {TOL})")
    assert ez <= TOL, ez
    assert ev <= TOL, ev
    np.testing.assert_array_equal(outs[1], g1)
