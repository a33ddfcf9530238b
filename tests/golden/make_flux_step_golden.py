"""Writes the expected velocity of step 0 of the full FLUX.1-dev-shaped
denoise step (19 double + 38 single blocks at H 3072, 512 text + 4096 image
tokens, int8 weight-only linears, guidance 3.5, t 1 -> 1 - 1/28; the
flux-amd-rocm benchmarks page header fixes 28 steps, guidance 3.5 and int8
weight-only linears) by running the CPU oracle on the seeded synthetic
weights. It calls only the oracle and the input generator.

    python tests/golden/make_flux_step_golden.py

takes ~15-30 minutes on 8-16 cores (about 74 TFLOP in fp64) and ~25 GB of
host memory. Output: flux_step_int8_step0.npz (v of every image token as
float32, plus the step's scalars) and flux_step_int8_step0.json (weight
fingerprints: the GPU test regenerates the weights and checks them first).
"""
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from diffusion_transformer_image_mm_amd import synth  # noqa: E402

SHAPE = synth.FLUX_STEP
T0, T1, GUIDANCE = 1.0, 1.0 - 1.0 / 28.0, 3.5


def fingerprints(m) -> dict:
    """sha256 (first 16 hex digits) of a few layers' codes, scales and biases."""
    def fp(lin):
        h = hashlib.sha256()
        for a in (lin.q, lin.s, lin.b):
            h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()[:16]
    return {
        "img_in": fp(m["img_in"]),
        "time_in.1": fp(m["time_in"][1]),
        "double.0.img.fc1": fp(m["double"][0]["img"]["fc1"]),
        "double.18.txt.qkv": fp(m["double"][18]["txt"]["qkv"]),
        "single.37.linear2": fp(m["single"][37]["linear2"]),
        "final_out": fp(m["final_out"]),
    }


def main() -> None:
    t = time.time()
    m = synth.model_weights(SHAPE, int8=True)
    s = synth.step_inputs(SHAPE)
    print(f"weights generated in {time.time() - t:.0f} s", flush=True)
    t = time.time()
    _, v = O.denoise_step(s["z"], s["txt"], s["ids"], m, SHAPE, T0, T1, GUIDANCE)
    dt = time.time() - t
    print(f"oracle step in {dt:.0f} s, rms(v) = {np.sqrt(np.mean(v * v)):.4f}", flush=True)
    np.savez_compressed(os.path.join(HERE, "flux_step_int8_step0.npz"), v=v.astype(np.float32),
                        t0=np.float64(T0), t1=np.float64(T1), guidance=np.float64(GUIDANCE))
    meta = {
        "what": "velocity of step 0 of the FLUX.1-dev-shaped int8 denoise step, CPU oracle (fp64), stored as float32",
        "shape": SHAPE.name, "t0": T0, "t1": T1, "guidance": GUIDANCE,
        "writer": "tests/golden/make_flux_step_golden.py (oracle + synth only)",
        "numpy": np.__version__, "oracle_seconds": round(dt, 1),
        "weight_fingerprints": fingerprints(m),
    }
    with open(os.path.join(HERE, "flux_step_int8_step0.json"), "w") as f:
        json.dump(meta, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
