"""mmdit_modulation_batch_noalloc, the entry point that allocates nothing
(its scratch is a fixed device array in the library), against
mmdit_modulation_batch with a caller-provided workspace: bit for bit, on two
calls in a row, the second with fewer steps (so it reuses scratch that the
first call left filled), on a GELU model with int8 weights and on a
guidance-free SwiGLU one."""
import numpy as np
import pytest

from diffusion_transformer_image_mm_amd import binding as B
from diffusion_transformer_image_mm_amd import synth
from diffusion_transformer_image_mm_amd.device import dims_for
from gpu_helpers import DeviceArena, say, stream, sync

pytestmark = pytest.mark.gpu

STEP = synth.custom_shape("noalloc-step-h256-2d2s", 730, 256, 4, 1024, 64, (16, 16), n_double=2, n_single=2)
KLEIN = synth.custom_shape("noalloc-klein-h256-2d2s", 731, 256, 4, 768, 64, (8, 8), n_double=2, n_single=2,
                           **synth.KLEIN_KW)


@pytest.mark.parametrize("shape,int8", [(STEP, True), (KLEIN, False)])
def test_modulation_batch_noalloc_matches_workspace_entry(shape, int8):
    say(f"modulation batch noalloc {shape.name} int8={int8}")
    m = synth.model_weights(shape, int8=int8)
    A = DeviceArena()
    d = dims_for(shape, int8)
    mm = A.model(m)
    nf = B.mmdit_modulation_floats(d)
    ts = synth.sigma_schedule(28)
    for n_steps, g in ((7, 3.5), (3, 2.0)):        # the second call is smaller
        t = ts[5:5 + n_steps]
        ref = A.empty_f32(n_steps, nf)
        ws = A.workspace(B.mmdit_modulation_workspace_bytes(d, n_steps))
        B.check(B.mmdit_modulation_batch(d, mm, t, g, ref, ws, ws.numel(), stream()), "modbatch")
        got = A.empty_f32(n_steps, nf)
        got.fill_(float("nan"))
        B.check(B.mmdit_modulation_batch_noalloc(d, mm, t, g, got, stream()), "modbatch noalloc")
        sync()
        a, b = ref.cpu().numpy(), got.cpu().numpy()
        say(f"  n_steps={n_steps}: max |noalloc - workspace| = {np.max(np.abs(a - b)):.3e}")
        assert np.all(np.isfinite(b))
        np.testing.assert_array_equal(b, a)
