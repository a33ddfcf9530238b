"""Block inputs whose output depends strongly on q and k: the RMSNorm scales
of q and k doubled (exact in bf16; attention logits about four times
sharper than with the synthetic N(0,1) inputs, whose attention is nearly
uniform) and, in the double block, the MLP gate rows of the modulation
zeroed, so that x_out - x_in is the gated attention branch alone."""
from diffusion_transformer_image_mm_amd import synth


def sharp_block_inputs(shape, kind, int8=False):
    inp = synth.block_inputs(shape, kind, int8=int8)
    H = shape.hidden
    ws = [inp["w"][s] for s in ("txt", "img")] if kind == "double" else [inp["w"]]
    for w in ws:
        w["q_norm"] = w["q_norm"] * 2.0
        w["k_norm"] = w["k_norm"] * 2.0
        if kind == "double":   # gate2: modulation rows [5H, 6H)
            lin = w["mod"]
            if lin.w is not None:
                lin.w[5 * H:] = 0
            else:              # int8 layer: zero codes
                lin.q[5 * H:] = 0
            lin.b[5 * H:] = 0
    return inp


def update_rms_err(x_out, ref_out, x_in):
    """RMS of the error of the block's update over the RMS of the reference update."""
    import numpy as np
    du = np.asarray(x_out, np.float64) - x_in
    dr = np.asarray(ref_out, np.float64) - x_in
    return float(np.sqrt(np.mean((du - dr) ** 2)) / np.sqrt(np.mean(dr ** 2)))
