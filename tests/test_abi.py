"""The C-ABI library loads, exports every function include/mmdit.h declares,
and rejects bad arguments on the host before launching anything (these
calls return an error status without touching a GPU)."""
import ctypes

import pytest

from diffusion_transformer_image_mm_amd import binding as B
from diffusion_transformer_image_mm_amd import synth
from diffusion_transformer_image_mm_amd.device import dims_for

FAKE = 1 << 20  # a 16-byte aligned, never-dereferenced address


def test_exports_every_header_function():
    names = B.header_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(B.lib, n), n
        assert callable(getattr(B, n)), n


def test_abi_version_and_status_strings():
    assert B.mmdit_abi_version() == B.MMDIT_ABI_VERSION == 3
    for st in range(9):
        assert B.mmdit_status_string(st)
    assert B.mmdit_status_string(99) == "unknown status"


def _dims(**kw):
    d = dims_for(synth.TINY)
    for k, v in kw.items():
        if k == "rope_axes":
            for i in range(3):
                d.rope_axes[i] = v[i]
        else:
            setattr(d, k, v)
    return d


def _linear():
    return B.mmdit_linear(FAKE, 0, FAKE)


def _double():
    s = B.mmdit_stream_weights(_linear(), _linear(), _linear(), _linear(), _linear(), FAKE, FAKE)
    return B.mmdit_double_weights(s, s)


@pytest.mark.parametrize("kw,status", [
    ({"head_dim": 96, "hidden": 384}, B.MMDIT_E_SHAPE),
    ({"hidden": 320}, B.MMDIT_E_SHAPE),            # hidden != heads * head_dim
    ({"rope_axes": (8, 28, 26)}, B.MMDIT_E_SHAPE),  # axes do not sum to D
    ({"rope_axes": (9, 27, 28)}, B.MMDIT_E_SHAPE),  # odd axis
    ({"txt_len": 0}, B.MMDIT_E_SHAPE),
    ({"img_len": 0}, B.MMDIT_E_SHAPE),
    ({"mlp_hidden": 1000}, B.MMDIT_E_SHAPE),
    ({"mlp_hidden": 65536 + 64}, B.MMDIT_E_SHAPE),   # beyond the documented maximum
    ({"weight_dtype": 5}, B.MMDIT_E_DTYPE),
    ({"mlp_act": 2}, B.MMDIT_E_ARG),
    ({"guidance_embed": 2}, B.MMDIT_E_ARG),
    ({"ref_len": 256}, B.MMDIT_E_SHAPE),             # ref_len must be < img_len (256)
    ({"ref_len": -1}, B.MMDIT_E_SHAPE),
    ({"mlp_act": B.MMDIT_ACT_SWIGLU, "mlp_hidden": 1088}, B.MMDIT_E_SHAPE),   # SwiGLU: M % 128
    ({"mlp_act": B.MMDIT_ACT_SWIGLU, "hidden": 192, "heads": 3}, B.MMDIT_E_SHAPE),  # SwiGLU: H % 256
])
def test_block_rejects_bad_dims(kw, status):
    d = _dims(**kw)
    assert B.mmdit_workspace_bytes(d, B.MMDIT_WS_DOUBLE) == 0
    w = _double()
    assert B.mmdit_block_forward(d, w, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40) == status


def test_block_rejects_null_misaligned_small_workspace_and_missing_scales():
    d = _dims()
    w = _double()
    need = B.mmdit_workspace_bytes(d, B.MMDIT_WS_DOUBLE)
    assert need > 0
    assert B.mmdit_block_forward(d, w, 0, FAKE, FAKE, FAKE, FAKE, need) == B.MMDIT_E_NULL
    assert B.mmdit_block_forward(d, w, FAKE + 4, FAKE, FAKE, FAKE, FAKE, need) == B.MMDIT_E_ALIGN
    assert B.mmdit_block_forward(d, w, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1) == B.MMDIT_E_WORKSPACE
    w.img.fc2.bias = 0
    assert B.mmdit_block_forward(d, w, FAKE, FAKE, FAKE, FAKE, FAKE, need) == B.MMDIT_E_NULL
    d8 = _dims(weight_dtype=B.MMDIT_INT8)
    assert B.mmdit_block_forward(d8, _double(), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40) == B.MMDIT_E_DTYPE


def test_single_and_step_validation():
    d = _dims()
    sw = B.mmdit_single_weights(_linear(), _linear(), _linear(), FAKE, FAKE)
    need = B.mmdit_workspace_bytes(d, B.MMDIT_WS_SINGLE)
    assert B.mmdit_single_block_forward(d, sw, FAKE, FAKE, FAKE, FAKE, FAKE, need - 256) == B.MMDIT_E_WORKSPACE
    sw.q_norm = FAKE + 2
    assert B.mmdit_single_block_forward(d, sw, FAKE, FAKE, FAKE, FAKE, FAKE, need) == B.MMDIT_E_ALIGN
    m = B.mmdit_model()
    for f in ("img_in", "final_mod", "final_out"):
        setattr(m, f, _linear())
    for i in range(2):
        m.time_in[i] = _linear()
        m.guid_in[i] = _linear()
    d.n_double, d.n_single = 1, 0
    assert B.mmdit_denoise_step(d, m, FAKE, FAKE, FAKE, 1.0, 0.9, 3.5, FAKE, 1 << 40) == B.MMDIT_E_NULL  # no doubles
    d.n_double = 0
    need = B.mmdit_workspace_bytes(d, B.MMDIT_WS_STEP)
    assert B.mmdit_denoise_step(d, m, FAKE, FAKE, FAKE, 1.0, 0.9, 3.5, FAKE, need - 1) == B.MMDIT_E_WORKSPACE
    assert B.mmdit_denoise_step(d, m, FAKE, FAKE, FAKE, float("nan"), 0.9, 3.5, FAKE, need) == B.MMDIT_E_ARG
    d.in_channels = 48
    assert B.mmdit_denoise_step(d, m, FAKE, FAKE, FAKE, 1.0, 0.9, 3.5, FAKE, need) == B.MMDIT_E_SHAPE
    d.in_channels = 64
    m.guid_in[1] = B.mmdit_linear(0, 0, FAKE)
    assert B.mmdit_denoise_step(d, m, FAKE, FAKE, FAKE, 1.0, 0.9, 3.5, FAKE, need) == B.MMDIT_E_NULL
    d.guidance_embed = 0   # a guidance-free model does not read guid_in
    need = B.mmdit_workspace_bytes(d, B.MMDIT_WS_STEP)
    assert B.mmdit_denoise_step(d, m, FAKE, FAKE, FAKE, 1.0, 0.9, 3.5, FAKE, need - 1) == B.MMDIT_E_WORKSPACE


def test_modulation_batch_and_premod_validation():
    d = _dims()
    H = d.hidden
    d.n_double, d.n_single = 2, 3
    assert B.mmdit_modulation_floats(d) == 2 * 12 * H + 3 * 3 * H + 2 * H
    assert B.mmdit_modulation_workspace_bytes(d, 0) == 0
    assert B.mmdit_modulation_workspace_bytes(d, 257) == 0
    need = B.mmdit_modulation_workspace_bytes(d, 28)
    assert need > 0
    m = B.mmdit_model()
    for f in ("img_in", "final_mod", "final_out"):
        setattr(m, f, _linear())
    for i in range(2):
        m.time_in[i] = _linear()
        m.guid_in[i] = _linear()
    doubles = (B.mmdit_double_weights * 2)(_double(), _double())
    singles = (B.mmdit_single_weights * 3)(*[B.mmdit_single_weights(_linear(), _linear(), _linear(), FAKE, FAKE)
                                             for _ in range(3)])
    m.doubles, m.singles = doubles, singles
    ts = [1.0 - i / 28 for i in range(28)]
    assert B.mmdit_modulation_batch(d, m, [], 3.5, FAKE, FAKE, need) == B.MMDIT_E_SHAPE
    assert B.mmdit_modulation_batch(d, m, ts[:3] + [float("inf")], 3.5, FAKE, FAKE, need) == B.MMDIT_E_ARG
    assert B.mmdit_modulation_batch(d, m, ts, 3.5, FAKE + 4, FAKE, need) == B.MMDIT_E_ALIGN
    assert B.mmdit_modulation_batch(d, m, ts, 3.5, FAKE, FAKE, need - 1) == B.MMDIT_E_WORKSPACE
    step_ws = B.mmdit_workspace_bytes(d, B.MMDIT_WS_STEP)
    assert B.mmdit_denoise_step_premod(d, m, 0, FAKE, FAKE, FAKE, 1.0, 0.9, FAKE, step_ws) == B.MMDIT_E_NULL
    assert B.mmdit_denoise_step_premod(d, m, FAKE, FAKE, FAKE, FAKE, 1.0, float("nan"), FAKE, step_ws) == B.MMDIT_E_ARG
    assert B.mmdit_denoise_step_premod(d, m, FAKE, FAKE, FAKE, FAKE, 1.0, 0.9, FAKE, step_ws - 1) == \
        B.MMDIT_E_WORKSPACE


def test_kernel_entry_validation():
    assert B.mmdit_k_ln_modulate(FAKE, 10, 100, 0, FAKE, FAKE, FAKE, FAKE, 1e-6, FAKE) == B.MMDIT_E_SHAPE
    assert B.mmdit_k_ln_modulate(FAKE, 10, 256, 0, FAKE, FAKE, FAKE, FAKE, 0.0, FAKE) == B.MMDIT_E_ARG
    assert B.mmdit_k_attention(FAKE, FAKE, FAKE, 4, 100, 64, 96, FAKE, 256) == B.MMDIT_E_SHAPE  # l_pad % 64
    assert B.mmdit_k_attention(FAKE, FAKE, FAKE, 4, 100, 80, 128, FAKE, 320) == B.MMDIT_E_SHAPE
    assert B.mmdit_k_attention(FAKE, FAKE, FAKE, 4, 100, 64, 1 << 24, FAKE, 256) == B.MMDIT_E_SHAPE  # 32-bit offsets
    assert B.mmdit_k_qknorm_rope(FAKE, 768, 100, 4, 64, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6, 100,
                                 FAKE, FAKE, FAKE) == B.MMDIT_E_SHAPE
    g = B.mmdit_gemm(m=10, n=100, k=64, weight_dtype=0, a=FAKE, lda=64, w=_linear(), epilogue=0, out=FAKE, ldo=128)
    assert B.mmdit_k_gemm(g) == B.MMDIT_E_SHAPE  # n not a multiple of 64
    g.n = 128
    g.epilogue = 9
    assert B.mmdit_k_gemm(g) == B.MMDIT_E_ARG
    for internal in (64, 65, 66):   # the blocks' attention-layout epilogues are not public
        g.epilogue = internal
        assert B.mmdit_k_gemm(g) == B.MMDIT_E_ARG
    g.epilogue = B.MMDIT_EPI_GATE_RESID
    assert B.mmdit_k_gemm(g) == B.MMDIT_E_NULL  # gate / resid missing
    g.epilogue, g.weight_dtype = 0, B.MMDIT_INT8
    assert B.mmdit_k_gemm(g) == B.MMDIT_E_DTYPE  # int8 without scales
    g.weight_dtype = 4
    assert B.mmdit_k_gemm(g) == B.MMDIT_E_DTYPE
    g.weight_dtype = B.MMDIT_FP8           # fp8 operands: k a multiple of 128, a row scale, weight scales
    assert B.mmdit_k_gemm(g) == B.MMDIT_E_SHAPE
    g.k, g.lda = 128, 128
    assert B.mmdit_k_gemm(g) == B.MMDIT_E_NULL
    g.a_scale = FAKE
    assert B.mmdit_k_gemm(g) == B.MMDIT_E_DTYPE   # w.scale missing
    g.lda = 136
    assert B.mmdit_k_gemm(g) == B.MMDIT_E_SHAPE   # fp8 rows must stay 16-byte aligned
    g.k, g.lda, g.a_scale = 64, 64, None
    g.weight_dtype, g.epilogue, g.ldo = 0, B.MMDIT_EPI_SWIGLU, 64
    assert B.mmdit_k_gemm(g) == B.MMDIT_E_SHAPE  # SwiGLU: n (2M) a multiple of 256
    g.n, g.ldo = 256, 120
    assert B.mmdit_k_gemm(g) == B.MMDIT_E_SHAPE  # ldo < n / 2
    g.epilogue, g.n, g.ldo, g.split_n, g.out2, g.ldo2, g.out2_col = B.MMDIT_EPI_SPLIT_SWIGLU, 768, 256, 192, FAKE, 512, 256
    assert B.mmdit_k_gemm(g) == B.MMDIT_E_SHAPE  # split at 192: a SwiGLU tile would straddle it
    # 32-bit per-lane offsets within a 256-row tile: 256 * lda * 2 bytes and
    # 256 (SwiGLU: 256 + n/2) weight rows of k * 2 bytes must stay below 4 GiB
    g = B.mmdit_gemm(m=10, n=128, k=64, weight_dtype=0, a=FAKE, lda=(1 << 23), w=_linear(), epilogue=0,
                     out=FAKE, ldo=128)
    assert B.mmdit_k_gemm(g) == B.MMDIT_E_SHAPE
    g.lda, g.k = 1 << 23, 1 << 23
    assert B.mmdit_k_gemm(g) == B.MMDIT_E_SHAPE
    g.lda, g.k, g.n, g.ldo, g.epilogue = 4096, 4096, 1 << 20, 1 << 19, B.MMDIT_EPI_SWIGLU
    assert B.mmdit_k_gemm(g) == B.MMDIT_E_SHAPE  # (256 + n/2) rows x 8 KB > 4 GiB
    lin = _linear()
    assert B.mmdit_k_gemv(FAKE, 100, lin, 10, 0, 1, 0, FAKE) == B.MMDIT_E_SHAPE
    assert B.mmdit_k_gemv(FAKE, 128, lin, 10, 3, 1, 0, FAKE) == B.MMDIT_E_DTYPE
    assert B.mmdit_k_gemv(FAKE, 4160, lin, 10, 0, 1, 0, FAKE) == B.MMDIT_E_SHAPE  # k > 4096
    assert B.mmdit_k_euler(FAKE + 8, FAKE, 10, 0.1) == B.MMDIT_E_ALIGN


def test_quantize_fp8_validation():
    assert B.mmdit_quantize_fp8_rows(FAKE, B.MMDIT_INT8, 4, 64, 64, FAKE, 64, FAKE) == B.MMDIT_E_DTYPE
    assert B.mmdit_quantize_fp8_rows(FAKE, B.MMDIT_F16, 4, 40, 64, FAKE, 64, FAKE) == B.MMDIT_E_SHAPE
    assert B.mmdit_quantize_fp8_rows(FAKE, B.MMDIT_F16, 4, 64, 64, FAKE, 72, FAKE) == B.MMDIT_E_SHAPE
    assert B.mmdit_quantize_fp8_rows(FAKE, B.MMDIT_BF16, 4, 64, 60, FAKE, 64, FAKE) == B.MMDIT_E_SHAPE
    assert B.mmdit_quantize_fp8_rows(0, B.MMDIT_BF16, 4, 64, 64, FAKE, 64, FAKE) == B.MMDIT_E_NULL
    assert B.mmdit_quantize_fp8_rows(FAKE, B.MMDIT_BF16, 4, 64, 64, FAKE, 64, FAKE + 4) == B.MMDIT_E_ALIGN


def test_weight_conversion_validation():
    assert B.mmdit_weights_to_f16(0, FAKE, 8) == B.MMDIT_E_NULL
    assert B.mmdit_weights_to_f16(FAKE, FAKE + 2, 8) == B.MMDIT_E_ALIGN
    assert B.mmdit_weights_to_f16(FAKE, FAKE + 16, 64) == B.MMDIT_E_ARG   # overlapping ranges
    assert B.mmdit_weights_to_f16(FAKE, FAKE + 128, 0) == B.MMDIT_OK      # nothing to do
    d = _dims(weight_dtype=B.MMDIT_F16)
    assert B.mmdit_workspace_bytes(d, B.MMDIT_WS_DOUBLE) > 0
    assert B.mmdit_workspace_bytes(_dims(weight_dtype=4), B.MMDIT_WS_DOUBLE) == 0
    # fp8 blocks need the extra code and scale buffers; SwiGLU MLPs reject fp8
    d8 = _dims(weight_dtype=B.MMDIT_FP8)
    assert B.mmdit_workspace_bytes(d8, B.MMDIT_WS_DOUBLE) > B.mmdit_workspace_bytes(d, B.MMDIT_WS_DOUBLE)
    assert B.mmdit_workspace_bytes(d8, B.MMDIT_WS_SINGLE) > B.mmdit_workspace_bytes(d, B.MMDIT_WS_SINGLE)
    assert B.mmdit_workspace_bytes(_dims(weight_dtype=B.MMDIT_FP8, mlp_act=B.MMDIT_ACT_SWIGLU),
                                   B.MMDIT_WS_DOUBLE) == 0


def test_one_hip_runtime_per_process():
    """The library needs only the HIP runtime (by SONAME) and the binding
    loads PyTorch's runtime before it, so a process never holds two HSA
    runtimes (the system one next to PyTorch's)."""
    import subprocess
    import sys
    out = subprocess.run(["readelf", "-d", B.LIB_PATH], capture_output=True, text=True).stdout
    needed = [l for l in out.splitlines() if "NEEDED" in l]
    assert any("libamdhip64.so" in l for l in needed)
    assert not any("libhsa-runtime64" in l for l in needed), needed
    code = ("import sys; import diffusion_transformer_image_mm_amd.binding as b; "
            "print('torch' in sys.modules)")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       cwd=__import__("os").path.dirname(__import__("os").path.dirname(__file__)))
    assert r.stdout.strip() == "True", r.stderr


def test_modulation_batch_noalloc_rejects_sizes_beyond_its_scratch():
    shp = synth.custom_shape("noalloc-big-h4096", 732, 4096, 32, 4096, 8, (2, 2), n_double=1, n_single=1)
    d = dims_for(shp, True)
    need = B.mmdit_modulation_workspace_bytes(d, 256)
    assert need > B.MMDIT_NOALLOC_SCRATCH_BYTES
    m = B.mmdit_model()
    lin = B.mmdit_linear(FAKE, FAKE, FAKE)
    for k in ("img_in", "final_mod", "final_out"):
        setattr(m, k, lin)
    m.time_in[0] = m.time_in[1] = m.guid_in[0] = m.guid_in[1] = lin
    s = B.mmdit_stream_weights(lin, lin, lin, lin, lin, FAKE, FAKE)
    dbl = (B.mmdit_double_weights * 1)(B.mmdit_double_weights(s, s))
    sgl = (B.mmdit_single_weights * 1)(B.mmdit_single_weights(lin, lin, lin, FAKE, FAKE))
    m.doubles, m.singles = dbl, sgl
    st = B.mmdit_modulation_batch_noalloc(d, m, [0.5] * 256, 3.5, FAKE)
    assert st == B.MMDIT_E_SCRATCH, st
    assert "scratch" in B.mmdit_status_string(st)
