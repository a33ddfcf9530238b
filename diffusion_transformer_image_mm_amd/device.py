"""Device-side holders for the C ABI: upload seeded host arrays to HBM and
fill the ABI's weight structs with their addresses.

PyTorch is used only to allocate device memory, copy host arrays into it and
provide streams; every computation runs in libmmdit.so.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np
import torch

from . import binding as B
from . import synth


class DeviceArena:
    """Owns device tensors so that the addresses in ABI structs stay valid.
    With f16_weights, the bf16 weights of every non-int8 linear are uploaded
    and re-encoded on the device by mmdit_weights_to_f16 (MMDIT_F16); with
    fp8_weights, quantised per output channel on the device by
    mmdit_quantize_fp8_rows (MMDIT_FP8: e4m3 codes + fp32 scales)."""

    def __init__(self, device: str = "cuda", f16_weights: bool = False, fp8_weights: bool = False):
        assert not (f16_weights and fp8_weights)
        self.device = torch.device(device)
        self.keep: List[torch.Tensor] = []
        self.f16_weights = f16_weights
        self.fp8_weights = fp8_weights

    def _hold(self, t: torch.Tensor) -> torch.Tensor:
        self.keep.append(t)
        return t

    def _upload_bf16(self, a: np.ndarray) -> torch.Tensor:
        bits = synth.bf16_bits(np.asarray(a, dtype=np.float32))
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(self.device)

    def bf16(self, a: np.ndarray) -> torch.Tensor:
        return self._hold(self._upload_bf16(a))

    def f16(self, a: np.ndarray) -> torch.Tensor:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32).astype(np.float16))
        return self._hold(t.to(self.device))

    def f32(self, a: np.ndarray) -> torch.Tensor:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
        return self._hold(t.to(self.device))

    def i8(self, a: np.ndarray) -> torch.Tensor:
        return self._hold(torch.from_numpy(np.ascontiguousarray(a, dtype=np.int8)).to(self.device))

    def i32(self, a: np.ndarray) -> torch.Tensor:
        return self._hold(torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(self.device))

    def empty_f32(self, *shape) -> torch.Tensor:
        return self._hold(torch.empty(*shape, dtype=torch.float32, device=self.device))

    def empty_bf16(self, *shape) -> torch.Tensor:
        return self._hold(torch.empty(*shape, dtype=torch.bfloat16, device=self.device))

    def empty_f16(self, *shape) -> torch.Tensor:
        return self._hold(torch.empty(*shape, dtype=torch.float16, device=self.device))

    def workspace(self, nbytes: int) -> torch.Tensor:
        return self._hold(torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=self.device))

    # ------------------------------------------------------------ weights
    def linear(self, lin: synth.Linear) -> B.mmdit_linear:
        b = self.bf16(lin.b)
        if lin.is_int8:
            q = self.i8(lin.q)
            s = self.f32(lin.s)
            return B.mmdit_linear(q.data_ptr(), s.data_ptr(), b.data_ptr())
        if self.fp8_weights:
            codes, scales = to_fp8_weights(self._upload_bf16(lin.w))
            self._hold(codes)
            self._hold(scales)
            return B.mmdit_linear(codes.data_ptr(), scales.data_ptr(), b.data_ptr())
        if self.f16_weights:
            w = self._hold(to_f16_weights(self._upload_bf16(lin.w)))
        else:
            w = self.bf16(lin.w)
        return B.mmdit_linear(w.data_ptr(), None, b.data_ptr())

    def stream_weights(self, s: Dict) -> B.mmdit_stream_weights:
        return B.mmdit_stream_weights(
            self.linear(s["mod"]), self.linear(s["qkv"]), self.linear(s["proj"]), self.linear(s["fc1"]),
            self.linear(s["fc2"]), self.bf16(s["q_norm"]).data_ptr(), self.bf16(s["k_norm"]).data_ptr())

    def double_weights(self, w: Dict) -> B.mmdit_double_weights:
        return B.mmdit_double_weights(self.stream_weights(w["txt"]), self.stream_weights(w["img"]))

    def single_weights(self, w: Dict) -> B.mmdit_single_weights:
        return B.mmdit_single_weights(self.linear(w["mod"]), self.linear(w["linear1"]), self.linear(w["linear2"]),
                                      self.bf16(w["q_norm"]).data_ptr(), self.bf16(w["k_norm"]).data_ptr())

    def model(self, m: Dict) -> B.mmdit_model:
        nd, ns = len(m["double"]), len(m["single"])
        doubles = (B.mmdit_double_weights * max(nd, 1))(*[self.double_weights(w) for w in m["double"]])
        singles = (B.mmdit_single_weights * max(ns, 1))(*[self.single_weights(w) for w in m["single"]])
        self.keep_host = getattr(self, "keep_host", []) + [doubles, singles]
        mm = B.mmdit_model()
        mm.img_in = self.linear(m["img_in"])
        mm.time_in[0] = self.linear(m["time_in"][0])
        mm.time_in[1] = self.linear(m["time_in"][1])
        if m.get("guid_in") is not None:
            mm.guid_in[0] = self.linear(m["guid_in"][0])
            mm.guid_in[1] = self.linear(m["guid_in"][1])
        mm.final_mod = self.linear(m["final_mod"])
        mm.final_out = self.linear(m["final_out"])
        mm.doubles = doubles
        mm.singles = singles
        return mm


def to_f16_weights(w: torch.Tensor) -> torch.Tensor:
    """bf16 device weights -> the fp16 copy that mmdit_weights_to_f16 makes on
    the current stream (the torch allocator orders any reuse of w's memory
    after that stream's work, so w may be dropped right away)."""
    assert w.dtype == torch.bfloat16 and w.is_contiguous()
    out = torch.empty(w.shape, dtype=torch.float16, device=w.device)
    B.check(B.mmdit_weights_to_f16(w, out, w.numel(), torch.cuda.current_stream()))
    return out


def to_fp8_weights(w: torch.Tensor):
    """bf16 device weights [n, k] -> (e4m3 codes uint8 [n, k], fp32 scales
    [n]), one scale per output channel, made by mmdit_quantize_fp8_rows on the
    current stream (w may be dropped right away, as for to_f16_weights)."""
    assert w.dtype == torch.bfloat16 and w.is_contiguous() and w.dim() == 2
    n, k = w.shape
    codes = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    scales = torch.empty((n,), dtype=torch.float32, device=w.device)
    B.check(B.mmdit_quantize_fp8_rows(w, B.MMDIT_BF16, n, k, k, codes, k, scales,
                                      torch.cuda.current_stream()), "quantize fp8 weights")
    return codes, scales


class TimingModel:
    """A whole denoiser with random weights drawn directly in HBM (seeded torch
    device generator), for timing the full-depth step where host generation
    of ~12 B parameters would dominate. bf16 layers: N(0, 0.02) weights and
    biases; int8 layers: codes uniform on [-127, 127] with a per-channel scale
    of 0.02 / 73.6 (the codes' standard deviation), so W has std 0.02; fp8
    layers: the bf16 draws quantised per output channel on the device;
    RMSNorm scales U(0.5, 1.5). Values are not checked against the oracle
    (the parity tests use the host generator)."""

    def __init__(self, shp: synth.Shape, int8: bool, seed: int = 42, device: str = "cuda", f16: bool = False,
                 fp8: bool = False):
        self.dev = torch.device(device)
        self.gen = torch.Generator(device=self.dev)
        self.gen.manual_seed(seed)
        self.int8 = int8
        self.f16 = f16 and not int8
        self.fp8 = fp8 and not int8 and not f16
        self.keep: List[torch.Tensor] = []
        H, M, C, D = shp.hidden, shp.mlp, shp.in_channels, shp.head_dim
        MO = shp.mlp_out
        mk = self._linear
        norm = self._norm
        shared = {}

        def mod(key, n):
            # one modulation linear per block type when the shape shares them
            if not shp.shared_mod:
                return mk(n, H)
            if key not in shared:
                shared[key] = mk(n, H)
            return shared[key]

        def stream_w(key):
            return B.mmdit_stream_weights(mod(key, 6 * H), mk(3 * H, H), mk(H, H), mk(MO, H), mk(H, M), norm(D),
                                          norm(D))

        self.doubles = (B.mmdit_double_weights * max(shp.n_double, 1))(
            *[B.mmdit_double_weights(stream_w("txt"), stream_w("img")) for _ in range(shp.n_double)])
        self.singles = (B.mmdit_single_weights * max(shp.n_single, 1))(
            *[B.mmdit_single_weights(mod("single", 3 * H), mk(3 * H + MO, H), mk(H, H + M), norm(D), norm(D))
              for _ in range(shp.n_single)])
        m = B.mmdit_model()
        m.img_in = mk(H, C)
        m.time_in[0], m.time_in[1] = mk(H, 256), mk(H, H)
        if shp.guidance_embed:
            m.guid_in[0], m.guid_in[1] = mk(H, 256), mk(H, H)
        m.final_mod = mk(2 * H, H)
        m.final_out = mk(C, H)
        m.doubles = self.doubles
        m.singles = self.singles
        self.model = m

    def _hold(self, t):
        self.keep.append(t)
        return t.data_ptr()

    def _linear(self, n: int, k: int) -> B.mmdit_linear:
        b = self._hold((torch.randn(n, generator=self.gen, device=self.dev) * 0.02).to(torch.bfloat16))
        if self.int8:
            q = self._hold(torch.randint(-127, 128, (n, k), generator=self.gen, device=self.dev, dtype=torch.int8))
            s = self._hold(torch.full((n,), 0.02 / 73.6, device=self.dev, dtype=torch.float32))
            return B.mmdit_linear(q, s, b)
        w = (torch.randn(n, k, generator=self.gen, device=self.dev) * 0.02).to(torch.bfloat16)
        if self.fp8:
            codes, scales = to_fp8_weights(w)
            return B.mmdit_linear(self._hold(codes), self._hold(scales), b)
        if self.f16:
            w = to_f16_weights(w)
        return B.mmdit_linear(self._hold(w), None, b)

    def _norm(self, d: int) -> int:
        return self._hold((torch.rand(d, generator=self.gen, device=self.dev) + 0.5).to(torch.bfloat16))


def dims_for(shp: synth.Shape, int8: bool = False, f16: bool = False, fp8: bool = False) -> B.mmdit_dims:
    d = B.mmdit_dims()
    d.txt_len, d.img_len = shp.txt_len, shp.img_len
    d.hidden, d.heads, d.head_dim, d.mlp_hidden = shp.hidden, shp.heads, shp.head_dim, shp.mlp
    d.in_channels = shp.in_channels
    d.rope_axes[0], d.rope_axes[1], d.rope_axes[2] = shp.axes
    d.rope_theta, d.ln_eps, d.rms_eps = shp.theta, shp.ln_eps, shp.rms_eps
    d.weight_dtype = (B.MMDIT_INT8 if int8 else B.MMDIT_F16 if f16 else B.MMDIT_FP8 if fp8
                      else B.MMDIT_BF16)
    d.n_double, d.n_single = shp.n_double, shp.n_single
    d.mlp_act = B.MMDIT_ACT_SWIGLU if shp.mlp_act == "swiglu" else B.MMDIT_ACT_GELU_TANH
    d.guidance_embed = 1 if shp.guidance_embed else 0
    d.ref_len = shp.ref_len
    return d


def to_numpy_f32(t: torch.Tensor) -> np.ndarray:
    """Device tensor (fp32, fp16 or bf16) -> host float32 array (exact)."""
    if t.dtype == torch.bfloat16:
        return synth.bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
    if t.dtype == torch.float16:
        return t.view(torch.int16).cpu().numpy().view(np.float16).astype(np.float32)
    return t.cpu().numpy().astype(np.float32, copy=False)
